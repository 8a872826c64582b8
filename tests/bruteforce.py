"""Pure-Python (math module, nested loops) second evaluation of the Flux block
maths for tiny inputs.  It shares nothing with oracle/ and exists only to pin
the oracle: a transposed operand, a wrong axis or a dropped term in the numpy
code makes the two disagree.

It follows the same pages as the oracle ("Flux architecture deep dive", MMDiT
layer and Flux single block; "Flux model API reference", AdaLN, RMSNorm,
EmbedND) but is written element by element, and it computes softmax through a
log-sum-exp with math.fsum rather than max-subtraction.
"""
import math


def vec_linear(x, w, b):
    """x: list[in]; w: list[out][in]; b: list[out] -> list[out]."""
    return [math.fsum(w[o][i] * x[i] for i in range(len(x))) + b[o] for o in range(len(w))]


def silu(v):
    return v / (1.0 + math.exp(-v))


def gelu(v):
    return 0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0)))


def ln_mod(x, shift, scale, eps):
    n = len(x)
    mu = math.fsum(x) / n
    var = math.fsum((a - mu) ** 2 for a in x) / n
    r = 1.0 / math.sqrt(var + eps)
    return [(x[i] - mu) * r * (1.0 + scale[i]) + shift[i] for i in range(n)]


def rms(x, g, eps):
    n = len(x)
    r = 1.0 / math.sqrt(math.fsum(a * a for a in x) / n + eps)
    return [x[i] * r * g[i] for i in range(n)]


def rope_token(x, pos, axes_dim, theta):
    """Rotate one head vector: for each axis, pair j of that axis' slice."""
    out = list(x)
    off = 0
    for a, d in enumerate(axes_dim):
        for j in range(d // 2):
            ang = pos[a] / (theta ** (2.0 * j / d))
            i0 = off + 2 * j
            u, w = x[i0], x[i0 + 1]
            out[i0] = u * math.cos(ang) - w * math.sin(ang)
            out[i0 + 1] = u * math.sin(ang) + w * math.cos(ang)
        off += d
    return out


def attend(qs, ks, vs):
    """qs/ks/vs: list over tokens of head vectors -> list of outputs."""
    dh = len(qs[0])
    outs = []
    for q in qs:
        s = [math.fsum(q[d] * k[d] for d in range(dh)) / math.sqrt(dh) for k in ks]
        top = max(s)
        lse = top + math.log(math.fsum(math.exp(v - top) for v in s))
        p = [math.exp(v - lse) for v in s]
        outs.append([math.fsum(p[j] * vs[j][d] for j in range(len(ks))) for d in range(dh)])
    return outs


def _tolist(a):
    return a.tolist() if hasattr(a, "tolist") else a


def double_block(x_img, x_txt, vec, ids, w, heads, axes_dim, theta, eps):
    """x_img [B][Li][D], x_txt [B][Lt][D], vec [B][D], ids [B][Li+Lt][3]."""
    x_img, x_txt, vec, ids = map(_tolist, (x_img, x_txt, vec, ids))
    W = {k: _tolist(v) for k, v in w.items()}
    B, D = len(vec), len(vec[0])
    dh = D // heads
    out_img, out_txt = [], []
    for b in range(B):
        xs = {"img": x_img[b], "txt": x_txt[b]}
        sv = [silu(v) for v in vec[b]]
        mod, q, k, v = {}, {}, {}, {}
        for s in ("img", "txt"):
            m = vec_linear(sv, W[s + "_mod.w"], W[s + "_mod.b"])
            mod[s] = [m[i * D:(i + 1) * D] for i in range(6)]
            q[s], k[s], v[s] = [], [], []
            for tok in xs[s]:
                h = ln_mod(tok, mod[s][0], mod[s][1], eps)
                y = vec_linear(h, W[s + "_qkv.w"], W[s + "_qkv.b"])
                q[s].append([rms(y[hd * dh:(hd + 1) * dh], W[s + "_q_norm"], eps) for hd in range(heads)])
                k[s].append([rms(y[D + hd * dh:D + (hd + 1) * dh], W[s + "_k_norm"], eps) for hd in range(heads)])
                v[s].append([y[2 * D + hd * dh:2 * D + (hd + 1) * dh] for hd in range(heads)])
        joint = [("img", i) for i in range(len(xs["img"]))] + [("txt", i) for i in range(len(xs["txt"]))]
        Q = [[rope_token(q[s][i][hd], ids[b][n], axes_dim, theta) for hd in range(heads)]
             for n, (s, i) in enumerate(joint)]
        K = [[rope_token(k[s][i][hd], ids[b][n], axes_dim, theta) for hd in range(heads)]
             for n, (s, i) in enumerate(joint)]
        V = [v[s][i] for (s, i) in joint]
        O = [[] for _ in joint]
        for hd in range(heads):
            oh = attend([Q[n][hd] for n in range(len(joint))], [K[n][hd] for n in range(len(joint))],
                        [V[n][hd] for n in range(len(joint))])
            for n in range(len(joint)):
                O[n].extend(oh[n])
        res = {"img": [], "txt": []}
        for n, (s, i) in enumerate(joint):
            m = mod[s]
            p = vec_linear(O[n], W[s + "_proj.w"], W[s + "_proj.b"])
            x1 = [xs[s][i][c] + m[2][c] * p[c] for c in range(D)]
            h2 = ln_mod(x1, m[3], m[4], eps)
            u = [gelu(a) for a in vec_linear(h2, W[s + "_fc1.w"], W[s + "_fc1.b"])]
            f = vec_linear(u, W[s + "_fc2.w"], W[s + "_fc2.b"])
            res[s].append([x1[c] + m[5][c] * f[c] for c in range(D)])
        out_img.append(res["img"])
        out_txt.append(res["txt"])
    return out_img, out_txt


def single_block(x, vec, ids, w, heads, axes_dim, theta, eps):
    x, vec, ids = map(_tolist, (x, vec, ids))
    W = {k: _tolist(v) for k, v in w.items()}
    B, D = len(vec), len(vec[0])
    dh = D // heads
    out = []
    for b in range(B):
        sv = [silu(a) for a in vec[b]]
        m = vec_linear(sv, W["mod.w"], W["mod.b"])
        shift, scale, gate = m[:D], m[D:2 * D], m[2 * D:]
        Q, K, V, M = [], [], [], []
        for n, tok in enumerate(x[b]):
            h = ln_mod(tok, shift, scale, eps)
            y = vec_linear(h, W["lin1.w"], W["lin1.b"])
            Q.append([rope_token(rms(y[hd * dh:(hd + 1) * dh], W["q_norm"], eps), ids[b][n], axes_dim, theta)
                      for hd in range(heads)])
            K.append([rope_token(rms(y[D + hd * dh:D + (hd + 1) * dh], W["k_norm"], eps), ids[b][n], axes_dim,
                                 theta) for hd in range(heads)])
            V.append([y[2 * D + hd * dh:2 * D + (hd + 1) * dh] for hd in range(heads)])
            M.append([gelu(a) for a in y[3 * D:]])
        O = [[] for _ in x[b]]
        for hd in range(heads):
            oh = attend([q[hd] for q in Q], [k[hd] for k in K], [v[hd] for v in V])
            for n in range(len(O)):
                O[n].extend(oh[n])
        rows = []
        for n, tok in enumerate(x[b]):
            y2 = vec_linear(O[n] + M[n], W["lin2.w"], W["lin2.b"])
            rows.append([tok[c] + gate[c] * y2[c] for c in range(D)])
        out.append(rows)
    return out


def single_block_sequential(x, vec, ids, w, heads, axes_dim, theta, eps):
    """Sequential single block: six adaLN chunks; attention sub-block then MLP
    sub-block over the whole sequence, each with its gated residual."""
    x, vec, ids = map(_tolist, (x, vec, ids))
    W = {k: _tolist(v) for k, v in w.items()}
    B, D = len(vec), len(vec[0])
    dh = D // heads
    out = []
    for b in range(B):
        sv = [silu(a) for a in vec[b]]
        m = vec_linear(sv, W["mod.w"], W["mod.b"])
        ch = [m[i * D:(i + 1) * D] for i in range(6)]
        Q, K, V = [], [], []
        for n, tok in enumerate(x[b]):
            y = vec_linear(ln_mod(tok, ch[0], ch[1], eps), W["qkv.w"], W["qkv.b"])
            Q.append([rope_token(rms(y[hd * dh:(hd + 1) * dh], W["q_norm"], eps), ids[b][n], axes_dim, theta)
                      for hd in range(heads)])
            K.append([rope_token(rms(y[D + hd * dh:D + (hd + 1) * dh], W["k_norm"], eps), ids[b][n], axes_dim,
                                 theta) for hd in range(heads)])
            V.append([y[2 * D + hd * dh:2 * D + (hd + 1) * dh] for hd in range(heads)])
        O = [[] for _ in x[b]]
        for hd in range(heads):
            oh = attend([q[hd] for q in Q], [k[hd] for k in K], [v[hd] for v in V])
            for n in range(len(O)):
                O[n].extend(oh[n])
        rows = []
        for n, tok in enumerate(x[b]):
            p = vec_linear(O[n], W["proj.w"], W["proj.b"])
            x1 = [tok[c] + ch[2][c] * p[c] for c in range(D)]
            u = [gelu(a) for a in vec_linear(ln_mod(x1, ch[3], ch[4], eps), W["fc1.w"], W["fc1.b"])]
            f = vec_linear(u, W["fc2.w"], W["fc2.b"])
            rows.append([x1[c] + ch[5][c] * f[c] for c in range(D)])
        out.append(rows)
    return out


# --------------------------------------------------------------------------- #
# Conditioning vector and output head ("Flux architecture deep dive",
# Conditioning and Model components / Output processing; "Flux model API
# reference", Embeddings and AdaLNContinuous).  Written per sample and per
# element; the frequencies are powers of max_period, not exponentials of logs.
# --------------------------------------------------------------------------- #
def sinusoid(t, dim, time_factor=1000.0, max_period=10000.0):
    """[cos(tau f_0) .. cos(tau f_{n-1}) | sin(tau f_0) .. sin(tau f_{n-1})],
    tau = time_factor * t, f_j = max_period ** (-j / n), n = dim / 2."""
    n = dim // 2
    tau = time_factor * t
    freqs = [max_period ** (-float(j) / n) for j in range(n)]
    return [math.cos(tau * f) for f in freqs] + [math.sin(tau * f) for f in freqs]


def mlp_embed(x, w1, b1, w2, b2):
    """Linear -> SiLU -> Linear on one vector."""
    return vec_linear([silu(a) for a in vec_linear(x, w1, b1)], w2, b2)


def conditioning_vector(t, y, w, model_channels, guidance=None):
    """vec[b] = time MLP(sinusoid(t[b])) (+ pooled MLP(y[b])) (+ guidance
    Linear(g[b])): t [B], y [B][in] or None -> [B][D]."""
    t, y, guidance = map(_tolist, (t, y, guidance))
    W = {k: _tolist(v) for k, v in w.items()}
    out = []
    for b in range(len(t)):
        v = mlp_embed(sinusoid(t[b], model_channels), W["time_in1.w"], W["time_in1.b"], W["time_in2.w"],
                      W["time_in2.b"])
        if y is not None:
            p = mlp_embed(y[b], W["vector_in1.w"], W["vector_in1.b"], W["vector_in2.w"], W["vector_in2.b"])
            v = [v[i] + p[i] for i in range(len(v))]
        if guidance is not None:
            g = vec_linear([guidance[b]], W["guidance_in.w"], W["guidance_in.b"])
            v = [v[i] + g[i] for i in range(len(v))]
        out.append(v)
    return out


def patch_tokens(z):
    """[B][C][H][W] -> [B][H*W][C], token h*W + w."""
    z = _tolist(z)
    return [[[z[b][c][h][x] for c in range(len(z[b]))] for h in range(len(z[b][0])) for x in range(len(z[b][0][0]))]
            for b in range(len(z))]


def final_layer(x_img, vec, w, hh, ww, eps):
    """(shift, scale) = Linear(SiLU(vec)) split in two; each image token
    goes through LN(x)(1 + scale) + shift and the output Linear D -> C; the
    token h*W + w lands at [c][h][w].  x_img [B][H*W][D] -> [B][C][H][W]."""
    x_img, vec = map(_tolist, (x_img, vec))
    W = {k: _tolist(v) for k, v in w.items()}
    out = []
    for b in range(len(vec)):
        D = len(vec[b])
        m = vec_linear([silu(a) for a in vec[b]], W["final_mod.w"], W["final_mod.b"])
        shift, scale = m[:D], m[D:2 * D]
        toks = [vec_linear(ln_mod(x, shift, scale, eps), W["final_out.w"], W["final_out.b"]) for x in x_img[b]]
        C = len(toks[0])
        out.append([[[toks[h * ww + x][c] for x in range(ww)] for h in range(hh)] for c in range(C)])
    return out
