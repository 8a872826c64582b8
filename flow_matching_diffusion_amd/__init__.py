"""MI355X-native Flux MMDiT block forward and rectified-flow objective.

The compute lives in the HIP library ``libflux.so`` (built from ``csrc/``);
``flow_matching_diffusion_amd.flux`` is its ctypes binding.  Importing this
package does not load the library, so the CPU-only parts (``synth``) work on
machines without a GPU.
"""
__all__ = ["synth"]
