"""MI355X-native block-discrete-diffusion canvas denoising step.

The compute path lives in the HIP library ``libdg.so`` (C-ABI declared in
include/dg.h); :mod:`block_discrete_diffusion_amd.binding` marshals torch
tensors into it.  :mod:`block_discrete_diffusion_amd.synth` draws the seeded
synthetic inputs.  Importing this package loads nothing; the binding raises
if the library has not been built.
"""
__all__ = ["synth", "binding"]
