"""MI355X (gfx950) library for the batched DDIM sampling loop of Kimodo's
two-stage motion denoiser.

The compute lives in libkimodo.so (hand-written HIP kernels behind the C ABI of
include/kimodo.h). ``text_motion_diffusion_amd.kimodo`` is the ctypes binding
with the same entry-point names; ``text_motion_diffusion_amd.session.Session``
keeps weights and workspace resident in torch-allocated device memory. Build the
library with ``python -m text_motion_diffusion_amd.build``.
"""
