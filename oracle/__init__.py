"""CPU oracle (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package. The product path (text_motion_diffusion_amd) never imports it and
has no CPU fallback.
"""
from .kimodo_oracle import *  # noqa: F401,F403
