"""CPU oracle for the 3D-windowed joint-attention layer (test infrastructure only).

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  The product path (``video_dit_window_amd``) never
imports it and shares no code with it.
"""
from .wsp_oracle import *  # noqa: F401,F403
from .wsp_rope import *  # noqa: F401,F403,E402
from .wsp_fp8 import *  # noqa: F401,F403,E402
from .wsp_stack import *  # noqa: F401,F403,E402
