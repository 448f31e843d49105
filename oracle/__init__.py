"""FP64 CPU oracle for the routed MoE layer forward (test infrastructure only:
the test suite, the smoke check and the CPU baseline of the benchmark use it;
the HIP path never does)."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
