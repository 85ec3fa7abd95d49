"""Oracle package: plain CPU statement of the fused mixed-precision MoE layer.

Test infrastructure only (tests, smoke check, benchmark CPU baseline)."""
from .pagedweight_oracle import *  # noqa: F401,F403
