"""CPU oracle for the DSpark per-step verify path. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package. The product path (the HIP
library and its Python binding) never imports, links or calls it, and shares
no code, table or helper with it.

Each function is a plain, slow, single-threaded restatement of what the pages
define, checked against the pages' printed examples and against closed forms
and brute force in ``tests/test_oracle_*.py``. Page references used in the
docstrings:

* [Budget]  akiyangdev, "DSpark 自适应 Verify 怎样分配候选预算"
* [Round]   akiyangdev, "DeepSeek-V4 DSpark 一轮 Draft、Verify、Accept 与 Commit"
* [SGLang]  yingzheng, "DSpark 接入 SGLang：用置信度驱动可变长度验证"
* [CSSD]    charlestar, "DSpark confidence-scheduled speculative decoding"
            (2026-06-11)

Precision. Where a floating-point value decides an integer (survival values
decide the top-b selection and hence ``verify_lens``), the oracle takes the
decision in the same precision as the kernels: fp32 survival built from a
*correctly rounded* fp32 sigmoid, an exact sum for tau, an fp64 ratio. The
soft accept-rate (no integer depends on it inside the stage) is fp64.
"""

from .sigmoid import sigmoid32
from .plan import (
    COST_ADDITIVE,
    COST_SPS1D,
    DATA_BAD_CONF,
    DATA_BAD_COST,
    FX_SHIFT,
    IN_COND,
    IN_CONF_LOGITS,
    IN_SURVIVAL,
    plan,
    sps_floor,
    survival,
)
from .pack import DATA_BAD_LENS, pack
from .accept import accept, row_argmax
from .tv import tv_accept
from .strided import cap_accept, scatter_to_strided
from .sts import sts_fit
from .sampling import DATA_BAD_LOGITS, accept_sampling

__all__ = [
    "sigmoid32", "survival", "plan", "pack", "accept", "row_argmax", "tv_accept",
    "cap_accept", "scatter_to_strided", "sts_fit", "accept_sampling", "DATA_BAD_LOGITS",
    "IN_CONF_LOGITS", "IN_COND", "IN_SURVIVAL", "COST_ADDITIVE", "COST_SPS1D", "sps_floor",
    "DATA_BAD_COST", "DATA_BAD_CONF", "DATA_BAD_LENS", "FX_SHIFT",
]
