"""Layer shapes and seeded synthetic inputs shared by the tests, the harness
and the oracle's callers.  Holds no part of the layer's arithmetic."""
from .configs import (ALIASES, BY_NAME, CONFIGS, GLAM_4K, GLAM_TINY_FP32,  # noqa: F401
                      GLM45_DECODE, GLM45_DENSE, GLM45_GROUPED, GLM45_PREFILL, GLM5_ZIPF,
                      SWITCH_TOP1,
                      MoEConfig, get, shrink)
from .gen import TENSOR_ORDER, generate, host_inputs, to_host_array, torch_dtype  # noqa: F401
