"""MI355X-native SSM layer of "The Mamba in the Llama": chunked prefill and
speculative verify / commit, behind the C ABI of include/mil_ssm.h."""
from ._lib import (MIL_BF16, MIL_COMMIT_MATERIALIZE, MIL_F32, MIL_PREFILL_CONTINUE, MilError, lib)
from .ssm import SSMCache, cache_layout, supported

__all__ = ["SSMCache", "cache_layout", "supported", "lib", "MilError", "MIL_F32", "MIL_BF16",
           "MIL_PREFILL_CONTINUE", "MIL_COMMIT_MATERIALIZE"]
