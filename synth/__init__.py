"""Seeded synthetic inputs for block-wise low-rank KV attention.

This package only draws numbers: workload shapes (``configs``) and seeded
factor/query/tail arrays (``gen``).  It holds none of the attention arithmetic,
so both the fp64 oracle and the HIP path can consume its output.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .configs import ENCODE_CONFIGS, EncodeConfig, get_encode_config  # noqa: F401
from .gen import Workload, LogicalBlock, make_workload, bf16_bits_to_f32  # noqa: F401
from .gen import DenseContext, make_dense_context, make_spectra  # noqa: F401
