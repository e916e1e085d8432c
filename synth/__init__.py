"""Seeded synthetic inputs for the CSA/HCA layer step.

This package is the only code shared by the float64 oracle (``oracle/``) and the
HIP path (``long_context_sparse_04_amd``).  It holds shapes, seeds and storage
encoders (bf16, fp8 e4m3 with a row scale, MXFP4), and none of the method's
arithmetic: no pooling, scoring, selection or attention happens here.
"""
from .configs import CONFIGS, CSAConfig, get_config  # noqa: F401
from . import gen, formats  # noqa: F401
