"""Float64 CPU oracle for the CSA/HCA layer step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP path never calls it and shares no
code with it.  Every function follows the pages' definitions step by step in
float64 (numpy); see each function's docstring for the passage it restates.
"""
from .csa import (  # noqa: F401
    compress, index, topk, attend, hca_attend,
    rmsnorm, rope, rope_thetas,
)
from .proj import q_up_proj, grouped_out_proj  # noqa: F401
from .formats import (  # noqa: F401
    decode_bf16, encode_bf16, decode_fp8_e4m3, decode_e2m1, decode_e8m0, decode_mxfp4,
    dequant_rows, encode_fp8_rows, encode_mxfp4, fp8_e4m3_values, e2m1_values, encode_fp8_rope_rows,
    decode_fp8_rope_rows,
)
