"""CPU oracle for the MXFP4 quantize and GEMM (float64, NumPy).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import it. The HIP product path never imports it and it
imports nothing from the HIP path. Every function cites the passage it follows
in its module docstring; the acceptance criteria live in oracle.compare.
"""

from .mxfp4_ref import (  # noqa: F401
    BLOCK,
    E2M1_VALUES,
    bf16_bits_to_f64,
    scale_exponent,
    e2m1_nearest_even,
    quantize,
    quantize_2d,
    unpack_codes,
    dequantize,
    gemm,
    gemm_block,
    gemm_entries,
)
from .stochastic import (  # noqa: F401
    DIR_ROWWISE,
    DIR_COLUMNWISE,
    philox4x32,
    seed_key,
    sr_random_bytes,
    sr_magnitude_index,
    quantize_sr_with_bytes,
    quantize_sr,
    quantize_2d_sr,
)
from .swiglu import (  # noqa: F401
    SILU_ARGMIN,
    silu,
    silu_range,
    swiglu_tolerance,
    swiglu_reference,
)
from .shuffle import (  # noqa: F401
    shuffled_sizes,
    shuffle_b,
    unshuffle_b,
)
from .frag import (  # noqa: F401
    to_frag,
    from_frag,
)
from .compare import (  # noqa: F401
    FP32_REL_TOL,
    fp32_rel_tol,
    round_to_bf16,
    bf16_bits_of,
    bf16_ordinal,
    bf16_ulp,
    check_fp32,
    check_bf16,
    check_act_bf16,
)
