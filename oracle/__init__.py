"""Float64 CPU oracle of the Kalman Linear Attention (KLA) forward scan.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The product path (the
HIP library and its Python binding) never imports it, and it imports nothing
from the product path.
"""
from .kla_f64 import (  # noqa: F401
    kla_forward_f64,
    kla_decode_step_f64,
    filter_step,
    precision_scan_f64,
    precision_path_from_coeffs,
    predict_precision,
    update_precision,
    forget_gate,
    write_gate,
    readout,
)
from .kla_ou_f64 import ou_discretize_f64, kla_forward_ou_f64  # noqa: F401,E402
from .kla_vprec_f64 import kla_forward_vprec_f64  # noqa: F401,E402
from .kla_prologue_f64 import (  # noqa: F401,E402
    causal_conv_f64, silu_f64, softplus_f64, prologue_f64, kla_forward_prologue_f64)
