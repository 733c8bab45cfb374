"""GPU parity of kla_forward_prologue (the forward pass on raw projections:
causal conv1d + SiLU on q, k, v, softplus on the step length and the value
precision, OU prior discretised in the kernel) against the float64 oracle
oracle/kla_prologue_f64.py, needs an MI355X.

The oracle forms the activations in float64 and rounds them to the input
dtype, as the kernel stores them (bf16: nearest even).  The kernel's fp32
convolution can land on the other side of a bf16 rounding midpoint than the
float64 one, for activations within about 2^-23 relative of one (a few per
10^5: in the 1x4x1000 d64 case, k at token 195, channel 26 of head 0 lies
1.2e-7 from a midpoint).  Such a one-unit difference in one k moves that
channel's precision by up to about 2^-7 c / lambda and y by a like amount,
inside the bf16 bar.  Bars: fp32 inputs, every output 1e-5 relative (y and
M_T against the per-head RMS), as the forward pass; bf16 inputs, every
output (the precision included) 1e-2 + 2e-2 |r| (tests/kla_testutil.py).
Every case prints its name, seed and shape before touching the GPU.
"""
import numpy as np
import pytest

import kla_inputs as KI
from kla_testutil import check_forward, say
from oracle import kla_forward_prologue_f64

pytestmark = pytest.mark.gpu

TOK = ("xq", "xk", "xv", "dt_raw", "vp_raw")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import bius_scan_sequence_amd as K
    assert torch.cuda.is_available()
    yield K
    torch.cuda.synchronize()


def _f32(a):
    import torch
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def run(x, state=True):
    import torch
    import bius_scan_sequence_amd as K
    dt = torch.bfloat16 if x["dtype"] == "bf16" else torch.float32
    xd = {n: torch.from_numpy(np.ascontiguousarray(x[n])).cuda().to(dt) for n in TOK}
    res = K.forward_prologue(xd["xq"], xd["xk"], xd["xv"], xd["dt_raw"], _f32(x["theta"]), _f32(x["sigma2"]),
                             xd["vp_raw"], tuple(_f32(w) for w in x["conv_w"]), tuple(_f32(b) for b in x["conv_b"]),
                             _f32(x["lambda0"]) if state else None, _f32(x["M0"]) if state else None,
                             return_lambda_path=True)
    torch.cuda.synchronize()
    got = tuple(t.float().cpu().numpy() for t in res)
    ref = kla_forward_prologue_f64(*(x[n] for n in ("xq", "xk", "xv", "dt_raw", "theta", "sigma2", "vp_raw")),
                                   x["conv_w"], x["conv_b"], x["lambda0"] if state else None,
                                   x["M0"] if state else None, dtype=x["dtype"], return_lambda_path=True)
    return got, ref


SHAPES = [
    # (B, H, T, dk, dv, dtype)
    (1, 1, 256, 16, 16, "f32"),
    (2, 3, 300, 32, 64, "f32"),
    (1, 2, 200, 128, 32, "f32"),
    (2, 2, 130, 64, 64, "bf16"),
    (1, 4, 1000, 64, 64, "bf16"),
    (1, 2, 300, 64, 128, "bf16"),
    (1, 2, 300, 128, 128, "bf16"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_forward_prologue_matches_oracle(shape):
    B, H, T, dk, dv, dt = shape
    seed = 9700 + T + dk + dv
    say(f"[case] forward_prologue {shape}: seed={seed}")
    x = KI.make_prologue_inputs("pro_lm45m_bf16", B=B, H=H, T=T, dk=dk, dv=dv, seed=seed, dtype=dt)
    rng = np.random.default_rng(seed)
    x["lambda0"] = (0.5 + rng.random((B, H, dk))).astype(np.float32)
    x["M0"] = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    got, ref = run(x)
    stats = check_forward(x, got, ref, dt, exact_coeffs=False)
    say(f"[ok] forward_prologue {shape}: " + ", ".join(f"{k}={v:.2e}" for k, v in stats.items()))


@pytest.mark.parametrize("width", [1, 2, 3])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_prologue_conv_widths(width, dtype):
    """Narrower convolutions (the taps fill the last slots; the others read
    nothing), without biases."""
    seed = 9650 + width
    say(f"[case] forward_prologue width {width} {dtype}: B=1 H=2 T=150 d=32 seed={seed}")
    x = KI.make_prologue_inputs("pro_lm45m_bf16", B=1, H=2, T=150, dk=32, dv=32, seed=seed, dtype=dtype,
                                conv_width=width, bias=False)
    got, ref = run(x, state=False)
    stats = check_forward(x, got, ref, dtype, exact_coeffs=False)
    say(f"[ok] forward_prologue width {width} {dtype}: " + ", ".join(f"{k}={v:.2e}" for k, v in stats.items()))


@pytest.mark.parametrize("T", [1, 2, 3, 5, 64, 65, 67])
def test_forward_prologue_short_and_boundary_lengths(T):
    """Sequences shorter than the convolution window, and lengths around one
    segment: the window reaches back across the segment boundary (or into the
    zero history before token 0)."""
    seed = 9600 + T
    say(f"[case] forward_prologue T={T}: B=2 H=1 d=16 f32 seed={seed}")
    x = KI.make_prologue_inputs("pro_lm45m_bf16", B=2, H=1, T=T, dk=16, dv=16, seed=seed, dtype="f32")
    got, ref = run(x)
    stats = check_forward(x, got, ref, "f32")
    say(f"[ok] forward_prologue T={T}: " + ", ".join(f"{k}={v:.2e}" for k, v in stats.items()))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_prologue_strong_decay_exact_path(dtype):
    """Long steps (dt_raw + 40, so dt ~ 40): chunks whose prod f over half a
    chunk falls below 2^-64 take the kernel's exact path, which forms the
    activations of its chunk from the raw projections in global memory (for
    bf16, rounded as the staged ones are)."""
    say(f"[case] forward_prologue strong decay: B=1 H=2 T=200 d=32 {dtype} seed=9590")
    x = KI.make_prologue_inputs("pro_lm45m_bf16", B=1, H=2, T=200, dk=32, dv=32, seed=9590, dtype=dtype)
    dtr = x["dt_raw"].astype(np.float32) + 40.0
    x["dt_raw"] = KI.round_bf16(dtr) if dtype == "bf16" else dtr
    got, ref = run(x, state=False)
    stats = check_forward(x, got, ref, dtype, exact_coeffs=False)
    say("[ok] forward_prologue strong decay: " + ", ".join(f"{k}={v:.2e}" for k, v in stats.items()))


@pytest.mark.parametrize("dims", [(16, 16), (16, 64), (32, 128), (128, 64)], ids=lambda d: f"{d[0]}x{d[1]}")
def test_forward_prologue_bf16_widths(dims):
    """bf16 at other widths: the staging units then cover 2 to 16 channels per
    row and the carry waves are one or two."""
    dk, dv = dims
    seed = 9550 + dk + dv
    say(f"[case] forward_prologue bf16 dk={dk} dv={dv}: B=2 H=2 T=190 seed={seed}")
    x = KI.make_prologue_inputs("pro_lm45m_bf16", B=2, H=2, T=190, dk=dk, dv=dv, seed=seed, dtype="bf16")
    got, ref = run(x, state=False)
    stats = check_forward(x, got, ref, "bf16", exact_coeffs=False)
    say(f"[ok] forward_prologue bf16 dk={dk} dv={dv}: " + ", ".join(f"{k}={v:.2e}" for k, v in stats.items()))


def test_forward_prologue_empty_sequence():
    """T = 0 copies the state in to the state out."""
    import torch
    import bius_scan_sequence_amd as K
    say("[case] forward_prologue T=0: B=2 H=2 d=16 f32")
    x = KI.make_prologue_inputs("pro_lm45m_bf16", B=2, H=2, T=0, dk=16, dv=16, seed=9580, dtype="f32")
    rng = np.random.default_rng(9580)
    lam0 = _f32(0.5 + rng.random((2, 2, 16)))
    M0 = _f32(rng.standard_normal((2, 2, 16, 16)))
    xd = {n: torch.from_numpy(np.ascontiguousarray(x[n])).cuda() for n in TOK}
    y, lT, MT = K.forward_prologue(xd["xq"], xd["xk"], xd["xv"], xd["dt_raw"], _f32(x["theta"]), _f32(x["sigma2"]),
                                   xd["vp_raw"], tuple(_f32(w) for w in x["conv_w"]),
                                   tuple(_f32(b) for b in x["conv_b"]), lam0, M0)
    torch.cuda.synchronize()
    assert y.numel() == 0
    assert torch.equal(lT, lam0) and torch.equal(MT, M0)
    say("[ok] forward_prologue T=0")


def test_forward_prologue_full_size_sampled_heads():
    """The benchmark's prologue workload (B8 H8 T2048 d64 bf16) generated on
    the device; two sampled heads against the oracle."""
    import torch
    import bius_scan_sequence_amd as K
    w = KI.workload("pro_lm45m_bf16")
    say(f"[case] forward_prologue full size {w.B}x{w.H}x{w.T} d={w.dk} bf16 seed={w.seed}")
    xd = KI.make_prologue_inputs_torch(w, device="cuda")
    y, lT, MT = K.forward_prologue(xd["xq"], xd["xk"], xd["xv"], xd["dt_raw"], xd["theta"], xd["sigma2"],
                                   xd["vp_raw"], xd["conv_w"], xd["conv_b"])
    torch.cuda.synchronize()
    for b, h in ((0, 5), (6, 2)):
        x = {n: xd[n][b:b + 1, h:h + 1].float().cpu().numpy() for n in TOK}
        x["theta"] = xd["theta"][h:h + 1].cpu().numpy()
        x["sigma2"] = xd["sigma2"][h:h + 1].cpu().numpy()
        x["conv_w"] = tuple(t[h:h + 1].cpu().numpy() for t in xd["conv_w"])
        x["conv_b"] = tuple(t[h:h + 1].cpu().numpy() for t in xd["conv_b"])
        x["dtype"] = "bf16"
        ref = kla_forward_prologue_f64(*(x[n] for n in ("xq", "xk", "xv", "dt_raw", "theta", "sigma2", "vp_raw")),
                                       x["conv_w"], x["conv_b"], dtype="bf16")
        got = (y[b:b + 1, h:h + 1].float().cpu().numpy(), lT[b:b + 1, h:h + 1].cpu().numpy(),
               MT[b:b + 1, h:h + 1].cpu().numpy())
        stats = check_forward(x, got, ref, "bf16", exact_coeffs=False)
        say(f"[ok] forward_prologue full size head ({b},{h}): " + ", ".join(f"{k}={v:.2e}" for k, v in stats.items()))
