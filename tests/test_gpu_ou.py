"""GPU parity of kla_forward_ou (the forward pass with the OU prior given in
continuous time, discretised inside the kernel) against the float64 oracle
oracle/kla_ou_f64.py, needs an MI355X.

The oracle discretises exactly in float64 (log a = -theta dt,
pbar = sigma2 (1 - e^{-2 theta dt}) / (2 theta)) and runs the sequential
filter; the kernel forms the same two numbers in fp32 per token.  The bars are
those of the forward pass (tests/kla_testutil.py): fp32 inputs 1e-5 relative
(y and M_T against the per-head RMS), bf16 inputs 1e-2 + 2e-2 |r|.
Every case prints its name, seed and shape before touching the GPU.
"""
import numpy as np
import pytest

import kla_inputs as KI
from kla_testutil import check_forward, say
from oracle import kla_forward_ou_f64

pytestmark = pytest.mark.gpu

TOK = ("q", "k", "v", "dt", "val_prec")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import bius_scan_sequence_amd as K
    assert torch.cuda.is_available()
    yield K
    torch.cuda.synchronize()


def to_dev_ou(x):
    import torch
    dt = torch.bfloat16 if x["dtype"] == "bf16" else torch.float32
    out = {n: torch.from_numpy(np.ascontiguousarray(x[n])).cuda().to(dt) for n in TOK}
    for n in ("theta", "sigma2", "lambda0", "M0"):
        out[n] = torch.from_numpy(np.ascontiguousarray(x[n], np.float32)).cuda()
    return out


def run(x, state=True):
    import torch
    import bius_scan_sequence_amd as K
    xd = to_dev_ou(x)
    res = K.forward_ou(xd["q"], xd["k"], xd["v"], xd["dt"], xd["theta"], xd["sigma2"], xd["val_prec"],
                       xd["lambda0"] if state else None, xd["M0"] if state else None, return_lambda_path=True)
    torch.cuda.synchronize()
    got = tuple(t.float().cpu().numpy() for t in res)
    ref = kla_forward_ou_f64(*(x[n] for n in ("q", "k", "v", "dt", "theta", "sigma2", "val_prec")),
                             x["lambda0"] if state else None, x["M0"] if state else None, return_lambda_path=True)
    return got, ref


SHAPES = [
    # (B, H, T, dk, dv, dtype)
    (1, 1, 256, 16, 16, "f32"),
    (2, 3, 300, 32, 64, "f32"),
    (1, 2, 200, 128, 32, "f32"),
    (2, 2, 130, 64, 64, "bf16"),
    (1, 4, 1000, 64, 64, "bf16"),
    (1, 2, 300, 128, 128, "bf16"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_forward_ou_matches_oracle(shape):
    B, H, T, dk, dv, dt = shape
    seed = 9800 + T + dk + dv
    say(f"[case] forward_ou {shape}: seed={seed}")
    x = KI.make_ou_inputs("ou_lm45m_bf16", B=B, H=H, T=T, dk=dk, dv=dv, seed=seed, dtype=dt)
    rng = np.random.default_rng(seed)
    x["lambda0"] = (0.5 + rng.random((B, H, dk))).astype(np.float32)
    x["M0"] = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    got, ref = run(x)
    stats = check_forward(x, got, ref, dt)
    say(f"[ok] forward_ou {shape}: " + ", ".join(f"{k}={v:.2e}" for k, v in stats.items()))


@pytest.mark.parametrize("case", ["brownian", "stationary", "zero_step"])
def test_forward_ou_limits(case):
    """theta = 0 (Brownian steps, the kernel's series branch), long steps
    (the stationary variance, a -> 0), and dt = 0 (no time passes: a = 1 and
    no process noise, so the precision only accumulates evidence)."""
    say(f"[case] forward_ou limit {case}: B=1 H=2 T=200 d=32 f32 seed=9900")
    x = KI.make_ou_inputs("ou_lm45m_bf16", B=1, H=2, T=200, dk=32, dv=32, seed=9900, dtype="f32")
    if case == "brownian":
        x["theta"] = np.zeros_like(x["theta"])
        x["theta"][0, :4] = 1e-6  # also tiny rates, below the series threshold
    elif case == "stationary":
        x["dt"] = (x["dt"] * 40.0).astype(np.float32)
    else:
        x["dt"] = np.zeros_like(x["dt"])
    got, ref = run(x, state=False)
    stats = check_forward(x, got, ref, "f32")
    say(f"[ok] forward_ou limit {case}: " + ", ".join(f"{k}={v:.2e}" for k, v in stats.items()))


def test_forward_ou_full_size_sampled_heads():
    """The benchmark's OU workload (B8 H8 T2048 d64 bf16) generated on the
    device; two sampled heads against the oracle."""
    import torch
    import bius_scan_sequence_amd as K
    w = KI.workload("ou_lm45m_bf16")
    say(f"[case] forward_ou full size {w.B}x{w.H}x{w.T} d={w.dk} bf16 seed={w.seed}")
    xd = KI.make_ou_inputs_torch(w, device="cuda")
    y, lT, MT = K.forward_ou(xd["q"], xd["k"], xd["v"], xd["dt"], xd["theta"], xd["sigma2"], xd["val_prec"])
    torch.cuda.synchronize()
    for b, h in ((0, 5), (6, 2)):
        x = {n: xd[n][b:b + 1, h:h + 1].float().cpu().numpy() for n in TOK}
        x["theta"] = xd["theta"][h:h + 1].cpu().numpy()
        x["sigma2"] = xd["sigma2"][h:h + 1].cpu().numpy()
        x["dtype"] = "bf16"
        ref = kla_forward_ou_f64(*(x[n] for n in ("q", "k", "v", "dt", "theta", "sigma2", "val_prec")))
        got = (y[b:b + 1, h:h + 1].float().cpu().numpy(), lT[b:b + 1, h:h + 1].cpu().numpy(),
               MT[b:b + 1, h:h + 1].cpu().numpy())
        stats = check_forward(x, got, ref, "bf16")
        say(f"[ok] forward_ou full size head ({b},{h}): " + ", ".join(f"{k}={v:.2e}" for k, v in stats.items()))
