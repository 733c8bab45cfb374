"""GPU parity of kla_forward_vprec (value precision per value channel: a
d_k x d_v precision field) against the float64 oracle oracle/kla_vprec_f64.py,
needs an MI355X.

The bars are the forward pass's (tests/kla_testutil.py): fp32 inputs 1e-5
relative (lambda elementwise; y and M_T against the per-head RMS), bf16 inputs
1e-2 + 2e-2 |r| for y and M_T with lambda_T held to the fp32 bar.
Every case prints its name, seed and shape before touching the GPU.
"""
import numpy as np
import pytest

import kla_inputs as KI
from kla_testutil import check_bf16, check_f32, say
from oracle import kla_forward_vprec_f64

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "log_decay", "proc_noise", "val_prec")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import bius_scan_sequence_amd as K
    assert torch.cuda.is_available()
    yield K
    torch.cuda.synchronize()


def run_case(x, state=True):
    import torch
    import bius_scan_sequence_amd as K
    tdt = torch.bfloat16 if x["dtype"] == "bf16" else torch.float32
    xd = {n: torch.from_numpy(np.ascontiguousarray(x[n])).cuda().to(tdt) for n in NAMES}
    lam0 = torch.from_numpy(x["lambda0"]).cuda() if state else None
    M0 = torch.from_numpy(x["M0"]).cuda() if state else None
    y, lT, MT = K.forward_vprec(*(xd[n] for n in NAMES), lam0, M0)
    torch.cuda.synchronize()
    ry, rl, rM = kla_forward_vprec_f64(*(x[n] for n in NAMES), x["lambda0"] if state else None,
                                       x["M0"] if state else None)
    y, lT, MT = y.float().cpu().numpy(), lT.cpu().numpy(), MT.cpu().numpy()
    st = {"lambda_T": check_f32("lambda_T", lT, rl, per_head_floor=False)}
    if x["dtype"] == "f32":
        st["y"] = check_f32("y", y, ry, per_head_floor=True)
        st["M_T"] = check_f32("M_T", MT, rM, per_head_floor=True)
    else:
        st["y"] = check_bf16("y", y, ry)
        st["M_T"] = check_bf16("M_T", MT, rM)
    return st


SHAPES = [
    # (B, H, T, dk, dv, dtype, state)
    (1, 1, 1, 16, 16, "f32", True),
    (1, 2, 77, 16, 32, "f32", True),
    (2, 1, 200, 64, 16, "f32", False),
    (1, 2, 130, 32, 64, "f32", True),
    (1, 1, 100, 128, 128, "f32", True),
    (2, 2, 300, 64, 64, "bf16", True),
    (1, 2, 257, 128, 64, "bf16", False),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_vprec_matches_oracle(shape):
    B, H, T, dk, dv, dt, state = shape
    seed = 9950 + T + dk + dv
    say(f"[case] forward_vprec {shape}: seed={seed}")
    x = KI.make_vprec_inputs("vprec_lm45m_bf16", B=B, H=H, T=T, dk=dk, dv=dv, seed=seed, dtype=dt)
    if state:
        rng = np.random.default_rng(seed)
        x["lambda0"] = (0.5 + rng.random((B, H, dk, dv))).astype(np.float32)
        x["M0"] = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    st = run_case(x, state)
    say(f"[ok] forward_vprec {shape}: " + ", ".join(f"{k}={v:.2e}" for k, v in st.items()))


def test_vprec_shared_precision_equals_forward():
    """With one value precision per token (the same for every channel) the
    variant and kla_forward compute the same filter: their outputs agree
    within the fp32 bar, and lambda_T of the variant repeats kla_forward's
    over the value channels."""
    import torch
    import bius_scan_sequence_amd as K
    B, H, T, dk, dv = 1, 2, 150, 32, 32
    say(f"[case] forward_vprec vs forward, shared precision: B={B} H={H} T={T} d={dk} f32")
    x = KI.make_forward_inputs("tiny_f32", B=B, H=H, T=T, dk=dk, dv=dv, seed=9970)
    s = x["val_prec"][..., :1]
    xd = {n: torch.from_numpy(x[n]).cuda() for n in NAMES}
    xd_f = dict(xd, val_prec=torch.from_numpy(np.ascontiguousarray(np.broadcast_to(s, (B, H, T, dk)))).cuda())
    xd_v = dict(xd, val_prec=torch.from_numpy(np.ascontiguousarray(np.broadcast_to(s, (B, H, T, dv)))).cuda())
    y1, l1, M1 = K.forward(*(xd_f[n] for n in NAMES))
    y2, l2, M2 = K.forward_vprec(*(xd_v[n] for n in NAMES))
    torch.cuda.synchronize()
    y1, y2 = y1.cpu().numpy(), y2.cpu().numpy()
    scale = np.maximum(np.abs(y1), np.sqrt(np.mean(y1 ** 2)))
    assert np.max(np.abs(y2 - y1) / scale) <= 2e-5
    l1, l2 = l1.cpu().numpy(), l2.cpu().numpy()
    assert np.max(np.abs(l2 - l1[..., None]) / l1[..., None]) <= 2e-5
    say("[ok] forward_vprec vs forward")


def test_vprec_full_size_sampled_heads():
    """The benchmark's variant workload (B8 H8 T2048 d64 bf16) on the device;
    two sampled heads against the oracle."""
    import torch
    import bius_scan_sequence_amd as K
    w = KI.workload("vprec_lm45m_bf16")
    say(f"[case] forward_vprec full size {w.B}x{w.H}x{w.T} d={w.dk} bf16 seed={w.seed}")
    xd = KI.make_vprec_inputs_torch(w, device="cuda")
    y, lT, MT = K.forward_vprec(*(xd[n] for n in NAMES))
    torch.cuda.synchronize()
    for b, h in ((1, 4), (7, 0)):
        x = {n: xd[n][b:b + 1, h:h + 1].float().cpu().numpy() for n in NAMES}
        ry, rl, rM = kla_forward_vprec_f64(*(x[n] for n in NAMES))
        check_bf16("y", y[b:b + 1, h:h + 1].float().cpu().numpy(), ry)
        check_f32("lambda_T", lT[b:b + 1, h:h + 1].cpu().numpy(), rl, per_head_floor=False)
        check_bf16("M_T", MT[b:b + 1, h:h + 1].cpu().numpy(), rM)
        say(f"[ok] forward_vprec full size head ({b},{h})")
