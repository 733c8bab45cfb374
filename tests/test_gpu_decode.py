"""GPU parity of kla_decode_step (one token per head) against the float64 oracle.

Every case prints its name, seed and shape before touching the GPU.  Inputs
follow the workload recipes of kla_inputs at T = 1 (or T tokens fed one at a
time); the carried state is drawn here: lambda ~ 0.5 + U(0, 3), M ~ N(0, 1).
The precision and the state are held to the fp32 bar for both input dtypes
(the step runs in fp32 on exactly the values the oracle sees); y uses the
dtype's bar (tests/kla_testutil.py).
"""
import numpy as np
import pytest

import kla_inputs as KI
from kla_testutil import check_bf16, check_f32, oracle_forward, say, to_dev
from oracle import kla_decode_step_f64

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "log_decay", "proc_noise", "val_prec")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import bius_scan_sequence_amd as K
    assert torch.cuda.is_available()
    yield K
    torch.cuda.synchronize()


def step_inputs(B, H, dk, dv, dt, seed):
    w = KI.workload("lm180m_bf16" if dt == "bf16" else "tiny_f32")
    x = KI.make_forward_inputs(w, B=B, H=H, T=1, dk=dk, dv=dv, seed=seed, dtype=dt)
    x = {n: (x[n][:, :, 0] if n in NAMES else x[n]) for n in x}
    rng = np.random.default_rng(seed)
    x["lam"] = (0.5 + 3.0 * rng.random((B, H, dk))).astype(np.float32)
    x["M"] = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    return x


def gpu_step(xd, lam, M, inplace=False):
    import torch
    import bius_scan_sequence_amd as K
    y, l, m = K.decode_step(*(xd[n] for n in NAMES), lam, M, inplace=inplace)
    torch.cuda.synchronize()
    return y, l, m


def check_step(name, x, got, ref):
    y, lam, M = (t.float().cpu().numpy() for t in got)
    ry, rl, rM = ref
    s = {"lambda": check_f32("lambda", lam, rl, per_head_floor=False),
         "M": check_f32("M", M, rM, per_head_floor=True)}
    if x["dtype"] == "f32":
        s["y"] = check_f32("y", y, ry, per_head_floor=True)
    else:
        s["y"] = check_bf16("y", y, ry)
    say(f"[ok] {name}: " + ", ".join(f"{k}={v:.2e}" for k, v in s.items()))


SHAPES = [
    # (B, H, dk, dv, dtype)
    (1, 1, 16, 16, "f32"),
    (2, 3, 16, 128, "f32"),
    (1, 4, 32, 64, "f32"),
    (2, 1, 128, 16, "f32"),
    (1, 2, 128, 128, "f32"),
    (2, 2, 64, 64, "bf16"),
    (3, 5, 64, 32, "bf16"),
    (1, 3, 128, 128, "bf16"),
    (2, 2, 32, 16, "bf16"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_step_matches_oracle(shape):
    import torch
    B, H, dk, dv, dt = shape
    seed = 8100 + dk + 3 * dv
    say(f"[case] decode step {shape}: seed={seed}")
    x = step_inputs(B, H, dk, dv, dt, seed)
    xd = to_dev(x)
    lam = torch.from_numpy(x["lam"]).cuda()
    M = torch.from_numpy(x["M"]).cuda()
    got = gpu_step(xd, lam, M)
    ref = kla_decode_step_f64(*(x[n] for n in NAMES), x["lam"], x["M"])
    check_step(f"decode step {shape}", x, got, ref)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_in_place_equals_out_of_place(dt):
    import torch
    say(f"[case] decode in place {dt}")
    x = step_inputs(2, 3, 64, 64, dt, 8200)
    xd = to_dev(x)
    lam = torch.from_numpy(x["lam"]).cuda()
    M = torch.from_numpy(x["M"]).cuda()
    y1, l1, m1 = gpu_step(xd, lam, M, inplace=False)
    lam2, M2 = lam.clone(), M.clone()
    y2, l2, m2 = gpu_step(xd, lam2, M2, inplace=True)
    assert l2.data_ptr() == lam2.data_ptr() and m2.data_ptr() == M2.data_ptr()
    assert torch.equal(y1, y2) and torch.equal(l1, lam2) and torch.equal(m1, M2)
    say(f"[ok] decode in place {dt}")


def test_prior_when_no_state():
    import torch
    say("[case] decode from the prior")
    x = step_inputs(1, 2, 32, 32, "bf16", 8300)
    xd = to_dev(x)
    y1, l1, m1 = gpu_step(xd, None, None)
    y2, l2, m2 = gpu_step(xd, torch.ones((1, 2, 32), device="cuda"), torch.zeros((1, 2, 32, 32), device="cuda"))
    assert torch.equal(y1, y2) and torch.equal(l1, l2) and torch.equal(m1, m2)
    say("[ok] decode from the prior")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_token_by_token_equals_forward(dt):
    """T decode steps from (lambda0, M0) reproduce the forward pass over the
    same tokens (oracle), and agree with the GPU forward pass."""
    import torch
    import bius_scan_sequence_amd as K
    B, H, T, dk, dv = 2, 2, 48, 64, 32
    say(f"[case] decode chain {dt}: B={B} H={H} T={T} dk={dk} dv={dv}")
    w = KI.workload("lm180m_bf16" if dt == "bf16" else "tiny_f32")
    x = KI.make_forward_inputs(w, B=B, H=H, T=T, dk=dk, dv=dv, seed=8400, dtype=dt)
    rng = np.random.default_rng(8400)
    x["lambda0"] = (0.5 + rng.random((B, H, dk))).astype(np.float32)
    x["M0"] = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    xd = to_dev(x)
    lam, M = xd["lambda0"].clone(), xd["M0"].clone()
    ys = []
    for t in range(T):
        y, lam, M = K.decode_step(*(xd[n][:, :, t].contiguous() for n in NAMES), lam, M)
        ys.append(y)
    torch.cuda.synchronize()
    yg = torch.stack(ys, 2).float().cpu().numpy()
    ry, rl, rM = oracle_forward(x)
    check_f32("lambda_T", lam.cpu().numpy(), rl, per_head_floor=False)
    check_f32("M_T", M.cpu().numpy(), rM, per_head_floor=True)
    if dt == "f32":
        check_f32("y", yg, ry, per_head_floor=True)
    else:
        check_bf16("y", yg, ry)
    # Against the GPU forward pass: each side meets its bar against the oracle,
    # so they agree within the sum of the two bars (the forward's bf16 path
    # contracts split-bf16 operands, about 16 mantissa bits).
    fy, fl, fM = K.forward(*(xd[n] for n in NAMES), xd["lambda0"], xd["M0"])
    torch.cuda.synchronize()
    got, fwd = (lam.cpu().numpy(), M.cpu().numpy()), (fl.cpu().numpy(), fM.cpu().numpy())
    if dt == "f32":
        for name, g, f, floor in (("lambda_T", got[0], fwd[0], False), ("M_T", got[1], fwd[1], True)):
            scale = np.maximum(np.abs(f), np.sqrt(np.mean(f * f, axis=tuple(range(2, f.ndim)), keepdims=True))) \
                if floor else np.abs(f)
            assert np.max(np.abs(g - f) / scale) <= 2e-5, f"decode vs forward {name}"
    else:
        check_bf16("decode vs forward lambda_T", got[0], fwd[0])
        check_bf16("decode vs forward M_T", got[1], fwd[1])
    say(f"[ok] decode chain {dt}")


def test_continues_a_forward_pass():
    """Decode picks up the state a forward pass leaves (prefill, then generate)."""
    import torch
    import bius_scan_sequence_amd as K
    B, H, T1, T2, d = 1, 3, 130, 6, 64
    say(f"[case] prefill {T1} then decode {T2}")
    x = KI.make_forward_inputs("lm45m_bf16", B=B, H=H, T=T1 + T2, dk=d, dv=d, seed=8500)
    xd = to_dev(x)
    _, lam, M = K.forward(*(xd[n][:, :, :T1].contiguous() for n in NAMES))
    ys = []
    for t in range(T1, T1 + T2):
        y, lam, M = K.decode_step(*(xd[n][:, :, t].contiguous() for n in NAMES), lam, M)
        ys.append(y)
    torch.cuda.synchronize()
    ry, rl, rM = oracle_forward(x)
    # The carried mean went through the forward pass's bf16 path: its bar.
    check_bf16("y", torch.stack(ys, 2).float().cpu().numpy(), ry[:, :, T1:])
    check_f32("lambda_T", lam.cpu().numpy(), rl, per_head_floor=False)
    check_bf16("M_T", M.cpu().numpy(), rM)
    say("[ok] prefill then decode")


def test_decode_batch256_full_size():
    """The benchmark's batch-256 decode shape (B=256, H=8, d=64, bf16), every head."""
    import torch
    B, H, d = 256, 8, 64
    say(f"[case] decode batch: B={B} H={H} d={d} bf16 seed=8600")
    x = step_inputs(B, H, d, d, "bf16", 8600)
    xd = to_dev(x)
    lam = torch.from_numpy(x["lam"]).cuda()
    M = torch.from_numpy(x["M"]).cuda()
    got = gpu_step(xd, lam, M, inplace=True)
    ref = kla_decode_step_f64(*(x[n] for n in NAMES), x["lam"], x["M"])
    check_step("decode batch256", x, got, ref)


def test_decode_steps_replayed_from_a_graph():
    """A generation loop of decode steps captured once in a HIP graph (state
    updated in place, per-token outputs into fixed buffers) and replayed three
    times, with eager work between the replays, gives each time exactly the
    eager loop's outputs and final state."""
    import torch
    import bius_scan_sequence_amd as K
    B, H, T, dk, dv = 4, 8, 12, 64, 64
    say(f"[case] decode graph replay: B={B} H={H} T={T} d={dk} bf16")
    w = KI.workload("lm180m_bf16")
    x = KI.make_forward_inputs(w, B=B, H=H, T=T, dk=dk, dv=dv, seed=8500, dtype="bf16")
    rng = np.random.default_rng(8500)
    x["lambda0"] = (0.5 + rng.random((B, H, dk))).astype(np.float32)
    x["M0"] = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    xd = to_dev(x)
    toks = [{n: xd[n][:, :, t].contiguous() for n in NAMES} for t in range(T)]
    # Eager reference.
    lam, M = xd["lambda0"].clone(), xd["M0"].clone()
    ref_y = []
    for t in range(T):
        y, lam, M = K.decode_step(*(toks[t][n] for n in NAMES), lam, M)
        ref_y.append(y.clone())
    torch.cuda.synchronize()
    ref_lam, ref_M = lam.clone(), M.clone()
    # Captured loop over fixed buffers.
    glam, gM = xd["lambda0"].clone(), xd["M0"].clone()
    ys = [torch.empty((B, H, dv), dtype=torch.bfloat16, device="cuda") for _ in range(T)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream, as graph capture wants
        K.decode_step(*(toks[0][n] for n in NAMES), glam, gM, out=(ys[0], glam, gM))
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(T):
            K.decode_step(*(toks[t][n] for n in NAMES), glam, gM, out=(ys[t], glam, gM))
    for rep in range(3):
        glam.copy_(xd["lambda0"])
        gM.copy_(xd["M0"])
        for y in ys:
            y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t in range(T):
            assert torch.equal(ys[t], ref_y[t]), f"replay {rep}, token {t}"
        assert torch.equal(glam, ref_lam) and torch.equal(gM, ref_M), f"replay {rep}, state"
        _ = (xd["q"].float() * 2).sum().item()  # eager work between replays
    say("[ok] decode graph replay")
