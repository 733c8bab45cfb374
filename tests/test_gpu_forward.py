"""GPU parity of kla_forward against the float64 oracle (needs an MI355X).

Every case prints its name, seed and shape before touching the GPU.  Inputs are
the seeded workload recipes (kla_inputs); the oracle consumes exactly the
values handed to the GPU (bf16-rounded for bf16 workloads).  Tolerances are
those of tests/kla_testutil.py.
"""
import numpy as np
import pytest

import kla_inputs as KI
from kla_testutil import (check_bf16, check_f32, check_forward, gpu_forward, oracle_forward, say,
                          to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import bius_scan_sequence_amd as K
    assert torch.cuda.is_available()
    yield K
    torch.cuda.synchronize()


def run_case(name, x, with_path=True):
    say(f"[case] {name}: seed={x['seed']} shape q={x['q'].shape} v={x['v'].shape} dtype={x['dtype']}")
    xd = to_dev(x)
    got = gpu_forward(xd, return_lambda_path=with_path)
    ref = oracle_forward(x, return_lambda_path=with_path)
    stats = check_forward(x, got, ref, x["dtype"])
    say(f"[ok] {name}: " + ", ".join(f"{k}={v:.2e}" for k, v in stats.items()))
    return got, ref


# ----------------------------------------------------------------------------- workloads
def test_tiny_f32_full():
    run_case("tiny_f32", KI.make_forward_inputs("tiny_f32"))


def test_lm45m_bf16_full():
    run_case("lm45m_bf16", KI.make_forward_inputs("lm45m_bf16"))


def test_lm180m_bf16_full():
    run_case("lm180m_bf16", KI.make_forward_inputs("lm180m_bf16"), with_path=False)


def test_long_bf16_full_size_sampled_heads():
    """long_bf16 at its full shape (B=2, H=16, T=16384, d=128), generated on the
    device; the oracle checks four sampled heads over all 16384 tokens."""
    import torch
    import bius_scan_sequence_amd as K
    w = KI.workload("long_bf16")
    say(f"[case] long_bf16 full size: seed={w.seed} B={w.B} H={w.H} T={w.T} d={w.dk}")
    xd = KI.make_forward_inputs_torch(w)
    y, lT, MT = K.forward(xd["q"], xd["k"], xd["v"], xd["log_decay"], xd["proc_noise"], xd["val_prec"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed)
    for flat in rng.choice(w.B * w.H, size=4, replace=False):
        b, h = divmod(int(flat), w.H)
        x = {n: xd[n][b:b + 1, h:h + 1].float().cpu().numpy() for n in
             ("q", "k", "v", "log_decay", "proc_noise", "val_prec")}
        x["dtype"] = "bf16"
        ref = oracle_forward(x)
        got = (y[b:b + 1, h:h + 1].float().cpu().numpy(), lT[b:b + 1, h:h + 1].cpu().numpy(),
               MT[b:b + 1, h:h + 1].cpu().numpy())
        stats = check_forward(x, got, ref, "bf16")
        say(f"[ok] long_bf16 head ({b},{h}): " + ", ".join(f"{k}={v:.2e}" for k, v in stats.items()))
    del xd, y, lT, MT
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- shapes
SHAPES = [
    # (B, H, T, dk, dv, dtype)
    (1, 1, 1, 16, 16, "f32"),
    (1, 2, 17, 16, 32, "f32"),
    (2, 1, 65, 32, 64, "f32"),
    (1, 3, 200, 64, 32, "f32"),
    (1, 1, 130, 128, 128, "f32"),
    (1, 1, 96, 64, 128, "f32"),
    (1, 1, 1, 64, 64, "bf16"),
    (2, 2, 63, 16, 16, "bf16"),
    (1, 2, 64, 32, 128, "bf16"),
    (1, 1, 129, 128, 64, "bf16"),
    (2, 3, 300, 64, 64, "bf16"),
    (1, 1, 1000, 128, 128, "bf16"),
    (1, 2, 777, 16, 64, "bf16"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shapes_ragged(shape):
    B, H, T, dk, dv, dt = shape
    w = KI.workload("lm180m_bf16" if dt == "bf16" else "tiny_f32")
    x = KI.make_forward_inputs(w, B=B, H=H, T=T, dk=dk, dv=dv, seed=7000 + T + dk, dtype=dt)
    run_case(f"shape {shape}", x)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_nondefault_initial_state(dt):
    x = KI.make_forward_inputs("tiny_f32", B=2, H=2, T=150, dk=32, dv=16, seed=71, dtype=dt)
    rng = np.random.default_rng(5)
    x["lambda0"] = (0.2 + 3 * rng.random((2, 2, 32))).astype(np.float32)
    x["M0"] = rng.standard_normal((2, 2, 32, 16)).astype(np.float32)
    run_case(f"initial state {dt}", x)


def test_t_zero_copies_state():
    import torch
    import bius_scan_sequence_amd as K
    say("[case] T=0 state copy")
    x = KI.make_forward_inputs("lm45m_bf16", B=1, H=2, T=0, dk=64, dv=32)
    xd = to_dev(x)
    lam0 = torch.rand((1, 2, 64), device="cuda") + 0.5
    M0 = torch.randn((1, 2, 64, 32), device="cuda")
    y, lT, MT = K.forward(xd["q"], xd["k"], xd["v"], xd["log_decay"], xd["proc_noise"], xd["val_prec"],
                          lam0, M0)
    torch.cuda.synchronize()
    assert y.shape == (1, 2, 0, 32)
    assert torch.equal(lT, lam0) and torch.equal(MT, M0)
    y, lT, MT = K.forward(xd["q"], xd["k"], xd["v"], xd["log_decay"], xd["proc_noise"], xd["val_prec"])
    torch.cuda.synchronize()
    assert torch.all(lT == 1) and torch.all(MT == 0)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_state_carry_resumes(dt):
    """Two calls with the state passed on equal one call over all tokens."""
    import torch
    import bius_scan_sequence_amd as K
    say(f"[case] state carry {dt}")
    x = KI.make_forward_inputs("lm45m_bf16", B=2, H=2, T=700, dk=64, dv=64, seed=99, dtype=dt)
    xd = to_dev(x)
    names = ("q", "k", "v", "log_decay", "proc_noise", "val_prec")
    y, lT, MT = K.forward(*(xd[n] for n in names))
    T1 = 333
    y1, l1, M1 = K.forward(*(xd[n][:, :, :T1].contiguous() for n in names))
    y2, l2, M2 = K.forward(*(xd[n][:, :, T1:].contiguous() for n in names), l1, M1)
    torch.cuda.synchronize()
    ref = oracle_forward(x)
    got = (torch.cat([y1, y2], 2).float().cpu().numpy(), l2.cpu().numpy(), M2.cpu().numpy())
    check_forward(x, got, ref, dt)
    if dt == "f32":
        check_f32("carry vs single y", got[0], y.cpu().numpy(), per_head_floor=True)
    else:
        check_bf16("carry vs single y", got[0], y.float().cpu().numpy())
    say(f"[ok] state carry {dt}")


def test_deterministic_bitwise():
    """Repeated calls give identical bits (carries are folded in a fixed order
    whatever predecessor a look-back stops at)."""
    import torch
    import bius_scan_sequence_amd as K
    say("[case] determinism lm45m_bf16")
    x = KI.make_forward_inputs("lm45m_bf16")
    xd = to_dev(x)
    names = ("q", "k", "v", "log_decay", "proc_noise", "val_prec")
    first = K.forward(*(xd[n] for n in names))
    for _ in range(5):
        again = K.forward(*(xd[n] for n in names))
        torch.cuda.synchronize()
        for a, b in zip(first, again):
            assert torch.equal(a, b)
    ws = K._default_workspace(xd["q"].device, torch.cuda.current_stream().cuda_stream, "forward")
    assert ws.error() == 0
    say("[ok] determinism")


@pytest.mark.parametrize("case", ["lm180m_bf16", "deep_runs"])
def test_deterministic_bitwise_ten_repeats(case):
    """Ten repeated calls give the first call's bits, stopping at the first
    mismatch: lm180m_bf16 at full size (192 heads), and 8 heads x 8192 tokens
    (128 tiles per head, so the run kernel cuts each head into many runs and
    folds their carries through look-backs)."""
    import torch
    import bius_scan_sequence_amd as K
    if case == "lm180m_bf16":
        x = KI.make_forward_inputs("lm180m_bf16")
    else:
        x = KI.make_forward_inputs("lm45m_bf16", B=1, H=8, T=8192, seed=311)
    say(f"[case] determinism x10 {case}: q={x['q'].shape}")
    xd = to_dev(x)
    names = ("q", "k", "v", "log_decay", "proc_noise", "val_prec")
    ws = K.Workspace()
    first = K.forward(*(xd[n] for n in names), workspace=ws)
    torch.cuda.synchronize()
    for rep in range(10):
        again = K.forward(*(xd[n] for n in names), workspace=ws)
        torch.cuda.synchronize()
        for name, a, b in zip(("y", "lambda_T", "M_T"), first, again):
            assert torch.equal(a, b), f"repeat {rep}: {name} differs"
    assert ws.error() == 0
    say(f"[ok] determinism x10 {case}")


def test_many_heads_skipped_aggregates_deterministic():
    """With 128 or more heads a segment whose predecessor's inclusive mean is
    already out publishes no aggregate.  Results stay bitwise repeatable and
    match the oracle (two sampled heads)."""
    import torch
    import bius_scan_sequence_amd as K
    say("[case] many heads: B=2 H=80 T=700 d=64 bf16 seed=77")
    x = KI.make_forward_inputs("lm45m_bf16", B=2, H=80, T=700, seed=77)
    xd = to_dev(x)
    names = ("q", "k", "v", "log_decay", "proc_noise", "val_prec")
    first = K.forward(*(xd[n] for n in names))
    for _ in range(4):
        again = K.forward(*(xd[n] for n in names))
        torch.cuda.synchronize()
        for a, b in zip(first, again):
            assert torch.equal(a, b)
    for b, h in ((0, 3), (1, 77)):
        xs = {n: x[n][b:b + 1, h:h + 1] for n in names}
        xs["dtype"] = "bf16"
        ref = oracle_forward(xs)
        got = tuple(t[b:b + 1, h:h + 1].float().cpu().numpy() for t in first)
        check_forward(xs, got, ref, "bf16")
    say("[ok] many heads")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_extreme_decay_exact_path(dt):
    """Chunks whose decay over a half chunk underflows 2^-64 on some channel
    take the exact scalar path for their intra-chunk scores."""
    x = KI.make_forward_inputs("tiny_f32", B=1, H=2, T=160, dk=32, dv=16, seed=123, dtype=dt)
    ld = x["log_decay"].copy()
    ld[0, 0, 20:40, 3] = -9.0      # e^-9 per token: far below 2^-64 within a chunk
    ld[0, 1, 100:112, :] = -12.0
    ld[0, 1, 70, 5] = -60.0        # one token wipes a channel's memory
    x["log_decay"] = KI.round_bf16(ld) if dt == "bf16" else ld.astype(np.float32)
    run_case(f"extreme decay {dt}", x)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_strong_decay_middle_reference(dt):
    """Chunks whose decay over the whole chunk falls below 2^-64 while each
    half stays above it: their scores still come from the matrix cores, with
    the operands referred to the middle of the chunk.  Also a chunk whose
    first half alone falls below 2^-64 next to one whose second half does
    (both take the exact path)."""
    x = KI.make_forward_inputs("tiny_f32", B=1, H=2, T=200, dk=32, dv=16, seed=124, dtype=dt)
    ld = x["log_decay"].copy()
    ld[0, 0, 16:80, :] = -3.5      # about 2^-5 per token: 2^-81 per chunk, 2^-40 per half
    ld[0, 1, 32:48, 0:8] = -3.9
    ld[0, 1, 96:104, 9] = -7.0     # first half of a chunk only: 2^-81
    ld[0, 1, 120:128, 9] = -7.0    # second half of the next chunk only
    x["log_decay"] = KI.round_bf16(ld) if dt == "bf16" else ld.astype(np.float32)
    run_case(f"strong decay {dt}", x)


# ----------------------------------------------------------------------------- run-streaming kernel paths
# bf16 at d = 64 runs the run-streaming kernel.  At B8 H8 T2048 a head is cut
# into 4 runs of 8 tiles.  The lm45m recipe forgets fast (every tile after a
# run's two held tiles is free, and one window tile always converges), so the
# paths below need recipes of their own; every head is checked.
def _scaled(ld_s, pn_s, vp_s, seed):
    x = KI.make_forward_inputs("lm45m_bf16", seed=seed)
    x["log_decay"] = KI.round_bf16(ld_s * x["log_decay"].astype(np.float32))
    x["proc_noise"] = KI.round_bf16(pn_s * x["proc_noise"].astype(np.float32))
    x["val_prec"] = KI.round_bf16(vp_s * x["val_prec"].astype(np.float32))
    return x


@pytest.mark.parametrize("case", ["long_memory", "window_4_tiles", "window_to_start"])
def test_run_kernel_slow_forgetting(case):
    """Decays near 1: the entering mean still matters after the held tiles, so
    every later run resolves it mid-run (look-back, held tiles corrected,
    state folded) instead of dropping it.  The precision maps contract slowly:
    the window walk composes about 4 tiles (window_4_tiles), or 12 tiles and
    for the second run the whole prefix down to lambda0 (window_to_start)."""
    if case == "long_memory":
        x = KI.make_forward_inputs("long_bf16", B=8, H=8, T=2048, dk=64, dv=64, seed=8100)
    elif case == "window_4_tiles":
        x = _scaled(0.05, 0.05, 0.2, 8101)
    else:
        x = _scaled(0.02, 0.01, 0.01, 8102)
    run_case(f"run kernel {case}", x)


def test_run_kernel_several_rounds():
    """More runs than compute units: B24 H16 T1024 plans two 8-tile runs per
    head, 768 workgroups in three rounds, so tickets are drawn across rounds
    and a later run's look-back may meet predecessors that finished long ago
    (their inclusive means out, some aggregates never published).  Bitwise
    repeatable over three calls, and six heads against the oracle: from the
    first and the last tickets of each run index."""
    import torch
    import bius_scan_sequence_amd as K
    say("[case] run kernel several rounds: B=24 H=16 T=1024 d=64 bf16 seed=8104")
    x = KI.make_forward_inputs("lm45m_bf16", B=24, H=16, T=1024, seed=8104)
    xd = to_dev(x)
    names = ("q", "k", "v", "log_decay", "proc_noise", "val_prec")
    first = K.forward(*(xd[n] for n in names), return_lambda_path=True)
    for _ in range(2):
        again = K.forward(*(xd[n] for n in names), return_lambda_path=True)
        torch.cuda.synchronize()
        for a, b in zip(first, again):
            assert torch.equal(a, b)
    for b, h in ((0, 0), (0, 1), (11, 7), (12, 8), (23, 14), (23, 15)):
        xs = {n: x[n][b:b + 1, h:h + 1] for n in names}
        xs["dtype"] = "bf16"
        ref = oracle_forward(xs, return_lambda_path=True)
        got = tuple(t[b:b + 1, h:h + 1].float().cpu().numpy() for t in first)
        check_forward(xs, got, ref, "bf16")
    say("[ok] run kernel several rounds")


def test_run_kernel_extreme_decays():
    """Chunks whose decay underflows 2^-120 on some channel take the run
    kernel's exact per-token path: in a free tile, across the boundary of two
    runs, and inside a held tile of a later run (which then resolves the
    entering mean mid-run at that chunk)."""
    x = KI.make_forward_inputs("lm45m_bf16", seed=8103)
    ld = x["log_decay"].astype(np.float32).copy()
    ld[0, 0, 600:620, 3] = -9.0       # e^-9 per token: a chunk far below 2^-120 on one channel
    ld[0, 1, 1000, 5] = -60.0         # one token wipes a channel's memory
    ld[1, 2, 1500:1512, :] = -12.0    # every channel
    ld[2, 3, 504:520, 7] = -12.0      # across the boundary of runs 0 and 1 (token 512)
    ld[3, 4, 530:546, 0:4] = -9.0     # inside the first held tile of run 1
    ld[5, 6, 1540:1556, 60] = -12.0   # inside the first held tile of run 3
    x["log_decay"] = KI.round_bf16(ld)
    run_case("run kernel extreme decays", x)


def test_precision_only_inputs_shared_over_value_channels():
    """The precision path of kla_forward does not depend on q, v or M0."""
    import torch
    import bius_scan_sequence_amd as K
    say("[case] precision independent of q/v")
    x = KI.make_forward_inputs("lm45m_bf16", B=1, H=2, T=300)
    xd = to_dev(x)
    _, l1, _, p1 = K.forward(xd["q"], xd["k"], xd["v"], xd["log_decay"], xd["proc_noise"], xd["val_prec"],
                             return_lambda_path=True)
    _, l2, _, p2 = K.forward(-xd["q"], xd["k"], 2 * xd["v"], xd["log_decay"], xd["proc_noise"],
                             xd["val_prec"], None, torch.ones((1, 2, 64, 64), device="cuda"),
                             return_lambda_path=True)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2) and torch.equal(l1, l2)
    say("[ok] precision independent of q/v")
