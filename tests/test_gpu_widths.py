"""Every supported width pair, both dtypes, every entry point (needs an MI355X).

The kernels are compile-time instances per (d_k, d_v, dtype): 16 width pairs
x 2 dtypes for each of the forward modes (plain, OU prior, raw projections),
the per-channel value precision, the decode step and the backward.  The other
GPU tests cover a subset of these instances at several lengths; this sweep
runs each instance against the float64 oracle once, at a length that spans two
64-token segments and ends in a ragged chunk (T = 83), with a nondefault state
in (the decode step: three steps).  Tolerances and comparisons are the entry
points' own tests'.
"""
import numpy as np
import pytest

import kla_inputs as KI
from kla_testutil import check_forward, gpu_forward, oracle_forward, say, to_dev

import test_gpu_backward as TB
import test_gpu_ou as TO
import test_gpu_prologue as TP
import test_gpu_vprec as TV

pytestmark = pytest.mark.gpu

WIDTHS = (16, 32, 64, 128)
CASES = [(dk, dv, dt) for dt in ("f32", "bf16") for dk in WIDTHS for dv in WIDTHS]
IDS = [f"{dt}-{dk}x{dv}" for dk, dv, dt in CASES]
B, H, T = 1, 2, 83


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import bius_scan_sequence_amd as K
    assert torch.cuda.is_available()
    yield K
    torch.cuda.synchronize()


def _state(x, dk, dv, seed, per_value=False):
    rng = np.random.default_rng(seed)
    x["lambda0"] = (0.5 + rng.random((B, H, dk, dv) if per_value else (B, H, dk))).astype(np.float32)
    x["M0"] = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    return x


def _seed(base, dk, dv, dt):
    return base + 8 * WIDTHS.index(dk) + 2 * WIDTHS.index(dv) + (dt == "bf16")


@pytest.mark.parametrize("dk,dv,dt", CASES, ids=IDS)
def test_forward_every_width(dk, dv, dt):
    seed = _seed(12000, dk, dv, dt)
    say(f"[case] forward widths dk={dk} dv={dv} {dt}: B={B} H={H} T={T} seed={seed}")
    x = _state(KI.make_forward_inputs("lm180m_bf16" if dt == "bf16" else "tiny_f32", B=B, H=H, T=T, dk=dk,
                                      dv=dv, seed=seed, dtype=dt), dk, dv, seed)
    got = gpu_forward(to_dev(x), return_lambda_path=True)
    ref = oracle_forward(x, return_lambda_path=True)
    stats = check_forward(x, got, ref, dt)
    say(f"[ok] forward widths dk={dk} dv={dv} {dt}: " + ", ".join(f"{k}={v:.2e}" for k, v in stats.items()))


@pytest.mark.parametrize("dk,dv,dt", CASES, ids=IDS)
def test_forward_ou_every_width(dk, dv, dt):
    seed = _seed(12100, dk, dv, dt)
    say(f"[case] forward_ou widths dk={dk} dv={dv} {dt}: B={B} H={H} T={T} seed={seed}")
    x = _state(KI.make_ou_inputs("ou_lm45m_bf16", B=B, H=H, T=T, dk=dk, dv=dv, seed=seed, dtype=dt), dk, dv, seed)
    got, ref = TO.run(x)
    stats = check_forward(x, got, ref, dt)
    say(f"[ok] forward_ou widths dk={dk} dv={dv} {dt}: " + ", ".join(f"{k}={v:.2e}" for k, v in stats.items()))


@pytest.mark.parametrize("dk,dv,dt", CASES, ids=IDS)
def test_forward_prologue_every_width(dk, dv, dt):
    seed = _seed(12200, dk, dv, dt)
    say(f"[case] forward_prologue widths dk={dk} dv={dv} {dt}: B={B} H={H} T={T} seed={seed}")
    x = _state(KI.make_prologue_inputs("pro_lm45m_bf16", B=B, H=H, T=T, dk=dk, dv=dv, seed=seed, dtype=dt),
               dk, dv, seed)
    got, ref = TP.run(x)
    # bf16: q, k, v are rounded to bf16 on both sides, from fp32 and fp64
    # sums, so a value within an ulp of a rounding midpoint can round either
    # way; the precision outputs take the bf16 bar then.
    stats = check_forward(x, got, ref, dt, exact_coeffs=dt == "f32")
    say(f"[ok] forward_prologue widths dk={dk} dv={dv} {dt}: " + ", ".join(f"{k}={v:.2e}" for k, v in stats.items()))


@pytest.mark.parametrize("dk,dv,dt", CASES, ids=IDS)
def test_forward_vprec_every_width(dk, dv, dt):
    seed = _seed(12300, dk, dv, dt)
    say(f"[case] forward_vprec widths dk={dk} dv={dv} {dt}: B={B} H={H} T={T} seed={seed}")
    x = _state(KI.make_vprec_inputs("vprec_lm45m_bf16", B=B, H=H, T=T, dk=dk, dv=dv, seed=seed, dtype=dt),
               dk, dv, seed, per_value=True)
    st = TV.run_case(x, state=True)
    say(f"[ok] forward_vprec widths dk={dk} dv={dv} {dt}: " + ", ".join(f"{k}={v:.2e}" for k, v in st.items()))


@pytest.mark.parametrize("dk,dv,dt", CASES, ids=IDS)
def test_backward_every_width(dk, dv, dt):
    seed = _seed(12400, dk, dv, dt)
    say(f"[case] backward widths dk={dk} dv={dv} {dt}: B={B} H={H} T={T} seed={seed}")
    x, gh = TB.make_case(B, H, T, dk, dv, dt, seed, state=True)
    got = TB.gpu_backward(to_dev(x), TB.grads_to_dev(gh, dt), state_in=True)
    ref = TB.oracle_backward(x, gh, state_in=True)
    TB.compare(f"backward widths dk={dk} dv={dv} {dt}", x, got, ref, state_in=True)


@pytest.mark.parametrize("dk,dv,dt", CASES, ids=IDS)
def test_decode_step_every_width(dk, dv, dt):
    """Three decode steps in a row, each against the oracle's step from the
    oracle's previous state (so an error does not compound)."""
    import torch
    from oracle import kla_decode_step_f64
    import test_gpu_decode as TD
    seed = _seed(12500, dk, dv, dt)
    say(f"[case] decode widths dk={dk} dv={dv} {dt}: B={B} H={H} seed={seed}")
    x = TD.step_inputs(B, H, dk, dv, dt, seed)
    lam, M = x["lam"], x["M"]
    for s in range(3):
        xs = TD.step_inputs(B, H, dk, dv, dt, seed + 100 * (s + 1)) if s else x
        got = TD.gpu_step(to_dev(xs), torch.from_numpy(lam).cuda(), torch.from_numpy(M).cuda())
        ref = kla_decode_step_f64(*(xs[n] for n in TD.NAMES), lam, M)
        TD.check_step(f"decode widths dk={dk} dv={dv} {dt} step {s}", xs, got, ref)
        lam, M = ref[1].astype(np.float32), ref[2].astype(np.float32)
