"""GPU parity of kla_backward (gradients of the forward scan) against the
float64 autograd oracle (oracle/kla_backward_f64.py), needs an MI355X.

The path under test is the training path: the GPU forward pass writes the
precision path, and the GPU backward pass takes it with the inputs and the
upstream gradients.  The oracle differentiates the sequential float64 filter
on the same (dtype-rounded) inputs.

Tolerance (float64 oracle r, GPU result x, per (b, h) RMS floor as for y):
  |x - r| <= tol * max(|r|, rms_{b,h}(r)) + FLT_MIN
  tol = 1e-4 for float32 results (grad_lambda0 and grad_M0 always; every
  gradient for float32 inputs).  Derivation: a float32 emulation of the same
  decomposition reached 1.3e-5 on the lm45m and long input recipes (d_log_decay,
  a suffix sum over the sequence, is the worst); 1e-4 leaves 8x margin.
  tol = 2^-8 for bfloat16 results: one rounding to bf16 (2^-9 relative) on top
  of the float32 error.
grad_lambda0 takes a different floor.  The prior precision enters only the
first predict step, so dL/dlambda0 = -(a_1^2/lambda0^2) dL/dpbar_1; the same
expression at every token, -(a_t^2/lambda_{t-1}^2) dL/dpbar_t, is the adjoint
of the precision entering each predict step.  The filter forgets its prior
geometrically, so dL/dlambda0 can be ~1e-17 while that adjoint is O(1) and
float32 rounds at its scale: the floor is its RMS over the head's tokens.
Every case prints its name, seed and shape before touching the GPU.
"""
import numpy as np
import pytest

import kla_inputs as KI
from kla_testutil import F32_TINY, say, to_dev
from oracle import kla_forward_f64
from oracle.kla_backward_f64 import kla_backward_f64

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "log_decay", "proc_noise", "val_prec")
GRADS = ("dq", "dk", "dv", "d_log_decay", "d_proc_noise", "d_val_prec", "d_lambda0", "d_M0")
TOL_F32, TOL_BF16 = 1e-4, 2.0 ** -8


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import bius_scan_sequence_amd as K
    assert torch.cuda.is_available()
    yield K
    torch.cuda.synchronize()


def head_rms(r):
    return np.sqrt(np.mean(r * r, axis=tuple(range(2, r.ndim)), keepdims=True))


def check_grad(name, x, r, tol, floor=None):
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    assert x.shape == r.shape, (name, x.shape, r.shape)
    assert np.all(np.isfinite(x)), f"{name}: non-finite output"
    if r.size == 0:
        return 0.0
    scale = np.maximum(np.abs(r), head_rms(r) if floor is None else floor)
    err = np.maximum(np.abs(x - r) - F32_TINY, 0.0) / np.maximum(scale, 1e-300)
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= tol, f"{name}: max scaled error {err.max():.3e} at {worst}: got {x[worst]}, want {r[worst]}"
    return float(err.max())


def gpu_backward(xd, g, state_in=True):
    """GPU forward (for the precision path), then GPU backward."""
    import torch
    import bius_scan_sequence_amd as K
    lam0 = xd.get("lambda0") if state_in else None
    M0 = xd.get("M0") if state_in else None
    _, _, _, lpath = K.forward(*(xd[n] for n in NAMES), lam0, M0, return_lambda_path=True)
    out = K.backward(*(xd[n] for n in NAMES), g["grad_y"], lpath, lam0, M0, g.get("grad_lambda_T"),
                     g.get("grad_M_T"))
    torch.cuda.synchronize()
    return dict(zip(GRADS, (t.float().cpu().numpy() for t in out)))


def grads_to_dev(gh, dtype):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {"grad_y": torch.from_numpy(gh["grad_y"]).cuda().to(tdt)}
    for n in ("grad_lambda_T", "grad_M_T"):
        out[n] = None if gh[n] is None else torch.from_numpy(gh[n]).cuda()
    return out


def oracle_backward(x, gh, state_in=True):
    return kla_backward_f64(*(x[n] for n in NAMES), gh["grad_y"],
                            x["lambda0"] if state_in else None, x["M0"] if state_in else None,
                            gh["grad_lambda_T"], gh["grad_M_T"])


def lambda0_floor(x, ref, state_in=True):
    """Per-head RMS of -(a_t^2 / lambda_{t-1}^2) dL/dpbar_t over the tokens."""
    lam0 = x["lambda0"] if state_in else np.ones_like(x["lambda0"])
    lpath = kla_forward_f64(*(x[n] for n in NAMES), lam0, None, return_lambda_path=True)[3]
    lprev = np.concatenate([np.asarray(lam0, np.float64)[:, :, None], lpath[:, :, :-1]], axis=2)
    fam = ref["d_proc_noise"] * np.exp(2.0 * x["log_decay"].astype(np.float64)) / lprev ** 2
    return head_rms(fam)[..., 0]


def compare(label, x, got, ref, state_in=True):
    stats = {}
    for n in GRADS:
        tol = TOL_F32 if (x["dtype"] == "f32" or n in ("d_lambda0", "d_M0")) else TOL_BF16
        floor = lambda0_floor(x, ref, state_in) if n == "d_lambda0" and x["q"].shape[2] > 0 else None
        stats[n] = check_grad(f"{label} {n}", got[n], ref[n], tol, floor)
    say(f"[ok] {label}: " + ", ".join(f"{k}={v:.1e}" for k, v in stats.items()))


def make_case(B, H, T, dk, dv, dt, seed, state=True, recipe="lm45m_bf16"):
    x = KI.make_forward_inputs(recipe, B=B, H=H, T=T, dk=dk, dv=dv, seed=seed, dtype=dt)
    rng = np.random.default_rng(seed)
    if state:
        x["lambda0"] = (0.5 + rng.random((B, H, dk))).astype(np.float32)
        x["M0"] = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    gh = KI.make_backward_grads(B=B, H=H, T=T, dk=dk, dv=dv, seed=seed, dtype=dt, state=state)
    return x, gh


SHAPES = [
    # (B, H, T, dk, dv, dtype, state): one chunk, ragged chunks and segments, several segments
    (1, 1, 1, 16, 16, "f32", True),
    (1, 1, 16, 16, 16, "f32", False),
    (1, 2, 100, 16, 32, "f32", True),
    (2, 1, 200, 32, 16, "f32", True),
    (1, 2, 130, 64, 64, "f32", True),
    (1, 1, 64, 64, 32, "f32", False),
    (2, 2, 257, 64, 64, "bf16", True),
    (1, 3, 64, 32, 64, "bf16", False),
    (1, 2, 333, 16, 64, "bf16", True),
    # widths of 128 run as 64-wide halves: key halves, value halves, both
    (1, 2, 150, 128, 64, "f32", True),
    (1, 1, 100, 32, 128, "f32", True),
    (1, 2, 140, 128, 128, "f32", False),
    (2, 1, 200, 128, 128, "bf16", True),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_matches_oracle(shape):
    B, H, T, dk, dv, dt, state = shape
    seed = 9300 + T + dk + 7 * dv
    say(f"[case] backward {shape}: seed={seed}")
    x, gh = make_case(B, H, T, dk, dv, dt, seed, state)
    # Without a state in, both sides take the defaults (lambda0 = 1, M0 = 0; NULL on the GPU).
    got = gpu_backward(to_dev(x), grads_to_dev(gh, dt), state_in=state)
    ref = oracle_backward(x, gh, state_in=state)
    compare(f"backward {shape}", x, got, ref, state_in=state)


@pytest.mark.parametrize("recipe", ["lm180m_bf16", "long_bf16"])
def test_backward_other_recipes(recipe):
    """The value-precision spikes (x100 on 5% of tokens) and the slow-decay
    recipe, at d = 64."""
    say(f"[case] backward recipe {recipe}: B=1 H=2 T=300 d=64 seed=9400")
    x, gh = make_case(1, 2, 300, 64, 64, "bf16", 9400, state=True, recipe=recipe)
    got = gpu_backward(to_dev(x), grads_to_dev(gh, "bf16"))
    compare(f"backward {recipe}", x, got, oracle_backward(x, gh))


def _no_observation(x):
    x["val_prec"] = np.zeros_like(x["val_prec"])


def _extreme_decay(x):
    ld = x["log_decay"].copy()
    ld[0, 0, 20:40, 3] = -9.0     # in-chunk decay far below 2^-64
    ld[0, 1, 100:112, :] = -12.0
    ld[0, 1, 70, 5] = -60.0       # one token wipes a channel's memory
    x["log_decay"] = KI.round_bf16(ld) if x["dtype"] == "bf16" else ld.astype(np.float32)


def _no_decay_no_noise(x):
    x["log_decay"] = np.zeros_like(x["log_decay"])
    x["proc_noise"] = np.zeros_like(x["proc_noise"])


DEGENERATE = {"no_observation": _no_observation, "extreme_decay": _extreme_decay,
              "no_decay_no_noise": _no_decay_no_noise,
              "zero_query": lambda x: x.update(q=np.zeros_like(x["q"]))}


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("case", sorted(DEGENERATE))
def test_backward_degenerate(case, dt):
    say(f"[case] backward degenerate {case} {dt}: B=1 H=2 T=160 dk=32 dv=16 seed=9500")
    x, gh = make_case(1, 2, 160, 32, 16, dt, 9500, state=True)
    DEGENERATE[case](x)
    got = gpu_backward(to_dev(x), grads_to_dev(gh, dt))
    if case == "no_observation":
        assert np.all(got["dv"] == 0), "dv must vanish without observations (g = 0)"
    compare(f"backward {case} {dt}", x, got, oracle_backward(x, gh))


def test_backward_empty_sequence():
    import torch
    import bius_scan_sequence_amd as K
    say("[case] backward T=0")
    B, H, dk, dv = 2, 3, 32, 16
    e = lambda *s: torch.empty(s, device="cuda", dtype=torch.bfloat16)
    ins = [e(B, H, 0, dk), e(B, H, 0, dk), e(B, H, 0, dv), e(B, H, 0, dk), e(B, H, 0, dk), e(B, H, 0, dk)]
    gy = e(B, H, 0, dv)
    lp = torch.empty((B, H, 0, dk), device="cuda")
    glam = torch.randn((B, H, dk), device="cuda")
    gM = torch.randn((B, H, dk, dv), device="cuda")
    out = K.backward(*ins, gy, lp, None, None, glam, gM)
    torch.cuda.synchronize()
    assert torch.equal(out[6], glam) and torch.equal(out[7], gM)
    out = K.backward(*ins, gy, lp)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[6]) == 0 and torch.count_nonzero(out[7]) == 0
    say("[ok] backward T=0")


def test_backward_deterministic():
    import torch
    say("[case] backward determinism: B=2 H=2 T=300 d=64 bf16 seed=9600")
    x, gh = make_case(2, 2, 300, 64, 64, "bf16", 9600, state=True)
    xd, gd = to_dev(x), grads_to_dev(gh, "bf16")
    a = gpu_backward(xd, gd)
    b = gpu_backward(xd, gd)
    for n in GRADS:
        assert np.array_equal(a[n], b[n]), n
    say("[ok] backward determinism")


def test_autograd_scan_matches_backward():
    """K.scan is the forward pass as a torch autograd operation: its input
    gradients equal K.backward's for the same upstream gradients."""
    import torch
    import bius_scan_sequence_amd as K
    say("[case] autograd scan: B=1 H=2 T=100 dk=32 dv=16 f32 seed=9700")
    x, gh = make_case(1, 2, 100, 32, 16, "f32", 9700, state=True)
    xd = to_dev(x)
    leaves = [xd[n].clone().requires_grad_(True) for n in NAMES]
    lam0 = xd["lambda0"].clone().requires_grad_(True)
    M0 = xd["M0"].clone().requires_grad_(True)
    gd = grads_to_dev(gh, "f32")
    y, lT, MT = K.scan(*leaves, lam0, M0)
    loss = (y * gd["grad_y"]).sum() + (lT * gd["grad_lambda_T"]).sum() + (MT * gd["grad_M_T"]).sum()
    got = torch.autograd.grad(loss, leaves + [lam0, M0])
    ref = gpu_backward(xd, gd)
    for n, t in zip(GRADS, got):
        assert np.array_equal(t.detach().cpu().numpy(), ref[n]), n
    say("[ok] autograd scan")


def test_backward_full_size_sampled_heads():
    """The benchmark's backward shape (B=8, H=8, T=2048, d=64, bf16), generated
    on the device; every gradient of two sampled heads against the oracle."""
    import torch
    import bius_scan_sequence_amd as K
    w = KI.workload("bwd_lm45m_bf16")
    say(f"[case] backward full size {w.B}x{w.H}x{w.T} d={w.dk} bf16 seed={w.seed}")
    xd = KI.make_forward_inputs_torch(w, device="cuda")
    gy = KI.make_backward_grads_torch(w, device="cuda")
    _, _, _, lpath = K.forward(*(xd[n] for n in NAMES), return_lambda_path=True)
    out = K.backward(*(xd[n] for n in NAMES), gy, lpath)
    torch.cuda.synchronize()
    say("[step] full-size backward done")
    for b, h in ((0, 3), (7, 6)):
        x = {n: xd[n][b:b + 1, h:h + 1].float().cpu().numpy() for n in NAMES}
        x["dtype"] = "bf16"
        x["lambda0"] = np.ones((1, 1, w.dk), np.float32)
        x["M0"] = np.zeros((1, 1, w.dk, w.dv), np.float32)
        gh = {"grad_y": gy[b:b + 1, h:h + 1].float().cpu().numpy(), "grad_lambda_T": None, "grad_M_T": None}
        ref = oracle_backward(x, gh)
        got = dict(zip(GRADS, (t[b:b + 1, h:h + 1].float().cpu().numpy() for t in out)))
        compare(f"full size head ({b},{h})", x, got, ref)


def test_backward_long_full_size_sampled_head():
    """The long-context backward shape at full size (B=2, H=16, T=16384,
    d=128, bf16, long-memory decays), generated on the device and run in the
    launch configuration the benchmark times; every gradient of one sampled
    head against the oracle (about a minute and a half of float64 work)."""
    import torch
    import bius_scan_sequence_amd as K
    w = KI.workload("bwd_long_bf16")
    say(f"[case] backward full size {w.B}x{w.H}x{w.T} d={w.dk} bf16 seed={w.seed}")
    xd = KI.make_forward_inputs_torch(w, device="cuda")
    gy = KI.make_backward_grads_torch(w, device="cuda")
    _, _, _, lpath = K.forward(*(xd[n] for n in NAMES), return_lambda_path=True)
    out = K.backward(*(xd[n] for n in NAMES), gy, lpath)
    torch.cuda.synchronize()
    say("[step] full-size long backward done; oracle on one head")
    b, h = 1, 11
    x = {n: xd[n][b:b + 1, h:h + 1].float().cpu().numpy() for n in NAMES}
    x["dtype"] = "bf16"
    x["lambda0"] = np.ones((1, 1, w.dk), np.float32)
    x["M0"] = np.zeros((1, 1, w.dk, w.dv), np.float32)
    gh = {"grad_y": gy[b:b + 1, h:h + 1].float().cpu().numpy(), "grad_lambda_T": None, "grad_M_T": None}
    got = dict(zip(GRADS, (t[b:b + 1, h:h + 1].float().cpu().numpy() for t in out)))
    del out, xd, gy, lpath
    ref = oracle_backward(x, gh)
    compare(f"full size long head ({b},{h})", x, got, ref)


def test_backward_long_recipe_d128():
    """The long-memory recipe (log_decay = -softplus(N(-2, 1))) at d = 128 over
    4096 tokens, generated on the device; one sampled head against the
    oracle."""
    import torch
    import bius_scan_sequence_amd as K
    w = KI.Workload(91, "long_d128_4k", "backward", 1, 2, 4096, 128, 128, "bf16", decay_mean=-2.0)
    say(f"[case] backward long recipe B=1 H=2 T=4096 d=128 bf16 seed={w.seed}")
    xd = KI.make_forward_inputs_torch(w, device="cuda")
    gy = KI.make_backward_grads_torch(w, device="cuda")
    _, _, _, lpath = K.forward(*(xd[n] for n in NAMES), return_lambda_path=True)
    out = K.backward(*(xd[n] for n in NAMES), gy, lpath)
    torch.cuda.synchronize()
    say("[step] backward done")
    h = 1
    x = {n: xd[n][0:1, h:h + 1].float().cpu().numpy() for n in NAMES}
    x["dtype"] = "bf16"
    x["lambda0"] = np.ones((1, 1, 128), np.float32)
    x["M0"] = np.zeros((1, 1, 128, 128), np.float32)
    gh = {"grad_y": gy[0:1, h:h + 1].float().cpu().numpy(), "grad_lambda_T": None, "grad_M_T": None}
    ref = oracle_backward(x, gh)
    got = dict(zip(GRADS, (t[0:1, h:h + 1].float().cpu().numpy() for t in out)))
    compare("long recipe d128 head 1", x, got, ref)
