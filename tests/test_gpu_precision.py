"""GPU parity of kla_precision_scan against the float64 oracle (needs an MI355X).

Precision paths are compared element by element at |x - r| <= 1e-5 |r|.
"""
import numpy as np
import pytest

import kla_inputs as KI
from kla_testutil import check_f32, precision_oracle, say

pytestmark = pytest.mark.gpu


def run_scan(name, x, lam0=None):
    import torch
    import bius_scan_sequence_amd as K
    B, H, T, D = x["log_decay"].shape
    say(f"[case] {name}: seed={x['seed']} B={B} H={H} T={T} D={D} "
        f"workspace={K.kla_precision_scan_workspace_bytes(B, H, T, D)}")
    dev = {n: torch.from_numpy(x[n]).cuda() for n in ("log_decay", "proc_noise", "obs_prec")}
    l0 = None if lam0 is None else torch.from_numpy(lam0).cuda()
    path, lT = K.precision_scan(dev["log_decay"], dev["proc_noise"], dev["obs_prec"], l0)
    torch.cuda.synchronize()
    rp, rl = precision_oracle(x["log_decay"], x["proc_noise"], x["obs_prec"], lam0)
    e1 = check_f32("lambda_path", path.cpu().numpy(), rp, per_head_floor=False)
    e2 = check_f32("lambda_T", lT.cpu().numpy(), rl, per_head_floor=False)
    say(f"[ok] {name}: path err {e1:.2e}, lambda_T err {e2:.2e}")


@pytest.mark.parametrize("shape", [
    (1, 1, 1, 64), (1, 2, 100, 64), (2, 3, 777, 16), (1, 1, 5000, 64), (1, 1, 70001, 7),
    (4, 64, 300, 64), (1, 5, 2048, 100),
], ids=lambda s: "x".join(map(str, s)))
def test_precision_shapes(shape):
    B, H, T, D = shape
    x = KI.make_precision_inputs(B=B, H=H, T=T, D=D, seed=4000 + T)
    run_scan(f"pscan {shape}", x)


def test_precision_initial_state():
    x = KI.make_precision_inputs(B=1, H=3, T=3000, D=32, seed=9)
    lam0 = (0.01 + 5 * np.random.default_rng(1).random((1, 3, 32))).astype(np.float32)
    run_scan("pscan lambda0", x, lam0)


def test_precision_t_zero():
    import torch
    import bius_scan_sequence_amd as K
    say("[case] pscan T=0")
    z = torch.zeros((1, 2, 0, 8), device="cuda")
    l0 = torch.rand((1, 2, 8), device="cuda") + 1
    path, lT = K.precision_scan(z, z, z, l0)
    torch.cuda.synchronize()
    assert path.shape == (1, 2, 0, 8) and torch.equal(lT, l0)


def test_chains_f32_full_size_sampled():
    """chains_f32 at its full size: 65536 chains x 65536 tokens (B=1, H=1024,
    D=64; 68.7 GB of device arrays), generated on the device; 256 sampled
    chains are checked against the oracle over all 65536 tokens."""
    import torch
    import bius_scan_sequence_amd as K
    w = KI.workload("chains_f32")
    say(f"[case] chains_f32 full size: seed={w.seed} B={w.B} H={w.H} T={w.T} D={w.dk}")
    x = KI.make_precision_inputs_torch(B=w.B, H=w.H, T=w.T, D=w.dk, seed=w.seed)
    path, lT = K.precision_scan(x["log_decay"], x["proc_noise"], x["obs_prec"])
    torch.cuda.synchronize()
    say("[step] chains_f32 GPU scan done")
    rng = np.random.default_rng(w.seed)
    hs = torch.from_numpy(rng.integers(0, w.H, 256)).cuda()
    ds = torch.from_numpy(rng.integers(0, w.dk, 256)).cuda()
    pick = lambda t: t[0][hs, :, ds].T.contiguous().cpu().numpy()[None, None]  # [1,1,T,256]
    ld, pn, c = pick(x["log_decay"]), pick(x["proc_noise"]), pick(x["obs_prec"])
    got_path = pick(path)
    got_T = lT[0][hs, ds].cpu().numpy()
    del x, path, lT
    torch.cuda.empty_cache()
    rp, rl = precision_oracle(ld, pn, c)
    e1 = check_f32("chains path", got_path, rp, per_head_floor=False)
    e2 = check_f32("chains lambda_T", got_T, rl[0, 0], per_head_floor=False)
    say(f"[ok] chains_f32 sampled: path err {e1:.2e}, lambda_T err {e2:.2e}")
