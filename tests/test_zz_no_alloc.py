"""kla_forward_noalloc, the forward entry point that allocates nothing (its
scratch is a device array inside the library), against kla_forward with a
caller's workspace, through the C ABI: the same kernels, so the same bits.
Two calls in a row per path, the second on a smaller input, then a repeat of
the first: each call starts from the scratch the previous one left behind."""
import numpy as np
import pytest

import kla_inputs as KI
from kla_testutil import say

pytestmark = pytest.mark.gpu

# (B, H, T, dk, dv, dtype): the run kernel (bf16, d64: 16 and 5 runs per head,
# look-backs between them) and the segment kernels (f32, d32).
PAIRS = {
    "run_bf16_d64": [(2, 4, 1024, 64, 64, "bf16"), (1, 2, 300, 64, 64, "bf16")],
    "segments_f32_d32": [(2, 2, 700, 32, 32, "f32"), (1, 1, 130, 32, 32, "f32")],
}


def _inputs(shape, seed):
    import torch
    B, H, T, dk, dv, dt = shape
    x = KI.make_forward_inputs("lm45m_bf16", B=B, H=H, T=T, dk=dk, dv=dv, seed=seed, dtype=dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    xd = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to("cuda").to(tdt)
          for n in ("q", "k", "v", "log_decay", "proc_noise", "val_prec")}
    rng = np.random.default_rng(seed + 7)
    xd["lambda0"] = torch.from_numpy((0.5 + rng.random((B, H, dk))).astype(np.float32)).to("cuda")
    xd["M0"] = torch.from_numpy(rng.standard_normal((B, H, dk, dv)).astype(np.float32)).to("cuda")
    return xd


def _call(K, xd, shape, noalloc):
    import torch
    B, H, T, dk, dv, dt = shape
    code = K.KLA_BF16 if dt == "bf16" else K.KLA_F32
    y = torch.full((B, H, T, dv), float("nan"), dtype=xd["q"].dtype, device="cuda")
    lam_T = torch.full((B, H, dk), float("nan"), dtype=torch.float32, device="cuda")
    M_T = torch.full((B, H, dk, dv), float("nan"), dtype=torch.float32, device="cuda")
    lpath = torch.full((B, H, T, dk), float("nan"), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    ptrs = [xd[n].data_ptr() for n in ("q", "k", "v", "log_decay", "proc_noise", "val_prec")]
    ptrs += [xd["lambda0"].data_ptr(), xd["M0"].data_ptr(), y.data_ptr(), lam_T.data_ptr(), M_T.data_ptr(),
             lpath.data_ptr()]
    err = None
    if noalloc:
        err = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        rc = K.kla_forward_noalloc(*ptrs, B, H, T, dk, dv, code, err.data_ptr(), stream)
    else:
        need = K.kla_forward_workspace_bytes(B, H, T, dk, dv)
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        rc = K.kla_forward(*ptrs, B, H, T, dk, dv, code, ws.data_ptr(), need, stream)
    assert rc == 0, K.kla_status_string(rc)
    torch.cuda.synchronize()
    return (y, lam_T, M_T, lpath), err


@pytest.mark.parametrize("path", sorted(PAIRS))
def test_noalloc_matches_forward(path):
    import torch
    import bius_scan_sequence_amd as K
    big, small = PAIRS[path]
    for i, shape in enumerate((big, small, big)):
        say(f"[noalloc] {path} call {i}: B,H,T,dk,dv,dtype = {shape}")
        xd = _inputs(shape, seed=9100 + i)
        want, _ = _call(K, xd, shape, noalloc=False)
        got, err = _call(K, xd, shape, noalloc=True)
        assert int(err.item()) == 0
        for name, g, w in zip(("y", "lambda_T", "M_T", "lambda_path"), got, want):
            assert torch.isfinite(g.float()).all(), name
            assert torch.equal(g, w), f"{name}: max |diff| {(g.float() - w.float()).abs().max().item():.3e}"


def test_noalloc_empty_sequence():
    import torch
    import bius_scan_sequence_amd as K
    B, H, dk, dv = 2, 3, 64, 64
    lam0 = torch.rand((B, H, dk), device="cuda") + 0.5
    M0 = torch.randn((B, H, dk, dv), device="cuda")
    lam_T = torch.empty_like(lam0)
    M_T = torch.empty_like(M0)
    err = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    rc = K.kla_forward_noalloc(None, None, None, None, None, None, lam0.data_ptr(), M0.data_ptr(), None,
                               lam_T.data_ptr(), M_T.data_ptr(), None, B, H, 0, dk, dv, K.KLA_BF16,
                               err.data_ptr(), stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(lam_T, lam0) and torch.equal(M_T, M0)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    """B*H = 2048 heads at T = 2048 (bf16, d64) need about 69 MB of scratch:
    rejected on the host with KLA_ERR_TOO_LARGE, nothing launched; kla_forward
    with a workspace still serves the shape (not run here)."""
    import torch
    import bius_scan_sequence_amd as K
    B, H, T, dk, dv = 32, 64, 2048, 64, 64
    x = torch.zeros((B, H, T, dk), dtype=torch.bfloat16, device="cuda")
    lam_T = torch.empty((B, H, dk), dtype=torch.float32, device="cuda")
    M_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    p = x.data_ptr()
    stream = torch.cuda.current_stream().cuda_stream
    rc = K.kla_forward_noalloc(p, p, p, p, p, p, None, None, p, lam_T.data_ptr(), M_T.data_ptr(), None,
                               B, H, T, dk, dv, K.KLA_BF16, None, stream)
    assert rc == 5  # KLA_ERR_TOO_LARGE
    assert "KLA_NOALLOC_SCRATCH_BYTES" in K.kla_status_string(rc)
    assert K.kla_forward_workspace_bytes(B, H, T, dk, dv) > K.KLA_NOALLOC_SCRATCH_BYTES
