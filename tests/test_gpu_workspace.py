"""A workspace reused across calls of different shapes (needs an MI355X).

Flags of a call carry the call's epoch, which advances once every workgroup
of the call has counted itself done.  Each case first runs a call with few
units (heads or chain blocks) that leaves a large workspace, then calls with
more units on the same workspace.  The done counters of the extra units must
start from zero, so they live in a fixed region of every layout.  Otherwise
the epoch stops advancing and a later call takes an earlier call's records
for its own.  Every later call must equal, bit for bit, the same call on a
fresh workspace (a result does not depend on its workspace), and the epoch
must advance by one per call.
"""
import numpy as np
import pytest

import kla_inputs as KI
from kla_testutil import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import bius_scan_sequence_amd as K
    assert torch.cuda.is_available()
    yield K
    torch.cuda.synchronize()


def _epoch(ws):
    return int(ws.buf[:4].view(__import__("torch").int32).item())


NAMES = ("q", "k", "v", "log_decay", "proc_noise", "val_prec")


def _fwd_inputs(H, T, seed):
    import torch
    x = KI.make_forward_inputs("lm45m_bf16", B=1, H=H, T=T, seed=seed)
    return {n: torch.from_numpy(x[n]).cuda().to(torch.bfloat16) for n in NAMES}


def test_forward_workspace_reused_with_more_heads():
    """Three calls over 4 heads (16000 tokens) leave a large workspace with
    flags of three epochs; then two calls over 100 heads (260 tokens, other
    inputs each) on it.  The second must equal the same call on a fresh
    workspace: with a stale epoch it would take the first one's records."""
    import torch
    import bius_scan_sequence_amd as K
    say("[case] forward workspace reuse: 3 x (B1 H4 T16000), then B1 H100 T260 twice (other inputs), d64 bf16")
    ws = K.Workspace("cuda")
    a = _fwd_inputs(4, 16000, 31)
    for _ in range(3):
        K.forward(*(a[n] for n in NAMES), workspace=ws)
    torch.cuda.synchronize()
    del a
    assert K.kla_forward_workspace_bytes(1, 100, 260, 64, 64) <= ws.buf.numel()  # no regrowth (no re-zeroing)
    b1, b2 = _fwd_inputs(100, 260, 32), _fwd_inputs(100, 260, 33)
    e0 = _epoch(ws)
    K.forward(*(b1[n] for n in NAMES), workspace=ws)
    r2 = K.forward(*(b2[n] for n in NAMES), workspace=ws, return_lambda_path=True)
    fresh = K.forward(*(b2[n] for n in NAMES), workspace=K.Workspace("cuda"), return_lambda_path=True)
    torch.cuda.synchronize()
    for name, x2, xf in zip(("y", "lambda_T", "M_T", "lambda_path"), r2, fresh):
        assert torch.equal(x2, xf), f"second call on the reused workspace, {name}"
    assert _epoch(ws) == e0 + 2, (e0, _epoch(ws))
    assert ws.error() == 0
    say("[ok] forward workspace reuse")


def _pscan_inputs(H, T, D, seed):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    sp = torch.nn.functional.softplus
    rn = lambda: torch.randn((1, H, T, D), generator=g, device="cuda")
    return -sp(rn()), sp(rn()), sp(rn())


def test_precision_scan_workspace_reused_with_more_chain_blocks():
    """Three calls over 64 chain blocks (16384 tokens) leave a large workspace;
    then two calls over 80 chain blocks (2048 tokens, other inputs each).  The
    second must equal the same call on a fresh workspace."""
    import torch
    import bius_scan_sequence_amd as K
    say("[case] precision-scan workspace reuse: 3 x (64 chain blocks, T16384), then 80 blocks x T2048 twice")
    ws = K.Workspace("cuda")
    a = _pscan_inputs(256, 16384, 64, 41)  # 16384 chains = 64 blocks of 256, 16 segments
    for _ in range(3):
        K.precision_scan(*a, workspace=ws)
    torch.cuda.synchronize()
    del a
    assert K.kla_precision_scan_workspace_bytes(1, 320, 2048, 64) <= ws.buf.numel()
    b1, b2 = _pscan_inputs(320, 2048, 64, 42), _pscan_inputs(320, 2048, 64, 43)  # 80 blocks, 4 segments
    e0 = _epoch(ws)
    K.precision_scan(*b1, workspace=ws)
    r2 = K.precision_scan(*b2, workspace=ws)
    fresh = K.precision_scan(*b2, workspace=K.Workspace("cuda"))
    torch.cuda.synchronize()
    for name, x2, xf in zip(("lambda_path", "lambda_T"), r2, fresh):
        assert torch.equal(x2, xf), f"second call on the reused workspace, {name}"
    assert _epoch(ws) == e0 + 2, (e0, _epoch(ws))
    assert ws.error() == 0
    say("[ok] precision-scan workspace reuse")
