"""GPU parity of kla_forward on degenerate coefficients and at the largest
supported size (needs an MI355X).

Degenerate cases, each a textbook special case of the filter:
  * no process noise (pbar = 0): the precision only grows (long-memory decays,
    so that it stays inside the fp32 range);
  * no observation (Lambda^v = 0): g = 0 and f = a, so y is the decayed prior mean;
  * no decay and no process noise (a = 1, pbar = 0): recursive least squares;
  * q = 0: y = 0 exactly, the state still evolves.
The largest size: B*H*T*d_k just below 2^31 (B=1, H=1024, T=32767, d=64, bf16;
about 30 GB of inputs, outputs and workspace), generated on the device; the
oracle checks two sampled heads over all 32767 tokens (ragged last segment).
"""
import numpy as np
import pytest

import kla_inputs as KI
from kla_testutil import check_forward, gpu_forward, oracle_forward, say, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "log_decay", "proc_noise", "val_prec")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import bius_scan_sequence_amd as K
    assert torch.cuda.is_available()
    yield K
    torch.cuda.synchronize()


def _no_process_noise(x):
    # Without process noise the precision grows by 1/a^2 per token; decays
    # near 1 (a^2 about 0.96) keep it inside the fp32 range over 300 tokens
    # (the library's precondition: the precision must stay below FLT_MAX).
    ld = 0.02 * x["log_decay"].astype(np.float32)
    x.update(proc_noise=np.zeros_like(x["proc_noise"]),
             log_decay=KI.round_bf16(ld) if x["dtype"] == "bf16" else ld)


CASES = {
    "no_process_noise": _no_process_noise,
    "no_observation": lambda x: x.update(val_prec=np.zeros_like(x["val_prec"])),
    "no_decay_no_noise": lambda x: x.update(log_decay=np.zeros_like(x["log_decay"]),
                                            proc_noise=np.zeros_like(x["proc_noise"])),
    "zero_query": lambda x: x.update(q=np.zeros_like(x["q"])),
}


@pytest.mark.parametrize("dt,dk,dv", [("bf16", 64, 64), ("f32", 32, 16), ("bf16", 128, 128)],
                         ids=["bf16_d64", "f32_d32", "bf16_d128"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_degenerate_coefficients(case, dt, dk, dv):
    x = KI.make_forward_inputs("lm45m_bf16", B=1, H=2, T=300, dk=dk, dv=dv, seed=9100, dtype=dt)
    rng = np.random.default_rng(9100)
    x["lambda0"] = (0.5 + rng.random((1, 2, dk))).astype(np.float32)
    x["M0"] = rng.standard_normal((1, 2, dk, dv)).astype(np.float32)
    CASES[case](x)
    say(f"[case] degenerate {case} {dt} dk={dk} dv={dv}: seed=9100 T=300")
    got = gpu_forward(to_dev(x), return_lambda_path=True)
    ref = oracle_forward(x, return_lambda_path=True)
    stats = check_forward(x, got, ref, dt)
    if case == "zero_query":
        assert np.all(got[0] == 0), "y must vanish with q = 0"
    say(f"[ok] degenerate {case} {dt}: " + ", ".join(f"{k}={v:.2e}" for k, v in stats.items()))


def test_maximum_size_sampled_heads():
    import torch
    import bius_scan_sequence_amd as K
    B, H, T, d = 1, 1024, 32767, 64
    assert B * H * T * d < 2 ** 31
    w = KI.Workload(90, "max_bf16", "forward", B, H, T, d, d, "bf16")
    say(f"[case] maximum size: B={B} H={H} T={T} d={d} bf16 seed={w.seed} "
        f"({B * H * T * d} elements per tensor)")
    xd = KI.make_forward_inputs_torch(w, device="cuda")
    torch.cuda.synchronize()
    say("[step] inputs generated")
    ws = K.Workspace(xd["q"].device)
    y, lT, MT = K.forward(*(xd[n] for n in NAMES), workspace=ws)
    torch.cuda.synchronize()
    assert ws.error() == 0
    say("[step] forward done")
    for flat in (3, 1021):
        x = {n: xd[n][0:1, flat:flat + 1].float().cpu().numpy() for n in NAMES}
        x["dtype"] = "bf16"
        ref = oracle_forward(x)
        got = (y[0:1, flat:flat + 1].float().cpu().numpy(), lT[0:1, flat:flat + 1].cpu().numpy(),
               MT[0:1, flat:flat + 1].cpu().numpy())
        stats = check_forward(x, got, ref, "bf16")
        say(f"[ok] maximum size head {flat}: " + ", ".join(f"{k}={v:.2e}" for k, v in stats.items()))
    del xd, y, lT, MT, ws
    torch.cuda.empty_cache()
