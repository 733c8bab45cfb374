"""Float64 gradients of the KLA forward scan (the backward pass).

TEST INFRASTRUCTURE ONLY: imported by tests/ and the benchmark's CPU baseline,
never by the product path.

Training a KLA layer needs the gradients of the loss with respect to every
input of the scan ([KLA-nl] "Belangrijkste Bijdragen": KLA is trained as the
sequence mixer of a language model).  The forward pass is the sequential
filter of [KLA-nl] §1-§3 (predict / update of the precision, precision-ratio
gates, affine mean recursion, readout of the posterior mean); this module
writes that same filter with plain PyTorch CPU operations in float64 and lets
reverse-mode automatic differentiation produce the gradients.  No adjoint is
derived by hand here, so the result is the exact derivative of the filter up
to float64 rounding.  The tests pin it to central finite differences of the
numpy oracle (oracle/kla_f64.py).
"""
from __future__ import annotations

import numpy as np

__all__ = ["kla_forward_torch64", "kla_backward_f64"]


def _torch():
    import torch
    return torch


def kla_forward_torch64(q, k, v, log_decay, proc_noise, val_prec, lambda0, M0):
    """The sequential filter on float64 torch tensors (differentiable).

    Same steps, in the same order, as oracle.kla_f64.filter_step: predict
    lam^- = lam / (a^2 + pbar lam), update lam = lam^- + k^2 Lambda^v, gates
    f = a lam^- / lam and g = k Lambda^v / lam, M = f M + g v, y = q^T M.
    Returns (y [B,H,T,dv], lambda_T [B,H,dk], M_T [B,H,dk,dv]).
    """
    torch = _torch()
    T = k.shape[2]
    lam, M = lambda0, M0
    ys = []
    for t in range(T):
        a = torch.exp(log_decay[:, :, t])
        kt, lt = k[:, :, t], val_prec[:, :, t]
        lam_pred = lam / (a * a + proc_noise[:, :, t] * lam)
        lam_new = lam_pred + kt * kt * lt
        f = a * lam_pred / lam_new
        g = kt * lt / lam_new
        M = f[..., None] * M + g[..., None] * v[:, :, t, None, :]
        ys.append(torch.einsum("bhi,bhij->bhj", q[:, :, t], M))
        lam = lam_new
    y = torch.stack(ys, 2) if ys else torch.zeros(v.shape, dtype=torch.float64)
    return y, lam, M


def kla_backward_f64(q, k, v, log_decay, proc_noise, val_prec, dy, lambda0=None, M0=None,
                     d_lambda_T=None, d_M_T=None):
    """Gradients of L = <dy, y> + <d_lambda_T, lambda_T> + <d_M_T, M_T>.

    Inputs as oracle.kla_f64.kla_forward_f64 (numpy arrays, any float dtype),
    dy [B,H,T,dv]; lambda0 defaults to 1 and M0 to 0, the upstream state
    gradients to 0.  Returns a dict of float64 numpy arrays: dq, dk, dv,
    d_log_decay, d_proc_noise, d_val_prec ([B,H,T,*]), d_lambda0 [B,H,dk],
    d_M0 [B,H,dk,dv].
    """
    torch = _torch()
    B, H, T, dk = np.shape(k)
    dv = np.shape(v)[-1]
    t64 = lambda x: torch.tensor(np.asarray(x, np.float64), dtype=torch.float64, requires_grad=True)
    xs = {n: t64(x) for n, x in (("q", q), ("k", k), ("v", v), ("log_decay", log_decay),
                                   ("proc_noise", proc_noise), ("val_prec", val_prec))}
    lam0 = t64(np.ones((B, H, dk)) if lambda0 is None else lambda0)
    m0 = t64(np.zeros((B, H, dk, dv)) if M0 is None else M0)
    y, lamT, MT = kla_forward_torch64(xs["q"], xs["k"], xs["v"], xs["log_decay"], xs["proc_noise"],
                                      xs["val_prec"], lam0, m0)
    loss = (y * torch.tensor(np.asarray(dy, np.float64))).sum()
    if d_lambda_T is not None:
        loss = loss + (lamT * torch.tensor(np.asarray(d_lambda_T, np.float64))).sum()
    if d_M_T is not None:
        loss = loss + (MT * torch.tensor(np.asarray(d_M_T, np.float64))).sum()
    order = ["q", "k", "v", "log_decay", "proc_noise", "val_prec"]
    grads = torch.autograd.grad(loss, [xs[n] for n in order] + [lam0, m0], allow_unused=True)
    names = ["dq", "dk", "dv", "d_log_decay", "d_proc_noise", "d_val_prec", "d_lambda0", "d_M0"]
    ref = [xs[n] for n in order] + [lam0, m0]
    out = {}
    for name, g, r in zip(names, grads, ref):
        out[name] = np.zeros(tuple(r.shape)) if g is None else g.detach().numpy()
    return out
