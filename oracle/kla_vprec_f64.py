"""Float64 oracle of the KLA variant with the value precision indexed by value
channel (a d_k x d_v precision field).

TEST INFRASTRUCTURE ONLY: imported by tests/ and the benchmark's CPU baseline,
never by the product path.

[KLA-nl] §1 ("Observatiemodel") gives each value an observation precision
Lambda^v; the main path reads it as indexed like k (per key channel), so one
precision per (b,h,i) is shared over the value channels j.  This module takes
the other reading: Lambda^v_{t,j} per value channel.  Every element (i,j) is
then its own scalar Kalman filter with observation precision
c_{t,ij} = k_{t,i}^2 Lambda^v_{t,j}, so the precision lam_{t,ij}, the gates
f_{t,ij} = a_{t,i} lam^-_{t,ij} / lam_{t,ij} and g_{t,ij} = k_{t,i}
Lambda^v_{t,j} / lam_{t,ij} are all per element; the mean recursion and the
readout y_t = q_t^T M_t are unchanged ([KLA-nl] §1-§3).  The step functions of
oracle.kla_f64 are applied elementwise with broadcasting.
"""
from __future__ import annotations

import numpy as np

from . import kla_f64 as O

__all__ = ["kla_forward_vprec_f64"]


def kla_forward_vprec_f64(q, k, v, log_decay, proc_noise, val_prec, lambda0=None, M0=None,
                          return_lambda_path=False):
    """q, k, log_decay, proc_noise [B,H,T,dk]; v and val_prec [B,H,T,dv];
    lambda0 and M0 [B,H,dk,dv] (defaults 1 and 0).  Returns (y [B,H,T,dv],
    lambda_T [B,H,dk,dv], M_T [B,H,dk,dv]) and the precision path
    [B,H,T,dk,dv] if asked."""
    q, k, v, ld, pn, vp = (np.asarray(x, np.float64) for x in (q, k, v, log_decay, proc_noise, val_prec))
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    lam = np.ones((B, H, dk, dv)) if lambda0 is None else np.array(lambda0, np.float64)
    M = np.zeros((B, H, dk, dv)) if M0 is None else np.array(M0, np.float64)
    y = np.empty((B, H, T, dv))
    path = np.empty((B, H, T, dk, dv)) if return_lambda_path else None
    for t in range(T):
        a = np.exp(ld[:, :, t])[..., None]        # [B,H,dk,1]
        pb = pn[:, :, t][..., None]
        kk = k[:, :, t][..., None]
        L = vp[:, :, t][:, :, None, :]            # [B,H,1,dv]
        lam_pred = O.predict_precision(lam, a, pb)
        lam_new = O.update_precision(lam_pred, kk * kk * L)
        f = O.forget_gate(a, lam_pred, lam_new)
        g = O.write_gate(kk, L, lam_new)
        M = f * M + g * v[:, :, t][:, :, None, :]
        y[:, :, t] = O.readout(q[:, :, t], M)
        lam = lam_new
        if path is not None:
            path[:, :, t] = lam
    return (y, lam, M, path) if return_lambda_path else (y, lam, M)
