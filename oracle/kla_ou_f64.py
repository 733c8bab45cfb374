"""Float64 oracle of the KLA forward pass with the OU prior in continuous time.

TEST INFRASTRUCTURE ONLY: imported by tests/ and the benchmark's CPU baseline,
never by the product path.

[KLA-nl] §1 ("Probabilistische Formulering", bullet "Dynamics Prior") states
that the prior over each latent is an exactly discretised Ornstein-Uhlenbeck
process.  In continuous time dx = -theta x ds + sigma dW; over a step of length
dt the exact transition is

    x_t = e^{-theta dt} x_{t-1} + w,   Var w = integral_0^dt sigma^2 e^{-2 theta s} ds
                                             = sigma^2 (1 - e^{-2 theta dt}) / (2 theta),

with the Brownian limit sigma^2 dt as theta -> 0.  ou_discretize_f64 writes
this out; kla_forward_ou_f64 feeds the resulting (log_decay, proc_noise) to the
sequential filter of oracle.kla_f64.
"""
from __future__ import annotations

import numpy as np

from .kla_f64 import kla_forward_f64

__all__ = ["ou_discretize_f64", "kla_forward_ou_f64"]


def ou_discretize_f64(theta, sigma2, dt):
    """(log_decay, proc_noise) of OU steps: log a = -theta dt and
    pbar = sigma2 (1 - e^{-2 theta dt}) / (2 theta) (sigma2 dt when theta = 0).

    theta, sigma2 broadcast against dt (e.g. [H,dk] against [B,H,T,dk] after
    adding the T axis); all float64.
    """
    theta = np.asarray(theta, np.float64)
    sigma2 = np.asarray(sigma2, np.float64)
    dt = np.asarray(dt, np.float64)
    u = 2.0 * theta * dt
    with np.errstate(invalid="ignore", divide="ignore"):
        phi = np.where(u == 0.0, 1.0, -np.expm1(-u) / np.where(u == 0.0, 1.0, u))
    return -theta * dt, sigma2 * dt * phi


def kla_forward_ou_f64(q, k, v, dt, theta, sigma2, val_prec, lambda0=None, M0=None, return_lambda_path=False):
    """The forward pass with per-(h,i) OU rate theta and diffusion sigma2
    ([H,dk]) and per-token step lengths dt ([B,H,T,dk])."""
    th = np.asarray(theta, np.float64)[None, :, None, :]
    s2 = np.asarray(sigma2, np.float64)[None, :, None, :]
    log_decay, proc_noise = ou_discretize_f64(th, s2, dt)
    return kla_forward_f64(q, k, v, log_decay, proc_noise, val_prec, lambda0, M0,
                           return_lambda_path=return_lambda_path)
