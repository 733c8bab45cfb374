"""Float64 oracle of the KLA forward pass behind its coefficient prologue.

TEST INFRASTRUCTURE ONLY: imported by tests/ and the benchmark's CPU baseline,
never by the product path.

[KLA-nl] §4 ("Architectuur") places the scan in a fused MLP block of the Mamba
kind with 1D causal convolutions and SiLU activations; §1 ("Probabilistische
Formulering", bullet "Dynamics Prior") makes the prior an exactly discretised
OU process.  The prologue read here turns raw projections into the scan's
inputs:

    q, k, v   = SiLU(causal depthwise conv1d of the raw projections xq, xk, xv)
                u_t[c] = b[c] + sum_{s=0}^{W-1} w[c, s] x_{t-(W-1)+s}[c]
                (x_t = 0 for t < 0: the sequence starts from zero history),
                SiLU(u) = u / (1 + e^{-u});
                the activations are held in the input dtype (bf16 inputs:
                rounded to the nearest bfloat16, as an unfused bf16 block
                stores them);
    dt        = softplus(dt_raw)         step length of each token and channel;
    Lambda^v  = softplus(vp_raw)         value precision;
    (log a, pbar) = exact OU discretisation of (theta, sigma2, dt);

then the sequential filter of oracle.kla_f64.  Parity unpinned beyond the pins
in tests/oracle_pins.py (impulse response and numpy.convolve for the
convolution, closed forms for SiLU and softplus).
"""
from __future__ import annotations

import numpy as np

from .kla_ou_f64 import kla_forward_ou_f64

__all__ = ["causal_conv_f64", "silu_f64", "softplus_f64", "prologue_f64", "kla_forward_prologue_f64"]


def causal_conv_f64(x, w, b=None):
    """Causal depthwise convolution along the token axis.

    x [B,H,T,d]; w [H,d,W] (tap W-1 multiplies the current token, tap s the
    token W-1-s steps back); b [H,d] or None.  Returns u [B,H,T,d] float64.
    """
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    T = x.shape[2]
    W = w.shape[-1]
    u = np.zeros_like(x)
    if b is not None:
        u += np.asarray(b, np.float64)[None, :, None, :]
    for s in range(W):
        back = W - 1 - s  # how many tokens back tap s reaches
        if back >= T:
            continue
        u[:, :, back:, :] += w[None, :, None, :, s] * x[:, :, : T - back, :]
    return u


def silu_f64(u):
    """u * sigmoid(u) = u / (1 + e^{-u})."""
    u = np.asarray(u, np.float64)
    with np.errstate(over="ignore"):
        return u / (1.0 + np.exp(-u))


def softplus_f64(x):
    """log(1 + e^x)."""
    return np.logaddexp(0.0, np.asarray(x, np.float64))


def _to_input_dtype(x, dtype):
    if dtype == "bf16":
        import torch
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    return np.asarray(x, np.float32).astype(np.float64)


def prologue_f64(xq, xk, xv, dt_raw, vp_raw, conv_w, conv_b=(None, None, None), dtype="f32"):
    """(q, k, v, dt, val_prec) the scan consumes; conv_w / conv_b are the
    (q, k, v) weights [H,d,W] and biases [H,d] (None: no bias)."""
    acts = [_to_input_dtype(silu_f64(causal_conv_f64(x, w, b)), dtype)
            for x, w, b in zip((xq, xk, xv), conv_w, conv_b)]
    return acts[0], acts[1], acts[2], softplus_f64(dt_raw), softplus_f64(vp_raw)


def kla_forward_prologue_f64(xq, xk, xv, dt_raw, theta, sigma2, vp_raw, conv_w, conv_b=(None, None, None),
                             lambda0=None, M0=None, dtype="f32", return_lambda_path=False):
    """The forward pass on raw projections: prologue, OU discretisation, filter."""
    q, k, v, dt, vp = prologue_f64(xq, xk, xv, dt_raw, vp_raw, conv_w, conv_b, dtype)
    return kla_forward_ou_f64(q, k, v, dt, theta, sigma2, vp, lambda0, M0, return_lambda_path=return_lambda_path)
