"""Plain, sequential float64 oracle of the KLA forward scan.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the CPU
baseline of the benchmark, never by the product path.

Sources (gist.science summaries of arXiv 2602.10743, "Kalman Linear Attention"):
  [KLA-nl] "Technische Samenvatting: Kalman Linear Attention (KLA)"
           (gist.science/nl/paper/2602.10743)
  [KLA-de] "Kalman Linear Attention: Parallel Bayesian Filtering For Efficient
           Language Modelling and State Tracking" (gist.science/de/paper/2602.10743),
           section "Technisches Resümee"

What is computed.  The pages define KLA as *exact* Bayesian filtering in a
linear-Gaussian state-space model ([KLA-nl] "Methodologie"; "Belangrijkste
Bijdragen" item 1: diagonal linear-Gaussian Kalman filtering).  The parallel
Möbius scan reaches exactly (up to rounding order) the result of the plain
sequential filter, so this oracle is that filter written out, one scalar filter
per state element (b, h, i, j), vectorised over the independent elements and
looped over time:

  latent      x_t = a_t x_{t-1} + w_t,   w_t ~ N(0, pbar_t)
              (exactly discretised OU prior; [KLA-nl] §1 "Dynamics Prior")
  observation v_{t,j} = k_{t,i} x_{t,ij} + e,  e with precision Lambda^v_{t,i}
              ([KLA-nl] §1 "Observatiemodel")
  readout     y_{t,j} = sum_i q_{t,i} mu_{t,ij}, mu the posterior mean
              ([KLA-nl] §1 "Readout")
  prior       x_{0,ij} ~ N(M0[i,j], 1/lambda0[i])

The pages leave the OU discretisation, the order of predict/update and the
coefficients of the Möbius map open; readings taken here (documented with the
design):
  * inputs arrive discretised: a_t = exp(log_decay_t), pbar_t = proc_noise_t
    (a variance);
  * each step predicts, then updates; (lambda0, M0) is the posterior before the
    first token;
  * precision depends on (b, h, t, i) only and is shared over j; Lambda^v is
    indexed like k;
  * the readout uses the posterior (filtering) mean that includes token t.

No blocking, chunking, normalisation or reordering is applied: every step is
the textbook scalar predict/update in float64.  The step functions are
module-level so that tests can plant a mistake in one of them and show that a
pin catches it.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "predict_precision", "update_precision", "forget_gate", "write_gate", "readout",
    "filter_step", "kla_forward_f64", "kla_decode_step_f64", "precision_scan_f64",
    "precision_path_from_coeffs",
]


# --------------------------------------------------------------------------- #
# One filter step, in the information (precision) form.                        #
# Written with + - * / only, so the same functions run on float64 arrays and   #
# on exact rationals (fractions.Fraction) in the tests.                        #
# --------------------------------------------------------------------------- #

def predict_precision(lam, a, pbar):
    """Prior precision after the OU transition.

    Variance form: P^- = a^2 P + pbar with P = 1/lam, so
    lam^- = 1/P^- = lam / (a^2 + pbar * lam).
    ([KLA-nl] §1 "Dynamics Prior": the exactly discretised OU step decays the
    mean by a, the variance by a^2, and adds the process noise pbar.)
    """
    return lam / (a * a + pbar * lam)


def update_precision(lam_pred, c):
    """Posterior precision after observing a token: lam = lam^- + c, with the
    observation precision c = k^2 * Lambda^v ([KLA-nl] §1 "Observatiemodel").

    Composed with predict_precision this is the Möbius map of [KLA-nl] §2
    "Parallelisatie via Möbius-transformaties" (precision equation), with
    alpha = 1 + c*pbar, beta = c*a^2, gamma = pbar, delta = a^2.
    """
    return lam_pred + c


def forget_gate(a, lam_pred, lam):
    """Weight of the previous posterior mean: f = a * lam^- / lam.

    The posterior mean is the precision-weighted average of the predicted mean
    a*mu and the token evidence; the weight of the prediction is a ratio of
    precisions ([KLA-nl] §3 "Niet-lineaire Gating vanuit Onzekerheid").
    """
    return a * lam_pred / lam


def write_gate(k, val_prec, lam):
    """Weight of the token value: g = k * Lambda^v / lam ([KLA-nl] §3)."""
    return k * val_prec / lam


def readout(q_t, M):
    """y_t[j] = sum_i q_t[i] * M[i, j] over the posterior mean ([KLA-nl] §1 "Readout").

    q_t: [..., dk], M: [..., dk, dv] -> [..., dv].
    """
    return np.einsum("...i,...ij->...j", q_t, M)


def filter_step(q_t, k_t, v_t, log_decay_t, proc_noise_t, val_prec_t, lam, M):
    """One token of every filter: predict, update, gates, mean update, readout.

    Shapes: q_t, k_t, log_decay_t, proc_noise_t, val_prec_t, lam [..., dk];
    v_t [..., dv]; M [..., dk, dv].  Returns (y_t [..., dv], lam_t [..., dk],
    M_t [..., dk, dv], f [..., dk], g [..., dk]).

    The mean follows the affine recursion M_t = f M_{t-1} + g v_t ([KLA-nl] §2,
    the posterior-mean recursion) with the precision-ratio gates of §3.
    """
    a = np.exp(log_decay_t)
    lam_pred = predict_precision(lam, a, proc_noise_t)
    lam_new = update_precision(lam_pred, k_t * k_t * val_prec_t)
    f = forget_gate(a, lam_pred, lam_new)
    g = write_gate(k_t, val_prec_t, lam_new)
    M_new = f[..., None] * M + g[..., None] * v_t[..., None, :]
    return readout(q_t, M_new), lam_new, M_new, f, g


# --------------------------------------------------------------------------- #
# Full forward pass.                                                           #
# --------------------------------------------------------------------------- #

def kla_forward_f64(q, k, v, log_decay, proc_noise, val_prec, lambda0=None, M0=None,
                    return_lambda_path=False, return_gates=False):
    """Sequential float64 KLA forward pass.

    Shapes: q, k, log_decay, proc_noise, val_prec [B,H,T,dk]; v [B,H,T,dv];
    lambda0 [B,H,dk] (default 1); M0 [B,H,dk,dv] (default 0).

    Returns (y [B,H,T,dv], lambda_T [B,H,dk], M_T [B,H,dk,dv]) in float64, then
    the precision path [B,H,T,dk] if ``return_lambda_path`` and the gates
    (f, g) [B,H,T,dk] each if ``return_gates``.

    T = 0 returns (lambda0, M0) unchanged with an empty y.  Raises ValueError on
    non-finite inputs or a non-positive lambda0.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    ld = np.asarray(log_decay, np.float64)
    pn = np.asarray(proc_noise, np.float64)
    vp = np.asarray(val_prec, np.float64)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    for name, arr, shp in (("q", q, (B, H, T, dk)), ("log_decay", ld, (B, H, T, dk)),
                           ("proc_noise", pn, (B, H, T, dk)), ("val_prec", vp, (B, H, T, dk)),
                           ("v", v, (B, H, T, dv))):
        if arr.shape != shp:
            raise ValueError(f"{name} has shape {arr.shape}, expected {shp}")
    lam = np.ones((B, H, dk)) if lambda0 is None else np.array(lambda0, np.float64)
    M = np.zeros((B, H, dk, dv)) if M0 is None else np.array(M0, np.float64)
    if lam.shape != (B, H, dk) or M.shape != (B, H, dk, dv):
        raise ValueError("lambda0/M0 shape mismatch")
    for name, arr in (("q", q), ("k", k), ("v", v), ("log_decay", ld), ("proc_noise", pn),
                      ("val_prec", vp), ("lambda0", lam), ("M0", M)):
        if not np.all(np.isfinite(arr)):
            raise ValueError(f"{name} has non-finite entries")
    if np.any(lam <= 0):
        raise ValueError("lambda0 must be positive")

    y = np.empty((B, H, T, dv))
    lam_path = np.empty((B, H, T, dk)) if return_lambda_path else None
    f_path = np.empty((B, H, T, dk)) if return_gates else None
    g_path = np.empty((B, H, T, dk)) if return_gates else None
    for t in range(T):
        y[:, :, t], lam, M, f, g = filter_step(q[:, :, t], k[:, :, t], v[:, :, t], ld[:, :, t],
                                               pn[:, :, t], vp[:, :, t], lam, M)
        if return_lambda_path:
            lam_path[:, :, t] = lam
        if return_gates:
            f_path[:, :, t] = f
            g_path[:, :, t] = g
    out = (y, lam, M)
    if return_lambda_path:
        out = out + (lam_path,)
    if return_gates:
        out = out + (f_path, g_path)
    return out


# --------------------------------------------------------------------------- #
# Decode: one token per head.                                                  #
# --------------------------------------------------------------------------- #

def kla_decode_step_f64(q, k, v, log_decay, proc_noise, val_prec, lam, M):
    """One filter step per head, from the state (lam, M) before the token.

    Shapes: q, k, log_decay, proc_noise, val_prec [B,H,dk]; v [B,H,dv];
    lam [B,H,dk]; M [B,H,dk,dv].  Returns (y [B,H,dv], lam_new [B,H,dk],
    M_new [B,H,dk,dv]) in float64: the same step the forward pass takes for
    every token, so T decode steps from (lambda0, M0) reproduce a forward pass
    over T tokens.  Raises ValueError on shape mismatches, non-finite inputs or
    a non-positive lam.
    """
    arrs = {n: np.asarray(x, np.float64) for n, x in (("q", q), ("k", k), ("v", v), ("log_decay", log_decay),
                                                       ("proc_noise", proc_noise), ("val_prec", val_prec),
                                                       ("lam", lam), ("M", M))}
    B, H, dk = arrs["k"].shape
    dv = arrs["v"].shape[-1]
    want = {"q": (B, H, dk), "log_decay": (B, H, dk), "proc_noise": (B, H, dk), "val_prec": (B, H, dk),
            "v": (B, H, dv), "lam": (B, H, dk), "M": (B, H, dk, dv)}
    for n, shp in want.items():
        if arrs[n].shape != shp:
            raise ValueError(f"{n} has shape {arrs[n].shape}, expected {shp}")
    for n, x in arrs.items():
        if not np.all(np.isfinite(x)):
            raise ValueError(f"{n} has non-finite entries")
    if np.any(arrs["lam"] <= 0):
        raise ValueError("lam must be positive")
    y, lam_new, M_new, _, _ = filter_step(arrs["q"], arrs["k"], arrs["v"], arrs["log_decay"],
                                          arrs["proc_noise"], arrs["val_prec"], arrs["lam"], arrs["M"])
    return y, lam_new, M_new


# --------------------------------------------------------------------------- #
# Precision path only.                                                         #
# --------------------------------------------------------------------------- #

def precision_path_from_coeffs(a, pbar, c, lam0):
    """Precision path of one filter from already-formed coefficients.

    a, pbar, c: sequences of length T (any numeric type supporting + * /, e.g.
    float64 arrays with trailing chain axes, or fractions.Fraction); lam0 the
    starting precision.  Returns the list [lam_1, ..., lam_T].  Used by the
    exact-arithmetic pins; the float path below runs the same steps.
    """
    out = []
    lam = lam0
    for t in range(len(a)):
        lam = update_precision(predict_precision(lam, a[t], pbar[t]), c[t])
        out.append(lam)
    return out


def precision_scan_f64(log_decay, proc_noise, obs_prec, lambda0=None):
    """Precision-only filter: lambda path of independent chains.

    Inputs [B,H,T,D] (log_decay, proc_noise, obs_prec c = k^2 Lambda^v),
    lambda0 [B,H,D] (default 1).  Each chain runs
    lam_t = predict(lam_{t-1}) + c_t ([KLA-nl] §2, precision equation).
    Returns (lambda_path [B,H,T,D], lambda_T [B,H,D]) in float64.
    """
    ld = np.asarray(log_decay, np.float64)
    pn = np.asarray(proc_noise, np.float64)
    c = np.asarray(obs_prec, np.float64)
    B, H, T, D = ld.shape
    if pn.shape != ld.shape or c.shape != ld.shape:
        raise ValueError("coefficient shapes differ")
    lam = np.ones((B, H, D)) if lambda0 is None else np.array(lambda0, np.float64)
    if lam.shape != (B, H, D):
        raise ValueError("lambda0 shape mismatch")
    if np.any(lam <= 0) or not (np.all(np.isfinite(ld)) and np.all(np.isfinite(pn))
                                and np.all(np.isfinite(c)) and np.all(np.isfinite(lam))):
        raise ValueError("non-finite input or non-positive lambda0")
    path = np.empty((B, H, T, D))
    for t in range(T):
        lam = update_precision(predict_precision(lam, np.exp(ld[:, :, t]), pn[:, :, t]), c[:, :, t])
        path[:, :, t] = lam
    return path, lam
