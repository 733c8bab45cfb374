"""Helpers shared by the GPU parity tests: device transfer, oracle runs and the
tolerance checks the parity bar uses.

Tolerances (float64 oracle as reference r, GPU result x):
  fp32 inputs:  precision  |x - r| <= 1e-5 |r| + FLT_MIN
                y, M_T     |x - r| <= 1e-5 max(|r|, rms of r over the head) + FLT_MIN
                (y is a dot product that can cancel towards 0; the per-head RMS
                floor keeps the bound relative to the head's output scale;
                FLT_MIN = 1.18e-38 covers results below the fp32 normal range)
  bf16 inputs:  |x - r| <= 1e-2 + 2e-2 |r| for y, lambda_T and M_T
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import kla_forward_f64, precision_scan_f64

F32_REL = 1e-5
F32_TINY = float(np.finfo(np.float32).tiny)  # 1.18e-38, smallest normal fp32
BF16_ABS, BF16_REL = 1e-2, 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x: dict, names=("q", "k", "v", "log_decay", "proc_noise", "val_prec")):
    import torch
    dt = torch.bfloat16 if x["dtype"] == "bf16" else torch.float32
    out = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to("cuda").to(dt) for n in names}
    for n in ("lambda0", "M0"):
        if n in x and x[n] is not None:
            out[n] = torch.from_numpy(np.ascontiguousarray(x[n], np.float32)).to("cuda")
    return out


def gpu_forward(xd: dict, return_lambda_path=False, lambda0=True, M0=True, **kw):
    import torch
    import bius_scan_sequence_amd as K
    res = K.forward(xd["q"], xd["k"], xd["v"], xd["log_decay"], xd["proc_noise"], xd["val_prec"],
                    xd.get("lambda0") if lambda0 else None, xd.get("M0") if M0 else None,
                    return_lambda_path=return_lambda_path, **kw)
    torch.cuda.synchronize()
    return tuple(t.float().cpu().numpy() for t in res)


def oracle_forward(x: dict, return_lambda_path=False):
    return kla_forward_f64(x["q"], x["k"], x["v"], x["log_decay"], x["proc_noise"], x["val_prec"],
                           x.get("lambda0"), x.get("M0"), return_lambda_path=return_lambda_path)


def head_rms(r: np.ndarray, nbatch_axes=2) -> np.ndarray:
    axes = tuple(range(nbatch_axes, r.ndim))
    rms = np.sqrt(np.mean(r * r, axis=axes, keepdims=True))
    return np.broadcast_to(rms, r.shape)


def check_f32(name, x, r, per_head_floor: bool):
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    assert x.shape == r.shape, (name, x.shape, r.shape)
    assert np.all(np.isfinite(x)), f"{name}: non-finite output"
    scale = np.maximum(np.abs(r), head_rms(r)) if per_head_floor else np.abs(r)
    # Results below the fp32 normal range (e.g. a state decayed to 1e-98) have
    # no fp32 representation: differences up to FLT_MIN are not counted.
    err = np.maximum(np.abs(x - r) - F32_TINY, 0.0) / np.maximum(scale, 1e-300)
    worst = np.unravel_index(np.argmax(err), err.shape) if err.size else None
    assert err.size == 0 or err.max() <= F32_REL, (
        f"{name}: max scaled error {err.max():.3e} at {worst}: got {x[worst]}, want {r[worst]}")
    return float(err.max()) if err.size else 0.0


def check_bf16(name, x, r):
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    assert x.shape == r.shape, (name, x.shape, r.shape)
    assert np.all(np.isfinite(x)), f"{name}: non-finite output"
    bound = BF16_ABS + BF16_REL * np.abs(r)
    viol = np.abs(x - r) / bound
    worst = np.unravel_index(np.argmax(viol), viol.shape) if viol.size else None
    assert viol.size == 0 or viol.max() <= 1.0, (
        f"{name}: |x-r| reaches {viol.max():.3f} of the bound at {worst}: got {x[worst]}, want {r[worst]}")
    return float(viol.max()) if viol.size else 0.0


def normwise(x, r):
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    return float(np.linalg.norm(x - r) / max(np.linalg.norm(r), 1e-300))


def check_forward(x: dict, got, ref, dtype: str, exact_coeffs: bool = True):
    """Compare (y, lambda_T, M_T[, lambda_path]) against the oracle.

    y and M_T use the dtype's bar.  The precision outputs are held to the fp32
    bar for both dtypes when the scan runs in fp32 on exactly the
    (bf16-rounded) coefficients the oracle sees (exact_coeffs), so that
    nothing but fp32 rounding separates them; for bf16 inputs the bf16 bar is
    checked as well.  Without exact_coeffs (coefficients the kernel forms and
    rounds to bf16 itself, which can round apart from the float64 ones at a
    rounding midpoint) bf16 precision outputs get the bf16 bar only.
    """
    names = ("y", "lambda_T", "M_T", "lambda_path")[: len(ref)]
    stats = {}
    for n, g, r in zip(names, got, ref):
        if n in ("lambda_T", "lambda_path") and dtype == "bf16" and not exact_coeffs:
            stats[n] = check_bf16(n, g, r)
        elif n in ("lambda_T", "lambda_path"):
            stats[n] = check_f32(n, g, r, per_head_floor=False)
            if dtype == "bf16":
                check_bf16(n, g, r)
        elif dtype == "f32":
            stats[n] = check_f32(n, g, r, per_head_floor=True)
        else:
            stats[n] = check_bf16(n, g, r)
        stats[n + "_normwise"] = normwise(g, r)
    return stats


def precision_oracle(ld, pn, c, lam0=None):
    return precision_scan_f64(ld, pn, c, lam0)
