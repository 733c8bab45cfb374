"""Seeded synthetic inputs for the KLA forward scan and the precision-only scan.

This module is shared by the tests, the oracle runs and the benchmark. It holds
the input *recipes* only (distributions, shapes, bf16 rounding of the values
that both sides consume); it contains none of the filter's arithmetic.

Workloads (names used throughout the repository):

  tiny_f32      B=1,  H=1,  T=256,   d_k=d_v=16,  fp32
  lm45m_bf16    B=8,  H=8,  T=2048,  d_k=d_v=64,  bf16 inputs
  lm180m_bf16   B=16, H=12, T=2048,  d_k=d_v=64,  bf16, 5% of tokens with val_prec x100
  long_bf16     B=2,  H=16, T=16384, d_k=d_v=128, bf16, long-memory decay
  chains_f32    65536 chains x T=65536 (as B=1, H=1024, D=64), fp32, precision path only
  decode_lm45m_bf16   one decode step of lm45m_bf16's heads (B=8, H=8, d=64), bf16
  decode_b256_bf16    one decode step of a batch of 256 sequences (B=256, H=8, d=64), bf16

Distributions (all draws float64, then cast):
  q, k        ~ N(0, 1/d_k)                       (variance 1/d_k)
  v           ~ N(0, 1)
  log_decay   = -softplus(N(mu_decay, 1))          mu_decay = 0, or -2 for long_bf16
  proc_noise  = softplus(N(0, 1)) + 1e-3
  val_prec    = softplus(N(0, 1)) + 1e-3           (x100 on masked tokens, lm180m_bf16)
  lambda0 = 1, M0 = 0

Seeding: seed = 1000 + workload index; one PCG64 stream per tensor from
``SeedSequence(seed).spawn(7)`` in the order q, k, v, log_decay, proc_noise,
val_prec, mask.  bf16 workloads round every input once, round-to-nearest-even,
and both the GPU path and the oracle consume exactly those rounded values.
"""
from __future__ import annotations

from dataclasses import dataclass
import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "round_bf16", "bf16_bits",
    "make_forward_inputs", "make_forward_inputs_torch", "make_precision_inputs",
    "make_precision_inputs_torch",
    "softplus",
]


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    kind: str            # "forward", "forward_ou", "forward_prologue", "forward_vprec", "precision",
                         # "decode" or "backward"
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: str           # "f32" or "bf16"
    decay_mean: float = 0.0
    spike_frac: float = 0.0
    spike_scale: float = 1.0

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def tokens(self) -> int:
        return self.B * self.H * self.T


WORKLOADS = (
    Workload(0, "tiny_f32", "forward", 1, 1, 256, 16, 16, "f32"),
    Workload(1, "lm45m_bf16", "forward", 8, 8, 2048, 64, 64, "bf16"),
    Workload(2, "lm180m_bf16", "forward", 16, 12, 2048, 64, 64, "bf16",
             spike_frac=0.05, spike_scale=100.0),
    Workload(3, "long_bf16", "forward", 2, 16, 16384, 128, 128, "bf16", decay_mean=-2.0),
    Workload(4, "chains_f32", "precision", 1, 1024, 65536, 64, 64, "f32"),
    Workload(5, "decode_lm45m_bf16", "decode", 8, 8, 1, 64, 64, "bf16"),
    Workload(6, "decode_b256_bf16", "decode", 256, 8, 1, 64, 64, "bf16"),
    Workload(7, "bwd_lm45m_bf16", "backward", 8, 8, 2048, 64, 64, "bf16"),
    Workload(8, "ou_lm45m_bf16", "forward_ou", 8, 8, 2048, 64, 64, "bf16"),
    Workload(9, "vprec_lm45m_bf16", "forward_vprec", 8, 8, 2048, 64, 64, "bf16"),
    Workload(10, "bwd_long_bf16", "backward", 2, 16, 16384, 128, 128, "bf16", decay_mean=-2.0),
    Workload(11, "pro_lm45m_bf16", "forward_prologue", 8, 8, 2048, 64, 64, "bf16"),
)


def workload(key) -> Workload:
    """Look a workload up by index or by name."""
    for w in WORKLOADS:
        if key == w.index or key == w.name:
            return w
    raise KeyError(key)


def softplus(x: np.ndarray) -> np.ndarray:
    """log(1 + e^x), evaluated without overflow."""
    return np.logaddexp(0.0, x)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float32 values, round-to-nearest-even.

    Inputs must be finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    bits = bf16_bits(x).astype(np.uint32) << 16
    return bits.view(np.float32)


def _streams(seed: int, n: int = 7):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def make_forward_inputs(w: Workload | int | str, *, B=None, H=None, T=None, dk=None, dv=None,
                        seed=None, dtype=None) -> dict:
    """Seeded inputs of a forward workload, optionally at another shape.

    Returns a dict of float32 numpy arrays (bf16-rounded when the dtype is
    bf16): q, k, log_decay, proc_noise, val_prec [B,H,T,dk]; v [B,H,T,dv];
    lambda0 [B,H,dk]; M0 [B,H,dk,dv]; plus "dtype" and "seed".
    """
    if not isinstance(w, Workload):
        w = workload(w)
    B = w.B if B is None else B
    H = w.H if H is None else H
    T = w.T if T is None else T
    dk = w.dk if dk is None else dk
    dv = w.dv if dv is None else dv
    seed = w.seed if seed is None else seed
    dtype = w.dtype if dtype is None else dtype
    rq, rk, rv, rd, rp, rl, rm = _streams(seed)
    sk = (B, H, T, dk)
    q = rq.standard_normal(sk) / np.sqrt(dk)
    k = rk.standard_normal(sk) / np.sqrt(dk)
    v = rv.standard_normal((B, H, T, dv))
    log_decay = -softplus(rd.standard_normal(sk) + w.decay_mean)
    proc_noise = softplus(rp.standard_normal(sk)) + 1e-3
    val_prec = softplus(rl.standard_normal(sk)) + 1e-3
    if w.spike_frac > 0.0:
        mask = rm.random((B, H, T)) < w.spike_frac
        val_prec = np.where(mask[..., None], val_prec * w.spike_scale, val_prec)
    out = {}
    for name, arr in (("q", q), ("k", k), ("v", v), ("log_decay", log_decay),
                      ("proc_noise", proc_noise), ("val_prec", val_prec)):
        a32 = arr.astype(np.float32)
        out[name] = round_bf16(a32) if dtype == "bf16" else a32
    out["lambda0"] = np.ones((B, H, dk), np.float32)
    out["M0"] = np.zeros((B, H, dk, dv), np.float32)
    out["dtype"] = dtype
    out["seed"] = seed
    return out


def make_precision_inputs(*, B: int, H: int, T: int, D: int, seed: int = 1004) -> dict:
    """Host-side seeded inputs of the precision-only scan (chains_f32 recipe).

    log_decay = -softplus(N(0,1)); proc_noise = softplus(N(0,1));
    obs_prec = k^2 * Lambda^v with k ~ N(0,1), Lambda^v = softplus(N(0,1)),
    formed in float32 as the recipe's input; lambda0 = 1.  All float32.
    """
    rk, rl, rd, rp = _streams(seed, 4)
    shape = (B, H, T, D)
    log_decay = (-softplus(rd.standard_normal(shape))).astype(np.float32)
    proc_noise = softplus(rp.standard_normal(shape)).astype(np.float32)
    kk = rk.standard_normal(shape).astype(np.float32)
    lv = softplus(rl.standard_normal(shape)).astype(np.float32)
    obs_prec = (kk * kk * lv).astype(np.float32)
    return {"log_decay": log_decay, "proc_noise": proc_noise, "obs_prec": obs_prec,
            "lambda0": np.ones((B, H, D), np.float32), "seed": seed}


def make_precision_inputs_torch(*, B: int, H: int, T: int, D: int, seed: int = 1004,
                                device="cuda", chunk_rows: int = 1 << 26):
    """Device-side seeded inputs of the precision-only scan, for sizes the host cannot
    generate quickly (the full chains_f32 workload is 4.3 G elements per tensor).

    Same recipe as :func:`make_precision_inputs` but drawn with torch's generator on
    ``device``; the values differ from the host version.  Tensors are float32 and
    contiguous [B,H,T,D]; generation runs in slabs to bound temporaries.
    """
    import torch
    gens = []
    for i in range(4):
        g = torch.Generator(device=device)
        g.manual_seed(seed * 16 + i)
        gens.append(g)
    shape = (B, H, T, D)
    n = B * H * T * D
    ld = torch.empty(shape, dtype=torch.float32, device=device)
    pn = torch.empty(shape, dtype=torch.float32, device=device)
    op = torch.empty(shape, dtype=torch.float32, device=device)
    fl, fp, fo = ld.view(-1), pn.view(-1), op.view(-1)
    sp = torch.nn.functional.softplus
    for s in range(0, n, chunk_rows):
        e = min(n, s + chunk_rows)
        m = e - s
        fl[s:e] = -sp(torch.randn(m, generator=gens[0], device=device))
        fp[s:e] = sp(torch.randn(m, generator=gens[1], device=device))
        kk = torch.randn(m, generator=gens[2], device=device)
        lv = sp(torch.randn(m, generator=gens[3], device=device))
        fo[s:e] = kk * kk * lv
        del kk, lv
    lam0 = torch.ones((B, H, D), dtype=torch.float32, device=device)
    return {"log_decay": ld, "proc_noise": pn, "obs_prec": op, "lambda0": lam0, "seed": seed}


def make_forward_inputs_torch(w: Workload | int | str, *, seed=None, device="cuda", dtype=None):
    """Device-side seeded inputs of a forward workload at its full shape, for
    shapes the host generates slowly (long_bf16 draws 400 M values).

    Same recipe as :func:`make_forward_inputs`, drawn with torch's generator on
    ``device`` (values differ from the host version).  Returns torch tensors in
    the workload dtype (bf16: rounded to nearest even by the cast), plus
    float32 lambda0 = 1 and M0 = 0.
    """
    import torch
    if not isinstance(w, Workload):
        w = workload(w)
    seed = w.seed if seed is None else seed
    dtype = w.dtype if dtype is None else dtype
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    gens = []
    for i in range(7):
        g = torch.Generator(device=device)
        g.manual_seed(seed * 16 + i)
        gens.append(g)
    sp = torch.nn.functional.softplus
    sk, sv = (B, H, T, dk), (B, H, T, dv)

    def rn(shape, g):
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32)

    out = {
        "q": (rn(sk, gens[0]) / dk ** 0.5).to(tdt),
        "k": (rn(sk, gens[1]) / dk ** 0.5).to(tdt),
        "v": rn(sv, gens[2]).to(tdt),
        "log_decay": (-sp(rn(sk, gens[3]) + w.decay_mean)).to(tdt),
        "proc_noise": (sp(rn(sk, gens[4])) + 1e-3).to(tdt),
    }
    vp = sp(rn(sk, gens[5])) + 1e-3
    if w.spike_frac > 0.0:
        mask = torch.rand((B, H, T), generator=gens[6], device=device) < w.spike_frac
        vp = torch.where(mask[..., None], vp * w.spike_scale, vp)
    out["val_prec"] = vp.to(tdt)
    out["lambda0"] = torch.ones((B, H, dk), dtype=torch.float32, device=device)
    out["M0"] = torch.zeros((B, H, dk, dv), dtype=torch.float32, device=device)
    out["dtype"] = dtype
    out["seed"] = seed
    return out


def make_backward_grads(*, B: int, H: int, T: int, dk: int, dv: int, seed: int, dtype: str,
                        state: bool = False) -> dict:
    """Seeded upstream gradients for the backward pass (host side).

    grad_y ~ N(0, 1) [B,H,T,dv] (bf16-rounded when the dtype is bf16); with
    ``state``, also grad_lambda_T ~ N(0, 1) [B,H,dk] and grad_M_T ~ N(0, 1)
    [B,H,dk,dv] in float32, else None for both.  One PCG64 stream per tensor,
    spawned from SeedSequence([seed, 1]) (disjoint from the forward inputs'
    streams of the same seed).
    """
    ry, rl, rm = (np.random.default_rng(s) for s in np.random.SeedSequence([seed, 1]).spawn(3))
    gy = ry.standard_normal((B, H, T, dv)).astype(np.float32)
    out = {"grad_y": round_bf16(gy) if dtype == "bf16" else gy, "grad_lambda_T": None, "grad_M_T": None}
    if state:
        out["grad_lambda_T"] = rl.standard_normal((B, H, dk)).astype(np.float32)
        out["grad_M_T"] = rm.standard_normal((B, H, dk, dv)).astype(np.float32)
    return out


def make_backward_grads_torch(w: Workload | int | str, *, seed=None, device="cuda"):
    """Device-side grad_y ~ N(0, 1) [B,H,T,dv] of a workload's full shape, in
    its dtype (torch's generator; values differ from the host version)."""
    import torch
    if not isinstance(w, Workload):
        w = workload(w)
    seed = w.seed if seed is None else seed
    g = torch.Generator(device=device)
    g.manual_seed(seed * 16 + 7)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return torch.randn((w.B, w.H, w.T, w.dv), generator=g, device=device, dtype=torch.float32).to(tdt)


def make_ou_inputs(w: Workload | int | str, *, B=None, H=None, T=None, dk=None, dv=None, seed=None,
                   dtype=None) -> dict:
    """Seeded inputs of the forward pass with the OU prior in continuous time.

    q, k ~ N(0, 1/d_k), v ~ N(0, 1), val_prec = softplus(N(0, 1)) + 1e-3 as in
    the forward recipe; the step length dt = softplus(N(0, 1)) per (b,h,t,i);
    the OU rate theta = exp(N(0, 0.25^2)) and diffusion sigma2 =
    softplus(N(0, 1)) + 1e-3 per (h,i), float32.  With theta near 1 the
    per-token log decays -theta dt have the scale of the forward recipe's
    -softplus(N(0, 1)).  Per-token arrays are float32
    numpy arrays (bf16-rounded for bf16); lambda0 = 1, M0 = 0.  Streams: those
    of make_forward_inputs, with the log_decay stream drawing dt and the
    proc_noise stream drawing (theta, sigma2).
    """
    if not isinstance(w, Workload):
        w = workload(w)
    B = w.B if B is None else B
    H = w.H if H is None else H
    T = w.T if T is None else T
    dk = w.dk if dk is None else dk
    dv = w.dv if dv is None else dv
    seed = w.seed if seed is None else seed
    dtype = w.dtype if dtype is None else dtype
    rq, rk, rv, rd, rp, rl, _ = _streams(seed)
    sk = (B, H, T, dk)
    arrs = {"q": rq.standard_normal(sk) / np.sqrt(dk), "k": rk.standard_normal(sk) / np.sqrt(dk),
            "v": rv.standard_normal((B, H, T, dv)), "dt": softplus(rd.standard_normal(sk)),
            "val_prec": softplus(rl.standard_normal(sk)) + 1e-3}
    par = rp.standard_normal((2, H, dk))
    out = {}
    for name, arr in arrs.items():
        a32 = arr.astype(np.float32)
        out[name] = round_bf16(a32) if dtype == "bf16" else a32
    out["theta"] = np.exp(0.25 * par[0]).astype(np.float32)
    out["sigma2"] = (softplus(par[1]) + 1e-3).astype(np.float32)
    out["lambda0"] = np.ones((B, H, dk), np.float32)
    out["M0"] = np.zeros((B, H, dk, dv), np.float32)
    out["dtype"] = dtype
    out["seed"] = seed
    return out


def make_ou_inputs_torch(w: Workload | int | str, *, seed=None, device="cuda"):
    """Device-side version of make_ou_inputs at the workload's full shape
    (torch's generator; values differ from the host version)."""
    import torch
    if not isinstance(w, Workload):
        w = workload(w)
    seed = w.seed if seed is None else seed
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    gens = []
    for i in range(6):
        g = torch.Generator(device=device)
        g.manual_seed(seed * 16 + i)
        gens.append(g)
    sp = torch.nn.functional.softplus
    rn = lambda shape, g: torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    sk = (B, H, T, dk)
    return {
        "q": (rn(sk, gens[0]) / dk ** 0.5).to(tdt),
        "k": (rn(sk, gens[1]) / dk ** 0.5).to(tdt),
        "v": rn((B, H, T, dv), gens[2]).to(tdt),
        "dt": sp(rn(sk, gens[3])).to(tdt),
        "theta": torch.exp(0.25 * rn((H, dk), gens[4])),
        "sigma2": sp(rn((H, dk), gens[4])) + 1e-3,
        "val_prec": (sp(rn(sk, gens[5])) + 1e-3).to(tdt),
        "lambda0": torch.ones((B, H, dk), dtype=torch.float32, device=device),
        "M0": torch.zeros((B, H, dk, dv), dtype=torch.float32, device=device),
        "dtype": w.dtype, "seed": seed,
    }


def make_vprec_inputs(w: Workload | int | str, *, B=None, H=None, T=None, dk=None, dv=None, seed=None,
                      dtype=None) -> dict:
    """Seeded inputs of the variant with the value precision per value
    channel: the forward recipe, except val_prec = softplus(N(0, 1)) + 1e-3
    drawn with shape [B,H,T,dv] (from the same stream); lambda0 = 1 and M0 = 0
    as [B,H,dk,dv]."""
    if not isinstance(w, Workload):
        w = workload(w)
    x = make_forward_inputs(w, B=B, H=H, T=T, dk=dk, dv=dv, seed=seed, dtype=dtype)
    B, H, T, dk = x["k"].shape
    dv = x["v"].shape[-1]
    rl = _streams(x["seed"])[5]
    vp = (softplus(rl.standard_normal((B, H, T, dv))) + 1e-3).astype(np.float32)
    x["val_prec"] = round_bf16(vp) if x["dtype"] == "bf16" else vp
    x["lambda0"] = np.ones((B, H, dk, dv), np.float32)
    x["M0"] = np.zeros((B, H, dk, dv), np.float32)
    return x


def make_vprec_inputs_torch(w: Workload | int | str, *, seed=None, device="cuda"):
    """Device-side version of make_vprec_inputs at the workload's full shape."""
    import torch
    if not isinstance(w, Workload):
        w = workload(w)
    x = make_forward_inputs_torch(w, seed=seed, device=device)
    g = torch.Generator(device=device)
    g.manual_seed((w.seed if seed is None else seed) * 16 + 8)
    tdt = x["q"].dtype
    x["val_prec"] = (torch.nn.functional.softplus(torch.randn((w.B, w.H, w.T, w.dv), generator=g, device=device))
                     + 1e-3).to(tdt)
    x["lambda0"] = None
    x["M0"] = None
    return x


def make_prologue_inputs(w: Workload | int | str, *, B=None, H=None, T=None, dk=None, dv=None, seed=None,
                         dtype=None, conv_width=4, bias=True) -> dict:
    """Seeded inputs of the forward pass on raw projections (coefficient
    prologue: causal conv1d + SiLU on q, k, v; softplus on the step length and
    the value precision; OU prior).

    Raw projections xq, xk, xv ~ N(0, 1); dt_raw, vp_raw ~ N(0, 1) (so dt and
    val_prec are softplus(N(0, 1)), the OU recipe's distribution); theta =
    exp(N(0, 0.25^2)) and sigma2 = softplus(N(0, 1)) + 1e-3 per (h,i) as the
    OU recipe; convolution taps and biases ~ U(-1/sqrt(W), 1/sqrt(W)) per
    (h, channel) (the default initialisation of a depthwise torch Conv1d), as
    float32 [H,d,W] and [H,d].  Per-token arrays are float32 numpy arrays
    (bf16-rounded for bf16); lambda0 = 1, M0 = 0.  Streams: those of
    make_forward_inputs (q, k, v, log_decay -> dt_raw, proc_noise -> theta,
    sigma2, val_prec -> vp_raw, mask -> convolution parameters).
    """
    if not isinstance(w, Workload):
        w = workload(w)
    B = w.B if B is None else B
    H = w.H if H is None else H
    T = w.T if T is None else T
    dk = w.dk if dk is None else dk
    dv = w.dv if dv is None else dv
    seed = w.seed if seed is None else seed
    dtype = w.dtype if dtype is None else dtype
    rq, rk, rv, rd, rp, rl, rc = _streams(seed)
    sk = (B, H, T, dk)
    arrs = {"xq": rq.standard_normal(sk), "xk": rk.standard_normal(sk), "xv": rv.standard_normal((B, H, T, dv)),
            "dt_raw": rd.standard_normal(sk), "vp_raw": rl.standard_normal(sk)}
    out = {}
    for name, arr in arrs.items():
        a32 = arr.astype(np.float32)
        out[name] = round_bf16(a32) if dtype == "bf16" else a32
    par = rp.standard_normal((2, H, dk))
    out["theta"] = np.exp(0.25 * par[0]).astype(np.float32)
    out["sigma2"] = (softplus(par[1]) + 1e-3).astype(np.float32)
    bound = 1.0 / np.sqrt(conv_width)
    out["conv_w"] = tuple(rc.uniform(-bound, bound, (H, d, conv_width)).astype(np.float32) for d in (dk, dk, dv))
    cb = tuple(rc.uniform(-bound, bound, (H, d)).astype(np.float32) for d in (dk, dk, dv))
    out["conv_b"] = cb if bias else (None, None, None)
    out["lambda0"] = np.ones((B, H, dk), np.float32)
    out["M0"] = np.zeros((B, H, dk, dv), np.float32)
    out["dtype"] = dtype
    out["seed"] = seed
    return out


def make_prologue_inputs_torch(w: Workload | int | str, *, seed=None, device="cuda", conv_width=4):
    """Device-side version of make_prologue_inputs at the workload's full shape
    (torch's generator; values differ from the host version)."""
    import torch
    if not isinstance(w, Workload):
        w = workload(w)
    seed = w.seed if seed is None else seed
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    gens = []
    for i in range(7):
        g = torch.Generator(device=device)
        g.manual_seed(seed * 16 + i)
        gens.append(g)
    sp = torch.nn.functional.softplus
    rn = lambda shape, g: torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    bound = 1.0 / conv_width ** 0.5
    ru = lambda shape, g: (torch.rand(shape, generator=g, device=device, dtype=torch.float32) * 2 - 1) * bound
    sk = (B, H, T, dk)
    return {
        "xq": rn(sk, gens[0]).to(tdt), "xk": rn(sk, gens[1]).to(tdt), "xv": rn((B, H, T, dv), gens[2]).to(tdt),
        "dt_raw": rn(sk, gens[3]).to(tdt),
        "theta": torch.exp(0.25 * rn((H, dk), gens[4])),
        "sigma2": sp(rn((H, dk), gens[4])) + 1e-3,
        "vp_raw": rn(sk, gens[5]).to(tdt),
        "conv_w": tuple(ru((H, d, conv_width), gens[6]) for d in (dk, dk, dv)),
        "conv_b": tuple(ru((H, d), gens[6]) for d in (dk, dk, dv)),
        "lambda0": torch.ones((B, H, dk), dtype=torch.float32, device=device),
        "M0": torch.zeros((B, H, dk, dv), dtype=torch.float32, device=device),
        "dtype": w.dtype, "seed": seed,
    }
