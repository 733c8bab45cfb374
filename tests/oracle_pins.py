"""Pins of the float64 oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function raises AssertionError (or any exception) when the oracle
disagrees with an independent statement of what the filter computes:

  * the covariance-form Kalman filter (a textbook derivation other than the
    information form the oracle uses);
  * Gaussian conditioning of the dense joint distribution of (x_0..x_T, v_1..v_t);
  * exact rational composition of 2x2 projective matrices (the Möbius-map
    reading of the precision recursion) against the oracle's step functions;
  * closed forms of special cases (no observation, no process noise, the
    recursive-least-squares limit, the steady-state DARE root);
  * invariants: positivity and the OU bounds of the precision, monotonicity in
    lambda0, gate ranges, independence of the precision from q/v/M0,
    linearity of y;
  * state carry: two calls with the state passed on equal one call.

Sources: gist.science "Technische Samenvatting: Kalman Linear Attention (KLA)"
(arXiv 2602.10743 summary), §1 "Probabilistische Formulering", §2
"Parallelisatie via Möbius-transformaties" (precision equation), §3
"Niet-lineaire Gating vanuit Onzekerheid".

The functions look the oracle up at call time so that tests can plant a
mistake in one of its step functions and check that some pin fails.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import oracle.kla_f64 as O


def _rand_inputs(rng, B=2, H=1, T=24, dk=3, dv=2, scale_c=1.0):
    q = rng.standard_normal((B, H, T, dk)) / np.sqrt(dk)
    k = rng.standard_normal((B, H, T, dk)) * scale_c
    v = rng.standard_normal((B, H, T, dv))
    ld = -np.logaddexp(0.0, rng.standard_normal((B, H, T, dk)))
    pn = np.logaddexp(0.0, rng.standard_normal((B, H, T, dk))) + 1e-3
    vp = np.logaddexp(0.0, rng.standard_normal((B, H, T, dk))) + 1e-3
    lam0 = 0.5 + rng.random((B, H, dk))
    M0 = rng.standard_normal((B, H, dk, dv))
    return q, k, v, ld, pn, vp, lam0, M0


# --------------------------------------------------------------------------- #
# 1. covariance-form Kalman filter                                             #
# --------------------------------------------------------------------------- #

def covariance_form_filter(q, k, v, ld, pn, vp, lam0, M0):
    """Textbook Kalman filter in (mean, variance) form, per element (b,h,i,j).

    predict: m^- = a m,  P^- = a^2 P + pbar
    update:  S = k^2 P^- + 1/Lambda,  K = P^- k / S,
             m = m^- + K (v - k m^-),  P = (1 - K k) P^-
    """
    B, H, T, dk = k.shape
    P = 1.0 / lam0
    m = M0.copy()
    y = np.empty(v.shape[:3] + (v.shape[-1],))
    lam_path = np.empty(k.shape)
    for t in range(T):
        a = np.exp(ld[:, :, t])
        Pp = a * a * P + pn[:, :, t]
        mp = a[..., None] * m
        kt = k[:, :, t]
        S = kt * kt * Pp + 1.0 / vp[:, :, t]
        K = Pp * kt / S
        m = mp + K[..., None] * (v[:, :, t, None, :] - kt[..., None] * mp)
        P = (1.0 - K * kt) * Pp
        y[:, :, t] = np.einsum("bhi,bhij->bhj", q[:, :, t], m)
        lam_path[:, :, t] = 1.0 / P
    return y, 1.0 / P, m, lam_path


def pin_covariance_form(seed=11):
    rng = np.random.default_rng(seed)
    args = _rand_inputs(rng, B=2, H=2, T=40, dk=3, dv=5)
    y, lT, MT, path = O.kla_forward_f64(*args, return_lambda_path=True)
    y2, lT2, MT2, path2 = covariance_form_filter(*args)
    np.testing.assert_allclose(path, path2, rtol=1e-11, atol=0)
    np.testing.assert_allclose(lT, lT2, rtol=1e-11, atol=0)
    np.testing.assert_allclose(MT, MT2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(y, y2, rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------- #
# 2. dense joint Gaussian conditioning                                         #
# --------------------------------------------------------------------------- #

def dense_posterior(a, pbar, kk, lv, vv, lam0, m0):
    """Posterior mean and precision of x_t given v_1..v_t for one scalar element,
    by conditioning the dense joint Gaussian (numpy.linalg.solve).

    x_0 ~ N(m0, 1/lam0);  x_t = a_t x_{t-1} + w_t, w_t ~ N(0, pbar_t);
    v_t = k_t x_t + e_t, e_t ~ N(0, 1/lv_t).  Returns (means[T], precisions[T]).
    """
    T = len(a)
    # x = G @ z with z = (x_0, w_1..w_T) independent, Cov(z) = diag(1/lam0, pbar)
    G = np.zeros((T + 1, T + 1))
    for t in range(T + 1):
        for u in range(t + 1):
            G[t, u] = np.prod(a[u:t])  # product a_{u+1}..a_t (index shift: a[0] is a_1)
    Cz = np.diag(np.concatenate([[1.0 / lam0], pbar]))
    Cx = G @ Cz @ G.T
    mx = G[:, 0] * m0
    means, precs = np.empty(T), np.empty(T)
    for t in range(1, T + 1):
        Kmat = np.zeros((t, T + 1))
        for s in range(1, t + 1):
            Kmat[s - 1, s] = kk[s - 1]
        Cv = Kmat @ Cx @ Kmat.T + np.diag(1.0 / lv[:t])
        Cxv = Cx[t] @ Kmat.T
        mv = Kmat @ mx
        sol = np.linalg.solve(Cv, np.asarray(vv[:t]) - mv)
        means[t - 1] = mx[t] + Cxv @ sol
        var = Cx[t, t] - Cxv @ np.linalg.solve(Cv, Cxv)
        precs[t - 1] = 1.0 / var
    return means, precs


def pin_dense_gaussian(seed=5):
    rng = np.random.default_rng(seed)
    B, H, T, dk, dv = 1, 1, 7, 3, 2
    q, k, v, ld, pn, vp, lam0, M0 = _rand_inputs(rng, B, H, T, dk, dv)
    # readout of single elements: q = e_i reads row i of the posterior mean
    for i in range(dk):
        qi = np.zeros_like(q)
        qi[..., i] = 1.0
        y, lT, MT, path = O.kla_forward_f64(qi, k, v, ld, pn, vp, lam0, M0, return_lambda_path=True)
        for j in range(dv):
            mu, pr = dense_posterior(np.exp(ld[0, 0, :, i]), pn[0, 0, :, i], k[0, 0, :, i],
                                     vp[0, 0, :, i], v[0, 0, :, j], lam0[0, 0, i], M0[0, 0, i, j])
            np.testing.assert_allclose(y[0, 0, :, j], mu, rtol=1e-9, atol=1e-11)
            np.testing.assert_allclose(path[0, 0, :, i], pr, rtol=1e-9)
            np.testing.assert_allclose(MT[0, 0, i, j], mu[-1], rtol=1e-9, atol=1e-11)
    # general readout: y_t = sum_i q_{t,i} mu_{t,ij}
    y, _, _ = O.kla_forward_f64(q, k, v, ld, pn, vp, lam0, M0)
    mus = np.empty((T, dk, dv))
    for i in range(dk):
        for j in range(dv):
            mus[:, i, j] = dense_posterior(np.exp(ld[0, 0, :, i]), pn[0, 0, :, i], k[0, 0, :, i],
                                           vp[0, 0, :, i], v[0, 0, :, j], lam0[0, 0, i],
                                           M0[0, 0, i, j])[0]
    yref = np.einsum("ti,tij->tj", q[0, 0], mus)
    np.testing.assert_allclose(y[0, 0], yref, rtol=1e-9, atol=1e-11)


# --------------------------------------------------------------------------- #
# 3. exact 2x2 projective composition (Möbius map)                             #
# --------------------------------------------------------------------------- #

def mat_mul(A, B):
    return [[A[0][0] * B[0][0] + A[0][1] * B[1][0], A[0][0] * B[0][1] + A[0][1] * B[1][1]],
            [A[1][0] * B[0][0] + A[1][1] * B[1][0], A[1][0] * B[0][1] + A[1][1] * B[1][1]]]


def step_matrix(a, pbar, c):
    """2x2 matrix of one predict-then-update step acting on [lambda; 1]:
    predict = [[1, 0], [pbar, a^2]]  (lambda -> lambda / (pbar*lambda + a^2)),
    update  = [[1, c], [0, 1]]       (lambda -> lambda + c).
    """
    return mat_mul([[1, c], [0, 1]], [[1, 0], [pbar, a * a]])


def pin_mobius_exact(seed=3, T=12):
    rng = np.random.default_rng(seed)
    a = [Fraction(int(rng.integers(1, 20)), 20) for _ in range(T)]
    pb = [Fraction(int(rng.integers(1, 50)), int(rng.integers(1, 9))) for _ in range(T)]
    c = [Fraction(int(rng.integers(0, 30)), int(rng.integers(1, 7))) for _ in range(T)]
    lam0 = Fraction(7, 3)
    path = O.precision_path_from_coeffs(a, pb, c, lam0)
    P = [[Fraction(1), Fraction(0)], [Fraction(0), Fraction(1)]]
    for t in range(T):
        P = mat_mul(step_matrix(a[t], pb[t], c[t]), P)
        num = P[0][0] * lam0 + P[0][1]
        den = P[1][0] * lam0 + P[1][1]
        assert path[t] == num / den, (t, path[t], num / den)


def pin_mobius_mpmath(seed=4, T=64):
    """Float64 oracle vs 60-digit composition of the 2x2 step matrices."""
    import mpmath
    mpmath.mp.dps = 60
    rng = np.random.default_rng(seed)
    ld = -np.logaddexp(0.0, rng.standard_normal(T))
    pn = np.logaddexp(0.0, rng.standard_normal(T)) + 1e-3
    kk = rng.standard_normal(T) / 4
    vp = np.logaddexp(0.0, rng.standard_normal(T)) + 1e-3
    lam0 = 1.0
    y, lT, MT, path = O.kla_forward_f64(np.zeros((1, 1, T, 1)), kk.reshape(1, 1, T, 1),
                                         np.zeros((1, 1, T, 1)), ld.reshape(1, 1, T, 1),
                                         pn.reshape(1, 1, T, 1), vp.reshape(1, 1, T, 1),
                                         np.full((1, 1, 1), lam0), return_lambda_path=True)
    P = [[mpmath.mpf(1), mpmath.mpf(0)], [mpmath.mpf(0), mpmath.mpf(1)]]
    for t in range(T):
        a = mpmath.exp(mpmath.mpf(float(ld[t])))
        c = mpmath.mpf(float(kk[t])) ** 2 * mpmath.mpf(float(vp[t]))
        P = mat_mul(step_matrix(a, mpmath.mpf(float(pn[t])), c), P)
        ref = (P[0][0] * lam0 + P[0][1]) / (P[1][0] * lam0 + P[1][1])
        got = path[0, 0, t, 0]
        assert abs(mpmath.mpf(float(got)) - ref) <= mpmath.mpf("1e-13") * abs(ref), (t, got, ref)


# --------------------------------------------------------------------------- #
# 4. closed forms of special cases                                             #
# --------------------------------------------------------------------------- #

def _run(q, k, v, ld, pn, vp, lam0, M0):
    return O.kla_forward_f64(q, k, v, ld, pn, vp, lam0, M0, return_lambda_path=True,
                             return_gates=True)


def pin_steady_state_dare(T=400):
    """Constant coefficients: lambda_t tends to the positive root of
    pbar*L^2 - (1 + c*pbar - a^2)*L - c*a^2 = 0 (fixed point of the Möbius map)."""
    for a, pb, c in ((0.9, 0.3, 0.7), (0.5, 2.0, 0.01), (0.99, 0.01, 3.0)):
        k = np.full((1, 1, T, 1), np.sqrt(c))
        vp = np.ones((1, 1, T, 1))
        ld = np.full((1, 1, T, 1), np.log(a))
        pn = np.full((1, 1, T, 1), pb)
        _, lT, _, path = O.kla_forward_f64(np.zeros((1, 1, T, 1)), k, np.zeros((1, 1, T, 1)),
                                            ld, pn, vp, np.full((1, 1, 1), 1.0),
                                            return_lambda_path=True)
        bq = 1 + c * pb - a * a
        lstar = (bq + np.sqrt(bq * bq + 4 * pb * c * a * a)) / (2 * pb)
        assert abs(lT[0, 0, 0] - lstar) <= 1e-10 * lstar, (a, pb, c, lT, lstar)


def pin_no_observation(seed=8, T=30):
    """k = 0: variance follows P_t = a^2 P_{t-1} + pbar (geometric closed form for
    constant a, pbar); the mean only decays: M_t = a^t M0, gates f = a, g = 0."""
    rng = np.random.default_rng(seed)
    dk, dv = 2, 3
    a, pb = 0.8, 0.25
    q = rng.standard_normal((1, 1, T, dk))
    v = rng.standard_normal((1, 1, T, dv))
    k = np.zeros((1, 1, T, dk))
    ld = np.full((1, 1, T, dk), np.log(a))
    pn = np.full((1, 1, T, dk), pb)
    vp = np.ones((1, 1, T, dk))
    lam0 = np.array([[[2.0, 0.5]]])
    M0 = rng.standard_normal((1, 1, dk, dv))
    y, lT, MT, path, f, g = _run(q, k, v, ld, pn, vp, lam0, M0)
    t = np.arange(1, T + 1)[:, None]
    P = a ** (2 * t) / lam0[0, 0] + pb * (1 - a ** (2 * t)) / (1 - a * a)
    np.testing.assert_allclose(path[0, 0], 1 / P, rtol=1e-12)
    np.testing.assert_allclose(f[0, 0], a, rtol=1e-12)
    assert np.all(g == 0)
    yref = np.einsum("ti,ij->tj", q[0, 0] * a ** t, M0[0, 0])
    np.testing.assert_allclose(y[0, 0], yref, rtol=1e-11, atol=1e-13)


def pin_no_process_noise(T=25):
    """pbar = 0, constant a and c: lambda_t = lambda0 a^(-2t) + c * sum_{s<t} a^(-2s)."""
    a, c, lam0 = 0.95, 0.4, 1.3
    ld = np.full((1, 1, T, 1), np.log(a))
    pn = np.zeros((1, 1, T, 1))
    k = np.full((1, 1, T, 1), 2.0)
    vp = np.full((1, 1, T, 1), c / 4.0)
    _, _, _, path = O.kla_forward_f64(np.zeros((1, 1, T, 1)), k, np.zeros((1, 1, T, 1)),
                                       ld, pn, vp, np.full((1, 1, 1), lam0), return_lambda_path=True)
    t = np.arange(1, T + 1)
    ref = lam0 * a ** (-2.0 * t) + c * np.array([np.sum(a ** (-2.0 * np.arange(n))) for n in t])
    np.testing.assert_allclose(path[0, 0, :, 0], ref, rtol=1e-12)


def pin_least_squares(seed=9, T=20):
    """a = 1, pbar = 0: the filter is recursive weighted least squares,
    mu_t = (lam0 mu0 + sum_s k_s Lam_s v_s) / (lam0 + sum_s k_s^2 Lam_s)."""
    rng = np.random.default_rng(seed)
    dk, dv = 3, 2
    k = rng.standard_normal((1, 1, T, dk))
    vp = 0.1 + rng.random((1, 1, T, dk))
    v = rng.standard_normal((1, 1, T, dv))
    q = rng.standard_normal((1, 1, T, dk))
    lam0 = 0.5 + rng.random((1, 1, dk))
    M0 = rng.standard_normal((1, 1, dk, dv))
    y, lT, MT, path, f, g = _run(q, k, v, np.zeros((1, 1, T, dk)), np.zeros((1, 1, T, dk)),
                                 vp, lam0, M0)
    kl = (k * vp)[0, 0]                       # [T, dk]
    num = lam0[0, 0][:, None] * M0[0, 0] + np.einsum("ti,tj->ij", kl, v[0, 0])
    den = lam0[0, 0] + np.sum(k[0, 0] ** 2 * vp[0, 0], axis=0)
    np.testing.assert_allclose(MT[0, 0], num / den[:, None], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lT[0, 0], den, rtol=1e-12)
    mus = np.cumsum(np.einsum("ti,tj->tij", kl, v[0, 0]), axis=0) + (lam0[0, 0][:, None] * M0[0, 0])
    dens = lam0[0, 0] + np.cumsum(k[0, 0] ** 2 * vp[0, 0], axis=0)
    yref = np.einsum("ti,tij->tj", q[0, 0], mus / dens[:, :, None])
    np.testing.assert_allclose(y[0, 0], yref, rtol=1e-11, atol=1e-13)


def pin_zero_value_precision(seed=10, T=15):
    """Lambda^v = 0: tokens carry no evidence; f = a and y_t = q_t^T diag(prod a) M0."""
    rng = np.random.default_rng(seed)
    dk, dv = 4, 3
    q, k, v, ld, pn, vp, lam0, M0 = _rand_inputs(rng, 1, 1, T, dk, dv)
    vp = np.zeros_like(vp)
    y, lT, MT, path, f, g = _run(q, k, v, ld, pn, vp, lam0, M0)
    a = np.exp(ld[0, 0])
    np.testing.assert_allclose(f[0, 0], a, rtol=1e-12)
    cum = np.cumprod(a, axis=0)
    yref = np.einsum("ti,ij->tj", q[0, 0] * cum, M0[0, 0])
    np.testing.assert_allclose(y[0, 0], yref, rtol=1e-11, atol=1e-13)


# --------------------------------------------------------------------------- #
# 5. invariants                                                                #
# --------------------------------------------------------------------------- #

def pin_invariants(seed=12):
    rng = np.random.default_rng(seed)
    q, k, v, ld, pn, vp, lam0, M0 = _rand_inputs(rng, 2, 2, 50, 4, 3)
    y, lT, MT, path, f, g = _run(q, k, v, ld, pn, vp, lam0, M0)
    c = k * k * vp
    assert np.all(path > 0)
    # OU bounds: evidence adds c; the prior precision lies in (0, 1/pbar)
    assert np.all(path > c) and np.all(path < c + 1.0 / pn)
    a = np.exp(ld)
    assert np.all(f > 0) and np.all(f <= a * (1 + 1e-15)) and np.all(a < 1)
    # precision independent of q, v, M0
    _, lT2, _, path2, _, _ = _run(-2 * q, k, 3 * v, ld, pn, vp, lam0, M0 + 1)
    assert np.array_equal(path, path2)
    # monotone in lambda0 (det of each step matrix = a^2 > 0); once the two paths
    # have contracted onto each other only rounding separates them
    _, _, _, path3, _, _ = _run(q, k, v, ld, pn, vp, lam0 * 1.7, M0)
    assert np.all(path3 - path >= -4e-16 * path)
    assert np.all(path3[:, :, 0] > path[:, :, 0])
    # y is linear in (v, M0) jointly and in q
    q2, k2, v2, *_, M02 = _rand_inputs(np.random.default_rng(seed + 1), 2, 2, 50, 4, 3)
    ya = _run(q, k, v, ld, pn, vp, lam0, M0)[0]
    yb = _run(q, k, v2, ld, pn, vp, lam0, M02)[0]
    yab = _run(q, k, 2 * v - 3 * v2, ld, pn, vp, lam0, 2 * M0 - 3 * M02)[0]
    np.testing.assert_allclose(yab, 2 * ya - 3 * yb, rtol=1e-10, atol=1e-11)
    yq = _run(q + q2, k, v, ld, pn, vp, lam0, M0)[0]
    yq2 = _run(q2, k, v, ld, pn, vp, lam0, M0)[0]
    np.testing.assert_allclose(yq, ya + yq2, rtol=1e-10, atol=1e-11)


def pin_state_carry(seed=13):
    rng = np.random.default_rng(seed)
    q, k, v, ld, pn, vp, lam0, M0 = _rand_inputs(rng, 1, 2, 33, 3, 4)
    y, lT, MT = O.kla_forward_f64(q, k, v, ld, pn, vp, lam0, M0)
    s = slice(0, 13), slice(13, 33)
    y1, l1, M1 = O.kla_forward_f64(*(x[:, :, s[0]] for x in (q, k, v, ld, pn, vp)), lam0, M0)
    y2, l2, M2 = O.kla_forward_f64(*(x[:, :, s[1]] for x in (q, k, v, ld, pn, vp)), l1, M1)
    np.testing.assert_array_equal(np.concatenate([y1, y2], axis=2), y)
    np.testing.assert_array_equal(l2, lT)
    np.testing.assert_array_equal(M2, MT)
    # T = 0 is the identity
    y0, l0, Mz = O.kla_forward_f64(*(x[:, :, :0] for x in (q, k, v, ld, pn, vp)), lam0, M0)
    assert y0.shape == (1, 2, 0, 4)
    np.testing.assert_array_equal(l0, lam0)
    np.testing.assert_array_equal(Mz, M0)


def pin_precision_scan_matches_forward(seed=14):
    """The precision-only oracle equals the forward oracle's precision path when
    fed c = k^2 Lambda^v."""
    rng = np.random.default_rng(seed)
    q, k, v, ld, pn, vp, lam0, M0 = _rand_inputs(rng, 2, 3, 20, 5, 2)
    _, lT, _, path = O.kla_forward_f64(q, k, v, ld, pn, vp, lam0, M0, return_lambda_path=True)
    p2, l2 = O.precision_scan_f64(ld, pn, k * k * vp, lam0)
    np.testing.assert_allclose(p2, path, rtol=1e-14)
    np.testing.assert_allclose(l2, lT, rtol=1e-14)


# --------------------------------------------------------------------------- #
# decode step                                                                  #
# --------------------------------------------------------------------------- #

def pin_decode_covariance_form(seed=15):
    """One decode step from a random state equals one step of the
    covariance-form filter started from that state."""
    rng = np.random.default_rng(seed)
    q, k, v, ld, pn, vp, lam0, M0 = _rand_inputs(rng, B=3, H=2, T=1, dk=4, dv=5)
    y, lam, M = O.kla_decode_step_f64(q[:, :, 0], k[:, :, 0], v[:, :, 0], ld[:, :, 0], pn[:, :, 0],
                                      vp[:, :, 0], lam0, M0)
    y2, lam2, M2, _ = covariance_form_filter(q, k, v, ld, pn, vp, lam0, M0)
    np.testing.assert_allclose(lam, lam2, rtol=1e-12, atol=0)
    np.testing.assert_allclose(M, M2, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(y, y2[:, :, 0], rtol=1e-11, atol=1e-13)


def pin_decode_chain_is_dense_posterior(seed=16, T=8):
    """Decode steps chained from the prior give, at every token, the posterior
    mean and precision of Gaussian conditioning on the whole history."""
    rng = np.random.default_rng(seed)
    q, k, v, ld, pn, vp, lam0, M0 = _rand_inputs(rng, B=1, H=1, T=T, dk=2, dv=2)
    ref = {(i, j): dense_posterior(np.exp(ld[0, 0, :, i]), pn[0, 0, :, i], k[0, 0, :, i], vp[0, 0, :, i],
                                   v[0, 0, :, j], lam0[0, 0, i], M0[0, 0, i, j])
           for i in range(2) for j in range(2)}
    lam, M = lam0.copy(), M0.copy()
    for t in range(T):
        _, lam, M = O.kla_decode_step_f64(q[:, :, t], k[:, :, t], v[:, :, t], ld[:, :, t], pn[:, :, t],
                                          vp[:, :, t], lam, M)
        for (i, j), (means, precs) in ref.items():
            np.testing.assert_allclose(M[0, 0, i, j], means[t], rtol=1e-9, atol=1e-11)
            np.testing.assert_allclose(lam[0, 0, i], precs[t], rtol=1e-9)


# --------------------------------------------------------------------------- #
# backward pass                                                                #
# --------------------------------------------------------------------------- #

def _loss_parts(rng, B, H, T, dk, dv):
    dy = rng.standard_normal((B, H, T, dv))
    dlT = rng.standard_normal((B, H, dk))
    dMT = rng.standard_normal((B, H, dk, dv))
    return dy, dlT, dMT


def pin_backward_finite_differences(seed=17):
    """Gradients of <dy, y> + <dlam_T, lam_T> + <dM_T, M_T> equal central
    finite differences of the numpy oracle, for every input element."""
    import oracle.kla_backward_f64 as OB
    rng = np.random.default_rng(seed)
    B, H, T, dk, dv = 1, 2, 5, 3, 2
    q, k, v, ld, pn, vp, lam0, M0 = _rand_inputs(rng, B, H, T, dk, dv)
    dy, dlT, dMT = _loss_parts(rng, B, H, T, dk, dv)
    g = OB.kla_backward_f64(q, k, v, ld, pn, vp, dy, lam0, M0, dlT, dMT)

    def loss(q, k, v, ld, pn, vp, lam0, M0):
        y, lT, MT = O.kla_forward_f64(q, k, v, ld, pn, vp, lam0, M0)
        return float(np.sum(y * dy) + np.sum(lT * dlT) + np.sum(MT * dMT))

    args = [q, k, v, ld, pn, vp, lam0, M0]
    names = ["dq", "dk", "dv", "d_log_decay", "d_proc_noise", "d_val_prec", "d_lambda0", "d_M0"]
    for ai, name in enumerate(names):
        x = args[ai]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            h = 1e-6 * (1.0 + abs(x[idx]))
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            a_p = list(args); a_p[ai] = xp
            a_m = list(args); a_m[ai] = xm
            fd[idx] = (loss(*a_p) - loss(*a_m)) / (2 * h)
        np.testing.assert_allclose(g[name], fd, rtol=1e-6, atol=1e-8, err_msg=name)


def pin_backward_forward_is_the_oracle(seed=18):
    """The differentiable float64 filter of the backward oracle computes the
    numpy oracle's forward pass."""
    import torch
    import oracle.kla_backward_f64 as OB
    rng = np.random.default_rng(seed)
    args = _rand_inputs(rng, 2, 2, 30, 4, 3)
    y, lT, MT = O.kla_forward_f64(*args)
    yt, lTt, MTt = OB.kla_forward_torch64(*(torch.tensor(x, dtype=torch.float64) for x in args))
    np.testing.assert_allclose(yt.numpy(), y, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lTt.numpy(), lT, rtol=1e-13)
    np.testing.assert_allclose(MTt.numpy(), MT, rtol=1e-13, atol=1e-15)


def pin_backward_prior_precision_identity(seed=19):
    """lambda0 enters the filter only through the first predict step,
    lam^- = lambda0 / (a^2 + pbar lambda0), whose partial derivatives are
    a^2/D^2 in lambda0 and -lambda0^2/D^2 in pbar (D = a^2 + pbar lambda0).
    Hence dL/dlambda0 = -(a_1^2 / lambda0^2) dL/dpbar_1, whatever the rest of
    the filter does; the oracle's two gradients must obey it."""
    import oracle.kla_backward_f64 as OB
    rng = np.random.default_rng(seed)
    B, H, T, dk, dv = 2, 2, 12, 4, 3
    q, k, v, ld, pn, vp, lam0, M0 = _rand_inputs(rng, B, H, T, dk, dv)
    dy, dlT, dMT = _loss_parts(rng, B, H, T, dk, dv)
    g = OB.kla_backward_f64(q, k, v, ld, pn, vp, dy, lam0, M0, dlT, dMT)
    want = -np.exp(2 * ld[:, :, 0]) / lam0 ** 2 * g["d_proc_noise"][:, :, 0]
    np.testing.assert_allclose(g["d_lambda0"], want, rtol=1e-12, atol=1e-15)


def pin_ou_semigroup(seed=21):
    """OU transitions compose: a step of dt1 followed by one of dt2 is a step
    of dt1 + dt2, i.e. a(dt1 + dt2) = a(dt1) a(dt2) and
    pbar(dt1 + dt2) = a(dt2)^2 pbar(dt1) + pbar(dt2) (the first step's noise
    decays through the second)."""
    import oracle.kla_ou_f64 as OU
    rng = np.random.default_rng(seed)
    th = rng.uniform(0.0, 3.0, 200)
    s2 = rng.uniform(0.1, 2.0, 200)
    d1, d2 = rng.uniform(0.0, 2.0, 200), rng.uniform(0.0, 2.0, 200)
    l1, p1 = OU.ou_discretize_f64(th, s2, d1)
    l2, p2 = OU.ou_discretize_f64(th, s2, d2)
    l12, p12 = OU.ou_discretize_f64(th, s2, d1 + d2)
    np.testing.assert_allclose(l12, l1 + l2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(p12, np.exp(2 * l2) * p1 + p2, rtol=1e-12)


def pin_ou_transition_variance_quadrature(seed=22):
    """The step noise equals integral_0^dt sigma2 e^{-2 theta s} ds, evaluated
    by adaptive quadrature (scipy), and the decay equals e^{-theta dt}."""
    from scipy.integrate import quad
    import oracle.kla_ou_f64 as OU
    rng = np.random.default_rng(seed)
    for _ in range(20):
        th, s2, dt = rng.uniform(0.0, 4.0), rng.uniform(0.1, 3.0), rng.uniform(0.0, 3.0)
        want, _ = quad(lambda x: s2 * np.exp(-2.0 * th * x), 0.0, dt, epsabs=1e-14, epsrel=1e-13)
        ld, pn = OU.ou_discretize_f64(th, s2, dt)
        np.testing.assert_allclose(pn, want, rtol=1e-11, atol=1e-14)
        np.testing.assert_allclose(np.exp(ld), np.exp(-th * dt), rtol=1e-15)


def pin_ou_limits():
    """Brownian limit: theta = 0 gives a = 1 and pbar = sigma2 dt (and theta
    -> 0 approaches it); long steps reach the stationary variance
    sigma2 / (2 theta) with a -> 0."""
    import oracle.kla_ou_f64 as OU
    s2, dt = 1.7, 0.9
    ld, pn = OU.ou_discretize_f64(0.0, s2, dt)
    assert ld == 0.0 and abs(pn - s2 * dt) < 1e-15
    ld, pn = OU.ou_discretize_f64(1e-9, s2, dt)
    np.testing.assert_allclose(pn, s2 * dt, rtol=1e-8)
    ld, pn = OU.ou_discretize_f64(0.8, s2, 60.0)
    np.testing.assert_allclose(pn, s2 / (2 * 0.8), rtol=1e-14)
    assert np.exp(ld) < 1e-20


def pin_vprec_elements_are_dense_posteriors(seed=23):
    """With the value precision per value channel, every element (i,j) is its
    own scalar filter: its mean and precision after every token equal dense
    Gaussian conditioning (numpy.linalg.solve) with coefficients
    (a_i, pbar_i, k_i, Lambda^v_j, v_j), and y_t[j] = sum_i q_{t,i} mean_ij(t)."""
    import oracle.kla_vprec_f64 as OV
    rng = np.random.default_rng(seed)
    B, H, T, dk, dv = 1, 2, 9, 3, 4
    q, k, v, ld, pn, _, _, _ = _rand_inputs(rng, B, H, T, dk, dv)
    vpv = np.logaddexp(0.0, rng.standard_normal((B, H, T, dv))) + 1e-3
    lam0 = 0.5 + rng.random((B, H, dk, dv))
    M0 = rng.standard_normal((B, H, dk, dv))
    y, lT, MT, path = OV.kla_forward_vprec_f64(q, k, v, ld, pn, vpv, lam0, M0, return_lambda_path=True)
    for h in range(H):
        means = np.empty((T, dk, dv))
        for i in range(dk):
            for j in range(dv):
                m, prec = dense_posterior(np.exp(ld[0, h, :, i]), pn[0, h, :, i], k[0, h, :, i], vpv[0, h, :, j],
                                          v[0, h, :, j], lam0[0, h, i, j], M0[0, h, i, j])
                np.testing.assert_allclose(path[0, h, :, i, j], prec, rtol=1e-9)
                means[:, i, j] = m
        np.testing.assert_allclose(MT[0, h], means[-1], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(y[0, h], np.einsum("ti,tij->tj", q[0, h], means), rtol=1e-9, atol=1e-12)


def pin_vprec_shared_precision_is_the_main_path(seed=24):
    """When Lambda^v is one number per token (the same for every key and value
    channel), both readings coincide: the variant equals the main oracle."""
    import oracle.kla_vprec_f64 as OV
    rng = np.random.default_rng(seed)
    B, H, T, dk, dv = 2, 1, 20, 3, 5
    q, k, v, ld, pn, _, lam0, M0 = _rand_inputs(rng, B, H, T, dk, dv)
    s = np.logaddexp(0.0, rng.standard_normal((B, H, T, 1))) + 1e-3
    y1, l1, M1 = O.kla_forward_f64(q, k, v, ld, pn, np.broadcast_to(s, (B, H, T, dk)), lam0, M0)
    y2, l2, M2 = OV.kla_forward_vprec_f64(q, k, v, ld, pn, np.broadcast_to(s, (B, H, T, dv)),
                                          np.broadcast_to(lam0[..., None], (B, H, dk, dv)), M0)
    np.testing.assert_allclose(y2, y1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(M2, M1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l2, np.broadcast_to(l1[..., None], l2.shape), rtol=1e-13)


def pin_prologue_conv_impulse(seed=25):
    """A unit impulse at token t0 in channel c comes out of the causal
    convolution as the channel's taps, newest tap first: u_{t0+m} = w[c, W-1-m]
    for m < W and nothing before t0 or after t0 + W - 1 (plus the bias
    everywhere)."""
    import oracle.kla_prologue_f64 as OP
    rng = np.random.default_rng(seed)
    H, T, d, W = 2, 11, 3, 4
    w = rng.standard_normal((H, d, W))
    b = rng.standard_normal((H, d))
    for t0 in (0, 4, 9):
        x = np.zeros((1, H, T, d))
        x[0, 1, t0, 2] = 1.0
        u = OP.causal_conv_f64(x, w, b) - b[None, :, None, :]
        want = np.zeros_like(u)
        for m in range(W):
            if t0 + m < T:
                want[0, 1, t0 + m, 2] = w[1, 2, W - 1 - m]
        np.testing.assert_allclose(u, want, rtol=0, atol=1e-14)


def pin_prologue_streams_match_library_routines(seed=26):
    """Each prologue output against library routines: the convolution as
    numpy.convolve with the taps reversed (its first T outputs are the causal
    ones), SiLU as u (1 + tanh(u/2)) / 2, softplus as log1p(exp(x)); each
    stream with weights of its own, so a swapped weight or input fails."""
    import oracle.kla_prologue_f64 as OP
    rng = np.random.default_rng(seed)
    B, H, T, dk, dv, W = 2, 2, 13, 3, 2, 4
    xs = [rng.standard_normal((B, H, T, d)) for d in (dk, dk, dv)]
    ws = [rng.uniform(-0.5, 0.5, (H, d, W)) for d in (dk, dk, dv)]
    bs = [rng.uniform(-0.5, 0.5, (H, d)) for d in (dk, dk, dv)]
    dtr, vpr = rng.standard_normal((B, H, T, dk)), 3 * rng.standard_normal((B, H, T, dk))
    out = OP.prologue_f64(*xs, dtr, vpr, ws, bs, dtype="f32")
    for x, w, b, got in zip(xs, ws, bs, out[:3]):
        u = np.empty_like(x)
        for bi in range(B):
            for h in range(H):
                for c in range(x.shape[-1]):
                    u[bi, h, :, c] = np.convolve(x[bi, h, :, c], w[h, c, ::-1])[:T] + b[h, c]
        want = (u * 0.5 * (1.0 + np.tanh(0.5 * u))).astype(np.float32)
        np.testing.assert_allclose(got, want, rtol=2e-7, atol=1e-30)
    np.testing.assert_allclose(out[3], np.log1p(np.exp(dtr)), rtol=1e-14)
    np.testing.assert_allclose(out[4], np.log1p(np.exp(vpr)), rtol=1e-14)


def pin_prologue_closed_forms():
    """SiLU(0) = 0, SiLU(x) - SiLU(-x) = x, SiLU(x) / x -> 1 for large x;
    softplus(0) = ln 2, softplus(x) - softplus(-x) = x, and softplus' = sigmoid
    = SiLU(x) / x (central difference)."""
    import oracle.kla_prologue_f64 as OP
    x = np.linspace(-6.0, 6.0, 25)
    assert OP.silu_f64(0.0) == 0.0
    np.testing.assert_allclose(OP.silu_f64(x) - OP.silu_f64(-x), x, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(OP.silu_f64(40.0), 40.0, rtol=1e-15)
    np.testing.assert_allclose(OP.softplus_f64(0.0), np.log(2.0), rtol=1e-15)
    np.testing.assert_allclose(OP.softplus_f64(x) - OP.softplus_f64(-x), x, rtol=1e-13, atol=1e-15)
    xn = x[x != 0]
    h = 1e-5
    deriv = (OP.softplus_f64(xn + h) - OP.softplus_f64(xn - h)) / (2 * h)
    np.testing.assert_allclose(deriv, OP.silu_f64(xn) / xn, rtol=1e-8)


def pin_prologue_bf16_activations():
    """For bf16 inputs the activations are the nearest bfloat16 values: every
    one has a zero low half as float32 and lies within half a bf16 unit in the
    last place (at most 2^-8 relative) of the exact SiLU(conv)."""
    import oracle.kla_prologue_f64 as OP
    rng = np.random.default_rng(27)
    H, T, d, W = 1, 40, 8, 4
    x = rng.standard_normal((1, H, T, d))
    w = rng.uniform(-0.5, 0.5, (H, d, W))
    out = OP.prologue_f64(x, x, x, x[..., :1], x[..., :1], (w, w, w), dtype="bf16")
    exact = OP.silu_f64(OP.causal_conv_f64(x, w))
    for a in out[:3]:
        bits = np.asarray(a, np.float32).view(np.uint32)
        assert np.all(bits & 0xFFFF == 0)
        assert np.all(np.abs(a - exact) <= 2.0 ** -8 * np.abs(exact) + 1e-38)


ALL_PINS = [
    pin_covariance_form, pin_dense_gaussian, pin_mobius_exact, pin_mobius_mpmath,
    pin_steady_state_dare, pin_no_observation, pin_no_process_noise, pin_least_squares,
    pin_zero_value_precision, pin_invariants, pin_state_carry,
    pin_precision_scan_matches_forward, pin_decode_covariance_form, pin_decode_chain_is_dense_posterior,
    pin_backward_finite_differences, pin_backward_forward_is_the_oracle,
    pin_backward_prior_precision_identity, pin_ou_semigroup, pin_ou_transition_variance_quadrature,
    pin_ou_limits, pin_vprec_elements_are_dense_posteriors, pin_vprec_shared_precision_is_the_main_path,
    pin_prologue_conv_impulse, pin_prologue_streams_match_library_routines, pin_prologue_closed_forms,
    pin_prologue_bf16_activations,
]
