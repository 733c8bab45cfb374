// KLA backward pass: gradients of the forward scan with respect to q, k, v,
// log_decay, proc_noise, val_prec and the state in (lambda0, M0), given the
// gradients of y and of the state out (lambda_T, M_T).
//
// Sources: gist.science summaries of arXiv 2602.10743, "Kalman Linear Attention";
// [KLA-nl] = "Technische Samenvatting: Kalman Linear Attention (KLA)":
//   §2 "Parallelisatie via Möbius-transformaties"  precision equation; affine mean recursion
//   §3 "Niet-lineaire Gating vanuit Onzekerheid"   gates are precision ratios
//   "Belangrijkste Bijdragen"                      KLA is trained as a sequence mixer
// The forward step per token t and key channel i (a = exp(log_decay),
// pbar = proc_noise, c = k^2 Lambda^v):
//   lam^- = lam_{t-1} / (a^2 + pbar lam_{t-1}),  lam_t = lam^- + c,
//   f = a lam^- / lam_t,  g = k Lambda^v / lam_t,  M_t = f M_{t-1} + g v_t^T,
//   y_t = q_t^T M_t.
//
// Decomposition (segments of 64 tokens, chunks of 16; all arithmetic fp32):
//   1. segagg   per (head, segment): prod of f over the segment, and the two
//               segment aggregates sum_t (prod_{u>t} f) g_t v_t^T (mean) and
//               sum_t (prod_{u<=t} f) q_t dy_t^T (adjoint).
//   2. segscan  per head and state element: the mean entering every segment
//               (forward over segments) and the adjoint at every segment end
//               (backward over segments); dM0; the row sums of M_T * dM_T.
//   3. chunk    per (head, segment), its chunks last to first: the mean
//               entering the chunk (from the segment's, plus the tokens before
//               the chunk), the adjoint at its end (carried backwards), then
//               dq and dv (final) and, per channel, the write-gate gradient dg
//               and e = q dq - g dg.  In-chunk decays prod_{u=m+1..l} f_u are
//               formed as running products (never as ratios of cumulative
//               products, which can underflow), and inside the score matrix
//               as exp2 of differences of cumulative log2 f.
//   4. chain    per channel, backwards over tokens: d log f_t is the suffix
//               sum of e (plus the M_T * dM_T row sum), and the adjoint of the
//               precision obeys an affine recursion; both run as a two-level
//               scan over 64-token blocks (block composites, a carry pass over
//               blocks, and a pass that writes dk, d_log_decay, d_proc_noise,
//               d_val_prec).  dlambda0 is the adjoint left after token 1.
// Every sum has a fixed order: results are deterministic.
#include <type_traits>

#include "kla_device.h"
#include "kla_internal.h"

namespace kla {

namespace {
constexpr int kSL = 64;  // tokens per segment
constexpr int kC = 16;   // tokens per chunk
constexpr int kChunkThreads = 512;

template <bool BF16>
__device__ __forceinline__ float ldin(const void* p, size_t x) {
  using In = typename std::conditional<BF16, uint16_t, float>::type;
  return to_f32(static_cast<const In*>(p)[x]);
}

template <bool BF16>
__device__ __forceinline__ void stout(void* p, size_t x, float v) {
  using In = typename std::conditional<BF16, uint16_t, float>::type;
  static_cast<In*>(p)[x] = from_f32<In>(v);
}

// Forget and write gates of token t < T, channel i, from the saved precision path.
template <bool BF16>
__device__ __forceinline__ void gates(const BwdParams& p, size_t hd, int t, int i, int K, float& f, float& g) {
  const size_t x = (hd * p.T + t) * K + i;
  const float lam = p.lpath[x];
  const float lprev = t > 0 ? p.lpath[x - K] : (p.lam0 ? p.lam0[hd * K + i] : 1.f);
  const float a = __expf(ldin<BF16>(p.ld, x));
  const float lpred = lprev / fmaf(ldin<BF16>(p.pn, x), lprev, a * a);
  f = a * lpred / lam;
  g = ldin<BF16>(p.k, x) * ldin<BF16>(p.vp, x) / lam;
}

// Stages the segment's tokens: f, g, q as [64][K+1] and v, dy as [64][V+1]
// (rows padded by one word so that column walks hit distinct banks).  Tokens
// past T are identity steps: f = 1, g = q = v = dy = 0.
template <int K, int V, bool BF16, int NT>
__device__ __forceinline__ void stage_segment(const BwdParams& p, size_t hd, int t0, float* sf, float* sg,
                                              float* sq, float* sv, float* sd) {
  constexpr int KP = K + 1, VP = V + 1;
  for (int x = threadIdx.x; x < kSL * K; x += NT) {
    const int t = x / K, i = x % K;
    float f = 1.f, g = 0.f, q = 0.f;
    if (t0 + t < p.T) {
      gates<BF16>(p, hd, t0 + t, i, K, f, g);
      q = ldin<BF16>(p.q, (hd * p.T + t0 + t) * K + i);
    }
    sf[t * KP + i] = f;
    sg[t * KP + i] = g;
    sq[t * KP + i] = q;
  }
  for (int x = threadIdx.x; x < kSL * V; x += NT) {
    const int t = x / V, j = x % V;
    float v = 0.f, d = 0.f;
    if (t0 + t < p.T) {
      const size_t y = (hd * p.T + t0 + t) * V + j;
      v = ldin<BF16>(p.v, y);
      d = ldin<BF16>(p.dy, y);
    }
    sv[t * VP + j] = v;
    sd[t * VP + j] = d;
  }
}
}  // namespace

// ---------------------------------------------------------------------------
// 1. Segment aggregates.  Grid: nheads * nseg workgroups of 256 threads.
// ---------------------------------------------------------------------------
template <int K, int V, bool BF16>
__global__ __launch_bounds__(256) void kla_bwd_segagg_kernel(BwdParams p) {
  constexpr int KP = K + 1, VP = V + 1, NT = 256;
  __shared__ float sf[kSL * KP], sa[kSL * KP], sb[kSL * KP], sv[kSL * VP], sd[kSL * VP];
  const size_t hd = blockIdx.x / p.nseg;
  const int s = blockIdx.x % p.nseg;
  const int tid = threadIdx.x;
  stage_segment<K, V, BF16, NT>(p, hd, s * kSL, sf, sa, sb, sv, sd);
  __syncthreads();
  if (tid < K) {
    // alpha_t = g_t prod_{u>t} f_u (in place of g); beta_t = q_t prod_{u<=t} f_u (in place of q).
    float run = 1.f;
    for (int t = kSL - 1; t >= 0; --t) {
      sa[t * KP + tid] *= run;
      run *= sf[t * KP + tid];
    }
    p.F[(hd * p.nseg + s) * K + tid] = run;
    float pre = 1.f;
    for (int t = 0; t < kSL; ++t) {
      pre *= sf[t * KP + tid];
      sb[t * KP + tid] *= pre;
    }
  }
  __syncthreads();
  // Mean aggregate alpha^T v and adjoint aggregate beta^T dy, 4x4 tiles per thread.
  constexpr int NJ = V / 4, NTILE = (K / 4) * NJ;
  float* UM = p.Mseg + (hd * p.nseg + s) * (size_t)(K * V);
  float* UH = p.Gseg + (hd * p.nseg + s) * (size_t)(K * V);
  for (int tile = tid; tile < NTILE; tile += NT) {
    const int i0 = (tile / NJ) * 4, j0 = (tile % NJ) * 4;
    float am[4][4], ah[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) am[r][c] = ah[r][c] = 0.f;
    for (int t = 0; t < kSL; ++t) {
      float a[4], b[4], v[4], d[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        a[r] = sa[t * KP + i0 + r];
        b[r] = sb[t * KP + i0 + r];
        v[r] = sv[t * VP + j0 + r];
        d[r] = sd[t * VP + j0 + r];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          am[r][c] = fmaf(a[r], v[c], am[r][c]);
          ah[r][c] = fmaf(b[r], d[c], ah[r][c]);
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      *reinterpret_cast<float4*>(UM + (i0 + r) * V + j0) = make_float4(am[r][0], am[r][1], am[r][2], am[r][3]);
      *reinterpret_cast<float4*>(UH + (i0 + r) * V + j0) = make_float4(ah[r][0], ah[r][1], ah[r][2], ah[r][3]);
    }
  }
}

// ---------------------------------------------------------------------------
// 2. Scans over segments.  Grid: nheads * ceil(K*V/4 / 256) workgroups of 256
// threads; a thread owns four consecutive elements of one state row.
// ---------------------------------------------------------------------------
template <int K, int V>
__global__ __launch_bounds__(256) void kla_bwd_segscan_kernel(BwdParams p) {
  constexpr int NJ = V / 4, N4 = K * NJ;
  constexpr int NB = (N4 + 255) / 256;
  const size_t hd = blockIdx.x / NB;
  const int e4 = (blockIdx.x % NB) * 256 + threadIdx.x;
  const bool live = e4 < N4;
  const int i = e4 / NJ;
  const int nseg = p.nseg;
  float4* Ms = reinterpret_cast<float4*>(p.Mseg + hd * nseg * (size_t)(K * V));
  float4* Gs = reinterpret_cast<float4*>(p.Gseg + hd * nseg * (size_t)(K * V));
  const float* F = p.F + hd * nseg * (size_t)K + i;
  float part = 0.f;
  if (live) {
    float4 m = p.M0 ? reinterpret_cast<const float4*>(p.M0 + hd * (size_t)(K * V))[e4] : make_float4(0.f, 0.f, 0.f, 0.f);
    float4 u = Ms[e4];
    for (int s = 0; s < nseg; ++s) {
      const float4 un = s + 1 < nseg ? Ms[(size_t)(s + 1) * N4 + e4] : u;
      const float f = F[(size_t)s * K];
      Ms[(size_t)s * N4 + e4] = m;
      m = make_float4(fmaf(f, m.x, u.x), fmaf(f, m.y, u.y), fmaf(f, m.z, u.z), fmaf(f, m.w, u.w));
      u = un;
    }
    if (p.dMT) {
      const float4 d = reinterpret_cast<const float4*>(p.dMT + hd * (size_t)(K * V))[e4];
      part = m.x * d.x + m.y * d.y + m.z * d.z + m.w * d.w;
    }
  }
  // Row sum over the NJ threads of a row (consecutive lanes of one wave).
#pragma unroll
  for (int o = NJ / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o);
  if (live && e4 % NJ == 0) p.rs[hd * K + i] = part;
  if (live) {
    float4 h = p.dMT ? reinterpret_cast<const float4*>(p.dMT + hd * (size_t)(K * V))[e4] : make_float4(0.f, 0.f, 0.f, 0.f);
    float4 u = Gs[(size_t)(nseg - 1) * N4 + e4];
    for (int s = nseg - 1; s >= 0; --s) {
      const float4 un = s > 0 ? Gs[(size_t)(s - 1) * N4 + e4] : u;
      const float f = F[(size_t)s * K];
      Gs[(size_t)s * N4 + e4] = h;
      h = make_float4(fmaf(f, h.x, u.x), fmaf(f, h.y, u.y), fmaf(f, h.z, u.z), fmaf(f, h.w, u.w));
      u = un;
    }
    reinterpret_cast<float4*>(p.dM0 + hd * (size_t)(K * V))[e4] = h;
  }
}

// ---------------------------------------------------------------------------
// 3. Per-chunk gradients.  Grid: nheads * nseg workgroups of 512 threads.
// ---------------------------------------------------------------------------
template <int K, int V>
struct BwdChunkSmem {
  static constexpr int KP = K + 1, VP = V + 1;
  float f[kSL * KP], g[kSL * KP], q[kSL * KP], v[kSL * VP], d[kSL * VP];
  float M[K * VP], H[K * VP];      // mean entering the chunk; adjoint at its end
  float al[(kSL - kC) * KP];       // g_t prod_{u=t+1}^{c0-1} f_u for tokens before the chunk
  float lb[kC * KP];               // cumulative log2 f inside the chunk
  float cp[kC * KP];               // prod_{u<=l} f_u inside the chunk
  float sx[kC * KP];               // prod_{u>l} f_u inside the chunk
  float A[kC * kC], B[kC * kC];    // A[l][m] = q_l . (g_m decayed to l); B[l][m] = dy_l . v_m
  float P[K];                      // prod of f from the segment start to the chunk start
};

template <int K, int V, bool BF16>
__global__ __launch_bounds__(kChunkThreads) void kla_bwd_chunk_kernel(BwdParams p) {
  constexpr int KP = K + 1, VP = V + 1, NT = kChunkThreads, C = kC;
  static_assert(NT == 2 * C * C, "one score pair per thread for A and for B");
  __shared__ BwdChunkSmem<K, V> s;
  const size_t hd = blockIdx.x / p.nseg;
  const int seg = blockIdx.x % p.nseg;
  const int tid = threadIdx.x;
  const int t0 = seg * kSL;
  const int nvalid = min(kSL, p.T - t0);
  stage_segment<K, V, BF16, NT>(p, hd, t0, s.f, s.g, s.q, s.v, s.d);
  const size_t st = (hd * p.nseg + seg) * (size_t)(K * V);
  const float* Mg = p.Mseg + st;
  for (int x = tid; x < K * V; x += NT) s.H[(x / V) * VP + x % V] = p.Gseg[st + x];
  __syncthreads();

  for (int w = (nvalid - 1) / C; w >= 0; --w) {
    const int c0 = w * C;
    // (a) per-channel running products.
    if (tid < K) {
      const int i = tid;
      float run = 1.f;
      for (int t = c0 - 1; t >= 0; --t) {
        s.al[t * KP + i] = s.g[t * KP + i] * run;
        run *= s.f[t * KP + i];
      }
      s.P[i] = run;
      float cp = 1.f, lb = 0.f;
      for (int l = 0; l < C; ++l) {
        const float f = s.f[(c0 + l) * KP + i];
        cp *= f;
        lb += __log2f(fmaxf(f, 1e-37f));
        s.cp[l * KP + i] = cp;
        s.lb[l * KP + i] = lb;
      }
      float sx = 1.f;
      for (int l = C - 1; l >= 0; --l) {
        s.sx[l * KP + i] = sx;
        sx *= s.f[(c0 + l) * KP + i];
      }
    }
    __syncthreads();
    // (b) mean entering the chunk: diag(P) M_seg + sum_{t<c0} al_t v_t^T (4x2 tiles).
    {
      constexpr int NJ2 = V / 2, NTILE = (K / 4) * NJ2;
      for (int tile = tid; tile < NTILE; tile += NT) {
        const int i0 = (tile / NJ2) * 4, j0 = (tile % NJ2) * 2;
        float acc[4][2];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float P = s.P[i0 + r];
          const float2 m = *reinterpret_cast<const float2*>(Mg + (i0 + r) * V + j0);
          acc[r][0] = P * m.x;
          acc[r][1] = P * m.y;
        }
        for (int t = 0; t < c0; ++t) {
          const float v0 = s.v[t * VP + j0], v1 = s.v[t * VP + j0 + 1];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float al = s.al[t * KP + i0 + r];
            acc[r][0] = fmaf(al, v0, acc[r][0]);
            acc[r][1] = fmaf(al, v1, acc[r][1]);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s.M[(i0 + r) * VP + j0] = acc[r][0];
          s.M[(i0 + r) * VP + j0 + 1] = acc[r][1];
        }
      }
    }
    // (c) in-chunk scores for m <= l (zero above the diagonal).
    {
      const int pr = tid & (C * C - 1), l = pr / C, m = pr % C;
      float acc = 0.f;
      if (m <= l) {
        if (tid < C * C) {
          for (int i = 0; i < K; ++i)
            acc = fmaf(s.q[(c0 + l) * KP + i] * s.g[(c0 + m) * KP + i],
                       exp2f(s.lb[l * KP + i] - s.lb[m * KP + i]), acc);
        } else {
          for (int j = 0; j < V; ++j) acc = fmaf(s.d[(c0 + l) * VP + j], s.v[(c0 + m) * VP + j], acc);
        }
      }
      (tid < C * C ? s.A : s.B)[l * C + m] = acc;
    }
    __syncthreads();
    // (d) per (token, key channel): dq, dg, e;  per (token, value channel): dv.
    const size_t tok0 = hd * (size_t)p.T + t0 + c0;
    for (int x = tid; x < C * K; x += NT) {
      const int l = x / K, i = x % K;
      if (c0 + l >= nvalid) continue;
      float xs = 0.f, ys = 0.f;
      for (int j = 0; j < V; ++j) {
        xs = fmaf(s.d[(c0 + l) * VP + j], s.M[i * VP + j], xs);
        ys = fmaf(s.v[(c0 + l) * VP + j], s.H[i * VP + j], ys);
      }
      float dqi = 0.f, D = 1.f;
      for (int m = l; m >= 0; --m) {
        dqi = fmaf(s.B[l * C + m] * s.g[(c0 + m) * KP + i], D, dqi);
        D *= s.f[(c0 + m) * KP + i];
      }
      float dgi = 0.f;
      D = 1.f;
      for (int l2 = l; l2 < C; ++l2) {
        dgi = fmaf(s.B[l2 * C + l] * s.q[(c0 + l2) * KP + i], D, dgi);
        if (l2 + 1 < C) D *= s.f[(c0 + l2 + 1) * KP + i];
      }
      const float dq = fmaf(s.cp[l * KP + i], xs, dqi);
      const float dg = fmaf(s.sx[l * KP + i], ys, dgi);
      const size_t o = (tok0 + l) * K + i;
      stout<BF16>(p.dq, o, dq);
      p.dgw[o] = dg;
      p.ew[o] = s.q[(c0 + l) * KP + i] * dq - s.g[(c0 + l) * KP + i] * dg;
    }
    for (int x = tid; x < C * V; x += NT) {
      const int m = x / V, j = x % V;
      if (c0 + m >= nvalid) continue;
      float acc = 0.f;
      for (int l = m; l < C; ++l) acc = fmaf(s.A[l * C + m], s.d[(c0 + l) * VP + j], acc);
      for (int i = 0; i < K; ++i)
        acc = fmaf(s.g[(c0 + m) * KP + i] * s.sx[m * KP + i], s.H[i * VP + j], acc);
      stout<BF16>(p.dv, (tok0 + m) * V + j, acc);
    }
    __syncthreads();
    // (e) adjoint at the end of the previous chunk: diag(cp_end) H + sum_l (cp_l q_l) dy_l^T.
    if (w > 0) {
      constexpr int NJ2 = V / 2, NTILE = (K / 4) * NJ2;
      for (int tile = tid; tile < NTILE; tile += NT) {
        const int i0 = (tile / NJ2) * 4, j0 = (tile % NJ2) * 2;
        float acc[4][2];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ce = s.cp[(C - 1) * KP + i0 + r];
          acc[r][0] = ce * s.H[(i0 + r) * VP + j0];
          acc[r][1] = ce * s.H[(i0 + r) * VP + j0 + 1];
        }
        for (int l = 0; l < C; ++l) {
          const float d0 = s.d[(c0 + l) * VP + j0], d1 = s.d[(c0 + l) * VP + j0 + 1];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float b = s.cp[l * KP + i0 + r] * s.q[(c0 + l) * KP + i0 + r];
            acc[r][0] = fmaf(b, d0, acc[r][0]);
            acc[r][1] = fmaf(b, d1, acc[r][1]);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s.H[(i0 + r) * VP + j0] = acc[r][0];
          s.H[(i0 + r) * VP + j0 + 1] = acc[r][1];
        }
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// 4. Per-channel reverse chain.  State entering token t from the right:
// acc = sum_{s>t} e_s (+ the M_T * dM_T row sum) and L = dL/dlambda_t from
// later tokens.  Token t (reverse) maps it affinely:
//   acc' = acc + e_t
//   L'   = m_t (L + c1_t acc' + c0_t),  m_t = a^2/D^2, D = a^2 + pbar lam_{t-1},
//          c1_t = c/(lam lam^-) (= 1/lam^- - 1/lam), c0_t = -g dg / lam,
// where d log f_t = acc', df = acc'/f, and L' = dL/dlambda_{t-1}.
// ---------------------------------------------------------------------------
namespace {
struct ChainTok {
  float lam, lprev, a2, D, lpred, k, vp, dg, e;
};

template <bool BF16>
__device__ __forceinline__ ChainTok chain_tok(const BwdParams& p, size_t hd, long long ch, int t, int K, int i) {
  ChainTok c;
  const size_t x = (hd * p.T + t) * K + i;
  c.lam = p.lpath[x];
  c.lprev = t > 0 ? p.lpath[x - K] : (p.lam0 ? p.lam0[ch] : 1.f);
  const float a = __expf(ldin<BF16>(p.ld, x));
  c.a2 = a * a;
  c.D = fmaf(ldin<BF16>(p.pn, x), c.lprev, c.a2);
  c.lpred = c.lprev / c.D;
  c.k = ldin<BF16>(p.k, x);
  c.vp = ldin<BF16>(p.vp, x);
  c.dg = p.dgw[x];
  c.e = p.ew[x];
  return c;
}
}  // namespace

// Grid: ceil(nchains/256) * nseg workgroups; thread = chain, y = block of 64 tokens.
template <bool BF16>
__global__ __launch_bounds__(256) void kla_bwd_chain_comp_kernel(BwdParams p, int K, int ncb) {
  const long long ch = (long long)(blockIdx.x % ncb) * 256 + threadIdx.x;
  const int b = blockIdx.x / ncb;
  if (ch >= p.nchains) return;
  const size_t hd = ch / K;
  const int i = (int)(ch % K);
  const int tb = b * kSL, te = min(p.T, tb + kSL);
  float E = 0.f, Pm = 1.f, Qa = 0.f, R = 0.f;
  for (int t = te - 1; t >= tb; --t) {
    const ChainTok c = chain_tok<BF16>(p, hd, ch, t, K, i);
    const float g = c.k * c.vp / c.lam;
    const float m = c.a2 / (c.D * c.D);
    const float c1 = c.k * c.k * c.vp / (c.lam * c.lpred);
    const float c0 = -g * c.dg / c.lam;
    E += c.e;
    Pm *= m;
    Qa = m * (Qa + c1);
    R = m * fmaf(c1, E, R + c0);
  }
  reinterpret_cast<float4*>(p.comp)[(size_t)b * p.nchains + ch] = make_float4(E, Pm, Qa, R);
}

__global__ __launch_bounds__(256) void kla_bwd_chain_carry_kernel(BwdParams p) {
  const long long ch = (long long)blockIdx.x * 256 + threadIdx.x;
  if (ch >= p.nchains) return;
  float acc = p.rs[ch], L = p.dlamT ? p.dlamT[ch] : 0.f;
  for (int b = p.nseg - 1; b >= 0; --b) {
    reinterpret_cast<float2*>(p.cin)[(size_t)b * p.nchains + ch] = make_float2(acc, L);
    const float4 c = reinterpret_cast<const float4*>(p.comp)[(size_t)b * p.nchains + ch];
    L = fmaf(c.y, L, fmaf(c.z, acc, c.w));
    acc += c.x;
  }
  p.dlam0[ch] = L;
}

template <bool BF16>
__global__ __launch_bounds__(256) void kla_bwd_chain_out_kernel(BwdParams p, int K, int ncb) {
  const long long ch = (long long)(blockIdx.x % ncb) * 256 + threadIdx.x;
  const int b = blockIdx.x / ncb;
  if (ch >= p.nchains) return;
  const size_t hd = ch / K;
  const int i = (int)(ch % K);
  const int tb = b * kSL, te = min(p.T, tb + kSL);
  const float2 in = reinterpret_cast<const float2*>(p.cin)[(size_t)b * p.nchains + ch];
  float acc = in.x, L = in.y;
  for (int t = te - 1; t >= tb; --t) {
    const ChainTok c = chain_tok<BF16>(p, hd, ch, t, K, i);
    const float g = c.k * c.vp / c.lam;
    const float c0 = -g * c.dg / c.lam;
    acc += c.e;                                             // d log f_t
    const float dc = L - acc / c.lam + c0;                  // dL/dlambda_t = dL/dc_t
    const float Llp = fmaf(c.k * c.k * c.vp / (c.lam * c.lpred), acc, L + c0);  // dL/dlambda^-_t
    const float w = -Llp * c.lprev / (c.D * c.D);           // dL/d(a^2)
    const size_t x = (hd * p.T + t) * K + i;
    stout<BF16>(p.dld, x, fmaf(2.f * c.a2, w, acc));        // a dL/da = d log f + 2 a^2 dL/d(a^2)
    stout<BF16>(p.dpn, x, w * c.lprev);
    stout<BF16>(p.dk, x, c.vp / c.lam * c.dg + 2.f * c.k * c.vp * dc);
    stout<BF16>(p.dvp, x, c.k / c.lam * c.dg + c.k * c.k * dc);
    L = Llp * (c.a2 / (c.D * c.D));
  }
}

__global__ void kla_bwd_empty_kernel(const float* dlamT, const float* dMT, float* dlam0, float* dM0, long long nl,
                                     long long nm) {
  const long long x = (long long)blockIdx.x * 256 + threadIdx.x;
  if (x < nl) dlam0[x] = dlamT ? dlamT[x] : 0.f;
  if (x < nm) dM0[x] = dMT ? dMT[x] : 0.f;
}

// ---------------------------------------------------------------------------
// Launch sequence.
// ---------------------------------------------------------------------------
template <int K, int V, bool BF16>
static hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
  const unsigned nsb = (unsigned)((long long)p.nheads * p.nseg);
  hipLaunchKernelGGL((kla_bwd_segagg_kernel<K, V, BF16>), dim3(nsb), dim3(256), 0, stream, p);
  constexpr int NB = (K * V / 4 + 255) / 256;
  hipLaunchKernelGGL((kla_bwd_segscan_kernel<K, V>), dim3((unsigned)(p.nheads * NB)), dim3(256), 0, stream, p);
  hipLaunchKernelGGL((kla_bwd_chunk_kernel<K, V, BF16>), dim3(nsb), dim3(kChunkThreads), 0, stream, p);
  const int ncb = (int)((p.nchains + 255) / 256);
  const unsigned ncomp = (unsigned)((long long)ncb * p.nseg);
  hipLaunchKernelGGL((kla_bwd_chain_comp_kernel<BF16>), dim3(ncomp), dim3(256), 0, stream, p, K, ncb);
  hipLaunchKernelGGL(kla_bwd_chain_carry_kernel, dim3((unsigned)ncb), dim3(256), 0, stream, p);
  hipLaunchKernelGGL((kla_bwd_chain_out_kernel<BF16>), dim3(ncomp), dim3(256), 0, stream, p, K, ncb);
  return hipGetLastError();
}

template <int K, bool BF16>
static hipError_t bwd_dv(const BwdParams& p, int dv, hipStream_t stream) {
  switch (dv) {
    case 16: return launch_bwd<K, 16, BF16>(p, stream);
    case 32: return launch_bwd<K, 32, BF16>(p, stream);
    case 64: return launch_bwd<K, 64, BF16>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16>
static hipError_t bwd_dk(const BwdParams& p, int dk, int dv, hipStream_t stream) {
  switch (dk) {
    case 16: return bwd_dv<16, BF16>(p, dv, stream);
    case 32: return bwd_dv<32, BF16>(p, dv, stream);
    case 64: return bwd_dv<64, BF16>(p, dv, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_backward(const BwdParams& p, int dk, int dv, bool bf16, hipStream_t stream) {
  return bf16 ? bwd_dk<true>(p, dk, dv, stream) : bwd_dk<false>(p, dk, dv, stream);
}

hipError_t launch_backward_empty(const float* dlamT, const float* dMT, float* dlam0, float* dM0, long long nl,
                                 long long nm, hipStream_t stream) {
  const long long n = nl > nm ? nl : nm;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(kla_bwd_empty_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, dlamT, dMT,
                     dlam0, dM0, nl, nm);
  return hipGetLastError();
}

}  // namespace kla
