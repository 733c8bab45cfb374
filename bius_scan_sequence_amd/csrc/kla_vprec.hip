// KLA with the value precision indexed by value channel: one scalar Kalman
// filter per element (i, j), each with its own precision.
//
// Sources: gist.science summaries of arXiv 2602.10743, "Kalman Linear Attention";
// [KLA-nl] = "Technische Samenvatting: Kalman Linear Attention (KLA)":
//   §1 "Probabilistische Formulering"  observation model (here Lambda^v per value channel j);
//                                      readout of the posterior mean
//   §2 "Parallelisatie via Möbius-transformaties"  precision equation; affine mean recursion
//   §3 "Niet-lineaire Gating vanuit Onzekerheid"   gates are precision ratios
// Per element (i, j) of head (b, h), token t (a = exp(log_decay_{t,i}),
// pbar = proc_noise_{t,i}, c_{t,ij} = k_{t,i}^2 Lambda^v_{t,j}):
//   lam^- = lam / (a^2 + pbar lam),  lam' = lam^- + c,
//   f = a lam^- / lam',  g = k_{t,i} Lambda^v_{t,j} / lam',
//   M' = f M + g v_{t,j},  y_t[j] = sum_i q_{t,i} M'_{ij}.
// The gates differ per element, so there is no chunked matrix form: the work
// is elementwise (VALU), O(T d_k d_v).
//
// Decomposition.  One workgroup per (head, block of 16 value columns); thread
// (ig, jj) owns key channels 2 ig and 2 ig + 1 of column jj and walks the
// sequence, two independent element chains per thread.  (Four chains per
// thread left one wave per SIMD at B8 H8 d64 and ran about 25% longer.)  The
// precision is kept projectively as lam = n / d (the Möbius form of [KLA-nl]
// §2):
//   d' = pbar n + a^2 d,  n' = n + c d',
// for which lam^- / lam' = n / n', so f = a n / n' and g = k Lambda^v d' / n'.
// The mean is kept as its numerator m = M n: M' = f M + g v becomes
//   m' = a m + k Lambda^v d' v,
// with no reciprocal on the recursion; the one reciprocal per element and
// token serves the readout M' = m' / n'.  (n, d, m) are rescaled by one
// power of two every fourth token (n / d and m / n are unchanged).  Tokens
// are staged in blocks: the per-(t, i) coefficients (a, pbar, k, q) once
// per block in LDS, v and Lambda^v per (t, j).  The readout's sum over key
// channels is deferred: each thread keeps its two-channel partial per token
// in LDS, and after the block one thread per (t, j) adds the d_k/2 partials in
// a fixed order (deterministic).
#include <type_traits>

#include "kla_device.h"
#include "kla_internal.h"

namespace kla {

namespace {
constexpr int kVR = 2;   // key channels per thread
constexpr int kVJB = 16;  // value columns per workgroup

template <int DK>
constexpr int vprec_tb() { return DK >= 128 ? 16 : 32; }  // tokens per staged block

// R consecutive fp32 values from LDS in one access.
template <int R>
__device__ __forceinline__ void lds_vals(const float* src, float (&x)[R]) {
  if constexpr (R == 4) {
    const float4 w = *reinterpret_cast<const float4*>(src);
    x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
  } else {
    static_assert(R == 2, "two or four key channels per thread");
    const float2 w = *reinterpret_cast<const float2*>(src);
    x[0] = w.x; x[1] = w.y;
  }
}

template <int DK, int DV, bool BF16>
struct alignas(16) VprecSmem {
  static constexpr int TB = vprec_tb<DK>(), NI = DK / kVR;
  float a[TB][DK], pn[TB][DK], k[TB][DK], q[TB][DK];
  float v[TB][kVJB], L[TB][kVJB];
  float part[TB][kVJB][NI + 1];  // padded: the reduction walks NI consecutive words
};
}  // namespace

template <int DK, int DV, bool BF16>
__global__ __launch_bounds__(DK / kVR * kVJB) void kla_vprec_kernel(VprecParams p) {
  using In = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int NI = DK / kVR, NT = NI * kVJB, TB = vprec_tb<DK>(), NJB = DV / kVJB;
  __shared__ VprecSmem<DK, DV, BF16> s;
  const int tid = threadIdx.x;
  const int ig = tid % NI, jj = tid / NI;
  const size_t head = blockIdx.x / NJB;
  const int j0 = (blockIdx.x % NJB) * kVJB;
  const int j = j0 + jj;
  const int T = p.T;
  const In* q = static_cast<const In*>(p.q);
  const In* k = static_cast<const In*>(p.k);
  const In* ld = static_cast<const In*>(p.ld);
  const In* pn = static_cast<const In*>(p.pn);
  const In* v = static_cast<const In*>(p.v);
  const In* vp = static_cast<const In*>(p.vp);

  // Element state: precision n/d and mean numerator m = M n, for channels
  // kVR ig + r of column j.
  float n[kVR], d[kVR], m[kVR];
#pragma unroll
  for (int r = 0; r < kVR; ++r) {
    const size_t e = (head * DK + ig * kVR + r) * DV + j;
    n[r] = p.lam0 ? p.lam0[e] : 1.f;
    d[r] = 1.f;
    m[r] = p.M0 ? p.M0[e] * n[r] : 0.f;
  }

  // The next block's raw inputs are loaded into registers while the current
  // block is computed (U1 coefficient and U2 value elements per thread).
  constexpr int U1 = (TB * DK + NT - 1) / NT, U2 = (TB * kVJB + NT - 1) / NT;
  In rld[U1], rpn[U1], rk[U1], rq[U1], rv[U2], rvp[U2];
  auto load_block = [&](int tb) {
#pragma unroll
    for (int u = 0; u < U1; ++u) {
      const int x = tid + u * NT, t = x / DK, i = x % DK;
      rld[u] = rpn[u] = rk[u] = rq[u] = In(0);
      if (x < TB * DK && tb + t < T) {
        const size_t g = (head * T + tb + t) * DK + i;
        rld[u] = ld[g];
        rpn[u] = pn[g];
        rk[u] = k[g];
        rq[u] = q[g];
      }
    }
#pragma unroll
    for (int u = 0; u < U2; ++u) {
      const int x = tid + u * NT, t = x / kVJB, c = x % kVJB;
      rv[u] = rvp[u] = In(0);
      if (x < TB * kVJB && tb + t < T) {
        const size_t g = (head * T + tb + t) * DV + j0 + c;
        rv[u] = v[g];
        rvp[u] = vp[g];
      }
    }
  };
  load_block(0);
  for (int t0 = 0; t0 < T; t0 += TB) {
    // Stage the block from the registers: per-(t, i) coefficients and
    // per-(t, j) values.  Tokens past T are identity steps (a = 1, pbar = 0,
    // k = 0: their zero log_decay gives a = 1).
#pragma unroll
    for (int u = 0; u < U1; ++u) {
      const int x = tid + u * NT, t = x / DK, i = x % DK;
      if (x < TB * DK) {
        const float av = __expf(to_f32(rld[u]));
        s.a[t][i] = av;
        s.pn[t][i] = to_f32(rpn[u]);
        s.k[t][i] = to_f32(rk[u]);
        s.q[t][i] = to_f32(rq[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < U2; ++u) {
      const int x = tid + u * NT, t = x / kVJB, c = x % kVJB;
      if (x < TB * kVJB) {
        s.v[t][c] = to_f32(rv[u]);
        s.L[t][c] = to_f32(rvp[u]);
      }
    }
    __syncthreads();
    if (t0 + TB < T) load_block(t0 + TB);
#pragma unroll 4
    for (int t = 0; t < TB; ++t) {
      const float vj = s.v[t][jj], Lj = s.L[t][jj];
      float av[kVR], a2v[kVR], pv[kVR], kv[kVR], qv[kVR];
      lds_vals<kVR>(&s.a[t][ig * kVR], av);
#pragma unroll
      for (int r = 0; r < kVR; ++r) a2v[r] = av[r] * av[r];
      lds_vals<kVR>(&s.pn[t][ig * kVR], pv);
      lds_vals<kVR>(&s.k[t][ig * kVR], kv);
      lds_vals<kVR>(&s.q[t][ig * kVR], qv);
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < kVR; ++r) {
        const float kL = kv[r] * Lj;
        const float c = kv[r] * kL;
        const float dd = fmaf(pv[r], n[r], a2v[r] * d[r]);  // d' = pbar n + a^2 d
        const float nn = fmaf(c, dd, n[r]);                 // n' = n + c d'
        m[r] = fmaf(av[r], m[r], kL * (dd * vj));           // m' = a m + k Lambda^v d' v
        part = fmaf(qv[r] * fast_rcp(nn), m[r], part);      // q M' = q m' / n'
        n[r] = nn;
        d[r] = dd;
      }
      if ((t & 3) == 3) {
#pragma unroll
        for (int r = 0; r < kVR; ++r) {
          const int e = __builtin_amdgcn_frexp_expf(fmaxf(n[r], d[r]));
          n[r] = __builtin_amdgcn_ldexpf(n[r], -e);
          d[r] = __builtin_amdgcn_ldexpf(d[r], -e);
          m[r] = __builtin_amdgcn_ldexpf(m[r], -e);
        }
      }
      s.part[t][jj][ig] = part;
    }
    __syncthreads();
    // y_t[j] = sum over the key-channel groups, in a fixed order.
    for (int x = tid; x < TB * kVJB; x += NT) {
      const int t = x / kVJB, c = x % kVJB;
      if (t0 + t >= T) continue;
      float y = 0.f;
#pragma unroll
      for (int g = 0; g < NI; ++g) y += s.part[t][c][g];
      static_cast<In*>(p.y)[(head * T + t0 + t) * DV + j0 + c] = from_f32<In>(y);
    }
    // The next staging writes only the coefficient and value arrays, which
    // every thread finished reading before the barrier above; the partials
    // are next written after the staging barrier.
  }
#pragma unroll
  for (int r = 0; r < kVR; ++r) {
    const size_t e = (head * DK + ig * kVR + r) * DV + j;
    p.lamT[e] = n[r] / d[r];
    p.MT[e] = m[r] / n[r];
  }
}

template <int DK, int DV, bool BF16>
static hipError_t launch_vp(const VprecParams& p, long long nheads, hipStream_t stream) {
  constexpr int NT = DK / kVR * kVJB;
  hipLaunchKernelGGL((kla_vprec_kernel<DK, DV, BF16>), dim3((unsigned)(nheads * (DV / kVJB))), dim3(NT), 0, stream,
                     p);
  return hipGetLastError();
}

template <int DK, bool BF16>
static hipError_t vp_dv(const VprecParams& p, long long nheads, int dv, hipStream_t stream) {
  switch (dv) {
    case 16: return launch_vp<DK, 16, BF16>(p, nheads, stream);
    case 32: return launch_vp<DK, 32, BF16>(p, nheads, stream);
    case 64: return launch_vp<DK, 64, BF16>(p, nheads, stream);
    case 128: return launch_vp<DK, 128, BF16>(p, nheads, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16>
static hipError_t vp_dk(const VprecParams& p, long long nheads, int dk, int dv, hipStream_t stream) {
  switch (dk) {
    case 16: return vp_dv<16, BF16>(p, nheads, dv, stream);
    case 32: return vp_dv<32, BF16>(p, nheads, dv, stream);
    case 64: return vp_dv<64, BF16>(p, nheads, dv, stream);
    case 128: return vp_dv<128, BF16>(p, nheads, dv, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_vprec(const VprecParams& p, long long nheads, int dk, int dv, bool bf16, hipStream_t stream) {
  return bf16 ? vp_dk<true>(p, nheads, dk, dv, stream) : vp_dk<false>(p, nheads, dk, dv, stream);
}

}  // namespace kla
