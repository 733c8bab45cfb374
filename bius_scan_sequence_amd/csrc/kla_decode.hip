// KLA decode step: one token per head.  The gates from the precision
// recursion, the affine posterior-mean update and the q readout, in one pass
// over the state.
//
// Sources: gist.science summaries of arXiv 2602.10743, "Kalman Linear Attention";
// [KLA-nl] = "Technische Samenvatting: Kalman Linear Attention (KLA)":
//   §1 "Probabilistische Formulering"      observation model; readout of the posterior mean
//   §2 "Parallelisatie via Möbius-transformaties"  precision equation; affine mean recursion
//   §3 "Niet-lineaire Gating vanuit Onzekerheid"   gates are precision ratios
//
// Decomposition.  One workgroup (256 threads) per head.  The state M [dk][dv]
// (fp32) is the only sizeable data and is streamed once: thread (row group
// rg, column group cg) owns columns 4cg .. 4cg+3 of rows rg, rg + RPP, ...,
// read and written as 16-byte units, so consecutive threads touch
// consecutive addresses.  The state loads are issued before the gates are
// formed (they do not depend on them).  The first dk threads form the gates
// of their channel; the readout sums the row groups' partial sums in a fixed
// order, so results are deterministic.
//
// In place: a thread reads each state element it writes, and nothing else,
// and thread i alone reads and writes lambda[i], so the state in and out may
// be the same buffers.
#include <type_traits>

#include "kla_device.h"
#include "kla_internal.h"

namespace kla {

template <int DK, int DV, bool BF16>
__global__ __launch_bounds__(256) void kla_decode_kernel(DecodeParams p) {
  using In = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int CW = DV / 4;                // 16-byte units per state row
  constexpr int RPP = 256 / CW;             // rows per pass
  constexpr int NRG = RPP < DK ? RPP : DK;  // row groups that own rows
  constexpr int NP = (DK + RPP - 1) / RPP;  // passes
  __shared__ float sf[DK], sg[DK], sq[DK];
  __shared__ alignas(16) float sv[DV];
  __shared__ float red[NRG * DV];

  const int tid = threadIdx.x;
  const size_t head = blockIdx.x;
  const int cg = tid % CW, rg = tid / CW;

  // State entering the token (the prior M = 0 when none is given).
  float4 m[NP];
#pragma unroll
  for (int r = 0; r < NP; ++r) {
    const int row = rg + r * RPP;
    m[r] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (p.M_in && row < DK) m[r] = reinterpret_cast<const float4*>(p.M_in + head * DK * DV)[row * CW + cg];
  }

  // Gates of channel tid: predict, update, precision ratios.
  if (tid < DK) {
    const size_t x = head * DK + tid;
    const float q = to_f32(static_cast<const In*>(p.q)[x]);
    const float k = to_f32(static_cast<const In*>(p.k)[x]);
    const float ld = to_f32(static_cast<const In*>(p.ld)[x]);
    const float pb = to_f32(static_cast<const In*>(p.pn)[x]);
    const float vp = to_f32(static_cast<const In*>(p.vp)[x]);
    const float lam = p.lam_in ? p.lam_in[x] : 1.f;
    const float a = __expf(ld);
    const float kv = k * vp;
    float lam_pred;
    const float lam_new = lam_step(lam, a * a, pb, k * kv, lam_pred);
    const float inv = fast_rcp(lam_new);
    sf[tid] = a * lam_pred * inv;
    sg[tid] = kv * inv;
    sq[tid] = q;
    p.lam_out[x] = lam_new;
  }
  if (tid < DV) sv[tid] = to_f32(static_cast<const In*>(p.v)[head * DV + tid]);
  __syncthreads();

  // M <- diag(f) M + g v^T, and this thread's share of y = q^T M.
  const float4 v4 = *reinterpret_cast<const float4*>(sv + 4 * cg);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float4* const Mo = reinterpret_cast<float4*>(p.M_out + head * DK * DV);
#pragma unroll
  for (int r = 0; r < NP; ++r) {
    const int row = rg + r * RPP;
    if (row < DK) {
      const float f = sf[row], g = sg[row], q = sq[row];
      const float4 n = make_float4(fmaf(f, m[r].x, g * v4.x), fmaf(f, m[r].y, g * v4.y),
                                   fmaf(f, m[r].z, g * v4.z), fmaf(f, m[r].w, g * v4.w));
      Mo[row * CW + cg] = n;
      acc.x = fmaf(q, n.x, acc.x);
      acc.y = fmaf(q, n.y, acc.y);
      acc.z = fmaf(q, n.z, acc.z);
      acc.w = fmaf(q, n.w, acc.w);
    }
  }
  if (rg < NRG) *reinterpret_cast<float4*>(red + rg * DV + 4 * cg) = acc;
  __syncthreads();
  if (tid < DV) {
    float y = 0.f;
#pragma unroll
    for (int g = 0; g < NRG; ++g) y += red[g * DV + tid];
    static_cast<In*>(p.y)[head * DV + tid] = from_f32<In>(y);
  }
}

template <int DK, int DV, bool BF16>
static hipError_t launch_dec(const DecodeParams& p, long long nheads, hipStream_t stream) {
  hipLaunchKernelGGL((kla_decode_kernel<DK, DV, BF16>), dim3((unsigned)nheads), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int DK, bool BF16>
static hipError_t dispatch_dv(const DecodeParams& p, long long nheads, int dv, hipStream_t stream) {
  switch (dv) {
    case 16: return launch_dec<DK, 16, BF16>(p, nheads, stream);
    case 32: return launch_dec<DK, 32, BF16>(p, nheads, stream);
    case 64: return launch_dec<DK, 64, BF16>(p, nheads, stream);
    case 128: return launch_dec<DK, 128, BF16>(p, nheads, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16>
static hipError_t dispatch_dk(const DecodeParams& p, long long nheads, int dk, int dv, hipStream_t stream) {
  switch (dk) {
    case 16: return dispatch_dv<16, BF16>(p, nheads, dv, stream);
    case 32: return dispatch_dv<32, BF16>(p, nheads, dv, stream);
    case 64: return dispatch_dv<64, BF16>(p, nheads, dv, stream);
    case 128: return dispatch_dv<128, BF16>(p, nheads, dv, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeParams& p, long long nheads, int dk, int dv, bool bf16, hipStream_t stream) {
  return bf16 ? dispatch_dk<true>(p, nheads, dk, dv, stream) : dispatch_dk<false>(p, nheads, dk, dv, stream);
}

}  // namespace kla
