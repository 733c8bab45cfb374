// KLA forward scan: Möbius precision scan, precision-ratio gates, chunked
// gated posterior-mean recursion and q readout, fused in one kernel.
//
// Sources: gist.science summaries of arXiv 2602.10743, "Kalman Linear Attention";
// [KLA-nl] = "Technische Samenvatting: Kalman Linear Attention (KLA)":
//   §1 "Probabilistische Formulering"      model: OU prior, observation, readout
//   §2 "Parallelisatie via Möbius-transformaties"  precision equation; associative
//                                          composition; affine mean recursion
//   §3 "Niet-lineaire Gating vanuit Onzekerheid"   gates are precision ratios
//   §4 "Architectuur"                       expanded states never go to HBM
//
// Decomposition.  One workgroup (four wave64s; eight for bf16 at d_k = 128) owns one segment
// of L tokens of one head (b,h).  The segment's inputs are staged once in LDS.
//   1. Each walker thread (channel i, token group r) composes the 2x2 step
//      matrices of its tokens; the segment aggregate is the product of the
//      group aggregates.
//   2. Decoupled look-back over the head's earlier segments gives the
//      precision entering the segment (one 2x2 matrix or one float per
//      channel crosses workgroups).
//   3. The walk is repeated with the true entering precision to produce the
//      per-token gates f = a lam^-/lam and g = k Lambda^v / lam, folded into the
//      matrix-core operands of 16-token chunks, referred to the middle of the
//      chunk:
//        Qs = q * cp / F1,  Ks = g * F1 / cp,  Qg = q * cp * (prod of f over earlier chunks),
//        cp = in-chunk cumulative product of f, F1 = its value after the first
//        half, F2 = cp_end / F1 (Kd = g * prod_{w>u} f_w = Ks F2).
//   4. Chunk loop from a zero state: y_c = tril(Qs Ks^T) V + Qs (F1 M_c) and
//      M_{c+1} = diag(F2) (F1 M_c + Ks^T V), on 16x16 matrix-core tiles; the
//      state stays in accumulator registers, never in HBM.
//   5. Decoupled look-back of the mean carry (prod f over the segment, local
//      state), then y += Qg M_in and store.
// Every carry is folded forward in segment order with the same instructions,
// so results do not depend on which predecessor a look-back stops at.
//
// A chunk whose decay prod f over either half falls below 2^-64 on some
// channel could overflow Qs or Ks; such a chunk takes an exact scalar path for
// its intra-chunk scores instead (and chunk-start operands for the rest).
#include <type_traits>

#include "kla_device.h"
#include "kla_internal.h"

namespace kla {

#ifdef KLA_TIMELINE
// Timeline build only (-DKLA_TIMELINE): the first thread of every workgroup
// of the segmented kernel records the 100 MHz real-time counter at the start
// of each section, into kla_seg_timeline_buf[workgroup][slot]: 0 entry, 1
// ticket read, 2 inputs staged, 3 chunk aggregates done, 4 precision carry
// done, 5 gate walk done, 6 scores done, 7 chunk loop done, 8 mean carry done,
// 9 end; values: 10 segment, 11 segments the mean look-back folded (0: none).
constexpr int kStlSlots = 16, kStlGroups = 16384;
__device__ unsigned long long kla_seg_timeline_buf[kStlGroups * kStlSlots];
#define KLA_SSTAMP(k)                                                                               \
  do {                                                                                              \
    if (threadIdx.x == 0 && blockIdx.x < (unsigned)kStlGroups)                                      \
      kla_seg_timeline_buf[(size_t)blockIdx.x * kStlSlots + (k)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#define KLA_SVALUE(k, v)                                                                             \
  do {                                                                                               \
    if (threadIdx.x == 0 && blockIdx.x < (unsigned)kStlGroups)                                       \
      kla_seg_timeline_buf[(size_t)blockIdx.x * kStlSlots + (k)] = (unsigned long long)(v);          \
  } while (0)
#else
#define KLA_SSTAMP(k) \
  do {                \
  } while (0)
#define KLA_SVALUE(k, v) \
  do {                   \
  } while (0)
#endif

template <int DK, int DV, bool BF16>
struct FwdCfg {
  using In = typename std::conditional<BF16, uint16_t, float>::type;
  static constexpr int L = (BF16 || (DK <= 64 && DV <= 64)) ? 64 : 32;  // tokens per segment
  // Waves per workgroup: eight for bf16 at d_k = 128 (two walker waves per
  // chunk and one state column tile per wave keep the registers of a lane
  // within 256, so two waves share each SIMD), else four.
  static constexpr int NW = (BF16 && DK == 128) ? 8 : 4;
  static constexpr int NT = 64 * NW;                                    // threads
  static constexpr int NCH = L / 16;                                    // 16-token chunks
  // Walkers: one thread per (channel group of CPT channels, half chunk of 8
  // tokens); wave w walks chunk w % 4 (channel part w / 4), the halves of the
  // chunk in lanes l and l ^ 32.
  static constexpr int WPC = NW / 4;                                    // walker waves per chunk
  static constexpr int CPT = DK >= 64 ? DK / (32 * WPC) : 1;            // channels per walker
  static_assert(NCH <= 4, "one walker wave group per chunk");
  static constexpr int NRT = DK / 16;                                   // state row tiles
  static constexpr int NCT = DV / 16;                                   // state col tiles
  static constexpr int CPW = (NCT + NW - 1) / NW;                       // col tiles per wave
  // Stored operands: 16 bytes per 4 consecutive values (bf16: [hi x4 | lo x4];
  // fp32: the 4 values), rows padded by 16 bytes against bank conflicts.
  static constexpr int QROW = DK * 4 + 16;                              // Qs / Ks row (bytes)
  static constexpr int KROW = L * 4 + 16;                               // Kd^T row (bytes)
  // bf16: the chunk recursion reads Ks^T straight from the Ks rows with
  // transposing LDS loads; fp32 keeps a separate Kd^T copy.
  static constexpr bool KST = BF16;
  static constexpr int RAW_BYTES = 5 * L * DK * (int)sizeof(In);        // q, k, ld, pn, vp
  static constexpr int OPS_BYTES = 3 * L * QROW + (KST ? 0 : DK * KROW);  // Qs, Ks, Qg[, Kd^T]
  // The local readout Qs_c (F1_c M_c) waits until the local state has been published
  // (it then overlaps that publication and the first flag poll) when the local
  // chunk states fit in registers (NRT*CPW <= 4 tiles per lane); otherwise it
  // runs in the chunk loop.
  static constexpr bool LATE_LOCAL = NRT * CPW <= 4;
  static constexpr int UNION_BYTES = RAW_BYTES > OPS_BYTES ? RAW_BYTES : OPS_BYTES;
  static constexpr int A_BYTES = NCH * 64 * 16;                         // per chunk: scores, A-operand order
  static constexpr int RED_BYTES = 2 * 256 * 4;                         // exact path: per-wave partial sums
  static_assert(DK <= 128, "exact-path partial sums: at most two channel waves");
  static constexpr int CAGG_BYTES = NCH * DK * 16;                      // chunk 2x2 aggregates
  // Once the gate walk is done, the raw tiles beyond the stored operands are
  // free: the scores and the exact path's partial sums go there if they fit.
  static constexpr bool TAIL = RAW_BYTES - OPS_BYTES >= A_BYTES + RED_BYTES;
  // The chunk aggregates are needed only until the precision carry is done,
  // before v is staged: they use v's space when it is large enough.
  static constexpr bool CAGG_IN_V = CAGG_BYTES <= L * DV * (int)sizeof(In);
  static constexpr int AP_A = TAIL ? 0 : A_BYTES, AP_C = CAGG_IN_V ? 0 : CAGG_BYTES;
  static constexpr int AP_BYTES = (AP_A > AP_C ? AP_A : AP_C) > 16 ? (AP_A > AP_C ? AP_A : AP_C) : 16;
  // The walkers keep a, pbar, c, k*Lambda^v in registers between the two
  // walks when they own at most 16 token-channels.
  static constexpr bool KEEP = 8 * CPT <= 16;
};

template <int DK, int DV, bool BF16>
struct FwdSmem {
  using C = FwdCfg<DK, DV, BF16>;
  using In = typename C::In;
  // Raw inputs q, k, ld, pn, vp ([L][DK] each) until the gate walk is done;
  // afterwards the stored operands Qs [L][QROW], Ks [L][QROW] (Kd in the rows
  // of an unsafe chunk when KST), Qg [L][QROW] and, without KST, Kd^T [DK][KROW].
  alignas(16) unsigned char u[C::UNION_BYTES];
  // Chunk 2x2 aggregates until the precision carry is done (when CAGG_IN_V),
  // then raw v; staged y at the end.
  alignas(16) In v[C::L * DV];
  // Chunk aggregates and / or the causal intra-chunk scores of every chunk in
  // A-operand order, for the parts that have no place elsewhere.
  alignas(16) unsigned char ap[C::AP_BYTES];
  alignas(16) float cpe[C::NCH * DK];      // per chunk: prod of f over the chunk
  // Per chunk: the reference of its scores (prod of f over the first half, or
  // 1 for an unsafe chunk) and the factor that takes the state, once the
  // chunk's keys are added, to the chunk end (prod of f over the second half,
  // or cpe for an unsafe chunk); with KST, a safe chunk's cp2 then also takes
  // the next chunk's reference (folded in before the chunk loop).
  alignas(16) float cpm[C::NCH * DK];
  alignas(16) float cp2[C::NCH * DK];
  float lamc[C::NCH * DK];                 // per chunk: precision entering the chunk
  alignas(16) float fseg[DK];              // prod of f over the segment
  float red[C::TAIL ? 4 : C::RED_BYTES / 4];
  // Coefficient prologue: the three raw rows before the segment of xq, xk, xv.
  alignas(16) In halo[3 * (2 * DK + DV)];
  int unsafe[C::NCH];
  int ctl[4];

  __device__ In* raw(int which) { return reinterpret_cast<In*>(u) + which * C::L * DK; }
  __device__ float* cagg() { return C::CAGG_IN_V ? reinterpret_cast<float*>(v) : reinterpret_cast<float*>(ap); }
  __device__ unsigned char* scores() { return C::TAIL ? u + C::OPS_BYTES : ap; }
  __device__ float* partial() { return C::TAIL ? reinterpret_cast<float*>(u + C::OPS_BYTES + C::A_BYTES) : red; }
};

// Copy one [rows x width] tile between global memory and LDS (16-byte units;
// width*sizeof(In) is a multiple of 32 bytes for every supported width).
// Loads zero rows past `nvalid`: zeros are an identity filter step (a = 1,
// pbar = 0, c = 0) and contribute nothing to y.
template <typename In, int ROWS, int WIDTH, int NT>
__device__ __forceinline__ void stage_tile(In* dst, const In* src, int nvalid, int tid) {
  constexpr int UNITS = ROWS * WIDTH * (int)sizeof(In) / 16;
  constexpr int PER_UNIT = 16 / (int)sizeof(In);
  const int valid_units = nvalid * WIDTH / PER_UNIT;
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
  uint4* d4 = reinterpret_cast<uint4*>(dst);
  uint4 buf[(UNITS + NT - 1) / NT];
#pragma unroll
  for (int it = 0; it < (UNITS + NT - 1) / NT; ++it) {
    int u = tid + it * NT;
    buf[it] = (u < valid_units) ? s4[u] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int it = 0; it < (UNITS + NT - 1) / NT; ++it) {
    int u = tid + it * NT;
    if (u < UNITS) d4[u] = buf[it];
  }
}
// The two halves of stage_tile, for overlapping a load with other work.
template <typename In, int ROWS, int WIDTH, int NT>
__device__ __forceinline__ void load_tile(uint4 (&buf)[(ROWS * WIDTH * (int)sizeof(In) / 16 + NT - 1) / NT],
                                          const In* src, int nvalid, int tid) {
  constexpr int UNITS = ROWS * WIDTH * (int)sizeof(In) / 16;
  constexpr int PER_UNIT = 16 / (int)sizeof(In);
  const int valid_units = nvalid * WIDTH / PER_UNIT;
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
#pragma unroll
  for (int it = 0; it < (UNITS + NT - 1) / NT; ++it) {
    int u = tid + it * NT;
    buf[it] = (u < valid_units) ? s4[u] : make_uint4(0, 0, 0, 0);
  }
}
template <typename In, int ROWS, int WIDTH, int NT>
__device__ __forceinline__ void store_tile(In* dst, const uint4 (&buf)[(ROWS * WIDTH * (int)sizeof(In) / 16 + NT - 1) / NT],
                                           int tid) {
  constexpr int UNITS = ROWS * WIDTH * (int)sizeof(In) / 16;
  uint4* d4 = reinterpret_cast<uint4*>(dst);
#pragma unroll
  for (int it = 0; it < (UNITS + NT - 1) / NT; ++it) {
    int u = tid + it * NT;
    if (u < UNITS) d4[u] = buf[it];
  }
}
template <typename In, int ROWS, int WIDTH, int NT>
__device__ __forceinline__ void unstage_tile(In* dst, const In* src, int nvalid, int tid) {
  constexpr int PER_UNIT = 16 / (int)sizeof(In);
  const int valid_units = nvalid * WIDTH / PER_UNIT;
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
  uint4* d4 = reinterpret_cast<uint4*>(dst);
  for (int u = tid; u < valid_units; u += NT) d4[u] = s4[u];
}

__device__ __forceinline__ v4f ld4(const float* p) { return *reinterpret_cast<const v4f*>(p); }

// Sum over the 64 lanes of a wave, in a fixed order.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// One stored value of a 4-value block: bf16 hi at byte 2*j, lo at 8 + 2*j;
// fp32 at byte 4*j.
template <bool BF16>
__device__ __forceinline__ void put1(unsigned char* block, int j, float x) {
  if constexpr (BF16) {
    const uint16_t h = bf16_rne(x);
    reinterpret_cast<uint16_t*>(block)[j] = h;
    reinterpret_cast<uint16_t*>(block)[4 + j] = bf16_rne(x - to_f32(h));
  } else {
    reinterpret_cast<float*>(block)[j] = x;
  }
}

// CPT consecutive input values (CPT * sizeof(In)-aligned) as floats.
template <int CPT>
__device__ __forceinline__ void load_vals(const uint16_t* p, float (&o)[CPT]) {
  if constexpr (CPT == 1) {
    o[0] = to_f32(p[0]);
  } else if constexpr (CPT == 2) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    o[0] = __uint_as_float(w << 16);
    o[1] = __uint_as_float(w & 0xffff0000u);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    o[0] = __uint_as_float(w.x << 16);
    o[1] = __uint_as_float(w.x & 0xffff0000u);
    o[2] = __uint_as_float(w.y << 16);
    o[3] = __uint_as_float(w.y & 0xffff0000u);
  }
}
template <int CPT>
__device__ __forceinline__ void load_vals(const float* p, float (&o)[CPT]) {
#pragma unroll
  for (int k = 0; k < CPT; ++k) o[k] = p[k];
}

// Exact discretisation of an OU step of length dt with rate theta and
// diffusion sigma2 ([KLA-nl] §1, "Dynamics Prior": the prior is an exactly
// discretised OU process): x_t = e^{-theta dt} x_{t-1} + w with
// Var w = sigma2 (1 - e^{-2 theta dt}) / (2 theta) = sigma2 dt phi(2 theta dt),
// phi(u) = (1 - e^{-u}) / u (phi -> 1 as theta -> 0, the Brownian step).
// For |u| > 0.5, phi = (1 - a^2) / u with a = e^{-theta dt}, the decay the
// walk forms anyway (the cancellation in 1 - a^2 costs well under 1e-6
// relative there); below, the series sum_{n<=7} (-u)^n / (n+1)! (error
// below u^8/9!, about 1e-8).  Both forms are evaluated and one is selected,
// so a wave whose lanes fall on both sides runs no branch; the decay a is
// returned for the walk.
__device__ __forceinline__ float ou_coef(float th, float s2, float dt, float& ld, float& pn) {
  const float x = th * dt;
  ld = -x;
  const float a = __expf(ld);
  const float u = 2.f * x;
  float s = -1.f / 40320.f;                   // (-1)^7 / 8!
  s = fmaf(u, s, 1.f / 5040.f);
  s = fmaf(u, s, -1.f / 720.f);
  s = fmaf(u, s, 1.f / 120.f);
  s = fmaf(u, s, -1.f / 24.f);
  s = fmaf(u, s, 1.f / 6.f);
  s = fmaf(u, s, -0.5f);
  const float phi = fabsf(u) > 0.5f ? (1.f - a * a) * fast_rcp(u) : fmaf(u, s, 1.f);
  pn = s2 * dt * phi;
  return a;
}

// Input modes of the kernel: log_decay and proc_noise given per token
// (kPlain); the OU prior in continuous time, discretised per token (kOU); the
// OU prior behind the coefficient prologue (kPrologue: raw projections and
// raw coefficients, see below).
enum FwdMode { kPlain = 0, kOU = 1, kPrologue = 2 };

// Coefficient prologue of the Mamba-like block ([KLA-nl] §4 "Architectuur":
// the scan sits between causal 1D convolutions with SiLU activations):
// q, k, v = SiLU(causal depthwise conv1d of the raw projections), stored in the
// input dtype; the step length and the value precision are softplus of their
// raw values, formed in fp32 where they are used.
// softplus(x) = max(x, 0) + log1p(e) with e = e^{-|x|} in (0, 1], and
// log1p(e) = 2 atanh(z) = 2 z (1 + z^2/3 + z^4/5 + ...), z = e / (2 + e) <= 1/3:
// terms to z^12/13 leave a relative error below 2e-8 (branch-free, unlike the
// library log1pf).
__device__ __forceinline__ float softplus_f(float x) {
  const float e = __expf(-fabsf(x));
  const float z = e * fast_rcp(2.f + e), z2 = z * z;
  float t = 1.f / 13.f;
  t = fmaf(t, z2, 1.f / 11.f);
  t = fmaf(t, z2, 1.f / 9.f);
  t = fmaf(t, z2, 1.f / 7.f);
  t = fmaf(t, z2, 1.f / 5.f);
  t = fmaf(t, z2, 1.f / 3.f);
  t = fmaf(t, z2, 1.f);
  return fmaxf(x, 0.f) + 2.f * z * t;
}
__device__ __forceinline__ float silu_f(float u) { return u * fast_rcp(1.f + __expf(-u)); }

// Convolution taps of channels c0 .. c0 + N - 1 (weights [d][W] of one head,
// W <= 4) as four slots, slot j multiplying the token 3 - j steps back; slots
// before the first tap hold zero.
template <int N>
__device__ __forceinline__ void conv_slots(const float* w, const float* b, int W, int c0, float (&ws)[N][4],
                                           float (&bs)[N]) {
  // One uniform branch per set (not per channel); the loads of the general
  // width are clamped into the channel's taps and then selected.
  if (W == 4) {
#pragma unroll
    for (int c = 0; c < N; ++c) {
      const float4 v = *reinterpret_cast<const float4*>(w + (size_t)(c0 + c) * 4);
      ws[c][0] = v.x; ws[c][1] = v.y; ws[c][2] = v.z; ws[c][3] = v.w;
    }
  } else {
#pragma unroll
    for (int c = 0; c < N; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tap = j - (4 - W);
        const float v = w[(size_t)(c0 + c) * W + (tap > 0 ? tap : 0)];
        ws[c][j] = tap >= 0 ? v : 0.f;
      }
  }
  if (b) {
#pragma unroll
    for (int c = 0; c < N; ++c) bs[c] = b[c0 + c];
  } else {
#pragma unroll
    for (int c = 0; c < N; ++c) bs[c] = 0.f;
  }
}

// Values of one 16-byte unit as floats, and back (bf16: round to nearest even).
template <typename In>
__device__ __forceinline__ void unpack_unit(const uint4& u, float (&x)[16 / sizeof(In)]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  if constexpr (sizeof(In) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
  }
}
template <typename In>
__device__ __forceinline__ uint4 pack_unit(const float (&x)[16 / sizeof(In)]) {
  uint32_t w[4];
  if constexpr (sizeof(In) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __builtin_bit_cast(uint32_t, bf16x2(x[2 * i], x[2 * i + 1]));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(x[i]);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// The three raw rows before a tile (tokens t0 - 3 .. t0 - 1; zero before the
// sequence start) from global memory into LDS, [3][WIDTH].
template <typename In, int WIDTH, int NT>
__device__ __forceinline__ void stage_halo(In* dst, const In* src, int t0, int tid) {
  constexpr int PER = 16 / (int)sizeof(In), UPR = WIDTH / PER;
  static_assert(3 * UPR <= NT, "one unit per thread");
  if (tid < 3 * UPR) {
    const int r = tid / UPR, c0 = (tid % UPR) * PER;
    const bool ok = t0 - 3 + r >= 0;
    reinterpret_cast<uint4*>(dst)[tid] =
        ok ? *reinterpret_cast<const uint4*>(src + (ptrdiff_t)(r - 3) * WIDTH + c0) : make_uint4(0, 0, 0, 0);
  }
}

// SiLU of the causal convolution over a staged [ROWS x WIDTH] raw tile (rows
// r < 0 in `halo`), for rows r < nvalid; rows past nvalid are zero.  The
// result, in the input dtype, is left in registers in store_tile's unit
// order.  Each thread's units share one channel group, so it loads its taps
// once.
template <typename In, int ROWS, int WIDTH, int NT>
__device__ __forceinline__ void conv_lds(uint4 (&buf)[(ROWS * WIDTH * (int)sizeof(In) / 16 + NT - 1) / NT],
                                         const In* tile, const In* halo, int nvalid, const float* w, const float* b,
                                         int W, int tid) {
  constexpr int PER = 16 / (int)sizeof(In), UPR = WIDTH / PER, UNITS = ROWS * UPR;
  constexpr int U = (UNITS + NT - 1) / NT;
  static_assert(NT % UPR == 0, "a thread's units must share their channels");
  const int c0 = (tid % UPR) * PER;
  float ws[PER][4], bs[PER];
  conv_slots<PER>(w, b, W, c0, ws, bs);
#pragma unroll
  for (int it = 0; it < U; ++it) {
    const int u = tid + it * NT, r = u / UPR;
    const bool live = u < UNITS && r < nvalid;
    float acc[PER];
#pragma unroll
    for (int c = 0; c < PER; ++c) acc[c] = bs[c];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rr = min(r - 3 + j, ROWS - 1);  // (units past the tile read its last row, unused)
      float x[PER];
      // Always in bounds (rr >= -3; rows past nvalid and before the sequence
      // start are staged as zero), so read unconditionally: a slot before the
      // first tap has weight zero, and a row past nvalid gives no output.
      const uint4 raw = *reinterpret_cast<const uint4*>(rr >= 0 ? tile + rr * WIDTH + c0 : halo + (rr + 3) * WIDTH + c0);
      unpack_unit<In>(raw, x);
#pragma unroll
      for (int c = 0; c < PER; ++c) acc[c] = fmaf(ws[c][j], x[c], acc[c]);
    }
#pragma unroll
    for (int c = 0; c < PER; ++c) acc[c] = live ? silu_f(acc[c]) : 0.f;
    buf[it] = pack_unit<In>(acc);
  }
}

// The same activations for one channel over one 16-token chunk whose first
// row is tile row r0 (x points at the channel's raw value in that row, rows
// `stride` apart; tg0 is that row's token in the sequence), with the
// instructions of conv_lds: the 19 raw values of the window are loaded once
// (rows before the sequence start or past nvalid read as zero), and the
// results are rounded to the input dtype.
template <typename In>
__device__ __forceinline__ void conv_chunk(float (&out)[16], const In* x, int stride, int tg0, int r0, int nvalid,
                                           const float (&ws)[4], float b) {
  float win[19];
#pragma unroll
  for (int i = 0; i < 19; ++i) {
    const int r = r0 - 3 + i;  // tile row
    const bool ok = tg0 - 3 + i >= 0 && r < nvalid;
    // Rows out of range are read at row r0 (in bounds) and replaced by zero.
    const float raw = to_f32(x[ok ? (ptrdiff_t)(i - 3) * stride : 0]);
    win[i] = ok ? raw : 0.f;
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float acc = b;
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = fmaf(ws[j], win[e + j], acc);
    out[e] = r0 + e < nvalid ? to_f32(from_f32<In>(silu_f(acc))) : 0.f;
  }
}

// log_decay, proc_noise and val_prec of CPT channels of one token: read from
// the staged tiles; or (OU) log_decay and proc_noise formed from the staged
// step length and the channels' theta and sigma2; or (prologue) the same
// after softplus of the staged raw step length and value precision.  A token
// past the end (tv false) is an identity step: zero step length and value
// precision.
template <int MODE, int CPT, typename In>
__device__ __forceinline__ void coef_vals(const In* rld, const In* rpn, const In* rvp, const float (&th)[CPT],
                                          const float (&s2)[CPT], bool tv, float (&av)[CPT], float (&pnv)[CPT],
                                          float (&vpv)[CPT]) {
  float ldv[CPT];
  load_vals<CPT>(rvp, vpv);
  if constexpr (MODE == kPrologue) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) vpv[k] = tv ? softplus_f(vpv[k]) : 0.f;
  }
  if constexpr (MODE != kPlain) {
    float dt[CPT];
    load_vals<CPT>(rld, dt);
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      float d = dt[k];
      if constexpr (MODE == kPrologue) d = tv ? softplus_f(d) : 0.f;
      av[k] = ou_coef(th[k], s2[k], d, ldv[k], pnv[k]);
    }
  } else {
    load_vals<CPT>(rld, ldv);
    load_vals<CPT>(rpn, pnv);
#pragma unroll
    for (int k = 0; k < CPT; ++k) av[k] = __expf(ldv[k]);
  }
}

// CPT consecutive stored values starting at slot j of a 4-value block (see put1).
template <bool BF16, int CPT>
__device__ __forceinline__ void put_vals(unsigned char* block, int j, const float (&x)[CPT]) {
  if constexpr (CPT == 1) {
    put1<BF16>(block, j, x[0]);
  } else if constexpr (BF16 && CPT == 2) {
    const v2s h = bf16x2(x[0], x[1]);
    const v2s l = bf16x2(x[0] - to_f32((uint16_t)h[0]), x[1] - to_f32((uint16_t)h[1]));
    *reinterpret_cast<v2s*>(block + 2 * j) = h;
    *reinterpret_cast<v2s*>(block + 8 + 2 * j) = l;
  } else if constexpr (BF16) {
    Mma<true>::put(block, v4f{x[0], x[1], x[2], x[3]});
  } else {
#pragma unroll
    for (int k = 0; k < CPT; ++k) reinterpret_cast<float*>(block)[j + k] = x[k];
  }
}

// Waves per SIMD the kernel is compiled for: two workgroups per compute unit
// when two fit in LDS, else one, times the workgroup's waves per SIMD (two
// waves per SIMD allow at most 256 registers per lane).  (Three
// fit in LDS at d = 64 but were slower: the 168-register budget spills and
// twelve segments of a head in flight deepen the look-backs.)
template <int DK, int DV, bool BF16>
constexpr int fwd_waves_per_eu() {
  return (sizeof(FwdSmem<DK, DV, BF16>) <= 80 * 1024 ? 2 : 1) * FwdCfg<DK, DV, BF16>::NW / 4;
}

template <int DK, int DV, bool BF16, int MODE>
__global__ __launch_bounds__((FwdCfg<DK, DV, BF16>::NT), (fwd_waves_per_eu<DK, DV, BF16>())) void kla_fwd_kernel(FwdParams p) {
  using C = FwdCfg<DK, DV, BF16>;
  using In = typename C::In;
  using M = Mma<BF16>;
  using Op = typename M::Op;
  constexpr int L = C::L, NCH = C::NCH, CPT = C::CPT, NW = C::NW, NT = C::NT;
  constexpr int NRT = C::NRT, NCT = C::NCT, CPW = C::CPW, QROW = C::QROW, KROW = C::KROW;
  constexpr bool OU = MODE != kPlain;
  __shared__ FwdSmem<DK, DV, BF16> s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lc = lane & 15;  // lane group (k block) / lane column
  const int nheads = p.nheads, T = p.T, nseg = p.nseg;
  KLA_SSTAMP(0);
  // The inputs of the (head, segment) the workgroup index predicts are
  // requested before the ticket is drawn (workgroups of a group mostly draw
  // their tickets in index order); a wrong guess costs only these loads.
  constexpr int UK = (L * DK * (int)sizeof(In) / 16 + NT - 1) / NT, UV = (L * DV * (int)sizeof(In) / 16 + NT - 1) / NT;
  uint4 gq[UK], gv[UV], gk[UK], gld[UK], gpn[UK], gvp[UK];
  int g_seg = -1, g_head = -1;
  {
    const unsigned tgg = nseg > 1 ? (unsigned)p.tgroups : 1u, hpgg = (unsigned)nheads / tgg;
    const unsigned gt = nseg > 1 ? blockIdx.x / tgg : blockIdx.x;
    g_seg = (int)(gt / hpgg);
    g_head = (int)((gt % hpgg) * tgg + blockIdx.x % tgg);
    const int gnv = min(L, T - g_seg * L);
    const size_t gko = ((size_t)g_head * T + (size_t)g_seg * L) * DK, gvo = ((size_t)g_head * T + (size_t)g_seg * L) * DV;
    load_tile<In, L, DK, NT>(gq, static_cast<const In*>(p.q) + gko, gnv, tid);
    load_tile<In, L, DV, NT>(gv, static_cast<const In*>(p.v) + gvo, gnv, tid);
    load_tile<In, L, DK, NT>(gk, static_cast<const In*>(p.k) + gko, gnv, tid);
    load_tile<In, L, DK, NT>(gld, static_cast<const In*>(p.ld) + gko, gnv, tid);
    if constexpr (MODE == kPlain) load_tile<In, L, DK, NT>(gpn, static_cast<const In*>(p.pn) + gko, gnv, tid);
    load_tile<In, L, DK, NT>(gvp, static_cast<const In*>(p.vp) + gko, gnv, tid);
  }
  // (head, segment) from a ticket when segments wait on predecessors: group
  // x = blockIdx % tgroups serves heads x, x + tgroups, ..., segment-major, so
  // every segment a workgroup waits on holds a smaller ticket of its own
  // counter and started earlier.
  if (nseg > 1 && tid == 0)
    s.ctl[2] = (int)draw_ticket(p.tick, (unsigned)p.tgroups, (unsigned)nheads / (unsigned)p.tgroups * (unsigned)nseg);
  if (tid == 0) s.ctl[1] = nseg > 1 ? (int)ld_relaxed(p.ctrl + kEpoch) : 0;
  if (nseg > 1) __syncthreads();
  const unsigned ticket = nseg > 1 ? (unsigned)s.ctl[2] : blockIdx.x;
  const unsigned tg = nseg > 1 ? (unsigned)p.tgroups : 1u, hpg = (unsigned)nheads / tg;
  const int seg = (int)(ticket / hpg), head = (int)((ticket % hpg) * tg + blockIdx.x % tg);
  const int t0 = seg * L;
  const int nvalid = min(L, T - t0);
  const bool last = (seg == nseg - 1);
  const size_t hs = (size_t)head * nseg + seg;  // (head, segment) slot
  KLA_SSTAMP(1);
  KLA_SVALUE(10, seg);
  const size_t hb = (size_t)head * nseg;

  if (tid < NCH) s.unsafe[tid] = 0;

  In* const rq = s.raw(0);
  In* const rk = s.raw(1);
  In* const rld = s.raw(2);
  In* const rpn = s.raw(3);
  In* const rvp = s.raw(4);

  // ---------------------------------------------------------------- stage inputs
  // All six tiles are requested at once; the coefficient tiles are written to
  // LDS first and q, v only after the aggregate walk, so their load latency
  // overlaps the walk.
  const size_t offk = ((size_t)head * T + t0) * DK, offv = ((size_t)head * T + t0) * DV;
  uint4 bq[UK], bv[UV];
  if constexpr (MODE == kPrologue) {
    // q, k, v are SiLU(conv) of the raw projections.  The raw tiles go to LDS
    // once (xk in the proc_noise slot, which this mode leaves free; xq and xv
    // in their own slots, written after the aggregate walk as in the other
    // modes), with the three rows before the segment beside them.  The
    // walkers form k from the raw rows as they start the aggregate walk
    // (section 1); q and v are formed during the precision carry by the waves
    // that do not carry (section 2).  k itself is never stored, so the chunk
    // aggregates go to k's slot.
    In* const hk = s.halo + 3 * DK;
    if (seg == g_seg && head == g_head) {  // the guess was right: the tiles are in flight
#pragma unroll
      for (int u = 0; u < UK; ++u) bq[u] = gq[u];
#pragma unroll
      for (int u = 0; u < UV; ++u) bv[u] = gv[u];
      store_tile<In, L, DK, NT>(rpn, gk, tid);
    } else {
      load_tile<In, L, DK, NT>(bq, static_cast<const In*>(p.q) + offk, nvalid, tid);
      load_tile<In, L, DV, NT>(bv, static_cast<const In*>(p.v) + offv, nvalid, tid);
      stage_tile<In, L, DK, NT>(rpn, static_cast<const In*>(p.k) + offk, nvalid, tid);
    }
    stage_halo<In, DK, NT>(hk, static_cast<const In*>(p.k) + offk, t0, tid);
    stage_halo<In, DK, NT>(s.halo, static_cast<const In*>(p.q) + offk, t0, tid);
    stage_halo<In, DV, NT>(s.halo + 6 * DK, static_cast<const In*>(p.v) + offv, t0, tid);
    if (seg == g_seg && head == g_head) {
      store_tile<In, L, DK, NT>(rld, gld, tid);  // raw step length
      store_tile<In, L, DK, NT>(rvp, gvp, tid);  // raw value precision
    } else {
      stage_tile<In, L, DK, NT>(rld, static_cast<const In*>(p.ld) + offk, nvalid, tid);  // raw step length
      stage_tile<In, L, DK, NT>(rvp, static_cast<const In*>(p.vp) + offk, nvalid, tid);  // raw value precision
    }
  } else if (seg == g_seg && head == g_head) {  // the guess was right: the tiles are in flight
#pragma unroll
    for (int u = 0; u < UK; ++u) bq[u] = gq[u];
#pragma unroll
    for (int u = 0; u < UV; ++u) bv[u] = gv[u];
    store_tile<In, L, DK, NT>(rk, gk, tid);
    store_tile<In, L, DK, NT>(rld, gld, tid);
    if constexpr (!OU) store_tile<In, L, DK, NT>(rpn, gpn, tid);
    store_tile<In, L, DK, NT>(rvp, gvp, tid);
  } else {
    load_tile<In, L, DK, NT>(bq, static_cast<const In*>(p.q) + offk, nvalid, tid);
    load_tile<In, L, DV, NT>(bv, static_cast<const In*>(p.v) + offv, nvalid, tid);
    stage_tile<In, L, DK, NT>(rk, static_cast<const In*>(p.k) + offk, nvalid, tid);
    stage_tile<In, L, DK, NT>(rld, static_cast<const In*>(p.ld) + offk, nvalid, tid);  // OU: the step length
    if constexpr (!OU) stage_tile<In, L, DK, NT>(rpn, static_cast<const In*>(p.pn) + offk, nvalid, tid);
    stage_tile<In, L, DK, NT>(rvp, static_cast<const In*>(p.vp) + offk, nvalid, tid);
  }
  __syncthreads();
  const unsigned epoch = (unsigned)s.ctl[1];
  const unsigned FAGG = 2u * epoch + 2u, FINC = 2u * epoch + 3u;
  // The precision carry waves ask for the predecessor's inclusive precision
  // record now; if it has been published by the end of the aggregate walk,
  // the look-back is skipped (see section 2).
  constexpr int PW = (DK + 63) / 64;  // precision carry waves
  const bool pwave = wave < PW, pch = tid < DK;
  // Chunk 2x2 aggregates: in v's space (or the spare operand area); with the
  // prologue in k's slot, since raw xv goes to v's space before the carry.
  float* const cagg = MODE == kPrologue ? reinterpret_cast<float*>(rk) : s.cagg();
  unsigned long long early = 0ull;
  if (pwave && pch && seg > 0) early = ld_record(p.pinc + (hb + seg - 1) * DK + tid);

  KLA_SSTAMP(2);
  // ---------------------------------------------------------------- 1. chunk aggregates
  // Walker (chunk wc, half wh) owns channels wch .. wch + CPT - 1 and tokens
  // wt0 .. wt0 + 7 and composes their 2x2 step matrices; the halves of a
  // chunk are joined with a lane exchange.
  const int wc = wave & 3, wh = lane >> 5;
  const int wch = (wave >> 2) * 32 * CPT + (lane & 31) * CPT, wt0 = wc * 16 + wh * 8;
  const bool walker = wc < NCH && wch < DK;
  // OU inputs: the walker's channels' rate and diffusion (unused otherwise).
  float th[CPT], s2[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    th[k] = 0.f;
    s2[k] = 0.f;
    if constexpr (OU) {
      if (walker) {
        const size_t hc = (size_t)(head % p.H) * DK + wch + k;
        th[k] = p.theta[hc];
        s2[k] = p.sigma2[hc];
      }
    }
  }
  constexpr int KT = C::KEEP ? 8 : 1;
  float ca[KT][CPT], cpn[KT][CPT], cc2[KT][CPT], ckv[KT][CPT];  // a, pbar, c, k*Lambda^v
  // Prologue: each walker forms k for its own tokens and channels from the
  // staged raw xk (rows before the segment in the halo), with conv_lds's
  // instructions, so the values equal those of the exact path bit for bit.
  // k is never stored: the gate walk keeps what it needs in registers, or
  // (more than 16 token-channels per walker) forms k again the same way.
  float kact[MODE == kPrologue ? 8 : 1][CPT];
  auto walker_k = [&]() {
    if constexpr (MODE == kPrologue) {
      const In* const hk = s.halo + 3 * DK;
      const int hh = head % p.H;
      float ws[CPT][4], bs[CPT];
      conv_slots<CPT>(p.cw[1] + (size_t)hh * DK * p.cwidth, p.cb[1] ? p.cb[1] + (size_t)hh * DK : nullptr, p.cwidth,
                      wch, ws, bs);
      float win[11][CPT];  // raw rows wt0 - 3 .. wt0 + 7 (rows past nvalid are staged as zero)
#pragma unroll
      for (int i = 0; i < 11; ++i) {
        const int r = wt0 - 3 + i;
        load_vals<CPT>(r >= 0 ? rpn + r * DK + wch : hk + (r + 3) * DK + wch, win[i]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
          float acc = bs[k];
#pragma unroll
          for (int j = 0; j < 4; ++j) acc = fmaf(ws[k][j], win[e + j][k], acc);
          kact[e][k] = wt0 + e < nvalid ? to_f32(from_f32<In>(silu_f(acc))) : 0.f;
        }
    }
  };
  if (walker) walker_k();
  Mob Pg[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) Pg[k] = mob_identity();
  if (walker) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int x = (wt0 + e) * DK + wch;
      float kk[CPT], vpv[CPT], av[CPT], pnv[CPT];
      if constexpr (MODE == kPrologue) {
#pragma unroll
        for (int k = 0; k < CPT; ++k) kk[k] = kact[e][k];
      } else {
        load_vals<CPT>(rk + x, kk);
      }
      coef_vals<MODE, CPT>(rld + x, rpn + x, rvp + x, th, s2, wt0 + e < nvalid, av, pnv, vpv);
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const float kv = kk[k] * vpv[k];
        const float a = av[k];
        const float c = kk[k] * kv;
        if constexpr (C::KEEP) {
          ca[e][k] = a;
          cpn[e][k] = pnv[k];
          cc2[e][k] = c;
          ckv[e][k] = kv;
        }
        Pg[k] = mob_step_raw(Pg[k], a * a, pnv[k], c);
        if ((e & 3) == 3) Pg[k] = mob_normalize(Pg[k]);
      }
    }
  }
  // Chunk aggregate = (second half) . (first half); both halves form the same
  // product.  The second half keeps the first half's aggregate to find its
  // entering precision.
  Mob Pfirst[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const Mob Pp = Mob{__shfl_xor(Pg[k].m00, 32, 64), __shfl_xor(Pg[k].m01, 32, 64), __shfl_xor(Pg[k].m10, 32, 64),
                       __shfl_xor(Pg[k].m11, 32, 64)};
    Pfirst[k] = wh ? Pp : Pg[k];
    const Mob Pc = wh ? mob_mul(Pg[k], Pp) : mob_mul(Pp, Pg[k]);
    if (walker && wh == 0) *reinterpret_cast<v4f*>(cagg + (wc * DK + wch + k) * 4) = v4f{Pc.m00, Pc.m01, Pc.m10, Pc.m11};
  }
  store_tile<In, L, DK, NT>(rq, bq, tid);
  if constexpr (MODE == kPrologue || !C::CAGG_IN_V) store_tile<In, L, DV, NT>(s.v, bv, tid);
  __syncthreads();

  KLA_SSTAMP(3);
  // ---------------------------------------------------------------- 2. precision carry
  // The carry waves (one lane per channel; a second wave when DK = 128) each
  // run their own look-back over their channels, with flags of their own, so
  // no workgroup barrier sits inside the carry.  The inclusive precision of a
  // segment is published as {value, flag} records.  When the predecessor's
  // records, requested before the aggregate walk, already carry this call's
  // flag, they are the precision entering the segment: no aggregate is
  // published and no look-back runs (successors then wait for this segment's
  // inclusive flag, which follows at once).  Otherwise the aggregate is
  // published first; the first flag poll is issued before waiting for its
  // stores.  The inclusive flag is raised after the barrier that releases
  // the other waves.
  unsigned* const pfl = p.pflag + hb * 2 + wave;  // flag of segment r: pfl[2 * r]
  if (pwave) {
    // pre[c]: the map from the segment start to the start of chunk c + 1.
    Mob pre[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      Mob cg = mob_identity();
      if (pch) {
        const v4f d = ld4(cagg + (c * DK + tid) * 4);
        cg = Mob{d[0], d[1], d[2], d[3]};
      }
      pre[c] = c == 0 ? cg : mob_mul(cg, pre[c - 1]);
    }
    const Mob Pseg = pre[NCH - 1];
    float lam_in = 1.f;
    const bool fast = seg > 0 && __ballot(pch && record_flag(early) != FINC) == 0ull;
    if (seg == 0) {
      if (pch && p.lam0) lam_in = p.lam0[(size_t)head * DK + tid];
    } else if (fast) {
      lam_in = pch ? record_value(early) : 1.f;
    } else {
      if (!last && pch) {  // publish the aggregate first so successors need not wait on us
        const auto r = coherent_rsrc(p.pagg + hs * DK * 4, DK * 16);
        st_coherent(r, tid * 16, v4f{Pseg.m00, Pseg.m01, Pseg.m10, Pseg.m11});
      }
      const unsigned f0 = lookback_peek(pfl, 2, seg - 1);
      // A second look at the predecessor's records, in the same round trip.
      const unsigned long long again = pch ? ld_record(p.pinc + (hb + seg - 1) * DK + tid) : 0ull;
      wait_stores();
      if (!last && lane == 0) st_relaxed(pfl + 2 * seg, FAGG);
      if (__ballot(pch && record_flag(again) != FINC) == 0ull) {
        lam_in = pch ? record_value(again) : 1.f;
      } else {
        const int r0 = lookback_find(pfl, 2, seg, FAGG, FINC, p.ctrl, f0);
        // Fold the carries of segments r0 .. seg-1, loading up to eight at once.
        float lam = pch ? record_value(ld_record(p.pinc + (hb + r0) * DK + tid)) : 1.f;
        for (int u0 = r0 + 1; u0 < seg; u0 += 8) {
          v4f m[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (u0 + j < seg) m[j] = ld_coherent(coherent_rsrc(p.pagg + (hb + u0 + j) * DK * 4, DK * 16), tid * 16);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (u0 + j < seg) lam = mob_apply(Mob{m[j][0], m[j][1], m[j][2], m[j][3]}, lam);
        }
        lam_in = lam;
      }
    }
    if (!last && pch) st_record(p.pinc + hs * DK + tid, mob_apply(Pseg, lam_in), FINC);
    if (pch) {  // precision entering every chunk
#pragma unroll
      for (int c = 0; c < NCH; ++c) s.lamc[c * DK + tid] = c == 0 ? lam_in : mob_apply(pre[c - 1], lam_in);
    }
  }
  // Prologue: the waves that do not carry form q and v from the staged raw
  // tiles meanwhile (into registers; stored in place after the barrier).
  constexpr int NTC = NT - 64 * PW;
  constexpr int UKC = (L * DK * (int)sizeof(In) / 16 + NTC - 1) / NTC;
  constexpr int UVC = (L * DV * (int)sizeof(In) / 16 + NTC - 1) / NTC;
  uint4 cq[MODE == kPrologue ? UKC : 1], cv[MODE == kPrologue ? UVC : 1];
  const int tc = tid - 64 * PW;
  if constexpr (MODE == kPrologue) {
    if (!pwave) {
      const int hh = head % p.H, W = p.cwidth;
      conv_lds<In, L, DK, NTC>(cq, rq, s.halo, nvalid, p.cw[0] + (size_t)hh * DK * W,
                               p.cb[0] ? p.cb[0] + (size_t)hh * DK : nullptr, W, tc);
      conv_lds<In, L, DV, NTC>(cv, s.v, s.halo + 6 * DK, nvalid, p.cw[2] + (size_t)hh * DV * W,
                               p.cb[2] ? p.cb[2] + (size_t)hh * DV : nullptr, W, tc);
    }
  }
  __syncthreads();
  if (pwave && !last) {
    wait_stores();
    if (lane == 0) st_relaxed(pfl + 2 * seg, FINC);
  }
  if constexpr (MODE == kPrologue) {
    if (!pwave) {
      store_tile<In, L, DK, NTC>(rq, cq, tc);
      store_tile<In, L, DV, NTC>(s.v, cv, tc);
    }
    __syncthreads();  // the gate walk reads q
  } else if constexpr (C::CAGG_IN_V) {
    store_tile<In, L, DV, NT>(s.v, bv, tid);  // the aggregates are consumed
  }

  KLA_SSTAMP(4);
  // ---------------------------------------------------------------- 3. gate walk
  // Results stay in registers until every walker has finished reading the raw
  // inputs, then overwrite them as stored operands.  A second-half walker
  // starts from the precision after the first half and, once the halves have
  // exchanged their prod f, rescales its cumulative products to the chunk start.
  float wq[8][CPT], wk[8][CPT], wd[8][CPT];
  float Fg[CPT];  // prod f over this walker's tokens
#pragma unroll
  for (int k = 0; k < CPT; ++k) Fg[k] = 1.f;
  // The precision is walked projectively, lam = n / d ([KLA-nl] §2, the
  // Möbius form): d' = pbar n + a^2 d and n' = n + c d', so lam^- / lam' =
  // n / n', f = a n / n' and g = k Lambda^v d' / n'.  The recursion carries
  // two FMAs per token and no reciprocal; one reciprocal per token serves the
  // gates.  (n, d) are rescaled by a power of two every fourth token.
  if constexpr (MODE == kPrologue && !C::KEEP) {
    if (walker) walker_k();  // raw xk is still staged
  }
  auto walk = [&](auto with_path) {
    constexpr bool PATH = decltype(with_path)::value;
    float pn_[CPT], pd_[CPT], cp[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      pn_[k] = s.lamc[wc * DK + wch + k];
      if (wh) pn_[k] = mob_apply(Pfirst[k], pn_[k]);
      pd_[k] = 1.f;
      cp[k] = 1.f;
    }
    float* const lp = PATH ? p.lpath + ((size_t)head * T + t0) * DK + wch : nullptr;
    float fr[8][CPT], gr[8][CPT];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = wt0 + e;
      const int x = t * DK + wch;
      float qv[CPT];
      load_vals<CPT>(rq + x, qv);
      float a[CPT], pnv[CPT], c[CPT], kv[CPT];
      if constexpr (C::KEEP) {
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
          a[k] = ca[e][k];
          pnv[k] = cpn[e][k];
          c[k] = cc2[e][k];
          kv[k] = ckv[e][k];
        }
      } else {
        float kk[CPT], vpv[CPT];
        if constexpr (MODE == kPrologue) {
#pragma unroll
          for (int k = 0; k < CPT; ++k) kk[k] = kact[e][k];
        } else {
          load_vals<CPT>(rk + x, kk);
        }
        coef_vals<MODE, CPT>(rld + x, rpn + x, rvp + x, th, s2, t < nvalid, a, pnv, vpv);
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
          kv[k] = kk[k] * vpv[k];
          c[k] = kk[k] * kv[k];
        }
      }
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const float d1 = fmaf(pnv[k], pn_[k], a[k] * a[k] * pd_[k]);  // d' = pbar n + a^2 d
        const float n1 = fmaf(c[k], d1, pn_[k]);                       // n' = n + c d'
        const float inv = fast_rcp(n1);
        const float f = a[k] * pn_[k] * inv;
        const float g = kv[k] * d1 * inv;
        cp[k] *= f;
        wq[e][k] = qv[k] * cp[k];
        wk[e][k] = g * fast_rcp(cp[k]);
        fr[e][k] = f;
        gr[e][k] = g;
        pn_[k] = n1;
        pd_[k] = d1;
        if constexpr (PATH) {
          if (t < nvalid) lp[(size_t)t * DK + k] = n1 * fast_rcp(d1);
        }
      }
      if ((e & 3) == 3) {
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
          const int ex = __builtin_amdgcn_frexp_expf(fmaxf(pn_[k], pd_[k]));
          pn_[k] = __builtin_amdgcn_ldexpf(pn_[k], -ex);
          pd_[k] = __builtin_amdgcn_ldexpf(pd_[k], -ex);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      float sp = 1.f;
#pragma unroll
      for (int e = 7; e >= 0; --e) {
        wd[e][k] = gr[e][k] * sp;
        sp *= fr[e][k];
      }
      Fg[k] = cp[k];
      if (last && wc == NCH - 1 && wh) p.lamT[(size_t)head * DK + wch + k] = pn_[k] / pd_[k];
    }
  };
  if (walker) {
    if (p.lpath)
      walk(std::true_type{});
    else
      walk(std::false_type{});
  }
  // The scores of a chunk take the middle of the chunk as reference point:
  // Qs = q cp / F1 and Ks = g F1 / cp, with cp the prod of f from the chunk
  // start and F1 its value at the end of the first half, so that every factor
  // is bounded by the decay over one half (Qs Ks^T still pairs q_t g_u with
  // the decay from u to t).  A chunk is unsafe when some channel's prod f over
  // either half falls below 2^-64 (Qs or Ks could overflow); the chunk's
  // walker waves flag it in LDS, and its rows then hold the chunk-start
  // versions Qs = q cp and (with KST) Kd for the exact path.
  bool unsafe_w = false;
  float FpA[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const float Fp = FpA[k] = __shfl_xor(Fg[k], 32, 64);  // the other half's prod f
    const float cpe = wh ? Fp * Fg[k] : Fg[k] * Fp;
    unsafe_w |= __ballot(walker && !(Fg[k] >= 0x1p-64f)) != 0ull;
    if (walker && wh == 0) s.cpe[wc * DK + wch + k] = cpe;
  }
  if (walker && unsafe_w && lane == 0) s.unsafe[wc] = 1;
  __syncthreads();
  const bool unsafe_c = walker && s.unsafe[wc] != 0;  // uniform over the chunk's walker waves
  float F1[CPT];  // prod of f over the first half of the chunk
  if (walker) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      F1[k] = wh ? FpA[k] : Fg[k];
      if (unsafe_c) {  // chunk-start reference: the second half is rescaled
        if (wh) {
          const float r = fast_rcp(FpA[k]);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            wq[e][k] *= FpA[k];
            wk[e][k] *= r;
          }
        }
      } else if (!wh) {  // middle reference: the first half is rescaled
        const float r = fast_rcp(Fg[k]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          wq[e][k] *= r;
          wk[e][k] *= Fg[k];
        }
      }
      if (wh == 0) {
        s.cpm[wc * DK + wch + k] = unsafe_c ? 1.f : Fg[k];
        s.cp2[wc * DK + wch + k] = unsafe_c ? Fg[k] * FpA[k] : FpA[k];
      }
    }
  }
  if (walker && (unsafe_c || !C::KST) && !wh) {  // Kd is stored: rescale the first half to the chunk end
#pragma unroll
    for (int k = 0; k < CPT; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) wd[e][k] *= FpA[k];
  }
  unsigned char* const Qs = s.u;
  unsigned char* const Ks = s.u + L * QROW;
  unsigned char* const Qg = s.u + 2 * L * QROW;
  unsigned char* const KdT = s.u + 3 * L * QROW;  // without KST only
  if (walker) {
    const int cb = (wch >> 2) * 16, cj = wch & 3;  // block and slot of channel wch in a row
    // Qg = q times the prod of f from the segment start: the chunk-start
    // version of Qs scaled by the decays of the earlier chunks.  The carried
    // state enters y only through it.
    float dec[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      dec[k] = unsafe_c ? 1.f : F1[k];
#pragma unroll
      for (int c = 0; c < NCH - 1; ++c)
        if (c < wc) dec[k] *= s.cpe[c * DK + wch + k];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = wt0 + e;
      put_vals<BF16, CPT>(Qs + t * QROW + cb, cj, wq[e]);
      float qg[CPT];
#pragma unroll
      for (int k = 0; k < CPT; ++k) qg[k] = wq[e][k] * dec[k];
      put_vals<BF16, CPT>(Qg + t * QROW + cb, cj, qg);
      // With KST the rows of an unsafe chunk hold Kd (its scores take the
      // exact path and never read Ks).
      put_vals<BF16, CPT>(Ks + t * QROW + cb, cj, (C::KST && unsafe_c) ? wd[e] : wk[e]);
    }
    if constexpr (!C::KST) {
#pragma unroll
      for (int k = 0; k < CPT; ++k)  // Kd^T row wch + k: four tokens per block
#pragma unroll
        for (int e = 0; e < 8; e += 4)
          M::put(KdT + (wch + k) * KROW + (wt0 + e) * 4, v4f{wd[e][k], wd[e + 1][k], wd[e + 2][k], wd[e + 3][k]});
    }
  }
  if (tid < DK) {
    float F = 1.f;
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) F *= s.cpe[cc * DK + tid];
    s.fseg[tid] = F;
  }
  __syncthreads();

  KLA_SSTAMP(5);
  // ---------------------------------------------------------------- 4a. intra-chunk scores
  // A[t][u] = sum_i Qs[t][i] Ks[u][i] for u <= t (0 above the diagonal),
  // stored in A-operand order: lane l, element e -> A[t = l%16][u = 4*(l/16) + e].
  // A chunk flagged unsafe gets exact scores instead: each channel lane
  // re-derives f, g of its channel (same instructions as the walk, raw inputs
  // from global memory) and the channels are summed with wave reductions, in
  // a fixed order.
  unsigned char* const A = s.scores();
#pragma unroll 1
  for (int cc = 0; cc < NCH; ++cc) {
    if (!s.unsafe[cc]) continue;  // uniform: every thread reads the same flag
    float f[16], g[16], q[16];
    const bool chan = tid < DK;
    if (chan) {
      float th1 = 0.f, s21 = 0.f;
      if constexpr (OU) {
        th1 = p.theta[(size_t)(head % p.H) * DK + tid];
        s21 = p.sigma2[(size_t)(head % p.H) * DK + tid];
      }
      float qa[16], ka[16];  // prologue: this channel's q and k activations over the chunk
      if constexpr (MODE == kPrologue) {
        const size_t hh = head % p.H;
        float ws[1][4], bs[1];
        const size_t gx0 = ((size_t)head * T + t0 + cc * 16) * DK + tid;
        conv_slots<1>(p.cw[0] + hh * DK * p.cwidth, p.cb[0] ? p.cb[0] + hh * DK : nullptr, p.cwidth, tid, ws, bs);
        conv_chunk<In>(qa, static_cast<const In*>(p.q) + gx0, DK, t0 + cc * 16, cc * 16, nvalid, ws[0], bs[0]);
        conv_slots<1>(p.cw[1] + hh * DK * p.cwidth, p.cb[1] ? p.cb[1] + hh * DK : nullptr, p.cwidth, tid, ws, bs);
        conv_chunk<In>(ka, static_cast<const In*>(p.k) + gx0, DK, t0 + cc * 16, cc * 16, nvalid, ws[0], bs[0]);
      }
      float lam = s.lamc[cc * DK + tid];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = cc * 16 + e;
        float kk = 0.f, ldv = 0.f, pnv = 0.f, vpv = 0.f, qv = 0.f, a = 1.f;
        if (t < nvalid) {
          const size_t gx = ((size_t)head * T + t0 + t) * DK + tid;
          ldv = to_f32(static_cast<const In*>(p.ld)[gx]);
          vpv = to_f32(static_cast<const In*>(p.vp)[gx]);
          if constexpr (MODE == kPrologue) {
            kk = ka[e];
            qv = qa[e];
            ldv = softplus_f(ldv);
            vpv = softplus_f(vpv);
          } else {
            kk = to_f32(static_cast<const In*>(p.k)[gx]);
            qv = to_f32(static_cast<const In*>(p.q)[gx]);
          }
          if constexpr (OU) {
            a = ou_coef(th1, s21, ldv, ldv, pnv);
          } else {
            pnv = to_f32(static_cast<const In*>(p.pn)[gx]);
            a = __expf(ldv);
          }
        }
        const float kv = kk * vpv;
        float lam_pred;
        const float lam_new = lam_step(lam, a * a, pnv, kk * kv, lam_pred);
        const float inv = fast_rcp(lam_new);
        f[e] = a * lam_pred * inv;
        g[e] = kv * inv;
        q[e] = qv;
        lam = lam_new;
      }
    }
    // pair (t, u), u <= t: sum over channels of q_t g_u prod_{w=u+1..t} f_w
    // (rarely taken: kept rolled to keep the kernel's code small)
#pragma unroll 1
    for (int uu = 0; uu < 16; ++uu) {
      float d = chan ? g[uu] : 0.f;
#pragma unroll 1
      for (int tt = uu; tt < 16; ++tt) {
        if (tt > uu) d *= chan ? f[tt] : 0.f;
        const float part = wave_sum(chan ? q[tt] * d : 0.f);
        if (lane == 0 && wave < (DK + 63) / 64) s.partial()[wave * 256 + tt * 16 + uu] = part;
      }
    }
    __syncthreads();
    if (tid < 256) {
      const int tt = tid >> 4, uu = tid & 15;
      float acc = 0.f;
      if (uu <= tt)
        for (int w = 0; w < (DK + 63) / 64; ++w) acc += s.partial()[w * 256 + tt * 16 + uu];
      put1<BF16>(A + (cc * 64 + tt + 16 * (uu >> 2)) * 16, uu & 3, acc);
    }
    __syncthreads();
  }
  for (int cc = wave; cc < NCH; cc += NW) {
    if (s.unsafe[cc]) continue;
    Op qo[NRT], ko[NRT];
#pragma unroll
    for (int mt = 0; mt < NRT; ++mt) {
      qo[mt] = M::get(Qs + (cc * 16 + lc) * QROW + (16 * mt + 4 * lg) * 4);
      ko[mt] = M::get(Ks + (cc * 16 + lc) * QROW + (16 * mt + 4 * lg) * 4);
    }
    // D[u][t] = sum_i Ks[u][i] Qs[t][i]: lane l, element e holds S[t = l%16][u = 4*(l/16) + e]
    v4f st = M::dot(v4f{0.f, 0.f, 0.f, 0.f}, ko, qo);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * lg + e > lc) st[e] = 0.f;  // causal: u <= t
    M::put(A + (cc * 64 + lane) * 16, st);
  }
  if (C::KST && tid < DK) {  // a safe chunk's update ends with one multiply: F2 times the next reference
#pragma unroll
    for (int cc = 0; cc + 1 < NCH; ++cc)
      if (!s.unsafe[cc]) s.cp2[cc * DK + tid] *= s.cpm[(cc + 1) * DK + tid];
  }
  __syncthreads();

  KLA_SSTAMP(6);
  // ---------------------------------------------------------------- 4b. chunk loop
  // Local chunk states from a zero state: M_{c+1} = diag(cp_end_c) M_c + Kd_c^T V_c.
  // y_c gets its local part A_c V_c + q cp M_c, here or (LATE_LOCAL) from the
  // kept states once the local state is on its way out; the carried state is
  // added once it is known.  The accumulators hold the state entering chunk c
  // times the chunk's score reference (diag(cpm_c) M_c), so the readout is
  // Qs_c times them; after the chunk's update the state is taken to the next
  // chunk's reference (1 after the last chunk: the local state).
  // The mean-carry waves ask for the predecessor's mean flag now (used in
  // section 5; a lane's flag of segment seg - 1 - lane).
  const unsigned early_mflag =
      (p.mskip && wave < NCT && seg > 0) ? lookback_peek(p.mflag + hb * NW + wave, NW, seg - 1) : 0u;
  v4f yl[NCH][CPW];
  v4f Macc[NRT][CPW];
  constexpr int NKEEP = C::LATE_LOCAL ? NCH : 1;
  v4f Mkeep[NKEEP][NRT][CPW];  // LATE_LOCAL: local state entering chunk c (c >= 1)
#pragma unroll
  for (int pp = 0; pp < CPW; ++pp)
#pragma unroll
    for (int mt = 0; mt < NRT; ++mt) Macc[mt][pp] = v4f{0.f, 0.f, 0.f, 0.f};

  if (wave < NCT) {
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      const Op ao = M::get(A + (cc * 64 + lane) * 16);
      Op qo[NRT];
      if (!C::LATE_LOCAL && cc > 0) {
#pragma unroll
        for (int mt = 0; mt < NRT; ++mt) qo[mt] = M::get(Qs + (cc * 16 + lc) * QROW + (16 * mt + 4 * lg) * 4);
      }
#pragma unroll
      for (int pp = 0; pp < CPW; ++pp) {
        const int nt = wave + NW * pp;
        if (nt < NCT) {
          // V block: rows u = cc*16 + 4*lg + e, column 16*nt + lc.
          const typename M::VOp vo = M::vop(s.v + (cc * 16 + 4 * lg) * DV + 16 * nt + lc, DV);
          v4f acc = M::dotv(v4f{0.f, 0.f, 0.f, 0.f}, ao, vo);
          if (!C::LATE_LOCAL && cc > 0) {  // the local state entering chunk 0 is zero
            Op mo[NRT];
#pragma unroll
            for (int mt = 0; mt < NRT; ++mt) mo[mt] = M::op(Macc[mt][pp]);
            acc = M::dot(acc, qo, mo);
          }
          yl[cc][pp] = acc;
#pragma unroll
          for (int mt = 0; mt < NRT; ++mt) {
            const v4f ce = ld4(s.cp2 + cc * DK + 16 * mt + 4 * lg);
            auto next_ref = [&]() {
              return cc + 1 < NCH ? ld4(s.cpm + (cc + 1) * DK + 16 * mt + 4 * lg) : v4f{1.f, 1.f, 1.f, 1.f};
            };
            if constexpr (C::KST) {
              // Ks^T block (channels 16mt.., tokens of chunk cc) read transposed
              // from the Ks rows: input lane j of a 16-lane group reads the hi
              // (then lo) half of block 4mt + j%4 in token row 4*(l/16) + j/4.
              const int j = lane & 15;
              const unsigned char* a = Ks + (cc * 16 + 4 * lg + (j >> 2)) * QROW + (4 * mt + (j & 3)) * 16;
              const Op kso = cat(lds_read_tr16(a), lds_read_tr16(a + 8));
              if (s.unsafe[cc])  // rows hold Kd: M' = diag(cp_end) M + Kd^T V (reference 1)
                Macc[mt][pp] = M::dotv(Macc[mt][pp] * ce, kso, vo) * next_ref();
              else  // M' = diag(F2) (F1 M + Ks^T V), since Kd = Ks F2 (ce includes the next reference)
                Macc[mt][pp] = M::dotv(Macc[mt][pp], kso, vo) * ce;
            } else {  // M' = diag(cp_end) M + Kd^T V, with cp_end M = F2 (F1 M)
              const v4f m = cc == 0 ? Macc[mt][pp] : Macc[mt][pp] * ce;
              const Op kdo = M::get(KdT + (16 * mt + lc) * KROW + (cc * 16 + 4 * lg) * 4);
              Macc[mt][pp] = M::dotv(m, kdo, vo) * next_ref();
            }
            if constexpr (C::LATE_LOCAL) {
              if (cc + 1 < NCH) Mkeep[cc + 1 < NKEEP ? cc + 1 : 0][mt][pp] = Macc[mt][pp];
            }
          }
        }
      }
    }
  }

  KLA_SSTAMP(7);
  // ---------------------------------------------------------------- 5. mean carry
  // Each lane owns, per tile (mt, nt), rows 16*mt + 4*lg + e of column 16*nt + lc.
  // Workspace payloads are stored in this fragment order, 16 bytes per lane.
  // The carry of a column tile depends only on the same columns of earlier
  // segments, so each wave carries its own tiles with flags (and a copy of
  // prod f) of its own: no workgroup barrier sits inside the carry.
  constexpr uint32_t MBYTES = (uint32_t)DK * DV * 4;
  constexpr int FB = NRT * CPW <= 8 ? 2 : 1;  // aggregates folded per round trip
  auto frag_off = [&](int mt, int nt) -> uint32_t { return ((uint32_t)(nt * NRT + mt) * 64 + lane) * 16; };
  v4f Min[NRT][CPW];
  auto local_readout = [&]() {  // LATE_LOCAL: y_c += Qs_c (F1_c M_c) for c >= 1
    if constexpr (C::LATE_LOCAL) {
#pragma unroll
      for (int cc = 1; cc < NCH; ++cc) {
        Op qo[NRT];
#pragma unroll
        for (int mt = 0; mt < NRT; ++mt) qo[mt] = M::get(Qs + (cc * 16 + lc) * QROW + (16 * mt + 4 * lg) * 4);
#pragma unroll
        for (int pp = 0; pp < CPW; ++pp) {
          if (wave + NW * pp < NCT) {
            Op mo[NRT];
#pragma unroll
            for (int mt = 0; mt < NRT; ++mt) mo[mt] = M::op(Mkeep[cc < NKEEP ? cc : 0][mt][pp]);
            yl[cc][pp] = M::dot(yl[cc][pp], qo, mo);
          }
        }
      }
    }
  };
  if (wave < NCT) {
    unsigned* const mfl = p.mflag + hb * NW + wave;  // flag of segment r: mfl[NW * r]
    auto store_inclusive = [&]() {
      const auto r = coherent_rsrc(p.minc + hs * DK * DV, MBYTES);
#pragma unroll
      for (int pp = 0; pp < CPW; ++pp) {
        const int nt = wave + NW * pp;
        if (nt < NCT) {
#pragma unroll
          for (int mt = 0; mt < NRT; ++mt) {
            const v4f F = ld4(s.fseg + 16 * mt + 4 * lg);
            v4f o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = fmaf(F[e], Min[mt][pp][e], Macc[mt][pp][e]);
            st_coherent(r, frag_off(mt, nt), o);
          }
        }
      }
      wait_stores();
      if (lane == 0) st_relaxed(mfl + NW * seg, FINC);
    };
    if (seg == 0) {
#pragma unroll
      for (int pp = 0; pp < CPW; ++pp) {
        const int nt = wave + NW * pp;
#pragma unroll
        for (int mt = 0; mt < NRT; ++mt) {
          v4f m = v4f{0.f, 0.f, 0.f, 0.f};
          if (nt < NCT && p.M0) {
            const float* src = p.M0 + (size_t)head * DK * DV + (size_t)(16 * mt + 4 * lg) * DV + 16 * nt + lc;
            m = v4f{src[0], src[DV], src[2 * DV], src[3 * DV]};
          }
          Min[mt][pp] = m;
        }
      }
      local_readout();
      if (!last) store_inclusive();
    } else {
      // If the predecessor's flag read before the chunk loop already showed
      // its inclusive state, that is the carry: this segment publishes no
      // aggregate and runs no look-back (successors then wait for its
      // inclusive flag, which follows at once).  Only with many heads
      // (p.mskip): consecutive segments of a head are then dispatched far
      // apart, so no successor is left waiting; with few heads they run side
      // by side and the aggregate is what lets them proceed.
      const bool pred_inc = p.mskip && __ballot(lane == 0 && early_mflag == FINC) != 0ull;
      int r0 = seg - 1;
      if (pred_inc) local_readout();
      if (!pred_inc) {
        const size_t fslot = (hs * NW + wave) * DK;  // this wave's copy of prod f
        if (!last) {
          for (int r = lane; r < DK; r += 64) st_coherent(p.mF + fslot + r, s.fseg[r]);
          const auto r = coherent_rsrc(p.magg + hs * DK * DV, MBYTES);
#pragma unroll
          for (int pp = 0; pp < CPW; ++pp) {
            const int nt = wave + NW * pp;
            if (nt < NCT) {
#pragma unroll
              for (int mt = 0; mt < NRT; ++mt) st_coherent(r, frag_off(mt, nt), Macc[mt][pp]);
            }
          }
        }
        const unsigned f1 = lookback_peek(mfl, NW, seg - 1);
        local_readout();  // overlaps the stores above and the flag poll
        wait_stores();
        if (!last && lane == 0) st_relaxed(mfl + NW * seg, FAGG);
        r0 = lookback_find(mfl, NW, seg, FAGG, FINC, p.ctrl, f1);
        KLA_SVALUE(11, seg - r0);
      }
      // Fold the carries of segments r0 .. seg-1 (M <- diag(prod f) M + local
      // state), FB aggregates per round trip.
#pragma unroll
      for (int pp = 0; pp < CPW; ++pp) {
        const int nt = wave + NW * pp;
#pragma unroll
        for (int mt = 0; mt < NRT; ++mt)
          Min[mt][pp] = nt < NCT ? ld_coherent(coherent_rsrc(p.minc + (hb + r0) * DK * DV, MBYTES), frag_off(mt, nt))
                                 : v4f{0.f, 0.f, 0.f, 0.f};
      }
      for (int u0 = r0 + 1; u0 < seg; u0 += FB) {
        v4f A[FB][NRT][CPW], F[FB][NRT];
#pragma unroll
        for (int j = 0; j < FB; ++j) {
          if (u0 + j < seg) {
            const size_t us = hb + u0 + j;
            const auto ra = coherent_rsrc(p.magg + us * DK * DV, MBYTES);
            const auto rf = coherent_rsrc(p.mF + (us * NW + wave) * DK, DK * 4);
#pragma unroll
            for (int mt = 0; mt < NRT; ++mt) {
              F[j][mt] = ld_coherent(rf, (16 * mt + 4 * lg) * 4);
#pragma unroll
              for (int pp = 0; pp < CPW; ++pp) {
                const int nt = wave + NW * pp;
                A[j][mt][pp] = nt < NCT ? ld_coherent(ra, frag_off(mt, nt)) : v4f{0.f, 0.f, 0.f, 0.f};
              }
            }
          }
        }
#pragma unroll
        for (int j = 0; j < FB; ++j) {
          if (u0 + j < seg) {
#pragma unroll
            for (int mt = 0; mt < NRT; ++mt)
#pragma unroll
              for (int pp = 0; pp < CPW; ++pp)
#pragma unroll
                for (int e = 0; e < 4; ++e) Min[mt][pp][e] = fmaf(F[j][mt][e], Min[mt][pp][e], A[j][mt][pp][e]);
          }
        }
      }
      if (!last) store_inclusive();
    }
  }
  // Every thread read the epoch before the first barrier; count this
  // workgroup done (other waves may still be polling flags of this call).
  if (nseg > 1 && tid == 0) epoch_done_units(p.ctrl, p.hdone, (unsigned)head, (unsigned)nheads, (unsigned)nseg, epoch);
  if (last) {  // final state, row-major
#pragma unroll
    for (int pp = 0; pp < CPW; ++pp) {
      const int nt = wave + NW * pp;
      if (nt < NCT) {
#pragma unroll
        for (int mt = 0; mt < NRT; ++mt) {
          const v4f F = ld4(s.fseg + 16 * mt + 4 * lg);
          float* dst = p.MT + (size_t)head * DK * DV + (size_t)(16 * mt + 4 * lg) * DV + 16 * nt + lc;
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[e * DV] = fmaf(F[e], Min[mt][pp][e], Macc[mt][pp][e]);
        }
      }
    }
  }

  KLA_SSTAMP(8);
  // ---------------------------------------------------------------- 6. carried-state readout + store
  // With M_in the state entering the segment, the true state entering chunk c
  // is M_c + diag(prod of earlier chunk decays) M_in, so
  //   y_c = (A_c V_c + Qs_c F1_c M_c) + Qg_c M_in,
  // the bracket from the chunk loop; M_in is split into matrix-core operands
  // once for all chunks.  y is staged in LDS over v (dead once every wave has
  // left the chunk loop) and written out in 16-byte units.  A wave's y
  // columns are the V columns only it read in the chunk loop, so no barrier
  // is needed before staging.
  if (wave < NCT) {
#pragma unroll
    for (int pp = 0; pp < CPW; ++pp) {
      const int nt = wave + NW * pp;
      if (nt < NCT) {
        Op mo[NRT];
#pragma unroll
        for (int mt = 0; mt < NRT; ++mt) mo[mt] = M::op(Min[mt][pp]);
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc) {
          Op go[NRT];
#pragma unroll
          for (int mt = 0; mt < NRT; ++mt) go[mt] = M::get(Qg + (cc * 16 + lc) * QROW + (16 * mt + 4 * lg) * 4);
          const v4f acc = M::dot(yl[cc][pp], go, mo);
#pragma unroll
          for (int e = 0; e < 4; ++e) s.v[(cc * 16 + 4 * lg + e) * DV + 16 * nt + lc] = from_f32<In>(acc[e]);
        }
      }
    }
  }
  __syncthreads();
  unstage_tile<In, L, DV, NT>(static_cast<In*>(p.y) + ((size_t)head * T + t0) * DV, s.v, nvalid, tid);
  KLA_SSTAMP(9);
}

// ------------------------------------------------------------------------------
// Host-side launch.
// ------------------------------------------------------------------------------
template <int DK, int DV, bool BF16>
static hipError_t launch_fwd(const FwdParams& p, hipStream_t stream) {
  const unsigned nblocks = (unsigned)p.nheads * (unsigned)p.nseg;
  constexpr int NT = FwdCfg<DK, DV, BF16>::NT;
  if (p.cw[0])
    hipLaunchKernelGGL((kla_fwd_kernel<DK, DV, BF16, kPrologue>), dim3(nblocks), dim3(NT), 0, stream, p);
  else if (p.theta)
    hipLaunchKernelGGL((kla_fwd_kernel<DK, DV, BF16, kOU>), dim3(nblocks), dim3(NT), 0, stream, p);
  else
    hipLaunchKernelGGL((kla_fwd_kernel<DK, DV, BF16, kPlain>), dim3(nblocks), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

int fwd_segment_len(int dk, int dv, bool bf16) {
  return (bf16 || (dk <= 64 && dv <= 64)) ? 64 : 32;
}

hipError_t launch_forward(const FwdParams& p, int dk, int dv, bool bf16, hipStream_t stream) {
#define KLA_FWD_CASE(DK_, DV_)                                                          \
  if (dk == DK_ && dv == DV_) return bf16 ? launch_fwd<DK_, DV_, true>(p, stream)        \
                                          : launch_fwd<DK_, DV_, false>(p, stream);
#define KLA_FWD_ROW(DK_) KLA_FWD_CASE(DK_, 16) KLA_FWD_CASE(DK_, 32) KLA_FWD_CASE(DK_, 64) KLA_FWD_CASE(DK_, 128)
  KLA_FWD_ROW(16)
  KLA_FWD_ROW(32)
  KLA_FWD_ROW(64)
  KLA_FWD_ROW(128)
#undef KLA_FWD_ROW
#undef KLA_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace kla

#ifdef KLA_TIMELINE
extern "C" int kla_seg_timeline_read(void* host, size_t bytes) {
  const size_t n = sizeof(kla::kla_seg_timeline_buf);
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(kla::kla_seg_timeline_buf), bytes < n ? bytes : n, 0,
                                  hipMemcpyDeviceToHost);
}
extern "C" int kla_seg_timeline_clear() {
  static unsigned long long zeros[kla::kStlGroups * kla::kStlSlots];
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(kla::kla_seg_timeline_buf), zeros, sizeof(zeros), 0, hipMemcpyHostToDevice);
}
#endif

