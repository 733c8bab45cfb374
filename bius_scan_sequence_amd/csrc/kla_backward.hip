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
//               and e = q dq - g dg.  Decays prod_{u=m+1..l} f_u are exp2 of
//               short sums of log2 f: differences of cumulative sums inside
//               one 16-token chunk plus whole chunks' totals (never ratios of
//               products over the segment, which can underflow).
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

#ifdef KLA_TIMELINE
// Timeline build only (-DKLA_TIMELINE): every wave of the chunk kernel sums
// the shader clock (s_memtime) spent in each phase of its work over all its
// segments, and lane 0 writes the sums to kla_bwd_timeline_buf[workgroup]
// [wave][phase] at the end.  Phases: 0 state loads issued at a segment's
// start, 10 the staging proper (seg_store), 11 the wait for the segment's loads
// (and the stores before them), 12 the next segment's loads issued (a share
// per chunk), 1 work before the chunk loop, 2 barrier before the loop; per
// chunk: 15 the barrier after the chunk before (and a flag read), 3 mean
// tiles, 13 and 14 the key waves' Xs / Ys and in-chunk parts of the outputs,
// 4 the rest of the outputs, 5 adjoint update, 6 operands of the next chunk;
// 7 the barrier after a segment's last chunk.  Slot 8 counts segments, slot 9
// holds the wave's whole life in cycles.
constexpr int kBtlPhases = 16, kBtlGroups = 4096;
__device__ unsigned long long kla_bwd_timeline_buf[kBtlGroups * 8 * kBtlPhases];
#define KLA_BTL_DECL                                 \
  unsigned long long btl_acc[kBtlPhases] = {};       \
  const unsigned long long btl_t0 = __builtin_amdgcn_s_memtime(); \
  unsigned long long btl_t = btl_t0
#define KLA_BTL(k)                                                \
  do {                                                            \
    const unsigned long long btl_n = __builtin_amdgcn_s_memtime(); \
    btl_acc[k] += btl_n - btl_t;                                  \
    btl_t = btl_n;                                                \
  } while (0)
#define KLA_BTL_END()                                                                          \
  do {                                                                                         \
    btl_acc[9] = __builtin_amdgcn_s_memtime() - btl_t0;                                        \
    if ((threadIdx.x & 63) == 0 && blockIdx.x < (unsigned)kBtlGroups) _Pragma("unroll")         \
      for (int btl_k = 0; btl_k < kBtlPhases; ++btl_k)                                         \
        kla_bwd_timeline_buf[((size_t)blockIdx.x * 8 + (threadIdx.x >> 6)) * kBtlPhases + btl_k] = \
            btl_acc[btl_k];                                                                    \
  } while (0)
#else
#define KLA_BTL_DECL \
  do {               \
  } while (0)
#define KLA_BTL(k) \
  do {             \
  } while (0)
#define KLA_BTL_END() \
  do {                \
  } while (0)
#endif

namespace {
constexpr int kSL = 64;  // tokens per segment
constexpr int kC = 16;   // tokens per chunk
constexpr int kChunkThreads = 512;
// LDS row strides, in elements.  Rows of the 64-token [t][channel] arrays are
// K + 4 long (a multiple of 4 that is 4 modulo 32): a matrix-core operand read
// (rows 4 lg + e, columns lr of a 16-lane group) then hits distinct banks, and
// staging writes four channels at once.  The 16-row per-chunk arrays are read
// both by rows lr and by rows 4 lg + e: K + 3 keeps both at two-way at most.
// The 16 x 16 score tiles use rows of 17 for the same reason.
template <int K> constexpr int kRowP = K + 4;
template <int K> constexpr int kRow16P = K + 3;
constexpr int kCP = 17;
// s_waitcnt operand that waits for every vector memory operation (vmcnt 0)
// and leaves the export and LDS/scalar counters at their maxima.
constexpr int kVmcntZero = 0x0F70;

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

// Four consecutive elements x .. x+3 of a per-token output (x a multiple of
// 4): one 8-byte store for bf16, one 16-byte store for fp32.
template <bool BF16>
__device__ __forceinline__ void stout4(void* p, size_t x, v4f v) {
  if constexpr (BF16) {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + x) =
        make_uint2((uint32_t)bf16_rne(v[0]) | ((uint32_t)bf16_rne(v[1]) << 16),
                   (uint32_t)bf16_rne(v[2]) | ((uint32_t)bf16_rne(v[3]) << 16));
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(p) + x) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// Four consecutive elements x .. x+3 of a per-token input (16-byte aligned
// rows; x a multiple of 4): one 8-byte load for bf16, one 16-byte load for fp32.
template <bool BF16>
__device__ __forceinline__ float4 ldin4(const void* p, size_t x) {
  if constexpr (BF16) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + x);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  } else {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + x);
  }
}

// log2 of the forget gate and the write gate of one element (token t < T),
// from the saved precision after the token (lam) and before it (lprev).
// log2 f = log2 a + log2(lam^-/lam) is formed without forming f, so strong
// decays (f below the fp32 range) stay exact.
__device__ __forceinline__ void gate1(float lam, float lprev, float ld, float pn, float k, float vp, float& lf,
                                      float& g) {
  const float a = __expf(ld);
  const float inv = fast_rcp(lam);
  const float lpred = lprev * fast_rcp(fmaf(pn, lprev, a * a));
  lf = fmaf(ld, 1.44269504088896341f, __log2f(lpred * inv));
  g = k * vp * inv;
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Four consecutive staged v / dy values of one row (8-byte aligned for bf16
// rows, whose stride is a multiple of 4 elements): one 8-byte LDS read for bf16.
__device__ __forceinline__ v4f row4(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return v4f{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
             __uint_as_float(u.y & 0xffff0000u)};
}
__device__ __forceinline__ v4f row4(const float* p) { return v4f{p[0], p[1], p[2], p[3]}; }

// bf16 inputs: a product whose one operand is exact in bf16 (the inputs v and
// dy, held as their bit patterns) runs on v_mfma_f32_16x16x32_bf16.  The fp32
// operand y is split into three bf16 terms, hi = bf16(y), mid = bf16(y - hi),
// lo = bf16(y - hi - mid), about 24 bits of y together (two terms, 17 bits,
// are too few: d log_decay sums the per-token products over the whole
// sequence and their errors with it).  One instruction forms x.hi + x.mid,
// a second x.lo: two instructions per K = 16 block against four of
// v_mfma_f32_16x16x4_f32, at half the cycles each.  Products of two fp32
// operands keep the fp32 path.
struct Split3 {
  v8s hm;  // [hi | mid]
  v8s l0;  // [lo | 0]
};
__device__ __forceinline__ Split3 split3(v4f y) {
  v4s h, m, l, r2;
  split4(y, h, m);
  v4f r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = (y[e] - to_f32((uint16_t)h[e])) - to_f32((uint16_t)m[e]);
  split4(r, l, r2);
  return Split3{cat(h, m), cat(l, v4s{0, 0, 0, 0})};
}
__device__ __forceinline__ v4f mma_ex(v4f acc, v4s x, const Split3& y) {  // x on the A side
  acc = mma_x32(acc, cat(x, x), y.hm);
  return mma_x32(acc, cat(x, v4s{0, 0, 0, 0}), y.l0);
}
__device__ __forceinline__ v4f mma_xe(v4f acc, const Split3& y, v4s x) {  // x on the B side
  acc = mma_x32(acc, y.hm, cat(x, x));
  return mma_x32(acc, y.l0, cat(x, v4s{0, 0, 0, 0}));
}
// Bit patterns of four bf16 values: consecutive (8-byte aligned) or strided.
__device__ __forceinline__ v4s bits4(const uint16_t* p) { return *reinterpret_cast<const v4s*>(p); }
__device__ __forceinline__ v4s bits4(const uint16_t* p, int stride) {
  return v4s{(short)p[0], (short)p[stride], (short)p[2 * stride], (short)p[3 * stride]};
}

// v and dy are kept in their input type (bf16 bits are exact); the row
// stride of those arrays, in elements: bf16 rows padded by 4 elements, so that
// the four 4-row groups of a matrix-core operand read fall on distinct banks.
template <int V, bool BF16> struct VRow {
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  static constexpr int P = BF16 ? V + 4 : V + 1;
};

// A segment's raw inputs in registers: the first half of staging, issued a
// segment ahead by the segment-aggregate and chunk kernels so that their
// loads overlap the work on the segment before.  Four consecutive elements per load: 8 bytes for bf16,
// 16 for fp32; pass x of the key side covers (token x / K4, channels
// 4 (x % K4) ..), pass x of the value side likewise.
template <bool BF16> using Raw4 = typename std::conditional<BF16, uint2, float4>::type;
template <int K, int V, bool BF16, int NT>
struct SegLoads {
  static constexpr int PK = (kSL * (K / 4) + NT - 1) / NT, PV = (kSL * (V / 4) + NT - 1) / NT;
  // Load parts that can be issued separately: each pass of the key side, then
  // the whole value side.
  static constexpr int NPART = PK + 1;
  float4 lam[PK], lprev[PK];  // the precision path at the token and one token earlier
  Raw4<BF16> ld[PK], pn[PK], k[PK], vp[PK], q[PK];
  Raw4<BF16> v[PV], d[PV];
};

template <bool BF16>
__device__ __forceinline__ Raw4<BF16> ldraw4(const void* p, size_t x) {
  if constexpr (BF16)
    return *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + x);
  else
    return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + x);
}
__device__ __forceinline__ float4 raw_f4(uint2 u) {
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}
__device__ __forceinline__ float4 raw_f4(float4 f) { return f; }

// Part PART of a segment's loads (SegLoads::NPART parts: pass PART of the key
// side, or for the last part the value side).
template <int PART, int K, int V, bool BF16, int NT>
__device__ __forceinline__ void seg_load_part(const BwdParams& p, size_t hd, int t0, SegLoads<K, V, BF16, NT>& r) {
  constexpr int K4 = K / 4, V4 = V / 4;
  using L = SegLoads<K, V, BF16, NT>;
  const Raw4<BF16> z{};
  // The thread index through an empty asm: the addresses are formed here,
  // where the loads go out, not hoisted out of a loop that issues them and
  // held in registers across it.
  int tix = (int)threadIdx.x;
  asm volatile("" : "+v"(tix));
  if constexpr (PART < L::PK) {
    constexpr int pk = PART;
    const int x = tix + pk * NT, t = x / K4, i = (x % K4) * 4;
    r.lam[pk] = make_float4(0.f, 0.f, 0.f, 0.f);
    r.lprev[pk] = make_float4(1.f, 1.f, 1.f, 1.f);
    r.ld[pk] = r.pn[pk] = r.k[pk] = r.vp[pk] = r.q[pk] = z;
    if (x < kSL * K4 && t0 + t < p.T) {
      const size_t e = (hd * p.T + t0 + t) * p.ks + i;
      r.lam[pk] = *reinterpret_cast<const float4*>(p.lpath + e);
      // The precision before the token: the path one token earlier, or the prior.
      if (t0 + t > 0) {
        r.lprev[pk] = *reinterpret_cast<const float4*>(p.lpath + e - p.ks);
      } else if (p.lam0) {
        const float* l0 = p.lam0 + hd * p.ksh + i;
        r.lprev[pk] = make_float4(l0[0], l0[1], l0[2], l0[3]);
      }
      r.ld[pk] = ldraw4<BF16>(p.ld, e);
      r.pn[pk] = ldraw4<BF16>(p.pn, e);
      r.k[pk] = ldraw4<BF16>(p.k, e);
      r.vp[pk] = ldraw4<BF16>(p.vp, e);
      r.q[pk] = ldraw4<BF16>(p.q, e);
    }
  } else {
#pragma unroll
    for (int pv = 0; pv < L::PV; ++pv) {
      const int x = tix + pv * NT, t = x / V4, j = (x % V4) * 4;
      r.v[pv] = r.d[pv] = z;
      if (x < kSL * V4 && t0 + t < p.T) {
        const size_t y = (hd * p.T + t0 + t) * p.vs + j;
        r.v[pv] = ldraw4<BF16>(p.v, y);
        r.d[pv] = ldraw4<BF16>(p.dy, y);
      }
    }
  }
}

// Parts PART, PART + 1, ... of a segment's loads; with `only` >= 0 just part
// `only` (a wave-uniform index; none if it is past the last part).
template <int PART = 0, int K, int V, bool BF16, int NT>
__device__ __forceinline__ void seg_load(const BwdParams& p, size_t hd, int t0, SegLoads<K, V, BF16, NT>& r,
                                         int only = -1) {
  if constexpr (PART < SegLoads<K, V, BF16, NT>::NPART) {
    if (only < 0 || only == PART) seg_load_part<PART>(p, hd, t0, r);
    seg_load<PART + 1>(p, hd, t0, r, only);
  }
}

// The second half of staging: log2 f, g, q as [64][K+1] (q in fp32 or, for
// bf16 inputs, in its own bf16 bits) and v, dy as [64][VRow::P] (rows padded
// so that column walks hit distinct banks), then log2 f turned into the
// cumulative sum inside each 16-token chunk (lb) with each chunk's total in
// T[4][K].  Tokens past T are identity steps: log2 f = 0, g = q = v = dy = 0.
// Every decay the kernels need is then exp2 of a short sum: inside a chunk
// lb_l - lb_m, across chunks the chunk totals in between (never a difference
// of two long cumulative sums).
template <int K, int V, bool BF16, int NT, typename QT>
__device__ __forceinline__ void seg_store(const BwdParams& p, size_t hd, int t0, const SegLoads<K, V, BF16, NT>& r, float* slb,
                                          float* sg, QT* sq, typename VRow<V, BF16>::T* sv,
                                          typename VRow<V, BF16>::T* sd, float* sT, int* unsafe) {
  using In = typename std::conditional<BF16, uint16_t, float>::type;
  using L = SegLoads<K, V, BF16, NT>;
  constexpr int KP = kRowP<K>, VP = VRow<V, BF16>::P, K4 = K / 4, V4 = V / 4;
#pragma unroll
  for (int pk = 0; pk < L::PK; ++pk) {
    const int x = threadIdx.x + pk * NT, t = x / K4, i = (x % K4) * 4;
    if (x >= kSL * K4) continue;
    float lf[4] = {0.f, 0.f, 0.f, 0.f}, g[4] = {0.f, 0.f, 0.f, 0.f}, q[4] = {0.f, 0.f, 0.f, 0.f};
    if (t0 + t < p.T) {
      const float4 lam = r.lam[pk], lprev = r.lprev[pk];
      const float4 ld = raw_f4(r.ld[pk]), pn = raw_f4(r.pn[pk]), k = raw_f4(r.k[pk]), vp = raw_f4(r.vp[pk]),
                   qq = raw_f4(r.q[pk]);
      gate1(lam.x, lprev.x, ld.x, pn.x, k.x, vp.x, lf[0], g[0]);
      gate1(lam.y, lprev.y, ld.y, pn.y, k.y, vp.y, lf[1], g[1]);
      gate1(lam.z, lprev.z, ld.z, pn.z, k.z, vp.z, lf[2], g[2]);
      gate1(lam.w, lprev.w, ld.w, pn.w, k.w, vp.w, lf[3], g[3]);
      q[0] = qq.x; q[1] = qq.y; q[2] = qq.z; q[3] = qq.w;
    }
    *reinterpret_cast<float4*>(slb + t * KP + i) = make_float4(lf[0], lf[1], lf[2], lf[3]);
    *reinterpret_cast<float4*>(sg + t * KP + i) = make_float4(g[0], g[1], g[2], g[3]);
    if constexpr (std::is_same<QT, float>::value) {
      *reinterpret_cast<float4*>(sq + t * KP + i) = make_float4(q[0], q[1], q[2], q[3]);
    } else {  // bf16 bits of q (exact: q is a bf16 value)
      *reinterpret_cast<uint2*>(sq + t * KP + i) =
          make_uint2((__float_as_uint(q[0]) >> 16) | (__float_as_uint(q[1]) & 0xffff0000u),
                     (__float_as_uint(q[2]) >> 16) | (__float_as_uint(q[3]) & 0xffff0000u));
    }
  }
#pragma unroll
  for (int pv = 0; pv < L::PV; ++pv) {
    const int x = threadIdx.x + pv * NT, t = x / V4, j = (x % V4) * 4;
    if (x >= kSL * V4) continue;
    In vv[4], dd[4];
    if constexpr (BF16) {  // the inputs' own bits
      const uint2 uv = r.v[pv], ud = r.d[pv];
      vv[0] = (In)uv.x; vv[1] = (In)(uv.x >> 16); vv[2] = (In)uv.y; vv[3] = (In)(uv.y >> 16);
      dd[0] = (In)ud.x; dd[1] = (In)(ud.x >> 16); dd[2] = (In)ud.y; dd[3] = (In)(ud.y >> 16);
    } else {
      const float4 fv = r.v[pv], fd = r.d[pv];
      vv[0] = fv.x; vv[1] = fv.y; vv[2] = fv.z; vv[3] = fv.w;
      dd[0] = fd.x; dd[1] = fd.y; dd[2] = fd.z; dd[3] = fd.w;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sv[t * VP + j + e] = vv[e];
      sd[t * VP + j + e] = dd[e];
    }
  }
  __syncthreads();
  // One thread per (channel, chunk): cumulative log2 f inside the chunk.  A
  // chunk is marked in `unsafe` (when given) if a channel's log2 decay over
  // either half of it falls below -96.
  // The chunk's 16 values are read before any is written back, so that the
  // reads are in flight together.
  for (int x = threadIdx.x; x < 4 * K; x += NT) {
    const int c = x / K, i = x % K;
    float r[kC];
#pragma unroll
    for (int l = 0; l < kC; ++l) r[l] = slb[(c * kC + l) * KP + i];
    float acc = 0.f, mid = 0.f;
#pragma unroll
    for (int l = 0; l < kC; ++l) {
      acc += r[l];
      r[l] = acc;
      if (l == 7) mid = acc;
    }
#pragma unroll
    for (int l = 0; l < kC; ++l) slb[(c * kC + l) * KP + i] = r[l];
    sT[c * K + i] = acc;
    const float first = r[0];
    if (unsafe && (first - mid > 96.f || mid - acc > 96.f)) unsafe[c] = 1;  // benign race: all write 1
  }
  __syncthreads();
}

}  // namespace

// ---------------------------------------------------------------------------
// 1. Segment aggregates.  Workgroups of 512 threads, each taking segments
// blockIdx, blockIdx + gridDim, ...; for bf16 inputs the next segment's inputs
// are loaded into registers while the current one is reduced.
// ---------------------------------------------------------------------------
template <int K, int V, bool BF16>
__global__ __launch_bounds__(512) void kla_bwd_segagg_kernel(BwdParams p) {
  using SV = typename VRow<V, BF16>::T;
  constexpr int KP = kRowP<K>, VP = VRow<V, BF16>::P, NT = 512;
  __shared__ __align__(16) float sl[kSL * KP];
  __shared__ __align__(16) float sa[kSL * KP];
  __shared__ __align__(16) float sb[kSL * KP];
  __shared__ float sT[4 * K];
  __shared__ SV sv[kSL * VP], sd[kSL * VP];
  const int tid = threadIdx.x;
  constexpr bool PREFETCH = BF16;
  const unsigned nsb = (unsigned)p.nheads * (unsigned)p.nseg;
  SegLoads<K, V, BF16, NT> nxt;
  if constexpr (PREFETCH)
    if (blockIdx.x < nsb) seg_load(p, blockIdx.x / p.nseg, (int)(blockIdx.x % p.nseg) * kSL, nxt);
  for (unsigned sg = blockIdx.x; sg < nsb; sg += gridDim.x) {
  const size_t hd = sg / p.nseg;
  const int s = (int)(sg % p.nseg);
  if (sg != blockIdx.x) __syncthreads();  // the previous segment's tiles are read
  if constexpr (!PREFETCH) seg_load(p, hd, s * kSL, nxt);
  seg_store<K, V, BF16, NT>(p, hd, s * kSL, nxt, sl, sa, sb, sv, sd, sT, static_cast<int*>(nullptr));
  if constexpr (PREFETCH) {
    const unsigned nb = sg + gridDim.x;
    if (nb < nsb) seg_load(p, nb / p.nseg, (int)(nb % p.nseg) * kSL, nxt);
  }
  // alpha_t = g_t prod_{u>t} f_u (in place of g), beta_t = q_t prod_{u<=t} f_u
  // (in place of q), for t in chunk c: the products are exp2 of the chunk's
  // partial sums plus the totals of the later / earlier chunks.  A thread
  // keeps one channel (NT is a multiple of K), so its four chunks' offsets
  // are formed once.
  {
    static_assert(NT % K == 0, "one channel per thread");
    const int i = tid % K;
    float tot[4], aft[4], bef[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) tot[c] = sT[c * K + i];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      aft[c] = 0.f;
      bef[c] = 0.f;
#pragma unroll
      for (int c2 = 0; c2 < 4; ++c2) {
        if (c2 > c) aft[c] += tot[c2];
        if (c2 < c) bef[c] += tot[c2];
      }
    }
#pragma unroll
    for (int u = 0; u < kSL * K / NT; ++u) {
      const int t = tid / K + u * (NT / K), c = t / kC;
      // c is a compile-time function of u when a pass covers whole chunks;
      // otherwise pick among the four without indexing the register arrays.
      const float Tc = c == 0 ? tot[0] : c == 1 ? tot[1] : c == 2 ? tot[2] : tot[3];
      const float A = c == 0 ? aft[0] : c == 1 ? aft[1] : c == 2 ? aft[2] : aft[3];
      const float Bf = c == 0 ? bef[0] : c == 1 ? bef[1] : c == 2 ? bef[2] : bef[3];
      const float lb = sl[t * KP + i];
      sa[t * KP + i] *= ex2((Tc - lb) + A);
      sb[t * KP + i] *= ex2(lb + Bf);
    }
  }
  if (tid < K) p.F[(hd * p.nseg + s) * K + tid] = ex2(sT[tid] + sT[K + tid] + sT[2 * K + tid] + sT[3 * K + tid]);
  __syncthreads();
  // Mean aggregate alpha^T v and adjoint aggregate beta^T dy as 16x16
  // matrix-core tiles over the 64 tokens.  A wave takes one (aggregate, key
  // block) pair and every value block, so each coefficient block is read
  // (and, for bf16 inputs, split) once.
  constexpr int KB = K / 16, VB = V / 16;
  const int wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  const size_t base = (hd * p.nseg + s) * (size_t)(K * V);
  for (int pr = wave; pr < 2 * KB; pr += NT / 64) {
    const bool adj = pr >= KB;
    const int ib = adj ? pr - KB : pr;
    const float* X = adj ? sb : sa;  // coefficient [t][i]
    const SV* Y = adj ? sd : sv;     // [t][j]
    v4f acc[VB];
#pragma unroll
    for (int jb = 0; jb < VB; ++jb) acc[jb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < kSL; kb += 16) {
      v4f a;
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = X[(kb + 4 * lg + e) * KP + ib * 16 + lr];
      if constexpr (BF16) {  // v and dy exact in bf16: the three-term split
        const Split3 as = split3(a);
#pragma unroll
        for (int jb = 0; jb < VB; ++jb)
          acc[jb] = mma_xe(acc[jb], as, bits4(&Y[(kb + 4 * lg) * VP + jb * 16 + lr], VP));
      } else {
#pragma unroll
        for (int jb = 0; jb < VB; ++jb) {
          v4f b;
#pragma unroll
          for (int e = 0; e < 4; ++e) b[e] = to_f32(Y[(kb + 4 * lg + e) * VP + jb * 16 + lr]);
          acc[jb] = mma_f32(acc[jb], a, b);
        }
      }
    }
    float* U = (adj ? p.Gseg : p.Mseg) + base;
#pragma unroll
    for (int jb = 0; jb < VB; ++jb)
#pragma unroll
      for (int e = 0; e < 4; ++e) U[(ib * 16 + 4 * lg + e) * V + jb * 16 + lr] = acc[jb][e];
  }
  }  // segments
}

// ---------------------------------------------------------------------------
// 2. Scans over segments.  Grid: nheads * ceil(K*V / 256) workgroups of 256
// threads; one thread per state element, eight segments' loads in flight.
// ---------------------------------------------------------------------------
template <int K, int V>
__global__ __launch_bounds__(256) void kla_bwd_segscan_kernel(BwdParams p) {
  constexpr int N = K * V, NB = (N + 255) / 256, G = 8;
  const size_t hd = blockIdx.x / NB;
  const int el = (blockIdx.x % NB) * 256 + threadIdx.x;
  const bool live = el < N;
  const int i = el / V;
  const size_t me = hd * (size_t)p.mhead + (size_t)i * p.mrow + el % V;  // element of M0 / dMT / dM0
  const int nseg = p.nseg;
  float* Ms = p.Mseg + hd * nseg * (size_t)N;
  float* Gs = p.Gseg + hd * nseg * (size_t)N;
  const float* F = p.F + hd * nseg * (size_t)K + i;
  float part = 0.f;
  if (live) {
    float m = p.M0 ? p.M0[me] : 0.f;
    int s = 0;
    for (; s + G <= nseg; s += G) {
      float u[G], f[G];
#pragma unroll
      for (int r = 0; r < G; ++r) {
        u[r] = Ms[(size_t)(s + r) * N + el];
        f[r] = F[(size_t)(s + r) * K];
      }
#pragma unroll
      for (int r = 0; r < G; ++r) {
        Ms[(size_t)(s + r) * N + el] = m;
        m = fmaf(f[r], m, u[r]);
      }
    }
    for (; s < nseg; ++s) {
      const float u = Ms[(size_t)s * N + el];
      Ms[(size_t)s * N + el] = m;
      m = fmaf(F[(size_t)s * K], m, u);
    }
    if (p.dMT) part = m * p.dMT[me];
  }
  // Row sum over the V threads of a row (consecutive lanes of one wave).
#pragma unroll
  for (int o = V / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o);
  if (live && el % V == 0) p.rs[hd * p.ksh + i] = p.add_rs ? p.rs[hd * p.ksh + i] + part : part;
  if (live) {
    float h = p.dMT ? p.dMT[me] : 0.f;
    int s = nseg - 1;
    for (; s - G + 1 >= 0; s -= G) {
      float u[G], f[G];
#pragma unroll
      for (int r = 0; r < G; ++r) {
        u[r] = Gs[(size_t)(s - r) * N + el];
        f[r] = F[(size_t)(s - r) * K];
      }
#pragma unroll
      for (int r = 0; r < G; ++r) {
        Gs[(size_t)(s - r) * N + el] = h;
        h = fmaf(f[r], h, u[r]);
      }
    }
    for (; s >= 0; --s) {
      const float u = Gs[(size_t)s * N + el];
      Gs[(size_t)s * N + el] = h;
      h = fmaf(F[(size_t)s * K], h, u);
    }
    p.dM0[me] = h;
  }
}

// ---------------------------------------------------------------------------
// 3. Per-chunk gradients.  Grid: nheads * nseg workgroups of 512 threads
// (eight waves); the segment's chunks are taken last to first.  The
// contractions run on the matrix cores in fp32 (v_mfma_f32_16x16x4_f32,
// 16x16 tiles; lane layout in kla_device.h).  Waves 0-3 are key-side: key
// wave w keeps, in registers, tiles of M_c^T and of H^T whose columns are key
// block w; waves 4-7 are value-side: value wave w keeps the tiles of H whose
// columns are value block w.  Each tile set is in the orientation in which it
// is the B operand of the product that needs it:
//   Mt[jb] = tile (jb, w) of M_c^T   (rows j, cols i in key block w):   dY M_c^T
//   Ht[jb] = tile (jb, w) of H^T                                       V H^T
//   Hc[ib] = tile (ib, w) of H       (rows i, cols j in value block w): Kd H
// so the key-side outputs (dq, dg) of key block w and the value-side output
// (dv) of value block w each come out of one wave with no cross-wave
// reduction, and two waves share each SIMD.
//
// In-chunk decays D(l, m) = prod_{u=m+1..l} f_u = exp2(lb_l - lb_m).  When
// every channel's log2 decay over each half of the chunk stays above -96
// ("safe" chunk), D(l, m) = E_l F_m with E_l = exp2(lb_l - lb_7) and
// F_m = exp2(lb_7 - lb_m) both inside the fp32 range, and the in-chunk terms
// are matrix-core products of (q E), (g F) and the score matrices.  Other
// chunks take the exact elementwise path, with every D(l, m) from its own
// exp2.
// ---------------------------------------------------------------------------
// The in-chunk decays E_l = exp2(lb_l - lb_7), F_l = exp2(lb_7 - lb_l),
// cp_l = exp2(lb_l) (prod_{u<=l} f_u) and sx_l = exp2(T_c - lb_l)
// (prod_{u>l} f_u) are formed where they are used, from the staged lb.
// The chunk kernel's per-segment state tiles from global memory: a value wave
// takes H tiles (Hx[ib] = H[16 ib + 4 lg + e][16 vb + lr], ib < K/16), a key
// wave H^T tiles (Hx[jb] = H[16 kb + lr][16 jb + 4 lg + e], jb < V/16) and the
// same tiles of the mean M (Ms); the rest stay zero.
template <int K, int V, int HB>
__device__ __forceinline__ void load_state(const float* Gg, const float* Mg, bool vw, bool kw, int kb, int vb, int lg,
                                           int lr, v4f (&Hx)[HB], v4f (&Ms)[V / 16]) {
  constexpr int KB = K / 16, VB = V / 16;
#pragma unroll
  for (int b = 0; b < HB; ++b) {
    Hx[b] = v4f{0.f, 0.f, 0.f, 0.f};
    if (b < VB) Ms[b] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  if (vw) {  // wave-uniform branches: every load of a wave issued together
#pragma unroll
    for (int ib = 0; ib < KB; ++ib)
#pragma unroll
      for (int e = 0; e < 4; ++e) Hx[ib][e] = Gg[(ib * 16 + 4 * lg + e) * V + vb * 16 + lr];
  } else if (kw) {
#pragma unroll
    for (int jb = 0; jb < VB; ++jb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Hx[jb][e] = Gg[(kb * 16 + lr) * V + jb * 16 + 4 * lg + e];
        Ms[jb][e] = Mg[(kb * 16 + lr) * V + jb * 16 + 4 * lg + e];
      }
  }
}

template <int K, int V, bool BF16>
struct alignas(16) BwdChunkSmem {
  using SV = typename VRow<V, BF16>::T;
  static constexpr int KP = kRowP<K>, K16 = kRow16P<K>, VP = VRow<V, BF16>::P;
  float lb[kSL * KP], g[kSL * KP];
  SV q[kSL * KP];
  SV v[kSL * VP], d[kSL * VP];
  // Per-chunk operands, two buffers: chunk w's in buffer w & 1 while chunk
  // w - 1's are being formed.
  float qE[2][kC * K16];      // q_l E_l
  float gF[2][kC * K16];      // g_l F_l
  float kd[2][kC * K16];      // g_l sx_l (write gate decayed to the chunk end)
  float be[2][kC * K16];      // q_l cp_l (query decayed from the chunk start)
  float A[2][kC * kCP], B[2][kC * kCP];  // A[l][m] = q_l . (g_m decayed to l); B[l][m] = dy_l . v_m (m <= l; 0 above)
  float cdec[2][K];           // prod f over the chunk, per channel (exp2 of its total)
  float T[4 * K];             // sum of log2 f over each chunk of the segment
  int unsafe[4];              // chunk needs the exact in-chunk path
};

// Operands of chunk w (tokens 16 w ..) into buffer `buf`: the decayed rows
// qE, gF, kd, be and the chunk's decay per channel, elements x = grp, grp +
// gsize, ... below xend (none if grp < 0) (E = prod f from the chunk's token 7
// to l, F its inverse, cp = prod f from the chunk start, sx = prod f to the
// chunk end, all exp2 of short sums); the score tile B when do_b; the score
// tile A by wave 6 from the same products (or, on the exact path, one (l, m)
// pair per thread xp < 256 of the workgroup).
template <int K, int V, bool BF16>
__device__ __forceinline__ void chunk_operands(BwdChunkSmem<K, V, BF16>& s, int w, int buf, int grp, int xend,
                                               int gsize, bool do_b, int xp, int wave, int lg, int lr) {
  constexpr int KP = kRowP<K>, K16 = kRow16P<K>, VP = VRow<V, BF16>::P, C = kC, CP = kCP, VB = V / 16;
  const int c0 = w * C;
  for (int x = grp; grp >= 0 && x < xend; x += gsize) {
    const int l = x / K, i = x % K;
    const float lb = s.lb[(c0 + l) * KP + i], lb7 = s.lb[(c0 + 7) * KP + i];
    const float tot = s.T[w * K + i];
    const float E = ex2(lb - lb7), F = ex2(lb7 - lb), cp = ex2(lb), sx = ex2(tot - lb);
    const float q = to_f32(s.q[(c0 + l) * KP + i]), g = s.g[(c0 + l) * KP + i];
    s.qE[buf][l * K16 + i] = q * E;
    s.gF[buf][l * K16 + i] = g * F;
    s.kd[buf][l * K16 + i] = g * sx;
    s.be[buf][l * K16 + i] = q * cp;
    if (l == C - 1) s.cdec[buf][i] = cp;  // exp2 of the chunk's last cumulative value: its total
  }
  if (do_b) {
    // B[l][m] = dy_l . v_m (one tile, V/16 blocks; bf16 inputs: exact
    // products, two blocks per instruction).
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
    if constexpr (BF16) {
#pragma unroll
      for (int jb = 0; jb < VB; jb += 2) {
        const v4s a0 = bits4(&s.d[(c0 + lr) * VP + jb * 16 + 4 * lg]);
        const v4s b0 = bits4(&s.v[(c0 + lr) * VP + jb * 16 + 4 * lg]);
        const v4s a1 = jb + 1 < VB ? bits4(&s.d[(c0 + lr) * VP + (jb + 1) * 16 + 4 * lg]) : v4s{0, 0, 0, 0};
        const v4s b1 = jb + 1 < VB ? bits4(&s.v[(c0 + lr) * VP + (jb + 1) * 16 + 4 * lg]) : v4s{0, 0, 0, 0};
        acc = mma_x32(acc, cat(a0, a1), cat(b0, b1));
      }
    } else {
#pragma unroll
      for (int jb = 0; jb < VB; ++jb) {
        const v4f a = row4(&s.d[(c0 + lr) * VP + jb * 16 + 4 * lg]);
        const v4f b = row4(&s.v[(c0 + lr) * VP + jb * 16 + 4 * lg]);
        acc = mma_f32(acc, a, b);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) s.B[buf][(4 * lg + e) * CP + lr] = lr <= 4 * lg + e ? acc[e] : 0.f;
  }
  if (s.unsafe[w] == 0) {
    if (wave == 6) {
      // A = tril((q E)(g F)^T) (one tile, K/16 blocks).
      v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < K; kb += 16) {
        v4f a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = kb + 4 * lg + e;
          const float lb = s.lb[(c0 + lr) * KP + i], lb7 = s.lb[(c0 + 7) * KP + i];
          a[e] = to_f32(s.q[(c0 + lr) * KP + i]) * ex2(lb - lb7);
          b[e] = s.g[(c0 + lr) * KP + i] * ex2(lb7 - lb);
        }
        acc = mma_f32(acc, a, b);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) s.A[buf][(4 * lg + e) * CP + lr] = lr <= 4 * lg + e ? acc[e] : 0.f;
    }
  } else if (xp >= 0 && xp < C * C) {
    // Exact scores: A[l][m] = sum_i q_l g_m exp2(lb_l - lb_m), m <= l.
    const int l = xp / C, m = xp % C;
    float acc = 0.f;
    if (m <= l)
      for (int i = 0; i < K; ++i)
        acc = fmaf(to_f32(s.q[(c0 + l) * KP + i]) * s.g[(c0 + m) * KP + i],
                   ex2(s.lb[(c0 + l) * KP + i] - s.lb[(c0 + m) * KP + i]), acc);
    s.A[buf][l * CP + m] = acc;
  }
}

// M_c^T tiles of key wave kb (block kb of the key channels) for chunk w: the
// segment state decayed to the chunk start plus the tokens before the chunk
// (v^T al over t < 16 w).  Reads only the staged rows.
template <int K, int V, bool BF16>
__device__ __forceinline__ void mean_tiles(const BwdChunkSmem<K, V, BF16>& s, int w, int kb_w, int lg, int lr,
                                           const v4f (&Ms)[V / 16], v4f (&Mt)[V / 16]) {
  constexpr int KP = kRowP<K>, VP = VRow<V, BF16>::P, C = kC, VB = V / 16;
  const int i = kb_w * 16 + lr;
  float lP = 0.f;
  for (int c3 = 0; c3 < w; ++c3) lP += s.T[c3 * K + i];
  const float Pi = ex2(lP);
#pragma unroll
  for (int jb = 0; jb < VB; ++jb)
#pragma unroll
    for (int e = 0; e < 4; ++e) Mt[jb][e] = Pi * Ms[jb][e];
  // Tokens t of an earlier chunk c2 enter with g_t prod_{u=t+1}^{c0-1} f_u
  // = g_t exp2((T[c2] - lb_t) + sum of the chunk totals in between).
  for (int c2 = 0; c2 < w; ++c2) {
    float off = s.T[c2 * K + i];
    for (int c3 = c2 + 1; c3 < w; ++c3) off += s.T[c3 * K + i];
    v4f b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = c2 * C + 4 * lg + e;
      b[e] = s.g[t * KP + i] * ex2(off - s.lb[t * KP + i]);
    }
    // one 16-token block of this chunk: four k-groups of 4 (e), tiles jb interleaved
    if constexpr (BF16) {
      const Split3 bs = split3(b);
#pragma unroll
      for (int jb = 0; jb < VB; ++jb)
        Mt[jb] = mma_ex(Mt[jb], bits4(&s.v[(c2 * C + 4 * lg) * VP + jb * 16 + lr], VP), bs);
    } else {
#pragma unroll
      for (int jb = 0; jb < VB; ++jb) {
        v4f a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = to_f32(s.v[(c2 * C + 4 * lg + e) * VP + jb * 16 + lr]);
        Mt[jb] = mma_f32(Mt[jb], a, b);
      }
    }
  }
}

template <int K, int V, bool BF16>
__global__ __launch_bounds__(kChunkThreads) void kla_bwd_chunk_kernel(BwdParams p) {
  constexpr int KP = kRowP<K>, K16 = kRow16P<K>, VP = VRow<V, BF16>::P, NT = kChunkThreads, C = kC, CP = kCP;
  constexpr int KB = K / 16, VB = V / 16;
  static_assert(NT == 2 * C * C && NT == 512, "eight waves; one score pair per thread of the first four");
  __shared__ BwdChunkSmem<K, V, BF16> s;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  const int kb_w = wave, vb_w = wave - 4;       // key block of a key wave, value block of a value wave
  const bool kw = wave < KB, vw = wave >= 4 && vb_w < VB;
  // Each workgroup takes segments blockIdx, blockIdx + gridDim, ...; for bf16
  // inputs the next segment's inputs are loaded into registers while this
  // one's chunks run, so their latency is hidden (one workgroup per CU leaves
  // nothing else to hide it behind).  fp32 inputs (twice the registers) load
  // each segment when it starts.
  constexpr bool PREFETCH = BF16;
  const unsigned nsb = (unsigned)p.nheads * (unsigned)p.nseg;
  KLA_BTL_DECL;
  SegLoads<K, V, BF16, NT> nxt;
  if constexpr (PREFETCH)
    if (blockIdx.x < nsb)
    seg_load(p, blockIdx.x / p.nseg, (int)(blockIdx.x % p.nseg) * kSL, nxt);
  for (unsigned sb = blockIdx.x; sb < nsb; sb += gridDim.x) {
  KLA_BTL(7);
#ifdef KLA_TIMELINE
  ++btl_acc[8];
#endif
  const size_t hd = sb / p.nseg;
  const int seg = (int)(sb % p.nseg);
  const int t0 = seg * kSL;
  const int nvalid = min(kSL, p.T - t0);
  const size_t st = (hd * p.nseg + seg) * (size_t)(K * V);
  const float* Mg = p.Mseg + st;
  const float* Gg = p.Gseg + st;
  // Adjoint at the segment end and the mean entering the segment.  A value
  // wave keeps H tiles (Hc[ib], ib < KB), a key wave H^T tiles (Ht[jb],
  // jb < VB) in the same registers, and M^T (Ms).  With the prefetch their
  // loads go out first and land during staging; without it (fp32 inputs,
  // more registers held by the staging) they follow the staging.
  constexpr int HB = KB > VB ? KB : VB;
  v4f Hx[HB], Mt[VB], Ms[VB];
  v4f(&Hc)[HB] = Hx;
  v4f(&Ht)[HB] = Hx;
  if constexpr (PREFETCH) load_state<K, V>(Gg, Mg, vw, kw, kb_w, vb_w, lg, lr, Hx, Ms);
  if (tid < 4) s.unsafe[tid] = 0;
  if constexpr (!PREFETCH) seg_load(p, hd, t0, nxt);
  KLA_BTL(0);
  seg_store<K, V, BF16, NT>(p, hd, t0, nxt, s.lb, s.g, s.q, s.v, s.d, s.T, s.unsafe);
  if constexpr (!PREFETCH) load_state<K, V>(Gg, Mg, vw, kw, kb_w, vb_w, lg, lr, Hx, Ms);
  KLA_BTL(10);
  // Every load of this segment has landed before the chunk loop starts.
  // Global stores share the load counter and it drains in order: a load
  // still pending inside the loop would make each chunk wait for the stores
  // of the chunk before it.
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  KLA_BTL(11);
  // The next segment's loads go out in parts, one at the start of each chunk
  // (the rest after the last chunk), so that they queue behind the chunks'
  // work rather than stall the waves all at once; only the next staging
  // waits for them.
  const unsigned nb = sb + gridDim.x;
  const bool more = PREFETCH && nb < nsb;
  const size_t nhd = nb / p.nseg;
  const int nt0 = (int)(nb % p.nseg) * kSL;

  // Inside the loop every wave works on chunk w and then forms its share of
  // chunk w - 1's operands in the other buffer: one barrier per chunk.  The
  // rows go to waves 4, 5 and 7 in whole passes of 192 elements, the rest
  // (and the score tile B) to waves 0..3, which wait at the barriers longer;
  // wave 6 forms the score tile A.  Before the loop the waves form the last
  // chunk's operands the same way while the key waves rebuild its mean tiles.
  constexpr int kRowsV = (C * K / 192) * 192;  // row elements of waves 4, 5, 7
  const int wl = (nvalid - 1) / C;
  const int grp_v = wave == 6 ? -1 : wave == 7 ? tid - 320 : tid - 256;
  if (wave >= 4) {
    chunk_operands<K, V, BF16>(s, wl, wl & 1, grp_v, kRowsV, 192, false, tid - 256, wave, lg, lr);
  } else {
    if (kw) mean_tiles<K, V, BF16>(s, wl, kb_w, lg, lr, Ms, Mt);
    chunk_operands<K, V, BF16>(s, wl, wl & 1, kRowsV + tid, C * K, 256, wave == 3, -1, wave, lg, lr);
  }
  KLA_BTL(1);
  __syncthreads();
  KLA_BTL(2);
  for (int w = wl; w >= 0; --w) {
    const int c0 = w * C, cur = w & 1;
    const bool safe = s.unsafe[w] == 0;
    KLA_BTL(15);
    if (more) seg_load(p, nhd, nt0, nxt, wl - w);
    KLA_BTL(12);
    // (b) M_c^T tiles (for the last chunk, formed before the loop).
    if (kw && w != wl) mean_tiles<K, V, BF16>(s, w, kb_w, lg, lr, Ms, Mt);
    KLA_BTL(3);
    // (c) outputs.
    const size_t tok0 = hd * (size_t)p.T + t0 + c0;
    if (kw) {
      // Xs = dY M_c^T, Ys = V H^T; in-chunk parts dqi = E (tril(B) (g F)),
      // dgi = F (tril(B)^T (q E)) for key block `wave`, each formed transposed
      // (the operands of every product swapped): lane (lg, lr) holds token lr
      // of the chunk and channels i0 .. i0 + 3, so that its outputs go out as
      // one vector store per array.
      const int i = kb_w * 16 + lr, i0 = kb_w * 16 + 4 * lg;
      v4f xs = v4f{0.f, 0.f, 0.f, 0.f}, ys = xs, dqi = xs, dgi = xs;
      if constexpr (BF16) {
#pragma unroll
        for (int jb = 0; jb < VB; ++jb) {
          xs = mma_xe(xs, split3(Mt[jb]), bits4(&s.d[(c0 + lr) * VP + jb * 16 + 4 * lg]));
          ys = mma_xe(ys, split3(Ht[jb]), bits4(&s.v[(c0 + lr) * VP + jb * 16 + 4 * lg]));
        }
      } else {
#pragma unroll
        for (int jb = 0; jb < VB; ++jb) {
          const v4f a = row4(&s.d[(c0 + lr) * VP + jb * 16 + 4 * lg]);
          const v4f b = row4(&s.v[(c0 + lr) * VP + jb * 16 + 4 * lg]);
          xs = mma_f32(xs, Mt[jb], a);
          ys = mma_f32(ys, Ht[jb], b);
        }
      }
      KLA_BTL(13);
      const v4f lb = *reinterpret_cast<const v4f*>(&s.lb[(c0 + lr) * KP + i0]);
      if (safe) {
        v4f a, b, c, d;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int n = 4 * lg + e;
          a[e] = s.B[cur][lr * CP + n];  // tril(B)[l = lr][m = n]
          b[e] = s.gF[cur][n * K16 + i];
          c[e] = s.B[cur][n * CP + lr];  // tril(B)^T[l = lr][n]
          d[e] = s.qE[cur][n * K16 + i];
        }
        dqi = mma_f32(dqi, b, a);
        dgi = mma_f32(dgi, d, c);
        const v4f lb7 = *reinterpret_cast<const v4f*>(&s.lb[(c0 + 7) * KP + i0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dqi[e] *= ex2(lb[e] - lb7[e]);
          dgi[e] *= ex2(lb7[e] - lb[e]);
        }
      } else {
        const int l = lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ic = i0 + e;
          float aq = 0.f, ag = 0.f;
          for (int m = 0; m < C; ++m) {
            const float lbm = s.lb[(c0 + m) * KP + ic];
            if (m <= l) aq = fmaf(s.B[cur][l * CP + m] * s.g[(c0 + m) * KP + ic], ex2(lb[e] - lbm), aq);
            if (m >= l) ag = fmaf(s.B[cur][m * CP + l] * to_f32(s.q[(c0 + m) * KP + ic]), ex2(lbm - lb[e]), ag);
          }
          dqi[e] = aq;
          dgi[e] = ag;
        }
      }
      KLA_BTL(14);
      if (c0 + lr < nvalid) {
        const v4f tot = *reinterpret_cast<const v4f*>(&s.T[w * K + i0]);
        const v4f gl = *reinterpret_cast<const v4f*>(&s.g[(c0 + lr) * KP + i0]);
        v4f ql;
        if constexpr (BF16)
          ql = row4(&s.q[(c0 + lr) * KP + i0]);
        else
          ql = *reinterpret_cast<const v4f*>(&s.q[(c0 + lr) * KP + i0]);
        v4f dq, dg, ee;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dq[e] = fmaf(ex2(lb[e]), xs[e], dqi[e]);
          dg[e] = fmaf(ex2(tot[e] - lb[e]), ys[e], dgi[e]);
          ee[e] = ql[e] * dq[e] - gl[e] * dg[e];
        }
        const size_t ow = (tok0 + lr) * p.kws + i0;
        if (p.dq_acc)
          *reinterpret_cast<float4*>(p.dq_acc + ow) = make_float4(dq[0], dq[1], dq[2], dq[3]);
        else
          stout4<BF16>(p.dq, (tok0 + lr) * p.ks + i0, dq);
        *reinterpret_cast<float4*>(p.dgw + ow) = make_float4(dg[0], dg[1], dg[2], dg[3]);
        *reinterpret_cast<float4*>(p.ew + ow) = make_float4(ee[0], ee[1], ee[2], ee[3]);
      }
    }
    if (vw) {
      // dv = Kd H + tril(A)^T dY for value block `wave - 4`, Kd = g sx, formed
      // transposed like the key side: lane (lg, lr) holds token lr and value
      // columns j0 .. j0 + 3.
      const int j = vb_w * 16 + lr, j0 = vb_w * 16 + 4 * lg;
      v4f dv = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ib = 0; ib < KB; ++ib) {
        v4f a;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = ib * 16 + 4 * lg + e;
          a[e] = s.kd[cur][lr * K16 + i];
        }
        dv = mma_f32(dv, Hc[ib], a);
      }
      {
        v4f a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = s.A[cur][(4 * lg + e) * CP + lr];  // tril(A)[l][m = lr]
          if constexpr (!BF16) b[e] = to_f32(s.d[(c0 + 4 * lg + e) * VP + j]);
        }
        if constexpr (BF16) {
          // its own accumulator: no matrix-core instruction of one shape reads
          // an accumulator that one of the other shape has just written
          dv += mma_ex(v4f{0.f, 0.f, 0.f, 0.f}, bits4(&s.d[(c0 + 4 * lg) * VP + j], VP), split3(a));
        } else {
          dv = mma_f32(dv, b, a);
        }
      }
      if (c0 + lr < nvalid) {
        if (p.dv_acc)
          *reinterpret_cast<float4*>(p.dv_acc + (tok0 + lr) * p.vacc + j0) = make_float4(dv[0], dv[1], dv[2], dv[3]);
        else
          stout4<BF16>(p.dv, (tok0 + lr) * p.vs + j0, dv);
      }
    }
    KLA_BTL(4);
    // (d) adjoint at the end of the previous chunk: diag(cp_end) H + (cp q)^T dY,
    // in both orientations (registers of this wave; LDS operands of this chunk).
    if (w > 0) {
      if (vw) {
        v4s bx = v4s{0, 0, 0, 0};
        if constexpr (BF16) bx = bits4(&s.d[(c0 + 4 * lg) * VP + vb_w * 16 + lr], VP);
#pragma unroll
        for (int ib = 0; ib < KB; ++ib) {
          v4f a, b;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            Hc[ib][e] *= s.cdec[cur][ib * 16 + 4 * lg + e];
            a[e] = s.be[cur][(4 * lg + e) * K16 + ib * 16 + lr];
            if constexpr (!BF16) b[e] = to_f32(s.d[(c0 + 4 * lg + e) * VP + vb_w * 16 + lr]);
          }
          if constexpr (BF16)
            Hc[ib] = mma_xe(Hc[ib], split3(a), bx);
          else
            Hc[ib] = mma_f32(Hc[ib], a, b);
        }
      }
      if (kw) {
        const int i = kb_w * 16 + lr;
        const float ce = s.cdec[cur][i];
        if constexpr (BF16) {
          v4f b;
#pragma unroll
          for (int e = 0; e < 4; ++e) b[e] = s.be[cur][(4 * lg + e) * K16 + i];
          const Split3 bs = split3(b);
#pragma unroll
          for (int jb = 0; jb < VB; ++jb) {
#pragma unroll
            for (int e = 0; e < 4; ++e) Ht[jb][e] *= ce;
            Ht[jb] = mma_ex(Ht[jb], bits4(&s.d[(c0 + 4 * lg) * VP + jb * 16 + lr], VP), bs);
          }
        } else {
#pragma unroll
          for (int jb = 0; jb < VB; ++jb) {
            v4f a, b;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              Ht[jb][e] *= ce;
              a[e] = to_f32(s.d[(c0 + 4 * lg + e) * VP + jb * 16 + lr]);
              b[e] = s.be[cur][(4 * lg + e) * K16 + i];
            }
            Ht[jb] = mma_f32(Ht[jb], a, b);
          }
        }
      }
    }
    KLA_BTL(5);
    if (w > 0) {
      if (wave >= 4)
        chunk_operands<K, V, BF16>(s, w - 1, (w - 1) & 1, grp_v, kRowsV, 192, false, tid - 256, wave, lg, lr);
      else
        chunk_operands<K, V, BF16>(s, w - 1, (w - 1) & 1, kRowsV + tid, C * K, 256, wave == 3, -1, wave, lg, lr);
    }
    KLA_BTL(6);
    __syncthreads();
  }
  if (more)
    for (int pt = wl + 1; pt < SegLoads<K, V, BF16, NT>::NPART; ++pt) seg_load(p, nhd, nt0, nxt, pt);
  }  // segments
  KLA_BTL(7);
  KLA_BTL_END();
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
  float lam, lprev, a2, D, k, vp, dg, e;
  float ilam, iD, ilprev;  // hardware reciprocals (about 1 ulp)
};

template <bool BF16>
// Token data of one chain at key-side index x and workspace index xw;
// lam0v is the precision before the first token (used when first).
__device__ __forceinline__ ChainTok chain_tok(const BwdParams& p, size_t x, size_t xw, bool first, float lam0v) {
  ChainTok c;
  c.lam = p.lpath[x];
  c.lprev = first ? lam0v : p.lpath[x - p.ks];
  const float a = __expf(ldin<BF16>(p.ld, x));
  c.a2 = a * a;
  c.D = fmaf(ldin<BF16>(p.pn, x), c.lprev, c.a2);
  c.ilam = fast_rcp(c.lam);
  c.iD = fast_rcp(c.D);
  c.ilprev = fast_rcp(c.lprev);
  c.k = ldin<BF16>(p.k, x);
  c.vp = ldin<BF16>(p.vp, x);
  c.dg = p.dgw[xw];
  c.e = p.ew[xw];
  if (p.ehalf) {  // the second value half's partials, added to the first's
    c.dg += p.dgw[xw + p.ehalf];
    c.e += p.ew[xw + p.ehalf];
  }
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
  // Per-thread bases; each token adds a uniform offset (scalar arithmetic).
  const size_t bk = (hd * p.T + tb) * p.ks + i, bw = (hd * p.T + tb) * p.kws + i;
  const float lam0v = (tb == 0 && p.lam0) ? p.lam0[hd * p.ksh + i] : 1.f;
  float E = 0.f, Pm = 1.f, Qa = 0.f, R = 0.f;
  auto step = [&](int t) {
    const int u = t - tb;
    const ChainTok c = chain_tok<BF16>(p, bk + (size_t)u * p.ks, bw + (size_t)u * p.kws, t == 0, lam0v);
    const float g = c.k * c.vp * c.ilam;
    const float m = c.a2 * c.iD * c.iD;
    const float c1 = c.k * c.k * c.vp * c.ilam * c.D * c.ilprev;  // c / (lam lam^-), lam^- = lprev / D
    const float c0 = -g * c.dg * c.ilam;
    E += c.e;
    Pm *= m;
    Qa = m * (Qa + c1);
    R = m * fmaf(c1, E, R + c0);
  };
  if (te - tb == kSL) {
    // Full block: unrolled, so that several tokens' loads are in flight.
#pragma unroll 8
    for (int u = kSL - 1; u >= 0; --u) step(tb + u);
  } else {
    for (int t = te - 1; t >= tb; --t) step(t);
  }
  reinterpret_cast<float4*>(p.comp)[(size_t)b * p.nchains + ch] = make_float4(E, Pm, Qa, R);
}

__global__ __launch_bounds__(256) void kla_bwd_chain_carry_kernel(BwdParams p, int K) {
  const long long ch = (long long)blockIdx.x * 256 + threadIdx.x;
  if (ch >= p.nchains) return;
  const size_t kv = (size_t)(ch / K) * p.ksh + ch % K;  // this channel in the key vectors
  float acc = p.rs[kv], L = p.dlamT ? p.dlamT[kv] : 0.f;
  const float4* comp = reinterpret_cast<const float4*>(p.comp);
  float2* cin = reinterpret_cast<float2*>(p.cin);
  int b = p.nseg - 1;
  // Blocks in batches of eight, the batch's loads issued together (the
  // recursion itself is a few multiply-adds per block).
  for (; b >= 7; b -= 8) {
    float4 c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) c[u] = comp[(size_t)(b - u) * p.nchains + ch];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      cin[(size_t)(b - u) * p.nchains + ch] = make_float2(acc, L);
      L = fmaf(c[u].y, L, fmaf(c[u].z, acc, c[u].w));
      acc += c[u].x;
    }
  }
  for (; b >= 0; --b) {
    cin[(size_t)b * p.nchains + ch] = make_float2(acc, L);
    const float4 c = comp[(size_t)b * p.nchains + ch];
    L = fmaf(c.y, L, fmaf(c.z, acc, c.w));
    acc += c.x;
  }
  p.dlam0[kv] = L;
}

template <bool BF16>
__global__ __launch_bounds__(256) void kla_bwd_chain_out_kernel(BwdParams p, int K, int ncb) {
  const long long ch = (long long)(blockIdx.x % ncb) * 256 + threadIdx.x;
  const int b = blockIdx.x / ncb;
  if (ch >= p.nchains) return;
  const size_t hd = ch / K;
  const int i = (int)(ch % K);
  const int tb = b * kSL, te = min(p.T, tb + kSL);
  const size_t bk = (hd * p.T + tb) * p.ks + i, bw = (hd * p.T + tb) * p.kws + i;
  const float lam0v = (tb == 0 && p.lam0) ? p.lam0[hd * p.ksh + i] : 1.f;
  const float2 in = reinterpret_cast<const float2*>(p.cin)[(size_t)b * p.nchains + ch];
  float acc = in.x, L = in.y;
  auto step = [&](int t) {
    const int u = t - tb;
    const size_t x = bk + (size_t)u * p.ks;
    const ChainTok c = chain_tok<BF16>(p, x, bw + (size_t)u * p.kws, t == 0, lam0v);
    const float g = c.k * c.vp * c.ilam;
    const float c0 = -g * c.dg * c.ilam;
    acc += c.e;                                                   // d log f_t
    const float dc = fmaf(-acc, c.ilam, L + c0);                  // dL/dlambda_t = dL/dc_t
    const float c1 = c.k * c.k * c.vp * c.ilam * c.D * c.ilprev;  // c / (lam lam^-)
    const float Llp = fmaf(c1, acc, L + c0);                      // dL/dlambda^-_t
    const float w = -Llp * c.lprev * c.iD * c.iD;                 // dL/d(a^2)
    stout<BF16>(p.dld, x, fmaf(2.f * c.a2, w, acc));              // a dL/da = d log f + 2 a^2 dL/d(a^2)
    stout<BF16>(p.dpn, x, w * c.lprev);
    stout<BF16>(p.dk, x, c.vp * c.ilam * c.dg + 2.f * c.k * c.vp * dc);
    stout<BF16>(p.dvp, x, c.k * c.ilam * c.dg + c.k * c.k * dc);
    L = Llp * (c.a2 * c.iD * c.iD);
  };
  if (te - tb == kSL) {
#pragma unroll 8
    for (int u = kSL - 1; u >= 0; --u) step(tb + u);
  } else {
    for (int t = te - 1; t >= tb; --t) step(t);
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
static hipError_t launch_front(const BwdParams& p, hipStream_t stream) {
  const unsigned nsb = (unsigned)((long long)p.nheads * p.nseg);
  // Two workgroups per compute unit fit its LDS; each walks several segments.
  const unsigned nagg = nsb < 2u * (unsigned)p.ncu ? nsb : 2u * (unsigned)p.ncu;
  hipLaunchKernelGGL((kla_bwd_segagg_kernel<K, V, BF16>), dim3(nagg), dim3(512), 0, stream, p);
  constexpr int NB = (K * V + 255) / 256;
  hipLaunchKernelGGL((kla_bwd_segscan_kernel<K, V>), dim3((unsigned)(p.nheads * NB)), dim3(256), 0, stream, p);
  // One workgroup per compute unit (its registers allow no more), each
  // walking several segments.
  const unsigned nchunk = nsb < (unsigned)p.ncu ? nsb : (unsigned)p.ncu;
  hipLaunchKernelGGL((kla_bwd_chunk_kernel<K, V, BF16>), dim3(nchunk), dim3(kChunkThreads), 0, stream, p);
  return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_chain(const BwdParams& p, int K, hipStream_t stream) {
  const int ncb = (int)((p.nchains + 255) / 256);
  const unsigned ncomp = (unsigned)((long long)ncb * p.nseg);
  hipLaunchKernelGGL((kla_bwd_chain_comp_kernel<BF16>), dim3(ncomp), dim3(256), 0, stream, p, K, ncb);
  hipLaunchKernelGGL(kla_bwd_chain_carry_kernel, dim3((unsigned)ncb), dim3(256), 0, stream, p, K);
  hipLaunchKernelGGL((kla_bwd_chain_out_kernel<BF16>), dim3(ncomp), dim3(256), 0, stream, p, K, ncb);
  return hipGetLastError();
}

template <int K, bool BF16>
static hipError_t front_dv(const BwdParams& p, int dv, hipStream_t stream) {
  switch (dv) {
    case 16: return launch_front<K, 16, BF16>(p, stream);
    case 32: return launch_front<K, 32, BF16>(p, stream);
    case 64: return launch_front<K, 64, BF16>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16>
static hipError_t front_dk(const BwdParams& p, int dk, int dv, hipStream_t stream) {
  switch (dk) {
    case 16: return front_dv<16, BF16>(p, dv, stream);
    case 32: return front_dv<32, BF16>(p, dv, stream);
    case 64: return front_dv<64, BF16>(p, dv, stream);
    default: return hipErrorInvalidValue;
  }
}

// Segment aggregates, segment scans and the chunk kernel of one sub-problem
// (dk, dv <= 64).
hipError_t launch_backward_front(const BwdParams& p, int dk, int dv, bool bf16, hipStream_t stream) {
  return bf16 ? front_dk<true>(p, dk, dv, stream) : front_dk<false>(p, dk, dv, stream);
}

// The per-channel reverse chain of dk channels (after every value half of
// them has been through the front).
hipError_t launch_backward_chain(const BwdParams& p, int dk, bool bf16, hipStream_t stream) {
  return bf16 ? launch_chain<true>(p, dk, stream) : launch_chain<false>(p, dk, stream);
}

template <bool BF16>
__global__ __launch_bounds__(256) void kla_bwd_convert_kernel(const float* acc, void* out, long long n) {
  const long long x = (long long)blockIdx.x * 256 + threadIdx.x;
  if (x < n) stout<BF16>(out, x, acc[x] + acc[x + n]);
}

// Two fp32 partials (acc[0 .. n) and acc[n .. 2n), the two halves of a
// 128-wide sum) -> their sum in the output dtype.
hipError_t launch_backward_convert(const float* acc, void* out, long long n, bool bf16, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(kla_bwd_convert_kernel<true>, grid, dim3(256), 0, stream, acc, out, n);
  else
    hipLaunchKernelGGL(kla_bwd_convert_kernel<false>, grid, dim3(256), 0, stream, acc, out, n);
  return hipGetLastError();
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

#ifdef KLA_TIMELINE
extern "C" int kla_bwd_timeline_read(void* host, size_t bytes) {
  const size_t n = sizeof(kla::kla_bwd_timeline_buf);
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(kla::kla_bwd_timeline_buf), bytes < n ? bytes : n, 0,
                                  hipMemcpyDeviceToHost);
}
#endif
