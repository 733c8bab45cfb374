// Device-side building blocks shared by the KLA kernels (gfx950 / CDNA4).
//
// Sources: gist.science summaries of arXiv 2602.10743, "Kalman Linear Attention";
// [KLA-nl] = "Technische Samenvatting: Kalman Linear Attention (KLA)".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kla_internal.h"

namespace kla {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// A wait on a predecessor gives up after this many polls (each followed by a
// short sleep, ~1-2 s in total) and records an error instead of hanging.
constexpr int kSpinLimit = 1 << 25;

// ----------------------------------------------------------------------------
// Element conversion.  bf16 values travel as their 16-bit patterns.
// ----------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float to_f32(float x) { return x; }

// float32 -> bfloat16, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename In> __device__ __forceinline__ In from_f32(float x);
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) { return bf16_rne(x); }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// ----------------------------------------------------------------------------
// 16x16 matrix-core tiles.
//
// Layout of one 16x16 fp32 accumulator tile D (64 lanes, 4 values per lane):
//   lane l, element e holds D[4*(l/16) + e][l % 16].
// A K=16 operand block holds 4 values per lane along k:
//   A operand (m x k): lane l, element e holds A[l % 16][4*(l/16) + e]
//   B operand (k x n): lane l, element e holds B[4*(l/16) + e][l % 16]
// so an accumulator tile serves directly as a B operand (its rows become k),
// and its transpose as an A operand.
//
// Precision.  Gated operands (q*cp, g/cp, the state, the scores) are fp32
// values; rounding them once to bf16 costs up to 2^-9 relative per product,
// which the cancellation inside y amplifies beyond the bf16-input tolerance
// (the x100 value-precision spikes make it visible).  Each such operand is
// therefore split into hi = bf16(x) and lo = bf16(x - hi) (about 16 mantissa
// bits together) and a product takes hi*hi + lo*hi + hi*lo; the bf16 input V
// is exact and needs no split.  Two K=16 blocks are packed into one
// v_mfma_f32_16x16x32_bf16 (elements 0-3 of a lane hold the first block,
// 4-7 the second, identically for A and B, so the instruction adds the two
// block products).  Every bf16 contraction uses this one instruction shape:
// a v_mfma_f32_16x16x16_bf16 issued right after a 16x16x32 that feeds its
// accumulator read that accumulator before the 16x16x32 had written it (no
// wait states were emitted between the two shapes), so an odd leftover block
// is padded with zeros instead.  The fp32 path uses v_mfma_f32_16x16x4_f32 four times per
// block (step e contracts k = 4*(l/16) + e over the four lane groups).
// ----------------------------------------------------------------------------
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

struct SFrag {  // split fp32 block: hi and lo bf16 parts
  v4s hi, lo;
};

__device__ __forceinline__ SFrag split4(v4f x) {
  SFrag f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint16_t h = bf16_rne(x[e]);
    f.hi[e] = (short)h;
    f.lo[e] = (short)bf16_rne(x[e] - to_f32(h));
  }
  return f;
}

__device__ __forceinline__ v4f mma_x32(v4f acc, v4s a0, v4s a1, v4s b0, v4s b1) {
  const v8s a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
  const v8s b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b),
                                                 acc, 0, 0, 0);
}
__device__ __forceinline__ v4f mma_f32(v4f acc, v4f a, v4f b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
  return acc;
}

// Operand policy per input dtype.
//   Op  : a gated fp32 operand block (split for bf16 inputs, plain for fp32)
//   VOp : an operand block read from the inputs (exact in its own dtype)
template <bool BF16> struct Mma;

template <> struct Mma<true> {
  using Op = SFrag;
  using VOp = v4s;
  static __device__ __forceinline__ Op op(v4f x) { return split4(x); }
  static __device__ __forceinline__ VOp vop(const uint16_t* p, int stride) {
    return v4s{(short)p[0], (short)p[stride], (short)p[2 * stride], (short)p[3 * stride]};
  }
  // acc += sum_b A[b] . B[b], both operands split.
  template <int NB>
  static __device__ __forceinline__ v4f dot(v4f acc, const Op (&A)[NB], const Op (&B)[NB]) {
#pragma unroll
    for (int b = 0; b < NB; ++b) acc = mma_x32(acc, A[b].hi, A[b].lo, B[b].hi, B[b].hi);
#pragma unroll
    for (int b = 0; b + 1 < NB; b += 2) acc = mma_x32(acc, A[b].hi, A[b + 1].hi, B[b].lo, B[b + 1].lo);
    if (NB % 2) {  // odd leftover: x32 with a zero second half
      const v4s z = v4s{0, 0, 0, 0};
      acc = mma_x32(acc, A[NB - 1].hi, z, B[NB - 1].lo, z);
    }
    return acc;
  }
  // acc += A . V, A split, V exact.
  static __device__ __forceinline__ v4f dotv(v4f acc, const Op& A, VOp V) {
    return mma_x32(acc, A.hi, A.lo, V, V);
  }
};

template <> struct Mma<false> {
  using Op = v4f;
  using VOp = v4f;
  static __device__ __forceinline__ Op op(v4f x) { return x; }
  static __device__ __forceinline__ VOp vop(const float* p, int stride) {
    return v4f{p[0], p[stride], p[2 * stride], p[3 * stride]};
  }
  template <int NB>
  static __device__ __forceinline__ v4f dot(v4f acc, const Op (&A)[NB], const Op (&B)[NB]) {
#pragma unroll
    for (int b = 0; b < NB; ++b) acc = mma_f32(acc, A[b], B[b]);
    return acc;
  }
  static __device__ __forceinline__ v4f dotv(v4f acc, const Op& A, VOp V) { return mma_f32(acc, A, V); }
};

// ----------------------------------------------------------------------------
// One filter step ([KLA-nl] §1-§2).  Coefficients of token t for one channel:
//   a2 = a^2 (a = exp(log_decay)), pb = process-noise variance,
//   c  = k^2 Lambda^v (observation precision).
// Predict then update in precision form:
//   lam^- = lam / (a2 + pb*lam),  lam_t = lam^- + c.
// As a projective 2x2 matrix acting on [lam; 1] (the Möbius map's alpha..delta):
//   [[1 + c*pb, c*a2], [pb, a2]] = [[1, c],[0, 1]] . [[1, 0],[pb, a2]].
// ----------------------------------------------------------------------------
struct Mob {
  float m00, m01, m10, m11;
};

__device__ __forceinline__ Mob mob_identity() { return Mob{1.f, 0.f, 0.f, 1.f}; }

// Rescale by a power of two so the largest entry lies in [0.5, 1): exact, and
// a projective matrix is unchanged by any positive scale.
__device__ __forceinline__ Mob mob_normalize(Mob m) {
  float mx = fmaxf(fmaxf(m.m00, m.m01), fmaxf(m.m10, m.m11));
  int e = __builtin_amdgcn_frexp_expf(mx);
  return Mob{__builtin_amdgcn_ldexpf(m.m00, -e), __builtin_amdgcn_ldexpf(m.m01, -e),
             __builtin_amdgcn_ldexpf(m.m10, -e), __builtin_amdgcn_ldexpf(m.m11, -e)};
}

// step(a2, pb, c) . P, normalised.
__device__ __forceinline__ Mob mob_step(Mob P, float a2, float pb, float c) {
  const float al = fmaf(c, pb, 1.f), be = c * a2;
  Mob n;
  n.m00 = fmaf(al, P.m00, be * P.m10);
  n.m01 = fmaf(al, P.m01, be * P.m11);
  n.m10 = fmaf(pb, P.m00, a2 * P.m10);
  n.m11 = fmaf(pb, P.m01, a2 * P.m11);
  return mob_normalize(n);
}

// A . B (B applied first), normalised.
__device__ __forceinline__ Mob mob_mul(Mob A, Mob B) {
  Mob n;
  n.m00 = fmaf(A.m00, B.m00, A.m01 * B.m10);
  n.m01 = fmaf(A.m00, B.m01, A.m01 * B.m11);
  n.m10 = fmaf(A.m10, B.m00, A.m11 * B.m10);
  n.m11 = fmaf(A.m10, B.m01, A.m11 * B.m11);
  return mob_normalize(n);
}

// The Möbius map of P applied to lam.  Every fold of carries uses this one
// function, so the carried precision is the same bits whichever predecessor
// a look-back starts from.
__device__ __forceinline__ float mob_apply(Mob P, float lam) {
  return fmaf(P.m00, lam, P.m01) / fmaf(P.m10, lam, P.m11);
}

// Scalar predict/update step; returns lam_t and writes lam^-.
__device__ __forceinline__ float lam_step(float lam, float a2, float pb, float c, float& lam_pred) {
  lam_pred = lam * fast_rcp(fmaf(pb, lam, a2));
  return lam_pred + c;
}

// ----------------------------------------------------------------------------
// Inter-workgroup publication (decoupled look-back).  Payload stores are
// ordinary stores followed by an agent-scope release fence in every writing
// thread; the flag is stored with release semantics by one thread after a
// workgroup barrier.  Readers poll with acquire loads, then every reading
// thread issues an agent-scope acquire fence before touching the payload.
// ----------------------------------------------------------------------------
__device__ __forceinline__ unsigned ld_acquire(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_release(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_release() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}
__device__ __forceinline__ void fence_acquire() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Walk back from segment `s - 1` to the nearest predecessor that has published
// its inclusive carry (flag == finc); predecessors that have published only
// their own aggregate (flag == fagg) are stepped over.  Segment 0 always
// publishes an inclusive carry, so the walk ends.  Returns the index found.
// Called by one thread.
__device__ inline int lookback_find(const unsigned* flags, int s, unsigned fagg, unsigned finc,
                                    unsigned* ctrl) {
  int r = s - 1;
  int spins = 0;
  while (r > 0) {
    unsigned f = ld_acquire(flags + r);
    if (f == finc) return r;
    if (f == fagg) {
      --r;
      continue;
    }
    if (++spins > kSpinLimit) {
      __hip_atomic_store(ctrl + kError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return r;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  // r == 0: wait for segment 0's inclusive carry.
  while (ld_acquire(flags) != finc) {
    if (++spins > kSpinLimit) {
      __hip_atomic_store(ctrl + kError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return 0;
}

// Workgroup order: a ticket taken at start, so every workgroup a segment waits
// on has started before it (no wait on a workgroup that cannot be scheduled).
__device__ __forceinline__ unsigned take_ticket(unsigned* ctrl) {
  return __hip_atomic_fetch_add(ctrl + kTicket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Last workgroup out resets the ticket and exit counters and advances the
// epoch, so flags of this call never match the next call's.
__device__ __forceinline__ void finish_call(unsigned* ctrl, unsigned epoch, unsigned nblocks) {
  unsigned old = __hip_atomic_fetch_add(ctrl + kDone, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  if (old == nblocks - 1) {
    __hip_atomic_store(ctrl + kDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(ctrl + kTicket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(ctrl + kEpoch, epoch + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace kla
