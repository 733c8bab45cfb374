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

// float32 -> bfloat16, round to nearest even, by the hardware conversion
// (v_cvt_pk_bf16_f32 converts two values per instruction).
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v2s __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v2s bf16x2(float a, float b) {
  return __builtin_bit_cast(v2s, __builtin_convertvector(v2f{a, b}, v2bf));
}
__device__ __forceinline__ uint16_t bf16_rne(float x) {
  return (uint16_t)__builtin_bit_cast(short, static_cast<__bf16>(x));
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

// hi = bf16(x) (nearest even), lo = bf16(x - hi): about 16 mantissa bits together.
__device__ __forceinline__ void split4(v4f x, v4s& hi, v4s& lo) {
  const v2s h01 = bf16x2(x[0], x[1]), h23 = bf16x2(x[2], x[3]);
  const v2s l01 = bf16x2(x[0] - to_f32((uint16_t)h01[0]), x[1] - to_f32((uint16_t)h01[1]));
  const v2s l23 = bf16x2(x[2] - to_f32((uint16_t)h23[0]), x[3] - to_f32((uint16_t)h23[1]));
  hi = v4s{h01[0], h01[1], h23[0], h23[1]};
  lo = v4s{l01[0], l01[1], l23[0], l23[1]};
}
__device__ __forceinline__ v8s cat(v4s a, v4s b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }
// first / second half of a split block: the hi part / the lo part
__device__ __forceinline__ v4s part_hi(v8s a) { return __builtin_shufflevector(a, a, 0, 1, 2, 3); }
__device__ __forceinline__ v4s part_lo(v8s a) { return __builtin_shufflevector(a, a, 4, 5, 6, 7); }

__device__ __forceinline__ v4f mma_x32(v4f acc, v8s a, v8s b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), acc,
                                                 0, 0, 0);
}
__device__ __forceinline__ v4f mma_f32(v4f acc, v4f a, v4f b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
  return acc;
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of
// 16 lanes, lane i receives element i % 4 of the 8-byte rows read by lanes
// 4r + i / 4 (as element r, r = 0..3): the 4 x 16 block the group reads as
// sixteen 4-element pieces comes back transposed.  (Lane layout checked on
// the device with a probe that filled LDS with each element's own index.)
typedef __attribute__((address_space(3))) v4s lds_v4s;
__device__ __forceinline__ v4s lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p));
}

// Operand policy per input dtype.
//   Op   one K=16 block of a gated fp32 operand.  bf16 inputs: the block's hi
//        and lo parts as one 8-element vector [hi0..3 | lo0..3] (so an A-side
//        block feeds v_mfma_f32_16x16x32_bf16 as it is loaded); fp32 inputs:
//        the four fp32 values.
//   VOp  one block read from the inputs, exact in its own dtype.
// Stored operands keep this layout in LDS: 16 bytes per block (bf16) or
// 16 bytes per 4 values (fp32), so one aligned 16-byte load fetches a block.
template <bool BF16> struct Mma;

template <> struct Mma<true> {
  using Op = v8s;
  using VOp = v4s;
  static __device__ __forceinline__ Op op(v4f x) {
    v4s h, l;
    split4(x, h, l);
    return cat(h, l);
  }
  static __device__ __forceinline__ Op get(const unsigned char* p) { return *reinterpret_cast<const v8s*>(p); }
  static __device__ __forceinline__ void put(unsigned char* p, v4f x) { *reinterpret_cast<v8s*>(p) = op(x); }
  static __device__ __forceinline__ VOp vop(const uint16_t* p, int stride) {
    return v4s{(short)p[0], (short)p[stride], (short)p[2 * stride], (short)p[3 * stride]};
  }
  // acc += sum_b A[b] . B[b]; each product takes hi*hi + lo*hi + hi*lo.
  template <int NB>
  static __device__ __forceinline__ v4f dot(v4f acc, const Op (&A)[NB], const Op (&B)[NB]) {
#pragma unroll
    for (int b = 0; b < NB; ++b) acc = mma_x32(acc, A[b], cat(part_hi(B[b]), part_hi(B[b])));
#pragma unroll
    for (int b = 0; b + 1 < NB; b += 2)
      acc = mma_x32(acc, cat(part_hi(A[b]), part_hi(A[b + 1])), cat(part_lo(B[b]), part_lo(B[b + 1])));
    if (NB % 2) {  // odd leftover: x32 with a zero second half
      const v4s z = v4s{0, 0, 0, 0};
      acc = mma_x32(acc, cat(part_hi(A[NB - 1]), z), cat(part_lo(B[NB - 1]), z));
    }
    return acc;
  }
  // acc += A . V, A split, V exact.
  static __device__ __forceinline__ v4f dotv(v4f acc, const Op& A, VOp V) { return mma_x32(acc, A, cat(V, V)); }
};

template <> struct Mma<false> {
  using Op = v4f;
  using VOp = v4f;
  static __device__ __forceinline__ Op op(v4f x) { return x; }
  static __device__ __forceinline__ Op get(const unsigned char* p) { return *reinterpret_cast<const v4f*>(p); }
  static __device__ __forceinline__ void put(unsigned char* p, v4f x) { *reinterpret_cast<v4f*>(p) = x; }
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
  float mx = __builtin_fmaxf(__builtin_fmaxf(m.m00, m.m01), __builtin_fmaxf(m.m10, m.m11));
  int e = __builtin_amdgcn_frexp_expf(mx);
  return Mob{__builtin_amdgcn_ldexpf(m.m00, -e), __builtin_amdgcn_ldexpf(m.m01, -e),
             __builtin_amdgcn_ldexpf(m.m10, -e), __builtin_amdgcn_ldexpf(m.m11, -e)};
}

// step(a2, pb, c) . P as two row operations (predict, then update); not
// normalised.  An entry grows per step by at most the step matrix's largest
// row sum, so normalising every fourth step keeps every entry inside the fp32
// range while that sum stays below about 10^9 (1 + c*pb + c*a2 for realistic
// coefficients is many orders smaller).  The (0,0) entry never shrinks below
// its value before the step, so nothing that matters underflows.
__device__ __forceinline__ Mob mob_step_raw(Mob P, float a2, float pb, float c) {
  Mob n;
  n.m10 = fmaf(pb, P.m00, a2 * P.m10);  // predict: row1 <- pb*row0 + a2*row1
  n.m11 = fmaf(pb, P.m01, a2 * P.m11);
  n.m00 = fmaf(c, n.m10, P.m00);        // update:  row0 <- row0 + c*row1
  n.m01 = fmaf(c, n.m11, P.m01);
  return n;
}
__device__ __forceinline__ Mob mob_step(Mob P, float a2, float pb, float c) {
  return mob_normalize(mob_step_raw(P, a2, pb, c));
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

// The Möbius map of P applied to lam (hardware reciprocal: about 1 ulp).
// Every fold of carries uses this one function, so the carried precision is
// the same bits whichever predecessor a look-back starts from.
__device__ __forceinline__ float mob_apply(Mob P, float lam) {
  return fmaf(P.m00, lam, P.m01) * fast_rcp(fmaf(P.m10, lam, P.m11));
}

// Scalar predict/update step; returns lam_t and writes lam^-.
__device__ __forceinline__ float lam_step(float lam, float a2, float pb, float c, float& lam_pred) {
  lam_pred = lam * fast_rcp(fmaf(pb, lam, a2));
  return lam_pred + c;
}

// ----------------------------------------------------------------------------
// Inter-workgroup publication (decoupled look-back).
// Payloads and flags are written and read with agent-coherent accesses
// (the sc1 cache policy that agent-scope atomics use), so no cache-wide write
// back or invalidate is needed:
//   publish: every writing thread stores its part of the payload coherently
//            and waits for its stores to complete; a workgroup barrier; one
//            thread stores the flag coherently.
//   consume: one thread polls the flag with coherent loads (sleeping between
//            polls); a workgroup barrier; the threads load the payload
//            coherently.
// A payload store that has completed is visible to every coherent load on
// the device, and the flag is stored only after all payload stores of the
// workgroup completed, so a reader that sees the flag sees the payload.
// ----------------------------------------------------------------------------
constexpr int kCoherent = 16;  // buffer cache-policy operand: sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
typedef unsigned v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, v4f x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, x), r, (int)off, 0, kCoherent);
}
__device__ __forceinline__ v4f ld_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCoherent));
}
__device__ __forceinline__ void st_coherent(float* p, float x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_relaxed(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A float published together with its flag in one 64-bit word (value bits
// low, flag high).  Aligned 64-bit accesses are single-copy atomic, so a
// reader that sees the flag sees the value stored with it, without waiting
// for any other store.
__device__ __forceinline__ void st_record(unsigned long long* p, float v, unsigned flag) {
  __hip_atomic_store(p, ((unsigned long long)flag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_record(const unsigned long long* p) {
  return __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float record_value(unsigned long long r) { return __uint_as_float((unsigned)r); }
__device__ __forceinline__ unsigned record_flag(unsigned long long r) { return (unsigned)(r >> 32); }

// Wait until this thread's outstanding memory operations have completed.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); /* vmcnt(0) */ }

// Find the nearest predecessor of segment `s` that has published its
// inclusive carry (flag == finc) such that every segment between them has
// published at least its aggregate (flag == fagg).  Segment 0 always
// publishes an inclusive carry, so the search ends.  One wavefront polls a
// window of 64 predecessors at once (lane j reads segment s-1-j), so a
// look-back costs one memory round trip per window instead of one per
// predecessor.  `stride` is the distance between the flags of consecutive
// segments.  Called by all 64 lanes of one wavefront (uniform result); on
// giving up after kSpinLimit polls it records an error and returns.
//
// lookback_peek issues the first window's flag loads on their own, so that
// their round trip can overlap the publication of the caller's own aggregate;
// its result is handed to lookback_find.
__device__ __forceinline__ unsigned lookback_peek(const unsigned* flags, int stride, int top) {
  const int r = top - (int)(threadIdx.x & 63);
  return r >= 0 ? ld_relaxed(flags + (size_t)r * stride) : 0u;
}
__device__ inline int lookback_find(const unsigned* flags, int stride, int s, unsigned fagg, unsigned finc,
                                    unsigned* ctrl, unsigned f) {
  const int lane = threadIdx.x & 63;
  int top = s - 1;  // newest predecessor of the current window; f holds its flags
  int spins = 0;
  while (true) {
    const int r = top - lane;
    const unsigned long long inc = __ballot(r >= 0 && f == finc);
    const unsigned long long ready = __ballot(r >= 0 && (f == finc || f == fagg));
    if (inc) {
      const int j = __builtin_ctzll(inc);  // nearest inclusive carry in the window
      const unsigned long long below = j ? ((1ull << j) - 1) : 0ull;
      if ((ready & below) == below) return top - j;
    } else if (ready == ~0ull) {
      top -= 64;  // the whole window holds aggregates only: look further back
      f = lookback_peek(flags, stride, top);
      continue;
    }
    if (++spins > kSpinLimit) {
      if (lane == 0) st_relaxed(ctrl + kError, 1u);
      return top;
    }
    __builtin_amdgcn_s_sleep(1);
    f = lookback_peek(flags, stride, top);
  }
}
__device__ inline int lookback_find(const unsigned* flags, int stride, int s, unsigned fagg, unsigned finc,
                                    unsigned* ctrl) {
  return lookback_find(flags, stride, s, fagg, finc, ctrl, lookback_peek(flags, stride, s - 1));
}

// Draws this workgroup's ticket from the counter of its group (blockIdx %
// groups), which takes `per_group` tickets per call; the workgroup that draws
// the last one sets the counter back to zero for the next call.
__device__ __forceinline__ unsigned draw_ticket(unsigned* tick, unsigned groups, unsigned per_group) {
  unsigned* const tk = tick + kTicketStride * (blockIdx.x % groups);
  const unsigned t = __hip_atomic_fetch_add(tk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (t == per_group - 1u) st_relaxed(tk, 0u);
  return t;
}

// Call epochs.  Every workgroup reads the workspace epoch e before touching
// flags, so flags of this call (values 2e+2, 2e+3) never match those left by
// earlier calls, whatever their shapes.  Each workgroup counts itself done
// once it no longer needs the epoch; the last of the `ngroups` workgroups
// resets the counter and advances the epoch for the next call (calls on one
// workspace are ordered on one stream, so no workgroup of the next call runs
// before every workgroup of this one has finished).
enum CtrlEpoch { kEpoch = 0, kGroupsDone = 1 };
__device__ __forceinline__ void epoch_done(unsigned* ctrl, unsigned ngroups, unsigned e) {
  if (__hip_atomic_fetch_add(ctrl + kGroupsDone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != ngroups - 1)
    return;
  st_relaxed(ctrl + kGroupsDone, 0u);
  st_relaxed(ctrl + kEpoch, e + 1u);
}

// The same with workgroups counted in groups first (one counter per group, then
// one for the groups), which spreads the counting atomics over many addresses
// when many workgroups finish together.
__device__ __forceinline__ void epoch_done_grouped(unsigned* ctrl, unsigned* group_done, unsigned group_size,
                                                   unsigned ngroups, unsigned e) {
  if (__hip_atomic_fetch_add(group_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != group_size - 1) return;
  st_relaxed(group_done, 0u);
  epoch_done(ctrl, ngroups, e);
}

// The same for `nunits` units of `per_unit` workgroups each, counted on the
// fixed array of kDoneCounters words `done` (unit u on word u % kDoneCounters,
// whose group then holds every unit congruent to it).
__device__ __forceinline__ void epoch_done_units(unsigned* ctrl, unsigned* done, unsigned unit, unsigned nunits,
                                                 unsigned per_unit, unsigned e) {
  constexpr unsigned NC = (unsigned)kDoneCounters;
  const unsigned g = unit % NC;
  const unsigned members = nunits / NC + (g < nunits % NC ? 1u : 0u);
  epoch_done_grouped(ctrl, done + g, per_unit * members, nunits < NC ? nunits : NC, e);
}

}  // namespace kla
