// Precision path only: independent Möbius chains lam_t = step_t(lam_{t-1}).
//
// Source: gist.science "Technische Samenvatting: Kalman Linear Attention (KLA)"
// (summary of arXiv 2602.10743), §2 "Parallelisatie via Möbius-transformaties":
// the posterior precision is a Möbius map of the previous one, and Möbius maps
// compose associatively (2x2 matrix products), which permits a prefix scan.
//
// Layout [B,H,T,D]: at a fixed token the D chains of a head are contiguous, so
// one lane per chain makes every token one coalesced row per wavefront.  Each
// lane walks its chain over a T-segment with loads issued a block of tokens
// ahead.  When there are too few chains to fill the GPU, T is split into
// segments: each segment first composes its 2x2 aggregate, publishes it, and a
// decoupled look-back over earlier segments gives the entering precision before
// the segment is walked again to write the path.
#include "kla_device.h"
#include "kla_internal.h"

namespace kla {

constexpr int kPB = 8;  // tokens per prefetch block

__global__ __launch_bounds__(256) void kla_pscan_kernel(PscanParams p) {
  __shared__ int sh[4];
  const int tid = threadIdx.x;
  const int nseg = p.nseg;
  // (chain block, segment) from a ticket when segments wait on predecessors:
  // group x = blockIdx % tgroups serves chain blocks x, x + tgroups, ...,
  // segment-major, so every segment a workgroup waits on holds a smaller
  // ticket of its own counter and started earlier.
  if (nseg > 1 && tid == 0)
    sh[3] = (int)draw_ticket(p.tick, (unsigned)p.tgroups, (unsigned)p.ncblocks / (unsigned)p.tgroups * (unsigned)nseg);
  if (tid == 0) sh[1] = nseg > 1 ? (int)ld_relaxed(p.ctrl + kEpoch) : 0;
  if (nseg > 1) __syncthreads();
  const unsigned ticket = nseg > 1 ? (unsigned)sh[3] : blockIdx.x;
  const unsigned tg = nseg > 1 ? (unsigned)p.tgroups : 1u, cpg = (unsigned)p.ncblocks / tg;
  const int seg = (int)(ticket / cpg), cb = (int)((ticket % cpg) * tg + blockIdx.x % tg);
  const bool last = seg == nseg - 1;
  const long long chain = (long long)cb * 256 + tid;
  const bool valid = chain < p.nchains;
  const int D = p.D, T = p.T;
  const long long bh = valid ? chain / D : 0, d = valid ? chain % D : 0;
  const long long base = bh * T * (long long)D + d;  // element (bh, t=0, d)
  const int tb = seg * p.seglen, te = min(T, tb + p.seglen);
  const int n = valid ? te - tb : 0;
  const size_t slot = (size_t)(seg * p.ncblocks + cb);  // (segment, chain block)
  const size_t cslot = slot * 256 + tid;                // per-chain payload

  // Loads one block of kPB tokens starting at token t (identity past the end).
  auto load_block = [&](int t, float* l, float* q, float* c) {
#pragma unroll
    for (int e = 0; e < kPB; ++e) {
      if (t + e < n) {
        const long long x = base + (long long)(tb + t + e) * D;
        l[e] = p.ld[x];
        q[e] = p.pn[x];
        c[e] = p.c[x];
      } else {
        l[e] = 0.f;
        q[e] = 0.f;
        c[e] = 0.f;
      }
    }
  };

  float lam = 1.f;
  if (valid && p.lam0) lam = p.lam0[chain];

  if (nseg > 1) {
    // ---- segment aggregate
    Mob P = mob_identity();
    {
      float l0[kPB], q0[kPB], c0[kPB], l1[kPB], q1[kPB], c1[kPB];
      load_block(0, l0, q0, c0);
      for (int t = 0; t < n; t += 2 * kPB) {
        load_block(t + kPB, l1, q1, c1);
#pragma unroll
        for (int e = 0; e < kPB; ++e) {
          const float a = __expf(l0[e]);
          P = mob_step(P, a * a, q0[e], c0[e]);
        }
        load_block(t + 2 * kPB, l0, q0, c0);
#pragma unroll
        for (int e = 0; e < kPB; ++e) {
          const float a = __expf(l1[e]);
          P = mob_step(P, a * a, q1[e], c1[e]);
        }
      }
    }
    // ---- publish and look back
    __syncthreads();
    const unsigned epoch = (unsigned)sh[1];
    const unsigned FAGG = 2u * epoch + 2u, FINC = 2u * epoch + 3u;
    if (seg == 0) {
      if (!last) {
        st_coherent(p.inc + cslot, mob_apply(P, lam));
        wait_stores();
        __syncthreads();
        if (tid == 0) st_relaxed(p.flag + slot, FINC);
      }
    } else {
      if (!last) {
        st_coherent(coherent_rsrc(p.agg + slot * 256 * 4, 256 * 16), tid * 16, v4f{P.m00, P.m01, P.m10, P.m11});
        wait_stores();
        __syncthreads();
        if (tid == 0) st_relaxed(p.flag + slot, FAGG);
      }
      // flags of this chain block for segments 0..seg-1 sit ncblocks apart
      if (tid < 64) {
        const int r = lookback_find(p.flag + cb, p.ncblocks, seg, FAGG, FINC, p.ctrl);
        if (tid == 0) sh[2] = r;
      }
      __syncthreads();
      const int r0 = sh[2];
      float x = ld_coherent(p.inc + ((size_t)r0 * p.ncblocks + cb) * 256 + tid);
      for (int u = r0 + 1; u < seg; ++u) {
        const v4f m = ld_coherent(coherent_rsrc(p.agg + ((size_t)u * p.ncblocks + cb) * 256 * 4, 256 * 16), tid * 16);
        x = mob_apply(Mob{m[0], m[1], m[2], m[3]}, x);
      }
      lam = x;
      if (!last) {
        st_coherent(p.inc + cslot, mob_apply(P, lam));
        wait_stores();
        __syncthreads();
        if (tid == 0) st_relaxed(p.flag + slot, FINC);
      }
    }
    // Every flag access of this workgroup is done.
    if (tid == 0) epoch_done_units(p.ctrl, p.bdone, (unsigned)cb, (unsigned)p.ncblocks, (unsigned)nseg, epoch);
  }

  // ---- walk, writing the path
  {
    float l0[kPB], q0[kPB], c0[kPB], l1[kPB], q1[kPB], c1[kPB];
    load_block(0, l0, q0, c0);
    float* out = p.lpath + base + (long long)tb * D;
    for (int t = 0; t < n; t += 2 * kPB) {
      load_block(t + kPB, l1, q1, c1);
#pragma unroll
      for (int e = 0; e < kPB; ++e) {
        const float a = __expf(l0[e]);
        float lp;
        const float nl = lam_step(lam, a * a, q0[e], c0[e], lp);
        if (t + e < n) {
          lam = nl;
          out[(long long)(t + e) * D] = lam;
        }
      }
      load_block(t + 2 * kPB, l0, q0, c0);
#pragma unroll
      for (int e = 0; e < kPB; ++e) {
        const float a = __expf(l1[e]);
        float lp;
        const float nl = lam_step(lam, a * a, q1[e], c1[e], lp);
        if (t + kPB + e < n) {
          lam = nl;
          out[(long long)(t + kPB + e) * D] = lam;
        }
      }
    }
  }
  if (last && valid && p.lamT) p.lamT[chain] = lam;
}

hipError_t launch_pscan(const PscanParams& p, hipStream_t stream) {
  const unsigned nblocks = (unsigned)p.ncblocks * (unsigned)p.nseg;
  hipLaunchKernelGGL(kla_pscan_kernel, dim3(nblocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kla
