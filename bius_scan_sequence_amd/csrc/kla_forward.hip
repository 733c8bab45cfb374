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
// Decomposition.  One workgroup (256 threads, four wave64s) owns one segment
// of L tokens of one head (b,h).  The segment's inputs are staged once in LDS.
//   1. Each walker thread (channel i, token group r) composes the 2x2 step
//      matrices of its tokens; the segment aggregate is the product of the
//      group aggregates.
//   2. Decoupled look-back over the head's earlier segments gives the
//      precision entering the segment (one 2x2 matrix or one float per
//      channel crosses workgroups).
//   3. The walk is repeated with the true entering precision to produce the
//      per-token gates f = a lam^-/lam and g = k Lambda^v / lam, folded into the
//      matrix-core operands of 16-token chunks:
//        Qs = q * cp,  Ks = g / cp,  Kd = g * prod_{w>u} f_w,  cp = in-chunk
//        cumulative product of f.
//   4. Chunk loop from a zero state: y_c = tril(Qs Ks^T) V + Qs M_c and
//      M_{c+1} = diag(cp_end) M_c + Kd^T V, on 16x16 matrix-core tiles; the state
//      stays in accumulator registers, never in HBM.
//   5. Decoupled look-back of the mean carry (prod f over the segment, local
//      state), then y += Qs (diag(prod of earlier chunk decays) M_in) and store.
// Every carry is folded forward in segment order with the same instructions,
// so results do not depend on which predecessor a look-back stops at.
//
// A chunk whose in-chunk decay prod f falls below 2^-64 on some channel would
// overflow Ks = g / cp; such a chunk takes an exact scalar path for its
// intra-chunk scores instead.
#include "kla_device.h"
#include "kla_internal.h"

namespace kla {

template <int DK, int DV, bool BF16>
struct FwdCfg {
  using In = typename std::conditional<BF16, uint16_t, float>::type;
  static constexpr int L = (BF16 || (DK <= 64 && DV <= 64)) ? 64 : 32;  // tokens per segment
  static constexpr int NT = 256;
  static constexpr int NCH = L / 16;                                    // 16-token chunks
  static constexpr int NG = (NT / DK < NCH) ? NT / DK : NCH;            // walker token groups
  static constexpr int TG = L / NG;                                     // tokens per group
  static constexpr int CPG = TG / 16;                                   // chunks per group
  static constexpr int NRT = DK / 16;                                   // state row tiles
  static constexpr int NCT = DV / 16;                                   // state col tiles
  static constexpr int CPW = (NCT + 3) / 4;                             // col tiles per wave
  static constexpr int QLD = DK + 4;                                    // padded Qs/Ks row (floats)
  static constexpr int KDT_LD = L + 4;                                  // padded Kd^T row (floats)
  static constexpr int RAW_BYTES = 5 * L * DK * (int)sizeof(In);        // q, k, ld, pn, vp
  static constexpr int OPS_BYTES = (2 * L * QLD + DK * KDT_LD) * 4;     // Qs, Ks, Kd^T (fp32)
  static constexpr int UNION_BYTES = RAW_BYTES > OPS_BYTES ? RAW_BYTES : OPS_BYTES;
  static_assert(TG % 16 == 0, "walker groups must own whole chunks");
};

template <int DK, int DV, bool BF16>
struct FwdSmem {
  using C = FwdCfg<DK, DV, BF16>;
  using In = typename C::In;
  // Staged raw inputs q, k, ld, pn, vp ([L][DK] each) until the gate walk is
  // done; afterwards the fp32 operands Qs [L][QLD], Ks [L][QLD], Kd^T [DK][KDT_LD].
  alignas(16) unsigned char u[C::UNION_BYTES];
  alignas(16) In v[C::L * DV];     // raw v
  float scr_f[16 * DK];            // slow path: f, g of one chunk
  float scr_g[16 * DK];
  float cpe[C::NCH * DK];          // per chunk: prod of f over the chunk
  float lamc[C::NCH * DK];         // per chunk: precision entering the chunk
  float pagg[C::NG * DK * 4];      // walker-group aggregates (2x2 per channel)
  float lam_in[DK];                // precision entering the segment
  float fseg[DK];                  // prod of f over the segment
  float S[16 * 16];                // slow-path intra-chunk scores S[t][u]
  int unsafe[C::NCH];
  int ctl[4];

  __device__ In* raw(int which) { return reinterpret_cast<In*>(u) + which * C::L * DK; }
  __device__ float* Qs() { return reinterpret_cast<float*>(u); }
  __device__ float* Ks() { return reinterpret_cast<float*>(u) + C::L * C::QLD; }
  __device__ float* KdT() { return reinterpret_cast<float*>(u) + 2 * C::L * C::QLD; }
};

// Copy one [rows x width] tile (contiguous in global memory) into LDS, zero
// rows past `nvalid` (zeros are an identity filter step: a = 1, pbar = 0, c = 0,
// and contribute nothing to y).  16-byte units; width*sizeof(In) is a
// multiple of 32 bytes for every supported width.
template <typename In, int ROWS, int WIDTH>
__device__ __forceinline__ void stage_tile(In* dst, const In* src, int nvalid, int tid) {
  constexpr int UNITS = ROWS * WIDTH * (int)sizeof(In) / 16;
  constexpr int PER_UNIT = 16 / (int)sizeof(In);
  const int valid_units = nvalid * WIDTH / PER_UNIT;
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
  uint4* d4 = reinterpret_cast<uint4*>(dst);
  uint4 buf[(UNITS + 255) / 256];
#pragma unroll
  for (int it = 0; it < (UNITS + 255) / 256; ++it) {
    int u = tid + it * 256;
    buf[it] = (u < valid_units) ? s4[u] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int it = 0; it < (UNITS + 255) / 256; ++it) {
    int u = tid + it * 256;
    if (u < UNITS) d4[u] = buf[it];
  }
}

__device__ __forceinline__ v4f ld4(const float* p) { return *reinterpret_cast<const v4f*>(p); }

template <int DK, int DV, bool BF16>
__global__ __launch_bounds__(256) void kla_fwd_kernel(FwdParams p) {
  using C = FwdCfg<DK, DV, BF16>;
  using In = typename C::In;
  using M = Mma<BF16>;
  using Op = typename M::Op;
  constexpr int L = C::L, NCH = C::NCH, NG = C::NG, TG = C::TG, CPG = C::CPG;
  constexpr int NRT = C::NRT, NCT = C::NCT, CPW = C::CPW, QLD = C::QLD, KDT_LD = C::KDT_LD;
  __shared__ FwdSmem<DK, DV, BF16> s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lc = lane & 15;  // lane group (k block) / lane column
  const unsigned nblocks = gridDim.x;

  // ---------------------------------------------------------------- ticket
  if (tid == 0) {
    unsigned e = __hip_atomic_load(p.ctrl + kEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned tk = take_ticket(p.ctrl) % nblocks;
    s.ctl[0] = (int)tk;
    s.ctl[1] = (int)e;
  }
  if (tid < NCH) s.unsafe[tid] = 0;
  __syncthreads();
  const int ticket = s.ctl[0];
  const unsigned epoch = (unsigned)s.ctl[1];
  const unsigned FAGG = 2u * epoch + 2u, FINC = 2u * epoch + 3u;
  const int nheads = p.nheads, T = p.T, nseg = p.nseg;
  const int seg = ticket / nheads, head = ticket % nheads;
  const int t0 = seg * L;
  const int nvalid = min(L, T - t0);
  const bool last = (seg == nseg - 1);
  const size_t hs = (size_t)head * nseg + seg;  // (head, segment) slot

  In* const rq = s.raw(0);
  In* const rk = s.raw(1);
  In* const rld = s.raw(2);
  In* const rpn = s.raw(3);
  In* const rvp = s.raw(4);

  // ---------------------------------------------------------------- stage inputs
  {
    const size_t offk = ((size_t)head * T + t0) * DK, offv = ((size_t)head * T + t0) * DV;
    stage_tile<In, L, DK>(rq, static_cast<const In*>(p.q) + offk, nvalid, tid);
    stage_tile<In, L, DK>(rk, static_cast<const In*>(p.k) + offk, nvalid, tid);
    stage_tile<In, L, DK>(rld, static_cast<const In*>(p.ld) + offk, nvalid, tid);
    stage_tile<In, L, DK>(rpn, static_cast<const In*>(p.pn) + offk, nvalid, tid);
    stage_tile<In, L, DK>(rvp, static_cast<const In*>(p.vp) + offk, nvalid, tid);
    stage_tile<In, L, DV>(s.v, static_cast<const In*>(p.v) + offv, nvalid, tid);
  }
  __syncthreads();

  // ---------------------------------------------------------------- 1. group aggregates
  const int wi = tid % DK, wr = tid / DK;
  const bool walker = wr < NG;
  if (walker) {
    Mob P = mob_identity();
    for (int t = wr * TG; t < (wr + 1) * TG; ++t) {
      const int x = t * DK + wi;
      const float kk = to_f32(rk[x]), a = __expf(to_f32(rld[x]));
      const float c = kk * kk * to_f32(rvp[x]);
      P = mob_step(P, a * a, to_f32(rpn[x]), c);
    }
    float* d = s.pagg + (wr * DK + wi) * 4;
    d[0] = P.m00; d[1] = P.m01; d[2] = P.m10; d[3] = P.m11;
  }
  __syncthreads();

  // ---------------------------------------------------------------- 2. precision carry
  Mob Pseg = mob_identity();
  if (tid < DK) {
    for (int r = 0; r < NG; ++r) {
      const float* d = s.pagg + (r * DK + tid) * 4;
      Pseg = mob_mul(Mob{d[0], d[1], d[2], d[3]}, Pseg);
    }
  }
  float lam_in = 1.f;
  if (seg == 0) {
    if (tid < DK) lam_in = p.lam0 ? p.lam0[(size_t)head * DK + tid] : 1.f;
    if (!last) {
      if (tid < DK) {
        p.pinc[hs * DK + tid] = mob_apply(Pseg, lam_in);
        fence_release();
      }
      __syncthreads();
      if (tid == 0) st_release(p.pflag + hs, FINC);
    }
  } else {
    if (!last) {  // publish the aggregate first so successors need not wait on us
      if (tid < DK) {
        float4* d = reinterpret_cast<float4*>(p.pagg) + hs * DK + tid;
        *d = make_float4(Pseg.m00, Pseg.m01, Pseg.m10, Pseg.m11);
        fence_release();
      }
      __syncthreads();
      if (tid == 0) st_release(p.pflag + hs, FAGG);
    }
    if (tid == 0) s.ctl[2] = lookback_find(p.pflag + (size_t)head * nseg, seg, FAGG, FINC, p.ctrl);
    __syncthreads();
    const int r0 = s.ctl[2];
    if (tid < DK) {
      fence_acquire();
      const size_t hb = (size_t)head * nseg;
      float lam = p.pinc[(hb + r0) * DK + tid];
      for (int u = r0 + 1; u < seg; ++u) {
        const float4 m = reinterpret_cast<const float4*>(p.pagg)[(hb + u) * DK + tid];
        lam = mob_apply(Mob{m.x, m.y, m.z, m.w}, lam);
      }
      lam_in = lam;
      if (!last) {
        p.pinc[hs * DK + tid] = mob_apply(Pseg, lam_in);
        fence_release();
      }
    }
    if (!last) {
      __syncthreads();
      if (tid == 0) st_release(p.pflag + hs, FINC);
    }
  }
  if (tid < DK) s.lam_in[tid] = lam_in;
  __syncthreads();

  // ---------------------------------------------------------------- 3. gate walk
  // Results stay in registers until every walker has finished reading the raw
  // inputs, then overwrite them as fp32 operands.
  float wq[TG], wk[TG], wd[TG];
  if (walker) {
    float lam = s.lam_in[wi];
    for (int r = 0; r < wr; ++r) {
      const float* d = s.pagg + (r * DK + wi) * 4;
      lam = mob_apply(Mob{d[0], d[1], d[2], d[3]}, lam);
    }
#pragma unroll
    for (int cl = 0; cl < CPG; ++cl) {
      const int cc = wr * CPG + cl;
      s.lamc[cc * DK + wi] = lam;
      float cp = 1.f;
      float fr[16], gr[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = cc * 16 + e;
        const int x = t * DK + wi;
        const float kk = to_f32(rk[x]), vpv = to_f32(rvp[x]);
        const float a = __expf(to_f32(rld[x]));
        float lam_pred;
        const float lam_new = lam_step(lam, a * a, to_f32(rpn[x]), kk * kk * vpv, lam_pred);
        const float inv = fast_rcp(lam_new);
        const float f = a * lam_pred * inv;
        const float g = kk * vpv * inv;
        cp *= f;
        wq[cl * 16 + e] = to_f32(rq[x]) * cp;
        wk[cl * 16 + e] = g * fast_rcp(cp);
        fr[e] = f;
        gr[e] = g;
        lam = lam_new;
        if (p.lpath && t < nvalid) p.lpath[((size_t)head * T + t0 + t) * DK + wi] = lam;
      }
      s.cpe[cc * DK + wi] = cp;
      if (!(cp >= 0x1p-64f)) s.unsafe[cc] = 1;
      float sp = 1.f;
#pragma unroll
      for (int e = 15; e >= 0; --e) {
        wd[cl * 16 + e] = gr[e] * sp;
        sp *= fr[e];
      }
    }
    if (last && wr == NG - 1) p.lamT[(size_t)head * DK + wi] = lam;
  }
  __syncthreads();
  float* const Qs = s.Qs();
  float* const Ks = s.Ks();
  float* const KdT = s.KdT();
  if (walker) {
#pragma unroll
    for (int e = 0; e < TG; ++e) {
      const int t = wr * TG + e;
      Qs[t * QLD + wi] = wq[e];
      Ks[t * QLD + wi] = wk[e];
      KdT[wi * KDT_LD + t] = wd[e];
    }
  }
  if (tid < DK) {
    float F = 1.f;
    for (int cc = 0; cc < NCH; ++cc) F *= s.cpe[cc * DK + tid];
    s.fseg[tid] = F;
  }
  __syncthreads();

  // ---------------------------------------------------------------- 4. chunk loop
  v4f yl[NCH][CPW];
  v4f Macc[NRT][CPW];
#pragma unroll
  for (int pp = 0; pp < CPW; ++pp)
#pragma unroll
    for (int mt = 0; mt < NRT; ++mt) Macc[mt][pp] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int cc = 0; cc < NCH; ++cc) {
    const bool unsafe = s.unsafe[cc] != 0;
    if (unsafe) {
      // Exact intra-chunk scores: re-walk the chunk from its entering precision
      // (same instructions as the walk above, raw inputs from global memory),
      // then S[t][u] = sum_i q_ti g_ui prod_{w=u+1..t} f_wi by plain products.
      if (tid < DK) {
        float lam = s.lamc[cc * DK + tid];
        for (int e = 0; e < 16; ++e) {
          const int t = cc * 16 + e;
          float kk = 0.f, ldv = 0.f, pnv = 0.f, vpv = 0.f;
          if (t < nvalid) {
            const size_t gx = ((size_t)head * T + t0 + t) * DK + tid;
            kk = to_f32(static_cast<const In*>(p.k)[gx]);
            ldv = to_f32(static_cast<const In*>(p.ld)[gx]);
            pnv = to_f32(static_cast<const In*>(p.pn)[gx]);
            vpv = to_f32(static_cast<const In*>(p.vp)[gx]);
          }
          const float a = __expf(ldv);
          float lam_pred;
          const float lam_new = lam_step(lam, a * a, pnv, kk * kk * vpv, lam_pred);
          const float inv = fast_rcp(lam_new);
          s.scr_f[e * DK + tid] = a * lam_pred * inv;
          s.scr_g[e * DK + tid] = kk * vpv * inv;
          lam = lam_new;
        }
      }
      __syncthreads();
      {
        const int tt = tid >> 4, uu = tid & 15;
        float acc = 0.f;
        const int t = cc * 16 + tt;
        if (uu <= tt && t < nvalid) {
          const In* qrow = static_cast<const In*>(p.q) + ((size_t)head * T + t0 + t) * DK;
          for (int i = 0; i < DK; ++i) {
            float d = s.scr_g[uu * DK + i];
            for (int w = uu + 1; w <= tt; ++w) d *= s.scr_f[w * DK + i];
            acc = fmaf(to_f32(qrow[i]), d, acc);
          }
        }
        s.S[tt * 16 + uu] = acc;
      }
      __syncthreads();
    }

    // Qs blocks of this chunk: lane -> token cc*16 + lc, channels 16*mt + 4*lg + e.
    Op qo[NRT];
#pragma unroll
    for (int mt = 0; mt < NRT; ++mt) qo[mt] = M::op(ld4(Qs + (cc * 16 + lc) * QLD + 16 * mt + 4 * lg));

    // Intra-chunk scores, transposed: st[e] = S[t = lc][u = 4*lg + e].
    v4f st = v4f{0.f, 0.f, 0.f, 0.f};
    if (!unsafe) {
      Op ko[NRT];
#pragma unroll
      for (int mt = 0; mt < NRT; ++mt) ko[mt] = M::op(ld4(Ks + (cc * 16 + lc) * QLD + 16 * mt + 4 * lg));
      st = M::dot(st, ko, qo);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) st[e] = s.S[lc * 16 + 4 * lg + e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * lg + e > lc) st[e] = 0.f;  // causal: u <= t
    const Op ao = M::op(st);

#pragma unroll
    for (int pp = 0; pp < CPW; ++pp) {
      const int nt = wave + 4 * pp;
      if (nt < NCT) {
        // V block: rows u = cc*16 + 4*lg + e, column 16*nt + lc.
        const typename M::VOp vo = M::vop(s.v + (cc * 16 + 4 * lg) * DV + 16 * nt + lc, DV);
        v4f acc = M::dotv(v4f{0.f, 0.f, 0.f, 0.f}, ao, vo);
        Op mo[NRT];
#pragma unroll
        for (int mt = 0; mt < NRT; ++mt) mo[mt] = M::op(Macc[mt][pp]);
        acc = M::dot(acc, qo, mo);
        yl[cc][pp] = acc;
#pragma unroll
        for (int mt = 0; mt < NRT; ++mt) {
          v4f m = Macc[mt][pp];
          const v4f ce = ld4(s.cpe + cc * DK + 16 * mt + 4 * lg);
          m = m * ce;
          const Op kdo = M::op(ld4(KdT + (16 * mt + lc) * KDT_LD + cc * 16 + 4 * lg));
          Macc[mt][pp] = M::dotv(m, kdo, vo);
        }
      }
    }
  }

  // ---------------------------------------------------------------- 5. mean carry
  // Each lane owns, per tile (mt, nt), rows 16*mt + 4*lg + e of column 16*nt + lc.
  // Workspace payloads are stored in this fragment order, one float4 per lane.
  const size_t MSZ = (size_t)DK * DV;
  auto frag_index = [&](int mt, int nt) -> size_t { return ((size_t)(nt * NRT + mt) * 64 + lane) * 4; };
  v4f Min[NRT][CPW];
  auto publish_inclusive = [&]() {
#pragma unroll
    for (int pp = 0; pp < CPW; ++pp) {
      const int nt = wave + 4 * pp;
      if (nt < NCT) {
#pragma unroll
        for (int mt = 0; mt < NRT; ++mt) {
          const v4f F = ld4(s.fseg + 16 * mt + 4 * lg);
          v4f o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = fmaf(F[e], Min[mt][pp][e], Macc[mt][pp][e]);
          *reinterpret_cast<v4f*>(p.minc + hs * MSZ + frag_index(mt, nt)) = o;
        }
      }
    }
    fence_release();
    __syncthreads();
    if (tid == 0) st_release(p.mflag + hs, FINC);
  };
  if (seg == 0) {
#pragma unroll
    for (int pp = 0; pp < CPW; ++pp) {
      const int nt = wave + 4 * pp;
#pragma unroll
      for (int mt = 0; mt < NRT; ++mt) {
        v4f m = v4f{0.f, 0.f, 0.f, 0.f};
        if (nt < NCT && p.M0) {
          const float* src = p.M0 + (size_t)head * MSZ + (size_t)(16 * mt + 4 * lg) * DV + 16 * nt + lc;
          m = v4f{src[0], src[DV], src[2 * DV], src[3 * DV]};
        }
        Min[mt][pp] = m;
      }
    }
    if (!last) publish_inclusive();
  } else {
    if (!last) {
      if (tid < DK) p.mF[hs * DK + tid] = s.fseg[tid];
#pragma unroll
      for (int pp = 0; pp < CPW; ++pp) {
        const int nt = wave + 4 * pp;
        if (nt < NCT) {
#pragma unroll
          for (int mt = 0; mt < NRT; ++mt)
            *reinterpret_cast<v4f*>(p.magg + hs * MSZ + frag_index(mt, nt)) = Macc[mt][pp];
        }
      }
      fence_release();
      __syncthreads();
      if (tid == 0) st_release(p.mflag + hs, FAGG);
    }
    if (tid == 0) s.ctl[3] = lookback_find(p.mflag + (size_t)head * nseg, seg, FAGG, FINC, p.ctrl);
    __syncthreads();
    const int r0 = s.ctl[3];
    fence_acquire();
    const size_t hb = (size_t)head * nseg;
#pragma unroll
    for (int pp = 0; pp < CPW; ++pp) {
      const int nt = wave + 4 * pp;
#pragma unroll
      for (int mt = 0; mt < NRT; ++mt) {
        v4f m = v4f{0.f, 0.f, 0.f, 0.f};
        if (nt < NCT) {
          m = *reinterpret_cast<const v4f*>(p.minc + (hb + r0) * MSZ + frag_index(mt, nt));
          for (int u = r0 + 1; u < seg; ++u) {
            const v4f a = *reinterpret_cast<const v4f*>(p.magg + (hb + u) * MSZ + frag_index(mt, nt));
            const v4f F = *reinterpret_cast<const v4f*>(p.mF + (hb + u) * DK + 16 * mt + 4 * lg);
#pragma unroll
            for (int e = 0; e < 4; ++e) m[e] = fmaf(F[e], m[e], a[e]);
          }
        }
        Min[mt][pp] = m;
      }
    }
    if (!last) publish_inclusive();
  }
  if (last) {  // final state, row-major
#pragma unroll
    for (int pp = 0; pp < CPW; ++pp) {
      const int nt = wave + 4 * pp;
      if (nt < NCT) {
#pragma unroll
        for (int mt = 0; mt < NRT; ++mt) {
          const v4f F = ld4(s.fseg + 16 * mt + 4 * lg);
          float* dst = p.MT + (size_t)head * MSZ + (size_t)(16 * mt + 4 * lg) * DV + 16 * nt + lc;
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[e * DV] = fmaf(F[e], Min[mt][pp][e], Macc[mt][pp][e]);
        }
      }
    }
  }

  // ---------------------------------------------------------------- 6. correction + store
  {
    v4f decay[NRT];  // prod of chunk decays before chunk cc, per owned row
#pragma unroll
    for (int mt = 0; mt < NRT; ++mt) decay[mt] = v4f{1.f, 1.f, 1.f, 1.f};
    In* yout = static_cast<In*>(p.y) + ((size_t)head * T + t0) * DV;
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      Op qo[NRT];
#pragma unroll
      for (int mt = 0; mt < NRT; ++mt) qo[mt] = M::op(ld4(Qs + (cc * 16 + lc) * QLD + 16 * mt + 4 * lg));
#pragma unroll
      for (int pp = 0; pp < CPW; ++pp) {
        const int nt = wave + 4 * pp;
        if (nt < NCT) {
          Op mo[NRT];
#pragma unroll
          for (int mt = 0; mt < NRT; ++mt) mo[mt] = M::op(decay[mt] * Min[mt][pp]);
          const v4f acc = M::dot(yl[cc][pp], qo, mo);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = cc * 16 + 4 * lg + e;
            if (t < nvalid) yout[(size_t)t * DV + 16 * nt + lc] = from_f32<In>(acc[e]);
          }
        }
      }
#pragma unroll
      for (int mt = 0; mt < NRT; ++mt) decay[mt] = decay[mt] * ld4(s.cpe + cc * DK + 16 * mt + 4 * lg);
    }
  }

  __syncthreads();
  if (tid == 0) finish_call(p.ctrl, epoch, nblocks);
}

// ------------------------------------------------------------------------------
// Host-side launch.
// ------------------------------------------------------------------------------
template <int DK, int DV, bool BF16>
static hipError_t launch_fwd(const FwdParams& p, hipStream_t stream) {
  const unsigned nblocks = (unsigned)p.nheads * (unsigned)p.nseg;
  hipLaunchKernelGGL((kla_fwd_kernel<DK, DV, BF16>), dim3(nblocks), dim3(256), 0, stream, p);
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
