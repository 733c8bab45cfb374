// KLA forward scan for bf16 inputs at d_k = d_v = 64: one workgroup streams a
// run of consecutive 64-token tiles of one head.
//
// Sources: gist.science summaries of arXiv 2602.10743, "Kalman Linear Attention";
// [KLA-nl] = "Technische Samenvatting: Kalman Linear Attention (KLA)":
//   §1 "Probabilistische Formulering"      model: OU prior, observation, readout
//   §2 "Parallelisatie via Möbius-transformaties"  precision equation; associative
//                                          composition; affine mean recursion
//   §3 "Niet-lineaire Gating vanuit Onzekerheid"   gates are precision ratios
//   §4 "Architectuur"                       expanded states never go to HBM
//
// Work decomposition.  A head's T tokens are cut into runs of R tiles of 64
// tokens; one workgroup (512 threads) owns one run and walks its tiles in
// order, the next tile's inputs in flight in registers while the current one
// is computed.  Its eight waves have two roles, one tile apart:
//   walkers (waves 0-3): the precision recursion and the gates of tile j.
//     Thread (channel, 16-token chunk) composes the 2x2 step matrices of its
//     chunk; the four chunks of a channel are joined by a scan across lanes;
//     a second walk from the chunk's entering precision forms the gates,
//     folded into matrix-core operands referred to the chunk end:
//       Qt = q cp / cp16,   Kt = g cp16 / cp
//     (cp = in-chunk cumulative product of the forget gate f, cp16 its value
//     over the chunk, g the write gate).  The walk is projective (lam = n / d),
//     so g / cp = k Lambda^v d / (a-product * lam_in) needs no reciprocal of n.
//     Walker wave w then forms the causal scores of chunk w, S = tril(Qt Kt^T),
//     once for all four matrix waves, and keeps the decay from the run start.
//   matrix waves (4-7): wave 4 + c owns value columns 16c..16c+15 of the
//     state M (a 64 x 16 strip, in registers across the whole run).  Per chunk
//       W = diag(cp16) M,   y = Qt W + S V,   M <- W + Kt^T V,
//     on v_mfma_f32_16x16x32_bf16 with split (hi + lo bf16) operands.
// Carries between runs:
//   precision: none.  The precision entering a run is a Möbius image of the
//     one W tokens earlier; the composed map of those W tokens sends every
//     positive precision into an interval that shrinks geometrically with W
//     ([KLA-nl] §2: the maps compose associatively; with process noise they
//     contract).  The run composes the step matrices of the tile before it
//     (then earlier tiles, until the interval is below fp32 resolution or the
//     sequence start is reached, where lambda0 is applied exactly).
//   mean: one decoupled look-back per run (not per tile) over (prod f over
//     the run, local state), in ticket order.  Until the state entering the
//     run is known, the outputs of its first two tiles are held in registers
//     and corrected at the end (y += Qt diag(cp16 * decay from the run start)
//     M_in); a later tile whose decay from the run start is below 2^-100 on
//     every channel gets no correction (the entering state is checked to stay
//     below 2^40, else the error word is set); any other tile first waits for
//     the entering state.
// A chunk whose decay falls below 2^-120 on some channel could overflow Qt;
// it takes an exact per-token path instead (the walkers hand over f and g in
// fp32).
#include <type_traits>

#include "kla_device.h"
#include "kla_internal.h"

namespace kla {

#ifdef KLA_TIMELINE
// Timeline tracing, built only with -DKLA_TIMELINE (build.py --timeline; the
// library then also exports kla_timeline_read and kla_timeline_clear).  The
// first lane of wave 0 (a walker) and of wave 4 (a matrix wave) of every
// workgroup records the 100 MHz real-time counter at fixed points of its
// role, into kla_timeline_buf[workgroup][role][slot].
constexpr int kTlSlots = 64, kTlGroups = 4096;
__device__ unsigned long long kla_timeline_buf[kTlGroups * 2 * kTlSlots];
#define KLA_STAMP(role, k)                                                                              \
  do {                                                                                                  \
    const int kla_slot_ = (k);                                                                          \
    if ((threadIdx.x & 255) == 0 && blockIdx.x < (unsigned)kTlGroups && kla_slot_ < kTlSlots)           \
      kla_timeline_buf[((size_t)blockIdx.x * 2 + (role)) * kTlSlots + kla_slot_] =                      \
          __builtin_amdgcn_s_memrealtime();                                                             \
  } while (0)
// A value (a path counter) in place of a time.
#define KLA_VALUE(role, k, v)                                                                           \
  do {                                                                                                  \
    if ((threadIdx.x & 255) == 0 && blockIdx.x < (unsigned)kTlGroups)                                   \
      kla_timeline_buf[((size_t)blockIdx.x * 2 + (role)) * kTlSlots + (k)] = (unsigned long long)(v);   \
  } while (0)
#else
#define KLA_STAMP(role, k) \
  do {                     \
  } while (0)
#define KLA_VALUE(role, k, v) \
  do {                        \
  } while (0)
#endif

namespace {

constexpr int RD = 64;     // d_k = d_v
constexpr int RTL = 64;    // tokens per tile
constexpr int RNT = 512;   // threads
constexpr int RHOLD = 2;   // leading tiles of a run held for the entering-mean correction
constexpr int kNoSlot = 1 << 20;  // a timeline slot past the end: not recorded
constexpr float kTiny = 0x1p-100f;
constexpr float kMinBig = 0x1p40f;

// Control words in LDS.
enum RunCtl {
  cTicket = 0, cEpoch = 1, cWSync = 2, cXSync = 3,
  cUnsafe = 4,    // [2 tile parities][4 walker waves]: chunks that take the exact path
  cNotFree = 12,  // [2][4]: some channel's decay from the run start to the tile start above 2^-100
  cVote = 20,     // [4]: window walk not converged
  cLamReady = 24,  // the window walk's precision is in lamst
  cCorr = 25       // [4]: walker wave w's share of the held-tile correction (1: tile 1 to correct, 2: nothing)
};

struct alignas(16) RunSmem {
  unsigned char raw[5][RTL * RD * 2];     // q, k, log_decay, proc_noise, val_prec: [token][channel] bf16
  unsigned char vb[RTL * RD * 2];         // v: [token][column] bf16
  unsigned char qop[4][2][4][RD * 32];    // Qt hi / lo per chunk: [channel][16 tokens] bf16 (slots 0, 1: held tiles)
  unsigned char kop[2][2][4][RD * 32];    // Kt hi / lo per chunk: [channel][16 tokens] bf16
  unsigned char sop[2][4][64 * 16];       // per chunk: the causal scores as split B operands, 16 bytes per lane
  float fac[2][4][RD];                    // per chunk: cp16, the decay over the chunk
  float dtile[2][RD];                     // decay from the run start to the tile start
  float hfac[RHOLD][4][RD];               // held chunks: cp16 * decay from the run start to the chunk start
  float dend[RD];                         // decay over the whole run
  float lamst[RD];                        // precision entering the run (from the window walk)
  unsigned ctl[32];
};

// LDS layouts.  Every array is addressed in 8-byte pieces (4 bf16); a piece
// index is permuted by XOR with a few bits of its row so that the accesses
// of a half-wave (32 lanes, 256 bytes, 64 banks) hit distinct banks; the
// permutations are even, so 16-byte units stay whole and in order.
//
// Raw inputs [64 tokens][64 channels]: the walkers' transposing reads take
// rows 4b..4b+3 and 16 + 4b..16 + 4b + 3 (two chunks) in one half-wave, so
// piece p of row r sits at p ^ (4 r1 + 8 r4) (r_i: bit i of the row).
__device__ __forceinline__ int raw_off(int row, int x) {
  const int f = (((row >> 1) & 1) << 2) | (((row >> 4) & 1) << 3);
  return row * 128 + ((((x >> 2) ^ f) & 15) << 3) + ((x & 3) << 1);
}
// V [64 tokens][64 columns]: the matrix waves' transposing reads take rows
// 16r..16r+7 in one half-wave: piece p of row r at p ^ (4 r1 + 8 r2).
__device__ __forceinline__ int v_off(int row, int x) {
  const int f = (((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 3);
  return row * 128 + ((((x >> 2) ^ f) & 15) << 3) + ((x & 3) << 1);
}
// Operand chunk arrays [64 channels][16 tokens] (32-byte rows): piece p of
// channel ch at p ^ 2 ch3.  Transposing reads (eight consecutive channels,
// four pieces) and plain reads of one piece for 16 consecutive channels are
// both conflict-free; a chunk's index and a channel block's enter as
// constant offsets.
__device__ __forceinline__ int op_off(int ch, int t) {
  return ch * 32 + ((((t >> 2) ^ (((ch >> 3) & 1) << 1)) & 3) << 3) + ((t & 3) << 1);
}

typedef unsigned v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bfv(short x) { return __uint_as_float((uint32_t)(uint16_t)x << 16); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) { return __builtin_bit_cast(uint32_t, bf16x2(a, b)); }

// The 16 tokens of channel ch in a chunk's operand arrays `hi` and `lo`, as
// bf16 hi and lo parts (hi = bf16(x), lo = bf16(x - hi)), in 16-byte units.
__device__ __forceinline__ void put_split16(unsigned char* hi, unsigned char* lo, int ch, const float (&x)[16]) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const v2s hh = bf16x2(x[2 * k], x[2 * k + 1]);
    h[k] = __builtin_bit_cast(uint32_t, hh);
    l[k] = pack_bf16(x[2 * k] - to_f32((uint16_t)hh[0]), x[2 * k + 1] - to_f32((uint16_t)hh[1]));
  }
  const int o0 = op_off(ch, 0), o1 = op_off(ch, 8);
  *reinterpret_cast<uint4*>(hi + o0) = make_uint4(h[0], h[1], h[2], h[3]);
  *reinterpret_cast<uint4*>(hi + o1) = make_uint4(h[4], h[5], h[6], h[7]);
  *reinterpret_cast<uint4*>(lo + o0) = make_uint4(l[0], l[1], l[2], l[3]);
  *reinterpret_cast<uint4*>(lo + o1) = make_uint4(l[4], l[5], l[6], l[7]);
}

// A barrier among the four waves of one role (walkers or matrix waves),
// counted in an LDS word: one lane per wave adds one after its earlier LDS
// accesses completed, and every wave waits for 4 * k arrivals.
__device__ __forceinline__ void role_sync(unsigned* cnt, unsigned target) {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS accesses are done
  if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  while (__hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < target) __builtin_amdgcn_s_sleep(1);
}

__device__ __forceinline__ Mob shfl_up_mob(const Mob& m, int d) {
  return Mob{__shfl_up(m.m00, d, 64), __shfl_up(m.m01, d, 64), __shfl_up(m.m10, d, 64), __shfl_up(m.m11, d, 64)};
}
__device__ __forceinline__ Mob shfl_mob(const Mob& m, int src) {
  return Mob{__shfl(m.m00, src, 64), __shfl(m.m01, src, 64), __shfl(m.m10, src, 64), __shfl(m.m11, src, 64)};
}

// Lane geometry.  Walkers: wave w (0-3), lane l: chunk g = l / 16 (tokens
// 16g..16g+15 of the tile), channel ch = 16w + l % 16.  For the matrix-core
// operands of every wave: G = l / 16, li = l % 16, and the transposing reads
// take their 8-byte row from (row 4G + li / 4 of a 16-row block, column
// piece li % 4).
struct WLane {
  int g, i, ch, rr, mm;
};

// The raw values of one array for the walker's 16 tokens, four per
// transposing read: element r of part sb is token 16g + 4sb + r.
__device__ __forceinline__ void read_raw16(const unsigned char* arr, const WLane& L, int w, v4s (&o)[4]) {
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) o[sb] = lds_read_tr16(arr + raw_off(16 * L.g + 4 * sb + L.rr, 16 * w + 4 * L.mm));
}

// Composes the step matrices of the walker's 16 tokens (predict then update:
// [[1 + c pb, c a^2], [pb, a^2]], [KLA-nl] §2) as two independent 8-token
// products walked side by side (twice the independent work per step of the
// dependent chain), keeping (a, a^2, pb, c, k Lambda^v) per token for the
// gate walk when asked.  Returns the chunk's product and sets `first` to that
// of its first eight tokens.
// `arr` holds the tile's k, log_decay, proc_noise and val_prec arrays, 8 KB
// apart, in the raw-input layout.
template <bool KEEP>
__device__ __forceinline__ Mob agg_walk16(const unsigned char* arr, const WLane& L, int w, Mob& first,
                                          float (&ka)[16], float (&ka2)[16], float (&kp)[16], float (&kc)[16],
                                          float (&kv)[16]) {
  v4s rk[4], rl[4], rp[4], rv[4];
  read_raw16(arr, L, w, rk);
  read_raw16(arr + RTL * RD * 2, L, w, rl);
  read_raw16(arr + 2 * RTL * RD * 2, L, w, rp);
  read_raw16(arr + 3 * RTL * RD * 2, L, w, rv);
  // Software-pipelined: the coefficients of tokens u + 1 and u + 9 are formed
  // beside the chain steps of tokens u and u + 8, and each step is its own
  // scheduling region, so the dependent chain steps of both halves sit
  // between independent work.
  float A2[2][2], PB[2][2], C[2][2];  // [buffer][half]
  auto coef = [&](int u, int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = u + 8 * h, sb = t >> 2, e = t & 3;
      const float k = bfv(rk[sb][e]), ld = bfv(rl[sb][e]), pb = bfv(rp[sb][e]), vp = bfv(rv[sb][e]);
      const float a = __expf(ld);
      const float kvv = k * vp, c = k * kvv, a2 = a * a;
      A2[buf][h] = a2;
      PB[buf][h] = pb;
      C[buf][h] = c;
      if constexpr (KEEP) {
        ka[t] = a;
        ka2[t] = a2;
        kp[t] = pb;
        kc[t] = c;
        kv[t] = kvv;
      }
    }
  };
  Mob P[2] = {mob_identity(), mob_identity()};
  coef(0, 0);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (u + 1 < 8) coef(u + 1, (u + 1) & 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) P[h] = mob_step_raw(P[h], A2[u & 1][h], PB[u & 1][h], C[u & 1][h]);
    if ((u & 3) == 3) {
      P[0] = mob_normalize(P[0]);
      P[1] = mob_normalize(P[1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  first = P[0];
  return mob_mul(P[1], P[0]);
}

// Inclusive scan of the chunk products over the tile's four chunks (lanes
// 16 apart hold the same channel); returns the product of chunks 0..g and
// sets `excl` to that of chunks 0..g-1.
__device__ __forceinline__ Mob scan_chunks(Mob P, int g, Mob& excl) {
  Mob Q = shfl_up_mob(P, 16);
  if (g >= 1) P = mob_mul(P, Q);
  Q = shfl_up_mob(P, 32);
  if (g >= 2) P = mob_mul(P, Q);
  excl = shfl_up_mob(P, 16);
  if (g == 0) excl = mob_identity();
  return P;
}

// acc + A B over 64 channels with split operands, A = (Ah, Al) and B = (Bh,
// Bl) per 16-channel block: hi*hi + lo*hi + hi*lo, blocks paired into one
// 16x16x32 instruction each (6 instructions).
__device__ __forceinline__ v4f mma_split64(v4f acc, const v4s (&Ah)[4], const v4s (&Al)[4], const v4s (&Bh)[4],
                                           const v4s (&Bl)[4]) {
#pragma unroll
  for (int kb = 0; kb < 4; kb += 2) {
    const v8s bh = cat(Bh[kb], Bh[kb + 1]);
    acc = mma_x32(acc, cat(Ah[kb], Ah[kb + 1]), bh);
    acc = mma_x32(acc, cat(Al[kb], Al[kb + 1]), bh);
    acc = mma_x32(acc, cat(Ah[kb], Ah[kb + 1]), cat(Bl[kb], Bl[kb + 1]));
  }
  return acc;
}

// What both roles of a workgroup know about its run.
struct RunCtx {
  int tid, lane, wave;
  int head, run, tb, ntl, T, nrun;
  size_t hoff;  // element offset of the head in [B,H,T,64] arrays
  bool last_run;
  unsigned FAGG, FINC;
};

// ---------------------------------------------------------------------------
// Walker waves (0-3): precision scan, gates and causal scores of tile j during
// step j.
// ---------------------------------------------------------------------------
// Held chunk r of Qt slot `slot` (tile `tile`), value columns 16c..16c+15:
// y = y0 + Qt diag(h) M_in (h: the chunk's per-channel factor), stored as
// bf16.  Lane layout of the matrix waves; any wave runs it for any column
// block c (the walkers take the second held tile at the end of a run).
__device__ __forceinline__ void correct_held(RunSmem& s, int lane, int c, int tile, int slot, int r, const float* h,
                                             const v4f& y0, const v4f (&Min)[4], __amdgpu_buffer_rsrc_t yrs) {
  const int G = lane >> 4, li = lane & 15, xe = li >> 2, xj = li & 3;
  v4s Ah[4], Al[4], Bh[4], Bl[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const v4f W = Min[kb] * *reinterpret_cast<const v4f*>(h + 16 * kb + 4 * G);
    split4(W, Ah[kb], Al[kb]);
    const int off = op_off(16 * kb + 4 * G + xe, 4 * xj);
    Bh[kb] = lds_read_tr16(s.qop[slot][0][r] + off);
    Bl[kb] = lds_read_tr16(s.qop[slot][1][r] + off);
  }
  const v4f Y = mma_split64(y0, Ah, Al, Bh, Bl);
  const int tok = tile * RTL + 16 * r + li;
  const v2u wv = v2u{pack_bf16(Y[0], Y[1]), pack_bf16(Y[2], Y[3])};
  __builtin_amdgcn_raw_buffer_store_b64(wv, yrs, tok * (RD * 2) + (16 * c + 4 * G) * 2, 0, 0);
}

__device__ __forceinline__ void walker_role(const FwdRunParams& p, RunSmem& s, const RunCtx& x, uint4 (&pf)[10],
                                            bool have_first) {
  const int tid = x.tid, lane = x.lane, w = x.wave, T = x.T, tb = x.tb, ntl = x.ntl;
  const size_t hoff = x.hoff;
  WLane L;
  L.g = lane >> 4;
  L.i = lane & 15;
  L.ch = 16 * w + L.i;
  L.rr = L.i >> 2;
  L.mm = L.i & 3;
  // 16-byte units of q, k, ld, pn, vp of one tile: unit tid + 256 (it & 1) of
  // array it / 2.
  auto load = [&](int tile, uint4 (&buf)[10], int first) {
    const int t0 = tile * RTL;
#pragma unroll
    for (int it = 0; it < 10; ++it) {
      if (it < first) continue;
      const int a = it >> 1, u = tid + 256 * (it & 1), row = u >> 3, xx = (u & 7) << 3;
      const uint16_t* src = a == 0 ? p.q : a == 1 ? p.k : a == 2 ? p.ld : a == 3 ? p.pn : p.vp;
      buf[it] = t0 + row < T ? *reinterpret_cast<const uint4*>(src + hoff + (size_t)(t0 + row) * RD + xx)
                             : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](const uint4 (&buf)[10], int first) {
#pragma unroll
    for (int it = 0; it < 10; ++it) {
      if (it < first) continue;
      const int a = it >> 1, u = tid + 256 * (it & 1), row = u >> 3, xx = (u & 7) << 3;
      *reinterpret_cast<uint4*>(s.raw[a] + raw_off(row, xx)) = buf[it];
    }
  };
  // pf: the next tile's units, in flight.  The first tile's are in flight
  // already when the workgroup guessed its run right (have_first).
  if (!have_first) load(tb, pf, 0);
  // The precision entering the run: lambda0 for the first run, else the
  // matrix waves' window walk (read in step 0, once they have published it).
  float lam_start = p.lam0 ? p.lam0[(size_t)x.head * RD + L.ch] : 1.f;
  store(pf, 0);
  if (ntl > 1) load(tb + 1, pf, 0);
  __syncthreads();
  KLA_STAMP(0, 2);

  unsigned wsync = 0;
  float dtile = 1.f;  // decay of this channel from the run start to the tile start
  float* const lp = p.lpath;
  const int G = L.g, li = L.i, xe = L.rr, xj = L.mm;
  for (int j = 0; j <= ntl; ++j) {
    if (j < ntl) {
      const int tile = tb + j;
      const int qs = j < RHOLD ? j : RHOLD + (j & 1), ks = j & 1;
      float ka[16], ka2[16], kp[16], kc[16], kv[16];
      Mob excl, first;
      [[maybe_unused]] const int ts = j < 8 ? 3 + 7 * j : kNoSlot;  // timeline slots of this step
      KLA_STAMP(0, ts);
      (void)scan_chunks(agg_walk16<true>(s.raw[1], L, w, first, ka, ka2, kp, kc, kv), L.g, excl);
      KLA_STAMP(0, ts + 1);
      if (j == 0 && x.run > 0) {
        while (__hip_atomic_load(&s.ctl[cLamReady], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0u)
          __builtin_amdgcn_s_sleep(1);
        lam_start = s.lamst[L.ch];
      }
      const float lam_g = mob_apply(excl, lam_start);
      const float lam_g8 = mob_apply(first, lam_g);  // precision after the chunk's first 8 tokens
      v4s rq[4];
      read_raw16(s.raw[0], L, w, rq);
      // Gate walk, projective, as two 8-token halves walked side by side: half
      // h starts from (lam_h, 1) (lam_0 = lam_g, lam_1 = lam_g8) and is
      // rescaled by 2^-ex[h][g] after its token group g (4 tokens), so within
      // group g both n and d' carry 2^-E_g (E_0 = 0, E_1 = ex[h][0]).  With
      // Ab the product of a over the half so far (f = a n_prev / n, g =
      // k Lambda^v d' / n), cp_t = Ab_t lam_h / n_t within the half, and
      // referred to the half's end
      //   Qt_t = q_t (Ab_t / n_t) (n_8 / Ab_8),   Kt_t = k Lambda^v d'_t (Ab_8 / Ab_t) / n_8:
      // Qt from this forward pass and one factor per group, Kt from this pass
      // and a backward (suffix) product of a.  Referred to the chunk end,
      // the first half's Qt takes a further 1 / cp8b and its Kt a further
      // cp8b (cp8b: the second half's decay), and cp16 = cp8a cp8b.
      float n[2] = {lam_g, lam_g8}, d[2] = {1.f, 1.f}, Ab[2] = {1.f, 1.f}, n8[2], rn8[2];
      float qt[16], kt[16];
      int exg[2][2];
      // Software-pipelined like the composition walk: step u advances both
      // chains (token u of each half) and finishes the per-token work of the
      // step before it.
      float pn1[2] = {1.f, 1.f}, pd1[2] = {1.f, 1.f};
#pragma unroll
      for (int u = 0; u <= 8; ++u) {
        float cn1[2], cd1[2];
        if (u < 8) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int t = u + 8 * h;
            const float d1 = fmaf(kp[t], n[h], ka2[t] * d[h]);  // d' = pb n + a^2 d (predict)
            const float n1 = fmaf(kc[t], d1, n[h]);              // n' = n + c d'      (update)
            cn1[h] = n1;
            cd1[h] = d1;
            n[h] = n1;
            d[h] = d1;
          }
        }
        if (u > 0) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int t = u - 1 + 8 * h;
            const float rn = fast_rcp(pn1[h]);
            Ab[h] *= ka[t];
            qt[t] = bfv(rq[t >> 2][t & 3]) * (Ab[h] * rn);
            kt[t] = kv[t] * pd1[h];
            if (u - 1 == 7) {
              n8[h] = pn1[h];
              rn8[h] = rn;
            }
            if (lp) {
              const int tok = tile * RTL + 16 * L.g + t;
              if (tok < T) lp[hoff + (size_t)tok * RD + L.ch] = pn1[h] * fast_rcp(pd1[h]);
            }
          }
        }
        if (u < 8) {
          if ((u & 3) == 3) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int ex = __builtin_amdgcn_frexp_expf(fmaxf(n[h], d[h]));
              n[h] = __builtin_amdgcn_ldexpf(n[h], -ex);
              d[h] = __builtin_amdgcn_ldexpf(d[h], -ex);
              exg[h][u >> 2] = ex;
            }
          }
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            pn1[h] = cn1[h];
            pd1[h] = cd1[h];
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      KLA_STAMP(0, ts + 2);
      // Precision after the tile, for the next tile (from chunk 3's walk).
      const float lam_end = __shfl(n[1] * fast_rcp(d[1]), 48 + L.i, 64);
      const float cp8a = __builtin_amdgcn_ldexpf(Ab[0] * rn8[0] * lam_g, -exg[0][0]);
      const float cp8b = __builtin_amdgcn_ldexpf(Ab[1] * rn8[1] * lam_g8, -exg[1][0]);
      const float cp16 = cp8a * cp8b;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float fq = n8[h] * fast_rcp(Ab[h]);  // group 1 of the half
        float sk = rn8[h];
        if (h == 0) {
          fq *= fast_rcp(cp8b);
          sk *= cp8b;
        }
#pragma unroll
        for (int u = 7; u >= 0; --u) {
          const int t = u + 8 * h;
          qt[t] *= fq;
          kt[t] *= sk;
          sk *= ka[t];
          if (u == 4) {
            fq = __builtin_amdgcn_ldexpf(fq, exg[h][0]);
            sk = __builtin_amdgcn_ldexpf(sk, -exg[h][0]);
          }
        }
      }
      // The matrix path needs every operand and score of the chunk inside the
      // fp32 range: the chunk's decay at least 2^-120 on every channel and Qt
      // finite (Kt is bounded by the write gate).
      float qmag = 0.f;
#pragma unroll
      for (int t = 0; t < 16; t += 2) qmag = fmaxf(qmag, fmaxf(fabsf(qt[t]), fabsf(qt[t + 1])));
      const bool unsafe = !(cp16 >= 0x1p-120f) || !(qmag < 0x1p126f);
      put_split16(s.qop[qs][0][L.g], s.qop[qs][1][L.g], L.ch, qt);
      put_split16(s.kop[ks][0][L.g], s.kop[ks][1][L.g], L.ch, kt);
      s.fac[ks][L.g][L.ch] = cp16;
      // Decay from the run start to each chunk start: an exclusive product
      // over the tile's chunks, on top of the decay to the tile start.
      float ip = cp16;
      {
        float o = __shfl_up(ip, 16, 64);
        if (L.g >= 1) ip *= o;
        o = __shfl_up(ip, 32, 64);
        if (L.g >= 2) ip *= o;
      }
      float ep = __shfl_up(ip, 16, 64);
      if (L.g == 0) ep = 1.f;
      if (j < RHOLD) s.hfac[j][L.g][L.ch] = cp16 * (dtile * ep);
      if (L.g == 0) s.dtile[ks][L.ch] = dtile;
      const unsigned long long bad = __ballot(unsafe);
      const unsigned long long notfree = __ballot(!(dtile <= kTiny));
      if (lane == 0) {
        unsigned m = 0;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) m |= ((bad >> (16 * gg)) & 0xffffull) ? (1u << gg) : 0u;
        s.ctl[cUnsafe + 4 * ks + w] = m;
        s.ctl[cNotFree + 4 * ks + w] = notfree ? 1u : 0u;
      }
      dtile *= __shfl(ip, 48 + L.i, 64);
      KLA_STAMP(0, ts + 3);
      wsync += 4;
      role_sync(&s.ctl[cWSync], wsync);
      KLA_STAMP(0, ts + 4);
      // Causal scores of chunk w for every matrix wave: S^T[u][t] = Kt_u . Qt_t
      // (u, t tokens of the chunk; zero where u > t), as split B operands.
      {
        const int r = w;
        v4s Ah[4], Al[4], Bh[4], Bl[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const int off = op_off(16 * kb + 4 * G + xe, 4 * xj);
          Ah[kb] = lds_read_tr16(s.kop[ks][0][r] + off);
          Al[kb] = lds_read_tr16(s.kop[ks][1][r] + off);
          Bh[kb] = lds_read_tr16(s.qop[qs][0][r] + off);
          Bl[kb] = lds_read_tr16(s.qop[qs][1][r] + off);
        }
        v4f S = mma_split64(v4f{0.f, 0.f, 0.f, 0.f}, Ah, Al, Bh, Bl);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * G + e > li) S[e] = 0.f;
        v4s Sh, Sl;
        split4(S, Sh, Sl);
        *reinterpret_cast<v8s*>(s.sop[ks][r] + 16 * lane) = cat(Sh, Sl);
      }
      KLA_STAMP(0, ts + 5);
      const unsigned um = s.ctl[cUnsafe + 4 * ks] | s.ctl[cUnsafe + 4 * ks + 1] | s.ctl[cUnsafe + 4 * ks + 2] |
                          s.ctl[cUnsafe + 4 * ks + 3];
      if ((um >> L.g) & 1u) {
        // Exact path for this chunk: f and g per token in fp32, in the
        // chunk's operand bytes (tokens 0-7 in the hi block, 8-15 in lo).
        float nn = lam_g, dd = 1.f;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const float a = ka[t];
          const float d1 = fmaf(kp[t], nn, a * a * dd);
          const float n1 = fmaf(kc[t], d1, nn);
          const float rn = fast_rcp(n1);
          const int off = op_off(L.ch, 8 * ((t & 7) >> 2)) + 4 * (t & 3);
          *reinterpret_cast<float*>(s.qop[qs][t >> 3][L.g] + off) = a * nn * rn;
          *reinterpret_cast<float*>(s.kop[ks][t >> 3][L.g] + off) = kv[t] * d1 * rn;
          nn = n1;
          dd = d1;
          if ((t & 3) == 3) {
            const int ex = __builtin_amdgcn_frexp_expf(fmaxf(nn, dd));
            nn = __builtin_amdgcn_ldexpf(nn, -ex);
            dd = __builtin_amdgcn_ldexpf(dd, -ex);
          }
        }
      }
      lam_start = lam_end;
      if (j + 1 < ntl) {
        store(pf, 0);
        if (j + 2 < ntl) load(tile + 2, pf, 0);
      } else {
        if (L.g == 0) s.dend[L.ch] = dtile;
        if (x.last_run && L.g == 0) p.lamT[(size_t)x.head * RD + L.ch] = lam_start;
      }
      KLA_STAMP(0, ts + 6);
    }
    __syncthreads();
  }
  // End of a later run: the second held tile's correction for column block
  // w, once the matrix waves have the entering mean (they correct the first).
  if (x.run > 0) {
    unsigned f;
    while ((f = __hip_atomic_load(&s.ctl[cCorr + w], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) == 0u)
      __builtin_amdgcn_s_sleep(1);
    if (f == 1u) {
      const unsigned char* hb = s.raw[w];
      v4f Min[4], y0[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) Min[rt] = *reinterpret_cast<const v4f*>(hb + (rt * 64 + lane) * 16);
#pragma unroll
      for (int r = 0; r < 4; ++r) y0[r] = *reinterpret_cast<const v4f*>(hb + 4096 + (r * 64 + lane) * 16);
      const __amdgpu_buffer_rsrc_t yrs =
          __builtin_amdgcn_make_buffer_rsrc(p.y + hoff, (short)0, T * RD * 2, 0x00020000);
#pragma unroll
      for (int r = 0; r < 4; ++r) correct_held(s, lane, w, tb + 1, 1, r, s.hfac[1][r], y0[r], Min, yrs);
    }
  }
}

// The 16-byte units of tile wt's k, log_decay, proc_noise and val_prec that
// matrix-wave thread tv (0..255) stages for the window walk: unit tv + 256
// (it & 1) of array it / 2.  A full tile (it precedes a run), so no row check.
__device__ __forceinline__ void window_tile_load(const FwdRunParams& p, size_t hoff, int wt, int tv, uint4 (&buf)[8]) {
  const int t0 = wt * RTL;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int a = it >> 1, u = tv + 256 * (it & 1), row = u >> 3, xx = (u & 7) << 3;
    const uint16_t* src = a == 0 ? p.k : a == 1 ? p.ld : a == 2 ? p.pn : p.vp;
    buf[it] = *reinterpret_cast<const uint4*>(src + hoff + (size_t)(t0 + row) * RD + xx);
  }
}

// ---------------------------------------------------------------------------
// Matrix waves (4-7): wave 4 + c owns value columns 16c..16c+15; tile j-1
// during step j; the mean carry at the end of the run.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void matrix_role(const FwdRunParams& p, RunSmem& s, const RunCtx& x, uint4 (&wbuf)[8],
                                            bool have_window) {
  const int lane = x.lane, c = x.wave - 4, T = x.T, tb = x.tb, ntl = x.ntl, run = x.run, head = x.head;
  const int nrun = x.nrun;
  const size_t hoff = x.hoff;
  const int G = lane >> 4, li = lane & 15;
  const int xe = li >> 2, xj = li & 3;  // transposing-read supply row / column piece
  const int tv = x.tid - 256;
  uint4 vpf[2];
  auto v_load = [&](int tile) {
    const int t0 = tile * RTL;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int u = tv + 256 * it, row = u >> 3, xx = (u & 7) << 3;
      vpf[it] = t0 + row < T ? *reinterpret_cast<const uint4*>(p.v + hoff + (size_t)(t0 + row) * RD + xx)
                             : make_uint4(0, 0, 0, 0);
    }
  };
  auto v_store = [&]() {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int u = tv + 256 * it, row = u >> 3, xx = (u & 7) << 3;
      *reinterpret_cast<uint4*>(s.vb + v_off(row, xx)) = vpf[it];
    }
  };
  v4f Mst[4];
  v4f Yh[4 * RHOLD];  // held chunks' y, chunk-major (tile j, chunk r at 4 j + r)
#pragma unroll
  for (int k = 0; k < 4 * RHOLD; ++k) Yh[k] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      Mst[rt][e] = (run == 0 && p.M0) ? p.M0[(size_t)head * 4096 + (16 * rt + 4 * G + e) * RD + 16 * c + li] : 0.f;
  // The state's loads complete here, before the next tile's values are in
  // flight: no wait inside the chunk loop then stands for them.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  v_load(tb);
  bool mres = run == 0;  // state entering the run known (and folded into Mst)
  bool dropped = false;  // some chunk skipped the entering-mean correction
  const size_t hs = (size_t)head * nrun + run;  // (head, run) slot
  unsigned* const hflag = p.flag + (size_t)head * nrun * 4 + c;  // flag of run r: hflag[4 r]

  // y of 16 tokens (this wave's 16 columns) as bf16, 8 bytes per lane.
  // A buffer store: the hardware drops the tokens at or past T (the head's
  // record ends there), so no branch splits the chunk loop.
  const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(p.y + hoff, (short)0, T * RD * 2, 0x00020000);
  auto store_y = [&](int tile, int r, const v4f& Y) {
    const int tok = tile * RTL + 16 * r + li;
    const v2u wv = v2u{pack_bf16(Y[0], Y[1]), pack_bf16(Y[2], Y[3])};
    __builtin_amdgcn_raw_buffer_store_b64(wv, yrs, tok * (RD * 2) + (16 * c + 4 * G) * 2, 0, 0);
  };
  // Four consecutive per-channel values of an LDS vector, for rows 16 rt + 4 G
  // .. + 3 of the state strip.
  auto lds4 = [&](const float* vec, int rt) { return *reinterpret_cast<const v4f*>(vec + 16 * rt + 4 * G); };
  // Y + Qt W for the 16 tokens of chunk r of an operand slot (W in the state's
  // register layout: rows = channels, columns = this wave's value columns).
  auto readout = [&](v4f Y, const v4f (&W)[4], int qs, int r) {
    v4s Ah[4], Al[4], Bh[4], Bl[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      split4(W[kb], Ah[kb], Al[kb]);
      const int off = op_off(16 * kb + 4 * G + xe, 4 * xj);
      Bh[kb] = lds_read_tr16(s.qop[qs][0][r] + off);
      Bl[kb] = lds_read_tr16(s.qop[qs][1][r] + off);
    }
    return mma_split64(Y, Ah, Al, Bh, Bl);
  };
  // One chunk on the matrix cores: W = diag(cp16) M, y = Qt W + S V,
  // M <- W + Kt^T V.  Returns y (this wave's columns).
  auto chunk = [&](int qs, int ks, int r) {
    v4f W[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) W[rt] = Mst[rt] * lds4(s.fac[ks][r], rt);
    const v4s Vf = lds_read_tr16(s.vb + v_off(16 * r + 4 * G + xe, 16 * c + 4 * xj));
    const v8s Vb = cat(Vf, Vf);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int off = op_off(16 * rt + li, 4 * G);
      const v4s th = *reinterpret_cast<const v4s*>(s.kop[ks][0][r] + off);
      const v4s tl = *reinterpret_cast<const v4s*>(s.kop[ks][1][r] + off);
      Mst[rt] = mma_x32(W[rt], cat(th, tl), Vb);
    }
    const v8s Sv = *reinterpret_cast<const v8s*>(s.sop[ks][r] + 16 * lane);
    return readout(mma_x32(v4f{0.f, 0.f, 0.f, 0.f}, Vb, Sv), W, qs, r);
  };
  // Entering mean for this wave's strip: look back over the head's earlier
  // runs and fold their carries forward, M_end(u) = diag(D_u) M_end(u-1) +
  // Magg_u, with the same instructions whatever run the look-back stops at.
  // With up to three aggregates to fold (PREFETCH), every load is issued
  // before the first fold.
  auto lookback_mean = [&](v4f (&Min)[4], auto prefetch) {
    const int r0 = __builtin_amdgcn_readfirstlane(lookback_find(hflag, 4, run, x.FAGG, x.FINC, p.ctrl));
    const auto rinc = coherent_rsrc(p.minc + ((size_t)head * nrun + r0) * 4096 + c * 1024, 4096);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) Min[rt] = ld_coherent(rinc, (rt * 64 + lane) * 16);
    auto agg_rsrc = [&](int u) { return coherent_rsrc(p.magg + ((size_t)head * nrun + u) * 4096 + c * 1024, 4096); };
    auto dv_rsrc = [&](int u) { return coherent_rsrc(p.dv + (((size_t)head * nrun + u) * 4 + c) * 64, 256); };
    const int nfold = run - r0 - 1;
    if (decltype(prefetch)::value && nfold <= 3) {
      v4f A[3][4], Dd[3][4];
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        if (k < nfold) {
          const auto ragg = agg_rsrc(r0 + 1 + k);
          const auto rdv = dv_rsrc(r0 + 1 + k);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            A[k][rt] = ld_coherent(ragg, (rt * 64 + lane) * 16);
            Dd[k][rt] = ld_coherent(rdv, (16 * rt + 4 * G) * 4);
          }
        }
      }
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        if (k < nfold) {
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) Min[rt][e] = fmaf(Dd[k][rt][e], Min[rt][e], A[k][rt][e]);
        }
      }
    } else {
      for (int u = r0 + 1; u < run; ++u) {
        const auto ragg = agg_rsrc(u);
        const auto rdv = dv_rsrc(u);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const v4f a = ld_coherent(ragg, (rt * 64 + lane) * 16);
          const v4f d = ld_coherent(rdv, (16 * rt + 4 * G) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) Min[rt][e] = fmaf(d[e], Min[rt][e], a[e]);
        }
      }
    }
    if (dropped) {
      // Outputs after the run's held tiles skipped the entering mean where
      // its decay was below 2^-100: fine while the mean stays below 2^40.
      float mx = 0.f;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fabsf(Min[rt][e]));
      if (__ballot(!(mx < kMinBig)) && lane == 0) st_relaxed(p.ctrl + kError, 1u);
    }
  };
  // Held chunk k (tile k / 4, chunk k % 4): y += Qt diag(cp16 * decay from
  // the run start to the chunk start) M_in, stored.
  auto correct = [&](int k, const v4f& y0, const v4f (&Min)[4]) {
    const int j = k >> 2, r = k & 3;
    correct_held(s, lane, c, tb + j, j, r, s.hfac[j][r], y0, Min, yrs);
  };
  // Tells walker wave c (this wave's partner) what it corrects at the end of
  // the run: 1 = the second held tile (its inputs are in raw[c]), 2 = nothing.
  auto tell_walker = [&](unsigned what) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
    if (lane == 0) __hip_atomic_store(&s.ctl[cCorr + c], what, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  // Resolve the entering mean mid-run: fold the predecessors' carries
  // (M_in), correct the first `nheld` held chunks, and add diag(D) M_in to
  // the state (D: the decay from the run start to this point).
  [[maybe_unused]] int tl_resolves = 0, tl_exact = 0, tl_window = 0;  // path counters of the timeline build
  auto resolve_mid = [&](int nheld, const v4f (&D)[4]) {
    ++tl_resolves;
    v4f Min[4];
    lookback_mean(Min, std::false_type{});
#pragma unroll 1
    for (int k = 0; k < nheld; ++k) {
      v4f y0;
      switch (__builtin_amdgcn_readfirstlane(k)) {  // static register indices
        case 0: y0 = Yh[0]; break;
        case 1: y0 = Yh[1]; break;
        case 2: y0 = Yh[2]; break;
        case 3: y0 = Yh[3]; break;
        case 4: y0 = Yh[4]; break;
        case 5: y0 = Yh[5]; break;
        case 6: y0 = Yh[6]; break;
        default: y0 = Yh[7]; break;
      }
      correct(k, y0, Min);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) Mst[rt][e] = fmaf(D[rt][e], Min[rt][e], Mst[rt][e]);
    mres = true;
  };

  // Precision entering the run (not the first): compose the step matrices of
  // the tiles before it, newest first, until the image of (0, inf) under the
  // composed map is below fp32 resolution on every channel, or down to the
  // sequence start, where lambda0 is applied.  The matrix waves do this while
  // the walkers stage and compose tile 0; the window tiles go to the first
  // two Q slots, which the walkers first write after reading the result.
  unsigned char* const stage = &s.qop[0][0][0][0];
  auto put_tile = [&](const uint4 (&buf)[8]) {
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int a = it >> 1, u = tv + 256 * (it & 1), row = u >> 3, xx = (u & 7) << 3;
      *reinterpret_cast<uint4*>(stage + a * RTL * RD * 2 + raw_off(row, xx)) = buf[it];
    }
  };
  auto stage_tile = [&](int wt) {
    uint4 buf[8];
    window_tile_load(p, hoff, wt, tv, buf);
    put_tile(buf);
  };
  unsigned msync = 0;
  if (run > 0) {  // a full tile: it precedes the run
    if (have_window)
      put_tile(wbuf);  // loaded before the ticket, for the run guessed right
    else
      stage_tile(tb - 1);
  }
  __syncthreads();
  if (run > 0) {
    WLane L;
    L.g = G;
    L.i = li;
    L.ch = 16 * c + li;
    L.rr = xe;
    L.mm = xj;
    const float lam0 = p.lam0 ? p.lam0[(size_t)head * RD + L.ch] : 1.f;
    Mob Ptot = mob_identity();
    int wt = tb - 1;
    float lam_in;
    while (true) {
      ++tl_window;
      float ka[16], ka2[16], kp[16], kc[16], kv[16];
      Mob excl, first;
      const Mob Pc = scan_chunks(agg_walk16<false>(stage, L, c, first, ka, ka2, kp, kc, kv), L.g, excl);
      const Mob Pw = shfl_mob(Pc, 48 + L.i);  // product over the whole tile
      Ptot = mob_mul(Ptot, Pw);               // the older tile acts first
      const float lo = Ptot.m01 * fast_rcp(Ptot.m11), hi = Ptot.m00 * fast_rcp(Ptot.m10);
      const bool conv = hi - lo <= 0x1p-21f * lo;
      const unsigned long long bad = __ballot(!conv);
      if (lane == 0) s.ctl[cVote + c] = bad ? 1u : 0u;
      msync += 4;
      role_sync(&s.ctl[cXSync], msync);
      const bool all = (s.ctl[cVote] | s.ctl[cVote + 1] | s.ctl[cVote + 2] | s.ctl[cVote + 3]) == 0u;
      if (all || wt == 0) {
        lam_in = mob_apply(Ptot, wt == 0 ? lam0 : 1.f);
        break;
      }
      --wt;
      msync += 4;
      role_sync(&s.ctl[cXSync], msync);  // every matrix wave has read the votes and the staged tile
      stage_tile(wt);
      msync += 4;
      role_sync(&s.ctl[cXSync], msync);
    }
    if (L.g == 0) s.lamst[L.ch] = lam_in;
    msync += 4;
    role_sync(&s.ctl[cXSync], msync);  // all 64 channels written
    if (x.wave == 4 && lane == 0)
      __hip_atomic_store(&s.ctl[cLamReady], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  }

  KLA_STAMP(1, 2);
  unsigned xsync = msync;
  for (int j = 0; j <= ntl; ++j) {
    if (j >= 1) {
      const int jt = j - 1, tile = tb + jt;
      const int qs = jt < RHOLD ? jt : RHOLD + (jt & 1), ks = jt & 1;
      const unsigned um = s.ctl[cUnsafe + 4 * ks] | s.ctl[cUnsafe + 4 * ks + 1] | s.ctl[cUnsafe + 4 * ks + 2] |
                          s.ctl[cUnsafe + 4 * ks + 3];
      const unsigned nf = s.ctl[cNotFree + 4 * ks] | s.ctl[cNotFree + 4 * ks + 1] | s.ctl[cNotFree + 4 * ks + 2] |
                          s.ctl[cNotFree + 4 * ks + 3];
      // One decision for the whole tile about the entering mean: hold (the
      // run's first tiles), drop (the decay from the run start is below
      // 2^-100 on every channel at the tile start, hence at every chunk
      // start), or wait for it here.  A tile with a chunk on the exact path
      // holds only the chunks before it.
      const bool fast = um == 0u;
      bool hold_tile = false;
      if (!mres) {
        if (jt < RHOLD) {
          hold_tile = fast;
        } else if (fast && nf == 0u) {
          dropped = true;
        } else {
          v4f D[4];
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) D[rt] = lds4(s.dtile[ks], rt);
          resolve_mid(4 * RHOLD, D);
        }
      }
      if (fast) {
        // The four chunks as one branch-free block, outputs placed after it.
        v4f Yc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) Yc[r] = chunk(qs, ks, r);
        if (!hold_tile) {
#pragma unroll
          for (int r = 0; r < 4; ++r) store_y(tile, r, Yc[r]);
        } else if (jt == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) Yh[r] = Yc[r];
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) Yh[4 + r] = Yc[r];
        }
      }
      for (int r = 0; r < 4 && !fast; ++r) {
        const bool unsafe = (um >> r) & 1u;
        bool hold = false;
        if (!mres) {  // a held tile (jt < RHOLD)
          if (!unsafe) {
            hold = true;
          } else {
            v4f D[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
              D[rt] = lds4(s.dtile[ks], rt);
              for (int q = 0; q < r; ++q) D[rt] = D[rt] * lds4(s.fac[ks][q], rt);
            }
            resolve_mid(4 * jt + r, D);
          }
        }
        if (!unsafe) {
          const v4f Y = chunk(qs, ks, r);
          if (hold) {
            const int idx = 4 * jt + r;
#pragma unroll
            for (int k = 0; k < 4 * RHOLD; ++k)
              if (k == idx) Yh[k] = Y;
          } else {
            store_y(tile, r, Y);
          }
        } else {
          // Exact per-token path (the state here is the true state).
          ++tl_exact;
          for (int t = 0; t < 16; ++t) {
            const int tok = tile * RTL + 16 * r + t;
            float qv[16];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
              uint2 qw = make_uint2(0, 0);
              if (tok < T) qw = *reinterpret_cast<const uint2*>(p.q + hoff + (size_t)tok * RD + 16 * rt + 4 * G);
              qv[4 * rt + 0] = __uint_as_float(qw.x << 16);
              qv[4 * rt + 1] = __uint_as_float(qw.x & 0xffff0000u);
              qv[4 * rt + 2] = __uint_as_float(qw.y << 16);
              qv[4 * rt + 3] = __uint_as_float(qw.y & 0xffff0000u);
            }
            const float vv = bfv(*reinterpret_cast<const short*>(s.vb + v_off(16 * r + t, 16 * c + li)));
            float part = 0.f;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int off = op_off(16 * rt + 4 * G + e, 8 * ((t & 7) >> 2)) + 4 * (t & 3);
                const float f = *reinterpret_cast<const float*>(s.qop[qs][t >> 3][r] + off);
                const float gg = *reinterpret_cast<const float*>(s.kop[ks][t >> 3][r] + off);
                Mst[rt][e] = fmaf(f, Mst[rt][e], gg * vv);
                part = fmaf(qv[4 * rt + e], Mst[rt][e], part);
              }
            part += __shfl_xor(part, 16, 64);
            part += __shfl_xor(part, 32, 64);
            if (G == 0 && tok < T) p.y[hoff + (size_t)tok * RD + 16 * c + li] = bf16_rne(part);
          }
        }
      }
    }
    KLA_STAMP(1, j < 10 ? 3 + 2 * j : kNoSlot);
    if (j < ntl) {
      xsync += 4;
      role_sync(&s.ctl[cXSync], xsync);
      v_store();
      if (j + 1 < ntl) v_load(tb + j + 1);
    }
    KLA_STAMP(1, j < 10 ? 4 + 2 * j : kNoSlot);
    __syncthreads();
  }

  // End of the run: the mean carry.
  KLA_STAMP(1, 40);
  v4f D[4];
  bool agg_out = false;  // this run's aggregate is published
  if (!mres) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) D[rt] = lds4(s.dend, rt);
    // Publish the run's aggregate (prod f over the run, local state) unless
    // nothing follows.  When all runs of a head are resident together, this
    // is done even if the predecessor's inclusive carry is already out: the
    // later runs, which end their loops at the same time, then fold it at
    // once instead of waiting for this run's own look-back.  With several
    // rounds of workgroups the predecessors have mostly finished, and the
    // aggregate is skipped when the inclusive carry is there.
    const bool skip = !p.agg_always && ld_relaxed(hflag + 4 * (run - 1)) == x.FINC;
    if (!x.last_run && !skip) {
      agg_out = true;
      const auto ragg = coherent_rsrc(p.magg + hs * 4096 + c * 1024, 4096);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) st_coherent(ragg, (rt * 64 + lane) * 16, Mst[rt]);
      if (li == 0) {
        const auto rdv = coherent_rsrc(p.dv + (hs * 4 + c) * 64, 256);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) st_coherent(rdv, (16 * rt + 4 * G) * 4, D[rt]);
      }
      wait_stores();
      if (lane == 0) st_relaxed(hflag + 4 * run, x.FAGG);
    }
  }
  // The state after the run (inclusive mean): written as M_T by the last run,
  // else published for the runs after it.  When all runs of a head are
  // resident together and this run published its aggregate, the runs after
  // it fold that aggregate down to the first run's inclusive state, and this
  // run's inclusive state would never be read: it is skipped.
  auto publish = [&]() {
    if (x.last_run) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) p.MT[(size_t)head * 4096 + (16 * rt + 4 * G + e) * RD + 16 * c + li] = Mst[rt][e];
    } else if (!(p.agg_always && agg_out)) {
      const auto rinc = coherent_rsrc(p.minc + hs * 4096 + c * 1024, 4096);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) st_coherent(rinc, (rt * 64 + lane) * 16, Mst[rt]);
      wait_stores();
      if (lane == 0) st_relaxed(hflag + 4 * run, x.FINC);
    }
  };
  if (!mres) {
    KLA_STAMP(1, 41);
    v4f Min[4];
    lookback_mean(Min, std::true_type{});
    KLA_STAMP(1, 42);
    // The inclusive mean goes out before the held tiles are corrected (the
    // correction changes outputs only): a successor waiting on it does not
    // wait for the correction too.
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) Mst[rt][e] = fmaf(D[rt][e], Min[rt][e], Mst[rt][e]);
    publish();
    KLA_STAMP(1, 43);
    static_assert(RHOLD == 2, "the walkers take the second of two held tiles");
    if (ntl >= RHOLD) {
      // The second held tile goes to the walker wave of the same column
      // block: the entering mean and the held outputs through LDS (the raw
      // input tiles are no longer read).
      unsigned char* const hb = s.raw[c];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) *reinterpret_cast<v4f*>(hb + (rt * 64 + lane) * 16) = Min[rt];
#pragma unroll
      for (int r = 0; r < 4; ++r) *reinterpret_cast<v4f*>(hb + 4096 + (r * 64 + lane) * 16) = Yh[4 + r];
      tell_walker(1u);
    } else {
      tell_walker(2u);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) correct(k, Yh[k], Min);
  } else {
    publish();
    KLA_STAMP(1, 43);
    if (run > 0) tell_walker(2u);
  }
  KLA_STAMP(1, 44);
  KLA_VALUE(1, 50, tl_window);
  KLA_VALUE(1, 51, tl_resolves);
  KLA_VALUE(1, 52, tl_exact);
}

}  // namespace

// Eight waves share four SIMDs: two waves per SIMD, 256 registers per lane.
__global__ __launch_bounds__(RNT, 2) void kla_fwd_run_kernel(FwdRunParams p) {
  __shared__ RunSmem s;
  const int tid = threadIdx.x;
  KLA_STAMP(tid >> 8, 0);
  // Group x = blockIdx % tgroups serves heads x, x + tgroups, ...: its
  // tickets run over those heads, run-major.  Ticket order is run-major within
  // a group, and all runs of a head fall in one group, so every run a
  // workgroup waits on holds a smaller ticket of its own counter and started
  // earlier.
  const unsigned hpg = (unsigned)p.nheads / (unsigned)p.tgroups;
  auto run_head = [&](unsigned t, int& run, int& head) {
    run = (int)(t / hpg);
    head = (int)((t % hpg) * (unsigned)p.tgroups + blockIdx.x % (unsigned)p.tgroups);
  };
  // Run 0 takes R0 tiles, the others Rb or Rb + 1 (the first Rx of them).
  auto run_start = [&](int run) { return run == 0 ? 0 : p.R0 + (run - 1) * p.Rb + min(run - 1, p.Rx); };
  // The run context, once the ticket is out (after the barrier each role takes).
  auto context = [&]() {
    RunCtx x;
    const unsigned ticket = s.ctl[cTicket];
    const unsigned epoch = s.ctl[cEpoch];
    x.tid = tid;
    x.lane = tid & 63;
    x.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    x.FAGG = 2u * epoch + 2u;
    x.FINC = 2u * epoch + 3u;
    x.nrun = p.nrun;
    run_head(ticket, x.run, x.head);
    x.T = p.T;
    x.tb = run_start(x.run);
    x.ntl = x.run == 0 ? p.R0 : p.Rb + (x.run - 1 < p.Rx ? 1 : 0);
    x.hoff = (size_t)x.head * p.T * RD;
    x.last_run = x.run == p.nrun - 1;
    KLA_STAMP(tid >> 8, 1);
#ifdef KLA_TIMELINE
    if (tid == 0 && blockIdx.x < (unsigned)kTlGroups) {
      kla_timeline_buf[(size_t)blockIdx.x * 2 * kTlSlots + 62] = (unsigned long long)x.run;
      kla_timeline_buf[(size_t)blockIdx.x * 2 * kTlSlots + 63] = (unsigned long long)x.ntl;
    }
#endif
    return x;
  };
  if (tid < 256) {
    // The workgroups of a group mostly draw their tickets in index order, so
    // the walkers start the first tile's loads for the run of ticket
    // blockIdx / tgroups before their own ticket is known; a wrong guess
    // costs only those loads (the tile is loaded again).
    int g_run, g_head;
    run_head(blockIdx.x / (unsigned)p.tgroups, g_run, g_head);
    const size_t ghoff = (size_t)g_head * p.T * RD;
    const int t0 = run_start(g_run) * RTL;
    uint4 pf[10];
#pragma unroll
    for (int it = 0; it < 10; ++it) {
      const int a = it >> 1, u = tid + 256 * (it & 1), row = u >> 3, xx = (u & 7) << 3;
      const uint16_t* src = a == 0 ? p.q : a == 1 ? p.k : a == 2 ? p.ld : a == 3 ? p.pn : p.vp;
      pf[it] = t0 + row < p.T ? *reinterpret_cast<const uint4*>(src + ghoff + (size_t)(t0 + row) * RD + xx)
                              : make_uint4(0, 0, 0, 0);
    }
    // The ticket, drawn once those loads are on their way.
    if (tid == 0) {
      s.ctl[cTicket] =
          draw_ticket(p.tick, (unsigned)p.tgroups, (unsigned)p.nheads / (unsigned)p.tgroups * (unsigned)p.nrun);
      s.ctl[cEpoch] = p.nrun > 1 ? ld_relaxed(p.ctrl + kEpoch) : 0u;
      s.ctl[cWSync] = 0u;
      s.ctl[cXSync] = 0u;
      s.ctl[cLamReady] = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) s.ctl[cCorr + i] = 0u;
    }
    __syncthreads();  // the ticket is out
    const RunCtx x = context();
    walker_role(p, s, x, pf, x.head == g_head && x.run == g_run);
  } else {
    // Likewise the matrix waves load the guessed run's window tile (the tile
    // before the run) for the walk to the run's entering precision.
    int g_run, g_head;
    run_head(blockIdx.x / (unsigned)p.tgroups, g_run, g_head);
    uint4 wbuf[8];
    if (g_run > 0) {
      window_tile_load(p, (size_t)g_head * p.T * RD, run_start(g_run) - 1, tid - 256, wbuf);
    } else {
#pragma unroll
      for (int it = 0; it < 8; ++it) wbuf[it] = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();  // the ticket is out
    const RunCtx x = context();
    matrix_role(p, s, x, wbuf, g_run > 0 && x.head == g_head && x.run == g_run);
  }
  __syncthreads();
  // Count the workgroup done; the last one resets the counter and advances
  // the call epoch (the flags of the next call differ).
  if (tid == 0) {
    const unsigned ng = (unsigned)p.nheads * (unsigned)p.nrun;
    if (__hip_atomic_fetch_add(p.ctrl + kGroupsDone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ng - 1) {
      st_relaxed(p.ctrl + kGroupsDone, 0u);
      if (p.nrun > 1) st_relaxed(p.ctrl + kEpoch, s.ctl[cEpoch] + 1u);
    }
  }
}

// Runs per head: the count that minimises (rounds of workgroups) x (tiles
// per workgroup) on `ncu` compute units, fewest runs on ties; the tiles are
// split as evenly as they go (the first Rx runs after run 0 take one more).
// one_round: every run of every head is resident at once.
// A run's start (workgroup launch, ticket, first tile's loads) and end (the
// look-back, the held tiles' correction) cost about four tile steps; a round of
// runs is priced at its tiles plus that.  (lm180m_bf16, 192 heads x 32 tiles:
// three rounds of 8-tile runs took 152 us, one round of 32-tile runs 139 us.)
constexpr int kRunOverheadTiles = 4;

void fwd_run_plan(int nheads, int T, int ncu, int& R0, int& Rb, int& Rx, int& nrun, bool& one_round) {
  const int ntiles = (T + RTL - 1) / RTL;
  long long best = -1, best_rounds = 1;
  int bestn = 1;
  for (int n = 1; n <= ntiles; ++n) {
    const int r = (ntiles + n - 1) / n;
    const int nr = (ntiles + r - 1) / r;  // runs actually needed at r tiles each
    if (nr != n) continue;
    const long long rounds = ((long long)nheads * n + ncu - 1) / ncu;
    const long long cost = rounds * (r + kRunOverheadTiles);
    if (best < 0 || cost < best) {
      best = cost;
      best_rounds = rounds;
      bestn = n;
    }
  }
  nrun = bestn;
  one_round = best_rounds == 1;
  if (nrun == 1) {
    R0 = ntiles;
    Rb = Rx = 0;
    return;
  }
  R0 = min((ntiles + nrun - 1) / nrun, ntiles - (nrun - 1));
  const int rest = ntiles - R0;
  Rb = rest / (nrun - 1);
  Rx = rest % (nrun - 1);
}

hipError_t launch_forward_run(const FwdRunParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(kla_fwd_run_kernel, dim3((unsigned)p.nheads * (unsigned)p.nrun), dim3(RNT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kla

#ifdef KLA_TIMELINE
extern "C" int kla_timeline_read(void* host, size_t bytes) {
  const size_t n = sizeof(kla::kla_timeline_buf);
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(kla::kla_timeline_buf), bytes < n ? bytes : n, 0,
                                  hipMemcpyDeviceToHost);
}
extern "C" int kla_timeline_clear() {
  static unsigned long long zeros[kla::kTlGroups * 2 * kla::kTlSlots];
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(kla::kla_timeline_buf), zeros, sizeof(zeros), 0, hipMemcpyHostToDevice);
}
#endif
