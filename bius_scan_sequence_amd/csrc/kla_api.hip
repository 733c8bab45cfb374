// C ABI of the KLA library: argument validation, workspace layout, launches.
// The public contract (argument meaning, layout, ownership, errors) is in
// include/kla.h.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/kla.h"
#include "kla_internal.h"

namespace kla {
namespace {

thread_local char g_hip_error[256] = "";

int hip_fail(hipError_t e, const char* where) {
  snprintf(g_hip_error, sizeof(g_hip_error), "HIP error in %s: %s", where, hipGetErrorString(e));
  return KLA_ERR_HIP;
}

bool supported_width(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
size_t round256(size_t x) { return (x + 255) / 256 * 256; }

constexpr size_t kHeader = 256;

struct FwdLayout {
  size_t hdone, tick, pflag, mflag, pagg, pinc, mF, magg, minc, total;
};

// The largest divisor of `units` that has a ticket counter.
int ticket_groups(long long units) {
  for (int g = kTicketGroups; g > 1; --g)
    if (units % g == 0) return g;
  return 1;
}

bool fwd_shape_ok(int B, int H, int T, int dk, int dv) {
  if (B < 1 || H < 1 || T < 0) return false;
  if (!supported_width(dk) || !supported_width(dv)) return false;
  const long long wide = dk > dv ? dk : dv;
  return (long long)B * H * (long long)T * wide < (1LL << 31) && (long long)B * H < (1LL << 24);
}

FwdLayout fwd_layout(int B, int H, int T, int dk, int dv, int nseg) {
  const size_t slots = (size_t)B * H * nseg;
  FwdLayout l;
  size_t o = kHeader;
  l.hdone = o; o += (size_t)kDoneCounters * 4;  // fixed place and size in every layout
  l.tick = o; o += (size_t)kTicketWords * 4;     // likewise
  l.pflag = o; o += round256(slots * 2 * 4);  // one flag per carry wave (two when dk = 128)
  l.mflag = o; o += round256(slots * 8 * 4);  // one flag per wave (up to eight)
  l.pagg = o; o += round256(slots * dk * 16);
  l.pinc = o; o += round256(slots * dk * 8);  // {value, flag} records
  l.mF = o; o += round256(slots * 8 * dk * 4);  // one copy per wave (up to eight)
  l.magg = o; o += round256(slots * (size_t)dk * dv * 4);
  l.minc = o; o += round256(slots * (size_t)dk * dv * 4);
  l.total = o;
  return l;
}

int fwd_nseg(int T, int dk, int dv, bool bf16) {
  const int L = fwd_segment_len(dk, dv, bf16);
  return (T + L - 1) / L;
}

// The run-streaming kernel (kla_forward_run.hip) serves bf16 inputs at
// d_k = d_v = 64 with log_decay and proc_noise given per token.
bool fwd_uses_run(int dk, int dv, bool bf16, bool plain) { return bf16 && plain && dk == 64 && dv == 64; }

struct RunLayout {
  size_t tick, flag, dv, magg, minc, total;
};

RunLayout run_layout(long long nheads, int nrun) {
  const size_t slots = (size_t)nheads * nrun;
  RunLayout l;
  size_t o = kHeader;
  o += (size_t)kDoneCounters * 4;  // the fixed done-counter region of every layout (unused here)
  l.tick = o; o += (size_t)kTicketWords * 4;  // the fixed ticket region
  l.flag = o; o += round256(slots * 4 * 4);
  l.dv = o; o += round256(slots * 4 * 64 * 4);
  l.magg = o; o += round256(slots * 4096 * 4);
  l.minc = o; o += round256(slots * 4096 * 4);
  l.total = o;
  return l;
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

struct PscanPlan {
  int ncblocks, nseg, seglen;
  size_t bdone, tick, flag, agg, inc, total;
};

bool pscan_shape_ok(int B, int H, int T, int D) {
  if (B < 1 || H < 1 || D < 1 || T < 0) return false;
  const long long chains = (long long)B * H * D;
  return chains < (1LL << 31) && chains * (long long)T < (1LL << 62);
}

PscanPlan pscan_plan(int B, int H, int T, int D) {
  PscanPlan pl;
  const long long chains = (long long)B * H * D;
  pl.ncblocks = (int)((chains + 255) / 256);
  // One walk per chain when the chains alone fill the GPU (a workgroup per
  // compute unit); otherwise split T so that about 1024 workgroups run, with
  // segments of at least 512 tokens.
  int nseg = 1;
  if (pl.ncblocks < 256 && T >= 1024) {
    nseg = (1024 + pl.ncblocks - 1) / pl.ncblocks;
    const int cap = T / 512;
    if (nseg > cap) nseg = cap;
    if (nseg < 1) nseg = 1;
  }
  int seglen = T > 0 ? (T + nseg - 1) / nseg : 16;
  seglen = (seglen + 15) / 16 * 16;
  pl.seglen = seglen;
  pl.nseg = T > 0 ? (T + seglen - 1) / seglen : 1;
  const size_t slots = (size_t)pl.ncblocks * pl.nseg;
  size_t o = kHeader;
  pl.bdone = o; o += (size_t)kDoneCounters * 4;  // fixed place and size in every layout
  pl.tick = o; o += (size_t)kTicketWords * 4;     // likewise
  pl.flag = o; o += round256(slots * 4);
  if (pl.nseg > 1) {
    pl.agg = o; o += round256(slots * 256 * 16);
    pl.inc = o; o += round256(slots * 256 * 4);
  } else {
    pl.agg = pl.inc = o;
  }
  pl.total = o;
  return pl;
}

constexpr int kBwdSeg = 64;  // tokens per segment of the backward pass

// Widths of 128 run as 64-wide sub-problems (the kernels take d <= 64).
int bwd_sub(int d) { return d > 64 ? 64 : d; }

struct BwdLayout {
  size_t F, Mseg, Gseg, rs, dgw, ew, comp, cin, dqacc, dvacc, total;
};

bool bwd_shape_ok(int B, int H, int T, int dk, int dv) {
  if (B < 1 || H < 1 || T < 0) return false;
  if (!supported_width(dk) || !supported_width(dv)) return false;
  const long long wide = dk > dv ? dk : dv;
  return (long long)B * H * (long long)T * wide < (1LL << 31) && (long long)B * H < (1LL << 24);
}

BwdLayout bwd_layout(int B, int H, int T, int dk, int dv) {
  const size_t nh = (size_t)B * H;
  const size_t nseg = T > 0 ? (size_t)(T + kBwdSeg - 1) / kBwdSeg : 1;
  const size_t sk = bwd_sub(dk), sv = bwd_sub(dv);
  BwdLayout l;
  size_t o = kHeader;
  l.F = o; o += round256(nh * nseg * sk * 4);
  l.Mseg = o; o += round256(nh * nseg * sk * sv * 4);
  l.Gseg = o; o += round256(nh * nseg * sk * sv * 4);
  l.rs = o; o += round256(nh * dk * 4);
  // dgw, ew: one [nh][T][dk] partial per value half; dq and dv partials one
  // per value half and key half when there are two.
  const size_t vh = (size_t)(dv / sv), kh = (size_t)(dk / sk);
  l.dgw = o; o += round256(vh * nh * (size_t)T * dk * 4);
  l.ew = o; o += round256(vh * nh * (size_t)T * dk * 4);
  l.comp = o; o += round256(nseg * nh * sk * 16);
  l.cin = o; o += round256(nseg * nh * sk * 8);
  l.dqacc = o; if (vh > 1) o += round256(vh * nh * (size_t)T * dk * 4);
  l.dvacc = o; if (kh > 1) o += round256(kh * nh * (size_t)T * dv * 4);
  l.total = o;
  return l;
}

}  // namespace
}  // namespace kla

using namespace kla;

extern "C" size_t kla_backward_workspace_bytes(int B, int H, int T, int dk, int dv) {
  if (!bwd_shape_ok(B, H, T, dk, dv)) return 0;
  return bwd_layout(B, H, T, dk, dv).total;
}

extern "C" int kla_backward(const void* q, const void* k, const void* v, const void* log_decay,
                            const void* proc_noise, const void* val_prec, const float* lambda0, const float* M0,
                            const float* lambda_path, const void* grad_y, const float* grad_lambda_T,
                            const float* grad_M_T, void* grad_q, void* grad_k, void* grad_v,
                            void* grad_log_decay, void* grad_proc_noise, void* grad_val_prec,
                            float* grad_lambda0, float* grad_M0, int B, int H, int T, int dk, int dv, int dtype,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 1 || H < 1 || T < 0) return KLA_ERR_INVALID_ARG;
  if (!grad_lambda0 || !grad_M0) return KLA_ERR_INVALID_ARG;
  const void* tok[14] = {q, k, v, log_decay, proc_noise, val_prec, lambda_path, grad_y,
                         grad_q, grad_k, grad_v, grad_log_decay, grad_proc_noise, grad_val_prec};
  if (T > 0)
    for (const void* x : tok)
      if (!x) return KLA_ERR_INVALID_ARG;
  if (dtype != KLA_F32 && dtype != KLA_BF16) return KLA_ERR_UNSUPPORTED;
  if (!supported_width(dk) || !supported_width(dv)) return KLA_ERR_UNSUPPORTED;
  if (!bwd_shape_ok(B, H, T, dk, dv)) return KLA_ERR_INVALID_ARG;
  // Per-token arrays are read and written four elements at a time.
  for (int x = 0; x < 14; ++x)
    if (tok[x] && !aligned(tok[x], 16)) return KLA_ERR_INVALID_ARG;
  if ((lambda0 && !aligned(lambda0, 4)) || (grad_lambda_T && !aligned(grad_lambda_T, 4)) ||
      !aligned(grad_lambda0, 4) || (M0 && !aligned(M0, 16)) || (grad_M_T && !aligned(grad_M_T, 16)) ||
      !aligned(grad_M0, 16))
    return KLA_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, 256)) return KLA_ERR_WORKSPACE;
  if (workspace_bytes < kla_backward_workspace_bytes(B, H, T, dk, dv)) return KLA_ERR_WORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const long long nheads = (long long)B * H;
  if (T == 0) {
    hipError_t e = launch_backward_empty(grad_lambda_T, grad_M_T, grad_lambda0, grad_M0, nheads * dk,
                                         nheads * dk * dv, st);
    return e == hipSuccess ? KLA_OK : hip_fail(e, "kla_backward (T = 0)");
  }
  const bool bf16 = dtype == KLA_BF16;
  const size_t esz = bf16 ? 2 : 4;
  const int sk = bwd_sub(dk), sv = bwd_sub(dv), KH = dk / sk, VH = dv / sv;
  const BwdLayout l = bwd_layout(B, H, T, dk, dv);
  char* ws = static_cast<char*>(workspace);
  auto kbyte = [&](const void* base, int off) {  // key-side array shifted by `off` channels
    return base ? static_cast<const char*>(base) + (size_t)off * esz : nullptr;
  };
  BwdParams p{};
  p.nheads = (int)nheads; p.T = T; p.nseg = (T + kBwdSeg - 1) / kBwdSeg;
  p.ncu = device_cus();
  p.nchains = nheads * sk;
  p.F = reinterpret_cast<float*>(ws + l.F);
  p.Mseg = reinterpret_cast<float*>(ws + l.Mseg);
  p.Gseg = reinterpret_cast<float*>(ws + l.Gseg);
  p.comp = reinterpret_cast<float*>(ws + l.comp);
  p.cin = reinterpret_cast<float*>(ws + l.cin);
  p.ks = dk; p.vs = dv; p.kws = dk; p.ksh = dk; p.mrow = dv; p.mhead = dk * dv; p.vacc = dv;
  float* const rs = reinterpret_cast<float*>(ws + l.rs);
  float* const dgw = reinterpret_cast<float*>(ws + l.dgw);
  float* const ew = reinterpret_cast<float*>(ws + l.ew);
  float* const dqacc = VH > 1 ? reinterpret_cast<float*>(ws + l.dqacc) : nullptr;
  float* const dvacc = KH > 1 ? reinterpret_cast<float*>(ws + l.dvacc) : nullptr;
  hipError_t e = hipSuccess;
  for (int kh = 0; kh < KH && e == hipSuccess; ++kh) {
    const int ko = kh * sk;
    p.q = kbyte(q, ko); p.k = kbyte(k, ko); p.ld = kbyte(log_decay, ko); p.pn = kbyte(proc_noise, ko);
    p.vp = kbyte(val_prec, ko);
    p.lpath = lambda_path + ko;
    p.lam0 = lambda0 ? lambda0 + ko : nullptr;
    p.dlamT = grad_lambda_T ? grad_lambda_T + ko : nullptr;
    p.dlam0 = grad_lambda0 + ko;
    p.rs = rs + ko;
    p.dq = const_cast<char*>(kbyte(grad_q, ko)); p.dk = const_cast<char*>(kbyte(grad_k, ko));
    p.dld = const_cast<char*>(kbyte(grad_log_decay, ko)); p.dpn = const_cast<char*>(kbyte(grad_proc_noise, ko));
    p.dvp = const_cast<char*>(kbyte(grad_val_prec, ko));
    // Each value half writes its own partials of dg, e and dq (and each key
    // half its own of dv); the chain and the conversion add them.
    const size_t half_k = (size_t)nheads * T * dk, half_v = (size_t)nheads * T * dv;
    for (int vh = 0; vh < VH && e == hipSuccess; ++vh) {
      const int vo = vh * sv;
      p.dgw = dgw + vh * half_k + ko; p.ew = ew + vh * half_k + ko;
      p.dq_acc = dqacc ? dqacc + vh * half_k + ko : nullptr;
      p.v = kbyte(v, vo); p.dy = kbyte(grad_y, vo);
      p.dv = const_cast<char*>(kbyte(grad_v, vo));
      p.dv_acc = dvacc ? dvacc + kh * half_v + vo : nullptr;
      const size_t mo = (size_t)ko * dv + vo;
      p.M0 = M0 ? M0 + mo : nullptr;
      p.dMT = grad_M_T ? grad_M_T + mo : nullptr;
      p.dM0 = grad_M0 + mo;
      p.add_rs = vh > 0;
      e = launch_backward_front(p, sk, sv, bf16, st);
    }
    p.dgw = dgw + ko; p.ew = ew + ko;
    p.ehalf = VH > 1 ? half_k : 0;
    if (e == hipSuccess) e = launch_backward_chain(p, sk, bf16, st);
  }
  if (e == hipSuccess && dqacc) e = launch_backward_convert(dqacc, grad_q, nheads * (long long)T * dk, bf16, st);
  if (e == hipSuccess && dvacc) e = launch_backward_convert(dvacc, grad_v, nheads * (long long)T * dv, bf16, st);
  return e == hipSuccess ? KLA_OK : hip_fail(e, "kla_backward");
}

extern "C" size_t kla_forward_workspace_bytes(int B, int H, int T, int dk, int dv) {
  if (!fwd_shape_ok(B, H, T, dk, dv)) return 0;
  // The layout does not depend on the dtype except through the segment
  // length; size for the shorter segment (more segments) to cover both, and
  // for the run-streaming kernel at its most runs (one tile each).
  const int nseg = T > 0 ? fwd_nseg(T, dk, dv, false) : 1;
  const int nseg_b = T > 0 ? fwd_nseg(T, dk, dv, true) : 1;
  size_t need = fwd_layout(B, H, T, dk, dv, nseg > nseg_b ? nseg : nseg_b).total;
  if (fwd_uses_run(dk, dv, true, true) && T > 0) {
    const size_t r = run_layout((long long)B * H, (T + 63) / 64).total;
    if (r > need) need = r;
  }
  return need;
}

namespace kla {
namespace {
// The scratch array of kla_forward_noalloc.  In host code `scratch` names a
// host-side stand-in, not the device array: only the address looked up with
// hipGetSymbolAddress (per device, with that device current) is ever passed
// to a kernel or a fill.
constexpr size_t kScratchBytes = KLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "kla_forward_noalloc (hipGetDevice)");
  if (dev < 0 || dev >= kMaxDevices) return KLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "kla_forward_noalloc (hipGetSymbolAddress)");
    if (!ptr || !aligned(ptr, 256)) return hip_fail(hipErrorInvalidSymbol, "kla_forward_noalloc (scratch address)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KLA_OK;
}
}  // namespace
}  // namespace kla

namespace kla {
namespace {
// kla_forward and kla_forward_ou: with theta == NULL, log_decay and
// proc_noise are per-token inputs; otherwise `log_decay` holds the OU step
// length and theta, sigma2 ([H][dk]) the rate and diffusion.
int forward_impl(const char* name, const void* q, const void* k, const void* v, const void* log_decay,
                 const void* proc_noise, const float* theta, const float* sigma2, const void* val_prec,
                 const float* lambda0, const float* M0, void* y, float* lambda_T, float* M_T, float* lambda_path,
                 int B, int H, int T, int dk, int dv, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream, const float* const* conv_w = nullptr, const float* const* conv_b = nullptr,
                 int conv_width = 0, bool lib_scratch = false) {
  if (B < 1 || H < 1 || T < 0) return KLA_ERR_INVALID_ARG;
  if (!lambda_T || !M_T) return KLA_ERR_INVALID_ARG;
  const bool ou = theta != nullptr;
  if (conv_w) {  // coefficient prologue: three weight arrays, taps 1..4, 16-byte aligned
    if (conv_width < 1 || conv_width > 4) return KLA_ERR_INVALID_ARG;
    for (int i = 0; i < 3; ++i) {
      if (!conv_w[i] || !aligned(conv_w[i], 16)) return KLA_ERR_INVALID_ARG;
      if (conv_b[i] && !aligned(conv_b[i], 4)) return KLA_ERR_INVALID_ARG;
    }
  }
  // With T = 0 the per-token arrays are empty and never touched (may be null).
  if (T > 0 && (!q || !k || !v || !log_decay || (!ou && !proc_noise) || !val_prec || !y))
    return KLA_ERR_INVALID_ARG;
  if (ou && (!sigma2 || !aligned(theta, 4) || !aligned(sigma2, 4))) return KLA_ERR_INVALID_ARG;
  if (dtype != KLA_F32 && dtype != KLA_BF16) return KLA_ERR_UNSUPPORTED;
  if (!supported_width(dk) || !supported_width(dv)) return KLA_ERR_UNSUPPORTED;
  if (!fwd_shape_ok(B, H, T, dk, dv)) return KLA_ERR_INVALID_ARG;
  const size_t esz = dtype == KLA_BF16 ? 2 : 4;
  const void* ins[6] = {q, k, v, log_decay, ou ? q : proc_noise, val_prec};
  for (const void* p : ins)
    if (!aligned(p, 16)) return KLA_ERR_INVALID_ARG;
  // y is written in 16-byte units.
  if (!aligned(y, 16) || !aligned(lambda_T, 4) || !aligned(M_T, 4)) return KLA_ERR_INVALID_ARG;
  if ((lambda0 && !aligned(lambda0, 4)) || (M0 && !aligned(M0, 4)) ||
      (lambda_path && !aligned(lambda_path, 4)))
    return KLA_ERR_INVALID_ARG;
  // A caller's workspace covers every layout of the shape; the library's
  // scratch array (kla_forward_noalloc) is checked against the layout this
  // call takes, below.
  if (!lib_scratch) {
    if (!workspace || !aligned(workspace, 256)) return KLA_ERR_WORKSPACE;
    if (workspace_bytes < kla_forward_workspace_bytes(B, H, T, dk, dv)) return KLA_ERR_WORKSPACE;
  }

  hipStream_t st = static_cast<hipStream_t>(stream);
  const long long nheads = (long long)B * H;
  if (T == 0) {
    hipError_t e = launch_state_copy(lambda0, M0, lambda_T, M_T, nheads * dk, nheads * dk * dv, st);
    return e == hipSuccess ? KLA_OK : hip_fail(e, name);
  }
  const bool bf16 = dtype == KLA_BF16;
  char* ws = static_cast<char*>(workspace);
  // The workspace of the layout this call takes: the caller's (checked above
  // against every layout), or the library's scratch array, checked here before
  // its address is looked up, its first `clear` bytes (control words,
  // counters, flags) then zero-filled on the stream.
  auto take = [&](size_t need, size_t clear) -> int {
    if (!lib_scratch) return workspace_bytes < need ? KLA_ERR_WORKSPACE : KLA_OK;
    if (need > kScratchBytes) return KLA_ERR_TOO_LARGE;
    void* base = nullptr;
    const int rc = scratch_address(&base);
    if (rc != KLA_OK) return rc;
    ws = static_cast<char*>(base);
    hipError_t e = launch_fill_zero(ws, clear / 4, st);
    return e == hipSuccess ? KLA_OK : hip_fail(e, name);
  };
  if (fwd_uses_run(dk, dv, bf16, !ou && !conv_w)) {
    FwdRunParams r;
    r.q = static_cast<const uint16_t*>(q); r.k = static_cast<const uint16_t*>(k);
    r.v = static_cast<const uint16_t*>(v); r.ld = static_cast<const uint16_t*>(log_decay);
    r.pn = static_cast<const uint16_t*>(proc_noise); r.vp = static_cast<const uint16_t*>(val_prec);
    r.lam0 = lambda0; r.M0 = M0; r.y = static_cast<uint16_t*>(y); r.lamT = lambda_T; r.MT = M_T;
    r.lpath = lambda_path;
    r.nheads = (int)nheads; r.T = T; r.ntiles = (T + 63) / 64;
    bool one_round = false;
    fwd_run_plan(r.nheads, T, device_cus(), r.R0, r.Rb, r.Rx, r.nrun, one_round);
    r.agg_always = one_round ? 1 : 0;
    r.tgroups = ticket_groups(r.nheads);
    const RunLayout rl = run_layout(nheads, r.nrun);
    const int rc = take(rl.total, rl.dv);
    if (rc != KLA_OK) return rc;
    r.ctrl = reinterpret_cast<unsigned*>(ws);
    r.tick = reinterpret_cast<unsigned*>(ws + rl.tick);
    r.flag = reinterpret_cast<unsigned*>(ws + rl.flag);
    r.dv = reinterpret_cast<float*>(ws + rl.dv);
    r.magg = reinterpret_cast<float*>(ws + rl.magg);
    r.minc = reinterpret_cast<float*>(ws + rl.minc);
    hipError_t e = launch_forward_run(r, st);
    return e == hipSuccess ? KLA_OK : hip_fail(e, name);
  }
  const int nseg = fwd_nseg(T, dk, dv, bf16);
  const FwdLayout l = fwd_layout(B, H, T, dk, dv, nseg);
  const int rc = take(l.total, l.mF);  // the flagged precision records (pinc) lie before mF
  if (rc != KLA_OK) return rc;
  FwdParams p;
  p.q = q; p.k = k; p.v = v; p.ld = log_decay; p.pn = ou ? nullptr : proc_noise; p.vp = val_prec;
  p.lam0 = lambda0; p.M0 = M0; p.y = y; p.lamT = lambda_T; p.MT = M_T; p.lpath = lambda_path;
  p.theta = theta; p.sigma2 = ou ? sigma2 : nullptr;
  for (int i = 0; i < 3; ++i) {
    p.cw[i] = conv_w ? conv_w[i] : nullptr;
    p.cb[i] = conv_w ? conv_b[i] : nullptr;
  }
  p.cwidth = conv_w ? conv_width : 0;
  p.nheads = (int)nheads; p.T = T; p.nseg = nseg; p.H = H;
  p.tgroups = ticket_groups(nheads);
  // With 128 or more heads a head's consecutive segments are dispatched at
  // least 128 workgroups apart (segment-major order), and a segment seldom
  // has a successor waiting on its aggregate.
  p.mskip = nheads >= 128;
  p.ctrl = reinterpret_cast<unsigned*>(ws);
  p.tick = reinterpret_cast<unsigned*>(ws + l.tick);
  p.hdone = reinterpret_cast<unsigned*>(ws + l.hdone);
  p.pflag = reinterpret_cast<unsigned*>(ws + l.pflag);
  p.mflag = reinterpret_cast<unsigned*>(ws + l.mflag);
  p.pagg = reinterpret_cast<float*>(ws + l.pagg);
  p.pinc = reinterpret_cast<unsigned long long*>(ws + l.pinc);
  p.mF = reinterpret_cast<float*>(ws + l.mF);
  p.magg = reinterpret_cast<float*>(ws + l.magg);
  p.minc = reinterpret_cast<float*>(ws + l.minc);
  hipError_t e = launch_forward(p, dk, dv, bf16, st);
  return e == hipSuccess ? KLA_OK : hip_fail(e, name);
}
}  // namespace
}  // namespace kla

extern "C" int kla_forward(const void* q, const void* k, const void* v, const void* log_decay,
                           const void* proc_noise, const void* val_prec, const float* lambda0,
                           const float* M0, void* y, float* lambda_T, float* M_T, float* lambda_path,
                           int B, int H, int T, int dk, int dv, int dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return forward_impl("kla_forward", q, k, v, log_decay, proc_noise, nullptr, nullptr, val_prec, lambda0, M0, y,
                      lambda_T, M_T, lambda_path, B, H, T, dk, dv, dtype, workspace, workspace_bytes, stream);
}


extern "C" int kla_forward_noalloc(const void* q, const void* k, const void* v, const void* log_decay,
                                   const void* proc_noise, const void* val_prec, const float* lambda0,
                                   const float* M0, void* y, float* lambda_T, float* M_T, float* lambda_path,
                                   int B, int H, int T, int dk, int dv, int dtype, int* error_flag, void* stream) {
  if (error_flag && !aligned(error_flag, 4)) return KLA_ERR_INVALID_ARG;
  int rc = forward_impl("kla_forward_noalloc", q, k, v, log_decay, proc_noise, nullptr, nullptr, val_prec, lambda0, M0,
                        y, lambda_T, M_T, lambda_path, B, H, T, dk, dv, dtype, nullptr, 0, stream, nullptr, nullptr, 0,
                        true);
  if (rc != KLA_OK || !error_flag) return rc;
  // T = 0 launches no scan and leaves the scratch alone: its error word is 0.
  void* ws = nullptr;
  if (T > 0 && (rc = scratch_address(&ws)) != KLA_OK) return rc;
  const unsigned* word = T > 0 ? static_cast<const unsigned*>(ws) + kError : nullptr;
  hipError_t e = launch_word_copy(word, error_flag, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KLA_OK : hip_fail(e, "kla_forward_noalloc (error word)");
}

extern "C" int kla_forward_ou(const void* q, const void* k, const void* v, const void* dt, const float* theta,
                              const float* sigma2, const void* val_prec, const float* lambda0, const float* M0,
                              void* y, float* lambda_T, float* M_T, float* lambda_path, int B, int H, int T,
                              int dk, int dv, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!theta) return KLA_ERR_INVALID_ARG;
  return forward_impl("kla_forward_ou", q, k, v, dt, nullptr, theta, sigma2, val_prec, lambda0, M0, y, lambda_T,
                      M_T, lambda_path, B, H, T, dk, dv, dtype, workspace, workspace_bytes, stream);
}

extern "C" int kla_forward_prologue(const void* xq, const void* xk, const void* xv, const void* dt_raw,
                                    const float* theta, const float* sigma2, const void* vp_raw,
                                    const float* conv_wq, const float* conv_wk, const float* conv_wv,
                                    const float* conv_bq, const float* conv_bk, const float* conv_bv, int conv_width,
                                    const float* lambda0, const float* M0, void* y, float* lambda_T, float* M_T,
                                    float* lambda_path, int B, int H, int T, int dk, int dv, int dtype,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (!theta) return KLA_ERR_INVALID_ARG;
  const float* cw[3] = {conv_wq, conv_wk, conv_wv};
  const float* cb[3] = {conv_bq, conv_bk, conv_bv};
  for (const float* w : cw)
    if (!w) return KLA_ERR_INVALID_ARG;
  return forward_impl("kla_forward_prologue", xq, xk, xv, dt_raw, nullptr, theta, sigma2, vp_raw, lambda0, M0, y,
                      lambda_T, M_T, lambda_path, B, H, T, dk, dv, dtype, workspace, workspace_bytes, stream, cw, cb,
                      conv_width);
}

extern "C" int kla_forward_vprec(const void* q, const void* k, const void* v, const void* log_decay,
                                 const void* proc_noise, const void* val_prec, const float* lambda0, const float* M0,
                                 void* y, float* lambda_T, float* M_T, int B, int H, int T, int dk, int dv, int dtype,
                                 void* stream) {
  if (B < 1 || H < 1 || T < 0) return KLA_ERR_INVALID_ARG;
  if (!lambda_T || !M_T) return KLA_ERR_INVALID_ARG;
  if (T > 0 && (!q || !k || !v || !log_decay || !proc_noise || !val_prec || !y)) return KLA_ERR_INVALID_ARG;
  if (dtype != KLA_F32 && dtype != KLA_BF16) return KLA_ERR_UNSUPPORTED;
  if (!supported_width(dk) || !supported_width(dv)) return KLA_ERR_UNSUPPORTED;
  if (!fwd_shape_ok(B, H, T, dk, dv)) return KLA_ERR_INVALID_ARG;
  const size_t esz = dtype == KLA_BF16 ? 2 : 4;
  const void* ins[7] = {q, k, v, log_decay, proc_noise, val_prec, y};
  for (const void* x : ins)
    if (x && !aligned(x, esz)) return KLA_ERR_INVALID_ARG;
  const void* st4[4] = {lambda0, M0, lambda_T, M_T};
  for (const void* x : st4)
    if (x && !aligned(x, 4)) return KLA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const long long nheads = (long long)B * H;
  if (T == 0) {
    hipError_t e = launch_state_copy(lambda0, M0, lambda_T, M_T, nheads * dk * dv, nheads * dk * dv, st);
    return e == hipSuccess ? KLA_OK : hip_fail(e, "kla_forward_vprec (T = 0 state copy)");
  }
  VprecParams p;
  p.q = q; p.k = k; p.v = v; p.ld = log_decay; p.pn = proc_noise; p.vp = val_prec;
  p.lam0 = lambda0; p.M0 = M0; p.y = y; p.lamT = lambda_T; p.MT = M_T; p.T = T;
  hipError_t e = launch_vprec(p, nheads, dk, dv, dtype == KLA_BF16, st);
  return e == hipSuccess ? KLA_OK : hip_fail(e, "kla_forward_vprec");
}

extern "C" size_t kla_precision_scan_workspace_bytes(int B, int H, int T, int D) {
  if (!pscan_shape_ok(B, H, T, D)) return 0;
  return pscan_plan(B, H, T, D).total;
}

extern "C" int kla_precision_scan(const float* log_decay, const float* proc_noise, const float* obs_prec,
                                  const float* lambda0, float* lambda_path, float* lambda_T, int B, int H,
                                  int T, int D, void* workspace, size_t workspace_bytes, void* stream) {
  if (!pscan_shape_ok(B, H, T, D)) return KLA_ERR_INVALID_ARG;
  if (T > 0 && (!log_decay || !proc_noise || !obs_prec || !lambda_path)) return KLA_ERR_INVALID_ARG;
  const void* ptrs[6] = {log_decay, proc_noise, obs_prec, lambda_path, lambda0, lambda_T};
  for (const void* p : ptrs)
    if (p && !aligned(p, 4)) return KLA_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, 256)) return KLA_ERR_WORKSPACE;
  const PscanPlan pl = pscan_plan(B, H, T, D);
  if (workspace_bytes < pl.total) return KLA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const long long chains = (long long)B * H * D;
  if (T == 0) {
    if (!lambda_T) return KLA_OK;
    hipError_t e = launch_state_copy(lambda0, nullptr, lambda_T, nullptr, chains, 0, st);
    return e == hipSuccess ? KLA_OK : hip_fail(e, "kla_precision_scan (T = 0 state copy)");
  }
  char* ws = static_cast<char*>(workspace);
  PscanParams p;
  p.ld = log_decay; p.pn = proc_noise; p.c = obs_prec; p.lam0 = lambda0;
  p.lpath = lambda_path; p.lamT = lambda_T;
  p.nchains = chains; p.D = D; p.T = T;
  p.nseg = pl.nseg; p.seglen = pl.seglen; p.ncblocks = pl.ncblocks;
  p.tgroups = ticket_groups(pl.ncblocks);
  p.ctrl = reinterpret_cast<unsigned*>(ws);
  p.tick = reinterpret_cast<unsigned*>(ws + pl.tick);
  p.bdone = reinterpret_cast<unsigned*>(ws + pl.bdone);
  p.flag = reinterpret_cast<unsigned*>(ws + pl.flag);
  p.agg = reinterpret_cast<float*>(ws + pl.agg);
  p.inc = reinterpret_cast<float*>(ws + pl.inc);
  hipError_t e = launch_pscan(p, st);
  return e == hipSuccess ? KLA_OK : hip_fail(e, "kla_precision_scan");
}

extern "C" int kla_decode_step(const void* q, const void* k, const void* v, const void* log_decay,
                               const void* proc_noise, const void* val_prec, const float* lambda_in,
                               const float* M_in, float* lambda_out, float* M_out, void* y, int B, int H,
                               int dk, int dv, int dtype, void* stream) {
  if (B < 1 || H < 1) return KLA_ERR_INVALID_ARG;
  if (!q || !k || !v || !log_decay || !proc_noise || !val_prec || !lambda_out || !M_out || !y)
    return KLA_ERR_INVALID_ARG;
  if (dtype != KLA_F32 && dtype != KLA_BF16) return KLA_ERR_UNSUPPORTED;
  if (!supported_width(dk) || !supported_width(dv)) return KLA_ERR_UNSUPPORTED;
  const long long nheads = (long long)B * H;
  if (nheads >= (1LL << 31)) return KLA_ERR_INVALID_ARG;
  const size_t esz = dtype == KLA_BF16 ? 2 : 4;
  const void* ins[7] = {q, k, v, log_decay, proc_noise, val_prec, y};
  for (const void* p : ins)
    if (!aligned(p, esz)) return KLA_ERR_INVALID_ARG;
  if (!aligned(lambda_out, 4) || !aligned(M_out, 16) || (lambda_in && !aligned(lambda_in, 4)) ||
      (M_in && !aligned(M_in, 16)))
    return KLA_ERR_INVALID_ARG;
  DecodeParams p;
  p.q = q; p.k = k; p.v = v; p.ld = log_decay; p.pn = proc_noise; p.vp = val_prec;
  p.lam_in = lambda_in; p.M_in = M_in; p.lam_out = lambda_out; p.M_out = M_out; p.y = y;
  hipError_t e = launch_decode(p, nheads, dk, dv, dtype == KLA_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KLA_OK : hip_fail(e, "kla_decode_step");
}

extern "C" int kla_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || !aligned(workspace, 256)) return KLA_ERR_WORKSPACE;
  if (workspace_bytes < kHeader || workspace_bytes % 4) return KLA_ERR_INVALID_ARG;
  hipError_t e = launch_fill_zero(workspace, workspace_bytes / 4, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KLA_OK : hip_fail(e, "kla_workspace_init");
}

extern "C" int kla_workspace_error(const void* workspace, int* error_out, void* stream) {
  if (!workspace || !error_out || !aligned(workspace, 256)) return KLA_ERR_INVALID_ARG;
  // Ordered after the work already queued on `stream` (which may be a
  // non-blocking stream that the null stream does not wait for).
  hipStream_t st = static_cast<hipStream_t>(stream);
  unsigned w = 0;
  hipError_t e = hipMemcpyAsync(&w, static_cast<const char*>(workspace) + 4 * kError, 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "kla_workspace_error");
  *error_out = (int)w;
  return KLA_OK;
}

extern "C" const char* kla_status_string(int status) {
  switch (status) {
    case KLA_OK: return "success";
    case KLA_ERR_INVALID_ARG: return "invalid argument (null pointer, size or alignment)";
    case KLA_ERR_UNSUPPORTED: return "unsupported d_k/d_v or dtype (widths 16, 32, 64, 128; dtype f32 or bf16)";
    case KLA_ERR_WORKSPACE: return "workspace missing, not 256-byte aligned, or smaller than required";
    case KLA_ERR_HIP: return g_hip_error[0] ? g_hip_error : "HIP error";
    case KLA_ERR_TOO_LARGE:
      return "kla_forward_noalloc: the shape needs more than KLA_NOALLOC_SCRATCH_BYTES of scratch (use kla_forward)";
    default: return "unknown status";
  }
}
