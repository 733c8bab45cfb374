// Internal interface between the C ABI (kla_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kla {

// Control words at the head of every workspace (32-bit each).  Words 0 and 1
// hold the call epoch and the groups-done counter (kla_device.h).
enum CtrlWord { kError = 3 };

// Done counters: a fixed region of kDoneCounters words right after the
// 256-byte header, at the same place and of the same size whatever the call's
// shape, so that no call ever lays flags or payloads over them (a counter
// that starts from another array's leftover never fires, and the call epoch
// would then stop advancing).  Unit u (a head, a chain block) counts on word
// u % kDoneCounters.
constexpr int kDoneCounters = 4096;

// Ticket counters: a fixed region right after the done counters, one counter
// per 64-byte line (so that the atomics of many workgroups starting together
// spread over many lines), zero whenever no call runs.  A kernel whose
// workgroups wait on each other numbers them with tickets: group x =
// blockIdx % tgroups (tgroups divides the unit count, at most kTicketGroups)
// draws from counter x, and the workgroup that draws a counter's last ticket
// sets it back to zero.
constexpr int kTicketStride = 16;
constexpr int kTicketGroups = 256;
constexpr int kTicketWords = kTicketStride * kTicketGroups;

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* ld;   // log_decay
  const void* pn;   // proc_noise
  const void* vp;   // val_prec
  const float* lam0;  // nullable
  const float* M0;    // nullable
  void* y;
  float* lamT;
  float* MT;
  float* lpath;       // nullable
  const float* theta;   // OU inputs only ([H][dk] rate; ld then holds the step length), else null
  const float* sigma2;  // OU inputs only ([H][dk] diffusion)
  // Coefficient prologue (cw[0] non-null): q, k, v hold the raw projections,
  // ld the raw step length and vp the raw value precision; cw[] are the
  // causal convolution taps of q, k, v ([H][d][cwidth]), cb[] their biases
  // ([H][d], nullable).
  const float* cw[3];
  const float* cb[3];
  int cwidth;
  int nheads, T, nseg;
  int tgroups;        // ticket groups (divides nheads, at most kTicketGroups): group x takes the heads h = x mod tgroups
  unsigned* tick;     // ticket counters, group x at word kTicketStride * x
  int H;              // heads per batch row (indexes theta / sigma2)
  int mskip;          // a segment whose predecessor's inclusive mean is already out publishes no aggregate
  unsigned* ctrl;     // workspace control words
  unsigned* hdone;    // [kDoneCounters] segments done with their flags, per head group
  unsigned* pflag;    // [nheads*nseg][2] precision-carry flags, one per carry wave
  unsigned* mflag;    // [nheads*nseg][waves] mean-carry flags, one per wave
  float* pagg;        // [nheads*nseg][dk][4] segment 2x2 aggregates
  unsigned long long* pinc;  // [nheads*nseg][dk] precision after the segment: {value bits, flag}
  float* mF;          // [nheads*nseg][waves][dk] prod of forget gates over the segment (per wave)
  float* magg;        // [nheads*nseg][dk*dv] local mean state (fragment order)
  float* minc;        // [nheads*nseg][dk*dv] mean state after the segment (fragment order)
};

struct PscanParams {
  const float* ld;
  const float* pn;
  const float* c;
  const float* lam0;  // nullable
  float* lpath;
  float* lamT;        // nullable
  long long nchains;  // B*H*D
  int D, T, nseg, seglen, ncblocks;
  int tgroups;        // ticket groups (divides ncblocks, at most kTicketGroups): group x takes the chain blocks cb = x mod tgroups
  unsigned* tick;     // ticket counters, group x at word kTicketStride * x
  unsigned* ctrl;
  unsigned* bdone;    // [kDoneCounters] segments done with their flags, per chain-block group
  unsigned* flag;     // [nseg*ncblocks]
  float* agg;         // [ncblocks*nseg*256][4]
  float* inc;         // [ncblocks*nseg*256]
};

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const void* ld;     // log_decay
  const void* pn;     // proc_noise
  const void* vp;     // val_prec
  const float* lam_in;  // nullable (prior precision 1)
  const float* M_in;    // nullable (prior mean 0)
  float* lam_out;       // may equal lam_in
  float* M_out;         // may equal M_in
  void* y;
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* ld;     // log_decay
  const void* pn;     // proc_noise
  const void* vp;     // val_prec
  const void* dy;     // gradient of y
  const float* lam0;  // nullable (prior precision 1)
  const float* M0;    // nullable (prior mean 0)
  const float* lpath; // precision after every token [nheads][T][dk]
  const float* dlamT; // nullable
  const float* dMT;   // nullable
  void* dq;
  void* dk;
  void* dv;
  void* dld;
  void* dpn;
  void* dvp;
  float* dlam0;
  float* dM0;
  int nheads, T, nseg;
  int ncu;            // compute units of the device (the chunk kernel's grid)
  long long nchains;  // nheads * dk
  float* F;           // [nheads][nseg][dk] product of forget gates over the segment
  float* Mseg;        // [nheads][nseg][dk][dv] segment aggregate, then the mean entering the segment
  float* Gseg;        // [nheads][nseg][dk][dv] segment aggregate, then the adjoint at the segment end
  float* rs;          // [nheads][dk] sum_j M_T[i][j] dM_T[i][j]
  float* dgw;         // [nheads][T][dk] gradient of the write gate
  float* ew;          // [nheads][T][dk] q dq - g dg (per-token share of the log-forget-gate gradient)
  size_t ehalf;       // nonzero: dgw and ew hold a second value half's partials ehalf elements on,
                      // which the chain adds to the first's
  float* comp;        // [nseg][nchains][4] reverse-chain block composites
  float* cin;         // [nseg][nchains][2] reverse-chain state entering each block from the right
  // Strides (elements).  A call with d_k or d_v = 128 runs as 64-wide
  // sub-problems on strided views of the full arrays; otherwise every stride
  // is the plain one (ks = kws = ksh = dk, vs = dv, mrow = dv, mhead = dk*dv).
  int ks;             // row of the key-side per-token arrays (inputs, lpath, dq, dk, dld, dpn, dvp)
  int vs;             // row of the value-side per-token arrays (v, dy, dv)
  int kws;            // row of dgw, ew and dq_acc
  int ksh;            // head of the key vectors (lam0, dlamT, dlam0, rs)
  int mrow, mhead;    // row and head of the state matrices (M0, dMT, dM0)
  int vacc;           // row of dv_acc
  float* dq_acc;      // nullable: this value half's fp32 partial of dq, written instead of dq
  float* dv_acc;      // nullable: this key half's fp32 partial of dv, written instead of dv
  int add_rs;         // add into rs (a later value half) instead of writing
};

struct VprecParams {
  const void* q;
  const void* k;
  const void* v;
  const void* ld;     // log_decay
  const void* pn;     // proc_noise
  const void* vp;     // val_prec, [B,H,T,dv]
  const float* lam0;  // nullable, [B,H,dk,dv]
  const float* M0;    // nullable
  void* y;
  float* lamT;        // [B,H,dk,dv]
  float* MT;
  int T;
};

// The run-streaming forward kernel (bf16, d_k = d_v = 64, log_decay and
// proc_noise given per token): one workgroup per (head, run of R tiles of 64
// tokens), taken in ticket order.
struct FwdRunParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* ld;  // log_decay
  const uint16_t* pn;  // proc_noise
  const uint16_t* vp;  // val_prec
  const float* lam0;   // nullable
  const float* M0;     // nullable
  uint16_t* y;
  float* lamT;
  float* MT;
  float* lpath;        // nullable
  int nheads, T, ntiles, nrun;
  int R0, Rb, Rx;      // run 0 takes R0 tiles; run r >= 1 takes Rb, plus one if r - 1 < Rx
  int agg_always;      // every run but the last publishes its aggregate (all runs resident at once)
  int tgroups;         // ticket groups (divides nheads, at most kTicketGroups): group x takes the heads h = x mod tgroups
  unsigned* ctrl;      // workspace control words (epoch, groups done, error)
  unsigned* tick;      // ticket counters, group x at word kTicketStride * x
  unsigned* flag;      // [nheads*nrun][4] mean-carry flags, one per matrix wave
  float* dv;           // [nheads*nrun][4][64] prod of forget gates over the run (a copy per wave)
  float* magg;         // [nheads*nrun][4096] local mean state of the run (fragment order)
  float* minc;         // [nheads*nrun][4096] mean state after the run (fragment order)
};
void fwd_run_plan(int nheads, int T, int ncu, int& R0, int& Rb, int& Rx, int& nrun, bool& one_round);
hipError_t launch_forward_run(const FwdRunParams& p, hipStream_t stream);

int fwd_segment_len(int dk, int dv, bool bf16);
hipError_t launch_forward(const FwdParams& p, int dk, int dv, bool bf16, hipStream_t stream);
hipError_t launch_pscan(const PscanParams& p, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, long long nheads, int dk, int dv, bool bf16, hipStream_t stream);
hipError_t launch_backward_front(const BwdParams& p, int dk, int dv, bool bf16, hipStream_t stream);
hipError_t launch_backward_chain(const BwdParams& p, int dk, bool bf16, hipStream_t stream);
hipError_t launch_backward_convert(const float* acc, void* out, long long n, bool bf16, hipStream_t stream);
hipError_t launch_backward_empty(const float* dlamT, const float* dMT, float* dlam0, float* dM0,
                                 long long nl, long long nm, hipStream_t stream);
hipError_t launch_vprec(const VprecParams& p, long long nheads, int dk, int dv, bool bf16, hipStream_t stream);
hipError_t launch_fill_zero(void* ptr, size_t words, hipStream_t stream);
// *dst = *src (0 when src is null), one thread.
hipError_t launch_word_copy(const unsigned* src, int* dst, hipStream_t stream);
hipError_t launch_state_copy(const float* lam0, const float* M0, float* lamT, float* MT,
                             long long nl, long long nm, hipStream_t stream);

}  // namespace kla
