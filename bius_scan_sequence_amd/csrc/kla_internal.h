// Internal interface between the C ABI (kla_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kla {

// Control words at the head of every workspace (32-bit each).
enum CtrlWord { kError = 3 };

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
  int nheads, T, nseg;
  unsigned* ctrl;     // workspace control words
  unsigned* hdone;    // [nheads] segments of the head done with their flags
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
  unsigned* ctrl;
  unsigned* bdone;    // [ncblocks] segments of the block done with their flags
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

int fwd_segment_len(int dk, int dv, bool bf16);
hipError_t launch_forward(const FwdParams& p, int dk, int dv, bool bf16, hipStream_t stream);
hipError_t launch_pscan(const PscanParams& p, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, long long nheads, int dk, int dv, bool bf16, hipStream_t stream);
hipError_t launch_fill_zero(void* ptr, size_t words, hipStream_t stream);
hipError_t launch_state_copy(const float* lam0, const float* M0, float* lamT, float* MT,
                             long long nl, long long nm, hipStream_t stream);

}  // namespace kla
