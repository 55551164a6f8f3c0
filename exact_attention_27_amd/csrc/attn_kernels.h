// attn_kernels.h - launch interface between the C ABI (attn_api.hip) and the kernels.
// Arguments here are already validated; launchers only pick a kernel and a grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Scores are s = c_sign * <q, k> * scale.  The kernels keep c = |scale| * log2(e) > 0 and
// apply the sign (or a zero scale) to Q as it is loaded: every 32-bit word of Q is
// transformed as (w & q_and) ^ q_xor, which negates (q_xor = 0x80008000) or zeroes
// (q_and = 0) bf16 pairs exactly.  A zero scale is run as Q = 0 with c = 1.
struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, S;
  float c;
  uint32_t q_and, q_xor;
  float tau;
  // Variable-length (packed) batches; nullptr for the dense [B, H, S, d] layout.  With
  // cu_seqlens set, B is the number of sequences, S the longest sequence (grid size),
  // q/o are [total, Hq, d], k/v [total, Hkv, d] and lse [Hq, total]; sequence b is the
  // rows cu_seqlens[b] .. cu_seqlens[b + 1] - 1 (clamped to [0, total]).
  const int* cu_seqlens;
  int total;
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const float* lse;
  const uint16_t* dO;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;   // [B*Hq][S_pad] fp32 workspace: -D_i = -<dO_i, O_i> (S_pad = S rounded up to 64)
  float* lse2;    // [B*Hq][S_pad] fp32 workspace: LSE_i * log2(e)
  int B, Hq, Hkv, S;
  float c;        // |scale| * log2(e) (1 for a zero scale)
  float scale;    // the caller's scale (dQ and dK carry it)
  uint32_t q_and, q_xor;
};

hipError_t launch_fwd(const FwdArgs& a, int d, bool causal, int exp_mode, bool pingpong, hipStream_t stream);
// The same forward over a variable-length packed batch (a.cu_seqlens != nullptr).
hipError_t launch_fwd_varlen(const FwdArgs& a, int d, bool causal, int exp_mode, bool pingpong, hipStream_t stream);
// phases: bit 0 = preprocess (D, LSE log2 e), bit 1 = dK/dV kernel, bit 2 = dQ kernel.
// 7 runs the whole backward.
hipError_t launch_bwd(const BwdArgs& a, int d, bool causal, int exp_mode, int phases, hipStream_t stream);
hipError_t launch_exp2_eval(const float* x, float* y, long n, int exp_mode, hipStream_t stream);

}  // namespace attn
