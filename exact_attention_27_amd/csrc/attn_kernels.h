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
  // KV groups per dispatch chunk (set by the launcher, dispatch_chunk below).
  int grp_chunk;
};

// Workgroups of the backward preprocess per (batch, KV head); each leaves one set of
// partial maxima in the workspace (BwdArgs::pmax), so the later kernels reduce this many.
constexpr int kPreBlocks = 64;

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
  // Workspace (S_pad = S rounded up to 64; a "group" is one (batch, KV head)):
  float* delta;   // [B*Hq][S_pad] fp32: -D_i = -<dO_i, O_i> from the stored bf16 O (preprocess)
  float* lse2;    // [B*Hq][S_pad] fp32: LSE_i * log2(e) (preprocess)
  float* ndx;     // [B*Hq][S_pad] fp32: -D_i = -sum_j P_ij dP_ij, times 2^(e_dO + e_V) (dQ kernel)
  float* pmax;    // [B*Hkv][kPreBlocks][4] fp32: partial maxima of |dO|, |V|, |Q|, |K| per group (preprocess)
  uint16_t* do16; // [B*Hq][S][d] fp16: dO * 2^e_dO (dQ kernel), the dK/dV kernel's dO operand
  uint16_t* q16;  // [B*Hq][S][d] fp16: Q * 2^e_Q (dQ kernel), the dK/dV kernel's Q operand
  int B, Hq, Hkv, S;
  float c;        // |scale| * log2(e) (1 for a zero scale)
  float scale;    // the caller's scale (dQ and dK carry it)
  uint32_t q_and, q_xor;
  // KV groups per dispatch chunk of the dQ and the dK/dV kernels (set by the launcher).
  int dq_chunk, kv_chunk;
  // Variable-length (packed) batches; nullptr for the dense [B, H, S, d] layout.  With
  // cu_seqlens set, B is the number of sequences and S the longest sequence (it sizes the
  // grids); q, o, dO, dq are [total, Hq, d], k, v, dk, dv [total, Hkv, d] and lse
  // [Hq, total]; sequence b is the rows cu_seqlens[b] .. cu_seqlens[b + 1] - 1 (clamped to
  // [0, total]), of which the first S are used; the workspace's row arrays and fp16 copies
  // are laid out by token (varlen_ws_rows below) instead of [B*Hq][S_pad] and [B*Hq][S][d].
  const int* cu_seqlens;
  int total;
};

// The packed backward's workspace rows (every row array, and the fp16 copies' rows): per
// query head h, varlen_ws_rows(B, total) rows at h * varlen_ws_rows; sequence b's rows from
// varlen_ws_start(b, start), start being its first token.  Starts are multiples of 64 and
// a sequence of L tokens owns at least L rounded up to 64 rows before the next one's start
// (start_{b+1} >= start_b + L_b), so 64-row blocks stay aligned and inside the sequence's
// rows; the whole takes rows in proportion to the tokens, not to B times the longest.
__host__ __device__ inline size_t varlen_ws_rows(int B, int total) {
  return (size_t)64 * ((size_t)B + ((size_t)total + 63) / 64);
}
__host__ __device__ inline size_t varlen_ws_start(int b, int start) {
  return (size_t)64 * ((size_t)b + ((size_t)start + 63) / 64);
}

// Dispatch chunks.  A launch whose workgroups of one (batch, KV head) group all re-read
// that group's group_bytes of operands (K and V; Q and dO) runs its grid in chunks of
// groups, one chunk after the other, so that the resident workgroups share a few groups'
// operands in L2 and the memory-side cache instead of streaming every group's from HBM.
// Chunks are used when the operands of all groups exceed 160 MiB (the 256 MiB
// memory-side cache holds less beside the other streams) and sequences have at most 4096
// keys: the fewest equal chunks of at most about 96 MiB each, rounded up to a multiple of
// 8 groups.  Longer sequences keep one chunk: there a causal launch's longest workgroups
// are a large share of its run and must start first.  Returns groups per chunk.
inline int dispatch_chunk(int ngrp, int S, long group_bytes) {
  const long budget = 96L << 20;
  const long total = (long)ngrp * group_bytes;
  if (S > 4096 || S < 1 || group_bytes < 1 || total <= (160L << 20)) return ngrp;
  const long nch = (total + budget - 1) / budget;
  const long c = ((ngrp + nch - 1) / nch + 7) & ~7L;
  return c >= ngrp ? ngrp : (int)c;
}

// Groups per dispatch chunk of each chunked kernel: the forward and the dQ kernel re-read
// a group's K and V (4 S d bytes), the dK/dV kernel its G query heads' fp16 Q and dO
// (4 G S d bytes).
inline int fwd_chunk_groups(int B, int Hkv, int S, int d) { return dispatch_chunk(B * Hkv, S, 4L * S * d); }
inline int dq_chunk_groups(int B, int Hkv, int S, int d) { return dispatch_chunk(B * Hkv, S, 4L * S * d); }
inline int dkdv_chunk_groups(int B, int Hq, int Hkv, int S, int d) {
  return dispatch_chunk(B * Hkv, S, 4L * (Hq / Hkv) * S * d);
}
// Packed batches (every chunked kernel): chunks of 8 groups, one (sequence, KV head) per
// XCD at a time, so that the resident workgroups of an XCD walk one sequence's operands
// together.  In the unchunked order each XCD runs tiles of about 32 sequences at once, each
// streaming its own rows past the shared L2.  (Measured on 32 sequences of 268-7377
// tokens, GQA 32:8: backward 13.7 -> 9.75 ms, forward -0.9%; chunks of 16 or 32 groups
// gained less or lost.)
inline int varlen_chunk_groups(int nseq, int Hkv) { return nseq * Hkv < 8 ? nseq * Hkv : 8; }

hipError_t launch_fwd(const FwdArgs& a, int d, bool causal, int exp_mode, bool pingpong, hipStream_t stream);
// The same forward over a variable-length packed batch (a.cu_seqlens != nullptr).
hipError_t launch_fwd_varlen(const FwdArgs& a, int d, bool causal, int exp_mode, bool pingpong, hipStream_t stream);
// phases: bit 0 = preprocess (D, LSE log2 e), bit 1 = dK/dV kernel, bit 2 = dQ kernel.
// A packed batch when a.cu_seqlens is set.
// 7 runs the whole backward.
// four_wave: the dK/dV kernel in four-wave workgroups, two per CU (d = 64 always; at
// d = 128 only with the hardware exponential); otherwise eight-wave workgroups, one per CU.
hipError_t launch_bwd(const BwdArgs& a, int d, bool causal, int exp_mode, bool four_wave, int phases,
                      hipStream_t stream);
hipError_t launch_exp2_eval(const float* x, float* y, long n, int exp_mode, hipStream_t stream);

}  // namespace attn
