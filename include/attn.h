/*
 * attn.h - C ABI of the MI355X (gfx950) exact-attention library, libattn.so.
 *
 * What the library computes
 * -------------------------
 * Exact scaled-dot-product attention over full sequences, forward and backward:
 * the operation the FlashAttention-4 pages describe (hyper.ai FlashAttention-4
 * story, single paragraph: self-attention over the whole sequence, quadratic in
 * its length, with a backward pass whose intermediates are kept on chip;
 * "NVIDIA Blackwell: FlashAttention-4 Overcomes Memory Bottlenecks", body
 * paragraph: both passes, less memory traffic).  The pages print no formula; the
 * library follows the textbook definition.  For batch b, query head hq and its
 * key/value head hkv = hq / (Hq / Hkv):
 *
 *     s_ij  = scale * <q_i, k_j>,  visible keys V(i) = {j <= i} if causal else all
 *     LSE_i = ln sum_{j in V(i)} exp(s_ij)
 *     O_i   = sum_{j in V(i)} exp(s_ij - LSE_i) v_j
 *
 * and the exact gradients dQ, dK, dV of a scalar loss given dO (dK and dV of a
 * key/value head are summed over the Hq/Hkv query heads that read it: the
 * GQA/MQA sharing that "NVIDIA's FlashAttention-4: Cementing AI Infrastructure
 * Dominance in 2025", section "Limitations and the Road Ahead", lists as absent
 * from FA4).  The S x S score matrix is never written to device memory.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Tensor pointers are DEVICE pointers, owned by the caller, contiguous
 *    row-major, 16-byte aligned.  bf16 is IEEE bfloat16 (uint16 storage).
 *      q, o, dO, dq : [B, Hq,  S, d] bf16
 *      k, v, dk, dv : [B, Hkv, S, d] bf16
 *      lse          : [B, Hq,  S]    fp32, natural-log logsumexp of the scaled scores
 *  - d must be 64 or 128; Hq must be a multiple of Hkv; scale is any finite float.
 *  - B == 0 or S == 0 is an empty problem: ATTN_OK, nothing is launched or written,
 *    and the pointers may be NULL.
 *  - stream is a hipStream_t (NULL = the default stream).  Calls are asynchronous
 *    on that stream; results are valid once the stream has synchronized.  No call
 *    synchronizes the host.
 *  - Every argument is checked before anything is launched.  On any error the
 *    status is returned and nothing is written.  Launch failures report
 *    ATTN_ERR_HIP.  No C++ exception crosses this boundary.
 *  - Outputs are overwritten, never accumulated into.  The library allocates no
 *    device memory: the backward pass takes its scratch from the caller's
 *    workspace.  The library holds no state between calls.
 */
#ifndef EXACT_ATTENTION_ATTN_H
#define EXACT_ATTENTION_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,        /* a required pointer is NULL                       */
    ATTN_ERR_SHAPE = 2,       /* negative size, Hq or Hkv < 1, Hq % Hkv != 0,
                                 or a size too large for the library              */
    ATTN_ERR_UNSUPPORTED = 3, /* d not in {64, 128}, or an unknown option value   */
    ATTN_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned          */
    ATTN_ERR_WORKSPACE = 5,   /* backward workspace NULL or smaller than required */
    ATTN_ERR_HIP = 6,         /* the HIP runtime reported an error                */
    ATTN_ERR_VALUE = 7        /* scale (or tau) is not finite / out of range      */
} attn_status;

/* exp2 evaluation used by the softmax. */
enum {
    ATTN_EXP_HW = 0,   /* the hardware transcendental (v_exp_f32)                  */
    ATTN_EXP_POLY3 = 1 /* cubic polynomial on FMA units with exponent-field scaling:
                          the software exponential of "NVIDIA's FlashAttention-4"
                          (section "The Technical Edge") and of the gist.science
                          summary (section 2.B)                                    */
};

/* Forward schedules (attn_options.variant). */
enum {
    ATTN_VARIANT_AUTO = 0,     /* the library picks per launch (the default)          */
    ATTN_VARIANT_PINGPONG = 1, /* 8-wave workgroups in two half-step-staggered groups */
    ATTN_VARIANT_FOURWAVE = 2  /* 4-wave workgroups, two per CU                      */
};

/*
 * Tuning knobs of the forward and backward kernels.  The plain entry points use
 * the defaults (attn_default_options): the choices that measured fastest.
 *   exp_mode : ATTN_EXP_HW or ATTN_EXP_POLY3.
 *   tau      : rescale threshold in log2 units, >= 0 and finite.  The output
 *              accumulator and the running sum are rescaled only when a row's
 *              running maximum grows by more than tau (the "adaptive online
 *              softmax rescaling" of "NVIDIA's FlashAttention-4", section "The
 *              Technical Edge").  The result is the same for every tau; tau only
 *              bounds the unnormalised probabilities by 2^tau.  tau <= 30.
 *   variant  : forward schedule (the backward has one schedule and ignores it).
 *              ATTN_VARIANT_FOURWAVE (2): 4-wave workgroups of 128 queries, two per
 *              CU, every wave in the same phase order.  ATTN_VARIANT_PINGPONG (1):
 *              8-wave workgroups of 256 queries, one per CU, whose two 4-wave
 *              halves run half a step apart, so that of the two waves sharing a
 *              SIMD one exponentiates while the other runs matrix products (the
 *              two-team pipelining of the gist.science summary, section 2.A, and
 *              the overlap of "NVIDIA's FlashAttention-4", section "The Technical
 *              Edge").  ATTN_VARIANT_AUTO (0, the default): the ping-pong schedule
 *              for dense launches with S >= 8192 that give every CU at least one
 *              256-query workgroup (B * Hq * ceil(S / 256) >= 256), the 4-wave
 *              schedule otherwise and for packed batches (which measured faster
 *              each way).  All schedules give bit-identical results, so the choice
 *              affects speed only.  Other values: ATTN_ERR_UNSUPPORTED.
 */
typedef struct attn_options {
    int exp_mode;
    float tau;
    int variant;
} attn_options;

/* The options the plain entry points use. */
attn_options attn_default_options(void);

/*
 * Forward pass: o = attention(q, k, v) and lse (see above).
 * Inputs q, k, v are read only; o and lse are written in full.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int S, int d, float scale, int causal,
             void* stream);

/* attn_fwd with explicit options (opt == NULL means the defaults). */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int Hq, int Hkv, int S, int d, float scale, int causal,
                const attn_options* opt, void* stream);

/*
 * Forward pass over a variable-length (packed) batch: nseq sequences of different
 * lengths laid end to end, as a prefill server batches prompts (the pages' integration
 * target: prefill in SGLang and vLLM, hyper.ai FlashAttention-4 story).  Attention is
 * taken within each sequence only (causal: key j visible to query i of the same sequence
 * iff j <= i).  Layout, token-major:
 *     q, o : [total, Hq,  d] bf16     k, v : [total, Hkv, d] bf16
 *     lse  : [Hq, total]     fp32 (natural log, as in attn_fwd)
 *     cu_seqlens : [nseq + 1] int32 DEVICE array, 0 <= cu_seqlens[0] <= ... <=
 *                  cu_seqlens[nseq] <= total; sequence b is rows cu_seqlens[b] ..
 *                  cu_seqlens[b + 1] - 1.
 * max_seqlen should be >= every sequence's length: it sizes the launch.  Query rows at
 * positions >= max_seqlen within their sequence are not written; the rows that are
 * written still attend over their whole sequence's keys (all of them when non-causal).
 * The library does not read cu_seqlens on the host (it is device memory and the call is
 * asynchronous); offsets outside [0, total] are clamped and a sequence whose end lies
 * before its start is empty, so no access leaves the tensors.  Offsets that are not
 * non-decreasing can make two sequences overlap; rows written by both then hold either
 * result (unspecified).  Rows not covered by any sequence
 * are left unwritten.  nseq == 0, total == 0 or max_seqlen == 0 is an empty problem
 * (ATTN_OK, nothing launched).  Other conventions as above; opt == NULL means the
 * defaults.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens, int nseq, int total, int max_seqlen,
                    int Hq, int Hkv, int d, float scale, int causal,
                    const attn_options* opt, void* stream);

/*
 * Bytes of device workspace attn_bwd needs for these sizes: two fp32 row arrays
 * [B*Hq][S_pad] (the row terms -D_i = -<dO_i, O_i> and LSE_i log2(e), S_pad = S
 * rounded up to a multiple of 64), each rounded up to 256 bytes.  Returns 0 for invalid or
 * empty sizes.
 */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int d);

/*
 * Backward pass.  Inputs: q, k, v, the forward outputs o and lse (as written by
 * attn_fwd, or any consistent pair), and the upstream gradient dO.  Outputs dq,
 * dk, dv are written in full.  workspace: device memory of at least
 * attn_bwd_workspace_bytes(...) bytes, 256-byte aligned, owned by the caller;
 * its contents on entry do not matter and on exit are unspecified.  All outputs
 * are deterministic (no atomics).
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dO, void* dq, void* dk, void* dv,
             int B, int Hq, int Hkv, int S, int d, float scale, int causal,
             void* workspace, size_t workspace_bytes, void* stream);

/* attn_bwd with explicit options (opt == NULL means the defaults). */
int attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dO, void* dq, void* dk, void* dv,
                int B, int Hq, int Hkv, int S, int d, float scale, int causal,
                void* workspace, size_t workspace_bytes, const attn_options* opt, void* stream);

/*
 * One phase of attn_bwd_ex, for callers that schedule or time the backward's launches
 * separately.  Running ATTN_BWD_PREPROCESS, ATTN_BWD_MAIN and ATTN_BWD_DQ in that
 * order on one stream, with the same arguments and workspace, is exactly attn_bwd_ex
 * (ATTN_BWD_ALL); MAIN and DQ are independent of each other.  The phases communicate
 * through the workspace:
 *   PREPROCESS  reads o, dO, lse; writes -D = -rowsum(dO * O) and LSE log2(e);
 *   MAIN        reads q, k, v, dO, D and LSE log2(e); writes dk, dv;
 *   DQ          reads q, k, v, dO, D and LSE log2(e); writes dq.
 * Arguments are validated as for attn_bwd_ex; an unknown phase is ATTN_ERR_UNSUPPORTED.
 */
enum {
    ATTN_BWD_ALL = 0,
    ATTN_BWD_PREPROCESS = 1,
    ATTN_BWD_MAIN = 2,
    ATTN_BWD_DQ = 3
};
int attn_bwd_phase(int phase, const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, void* dq, void* dk, void* dv,
                   int B, int Hq, int Hkv, int S, int d, float scale, int causal,
                   void* workspace, size_t workspace_bytes, const attn_options* opt, void* stream);

/* Human-readable name of a status code (never NULL). */
const char* attn_status_string(int status);

/*
 * Evaluate the softmax's exp2 on the device, y[i] = 2^x[i] for i < n, with the
 * given exp_mode, exactly as the forward does (device pointers x, y; n >= 0).
 * For testing the polynomial and the hardware instruction in isolation.  The
 * polynomial clamps x to [-127, 64]: below -127 it gives 0, above 64 it gives
 * 2^64 (the backward, whose arguments stay near or below 0, omits the upper
 * clamp).
 */
int attn_exp2_eval(const float* x, float* y, long n, int exp_mode, void* stream);

/* Host evaluation of the same cubic polynomial exp2 (host pointers x, y). */
void attn_exp2_poly_host(const float* x, float* y, long n);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_ATTN_H */
