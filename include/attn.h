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
    ATTN_ERR_VALUE = 7,       /* scale (or tau) is not finite / out of range      */
    ATTN_ERR_SCRATCH = 8      /* attn_bwd_noalloc: the problem needs more scratch
                                 than its static buffer holds                     */
} attn_status;

/* exp2 evaluation used by the softmax. */
enum {
    ATTN_EXP_HW = 0,   /* the hardware transcendental (v_exp_f32)                  */
    ATTN_EXP_POLY3 = 1 /* cubic polynomial on FMA units with exponent-field scaling:
                          the software exponential of "NVIDIA's FlashAttention-4"
                          (section "The Technical Edge") and of the gist.science
                          summary (section 2.B)                                    */
};

/* Schedules (attn_options.variant), for the forward and the backward's dK/dV kernel. */
enum {
    ATTN_VARIANT_AUTO = 0,     /* the library picks per launch (the default)          */
    ATTN_VARIANT_PINGPONG = 1, /* 8-wave workgroups (forward: two half-step-staggered
                                  groups; dK/dV: the query halves of each step split
                                  between wave pairs), one per CU                    */
    ATTN_VARIANT_FOURWAVE = 2  /* 4-wave workgroups, several per CU                  */
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
 *   variant  : schedule.  Forward:
 *              ATTN_VARIANT_FOURWAVE (2): 4-wave workgroups of 128 queries walking
 *              32-key tiles, three per CU (three waves per SIMD), every wave in the
 *              same phase order.  ATTN_VARIANT_PINGPONG (1): 8-wave workgroups of 256
 *              queries walking 64-key tiles, one per CU, whose two 4-wave halves run
 *              half a step apart, so that of the two waves sharing a SIMD one
 *              exponentiates while the other runs matrix products (the two-team
 *              pipelining of the gist.science summary, section 2.A, and the overlap
 *              of "NVIDIA's FlashAttention-4", section "The Technical Edge").
 *              ATTN_VARIANT_AUTO (0, the default): the ping-pong schedule for dense
 *              non-causal launches with S >= 8192 that give every CU at least one
 *              256-query workgroup (B * Hq * ceil(S / 256) >= 256), the four-wave
 *              schedule otherwise (which measured faster each way).  The schedules
 *              round differently (their tiles differ, and with them the rescale
 *              points and the order of the row sums), so their results agree to the
 *              accuracy the library states, not bit for bit; a given schedule is
 *              deterministic.
 *              Backward (the dK/dV kernel; the other two launches have one schedule):
 *              ATTN_VARIANT_FOURWAVE (2): 4-wave workgroups of 128 keys stepping 32
 *              queries at a time, two per CU, so that one workgroup's K/V load and
 *              closing stores overlap the other's steps.  ATTN_VARIANT_PINGPONG (1):
 *              8-wave workgroups of 128 keys stepping 64 queries, one per CU, whose
 *              wave pairs split each step's queries and add their partial dK/dV at the
 *              end.  ATTN_VARIANT_AUTO (0): four-wave when G * ceil(S / 64) <= 256
 *              (G = Hq / Hkv), eight-wave otherwise.  With d = 64 the four-wave
 *              schedule is always used, and with d = 128 and ATTN_EXP_POLY3 the
 *              eight-wave one (its kernel cannot hold K in registers, which four-wave
 *              workgroups need).  The schedules add dK and dV in different orders, so
 *              they agree to the stated accuracy, not bit for bit.
 *              Other values: ATTN_ERR_UNSUPPORTED.
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
 * Bytes of device workspace attn_bwd needs for these sizes, each part rounded up to 256
 * bytes (S_pad = S rounded up to a multiple of 64): three fp32 row arrays [B*Hq][S_pad]
 * (the row term -D_i = -<dO_i, O_i> from the stored O, LSE_i log2(e), and -D_i formed
 * from its definition sum_j P_ij dP_ij, scaled), the preprocess's partial maxima of |dO|,
 * |V|, |Q| and |K| (fp32 [B*Hkv][64][4]), and dO scaled by a power of two per (batch, KV head) in
 * fp16 ([B*Hq][S][d], 2 bytes per element), and Q likewise.  About B*Hq*S*(4d + 12) bytes.
 * Returns 0 for invalid or empty sizes.
 */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int d);

/*
 * Backward pass.  Inputs: q, k, v, the forward outputs o and lse, and the upstream
 * gradient dO.  lse must be the logsumexp of these q, k and scale up to fp32 rounding (as
 * attn_fwd writes it) and o the matching output in bf16; with an lse far from that (say
 * 80 below) the recomputed probabilities overflow and the outputs are not meaningful.
 * Outputs dq, dk, dv are written in full.  workspace: device memory of at least
 * attn_bwd_workspace_bytes(...) bytes, 256-byte aligned, owned by the caller;
 * its contents on entry do not matter and on exit are unspecified.  All outputs
 * are deterministic (no atomics).
 *
 * Rounding: the products run on the MFMA units with fp32 accumulation.  The products
 * that give dK and dV (S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS) take their
 * operands in fp16: Q, K, V and dO are scaled by a power of two per (batch, KV head),
 * found by the preprocess, that makes every value exact in fp16 (bar values more than
 * 2^19 below the group's largest, whose rounding there is far below the outputs'), and P
 * and dS are rounded to fp16 (11 significant bits).  The dQ products take bf16 operands,
 * with dS rounded to bf16.  dK and dV use the row term D_i = sum_j P_ij dP_ij as defined;
 * dQ uses D_i = <dO_i, O_i> with the stored bf16 O.
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
 * Backward pass over a variable-length (packed) batch: the gradients of attn_fwd_varlen,
 * for training on sequences of different lengths laid end to end (the packed batches of
 * the pages' integration targets, hyper.ai FlashAttention-4 story; the backward itself:
 * "NVIDIA Blackwell: FlashAttention-4 Overcomes Memory Bottlenecks", body paragraph).
 * Each sequence is its own attention problem, exactly as attn_bwd computes it.  Layout,
 * token-major, as attn_fwd_varlen:
 *     q, o, dO, dq : [total, Hq,  d] bf16     k, v, dk, dv : [total, Hkv, d] bf16
 *     lse          : [Hq, total]     fp32 (as attn_fwd_varlen writes it)
 *     cu_seqlens   : [nseq + 1] int32 DEVICE array, as for attn_fwd_varlen.
 * max_seqlen must be >= every sequence's length: a longer sequence is taken as its first
 * max_seqlen rows (keys and queries), and its later rows of dq, dk and dv are not
 * written.  Rows not covered by any sequence are not written; overlapping sequences (offsets
 * that are not non-decreasing) leave the rows they share unspecified.  Offsets outside
 * [0, total] are clamped, so no access leaves the tensors.  workspace: at least
 * attn_bwd_varlen_workspace_bytes(nseq, total, Hq, Hkv, d) bytes, 256-byte aligned, owned
 * by the caller (contents on entry do not matter).  nseq == 0, total == 0 or
 * max_seqlen == 0 is an empty problem (ATTN_OK, nothing launched).  Rounding, determinism,
 * checks and the other conventions are those of attn_bwd_ex; opt == NULL means the
 * defaults.
 */
/*
 * Bytes of device workspace attn_bwd_varlen needs: the parts of attn_bwd's workspace, with
 * the row arrays and the fp16 copies of dO and Q laid out by token: per query head,
 * 64 (nseq + ceil(total / 64)) rows (each sequence's rows start on a multiple of 64 and
 * are followed by their padding to 64).  About Hq (total + 64 nseq)(4d + 12) bytes, however
 * the lengths are spread.  Returns 0 for invalid or empty sizes.
 */
size_t attn_bwd_varlen_workspace_bytes(int nseq, int total, int Hq, int Hkv, int d);

int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dO, void* dq, void* dk, void* dv,
                    const int* cu_seqlens, int nseq, int total, int max_seqlen,
                    int Hq, int Hkv, int d, float scale, int causal,
                    void* workspace, size_t workspace_bytes, const attn_options* opt, void* stream);

/*
 * attn_bwd for callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation.  It
 * calls no allocating routine.  Its scratch is a static device array of 64 MiB that the
 * library holds on each GPU it runs on until the process ends (the array's device
 * address is looked up on the first call on each device; the current device's array is
 * used, so stream must belong to the current device).  Problems whose workspace
 * (attn_bwd_workspace_bytes) exceeds 64 MiB return ATTN_ERR_SCRATCH before anything is
 * launched: with d = 128 that is B * Hq * S above about 128 Ki rows (e.g. B = 1, Hq = 16,
 * S = 7680 fits).  Every call on one GPU uses that GPU's one array, whose contents need
 * not be cleared (the backward overwrites what it reads): calls that overlap in time on
 * one GPU (on different streams, or from different host threads) race on it and give
 * wrong results; calls ordered on one stream are safe.  Arguments, checks, outputs and
 * results are those of attn_bwd with the default options.
 */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dO, void* dq, void* dk, void* dv,
                     int B, int Hq, int Hkv, int S, int d, float scale, int causal, void* stream);

/*
 * One phase of attn_bwd_ex, for callers that schedule or time the backward's launches
 * separately.  Running ATTN_BWD_PREPROCESS, ATTN_BWD_DQ and ATTN_BWD_MAIN in that
 * order on one stream, with the same arguments and workspace, is exactly attn_bwd_ex
 * (ATTN_BWD_ALL); each phase needs the ones before it.  The phases communicate through
 * the workspace:
 *   PREPROCESS  reads o, dO, lse, q, k, v; writes -D = -rowsum(dO * O), LSE log2(e) and
 *               the partial maxima of |dO|, |V|, |Q|, |K|;
 *   DQ          reads q, k, v, dO and the above; writes dq, the defined -D (scaled) and
 *               dO and Q in fp16 (scaled);
 *   MAIN        reads k, v, LSE log2(e), the maxima and the DQ phase's -D, fp16 dO and
 *               fp16 Q; writes dk, dv.
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

/*
 * The launch plan that attn_fwd_ex and attn_bwd_ex follow for these sizes and options,
 * computed on the host (no device is touched); for inspection and tests.  Arguments as
 * for attn_fwd_ex (opt may be NULL for the defaults); out receives:
 *   fwd_schedule  : ATTN_VARIANT_PINGPONG or ATTN_VARIANT_FOURWAVE, the dense forward's
 *                   workgroup schedule;
 *   fwd_chunk, dq_chunk, dkdv_chunk : (batch, KV head) groups per dispatch chunk of the
 *                   forward, the dQ kernel and the dK/dV kernel (B * Hkv: one chunk).
 *                   Large launches of sequences of at most 4096 keys run their grid in
 *                   chunks of groups, one after the other, so that the operands the
 *                   resident workgroups re-read stay in the memory-side cache;
 *   dkdv_schedule : ATTN_VARIANT_PINGPONG (eight-wave) or ATTN_VARIANT_FOURWAVE, the
 *                   dK/dV kernel's workgroup shape.
 * Returns ATTN_OK, ATTN_ERR_NULL if out is NULL, or the size / option error that the
 * entry points would return (out is then left unchanged).
 */
typedef struct attn_plan {
    int fwd_schedule;
    int fwd_chunk;
    int dq_chunk;
    int dkdv_chunk;
    int dkdv_schedule;
} attn_plan;
int attn_launch_plan(int B, int Hq, int Hkv, int S, int d, int causal, const attn_options* opt,
                     attn_plan* out);

/* Human-readable name of a status code (never NULL). */
const char* attn_status_string(int status);

/*
 * Evaluate the softmax's exp2 on the device, y[i] = 2^x[i] for i < n, with the
 * given exp_mode, exactly as the forward and backward do (device pointers x, y;
 * n >= 0).  For testing the polynomial and the hardware instruction in isolation.
 * The polynomial clamps x to [-127, 64]: below -127 it gives 0, above 64 it gives
 * 2^64.
 */
int attn_exp2_eval(const float* x, float* y, long n, int exp_mode, void* stream);

/* Host evaluation of the same cubic polynomial exp2 (host pointers x, y). */
void attn_exp2_poly_host(const float* x, float* y, long n);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_ATTN_H */
