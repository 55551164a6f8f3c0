// attn_api.hip - the C ABI of libattn.so (declared and documented in include/attn.h).
//
// Host side only: argument validation, status codes, workspace layout, and the choice
// of kernel.  Every check runs before any HIP call, so invalid arguments never launch
// anything and never touch the caller's memory.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "attn.h"
#include "attn_device.h"
#include "attn_kernels.h"

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates sizes.  Returns ATTN_OK, or the error; sets *empty for B == 0 or S == 0.
int check_sizes(int B, int Hq, int Hkv, int S, int d, bool* empty) {
  if (B < 0 || S < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  // Grid and index limits: workgroup counts must fit in 31 bits, and per-head element
  // offsets are computed in 64 bits but row indices in 32 bits.
  const int64_t tiles = ((int64_t)S + 127) / 128;
  if ((int64_t)B * Hq * tiles >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  if ((int64_t)S * d >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  // The backward preprocess runs one thread per 8 elements of each padded row.
  const int64_t pre_blocks = ((int64_t)B * Hq * ((S + 63) / 64 * 64) * (d / 8) + 255) / 256;
  if (pre_blocks >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  *empty = (B == 0 || S == 0);
  return ATTN_OK;
}

int check_options(const attn_options& o) {
  if (o.exp_mode != ATTN_EXP_HW && o.exp_mode != ATTN_EXP_POLY3) return ATTN_ERR_UNSUPPORTED;
  if (o.variant != ATTN_VARIANT_AUTO && o.variant != ATTN_VARIANT_PINGPONG && o.variant != ATTN_VARIANT_FOURWAVE)
    return ATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(o.tau) || o.tau < 0.0f || o.tau > 30.0f) return ATTN_ERR_VALUE;
  return ATTN_OK;
}

// Scale handling shared by both passes: the kernels see c = |scale| log2(e) > 0 and a
// Q transform that applies the sign (see attn_kernels.h).
void scale_setup(float scale, float* c, uint32_t* q_and, uint32_t* q_xor) {
  *q_and = 0xffffffffu;
  *q_xor = 0u;
  if (scale == 0.0f) {
    *c = 1.0f;
    *q_and = 0u;
  } else {
    *c = std::fabs(scale) * attn::kLog2e;
    if (scale < 0.0f) *q_xor = 0x80008000u;
  }
}

int hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// The forward schedule a launch runs (true: ping-pong).  ATTN_VARIANT_AUTO takes the
// ping-pong schedule for dense launches of S >= 8192 with at least one 256-query
// workgroup per CU, where it measured 1-3% faster; on shorter sequences, small grids
// and packed batches the 4-wave schedule measured faster.
bool use_pingpong(int variant, bool packed, int B, int Hq, int S) {
  if (variant != ATTN_VARIANT_AUTO) return variant == ATTN_VARIANT_PINGPONG;
  return !packed && S >= 8192 && (int64_t)B * Hq * ((S + 255) / 256) >= 256;
}

}  // namespace

extern "C" {

attn_options attn_default_options(void) {
  attn_options o;
  o.exp_mode = ATTN_EXP_HW;
  o.tau = 8.0f;
  o.variant = ATTN_VARIANT_AUTO;
  return o;
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_NULL: return "ATTN_ERR_NULL: a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "ATTN_ERR_SHAPE: invalid or too large B/Hq/Hkv/S, or Hq not a multiple of Hkv";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED: head dim not in {64,128} or unknown option";
    case ATTN_ERR_ALIGN: return "ATTN_ERR_ALIGN: tensor pointer not 16-byte aligned";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE: backward workspace missing, misaligned or too small";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: the HIP runtime reported an error";
    case ATTN_ERR_VALUE: return "ATTN_ERR_VALUE: scale or tau not finite or out of range";
    default: return "unknown attn status";
  }
}

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int Hq, int Hkv, int S, int d, float scale, int causal,
                const attn_options* opt, void* stream) {
  bool empty = false;
  int st = check_sizes(B, Hq, Hkv, S, d, &empty);
  if (st != ATTN_OK) return st;
  const attn_options o_ = opt ? *opt : attn_default_options();
  if ((st = check_options(o_)) != ATTN_OK) return st;
  if (!std::isfinite(scale)) return ATTN_ERR_VALUE;
  if (empty) return ATTN_OK;
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_ALIGN;

  attn::FwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S = S;
  scale_setup(scale, &a.c, &a.q_and, &a.q_xor);
  a.tau = o_.tau;
  a.cu_seqlens = nullptr;
  a.total = 0;
  (void)hipGetLastError();  // a stale error from earlier work is not this call's failure
  return hip_status(attn::launch_fwd(a, d, causal != 0, o_.exp_mode, use_pingpong(o_.variant, false, B, Hq, S),
                                     static_cast<hipStream_t>(stream)));
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int S, int d, float scale, int causal, void* stream) {
  return attn_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, S, d, scale, causal, nullptr, stream);
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens, int nseq, int total, int max_seqlen,
                    int Hq, int Hkv, int d, float scale, int causal,
                    const attn_options* opt, void* stream) {
  if (nseq < 0 || total < 0 || max_seqlen < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  // Workgroups (sequences x heads x query tiles) must fit in 31 bits; row offsets are
  // computed in 64 bits, per-tile offsets in 32.
  const int64_t tiles = ((int64_t)max_seqlen + 127) / 128;
  if ((int64_t)nseq * Hq * tiles >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  if ((int64_t)Hq * d * 64 * 2 >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  const attn_options o_ = opt ? *opt : attn_default_options();
  int st = check_options(o_);
  if (st != ATTN_OK) return st;
  if (!std::isfinite(scale)) return ATTN_ERR_VALUE;
  if (nseq == 0 || total == 0 || max_seqlen == 0) return ATTN_OK;
  if (!q || !k || !v || !o || !lse || !cu_seqlens) return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0)
    return ATTN_ERR_ALIGN;

  attn::FwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.B = nseq; a.Hq = Hq; a.Hkv = Hkv; a.S = max_seqlen;
  scale_setup(scale, &a.c, &a.q_and, &a.q_xor);
  a.tau = o_.tau;
  a.cu_seqlens = cu_seqlens;
  a.total = total;
  (void)hipGetLastError();
  return hip_status(attn::launch_fwd_varlen(a, d, causal != 0, o_.exp_mode,
                                            use_pingpong(o_.variant, true, nseq, Hq, max_seqlen),
                                            static_cast<hipStream_t>(stream)));
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int d) {
  bool empty = false;
  if (check_sizes(B, Hq, Hkv, S, d, &empty) != ATTN_OK || empty) return 0;
  const size_t prows = (size_t)B * Hq * (((size_t)S + 63) / 64 * 64);
  return 2 * round_up(prows * sizeof(float));
}

int attn_bwd_phase(int phase, const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, void* dq, void* dk, void* dv,
                   int B, int Hq, int Hkv, int S, int d, float scale, int causal,
                   void* workspace, size_t workspace_bytes, const attn_options* opt, void* stream) {
  int phases;
  switch (phase) {
    case ATTN_BWD_ALL: phases = 7; break;
    case ATTN_BWD_PREPROCESS: phases = 1; break;
    case ATTN_BWD_MAIN: phases = 2; break;
    case ATTN_BWD_DQ: phases = 4; break;
    default: return ATTN_ERR_UNSUPPORTED;
  }
  bool empty = false;
  int st = check_sizes(B, Hq, Hkv, S, d, &empty);
  if (st != ATTN_OK) return st;
  const attn_options o_ = opt ? *opt : attn_default_options();
  if ((st = check_options(o_)) != ATTN_OK) return st;
  if (!std::isfinite(scale)) return ATTN_ERR_VALUE;
  if (empty) return ATTN_OK;
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(dO) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return ATTN_ERR_ALIGN;
  const size_t need = attn_bwd_workspace_bytes(B, Hq, Hkv, S, d);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
    return ATTN_ERR_WORKSPACE;

  attn::BwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.lse = lse;
  a.dO = static_cast<const uint16_t*>(dO);
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  const size_t prows = (size_t)B * Hq * (((size_t)S + 63) / 64 * 64);
  a.delta = static_cast<float*>(workspace);
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + round_up(prows * sizeof(float)));
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S = S;
  a.scale = scale;
  scale_setup(scale, &a.c, &a.q_and, &a.q_xor);
  (void)hipGetLastError();
  return hip_status(attn::launch_bwd(a, d, causal != 0, o_.exp_mode, phases, static_cast<hipStream_t>(stream)));
}

int attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dO, void* dq, void* dk, void* dv,
                int B, int Hq, int Hkv, int S, int d, float scale, int causal,
                void* workspace, size_t workspace_bytes, const attn_options* opt, void* stream) {
  return attn_bwd_phase(ATTN_BWD_ALL, q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, S, d, scale, causal,
                        workspace, workspace_bytes, opt, stream);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dO, void* dq, void* dk, void* dv,
             int B, int Hq, int Hkv, int S, int d, float scale, int causal,
             void* workspace, size_t workspace_bytes, void* stream) {
  return attn_bwd_ex(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, S, d, scale, causal,
                     workspace, workspace_bytes, nullptr, stream);
}

int attn_exp2_eval(const float* x, float* y, long n, int exp_mode, void* stream) {
  if (n < 0) return ATTN_ERR_SHAPE;
  if (exp_mode != ATTN_EXP_HW && exp_mode != ATTN_EXP_POLY3) return ATTN_ERR_UNSUPPORTED;
  if (n == 0) return ATTN_OK;
  if (!x || !y) return ATTN_ERR_NULL;
  if (n > ((long)1 << 40)) return ATTN_ERR_SHAPE;
  (void)hipGetLastError();
  return hip_status(attn::launch_exp2_eval(x, y, n, exp_mode, static_cast<hipStream_t>(stream)));
}

void attn_exp2_poly_host(const float* x, float* y, long n) {
  for (long i = 0; i < n; ++i) y[i] = attn::exp2_poly3(x[i]);
}

}  // extern "C"
