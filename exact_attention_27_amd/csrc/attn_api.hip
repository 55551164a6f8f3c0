// attn_api.hip - the C ABI of libattn.so (declared and documented in include/attn.h).
//
// Host side only: argument validation, status codes, workspace layout, and the choice
// of kernel.  Every check runs before any HIP call, so invalid arguments never launch
// anything and never touch the caller's memory.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

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
  // The backward preprocess launches kPreBlocks workgroups per (batch, KV head).
  if ((int64_t)B * Hkv * attn::kPreBlocks >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
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
// four-wave schedule (32-key tiles, three waves per SIMD), which measured 2-5% faster than
// the ping-pong schedule on causal launches from S = 2k to 64k, GQA and packed batches,
// except for dense non-causal launches of S >= 8192 with at least one 256-query
// workgroup per CU, where the ping-pong schedule measured about 1% faster.
// The dK/dV kernel's workgroup shape (where both exist: d = 128 with the hardware
// exponential).  Each workgroup walks G * ceil(S / 64) query blocks at most.  Four-wave
// workgroups, two per CU, overlap one workgroup's K/V load and closing stores with the other's
// steps, and win while the walks are short; eight-wave workgroups, one per CU, take half the
// barriers per product and win on long walks.  Measured: four waves 5-15% faster up to
// G * ceil(S / 64) = 256 (S = 2k-16k at G = 1, S = 2k-4k at G = 4), 1-4% slower at 512.
bool bwd_four_wave(int variant, int G, int S) {
  if (variant == ATTN_VARIANT_PINGPONG) return false;
  if (variant == ATTN_VARIANT_FOURWAVE) return true;
  return (long)G * ((S + 63) / 64) <= 256;
}

bool use_pingpong(int variant, bool packed, bool causal, int B, int Hq, int S) {
  if (variant != ATTN_VARIANT_AUTO) return variant == ATTN_VARIANT_PINGPONG;
  return !packed && !causal && S >= 8192 && (int64_t)B * Hq * ((S + 255) / 256) >= 256;
}

// Backward workspace, in order, each part aligned to 256 bytes (S_pad = S rounded up to
// 64): -D from the bf16 O, LSE log2(e), the exact -D in the dK/dV kernel's units (three fp32
// [B*Hq][S_pad] arrays), the preprocess's partial maxima (fp32 [B*Hkv][64][4]), and dO and
// Q in fp16 (two [B*Hq][S][d] arrays).
struct BwdWorkspace {
  size_t delta, lse2, ndx, pmax, do16, q16, total;
};

BwdWorkspace bwd_workspace(int B, int Hq, int Hkv, int S, int d) {
  const size_t prows = (size_t)B * Hq * (((size_t)S + 63) / 64 * 64);
  BwdWorkspace w;
  w.delta = 0;
  w.lse2 = w.delta + round_up(prows * sizeof(float));
  w.ndx = w.lse2 + round_up(prows * sizeof(float));
  w.pmax = w.ndx + round_up(prows * sizeof(float));
  w.do16 = w.pmax + round_up((size_t)B * Hkv * attn::kPreBlocks * 4 * sizeof(float));
  w.q16 = w.do16 + round_up((size_t)B * Hq * S * d * sizeof(uint16_t));
  w.total = w.q16 + round_up((size_t)B * Hq * S * d * sizeof(uint16_t));
  return w;
}
// The packed backward's workspace: the same parts, the row arrays and the fp16 copies laid
// out by token (attn::varlen_ws_rows rows per query head, a sequence's rows from
// attn::varlen_ws_start), so that it grows with the tokens, not with nseq x the longest.
BwdWorkspace bwd_workspace_varlen(int nseq, int total, int Hq, int Hkv, int d) {
  const size_t prows = (size_t)Hq * attn::varlen_ws_rows(nseq, total);
  BwdWorkspace w;
  w.delta = 0;
  w.lse2 = w.delta + round_up(prows * sizeof(float));
  w.ndx = w.lse2 + round_up(prows * sizeof(float));
  w.pmax = w.ndx + round_up(prows * sizeof(float));
  w.do16 = w.pmax + round_up((size_t)nseq * Hkv * attn::kPreBlocks * 4 * sizeof(float));
  w.q16 = w.do16 + round_up(prows * d * sizeof(uint16_t));
  w.total = w.q16 + round_up(prows * d * sizeof(uint16_t));
  return w;
}
// Sizes of a packed backward, as attn_bwd_varlen checks them (ATTN_OK or the error).
int check_varlen_sizes(int nseq, int total, int max_seqlen, int Hq, int Hkv, int d, bool* empty) {
  if (nseq < 0 || total < 0 || max_seqlen < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  // The grids are those of a dense batch of nseq sequences of max_seqlen rows; per-lane
  // offsets within a tile of token-major rows are 32-bit.
  int st = check_sizes(nseq, Hq, Hkv, max_seqlen, d, empty);
  if (st != ATTN_OK) return st;
  if ((int64_t)Hq * d * 64 * 2 >= (int64_t)1 << 31) return ATTN_ERR_SHAPE;
  *empty = *empty || total == 0;
  return ATTN_OK;
}

// ---------------------------------------------------------------------------------
// Scratch for attn_bwd_noalloc: a file-scope device array (each GPU the library runs on
// holds its own copy until the process ends).  In host code `scratch` names a host-side
// stand-in, not device memory: its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept in scratch_ptr; only that
// address is ever handed to kernels.
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on its first use), or an error.
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ATTN_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return ATTN_OK;
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
    case ATTN_ERR_SCRATCH:
      return "ATTN_ERR_SCRATCH: the backward needs more scratch than attn_bwd_noalloc's static 64 MiB";
    default: return "unknown attn status";
  }
}

int attn_launch_plan(int B, int Hq, int Hkv, int S, int d, int causal, const attn_options* opt,
                     attn_plan* out) {
  if (!out) return ATTN_ERR_NULL;
  bool empty = false;
  int st = check_sizes(B, Hq, Hkv, S, d, &empty);
  if (st != ATTN_OK) return st;
  const attn_options o_ = opt ? *opt : attn_default_options();
  if ((st = check_options(o_)) != ATTN_OK) return st;
  attn_plan p;
  p.fwd_schedule = use_pingpong(o_.variant, false, causal != 0, B, Hq, S) ? ATTN_VARIANT_PINGPONG
                                                                          : ATTN_VARIANT_FOURWAVE;
  p.fwd_chunk = attn::fwd_chunk_groups(B, Hkv, S, d);
  p.dq_chunk = attn::dq_chunk_groups(B, Hkv, S, d);
  p.dkdv_chunk = attn::dkdv_chunk_groups(B, Hq, Hkv, S, d);
  // The launcher's rule: four waves always at d = 64; at d = 128 with the hardware
  // exponential only, by bwd_four_wave; eight waves for the cubic exponential at d = 128.
  const bool four = d == 64 || (o_.exp_mode == ATTN_EXP_HW && bwd_four_wave(o_.variant, Hq / Hkv, S));
  p.dkdv_schedule = four ? ATTN_VARIANT_FOURWAVE : ATTN_VARIANT_PINGPONG;
  *out = p;
  return ATTN_OK;
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
  return hip_status(attn::launch_fwd(a, d, causal != 0, o_.exp_mode, use_pingpong(o_.variant, false, causal != 0, B, Hq, S),
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
                                            use_pingpong(o_.variant, true, causal != 0, nseq, Hq, max_seqlen),
                                            static_cast<hipStream_t>(stream)));
}


size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int d) {
  bool empty = false;
  if (check_sizes(B, Hq, Hkv, S, d, &empty) != ATTN_OK || empty) return 0;
  return bwd_workspace(B, Hq, Hkv, S, d).total;
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
  const BwdWorkspace wl = bwd_workspace(B, Hq, Hkv, S, d);
  char* ws = static_cast<char*>(workspace);
  a.delta = reinterpret_cast<float*>(ws + wl.delta);
  a.lse2 = reinterpret_cast<float*>(ws + wl.lse2);
  a.ndx = reinterpret_cast<float*>(ws + wl.ndx);
  a.pmax = reinterpret_cast<float*>(ws + wl.pmax);
  a.do16 = reinterpret_cast<uint16_t*>(ws + wl.do16);
  a.q16 = reinterpret_cast<uint16_t*>(ws + wl.q16);
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S = S;
  a.scale = scale;
  scale_setup(scale, &a.c, &a.q_and, &a.q_xor);
  a.cu_seqlens = nullptr;
  a.total = 0;
  (void)hipGetLastError();
  return hip_status(attn::launch_bwd(a, d, causal != 0, o_.exp_mode, bwd_four_wave(o_.variant, Hq / Hkv, S), phases,
                                     static_cast<hipStream_t>(stream)));
}

size_t attn_bwd_varlen_workspace_bytes(int nseq, int total, int Hq, int Hkv, int d) {
  bool empty = false;
  if (check_varlen_sizes(nseq, total, 0, Hq, Hkv, d, &empty) != ATTN_OK || nseq == 0 || total == 0) return 0;
  return bwd_workspace_varlen(nseq, total, Hq, Hkv, d).total;
}

int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dO, void* dq, void* dk, void* dv,
                    const int* cu_seqlens, int nseq, int total, int max_seqlen,
                    int Hq, int Hkv, int d, float scale, int causal,
                    void* workspace, size_t workspace_bytes, const attn_options* opt, void* stream) {
  bool empty = false;
  int st = check_varlen_sizes(nseq, total, max_seqlen, Hq, Hkv, d, &empty);
  if (st != ATTN_OK) return st;
  const attn_options o_ = opt ? *opt : attn_default_options();
  if ((st = check_options(o_)) != ATTN_OK) return st;
  if (!std::isfinite(scale)) return ATTN_ERR_VALUE;
  if (empty) return ATTN_OK;
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv || !cu_seqlens) return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(dO) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0)
    return ATTN_ERR_ALIGN;
  const size_t need = attn_bwd_varlen_workspace_bytes(nseq, total, Hq, Hkv, d);
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
  const BwdWorkspace wl = bwd_workspace_varlen(nseq, total, Hq, Hkv, d);
  char* ws = static_cast<char*>(workspace);
  a.delta = reinterpret_cast<float*>(ws + wl.delta);
  a.lse2 = reinterpret_cast<float*>(ws + wl.lse2);
  a.ndx = reinterpret_cast<float*>(ws + wl.ndx);
  a.pmax = reinterpret_cast<float*>(ws + wl.pmax);
  a.do16 = reinterpret_cast<uint16_t*>(ws + wl.do16);
  a.q16 = reinterpret_cast<uint16_t*>(ws + wl.q16);
  a.B = nseq; a.Hq = Hq; a.Hkv = Hkv; a.S = max_seqlen;
  a.scale = scale;
  scale_setup(scale, &a.c, &a.q_and, &a.q_xor);
  a.cu_seqlens = cu_seqlens;
  a.total = total;
  (void)hipGetLastError();
  // The dK/dV workgroup shape by the walk of a sequence of the mean length (total / nseq)
  // rather than the longest: in a mix of lengths most walks are much shorter than the
  // longest one (packed training batch of 32 sequences, 268-7377 tokens: four waves 1.4%
  // faster, where the longest length alone chooses eight).
  const int mean_len = (int)(((int64_t)total + nseq - 1) / nseq);
  return hip_status(attn::launch_bwd(a, d, causal != 0, o_.exp_mode,
                                     bwd_four_wave(o_.variant, Hq / Hkv, std::min(mean_len, max_seqlen)), 7,
                                     static_cast<hipStream_t>(stream)));
}

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dO, void* dq, void* dk, void* dv,
                     int B, int Hq, int Hkv, int S, int d, float scale, int causal, void* stream) {
  // Every check before any HIP call, as for attn_bwd; then the size against the scratch.
  bool empty = false;
  int st = check_sizes(B, Hq, Hkv, S, d, &empty);
  if (st != ATTN_OK) return st;
  if (!std::isfinite(scale)) return ATTN_ERR_VALUE;
  if (empty) return ATTN_OK;
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(dO) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return ATTN_ERR_ALIGN;
  const size_t need = attn_bwd_workspace_bytes(B, Hq, Hkv, S, d);
  if (need > kScratchBytes) return ATTN_ERR_SCRATCH;
  void* ws = nullptr;
  if ((st = current_scratch(&ws)) != ATTN_OK) return st;
  return attn_bwd_phase(ATTN_BWD_ALL, q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, S, d, scale, causal, ws,
                        kScratchBytes, nullptr, stream);
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
