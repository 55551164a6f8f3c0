// attn_bwd.hip - backward pass of exact attention on gfx950 (CDNA4).
//
// The backward recomputes the probabilities from the saved logsumexp instead of
// storing them (the pages keep backward intermediates on chip: hyper.ai
// FlashAttention-4 story; "NVIDIA Blackwell: FlashAttention-4 Overcomes Memory
// Bottlenecks", body paragraph).  Three launches on the caller's stream:
//
//  1. bwd_pre:  -D_i = -<dO_i, O_i> in fp32 from the stored bf16 O and dO, and LSE_i log2(e),
//               into the workspace.  Bound by HBM bandwidth.
//  2. bwd_main: dK and dV.  One workgroup per (batch, KV head, tile of 128 keys) keeps dK
//               and dV for its keys in registers for the whole run and walks the query
//               tiles (64 or 32 queries, by workgroup shape) that can see its keys (causal:
//               only tiles at or below the diagonal), from the last one down, for every
//               query head of the GQA group.  Per step, with Q, dO, LSE and D staged in LDS:
//                   S   = Q K^T,  dP = dO V^T     (MFMA; K and V stay on chip for the run:
//                                                 K's operand fragments in registers, V in
//                                                 LDS, and with d = 64 V's in registers too)
//                   P   = 2^(S c - LSE log2 e), 0 where masked  (c = scale log2 e)
//                   dS  = P (dP - D)
//                   dV^T += dO^T P,  dK^T += Q^T dS   (dO^T and Q^T by LDS transpose reads)
//               Because the group's query heads loop inside the workgroup, dK and dV are
//               summed over the group without atomics.
//  3. bwd_dq:   dQ, per query tile, recomputing S and dP (see below); no atomics.
//
// Both bwd_dq and bwd_main keep every tile of one (batch, KV head) group on one XCD when
// the group count allows, and large launches of short sequences run in chunks of groups
// (dispatch_chunk in attn_kernels.h) so that the re-read K/V (dQ) and Q/dO (dK/dV) of the
// resident workgroups fit the memory-side cache.
//
// Packed batches (VARLEN, attn_bwd_varlen): the same kernels with per-sequence lengths
// from cu_seqlens and token-major rows for the caller's tensors; the workspace keeps the
// dense layout of B sequences of S rows (S the longest), and the grids run in chunks of 8
// (sequence, KV head) groups, one per XCD (varlen_chunk_groups).  Workgroups whose tile
// lies past their sequence's end return at once.
//
// In the S accumulator layout of bwd_main (v_mfma_f32_32x32x16_f16, A = Q rows, B = K^T,
// all four products on fp16 operands scaled by powers of two, see below) a lane holds one
// key column and 16 query rows; P and dS are packed to fp16 in registers and used directly
// as the B operand of the dV^T and dK^T products.
#include <type_traits>

#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

constexpr int kBwdBN = 128;  // keys per workgroup (4 waves x 32)
constexpr int kBwdBM = 64;   // queries per step

// ------------------------------------------------------------------ preprocess
// Rows are taken in the padded layout [B*Hq][S_pad] (S_pad = S rounded up to a multiple
// of the 64-query step): -D_i = -<dO_i, O_i> and LSE_i log2(e) go to the workspace there and
// padding rows get 0.  The dQ kernel reads one of each per lane and starts its dP
// products from -D, so dS = P (dP - D) is one multiply.
//
// The launch is kPreBlocks workgroups per KV group (b, hkv): workgroup nb takes an equal
// share of the group's G * S_pad padded rows of O, dO and Q and of its S rows of K and V,
// and writes the largest |dO|, |V|, |Q| and |K| it saw to pmax[group][nb][0..3] (no
// atomics, so nothing needs clearing beforehand).  The later kernels reduce those to the
// power-of-two scales that put the group's operands into fp16 exactly (fp16_exponent).
constexpr int kMaxDO = 0, kMaxV = 1, kMaxQ = 2, kMaxK = 3, kMaxes = 4;

__device__ __forceinline__ float absmax8(float m, const u32x4& w) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    m = fmaxf(m, fmaxf(fabsf(__builtin_bit_cast(float, w[e] << 16)), fabsf(__builtin_bit_cast(float, w[e] & 0xffff0000u))));
  return m;
}

template <int D, bool VARLEN>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a, int S_pad) {
  constexpr int LPR = D / 8;     // lanes per row, 8 bf16 each
  constexpr int RPI = 256 / LPR;  // rows per pass of the workgroup
  const int tid = threadIdx.x;
  const int part = tid % LPR;
  const int G = a.Hq / a.Hkv;
  const int grp = blockIdx.x / kPreBlocks;  // b * Hkv + hkv
  const int nb = blockIdx.x - grp * kPreBlocks;
  const int b = grp / a.Hkv;
  const int hkv = grp - b * a.Hkv;
  // This sequence's rows: S of them; row i of query head h of O, dO, Q at element
  // qbase + i rs_q + h D, of LSE at lse[lbase + h ls_h + i], row i of K and V at
  // kvb + i rs_kv.  (a.S is the rows of a (batch, head) in the workspace's layout.)
  int S;
  size_t qbase, kvb, lbase, ls_h;
  int rs_q = D, rs_kv = D;
  size_t wrow0 = 0, wstride = S_pad;  // workspace row of (this group's first head, row 0); rows per head
  if constexpr (VARLEN) {
    const int start = min(max(a.cu_seqlens[b], 0), a.total);
    const int end = min(max(a.cu_seqlens[b + 1], start), a.total);
    S = min(end - start, a.S);
    rs_q = a.Hq * D;
    rs_kv = a.Hkv * D;
    qbase = (size_t)start * rs_q;
    kvb = (size_t)start * rs_kv + (size_t)hkv * D;
    lbase = start;
    ls_h = a.total;
    wstride = varlen_ws_rows(a.B, a.total);
    wrow0 = (size_t)hkv * G * wstride + varlen_ws_start(b, start);
  } else {
    S = a.S;
    qbase = (size_t)b * a.Hq * S * D;
    kvb = (size_t)grp * S * D;
    lbase = (size_t)b * a.Hq * S;
    ls_h = S;
  }

  // O, dO, Q: the group's padded rows [row0, row0 + G * S_pad), this workgroup's share.
  // Packed batches take only the sequence's own rows rounded up to 64 (what the later
  // kernels read), token by token with the G heads of a token adjacent as they are in
  // memory, so that the group's workgroups share real rows; dense batches head by head.
  const long row0 = ((long)b * a.Hq + (long)hkv * G) * S_pad;
  const long nrows = (long)G * (VARLEN ? (S + kBwdBM - 1) / kBwdBM * kBwdBM : S_pad);
  const long per = ((nrows + kPreBlocks - 1) / kPreBlocks + RPI - 1) / RPI * RPI;
  const long r_end = min(nrows, (nb + 1) * per);
  float mdo = 0.0f, mq = 0.0f;
  // Two rows per thread and pass, their loads issued together.
  for (long r0 = nb * per; r0 < r_end; r0 += 2 * RPI) {
    long row[2], wi[2];
    bool real[2];
    u32x4 ov[2], dv[2], qv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const long r = r0 + u * RPI + tid / LPR;  // group-relative padded row
      int hl, srow;
      if constexpr (VARLEN) {
        srow = (int)(r / G);
        hl = (int)(r - (long)srow * G);
      } else {
        hl = (int)(r / S_pad);
        srow = (int)(r - (long)hl * S_pad);
      }
      wi[u] = VARLEN ? (long)(wrow0 + (size_t)hl * wstride) + srow : row0 + r;  // workspace row
      real[u] = r < r_end && srow < S;
      const int h = hkv * G + hl;  // query head
      row[u] = real[u] ? (long)(lbase + (size_t)h * ls_h) + srow : 0;  // LSE index of the row
      const size_t e = VARLEN ? qbase + (size_t)srow * rs_q + (size_t)h * D : (size_t)row[u] * D;
      if (real[u]) {
        ov[u] = *(const u32x4*)(a.o + e + part * 8);
        dv[u] = *(const u32x4*)(a.dO + e + part * 8);
        qv[u] = *(const u32x4*)(a.q + e + part * 8);
      } else {
        ov[u] = dv[u] = qv[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const long r = r0 + u * RPI + tid / LPR;
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float o0 = __builtin_bit_cast(float, ov[u][e] << 16), o1 = __builtin_bit_cast(float, ov[u][e] & 0xffff0000u);
        const float d0 = __builtin_bit_cast(float, dv[u][e] << 16), d1 = __builtin_bit_cast(float, dv[u][e] & 0xffff0000u);
        acc = fmaf(o0, d0, acc);
        acc = fmaf(o1, d1, acc);
      }
      mdo = absmax8(mdo, dv[u]);
      mq = absmax8(mq, qv[u]);
#pragma unroll
      for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
      if (r < r_end && part == 0) {
        a.delta[wi[u]] = -acc;  // -D: the dQ kernel's dP products start from it
        a.lse2[wi[u]] = real[u] ? a.lse[row[u]] * kLog2e : 0.0f;
      }
    }
  }
  // K, V: the group's S rows, this workgroup's share.
  const long vper = (((long)S + kPreBlocks - 1) / kPreBlocks + RPI - 1) / RPI * RPI;
  const long v_end = min((long)S, (nb + 1) * vper);
  float mv = 0.0f, mk = 0.0f;
  for (long r = nb * vper + tid / LPR; r < v_end; r += RPI) {
    mv = absmax8(mv, *(const u32x4*)(a.v + kvb + r * rs_kv + part * 8));
    mk = absmax8(mk, *(const u32x4*)(a.k + kvb + r * rs_kv + part * 8));
  }
  // Workgroup maxima: within each wave, then across the 4 waves through LDS.
  float m[kMaxes];
  m[kMaxDO] = mdo;
  m[kMaxV] = mv;
  m[kMaxQ] = mq;
  m[kMaxK] = mk;
  __shared__ float red[4][kMaxes];
#pragma unroll
  for (int i = 0; i < kMaxes; ++i) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m[i] = fmaxf(m[i], __shfl_xor(m[i], off));
    if ((tid & 63) == 0) red[tid >> 6][i] = m[i];
  }
  __syncthreads();
  if (tid < kMaxes) {
    const float x = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
    a.pmax[((size_t)grp * kPreBlocks + nb) * kMaxes + tid] = x;
  }
}

// Power of two 2^e that brings a group's largest magnitude mx into [2^(top-1), 2^top):
// every bf16 value x of the group then has x 2^e exactly representable in fp16 (top <= 15),
// unless |x| < 2^(-16-top) mx: its scaled value then lies below 2^-17, where fp16's
// subnormal spacing 2^-24 no longer holds bf16's 8 significant bits (the rounding error
// there is at most 2^-25, below 2^(-24-top) mx after unscaling).  0 for an all-zero group
// and for inf or NaN (the results are then inf or NaN anyway); at most 60 either way.
__device__ __forceinline__ int fp16_exponent(float mx, int top) {
  if (!(mx > 0.0f) || !(mx < INFINITY)) return 0;
  int e;
  (void)frexpf(mx, &e);  // mx = f 2^e, f in [1/2, 1)
  return min(max(top - e, -60), 60);
}

// Scale exponents of a group's fp16 operands.  dO and V are brought under 2^3, so that in
// the dK/dV kernel |dP| <= d 2^6 and |dS| = P |dP - D| <= 2 d 2^6 <= 2^14 stay within fp16
// (D is a P-weighted mean of dP); Q and K use fp16's whole range (their products are only
// accumulated in fp32).
struct GroupScales {
  int e_do, e_v, e_q, e_k;
};

// The reduction runs over the wave, so the result is the same in every lane (and is moved
// to scalar registers).
__device__ __forceinline__ GroupScales group_scales(const float* __restrict__ pmax, int grp) {
  const int lane = threadIdx.x & 63;
  float m[kMaxes];
#pragma unroll
  for (int i = 0; i < kMaxes; ++i) {
    m[i] = lane < kPreBlocks ? pmax[((size_t)grp * kPreBlocks + lane) * kMaxes + i] : 0.0f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m[i] = fmaxf(m[i], __shfl_xor(m[i], off));
  }
  GroupScales g;
  g.e_do = __builtin_amdgcn_readfirstlane(fp16_exponent(m[kMaxDO], 3));
  g.e_v = __builtin_amdgcn_readfirstlane(fp16_exponent(m[kMaxV], 3));
  g.e_q = __builtin_amdgcn_readfirstlane(fp16_exponent(m[kMaxQ], 15));
  g.e_k = __builtin_amdgcn_readfirstlane(fp16_exponent(m[kMaxK], 15));
  return g;
}

// Two floats (exact in fp16, or rounded to nearest even) packed as an fp16 pair.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 r;
  r[0] = (_Float16)lo;
  r[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// Eight bf16 (one 16-byte chunk) times 2^e (sc) as eight fp16.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 w, float sc) {
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    r[e] = pack_f16x2(__builtin_bit_cast(float, w[e] << 16) * sc, __builtin_bit_cast(float, w[e] & 0xffff0000u) * sc);
  return r;
}

// ------------------------------------------------------------------ main

// A workgroup owns a tile of 128 keys; wave w owns key block kq = w % 4 (32 keys).  Two
// shapes (NW waves, two waves per SIMD either way):
//  * NW = 8, one workgroup per CU: each step covers 64 queries, and wave w takes query half
//    qh = w / 4 of it, so waves w and w + 4 accumulate partial dK and dV for the same keys
//    over different queries; the two partials are added through LDS at the end.
//  * NW = 4, two workgroups per CU: each step covers 32 queries, every wave all of them, and
//    no partials need adding.  V's tile takes K's place in LDS once each wave holds its K
//    fragments, so the workgroup needs 64.5 KiB (d = 128) and two fit on a CU: one's K/V
//    load and closing stores overlap the other's steps.  That pays on short walks (each
//    workgroup's fixed cost is spread over few steps); on long ones the eight-wave shape,
//    with half the barriers per product, is faster (the launcher chooses).
//
// K, V (resident; each wave also holds its operand fragments of K, and with d = 64 of V,
// in registers) and the Q, dO stages sit in LDS as XOR chunk-inner blocks (see
// attn_device.h): MFMA-operand reads of 16 rows at one chunk and the transpose reads of
// dO^T and Q^T are both free of bank conflicts, every lane keeps a few base addresses
// and the rest are immediate offsets, and each 4 DMA lanes fetch one 64-byte piece of a
// row.  One step is 32 fenced slots of one product each, in four phases:
//   S  = Q K^T                       (8 products)
//   dP = dO V^T   beside P = 2^(S c - LSE log2 e), computed in place of S
//   dV^T += dO^T P   beside dS = P (dP - D), computed in place of dP
//   dK^T += Q^T dS
// so the vector work of each phase runs next to matrix products that do not need it;
// LDS reads run two slots ahead of their products.
template <int D, bool CAUSAL, int EXPMODE, int NW, bool VARLEN>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2, 2)))
void bwd_main_kernel(BwdArgs a) {
  static_assert(NW == 4 || NW == 8, "4 or 8 waves per workgroup");
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int CG = D / 32;                   // 4-chunk groups per row
  constexpr int ROWB = D * 2;                  // bytes per row of the fp16 Q and dO copies
  constexpr int BM = 32 * (NW / 4);            // queries per step
  constexpr int NT = 64 * NW;                  // threads
  constexpr int KT = kBwdBN * D;               // elements of the K (or V) tile
  constexpr int QT = BM * D;                   // elements of one Q (or dO) tile
  constexpr int KDMAS = kBwdBN / 16 * CG / NW; // 1024-byte blocks per wave, K or V tile
  constexpr int QDMAS = BM / 16 * CG / NW;     // 1024-byte blocks per wave, Q or dO tile
  constexpr int PD = 2;                        // slots between an LDS read and its product
  constexpr int NS = 4 * KSTEPS;               // slots per step (== 4 * 2 * DBLK)
  static_assert(KSTEPS == 2 * DBLK && KDMAS * NW * 16 == kBwdBN * CG && QDMAS * NW * 16 == BM * CG, "tiling");
  // The wave's operand fragments of K (S products) and, with d = 64, of V (dP products)
  // stay in registers for the whole run: they are read from LDS once, after the fp16
  // conversion, instead of once per step.  With d = 64 that is 32 registers and a third of
  // the kernel's LDS reads (the kernel runs 5-8% faster); with d = 128, K's 32 registers
  // are what the two-waves-per-SIMD budget has left (a sixth of the LDS reads, 2.5-4.5%
  // faster), and the cubic exponential's few extra registers leave no room for them.
  constexpr int NKV = D == 64 ? 2 * KSTEPS : (EXPMODE == 0 ? KSTEPS : 0);  // fragments held
  // With K in registers, K's LDS tile is only needed until its fragments are loaded, and V
  // then takes its place: the four-wave workgroup's LDS (one K/V tile, two Q/dO stages of
  // 32 queries, LSE and D: 64.5 KiB at d = 128) lets two workgroups share a CU.
  constexpr bool SHARED_KV = NW == 4;
  static_assert(!SHARED_KV || NKV >= KSTEPS, "V can only replace K when K's fragments are in registers");
  // One LDS buffer, [K | V | Q stage 0 | Q stage 1 | dO stage 0 | dO stage 1 | LSE, D]
  // (K and V in one tile when SHARED_KV): every operand read reaches its tile from a
  // lane's base register by an immediate offset below 64 KiB (K and V from the K base; the
  // four stages from the Q base).
  constexpr int K_OFF = 0, V_OFF = SHARED_KV ? 0 : 2 * KT, Q_OFF = V_OFF + 2 * KT, DO_OFF = Q_OFF + 4 * QT,
                SD_OFF = DO_OFF + 4 * QT;
  static_assert(V_OFF + 2 * KT - K_OFF <= 65536 && SD_OFF - Q_OFF <= 65536, "immediate LDS offsets");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SD_OFF + 2 * 2 * BM * 4];
  uint16_t* const k_lds = (uint16_t*)(smem + K_OFF);
  uint16_t* const v_lds = (uint16_t*)(smem + V_OFF);
  uint16_t* const q_lds[2] = {(uint16_t*)(smem + Q_OFF), (uint16_t*)(smem + Q_OFF + 2 * QT)};
  uint16_t* const do_lds[2] = {(uint16_t*)(smem + DO_OFF), (uint16_t*)(smem + DO_OFF + 2 * QT)};
  float (*const sd_lds)[2 * BM] = (float (*)[2 * BM])(smem + SD_OFF);  // [stage][LSE log2e | D]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kq = wave & 3;                  // key block of this wave
  const int qh = NW == 8 ? wave >> 2 : 0;   // query half of each step (NW = 8)
  const int col = lane & 31;
  const int half = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int G = a.Hq / a.Hkv;

  // Dispatch order: chunks of kv_chunk KV groups one after the other (dispatch_chunk);
  // within a chunk, key tile by key tile, the lowest key index first (it has the most
  // query tiles under the causal mask).  With the chunk's group count a multiple of 8,
  // all key tiles of one group run on one XCD (XCD = block index % 8) and share its L2
  // for the group's Q and dO.
  const int ngrp = a.B * a.Hkv;
  const int nkt = (a.S + kBwdBN - 1) / kBwdBN;
  const int per_chunk = a.kv_chunk * nkt;
  const int chunk = (int)blockIdx.x / per_chunk;
  const int pos = (int)blockIdx.x - chunk * per_chunk;
  const int ncg = min(a.kv_chunk, ngrp - chunk * a.kv_chunk);  // groups in this chunk
  const int kt = pos / ncg;
  const int bh = chunk * a.kv_chunk + (pos - kt * ncg);
  const int b = bh / a.Hkv;
  const int hkv = bh - b * a.Hkv;
  const int k0 = kt * kBwdBN;
  const int kw = k0 + kq * 32;
  const int key = kw + col;  // this lane's key (column of S)
  // This sequence's rows: S of them; row i of K, V, dK, dV at element kvbase + i rs_kv
  // (kvbase includes the head).  a.S is the rows of a (batch, head) in the workspace's
  // dense layout (the fp16 Q and dO copies, LSE and D): with VARLEN the longest sequence.
  int S;
  size_t kvbase;
  int rs_kv = D;
  size_t wq0 = 0, wstride = 0;  // packed: workspace row of (query head 0, row 0), rows per head
  if constexpr (VARLEN) {
    const int start = min(max(a.cu_seqlens[b], 0), a.total);
    const int end = min(max(a.cu_seqlens[b + 1], start), a.total);
    S = min(end - start, a.S);
    if (k0 >= S) return;  // the whole workgroup: this key tile lies past its sequence
    rs_kv = a.Hkv * D;
    kvbase = (size_t)start * rs_kv + (size_t)hkv * D;
    wstride = varlen_ws_rows(a.B, a.total);
    wq0 = varlen_ws_start(b, start);
  } else {
    S = a.S;
    kvbase = ((size_t)b * a.Hkv + hkv) * (size_t)S * D;
  }

  // DMA: wave w fills blocks i * NW + w of a tile; block bl holds rows 16 (bl / CG) ..,
  // chunks 4 (bl % CG) ..; lane l fetches row l / 4 of it, chunk (l % 4) ^ ((l / 16) % 4).
  const int dl_r = lane >> 2, dl_c = (lane & 3) ^ ((lane >> 4) & 3);
  // K and V tiles -> LDS (rows past the end are clamped to a real row; their
  // probabilities are masked to 0).  With SHARED_KV, V follows once K's fragments are in
  // registers.
  auto dma_kv = [&](const uint16_t* __restrict__ src_t, uint16_t* dst) {
#pragma unroll
    for (int i = 0; i < KDMAS; ++i) {
      const int bl = i * NW + wave;
      const int r = (bl / CG) * 16 + dl_r;
      const size_t src = kvbase + (size_t)min(k0 + r, S - 1) * rs_kv + ((bl % CG) * 4 + dl_c) * 8;
      dma16(src_t + src, dst + (i * NW + wave_u) * 512);
    }
  };
  dma_kv(a.k, k_lds);
  if constexpr (!SHARED_KV) dma_kv(a.v, v_lds);

  const int nqt = (S + BM - 1) / BM;
  const int q_first = CAUSAL ? (k0 / BM) : 0;
  const int per_head = nqt - q_first;
  const int steps = G * per_head;
  const int S_pad = (a.S + kBwdBM - 1) / kBwdBM * kBwdBM;

  // Per-lane byte offsets of the Q / dO DMA within a tile.
  uint32_t qd_off[QDMAS];
#pragma unroll
  for (int i = 0; i < QDMAS; ++i) {
    const int bl = i * NW + wave;
    qd_off[i] = (uint32_t)(((bl / CG) * 16 + dl_r) * ROWB + ((bl % CG) * 4 + dl_c) * 16);
  }
  // Step order: query tiles from the last one down, the group's heads innermost, so the
  // workgroups of one (batch, KV head), which share an XCD when B*Hkv is a multiple of
  // 8, read the same Q/dO rows at about the same time.  Steps are staged in order, so the
  // (head, query tile) of the next one is a pair of counters rather than a division per
  // step (scalar work that every wave of the CU repeats right after the barrier).
  int stage_g = 0, stage_qt = nqt - 1;
  auto stage_in = [&](int st) {
    const int g = stage_g;
    const int qt = stage_qt;
    if (++stage_g == G) {
      stage_g = 0;
      --stage_qt;
    }
    const int hq = hkv * G + g;
    const size_t rbase = VARLEN ? hq * wstride + wq0 : ((size_t)b * a.Hq + hq) * (size_t)a.S;
    const int q0 = qt * BM;
    const char* qb = (const char*)(a.q16 + (rbase + q0) * D);
    const char* ob = (const char*)(a.do16 + (rbase + q0) * D);
    if (q0 + BM <= S) {
#pragma unroll
      for (int i = 0; i < QDMAS; ++i) {
        dma16_s(qb, qd_off[i], q_lds[st] + (i * NW + wave_u) * 512);
        dma16_s(ob, qd_off[i], do_lds[st] + (i * NW + wave_u) * 512);
      }
    } else {
      int lr = dl_r;
      __asm__ volatile("" : "+v"(lr));  // keep this rare path's row arithmetic inside it
#pragma unroll
      for (int i = 0; i < QDMAS; ++i) {
        const int row = ((i * NW + wave) / CG) * 16 + lr;  // row within the tile
        const int rc = min(q0 + row, S - 1) - q0;
        const uint32_t off = qd_off[i] + (uint32_t)((rc - row) * ROWB);
        dma16_s(qb, off, q_lds[st] + (i * NW + wave_u) * 512);
        dma16_s(ob, off, do_lds[st] + (i * NW + wave_u) * 512);
      }
    }
    // LSE log2e (wave 0) and D (wave 1) of the BM queries: BM / 4 lanes x 16 bytes each.
    if (wave_u < 2) {
      const size_t pbase = (VARLEN ? hq * wstride + wq0 : ((size_t)b * a.Hq + hq) * (size_t)S_pad) + q0;
      const void* src = uniform_ptr((wave_u == 0 ? a.lse2 : a.ndx) + pbase);
      if (lane < BM / 4) dma16_s(src, (uint32_t)lane * 16u, &sd_lds[st][wave_u * BM]);
    }
  };

  // Per-lane LDS byte offsets.  Operand reads (16 rows at one chunk): chunk ks*2 + half,
  // one register per parity of ks, the rest by (ks / 2) * 1024.
  const int ra0 = opaque(Q_OFF + blk_chunk_inner_x<D>(qh * 32 + col, half));
  const int ra1 = opaque(Q_OFF + blk_chunk_inner_x<D>(qh * 32 + col, 2 + half));
  const int rb0 = opaque(K_OFF + blk_chunk_inner_x<D>(kq * 32 + col, half));
  const int rb1 = opaque(K_OFF + blk_chunk_inner_x<D>(kq * 32 + col, 2 + half));
  // Transpose reads of dO^T and Q^T: source lane s reads 4 d-values of query row
  // qh*32 + t*16 + (s / 32) * 4 + (s % 16) / 4 (+ 8 for the second read) at column
  // 16 * ((s / 16) % 2) + 4 * (s % 4) of d block db; the rest by (t * CG + db) * 1024.
  const int trow = (lane >> 5) * 4 + ((lane >> 2) & 3);
  const int tcl = ((lane >> 4) & 1) * 2 + ((lane >> 1) & 1);
  const int tq = Q_OFF + (2 * qh * CG) * 1024 + (lane & 1) * 8;
  const int tr0 = opaque(tq + (trow * 4 + (tcl ^ ((trow >> 2) & 3))) * 16);
  const int tr1 = opaque(tq + ((trow + 8) * 4 + (tcl ^ (((trow + 8) >> 2) & 3))) * 16);
  // LSE log2e and -D of the lane's query rows: one base (the area lies past the 16-bit
  // immediate range of the other bases), every stage and row group by an immediate offset.
  const int sdb = opaque(SD_OFF + (qh * 32 + half * 4) * 4);

  f32x16 dk_acc[DBLK], dv_acc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
    dk_acc[db] = f32x16{};
    dv_acc[db] = f32x16{};
  }
  // The group's fp16 scales (see the conversion before the step loop).  S is computed from
  // Q 2^e_q and K 2^e_k, so c carries 2^-(e_q + e_k); c is signed: no running maximum is
  // needed here.
  const GroupScales gs = group_scales(a.pmax, bh);
  const float c = ldexpf(a.scale * kLog2e, -(gs.e_q + gs.e_k));

  bf16x8 kvf[NKV > 0 ? NKV : 1];
  // One step on stage ST; MASKED adds the causal / end-of-sequence mask to P.
  auto compute = [&](const int q0, auto stage, auto masked) {
    constexpr int ST = decltype(stage)::value;
    constexpr bool MASKED = decltype(masked)::value;
    // Tile offsets from the lane bases (ra*, tr* hold Q stage 0; rb* hold K).
    constexpr int QS = ST * 2 * QT, OS = DO_OFF - Q_OFF + ST * 2 * QT, VS = V_OFF - K_OFF;
    const char* L = (const char*)smem;
    // Mask (MASKED only): register v holds query qb + e_v, e_v = (v/4)*8 + v%4, with
    // qb = q0 + qh*32 + half*4; P = 0 where e_v < lim_c (key > query) or e_v >= lim_s
    // (query past the end), and everywhere if the key is past the end.
    int lim_c = -1, lim_s = 64;
    if constexpr (MASKED) {
      const int qb = q0 + qh * 32 + half * 4;
      lim_s = S - qb;
      lim_c = key >= S ? 64 : (CAUSAL ? key - qb : -1);
    }

    bf16x8 fa[NS], fb[NS];  // operand fragments of phase A/B slots
    i16x4 tlo[NS], thi[NS];   // transpose-read halves of phase C/D slots
    f32x4 l4[4], d4[4];       // LSE log2e and D of this lane's 16 query rows
    // The slot that computes P of register v: registers [j 16 / n, (j + 1) 16 / n) in slot
    // KSTEPS + 2 + j, n = KSTEPS - 2 (two slots after the last S product).
    auto p_slot = [](const int v) {
      int j = 0;
      while ((j + 1) * 16 / (KSTEPS - 2) <= v) ++j;
      return KSTEPS + 2 + j;
    };
    auto issue = [&](const int i) {
      if (i < 2 * KSTEPS) {
        const int ks = i % KSTEPS;
        const int o = (ks >> 1) * 1024;
        const int ao = (i < KSTEPS ? QS : OS) + o, bo = (i < KSTEPS ? 0 : VS) + o;
        fa[i] = *(const bf16x8*)(L + ((ks & 1) ? ra1 : ra0) + ao);
        if (i < NKV) {
          fb[i] = kvf[i];
        } else {
          fb[i] = *(const bf16x8*)(L + ((ks & 1) ? rb1 : rb0) + bo);
        }
      } else if (i < NS) {
        const int p = (i - 2 * KSTEPS) % (2 * DBLK), t = p / DBLK, db = p % DBLK;
        const int o = (i < 3 * KSTEPS ? OS : QS) + (t * CG + db) * 1024;
        tlo[i] = lds_read_tr16((const uint16_t*)(L + tr0 + o));
        thi[i] = lds_read_tr16((const uint16_t*)(L + tr1 + o));
      }
      // LSE log2e of the rows of registers 4 g4 .. 4 g4 + 3, two slots before the first
      // slot whose share of the P computation (below) needs them: loaded late, so that the
      // 16 registers are not held through the S products.
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        if (i == p_slot(4 * g4)) l4[g4] = *(const f32x4*)(L + sdb + ST * BM * 8 + g4 * 32);
      // -D of the lane's 16 query rows, in the accumulator's register order: the first dP
      // product takes it as its accumulator input, so the chain ends at dP - D.
      if (i >= KSTEPS - 4 && i < KSTEPS) {
        const int g4 = i - (KSTEPS - 4);
        d4[g4] = *(const f32x4*)(L + sdb + ST * BM * 8 + BM * 4 + g4 * 32);
      }
    };

    f32x16 sacc = f32x16{}, dpacc;
    uint32_t pw[2][4], sw[2][4];  // P and dS packed to fp16 pairs: [t][pair], registers v = 8t ..
#pragma unroll
    for (int i = 0; i < PD; ++i) issue(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      issue(i + PD);
      if (i < KSTEPS) {
        sacc = mfma32_f16(fa[i], fb[i], sacc);
      } else if (i < 2 * KSTEPS) {
        if (i == KSTEPS) {
          const f32x16 nd = {d4[0][0], d4[0][1], d4[0][2], d4[0][3], d4[1][0], d4[1][1], d4[1][2], d4[1][3],
                             d4[2][0], d4[2][1], d4[2][2], d4[2][3], d4[3][0], d4[3][1], d4[3][2], d4[3][3]};
          dpacc = mfma32_f16(fa[i], fb[i], nd);
        } else {
          dpacc = mfma32_f16(fa[i], fb[i], dpacc);
        }
        // P for a share of the 16 registers, once S has had two slots to finish.
        const int j = i - KSTEPS - 2;
        if (j >= 0) {
          const int n = KSTEPS - 2, e0 = j * 16 / n, e1 = (j + 1) * 16 / n;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            if (v < e0 || v >= e1) continue;
            float p = exp2_sm<EXPMODE>(fmaf(sacc[v], c, -l4[v >> 2][v & 3]));
            if constexpr (MASKED) {
              const int ev = (v >> 2) * 8 + (v & 3);
              p = (ev < lim_c || ev >= lim_s) ? 0.0f : p;
            }
            sacc[v] = p;
            if (v & 1) pw[v >> 3][(v & 7) >> 1] = pack_f16x2(sacc[v - 1], p);
          }
        }
      } else if (i < 3 * KSTEPS) {
        const int p = i - 2 * KSTEPS, t = p / DBLK, db = p % DBLK;
        const u32x4 w = {pw[t][0], pw[t][1], pw[t][2], pw[t][3]};
        dv_acc[db] = mfma32_f16(join(tlo[i], thi[i]), __builtin_bit_cast(bf16x8, w), dv_acc[db]);
        // dS for a share of the 16 registers, once dP has had two slots to finish.
        const int j = p - 2;
        if (j >= 0) {
          const int n = 2 * DBLK - 2, e0 = j * 16 / n, e1 = (j + 1) * 16 / n;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            if (v < e0 || v >= e1) continue;
            const float ds = sacc[v] * dpacc[v];
            dpacc[v] = ds;
            if (v & 1) sw[v >> 3][(v & 7) >> 1] = pack_f16x2(dpacc[v - 1], ds);
          }
        }
      } else {
        const int p = i - 3 * KSTEPS, t = p / DBLK, db = p % DBLK;
        const u32x4 w = {sw[t][0], sw[t][1], sw[t][2], sw[t][3]};
        dk_acc[db] = mfma32_f16(join(tlo[i], thi[i]), __builtin_bit_cast(bf16x8, w), dk_acc[db]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  int step_g = 0, step_qt = nqt - 1;  // query tile of the step being computed, as above
  auto do_step = [&](const int step, auto stage) {
    constexpr int ST = decltype(stage)::value;
    wait_dma();
    __syncthreads();  // this step's Q, dO, LSE, D are in LDS; every wave is done with the previous stage
    if (step + 1 < steps) stage_in(ST ^ 1);
    const int qt = step_qt;
    if (++step_g == G) {
      step_g = 0;
      --step_qt;
    }
    const int q0 = qt * BM;
    const int qs = q0 + qh * 32;  // first query of this wave's half
    if (!CAUSAL || kw <= qs + 31) {
      const bool need_mask = (kw + 32 > S) || (qs + 32 > S) || (CAUSAL && kw + 31 > qs);
      if (need_mask) {
        compute(q0, stage, std::true_type{});
      } else {
        compute(q0, stage, std::false_type{});
      }
    }
  };

  if (steps > 0) stage_in(0);
  // K and V into fp16 in place, times 2^e_k and 2^e_v (exact, see fp16_exponent).  Every
  // product runs in fp16, on Q 2^e_q and dO 2^e_do staged from the dQ kernel's copies: S
  // carries 2^(e_q + e_k) (taken out through c), dP, -D and dS 2^(e_do + e_v), dV 2^e_do
  // and dK 2^(e_q + e_do + e_v); the last two are taken out at the end.
  // A tile of bf16 into fp16 in place, times 2^e.
  auto to_f16 = [&](uint16_t* t, int e) {
    const float sc = ldexpf(1.0f, e);
    u32x4* tt = (u32x4*)t;
#pragma unroll
    for (int i = 0; i < KT / 8 / NT; ++i) tt[i * NT + tid] = bf16x8_to_f16x8(tt[i * NT + tid], sc);
  };
  // Fragments i0 .. i1 - 1 of kvf (K's, then V's) from the converted tiles.
  auto load_frags = [&](const int i0, const int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const int ks = i % KSTEPS;
      const int bo = (i < KSTEPS ? 0 : V_OFF - K_OFF) + (ks >> 1) * 1024;
      kvf[i] = *(const bf16x8*)((const char*)smem + ((ks & 1) ? rb1 : rb0) + bo);
    }
  };
  wait_dma();
  __syncthreads();  // K (and V) are in LDS
  to_f16(k_lds, gs.e_k);
  if constexpr (SHARED_KV) {
    __syncthreads();  // the converted K is in LDS
    load_frags(0, KSTEPS);
    __syncthreads();  // every wave holds its K fragments: V takes K's place
    dma_kv(a.v, v_lds);
    wait_dma();
    __syncthreads();  // V is in LDS
    to_f16(v_lds, gs.e_v);
    if constexpr (NKV > KSTEPS) {
      __syncthreads();  // the converted V is in LDS
      load_frags(KSTEPS, NKV);
    }
  } else {
    to_f16(v_lds, gs.e_v);
    if constexpr (NKV > 0) {
      __syncthreads();  // the converted K and V are in LDS
      load_frags(0, NKV);
    }
  }
  // (the first step's barrier orders the conversion's writes before any other read of V)
  for (int step = 0; step < steps; step += 2) {
    do_step(step, std::integral_constant<int, 0>{});
    if (step + 1 < steps) do_step(step + 1, std::integral_constant<int, 1>{});
  }

  // With NW = 8, add the two query halves' partial dK, dV through LDS (the Q/dO stages
  // are free now); then dK = scale dK_acc, dV = dV_acc.
  if constexpr (NW == 8) {
  float* red = reinterpret_cast<float*>(smem + Q_OFF);  // 4 waves x DBLK x 16 x 64 floats
  static_assert(NW != 8 || SD_OFF - Q_OFF >= 4 * DBLK * 16 * 64 * (int)sizeof(float), "reduction space");
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    f32x16* acc = pass == 0 ? dv_acc : dk_acc;
    if (qh == 1) {
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
#pragma unroll
        for (int v = 0; v < 16; ++v) red[((kq * DBLK + db) * 16 + v) * 64 + lane] = acc[db][v];
      }
    }
    __syncthreads();
    if (qh == 0) {
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] += red[((kq * DBLK + db) * 16 + v) * 64 + lane];
      }
    }
    __syncthreads();
  }
  }
  if (qh == 0 && key < S) {
    // dK = scale 2^-(e_do + e_v) (2^-e_q acc), in two factors that each stay in range.
    const float kq = ldexpf(1.0f, -gs.e_q);
    const float ks = ldexpf(a.scale, -(gs.e_do + gs.e_v));
    const float vs = ldexpf(1.0f, -gs.e_do);
    // The lane's half, recomputed here rather than kept live across the loop.
    const int half = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) >> 5;
    uint16_t* dkr = a.dk + kvbase + (size_t)key * rs_kv;
    uint16_t* dvr = a.dv + kvbase + (size_t)key * rs_kv;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        u32x2 wk, wv;
        wk[0] = pack_bf16x2(dk_acc[db][g4 * 4 + 0] * kq * ks, dk_acc[db][g4 * 4 + 1] * kq * ks);
        wk[1] = pack_bf16x2(dk_acc[db][g4 * 4 + 2] * kq * ks, dk_acc[db][g4 * 4 + 3] * kq * ks);
        wv[0] = pack_bf16x2(dv_acc[db][g4 * 4 + 0] * vs, dv_acc[db][g4 * 4 + 1] * vs);
        wv[1] = pack_bf16x2(dv_acc[db][g4 * 4 + 2] * vs, dv_acc[db][g4 * 4 + 3] * vs);
        *(u32x2*)(dkr + db * 32 + g4 * 8 + half * 4) = wk;
        *(u32x2*)(dvr + db * 32 + g4 * 8 + half * 4) = wv;
      }
    }
  }
}

// ------------------------------------------------------------------ dQ
// dQ without atomics: one workgroup of 4 waves owns 128 queries of one (batch, query
// head) and walks the key tiles (64 keys, staged in LDS by DMA, double-buffered) that its
// queries can see, like the forward.  Per tile, with one query per lane (the transposed
// score layout of the forward):
//     S^T  = K Q^T,   dP^T = V dO^T                 (Q^T, dO^T held in registers)
//     dS^T = P^T (dP^T - D),  P^T = 2^(S^T c - LSE log2 e)   (LSE and D: one value per lane)
//     dQ^T += K^T dS^T                              (K^T by LDS transpose reads)
// It recomputes S and dP (two of the backward's five products) instead of adding
// partial dQ blocks from every key tile with fp32 atomics, and it is deterministic.
//
// Two by-products for the dK/dV kernel, which runs after this one:
//  * the exact row term D_i = sum_j P_ij dP_ij.  The -D the dP chains start from comes
//    from the stored bf16 O (<dO_i, O_i>), so the dS row sums are D_i - D_i(bf16 O) (the
//    probabilities of a row sum to one); adding them gives D without O's rounding.  It is
//    stored negated and times 2^(e_dO + e_V) in the units of the dK/dV kernel's dP.
//  * dO and Q in fp16, each times its group's power of two (exact, see fp16_exponent),
//    from the fragments this kernel holds anyway: the dK/dV kernel's products run in
//    fp16, so that P enters dV^T += dO^T P, and dS enters dK^T += Q^T dS, with fp16's
//    11-bit significand instead of bf16's 8.
//
// K and V tiles sit in LDS as XOR chunk-inner blocks (attn_device.h), filled by coalesced
// DMA; both the operand reads of K and V and the transpose reads of K^T are free of bank
// conflicts.  One tile is 48 fenced slots of one product each: S^T (16), then dP^T
// beside P^T = 2^(S^T c - LSE log2 e) computed in place of S^T, then dQ^T beside
// dS^T = P^T (dP^T - D) computed in place of dP^T, one 8-key block ahead of the products
// that use it.  LDS reads run two slots ahead.
constexpr int kDqBM = 128;  // queries per workgroup
constexpr int kDqBN = 64;   // keys per tile

template <int D, bool CAUSAL, int EXPMODE, bool VARLEN>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdArgs a) {
  constexpr int BN = kDqBN;
  constexpr int KB = BN / 32;           // 32-key blocks per tile
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int CG = D / 32;            // 4-chunk groups per row
  constexpr int TILE = BN * D;          // elements of one K or V tile
  constexpr int DMAS = BN / 16 * CG / 4;  // 1024-byte blocks per wave per tile
  constexpr int NA = KSTEPS * KB;       // S^T slots
  constexpr int NC = 2 * KB * DBLK;     // dQ^T slots
  constexpr int NS = 2 * NA + NC;       // slots per tile
  constexpr int PD = 2;
  static_assert(DMAS * 4 * 16 == BN * CG && KB == 2, "tiling");
  __shared__ __attribute__((aligned(1024))) uint16_t smem[4 * TILE];  // K ring (2 tiles), V ring (2 tiles)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;
  const int half = lane >> 5;
  // a.S: rows of a (batch, head) in the workspace's dense layout, and the grid's; with
  // VARLEN the longest sequence, otherwise every sequence's length.
  const int S_pad = (a.S + kBwdBM - 1) / kBwdBM * kBwdBM;

  const int nqt = (a.S + kDqBM - 1) / kDqBM;
  const int bid = blockIdx.x;
  // Dispatch order and head of this workgroup, as in the forward: chunks of dq_chunk KV
  // groups (dispatch_chunk), within a chunk the longest query tiles first; with the
  // chunk's group count a multiple of 8, every query head and query tile of one KV group
  // lands on one XCD (XCD = bid % 8) and reads K and V through one L2.
  const int G = a.Hq / a.Hkv;
  const int ngrp = a.B * a.Hkv;
  const int per_chunk = a.dq_chunk * G * nqt;
  const int chunk = bid / per_chunk;
  const int pos = bid - chunk * per_chunk;
  const int g0 = chunk * a.dq_chunk;
  const int ncg = min(a.dq_chunk, ngrp - g0);  // KV groups in this chunk
  const int nbh = ncg * G;
  const int level = pos / nbh;
  const int qt = CAUSAL ? (nqt - 1 - level) : level;
  const int u = pos - level * nbh;
  int kvg, g;
  if ((ncg & 7) == 0) {
    const int jj = u >> 3;
    kvg = g0 + (jj / G) * 8 + (u & 7);
    g = jj - (jj / G) * G;
  } else {
    kvg = g0 + u / G;
    g = u - (u / G) * G;
  }
  const int b = kvg / a.Hkv;
  const int hkv = kvg - b * a.Hkv;
  const int hq = hkv * G + g;
  const int q0 = qt * kDqBM;
  // This sequence's rows: S of them; row i of head h of Q, dO, dQ (K, V) at element
  // qbase + i rs_q (kvbase + i rs_kv), where qbase and kvbase include the head.
  int S;
  size_t qbase, kvbase;
  int rs_q = D, rs_kv = D;
  // Workspace row of this (batch or sequence, head)'s row 0: in the row arrays (prow0) and
  // in the fp16 Q and dO copies (wrow0); and the rows a tile may write past S (ws_rows).
  size_t prow0, wrow0;
  int ws_rows;
  if constexpr (VARLEN) {
    const int start = min(max(a.cu_seqlens[b], 0), a.total);
    const int end = min(max(a.cu_seqlens[b + 1], start), a.total);
    S = min(end - start, a.S);
    if (q0 >= S) return;  // the whole workgroup: this tile lies past its sequence
    rs_q = a.Hq * D;
    rs_kv = a.Hkv * D;
    qbase = (size_t)start * rs_q + (size_t)hq * D;
    kvbase = (size_t)start * rs_kv + (size_t)hkv * D;
    prow0 = wrow0 = hq * varlen_ws_rows(a.B, a.total) + varlen_ws_start(b, start);
    ws_rows = (S + kBwdBM - 1) / kBwdBM * kBwdBM;  // the sequence's own rows, up to 64
  } else {
    S = a.S;
    qbase = ((size_t)b * a.Hq + hq) * (size_t)S * D;
    kvbase = ((size_t)b * a.Hkv + hkv) * (size_t)S * D;
    prow0 = ((size_t)b * a.Hq + hq) * (size_t)S_pad;
    wrow0 = ((size_t)b * a.Hq + hq) * (size_t)a.S;
    ws_rows = S_pad;
  }
  const int ROWB = rs_kv * 2;  // bytes between K/V rows in memory
  const size_t wbase = wrow0 * D;
  const int qw = q0 + wave * 32;
  const int qi = qw + col;  // this lane's query
  const int qc = min(qi, S - 1);  // rows past the end read the last row; never stored
  // Causal bound of the wave's first query.  The non-causal kernels use the same tests
  // against a bound past any sequence (kept opaque): with the tests folded away at compile
  // time the compiler's allocation for them exceeds the 256 registers and spills.
  const int qhi = CAUSAL ? qw : opaque(0x3fffffff);
  const uint16_t* __restrict__ Kg = a.k + kvbase;
  const uint16_t* __restrict__ Vg = a.v + kvbase;

  // DMA of a tile: wave w fills blocks 4 i + w; lane l fetches row l / 4 of the block,
  // chunk (l % 4) ^ ((l / 16) % 4).  Fixed per-lane offsets from a scalar tile base; the
  // last tile, if it runs past the end of the sequence, clamps its rows (their scores
  // are masked).
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int dl_r = lane >> 2, dl_c = (lane & 3) ^ ((lane >> 4) & 3);
  uint32_t dma_off[DMAS];
#pragma unroll
  for (int i = 0; i < DMAS; ++i) {
    const int bl = i * 4 + wave;
    dma_off[i] = (uint32_t)(((bl / CG) * 16 + dl_r) * ROWB + ((bl % CG) * 4 + dl_c) * 16);
  }
  auto dma_tile = [&](const uint16_t* __restrict__ src, int j, uint16_t* slot) {
    const char* base = (const char*)(src + (size_t)j * BN * rs_kv);
    if (j * BN + BN <= S) {
#pragma unroll
      for (int i = 0; i < DMAS; ++i) dma16_s(base, dma_off[i], slot + (i * 4 + wave_u) * 512);
    } else {
      int lr = dl_r;
      __asm__ volatile("" : "+v"(lr));  // keep this rare path's row arithmetic inside it
#pragma unroll
      for (int i = 0; i < DMAS; ++i) {
        const int row = ((i * 4 + wave) / CG) * 16 + lr;  // row within the tile
        const int rc = min(j * BN + row, S - 1) - j * BN;
        dma16_s(base, dma_off[i] + (uint32_t)((rc - row) * ROWB), slot + (i * 4 + wave_u) * 512);
      }
    }
  };
  uint16_t* const Kring = smem;
  uint16_t* const Vring = smem + 2 * TILE;

  // The first K and V tiles are on their way while the Q and dO rows load.
  dma_tile(Kg, 0, Kring);
  dma_tile(Vg, 0, Vring);

  // Q^T and dO^T fragments (B operands): query qc, d = ks*16 + half*8 .. +7.
  bf16x8 qf[KSTEPS], of[KSTEPS];
  {
    const u32x4* qrow = (const u32x4*)(a.q + qbase + (size_t)qc * rs_q + half * 8);
    const u32x4* orow = (const u32x4*)(a.dO + qbase + (size_t)qc * rs_q + half * 8);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      qf[ks] = __builtin_bit_cast(bf16x8, qrow[ks * 2]);
      of[ks] = __builtin_bit_cast(bf16x8, orow[ks * 2]);
    }
  }
  // The group's fp16 scales; this workgroup's rows of dO and Q in fp16 (scaled) for the
  // dK/dV kernel, from the fragments held here anyway.
  const GroupScales gs = group_scales(a.pmax, kvg);
  if (qi < S) {
    const float so = ldexpf(1.0f, gs.e_do), sq = ldexpf(1.0f, gs.e_q);
    u32x4* dst_o = (u32x4*)(a.do16 + wbase + (size_t)qi * D + half * 8);
    u32x4* dst_q = (u32x4*)(a.q16 + wbase + (size_t)qi * D + half * 8);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      dst_o[ks * 2] = bf16x8_to_f16x8(__builtin_bit_cast(u32x4, of[ks]), so);
      dst_q[ks * 2] = bf16x8_to_f16x8(__builtin_bit_cast(u32x4, qf[ks]), sq);
    }
  }
  const size_t prow = prow0 + qc;
  const float lse2 = a.lse2[prow];
  float dsum = 0.0f;  // this lane's part of sum_j dS_ij
  // -D from the bf16 O (every register of a lane belongs to its query), subtracted as dS
  // is formed.  (Starting each dP chain from -D instead saves that subtraction but holds
  // 16 copies of it in registers, which the kernel, with the fp16 copies and the D sums it
  // now also produces, cannot spare without spilling.)
  const float nd0 = a.delta[prow];
  const float c = a.scale * kLog2e;  // signed: no running maximum is needed here

  const int kv_end = CAUSAL ? min(S, q0 + kDqBM) : S;
  const int nkv = (kv_end + BN - 1) / BN;

  // Per-lane LDS byte offsets.  K and V operand reads: key row kb*32 + col, chunk
  // ks*2 + half (one register per parity of ks).  K^T transpose reads: source lane s
  // reads 4 d-values of key row kb*32 + t*16 + (s / 32) * 4 + (s % 16) / 4 (+ 8 for the
  // second read) at column 16 * ((s / 16) % 2) + 4 * (s % 4) of d block db.
  const int ka0 = opaque(blk_chunk_inner_x<D>(col, half)), ka1 = opaque(blk_chunk_inner_x<D>(col, 2 + half));
  const int trow = (lane >> 5) * 4 + ((lane >> 2) & 3);
  const int tcl = ((lane >> 4) & 1) * 2 + ((lane >> 1) & 1);
  const int tr0 = opaque((trow * 4 + (tcl ^ ((trow >> 2) & 3))) * 16 + (lane & 1) * 8);
  const int tr1 = opaque(((trow + 8) * 4 + (tcl ^ (((trow + 8) >> 2) & 3))) * 16 + (lane & 1) * 8);

  f32x16 dq[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) dq[db] = f32x16{};

  // One key tile on ring slot P; MASKED adds the causal / end-of-sequence mask to P^T.
  auto compute = [&](const int j, auto parity, auto masked) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    constexpr bool MASKED = decltype(masked)::value;
    constexpr int KO = P * TILE * 2, VO = (2 + P) * TILE * 2;  // byte offsets of K_j, V_j
    const char* L = (const char*)smem;
    const int k0 = j * BN;
    int lim = BN;  // keys at tile positions e > lim are masked
    if constexpr (MASKED) {
      const int lim_s = S - 1 - k0 - half * 4;
      lim = min(lim_s, qhi + col - k0 - half * 4);
    }
    bf16x8 fr[2 * NA];      // K / V fragments of the S^T and dP^T slots
    i16x4 tlo[NC], thi[NC];  // K^T transpose-read halves of the dQ^T slots
    auto issue = [&](const int i) __attribute__((always_inline)) {
      if (i < 2 * NA) {
        const int k = i % NA, kb = k % KB, ks = k / KB;
        const int o = (i < NA ? KO : VO) + kb * 32 / 16 * CG * 1024 + (ks >> 1) * 1024;
        fr[i] = *(const bf16x8*)(L + ((ks & 1) ? ka1 : ka0) + o);
      } else if (i < NS) {
        const int p = i - 2 * NA, u = p / DBLK, db = p % DBLK;  // u = kb * 2 + t
        const int o = KO + (u * CG + db) * 1024;
        tlo[p] = lds_read_tr16((const uint16_t*)(L + tr0 + o));
        thi[p] = lds_read_tr16((const uint16_t*)(L + tr1 + o));
      }
    };
    f32x16 s[KB], dp[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = f32x16{};
    }
    uint32_t dw[2 * KB][4];  // dS^T packed to bf16 pairs: [kb * 2 + t][pair]
    // dS for 8-key block u (registers v = 8t .. 8t+7 of key block kb).
    auto ds_block = [&](const int u, const int v0, const int v1) __attribute__((always_inline)) {
      const int kb = u >> 1;
#pragma unroll
      for (int vv = 0; vv < 8; ++vv) {
        if (vv < v0 || vv >= v1) continue;
        const int v = (u & 1) * 8 + vv;
        const float ds = s[kb][v] * (dp[kb][v] + nd0);
        dp[kb][v] = ds;
        dsum += ds;
        if (v & 1) dw[u][(v & 7) >> 1] = pack_bf16x2(dp[kb][v - 1], ds);
      }
    };
#pragma unroll
    for (int i = 0; i < PD; ++i) issue(i);
    __builtin_amdgcn_sched_barrier(0);
    // Three loops, one per phase (each small enough to unroll completely).
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      issue(i + PD);
      const int kb = i % KB, ks = i / KB;
      s[kb] = mfma32(fr[i], qf[ks], s[kb]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = NA; i < 2 * NA; ++i) {
      issue(i + PD);
      const int k = i - NA, kb = k % KB, ks = k / KB;
      dp[kb] = mfma32(fr[i], of[ks], ks == 0 ? f32x16{} : dp[kb]);
      // P^T for a share of the 32 scores, once S^T has had a slot to finish.
      if (k >= 1) {
        const int n = NA - 1, e0 = (k - 1) * 2 * 16 / n, e1 = k * 2 * 16 / n;
#pragma unroll
        for (int e = 0; e < 2 * 16; ++e) {
          if (e < e0 || e >= e1) continue;
          float p = exp2_sm<EXPMODE>(fmaf(s[e >> 4][e & 15], c, -lse2));
          if constexpr (MASKED) {
            const int ek = (e >> 4) * 32 + ((e & 15) >> 2) * 8 + (e & 3);  // key - k0 - half*4
            p = ek > lim ? 0.0f : p;
          }
          s[e >> 4][e & 15] = p;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 2 * NA; i < NS; ++i) {
      issue(i + PD);
      const int p = i - 2 * NA, u = p / DBLK, db = p % DBLK;
      // dS for block u before its first product, and for block u + 1 beside the
      // products of block u.
      if (p == 0) ds_block(0, 0, 8);
      if (u + 1 < 2 * KB) {
        const int r = p % DBLK;
        ds_block(u + 1, r * 8 / DBLK, (r + 1) * 8 / DBLK);
      }
      const u32x4 w = {dw[u][0], dw[u][1], dw[u][2], dw[u][3]};
      dq[db] = mfma32(join(tlo[p], thi[p]), __builtin_bit_cast(bf16x8, w), dq[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto step = [&](const int j, auto parity) {
    constexpr int P = decltype(parity)::value;
    if (j + 1 < nkv) {
      dma_tile(Kg, j + 1, Kring + (1 - P) * TILE);
      dma_tile(Vg, j + 1, Vring + (1 - P) * TILE);
    }
    const int k0 = j * BN;
    // No products for a tile wholly above the wave's rows, nor for a wave whose 32 rows
    // all lie past the end of the sequence (nothing of theirs is stored).
    if (k0 <= qhi + 31 && qw < S) {
      const bool need_mask = (k0 + BN > S) || (k0 + BN - 1 > qhi);
      if (need_mask) {
        compute(j, parity, std::true_type{});
      } else {
        compute(j, parity, std::false_type{});
      }
    }
    wait_dma();
    __syncthreads();
  };

  wait_dma();
  __syncthreads();
  for (int j = 0; j < nkv; j += 2) {
    step(j, std::integral_constant<int, 0>{});
    if (j + 1 < nkv) step(j + 1, std::integral_constant<int, 1>{});
  }

  // -D_i = -(D_i(bf16 O) + sum_j dS_ij) for the dK/dV kernel, in its dP units; 0 on the
  // padding rows up to the next multiple of 64 (that kernel moves whole 64-row blocks of it
  // into LDS).
  const float dtot = sum_halves(dsum);
  if (half == 0 && qi < ws_rows) {
    const size_t pr = prow0 + qi;
    a.ndx[pr] = qi < S ? (nd0 - dtot) * ldexpf(1.0f, gs.e_do + gs.e_v) : 0.0f;
  }
  if (qi < S) {
    uint16_t* dqr = a.dq + qbase + (size_t)qi * rs_q;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16x2(dq[db][g * 4 + 0] * sc, dq[db][g * 4 + 1] * sc);
        w[1] = pack_bf16x2(dq[db][g * 4 + 2] * sc, dq[db][g * 4 + 3] * sc);
        *(u32x2*)(dqr + db * 32 + g * 8 + half * 4) = w;
      }
    }
  }
}

template <int D, bool CAUSAL, int EXPMODE, bool VARLEN>
hipError_t launch_bwd_t(const BwdArgs& a0, bool four_wave, int phases, hipStream_t stream) {
  hipError_t e = hipSuccess;
  BwdArgs a = a0;
  a.dq_chunk = VARLEN ? varlen_chunk_groups(a.B, a.Hkv) : dq_chunk_groups(a.B, a.Hkv, a.S, D);
  a.kv_chunk = VARLEN ? varlen_chunk_groups(a.B, a.Hkv) : dkdv_chunk_groups(a.B, a.Hq, a.Hkv, a.S, D);
  // Order: preprocess, dQ (which also writes the exact -D and the fp16 dO that the dK/dV
  // kernel reads), dK/dV.
  if (phases & 1) {
    const int S_pad = (a.S + kBwdBM - 1) / kBwdBM * kBwdBM;
    hipLaunchKernelGGL((bwd_pre_kernel<D, VARLEN>), dim3((unsigned)(a.B * a.Hkv * kPreBlocks)), dim3(256), 0, stream, a,
                       S_pad);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (phases & 4) {
    const int nqt = (a.S + kDqBM - 1) / kDqBM;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, EXPMODE, VARLEN>), dim3((unsigned)(nqt * a.B * a.Hq)), dim3(256), 0,
                       stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (phases & 2) {
    const int nkt = (a.S + kBwdBN - 1) / kBwdBN;
    const dim3 grid((unsigned)(nkt * a.B * a.Hkv));
    // Four-wave workgroups (two per CU) need K's fragments in registers: always at d = 64,
    // at d = 128 with the hardware exponential only.
    if constexpr (D == 64) {
      hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL, EXPMODE, 4, VARLEN>), grid, dim3(256), 0, stream, a);
    } else if constexpr (EXPMODE == 0) {
      if (four_wave) {
        hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL, EXPMODE, 4, VARLEN>), grid, dim3(256), 0, stream, a);
      } else {
        hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL, EXPMODE, 8, VARLEN>), grid, dim3(512), 0, stream, a);
      }
    } else {
      hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL, EXPMODE, 8, VARLEN>), grid, dim3(512), 0, stream, a);
    }
    e = hipGetLastError();
  }
  return e;
}

template <int D, bool VARLEN>
hipError_t launch_bwd_d(const BwdArgs& a, bool causal, int exp_mode, bool four_wave, int phases, hipStream_t stream) {
  if (causal) {
    return exp_mode == 0 ? launch_bwd_t<D, true, 0, VARLEN>(a, four_wave, phases, stream)
                         : launch_bwd_t<D, true, 1, VARLEN>(a, four_wave, phases, stream);
  }
  return exp_mode == 0 ? launch_bwd_t<D, false, 0, VARLEN>(a, four_wave, phases, stream)
                       : launch_bwd_t<D, false, 1, VARLEN>(a, four_wave, phases, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int d, bool causal, int exp_mode, bool four_wave, int phases,
                      hipStream_t stream) {
  if (a.cu_seqlens != nullptr) {
    return d == 64 ? launch_bwd_d<64, true>(a, causal, exp_mode, four_wave, phases, stream)
                   : launch_bwd_d<128, true>(a, causal, exp_mode, four_wave, phases, stream);
  }
  return d == 64 ? launch_bwd_d<64, false>(a, causal, exp_mode, four_wave, phases, stream)
                 : launch_bwd_d<128, false>(a, causal, exp_mode, four_wave, phases, stream);
}

}  // namespace attn
