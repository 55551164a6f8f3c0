// attn_fwd.hip - forward pass of exact attention on gfx950 (CDNA4).
//
// One workgroup of W waves (4 for the four-wave schedule, 8 for the ping-pong schedule)
// owns 32 W consecutive queries of one (batch, query head); each wave owns 32 of them.
// The workgroup walks the key/value sequence in tiles of BN keys (32 for the four-wave
// schedule, which then fits three workgroups, three waves per SIMD, on a CU; 64 for the
// ping-pong schedule) that are staged through LDS and shared by its waves; the S x S
// score matrix never leaves registers (the
// memory-traffic argument of "NVIDIA Blackwell: FlashAttention-4 Overcomes Memory
// Bottlenecks", body paragraph, and of the hyper.ai FlashAttention-4 story).
//
// Per key tile, each wave computes the transposed scores S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (K from LDS as the A operand, Q^T held in registers as the
// B operand).  In that accumulator layout a lane holds 16 keys of ONE query column,
// so the running row maximum and row sum of the online softmax are in-lane
// reductions plus one v_permlane32_swap between the two wave halves.  The
// probabilities P^T are packed to bf16 straight from the accumulator registers and
// used as the B operand of O^T += V^T P^T; V^T comes from the V tile through
// ds_read_b64_tr_b16 (LDS transpose reads).  The output accumulator O^T keeps the
// same one-query-per-lane layout, so rescaling it by a per-row factor is a plain
// per-lane multiply.
//
// Online softmax with conditional rescaling (the "adaptive online softmax rescaling"
// of "NVIDIA's FlashAttention-4", section "The Technical Edge": rescale only when the
// maximum changes significantly): each row keeps a reference maximum m_ref in log2
// units.  When a tile's maximum exceeds m_ref + tau anywhere in the wave, the wave
// rescales O^T and the running sum by 2^(m_ref - m_new) and moves m_ref; otherwise
// the probabilities 2^(x - m_ref) are used as they are (they stay <= 2^tau).  Since
// O and the sum always share m_ref, the final O = O_acc / l is exact for every tau.
// The tile maximum itself is only taken when the test can fire: the exponentials are
// computed with m_ref first, and unless some lane's partial row sum reaches 2^(tau-1)
// (which any score above m_ref + tau forces) no rescale is due.
//
// Software pipeline of one key tile j (a "step"), per wave: the products of tile j+1's
// scores S_{j+1} = K_{j+1} Q^T are issued while the vector units exponentiate S_j
// (phase 1), then, after the rescale test, O^T += V_j^T P_j^T (phase 2).
// Both phases are written out as slots of one matrix product each, fenced so the
// compiler keeps them: a slot issues the LDS reads of the slot two ahead, its product,
// and its share of the vector work.  The matrix cores of a SIMD are shared by two
// waves, which fill each other's gaps: of two different workgroups for W = 4, or of the
// two halves of one workgroup, kept half a step apart, for W = 8.
//
// Causal masking: key tiles above the diagonal of the workgroup are never loaded, and a
// wave skips the loaded tiles that lie wholly above its own queries; only tiles that
// straddle the diagonal or the end of the sequence are masked.
// Workgroups are dispatched longest-first (largest query tile index first; under the causal
// mask the longer ones also run at a higher wave priority), and when the number of KV
// groups is a multiple of 8 all query heads and query tiles of one KV group run on one XCD
// and share its L2 for K and V.  Large launches of short sequences run in chunks of KV
// groups (dispatch_chunk in attn_kernels.h) so that the resident workgroups' K and V fit
// the memory-side cache; packed batches run in chunks of 8 (sequence, KV head) groups,
// one per XCD (varlen_chunk_groups).
#include <type_traits>

#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

// Keys per LDS tile and waves per SIMD of a schedule.  The four-wave schedule uses
// 32-key tiles: half the score registers of 64-key tiles, so that three waves share
// each SIMD (168 registers each) and hide more of each other's latency.  The cubic
// exponential needs a few registers more than that, so its four-wave kernels keep two
// waves per SIMD.
template <int W>
constexpr int fwd_bn() { return W == 4 ? 32 : 64; }
template <int W, int EXPMODE>
constexpr int fwd_waves_per_simd() { return W == 4 && EXPMODE == 0 ? 3 : 2; }
// Slots between an LDS read and the product that uses it: two hide the read latency
// behind the two products in between; three or four measured slower on both schedules.
constexpr int kFwdPD = 2;

// VARLEN: a packed batch of sequences of different lengths (FwdArgs::cu_seqlens), with
// token-major rows (row stride H*d instead of d); otherwise the dense [B, H, S, d] layout.
// W: waves per workgroup.  W = 4: every wave meets the barrier after phase 2, and two
// workgroups share a CU.  W = 8: the staggered two-group schedule described below, one
// workgroup per CU.
template <int D, bool CAUSAL, int EXPMODE, bool VARLEN, int W>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * W, 64 * W),
                          amdgpu_waves_per_eu(fwd_waves_per_simd<W, EXPMODE>(), fwd_waves_per_simd<W, EXPMODE>())))
void fwd_kernel(FwdArgs a) {
  static_assert(W == 4 || W == 8, "4 or 8 waves per workgroup");
  constexpr int BN = fwd_bn<W>();
  constexpr int BM = 32 * W;            // queries per workgroup
  constexpr int KB = BN / 32;           // 32-key blocks per tile
  constexpr int KSTEPS = D / 16;        // MFMA k-steps of S^T = K Q^T
  constexpr int DBLK = D / 32;          // 32-row blocks of O^T
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int TILE = BN * D;          // bf16 elements of one K or V tile
  constexpr int DMAS = BN * CPR / (64 * W);  // 16-byte chunks per thread per tile
  constexpr int NQK = KSTEPS * KB;      // phase-1 slots (products of S_{j+1})
  constexpr int NPV = 2 * KB * DBLK;    // phase-2 slots (products of O^T)
  constexpr int NE = KB * 16;           // scores per lane per tile
  constexpr int EPS = NE / NQK;         // exponentials per phase-1 slot
  constexpr int PD = kFwdPD;
  static_assert(NE % NQK == 0 && EPS % 2 == 0, "exponentials must pair up per slot");
  static_assert(BN % 32 == 0 && DMAS * 64 * W == BN * CPR, "tile must split evenly over the threads");
  constexpr int VR = W == 8 ? 3 : 2;    // V ring slots (the K ring has 2)
  // K ring then V ring, each tile [BN][D] in 1024-byte blocks.
  __shared__ __attribute__((aligned(1024))) uint16_t smem[(2 + VR) * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;
  const int half = lane >> 5;

  const int nqt = (a.S + BM - 1) / BM;
  const int bid = blockIdx.x;
  // Dispatch order.  The grid is cut into chunks of grp_chunk KV groups (the last chunk
  // may be smaller), run one after the other; within a chunk the workgroups go level by
  // level, a level being one query tile of every query head of the chunk, causal: the
  // longest (last) query tile first.  Chunks keep the K and V that the resident
  // workgroups read to a few heads per XCD, so that their re-reads hit L2 and the
  // memory-side cache instead of HBM when B x H is large.
  // Head of this workgroup: workgroups go to the 8 XCDs round-robin (XCD = bid % 8).  When
  // the chunk's group count is a multiple of 8 (then so is every chunk's start), position
  // u in a level maps to KV group ((u / 8) / G) * 8 + u % 8 of the chunk and query head
  // g = (u / 8) % G of it, so every query head and query tile of one KV group runs on one
  // XCD and reads its K and V through one L2.
  const int G = a.Hq / a.Hkv;
  const int ngrp = a.B * a.Hkv;
  const int per_chunk = a.grp_chunk * G * nqt;
  const int chunk = bid / per_chunk;
  const int pos = bid - chunk * per_chunk;
  const int g0 = chunk * a.grp_chunk;
  const int ncg = min(a.grp_chunk, ngrp - g0);  // KV groups in this chunk
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
  const int q0 = qt * BM;
  // Causal four-wave launches: a workgroup's work grows with its query tile, and the
  // longest ones, dispatched first, set when the launch ends.  Their waves get a higher
  // issue priority (four levels by query tile), so they take the SIMD whenever they are
  // ready and the shorter workgroups that share the CU fill the gaps.  (The arithmetic is
  // unchanged; short causal launches, where three workgroups of very different lengths
  // share each CU, end 3-4% sooner.)
  if constexpr (CAUSAL && W == 4) {
    const int lvl = (4 * (qt + 1)) / (nqt + 1);
    if (lvl >= 3) {
      __builtin_amdgcn_s_setprio(3);
    } else if (lvl == 2) {
      __builtin_amdgcn_s_setprio(2);
    } else if (lvl == 1) {
      __builtin_amdgcn_s_setprio(1);
    }
  }
  // Rows of this (batch or sequence, head): S of them, D elements each, rs_q / rs_kv
  // elements apart; LSE of query i at lse[lse0 + i].
  int S, Sq;  // keys (the sequence's length) and the queries this launch writes
  size_t qbase, kvbase, lse0;
  constexpr int RS_DENSE = D;
  int rs_q = RS_DENSE, rs_kv = RS_DENSE;
  if constexpr (VARLEN) {
    const int start = min(max(a.cu_seqlens[b], 0), a.total);
    const int end = min(max(a.cu_seqlens[b + 1], start), a.total);
    S = end - start;
    Sq = min(S, a.S);     // queries past max_seqlen (a.S) are not written
    if (q0 >= Sq) return;  // the whole workgroup: this tile lies past its sequence
    rs_q = a.Hq * D;
    rs_kv = a.Hkv * D;
    qbase = (size_t)start * rs_q + (size_t)hq * D;
    kvbase = (size_t)start * rs_kv + (size_t)hkv * D;
    lse0 = (size_t)hq * a.total + start;
  } else {
    S = Sq = a.S;
    qbase = ((size_t)b * a.Hq + hq) * (size_t)S * D;
    kvbase = ((size_t)b * a.Hkv + hkv) * (size_t)S * D;
    lse0 = ((size_t)b * a.Hq + hq) * S;
  }
  const int qw = q0 + wave * 32;  // first query of this wave
  const int qi = qw + col;        // this lane's query
  const uint16_t* __restrict__ Kg = a.k + kvbase;
  const uint16_t* __restrict__ Vg = a.v + kvbase;

  // Q^T fragments (B operand): query qi, d = ks*16 + half*8 .. +7.  Rows past the end
  // of the sequence load the last row instead (their outputs are never stored); no
  // branch, so all the loads are in flight together.  With d = 128 they are issued after
  // the first K and V tiles' DMA, so that the two overlap (2k prefill 1.5-2% faster); with
  // d = 64 before it (1.5% faster that way).
  bf16x8 qf[KSTEPS];
  const u32x4* qrow = (const u32x4*)(a.q + qbase + (size_t)min(qi, S - 1) * rs_q + half * 8);
  if constexpr (D == 64) {
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, (qrow[ks * 2] & a.q_and) ^ a.q_xor);
  }

  const int kv_end = CAUSAL ? min(S, q0 + BM) : S;
  const int nkv = (kv_end + BN - 1) / BN;

  // LDS tiles use the blocked layouts of attn_device.h: K chunk-inner with XOR (read as
  // MFMA A operands, 16 rows at one chunk), V chunk-inner (read by transpose reads).  A
  // tile is (BN / 16) x (D / 32) blocks of 1024 bytes; wave w of W DMAs blocks W i + w,
  // i < DMAS.  Lane l fetches row l / 4 of the block, chunk l % 4 (K: XOR (l / 16) % 4),
  // so every 4 lanes read one aligned 64-byte piece of a row.  The per-lane global byte offsets are
  // fixed and the tile base is a scalar; only the last tile, if it runs past the end of
  // the sequence, clamps its rows to a real row (their scores are masked, so any finite
  // data will do).
  constexpr int CG = D / 32;    // 4-chunk groups per row
  const int ROWB = rs_kv * 2;   // bytes between K/V rows in memory (2 D when dense)
  static_assert(W % CG == 0 && (BN / 16) * CG == W * DMAS, "DMA block assignment");
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int w_rg = wave_u / CG, w_cg = wave_u % CG;  // block (w_rg, w_cg) for i = 0
  const int k_lr = lane >> 2, k_lc = (lane & 3) ^ ((lane >> 4) & 3);
  const int v_lr = lane >> 2, v_lc = lane & 3;
  const uint32_t k_goff = (uint32_t)((w_rg * 16 + k_lr) * ROWB + (w_cg * 4 + k_lc) * 16);
  const uint32_t v_goff = (uint32_t)((w_rg * 16 + v_lr) * ROWB + (w_cg * 4 + v_lc) * 16);
  auto dma_tile = [&](const uint16_t* __restrict__ src, int j, uint16_t* slot, int lr, int lc, uint32_t goff) {
    const char* base = (const char*)(src + (size_t)j * BN * rs_kv);
    if (j * BN + BN <= S) {
#pragma unroll
      for (int i = 0; i < DMAS; ++i)
        dma16_s(base + i * (W / CG) * 16 * ROWB, goff, slot + (i * W + wave_u) * 512);
    } else {
      __asm__ volatile("" : "+v"(lr));  // keep this rare path's row arithmetic inside it
#pragma unroll
      for (int i = 0; i < DMAS; ++i) {
        const int r = (i * (W / CG) + w_rg) * 16 + lr;  // row within the tile
        const int rc = min(j * BN + r, S - 1) - j * BN;
        dma16_s(base, (uint32_t)(rc * ROWB + (w_cg * 4 + lc) * 16), slot + (i * W + wave_u) * 512);
      }
    }
  };
  auto dma_k = [&](int j, uint16_t* slot) { dma_tile(Kg, j, slot, k_lr, k_lc, k_goff); };
  auto dma_v = [&](int j, uint16_t* slot) { dma_tile(Vg, j, slot, v_lr, v_lc, v_goff); };
  uint16_t* const Kring = smem;
  uint16_t* const Vring = smem + 2 * TILE;

  // Per-lane byte offsets of the LDS reads; every other read of a tile adds a constant.
  // K (A operand of S^T = K Q^T): lane l reads key row l % 32, chunk l / 32 + 2 ks; one
  // register per parity of ks.
  const int k_lds0 = blk_chunk_inner_x<D>(col, half), k_lds1 = blk_chunk_inner_x<D>(col, 2 + half);
  auto k_off = [&](int kb, int ks) { return ((ks & 1) ? k_lds1 : k_lds0) + blk_chunk_inner_x<D>(kb * 32, (ks >> 1) * 4); };
  // V^T by transpose reads: source lane s reads 4 d-values of key row
  // (s / 32) * 4 + (s % 16) / 4 (+ 8 for the second read) at column
  // 16 * ((s / 16) % 2) + 4 * (s % 4) of a 32-wide d block.
  const int v_lds = blk_chunk_inner<D>((lane >> 5) * 4 + ((lane >> 2) & 3), ((lane >> 4) & 1) * 2 + ((lane >> 1) & 1)) +
                    (lane & 1) * 8;

  f32x16 oacc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) oacc[db] = f32x16{};
  float m_ref = -INFINITY;  // reference row maximum, log2 units (scaled scores)
  float l_run = 0.0f;       // this lane's part of the running row sum
  const float c = a.c;
  const float tau = a.tau;
  const float thr = exp2f(tau - 1.0f);  // partial row sum that calls for the rescale test

  // Tiles that reach past the end of the sequence or (causal) past the wave's first
  // query: the only ones with masked scores.
  auto needs_mask = [&](int k0) { return (k0 + BN > S) || (CAUSAL && k0 + BN - 1 > qw); };
  auto mask = [&](f32x16* s, int k0) {
    // The lane's half and column, recomputed here from the lane id: kept live across the
    // loop for this rare path they would cost registers.
    const int ln = lane_id_here();
    const int hf = ln >> 5;
    const int lim_s = S - 1 - k0 - hf * 4;                                   // key <= S - 1
    int lim = CAUSAL ? min(lim_s, qw + (ln & 31) - k0 - hf * 4) : lim_s;     // key <= query
    __asm__ volatile("" : "+v"(lim));  // keep the comparisons inside this rare path
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int e = kb * 32 + (v >> 2) * 8 + (v & 3);  // key - k0 - half*4
        s[kb][v] = e > lim ? -INFINITY : s[kb][v];
      }
  };
  // Scaled row maximum (log2 units) of a score tile, both wave halves combined.
  auto tile_max = [&](const f32x16* s) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
    return max_halves(mx) * c;
  };

  // Ring discipline.  Every wave issues its share of the next tiles right after a
  // barrier and waits for that share before its next barrier, so a tile issued after
  // barrier m is complete for everyone after barrier m+1.  After barrier m the tiles
  // K_{m+2} (into K_m's slot) and V_{m+1} (into slot (m+1) % VR) are issued.
  //
  // W = 8 (two-wave-group ping-pong): the halves of the workgroup run the same steps
  // half a step apart, so the two waves sharing a SIMD (waves w and w+4) are in
  // complementary phases.  Group 0 meets each barrier after phase 2 of a step, group 1
  // after phase 1.  Between two barriers group 0 runs phases 1 and 2 of step s while
  // group 1 runs phase 2 of step s-1 and phase 1 of step s: the tiles read are K_{s+1},
  // V_s and V_{s-1} while K_{s+2} and V_{s+1} land, hence 3 V slots.
  const int grp = W == 8 ? (wave_u >= W / 2) : 0;
  // Prologue: K_0, K_1, V_0 resident; S_0 computed; a second barrier frees K_0's slot;
  // then K_2 and V_1 in flight.
  dma_k(0, Kring);
  if (nkv > 1) dma_k(1, Kring + TILE);
  dma_v(0, Vring);
  if constexpr (D != 64) {
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, (qrow[ks * 2] & a.q_and) ^ a.q_xor);
  }
  wait_dma();
  __syncthreads();
  f32x16 sc[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) sc[kb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      sc[kb] = mfma32(*(const bf16x8*)((const char*)Kring + k_off(kb, ks)), qf[ks], sc[kb]);
  if (needs_mask(0)) mask(sc, 0);
  // The first reference maximum is S_0's (O and the row sum are still zero, so nothing
  // needs rescaling).
  m_ref = tile_max(sc);
  // -m_ref as the exponent offset (0 while m_ref is -inf), kept in its own register: it
  // changes only when the reference moves.
  float nmu = m_ref == -INFINITY ? 0.0f : -m_ref;
  __syncthreads();  // every wave has read K_0
  if (nkv > 2) dma_k(2, Kring);
  if (nkv > 1) dma_v(1, Vring + TILE);
  int r_cur = 0;  // V ring slot of V_s, s % VR

  // One key tile: S_j (in cur) -> O; S_{j+1} (into nxt).  P is the K ring parity of j,
  // a constant in computing steps: their loop is unrolled by two so that the K slot
  // offsets are constants and the score registers swap roles instead of being copied
  // (the V slot, r_cur, is one wave-uniform value per step).  A dead step (DEAD true:
  // a tile wholly above the wave's queries) only meets the barrier and issues the wave's
  // share of the DMA, in which every wave of the workgroup takes part.
  auto step = [&](const int j, f32x16 (&cur)[KB], f32x16 (&nxt)[KB], auto parity, auto dead) {
    const int P = parity;  // j % 2
    constexpr bool DEAD = decltype(dead)::value;
    const int r1 = r_cur == VR - 1 ? 0 : r_cur + 1;                 // V slot of V_{j+1}
    const int r2 = r1 == VR - 1 ? 0 : r1 + 1;                       // V slot of V_{j+2}
    const char* Ks = (const char*)(Kring + (1 - P) * TILE);          // K_{j+1}
    const char* Vs = (const char*)(Vring + r_cur * TILE) + v_lds;    // V_j
    // This step's barrier (j+1): wait for this wave's share of K_{j+2} and V_{j+1}, meet
    // the other waves, then start K_{j+3} (into K_{j+1}'s slot, read by both groups in
    // phase 1, before their barrier) and V_{j+2}: for W = 8 into the slot of V_{j-1},
    // whose last reader (group 1, phase 2 of step j-1) finished before reaching this
    // barrier; for W = 4 into the slot of V_j, read by every wave in phase 2, before it.
    auto barrier = [&]() {
      wait_dma();
      __syncthreads();
      if (j + 3 < nkv) dma_k(j + 3, Kring + (1 - P) * TILE);
      if (j + 2 < nkv) dma_v(j + 2, Vring + r2 * TILE);
    };
    if constexpr (DEAD) {
      barrier();
      r_cur = r1;
      return;
    }

    // LDS reads of slot i: the K fragment of product i of phase 1, or the two V^T
    // halves of product i - NQK of phase 2.
    bf16x8 kfrag[NQK];
    i16x4 vlo[NPV], vhi[NPV];
    auto issue = [&](const int i) {
      if (i < NQK) {
        kfrag[i] = *(const bf16x8*)(Ks + k_off(i % KB, i / KB));
      } else if (i < NQK + NPV) {
        const int p = i - NQK, db = p % DBLK, row = (p / DBLK) * 16;
        vlo[p] = lds_read_tr16((const uint16_t*)(Vs + blk_chunk_inner<D>(row, db * 4)));
        vhi[p] = lds_read_tr16((const uint16_t*)(Vs + blk_chunk_inner<D>(row + 8, db * 4)));
      }
    };
#pragma unroll
    for (int i = 0; i < PD; ++i) issue(i);


#pragma unroll
    for (int kb = 0; kb < KB; ++kb) nxt[kb] = f32x16{};
    uint32_t pw[KB][2][4];  // P_j packed to bf16 pairs: [key block][16-key half][pair]
    // The row sums start at -0: -0 + p is exactly p for every p, so the first additions
    // fold away (+0 + p is not an identity in floating point: it maps -0 to +0).
    float lt0 = -0.0f, lt1 = -0.0f;
    // Exponentials of S_j registers e, e+1 with the reference maximum m_ref, into pw and
    // (lt0, lt1).  Called with compile-time e only (unrolled loops), so pw stays in
    // registers.
    auto exp_pair = [&](const int e) {
      const float p0 = exp2_sm<EXPMODE>(fmaf(cur[e >> 4][e & 15], c, nmu));
      const float p1 = exp2_sm<EXPMODE>(fmaf(cur[e >> 4][(e & 15) + 1], c, nmu));
      lt0 += p0;
      lt1 += p1;
      pw[e >> 4][(e >> 3) & 1][(e & 7) >> 1] = pack_bf16x2(p0, p1);
    };
    __builtin_amdgcn_sched_barrier(0);
    // Phase 1: the NQK products of S_{j+1}, EPS exponentials of S_j beside each.
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      issue(i + PD);
      const int kb = i % KB, ks = i / KB;
      nxt[kb] = mfma32(kfrag[i], qf[ks], nxt[kb]);
#pragma unroll
      for (int e = i * EPS; e < (i + 1) * EPS; e += 2) exp_pair(e);
      // Keep the row-sum additions in this slot (they would otherwise sink below the
      // barrier, where no matrix product runs beside them).
      __asm__ volatile("" : "+v"(lt0), "+v"(lt1));
      __builtin_amdgcn_sched_barrier(0);
    }
    // The (rare) rescale, decided after the exponentials.  A score more than tau above
    // m_ref gives p > 2^tau, so while every lane's partial sum stays below 2^(tau-1) no
    // rescale is due.  Otherwise take S_j's maximum and apply the rule exactly: if it
    // exceeds m_ref + tau anywhere in the wave, rescale O^T and the running sum by
    // 2^(m_ref - m_new), move m_ref and redo the exponentials.  One wave-uniform branch
    // per step.
    if (wave_any(!(lt0 + lt1 < thr) || m_ref == -INFINITY)) {
      const float mt = tile_max(cur);
      if (wave_any(mt > m_ref + tau)) {
        const float m_new = fmaxf(m_ref, mt);
        const float alpha = (m_new == -INFINITY) ? 1.0f : exp2_sm<0>(m_ref - m_new);
#pragma unroll
        for (int db = 0; db < DBLK; ++db) oacc[db] *= alpha;
        l_run *= alpha;
        m_ref = m_new;
        nmu = m_ref == -INFINITY ? 0.0f : -m_ref;
        lt0 = lt1 = -0.0f;
#pragma unroll
        for (int e = 0; e < NE; e += 2) exp_pair(e);
      }
    }
    if (grp != 0) barrier();
    __builtin_amdgcn_sched_barrier(0);
    // Phase 2: the NPV products of O^T.
#pragma unroll
    for (int i = NQK; i < NQK + NPV; ++i) {
      issue(i + PD);
      const int p = i - NQK, db = p % DBLK, kb = p / (2 * DBLK), t = (p / DBLK) & 1;
      const u32x4 w = {pw[kb][t][0], pw[kb][t][1], pw[kb][t][2], pw[kb][t][3]};
      oacc[db] = mfma32(join(vlo[p], vhi[p]), __builtin_bit_cast(bf16x8, w), oacc[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += lt0 + lt1;
    if (grp == 0) barrier();
    r_cur = r1;
    // S_{j+1} as computed is exact except on tiles that need a mask (at most the last
    // two of a wave).
    if (j + 1 < nkv && needs_mask((j + 1) * BN)) mask(nxt, (j + 1) * BN);
  };

  // This wave's live tiles: all nkv, or under the causal mask those holding a key at or
  // below its last query (wave-uniform).  The steps past them are dead.  (The last live
  // step still forms S_{nlive} and discards it: peeling that step off costs more registers
  // than the 16 products it would save.)  In the four-wave schedule a wave whose 32 rows
  // all lie past the end of the sequence has none: its products would be discarded.  (The
  // ping-pong groups keep every wave live: their barriers are staggered by group.)
  const int nlive = (W == 4 && q0 + wave_u * 32 >= Sq)
                        ? 0
                        : (CAUSAL ? min(nkv, (min(S, q0 + wave_u * 32 + 32) + BN - 1) / BN) : nkv);
  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;
  f32x16 sn[KB];
  for (int j = 0; j < nlive; j += 2) {
    step(j, sc, sn, Even{}, std::false_type{});
    if (j + 1 < nlive) step(j + 1, sn, sc, Odd{}, std::false_type{});
  }
  for (int j = nlive; j < nkv; ++j) step(j, sc, sn, j & 1, std::true_type{});

  // Epilogue: O = O_acc / l (bf16, round to nearest even) and LSE in natural log.
  const float l = sum_halves(l_run);
  const float inv = 1.0f / l;
  // The lane's query and half, recomputed from the lane id (not held across the loop).
  const int ln = lane_id_here();
  const int qo = qw + (ln & 31), ho = ln >> 5;
  if (qo < Sq) {
    uint16_t* orow = a.o + qbase + (size_t)qo * rs_q;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][g * 4 + 0] * inv, oacc[db][g * 4 + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][g * 4 + 2] * inv, oacc[db][g * 4 + 3] * inv);
        *(u32x2*)(orow + db * 32 + g * 8 + ho * 4) = w;
      }
    }
    if (ho == 0) a.lse[lse0 + qo] = (m_ref + log2f(l)) * kLn2;
  }
}

template <int D, bool CAUSAL, int EXPMODE, bool VARLEN, int W>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const int nqt = (a.S + 32 * W - 1) / (32 * W);
  const dim3 grid((unsigned)(nqt * a.B * a.Hq));
  FwdArgs c = a;
  // (Measured with 256-512 heads at S = 2048: 15-25% faster than one chunk; at S = 8192,
  // chunks of 24-48 groups were 1-4% slower.)
  c.grp_chunk = VARLEN ? varlen_chunk_groups(a.B, a.Hkv) : fwd_chunk_groups(a.B, a.Hkv, a.S, D);
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, EXPMODE, VARLEN, W>), grid, dim3(64 * W), 0, stream, c);
  return hipGetLastError();
}

template <int D, bool VARLEN, int W>
hipError_t launch_fwd_w(const FwdArgs& a, bool causal, int exp_mode, hipStream_t stream) {
  if (causal) {
    return exp_mode == 0 ? launch_fwd_t<D, true, 0, VARLEN, W>(a, stream)
                         : launch_fwd_t<D, true, 1, VARLEN, W>(a, stream);
  }
  return exp_mode == 0 ? launch_fwd_t<D, false, 0, VARLEN, W>(a, stream)
                       : launch_fwd_t<D, false, 1, VARLEN, W>(a, stream);
}

template <int D, bool VARLEN>
hipError_t launch_fwd_d(const FwdArgs& a, bool causal, int exp_mode, bool pingpong, hipStream_t stream) {
  return pingpong ? launch_fwd_w<D, VARLEN, 8>(a, causal, exp_mode, stream)
                      : launch_fwd_w<D, VARLEN, 4>(a, causal, exp_mode, stream);
}

__global__ void exp2_eval_kernel(const float* x, float* y, long n, int mode) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = mode == 0 ? exp2_sm<0>(x[i]) : exp2_sm<1>(x[i]);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, int d, bool causal, int exp_mode, bool pingpong, hipStream_t stream) {
  return d == 64 ? launch_fwd_d<64, false>(a, causal, exp_mode, pingpong, stream)
                 : launch_fwd_d<128, false>(a, causal, exp_mode, pingpong, stream);
}

hipError_t launch_fwd_varlen(const FwdArgs& a, int d, bool causal, int exp_mode, bool pingpong, hipStream_t stream) {
  return d == 64 ? launch_fwd_d<64, true>(a, causal, exp_mode, pingpong, stream)
                 : launch_fwd_d<128, true>(a, causal, exp_mode, pingpong, stream);
}

hipError_t launch_exp2_eval(const float* x, float* y, long n, int exp_mode, hipStream_t stream) {
  const long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(exp2_eval_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, y, n, exp_mode);
  return hipGetLastError();
}

}  // namespace attn
