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
//               tiles (64 queries) that can see its keys (causal: only tiles at or below
//               the diagonal), from the last one down, for every query head of the GQA
//               group.  Per step, with Q, dO, LSE and D staged in LDS:
//                   S   = Q K^T,  dP = dO V^T     (MFMA; K and V stay in LDS for the run)
//                   P   = 2^(S c - LSE log2 e), 0 where masked  (c = scale log2 e)
//                   dS  = P (dP - D)
//                   dV^T += dO^T P,  dK^T += Q^T dS   (dO^T and Q^T by LDS transpose reads)
//               Because the group's query heads loop inside the workgroup, dK and dV are
//               summed over the group without atomics.
//  3. bwd_dq:   dQ, per query tile, recomputing S and dP (see below); no atomics.
//
// In the S accumulator layout of bwd_main (v_mfma_f32_32x32x16_bf16, A = Q rows, B = K^T)
// a lane holds one key column and 16 query rows; P and dS are packed to bf16 in registers
// and used directly as the B operand of the dV^T and dK^T products.
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
// padding rows get 0.  The main kernel then moves whole 64-row blocks of -D and LSE into
// LDS with no bounds checks; the dQ kernel reads one of each per lane.  Both start their
// dP products from -D, so dS = P (dP - D) is one multiply.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dO,
                                                      const float* __restrict__ lse, float* __restrict__ delta,
                                                      float* __restrict__ lse2, long prows, int S, int S_pad) {
  constexpr int LPR = D / 8;  // lanes per row, 8 bf16 each
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long prow = gid / LPR;
  const int part = (int)(gid % LPR);
  const long bhr = prow / S_pad;
  const int srow = (int)(prow - bhr * S_pad);
  const bool real = prow < prows && srow < S;
  const long row = bhr * S + srow;  // row in the unpadded [B*Hq][S] tensors
  float acc = 0.0f;
  if (real) {
    const u32x4 ov = *(const u32x4*)(o + row * D + part * 8);
    const u32x4 dv = *(const u32x4*)(dO + row * D + part * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float o0 = __builtin_bit_cast(float, ov[e] << 16), o1 = __builtin_bit_cast(float, ov[e] & 0xffff0000u);
      const float d0 = __builtin_bit_cast(float, dv[e] << 16), d1 = __builtin_bit_cast(float, dv[e] & 0xffff0000u);
      acc = fmaf(o0, d0, acc);
      acc = fmaf(o1, d1, acc);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (prow < prows && part == 0) {
    delta[prow] = -acc;  // -D: the dP products start from it
    lse2[prow] = real ? lse[row] * kLog2e : 0.0f;
  }
}

// ------------------------------------------------------------------ main

// Workgroup of 8 waves (two per SIMD) on a tile of 128 keys.  Wave w owns key block
// kq = w % 4 (32 keys) for query half qh = w / 4 of every 64-query step: waves w and
// w + 4 accumulate partial dK and dV for the same keys over different queries, and
// the two partials are added through LDS at the end.
//
// K, V (resident) and the Q, dO stages sit in LDS as XOR chunk-inner blocks (see
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
template <int D, bool CAUSAL, int EXPMODE>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void bwd_main_kernel(BwdArgs a) {
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int CG = D / 32;                   // 4-chunk groups per row
  constexpr int ROWB = D * 2;                  // bytes per row in memory
  constexpr int KT = kBwdBN * D;               // elements of the K (or V) tile
  constexpr int QT = kBwdBM * D;               // elements of one Q (or dO) tile
  constexpr int KDMAS = kBwdBN / 16 * CG / 8;  // 1024-byte blocks per wave, K or V tile
  constexpr int QDMAS = kBwdBM / 16 * CG / 8;  // 1024-byte blocks per wave, Q or dO tile
  constexpr int PD = 2;                        // slots between an LDS read and its product
  constexpr int NS = 4 * KSTEPS;               // slots per step (== 4 * 2 * DBLK)
  static_assert(KSTEPS == 2 * DBLK && KDMAS * 8 * 16 == kBwdBN * CG && QDMAS * 8 * 16 == kBwdBM * CG, "tiling");
  // One LDS buffer, [K | V | Q stage 0 | Q stage 1 | dO stage 0 | dO stage 1 | LSE, D]: every
  // operand read reaches its tile from a lane's base register by an immediate offset
  // below 64 KiB (K and V from the K base; the four stages from the Q base).
  constexpr int K_OFF = 0, V_OFF = 2 * KT, Q_OFF = 4 * KT, DO_OFF = Q_OFF + 4 * QT, SD_OFF = DO_OFF + 4 * QT;
  static_assert(V_OFF + 2 * KT - K_OFF <= 65536 && SD_OFF - Q_OFF <= 65536, "immediate LDS offsets");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SD_OFF + 2 * 2 * kBwdBM * 4];
  uint16_t* const k_lds = (uint16_t*)(smem + K_OFF);
  uint16_t* const v_lds = (uint16_t*)(smem + V_OFF);
  uint16_t* const q_lds[2] = {(uint16_t*)(smem + Q_OFF), (uint16_t*)(smem + Q_OFF + 2 * QT)};
  uint16_t* const do_lds[2] = {(uint16_t*)(smem + DO_OFF), (uint16_t*)(smem + DO_OFF + 2 * QT)};
  float (*const sd_lds)[2 * kBwdBM] = (float (*)[2 * kBwdBM])(smem + SD_OFF);  // [stage][LSE log2e | D]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kq = wave & 3;   // key block of this wave
  const int qh = wave >> 2;  // query half of each step
  const int col = lane & 31;
  const int half = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int S = a.S;
  const int G = a.Hq / a.Hkv;

  // Tiles with the lowest key index have the most query tiles under the causal mask:
  // launch them first.
  const int nbh = a.B * a.Hkv;
  const int kt = blockIdx.x / nbh;
  const int bh = blockIdx.x % nbh;
  const int b = bh / a.Hkv;
  const int hkv = bh - b * a.Hkv;
  const int k0 = kt * kBwdBN;
  const int kw = k0 + kq * 32;
  const int key = kw + col;  // this lane's key (column of S)
  const size_t kvbase = ((size_t)b * a.Hkv + hkv) * (size_t)S * D;

  // DMA: wave w fills blocks i * 8 + w of a tile; block bl holds rows 16 (bl / CG) ..,
  // chunks 4 (bl % CG) ..; lane l fetches row l / 4 of it, chunk (l % 4) ^ ((l / 16) % 4).
  const int dl_r = lane >> 2, dl_c = (lane & 3) ^ ((lane >> 4) & 3);
  // K and V tiles -> LDS for the whole run (rows past the end are clamped to a real
  // row; their probabilities are masked to 0).
#pragma unroll
  for (int i = 0; i < KDMAS; ++i) {
    const int bl = i * 8 + wave;
    const int r = (bl / CG) * 16 + dl_r;
    const size_t src = kvbase + (size_t)min(k0 + r, S - 1) * D + ((bl % CG) * 4 + dl_c) * 8;
    dma16(a.k + src, k_lds + (i * 8 + wave_u) * 512);
    dma16(a.v + src, v_lds + (i * 8 + wave_u) * 512);
  }

  const int nqt = (S + kBwdBM - 1) / kBwdBM;
  const int q_first = CAUSAL ? (k0 / kBwdBM) : 0;
  const int per_head = nqt - q_first;
  const int steps = G * per_head;
  const int S_pad = (S + kBwdBM - 1) / kBwdBM * kBwdBM;

  // Per-lane byte offsets of the Q / dO DMA within a tile.
  uint32_t qd_off[QDMAS];
#pragma unroll
  for (int i = 0; i < QDMAS; ++i) {
    const int bl = i * 8 + wave;
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
    const size_t rbase = ((size_t)b * a.Hq + hq) * (size_t)S;
    const int q0 = qt * kBwdBM;
    const char* qb = (const char*)(a.q + (rbase + q0) * D);
    const char* ob = (const char*)(a.dO + (rbase + q0) * D);
    if (q0 + kBwdBM <= S) {
#pragma unroll
      for (int i = 0; i < QDMAS; ++i) {
        dma16_s(qb, qd_off[i], q_lds[st] + (i * 8 + wave_u) * 512);
        dma16_s(ob, qd_off[i], do_lds[st] + (i * 8 + wave_u) * 512);
      }
    } else {
      int lr = dl_r;
      __asm__ volatile("" : "+v"(lr));  // keep this rare path's row arithmetic inside it
#pragma unroll
      for (int i = 0; i < QDMAS; ++i) {
        const int row = ((i * 8 + wave) / CG) * 16 + lr;  // row within the tile
        const int rc = min(q0 + row, S - 1) - q0;
        const uint32_t off = qd_off[i] + (uint32_t)((rc - row) * ROWB);
        dma16_s(qb, off, q_lds[st] + (i * 8 + wave_u) * 512);
        dma16_s(ob, off, do_lds[st] + (i * 8 + wave_u) * 512);
      }
    }
    // LSE log2e (wave 0) and D (wave 1) of the 64 queries: 16 lanes x 16 bytes each.
    if (wave_u < 2) {
      const size_t pbase = ((size_t)b * a.Hq + hq) * (size_t)S_pad + q0;
      const void* src = uniform_ptr((wave_u == 0 ? a.lse2 : a.delta) + pbase);
      if (lane < 16) dma16_s(src, (uint32_t)lane * 16u, &sd_lds[st][wave_u * kBwdBM]);
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

  f32x16 dk_acc[DBLK], dv_acc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
    dk_acc[db] = f32x16{};
    dv_acc[db] = f32x16{};
  }
  const float c = a.scale * kLog2e;  // signed: no running maximum is needed here

  // One step on stage ST; MASKED adds the causal / end-of-sequence mask to P.
  auto compute = [&](const int q0, auto stage, auto masked) {
    constexpr int ST = decltype(stage)::value;
    constexpr bool MASKED = decltype(masked)::value;
    // Tile offsets from the lane bases (ra*, tr* hold Q stage 0; rb* hold K).
    constexpr int QS = ST * 2 * QT, OS = DO_OFF - Q_OFF + ST * 2 * QT, VS = V_OFF - K_OFF;
    const char* L = (const char*)smem;
    const float* sd = sd_lds[ST];
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
    auto issue = [&](const int i) {
      if (i < 2 * KSTEPS) {
        const int ks = i % KSTEPS;
        const int o = (ks >> 1) * 1024;
        const int ao = (i < KSTEPS ? QS : OS) + o, bo = (i < KSTEPS ? 0 : VS) + o;
        fa[i] = *(const bf16x8*)(L + ((ks & 1) ? ra1 : ra0) + ao);
        fb[i] = *(const bf16x8*)(L + ((ks & 1) ? rb1 : rb0) + bo);
      } else if (i < NS) {
        const int p = (i - 2 * KSTEPS) % (2 * DBLK), t = p / DBLK, db = p % DBLK;
        const int o = (i < 3 * KSTEPS ? OS : QS) + (t * CG + db) * 1024;
        tlo[i] = lds_read_tr16((const uint16_t*)(L + tr0 + o));
        thi[i] = lds_read_tr16((const uint16_t*)(L + tr1 + o));
      }
      if (i < 4) l4[i] = *(const f32x4*)(&sd[qh * 32 + i * 8 + half * 4]);
      // -D of the lane's 16 query rows, in the accumulator's register order: the first dP
      // product takes it as its accumulator input, so the chain ends at dP - D.
      if (i >= KSTEPS - 4 && i < KSTEPS) {
        const int g4 = i - (KSTEPS - 4);
        d4[g4] = *(const f32x4*)(&sd[kBwdBM + qh * 32 + g4 * 8 + half * 4]);
      }
    };

    f32x16 sacc = f32x16{}, dpacc;
    uint32_t pw[2][4], sw[2][4];  // P and dS packed to bf16 pairs: [t][pair], registers v = 8t ..
#pragma unroll
    for (int i = 0; i < PD; ++i) issue(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      issue(i + PD);
      if (i < KSTEPS) {
        sacc = mfma32(fa[i], fb[i], sacc);
      } else if (i < 2 * KSTEPS) {
        if (i == KSTEPS) {
          const f32x16 nd = {d4[0][0], d4[0][1], d4[0][2], d4[0][3], d4[1][0], d4[1][1], d4[1][2], d4[1][3],
                             d4[2][0], d4[2][1], d4[2][2], d4[2][3], d4[3][0], d4[3][1], d4[3][2], d4[3][3]};
          dpacc = mfma32(fa[i], fb[i], nd);
        } else {
          dpacc = mfma32(fa[i], fb[i], dpacc);
        }
        // P for a share of the 16 registers, once S has had two slots to finish.
        const int j = i - KSTEPS - 2;
        if (j >= 0) {
          const int n = KSTEPS - 2, e0 = j * 16 / n, e1 = (j + 1) * 16 / n;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            if (v < e0 || v >= e1) continue;
            float p = exp2_sm<EXPMODE, false>(fmaf(sacc[v], c, -l4[v >> 2][v & 3]));
            if constexpr (MASKED) {
              const int ev = (v >> 2) * 8 + (v & 3);
              p = (ev < lim_c || ev >= lim_s) ? 0.0f : p;
            }
            sacc[v] = p;
            if (v & 1) pw[v >> 3][(v & 7) >> 1] = pack_bf16x2(sacc[v - 1], p);
          }
        }
      } else if (i < 3 * KSTEPS) {
        const int p = i - 2 * KSTEPS, t = p / DBLK, db = p % DBLK;
        const u32x4 w = {pw[t][0], pw[t][1], pw[t][2], pw[t][3]};
        dv_acc[db] = mfma32(join(tlo[i], thi[i]), __builtin_bit_cast(bf16x8, w), dv_acc[db]);
        // dS for a share of the 16 registers, once dP has had two slots to finish.
        const int j = p - 2;
        if (j >= 0) {
          const int n = 2 * DBLK - 2, e0 = j * 16 / n, e1 = (j + 1) * 16 / n;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            if (v < e0 || v >= e1) continue;
            const float ds = sacc[v] * dpacc[v];
            dpacc[v] = ds;
            if (v & 1) sw[v >> 3][(v & 7) >> 1] = pack_bf16x2(dpacc[v - 1], ds);
          }
        }
      } else {
        const int p = i - 3 * KSTEPS, t = p / DBLK, db = p % DBLK;
        const u32x4 w = {sw[t][0], sw[t][1], sw[t][2], sw[t][3]};
        dk_acc[db] = mfma32(join(tlo[i], thi[i]), __builtin_bit_cast(bf16x8, w), dk_acc[db]);
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
    const int q0 = qt * kBwdBM;
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
  for (int step = 0; step < steps; step += 2) {
    do_step(step, std::integral_constant<int, 0>{});
    if (step + 1 < steps) do_step(step + 1, std::integral_constant<int, 1>{});
  }

  // Add the two query halves' partial dK, dV through LDS (the Q/dO stages are free now),
  // then dK = scale dK_acc, dV = dV_acc.
  float* red = reinterpret_cast<float*>(smem + Q_OFF);  // 4 waves x DBLK x 16 x 64 floats
  static_assert(SD_OFF - Q_OFF >= 4 * DBLK * 16 * 64 * (int)sizeof(float), "reduction space");
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
  if (qh == 0 && key < S) {
    const float ks = a.scale;
    // The lane's half, recomputed here rather than kept live across the loop.
    const int half = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) >> 5;
    uint16_t* dkr = a.dk + kvbase + (size_t)key * D;
    uint16_t* dvr = a.dv + kvbase + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        u32x2 wk, wv;
        wk[0] = pack_bf16x2(dk_acc[db][g4 * 4 + 0] * ks, dk_acc[db][g4 * 4 + 1] * ks);
        wk[1] = pack_bf16x2(dk_acc[db][g4 * 4 + 2] * ks, dk_acc[db][g4 * 4 + 3] * ks);
        wv[0] = pack_bf16x2(dv_acc[db][g4 * 4 + 0], dv_acc[db][g4 * 4 + 1]);
        wv[1] = pack_bf16x2(dv_acc[db][g4 * 4 + 2], dv_acc[db][g4 * 4 + 3]);
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
// K and V tiles sit in LDS as XOR chunk-inner blocks (attn_device.h), filled by coalesced
// DMA; both the operand reads of K and V and the transpose reads of K^T are free of bank
// conflicts.  One tile is 48 fenced slots of one product each: S^T (16), then dP^T
// beside P^T = 2^(S^T c - LSE log2 e) computed in place of S^T, then dQ^T beside
// dS^T = P^T (dP^T - D) computed in place of dP^T, one 8-key block ahead of the products
// that use it.  LDS reads run two slots ahead.
constexpr int kDqBM = 128;  // queries per workgroup
constexpr int kDqBN = 64;   // keys per tile

template <int D, bool CAUSAL, int EXPMODE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdArgs a) {
  constexpr int BN = kDqBN;
  constexpr int KB = BN / 32;           // 32-key blocks per tile
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int CG = D / 32;            // 4-chunk groups per row
  constexpr int ROWB = D * 2;           // bytes per row in memory
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
  const int S = a.S;
  const int S_pad = (S + kBwdBM - 1) / kBwdBM * kBwdBM;

  const int nbh = a.B * a.Hq;
  const int nqt = (S + kDqBM - 1) / kDqBM;
  const int bid = blockIdx.x;
  const int qt = CAUSAL ? (nqt - 1 - bid / nbh) : (bid / nbh);
  // Head of this workgroup, as in the forward: with B * Hkv a multiple of 8, every query
  // head and query tile of one KV group lands on one XCD (XCD = bid % 8) and reads K and
  // V through one L2.
  const int G = a.Hq / a.Hkv;
  const int u = bid % nbh;
  int kvg, g;
  if (((a.B * a.Hkv) & 7) == 0) {
    const int jj = u >> 3;
    kvg = (jj / G) * 8 + (u & 7);
    g = jj - (jj / G) * G;
  } else {
    kvg = u / G;
    g = u - kvg * G;
  }
  const int b = kvg / a.Hkv;
  const int hkv = kvg - b * a.Hkv;
  const int hq = hkv * G + g;
  const int q0 = qt * kDqBM;
  const int qw = q0 + wave * 32;
  const int qi = qw + col;  // this lane's query
  const int qc = min(qi, S - 1);  // rows past the end read the last row; never stored
  const size_t qbase = ((size_t)b * a.Hq + hq) * (size_t)S * D;
  const size_t kvbase = ((size_t)b * a.Hkv + hkv) * (size_t)S * D;
  const uint16_t* __restrict__ Kg = a.k + kvbase;
  const uint16_t* __restrict__ Vg = a.v + kvbase;

  // Q^T and dO^T fragments (B operands): query qc, d = ks*16 + half*8 .. +7.
  bf16x8 qf[KSTEPS], of[KSTEPS];
  {
    const u32x4* qrow = (const u32x4*)(a.q + qbase + (size_t)qc * D + half * 8);
    const u32x4* orow = (const u32x4*)(a.dO + qbase + (size_t)qc * D + half * 8);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      qf[ks] = __builtin_bit_cast(bf16x8, qrow[ks * 2]);
      of[ks] = __builtin_bit_cast(bf16x8, orow[ks * 2]);
    }
  }
  const size_t prow = ((size_t)b * a.Hq + hq) * (size_t)S_pad + qc;
  const float lse2 = a.lse2[prow];
  const float nd = a.delta[prow];  // -D
  // dP^T chains start from -D (every register of a lane belongs to its query), so the
  // products give dP^T - D directly and dS^T = P^T (dP^T - D) is one multiply.
  f32x16 negd;
#pragma unroll
  for (int v = 0; v < 16; ++v) negd[v] = nd;
  const float c = a.scale * kLog2e;  // signed: no running maximum is needed here

  const int kv_end = CAUSAL ? min(S, q0 + kDqBM) : S;
  const int nkv = (kv_end + BN - 1) / BN;

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
    const char* base = (const char*)(src + (size_t)j * BN * D);
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
      lim = CAUSAL ? min(lim_s, qi - k0 - half * 4) : lim_s;
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
        const float ds = s[kb][v] * dp[kb][v];
        dp[kb][v] = ds;
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
      dp[kb] = mfma32(fr[i], of[ks], ks == 0 ? negd : dp[kb]);
      // P^T for a share of the 32 scores, once S^T has had a slot to finish.
      if (k >= 1) {
        const int n = NA - 1, e0 = (k - 1) * 2 * 16 / n, e1 = k * 2 * 16 / n;
#pragma unroll
        for (int e = 0; e < 2 * 16; ++e) {
          if (e < e0 || e >= e1) continue;
          float p = exp2_sm<EXPMODE, false>(fmaf(s[e >> 4][e & 15], c, -lse2));
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
    if (!CAUSAL || k0 <= qw + 31) {
      const bool need_mask = (k0 + BN > S) || (CAUSAL && k0 + BN - 1 > qw);
      if (need_mask) {
        compute(j, parity, std::true_type{});
      } else {
        compute(j, parity, std::false_type{});
      }
    }
    wait_dma();
    __syncthreads();
  };

  dma_tile(Kg, 0, Kring);
  dma_tile(Vg, 0, Vring);
  wait_dma();
  __syncthreads();
  for (int j = 0; j < nkv; j += 2) {
    step(j, std::integral_constant<int, 0>{});
    if (j + 1 < nkv) step(j + 1, std::integral_constant<int, 1>{});
  }

  if (qi < S) {
    uint16_t* dqr = a.dq + qbase + (size_t)qi * D;
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

template <int D, bool CAUSAL, int EXPMODE>
hipError_t launch_bwd_t(const BwdArgs& a, int phases, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (phases & 1) {
    const int S_pad = (a.S + kBwdBM - 1) / kBwdBM * kBwdBM;
    const long prows = (long)a.B * a.Hq * S_pad;
    const long pre_threads = prows * (D / 8);
    hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((unsigned)((pre_threads + 255) / 256)), dim3(256), 0, stream,
                       a.o, a.dO, a.lse, a.delta, a.lse2, prows, a.S, S_pad);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (phases & 2) {
    const int nkt = (a.S + kBwdBN - 1) / kBwdBN;
    hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL, EXPMODE>), dim3((unsigned)(nkt * a.B * a.Hkv)), dim3(512), 0,
                       stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (phases & 4) {
    const int nqt = (a.S + kDqBM - 1) / kDqBM;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, EXPMODE>), dim3((unsigned)(nqt * a.B * a.Hq)), dim3(256), 0,
                       stream, a);
    e = hipGetLastError();
  }
  return e;
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, bool causal, int exp_mode, int phases, hipStream_t stream) {
  if (causal) {
    return exp_mode == 0 ? launch_bwd_t<D, true, 0>(a, phases, stream) : launch_bwd_t<D, true, 1>(a, phases, stream);
  }
  return exp_mode == 0 ? launch_bwd_t<D, false, 0>(a, phases, stream) : launch_bwd_t<D, false, 1>(a, phases, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int d, bool causal, int exp_mode, int phases, hipStream_t stream) {
  return d == 64 ? launch_bwd_d<64>(a, causal, exp_mode, phases, stream)
                 : launch_bwd_d<128>(a, causal, exp_mode, phases, stream);
}

}  // namespace attn
