// attn_fwd.hip - forward pass of exact attention on gfx950 (CDNA4).
//
// One workgroup of 4 waves owns 128 consecutive queries of one (batch, query head);
// each wave owns 32 of them.  The workgroup walks the key/value sequence in tiles of
// 64 keys that are staged through LDS and shared by its 4 waves; the S x S score
// matrix never leaves registers (the memory-traffic argument of "NVIDIA Blackwell:
// FlashAttention-4 Overcomes Memory Bottlenecks", body paragraph, and of the
// hyper.ai FlashAttention-4 story).
//
// Per key tile, each wave computes the transposed scores S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (K from LDS as the A operand, Q^T held in registers as the
// B operand).  In that accumulator layout a lane holds 16 keys of ONE query column,
// so the running row maximum and row sum of the online softmax are in-lane
// reductions plus one v_permlane32_swap between the two wave halves.  The
// probabilities P^T are packed to bf16 straight from the accumulator registers and
// used as the B operand of O^T += V^T P^T; V^T comes from the row-major V tile
// through ds_read_b64_tr_b16 (LDS transpose reads).  The output accumulator O^T keeps
// the same one-query-per-lane layout, so rescaling it by a per-row factor is a plain
// per-lane multiply.
//
// Online softmax with conditional rescaling (the "adaptive online softmax rescaling"
// of "NVIDIA's FlashAttention-4", section "The Technical Edge": rescale only when the
// maximum changes significantly): each row keeps a reference maximum m_ref in log2
// units.  When a tile's maximum exceeds m_ref + tau anywhere in the wave, the wave
// rescales O^T and the running sum by 2^(m_ref - m_new) and moves m_ref; otherwise
// the probabilities 2^(x - m_ref) are used as they are (they stay <= 2^tau).  Since
// O and the sum always share m_ref, the final O = O_acc / l is exact for every tau.
//
// Causal masking: key tiles above the diagonal of the workgroup are never loaded;
// only tiles that straddle the diagonal or the end of the sequence are masked.
// Workgroups are dispatched longest-first (largest query tile index first), and all
// query tiles of one head are spaced B*Hq workgroups apart so that, when B*Hq is a
// multiple of 8, they run on one XCD and share its L2 for K and V.
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

constexpr int kFwdWaves = 4;
constexpr int kFwdBN = 64;  // keys per LDS tile


// NQB = 32-query column blocks per wave.  NQB = 2 reuses every K and V operand read
// from LDS for two MFMAs (half the LDS traffic per MFMA) at twice the registers, so it
// runs one wave per SIMD; NQB = 1 runs two.
template <int D, bool CAUSAL, int EXPMODE, int NQB>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(NQB == 1 ? 2 : 1, NQB == 1 ? 2 : 1)))
void fwd_kernel(FwdArgs a) {
  constexpr int BN = kFwdBN;
  constexpr int WQ = 32 * NQB;          // queries per wave
  constexpr int BM = WQ * kFwdWaves;    // queries per workgroup
  constexpr int KSTEPS = D / 16;        // MFMA k-steps of S^T = K Q^T
  constexpr int DBLK = D / 32;          // 32-row blocks of O^T
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int TILE = BN * D;          // bf16 elements of one K or V tile
  constexpr int DMAS = BN * CPR / 256;  // 16-byte chunks per thread per tile
  // K ring (2 tiles) then V ring (2 tiles), each tile [BN][D] with swizzled chunks.
  __shared__ __attribute__((aligned(1024))) uint16_t smem[4 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;
  const int half = lane >> 5;

  const int nbh = a.B * a.Hq;
  const int nqt = (a.S + BM - 1) / BM;
  const int bid = blockIdx.x;
  const int qt = CAUSAL ? (nqt - 1 - bid / nbh) : (bid / nbh);
  const int bh = bid % nbh;
  const int b = bh / a.Hq;
  const int hq = bh - b * a.Hq;
  const int hkv = hq / (a.Hq / a.Hkv);
  const int S = a.S;
  const int q0 = qt * BM;
  const int qw = q0 + wave * WQ;  // first query of this wave; block qb holds qw + 32 qb ..
  const size_t qbase = ((size_t)b * a.Hq + hq) * (size_t)S * D;
  const size_t kvbase = ((size_t)b * a.Hkv + hkv) * (size_t)S * D;
  const uint16_t* __restrict__ Kg = a.k + kvbase;
  const uint16_t* __restrict__ Vg = a.v + kvbase;

  // Q^T fragments (B operand): query qw + 32 qb + col, d = ks*16 + half*8 .. +7.
  bf16x8 qf[NQB][KSTEPS];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int qi = qw + qb * 32 + col;
    // Rows past the end of the sequence load the last row instead (their outputs are
    // never stored); no branch, so all the loads are in flight together.
    const u32x4* qrow = (const u32x4*)(a.q + qbase + (size_t)min(qi, S - 1) * D + half * 8);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const u32x4 w = (qrow[ks * 2] & a.q_and) ^ a.q_xor;
      qf[qb][ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int kv_end = CAUSAL ? min(S, q0 + BM) : S;
  const int nkv = (kv_end + BN - 1) / BN;

  // DMA of one tile into a ring slot.  Thread tid, chunk i covers LDS chunk
  // p = (i * 4 + wave) * 64 + lane = (row, physical chunk); it fetches the logical chunk
  // physical ^ f(row) of key row j*BN + row.  The per-lane byte offsets within a tile
  // are fixed, the tile base is a scalar; only the last tile, if it runs past the end of
  // the sequence, clamps its rows to a real row (their scores are masked, so any finite
  // data will do).
  uint32_t dma_off[DMAS];
#pragma unroll
  for (int i = 0; i < DMAS; ++i) {
    const int pch = (i * 4 + wave) * 64 + lane;
    const int r = pch / CPR;
    dma_off[i] = (uint32_t)(r * D + swz_chunk<D>(r, pch % CPR) * 8) * 2u;
  }
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto dma_tile = [&](const uint16_t* __restrict__ src, int j, uint16_t* slot) {
    const uint16_t* base = src + (size_t)j * BN * D;
    if (j * BN + BN <= S) {
#pragma unroll
      for (int i = 0; i < DMAS; ++i) dma16_s(base, dma_off[i], slot + (i * 4 + wave_u) * 512);
    } else {
#pragma unroll
      for (int i = 0; i < DMAS; ++i) {
        const int pch = (i * 4 + wave) * 64 + lane;
        const int r = pch / CPR;
        const int rc = min(j * BN + r, S - 1) - j * BN;
        const uint32_t off = (uint32_t)(rc * D + swz_chunk<D>(r, pch % CPR) * 8) * 2u;
        dma16_s(base, off, slot + (i * 4 + wave_u) * 512);
      }
    }
  };
  uint16_t* const Kring = smem;
  uint16_t* const Vring = smem + 2 * TILE;

  // Per-lane parts of the V^T transpose-read addresses (see attn_device.h): source
  // lane s reads 4 d-values of key row (s / 32) * 4 + (s % 16) / 4 (+ 8 for the second
  // read), at column 16 * ((s / 16) % 2) + 4 * (s % 4) of a 32-wide d block.
  const int vrow = (lane >> 5) * 4 + ((lane >> 2) & 3);
  const int vcol = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;

  f32x16 oacc[NQB][DBLK];
  float m_ref[NQB], l_run[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
    for (int db = 0; db < DBLK; ++db) oacc[qb][db] = f32x16{};
    m_ref[qb] = -INFINITY;  // reference row maximum, log2 units (scaled scores)
    l_run[qb] = 0.0f;       // this lane's part of the running row sum
  }
  const float c = a.c;
  const float tau = a.tau;

  // S^T = K Q^T for every query block: each K fragment read from LDS feeds NQB MFMAs.
  auto qk = [&](const uint16_t* Ks, f32x16 (*s)[2]) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) s[qb][0] = s[qb][1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 ka = *(const bf16x8*)(Ks + swz<D>(kb * 32 + col, ks * 16 + half * 8));
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) s[qb][kb] = mfma32(ka, qf[qb][ks], s[qb][kb]);
      }
    }
  };
  auto mask = [&](f32x16 (*s)[2], int k0) {
    if ((k0 + BN > S) || (CAUSAL && k0 + BN - 1 > qw)) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int qi = qw + qb * 32 + col;
        const int lim_s = S - 1 - k0 - half * 4;               // key <= S - 1
        const int lim = CAUSAL ? min(lim_s, qi - k0 - half * 4) : lim_s;  // key <= query
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int e = kb * 32 + (v >> 2) * 8 + (v & 3);  // key - k0 - half*4
            s[qb][kb][v] = e > lim ? -INFINITY : s[qb][kb][v];
          }
        }
      }
    }
  };
  // P = 2^(s c - m) packed to bf16 in the B-operand layout of O^T += V^T P^T.
  auto softmax_exp = [&](const f32x16* s, float m, bf16x8 (*pf)[2]) {
    float lt = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = exp2_sm<EXPMODE>(fmaf(s[kb][t * 8 + 2 * e], c, -m));
          const float p1 = exp2_sm<EXPMODE>(fmaf(s[kb][t * 8 + 2 * e + 1], c, -m));
          lt += p0 + p1;
          w[e] = pack_bf16x2(p0, p1);
        }
        pf[kb][t] = __builtin_bit_cast(bf16x8, w);
      }
    }
    return lt;
  };

  // Prologue: K_0, V_0, K_1 in flight; S_0 computed.
  dma_tile(Kg, 0, Kring);
  dma_tile(Vg, 0, Vring);
  if (nkv > 1) dma_tile(Kg, 1, Kring + TILE);
  wait_dma();
  __syncthreads();
  f32x16 sc[NQB][2];
  qk(Kring, sc);
  mask(sc, 0);

  for (int j = 0; j < nkv; ++j) {
    // Free slots: K_j's (read by the previous step's QK) and V_{j-1}'s (read by its PV).
    if (j + 2 < nkv) dma_tile(Kg, j + 2, Kring + (j & 1) * TILE);
    if (j + 1 < nkv) dma_tile(Vg, j + 1, Vring + ((j + 1) & 1) * TILE);
    // Free slots: K_j's (read by the previous step's QK) and V_{j-1}'s (read by its PV).

    // Running maximum and the (rare) rescale, before the step's main block.  One
    // wave-uniform branch covers every query block of the wave.
    float mt[NQB];
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[qb][kb][v]);
      }
      mt[qb] = max_halves(mx) * c;
      grow = grow || (mt[qb] > m_ref[qb] + tau);
    }
    if (wave_any(grow)) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const float m_new = fmaxf(m_ref[qb], mt[qb]);
        const float alpha = (m_new == -INFINITY) ? 1.0f : exp2_sm<0>(m_ref[qb] - m_new);
#pragma unroll
        for (int db = 0; db < DBLK; ++db) oacc[qb][db] *= alpha;
        l_run[qb] *= alpha;
        m_ref[qb] = m_new;
      }
    }

    // Main block, free of branches: S_{j+1} = K_{j+1} Q^T on the matrix cores (its slot
    // holds stale data on the last step; the result is then unused) while the vector
    // units exponentiate S_j; then O^T += V_j^T P_j^T.
    f32x16 sn[NQB][2];
    qk(Kring + ((j + 1) & 1) * TILE, sn);
    bf16x8 pf[NQB][2][2];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
      l_run[qb] += softmax_exp(sc[qb], m_ref[qb] == -INFINITY ? 0.0f : m_ref[qb], pf[qb]);

    const uint16_t* Vs = Vring + (j & 1) * TILE;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int row = kb * 32 + t * 16 + vrow;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          const bf16x8 va = join(lds_read_tr16(Vs + swz<D>(row, db * 32 + vcol)),
                                 lds_read_tr16(Vs + swz<D>(row + 8, db * 32 + vcol)));
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) oacc[qb][db] = mfma32(va, pf[qb][kb][t], oacc[qb][db]);
        }
        // Bound the transpose reads in flight to one 16-key sub-block (register budget).
        if (kb * 2 + t < 3) __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_dma();
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      sc[qb][0] = sn[qb][0];
      sc[qb][1] = sn[qb][1];
    }
    if (j + 1 < nkv) mask(sc, (j + 1) * BN);
  }

  // Epilogue: O = O_acc / l (bf16, round to nearest even) and LSE in natural log.
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int qi = qw + qb * 32 + col;
    const float l = sum_halves(l_run[qb]);
    const float inv = 1.0f / l;
    if (qi < S) {
      uint16_t* orow = a.o + qbase + (size_t)qi * D;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w;
          w[0] = pack_bf16x2(oacc[qb][db][g * 4 + 0] * inv, oacc[qb][db][g * 4 + 1] * inv);
          w[1] = pack_bf16x2(oacc[qb][db][g * 4 + 2] * inv, oacc[qb][db][g * 4 + 3] * inv);
          *(u32x2*)(orow + db * 32 + g * 8 + half * 4) = w;
        }
      }
      if (half == 0) a.lse[((size_t)b * a.Hq + hq) * S + qi] = (m_ref[qb] + log2f(l)) * kLn2;
    }
  }
}

template <int D, bool CAUSAL, int EXPMODE, int NQB>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  constexpr int BM = 32 * NQB * kFwdWaves;
  const int nqt = (a.S + BM - 1) / BM;
  const dim3 grid((unsigned)(nqt * a.B * a.Hq));
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, EXPMODE, NQB>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

#ifndef FWD_NQB
#define FWD_NQB 1
#endif

template <int D>
hipError_t launch_fwd_d(const FwdArgs& a, bool causal, int exp_mode, hipStream_t stream) {
  constexpr int N = FWD_NQB;
  if (causal) {
    return exp_mode == 0 ? launch_fwd_t<D, true, 0, N>(a, stream) : launch_fwd_t<D, true, 1, N>(a, stream);
  }
  return exp_mode == 0 ? launch_fwd_t<D, false, 0, N>(a, stream) : launch_fwd_t<D, false, 1, N>(a, stream);
}

__global__ void exp2_eval_kernel(const float* x, float* y, long n, int mode) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = mode == 0 ? exp2_sm<0>(x[i]) : exp2_sm<1>(x[i]);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, int d, bool causal, int exp_mode, hipStream_t stream) {
  return d == 64 ? launch_fwd_d<64>(a, causal, exp_mode, stream) : launch_fwd_d<128>(a, causal, exp_mode, stream);
}

hipError_t launch_exp2_eval(const float* x, float* y, long n, int exp_mode, hipStream_t stream) {
  const long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(exp2_eval_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, y, n, exp_mode);
  return hipGetLastError();
}

}  // namespace attn
