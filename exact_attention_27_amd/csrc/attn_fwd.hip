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
constexpr int kFwdBM = 32 * kFwdWaves;  // queries per workgroup
constexpr int kFwdBN = 64;              // keys per LDS tile

template <int D, bool CAUSAL, int EXPMODE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdArgs a) {
  constexpr int BN = kFwdBN;
  constexpr int KSTEPS = D / 16;  // MFMA k-steps of S^T = K Q^T
  constexpr int DBLK = D / 32;    // 32-row blocks of O^T
  constexpr int CPR = D / 8;      // 16-byte chunks per row
  constexpr int TILE = BN * D;    // bf16 elements of one K or V tile
  constexpr int LOADS = BN * CPR / 256;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * TILE];  // [stage][K|V][BN][D]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;
  const int half = lane >> 5;

  const int nbh = a.B * a.Hq;
  const int nqt = (a.S + kFwdBM - 1) / kFwdBM;
  const int bid = blockIdx.x;
  const int qt = CAUSAL ? (nqt - 1 - bid / nbh) : (bid / nbh);
  const int bh = bid % nbh;
  const int b = bh / a.Hq;
  const int hq = bh - b * a.Hq;
  const int hkv = hq / (a.Hq / a.Hkv);
  const int S = a.S;
  const int q0 = qt * kFwdBM;
  const int qw = q0 + wave * 32;
  const int qi = qw + col;  // this lane's query
  const size_t qbase = ((size_t)b * a.Hq + hq) * (size_t)S * D;
  const size_t kvbase = ((size_t)b * a.Hkv + hkv) * (size_t)S * D;
  const uint16_t* __restrict__ Kg = a.k + kvbase;
  const uint16_t* __restrict__ Vg = a.v + kvbase;

  // Q^T fragments (B operand): query qi, d = ks*16 + half*8 .. +7.
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (qi < S) {
      w = *(const u32x4*)(a.q + qbase + (size_t)qi * D + ks * 16 + half * 8);
      w = (w & a.q_and) ^ a.q_xor;
    }
    qf[ks] = __builtin_bit_cast(bf16x8, w);
  }

  const int kv_end = CAUSAL ? min(S, q0 + kFwdBM) : S;
  const int nkv = (kv_end + BN - 1) / BN;

  // Global -> register staging of one K tile and one V tile (16-byte chunks, rows past
  // the end of the sequence are zero so that masked probabilities meet finite values).
  u32x4 kreg[LOADS], vreg[LOADS];
  auto gload = [&](int j) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int id = i * 256 + tid;
      const int r = id / CPR, c = id % CPR;
      const int key = j * BN + r;
      if (key < S) {
        kreg[i] = *(const u32x4*)(Kg + (size_t)key * D + c * 8);
        vreg[i] = *(const u32x4*)(Vg + (size_t)key * D + c * 8);
      } else {
        kreg[i] = u32x4{0u, 0u, 0u, 0u};
        vreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto sstore = [&](int stage) {
    uint16_t* Ks = smem + stage * 2 * TILE;
    uint16_t* Vs = Ks + TILE;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int id = i * 256 + tid;
      const int r = id / CPR, c = id % CPR;
      const int off = r * D + (swz_chunk<D>(r, c) << 3);
      *(u32x4*)(Ks + off) = kreg[i];
      *(u32x4*)(Vs + off) = vreg[i];
    }
  };

  // Per-lane parts of the V^T transpose-read addresses (see attn_device.h): source
  // lane s reads 4 d-values of key row (s / 32) * 4 + (s % 16) / 4 (+ 8 for the second
  // read), at column 16 * ((s / 16) % 2) + 4 * (s % 4) of a 32-wide d block.
  const int vrow = (lane >> 5) * 4 + ((lane >> 2) & 3);
  const int vcol = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;

  f32x16 oacc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) oacc[db] = f32x16{};
  float m_ref = -INFINITY;  // reference row maximum, log2 units (scaled scores)
  float l_part = 0.0f;      // this lane's part of the running row sum
  const float c = a.c;
  const float tau = a.tau;

  gload(0);
  sstore(0);
  __syncthreads();

  for (int j = 0; j < nkv; ++j) {
    const int stage = j & 1;
    if (j + 1 < nkv) gload(j + 1);
    const int k0 = j * BN;
    // A wave skips tiles whose keys all lie above its last query (causal).
    if (!CAUSAL || k0 <= qw + 31) {
      const uint16_t* Ks = smem + stage * 2 * TILE;
      const uint16_t* Vs = Ks + TILE;

      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 ka = *(const bf16x8*)(Ks + swz<D>(kb * 32 + col, ks * 16 + half * 8));
          s[kb] = mfma32(ka, qf[ks], s[kb]);
        }
      }

      const bool need_mask = (k0 + BN > S) || (CAUSAL && k0 + BN - 1 > qw);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = k0 + kb * 32 + (v >> 2) * 8 + half * 4 + (v & 3);
            if (key >= S || (CAUSAL && key > qi)) s[kb][v] = -INFINITY;
          }
        }
      }

      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
      }
      mx = max_halves(mx);
      const float mt = mx * c;
      if (wave_any(mt > m_ref + tau)) {
        const float m_new = fmaxf(m_ref, mt);
        const float alpha = (m_new == -INFINITY) ? 1.0f : exp2_sm<0>(m_ref - m_new);
#pragma unroll
        for (int db = 0; db < DBLK; ++db) oacc[db] *= alpha;
        l_part *= alpha;
        m_ref = m_new;
      }
      const float mu = (m_ref == -INFINITY) ? 0.0f : m_ref;

      bf16x8 pf[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = exp2_sm<EXPMODE>(fmaf(s[kb][t * 8 + 2 * e], c, -mu));
            const float p1 = exp2_sm<EXPMODE>(fmaf(s[kb][t * 8 + 2 * e + 1], c, -mu));
            l_part += p0 + p1;
            w[e] = pack_bf16x2(p0, p1);
          }
          pf[kb][t] = __builtin_bit_cast(bf16x8, w);
        }
      }

#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int row = kb * 32 + t * 16 + vrow;
#pragma unroll
          for (int db = 0; db < DBLK; ++db) {
            const i16x4 lo = lds_read_tr16(Vs + swz<D>(row, db * 32 + vcol));
            const i16x4 hi = lds_read_tr16(Vs + swz<D>(row + 8, db * 32 + vcol));
            oacc[db] = mfma32(join(lo, hi), pf[kb][t], oacc[db]);
          }
        }
      }
    }
    if (j + 1 < nkv) sstore(stage ^ 1);
    __syncthreads();
  }

  // Epilogue: O = O_acc / l (bf16, round to nearest even) and LSE in natural log.
  const float l = sum_halves(l_part);
  const float inv = 1.0f / l;
  if (qi < S) {
    uint16_t* orow = a.o + qbase + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][g * 4 + 0] * inv, oacc[db][g * 4 + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][g * 4 + 2] * inv, oacc[db][g * 4 + 3] * inv);
        *(u32x2*)(orow + db * 32 + g * 8 + half * 4) = w;
      }
    }
    if (half == 0) a.lse[((size_t)b * a.Hq + hq) * S + qi] = (m_ref + log2f(l)) * kLn2;
  }
}

template <int D, bool CAUSAL, int EXPMODE>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const int nqt = (a.S + kFwdBM - 1) / kFwdBM;
  const dim3 grid((unsigned)(nqt * a.B * a.Hq));
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, EXPMODE>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_d(const FwdArgs& a, bool causal, int exp_mode, hipStream_t stream) {
  if (causal) {
    return exp_mode == 0 ? launch_fwd_t<D, true, 0>(a, stream) : launch_fwd_t<D, true, 1>(a, stream);
  }
  return exp_mode == 0 ? launch_fwd_t<D, false, 0>(a, stream) : launch_fwd_t<D, false, 1>(a, stream);
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
