// attn_bwd.hip - backward pass of exact attention on gfx950 (CDNA4).
//
// The backward recomputes the probabilities from the saved logsumexp instead of
// storing them (the pages keep backward intermediates on chip: hyper.ai
// FlashAttention-4 story; "NVIDIA Blackwell: FlashAttention-4 Overcomes Memory
// Bottlenecks", body paragraph).  Three launches on the caller's stream:
//
//  1. bwd_pre:    D_i = <dO_i, O_i> in fp32 from the stored bf16 O and dO, and the fp32
//                 dQ accumulator is zeroed.  Bound by HBM bandwidth.
//  2. bwd_main:   one workgroup per (batch, KV head, tile of 128 keys); each of its 4 waves
//                 owns 32 keys and keeps dK and dV for them in registers for the whole
//                 run.  The workgroup walks the query tiles (64 queries) of every query
//                 head of the GQA group that can see its keys (causal: only tiles at or
//                 below the diagonal).  Per step, with Q, dO, LSE and D staged in LDS:
//                     S   = Q K^T              (MFMA; K and V stay in LDS for the run)
//                     P   = 2^(S c - LSE log2 e), 0 where masked  (c = scale log2 e)
//                     dP  = dO V^T             (MFMA)
//                     dS  = P (dP - D)
//                     dV^T += dO^T P,  dK^T += Q^T dS   (dO^T and Q^T by LDS transpose reads)
//                 dS^T is written to LDS, and the 4 waves then compute the step's
//                 dQ = dS K over all 128 keys together (dS and K^T by transpose reads)
//                 and add it to the fp32 accumulator with hardware float atomics.
//                 Because the group's query heads loop inside the workgroup, dK and dV
//                 are summed over the group without atomics.
//  3. dq_convert: dQ = bf16(scale * accumulator).
//
// In the S accumulator layout (v_mfma_f32_32x32x16_bf16, A = Q rows, B = K^T) a lane
// holds one key column and 16 query rows; P and dS are packed to bf16 in registers and
// used directly as the B operand of the dV^T and dK^T products.
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {
namespace {

constexpr int kBwdBN = 128;  // keys per workgroup (4 waves x 32)
constexpr int kBwdBM = 64;   // queries per step

// ------------------------------------------------------------------ preprocess
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dO,
                                                      float* __restrict__ delta, float* __restrict__ dq_acc, long rows) {
  constexpr int LPR = D / 8;  // lanes per row, 8 bf16 each
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = gid / LPR;
  const int part = (int)(gid % LPR);
  float acc = 0.0f;
  if (row < rows) {
    const u32x4 ov = *(const u32x4*)(o + row * D + part * 8);
    const u32x4 dv = *(const u32x4*)(dO + row * D + part * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float o0 = __builtin_bit_cast(float, ov[e] << 16), o1 = __builtin_bit_cast(float, ov[e] & 0xffff0000u);
      const float d0 = __builtin_bit_cast(float, dv[e] << 16), d1 = __builtin_bit_cast(float, dv[e] & 0xffff0000u);
      acc = fmaf(o0, d0, acc);
      acc = fmaf(o1, d1, acc);
    }
    f32x4* z = (f32x4*)(dq_acc + row * D + part * 8);
    z[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    z[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) delta[row] = acc;
}

// ------------------------------------------------------------------ main
template <int D, bool CAUSAL, int EXPMODE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void bwd_main_kernel(BwdArgs a) {
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int CPR = D / 8;
  constexpr int QT = kBwdBM * D;               // elements of one Q or dO tile
  constexpr int QLOADS = kBwdBM * CPR / 256;   // 16-byte chunks per thread per tile
  constexpr int KLOADS = kBwdBN * CPR / 256;
  constexpr int NDB = DBLK / 2;                // dQ d-blocks per wave
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kBwdBN * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[kBwdBN * D];
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[QT];
  __shared__ __attribute__((aligned(16))) uint16_t do_lds[QT];
  __shared__ __attribute__((aligned(16))) uint16_t dst_lds[kBwdBN * kBwdBM];  // dS^T [key][query]
  __shared__ __attribute__((aligned(16))) float lse_lds[kBwdBM];
  __shared__ __attribute__((aligned(16))) float dd_lds[kBwdBM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;
  const int half = lane >> 5;
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
  const int kw = k0 + wave * 32;
  const int key = kw + col;  // this lane's key (column of S)
  const size_t kvbase = ((size_t)b * a.Hkv + hkv) * (size_t)S * D;

  // K and V tiles -> LDS for the whole run (rows past the end of the sequence are zero).
#pragma unroll
  for (int i = 0; i < KLOADS; ++i) {
    const int id = i * 256 + tid;
    const int r = id / CPR, c = id % CPR;
    u32x4 wk = {0u, 0u, 0u, 0u}, wv = {0u, 0u, 0u, 0u};
    if (k0 + r < S) {
      wk = *(const u32x4*)(a.k + kvbase + (size_t)(k0 + r) * D + c * 8);
      wv = *(const u32x4*)(a.v + kvbase + (size_t)(k0 + r) * D + c * 8);
    }
    const int off = r * D + (swz_chunk<D>(r, c) << 3);
    *(u32x4*)(k_lds + off) = wk;
    *(u32x4*)(v_lds + off) = wv;
  }

  const int nqt = (S + kBwdBM - 1) / kBwdBM;
  const int q_first = CAUSAL ? (k0 / kBwdBM) : 0;
  const int per_head = nqt - q_first;
  const int steps = G * per_head;

  // Register staging of the next step's Q, dO, LSE (log2 units) and D.
  u32x4 qreg[QLOADS], doreg[QLOADS];
  float lse_r = 0.0f, dd_r = 0.0f;
  auto gload = [&](int step) {
    const int g = step / per_head;
    const int qt = q_first + step - g * per_head;
    const int hq = hkv * G + g;
    const size_t rbase = ((size_t)b * a.Hq + hq) * (size_t)S;
    const int q0 = qt * kBwdBM;
#pragma unroll
    for (int i = 0; i < QLOADS; ++i) {
      const int id = i * 256 + tid;
      const int r = id / CPR, c = id % CPR;
      u32x4 wq = {0u, 0u, 0u, 0u}, wd = {0u, 0u, 0u, 0u};
      if (q0 + r < S) {
        wq = *(const u32x4*)(a.q + (rbase + q0 + r) * D + c * 8);
        wd = *(const u32x4*)(a.dO + (rbase + q0 + r) * D + c * 8);
      }
      qreg[i] = wq;
      doreg[i] = wd;
    }
    if (tid < kBwdBM) {
      const bool in = q0 + tid < S;
      lse_r = in ? a.lse[rbase + q0 + tid] * kLog2e : 0.0f;
      dd_r = in ? a.delta[rbase + q0 + tid] : 0.0f;
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < QLOADS; ++i) {
      const int id = i * 256 + tid;
      const int r = id / CPR, c = id % CPR;
      const int off = r * D + (swz_chunk<D>(r, c) << 3);
      *(u32x4*)(q_lds + off) = qreg[i];
      *(u32x4*)(do_lds + off) = doreg[i];
    }
    if (tid < kBwdBM) {
      lse_lds[tid] = lse_r;
      dd_lds[tid] = dd_r;
    }
  };

  // Transpose-read lane offsets (see attn_device.h and attn_fwd.hip).
  const int trow = (lane >> 5) * 4 + ((lane >> 2) & 3);
  const int tcol = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;

  f32x16 dk_acc[DBLK], dv_acc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
    dk_acc[db] = f32x16{};
    dv_acc[db] = f32x16{};
  }
  const float c = a.scale * kLog2e;  // signed: no running maximum is needed here

  if (steps > 0) gload(0);
  for (int step = 0; step < steps; ++step) {
    sstore();
    __syncthreads();  // this step's tiles are in LDS; the previous dQ product is done
    const int g = step / per_head;
    const int qt = q_first + step - g * per_head;
    const int hq = hkv * G + g;
    const int q0 = qt * kBwdBM;
    if (step + 1 < steps) gload(step + 1);

    if (!CAUSAL || kw <= q0 + kBwdBM - 1) {
      f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int koff = swz<D>(wave * 32 + col, ks * 16 + half * 8);
        const bf16x8 kf = *(const bf16x8*)(k_lds + koff);
        const bf16x8 vf = *(const bf16x8*)(v_lds + koff);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int off = swz<D>(qb * 32 + col, ks * 16 + half * 8);
          s[qb] = mfma32(*(const bf16x8*)(q_lds + off), kf, s[qb]);
          dp[qb] = mfma32(*(const bf16x8*)(do_lds + off), vf, dp[qb]);
        }
      }
      const bool need_mask = (kw + 32 > S) || (q0 + kBwdBM > S) || (CAUSAL && kw + 31 > q0);
      // P and dS, packed to bf16 as soon as they are formed.  Register v of query block
      // qb holds query qb*32 + (v/4)*8 + half*4 + v%4; pb[qb][t] / sb[qb][t] hold
      // registers v = 8t .. 8t+7, the B operand layout of the dV^T and dK^T products.
      bf16x8 pb[2][2], sb[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          u32x4 wp, wsd;
#pragma unroll
          for (int gg = 0; gg < 2; ++gg) {
            const int g4 = 2 * t + gg;
            const int qr = qb * 32 + g4 * 8 + half * 4;
            const f32x4 l4 = *(const f32x4*)(lse_lds + qr);
            const f32x4 d4 = *(const f32x4*)(dd_lds + qr);
            float pv[4], dsv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int v = g4 * 4 + r;
              float p = exp2_sm<EXPMODE>(fmaf(s[qb][v], c, -l4[r]));
              if (need_mask) {
                const int q = q0 + qr + r;
                if (key >= S || q >= S || (CAUSAL && key > q)) p = 0.0f;
              }
              pv[r] = p;
              dsv[r] = p * (dp[qb][v] - d4[r]);
            }
            wp[2 * gg] = pack_bf16x2(pv[0], pv[1]);
            wp[2 * gg + 1] = pack_bf16x2(pv[2], pv[3]);
            wsd[2 * gg] = pack_bf16x2(dsv[0], dsv[1]);
            wsd[2 * gg + 1] = pack_bf16x2(dsv[2], dsv[3]);
          }
          pb[qb][t] = __builtin_bit_cast(bf16x8, wp);
          sb[qb][t] = __builtin_bit_cast(bf16x8, wsd);
          // dS^T -> LDS: row = this lane's key, 4 consecutive queries per 8-byte store.
#pragma unroll
          for (int gg = 0; gg < 2; ++gg) {
            const u32x2 w = {wsd[2 * gg], wsd[2 * gg + 1]};
            *(u32x2*)(dst_lds + swz<kBwdBM>(wave * 32 + col, qb * 32 + (2 * t + gg) * 8 + half * 4)) = w;
          }
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int row = qb * 32 + t * 16 + trow;
#pragma unroll
          for (int db = 0; db < DBLK; ++db) {
            const int o0 = swz<D>(row, db * 32 + tcol), o1 = swz<D>(row + 8, db * 32 + tcol);
            dv_acc[db] = mfma32(join(lds_read_tr16(do_lds + o0), lds_read_tr16(do_lds + o1)), pb[qb][t], dv_acc[db]);
            dk_acc[db] = mfma32(join(lds_read_tr16(q_lds + o0), lds_read_tr16(q_lds + o1)), sb[qb][t], dk_acc[db]);
          }
        }
      }
    } else {
      // All of this wave's keys lie above the tile's last query: its dS^T rows are zero.
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int id = i * 64 + lane;
        *(u32x4*)(dst_lds + (wave * 32 + id / 8) * kBwdBM + (id % 8) * 8) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    __syncthreads();  // dS^T complete

    // dQ[64 x D] += dS[64 x 128] K[128 x D]; wave -> query block (wave / 2) and NDB d-blocks.
    {
      const int qbw = wave >> 1;
      f32x16 dq[NDB];
#pragma unroll
      for (int n = 0; n < NDB; ++n) dq[n] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < kBwdBN / 16; ++kk) {
        const int row = kk * 16 + trow;
        const bf16x8 sa = join(lds_read_tr16(dst_lds + swz<kBwdBM>(row, qbw * 32 + tcol)),
                               lds_read_tr16(dst_lds + swz<kBwdBM>(row + 8, qbw * 32 + tcol)));
#pragma unroll
        for (int n = 0; n < NDB; ++n) {
          const int db = (wave & 1) * NDB + n;
          const bf16x8 kb = join(lds_read_tr16(k_lds + swz<D>(row, db * 32 + tcol)),
                                 lds_read_tr16(k_lds + swz<D>(row + 8, db * 32 + tcol)));
          dq[n] = mfma32(sa, kb, dq[n]);
        }
      }
      float* dqa = a.dq_acc + ((size_t)b * a.Hq + hq) * (size_t)S * D;
#pragma unroll
      for (int n = 0; n < NDB; ++n) {
        const int dcol = ((wave & 1) * NDB + n) * 32 + col;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int q = q0 + qbw * 32 + (v >> 2) * 8 + half * 4 + (v & 3);
          if (q < S) atomicAdd(dqa + (size_t)q * D + dcol, dq[n][v]);
        }
      }
    }
  }

  // dK = scale dK_acc, dV = dV_acc.
  if (key < S) {
    const float ks = a.scale;
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

// ------------------------------------------------------------------ dQ convert
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ acc, uint16_t* __restrict__ dq,
                                                         long n8, float scale) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 x0 = ((const f32x4*)acc)[2 * i];
  const f32x4 x1 = ((const f32x4*)acc)[2 * i + 1];
  u32x4 w;
  w[0] = pack_bf16x2(x0[0] * scale, x0[1] * scale);
  w[1] = pack_bf16x2(x0[2] * scale, x0[3] * scale);
  w[2] = pack_bf16x2(x1[0] * scale, x1[1] * scale);
  w[3] = pack_bf16x2(x1[2] * scale, x1[3] * scale);
  ((u32x4*)dq)[i] = w;
}

template <int D, bool CAUSAL, int EXPMODE>
hipError_t launch_bwd_t(const BwdArgs& a, int phases, hipStream_t stream) {
  const long rows = (long)a.B * a.Hq * a.S;
  hipError_t e = hipSuccess;
  if (phases & 1) {
    const long pre_threads = rows * (D / 8);
    hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((unsigned)((pre_threads + 255) / 256)), dim3(256), 0, stream,
                       a.o, a.dO, a.delta, a.dq_acc, rows);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (phases & 2) {
    const int nkt = (a.S + kBwdBN - 1) / kBwdBN;
    hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL, EXPMODE>), dim3((unsigned)(nkt * a.B * a.Hkv)), dim3(256), 0,
                       stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (phases & 4) {
    const long n8 = rows * D / 8;
    hipLaunchKernelGGL(dq_convert_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                       a.dq_acc, a.dq, n8, a.scale);
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
