// mfma_ceiling.hip - sustained v_mfma_f32_32x32x16_bf16 throughput of the whole chip.
//
// Not part of the library: a stand-alone measurement of the ceiling that the attention
// kernels' MFMA rates are read against.  Every CU runs two 256-thread workgroups (64 KiB of
// LDS each, so exactly two waves per SIMD), and every wave issues back-to-back MFMAs into
// four independent accumulators.  Two operand sets:
//   constant : one fixed fragment of small values for A and B in every product;
//   random   : eight fragments per operand of bf16 values ~ N(0, 1) (a fixed LCG, sum of
//              12 uniforms), a different (A, B) pair in each of eight consecutive products.
// The chip's clock under sustained load depends on the operand data (switching activity),
// so the random set is the ceiling that attention's N(0, 1) inputs meet.  Each set runs
// eight launches of about 10 ms back to back after a warm-up launch; the printed rate is
// dense bf16 flop (32*32*16*2 per product) over the event time.
//
// Build and run (any directory):
//   hipcc --offload-arch=gfx950 -O3 -o /tmp/mfma_ceiling <repo>/exact_attention_27_amd/csrc/probes/mfma_ceiling.hip
//   /tmp/mfma_ceiling           both operand sets, twice, as text
//   /tmp/mfma_ceiling --json    the random set once, as one JSON line (what bench.py reads)
//   /tmp/mfma_ceiling --chain   constant operands, one wave per SIMD, one dependent
//                               accumulation chain per wave against four independent ones
//                               (and two waves per SIMD with four): whether back-to-back
//                               products on one accumulator cost issue rate
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kBlocks = 512;         // two per CU on a 256-CU chip
constexpr int kFragWords = 4096;     // u32x4 words in the operand table (64 KiB)

template <bool RANDOM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mfma_loop(const u32x4* src, float* out, int iters) {
  __shared__ float pad[16384];  // 64 KiB: two workgroups per CU
  pad[threadIdx.x] = 0.f;
  __syncthreads();
  bf16x8 a[8], b[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = __builtin_bit_cast(bf16x8, src[(k * 256 + threadIdx.x) % kFragWords]);
    b[k] = __builtin_bit_cast(bf16x8, src[(k * 256 + 2048 + threadIdx.x) % kFragWords]);
  }
  if (!RANDOM) {
    bf16x8 s;
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = (__bf16)(0.01f * (float)((threadIdx.x + e) & 7));
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = b[k] = s;
  }
  f32x16 acc[4] = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[7 - k], acc[k & 3], 0, 0, 0);
  }
  float s = pad[(threadIdx.x + 1) & 255];
#pragma unroll
  for (int v = 0; v < 16; ++v) s += acc[0][v] + acc[1][v] + acc[2][v] + acc[3][v];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// One wave per SIMD (96 KiB of LDS: one workgroup per CU), NACC accumulators: NACC = 1
// makes every product depend on the one before it.
template <int NACC, int LDS_FLOATS>
__global__ __launch_bounds__(256) void mfma_chain(float* out, int iters) {
  __shared__ float pad[LDS_FLOATS];
  pad[threadIdx.x] = 0.f;
  __syncthreads();
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = (__bf16)(0.01f * (float)((threadIdx.x + e) & 7));
  f32x16 acc[NACC] = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k % NACC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[k % NACC], 0, 0, 0);
  }
  float s = pad[(threadIdx.x + 1) & 255];
#pragma unroll
  for (int j = 0; j < NACC; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[j][v];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

template <int NACC, int LDS_FLOATS>
bool run_chain(const char* name, float* out, int blocks) {
  const int iters = 4096;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return false;
  hipLaunchKernelGGL((mfma_chain<NACC, LDS_FLOATS>), dim3(blocks), dim3(256), 0, 0, out, iters);
  if (hipEventRecord(e0, 0) != hipSuccess) return false;
  for (int r = 0; r < 8; ++r) hipLaunchKernelGGL((mfma_chain<NACC, LDS_FLOATS>), dim3(blocks), dim3(256), 0, 0, out, iters);
  if (hipEventRecord(e1, 0) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) return false;
  float ms = 0.f;
  if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) return false;
  const double products = 8.0 * blocks * 4 * (double)iters * 8;
  std::printf("%-40s %8.2f ms for 8 launches, %7.1f TFLOP/s bf16 dense\n", name, ms,
              products * 32768.0 / (ms * 1e-3) / 1e12);
  std::fflush(stdout);
  return true;
}

template <bool RANDOM>
bool run(const char* name, const u32x4* src, float* out, int iters, bool json = false) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return false;
  hipLaunchKernelGGL((mfma_loop<RANDOM>), dim3(kBlocks), dim3(256), 0, 0, src, out, iters / 8);
  if (hipEventRecord(e0, 0) != hipSuccess) return false;
  for (int r = 0; r < 8; ++r) hipLaunchKernelGGL((mfma_loop<RANDOM>), dim3(kBlocks), dim3(256), 0, 0, src, out, iters);
  if (hipEventRecord(e1, 0) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) return false;
  float ms = 0.f;
  if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) return false;
  const double products = 8.0 * kBlocks * 4 * (double)iters * 8;
  const double tflops = products * 32768.0 / (ms * 1e-3) / 1e12;
  if (json) {
    std::printf("{\"operands\": \"%s\", \"tflops\": %.1f, \"ms\": %.2f, \"launches\": 8}\n", name, tflops, ms);
  } else {
    std::printf("%-9s operands: %8.2f ms for 8 launches, %7.1f TFLOP/s bf16 dense\n", name, ms, tflops);
  }
  std::fflush(stdout);
  return true;
}

}  // namespace

int main(int argc, char** argv) {
  const bool json = argc > 1 && std::strcmp(argv[1], "--json") == 0;
  if (argc > 1 && std::strcmp(argv[1], "--chain") == 0) {
    float* out = nullptr;
    if (hipMalloc(&out, (size_t)kBlocks * 256 * 4) != hipSuccess) return 1;
    // Twice, so that the second round runs at the settled clock.
    bool ok = true;
    for (int r = 0; r < 2 && ok; ++r) {
      ok = run_chain<1, 24576>("1 wave/SIMD, 1 dependent chain", out, kBlocks / 2) &&
           run_chain<4, 24576>("1 wave/SIMD, 4 independent chains", out, kBlocks / 2) &&
           run_chain<4, 16384>("2 waves/SIMD, 4 independent chains", out, kBlocks);
    }
    ok = ok && hipDeviceSynchronize() == hipSuccess;
    return ok ? 0 : 1;
  }
  static unsigned short h[kFragWords * 8];
  unsigned st = 12345u;
  for (int i = 0; i < kFragWords * 8; ++i) {
    float x = -6.0f;
    for (int t = 0; t < 12; ++t) {
      st = st * 1664525u + 1013904223u;
      x += (float)(st >> 8) * (1.0f / 16777216.0f);
    }
    unsigned u;
    std::memcpy(&u, &x, 4);
    h[i] = (unsigned short)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);  // round to nearest even
  }
  u32x4* src = nullptr;
  float* out = nullptr;
  if (hipMalloc(&src, sizeof(h)) != hipSuccess || hipMalloc(&out, (size_t)kBlocks * 256 * 4) != hipSuccess) return 1;
  if (hipMemcpy(src, h, sizeof(h), hipMemcpyHostToDevice) != hipSuccess) return 1;
  const int iters = 4096 * 8;
  bool ok = json ? run<true>("random", src, out, iters, true)
                 : (run<false>("constant", src, out, iters) && run<true>("random", src, out, iters) &&
                    run<false>("constant", src, out, iters) && run<true>("random", src, out, iters));
  ok = ok && hipDeviceSynchronize() == hipSuccess;
  return ok ? 0 : 1;
}
