// dq_atomics.hip - the fp32 atomic traffic of a dQ accumulated inside the dK/dV kernel,
// measured on its own.
//
// Not part of the library: a stand-alone measurement for the backward's design.  The
// separate dQ pass recomputes S and dP; the alternative folds dQ += dS K into the dK/dV
// kernel, where every workgroup (one per 128-key tile) would add its partial dQ of every
// step into an fp32 dQ in global memory with atomics, followed by one conversion launch.
// This probe issues exactly that atomic traffic and nothing else (no loads, no products):
//   - the dK/dV kernel's grid: one 512-thread workgroup per (KV group, 128-key tile), the
//     lowest key tile first;
//   - its step order: blocks of 64 queries from the last one down to the key tile's
//     diagonal (causal), the group's query heads innermost;
//   - per step, the workgroup's 64 x d partial block added to dQ rows with
//     global_atomic_add_f32, 16 per thread, each wave instruction covering 64 consecutive
//     floats of one row (the best coalescing the partial could be given).
// The time is a lower bound for that design's extra cost: it already contains none of the
// dQ product, the reduction of the key blocks' partials inside the workgroup, or the
// conversion launch.
//
// Build and run (any directory):
//   hipcc --offload-arch=gfx950 -O3 -o /tmp/dq_atomics <repo>/exact_attention_27_amd/csrc/probes/dq_atomics.hip
//   /tmp/dq_atomics [B Hq Hkv S]     default 2 32 8 8192 (d = 128, causal); one JSON line
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

constexpr int kD = 128;
constexpr int kKeys = 128;     // keys per workgroup
constexpr int kQueries = 64;   // queries per step
constexpr int kThreads = 512;
constexpr int kPerThread = kQueries * kD / kThreads;  // 16 atomics per thread per step

__global__ __launch_bounds__(kThreads) void dq_atomics(float* dq, int B, int Hq, int Hkv, int S) {
  const int ngrp = B * Hkv;
  const int kt = blockIdx.x / ngrp;  // lowest key tile first
  const int grp = blockIdx.x - kt * ngrp;
  const int b = grp / Hkv;
  const int hkv = grp - b * Hkv;
  const int G = Hq / Hkv;
  const int nqb = (S + kQueries - 1) / kQueries;
  const int q_first = (kt * kKeys) / kQueries;
  const float v = 1.0f / 1024.0f;
  for (int qb = nqb - 1; qb >= q_first; --qb) {
    for (int g = 0; g < G; ++g) {
      const int hq = hkv * G + g;
      float* base = dq + ((size_t)(b * Hq + hq) * S + (size_t)qb * kQueries) * kD;
#pragma unroll
      for (int p = 0; p < kPerThread; ++p) {
        const int e = p * kThreads + (int)threadIdx.x;  // element of the 64 x d block
        if (qb * kQueries + e / kD < S) unsafeAtomicAdd(base + e, v);
      }
    }
  }
}

}  // namespace

int main(int argc, char** argv) {
  int B = 2, Hq = 32, Hkv = 8, S = 8192;
  if (argc == 5) {
    B = std::atoi(argv[1]);
    Hq = std::atoi(argv[2]);
    Hkv = std::atoi(argv[3]);
    S = std::atoi(argv[4]);
  }
  if (B < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || S < kKeys || S % kKeys != 0) {
    std::fprintf(stderr, "usage: dq_atomics [B Hq Hkv S], S a multiple of %d\n", kKeys);
    return 2;
  }
  const size_t n = (size_t)B * Hq * S * kD;
  float* dq = nullptr;
  if (hipMalloc(&dq, n * sizeof(float)) != hipSuccess) return 1;
  const int nkt = S / kKeys;
  const dim3 grid((unsigned)(nkt * B * Hkv));
  hipEvent_t e0, e1;
  hipEventCreate(&e0);
  hipEventCreate(&e1);
  std::vector<float> ms;
  for (int rep = 0; rep < 6; ++rep) {
    hipMemset(dq, 0, n * sizeof(float));
    hipEventRecord(e0, 0);
    hipLaunchKernelGGL(dq_atomics, grid, dim3(kThreads), 0, 0, dq, B, Hq, Hkv, S);
    hipEventRecord(e1, 0);
    if (hipEventSynchronize(e1) != hipSuccess) return 1;
    float t = 0.f;
    hipEventElapsedTime(&t, e0, e1);
    if (rep > 0) ms.push_back(t);  // the first launch warms up
  }
  // Atomics issued: per group, G heads x 64 x d floats for every (key tile, query block
  // at or below it).
  double atomics = 0.0;
  const int nqb = S / kQueries;
  for (int kt = 0; kt < nkt; ++kt) atomics += (double)(nqb - (kt * kKeys) / kQueries) * (Hq / Hkv) * kQueries * kD;
  atomics *= (double)B * Hkv;
  std::sort(ms.begin(), ms.end());
  const double med = ms[ms.size() / 2];
  float check = 0.f;
  hipMemcpy(&check, dq, sizeof(float), hipMemcpyDeviceToHost);  // row 0: every key tile adds once
  std::printf("{\"probe\": \"dq_atomics\", \"B\": %d, \"Hq\": %d, \"Hkv\": %d, \"S\": %d, \"d\": %d, "
              "\"atomics\": %.0f, \"bytes\": %.0f, \"ms_median\": %.4f, \"ms_min\": %.4f, \"gb_per_s\": %.1f, "
              "\"row0_value\": %.6f}\n",
              B, Hq, Hkv, S, kD, atomics, atomics * 4.0, med, ms.front(), atomics * 4.0 / (med * 1e-3) / 1e9,
              (double)check);
  hipFree(dq);
  return 0;
}
