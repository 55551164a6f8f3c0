// attn_device.h - device-side building blocks shared by the gfx950 attention kernels.
//
// Register/lane layouts used throughout (CDNA4 MFMA, wave64), checked on the GPU by
// a one-instruction test against known matrices:
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l holds row (l % 32), k = (l / 32) * 8 + e, e = 0..7   (8 bf16)
//     B: lane l holds col (l % 32), k = (l / 32) * 8 + e, e = 0..7   (8 bf16)
//     D: lane l, register v holds row (v / 4) * 8 + (l / 32) * 4 + (v % 4), col (l % 32)
//   ds_read_b64_tr_b16 (LDS transpose read, 4 x bf16 per lane), within each group of
//     16 lanes: output lane i, element e = input element (i % 4) of the 8 bytes that
//     lane 4 * e + i / 4 of the same group addressed.
//   v_permlane32_swap(x, x): lane l < 32 gets {x[l], x[l + 32]}, lane l >= 32 gets
//     {x[l - 32], x[l]}; the two halves of a wave exchange values in one instruction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------------
// exp2.  The softmax evaluates every exponential as a power of two (the scale is
// folded into c = |scale| * log2(e)).  Two evaluations exist:
//  * the hardware transcendental, v_exp_f32;
//  * a cubic polynomial on the FMA units: the software exponential the FA4 pages
//    describe ("NVIDIA's FlashAttention-4", section "The Technical Edge": cubic
//    polynomials on ordinary cores instead of the special-function units; gist.science
//    summary, section 2.B).  The pages give no coefficients or range, so this one is
//    derived here: x is clamped to [-127, 64], split as x = n + f with n = round(x)
//    (the 1.5 * 2^23 addition trick) and f in [-1/2, 1/2]; 2^f is a degree-3
//    polynomial with p(0) = 1 whose coefficients minimise the maximum relative error
//    on [-1/2, 1/2] (a linear-programming minimax fit, fit_exp2_poly.py beside this
//    file); 2^n is applied by adding n to the exponent field.  Max relative error
//    1.02e-4 over the whole range, far below bf16's half-ulp (2^-9), and exactly
//    2^0 = 1 and 2^-inf = 0.  Arguments above 64 (and +inf) give 2^64: the forward
//    exponentiates a tile before its rescale test, which only needs such values to be
//    large (without the clamp the exponent add would overflow into the sign bit).
// ---------------------------------------------------------------------------------
constexpr float kExp2C1 = 0x1.62f5fap-1f;
constexpr float kExp2C2 = 0x1.f00c4cp-3f;
constexpr float kExp2C3 = 0x1.c2a216p-5f;

// HIGH: clamp the argument above at 64 as well as below at -127.  Without the upper clamp
// the result is still right for every x < 128 (2^127 is the largest power the exponent
// field holds) and wraps into the sign bit above; every kernel keeps the clamp, so an
// argument out of range saturates instead (the backward's arguments stay near or below 0
// for an LSE that matches its inputs, but the clamp costs one v_min).
template <bool HIGH = true>
__host__ __device__ inline float exp2_poly3(float x) {
  x = fmaxf(x, -127.0f);
  if constexpr (HIGH) x = fminf(x, 64.0f);
  const float t = x + 12582912.0f;  // 1.5 * 2^23: rounds x to an integer in the low mantissa bits
  const float n = t - 12582912.0f;
  const float f = x - n;
  const float p = fmaf(fmaf(fmaf(kExp2C3, f, kExp2C2), f, kExp2C1), f, 1.0f);
  const uint32_t ti = __builtin_bit_cast(uint32_t, t);
  return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, p) + (ti << 23));
}

template <int EXPMODE, bool HIGH = true>
__device__ __forceinline__ float exp2_sm(float x) {
  if constexpr (EXPMODE == 0) {
    return __builtin_amdgcn_exp2f(x);
  } else {
    return exp2_poly3<HIGH>(x);
  }
}

// ---------------------------------------------------------------------------------
// Cross-lane helpers.
// ---------------------------------------------------------------------------------
// Value held by lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float other_half(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t lo = r[0], hi = r[1];
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? lo : hi);
}

// max(x, value of lane l ^ 32) without a select: {r0, r1} is {own, other} in some order.
__device__ __forceinline__ float max_halves(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// The lane's index in the wave, computed where it is called: the asm keeps the compiler
// from computing it once and holding it in a register across a loop (for rare paths and
// epilogues of kernels at their register limit, recomputing costs less than the register).
__device__ __forceinline__ int lane_id_here() {
  int l;
  __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// ---------------------------------------------------------------------------------
// MFMA and LDS access.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_f16: the same shape and lane layouts with fp16 operands; the
// operands arrive as 16-bit lanes in the same vector type as the bf16 ones.
__device__ __forceinline__ f32x16 mfma32_f16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

__device__ __forceinline__ bf16x8 join(const i16x4& lo, const i16x4& hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, r);
}

// Tiles of D bf16 per row are stored in LDS with their 16-byte chunks permuted per row,
// chunk' = chunk ^ f(row).  f is chosen so that the two LDS access patterns of the
// kernels are free of bank conflicts (64 banks x 4 bytes):
//   * 16-byte MFMA-operand reads of 16 consecutive rows at one chunk, and
//   * 8-byte transpose reads of 4 consecutive rows x 4 consecutive chunks per 32 lanes.
template <int D>
__device__ __forceinline__ int swz_chunk(int r, int c) {
  if constexpr (D == 128) {
    return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
  } else {
    return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
}

// Element offset of (row r, column col) in a swizzled [rows][D] bf16 LDS tile.
template <int D>
__device__ __forceinline__ int swz(int r, int col) {
  return r * D + (swz_chunk<D>(r, col >> 3) << 3) + (col & 7);
}

// Blocked tile layouts (no swizzle).  A [rows][D] bf16 tile is cut into blocks of 16 rows
// x 4 chunks (a chunk is 16 bytes = 8 bf16): 64 chunks, 1024 bytes, exactly what one
// LDS DMA instruction writes.  Block (r / 16, c / 4) sits at byte
// ((r / 16) * (D / 32) + c / 4) * 1024 of the tile.  Inside a block the chunks are in
// one of two orders:
//   * row-inner, unit (c % 4) * 16 + r % 16: an MFMA-operand read of 16 consecutive rows
//     at one chunk is 256 contiguous bytes, free of bank conflicts;
//   * chunk-inner, unit (r % 16) * 4 + c % 4: a transpose read of 4 consecutive rows x
//     4 consecutive chunks (32 lanes) is 256 contiguous bytes, free of bank conflicts;
//   * chunk-inner with the chunk XORed by (r % 16) / 4, unit
//     (r % 16) * 4 + ((c % 4) ^ ((r % 16) / 4)): an MFMA-operand read of 16 consecutive
//     rows at one chunk touches every bank once.
// The DMA that fills a block gives lane l unit l, so in the two chunk-inner orders each
// group of 4 consecutive lanes fetches one aligned 64-byte piece of a row (the
// row-inner order scatters them over 4 rows).  The offsets are sums of a row part and
// a chunk part (for the XOR order: per parity of c / 2), so an address that a lane
// keeps in a register reaches every other block and row group by an immediate offset.
template <int D>
__host__ __device__ constexpr int blk_row_inner(int r, int c) {
  return ((r >> 4) * (D / 32) + (c >> 2)) * 1024 + ((c & 3) * 16 + (r & 15)) * 16;
}
template <int D>
__host__ __device__ constexpr int blk_chunk_inner(int r, int c) {
  return ((r >> 4) * (D / 32) + (c >> 2)) * 1024 + ((r & 15) * 4 + (c & 3)) * 16;
}
template <int D>
__host__ __device__ constexpr int blk_chunk_inner_x(int r, int c) {
  return ((r >> 4) * (D / 32) + (c >> 2)) * 1024 + ((r & 15) * 4 + ((c & 3) ^ ((r >> 2) & 3))) * 16;
}

// ---------------------------------------------------------------------------------
// Global -> LDS DMA (global_load_lds_dwordx4): lane l of the wave copies 16 bytes from
// its global address g to LDS bytes [lds_wave_base + 16 l, +16).  It is issued from an
// asm block so that the compiler, which cannot tell which LDS bytes the DMA writes, does
// not make every later LDS read wait for it.  The block has no register outputs; the
// LDS it writes is read only after wait_dma()/vmcnt waits and a barrier, which the
// kernels place explicitly.  lds_wave_base must be the same for all lanes of the wave.
// The DMA takes its LDS address from m0, which the block sets; the compiler treats m0 as
// reserved and warns about the clobber, but it uses m0 nowhere in these kernels (every
// m0 write in their assembly is one of these blocks; tests/test_isa.py checks that).
// ---------------------------------------------------------------------------------
// LDS byte address of a generic pointer into LDS: a generic LDS address is the LDS
// aperture in the upper 32 bits and the LDS byte address in the lower 32, so truncation
// gives it without the null-pointer check that an address-space cast emits.
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

__device__ __forceinline__ void dma16(const void* g, const void* lds_wave_base) {
  const uint32_t l = lds_addr(lds_wave_base);
  const uint32_t ls = __builtin_amdgcn_readfirstlane(l);
  __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                   :
                   : "s"(ls), "v"(g)
                   : "memory", "m0");
}

// A wave-uniform pointer moved to scalar registers (lane 0's copy).  For code where the
// compiler cannot prove uniformity (divergent branches) but a scalar base is required.
// readfirstlane returns a signed int: both halves go through uint32_t so that neither
// is sign-extended into the other.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t b64 = (uint64_t)(uintptr_t)p;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b64);
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo);
}

// dma16 with a scalar (wave-uniform) 64-bit base and a 32-bit per-lane byte offset:
// no per-lane address arithmetic when the offsets stay fixed across a loop.
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, const void* lds_wave_base) {
  const uint32_t l = lds_addr(lds_wave_base);
  const uint32_t ls = __builtin_amdgcn_readfirstlane(l);
  __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :
                   : "s"(ls), "v"(voff), "s"(sbase)
                   : "memory", "m0");
}

// A value the optimiser must treat as unknown: keeps a base address in one register
// instead of letting its constant part merge into per-use offsets past what the LDS
// instructions' 16-bit immediate can hold.
__device__ __forceinline__ int opaque(int x) {
  __asm__ volatile("" : "+v"(x));
  return x;
}

// Wait until every DMA (and every other vector memory operation) of the wave is done.
__device__ __forceinline__ void wait_dma() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

}  // namespace attn
