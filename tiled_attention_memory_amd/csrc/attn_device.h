// Device-side building blocks shared by the attention kernels (gfx950 only).
//
// MFMA operand layouts used throughout (checked on the device):
//   v_mfma_f32_32x32x16_bf16  C[32x32] += A[32x16] * B[16x32]
//     lane l holds A[l%32][8*(l/32) + t] and B[8*(l/32) + t][l%32], t = 0..7;
//     accumulator element v of lane l is C[8*(v/4) + 4*(l/32) + v%4][l%32].
//   ds_read_b64_tr_b16: within each group of 16 lanes, lane 4r+m supplies the
//     address of elements 4m..4m+3 of row r of a 4x16 block of 16-bit values;
//     lane i receives column i (rows 0..3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tam {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two 16-bit transposed LDS reads (rows r0..r0+3 and r0+8..r0+11 of the
// caller's layout) joined into one 8-element MFMA operand.
__device__ __forceinline__ bf16x8 lds_read_tr_pair(const uint16_t* p_lo, const uint16_t* p_hi) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p_lo));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p_hi));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Cross-half exchange: v_permlane32_swap(a, b) swaps the upper 32 lanes of a
// with the lower 32 lanes of b. With a = b = x, the first result holds the
// lower half of x in every lane and the second the upper half, so combining
// the two gives the same value in lanes l and l ^ 32. The second operand goes
// through an empty asm so the compiler cannot treat the two operands (and
// then the two results) as the same value.
__device__ __forceinline__ void swap_halves(float x, float* lo_half, float* hi_half) {
  uint32_t a = __builtin_bit_cast(uint32_t, x);
  uint32_t b = a;
  asm volatile("" : "+v"(b));
  auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  *lo_half = __builtin_bit_cast(float, (uint32_t)r[0]);
  *hi_half = __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ __forceinline__ float max_halves(float x) {
  float a, b;
  swap_halves(x, &a, &b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float min_halves(float x) {
  float a, b;
  swap_halves(x, &a, &b);
  return fminf(a, b);
}

__device__ __forceinline__ float sum_halves(float x) {
  float a, b;
  swap_halves(x, &a, &b);
  return a + b;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round two floats to bf16 (nearest even) and pack them, first in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* x) {
  u32x4 u = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]),
             pack_bf16(x[6], x[7])};
  return __builtin_bit_cast(bf16x8, u);
}

// x ~= hi + lo with hi = bf16(x) and lo = bf16(x - hi): two bf16 MFMA operands
// that together carry about 16 significant bits of x.
__device__ __forceinline__ void split_bf16x8(const float* x, bf16x8* hi, bf16x8* lo) {
  u32x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_bf16(x[2 * i], x[2 * i + 1]);
    const float r0 = x[2 * i] - __builtin_bit_cast(float, h[i] << 16);
    const float r1 = x[2 * i + 1] - __builtin_bit_cast(float, h[i] & 0xffff0000u);
    l[i] = pack_bf16(r0, r1);
  }
  *hi = __builtin_bit_cast(bf16x8, h);
  *lo = __builtin_bit_cast(bf16x8, l);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

// Scheduler shared by the query-tile kernels: work unit = (query head, query
// tile). Workgroup i runs on XCD i % 8; XCD x owns a contiguous range of
// heads (so the heads of one key/value group share that XCD's L2) and walks
// its units from the last query tile to the first, i.e. heaviest first under
// a causal mask.
struct TileSched {
  int BH;      // B * Hq
  int NT;      // query tiles per head
  int chunk;   // heads per XCD: ceil(BH / 8)
};

__host__ __device__ inline long long sched_grid(const TileSched& s) {
  return 8LL * s.chunk * s.NT;
}

__device__ __forceinline__ bool sched_decode(const TileSched& s, int bid, int* bh, int* qt) {
  const int x = bid & 7, slot = bid >> 3;
  const int h0 = x * s.chunk;
  const int hn = min(s.chunk, s.BH - h0);
  if (hn <= 0 || slot >= hn * s.NT) return false;
  *qt = s.NT - 1 - slot / hn;
  *bh = h0 + slot % hn;
  return true;
}

}  // namespace tam
