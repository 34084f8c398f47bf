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
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
// Kernel bodies are written with local lambdas; every one of them must be
// inlined, or its captured register arrays would be spilled to scratch memory.
#define TAM_INLINE __attribute__((always_inline))

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// The same product on fp16 operands (v_mfma_f32_32x32x16_f16, same layouts).
__device__ __forceinline__ f32x16 mfma32(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
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

// Store helper for accumulator rows: lanes l and l + 32 each hold 4 values of
// the same output row, x for columns [8i, 8i+4) + 4 * half and y for columns
// [8i+8, 8i+12) + 4 * half, as two packed 32-bit pairs. After the exchange the
// lower half holds columns 8i..8i+7 and the upper half 8i+8..8i+15 of that
// row, so one 16-byte store per lane covers 32 contiguous bytes per row.
__device__ __forceinline__ u32x4 pair_halves(u32x2 x, u32x2 y) {
  auto r0 = __builtin_amdgcn_permlane32_swap(x[0], y[0], false, false);
  auto r1 = __builtin_amdgcn_permlane32_swap(x[1], y[1], false, false);
  return u32x4{(uint32_t)r0[0], (uint32_t)r1[0], (uint32_t)r0[1], (uint32_t)r1[1]};
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

// Round two floats to fp16 (nearest even) and pack them, first in the low half.
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f32x2 v = {lo, hi};
  f16x2 h = __builtin_convertvector(v, f16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ f16x8 pack_f16x8(const float* x) {
  u32x4 u = {pack_f16(x[0], x[1]), pack_f16(x[2], x[3]), pack_f16(x[4], x[5]), pack_f16(x[6], x[7])};
  return __builtin_bit_cast(f16x8, u);
}

// Power-of-two scaling into fp16 operands. A block of values whose largest
// magnitude is m gets the exponent e = ceil(log2 m), clamped to
// [kMinExp, kMaxExp] (an all-zero block gets kMinExp), and is held as
// x * 2^(14 - e): every magnitude is then at most 2^14 (fp16 reaches 65504),
// and a bf16 value converts exactly unless it lies more than 2^28 below m.
constexpr int kMinExp = -60, kMaxExp = 128;
__device__ __forceinline__ int ceil_log2(float m) {
  const uint32_t u = __builtin_bit_cast(uint32_t, m) & 0x7fffffffu;
  const int E = (int)(u >> 23);
  if (E == 0) return kMinExp;  // zero, or below the fp32 normal range
  const int e = E - 127 + ((u & 0x7fffffu) != 0);
  return e < kMinExp ? kMinExp : e > kMaxExp ? kMaxExp : e;
}

// 2^e as a float, with e clamped to the normal range, built from the bits so
// that a wave-uniform e keeps the result in a scalar register.
__device__ __forceinline__ float pow2i(int e) {
  e = e < -126 ? -126 : e > 127 ? 127 : e;
  return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
}

// Largest magnitude among eight bf16 values, as a bf16 bit pattern (sign clear):
// for finite values the patterns order like the magnitudes.
__device__ __forceinline__ uint32_t bf16x8_max_mag(const bf16x8& x) {
  const u32x4 u = __builtin_bit_cast(u32x4, x);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = u[i] & 0x7fffu, hi = (u[i] >> 16) & 0x7fffu;
    m = m > lo ? m : lo;
    m = m > hi ? m : hi;
  }
  return m;
}

// Eight bf16 values times s (a power of two) as fp16, rounded to nearest even.
__device__ __forceinline__ f16x8 bf16x8_to_f16x8(const bf16x8& x, float s) {
  const u32x4 u = __builtin_bit_cast(u32x4, x);
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_f16(bf16_lo(u[i]) * s, bf16_hi(u[i]) * s);
  return __builtin_bit_cast(f16x8, r);
}

// Largest value over the 64 lanes of the wave (every lane gets it).
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t y = __shfl_xor(x, off);
    x = x > y ? x : y;
  }
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const int y = __shfl_xor(x, off);
    x = x > y ? x : y;
  }
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// ---------------------------------------------------------------------------
// 64-row LDS tiles of bf16 rows, filled straight from global memory
// ---------------------------------------------------------------------------
// Layout: 256-byte lines (one row of D = 128, or two rows of D = 64) whose
// 16-byte chunks are XOR-swizzled by the line index. The swizzle is chosen so
// that both read patterns the kernels use touch every LDS bank exactly once
// per cycle (checked with the LDS bank-conflict counter on the device):
//   * row reads: 16 lanes read the same 16-byte chunk of 16 consecutive rows;
//   * transposed 4x16 reads: 32 lanes read four 64-byte row segments of four
//     consecutive rows.
// For D = 128, chunk c of row r sits at chunk c ^ f(r) of line r with
// f(r) = ((r & 3) << 2) | ((r >> 2) & 3): a permutation of the 16 chunks over
// any 16 rows, giving the four rows of each aligned group distinct 64-byte
// groups. For D = 64, row r is half (r & 1) of line r / 2 and the 16 chunk
// slots are XORed with g(L) = ((L & 1) << 2) | ((L >> 1) & 3).
// The swizzle repeats every 16 rows, so moving by a multiple of 16 rows moves
// every address by the same number of bytes.
template <int D>
struct SwzTile {
  static_assert(D == 64 || D == 128, "head dim");
  static constexpr int ROWS = 64;
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int BYTES = ROWS * ROW_BYTES;   // 16 KiB or 8 KiB
  static constexpr int LOADS = BYTES / 1024;       // wave-wide 16-byte-per-lane loads per tile

  // byte offset of the 16-byte chunk c (elements 8c..8c+7) of row r
  __host__ __device__ static constexpr int chunk_off(int r, int c) {
    return D == 128 ? r * 256 + ((c ^ (((r & 3) << 2) | ((r >> 2) & 3))) << 4)
                    : (r >> 1) * 256 +
                          (((((r & 1) << 3) | c) ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3))) << 4);
  }
  // byte offset of element e (a multiple of 4) of row r
  __host__ __device__ static constexpr int elem_off(int r, int e) {
    return chunk_off(r, e >> 3) + ((e & 7) << 1);
  }
  // Source of the 16 bytes that lane l of the i-th 1-KiB load writes (LDS bytes
  // 1024 i + 16 l): byte offset of that chunk within the tile's rows in global memory.
  __host__ __device__ static constexpr int load_src(int i, int l) {
    return D == 128 ? src128(4 * i + (l >> 4), l & 15) : src64(4 * i + (l >> 4), l & 15);
  }

 private:
  __host__ __device__ static constexpr int src128(int line, int slot) {
    return line * 256 + ((slot ^ (((line & 3) << 2) | ((line >> 2) & 3))) << 4);
  }
  __host__ __device__ static constexpr int src64(int line, int slot) {
    return (2 * line + ((slot ^ (((line & 1) << 2) | ((line >> 1) & 3))) >> 3)) * 128 +
           (((slot ^ (((line & 1) << 2) | ((line >> 1) & 3))) & 7) << 4);
  }
};

// Buffer descriptor over `bytes` bytes from `base`: loads past the end read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// 16 bytes per lane from rsrc + voffset into LDS at lds_base + 16 * lane
// (lds_base must be the same for the whole wave).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, void* lds_base, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16,
                                           voffset, 0, 0, 0);
}
// 4 bytes per lane into LDS at lds_base + 4 * lane.
__device__ __forceinline__ void load_lds4(__amdgpu_buffer_rsrc_t r, void* lds_base, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 4,
                                           voffset, 0, 0, 0);
}

// The same 16-byte direct load, issued as inline assembly for kernels that keep
// every LDS buffer in one array: the compiler then does not treat the bytes it
// writes as aliasing later LDS reads of other parts of that array (which would
// make it wait for the load before those reads). Such kernels wait for their
// loads with wait_loads() and a barrier before reading the written bytes.
// lds_addr is the byte address in LDS (the same for the whole wave).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, int voffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voffset), "s"(r)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, int voffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voffset), "s"(r)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte address of a generic pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)p;
}

// Wait until this wave's outstanding global loads (including loads into LDS) are done.
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N of this wave's vector memory operations are
// outstanding. They complete in issue order, so the older ones are done.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier that orders LDS accesses only: every LDS access of this
// wave before it is complete and none after it starts early, but loads from
// global memory that are still in flight (into LDS stages nobody reads yet)
// are not waited for, as a full barrier would.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Dropout on the probabilities, with a keep mask regenerated from a
// counter-based generator instead of stored: Philox4x32-10 (Salmon, Moraes,
// Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011).
// A round multiplies words 0 and 2 by two constants (64-bit products split
// into high and low words) and mixes in the other two words and the key; the
// key advances by two Weyl increments between rounds.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  return u32x4{c0, c1, c2, c3};
}

// One generator call covers a 4 x 4 block of (query row i, key j) of one
// query head: counter (j / 4, i / 4, b * Hq + h, 0), key = the 64-bit seed;
// the pair's byte is byte j % 4 (low byte first) of word i % 4, and the pair
// is kept when that byte is at least t (dropout probability t / 256, kept
// probabilities scaled by r = 256 / (256 - t)).
struct DropParams {
  uint32_t seed_lo, seed_hi;
  uint32_t t;  // 0..255
  float r;
};

__host__ inline DropParams make_drop(int t, unsigned long long seed) {
  DropParams d;
  d.seed_lo = (uint32_t)seed;
  d.seed_hi = (uint32_t)(seed >> 32);
  d.t = (uint32_t)t;
  d.r = 256.f / (float)(256 - t);
  return d;
}

// Whether byte n (0..3) of a word of drop bytes keeps its pair.
__device__ __forceinline__ bool drop_keep(uint32_t bytes, int n, uint32_t t) {
  return ((bytes >> (8 * n)) & 0xFFu) >= t;
}

// 4 x 4 transpose across each quad of lanes (4m .. 4m + 3): on return,
// element i of lane 4m + j holds what element j of lane 4m + i held. Two
// butterfly steps (partner lane xor 1, then xor 2) with DPP quad permutes.
// Every lane of the quad must be active. Used to share generator calls: four
// neighbouring lanes that need the same four calls each make one and swap.
__device__ __forceinline__ u32x4 quad_transpose(u32x4 w) {
  const int q = (int)(__lane_id() & 3u);
#pragma unroll
  for (int k = 0; k < 4; k += 2) {   // partner lane ^ 1, elements k and k + 1
    const uint32_t send = (q & 1) ? w[k] : w[k + 1];
    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
    if (q & 1)
      w[k] = recv;
    else
      w[k + 1] = recv;
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {      // partner lane ^ 2, elements k and k + 2
    const uint32_t send = (q & 2) ? w[k] : w[k + 2];
    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
    if (q & 2)
      w[k] = recv;
    else
      w[k + 2] = recv;
  }
  return w;
}

// 4 x 4 transpose of the bytes of four words: byte r of word n of the result
// is byte n of word r of the input.
__device__ __forceinline__ u32x4 byte_transpose(u32x4 w) {
  const uint32_t lo01 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);  // w0.b0 w1.b0 w0.b1 w1.b1
  const uint32_t hi01 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);  // w0.b2 w1.b2 w0.b3 w1.b3
  const uint32_t lo23 = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
  const uint32_t hi23 = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
  return u32x4{__builtin_amdgcn_perm(lo23, lo01, 0x05040100u), __builtin_amdgcn_perm(lo23, lo01, 0x07060302u),
               __builtin_amdgcn_perm(hi23, hi01, 0x05040100u), __builtin_amdgcn_perm(hi23, hi01, 0x07060302u)};
}

// Rotary position embedding (rotate-half pairing): the pair (x_d, x_{d+D/2})
// of a row at position m turns by a_d = m * base^(-2d/D). The table holds
// (cos a_d, sin a_d) per position and d < D/2, computed from fp64 angles. One
// helper serves every kernel so that a rotated value is bit-identical
// wherever it is formed; inverse = 1 turns the other way (gradients).
__device__ __forceinline__ void rope_pair(float lo, float hi, float2 cs, bool inverse, float* out_lo, float* out_hi) {
  const float sn = inverse ? -cs.y : cs.y;
  *out_lo = __builtin_fmaf(lo, cs.x, -(hi * sn));
  *out_hi = __builtin_fmaf(hi, cs.x, lo * sn);
}

// Scheduler shared by the kernels: work unit = (stream, tile), a stream being
// a query head or a (key/value head, head subset) pair. Workgroup i runs on
// XCD i % 8. When the streams divide evenly over the 8 XCDs, XCD x owns a
// contiguous range of them (so the heads of one key/value group share that
// XCD's L2) and walks its units from the last tile to the first, i.e.
// heaviest first under a causal mask for the query-tile kernels. Otherwise
// the units are dealt out in one global heaviest-first order, so no XCD sits
// idle when there are fewer than 8 streams or a remainder.
struct TileSched {
  int BH;      // streams
  int NT;      // tiles per stream
  int chunk;   // streams per XCD: ceil(BH / 8)
};
__host__ __device__ inline long long sched_grid(const TileSched& s) {
  return s.BH % 8 == 0 ? 8LL * s.chunk * s.NT : (long long)s.BH * s.NT;
}

// Workgroups are dealt to the 8 XCDs in turn (workgroup i to XCD i % 8). For
// a grid that is a multiple of 8, unit = xcd_unit(i, n) gives each XCD a
// contiguous range of units, so that neighbouring units (which share inputs)
// share that XCD's L2.
__device__ __forceinline__ int xcd_unit(int bid, int n) {
  return n % 8 == 0 ? (bid & 7) * (n >> 3) + (bid >> 3) : bid;
}

__host__ __device__ inline bool sched_decode(const TileSched& s, int bid, int* bh, int* qt) {
  if (s.BH % 8 != 0) {
    if (bid >= s.BH * s.NT) return false;
    *qt = s.NT - 1 - bid / s.BH;
    *bh = bid % s.BH;
    return true;
  }
  const int x = bid & 7, slot = bid >> 3;
  const int h0 = x * s.chunk;
  const int hn = s.chunk;
  if (slot >= hn * s.NT) return false;
  *qt = s.NT - 1 - slot / hn;
  *bh = h0 + slot % hn;
  return true;
}

}  // namespace tam
