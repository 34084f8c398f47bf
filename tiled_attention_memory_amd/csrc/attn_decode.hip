// Decoding against a key/value cache, for gfx950.
//
// The page "使用 PyTorch FSDP 微調 Llama 2 70B" (agentlenshq.com), section
// "Flash Attention", computes exact attention tile by tile with an online
// softmax so that the score matrix never reaches HBM. In generation the query
// side shrinks to a few new tokens per head while the cached keys and values
// stay long, so every cached byte is read once and HBM bandwidth is the bound.
//
// One workgroup handles one (batch, kv head, key split): the Sq new tokens of
// all g query heads of that group are packed into R = g * Sq rows (row r is
// head r / Sq of the group, token r % Sq) that share one pass over the split's
// keys. Key and value tiles of 64 rows stream into a ring of LDS stages (four
// of 32 KiB for D = 128, eight of 16 KiB for D = 64) by direct-to-LDS loads,
// several tiles ahead of the tile being consumed, with one barrier per tile.
// With R <= 64 the two waves of each 32-row block take the two 32-key halves
// of every tile, each with its own online-softmax state, and combine their
// states through LDS at the end; with R > 64 each wave owns a 32-row block and
// both halves. A split writes its normalised fp32 output and log-sum-exp for
// attn_merge_kernel (attn_merge.hip) to combine; an unsplit key range writes
// the bf16 output and log-sum-exp directly.
//
// The splits are chosen so that the workgroups, one per CU at a time, finish
// their equal shares of the key tiles in as few rounds as possible.
#include <math.h>

#include <algorithm>

#include "attn_device.h"
#include "attn_launch.h"

namespace tam {
namespace {

constexpr int kThreads = 256;
constexpr int kBC = 64;                 // keys per tile
constexpr int kRingBytes = 128 * 1024;  // LDS ring of key/value stages
constexpr int kCUs = 256;

struct DecArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;       // bf16 output (one split), or
  float* o32;        // fp32 partial outputs: split s at o32 + s * o_stride
  float* lse;        // log-sum-exp (natural log): split s at lse + s * lse_stride
  long long o_stride, lse_stride;
  int Hq, Hkv, Sq, Sk, dlt;
  int g;             // query heads per kv head
  int kv_chunk;      // keys per split, a multiple of 64
  float c;           // softmax scale * log2(e)
  TileSched sched;   // streams = (batch, kv head), tiles = key splits
};

// The running row max only moves when a tile's max exceeds it by more than
// this (base-2 units): probabilities stay below 2^8 before normalisation, which
// fp32 sums and bf16 products carry without loss, and most tiles skip the
// rescale of the output accumulator.
constexpr float kLazyMax = 8.f;

// Workgroup barrier without a memory fence: the ring's loads are waited for
// explicitly (a fence would wait for the loads still in flight as well), and
// every LDS read before the barrier has been consumed by the time a wave gets
// there. The empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D, bool CAUSAL, bool KSPLIT>
__global__ __launch_bounds__(kThreads, 1) void attn_decode_kernel(DecArgs a) {
  using T = SwzTile<D>;
  constexpr int KS = D / 16;          // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;          // 32-row blocks of the O^T accumulator
  constexpr int STAGE = 2 * T::BYTES; // K tile then V tile
  constexpr int NST = kRingBytes / STAGE;
  constexpr int NLD = T::LOADS / 4;   // 1-KiB loads per wave per tensor per tile
  constexpr int LPS = 2 * NLD;        // loads per wave per stage
  constexpr int NKB = KSPLIT ? 1 : 2; // 32-key blocks of a tile one wave computes
  static_assert(kBC == T::ROWS, "key tile = LDS tile");
  static_assert(NST >= 3 && (NST - 2) * LPS < 64, "ring depth");
  static_assert(2 * (2 + 16 * DB) * 64 * 4 <= kRingBytes, "exchange area inside the ring");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[NST * STAGE];

  int bh, split;
  if (!sched_decode(a.sched, blockIdx.x, &bh, &split)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int Sq = a.Sq, Sk = a.Sk, dlt = a.dlt, g = a.g;
  const int rb = KSPLIT ? wave >> 1 : wave;  // 32-row block of this wave
  const int kb0 = KSPLIT ? wave & 1 : 0;     // its first 32-key block of each tile
  const bool wave_rows = rb * 32 < g * Sq;   // waves past the packed rows only load
  const int b = bh / a.Hkv, kvh = bh - b * a.Hkv;
  const int r = rb * 32 + col;               // packed row of this lane
  const int hoff = r / Sq, tok = r - hoff * Sq;
  const bool row_ok = hoff < g;
  const size_t row_off = ((size_t)(b * a.Hq + kvh * g + hoff) * Sq + tok) * D;
  const int kbeg = split * a.kv_chunk, kend = min(Sk, kbeg + a.kv_chunk);
  const uint16_t* kg = a.k + ((size_t)b * a.Hkv + kvh) * (size_t)Sk * D;
  const uint16_t* vg = a.v + ((size_t)b * a.Hkv + kvh) * (size_t)Sk * D;

  // Q rows as MFMA B operands (k = head dim), resident for the whole pass. A
  // negative scale is folded into Q as an exact sign flip, so the softmax
  // works with c >= 0 and takes a row max.
  const float c = fabsf(a.c);
  bf16x8 qf[KS];
  {
    const uint16_t* qp = a.q + row_off + 8 * half;
    const uint32_t flip = a.c < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 w = row_ok ? *reinterpret_cast<const u32x4*>(qp + 16 * ks) : u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, w ^ flip);
    }
  }

  // Per-lane LDS offsets within a stage: row reads of K (row col, chunk
  // 2ks + half) and transposed reads of V (rows 4half + (lane&15)/4 and +8,
  // elements 32db + dsub + 4(lane&3)).
  const int i16 = lane & 15;
  const int dsub = 16 * ((lane >> 4) & 1);
  int koff[KS], voff[DB][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = T::chunk_off(col, 2 * ks + half);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
      voff[db][hi] = T::elem_off(4 * half + (i16 >> 2) + 8 * hi, db * 32 + dsub + 4 * (i16 & 3));
  int loff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) loff[i] = T::load_src(wave * NLD + i, lane);

  // Key tiles [jbeg, jend) of the split; the last key any packed row may see
  // is Sq - 1 + dlt. Tiles from jplain on hold a key hidden from some row or
  // lie past the split's end.
  const int jbeg = kbeg / kBC;
  const int n_kv = (kend + kBC - 1) / kBC;
  const int jend = CAUSAL ? (Sq - 1 + dlt < kbeg ? jbeg : min(n_kv, (Sq - 1 + dlt) / kBC + 1)) : n_kv;
  const int jplain = max(jbeg, min(jend, (CAUSAL ? min(dlt + 1, kend) : kend) / kBC));

  // Tile j into ring stage st (this wave's share of its K and V rows). The
  // descriptors end at the split's last key: rows past it read as zeros, and
  // tiles past the split issue loads that touch no memory at all, which keeps
  // the number of loads per stage, and so every wait below, the same.
  const uint32_t ring_addr = lds_address(ring) + wave * NLD * 1024;
  auto issue = [&](int j, int st) TAM_INLINE {
    const int row0 = j * kBC;
    const int rows = max(0, kend - row0);
    const size_t base = rows > 0 ? (size_t)row0 * D : 0;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + base, rows * D * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + base, rows * D * 2);
    const uint32_t dst = ring_addr + st * STAGE;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      dma16(rk, dst + i * 1024, loff[i]);
      dma16(rv, dst + T::BYTES + i * 1024, loff[i]);
    }
  };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY;  // running (lazy) max of this row's base-2 scaled scores
  float l_run = 0.f;        // running sum of this lane's half of the row

  // One tile on ring stage `cur`: key blocks kb0 .. kb0 + NKB - 1 (32 keys
  // each) of the 64 keys from kv0. MASKED: some key is hidden from some row or
  // lies past the split's end, so each score is tested against a per-lane limit.
  auto tile = [&](auto masked_tag, int kv0, const unsigned char* cur) TAM_INLINE {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const unsigned char* Ks = cur + kb0 * 32 * T::ROW_BYTES;
    const unsigned char* Vs = cur + T::BYTES + kb0 * 32 * T::ROW_BYTES;

    // S^T for each 32-key block: lane holds keys 8(v/4) + 4half + v%4 of the
    // block for its row
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        s[kb] = mfma32(*reinterpret_cast<const bf16x8*>(Ks + kb * 32 * T::ROW_BYTES + koff[ks]), qf[ks], s[kb]);

    if (MASKED) {
      const int lim = (CAUSAL ? min(tok + dlt, kend - 1) : kend - 1) - (kv0 + 32 * kb0 + 4 * half);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kb][v] = kb * 32 + 8 * (v >> 2) + (v & 3) <= lim ? s[kb][v] : -INFINITY;
    }
    float ext = s[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) ext = fmaxf(ext, s[kb][v]);
    ext = max_halves(ext);
    // a tile with all of this row's keys hidden gives -inf (NaN when c == 0):
    // neither moves the running max
    const float mt = ext * c;
    const bool grow = mt > m_run + kLazyMax;
    if (MASKED || __builtin_amdgcn_ballot_w64(grow)) {
      // 0 on a row's first visible tile, 1 where the max does not move
      const float alpha = grow ? fast_exp2(m_run - mt) : 1.f;
      m_run = grow ? mt : m_run;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    float p[NKB][16];
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float e = fast_exp2(fmaf(s[kb][v], c, -m_run));
        if (MASKED) e = s[kb][v] == -INFINITY ? 0.f : e;
        p[kb][v] = e;
        lsum += e;
      }
    l_run += lsum;
    bf16x8 pb[NKB][2];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) pb[kb][k2] = pack_bf16x8(&p[kb][8 * k2]);

    // O^T += V^T P^T: the k index of product (kb, k2) slot t of lane half hh is
    // key 32kb + 16k2 + 8(t/4) + 4hh + t%4, where P sits in the S^T accumulator
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const unsigned char* vp = Vs + (kb * 32 + k2 * 16) * T::ROW_BYTES;
        bf16x8 vop[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
          vop[db] = lds_read_tr_pair(reinterpret_cast<const uint16_t*>(vp + voff[db][0]),
                                     reinterpret_cast<const uint16_t*>(vp + voff[db][1]));
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = mfma32(vop[db], pb[kb][k2], acc[db]);
      }
  };

  // The ring: tiles jbeg .. jbeg + NST - 2 go out first; at tile j, once every
  // wave has its share of tile j and has finished tile j - 1, tile j + NST - 1
  // goes into the stage tile j - 1 used. NST - 2 tiles stay in flight behind
  // the one being waited for.
  wait_loads();  // the Q loads, so that only ring loads are counted below
  int st_use = 0, st_fill = NST - 1;
  for (int t = 0; t < NST - 1; ++t) issue(jbeg + t, t);
  for (int j = jbeg; j < jend; ++j) {
    wait_vm<(NST - 2) * LPS>();
    ring_barrier();
    issue(j + NST - 1, st_fill);
    st_fill = st_fill + 1 == NST ? 0 : st_fill + 1;
    const unsigned char* cur = ring + st_use * STAGE;
    st_use = st_use + 1 == NST ? 0 : st_use + 1;
    if (wave_rows) {
      if (j < jplain)
        tile(std::false_type{}, j * kBC, cur);
      else
        tile(std::true_type{}, j * kBC, cur);
    }
  }
  wait_vm<0>();
  ring_barrier();  // the ring is idle from here on

  bool writer = wave_rows;
  if (KSPLIT) {
    // the wave of the second key half hands its state to the first through LDS
    float* xch = reinterpret_cast<float*>(ring) + rb * (2 + 16 * DB) * 64 + lane;
    if (wave_rows && kb0 == 1) {
      xch[0] = m_run;
      xch[64] = l_run;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) xch[(2 + 16 * db + v) * 64] = acc[db][v];
    }
    ring_barrier();
    writer = wave_rows && kb0 == 0;
    if (writer) {
      const float m1 = xch[0], l1 = xch[64];
      const float m = fmaxf(m_run, m1);
      // a half that saw no key of this row weighs 0
      const float a0 = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m);
      const float a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - m);
      m_run = m;
      l_run = a0 * l_run + a1 * l1;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] = a0 * acc[db][v] + a1 * xch[(2 + 16 * db + v) * 64];
    }
  }
  if (!writer) return;

  const float l_tot = sum_halves(l_run);
  if (!row_ok) return;
  // a row that saw no key of this split gets O = 0, LSE = -inf
  const bool seen = l_tot > 0.f;
  const float inv = seen ? 1.f / l_tot : 0.f;
  if (a.o32) {
    float* op = a.o32 + split * a.o_stride + row_off + 4 * half;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<f32x4*>(op + 32 * db + 8 * i) =
            f32x4{acc[db][4 * i] * inv, acc[db][4 * i + 1] * inv, acc[db][4 * i + 2] * inv, acc[db][4 * i + 3] * inv};
  } else {
    // lane holds columns 32db + 8i + 4half + (0..3); pairs of i are merged
    // across the halves so that each store writes 16 contiguous bytes
    uint16_t* op = a.o + row_off + 8 * half;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        u32x2 w[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int i = 2 * m + t;
          w[t] = u32x2{pack_bf16(acc[db][4 * i] * inv, acc[db][4 * i + 1] * inv),
                       pack_bf16(acc[db][4 * i + 2] * inv, acc[db][4 * i + 3] * inv)};
        }
        *reinterpret_cast<u32x4*>(op + 32 * db + 16 * m) = pair_halves(w[0], w[1]);
      }
  }
  if (half == 0) a.lse[split * a.lse_stride + row_off / D] = seen ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int D, bool CAUSAL>
hipError_t launch_t(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                    float* lse, void* workspace, hipStream_t stream) {
  const DecodePlan p = decode_plan(sh);
  const long long rows = (long long)sh.B * sh.Hq * sh.Sq;
  DecArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  if (p.splits > 1) {
    a.o = nullptr;
    a.o32 = static_cast<float*>(workspace);
    a.lse = a.o32 + (size_t)p.splits * rows * sh.D;
    a.o_stride = rows * sh.D;
    a.lse_stride = rows;
  } else {
    a.o = o;
    a.o32 = nullptr;
    a.lse = lse;
    a.o_stride = a.lse_stride = 0;
  }
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.Sq = sh.Sq;
  a.Sk = sh.Sk;
  a.dlt = sh.dlt;
  a.g = sh.Hq / sh.Hkv;
  a.kv_chunk = p.chunk;
  a.c = sh.scale * kLog2e;
  a.sched.BH = sh.B * sh.Hkv;
  a.sched.NT = p.splits;
  a.sched.chunk = (a.sched.BH + 7) / 8;
  // two waves per 32-row block when the packed rows fit in two blocks
  const bool ksplit = a.g * sh.Sq <= 64;
  const void* kern = ksplit ? reinterpret_cast<const void*>(&attn_decode_kernel<D, CAUSAL, true>)
                            : reinterpret_cast<const void*>(&attn_decode_kernel<D, CAUSAL, false>);
  void* args[] = {&a};
  hipError_t e = hipLaunchKernel(kern, dim3((unsigned)sched_grid(a.sched)), dim3(kThreads), args, 0, stream);
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_merge_strided(a.o32, a.lse, p.splits, rows * sh.D, rows, o, lse, rows, sh.D, stream);
}

}  // namespace

// Key splits: the workgroups run one per CU, so a launch of U = B * Hkv units
// split s ways takes ceil(U s / 256) rounds of ceil(T / s) tiles each (T key
// tiles per unit), plus a fixed start-up and write-out cost per round, taken
// as two tiles. The split count minimising that is used (the smallest one on
// ties, which also keeps the merge short).
DecodePlan decode_plan(const AttnShape& sh) {
  const long long units = (long long)sh.B * sh.Hkv;
  const int tiles = (sh.Sk + kBC - 1) / kBC;
  int best = 1;
  long long best_cost = -1;
  for (int s = 1; s <= tiles && s <= 1024; ++s) {
    const long long rounds = (units * s + kCUs - 1) / kCUs;
    const long long cost = rounds * ((tiles + s - 1) / s + 2);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = s;
    }
  }
  DecodePlan p;
  p.chunk = (tiles + best - 1) / best * kBC;
  p.splits = (sh.Sk + p.chunk - 1) / p.chunk;
  return p;
}

size_t decode_workspace_bytes(const AttnShape& sh) {
  const DecodePlan p = decode_plan(sh);
  const size_t rows = (size_t)sh.B * sh.Hq * sh.Sq;
  // unsplit ranges write the output directly; keep a small non-empty workspace
  return p.splits > 1 ? (size_t)p.splits * rows * (sh.D + 1) * 4 : 256;
}

hipError_t launch_decode(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                         float* lse, void* workspace, hipStream_t stream) {
  if (sh.D == 128) return sh.causal ? launch_t<128, true>(sh, q, k, v, o, lse, workspace, stream)
                                    : launch_t<128, false>(sh, q, k, v, o, lse, workspace, stream);
  return sh.causal ? launch_t<64, true>(sh, q, k, v, o, lse, workspace, stream)
                   : launch_t<64, false>(sh, q, k, v, o, lse, workspace, stream);
}

}  // namespace tam
