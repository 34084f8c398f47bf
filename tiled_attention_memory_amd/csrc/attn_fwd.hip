// Forward pass of exact attention for gfx950: one fused kernel.
//
// Follows the page "使用 PyTorch FSDP 微調 Llama 2 70B" (agentlenshq.com),
// section "Flash Attention": the score matrix is processed in tiles that stay
// on chip ("Tiling"), normalised with an online softmax, and fused with both
// products so that only O and one log-sum-exp per row are written to HBM
// ("Kernel Fusion").
//
// The same kernel serves a block pair of context-parallel attention: Sq query
// rows against Sk keys, key j visible to query row i when j <= i + dlt under a
// causal mask (dlt = query position - key position of the blocks' first rows).
// A row that sees no key gets O = 0 and LSE = -inf. With Sq = Sk and dlt = 0
// this is plain causal attention.
//
// Work unit: one (batch, query head, 128-row query tile); 4 waves, each owning
// 32 query rows. Sequences of at most 64 (32) rows would leave half (three
// quarters) of such a unit empty, so there 2 (4) query heads of one group
// share a unit, each in 64 (32) of its rows: they read the same K and V.
// Per 64-key tile:
//   S^T = K Q^T       (MFMA; A = K rows from LDS, B = Q rows held in registers)
//   online softmax    (each lane owns one query row: its running max, its
//                      partial row sum and its output column rescale are
//                      per-lane scalars; one cross-half exchange per tile)
//   O^T += V^T P^T    (MFMA; A = V read transposed from LDS, B = P straight
//                      from the S^T accumulator after bf16 rounding)
// K/V tiles go from global memory straight into double-buffered, swizzled LDS
// (no staging registers); the next tile's loads are in flight while the
// current one is consumed. Under a causal mask, key tiles past the diagonal
// are never visited and only tiles that straddle it evaluate the mask.
#include <math.h>

#include <type_traits>

#include "attn_device.h"
#include "attn_launch.h"

namespace tam {
namespace {

constexpr int kBR = 128;      // query rows per workgroup
constexpr int kBC = 64;       // keys per tile
constexpr int kThreads = 256;

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;      // bf16 output, or
  float* o32;       // fp32 output (partial results of a block pair)
  float* lse;
  int Hq, Hkv, Sq, Sk, dlt;
  float c;  // softmax scale * log2(e): scores are exponentiated in base 2
  DropParams drop;  // dropout on the probabilities (DROP kernels only)
  const float2* rope;  // (cos, sin) table [Sq][D/2]: rotate the Q rows at load; null = none
  int pack;            // log2 of the query heads a unit holds (Sq <= kBR >> pack)
  TileSched sched;
};

// The running row max only moves when a tile's max exceeds it by more than
// this (base-2 units); probabilities then stay below 2^8 before normalisation,
// which fp32 sums and bf16 products carry without loss, and the O rescale is
// skipped for most tiles.
constexpr float kLazyMax = 8.f;

template <int D, bool CAUSAL, bool DROP = false>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(FwdArgs a) {
  using T = SwzTile<D>;
  constexpr int KS = D / 16;          // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;          // 32-row blocks of the O^T accumulator
  constexpr int STAGE = 2 * T::BYTES; // K tile then V tile
  constexpr int NLD = T::LOADS / 4;   // 1-KiB loads per wave per tensor per tile
  static_assert(kBC == T::ROWS, "key tile = LDS tile");
  // Two separate LDS stages, so that loads into one are provably independent
  // of reads from the other and need no wait before those reads.
  __shared__ __attribute__((aligned(1024))) unsigned char stage0[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[STAGE];

  int bh, qt;
  if (!sched_decode(a.sched, blockIdx.x, &bh, &qt)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave
  const int col = lane & 31, half = lane >> 5;
  const int Sq = a.Sq, Sk = a.Sk, dlt = a.dlt;
  // unit = (batch, 2^pack query heads of one group, 128-row tile); each head
  // takes kBR >> pack rows of it, so a wave's 32 rows belong to one head
  const int rows_per_head = kBR >> a.pack;
  bh = (bh << a.pack) + wave * 32 / rows_per_head;   // this wave's (batch, query head)
  const int b = bh / a.Hq;
  const int kvh = (bh - b * a.Hq) / (a.Hq / a.Hkv);
  const int w_tmin = qt * kBR + wave * 32 % rows_per_head;  // the wave's first row
  const int w_tmax = w_tmin + 31;
  const int tok = w_tmin + col;                // the query row this lane owns
  const bool row_ok = tok < Sq;
  const size_t row_off = ((size_t)bh * Sq + tok) * D;  // element offset of the row in q, o (and / D in lse)
  const int t_last = min(qt * kBR + rows_per_head, Sq) - 1;  // the unit's last row (of any of its heads)
  constexpr int kbeg = 0;                      // the unit's keys: all of them
  const int kend = Sk;
  const uint16_t* kg = a.k + ((size_t)b * a.Hkv + kvh) * (size_t)Sk * D;
  const uint16_t* vg = a.v + ((size_t)b * a.Hkv + kvh) * (size_t)Sk * D;

  // Q rows as MFMA B operands (k = head dim), resident for the whole loop. A
  // negative scale is folded into Q (an exact sign flip), so the softmax below
  // always works with a scale c >= 0 and takes a row max.
  const float c = fabsf(a.c);
  bf16x8 qf[KS];
  {
    const uint16_t* qp = a.q + row_off + 8 * half;
    const uint32_t flip = a.c < 0.f ? 0x80008000u : 0u;
    u32x4 w[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) w[ks] = row_ok ? *reinterpret_cast<const u32x4*>(qp + 16 * ks) : u32x4{0, 0, 0, 0};
    if (a.rope && row_ok) {
      // rotary embedding at load: this lane holds elements 16 ks + 8 half + t,
      // and the partner of element d < D/2 (d + D/2) sits in chunk ks + KS/2
      const float2* cs = a.rope + (size_t)tok * (D / 2);
#pragma unroll
      for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 16 * ks + 8 * half + 2 * j;
          float l0, l1, h0, h1;
          rope_pair(bf16_lo(w[ks][j]), bf16_lo(w[ks + KS / 2][j]), cs[d], false, &l0, &h0);
          rope_pair(bf16_hi(w[ks][j]), bf16_hi(w[ks + KS / 2][j]), cs[d + 1], false, &l1, &h1);
          w[ks][j] = pack_bf16(l0, l1);
          w[ks + KS / 2][j] = pack_bf16(h0, h1);
        }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, w[ks] ^ flip);
  }

  // Per-lane LDS offsets, fixed for every tile: row reads of K (row col, chunk
  // 2ks + half; key block kb adds 32 rows) and transposed reads of V (rows
  // 4half + (lane&15)/4 and +8, elements 32db + dsub + 4(lane&3); blocks of 16
  // keys add 16 rows).
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

  // key tiles [jbeg, jend); the last key any row of the unit may see is t_last + dlt
  const int jbeg = kbeg / kBC;
  const int n_kv = (kend + kBC - 1) / kBC;
  const int jend = CAUSAL ? (t_last + dlt < kbeg ? jbeg : min(n_kv, (t_last + dlt) / kBC + 1)) : n_kv;

  // K and V tile j straight into an LDS stage; rows past S read as zeros.
  auto issue = [&](int j, unsigned char* stage) TAM_INLINE {
    const int row0 = j * kBC;
    const int bytes = (Sk - row0) * D * 2;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + (size_t)row0 * D, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + (size_t)row0 * D, bytes);
    unsigned char* dst = stage + wave * NLD * 1024;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      load_lds16(rk, dst + i * 1024, loff[i]);
      load_lds16(rv, dst + T::BYTES + i * 1024, loff[i]);
    }
  };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY;  // running (lazy) max of this row's base-2 scaled scores
  float l_run = 0.f;        // running sum of this lane's half of the row

  // Key blocks KB0 .. KB0 + NKB - 1 (32 keys each) of a 64-key tile. MASKED:
  // the tile straddles the diagonal or the end of the sequence for this wave,
  // so scores of hidden keys are excluded; such tiles run one 32-key block at
  // a time, which keeps fewer scores live. Every other tile runs both blocks
  // without any per-element test.
  auto tile = [&](auto masked_tag, auto kb0_tag, auto nkb_tag, int kv0, const unsigned char* cur,
                  auto&& after_scores) TAM_INLINE {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr int KB0 = decltype(kb0_tag)::value;
    constexpr int NKB = decltype(nkb_tag)::value;
    const unsigned char* Ks = cur + KB0 * 32 * T::ROW_BYTES;
    const unsigned char* Vs = cur + T::BYTES + KB0 * 32 * T::ROW_BYTES;

    // S^T for the 32-key blocks: lane holds keys kv0 + 32(KB0 + kb) + 8(v/4) + 4half + v%4
    // of this lane's row; independent accumulator chains, interleaved
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        s[kb] = mfma32(*reinterpret_cast<const bf16x8*>(Ks + kb * 32 * T::ROW_BYTES + koff[ks]), qf[ks], s[kb]);
    if (NKB == 2) {
      // keep three operand pairs in flight: six K reads first, then two
      // products per two reads (left alone, the scheduler reads each pair
      // just before its products and waits out every LDS round trip)
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);   // LDS reads
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0); // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    }

    // Whether this row may see the key of accumulator element v of block kb:
    // that key is kv0 + 32 KB0 + 4half + off with the constant
    // off = 32kb + 8(v/4) + v%4, so one compare against a per-lane limit decides it.
    const int lim = (CAUSAL ? min(tok + dlt, kend - 1) : kend - 1) - (kv0 + 32 * KB0 + 4 * half);
    auto visible = [&](int kb, int v) TAM_INLINE { return kb * 32 + 8 * (v >> 2) + (v & 3) <= lim; };
    if (MASKED) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kb][v] = visible(kb, v) ? s[kb][v] : -INFINITY;
    }
    after_scores();   // e.g. the next tile's loads, issued while the products run
    float ext = s[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) ext = fmaxf(ext, s[kb][v]);
    ext = max_halves(ext);
    // A tile where all of this row's keys are masked gives -inf, or NaN when
    // c == 0; neither moves the running max.
    const float mt = ext * c;
    const bool grow = mt > m_run + kLazyMax;
    // The few masked tiles rescale unconditionally: a branch here would make
    // the compiler copy the accumulators and spill.
    if (MASKED || __builtin_amdgcn_ballot_w64(grow)) {
      // 0 on a row's first visible tile, 1 where the max does not move (also
      // for a row that has seen no key yet, where m_run - m_new would be NaN)
      const float alpha = grow ? fast_exp2(m_run - mt) : 1.f;
      const float m_new = grow ? mt : m_run;
      m_run = m_new;
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
        // hidden scores hold -inf: exp2 gives 0, or NaN when c == 0; both become 0
        if (MASKED) e = s[kb][v] == -INFINITY ? 0.f : e;
        p[kb][v] = e;
        lsum += e;
      }
    l_run += lsum;
    if (DROP) {
      // the row sum above is taken before dropout; the product with V uses
      // the kept probabilities scaled by r
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        // The four lanes of a quad hold rows 4m .. 4m + 3 and need the same
        // four generator calls (key groups i = 0..3 of this half): lane 4m + j
        // makes call j and the quad swaps, leaving each lane its row's word of
        // every call.
        const uint32_t k4 = (uint32_t)(kv0 + 32 * (KB0 + kb) + 8 * (lane & 3) + 4 * half) >> 2;
        const u32x4 words = quad_transpose(
            philox4x32_10(k4, (uint32_t)tok >> 2, (uint32_t)bh, 0u, a.drop.seed_lo, a.drop.seed_hi));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            p[kb][4 * i + r4] = drop_keep(words[i], r4, a.drop.t) ? p[kb][4 * i + r4] * a.drop.r : 0.f;
      }
    }

    bf16x8 pb[NKB][2];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) pb[kb][k2] = pack_bf16x8(&p[kb][8 * k2]);

    // Keep the V reads below this point: hoisting them over the softmax would
    // hold 64 more registers and cost the second wave per SIMD.
    __builtin_amdgcn_sched_barrier(0);
    // O^T += V^T P^T: the k index of MFMA (kb, k2) slot t of lane half hh is key
    // 32kb + 16k2 + 8(t/4) + 4hh + t%4, matching where P sits in the S^T accumulator.
    // the DB accumulators form independent chains: head-dim block innermost
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

  // Tile j on stage cur while tile j + 1 loads into nxt; one barrier per tile
  // for every wave, whichever loop below runs it.
  auto step = [&](auto masked_tag, int j, const unsigned char* cur, unsigned char* nxt) TAM_INLINE {
    // the next tile's loads go out once this tile's score products are queued
    auto next = [&]() TAM_INLINE {
      if (j + 1 < jend) issue(j + 1, nxt);
    };
    tile(masked_tag, std::integral_constant<int, 0>{}, std::integral_constant<int, 2>{}, j * kBC, cur, next);
    // each tile is its own scheduling region: products moved across the
    // barrier would wait for the other waves or break up the next tile's
    // read-ahead pattern
    __builtin_amdgcn_sched_barrier(0);
    wait_loads();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Leading tiles lie entirely below this wave's diagonal and inside the
  // sequence: they run unmasked, two per iteration with fixed stages. The
  // remaining few tiles (diagonal, ragged end) run one by one.
  const int jplain = max(jbeg, min(jend, (CAUSAL ? min(w_tmin + dlt + 1, kend) : kend) / kBC));
  if (jend > jbeg) issue(jbeg, stage0);
  wait_loads();
  __syncthreads();
  if (w_tmin >= Sq) {
    // a wave whose rows all lie past the end of the sequence only loads its
    // share of each tile and meets the others at every barrier (its own loop
    // keeps that test out of the loops below)
    for (int jj = jbeg; jj < jend; ++jj) {
      if (jj + 1 < jend) issue(jj + 1, (jj - jbeg) & 1 ? stage0 : stage1);
      wait_loads();
      __syncthreads();
    }
    return;
  }
  int j = jbeg;
  for (; j + 2 <= jplain; j += 2) {
    step(std::false_type{}, j, stage0, stage1);
    step(std::false_type{}, j + 1, stage1, stage0);
  }
  // stages stay compile-time constants here too, so LDS addresses fold into
  // instruction offsets
  auto tail_step = [&](auto stage_tag, int jj) TAM_INLINE {
    constexpr int STG = decltype(stage_tag)::value;
    const unsigned char* cur = STG ? stage1 : stage0;
    unsigned char* nxt = STG ? stage0 : stage1;
    if (jj + 1 < jend) issue(jj + 1, nxt);
    const int kv0 = jj * kBC;
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    if (!CAUSAL || kv0 <= w_tmax + dlt) {   // some key of the tile is visible to this wave
      auto nothing = []() TAM_INLINE {};
      if (jj < jplain) {
        tile(std::false_type{}, C0{}, C2{}, kv0, cur, nothing);
      } else {
        tile(std::true_type{}, C0{}, C1{}, kv0, cur, nothing);
        // the second 32-key block, unless this wave sees none of its keys
        if ((!CAUSAL || kv0 + 32 <= w_tmax + dlt) && kv0 + 32 < kend)
          tile(std::true_type{}, C1{}, C1{}, kv0, cur, nothing);
      }
    }
    wait_loads();
    __syncthreads();
  };
  for (; j < jend; ++j) {
    if ((j - jbeg) & 1)
      tail_step(std::integral_constant<int, 1>{}, j);
    else
      tail_step(std::integral_constant<int, 0>{}, j);
  }

  const float l_tot = sum_halves(l_run);
  if (row_ok) {
    // a row that saw no key (possible with offset blocks) gets O = 0, LSE = -inf
    const bool seen = l_tot > 0.f;
    const float inv = seen ? 1.f / l_tot : 0.f;
    if (a.o32) {
      float* op = a.o32 + row_off + 4 * half;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<f32x4*>(op + 32 * db + 8 * i) =
              f32x4{acc[db][4 * i] * inv, acc[db][4 * i + 1] * inv, acc[db][4 * i + 2] * inv, acc[db][4 * i + 3] * inv};
    } else {
      // lane holds columns 32db + 8i + 4half + (0..3); pairs of i are merged
      // across the halves so each store writes 16 contiguous bytes per lane
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
    if (half == 0) a.lse[row_off / D] = seen ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// Whole sequences of at most 64 tokens: every row's keys fit one 64-key tile,
// so the softmax needs no running max and K, V can serve many query heads.
// Unit: (batch, kv head, subset of the group's query heads), 4 waves. K and V
// go to LDS once; waves 2p and 2p + 1 take rows 0..31 and 32..63 of the
// subset's heads p, p + 2, ..., with their rows of Q in two register sets
// used in turn: the first two heads' rows load together with K and V, and
// each later head's rows load while the head two before it is computed. With
// no barrier after the first, the waves run independently.
struct FwdShortArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int Hq, Hkv, S, nsplit;
  float c;  // softmax scale * log2(e)
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_short_kernel(FwdShortArgs a) {
  using T = SwzTile<D>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int NLD = T::LOADS / 4;
  static_assert(kBC == T::ROWS, "key tile = LDS tile");
  __shared__ __attribute__((aligned(1024))) unsigned char kv[2 * T::BYTES];  // K tile, then V tile

  const int S = a.S;
  const int unit = xcd_unit(blockIdx.x, gridDim.x);
  const int grp = unit / a.nsplit, sub = unit - grp * a.nsplit;  // grp = b * Hkv + kv head
  const int b = grp / a.Hkv;
  const int g = a.Hq / a.Hkv, hps = g / a.nsplit;
  const int h_end = (grp - b * a.Hkv) * g + sub * hps + hps;     // past the subset's last head
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int rb = wave & 1;                 // this wave's 32 rows of each head
  const int tok = 32 * rb + col;           // the query row this lane owns
  const bool row_ok = tok < S;
  const float c = fabsf(a.c);
  const uint32_t flip = a.c < 0.f ? 0x80008000u : 0u;  // a negative scale is folded into Q

  {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + (size_t)grp * S * D, S * D * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + (size_t)grp * S * D, S * D * 2);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int li = wave * NLD + i;
      load_lds16(rk, kv + li * 1024, T::load_src(li, lane));
      load_lds16(rv, kv + T::BYTES + li * 1024, T::load_src(li, lane));
    }
  }
  // This lane's Q chunks of head h through a bounded buffer: rows past S read
  // as zeros, and every wave issues exactly KS loads.
  auto load_q = [&](int h, u32x4 (&w)[KS]) TAM_INLINE {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + ((size_t)b * a.Hq + h) * S * D, S * D * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      w[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, (tok * D + 8 * half + 16 * ks) * 2, 0, 0));
  };
  // A wave's heads alternate between two register sets, so that the second
  // head's rows load together with K, V and the first head's rows.
  int h = h_end - hps + (wave >> 1);
  u32x4 qa[KS], qb[KS];
  if (h < h_end) load_q(h, qa);
  if (h + 2 < h_end) {
    __asm__ volatile("" ::: "memory");  // issued after the loads above
    load_q(h + 2, qb);
    wait_vm<KS>();   // K, V and the first head's rows; the second head's may still be in flight
  } else {
    wait_loads();
  }
  // A bare barrier: the wait above has put K and V into LDS, and a full
  // __syncthreads would also wait for the second head's rows. The empty asm
  // statements keep the compiler from moving memory accesses across it.
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");

  int koff[KS], voff[DB][2];
  const int i16 = lane & 15;
  const int dsub = 16 * ((lane >> 4) & 1);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = T::chunk_off(col, 2 * ks + half);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
      voff[db][hi] = T::elem_off(4 * half + (i16 >> 2) + 8 * hi, db * 32 + dsub + 4 * (i16 & 3));
  // the last key row tok may see, less this lane's key offset 4 half
  const int lim = (CAUSAL ? min(tok, S - 1) : S - 1) - 4 * half;
  auto visible = [&](int kb, int v) TAM_INLINE { return kb * 32 + 8 * (v >> 2) + (v & 3) <= lim; };

  // one head: S^T for key blocks 0 .. NKB - 1, softmax over the row, O^T = V^T P^T
  auto head = [&](auto nkb_tag, const bf16x8 (&qf)[KS], int hh) TAM_INLINE {
    constexpr int NKB = decltype(nkb_tag)::value;
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        s[kb] = mfma32(*reinterpret_cast<const bf16x8*>(kv + kb * 32 * T::ROW_BYTES + koff[ks]), qf[ks], s[kb]);
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = visible(kb, v) ? fmaxf(mx, s[kb][v]) : mx;
    const float mt = max_halves(mx) * c;  // every row sees key 0: finite
    float p[NKB][16];
    float l = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        p[kb][v] = visible(kb, v) ? fast_exp2(fmaf(s[kb][v], c, -mt)) : 0.f;
        l += p[kb][v];
      }
    l = sum_halves(l);
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const bf16x8 pb = pack_bf16x8(&p[kb][8 * k2]);
        const unsigned char* vp = kv + T::BYTES + (kb * 32 + k2 * 16) * T::ROW_BYTES;
#pragma unroll
        for (int db = 0; db < DB; ++db)
          acc[db] = mfma32(lds_read_tr_pair(reinterpret_cast<const uint16_t*>(vp + voff[db][0]),
                                            reinterpret_cast<const uint16_t*>(vp + voff[db][1])),
                           pb, acc[db]);
      }
    if (row_ok) {
      const float inv = 1.f / l;
      const size_t row = ((size_t)b * a.Hq + hh) * S + tok;
      uint16_t* op = a.o + row * D + 8 * half;
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
      if (half == 0) a.lse[row] = (mt + __log2f(l)) * kLn2;
    }
  };

  // rows 0..31 see only keys 0..31 under a causal mask, and so does every row of S <= 32
  const bool one_block = (CAUSAL && rb == 0) || S <= 32;
  // head hh from the register set w, whose rows are then reloaded for head hh + 4
  auto step = [&](u32x4 (&w)[KS], int hh) TAM_INLINE {
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, w[ks] ^ flip);
    if (hh + 4 < h_end) load_q(hh + 4, w);
    if (one_block)
      head(std::integral_constant<int, 1>{}, qf, hh);
    else
      head(std::integral_constant<int, 2>{}, qf, hh);
  };
  for (; h < h_end; h += 4) {
    step(qa, h);
    if (h + 2 < h_end) step(qb, h + 2);
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  uint16_t* o, float* o32, float* lse, hipStream_t stream) {
  FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.o32 = o32;
  a.lse = lse;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.Sq = sh.Sq;
  a.Sk = sh.Sk;
  a.dlt = sh.dlt;
  a.drop = make_drop(sh.drop_t, sh.seed);
  a.rope = sh.rope;
  a.c = sh.scale * kLog2e;
  a.pack = head_pack(sh, kBR);
  a.sched.BH = (sh.B * sh.Hq) >> a.pack;
  a.sched.NT = (sh.Sq + kBR - 1) / kBR;
  a.sched.chunk = (a.sched.BH + 7) / 8;
  const long long grid = sched_grid(a.sched);
  void* args[] = {&a};
  const void* kern = a.drop.t ? reinterpret_cast<const void*>(&attn_fwd_kernel<D, CAUSAL, true>)
                              : reinterpret_cast<const void*>(&attn_fwd_kernel<D, CAUSAL, false>);
  return hipLaunchKernel(kern, dim3((unsigned)grid), dim3(kThreads), args, 0, stream);
}

// The fewest head subsets (a divisor of the group) that give every compute
// unit two workgroups.
int fwd_short_split(const AttnShape& sh) {
  const int g = sh.Hq / sh.Hkv;
  const long long groups = (long long)sh.B * sh.Hkv;
  for (int ns = 1; ns < g; ++ns)
    if (g % ns == 0 && groups * ns >= 512) return ns;
  return g;
}

template <int D, bool CAUSAL>
hipError_t launch_short(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        uint16_t* o, float* lse, hipStream_t stream) {
  FwdShortArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.S = sh.Sq;
  a.nsplit = fwd_short_split(sh);
  a.c = sh.scale * kLog2e;
  const long long grid = (long long)sh.B * sh.Hkv * a.nsplit;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_short_kernel<D, CAUSAL>), dim3((unsigned)grid),
                         dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_fwd(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      uint16_t* o, float* o32, float* lse, hipStream_t stream) {
  // whole sequences of at most one key tile, bf16 output, no dropout or rotation
  if (o && !o32 && sh.Sq == sh.Sk && sh.Sq <= kBC && sh.dlt == 0 && !sh.drop_t && !sh.rope) {
    if (sh.D == 128) return sh.causal ? launch_short<128, true>(sh, q, k, v, o, lse, stream)
                                      : launch_short<128, false>(sh, q, k, v, o, lse, stream);
    return sh.causal ? launch_short<64, true>(sh, q, k, v, o, lse, stream)
                     : launch_short<64, false>(sh, q, k, v, o, lse, stream);
  }
  if (sh.D == 128) return sh.causal ? launch<128, true>(sh, q, k, v, o, o32, lse, stream)
                                    : launch<128, false>(sh, q, k, v, o, o32, lse, stream);
  return sh.causal ? launch<64, true>(sh, q, k, v, o, o32, lse, stream)
                   : launch<64, false>(sh, q, k, v, o, o32, lse, stream);
}

}  // namespace tam
