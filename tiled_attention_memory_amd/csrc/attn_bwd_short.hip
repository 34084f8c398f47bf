// Backward pass of exact attention for short sequences (gfx950): one kernel.
//
// Follows the "Recomputation" bullet of the page "使用 PyTorch FSDP 微調 Llama 2 70B"
// (agentlenshq.com), section "Flash Attention", like the general backward:
// the probabilities are recomputed from Q, K and the forward pass's
// log-sum-exp. A sequence of at most 64 tokens puts every row's keys into one
// 64-key tile, so a single pass over that tile gives every gradient:
//   S^T = K Q^T,  P = exp(scale S - LSE),  dP^T = V dO^T,
//   Delta_i = sum_j P_ij dP_ij   (the whole row is in the tile: exact, and O
//                                 is never read),
//   dS = P (dP - Delta),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// The general path instead needs three kernels (dQ, dK/dV, reduce), reads Q
// and dO twice and O once.
//
// Unit: (batch, kv head, subset of the group's query heads), 8 waves in two
// groups of four, two waves per SIMD. K and V stay in LDS for the whole unit;
// the groups take the subset's heads in pairs, one head each, side by side,
// each group in its own LDS region. The next pair's Q and dO load into
// registers while a pair is computed and go to LDS once it is done. dK and dV
// accumulate over each group's heads in registers; at the end group 1 hands
// its sums to group 0 through LDS, which adds them in that fixed order. Per
// head, with the 64 queries and 64 keys cut into 32 x 32 quadrants:
//   1. wave (qh, kb) forms quadrant (queries 32 qh.., keys 32 kb..) of S^T
//      and dP^T, P and its half of each row's Delta; the two halves of Delta
//      meet in LDS; then dS. P and dS go to LDS as hi + lo bf16 pairs
//      (about 16 significant bits), laid out [query][key];
//   2. wave (qh, kb) forms dQ^T for query half qh and the head-dim blocks of
//      half kb, from K^T and dS^T over all 64 keys, and stores dQ;
//   3. wave (kb, t) adds key block kb of dV^T = dO^T P (t = 0) or of
//      dK^T = Q^T dS (t = 1), every head-dim block.
// Under a causal mask quadrant (queries 0..31, keys 32..63) is empty: it is
// never formed, and steps 2 and 3 skip it. With one head subset dK and dV are
// stored as bf16; with several, as fp32 partials that a fixed-order sum
// finishes. Every output element comes from one thread in a fixed order, so
// the results are bitwise reproducible.
#include <math.h>

#include "attn_device.h"
#include "attn_launch.h"

namespace tam {
namespace {

constexpr int kThreads = 512;       // two groups of four waves
constexpr int kShortKeys = 64;      // the one key tile
constexpr long long kShortUnits = 256;  // one unit per compute unit, at least

struct ShortArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* part;  // several subsets: fp32 partials [nsplit][2][B*Hkv*S*D] (dK, then dV)
  int Hq, Hkv, S, nsplit;
  float c;      // softmax scale * log2(e): P = exp2(S c - LSE log2(e))
  float scale;
};

// LDS: K and V, then a region for each group of four waves: its head's Q and
// dO, and the [query][key] tiles of P and dS (hi and lo parts).
template <int D>
struct ShortLayout {
  using T = SwzTile<D>;
  using TP = SwzTile<64>;
  static constexpr int K0 = 0, V0 = T::BYTES;
  static constexpr int G0 = 2 * T::BYTES;     // group g's region at G0 + g GBYTES
  static constexpr int XQ = 0, XD = T::BYTES;  // within a region
  static constexpr int PH = 2 * T::BYTES, PL = PH + TP::BYTES, DH = PL + TP::BYTES, DL = DH + TP::BYTES;
  static constexpr int GBYTES = DL + TP::BYTES;
  static constexpr int BYTES = G0 + 2 * GBYTES;
};

// hi = bf16(x), lo = bf16(x - hi) for four values, packed in pairs.
__device__ __forceinline__ void split4(const float* x, u32x2* hi, u32x2* lo) {
  u32x2 h, l;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    h[i] = pack_bf16(x[2 * i], x[2 * i + 1]);
    l[i] = pack_bf16(x[2 * i] - bf16_lo(h[i]), x[2 * i + 1] - bf16_hi(h[i]));
  }
  *hi = h;
  *lo = l;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void attn_bwd_short_kernel(ShortArgs a) {
  using T = SwzTile<D>;
  using TP = SwzTile<64>;
  using L = ShortLayout<D>;
  constexpr int KS = D / 16;          // MFMA k-steps over the head dim
  constexpr int DB = D / 32;          // 32-wide head-dim blocks
  constexpr int DBQ = DB / 2;         // of them per wave in step 2
  constexpr int NKV = T::LOADS / 8;   // 1-KiB loads per wave per K or V tile (eight waves)
  constexpr int NX = T::LOADS / 4;    // per Q or dO tile (the group's four waves)
  static_assert(T::ROWS == kShortKeys && TP::ROW_BYTES == 128 && NKV >= 1, "tiles");
  static_assert(L::BYTES <= 160 * 1024, "LDS");
  static_assert(4 * DB * 16 * 64 * 4 <= L::GBYTES, "the dK/dV sums of a group fit its region");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[L::BYTES];

  const int S = a.S;
  const int unit = xcd_unit(blockIdx.x, gridDim.x);  // the subsets of a kv head share an XCD
  const int grp = unit / a.nsplit, sub = unit - grp * a.nsplit;  // grp = b * Hkv + kv head
  const int b = grp / a.Hkv, kvh = grp - b * a.Hkv;
  const int hps = a.Hq / a.Hkv / a.nsplit;          // query heads per subset
  const int h_first = kvh * (a.Hq / a.Hkv) + sub * hps;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave
  const int gw = wave >> 2, w4 = wave & 3;  // the wave's group and its place in it
  const int col = lane & 31, half = lane >> 5;
  const int i16 = lane & 15, dsub = 16 * ((lane >> 4) & 1);
  const int qh = w4 >> 1, kb = w4 & 1;      // steps 1 and 2: quadrant (qh, kb)
  const int kb3 = w4 >> 1;                  // step 3: key block kb3 of dV^T (w4 even) or dK^T (odd)
  const bool dk_role = w4 & 1;
  const int q = 32 * qh + col;              // the query row this lane owns in steps 1 and 2
  const int G = L::G0 + gw * L::GBYTES;     // the group's LDS region

  // Tile loads straight into LDS; rows past S read as zeros. K and V: each of
  // the eight waves issues an eighth; a group's Q and dO: each of its waves a
  // quarter.
  int lkv[NKV], lx[NX];
#pragma unroll
  for (int i = 0; i < NKV; ++i) lkv[i] = T::load_src(wave * NKV + i, lane);
#pragma unroll
  for (int i = 0; i < NX; ++i) lx[i] = T::load_src(w4 * NX + i, lane);
  auto load_kv = [&](const uint16_t* src, int dst) TAM_INLINE {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src, S * D * 2);
#pragma unroll
    for (int i = 0; i < NKV; ++i) load_lds16(r, smem + dst + (wave * NKV + i) * 1024, lkv[i]);
  };
  auto load_x = [&](const uint16_t* src, int dst) TAM_INLINE {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src, S * D * 2);
#pragma unroll
    for (int i = 0; i < NX; ++i) load_lds16(r, smem + dst + (w4 * NX + i) * 1024, lx[i]);
  };
  auto rows_of = [&](const uint16_t* base, int h) TAM_INLINE {
    return base + ((size_t)b * a.Hq + h) * S * D;
  };
  // LSE of this lane's row of head h, and LSE * log2(e) from it (+inf for a
  // row that sees no key or lies past the end: all its probabilities are 0).
  // The two are apart so that the next head's value loads during this one.
  auto lse_of = [&](int h) TAM_INLINE { return q < S ? a.lse[((size_t)b * a.Hq + h) * S + q] : -INFINITY; };
  auto lse2_from = [&](float l) TAM_INLINE { return l == -INFINITY ? INFINITY : l * kLog2e; };
  // The next pair's Q and dO come through registers while this pair runs:
  // lane l holds the 16 bytes that the direct loads would write at LDS byte
  // 1024 i + 16 l of the tile, and writes them there once the pair is done.
  u32x4 nq[NX], nd[NX];
  auto fetch_x = [&](int h) TAM_INLINE {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(rows_of(a.q, h), S * D * 2);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(rows_of(a.dout, h), S * D * 2);
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      nq[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, lx[i], 0, 0));
      nd[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rd, lx[i], 0, 0));
    }
  };

  // Per-lane offsets of the transposed reads: rows 4 half + (lane & 15) / 4
  // (+ 8 for the second read) of a 16-row block, elements 32 blk + dsub +
  // 4 (lane & 3); a lane receives element 32 blk + lane % 32 of 8 rows, and
  // k-slot t of lane half hh is row 8 (t / 4) + 4 hh + t % 4 of the block.
  int toff[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) toff[db][hi] = T::elem_off(4 * half + (i16 >> 2) + 8 * hi, db * 32 + dsub + 4 * (i16 & 3));
  int qoff[DBQ][2];  // step 2's blocks DBQ kb + j (a runtime index into toff would go to memory)
#pragma unroll
  for (int j = 0; j < DBQ; ++j)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
      qoff[j][hi] = T::elem_off(4 * half + (i16 >> 2) + 8 * hi, (DBQ * kb + j) * 32 + dsub + 4 * (i16 & 3));
  int poff[2];  // the same over the P and dS tiles, key block kb3
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) poff[hi] = TP::elem_off(4 * half + (i16 >> 2) + 8 * hi, kb3 * 32 + dsub + 4 * (i16 & 3));

  // dV^T (w4 even) or dK^T (w4 odd), head-dim block db x keys 32 kb3 + (0..31),
  // summed over the group's heads
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  // quadrant (qh, kb) holds a visible key
  const bool quad = !CAUSAL || kb <= qh;
  // the two halves of each row's Delta meet in the group's P-hi tile, before P
  float* const del = reinterpret_cast<float*>(smem + G + L::PH);
  const int xq = G + L::XQ, xd = G + L::XD;

  // The subset's heads in pairs: group 0 takes heads 0, 2, 4, ..., group 1
  // heads 1, 3, 5, ... Both groups pass the same barriers; with an odd count
  // group 1 only keeps step on the last pair.
  const int npairs = (hps + 1) / 2;
  float lse_cur = -INFINITY, lse_next = -INFINITY;
  // pair 0 goes straight into LDS with K and V; pair 1 starts into registers
  load_kv(a.k + (size_t)grp * S * D, L::K0);
  load_kv(a.v + (size_t)grp * S * D, L::V0);
  if (gw < hps) {
    load_x(rows_of(a.q, h_first + gw), xq);
    load_x(rows_of(a.dout, h_first + gw), xd);
    lse_cur = lse_of(h_first + gw);
  }
  wait_loads();
  if (2 + gw < hps) {
    fetch_x(h_first + 2 + gw);
    lse_next = lse_of(h_first + 2 + gw);
  }
  __syncthreads();
  for (int ip = 0; ip < npairs; ++ip) {
    const int h = h_first + 2 * ip + gw;
    const bool live = 2 * ip + gw < hps;  // uniform over the group
    if (ip > 0) {
      // this pair's rows, fetched during the last pair, into the freed region;
      // then the next pair's fetch
      if (live) {
#pragma unroll
        for (int i = 0; i < NX; ++i) {
          *reinterpret_cast<u32x4*>(smem + xq + (w4 * NX + i) * 1024 + 16 * lane) = nq[i];
          *reinterpret_cast<u32x4*>(smem + xd + (w4 * NX + i) * 1024 + 16 * lane) = nd[i];
        }
      }
      lse_cur = lse_next;
      if (2 * ip + 2 + gw < hps) {
        fetch_x(h + 2);
        lse_next = lse_of(h + 2);
      }
      lds_barrier();
    }
    const float lse2 = lse2_from(lse_cur);

    // 1. S^T and dP^T of the quadrant: element v of lane l is key
    //    32 kb + 8 (v / 4) + 4 half + v % 4 of row q
    float p[16], dp16[16];
    if (live) {
      f32x16 s = {}, dp = {};
      if (quad) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int kr = T::chunk_off(32 * kb + col, 2 * ks + half), qr = T::chunk_off(q, 2 * ks + half);
          s = mfma32(*reinterpret_cast<const bf16x8*>(smem + L::K0 + kr), *reinterpret_cast<const bf16x8*>(smem + xq + qr), s);
          dp = mfma32(*reinterpret_cast<const bf16x8*>(smem + L::V0 + kr), *reinterpret_cast<const bf16x8*>(smem + xd + qr), dp);
        }
      }
      float part = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = 32 * kb + 8 * (v >> 2) + 4 * half + (v & 3);
        const bool ok = quad & (key < S) & (!CAUSAL | (key <= q));  // branch-free
        const float e = fast_exp2(fmaf(s[v], a.c, -lse2));
        p[v] = ok ? e : 0.f;
        dp16[v] = dp[v];
        part = fmaf(p[v], dp[v], part);
      }
      part = sum_halves(part);  // sum over the quadrant's 32 keys, in both halves
      if (half == 0) del[kb * 64 + q] = part;
    }
    lds_barrier();
    const float delta = live ? del[q] + del[64 + q] : 0.f;  // the same order in both waves of the row
    lds_barrier();  // every wave has its Delta before P is written over it
    // P and dS (row q, four consecutive keys per group) into the [query][key] tiles
    if (live && quad) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float ds[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ds[r] = p[4 * g + r] * (dp16[4 * g + r] - delta);
        const int off = TP::elem_off(q, 32 * kb + 8 * g + 4 * half);
        u32x2 hv, lv;
        split4(p + 4 * g, &hv, &lv);
        *reinterpret_cast<u32x2*>(smem + G + L::PH + off) = hv;
        *reinterpret_cast<u32x2*>(smem + G + L::PL + off) = lv;
        split4(ds, &hv, &lv);
        *reinterpret_cast<u32x2*>(smem + G + L::DH + off) = hv;
        *reinterpret_cast<u32x2*>(smem + G + L::DL + off) = lv;
      }
    }
    lds_barrier();

    if (live) {
      // 2. dQ^T (head-dim blocks DBQ kb .., rows of query half qh) = K^T dS^T:
      //    A = K^T read transposed, B = dS^T rows of the tiles, k-slots matching
      f32x16 dq[DBQ];
#pragma unroll
      for (int j = 0; j < DBQ; ++j) dq[j] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (CAUSAL && kk > qh) continue;  // the empty quadrant
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int e0 = 32 * kk + 16 * k2 + 4 * half;
          const u32x2 h0 = *reinterpret_cast<const u32x2*>(smem + G + L::DH + TP::elem_off(q, e0));
          const u32x2 h1 = *reinterpret_cast<const u32x2*>(smem + G + L::DH + TP::elem_off(q, e0 + 8));
          const u32x2 l0 = *reinterpret_cast<const u32x2*>(smem + G + L::DL + TP::elem_off(q, e0));
          const u32x2 l1 = *reinterpret_cast<const u32x2*>(smem + G + L::DL + TP::elem_off(q, e0 + 8));
          const bf16x8 bh = __builtin_bit_cast(bf16x8, u32x4{h0[0], h0[1], h1[0], h1[1]});
          const bf16x8 bl = __builtin_bit_cast(bf16x8, u32x4{l0[0], l0[1], l1[0], l1[1]});
          const unsigned char* kt = smem + L::K0 + (32 * kk + 16 * k2) * T::ROW_BYTES;
#pragma unroll
          for (int j = 0; j < DBQ; ++j) {
            const bf16x8 ak = lds_read_tr_pair(reinterpret_cast<const uint16_t*>(kt + qoff[j][0]),
                                               reinterpret_cast<const uint16_t*>(kt + qoff[j][1]));
            dq[j] = mfma32(ak, bh, dq[j]);
            dq[j] = mfma32(ak, bl, dq[j]);
          }
        }
      }
      if (q < S) {
        // lane holds columns 32 db + 8 i + 4 half + (0..3) of row q; pairs of i
        // are merged across the halves into 16-byte stores
        uint16_t* op = a.dq + ((size_t)b * a.Hq + h) * S * D + (size_t)q * D + 8 * half;
#pragma unroll
        for (int j = 0; j < DBQ; ++j)
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            u32x2 w[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const int ii = 2 * m + t;
              w[t] = u32x2{pack_bf16(a.scale * dq[j][4 * ii], a.scale * dq[j][4 * ii + 1]),
                           pack_bf16(a.scale * dq[j][4 * ii + 2], a.scale * dq[j][4 * ii + 3])};
            }
            *reinterpret_cast<u32x4*>(op + 32 * (DBQ * kb + j) + 16 * m) = pair_halves(w[0], w[1]);
          }
      }

      // 3. key block kb3 of dV^T += dO^T P or dK^T += Q^T dS, over 16-row blocks of queries
      const int xt = dk_role ? xq : xd;
      const int yh = G + (dk_role ? L::DH : L::PH), yl = G + (dk_role ? L::DL : L::PL);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (CAUSAL && kb3 > qb) continue;  // the empty quadrant
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int r0 = 32 * qb + 16 * k2;
          const unsigned char* yhp = smem + yh + r0 * TP::ROW_BYTES;
          const unsigned char* ylp = smem + yl + r0 * TP::ROW_BYTES;
          const bf16x8 bh = lds_read_tr_pair(reinterpret_cast<const uint16_t*>(yhp + poff[0]),
                                             reinterpret_cast<const uint16_t*>(yhp + poff[1]));
          const bf16x8 bl = lds_read_tr_pair(reinterpret_cast<const uint16_t*>(ylp + poff[0]),
                                             reinterpret_cast<const uint16_t*>(ylp + poff[1]));
          const unsigned char* xp = smem + xt + r0 * T::ROW_BYTES;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x8 ax = lds_read_tr_pair(reinterpret_cast<const uint16_t*>(xp + toff[db][0]),
                                               reinterpret_cast<const uint16_t*>(xp + toff[db][1]));
            acc[db] = mfma32(ax, bh, acc[db]);
            acc[db] = mfma32(ax, bl, acc[db]);
          }
        }
      }
    }
    __syncthreads();  // the group's Q, dO and tiles are free for the next pair
  }

  // Group 1 hands its sums to group 0 through its own region; group 0 adds
  // them to its own (a fixed order) and stores.
  float* hand = reinterpret_cast<float*>(smem + L::G0 + L::GBYTES) + w4 * (DB * 16 * 64) + lane;
  if (gw == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) hand[(16 * db + v) * 64] = acc[db][v];
  }
  __syncthreads();
  if (gw == 1) return;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[db][v] += hand[(16 * db + v) * 64];

  // dV^T or dK^T: element v of lane l is head-dim column 32 db + 8 (v / 4) +
  // 4 half + v % 4 of key 32 kb3 + col
  const int key = 32 * kb3 + col;
  if (key < S) {
    const float f = dk_role ? a.scale : 1.f;
    const size_t row = ((size_t)grp * S + key) * D;
    if (a.nsplit == 1) {
      uint16_t* op = (dk_role ? a.dk : a.dv) + row + 8 * half;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          u32x2 w[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int ii = 2 * m + t;
            w[t] = u32x2{pack_bf16(f * acc[db][4 * ii], f * acc[db][4 * ii + 1]),
                         pack_bf16(f * acc[db][4 * ii + 2], f * acc[db][4 * ii + 3])};
          }
          *reinterpret_cast<u32x4*>(op + 32 * db + 16 * m) = pair_halves(w[0], w[1]);
        }
    } else {
      const size_t total = (size_t)gridDim.x / a.nsplit * S * D;
      float* op = a.part + ((size_t)sub * 2 + (dk_role ? 0 : 1)) * total + row + 4 * half;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          *reinterpret_cast<f32x4*>(op + 32 * db + 8 * ii) =
              f32x4{f * acc[db][4 * ii], f * acc[db][4 * ii + 1], f * acc[db][4 * ii + 2], f * acc[db][4 * ii + 3]};
    }
  }
}

}  // namespace

bool bwd_short_path(const AttnShape& sh) {
  return sh.Sq == sh.Sk && sh.Sq <= kShortKeys && sh.dlt == 0 && !sh.drop_t && !sh.rope;
}

// The fewest head subsets (a divisor of the group) that give every compute
// unit a workgroup; one subset needs no partials.
int bwd_short_split(const AttnShape& sh) {
  const int g = sh.Hq / sh.Hkv;
  const long long groups = (long long)sh.B * sh.Hkv;
  for (int ns = 1; ns < g; ++ns)
    if (g % ns == 0 && groups * ns >= kShortUnits) return ns;
  return g;
}

size_t bwd_short_workspace_bytes(const AttnShape& sh) {
  const int ns = bwd_short_split(sh);
  return ns > 1 ? (size_t)ns * 2 * sh.B * sh.Hkv * sh.Sk * sh.D * sizeof(float) : 0;
}

hipError_t launch_bwd_short(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const uint16_t* dout, const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                            float* part, hipStream_t stream) {
  ShortArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.part = part;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.S = sh.Sq;
  a.nsplit = bwd_short_split(sh);
  a.c = sh.scale * kLog2e;
  a.scale = sh.scale;
  const long long grid = (long long)sh.B * sh.Hkv * a.nsplit;
  void* args[] = {&a};
  const void* kern =
      sh.D == 128 ? (sh.causal ? reinterpret_cast<const void*>(&attn_bwd_short_kernel<128, true>)
                               : reinterpret_cast<const void*>(&attn_bwd_short_kernel<128, false>))
                  : (sh.causal ? reinterpret_cast<const void*>(&attn_bwd_short_kernel<64, true>)
                               : reinterpret_cast<const void*>(&attn_bwd_short_kernel<64, false>));
  return hipLaunchKernel(kern, dim3((unsigned)grid), dim3(kThreads), args, 0, stream);
}

}  // namespace tam
