// Backward pass of exact attention for gfx950.
//
// Follows the "Recomputation" bullet of the page "使用 PyTorch FSDP 微調 Llama 2 70B"
// (agentlenshq.com), section "Flash Attention": the probabilities are
// recomputed tile by tile from Q, K and the forward pass's log-sum-exp
// instead of being stored, so no N x N matrix is ever written.
//
// With P = exp(s - LSE), L = sum(O * dO):
//   dV = P^T dO,  dP = dO V^T,  Delta_i = sum_d dO_id O_id,
//   dS = P * (dP - Delta),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Kernels, all on the caller's stream:
//   1. prep:  Delta~ = sum_d dO_id O_id from the stored bf16 O, and
//             LSE * log2(e), per query row (workspace). Only the block
//             protocol runs it as a kernel of its own; on the whole-sequence
//             path the dQ kernel forms both for its rows (its dS wave holds
//             the row's dO already) and stores lse2 for kernel 3.
//   2. dq:    query-stationary, like the forward pass: dQ^T += K^T dS^T, with
//             the same wave-pair split as kernel 3 (one wave computes S, P and
//             P K, its partner dP, dS and dQ one key tile behind). It also
//             makes Delta exact: with dS~ = P (dP - Delta~) and sum_j P_ij = 1,
//             Delta_i - Delta~_i = sum_j dS~_ij =: c_i, so
//             dQ_i = scale (sum_j dS~_ij K_j - c_i sum_j P_ij K_j), and the exact
//             Delta_i = Delta~_i + c_i is written back for kernel 3. This removes
//             the error that rounding O to bf16 puts into Delta. For the fp16
//             dK/dV kernel it also writes fp16 copies of Q and dO and the
//             block exponents of Q, dO and Delta. Sequences of at most 64 (32)
//             rows pack 2 (4) query heads of a group into one 128-row unit.
//   1b. k16:  fp16 copy of K with tile exponents (and those of V), before an
//             fp16 dQ kernel.
//   1c. rows16: block protocol only, before an fp16 dK/dV call: the fp16
//             copies of the query block's Q and dO with the block exponents of
//             Q, dO and the exact Delta (which kernel 2 writes on the
//             whole-sequence path).
//   3. dkdv:  key-stationary. One unit = (batch, kv head, 128-key tile, subset
//             of the group's query heads); 8 waves in pairs own 32 keys per
//             pair while 64-row Q/dO tiles stream through LDS. In each pair one
//             wave keeps K and dV^T in registers and computes P, which it hands
//             to its partner through LDS; the partner keeps V and dK^T, computes
//             dP and dS, one tile behind, so that the two waves' vector work
//             and matrix products overlap. No atomics: each unit owns its output
//             rows; with more than one head subset, fp32 partials go to the
//             workspace.
//   4. reduce (only with several subsets): sums the partials in a fixed order.
// Precision of the gradient products (P for dV, dS for dK and dQ): for short
// sequences and the block protocol, the second operand enters the bf16 MFMA
// as a hi + lo pair of bf16 values, about 16 significant bits. Whole-sequence
// calls over 512 keys or more (with or without dropout) instead run every
// product of the dK/dV kernel, and those with K in the dQ kernel (S, P K and
// dQ), in fp16 (11 significant bits, one product each) on power-of-two scaled
// operands: copies of Q and dO that the dQ kernel writes, and a copy of K made
// by a small kernel of its own (1b) before it.
// Every output element is produced by one thread in a fixed order, so the
// results are bitwise reproducible.
#include <math.h>

#include <algorithm>
#include <functional>
#include <queue>
#include <type_traits>
#include <vector>

#include "attn_device.h"
#include "attn_launch.h"

namespace tam {
namespace {

constexpr int kThreads = 256;
constexpr int kBwdThreads = 512;   // dQ and dK/dV: 8 waves, two per SIMD
constexpr int kQBR = 128;   // dq: query rows per workgroup
constexpr int kQBC = 64;    // dq: keys per tile
constexpr int kKBC = 128;   // dkdv: keys per workgroup
constexpr int kKBR = 64;    // dkdv: query rows per streamed tile
constexpr int kTargetUnits = 1024;
constexpr int kF16MinKeys = 512;
// Block protocol: a separate pass converts the query block's Q and dO for each
// key block's dK/dV call, about twice the traffic of the dQ kernel's copies.
constexpr int kF16MinBlockKeys = 1024;

// ---------------------------------------------------------------------------
// workspace layout
// ---------------------------------------------------------------------------
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Head subsets per (batch, kv head, key tile) unit of the dK/dV kernel. More
// subsets give more, shorter units, which balance better over the CUs, at the
// cost of fp32 partials and the reduce pass.
//
// Whole-sequence calls: the smallest divisor of g whose units, dealt heaviest
// first onto kCUs workgroup slots (one resident unit per CU), finish within 2%
// of the ideal time, else the best one. Units are costed with the causal
// square mask whatever the call's mask, so that the workspace size (asked
// without the mask) and the launch agree. Block calls keep the simpler rule of
// enough units (their workspace is sized once for every offset).
constexpr int kCUs = 256;
constexpr long long kSimUnits = 1 << 14;  // beyond this many units the deal is balanced anyway

double deal_efficiency(const AttnShape& sh, int ns) {
  const int g = sh.Hq / sh.Hkv, hps = g / ns;
  const int NT = (sh.Sk + kKBC - 1) / kKBC, NQ = (sh.Sq + kKBR - 1) / kKBR;
  const long long streams = (long long)sh.B * sh.Hkv * ns;
  if (streams * NT >= kSimUnits) return 1.0;
  std::priority_queue<long long, std::vector<long long>, std::greater<long long>> load;
  for (int c = 0; c < kCUs; ++c) load.push(0);
  long long total = 0;
  for (int jt = 0; jt < NT; ++jt) {           // key tile 0 is the heaviest under the causal mask
    const int i_min = (jt * kKBC) / kKBR;
    const long long cost = (long long)std::max(0, NQ - i_min) * hps + 2;  // + loads and epilogue
    for (long long u = 0; u < streams; ++u) {
      const long long t = load.top();
      load.pop();
      load.push(t + cost);
      total += cost;
    }
  }
  long long makespan = 0;
  while (!load.empty()) {
    makespan = std::max(makespan, load.top());
    load.pop();
  }
  return makespan ? (double)total / kCUs / makespan : 1.0;
}

int choose_head_split(const AttnShape& sh, bool block) {
  const int g = sh.Hq / sh.Hkv;
  if (block) {
    const long long units = (long long)sh.B * sh.Hkv * ((sh.Sk + kKBC - 1) / kKBC);
    int ns = 1;
    while (units * ns < kTargetUnits && ns < g) {
      int next = ns + 1;
      while (g % next) ++next;
      ns = next;
    }
    return ns;
  }
  AttnShape sq = sh;
  sq.Sq = sq.Sk = std::max(sh.Sq, sh.Sk);
  int best = 1;
  double best_eff = -1.0;
  for (int ns = 1; ns <= g; ++ns) {
    if (g % ns) continue;
    const double eff = deal_efficiency(sq, ns);
    if (eff >= 0.98) return ns;
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = ns;
    }
  }
  return best;
}

struct WsLayout {
  size_t delta, lse2, csum, acc_dq, acc_pk, q16, do16, eq, edo, edl, k16, ek, ev, part, total;
  int nsplit;
};

// Backward workspace. Whole-sequence pass: Delta, lse2, the fp16 copies of Q
// and dO with their block exponents (and that of Delta) for the fp16 dK/dV
// kernel, the fp16 copy of K with its tile exponents (and those of V) for the
// fp16 dQ kernel, and the dK/dV partials. Block protocol (block = true): Delta, lse2,
// the running c = sum dS~ per row, the fp32 sums of dS~ K and P K over the key
// blocks seen so far, the fp16 copies of Q and dO with the block exponents
// (for the fp16 dK/dV kernel), the fp16 copy of the current key block's K
// with the tile exponents (for the fp16 dQ kernel), and the partials.
WsLayout ws_layout(const AttnShape& sh, bool block = false) {
  WsLayout w;
  const size_t rows = (size_t)sh.B * sh.Hq * sh.Sq;
  const size_t blocks = (size_t)sh.B * sh.Hq * ((sh.Sq + 31) / 32);
  w.nsplit = choose_head_split(sh, block);
  w.delta = 0;
  w.lse2 = align256(rows * 4);
  size_t off = w.lse2 + align256(rows * 4);
  w.csum = w.acc_dq = w.acc_pk = w.q16 = w.do16 = w.eq = w.edo = w.edl = w.k16 = w.ek = w.ev = 0;
  if (block) {
    w.csum = off;
    w.acc_dq = w.csum + align256(rows * 4);
    w.acc_pk = w.acc_dq + align256(rows * sh.D * 4);
    off = w.acc_pk + align256(rows * sh.D * 4);
  }
  {
    w.q16 = off;
    w.do16 = w.q16 + align256(rows * sh.D * 2);
    w.eq = w.do16 + align256(rows * sh.D * 2);
    w.edo = w.eq + align256(blocks * 4);
    w.edl = w.edo + align256(blocks * 4);
    off = w.edl + align256(blocks * 4);
  }
  {
    const size_t kv_tiles = (size_t)sh.B * sh.Hkv * ((sh.Sk + 63) / 64);
    w.k16 = off;
    w.ek = w.k16 + align256((size_t)sh.B * sh.Hkv * sh.Sk * sh.D * 2);
    w.ev = w.ek + align256(kv_tiles * 4);
    off = w.ev + align256(kv_tiles * 4);
  }
  w.part = off;
  const size_t kv_elems = (size_t)sh.B * sh.Hkv * sh.Sk * sh.D;
  w.total = w.part + (w.nsplit > 1 ? align256((size_t)w.nsplit * 2 * kv_elems * 4) : 0);
  // a whole-sequence call of at most 64 tokens may take the one-kernel path,
  // whose only workspace is its partials (from offset 0)
  if (!block) {
    AttnShape s = sh;
    s.drop_t = 0;
    s.rope = nullptr;
    if (bwd_short_path(s)) w.total = std::max(w.total, align256(bwd_short_workspace_bytes(s)));
  }
  return w;
}

// ---------------------------------------------------------------------------
// 1. prep: Delta_i = sum_d dO_id * O_id, lse2_i = LSE_i * log2(e)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void attn_bwd_prep_kernel(const uint16_t* o, const uint16_t* dout,
                                                                 const float* lse, float* delta,
                                                                 float* lse2, long long rows) {
  constexpr int TPR = D / 8;         // threads per row, 8 elements each
  constexpr int RPB = kThreads / TPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 ov = *reinterpret_cast<const u32x4*>(o + row * D + part * 8);
    const u32x4 dv = *reinterpret_cast<const u32x4*>(dout + row * D + part * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(bf16_lo(ov[w]), bf16_lo(dv[w]), acc);
      acc = fmaf(bf16_hi(ov[w]), bf16_hi(dv[w]), acc);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) {
    delta[row] = acc;
    // a row that sees no key at all has LSE = -inf; +inf here makes every
    // recomputed probability of that row exactly 0
    lse2[row] = lse[row] == -INFINITY ? INFINITY : lse[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// 1b. fp16 copy of K with one exponent per 64-key tile, and the exponent of
//     each V tile (for the fp16 dQ kernel): tile t of a kv head is stored as
//     K * 2^(14 - ek(t)), ek = ceil(log2 of the tile's largest |K|)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void attn_bwd_k16_kernel(const uint16_t* k, const uint16_t* v,
                                                                uint16_t* k16, int* ek, int* ev, int Sk,
                                                                int ntile) {
  constexpr int CPR = D / 8;                   // 16-byte chunks per row
  constexpr int NC = 64 * CPR / kThreads;      // chunks per thread
  __shared__ uint32_t red[2][kThreads / 64];
  const int tile = blockIdx.x % ntile;
  const size_t head = blockIdx.x / ntile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t base = (head * Sk + (size_t)tile * 64) * D;
  bf16x8 kc[NC];
  uint32_t mk = 0, mv = 0;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = tid + kThreads * i, row = c / CPR;
    const bool ok = tile * 64 + row < Sk;
    const size_t off = base + (size_t)c * 8;   // chunks of consecutive rows are contiguous
    kc[i] = ok ? *reinterpret_cast<const bf16x8*>(k + off) : __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    const bf16x8 vc = ok ? *reinterpret_cast<const bf16x8*>(v + off) : __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    const uint32_t a = bf16x8_max_mag(kc[i]), b = bf16x8_max_mag(vc);
    mk = mk > a ? mk : a;
    mv = mv > b ? mv : b;
  }
  mk = wave_max(mk);
  mv = wave_max(mv);
  if (lane == 0) {
    red[0][wave] = mk;
    red[1][wave] = mv;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    mk = mk > red[0][w] ? mk : red[0][w];
    mv = mv > red[1][w] ? mv : red[1][w];
  }
  const int e = ceil_log2(__builtin_bit_cast(float, mk << 16));
  const float sc = __builtin_ldexpf(1.f, 14 - e);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = tid + kThreads * i, row = c / CPR;
    if (tile * 64 + row < Sk) *reinterpret_cast<f16x8*>(k16 + base + (size_t)c * 8) = bf16x8_to_f16x8(kc[i], sc);
  }
  if (tid == 0) {
    ek[head * ntile + tile] = e;
    ev[head * ntile + tile] = ceil_log2(__builtin_bit_cast(float, mv << 16));
  }
}

// ---------------------------------------------------------------------------
// 1c. Block protocol: fp16 copies of a query block's Q and dO with the
//     exponents of each 32-row block of Q, dO and the exact Delta, for the
//     fp16 dK/dV kernel (on the whole-sequence path the dQ kernel writes
//     them): block b is stored as x * 2^(14 - e(b)), e = ceil(log2 of its
//     largest |x|). One workgroup per (batch * head, 32-row block).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void attn_bwd_rows16_kernel(const uint16_t* q, const uint16_t* dout,
                                                                   const float* delta, uint16_t* q16,
                                                                   uint16_t* do16, int* eq, int* edo, int* edl,
                                                                   int Sq, int nblk) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int NC = 32 * CPR / kThreads;    // chunks per thread
  static_assert(NC >= 1, "chunks");
  __shared__ uint32_t red[3][kThreads / 64];
  const int blk = blockIdx.x % nblk;
  const size_t bh = blockIdx.x / nblk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row0 = blk * 32;
  const size_t base = (bh * Sq + (size_t)row0) * D;
  const bf16x8 zero = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  bf16x8 qc[NC], dc[NC];
  uint32_t mq = 0, md = 0;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = tid + kThreads * i, row = c / CPR;
    const bool ok = row0 + row < Sq;
    const size_t off = base + (size_t)c * 8;   // chunks of consecutive rows are contiguous
    qc[i] = ok ? *reinterpret_cast<const bf16x8*>(q + off) : zero;
    dc[i] = ok ? *reinterpret_cast<const bf16x8*>(dout + off) : zero;
    const uint32_t a = bf16x8_max_mag(qc[i]), b = bf16x8_max_mag(dc[i]);
    mq = mq > a ? mq : a;
    md = md > b ? md : b;
  }
  const float dl = (tid < 32 && row0 + tid < Sq) ? fabsf(delta[bh * Sq + row0 + tid]) : 0.f;
  mq = wave_max(mq);
  md = wave_max(md);
  const uint32_t ml = __builtin_bit_cast(uint32_t, wave_max(dl));   // non-negative: bits order as values
  if (lane == 0) {
    red[0][wave] = mq;
    red[1][wave] = md;
    red[2][wave] = ml;
  }
  __syncthreads();
  uint32_t mlx = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    mq = mq > red[0][w] ? mq : red[0][w];
    md = md > red[1][w] ? md : red[1][w];
    mlx = mlx > red[2][w] ? mlx : red[2][w];
  }
  const int e_q = ceil_log2(__builtin_bit_cast(float, mq << 16));
  const int e_d = ceil_log2(__builtin_bit_cast(float, md << 16));
  const float sq = __builtin_ldexpf(1.f, 14 - e_q), sd = __builtin_ldexpf(1.f, 14 - e_d);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = tid + kThreads * i, row = c / CPR;
    if (row0 + row < Sq) {
      const size_t off = base + (size_t)c * 8;
      *reinterpret_cast<f16x8*>(q16 + off) = bf16x8_to_f16x8(qc[i], sq);
      *reinterpret_cast<f16x8*>(do16 + off) = bf16x8_to_f16x8(dc[i], sd);
    }
  }
  if (tid == 0) {
    const size_t o = bh * nblk + blk;
    eq[o] = e_q;
    edo[o] = e_d;
    edl[o] = ceil_log2(__builtin_bit_cast(float, mlx));
  }
}

// ---------------------------------------------------------------------------
// 2. dK/dV, key-stationary
// ---------------------------------------------------------------------------
struct DkdvArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* delta;
  const float* lse2;
  uint16_t* dk;
  uint16_t* dv;
  float* part;  // [nsplit][2][B*Hkv*Sk*D] fp32 partials when nsplit > 1
  int Hq, Hkv, Sq, Sk, dlt, nsplit;
  float c;      // scale * log2(e)
  float scale;
  DropParams drop;  // dropout on the probabilities (DROP kernels only)
  const float2* rope_inv;  // (cos, sin) table [Sk][D/2]: rotate dK back; null = none
  // fp16 kernels: q and dout are the dQ kernel's fp16 copies, and these its
  // block exponents of Q, dO and the exact Delta ([B*Hq][ceil(Sq/32)])
  const int* eq;
  const int* edo;
  const int* edl;
  TileSched sched;  // streams = (batch*Hkv + kv head) * nsplit + subset; tiles = key tiles
};

// LDS layout of the dK/dV kernel, one array. The two waves of a pair work one
// streamed tile apart (see the kernel), so Q is kept in three stages (step t in
// stage t % 3), dO in two (t % 2), the lse2/delta rows in three, and the
// probabilities one wave of each pair hands to the other in two.
template <int D>
struct DkdvLayout {
  using T = SwzTile<D>;
  static constexpr int Q0 = 0, DO0 = 3 * T::BYTES;
  static constexpr int F0 = 5 * T::BYTES;            // lse2[64], delta[64] per stage
  static constexpr int F_STAGE = 2 * kKBR * 4;
  static constexpr int PB = F0 + 3 * F_STAGE;         // P: 4 key blocks x 64 rows x 32 keys fp32 per stage
  static constexpr int PB_BLOCK = kKBR * 32 * 4;
  static constexpr int PB_STAGE = 4 * PB_BLOCK;
  static constexpr int BYTES = PB + 2 * PB_STAGE;
};

// F16: every product runs on fp16 operands, one product per gradient with no
// lo halves. Q and dO come as the dQ kernel's fp16 copies (each 32-row block
// b scaled by s_Q(b) = 2^(14 - eQ(b)), s_dO(b) = 2^(14 - eD(b))); each wave
// turns its 32 rows of K or V into fp16 with its own s_K or s_V. The block
// scales are folded into per-step scalars: S' = s_Q s_K S, so c' = c /
// (s_Q s_K); the probabilities go to the dV product as P W / s_dO(b), where
// W = 2^15 min_b s_dO(b) over the unit's blocks keeps them at or below 2^15;
// and dS goes to the dK product as dS U / s_Q(b), where U is the largest power
// of two keeping every block's dS at or below 2^15, from the bound
// |dS| <= r |dP| + |Delta| <= D 2^(eD + eV + eR) + 2^eDelta (r <= 2^eR the
// dropout scale, 1 without dropout). dV = r acc / W and
// dK = scale acc / U at the end.
template <int D, bool CAUSAL, bool DROP = false, bool F16 = false>
__global__ __attribute__((amdgpu_flat_work_group_size(kBwdThreads, kBwdThreads), amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv_kernel(DkdvArgs a) {
  using T = SwzTile<D>;
  using L = DkdvLayout<D>;
  using Op = std::conditional_t<F16, f16x8, bf16x8>;  // MFMA operand type
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int SLD = T::LOADS / 4;             // streamed Q/dO loads per wave per tile
  constexpr int kLog2D = D == 128 ? 7 : 6;
  static_assert(kKBR == T::ROWS && kKBC == 2 * T::ROWS, "tile sizes");
  static_assert(L::BYTES <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[L::BYTES];

  int stream, t;
  if (!sched_decode(a.sched, blockIdx.x, &stream, &t)) return;
  const int jt = a.sched.NT - 1 - t;  // key tile; ascending = heaviest first when causal
  const int grp = stream / a.nsplit, sub = stream - grp * a.nsplit;
  const int b = grp / a.Hkv;
  const int kvh = grp - b * a.Hkv;
  const int g = a.Hq / a.Hkv;
  const int hps = g / a.nsplit;           // query heads per subset
  const int h_first = kvh * g + sub * hps;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave
  const int kblk = wave & 3;         // this wave's 32 keys within the unit
  const bool vrole = wave < 4;       // P and dV (with K resident); else dP, dS and dK (with V resident)
  const int col = lane & 31, half = lane >> 5;
  const int Sq = a.Sq, Sk = a.Sk, dlt = a.dlt;
  const size_t kv_base = (size_t)grp * Sk * D;
  const int kvt0 = jt * kKBC;
  const int kvb0 = kvt0 + 32 * kblk;   // this wave's first key
  const int kvrow = kvb0 + col;        // the key this lane owns
  const uint32_t lds0 = lds_address(smem);

  // K (for S) or V (for dP) rows of this wave's keys as MFMA B operands; in
  // the fp16 kernels scaled by 2^(14 - e_kv) with the exponent of the wave's rows.
  Op kvf[KS];
  int e_kv = 0;
  {
    const uint16_t* src = (vrole ? a.k : a.v) + kv_base + (size_t)kvrow * D + 8 * half;
    bf16x8 raw[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      raw[ks] = kvrow < Sk ? *reinterpret_cast<const bf16x8*>(src + 16 * ks)
                          : __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    if constexpr (F16) {
      uint32_t m = 0;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t mk = bf16x8_max_mag(raw[ks]);
        m = m > mk ? m : mk;
      }
      e_kv = __builtin_amdgcn_readfirstlane(ceil_log2(__builtin_bit_cast(float, wave_max(m) << 16)));
      const float sc = __builtin_ldexpf(1.f, 14 - e_kv);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kvf[ks] = bf16x8_to_f16x8(raw[ks], sc);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kvf[ks] = raw[ks];
    }
  }

  // Per-lane LDS offsets (see SwzTile) into the stage this wave reads next: rr
  // for the row-by-key products (Q for the P role, dO for the dS role), tt for
  // the transposed reads (dO, resp. Q). They move to the next stage in place,
  // by a uniform step, so that a runtime stage costs no registers.
  const int i16 = lane & 15;
  const int dsub = 16 * ((lane >> 4) & 1);
  int rr[KS], tt[DB][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) rr[ks] = (vrole ? L::Q0 : L::DO0) + T::chunk_off(col, 2 * ks + half);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
      tt[db][hi] = (vrole ? L::DO0 : L::Q0) +
                   T::elem_off(4 * half + (i16 >> 2) + 8 * hi, db * 32 + dsub + 4 * (i16 & 3));
  // stage step after step st: Q stages cycle through three, dO stages through two
  auto q_next = [&](int st) TAM_INLINE { return st % 3 == 2 ? -2 * T::BYTES : T::BYTES; };
  auto do_next = [&](int st) TAM_INLINE { return (st & 1) ? -T::BYTES : T::BYTES; };
  auto move_rr = [&](int by) TAM_INLINE {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) rr[ks] += by;
  };
  auto move_tt = [&](int by) TAM_INLINE {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) tt[db][hi] += by;
  };
  auto f_at = [&](int st) TAM_INLINE { return L::F0 + (st % 3) * L::F_STAGE; };
  // this lane's slots of the P hand-off block of stage 0: element v of 32-row
  // block qs at (16 qs + v) * 64 + lane
  float* const pbuf = reinterpret_cast<float*>(smem + L::PB + kblk * L::PB_BLOCK) + lane;
  auto pb_at = [&](int st) TAM_INLINE { return pbuf + (st & 1) * (L::PB_STAGE / 4); };

  const int NQ = (Sq + kKBR - 1) / kKBR;
  // first query tile with a row that sees the unit's first key (row >= kvt0 - dlt)
  const int i_min = CAUSAL ? (kvt0 - dlt <= 0 ? 0 : (kvt0 - dlt) / kKBR) : 0;
  const int per_head = max(0, NQ - i_min);  // query tiles visited per head
  const int nsteps = per_head * hps;

  // fp16 kernels: unit-wide exponents over the 32-row blocks the unit visits,
  // E_dO = max eD (W = 2^(29 - E_dO)) and, for the dS role,
  // E_U = max (eQ + max(log2 D + eD + eV + eR, eDelta)) (U = 2^(28 - E_U)),
  // with 2^eR >= r the dropout scale (eR = 0 without dropout).
  const int nblk = (Sq + 31) / 32;
  int E_dO = kMinExp, E_U = kMinExp;
  if constexpr (F16) {
    const int eR = DROP ? ceil_log2(a.drop.r) : 0;
    const int nb = 2 * per_head;  // blocks per head: query tiles i_min .. NQ - 1
    for (int i = lane; i < nb * hps; i += 64) {
      const int hh = i / nb;
      const int blk = 2 * i_min + (i - hh * nb);
      if (blk < nblk) {
        const size_t o = ((size_t)b * a.Hq + h_first + hh) * nblk + blk;
        const int ed = a.edo[o];
        E_dO = max(E_dO, ed);
        if (!vrole) E_U = max(E_U, a.eq[o] + max(kLog2D + ed + e_kv + eR, a.edl[o]));
      }
    }
    E_dO = __builtin_amdgcn_readfirstlane(wave_max(E_dO));
    E_U = __builtin_amdgcn_readfirstlane(wave_max(E_U));
  }

  // Steps visit (query head, query tile) with tiles from the last one down and
  // the subset's heads innermost, so that the units resident at the same time
  // (whatever their key tile) stream the same Q/dO tiles together and share
  // them in L2. A cursor walks them without divisions.
  struct Cursor {
    int h, it;
  };
  auto advance = [&](Cursor& cu) TAM_INLINE {
    if (++cu.h == h_first + hps) {
      cu.h = h_first;
      --cu.it;
    }
  };
  // the whole workgroup takes the same branch: the tile meets the diagonal of
  // the unit's 128 keys, or the end of the sequence
  auto masked_at = [&](int it) TAM_INLINE {
    return (CAUSAL && it * kKBR + dlt < kvt0 + kKBC) || it * kKBR + kKBR > Sq || kvt0 + kKBC > Sk;
  };

  int sld[SLD];
#pragma unroll
  for (int i = 0; i < SLD; ++i) sld[i] = T::load_src((wave * SLD + i) % T::LOADS, lane);

  // fp16 kernels: the step's block exponents, loaded with its tiles; lanes
  // 0..3 hold eQ of blocks 0, 1 and eD of blocks 0, 1 of the query tile.
  int ex4 = 0;
  struct StepExp {
    int q[2], d[2];
  };
  auto step_exp = [&]() TAM_INLINE {
    StepExp e;
    e.q[0] = __builtin_amdgcn_readlane(ex4, 0);
    e.q[1] = __builtin_amdgcn_readlane(ex4, 1);
    e.d[0] = __builtin_amdgcn_readlane(ex4, 2);
    e.d[1] = __builtin_amdgcn_readlane(ex4, 3);
    return e;
  };

  // Q, dO tiles and their lse2, delta rows of step st (at cursor cu) straight
  // into its stages; rows past Sq read as zeros.
  auto issue = [&](int st, const Cursor& cu) TAM_INLINE {
    const int row0 = cu.it * kKBR;
    const size_t bh = (size_t)b * a.Hq + cu.h;
    if constexpr (F16) {
      // every lane loads (a block past the end reads the last one: its rows
      // are all masked), so no copy of the result has to wait for it
      const int blk = min(2 * cu.it + (lane & 1), nblk - 1);
      ex4 = ((lane & 2) ? a.edo : a.eq)[bh * nblk + blk];
    }
    const int rows_left = Sq - row0;
    const __amdgpu_buffer_rsrc_t rqd = make_rsrc(a.q + (bh * Sq + row0) * D, rows_left * D * 2);
    const __amdgpu_buffer_rsrc_t rdd = make_rsrc(a.dout + (bh * Sq + row0) * D, rows_left * D * 2);
    const uint32_t qb = lds0 + L::Q0 + (st % 3) * T::BYTES, dob = lds0 + L::DO0 + (st & 1) * T::BYTES;
#pragma unroll
    for (int i = 0; i < SLD; ++i) {
      const int gi = wave * SLD + i, which = gi / T::LOADS, li = gi % T::LOADS;
      dma16(which == 0 ? rqd : rdd, (which == 0 ? qb : dob) + li * 1024, sld[i]);
    }
    if (wave < 2) {
      const float* src = wave == 0 ? a.lse2 : a.delta;
      const __amdgpu_buffer_rsrc_t rf = make_rsrc(src + bh * Sq + row0, rows_left * 4);
      dma4(rf, lds0 + f_at(st) + wave * kKBR * 4, lane * 4);
    }
  };

  f32x16 acc[DB];   // dV^T (P role) or dK^T (dS role)
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  const float c = a.c;

  // x = A B^T over the head dim for the rows of the tile at rr and this
  // wave's keys: S = Q K^T (P role) or dP = dO V^T (dS role); lane holds key
  // kvrow, rows it*64 + 32qs + 8(v/4) + 4half + v%4. The two row blocks'
  // chains are interleaved (each operand read then has a product of the other
  // chain to hide behind). Both blocks run for every tile: a block entirely
  // before the wave's keys is masked whole (P = 0 by a select, dS = 0 times a
  // finite dP), and skipping it would cost a clear and a copy of x per step.
  auto rows_by_keys = [&](f32x16 (&x)[2]) TAM_INLINE {
    x[0] = f32x16{};
    x[1] = f32x16{};
    if (!vrole) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
        x[qs] = mfma32(*reinterpret_cast<const Op*>(smem + rr[ks] + qs * 32 * T::ROW_BYTES), kvf[ks], x[qs]);
    if (!vrole) __builtin_amdgcn_s_setprio(0);
  };

  // acc^T += A^T G for the rows of the tile at tt (read transposed) and the
  // gradient-side operand G given as hi + lo bf16 pairs: dV^T += dO^T P (P
  // role) or dK^T += Q^T dS (dS role). It runs for both row blocks of every
  // tile (a skipped block contributes exact zeros), and each role has one
  // copy of it per loop body: every accumulator value then feeds exactly one
  // matrix instruction, so the compiler accumulates in place instead of
  // keeping a second copy of dV^T/dK^T.
  // (fp16 kernels: one product on G alone; the lo array is unused.)
  // The dS wave runs both its product chains (dP in rows_by_keys, dK here)
  // at raised wave priority, so that once started they issue back to back
  // while the P wave fills the gaps with its exponentials (3% off the kernel;
  // raising the P wave's as well made it 5% slower).
  auto accumulate = [&](const Op (&hi)[2][2], const Op (&lo)[2][2]) TAM_INLINE {
    if (!vrole) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int ro = (qs * 32 + k2 * 16) * T::ROW_BYTES;
          const Op at = __builtin_bit_cast(Op, lds_read_tr_pair(reinterpret_cast<const uint16_t*>(smem + ro + tt[db][0]),
                                                                reinterpret_cast<const uint16_t*>(smem + ro + tt[db][1])));
          acc[db] = mfma32(at, hi[qs][k2], acc[db]);
          if constexpr (!F16) acc[db] = mfma32(at, lo[qs][k2], acc[db]);
        }
    if (!vrole) __builtin_amdgcn_s_setprio(0);
  };

  // P role, one step: P = exp2(S c - lse2) with the tile's mask, to the
  // partner (with dropout: the sign carries the keep bit) and as hi + lo
  // pairs for dV (with dropout: the kept probabilities scaled by r).
  // (fp16 kernels: with the step's scales, P W / s_dO as one fp16 operand;
  // the partner gets the same scaled values.)
  auto probabilities = [&](auto masked_tag, int st, int it, uint32_t bhq, bool masked, const f32x16 (&x)[2],
                           const StepExp& ex, Op (&hi)[2][2], Op (&lo)[2][2]) TAM_INLINE {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const float* Fs = reinterpret_cast<const float*>(smem + f_at(st));
    float* pb = pb_at(st);
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      // c' = c / (s_Q s_K) and log2(W / s_dO) of this 32-row block
      const float cq = F16 ? __builtin_ldexpf(c, ex.q[qs] + e_kv - 28) : c;
      const float lsh = F16 ? (float)(15 - E_dO + ex.d[qs]) : 0.f;
      float p[16];
      float ps[16];  // fp16 kernels with dropout: the partner's copy, sign = drop bit
      // Dropout bytes: the four lanes of a quad hold keys 4m .. 4m + 3 and need
      // the same four generator calls (row groups i = 0..3); lane 4m + j makes
      // call j, turns its words so that word n holds key n's bytes of rows
      // 0..3, and the quad swaps: dq4[i] then has byte r = row 8i + 4half + r
      // of this lane's key.
      u32x4 dq4 = {0u, 0u, 0u, 0u};
      if (DROP)
        dq4 = quad_transpose(byte_transpose(philox4x32_10(
            (uint32_t)kvrow >> 2, (uint32_t)(it * kKBR + qs * 32 + 8 * (lane & 3) + 4 * half) >> 2, bhq, 0u,
            a.drop.seed_lo, a.drop.seed_hi)));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 l2 = *reinterpret_cast<const f32x4*>(Fs + qs * 32 + 8 * i + 4 * half);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int v = 4 * i + r;
          float e = fast_exp2(fmaf(x[qs][v], cq, F16 ? lsh - l2[r] : -l2[r]));
          if (MASKED) {
            const int qrow = it * kKBR + qs * 32 + 8 * i + 4 * half + r;
            // bitwise &: every term is evaluated, so the select stays branch-free
            const bool ok = (qrow < Sq) & (kvrow < Sk) & (!CAUSAL | (kvrow <= qrow + dlt));
            e = ok ? e : 0.f;
          }
          if (DROP) {
            const bool keep = drop_keep(dq4[i], r, a.drop.t);
            if constexpr (F16) {
              // r is applied to dV at the end, so the operand stays below 2^15
              ps[v] = keep ? e : -e;
              p[v] = keep ? e : 0.f;
            } else {
              pb[(16 * qs + v) * 64] = keep ? e : -e;
              p[v] = keep ? e * a.drop.r : 0.f;
            }
          } else {
            p[v] = e;
            if constexpr (!F16) pb[(16 * qs + v) * 64] = e;
          }
        }
      }
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        if constexpr (F16) {
          // the partner takes the same fp16 pairs (with dropout, P with the
          // drop bit as sign): dword w of (qs, k2) holds elements 8 k2 + 2w
          // and 8 k2 + 2w + 1
          hi[qs][k2] = pack_f16x8(p + 8 * k2);
          const u32x4 w4 = __builtin_bit_cast(u32x4, DROP ? pack_f16x8(ps + 8 * k2) : hi[qs][k2]);
          uint32_t* pw = reinterpret_cast<uint32_t*>(pb);
#pragma unroll
          for (int w = 0; w < 4; ++w) pw[(8 * qs + 4 * k2 + w) * 64] = w4[w];
        } else {
          split_bf16x8(p + 8 * k2, &hi[qs][k2], &lo[qs][k2]);
        }
      }
    }
  };

  // dS role, second half of step st: dS = P (dP - Delta) from the partner's P
  // and the dP held in x since the step before, as hi + lo pairs. (fp16
  // kernels: P arrives as P W / s_dO and x holds s_dO s_V dP, so
  // P W/s_dO (x k - Delta m) with k = U / (W s_V s_Q) and m = s_dO s_V k is
  // dS U / s_Q, one fp16 operand.)
  auto grad_scores = [&](int st, const f32x16 (&x)[2], const StepExp& ex, Op (&hi)[2][2],
                         Op (&lo)[2][2]) TAM_INLINE {
    const float* Fs = reinterpret_cast<const float*>(smem + f_at(st));
    const float* pb = pb_at(st);
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const float kap = F16 ? __builtin_ldexpf(1.f, -29 - E_U + E_dO + e_kv + ex.q[qs]) : 1.f;
      const float mu = F16 ? __builtin_ldexpf(1.f, -1 - ex.d[qs] - E_U + E_dO + ex.q[qs]) : 1.f;
      const float kr = kap * a.drop.r;  // dropout: kept elements' dP factor
      float ds[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 dl4 = *reinterpret_cast<const f32x4*>(Fs + kKBR + qs * 32 + 8 * i + 4 * half);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int v = 4 * i + r;
          if constexpr (F16) {
            // P as the partner's fp16 pair; the widening folds into the multiply
            const uint32_t w = reinterpret_cast<const uint32_t*>(pb)[(8 * qs + 4 * (v >> 3) + ((v & 7) >> 1)) * 64];
            const float pv = (float)__builtin_bit_cast(f16x2, w)[v & 1];
            if constexpr (DROP)
              ds[v] = fmaf(fabsf(pv), fmaf(x[qs][v], __builtin_signbit(pv) ? 0.f : kr, -dl4[r] * mu), 0.f);
            else
              ds[v] = fmaf(pv, fmaf(x[qs][v], kap, -dl4[r] * mu), 0.f);
          } else {
            const float pv = pb[(16 * qs + v) * 64];
            ds[v] = DROP ? fabsf(pv) * ((__builtin_signbit(pv) ? 0.f : a.drop.r) * x[qs][v] - dl4[r])
                         : pv * (x[qs][v] - dl4[r]);
          }
        }
      }
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        if constexpr (F16)
          hi[qs][k2] = pack_f16x8(ds + 8 * k2);
        else
          split_bf16x8(ds + 8 * k2, &hi[qs][k2], &lo[qs][k2]);
      }
    }
  };

  // Software pipeline with one barrier per phase. In phase t the P wave of
  // each pair runs step t whole (S, P, dV) while its dS partner finishes step
  // t - 1 (whose P was handed over in phase t - 1: dS, dK) and then computes
  // dP of step t. The two waves of a pair share a SIMD, so the exponentials of
  // one overlap the matrix products of the other. Step t + 1's tiles load
  // meanwhile: its Q stage last served step t - 2, its dO stage step t - 1.
  // Both roles pass nsteps + 1 barriers after the first load.
  if (nsteps > 0) {
    Cursor cur = {h_first, NQ - 1};   // step t
    issue(0, cur);
    wait_loads();
    __syncthreads();
    Cursor nxt = cur;                 // step t + 1
    advance(nxt);
    if (vrole) {
      for (int st = 0; st < nsteps; ++st) {
        const int it = cur.it;
        const bool masked = masked_at(it);
        const uint32_t bhq = (uint32_t)(b * a.Hq + cur.h);
        StepExp ex{};
        if constexpr (F16) ex = step_exp();  // loaded with this step's tiles, before the barrier
        f32x16 x[2];
        rows_by_keys(x);
        if (st + 1 < nsteps) issue(st + 1, nxt);  // after the score products: the issue stalls overlap them
        Op hi[2][2], lo[2][2];
        if (masked)
          probabilities(std::true_type{}, st, it, bhq, masked, x, ex, hi, lo);
        else
          probabilities(std::false_type{}, st, it, bhq, masked, x, ex, hi, lo);
        accumulate(hi, lo);
        move_rr(q_next(st));
        move_tt(do_next(st));
        advance(cur);
        advance(nxt);
        wait_loads();
        __syncthreads();
      }
      __syncthreads();  // the partner's last phase
    } else {
      f32x16 x[2];  // dP of the step before, carried over the barrier
      StepExp ex_prev{};  // that step's exponents (fp16 kernels)
      if constexpr (F16) ex_prev = step_exp();
      if (nsteps > 1) issue(1, nxt);
      rows_by_keys(x);
      move_rr(do_next(0));
      advance(cur);
      advance(nxt);
      wait_loads();
      __syncthreads();
      for (int st = 1; st < nsteps; ++st) {
        StepExp ex_cur{};
        if constexpr (F16) ex_cur = step_exp();
        if (st + 1 < nsteps) issue(st + 1, nxt);
        Op hi[2][2], lo[2][2];
        grad_scores(st - 1, x, ex_prev, hi, lo);
        accumulate(hi, lo);
        move_tt(q_next(st - 1));
        rows_by_keys(x);
        move_rr(do_next(st));
        advance(cur);
        advance(nxt);
        ex_prev = ex_cur;
        wait_loads();
        __syncthreads();
      }
      Op hi[2][2], lo[2][2];
      grad_scores(nsteps - 1, x, ex_prev, hi, lo);
      accumulate(hi, lo);
      __syncthreads();
    }
  }

  // lane holds key kvrow, head-dim entries 32db + 8i + 4half + (0..3)
  if (kvrow < Sk) {
    // fp16 kernels: dV = acc / W, dK = scale acc / U
    const float mul = F16 ? (vrole ? (DROP ? a.drop.r : 1.f) * __builtin_ldexpf(1.f, E_dO - 29)
                                   : a.scale * __builtin_ldexpf(1.f, E_U - 28))
                          : (vrole ? 1.f : a.scale);
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] *= mul;
    if (!vrole && a.rope_inv) {
      // dK of the rotated keys back to the unrotated ones: element v of
      // block db is column 32db + 8(v/4) + 4half + v%4, its partner d + D/2
      // sits in block db + DB/2 of this lane
      const float2* cs = a.rope_inv + (size_t)kvrow * (D / 2);
#pragma unroll
      for (int db = 0; db < DB / 2; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float lo, hi;
          rope_pair(acc[db][v], acc[db + DB / 2][v], cs[32 * db + 8 * (v >> 2) + 4 * half + (v & 3)], true, &lo, &hi);
          acc[db][v] = lo;
          acc[db + DB / 2][v] = hi;
        }
    }
    if (a.nsplit == 1) {
      uint16_t* op = (vrole ? a.dv : a.dk) + kv_base + (size_t)kvrow * D + 8 * half;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const f32x16& A = acc[db];
          u32x2 w[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int i = 2 * m + t;
            w[t] = u32x2{pack_bf16(A[4 * i], A[4 * i + 1]), pack_bf16(A[4 * i + 2], A[4 * i + 3])};
          }
          *reinterpret_cast<u32x4*>(op + 32 * db + 16 * m) = pair_halves(w[0], w[1]);
        }
    } else {
      const size_t total = (size_t)(a.sched.BH / a.nsplit) * Sk * D;  // B*Hkv*Sk*D
      float* op = a.part + ((size_t)sub * 2 + (vrole ? 1 : 0)) * total + kv_base + (size_t)kvrow * D + 4 * half;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x16& A = acc[db];
          *reinterpret_cast<f32x4*>(op + 32 * db + 8 * i) = f32x4{A[4 * i], A[4 * i + 1], A[4 * i + 2], A[4 * i + 3]};
        }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. fixed-order sum of the per-subset partials -> bf16 dK, dV
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void attn_bwd_reduce_kernel(const float* part, uint16_t* dk,
                                                                   uint16_t* dv, long long n4,
                                                                   int nsplit) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;  // index of a 4-element group
  if (i >= n4) return;
  const size_t total = (size_t)n4 * 4;
  f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    sk += *reinterpret_cast<const f32x4*>(part + (size_t)s * 2 * total + (size_t)i * 4);
    sv += *reinterpret_cast<const f32x4*>(part + ((size_t)s * 2 + 1) * total + (size_t)i * 4);
  }
  *reinterpret_cast<u32x2*>(dk + (size_t)i * 4) = u32x2{pack_bf16(sk[0], sk[1]), pack_bf16(sk[2], sk[3])};
  *reinterpret_cast<u32x2*>(dv + (size_t)i * 4) = u32x2{pack_bf16(sv[0], sv[1]), pack_bf16(sv[2], sv[3])};
}

// ---------------------------------------------------------------------------
// 4. dQ, query-stationary
// ---------------------------------------------------------------------------
struct DqArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  float* delta;  // in: Delta~ from the stored O (unless o is set); out: exact Delta (final mode)
  float* lse2;   // in: LSE * log2(e) (unless o is set); out: the same, when o is set
  // Whole-sequence calls set o and lse: the kernel then forms Delta~ = sum_d dO O
  // and lse2 itself instead of reading them from the workspace.
  const uint16_t* o;
  const float* lse;
  uint16_t* dq;  // final mode: dQ = scale (sum dS~ K - c P K)
  // Accumulate mode (all three set, dq unused): this call's key block adds its
  // sum dS~ K, P K and c = sum dS~ to these fp32 buffers ([rows, D], [rows, D],
  // [rows]); the sum over all key blocks is finished later.
  float* acc_dq;
  float* acc_pk;
  float* acc_c;
  // When set (whole-sequence calls without dropout): fp16 copies of Q and dO
  // for the dK/dV kernel, each 32-row block scaled by 2^(14 - e), and the
  // block exponents e of Q, dO and the exact Delta, [B*Hq][ceil(Sq/32)] each.
  uint16_t* q16;
  uint16_t* do16;
  int* eq;
  int* edo;
  int* edl;
  // fp16 kernels: k is the fp16 copy of K, and these its tile exponents and
  // those of V ([B*Hkv][ceil(Sk/64)])
  const int* ek;
  const int* ev;
  int Hq, Hkv, Sq, Sk, dlt;
  float c;
  float scale;
  DropParams drop;  // dropout on the probabilities (DROP kernels only)
  const float2* rope_inv;  // (cos, sin) table [Sq][D/2]: rotate dQ back (final mode); null = none
  int pack;  // log2 of the query heads a unit holds (Sq <= kQBR >> pack)
  TileSched sched;
};

// LDS layout of the dQ kernel. The two waves of a pair work one key tile
// apart (see the kernel), so K is kept in three stages (tile t in stage t % 3),
// V in two (t % 2), and the probabilities one wave of each pair hands to the
// other in two.
template <int D>
struct DqLayout {
  using T = SwzTile<D>;
  static constexpr int K0 = 0, V0 = 3 * T::BYTES;
  static constexpr int PB = 5 * T::BYTES;
  static constexpr int PB_BLOCK = 32 * kQBC * 4;  // 32 rows x 64 keys fp32
  static constexpr int PB_STAGE = 4 * PB_BLOCK;
  static constexpr int EK = PB + 2 * PB_STAGE;    // fp16 kernels: K tile exponent per K stage (one wave load each)
  static constexpr int BYTES = EK + 3 * 256;
  static_assert(4 * (D / 32) * 16 * 64 * 4 <= PB, "final hand-off fits in the stages");
};

// F16: the products with K (S, P K and dQ) run on fp16 operands, one product
// each: K comes as the fp16 copy (tile t scaled by s_K(t) = 2^(14 - ek(t))),
// the P role turns its Q rows into fp16 with their block scale s_Q, so
// S' = s_K s_Q S and c' = c / (s_K s_Q) per tile; P goes to the P K product and
// to the partner as P W / s_K(t), W = 2^(29 - E_K) with E_K = max ek over the
// unit's tiles; the dS role forms dS U / s_K(t) from it with one unit-wide
// factor, U the largest power of two keeping every dS at or below 2^15 by
// |dS~| <= |dP| + |Delta~| <= 2 D 2^(eD + E_V) (E_V = max ev, since O is a
// mean of V rows; with dropout both terms grow by r <= 2^eR, so E_V takes eR
// on). dP = V dO^T stays in bf16. dQ = scale (acc / U - c PK / W).
template <int D, bool CAUSAL, bool DROP = false, bool F16 = false>
__global__ __attribute__((amdgpu_flat_work_group_size(kBwdThreads, kBwdThreads), amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_kernel(DqArgs a) {
  using T = SwzTile<D>;
  using L = DqLayout<D>;
  using KOp = std::conditional_t<F16, f16x8, bf16x8>;  // operand type of the products with K
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int kLog2D = D == 128 ? 7 : 6;
  constexpr int NLD = T::LOADS / 2;   // K and V loads per P-role wave per tile
  static_assert(kQBC == T::ROWS && kQBR == 128, "tile sizes");
  static_assert(L::BYTES <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[L::BYTES];

  int bh, qt;
  if (!sched_decode(a.sched, blockIdx.x, &bh, &qt)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave
  const int rblk = wave & 3;         // this pair's 32 query rows within the unit
  const bool prole = wave < 4;       // S, P and P K (with Q resident); else dP, dS and dQ (with dO resident)
  const int col = lane & 31, half = lane >> 5;
  const int Sq = a.Sq, Sk = a.Sk, dlt = a.dlt;
  // unit = (batch, 2^pack query heads of one group, 128-row tile); each head
  // takes kQBR >> pack rows of it, so a pair's 32 rows belong to one head
  const int rows_per_head = kQBR >> a.pack;
  bh = (bh << a.pack) + rblk * 32 / rows_per_head;  // this pair's (batch, query head)
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  const int kvh = h / (a.Hq / a.Hkv);
  const size_t q_base = (size_t)bh * Sq * D;
  const uint16_t* kg = a.k + ((size_t)b * a.Hkv + kvh) * (size_t)Sk * D;
  const uint16_t* vg = a.v + ((size_t)b * a.Hkv + kvh) * (size_t)Sk * D;
  const int q0 = qt * kQBR;
  const int wrow0 = q0 + rblk * 32 % rows_per_head;
  const int qrow = wrow0 + col;
  const uint32_t lds0 = lds_address(smem);

  // Q (for S) or dO (for dP) rows of this pair's queries as MFMA B operands.
  bf16x8 xf[KS];
  {
    const uint16_t* src = (prole ? a.q : a.dout) + q_base + (size_t)qrow * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      xf[ks] = qrow < Sq ? *reinterpret_cast<const bf16x8*>(src + 16 * ks)
                        : __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  }
  // lse2 (P role) or Delta~ (dS role) of this lane's row
  float rowval = 0.f;
  if (qrow < Sq) {
    const size_t r = (size_t)bh * Sq + qrow;
    if (!a.o) {
      rowval = (prole ? a.lse2 : a.delta)[r];
    } else if (prole) {
      // a row that sees no key has LSE = -inf; +inf makes all its probabilities 0
      const float l = a.lse[r];
      rowval = l == -INFINITY ? INFINITY : l * kLog2e;
      if (half == 0) a.lse2[r] = rowval;   // for the dK/dV kernel
    } else {
      // this lane's half of Delta~ = sum_d dO_d O_d: head-dim entries 16 ks + 8 half + (0..7)
      const uint16_t* op = a.o + q_base + (size_t)qrow * D + 8 * half;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 ov = *reinterpret_cast<const u32x4*>(op + 16 * ks);
        const u32x4 dv = __builtin_bit_cast(u32x4, xf[ks]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          rowval = fmaf(bf16_lo(ov[w]), bf16_lo(dv[w]), rowval);
          rowval = fmaf(bf16_hi(ov[w]), bf16_hi(dv[w]), rowval);
        }
      }
    }
  }
  if (a.o && !prole) rowval = sum_halves(rowval);  // every lane takes part in the exchange

  // fp16 copy of this pair's 32 rows of Q (P role) or dO (dS role) with the
  // rows' block exponent, for the dK/dV kernel. (Stored here, before the
  // tiles: stores count among the loads every barrier waits for, and spread
  // over the tile loop they cost registers.)
  // (fp16 kernels: the P role keeps these fp16 values of Q as its operands,
  // and both roles use the block exponent e_blk.)
  const int nblk = (Sq + 31) / 32;
  const size_t eidx = (size_t)bh * nblk + (wrow0 >> 5);
  int e_blk = 0;
  if (F16 || a.q16) {
    uint32_t m = 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t mk = bf16x8_max_mag(xf[ks]);
      m = m > mk ? m : mk;
    }
    e_blk = __builtin_amdgcn_readfirstlane(ceil_log2(__builtin_bit_cast(float, wave_max(m) << 16)));
    const float sc = __builtin_ldexpf(1.f, 14 - e_blk);
    f16x8 h[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) h[ks] = bf16x8_to_f16x8(xf[ks], sc);
    if (a.q16 && qrow < Sq) {
      uint16_t* dst = (prole ? a.q16 : a.do16) + q_base + (size_t)qrow * D + 8 * half;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) *reinterpret_cast<f16x8*>(dst + 16 * ks) = h[ks];
    }
    if (a.q16 && lane == 0 && wrow0 < Sq) (prole ? a.eq : a.edo)[eidx] = e_blk;
    if (F16 && prole) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) xf[ks] = __builtin_bit_cast(bf16x8, h[ks]);
    }
  }


  // Per-lane LDS offsets (see SwzTile) into the stage this wave reads next:
  // roff for the key-by-row products (K for the P role, V for the dS role),
  // toff for the transposed K reads. They move to the next stage in place, by
  // a uniform step, so that a runtime stage costs no registers.
  const int i16 = lane & 15;
  const int dsub = 16 * ((lane >> 4) & 1);
  int roff[KS], toff[DB][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) roff[ks] = (prole ? L::K0 : L::V0) + T::chunk_off(col, 2 * ks + half);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
      toff[db][hi] = L::K0 + T::elem_off(4 * half + (i16 >> 2) + 8 * hi, db * 32 + dsub + 4 * (i16 & 3));
  // stage step after tile j: K stages cycle through three, V stages through two
  auto k_next = [&](int j) TAM_INLINE { return j % 3 == 2 ? -2 * T::BYTES : T::BYTES; };
  auto v_next = [&](int j) TAM_INLINE { return (j & 1) ? -T::BYTES : T::BYTES; };
  auto move_roff = [&](int by) TAM_INLINE {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) roff[ks] += by;
  };
  auto move_toff = [&](int by) TAM_INLINE {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) toff[db][hi] += by;
  };
  // this lane's slots of the P hand-off block of stage 0: key v of 32-key
  // block kb at (16 kb + v) * 64 + lane
  float* const pbuf = reinterpret_cast<float*>(smem + L::PB + rblk * L::PB_BLOCK) + lane;
  auto pb_at = [&](int j) TAM_INLINE { return pbuf + (j & 1) * (L::PB_STAGE / 4); };

  const int last_row = min(q0 + rows_per_head, Sq) - 1;  // the unit's last row (of any of its heads)
  const int n_kv = (Sk + kQBC - 1) / kQBC;
  // the last key any row of the unit may see is last_row + dlt
  const int ntiles = CAUSAL ? (last_row + dlt < 0 ? 0 : min(n_kv, (last_row + dlt) / kQBC + 1)) : n_kv;

  // fp16 kernels: E_K and E_V over the unit's key tiles; the exponent of each
  // tile travels with it into LDS (beside its K stage), so that it waits with
  // the tile's own loads and holds no register across the loop
  const size_t tbase = ((size_t)b * a.Hkv + kvh) * n_kv;
  int E_K = kMinExp, E_V = kMinExp;
  if constexpr (F16) {
    for (int t = lane; t < ntiles; t += 64) {
      E_K = max(E_K, a.ek[tbase + t]);
      E_V = max(E_V, a.ev[tbase + t]);
    }
    E_K = __builtin_amdgcn_readfirstlane(wave_max(E_K));
    E_V = __builtin_amdgcn_readfirstlane(wave_max(E_V));
    // dropout scales the kept dP by r <= 2^eR: the dS scale takes it as part of E_V
    if (DROP) E_V += ceil_log2(a.drop.r);
  }
  auto tile_exp = [&](int j) TAM_INLINE {
    return __builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(smem + L::EK + (j % 3) * 256));
  };

  // K and V tiles of key tile j straight into their stages; rows past Sk read as
  // zeros. Only the four P-role waves call it, each issuing an eighth of the
  // loads, so a dS-role wave has no tile loads in flight and a wait on its own
  // loads never waits for the next tile (and the offsets take no dS-role
  // registers).
  auto issue = [&](int j) TAM_INLINE {
    if (F16 && wave == 0) dma4(make_rsrc(a.ek + tbase + j, 4), lds0 + L::EK + (j % 3) * 256, lane * 4);
    const int row0 = j * kQBC;
    const int bytes = (Sk - row0) * D * 2;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + (size_t)row0 * D, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + (size_t)row0 * D, bytes);
    const uint32_t kb = lds0 + L::K0 + (j % 3) * T::BYTES, vb = lds0 + L::V0 + (j & 1) * T::BYTES;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int gi = wave * NLD + i, which = gi / T::LOADS, li = gi % T::LOADS;
      dma16(which == 0 ? rk : rv, (which == 0 ? kb : vb) + li * 1024, T::load_src(li, lane));
    }
  };

  f32x16 acc[DB];  // (P K)^T (P role) or dQ^T with Delta~ (dS role)
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float csum = 0.f;  // dS role: this lane's half of c = sum_j dS~_j for its row
  const float c = a.c;

  // Key tiles of 64 keys, as two 32-key blocks, against this pair's 32 rows.
  // A tile is active for the pair when some key of it is visible to one of
  // its rows; it is masked when it meets the pair's diagonal or the end of
  // the sequence, and then hidden pairs get P = 0.
  auto active_at = [&](int j) TAM_INLINE { return !CAUSAL || j * kQBC <= wrow0 + 31 + dlt; };
  auto masked_at = [&](int j) TAM_INLINE {
    return (j * kQBC + kQBC > Sk) || (CAUSAL && j * kQBC + kQBC - 1 > wrow0 + dlt);
  };

  // The dS wave's matrix-product chains (dP and dQ) run at raised wave
  // priority, so that once started they issue back to back while the P wave
  // on the same SIMD fills the gaps with its exponentials (about 9% off the
  // kernel at S=4096 against no raised priority; raising both waves' chains
  // gained 2%, the P wave's alone lost 2%).
  // S^T = K Q^T (P role) or dP^T = V dO^T (dS role) from the tile at roff:
  // lane holds keys 32kb + 8(v/4) + 4half + v%4 of row qrow. Computed for
  // every tile: a tile no row of the pair sees is masked whole (P = 0, a
  // select, so any finite product is dropped), and a branch around the
  // products would cost a register clear of x per tile.
  // (fp16 kernels: the P role's products, with K, run in fp16.)
  auto scores = [&](auto prole_tag, f32x16 (&x)[2]) TAM_INLINE {
    using Op = std::conditional_t<F16 && decltype(prole_tag)::value, f16x8, bf16x8>;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) x[kb] = f32x16{};
    if (!decltype(prole_tag)::value) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        x[kb] = mfma32(*reinterpret_cast<const Op*>(smem + roff[ks] + kb * 32 * T::ROW_BYTES),
                       __builtin_bit_cast(Op, xf[ks]), x[kb]);
    if (!decltype(prole_tag)::value) __builtin_amdgcn_s_setprio(0);
  };
  // K^T rows kb*32 + k2*16 .. +15 of the tile at toff as A operands, read transposed
  auto kt_operands = [&](int kb, int k2, KOp (&a_k)[DB]) TAM_INLINE {
    const int ro = (kb * 32 + k2 * 16) * T::ROW_BYTES;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      a_k[db] = __builtin_bit_cast(KOp, lds_read_tr_pair(reinterpret_cast<const uint16_t*>(smem + ro + toff[db][0]),
                                                         reinterpret_cast<const uint16_t*>(smem + ro + toff[db][1])));
  };

  // P role, one tile: P = exp2(S c - lse2) with the tile's mask, handed to the
  // partner (with dropout: the sign carries the keep bit), and as bf16 B
  // operands (before dropout) for P K.
  // (fp16 kernels: with the tile's scales, P W / s_K as fp16 pairs, to the
  // partner as well.)
  auto probabilities = [&](auto masked_tag, int j, bool active, const f32x16 (&x)[2], int ekj,
                           KOp (&ph)[2][2]) TAM_INLINE {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int kv0 = j * kQBC;
    float* pb = pb_at(j);
    // c' = c / (s_K s_Q) and log2(W / s_K) of this tile
    const float cq = F16 ? __builtin_ldexpf(c, ekj + e_blk - 28) : c;
    const float arg0 = F16 ? (float)(15 - E_K + ekj) - rowval : -rowval;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float pf[16];
      float ps[16];  // fp16 kernels with dropout: the partner's copy, sign = drop bit
      // Dropout words: the four lanes of a quad hold rows 4m .. 4m + 3 and need
      // the same four generator calls (key groups of this half); lane 4m + j
      // makes call j and the quad swaps, leaving each lane its row's word of
      // every call (dwords[i] for keys kv0 + 32kb + 8i + 4half + 0..3).
      u32x4 dwords = {0u, 0u, 0u, 0u};
      if (DROP)
        dwords = quad_transpose(philox4x32_10((uint32_t)(kv0 + kb * 32 + 8 * (lane & 3) + 4 * half) >> 2,
                                              (uint32_t)qrow >> 2, (uint32_t)bh, 0u, a.drop.seed_lo,
                                              a.drop.seed_hi));
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float e = fast_exp2(fmaf(x[kb][v], cq, arg0));
        if (MASKED) {
          const int kv = kv0 + kb * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          const bool ok = active & (kv < Sk) & (!CAUSAL | (kv <= qrow + dlt));  // branch-free
          e = ok ? e : 0.f;
        }
        pf[v] = e;
        if (DROP && F16) {
          ps[v] = drop_keep(dwords[v >> 2], v & 3, a.drop.t) ? e : -e;
        } else if (DROP) {
          pb[(16 * kb + v) * 64] = drop_keep(dwords[v >> 2], v & 3, a.drop.t) ? e : -e;
        } else if (!F16) {
          pb[(16 * kb + v) * 64] = e;
        }
      }
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        if constexpr (F16) {
          // dword w of (kb, k2) holds keys 8 k2 + 2w and 8 k2 + 2w + 1 of block kb
          // (with dropout, P with the drop bit as sign)
          ph[kb][k2] = pack_f16x8(pf + 8 * k2);
          const u32x4 w4 = __builtin_bit_cast(u32x4, DROP ? pack_f16x8(ps + 8 * k2) : ph[kb][k2]);
          uint32_t* pw = reinterpret_cast<uint32_t*>(pb);
#pragma unroll
          for (int w = 0; w < 4; ++w) pw[(8 * kb + 4 * k2 + w) * 64] = w4[w];
        } else {
          ph[kb][k2] = pack_bf16x8(pf + 8 * k2);
        }
      }
    }
  };
  // (P K)^T += K^T P^T. It runs for every tile (an inactive one adds exact
  // zeros) and appears once in the loop, so that each accumulator value feeds
  // one matrix instruction and is updated in place.
  auto pk_product = [&](const KOp (&ph)[2][2]) TAM_INLINE {

#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        KOp a_k[DB];
        kt_operands(kb, k2, a_k);
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = mfma32(a_k[db], ph[kb][k2], acc[db]);
      }

  };

  // dS role, second half of tile j: dS~ = P (dP - Delta~) from the partner's
  // P and the dP held since the step before, c += sum dS~, and dQ^T +=
  // K^T dS~^T with hi and lo parts (once per loop body, for every tile).
  // (fp16 kernels: P arrives as P W / s_K, and P W/s_K (dP - Delta~) kap with
  // kap = U / W is dS~ U / s_K, one fp16 operand; c adds it times s_K / U.)
  // (the dS role's rowval then holds Delta~ kap, an exact power-of-two multiple)
  const float kap = F16 ? pow2i(-1 - kLog2D - e_blk - E_V) : 1.f;
  const float kr = kap * a.drop.r;  // dropout: kept elements' dP factor
  if (F16 && !prole) rowval *= kap;
  auto ds_tile = [&](int j, const f32x16 (&x)[2], int ekj) TAM_INLINE {
    const float* pb = pb_at(j);
    const float fj = F16 ? pow2i(-14 - ekj + kLog2D + e_blk + E_V + E_K) : 1.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float ds[16];
      float tsum = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        if constexpr (F16) {
          const uint32_t w = reinterpret_cast<const uint32_t*>(pb)[(8 * kb + 4 * (v >> 3) + ((v & 7) >> 1)) * 64];
          const float pv = (float)__builtin_bit_cast(f16x2, w)[v & 1];
          if constexpr (DROP)
            ds[v] = fmaf(fabsf(pv), fmaf(x[kb][v], __builtin_signbit(pv) ? 0.f : kr, -rowval), 0.f);
          else
            ds[v] = fmaf(pv, fmaf(x[kb][v], kap, -rowval), 0.f);
        } else {
          const float pv = pb[(16 * kb + v) * 64];
          ds[v] = DROP ? fabsf(pv) * ((__builtin_signbit(pv) ? 0.f : a.drop.r) * x[kb][v] - rowval)
                       : pv * (x[kb][v] - rowval);
        }
        if constexpr (F16)
          tsum += ds[v];
        else
          csum += ds[v];
      }
      if constexpr (F16) csum = fmaf(tsum, fj, csum);
      KOp dh[2], dl[2];
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        if constexpr (F16)
          dh[k2] = pack_f16x8(ds + 8 * k2);
        else
          split_bf16x8(ds + 8 * k2, &dh[k2], &dl[k2]);
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        KOp a_k[DB];
        kt_operands(kb, k2, a_k);
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = mfma32(a_k[db], dh[k2], acc[db]);
        if constexpr (!F16) {
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[db] = mfma32(a_k[db], dl[k2], acc[db]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }
  };

  // Software pipeline with one barrier per phase. In phase t the P wave of
  // each pair runs tile t whole (S, P, P K) while its dS partner finishes tile
  // t - 1 (whose P was handed over in phase t - 1: dS, dQ) and then computes
  // dP of tile t. The two waves of a pair share a SIMD, so the exponentials of
  // one overlap the matrix products of the other. The P waves load tile t + 1
  // meanwhile: its K stage last served tile t - 2, its V stage tile t - 1.
  // Both roles pass ntiles + 2 barriers.
  if (ntiles > 0) {
    if (prole) issue(0);
    wait_loads();
    __syncthreads();
    if (prole) {
      for (int j = 0; j < ntiles; ++j) {
        const int ekj = F16 ? tile_exp(j) : 0;  // loaded with tile j, before the barrier
        const bool active = active_at(j);
        f32x16 x[2];
        scores(std::true_type{}, x);
        if (j + 1 < ntiles) issue(j + 1);  // after the score products: the issue stalls overlap them
        KOp ph[2][2];
        if (masked_at(j))
          probabilities(std::true_type{}, j, active, x, ekj, ph);
        else
          probabilities(std::false_type{}, j, active, x, ekj, ph);
        pk_product(ph);
        move_roff(k_next(j));
        move_toff(k_next(j));
        wait_loads();
        __syncthreads();
      }
      __syncthreads();  // the partner's last phase
    } else {
      f32x16 x[2];  // dP of the tile before, carried over the barrier
      int ek_prev = F16 ? tile_exp(0) : 0;  // that tile's exponent (fp16 kernels)
      scores(std::false_type{}, x);
      move_roff(v_next(0));
      wait_loads();
      __syncthreads();
      for (int j = 1; j < ntiles; ++j) {
        const int ek_cur = F16 ? tile_exp(j) : 0;
        ds_tile(j - 1, x, ek_prev);
        move_toff(k_next(j - 1));
        scores(std::false_type{}, x);
        move_roff(v_next(j));
        ek_prev = ek_cur;
        wait_loads();
        __syncthreads();
      }
      ds_tile(ntiles - 1, x, ek_prev);
      __syncthreads();
    }
  }

  if (a.acc_dq) {
    // accumulate mode: each role adds its own sums for this key block (fp16
    // kernels: back in absolute units first, P K = acc / W, sum dS~ K = acc / U;
    // c is summed in absolute units already)
    if (qrow < Sq && ntiles > 0) {
      float* dst = (prole ? a.acc_pk : a.acc_dq) + q_base + (size_t)qrow * D + 4 * half;
      const float mul = !F16 ? 1.f
                        : prole ? __builtin_ldexpf(1.f, E_K - 29)
                                : __builtin_ldexpf(1.f, -28 + kLog2D + e_blk + E_V + E_K);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4* p4 = reinterpret_cast<f32x4*>(dst + 32 * db + 8 * i);
          *p4 += mul * f32x4{acc[db][4 * i], acc[db][4 * i + 1], acc[db][4 * i + 2], acc[db][4 * i + 3]};
        }
      if (!prole) {
        const float cs = sum_halves(csum);
        if (half == 0) a.acc_c[(size_t)bh * Sq + qrow] += cs;
      }
    }
    return;
  }
  // P K goes to the dS role through the (now idle) stages: element v of
  // accumulator db of lane l at float (16 db + v) * 64 + l of the pair's block.
  float* hand = reinterpret_cast<float*>(smem) + rblk * (DB * 16 * 64) + lane;
  if (prole) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) hand[(16 * db + v) * 64] = acc[db][v];
  }
  __syncthreads();
  if (prole) return;
  if (F16) rowval *= pow2i(1 + kLog2D + e_blk + E_V);  // Delta~ again
  const float corr = sum_halves(csum);  // Delta_i - Delta~_i
  if (a.edl) {
    const float dm = wave_max(qrow < Sq ? fabsf(rowval + corr) : 0.f);
    if (lane == 0 && wrow0 < Sq) a.edl[eidx] = ceil_log2(dm);
  }
  if (qrow < Sq) {
    // dQ = scale (sum dS~ K - c P K); element v of block db is column
    // 32db + 8(v/4) + 4half + v%4
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        if constexpr (F16) {
          // scale (acc / U - c P K / W)
          const float s1 = a.scale * __builtin_ldexpf(1.f, -28 + kLog2D + e_blk + E_V + E_K);
          const float s2 = a.scale * corr * __builtin_ldexpf(1.f, E_K - 29);
          acc[db][v] = fmaf(-s2, hand[(16 * db + v) * 64], s1 * acc[db][v]);
        } else {
          acc[db][v] = a.scale * fmaf(-corr, hand[(16 * db + v) * 64], acc[db][v]);
        }
      }
    if (a.rope_inv) {
      // back to the unrotated queries: the partner d + D/2 of column d sits in
      // block db + DB/2 of this lane
      const float2* cs = a.rope_inv + (size_t)qrow * (D / 2);
#pragma unroll
      for (int db = 0; db < DB / 2; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float lo, hi;
          rope_pair(acc[db][v], acc[db + DB / 2][v], cs[32 * db + 8 * (v >> 2) + 4 * half + (v & 3)], true, &lo, &hi);
          acc[db][v] = lo;
          acc[db + DB / 2][v] = hi;
        }
    }
    uint16_t* op = a.dq + q_base + (size_t)qrow * D + 8 * half;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        u32x2 w[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int i = 2 * m + t;
          w[t] = u32x2{pack_bf16(acc[db][4 * i], acc[db][4 * i + 1]), pack_bf16(acc[db][4 * i + 2], acc[db][4 * i + 3])};
        }
        *reinterpret_cast<u32x4*>(op + 32 * db + 16 * m) = pair_halves(w[0], w[1]);
      }
    if (half == 0) a.delta[(size_t)bh * Sq + qrow] = rowval + corr;
  }
}

// ---------------------------------------------------------------------------
// 5. small kernels of the block protocol
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void attn_fill_zero_kernel(f32x4* p, long long n4) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i < n4) p[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// dQ = scale (sum dS~ K - c P K) in bf16, and the exact Delta = Delta~ + c.
template <int D>
__global__ __launch_bounds__(kThreads) void attn_bwd_dq_end_kernel(const float* acc_dq, const float* acc_pk,
                                                                   const float* csum, float* delta,
                                                                   uint16_t* dq, float scale, long long rows) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements each
  constexpr int RPB = kThreads / TPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  if (row >= rows) return;
  const float c = csum[row];
  const f32x4* a = reinterpret_cast<const f32x4*>(acc_dq + row * D + part * 8);
  const f32x4* p = reinterpret_cast<const f32x4*>(acc_pk + row * D + part * 8);
  u32x4 w;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const f32x4 x = a[h], y = p[h];
    w[2 * h] = pack_bf16(scale * fmaf(-c, y[0], x[0]), scale * fmaf(-c, y[1], x[1]));
    w[2 * h + 1] = pack_bf16(scale * fmaf(-c, y[2], x[2]), scale * fmaf(-c, y[3], x[3]));
  }
  *reinterpret_cast<u32x4*>(dq + row * D + part * 8) = w;
  if (part == 0) delta[row] += c;
}

// ---------------------------------------------------------------------------
// host side: one launcher per stage, shared by the whole-sequence pass and
// the block protocol
// ---------------------------------------------------------------------------
struct Ws {
  float *delta, *lse2, *csum, *acc_dq, *acc_pk, *part;
  uint16_t *q16, *do16, *k16;
  int *eq, *edo, *edl, *ek, *ev;
  WsLayout w;
  bool block;
  Ws(const AttnShape& sh, void* base, bool block_) : w(ws_layout(sh, block_)), block(block_) {
    char* b = static_cast<char*>(base);
    delta = reinterpret_cast<float*>(b + w.delta);
    lse2 = reinterpret_cast<float*>(b + w.lse2);
    csum = block ? reinterpret_cast<float*>(b + w.csum) : nullptr;
    acc_dq = block ? reinterpret_cast<float*>(b + w.acc_dq) : nullptr;
    acc_pk = block ? reinterpret_cast<float*>(b + w.acc_pk) : nullptr;
    q16 = reinterpret_cast<uint16_t*>(b + w.q16);
    do16 = reinterpret_cast<uint16_t*>(b + w.do16);
    eq = reinterpret_cast<int*>(b + w.eq);
    edo = reinterpret_cast<int*>(b + w.edo);
    edl = reinterpret_cast<int*>(b + w.edl);
    k16 = reinterpret_cast<uint16_t*>(b + w.k16);
    ek = reinterpret_cast<int*>(b + w.ek);
    ev = reinterpret_cast<int*>(b + w.ev);
    part = reinterpret_cast<float*>(b + w.part);
  }
  // The fp16 kernels run on calls over at least kF16MinKeys keys (in the
  // block protocol from kF16MinBlockKeys keys): below
  // that their saving (which grows with the keys each row sees) does not repay
  // the fp16 copies of Q and dO (which grow with the rows alone).
  bool f16(const AttnShape& sh) const { return sh.Sk >= (block ? kF16MinBlockKeys : kF16MinKeys); }
};

template <int D>
hipError_t launch_prep(const AttnShape& sh, const uint16_t* o, const uint16_t* dout, const float* lse,
                       const Ws& ws, hipStream_t stream) {
  const long long rows = (long long)sh.B * sh.Hq * sh.Sq;
  constexpr int RPB = kThreads / (D / 8);
  const long long grid = (rows + RPB - 1) / RPB;
  float* delta = ws.delta;
  float* lse2 = ws.lse2;
  void* args[] = {(void*)&o, (void*)&dout, (void*)&lse, (void*)&delta, (void*)&lse2, (void*)&rows};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_prep_kernel<D>), dim3((unsigned)grid),
                         dim3(kThreads), args, 0, stream);
}

// Zero n floats (n a multiple of 4) with a kernel, so the protocol stays
// capturable in a graph.
hipError_t launch_fill_zero(float* p, long long n, hipStream_t stream) {
  long long n4 = n / 4;
  const long long grid = (n4 + kThreads - 1) / kThreads;
  f32x4* p4 = reinterpret_cast<f32x4*>(p);
  void* args[] = {(void*)&p4, (void*)&n4};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fill_zero_kernel), dim3((unsigned)grid),
                         dim3(kThreads), args, 0, stream);
}

// dQ kernel: final mode (dq set) or accumulate mode (dq null).
template <int D, bool CAUSAL>
hipError_t launch_dq(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     const uint16_t* dout, uint16_t* dq, const Ws& ws, hipStream_t stream,
                     const uint16_t* o = nullptr, const float* lse = nullptr) {
  DqArgs a;
  const bool f16 = ws.f16(sh);
  const bool copies = f16 && dq;  // whole-sequence path: the fp16 copies for the dK/dV kernel
  a.q = q;
  a.k = f16 ? ws.k16 : k;
  a.v = v;
  a.ek = f16 ? ws.ek : nullptr;
  a.ev = f16 ? ws.ev : nullptr;
  a.dout = dout;
  a.delta = ws.delta;
  a.lse2 = ws.lse2;
  a.o = o;
  a.lse = lse;
  a.dq = dq;
  a.acc_dq = dq ? nullptr : ws.acc_dq;
  a.acc_pk = dq ? nullptr : ws.acc_pk;
  a.acc_c = dq ? nullptr : ws.csum;
  a.q16 = copies ? ws.q16 : nullptr;
  a.do16 = copies ? ws.do16 : nullptr;
  a.eq = copies ? ws.eq : nullptr;
  a.edo = copies ? ws.edo : nullptr;
  a.edl = copies ? ws.edl : nullptr;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.Sq = sh.Sq;
  a.Sk = sh.Sk;
  a.dlt = sh.dlt;
  a.c = sh.scale * kLog2e;
  a.scale = sh.scale;
  a.drop = make_drop(sh.drop_t, sh.seed);
  a.rope_inv = sh.rope;
  a.pack = head_pack(sh, kQBR);
  a.sched.BH = (sh.B * sh.Hq) >> a.pack;
  a.sched.NT = (sh.Sq + kQBR - 1) / kQBR;
  a.sched.chunk = (a.sched.BH + 7) / 8;
  void* args[] = {&a};
  const void* kern = a.drop.t ? (f16 ? reinterpret_cast<const void*>(&attn_bwd_dq_kernel<D, CAUSAL, true, true>)
                                     : reinterpret_cast<const void*>(&attn_bwd_dq_kernel<D, CAUSAL, true>))
                     : f16 ? reinterpret_cast<const void*>(&attn_bwd_dq_kernel<D, CAUSAL, false, true>)
                           : reinterpret_cast<const void*>(&attn_bwd_dq_kernel<D, CAUSAL, false>);
  return hipLaunchKernel(kern, dim3((unsigned)sched_grid(a.sched)), dim3(kBwdThreads), args, 0, stream);
}

// fp16 copy of K and the tile exponents of K and V, for the fp16 dQ kernel
template <int D>
hipError_t launch_k16(const AttnShape& sh, const uint16_t* k, const uint16_t* v, const Ws& ws, hipStream_t stream) {
  int Sk = sh.Sk, ntile = (sh.Sk + 63) / 64;
  const long long grid = (long long)sh.B * sh.Hkv * ntile;
  uint16_t* k16 = ws.k16;
  int* ek = ws.ek;
  int* ev = ws.ev;
  void* args[] = {(void*)&k, (void*)&v, (void*)&k16, (void*)&ek, (void*)&ev, (void*)&Sk, (void*)&ntile};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_k16_kernel<D>), dim3((unsigned)grid),
                         dim3(kThreads), args, 0, stream);
}

// block protocol: fp16 copies of the query block's Q and dO and the block
// exponents of Q, dO and the exact Delta, for the fp16 dK/dV kernel
template <int D>
hipError_t launch_rows16(const AttnShape& sh, const uint16_t* q, const uint16_t* dout, const Ws& ws,
                         hipStream_t stream) {
  int Sq = sh.Sq, nblk = (sh.Sq + 31) / 32;
  const long long grid = (long long)sh.B * sh.Hq * nblk;
  const float* delta = ws.delta;
  uint16_t *q16 = ws.q16, *do16 = ws.do16;
  int *eq = ws.eq, *edo = ws.edo, *edl = ws.edl;
  void* args[] = {(void*)&q, (void*)&dout, (void*)&delta, (void*)&q16, (void*)&do16, (void*)&eq,
                  (void*)&edo, (void*)&edl, (void*)&Sq, (void*)&nblk};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_rows16_kernel<D>), dim3((unsigned)grid),
                         dim3(kThreads), args, 0, stream);
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const uint16_t* dout, uint16_t* dk, uint16_t* dv, const Ws& ws, hipStream_t stream) {
  DkdvArgs a;
  const bool f16 = ws.f16(sh);
  a.q = f16 ? ws.q16 : q;
  a.k = k;
  a.v = v;
  a.dout = f16 ? ws.do16 : dout;
  a.eq = f16 ? ws.eq : nullptr;
  a.edo = f16 ? ws.edo : nullptr;
  a.edl = f16 ? ws.edl : nullptr;
  a.delta = ws.delta;
  a.lse2 = ws.lse2;
  a.dk = dk;
  a.dv = dv;
  a.part = ws.part;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.Sq = sh.Sq;
  a.Sk = sh.Sk;
  a.dlt = sh.dlt;
  a.nsplit = ws.w.nsplit;
  a.c = sh.scale * kLog2e;
  a.scale = sh.scale;
  a.drop = make_drop(sh.drop_t, sh.seed);
  a.rope_inv = sh.rope;
  a.sched.BH = sh.B * sh.Hkv * ws.w.nsplit;
  a.sched.NT = (sh.Sk + kKBC - 1) / kKBC;
  a.sched.chunk = (a.sched.BH + 7) / 8;
  void* args[] = {&a};
  const void* kern = a.drop.t ? (f16 ? reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<D, CAUSAL, true, true>)
                                     : reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<D, CAUSAL, true>))
                     : f16 ? reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<D, CAUSAL, false, true>)
                           : reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<D, CAUSAL, false>);
  return hipLaunchKernel(kern, dim3((unsigned)sched_grid(a.sched)), dim3(kBwdThreads), args, 0, stream);
}

hipError_t launch_reduce(const AttnShape& sh, uint16_t* dk, uint16_t* dv, const Ws& ws, hipStream_t stream) {
  return launch_bwd_reduce(sh, ws.part, ws.w.nsplit, dk, dv, stream);
}

template <int D, bool CAUSAL>
hipError_t launch_all(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* o, const uint16_t* dout, const float* lse, uint16_t* dq,
                      uint16_t* dk, uint16_t* dv, void* workspace, hipStream_t stream,
                      hipEvent_t* ev) {
  hipError_t e;
  auto mark = [&](int i) { return ev ? hipEventRecord(ev[i], stream) : hipSuccess; };
  if (bwd_short_path(sh)) {
    // one kernel (between marks 0 and 1), then the sum of its partials (3 to 4)
    float* part = static_cast<float*>(workspace);
    if ((e = mark(0)) != hipSuccess ||
        (e = launch_bwd_short(sh, q, k, v, dout, lse, dq, dk, dv, part, stream)) != hipSuccess ||
        (e = mark(1)) != hipSuccess || (e = mark(2)) != hipSuccess || (e = mark(3)) != hipSuccess ||
        (e = launch_bwd_reduce(sh, part, bwd_short_split(sh), dk, dv, stream)) != hipSuccess)
      return e;
    return mark(4);
  }
  const Ws ws(sh, workspace, false);
  if ((e = mark(0)) != hipSuccess) return e;
  // 1. the fp16 copy of K for the fp16 dQ kernel (Delta~ and lse2 are formed
  //    inside the dQ kernel on this path)
  if (ws.f16(sh) && (e = launch_k16<D>(sh, k, v, ws, stream)) != hipSuccess) return e;
  if ((e = mark(1)) != hipSuccess) return e;
  // 2. dQ, which also writes lse2 and the exact Delta for the dK/dV kernel
  if ((e = launch_dq<D, CAUSAL>(sh, q, k, v, dout, dq, ws, stream, o, lse)) != hipSuccess ||
      (e = mark(2)) != hipSuccess)
    return e;
  // 3. dK/dV
  if ((e = launch_dkdv<D, CAUSAL>(sh, q, k, v, dout, dk, dv, ws, stream)) != hipSuccess ||
      (e = mark(3)) != hipSuccess)
    return e;
  // 4. fixed-order sum of the head-subset partials
  if ((e = launch_reduce(sh, dk, dv, ws, stream)) != hipSuccess) return e;
  return mark(4);
}

template <int D>
hipError_t block_begin(const AttnShape& sh, const uint16_t* o, const uint16_t* dout, const float* lse,
                       void* workspace, hipStream_t stream) {
  const Ws ws(sh, workspace, true);
  hipError_t e = launch_prep<D>(sh, o, dout, lse, ws, stream);
  // the three accumulators are contiguous: c [rows] then the two [rows, D]
  // sums, each padded to 256 bytes (the fp16 copies follow them)
  if (e == hipSuccess) e = launch_fill_zero(ws.csum, (long long)((ws.w.q16 - ws.w.csum) / 4), stream);
  return e;
}

template <int D>
hipError_t block_dq_end(const AttnShape& sh, uint16_t* dq, void* workspace, hipStream_t stream) {
  const Ws ws(sh, workspace, true);
  const long long rows = (long long)sh.B * sh.Hq * sh.Sq;
  constexpr int RPB = kThreads / (D / 8);
  const long long grid = (rows + RPB - 1) / RPB;
  const float* acc_dq = ws.acc_dq;
  const float* acc_pk = ws.acc_pk;
  const float* csum = ws.csum;
  float* delta = ws.delta;
  float scale = sh.scale;
  void* args[] = {(void*)&acc_dq, (void*)&acc_pk, (void*)&csum, (void*)&delta, (void*)&dq, (void*)&scale,
                  (void*)&rows};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_dq_end_kernel<D>), dim3((unsigned)grid),
                         dim3(kThreads), args, 0, stream);
}

template <int D, bool CAUSAL>
hipError_t block_dkdv(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* dout, uint16_t* dk, uint16_t* dv, void* workspace, hipStream_t stream) {
  const Ws ws(sh, workspace, true);
  hipError_t e;
  // the copies are rewritten by every call of the query block (the same values
  // each time), so that no call depends on another having run
  if (ws.f16(sh) && (e = launch_rows16<D>(sh, q, dout, ws, stream)) != hipSuccess) return e;
  if ((e = launch_dkdv<D, CAUSAL>(sh, q, k, v, dout, dk, dv, ws, stream)) != hipSuccess) return e;
  return launch_reduce(sh, dk, dv, ws, stream);
}

}  // namespace

hipError_t launch_bwd_reduce(const AttnShape& sh, const float* part, int ns, uint16_t* dk, uint16_t* dv,
                             hipStream_t stream) {
  if (ns <= 1) return hipSuccess;
  long long n4 = (long long)sh.B * sh.Hkv * sh.Sk * sh.D / 4;
  const long long grid = (n4 + kThreads - 1) / kThreads;
  void* args[] = {(void*)&part, (void*)&dk, (void*)&dv, (void*)&n4, (void*)&ns};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_reduce_kernel), dim3((unsigned)grid),
                         dim3(kThreads), args, 0, stream);
}

size_t bwd_workspace_bytes(const AttnShape& sh) { return ws_layout(sh).total; }
size_t bwd_block_workspace_bytes(const AttnShape& sh) { return ws_layout(sh, true).total; }

// A block call of a shorter key block can choose a larger head split, whose
// partials then outgrow those of the longest block, so the size that serves
// every call of a query block is the largest need over every key-block length
// up to sh.Sk. The need depends on the length through the number of 128-key
// tiles (which sets the split) and grows with the length at a fixed split; once
// the tiles alone give enough units the split is 1 and the longest block needs
// the most.
size_t bwd_block_workspace_bytes_upto(const AttnShape& sh) {
  const long long per_tile = (long long)sh.B * sh.Hkv;
  const int nt = (sh.Sk + kKBC - 1) / kKBC;
  size_t need = ws_layout(sh, true).total;
  for (int t = 1; t < nt && per_tile * t < kTargetUnits; ++t) {
    AttnShape s = sh;
    s.Sk = t * kKBC;
    need = std::max(need, ws_layout(s, true).total);
  }
  return need;
}

#define TAM_DISPATCH(F, ...)                                                              \
  (sh.D == 128 ? (sh.causal ? F<128, true>(__VA_ARGS__) : F<128, false>(__VA_ARGS__))   \
               : (sh.causal ? F<64, true>(__VA_ARGS__) : F<64, false>(__VA_ARGS__)))

hipError_t launch_bwd(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* o, const uint16_t* dout, const float* lse, uint16_t* dq,
                      uint16_t* dk, uint16_t* dv, void* workspace, hipStream_t stream,
                      hipEvent_t* ev) {
  return TAM_DISPATCH(launch_all, sh, q, k, v, o, dout, lse, dq, dk, dv, workspace, stream, ev);
}

hipError_t launch_bwd_block_begin(const AttnShape& sh, const uint16_t* o, const uint16_t* dout, const float* lse,
                                  void* workspace, hipStream_t stream) {
  return sh.D == 128 ? block_begin<128>(sh, o, dout, lse, workspace, stream)
                     : block_begin<64>(sh, o, dout, lse, workspace, stream);
}

hipError_t launch_bwd_block_dq(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const uint16_t* dout, void* workspace, hipStream_t stream) {
  const Ws ws(sh, workspace, true);
  if (ws.f16(sh)) {
    const hipError_t e = sh.D == 128 ? launch_k16<128>(sh, k, v, ws, stream) : launch_k16<64>(sh, k, v, ws, stream);
    if (e != hipSuccess) return e;
  }
  return TAM_DISPATCH(launch_dq, sh, q, k, v, dout, nullptr, ws, stream);
}

hipError_t launch_bwd_block_dq_end(const AttnShape& sh, uint16_t* dq, void* workspace, hipStream_t stream) {
  return sh.D == 128 ? block_dq_end<128>(sh, dq, workspace, stream) : block_dq_end<64>(sh, dq, workspace, stream);
}

hipError_t launch_bwd_block_dkdv(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const uint16_t* dout, uint16_t* dk, uint16_t* dv, void* workspace,
                                 hipStream_t stream) {
  return TAM_DISPATCH(block_dkdv, sh, q, k, v, dout, dk, dv, workspace, stream);
}

}  // namespace tam
