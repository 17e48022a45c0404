// bias_attn.hip -- [a5] token-gated attention forward: causal GQA flash
// attention over the kept tokens with a per-head, per-key additive gate
// bias and an optional per-query logit scale.
//
// TokenGate pages: ai.info summary "Key Contributions" items 2 and 3 and
// "Methodology in Plain English" -- each kept key's importance score, times
// a learned per-layer per-head gain, is added to the attention logits of
// every upper layer before the online softmax; a learned temperature driven
// by the ratio of a query's position to its rank among kept tokens rescales
// the logits.  The pages' own kernel is a patched FlashAttention-2 for
// NVIDIA parts; this is a gfx950 design of its own.
//
//   z[r,c] = c_r * (scale * <q_r, k_c> + gain_h * score_c),   c <= r
//
// bf16 path (gfx950, wave64):
//   * A workgroup (4 waves, or 8 for large grids) owns one KV head and a
//     block of query positions; each wave owns 32 query positions of one
//     query head, and the HPW query heads of the group that share the KV
//     head (and with 8 waves two query blocks) reuse every K/V tile staged
//     in LDS.
//   * Logits are computed transposed, S^T = K Q^T, on
//     v_mfma_f32_32x32x16_bf16: in the accumulator each lane holds one
//     query column and 16 keys of a 32-key block, so the running max and
//     sum of a query stay inside the lane (plus one exchange between the
//     two lane halves), and the probabilities P^T, converted to bf16 in
//     place, are exactly the B operand of the next product O^T += V^T P^T.
//     The keys that the accumulator layout puts in a lane's k-slots are
//     matched by reading V^T from LDS in the same order.
//   * Q stays in registers for the whole key loop.  K and V tiles go HBM ->
//     LDS with direct-to-LDS loads (no registers, no LDS write
//     instructions); the next tile's loads are issued before the current
//     tile's math and waited for (vmcnt 0) before the tile barrier.  K is
//     row-major with XOR-swizzled 16-byte chunks.  A lane's V^T operand (8
//     keys at one dim) is two transposing LDS reads (ds_read_b64_tr_b16):
//     within a 16-lane group, lane 4a + j reads 4 dims of one key and lane
//     4a' + b' receives dim b' of the 4 keys read by lanes a', a' + 4,
//     a' + 8, a' + 12.  V is stored blocked so that each such read is one
//     contiguous 512-byte run in lane order (a row-major tile, swizzled or
//     not, puts the 8 keys of a read on the same banks; measured on gfx950,
//     the blocked reads run at about 3x the rate).
//   * The two 32-key halves of a tile's logits are independent accumulation
//     chains, interleaved so no MFMA waits on its own predecessor.
//   * Key streams: when the grid is small (short prompts, where the longest
//     causal rows set the time), a workgroup runs two streams of 4 waves on
//     the even and odd key tiles, each with its own LDS buffers, and merges
//     their softmax states at the end; each wave's serial loop halves and
//     two waves share every SIMD.
//   * The bias gain_h*score_c (in dot-product units) is formed once per key
//     tile and head in LDS, in the accumulator layout's key order, and is the
//     initial value of the logit accumulators, so the MFMAs add the dot
//     products to it; logits use exp2 with log2(e) folded into the scale.
//   * The weights' reference is not the running max: a tile's max is taken,
//     and the output rescaled to it, only until every query has one, or
//     when a tile's weights would take some query's running sum past 2^32.
//     The running sum adds the bf16 weights that the PV product uses (two
//     per v_dot2c_f32_bf16), so the normaliser and P^T agree key by key.
//   * Workgroups are ordered longest-first (causal) and the KV head is the
//     fastest-varying index, so consecutive workgroups -- which the
//     dispatcher spreads over the 8 XCDs -- keep one KV head per XCD L2.
//
// f32 path: one thread per (query, head), fp32 online softmax.
#include <algorithm>
#include <deque>
#include <functional>
#include <memory>
#include <mutex>
#include <queue>
#include <type_traits>
#include <vector>

#include "tg_common.hpp"

namespace tg {
namespace {

constexpr int kBK = 64;           // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// K and V tiles, copied HBM -> LDS by direct-to-LDS loads, unpadded.
// K: row-major [key][D], the 16-byte chunk c of key row r stored at chunk
// c ^ (r & SW), so that the 32 rows a wave reads at one column fall in
// different banks.
// V: 512-byte blocks of 8 keys x 32 dims, block (key / 8) * (D / 32) +
// dim / 32; inside a block the 8-byte unit 16 g + 4 j + a holds dims
// 16 (g & 1) + 4 a .. + 3 of key 4 (g >> 1) + j (g, j, a in 0..3, 0..3,
// 0..3), which is lane 16 g + 4 j + a of the transposing read of those
// keys and dims.  A 16-byte chunk (8 dims of one key) stays contiguous, so
// the direct-to-LDS copy fills it with one load per lane.
template <int D>
struct AttnSmem {
  static constexpr int SW = (D / 8 < 16 ? D / 8 : 16) - 1;
  uint16_t ks[kBK * D];
  uint16_t vs[kBK * D];
  float bias[4][kBK];                       // per head, in accumulator order (bias_slot)
};
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ float bf16_val(uint32_t bits) {
  return __uint_as_float(bits << 16);
}

// Logits are tracked in log2 units, y = log2(e) * z.  A tile maximum below
// kMaskedLog2 counts as "no visible key" (a -inf score is encoded as a bias
// far below it).
constexpr float kMaskedLog2 = -524288.0f;
// The running sum of weights 2^(y - m) that makes the reference m move to the
// running max (and the output rescale to it).
constexpr float kSumCap = 0x1p32f;

// The bias of a key tile is the initial value of the logit accumulators: in
// the 32x32 accumulator layout, lane (query, half hh) holds in register r of
// key block kb the logit of key 32 kb + 8 (r / 4) + r % 4 + 4 hh, so the 64
// biases are stored in that order, and each lane reads its 16 with four
// 16-byte reads that every lane of its half shares (LDS broadcasts).
__device__ __forceinline__ int bias_slot(int key) {
  const int rem = key & 31;
  return (key & 32) + ((rem >> 2) & 1) * 16 + (rem >> 3) * 4 + (rem & 3);
}

// ---- key-chunk split ---------------------------------------------------------
// When the grid is small, the longest causal rows alone set the time: one
// workgroup walks every key tile of its row while most CUs have finished.
// The split cuts row p's key tiles [0, row_tiles(p)) into chunks of C tiles
// (items), and packs the items into at most one workgroup per resident slot
// (bins): largest first, each item to the bin with the least work so far.
// A bin walks its items one after the other.  An item of a row with more than one chunk writes its
// unnormalised softmax state (running max, sum, O^T) to the workspace, and
// attn_merge_kernel combines a row's chunks; the other items write their
// output directly.  Launching no more workgroups than the chip holds at once
// matters: workgroups beyond that are handed out in dispatch order as slots
// free up, late, whatever their size.
constexpr int kMaxChunks = 8;     // chunks per row
constexpr size_t kNoSlot = ~static_cast<size_t>(0);
constexpr int kMaxBins = 512;     // workgroups per query-head group
constexpr int kMaxItems = 1024;   // items per query-head group

struct SplitArgs {
  uint16_t* part_o;   // [slot][4 waves][D/32][64 lanes][16] fp16: scaled O^T accumulators
  float* part_ml;   // [slot][4 waves][64 lanes][2] f32: running max (log2 units), sum
  // slot of chunk c of split row p: ((npb - 1 - p) * nchunk + c) * query-head groups + group
  int32_t ctiles;   // C, key tiles per chunk
  int32_t nchunk;   // chunks of the longest row
};
// The chunk launch's kernel arguments: the split and its bins (about 3 KB).
struct SplitLaunch {
  SplitArgs a;
  uint16_t bin_first[kMaxBins + 1];   // bin b walks items [bin_first[b], bin_first[b + 1])
  uint16_t items[kMaxItems];          // item: row p << 3 | chunk c
};
struct NoSplit {};

__host__ __device__ inline int row_tiles(int p, int PB, int N, bool causal) {
  const int end = causal ? ((p + 1) * PB < N ? (p + 1) * PB : N) : N;
  return (end + kBK - 1) / kBK;
}

template <int D, int HPW, int KS, int QW, bool CAUSAL, bool HAS_BIAS, bool HAS_QSCALE,
          bool SPLIT>
__global__ __launch_bounds__(64 * QW * KS, (KS == 1 && QW == 4 && D <= 128) ? 2 : 1) void
attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ key_score,
    const float* __restrict__ gain, const float* __restrict__ q_scale, float scale,
    uint16_t* __restrict__ out, float* __restrict__ lse, int32_t N, int32_t Hq, int32_t Hkv,
    int32_t n_pblocks, int32_t n_hgroups, const int32_t* __restrict__ n_dyn,
    std::conditional_t<SPLIT, SplitLaunch, NoSplit> sp) {
  static_assert(!SPLIT || KS == 1, "a split chunk runs one key stream");
  static_assert(QW == 4 || (QW == 8 && KS == 1 && !SPLIT), "8 waves: one key stream, unsplit");
  constexpr int PB = 32 * (QW / HPW);       // query positions per workgroup
  constexpr int DK = D / 16;                // k-steps of S^T = K Q^T (plus one extra)
  constexpr int DB = D / 32;                // 32-row blocks of O^T
  // KS key streams: stream kh (waves 4kh .. 4kh+3, threads 256kh ..) takes
  // key tiles kh, kh + KS, kh + 2KS, ... with its own LDS buffers; the
  // streams' partial softmax states are merged at the end
  using Smem = AttnSmem<D>;
  __shared__ __attribute__((aligned(16))) Smem sm[2][KS];

  constexpr int NT = 64 * QW;               // threads per key stream
  const int tid = threadIdx.x % NT;         // thread index within the key stream
  const int kh = threadIdx.x / NT;          // key stream
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;                 // which half of the wave

  const int hg = blockIdx.x % n_hgroups;
  const int G = Hq / Hkv;
  const int hw = wave % HPW;
  // Ne: the kept count read at run time (N is then the capacity the launch
  // and its buffers are sized for): keys at or past it are masked, and query
  // rows at or past it are padding, written as O = 0, lse = -inf
  const int Ne = n_dyn != nullptr ? min(N, max(*n_dyn, 0)) : N;
  // key tiles with a visible key for query block p
  auto live_tiles = [&](int p) { return p * PB >= Ne ? 0 : row_tiles(p, PB, Ne, CAUSAL); };
  const int head = hg * HPW + hw;
  const int kvh = (hg * HPW) / G;

  const uint32_t q_row = static_cast<uint32_t>(Hq) * D * 2;     // bytes per token
  const __amdgpu_buffer_rsrc_t q_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(q), 0, static_cast<int>(static_cast<uint32_t>(N) * q_row), 0x00020000);

  // ---- staging -------------------------------------------------------------
  const float inv_scale = 1.0f / scale;
  // A -inf score becomes the bias -2^100 in dot-product units (exact, and it
  // absorbs any finite dot product).  Its logit, -2^100 scale log2(e) c_r log2 units, falls below
  // kMaskedLog2 whenever scale * c_r > 2^-80, and its weight underflows to
  // exactly 0, as deleting the key would give.
  const float masked_bias = -0x1p100f;
  float sreg = 0.0f;        // staged raw score (its bias is formed at store time)
  const int bias_key = tid % kBK;
  const float bias_gain = (HAS_BIAS && tid < HPW * kBK) ? gain[hg * HPW + tid / kBK] : 0.0f;
  const __amdgpu_buffer_rsrc_t s_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(key_score), 0, HAS_BIAS ? N * 4 : 0, 0x00020000);
  // each wave of the stream issues its share of the tile's 1-KB pieces
  // through buffer resources over K and V: a lane's byte offset within a
  // tile is the same for every tile (the compiler keeps it out of the key
  // loop), a tile adds one scalar, and rows past N fall outside the
  // resource and read as 0 (those keys are masked, and their weights are 0)
  constexpr int PIECES = kBK * D * 2 / 1024;
  constexpr int PPW = PIECES / QW;
  static_assert(PPW * QW == PIECES, "whole pieces per wave");
  const uint32_t kv_row = static_cast<uint32_t>(Hkv) * D * 2;   // bytes per key
  const int kv_bytes = static_cast<int>(static_cast<uint32_t>(N) * kv_row);
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(k), 0, kv_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(v), 0, kv_bytes, 0x00020000);
  auto dma_tile = [&](int t, Smem& b) {
    // wave-uniform (the key stream kh is)
    const uint32_t tb = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(t * kBK)) * kv_row;
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int u = wave * PPW + i;
      const int byte = u * 1024 + 16 * lane;
      const int r = byte / (2 * D), c = ((byte % (2 * D)) / 16) ^ (r & Smem::SW);
      const uint32_t koff = static_cast<uint32_t>(r) * kv_row + static_cast<uint32_t>(kvh * D + 8 * c) * 2u;
      // V: 16-byte slot u * 64 + lane of the blocked layout
      const int vb = (u * 64 + lane) >> 5, vsl = lane & 31;
      const int vkey = 8 * (vb / (D / 32)) + 4 * (vsl >> 4) + ((vsl >> 1) & 3);
      const int vdim = 32 * (vb % (D / 32)) + 16 * ((vsl >> 3) & 1) + 8 * (vsl & 1);
      const uint32_t voff = static_cast<uint32_t>(vkey) * kv_row + static_cast<uint32_t>(kvh * D + vdim) * 2u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          krs, (__attribute__((address_space(3))) void*)&b.ks[u * 512], 16, tb + koff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          vrs, (__attribute__((address_space(3))) void*)&b.vs[u * 512], 16, tb + voff, 0, 0, 0);
    }
    if (HAS_BIAS && tid < HPW * kBK)   // keys past N read 0
      sreg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           s_rs, 4u * static_cast<uint32_t>(t * kBK + bias_key), 0, 0));
  };
  auto store_bias = [&](Smem& b) {
    if (HAS_BIAS && tid < HPW * kBK)
      b.bias[tid / kBK][bias_slot(bias_key)] =
          sreg == -INFINITY ? masked_bias : bias_gain * sreg * inv_scale;
  };
  // vmcnt(0), other counters untouched: every direct-to-LDS load of this
  // wave has landed (each wave then passes the barrier)
  auto dma_wait = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };

  // One item: query block pblock against key tiles [t_first, t_end) of its
  // n_tiles; the final output, or (slot != kNoSlot) the unnormalised state.
  auto run_item = [&](const int pblock, const int t_first, const int t_end, const int n_tiles,
                      const size_t slot) {
  const int pos0 = pblock * PB + 32 * (wave / HPW);
  const int my_q = pos0 + l32;
  const bool q_ok = my_q < N;

  // y = ac * (<q, k> + bias'_k), with ac = scale * log2(e) * c_r and the
  // per-key bias'_k = gain * score_k / scale in dot-product units.
  const float cr = HAS_QSCALE ? (q_ok ? q_scale[my_q] : 1.0f) : 1.0f;
  const float ac = scale * kLog2e * cr;

  // Q^T as MFMA B operand (exact bf16): lane (query l32, half hh) holds dims
  // 16 ks + 8 hh .. +7.
  bf16x8 qf[DK];
  {
    const uint32_t base = static_cast<uint32_t>(my_q) * q_row +
                          static_cast<uint32_t>(head) * D * 2 + 16u * hh;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8,
                                  __builtin_amdgcn_raw_buffer_load_b128(q_rs, base + 32u * ks, 0, 0));
  }
  // reference of the weights 2^(y - m) (log2 units): -inf until a visible
  // key, then some running max of y that the weights never exceed by 32
  float m_run = -INFINITY;
  float m_use = 0.0f;       // m_run, or 0 while it is -inf
  const int lim = CAUSAL ? min(my_q, Ne - 1) : Ne - 1;   // last visible key

  // ---- running state --------------------------------------------------------
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float l_run = 0.0f;       // this lane's share of the running sum of 2^y

  if (t_first + kh < t_end) {
    dma_tile(t_first + kh, sm[0][kh]);
    store_bias(sm[0][kh]);
  }
  dma_wait();
  __syncthreads();

  const int n_rounds = (t_end - t_first + KS - 1) / KS;
  // one round; b is this round's buffer and nb the next one's.  Unsplit at
  // head dim <= 128 it is called with fixed buffers for even and odd rounds,
  // so every LDS address of a round is a loop-invariant register plus an
  // immediate.
  auto round = [&](const int j, const Smem& b, Smem& nb) __attribute__((always_inline)) {
    const int t = t_first + KS * j + kh;     // this stream's tile
    const int k0 = t * kBK;
    const bool more = t + KS < t_end;
    if (more) dma_tile(t + KS, nb);
    // keep the next tile's loads issued here, ahead of this tile's math
    __builtin_amdgcn_sched_barrier(0);
    if (KS == 1 || t < t_end) {   // uniform per wave: a stream may idle in the last round

    // S^T = bias' + K Q^T: the accumulators start from the tile's bias (in
    // dot-product units, zero without one); the two 32-key halves are
    // independent accumulation chains, interleaved so neither waits on its
    // own last MFMA
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (HAS_BIAS) {
        const f32x4* bp = reinterpret_cast<const f32x4*>(&b.bias[hw][32 * kb + 16 * hh]);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v4 = bp[q4];
#pragma unroll
          for (int e = 0; e < 4; ++e) s[kb][4 * q4 + e] = v4[e];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
      }
    }
#pragma unroll
    for (int ks = 0; ks < DK; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = 32 * kb + l32;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            &b.ks[row * D + 8 * ((2 * ks + hh) ^ (row & Smem::SW))]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
      }
    // operand reads run four K fragments ahead of their MFMAs (the bias
    // reads first): 1.5-2% faster at head dim <= 128, slower at 256
    if constexpr (D <= 128) {
      __builtin_amdgcn_sched_group_barrier(0x100, HAS_BIAS ? 12 : 4, 0);
#pragma unroll
      for (int i = 0; i < 2 * DK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }

    // causal / tail mask (only tiles that reach past a query or past N)
    const bool need_mask = (CAUSAL && k0 + kBK - 1 > pos0) || (k0 + kBK > Ne);
    if (need_mask) {
      const int rel = lim - k0 - 4 * hh;   // key index k0 + 4hh + c is visible iff c <= rel
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 32 * kb + 8 * (r >> 2) + (r & 3);
          s[kb][r] = c <= rel ? s[kb][r] : -INFINITY;
        }
    }

    // P^T = 2^(y - m) as bf16, already laid out as the PV B operand, with
    // the lane's reference m; lt is the running sum with this tile added.
    // The sum adds the bf16 weights themselves (two per v_dot2c with a pair
    // of ones), so the normaliser weighs each key exactly as P^T does.
    bf16x8 p[2][2];
    float lt;
    auto weights = [&]() __attribute__((always_inline)) {
      lt = l_run;
      const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          bf16x2 pr[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e0 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hf + 2 * i], ac, -m_use));
            const float e1 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hf + 2 * i + 1], ac, -m_use));
            pr[i] = bf16x2{static_cast<__bf16>(e0), static_cast<__bf16>(e1)};
            lt = __builtin_amdgcn_fdot2_f32_bf16(pr[i], ones, lt, false);
          }
          p[kb][hf] = __builtin_bit_cast(bf16x8, pr);
        }
    };
    // The reference is not kept at the running max: a tile's max is taken
    // only while some lane has no reference yet (its keys so far were all
    // masked, or none were seen), or when this tile's weights would take
    // some lane's sum past kSumCap (a logit about 32 log2 units above the
    // reference, or one that overflowed to inf).  Then every lane moves its
    // reference to its own running max, rescales its state and computes the
    // tile's weights again.  Otherwise no weight exceeds 2^32, and |O^T|
    // stays within 2^33 max|V|.
    const bool no_ref = __any(m_run == -INFINITY);
    if (!no_ref) weights();
    if (no_ref || __any(!(lt <= kSumCap))) {
      // tile max: one chain per 32-key half, each step taking two logits
      // (one v_max3), then the two lane halves through a lane-half swap
      float hmax[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        hmax[kb] = fmaxf(s[kb][0], s[kb][1]);
#pragma unroll
        for (int r = 2; r < 16; r += 2) hmax[kb] = fmaxf(fmaxf(hmax[kb], s[kb][r]), s[kb][r + 1]);
      }
      float tmax = fmaxf(hmax[0], hmax[1]);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax),
                                                         __float_as_uint(tmax), false, false);
        tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      // running max in log2 units (ac > 0 keeps the arg-max); maxima below
      // kMaskedLog2 are masked keys only
      float tm = tmax * ac;
      tm = tm > kMaskedLog2 ? tm : -INFINITY;
      const float m_new = fmaxf(m_run, tm);
      // 0 when nothing was accumulated yet; 1 for a lane whose max held
      const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      l_run *= alpha;
      m_run = m_new;
      m_use = m_run == -INFINITY ? 0.0f : m_run;
      weights();
    }
    l_run = lt;

    // O^T += V^T P^T: k-step (kb, hf) covers keys 32kb + 16hf + {4hh..4hh+3,
    // 8+4hh..8+4hh+3}, stored at slots 32kb + 16hf + 8hh .. +7: one 16-byte read
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          // two transposing reads: within each 16-lane group g, lane 4a + j
          // reads 4 dims (32 db + 16 (g & 1) + 4a ..) of key
          // 32 kb + 16 hf + 8 r + 4 (g >> 1) + j, and lane 4a' + b' receives
          // dim 32 db + 16 (g & 1) + 4a' + b' of the group's keys j = 0..3:
          // its V^T row, in the key order of the P^T operand
          // (blocked V: the read of keys 8 (4 kb + 2 hf + r) .. + 7, dims
          // 32 db .. + 31 is block (4 kb + 2 hf + r) * D / 32 + db, lane order)
          bf16x4 vh[2];
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int off = ((4 * kb + 2 * hf + r) * (D / 32) + db) * 256 + 4 * lane;
            vh[r] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4*)(const_cast<uint16_t*>(b.vs) + off));
          }
          const bf16x8 a8 = __builtin_shufflevector(vh[0], vh[1], 0, 1, 2, 3, 4, 5, 6, 7);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, p[kb][hf], o[db], 0, 0, 0);
        }
      }
    }

    }
    if (more) store_bias(nb);
    dma_wait();
    __syncthreads();
  };
  if constexpr (D <= 128 && !SPLIT) {
    int j = 0;
    for (; j + 1 < n_rounds; j += 2) {
      round(j, sm[0][kh], sm[1][kh]);
      round(j + 1, sm[1][kh], sm[0][kh]);
    }
    if (j < n_rounds) round(j, sm[0][kh], sm[1][kh]);
  } else {
    // head dim 256, or a split chunk: three copies of the round would not
    // fit the registers
    for (int j = 0; j < n_rounds; ++j) round(j, sm[j & 1][kh], sm[(j + 1) & 1][kh]);
  }
  if (KS > 1) {
    // merge the streams' (running max, partial sums, O^T) into stream 0
    constexpr int NV = DB * 16 + 2;
    float* xch = reinterpret_cast<float*>(&sm[0][0]);
    const int slot = wave * 64 + lane;
    if (kh > 0) {
      float* dst = xch + static_cast<size_t>((kh - 1) * 256 + slot) * NV;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[db * 16 + r] = o[db][r];
      dst[DB * 16] = m_run;
      dst[DB * 16 + 1] = l_run;
    }
    __syncthreads();
    if (kh > 0) return;
#pragma unroll
    for (int other = 1; other < KS; ++other) {
      const float* src = xch + static_cast<size_t>((other - 1) * 256 + slot) * NV;
      const float m1 = src[DB * 16];
      const float m = fmaxf(m_run, m1);
      const float a0 = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m);
      const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = o[db][r] * a0 + src[db * 16 + r] * a1;
      l_run = l_run * a0 + src[DB * 16 + 1] * a1;
      m_run = m;
    }
  }

  // ---- epilogue -------------------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if constexpr (SPLIT) {
    if (slot != kNoSlot) {
      // one chunk of a split row: hand the unnormalised state to the merge
      // O^T goes out in fp16 (half the bytes written here and read by the
      // merge).  The state (m, l, O) and (m - k, l 2^k, O 2^k) stand for the
      // same weights 2^(y - m), so each lane scales its O by the power of two
      // 2^k that puts its largest |O| in [2^14, 2^15): no fp16 overflow, and
      // one rounding of 2^-11 relative.  The max and sum stay fp32.
      float amax = 0.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(o[db][r]));
      int e = 0;
      (void)frexpf(amax, &e);                       // amax < 2^e (amax == 0: e == 0)
      const int k = amax > 0.0f ? min(max(15 - e, -60), 60) : 0;
      const float sc = ldexpf(1.0f, k);
      const size_t ws = slot * 4 + wave;
      uint16_t* po = sp.a.part_o + (ws * DB * 64 + lane) * 16;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
          f16x8 w;
#pragma unroll
          for (int i = 0; i < 8; ++i) w[i] = static_cast<_Float16>(o[db][8 * h8 + i] * sc);
          *reinterpret_cast<f16x8*>(po + db * 64 * 16 + 8 * h8) = w;
        }
      *reinterpret_cast<float2*>(sp.a.part_ml + ws * 128 + 2 * lane) =
          make_float2(m_run == -INFINITY ? m_run : m_run - static_cast<float>(k), l_tot * sc);
      return;
    }
  }
  // no visible key, or a padding row
  const bool empty = !(l_tot > 0.0f) || m_run == -INFINITY || my_q >= Ne;
  const float inv = empty ? 0.0f : 1.0f / l_tot;
  if (q_ok) {
    uint16_t* op = out + static_cast<int64_t>(my_q) * Hq * D + static_cast<int64_t>(head) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = static_cast<__bf16>(o[db][4 * j + i] * inv);
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * j + 4 * hh) = w;
      }
    }
    if (lse != nullptr && hh == 0)
      lse[static_cast<int64_t>(head) * N + my_q] =
          empty ? -INFINITY : kLn2 * (m_run + __builtin_log2f(l_tot));
  }
  };

  if constexpr (SPLIT) {
    const int bin = blockIdx.x / n_hgroups;
    const int i_end = sp.bin_first[bin + 1];
    for (int i = sp.bin_first[bin]; i < i_end; ++i) {
      const int item = sp.items[i];
      const int p = item >> 3, c = item & 7;
      const int nt = row_tiles(p, PB, N, CAUSAL);
      const int t0 = c * sp.a.ctiles;
      const size_t slot =
          nt > sp.a.ctiles
              ? (static_cast<size_t>(n_pblocks - 1 - p) * sp.a.nchunk + c) * n_hgroups + hg
              : kNoSlot;
      run_item(p, t0, min(t0 + sp.a.ctiles, live_tiles(p)), nt, slot);
    }
  } else {
    const int prank = blockIdx.x / n_hgroups;
    const int pblock = CAUSAL ? n_pblocks - 1 - prank : prank;
    const int nt = live_tiles(pblock);
    run_item(pblock, 0, nt, nt, kNoSlot);
  }
}

// Combines the chunks of every split row: with the chunks' running maxima
// m_c (log2 units), sums l_c and unnormalised O_c,
//   M = max_c m_c,  w_c = 2^(m_c - M),  O = sum_c w_c O_c / sum_c w_c l_c,
// the state one pass over all keys reaches.  One workgroup per (split row,
// query-head group, 32-dim block of O); thread (wave, lane) owns the
// accumulator entries that lane of that wave held in the chunk workgroups.
template <int D, int HPW, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_merge_kernel(SplitArgs sp, uint16_t* __restrict__ out,
                                                         float* __restrict__ lse, int32_t N,
                                                         int32_t Hq, int32_t n_pblocks,
                                                         int32_t n_hgroups,
                                                         const int32_t* __restrict__ n_dyn) {
  constexpr int PB = 32 * (4 / HPW);
  constexpr int DB = D / 32;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  // the query-head group is the fastest index, as in the chunk launch, so a
  // group's merge runs on the XCD whose L2 holds its chunk states
  const int hg = blockIdx.x % n_hgroups;
  const int db = (blockIdx.x / n_hgroups) % DB;
  const int rank = static_cast<int>(blockIdx.x) / (n_hgroups * DB);   // split rows, longest first
  const int pblock = n_pblocks - 1 - rank;
  const int head = hg * HPW + wave % HPW;
  const int my_q = pblock * PB + 32 * (wave / HPW) + l32;
  const int nc = (row_tiles(pblock, PB, N, CAUSAL) + sp.ctiles - 1) / sp.ctiles;

  // every load first (one round trip), then the combination
  float2 ml[kMaxChunks];
  f16x8 ov[kMaxChunks][2];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    if (c < nc) {
      const size_t slot = ((static_cast<size_t>(rank) * sp.nchunk + c) * n_hgroups + hg) * 4 + wave;
      ml[c] = *reinterpret_cast<const float2*>(sp.part_ml + slot * 128 + 2 * lane);
      const f16x8* po =
          reinterpret_cast<const f16x8*>(sp.part_o + ((slot * DB + db) * 64 + lane) * 16);
      ov[c][0] = po[0];
      ov[c][1] = po[1];
    }
  }
  float m_max = -INFINITY;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c)
    if (c < nc) m_max = fmaxf(m_max, ml[c].x);
  float l_tot = 0.0f;
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    if (c < nc) {
      const float w = ml[c].x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml[c].x - m_max);
      l_tot += w * ml[c].y;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[j][i] = fmaf(w, static_cast<float>(ov[c][j >> 1][4 * (j & 1) + i]), acc[j][i]);
    }
  }
  // no visible key, or a padding row past a run-time kept count
  const bool empty = !(l_tot > 0.0f) || m_max == -INFINITY ||
                     (n_dyn != nullptr && my_q >= *n_dyn);
  const float inv = empty ? 0.0f : 1.0f / l_tot;
  if (my_q >= N) return;
  uint16_t* op = out + static_cast<int64_t>(my_q) * Hq * D + static_cast<int64_t>(head) * D +
                 32 * db + 4 * hh;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bf16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = static_cast<__bf16>(acc[j][i] * inv);
    *reinterpret_cast<bf16x4*>(op + 8 * j) = v;
  }
  if (lse != nullptr && hh == 0 && db == 0)
    lse[static_cast<int64_t>(head) * N + my_q] =
        empty ? -INFINITY : kLn2 * (m_max + __builtin_log2f(l_tot));
}

// ---------------------------------------------------------------------------
// fp32 path: one thread per (query row, query head), online softmax in fp32.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ key_score, const float* __restrict__ gain,
    const float* __restrict__ q_scale, float scale, int causal, float* __restrict__ out,
    float* __restrict__ lse, int32_t N, int32_t Hq, int32_t Hkv,
    const int32_t* __restrict__ n_dyn) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(N) * Hq) return;
  const int r = static_cast<int>(idx / Hq);
  const int h = static_cast<int>(idx % Hq);
  // run-time kept count (N: capacity): later rows are padding, keys masked
  const int Ne = n_dyn != nullptr ? min(N, max(*n_dyn, 0)) : N;
  if (r >= Ne) {
    float* op = out + (static_cast<int64_t>(r) * Hq + h) * D;
    for (int e = 0; e < D; ++e) op[e] = 0.0f;
    if (lse) lse[static_cast<int64_t>(h) * N + r] = -INFINITY;
    return;
  }
  const int kvh = h / (Hq / Hkv);
  const float c = q_scale ? q_scale[r] : 1.0f;
  const float g = key_score ? gain[h] : 0.0f;
  float qr[D], acc[D];
  const float* qp = q + (static_cast<int64_t>(r) * Hq + h) * D;
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qr[e] = qp[e];
    acc[e] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  const int nk = causal ? r + 1 : Ne;
  for (int j = 0; j < nk; ++j) {
    const float* kp = k + (static_cast<int64_t>(j) * Hkv + kvh) * D;
    float dot = 0.0f;
#pragma unroll
    for (int e = 0; e < D; ++e) dot = fmaf(qr[e], kp[e], dot);
    const float z = c * (scale * dot + (key_score ? g * key_score[j] : 0.0f));
    if (z == -INFINITY) continue;
    const float* vp = v + (static_cast<int64_t>(j) * Hkv + kvh) * D;
    if (z > m) {
      const float a = expf(m - z);
      l = l * a + 1.0f;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(acc[e], a, vp[e]);
      m = z;
    } else {
      const float w = expf(z - m);
      l += w;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(w, vp[e], acc[e]);
    }
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  float* op = out + (static_cast<int64_t>(r) * Hq + h) * D;
#pragma unroll
  for (int e = 0; e < D; ++e) op[e] = acc[e] * inv;
  if (lse) lse[static_cast<int64_t>(h) * N + r] = l > 0.0f ? m + logf(l) : -INFINITY;
}

// Two key streams per workgroup halve each wave's serial key loop, at the
// cost of a whole CU's LDS per workgroup: they pay off while the grid is too
// small to keep every CU busy with one-stream workgroups for several rounds.
// Measured at 16/8 heads (grid = 8 ceil(N / 64)), unsplit: two streams took
// 116 / 130 us at N = 4500 / 5000 against 133 / 140 us for 8-wave one-stream
// workgroups, the same at 6000, and 217 / 272 / 282 us at 7000 / 8000 / 8192
// against 200 / 251 / 259 us.
constexpr int64_t kTwoStreamMaxGrid = 768;
// Workgroups resident at once on the chip (its compute units, 256 on
// MI355X, read from the device): two per CU for the one-stream kernel at
// head dim <= 128, one per CU for two-stream workgroups and at head dim 256
// (whose tile pair fills a CU's LDS).
constexpr int kMinChunkTiles = 4;
// Cost model, in units of one key tile of one workgroup (~2.4 us at head
// dim 128 with two workgroups per CU): each item adds its setup (Q and first
// tile loads) and epilogue, two units (with one and a half, the packing chose
// more and smaller chunks at N = 1500 that measured slower); the merge costs
// two units for its launch (with one, N = 3000 at 16/8 heads split and
// measured 55.6 against 52.1 us unsplit) plus the chunk states' bytes read
// back at about 10 MB per unit.
constexpr double kItemUnits = 2.0;
// A two-stream workgroup's round of two tiles (one per stream) costs about
// one unit, as measured with direct-to-LDS staging.
constexpr double kTwoStreamRoundUnits = 1.0;
constexpr double kMergeFixedUnits = 2.0;
constexpr double kMergeBytesPerUnit = 10.0e6;
// The split must beat the unsplit launch by this factor to be used.
constexpr double kSplitGain = 0.92;

struct AttnArgs {
  const uint16_t *q, *k, *v;
  const float *ks, *gain, *qs;
  float scale;
  uint16_t* out;
  float* lse;
  int32_t N, Hq, Hkv;
  bool causal, has_bias, has_qs;
  hipStream_t s;
  const int32_t* n_dyn;   // run-time kept count, or NULL
};

// Key-chunk split of a bf16 launch (ctiles == 0: the launch runs unsplit).
struct SplitPlan {
  int32_t ctiles = 0, nchunk = 0, n_bins = 0, n_split_rows = 0;
  size_t part_o_elems = 0, bytes = 0;   // fp16 elements of part_o; workspace bytes
  std::vector<uint16_t> bin_first, items;
};

// Greedy list schedule of tasks (sizes in tile units, in dispatch order) on
// `slots` identical workgroup slots: the time the last one ends.
double list_schedule(const std::vector<double>& tasks, int slots) {
  std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
  for (int i = 0; i < slots; ++i) free_at.push(0.0);
  double end = 0.0;
  for (double t : tasks) {
    const double s = free_at.top();
    free_at.pop();
    end = std::max(end, s + t);
    free_at.push(s + t);
  }
  return end;
}

SplitPlan make_split_plan(int64_t N, int64_t Hq, int64_t Hkv, int64_t D, bool causal,
                          int cus) {
  SplitPlan best_plan;
  if (N <= 0) return best_plan;
  const int64_t G = Hq / Hkv;
  const int hpw = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  const int PB = 32 * (4 / hpw);
  const int npb = static_cast<int>((N + PB - 1) / PB), nhg = static_cast<int>(Hq / hpw);
  if (static_cast<int64_t>(npb) * nhg > kTwoStreamMaxGrid) return best_plan;
  const int n = static_cast<int>(N);
  const int nt_max = row_tiles(npb - 1, PB, n, causal);
  const int slots = D <= 128 ? 2 * cus : cus;   // split workgroups resident at once
  const int max_bins = std::min(kMaxBins, slots / nhg);
  if (max_bins < 1) return best_plan;
  // unsplit: at head dim <= 128 two key streams per workgroup, each walking
  // half of its row, one workgroup per CU; at 256 one stream
  std::vector<double> tasks;
  for (int p = npb - 1; p >= 0; --p)
    for (int h = 0; h < nhg; ++h) {
      const int nt = row_tiles(p, PB, n, causal);
      tasks.push_back((D <= 128 ? (nt + 1) / 2 * kTwoStreamRoundUnits : nt) + kItemUnits);
    }
  double best = list_schedule(tasks, cus) * kSplitGain;
  // per state slot (4 waves): O^T in fp16, (max, sum) in fp32
  const size_t state_bytes =
      static_cast<size_t>(4) * ((D / 32) * 16 * 64 * sizeof(uint16_t) + 128 * sizeof(float));
  struct Item {
    int size, p, c;
  };
  std::vector<Item> items;
  std::vector<std::vector<uint16_t>> bins;
  for (int C = std::max((nt_max + kMaxChunks - 1) / kMaxChunks, kMinChunkTiles); C < nt_max;
       ++C) {
    const int nchunk = (nt_max + C - 1) / C;
    items.clear();
    int split_rows = 0;
    int64_t states = 0;   // chunk states written and merged, per query-head group
    for (int p = npb - 1; p >= 0; --p) {
      const int nt = row_tiles(p, PB, n, causal);
      if (nt > C) {
        ++split_rows;
        states += (nt + C - 1) / C;
      }
      for (int c = 0; c * C < nt; ++c) items.push_back(Item{std::min(C, nt - c * C), p, c});
    }
    if (items.size() > static_cast<size_t>(kMaxItems)) continue;
    // longest processing time first: items largest first (ties: longer row
    // first), each to the bin with the least work so far (ties: lowest bin)
    std::stable_sort(items.begin(), items.end(),
                     [](const Item& a, const Item& b) { return a.size > b.size; });
    using Load = std::pair<double, int>;
    std::priority_queue<Load, std::vector<Load>, std::greater<Load>> load;
    for (int b = 0; b < max_bins; ++b) load.push(Load(0.0, b));
    bins.assign(max_bins, {});
    for (size_t i = 0; i < items.size(); ++i) {
      Load l = load.top();
      load.pop();
      bins[l.second].push_back(static_cast<uint16_t>(i));
      l.first += items[i].size + kItemUnits;
      load.push(l);
    }
    double makespan = 0.0;
    while (!load.empty()) {
      makespan = std::max(makespan, load.top().first);
      load.pop();
    }
    const double t = makespan + kMergeFixedUnits +
                     static_cast<double>(states * nhg) * state_bytes / kMergeBytesPerUnit;
    if (t < best) {
      best = t;
      best_plan.ctiles = C;
      best_plan.nchunk = nchunk;
      best_plan.n_split_rows = split_rows;
      best_plan.bin_first.assign(1, 0);
      best_plan.items.clear();
      for (const auto& bin : bins) {
        if (bin.empty()) continue;   // fewer items than bins
        for (uint16_t i : bin)
          best_plan.items.push_back(static_cast<uint16_t>((items[i].p << 3) | items[i].c));
        best_plan.bin_first.push_back(static_cast<uint16_t>(best_plan.items.size()));
      }
      best_plan.n_bins = static_cast<int32_t>(best_plan.bin_first.size()) - 1;
    }
  }
  if (best_plan.ctiles == 0) return best_plan;
  const size_t n_states = static_cast<size_t>(best_plan.n_split_rows) * best_plan.nchunk * nhg;
  best_plan.part_o_elems = n_states * 4 * (D / 32) * 16 * 64;
  best_plan.bytes = n_states * state_bytes;
  return best_plan;
}

// Plans depend only on the shape and are kept for the last kPlanCache shapes
// (the kept-token count N changes from prompt to prompt, so the cache is
// bounded; the oldest entry goes first).  A caller holds its plan through a
// shared pointer, so an eviction by another thread never frees it early.
constexpr size_t kPlanCache = 256;
std::shared_ptr<const SplitPlan> split_plan(int64_t N, int64_t Hq, int64_t Hkv, int64_t D,
                                            bool causal) {
  struct Entry {
    int64_t N, Hq, Hkv, D;
    bool causal;
    int cus;
    std::shared_ptr<const SplitPlan> plan;
  };
  const int cus = device_cu_count();
  static std::mutex mu;
  static std::deque<Entry> cache;
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry& e : cache)
    if (e.N == N && e.Hq == Hq && e.Hkv == Hkv && e.D == D && e.causal == causal &&
        e.cus == cus)
      return e.plan;
  if (cache.size() >= kPlanCache) cache.pop_front();
  cache.push_back(Entry{N, Hq, Hkv, D, causal, cus,
                        std::make_shared<const SplitPlan>(
                            make_split_plan(N, Hq, Hkv, D, causal, cus))});
  return cache.back().plan;
}

template <int D, int HPW, bool CAUSAL, int KS, bool SPLIT, typename SP, int QW = 4>
void launch_bf16_attn_ks(const AttnArgs& a, dim3 grid, int32_t npb, int32_t nhg, const SP& sp) {
#define TG_ATTN_LAUNCH(B, Q)                                                                 \
  attn_bf16_kernel<D, HPW, KS, QW, CAUSAL, B, Q, SPLIT><<<grid, dim3(64 * QW * KS), 0, a.s>>>( \
      a.q, a.k, a.v, a.ks, a.gain, a.qs, a.scale, a.out, a.lse, a.N, a.Hq, a.Hkv, npb, nhg,   \
      a.n_dyn, sp)
  if (a.has_bias) {
    if (a.has_qs) TG_ATTN_LAUNCH(true, true); else TG_ATTN_LAUNCH(true, false);
  } else {
    if (a.has_qs) TG_ATTN_LAUNCH(false, true); else TG_ATTN_LAUNCH(false, false);
  }
#undef TG_ATTN_LAUNCH
}

template <int D, int HPW, bool CAUSAL>
void launch_bf16_attn(const AttnArgs& a, const SplitPlan& pl, void* workspace) {
  constexpr int PB = 32 * (4 / HPW);
  const int32_t npb = (a.N + PB - 1) / PB;
  const int32_t nhg = a.Hq / HPW;
  const NoSplit none{};
  {
    if (pl.ctiles > 0 && workspace != nullptr) {
      SplitLaunch sl{};
      sl.a.part_o = static_cast<uint16_t*>(workspace);
      sl.a.part_ml = reinterpret_cast<float*>(sl.a.part_o + pl.part_o_elems);
      sl.a.ctiles = pl.ctiles;
      sl.a.nchunk = pl.nchunk;
      std::copy(pl.bin_first.begin(), pl.bin_first.end(), sl.bin_first);
      std::copy(pl.items.begin(), pl.items.end(), sl.items);
      launch_bf16_attn_ks<D, HPW, CAUSAL, 1, true>(
          a, dim3(static_cast<uint32_t>(pl.n_bins * nhg)), npb, nhg, sl);
      attn_merge_kernel<D, HPW, CAUSAL>
          <<<dim3(static_cast<uint32_t>(pl.n_split_rows * (D / 32) * nhg)), dim3(256), 0, a.s>>>(
              sl.a, a.out, a.lse, a.N, a.Hq, npb, nhg, a.n_dyn);
      return;
    }
  }
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(npb) * nhg));
  // a head-dim 256 tile pair fills the LDS of a CU: one stream only
  if constexpr (D <= 128) {
    if (static_cast<int64_t>(grid.x) <= kTwoStreamMaxGrid) {
      launch_bf16_attn_ks<D, HPW, CAUSAL, 2, false>(a, grid, npb, nhg, none);
      return;
    }
    // large grids: 8-wave workgroups, two query blocks sharing each staged
    // key tile (half the staging work per wave at the same occupancy)
    constexpr int PB8 = 32 * (8 / HPW);
    const int32_t npb8 = (a.N + PB8 - 1) / PB8;
    launch_bf16_attn_ks<D, HPW, CAUSAL, 1, false, NoSplit, 8>(
        a, dim3(static_cast<uint32_t>(static_cast<int64_t>(npb8) * nhg)), npb8, nhg, none);
    return;
  }
  launch_bf16_attn_ks<D, HPW, CAUSAL, 1, false>(a, grid, npb, nhg, none);
}

template <int D, int HPW>
void launch_bf16_attn_c(const AttnArgs& a, const SplitPlan& pl, void* workspace) {
  if (a.causal)
    launch_bf16_attn<D, HPW, true>(a, pl, workspace);
  else
    launch_bf16_attn<D, HPW, false>(a, pl, workspace);
}

tg_status attn_fwd(tg_dtype dt, int64_t N, int64_t Hq, int64_t Hkv, int64_t D, const void* q,
                   const void* k, const void* v, const float* key_score, const float* gain,
                   const float* q_scale, float softmax_scale, int causal, void* out,
                   float* lse, void* workspace, size_t workspace_bytes, void* stream,
                   const int32_t* n_dyn) {
  if (dt != TG_DTYPE_F32 && dt != TG_DTYPE_BF16)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_bias_attn_fwd: unknown dtype %d", (int)dt);
  if (N < 0 || N > kMaxTokens || Hq < 1 || Hkv < 1 || Hq > 65536 || Hkv > 65536)
    return fail(TG_ERR_INVALID_ARGUMENT,
                "tg_bias_attn_fwd: need 0 <= N <= 2^31-1 and 1 <= Hkv, Hq (N=%lld Hq=%lld Hkv=%lld)",
                (long long)N, (long long)Hq, (long long)Hkv);
  if (Hq % Hkv != 0)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_bias_attn_fwd: Hq %% Hkv != 0 (%lld, %lld)",
                (long long)Hq, (long long)Hkv);
  if (D != 64 && D != 128 && D != 256)
    return fail(TG_ERR_UNSUPPORTED, "tg_bias_attn_fwd: head dim must be 64, 128 or 256 (D=%lld)",
                (long long)D);
  if (N * Hq > kMaxTokens)
    return fail(TG_ERR_UNSUPPORTED, "tg_bias_attn_fwd: N * Hq must fit in int32");
  if (dt == TG_DTYPE_BF16 && N * Hq * D * 2 > kMaxTokens)
    return fail(TG_ERR_UNSUPPORTED,
                "tg_bias_attn_fwd: bf16 path addresses Q/K/V with 32-bit offsets "
                "(N * Hq * D * 2 must be < 2^31)");
  static const SplitPlan kUnsplit;
  const std::shared_ptr<const SplitPlan> plan =
      dt == TG_DTYPE_BF16 ? split_plan(N, Hq, Hkv, D, causal != 0) : nullptr;
  const SplitPlan& pl = plan ? *plan : kUnsplit;
  if (workspace != nullptr) {
    if (!aligned(workspace, 16))
      return fail(TG_ERR_INVALID_ARGUMENT, "tg_bias_attn_fwd_ws: workspace must be 16-byte aligned");
    if (workspace_bytes < pl.bytes)
      return fail(TG_ERR_WORKSPACE, "tg_bias_attn_fwd_ws: workspace of %zu bytes, need %zu",
                  workspace_bytes, pl.bytes);
  }
  if (N == 0) {
    clear_error();
    return TG_OK;
  }
  if (!q || !k || !v || !out)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_bias_attn_fwd: NULL q/k/v/out");
  if (key_score && !gain)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_bias_attn_fwd: key_score given without gain");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_bias_attn_fwd: q/k/v/out must be 16-byte aligned");
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf(static_cast<float>(D));
  hipStream_t s = as_stream(stream);
  const int32_t n = static_cast<int32_t>(N), hq = static_cast<int32_t>(Hq),
                hkv = static_cast<int32_t>(Hkv);
  if (dt == TG_DTYPE_F32) {
    const int64_t threads = N * Hq;
    const dim3 grid(static_cast<uint32_t>((threads + 127) / 128));
    if (D == 64)
      attn_f32_kernel<64><<<grid, dim3(128), 0, s>>>(
          static_cast<const float*>(q), static_cast<const float*>(k),
          static_cast<const float*>(v), key_score, gain, q_scale, scale, causal ? 1 : 0,
          static_cast<float*>(out), lse, n, hq, hkv, n_dyn);
    else if (D == 256)
      attn_f32_kernel<256><<<grid, dim3(128), 0, s>>>(
          static_cast<const float*>(q), static_cast<const float*>(k),
          static_cast<const float*>(v), key_score, gain, q_scale, scale, causal ? 1 : 0,
          static_cast<float*>(out), lse, n, hq, hkv, n_dyn);
    else
      attn_f32_kernel<128><<<grid, dim3(128), 0, s>>>(
          static_cast<const float*>(q), static_cast<const float*>(k),
          static_cast<const float*>(v), key_score, gain, q_scale, scale, causal ? 1 : 0,
          static_cast<float*>(out), lse, n, hq, hkv, n_dyn);
    return check_launch("tg_bias_attn_fwd");
  }
  const int64_t G = Hq / Hkv;
  const int hpw = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  const AttnArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                   static_cast<const uint16_t*>(v), key_score, gain, q_scale, scale,
                   static_cast<uint16_t*>(out), lse, n, hq, hkv, causal != 0,
                   key_score != nullptr, q_scale != nullptr, s, n_dyn};
#define TG_ATTN_DISPATCH(DD, HH) launch_bf16_attn_c<DD, HH>(a, pl, workspace)
  if (D == 256) {
    if (hpw == 4) TG_ATTN_DISPATCH(256, 4);
    else if (hpw == 2) TG_ATTN_DISPATCH(256, 2);
    else TG_ATTN_DISPATCH(256, 1);
  } else if (D == 128) {
    if (hpw == 4) TG_ATTN_DISPATCH(128, 4);
    else if (hpw == 2) TG_ATTN_DISPATCH(128, 2);
    else TG_ATTN_DISPATCH(128, 1);
  } else {
    if (hpw == 4) TG_ATTN_DISPATCH(64, 4);
    else if (hpw == 2) TG_ATTN_DISPATCH(64, 2);
    else TG_ATTN_DISPATCH(64, 1);
  }
#undef TG_ATTN_DISPATCH
  return check_launch("tg_bias_attn_fwd");
}

}  // namespace

tg_status bias_attn_call(tg_dtype dt, int64_t N, int64_t Hq, int64_t Hkv, int64_t D,
                         const void* q, const void* k, const void* v, const float* key_score,
                         const float* gain, const float* q_scale, float softmax_scale,
                         int causal, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream, const int32_t* n_dyn) {
  return attn_fwd(dt, N, Hq, Hkv, D, q, k, v, key_score, gain, q_scale, softmax_scale, causal,
                  out, lse, workspace, workspace_bytes, stream, n_dyn);
}

}  // namespace tg

extern "C" tg_status tg_bias_attn_fwd(tg_dtype dt, int64_t N, int64_t Hq, int64_t Hkv,
                                      int64_t D, const void* q, const void* k, const void* v,
                                      const float* key_score, const float* gain,
                                      const float* q_scale, float softmax_scale, int causal,
                                      void* out, float* lse, void* stream) {
  return tg::bias_attn_call(dt, N, Hq, Hkv, D, q, k, v, key_score, gain, q_scale,
                            softmax_scale, causal, out, lse, nullptr, 0, stream, nullptr);
}

extern "C" size_t tg_bias_attn_workspace_size(tg_dtype dt, int64_t N, int64_t Hq, int64_t Hkv,
                                              int64_t D, int causal) {
  if (dt != TG_DTYPE_BF16 || N <= 0 || N > tg::kMaxTokens || Hq < 1 || Hkv < 1 ||
      Hq % Hkv != 0 || (D != 64 && D != 128 && D != 256) || N * Hq * D * 2 > tg::kMaxTokens)
    return 0;
  return tg::split_plan(N, Hq, Hkv, D, causal != 0)->bytes;
}

extern "C" tg_status tg_bias_attn_fwd_ws(tg_dtype dt, int64_t N, int64_t Hq, int64_t Hkv,
                                         int64_t D, const void* q, const void* k, const void* v,
                                         const float* key_score, const float* gain,
                                         const float* q_scale, float softmax_scale, int causal,
                                         void* out, float* lse, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  return tg::bias_attn_call(dt, N, Hq, Hkv, D, q, k, v, key_score, gain, q_scale,
                            softmax_scale, causal, out, lse, workspace, workspace_bytes, stream,
                            nullptr);
}
