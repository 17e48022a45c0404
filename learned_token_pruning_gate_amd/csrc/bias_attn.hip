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
//   * A workgroup (4 waves) owns one KV head and a block of query positions;
//     each wave owns 32 query positions of one query head, and the HPW query
//     heads of the group that share the KV head reuse every K/V tile staged
//     in LDS.
//   * Logits are computed transposed, S^T = K Q^T, on
//     v_mfma_f32_32x32x16_bf16: in the accumulator each lane holds one
//     query column and 16 keys of a 32-key block, so the running max and
//     sum of a query stay inside the lane (plus one exchange between the
//     two lane halves), and the probabilities P^T, converted to bf16 in
//     place, are exactly the B operand of the next product O^T += V^T P^T.
//     The keys that the accumulator layout puts in a lane's k-slots are
//     matched by reading V^T from LDS in the same order.
//   * Q stays in registers for the whole key loop.  K tiles are staged in
//     LDS row-major (padded); V tiles are transposed on their way into LDS
//     (4 keys x 8 dims per thread, packed with byte permutes), the keys of
//     every 16-key PV step stored in the order the P^T accumulator holds
//     them, so each lane's V^T operand is one 16-byte read.  The next tile's
//     global loads are issued before the current tile's math.
//   * The two 32-key halves of a tile's logits are independent accumulation
//     chains, interleaved so no MFMA waits on its own predecessor.
//   * Key streams: when the grid is small (short prompts, where the longest
//     causal rows set the time), a workgroup runs two streams of 4 waves on
//     the even and odd key tiles, each with its own LDS buffers, and merges
//     their softmax states at the end; each wave's serial loop halves and
//     two waves share every SIMD.
//   * The bias gain_h*log2(e)*score_c is formed once per key tile and head
//     in LDS; logits use exp2 with log2(e) folded into the scale; the output
//     is rescaled only when some query's running max grows.
//   * Workgroups are ordered longest-first (causal) and the KV head is the
//     fastest-varying index, so consecutive workgroups -- which the
//     dispatcher spreads over the 8 XCDs -- keep one KV head per XCD L2.
//
// f32 path: one thread per (query, head), fp32 online softmax.
#include "tg_common.hpp"

namespace tg {
namespace {

constexpr int kBK = 64;           // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Slot of the 4-key group g (0..3) of a 16-key PV k-step in V^T: lane half
// hh reads slots 8hh..8hh+7, which must hold keys 4hh..4hh+3 and 8+4hh..8+4hh+3
// (the order the P^T accumulator holds them in).
__device__ __forceinline__ int vgroup_slot(int g) { return ((g & 1) << 1) | (g >> 1); }

template <int D>
struct AttnSmem {
  static constexpr int KP = D + 8;          // K row pitch (bf16)
  static constexpr int VP = kBK + 8;        // V^T row pitch (bf16)
  uint16_t ks[kBK * KP];                    // K tile, row-major [key][dim]
  uint16_t vt[D * VP];                      // V tile transposed [dim][key slot]
  u32x2 bias[4][kBK];                       // per head: bf16 (hi | mid << 16, lo)
};

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}
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

// The bias enters the MFMA as three bf16 terms hi + mid + lo, which carry a
// fp32 value to within 2^-25 of itself: (hi | mid << 16, lo).
__device__ __forceinline__ u32x2 split_bf16_triple(float v) {
  const uint32_t hi = bf16_bits(v);
  const float r1 = v - bf16_val(hi);
  const uint32_t mid = bf16_bits(r1);
  const uint32_t lo = bf16_bits(r1 - bf16_val(mid));
  return u32x2{hi | (mid << 16), lo};
}

template <int D, int HPW, int KS, bool CAUSAL, bool HAS_BIAS, bool HAS_QSCALE>
__global__ __launch_bounds__(256 * KS, (KS == 1 && D <= 128) ? 2 : 1) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ key_score,
    const float* __restrict__ gain, const float* __restrict__ q_scale, float scale,
    uint16_t* __restrict__ out, float* __restrict__ lse, int32_t N, int32_t Hq, int32_t Hkv,
    int32_t n_pblocks, int32_t n_hgroups) {
  constexpr int PB = 32 * (4 / HPW);        // query positions per workgroup
  constexpr int DK = D / 16;                // k-steps of S^T = K Q^T (plus one extra)
  constexpr int DB = D / 32;                // 32-row blocks of O^T
  constexpr int CPR = D / 8;                // 16-byte chunks per K/V row
  constexpr int KRPI = 256 / CPR;           // K rows staged per pass
  constexpr int KI = kBK / KRPI;            // K staging passes
  constexpr int VT = (kBK / 4) * CPR;       // (4 keys x 8 dims) pieces of a V tile
  constexpr int VPC = (VT + 255) / 256;     // V pieces per staging thread
  // KS key streams: stream kh (waves 4kh .. 4kh+3, threads 256kh ..) takes
  // key tiles kh, kh + KS, kh + 2KS, ... with its own LDS buffers; the
  // streams' partial softmax states are merged at the end
  __shared__ __attribute__((aligned(16))) AttnSmem<D> sm[2][KS];

  const int tid = threadIdx.x & 255;        // thread index within the key stream
  const int kh = threadIdx.x >> 8;          // key stream
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;                 // which half of the wave

  const int hg = blockIdx.x % n_hgroups;
  const int prank = blockIdx.x / n_hgroups;
  const int pblock = CAUSAL ? n_pblocks - 1 - prank : prank;
  const int G = Hq / Hkv;
  const int hw = wave % HPW;
  const int head = hg * HPW + hw;
  const int kvh = (hg * HPW) / G;
  const int pos0 = pblock * PB + 32 * (wave / HPW);
  const int my_q = pos0 + l32;
  const bool q_ok = my_q < N;

  const uint32_t q_row = static_cast<uint32_t>(Hq) * D * 2;     // bytes per token
  const uint32_t kv_row = static_cast<uint32_t>(Hkv) * D * 2;
  const __amdgpu_buffer_rsrc_t q_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(q), 0, static_cast<int>(static_cast<uint32_t>(N) * q_row), 0x00020000);
  const __amdgpu_buffer_rsrc_t k_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(k), 0, static_cast<int>(static_cast<uint32_t>(N) * kv_row), 0x00020000);
  const __amdgpu_buffer_rsrc_t v_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(v), 0, static_cast<int>(static_cast<uint32_t>(N) * kv_row), 0x00020000);

  // y = ac * (<q, k> + bias'_k), with ac = scale * log2(e) * c_r and the
  // per-key bias'_k = gain * score_k / scale in dot-product units.
  const float cr = HAS_QSCALE ? (q_ok ? q_scale[my_q] : 1.0f) : 1.0f;
  const float ac = scale * kLog2e * cr;

  // Q^T as MFMA B operand (exact bf16): lane (query l32, half hh) holds dims
  // 16 ks + 8 hh .. +7.  k-step DK is the extra one: [1, 1, 1, 0...] in the
  // hh = 0 half, matched on the key side by [bias'_hi, bias'_mid, bias'_lo,
  // 0...], so the MFMA adds the gate bias to every logit.
  bf16x8 qf[DK + 1];
  {
    const uint32_t base = static_cast<uint32_t>(my_q) * q_row +
                          static_cast<uint32_t>(head) * D * 2 + 16u * hh;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8,
                                  __builtin_amdgcn_raw_buffer_load_b128(q_rs, base + 32u * ks, 0, 0));
  }
  qf[DK] = __builtin_bit_cast(bf16x8, hh == 0 ? u32x4{0x3F803F80u, 0x3F80u, 0, 0}
                                              : u32x4{0, 0, 0, 0});
  float m_run = -INFINITY;  // running max of y over visible keys (log2 units)

  const int wg_end = CAUSAL ? min((pblock + 1) * PB, N) : N;
  const int n_tiles = (wg_end + kBK - 1) / kBK;
  const int lim = CAUSAL ? min(my_q, N - 1) : N - 1;   // last visible key

  // ---- staging roles ------------------------------------------------------
  const int krow = tid / CPR, kchunk = tid % CPR;          // K: row-major copy
  // V: piece tid + 256 pc is keys 4 vkg .. +3 of dims 8 vdc .. +7, with
  // vkg = piece % 16 and vdc = piece / 16
  const float inv_scale = 1.0f / scale;
  // A -inf score becomes a bias of -2^21 log2 units (in dot-product units):
  // for any per-query scale >= 0.25 the logit falls below kMaskedLog2 and its
  // weight underflows to exactly 0, as deleting the key would give.
  const float masked_bias = -2097152.0f * inv_scale / kLog2e;
  u32x4 kreg[KI], vreg[VPC][4];
  float sreg = 0.0f;        // staged raw score (its bias is formed at store time)
  const int bias_key = tid % kBK;
  const float bias_gain = (HAS_BIAS && tid < HPW * kBK) ? gain[hg * HPW + tid / kBK] : 0.0f;
  const __amdgpu_buffer_rsrc_t s_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(key_score), 0, HAS_BIAS ? N * 4 : 0, 0x00020000);
  auto load_tile = [&](int t) {
    const int k0 = t * kBK;
    const uint32_t hoff = static_cast<uint32_t>(kvh) * D * 2;
#pragma unroll
    for (int i = 0; i < KI; ++i)
      kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(
          k_rs, static_cast<uint32_t>(k0 + krow + KRPI * i) * kv_row + hoff + 16u * kchunk, 0, 0);
#pragma unroll
    for (int pc = 0; pc < VPC; ++pc) {
      const int piece = tid + 256 * pc;
      const int vkg = piece % (kBK / 4), vdc = piece / (kBK / 4);
      if (piece < VT) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          vreg[pc][j] = __builtin_amdgcn_raw_buffer_load_b128(
              v_rs, static_cast<uint32_t>(k0 + 4 * vkg + j) * kv_row + hoff + 16u * vdc, 0, 0);
      }
    }
    if (HAS_BIAS && tid < HPW * kBK)   // keys past N read 0
      sreg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           s_rs, 4u * static_cast<uint32_t>(k0 + bias_key), 0, 0));
  };
  auto store_tile = [&](AttnSmem<D>& b) {
#pragma unroll
    for (int i = 0; i < KI; ++i)
      *reinterpret_cast<u32x4*>(&b.ks[(krow + KRPI * i) * AttnSmem<D>::KP + 8 * kchunk]) = kreg[i];
#pragma unroll
    for (int pc = 0; pc < VPC; ++pc) {
      const int piece = tid + 256 * pc;
      const int vkg = piece % (kBK / 4), vdc = piece / (kBK / 4);
      if (piece < VT) {
        // keys 4 vkg .. 4 vkg + 3 go to the slots the PV k-step reads them from
        const int vslot = 16 * (vkg >> 2) + 4 * vgroup_slot(vkg & 3);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // dims 8 vdc + 2w (low halves) and 8 vdc + 2w + 1 (high halves)
          u32x2 lo, hi;
          lo[0] = pack_lo(vreg[pc][0][w], vreg[pc][1][w]);
          lo[1] = pack_lo(vreg[pc][2][w], vreg[pc][3][w]);
          hi[0] = pack_hi(vreg[pc][0][w], vreg[pc][1][w]);
          hi[1] = pack_hi(vreg[pc][2][w], vreg[pc][3][w]);
          *reinterpret_cast<u32x2*>(&b.vt[(8 * vdc + 2 * w) * AttnSmem<D>::VP + vslot]) = lo;
          *reinterpret_cast<u32x2*>(&b.vt[(8 * vdc + 2 * w + 1) * AttnSmem<D>::VP + vslot]) = hi;
        }
      }
    }
    if (HAS_BIAS && tid < HPW * kBK)
      b.bias[tid / kBK][bias_key] = split_bf16_triple(
          sreg == -INFINITY ? masked_bias : bias_gain * sreg * inv_scale);
  };

  // ---- running state --------------------------------------------------------
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float l_run = 0.0f;       // this lane's share of the running sum of 2^y

  if (kh < n_tiles) {
    load_tile(kh);
    store_tile(sm[0][kh]);
  }
  __syncthreads();

  const int n_rounds = (n_tiles + KS - 1) / KS;
  for (int j = 0; j < n_rounds; ++j) {
    const int t = KS * j + kh;               // this stream's tile
    const AttnSmem<D>& b = sm[j & 1][kh];
    const int k0 = t * kBK;
    const bool more = t + KS < n_tiles;
    if (more) load_tile(t + KS);
    // keep the next tile's loads issued here, ahead of this tile's math
    __builtin_amdgcn_sched_barrier(0);
    if (KS == 1 || t < n_tiles) {   // uniform per wave: a stream may idle in the last round

    // S'^T = K' Q'^T = <q, k> + bias'; the two 32-key halves are independent
    // accumulation chains, interleaved so neither waits on its own last MFMA
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            &b.ks[(32 * kb + l32) * AttnSmem<D>::KP + 8 * hh + 16 * ks]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
      }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u32x4 ke = u32x4{0, 0, 0, 0};
      if (hh == 0) {
        const u32x2 bb = HAS_BIAS ? b.bias[hw][32 * kb + l32] : u32x2{0, 0};
        ke[0] = bb[0];                     // [bias'_hi, bias'_mid]
        ke[1] = bb[1];                     // [bias'_lo, 0]
      }
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ke), qf[DK],
                                                      s[kb], 0, 0, 0);
    }

    // causal / tail mask (only tiles that reach past a query or past N)
    const bool need_mask = (CAUSAL && k0 + kBK - 1 > pos0) || (k0 + kBK > N);
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

    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) tmax = fmaxf(tmax, fmaxf(s[kb][r], s[kb][r + 1]));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));

    // running max in log2 units (ac > 0 keeps the arg-max); maxima below
    // kMaskedLog2 are masked keys only
    float tm = tmax * ac;
    tm = tm > kMaskedLog2 ? tm : -INFINITY;
    const float m_new = fmaxf(m_run, tm);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    if (__any(m_new > m_run)) {
      // 0 when nothing was accumulated yet
      const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_use);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      l_run *= alpha;
    }
    m_run = m_new;

    // P^T = 2^(y - m) as bf16, already laid out as the PV B operand; the row
    // maximum gets weight exactly 1
    bf16x8 p[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hf + i], ac, -m_use));
          l_run += e;
          p[kb][hf][i] = static_cast<__bf16>(e);
        }

    // O^T += V^T P^T: k-step (kb, hf) covers keys 32kb + 16hf + {4hh..4hh+3,
    // 8+4hh..8+4hh+3}, stored at slots 32kb + 16hf + 8hh .. +7: one 16-byte read
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x4 a4 = *reinterpret_cast<const u32x4*>(
              &b.vt[(32 * db + l32) * AttnSmem<D>::VP + 32 * kb + 16 * hf + 8 * hh]);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4),
                                                          p[kb][hf], o[db], 0, 0, 0);
        }
      }
    }

    }
    if (more) store_tile(sm[(j + 1) & 1][kh]);
    __syncthreads();
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
  const bool empty = !(l_tot > 0.0f) || m_run == -INFINITY;  // no visible key
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
}

// ---------------------------------------------------------------------------
// fp32 path: one thread per (query row, query head), online softmax in fp32.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ key_score, const float* __restrict__ gain,
    const float* __restrict__ q_scale, float scale, int causal, float* __restrict__ out,
    float* __restrict__ lse, int32_t N, int32_t Hq, int32_t Hkv) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(N) * Hq) return;
  const int r = static_cast<int>(idx / Hq);
  const int h = static_cast<int>(idx % Hq);
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
  const int nk = causal ? r + 1 : N;
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
constexpr int64_t kTwoStreamMaxGrid = 1024;

template <int D, int HPW, bool CAUSAL, int KS>
void launch_bf16_attn_ks(bool has_bias, bool has_qs, dim3 grid, hipStream_t s,
                      const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const float* ks, const float* gain, const float* qs, float scale_log2,
                      uint16_t* out, float* lse, int32_t N, int32_t Hq, int32_t Hkv,
                      int32_t npb, int32_t nhg) {
#define TG_ATTN_LAUNCH(B, Q)                                                         \
  attn_bf16_kernel<D, HPW, KS, CAUSAL, B, Q><<<grid, dim3(256 * KS), 0, s>>>(        \
      q, k, v, ks, gain, qs, scale_log2, out, lse, N, Hq, Hkv, npb, nhg)
  if (has_bias) {
    if (has_qs) TG_ATTN_LAUNCH(true, true); else TG_ATTN_LAUNCH(true, false);
  } else {
    if (has_qs) TG_ATTN_LAUNCH(false, true); else TG_ATTN_LAUNCH(false, false);
  }
#undef TG_ATTN_LAUNCH
}

template <int D, int HPW, bool CAUSAL>
void launch_bf16_attn(bool has_bias, bool has_qs, dim3 grid, hipStream_t s,
                      const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const float* ks, const float* gain, const float* qs, float scale_log2,
                      uint16_t* out, float* lse, int32_t N, int32_t Hq, int32_t Hkv,
                      int32_t npb, int32_t nhg) {
  // a head-dim 256 tile pair fills the LDS of a CU: one stream only
  if constexpr (D <= 128) {
    if (static_cast<int64_t>(grid.x) <= kTwoStreamMaxGrid) {
      launch_bf16_attn_ks<D, HPW, CAUSAL, 2>(has_bias, has_qs, grid, s, q, k, v, ks, gain, qs,
                                             scale_log2, out, lse, N, Hq, Hkv, npb, nhg);
      return;
    }
  }
    launch_bf16_attn_ks<D, HPW, CAUSAL, 1>(has_bias, has_qs, grid, s, q, k, v, ks, gain, qs,
                                           scale_log2, out, lse, N, Hq, Hkv, npb, nhg);
}

template <int D, int HPW>
void launch_bf16_attn_c(bool causal, bool has_bias, bool has_qs, int32_t N, int32_t Hq,
                        int32_t Hkv, hipStream_t s, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const float* ks, const float* gain,
                        const float* qs, float scale_log2, uint16_t* out, float* lse) {
  constexpr int PB = 32 * (4 / HPW);
  const int32_t npb = (N + PB - 1) / PB;
  const int32_t nhg = Hq / HPW;
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(npb) * nhg));
  if (causal)
    launch_bf16_attn<D, HPW, true>(has_bias, has_qs, grid, s, q, k, v, ks, gain, qs,
                                   scale_log2, out, lse, N, Hq, Hkv, npb, nhg);
  else
    launch_bf16_attn<D, HPW, false>(has_bias, has_qs, grid, s, q, k, v, ks, gain, qs,
                                    scale_log2, out, lse, N, Hq, Hkv, npb, nhg);
}

}  // namespace
}  // namespace tg

extern "C" tg_status tg_bias_attn_fwd(tg_dtype dt, int64_t N, int64_t Hq, int64_t Hkv,
                                      int64_t D, const void* q, const void* k, const void* v,
                                      const float* key_score, const float* gain,
                                      const float* q_scale, float softmax_scale, int causal,
                                      void* out, float* lse, void* stream) {
  using namespace tg;
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
          static_cast<float*>(out), lse, n, hq, hkv);
    else if (D == 256)
      attn_f32_kernel<256><<<grid, dim3(128), 0, s>>>(
          static_cast<const float*>(q), static_cast<const float*>(k),
          static_cast<const float*>(v), key_score, gain, q_scale, scale, causal ? 1 : 0,
          static_cast<float*>(out), lse, n, hq, hkv);
    else
      attn_f32_kernel<128><<<grid, dim3(128), 0, s>>>(
          static_cast<const float*>(q), static_cast<const float*>(k),
          static_cast<const float*>(v), key_score, gain, q_scale, scale, causal ? 1 : 0,
          static_cast<float*>(out), lse, n, hq, hkv);
    return check_launch("tg_bias_attn_fwd");
  }
  const int64_t G = Hq / Hkv;
  const int hpw = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  const auto* qb = static_cast<const uint16_t*>(q);
  const auto* kb = static_cast<const uint16_t*>(k);
  const auto* vb = static_cast<const uint16_t*>(v);
  auto* ob = static_cast<uint16_t*>(out);
  const float sl2 = scale;
  const bool cz = causal != 0, hb = key_score != nullptr, hs = q_scale != nullptr;
#define TG_ATTN_DISPATCH(DD, HH) \
  launch_bf16_attn_c<DD, HH>(cz, hb, hs, n, hq, hkv, s, qb, kb, vb, key_score, gain, q_scale, sl2, ob, lse)
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
