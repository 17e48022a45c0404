// bias_attn_bwd.hip -- token-gated attention backward: the gradients of the
// forward of bias_attn.hip with respect to Q, K, V, the key scores and the
// per-head gains.
//
// TokenGate pages: ai.info summary "Key Contributions" items 2 and 3 (the
// gate is trained end to end: its scores reach the loss only through the
// per-key attention bias gain_h * score_k, so training the gate needs the
// gradient of the biased attention with respect to the scores and gains).
//
// With z[r,c] = c_r (alpha <q_r, k_c> + g_h s_c), P = softmax_c(z),
// O = P V and an upstream gradient dO:
//   dP = dO V^T,  Delta_r = <dO_r, O_r>,  dZ = P (dP - Delta)
//   dQ = (c alpha dZ) K,  dK = (c alpha dZ)^T Q,  dV = P^T dO
//   dscore_c = sum_h g_h A[h,c],  dgain_h = sum_c s_c A[h,c],
//   A[h,c] = sum_r c_r dZ[h,r,c]
// P is recomputed from the forward's log-sum-exp.  Four kernels:
//   * attn_bwd_pre_kernel: Delta and the log-sum-exp in log2 units;
//   * attn_bwd_dq_kernel: query-parallel, the forward's layout (S^T = K Q^T
//     with one query per lane), plus dP^T = V dO^T and dQ^T += K^T dZ^T
//     with K also staged transposed;
//   * attn_bwd_dkdv_kernel: key-parallel, logits oriented S = Q K^T so that
//     each lane holds one key; Q^T and dO^T are staged transposed (in the
//     key-slot order of the forward's V^T) as A operands of dK^T += Q^T dZ
//     and dV^T += dO^T P, and A[h,c] is summed per lane;
//   * attn_bwd_reduce_kernel: the dscore and dgain partials, summed in a
//     fixed order (deterministic).
// bf16 inputs on v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and dZ
// are rounded to bf16 only as operands of the dV, dK and dQ products.
#include <algorithm>
#include <type_traits>

#include "tg_common.hpp"

namespace tg {
namespace {

constexpr int kTile = 64;          // keys per tile (dQ), queries per tile (dK/dV)
constexpr int kKeysPerWg = 128;    // dK/dV: 4 waves x 32 keys
constexpr int kMaxKvChunks = 8;    // dK/dV query chunks per key block, at most
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int slot_of_group(int g) { return ((g & 1) << 1) | (g >> 1); }
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}
__device__ __forceinline__ uint32_t to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ float from_bf16_bits(uint32_t bits) {
  return __uint_as_float(bits << 16);
}
// fp32 value as three bf16 terms (hi | mid << 16, lo), within 2^-25 of it.
__device__ __forceinline__ u32x2 bf16_triple(float x) {
  const uint32_t hi = to_bf16_bits(x);
  const float r1 = x - from_bf16_bits(hi);
  const uint32_t mid = to_bf16_bits(r1);
  const uint32_t lo = to_bf16_bits(r1 - from_bf16_bits(mid));
  return u32x2{hi | (mid << 16), lo};
}

// A tile of 64 rows of one head, [row][dim] (padded), and the same tile
// transposed, [dim][row slot]: the rows of each 16-row MFMA k-step stored in
// the order the 32x32 accumulator holds them, so each lane's operand (8 rows
// at one dim) is one 16-byte read.
template <int D>
struct RowTile {
  static constexpr int P = D + 8;
  uint16_t a[kTile * P];
};
template <int D>
struct TrTile {
  static constexpr int P = kTile + 8;
  uint16_t a[D * P];
};

// Staging of a 64-row tile of a [rows][H][D] bf16 tensor by 256 threads:
// row-major as 16-byte chunks, or transposed as (4 rows x 8 dims) pieces.
template <int D>
struct Stage {
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int RPI = 256 / CPR;          // rows per pass
  static constexpr int RI = kTile / RPI;         // row-major passes
  static constexpr int PIECES = (kTile / 4) * CPR;
  static constexpr int PPT = (PIECES + 255) / 256;   // pieces per thread

  __device__ static void load_rows(u32x4 (&r)[RI], __amdgpu_buffer_rsrc_t rs, uint32_t row_bytes,
                                   uint32_t hoff, int row0, int tid) {
#pragma unroll
    for (int i = 0; i < RI; ++i)
      r[i] = __builtin_amdgcn_raw_buffer_load_b128(
          rs, static_cast<uint32_t>(row0 + tid / CPR + RPI * i) * row_bytes + hoff +
                  16u * (tid % CPR),
          0, 0);
  }
  __device__ static void store_rows(RowTile<D>& t, const u32x4 (&r)[RI], int tid) {
#pragma unroll
    for (int i = 0; i < RI; ++i)
      *reinterpret_cast<u32x4*>(&t.a[(tid / CPR + RPI * i) * RowTile<D>::P + 8 * (tid % CPR)]) =
          r[i];
  }
  __device__ static void load_pieces(u32x4 (&r)[PPT][4], __amdgpu_buffer_rsrc_t rs,
                                     uint32_t row_bytes, uint32_t hoff, int row0, int tid) {
#pragma unroll
    for (int pc = 0; pc < PPT; ++pc) {
      const int piece = tid + 256 * pc;
      if (piece < PIECES) {
        const int rg = piece % (kTile / 4), dc = piece / (kTile / 4);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          r[pc][j] = __builtin_amdgcn_raw_buffer_load_b128(
              rs, static_cast<uint32_t>(row0 + 4 * rg + j) * row_bytes + hoff + 16u * dc, 0, 0);
      }
    }
  }
  __device__ static void store_pieces(TrTile<D>& t, const u32x4 (&r)[PPT][4], int tid) {
#pragma unroll
    for (int pc = 0; pc < PPT; ++pc) {
      const int piece = tid + 256 * pc;
      if (piece < PIECES) {
        const int rg = piece % (kTile / 4), dc = piece / (kTile / 4);
        const int slot = 16 * (rg >> 2) + 4 * slot_of_group(rg & 3);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          u32x2 lo, hi;
          lo[0] = lo_halves(r[pc][0][w], r[pc][1][w]);
          lo[1] = lo_halves(r[pc][2][w], r[pc][3][w]);
          hi[0] = hi_halves(r[pc][0][w], r[pc][1][w]);
          hi[1] = hi_halves(r[pc][2][w], r[pc][3][w]);
          *reinterpret_cast<u32x2*>(&t.a[(8 * dc + 2 * w) * TrTile<D>::P + slot]) = lo;
          *reinterpret_cast<u32x2*>(&t.a[(8 * dc + 2 * w + 1) * TrTile<D>::P + slot]) = hi;
        }
      }
    }
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes),
                                           0x00020000);
}

// ---------------------------------------------------------------------------
// Delta[h][r] = <dO[r,h,:], O[r,h,:]> and lse2[h][r] = lse[h][r] * log2(e);
// a row with no visible key (lse = -inf) gets lse2 = +inf, so that every
// recomputed weight 2^(y - lse2) is 0.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(const uint16_t* __restrict__ out,
                                                           const uint16_t* __restrict__ dout,
                                                           const float* __restrict__ lse,
                                                           float* __restrict__ delta,
                                                           float* __restrict__ lse2, int32_t N,
                                                           int32_t Hq) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(N) * Hq) return;
  const int64_t r = i / Hq, h = i - r * Hq;   // i = r * Hq + h: the [N][Hq][D] row
  const u32x4* o = reinterpret_cast<const u32x4*>(out + i * D);
  const u32x4* d = reinterpret_cast<const u32x4*>(dout + i * D);
  float acc = 0.0f;
#pragma unroll 4
  for (int c = 0; c < D / 8; ++c) {
    const u32x4 a = o[c], b = d[c];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(__uint_as_float(a[w] << 16), __uint_as_float(b[w] << 16), acc);
      acc = fmaf(__uint_as_float(a[w] & 0xffff0000u), __uint_as_float(b[w] & 0xffff0000u), acc);
    }
  }
  const float l = lse[h * N + r];
  delta[h * N + r] = acc;
  lse2[h * N + r] = l == -INFINITY ? INFINITY : l * kLog2e;
}

// ---------------------------------------------------------------------------
// dQ: a workgroup (4 waves) owns one KV head and a block of queries, each
// wave 32 queries of one head (HPW heads of the group share the K/V tiles),
// and walks the key tiles of its rows.  Per 64-key tile:
//   S^T = K Q^T (+ bias k-step)   dP^T = V dO^T   (one query per lane)
//   dZ'^T = 2^(y - lse2) (dP^T - Delta) c alpha  -> bf16 B operand
//   dQ^T += K^T dZ'^T             (K^T staged transposed)
// ---------------------------------------------------------------------------
// The row tiles (S^T and dP^T operands, all D dims) and the transposed K
// tile (dQ^T operand, the DO output dims).  With DO < D (head dim 256) a
// launch produces the output dims [dof, dof + DO) of dQ and recomputes S
// and dP over all D; its row tiles are single-buffered (two buffers of them
// would not fit the LDS) and the next tile's rows are stored once every wave
// has finished the current tile's S and dP.
template <int D>
struct DqRows {
  RowTile<D> k, v;
  u32x2 bias[4][kTile];
};
template <int DO>
struct DqTr {
  TrTile<DO> kt;
};

template <int D, int DO, int HPW, bool CAUSAL, bool HAS_BIAS, bool HAS_QSCALE>
__global__ __launch_bounds__(256, 1) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ key_score,
    const float* __restrict__ gain, const float* __restrict__ q_scale, float scale,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse2,
    const float* __restrict__ delta, uint16_t* __restrict__ dq, int32_t N, int32_t Hq,
    int32_t Hkv, int32_t n_pblocks, int32_t n_hgroups, int32_t dof) {
  using St = Stage<D>;
  using So = Stage<DO>;
  constexpr int PB = 32 * (4 / HPW);
  constexpr int DK = D / 16;
  constexpr int DB = DO / 32;
  constexpr int RB = DO == D ? 2 : 1;   // row-tile buffers
  __shared__ __attribute__((aligned(16))) DqRows<D> rows[RB];
  __shared__ __attribute__((aligned(16))) DqTr<DO> trs[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
  const int hg = blockIdx.x % n_hgroups;
  const int prank = blockIdx.x / n_hgroups;
  const int pblock = CAUSAL ? n_pblocks - 1 - prank : prank;
  const int G = Hq / Hkv;
  const int hw = wave % HPW;
  const int head = hg * HPW + hw;
  const int kvh = (hg * HPW) / G;
  const int pos0 = pblock * PB + 32 * (wave / HPW);   // the wave's first query
  const int my_q = pos0 + l32;
  const bool q_ok = my_q < N;

  const uint32_t q_row = static_cast<uint32_t>(Hq) * D * 2;
  const uint32_t kv_row = static_cast<uint32_t>(Hkv) * D * 2;
  const auto q_rs = rsrc(q, static_cast<uint32_t>(N) * q_row);
  const auto d_rs = rsrc(dout, static_cast<uint32_t>(N) * q_row);
  const auto k_rs = rsrc(k, static_cast<uint32_t>(N) * kv_row);
  const auto v_rs = rsrc(v, static_cast<uint32_t>(N) * kv_row);
  const auto s_rs = rsrc(key_score, HAS_BIAS ? static_cast<uint32_t>(N) * 4 : 0);

  const float cr = HAS_QSCALE ? (q_ok ? q_scale[my_q] : 1.0f) : 1.0f;
  const float ac = scale * kLog2e * cr;   // y = ac * (<q,k> + bias')
  const float zs = scale * cr;            // dZ' = dZ c alpha
  const float l2q = q_ok ? lse2[static_cast<int64_t>(head) * N + my_q] : INFINITY;
  const float dlq = q_ok ? delta[static_cast<int64_t>(head) * N + my_q] : 0.0f;
  // P zs = 2^(y - lse2 + log2 zs): the factor zs rides in the exponent
  const float l2z = l2q - __builtin_log2f(zs);

  bf16x8 qf[DK + 1], df[DK];
  {
    const uint32_t base = static_cast<uint32_t>(my_q) * q_row +
                          static_cast<uint32_t>(head) * D * 2 + 16u * hh;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(q_rs, base + 32u * ks, 0, 0));
      df[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(d_rs, base + 32u * ks, 0, 0));
    }
  }
  qf[DK] = __builtin_bit_cast(bf16x8, hh == 0 ? u32x4{0x3F803F80u, 0x3F80u, 0, 0}
                                              : u32x4{0, 0, 0, 0});

  const float inv_scale = 1.0f / scale;
  // a -inf score: -2^100 in dot-product units absorbs any finite dot product,
  // and its weight underflows to exactly 0 whenever scale * c_r > 2^-80
  const float masked_bias = -0x1p100f;
  const int bias_key = tid % kTile;
  const float bias_gain = (HAS_BIAS && tid < HPW * kTile) ? gain[hg * HPW + tid / kTile] : 0.0f;
  const uint32_t hoff = static_cast<uint32_t>(kvh) * D * 2;

  u32x4 kr[St::RI], vr[St::RI], kp[So::PPT][4];
  float sreg = 0.0f;
  auto load_tile = [&](int t) {
    const int k0 = t * kTile;
    St::load_rows(kr, k_rs, kv_row, hoff, k0, tid);
    St::load_rows(vr, v_rs, kv_row, hoff, k0, tid);
    So::load_pieces(kp, k_rs, kv_row, hoff + 2u * static_cast<uint32_t>(dof), k0, tid);
    if (HAS_BIAS && tid < HPW * kTile)
      sreg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           s_rs, 4u * static_cast<uint32_t>(k0 + bias_key), 0, 0));
  };
  auto store_rows = [&](DqRows<D>& b) {
    St::store_rows(b.k, kr, tid);
    St::store_rows(b.v, vr, tid);
    if (HAS_BIAS && tid < HPW * kTile)
      b.bias[tid / kTile][bias_key] =
          bf16_triple(sreg == -INFINITY ? masked_bias : bias_gain * sreg * inv_scale);
  };
  auto store_tr = [&](DqTr<DO>& b) { So::store_pieces(b.kt, kp, tid); };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

  const int row_end = CAUSAL ? min((pblock + 1) * PB, N) : N;
  const int n_tiles = (row_end + kTile - 1) / kTile;
  const int lim = CAUSAL ? min(my_q, N - 1) : N - 1;
  load_tile(0);
  store_rows(rows[0]);
  store_tr(trs[0]);
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const DqRows<D>& b = rows[RB == 2 ? (t & 1) : 0];
    const DqTr<DO>& bt = trs[t & 1];
    const int k0 = t * kTile;
    const bool more = t + 1 < n_tiles;
    if (more) load_tile(t + 1);
    __builtin_amdgcn_sched_barrier(0);

    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = dp[kb][r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int off = (32 * kb + l32) * RowTile<D>::P + 8 * hh + 16 * ks;
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&b.k.a[off]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s[kb], 0, 0, 0);
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(&b.v.a[off]);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, df[ks], dp[kb], 0, 0, 0);
      }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u32x4 ke = u32x4{0, 0, 0, 0};
      if (hh == 0 && HAS_BIAS) {
        const u32x2 bb = b.bias[hw][32 * kb + l32];
        ke[0] = bb[0];
        ke[1] = bb[1];
      }
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ke), qf[DK],
                                                      s[kb], 0, 0, 0);
    }
    if constexpr (RB == 1) {   // every wave is done with this tile's rows
      __syncthreads();
      if (more) store_rows(rows[0]);
    }
    // weights, masked where the key is past the query or past N; a tile
    // whose last key (k0 + 63) no lane of the wave passes needs no mask
    const int rel = lim - k0 - 4 * hh;   // key k0 + 4hh + c visible iff c <= rel
    const bool full = k0 + kTile - 1 <= (CAUSAL ? min(pos0, N - 1) : N - 1);   // wave-uniform
    bf16x8 zb[2][2];
    auto weights = [&](const bool masked) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int r = 8 * hf + i;
            const int c = 32 * kb + 8 * (r >> 2) + (r & 3);
            const float pz = __builtin_amdgcn_exp2f(fmaf(s[kb][r], ac, -l2z));   // P zs
            zb[kb][hf][i] = static_cast<__bf16>((masked && c > rel) ? 0.0f : pz * (dp[kb][r] - dlq));
          }
    };
    if (full) weights(false); else weights(true);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x4 a4 = *reinterpret_cast<const u32x4*>(
              &bt.kt.a[(32 * db + l32) * TrTile<DO>::P + 32 * kb + 16 * hf + 8 * hh]);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4),
                                                            zb[kb][hf], acc[db], 0, 0, 0);
        }
    if (more) {
      if constexpr (RB == 2) store_rows(rows[(t + 1) & 1]);
      store_tr(trs[(t + 1) & 1]);
    }
    __syncthreads();
  }
  if (q_ok) {
    uint16_t* op = dq + static_cast<int64_t>(my_q) * Hq * D + static_cast<int64_t>(head) * D + dof;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = static_cast<__bf16>(acc[db][4 * j + i]);
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * j + 4 * hh) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV: a workgroup owns 128 keys of one KV head (4 waves x 32 keys, K and
// V fragments in registers as B operands) and walks, for each query head of
// the group, the 64-query tiles that see its keys.  Per tile:
//   S = Q K^T (+ bias k-step)   dP = dO V^T   (one key per lane)
//   P = 2^(y - lse2),  dZ = P (dP - Delta),  A += c dZ (per lane)
//   dV^T += dO^T P,  dK^T += Q^T (c alpha dZ)
// ---------------------------------------------------------------------------
// As in the dQ kernel, a launch with DO < D (head dim 256) produces the
// output dims [dof, dof + DO) of dK and dV, recomputing S and dP over all D.
// There the row tiles are single-buffered and filled by direct-to-LDS loads
// (no registers: the K and V fragments already take half the register
// file), unpadded with the 16-byte chunk c of row r at c ^ (r & 15) so that
// 16 rows read at one chunk fall in different banks; the next tile's rows
// are requested once every wave is done with the current ones, and the
// transposed tiles and per-query vectors stay double-buffered.  The dscore
// and dgain partials, the same in every launch, are written by the dof = 0
// launch.
template <int D>
struct DkvRows {
  RowTile<D> q, d;
};
template <int D>
struct DkvRowsSw {
  static constexpr int SW = (D / 8 < 16 ? D / 8 : 16) - 1;
  uint16_t q[kTile * D], d[kTile * D];
};
template <int DO>
struct DkvTr {
  TrTile<DO> qt, dt;
  float ac[kTile], acl[kTile], l2[kTile], dl[kTile];   // acl = ac ln 2
};

template <int D, int DO, bool CAUSAL, bool HAS_BIAS, bool HAS_QSCALE>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ key_score,
    const float* __restrict__ gain, const float* __restrict__ q_scale, float scale,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse2,
    const float* __restrict__ delta, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    float* __restrict__ part_kv, float* __restrict__ part_ds, float* __restrict__ part_dg,
    int32_t N, int32_t Hq, int32_t Hkv, int32_t nkb, int32_t qchunk, int32_t dof) {
  using St = Stage<D>;
  using So = Stage<DO>;
  constexpr int DK = D / 16;
  constexpr int DB = DO / 32;
  constexpr int RB = DO == D ? 2 : 1;   // row-tile buffers
  using Rows = std::conditional_t<RB == 2, DkvRows<D>, DkvRowsSw<D>>;
  __shared__ __attribute__((aligned(16))) Rows rows[RB];
  __shared__ __attribute__((aligned(16))) DkvTr<DO> trs[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hh = lane >> 5;
  // workgroup = (query chunk, key block, KV head), the KV head fastest; a key
  // block's query tiles are cut into chunks of qchunk tiles
  const int kvh = blockIdx.x % Hkv;
  const int kblock = (blockIdx.x / Hkv) % nkb;   // causal: lower key blocks see more queries
  const int chunk = blockIdx.x / (Hkv * nkb);
  const int key0 = kblock * kKeysPerWg;
  const int nq = (N + kTile - 1) / kTile;
  const int t_lo = (CAUSAL ? key0 / kTile : 0) + chunk * qchunk;
  if (t_lo >= nq) return;   // uniform: this key block has fewer chunks
  // several chunks: dK/dV go to fp32 partials, summed by attn_bwd_kv_reduce_kernel
  const bool split = (nq - (CAUSAL ? key0 / kTile : 0)) > qchunk;
  const size_t slot = (static_cast<size_t>(chunk) * nkb + kblock) * Hkv + kvh;
  const int my_k = key0 + 32 * wave + l32;
  const bool k_ok = my_k < N;
  const int G = Hq / Hkv;

  const uint32_t q_row = static_cast<uint32_t>(Hq) * D * 2;
  const uint32_t kv_row = static_cast<uint32_t>(Hkv) * D * 2;
  const auto q_rs = rsrc(q, static_cast<uint32_t>(N) * q_row);
  const auto d_rs = rsrc(dout, static_cast<uint32_t>(N) * q_row);
  const auto k_rs = rsrc(k, static_cast<uint32_t>(N) * kv_row);
  const auto v_rs = rsrc(v, static_cast<uint32_t>(N) * kv_row);

  // K, V fragments of this lane's key (B operands): dims 16 ks + 8 hh .. +7
  bf16x8 kf[DK + 1], vf[DK];
  {
    const uint32_t base = static_cast<uint32_t>(my_k) * kv_row +
                          static_cast<uint32_t>(kvh) * D * 2 + 16u * hh;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      kf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(k_rs, base + 32u * ks, 0, 0));
      vf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(v_rs, base + 32u * ks, 0, 0));
    }
  }
  const float s_key = (HAS_BIAS && k_ok) ? key_score[my_k] : 0.0f;
  const float inv_scale = 1.0f / scale;
  // a -inf score: -2^100 in dot-product units absorbs any finite dot product,
  // and its weight underflows to exactly 0 whenever scale * c_r > 2^-80
  const float masked_bias = -0x1p100f;
  // the query side of the bias k-step: [1, 1, 1, 0 ...] in the hh = 0 half
  const bf16x8 ones = __builtin_bit_cast(bf16x8, hh == 0 ? u32x4{0x3F803F80u, 0x3F80u, 0, 0}
                                                         : u32x4{0, 0, 0, 0});

  const int t_count = min(qchunk, nq - t_lo);   // query tiles per head
  const int n_iter = G * t_count;

  u32x4 qr[St::RI], dr[St::RI], qp[So::PPT][4], dpc[So::PPT][4];
  float vec_ac = 0.0f, vec_l2 = 0.0f, vec_dl = 0.0f;
  auto load_rows = [&](int it) {
    const int h = kvh * G + it / t_count;
    const int q0 = (t_lo + it % t_count) * kTile;
    const uint32_t hoff = static_cast<uint32_t>(h) * D * 2;
    St::load_rows(qr, q_rs, q_row, hoff, q0, tid);
    St::load_rows(dr, d_rs, q_row, hoff, q0, tid);
  };
  auto load_tile = [&](int it) {   // the transposed pieces and the vectors
    const int h = kvh * G + it / t_count;
    const int q0 = (t_lo + it % t_count) * kTile;
    const uint32_t hoff = static_cast<uint32_t>(h) * D * 2;
    So::load_pieces(qp, q_rs, q_row, hoff + 2u * static_cast<uint32_t>(dof), q0, tid);
    So::load_pieces(dpc, d_rs, q_row, hoff + 2u * static_cast<uint32_t>(dof), q0, tid);
    if (tid < kTile) {
      const int qi = q0 + tid;
      const bool ok = qi < N;
      vec_ac = ok ? scale * kLog2e * (HAS_QSCALE ? q_scale[qi] : 1.0f) : 0.0f;
      vec_l2 = ok ? lse2[static_cast<int64_t>(h) * N + qi] : INFINITY;
      vec_dl = ok ? delta[static_cast<int64_t>(h) * N + qi] : 0.0f;
    }
  };
  auto store_rows = [&](Rows& b) {
    if constexpr (RB == 2) {
      St::store_rows(b.q, qr, tid);
      St::store_rows(b.d, dr, tid);
    }
  };
  // single-buffered rows: each wave requests its share of the tile's 1-KB
  // pieces straight into the LDS; rows past N re-read row N - 1 (valid
  // memory; those queries have weight 0)
  auto dma_rows = [&](int it) {
    if constexpr (RB == 1) {
      const int h = kvh * G + it / t_count;
      const int q0 = (t_lo + it % t_count) * kTile;
      constexpr int PPW = kTile * D * 2 / 1024 / 4;
      Rows& b = rows[0];
      // the per-lane offsets are formed here, not kept live across the loop
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int wv = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
      for (int i = 0; i < PPW; ++i) {
        const int u = wv * PPW + i;
        const int byte = u * 1024 + 16 * ln;
        const int r = byte / (2 * D), c = ((byte % (2 * D)) / 16) ^ (r & Rows::SW);
        const int64_t off = (static_cast<int64_t>(min(q0 + r, N - 1)) * Hq + h) * D + 8 * c;
        __builtin_amdgcn_global_load_lds(q + off, (__attribute__((address_space(3))) void*)&b.q[u * 512],
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds(dout + off,
                                         (__attribute__((address_space(3))) void*)&b.d[u * 512], 16, 0, 0);
      }
    }
  };
  // vmcnt(0), other counters untouched: this wave's direct-to-LDS loads
  // have landed (each wave then passes the barrier)
  auto dma_wait = [] {
    if constexpr (RB == 1) __builtin_amdgcn_s_waitcnt(0x0F70);
  };
  auto store_tr = [&](DkvTr<DO>& b) {
    So::store_pieces(b.qt, qp, tid);
    So::store_pieces(b.dt, dpc, tid);
    if (tid < kTile) {
      b.ac[tid] = vec_ac;
      b.acl[tid] = vec_ac * kLn2;
      b.l2[tid] = vec_l2;
      b.dl[tid] = vec_dl;
    }
  };

  f32x16 dka[DB], dva[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dka[db][r] = dva[db][r] = 0.0f;
  float a_sum = 0.0f;    // sum over this lane's rows of ac * dZ, for the current head
  float ds_sum = 0.0f;   // sum over heads of gain_h * A[h, key]
  const float a_unit = 1.0f / (scale * kLog2e);   // ac = a_unit^-1 c_r

  if (n_iter > 0) {
    if constexpr (RB == 2) load_rows(0);
    dma_rows(0);
    load_tile(0);
    store_rows(rows[0]);
    store_tr(trs[0]);
    dma_wait();
  }
  __syncthreads();
  for (int it = 0; it < n_iter; ++it) {
    const Rows& br = rows[RB == 2 ? (it & 1) : 0];
    const DkvTr<DO>& b = trs[it & 1];
    const int h = kvh * G + it / t_count;
    const int q0 = (t_lo + it % t_count) * kTile;
    const bool more = it + 1 < n_iter;
    if (it % t_count == 0) {   // a new head: its bias k-step on the key side
      u32x4 kb4 = u32x4{0, 0, 0, 0};
      if (HAS_BIAS && hh == 0) {
        const float g = gain[h];
        const u32x2 t3 = bf16_triple(s_key == -INFINITY ? masked_bias : g * s_key * inv_scale);
        kb4[0] = t3[0];
        kb4[1] = t3[1];
      }
      kf[DK] = __builtin_bit_cast(bf16x8, kb4);
    }
    if (more) {
      if constexpr (RB == 2) load_rows(it + 1);
      load_tile(it + 1);
    }
    __builtin_amdgcn_sched_barrier(0);

    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[qb][r] = dp[qb][r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        bf16x8 qa, da;
        if constexpr (RB == 2) {
          const int off = (32 * qb + l32) * RowTile<D>::P + 8 * hh + 16 * ks;
          qa = *reinterpret_cast<const bf16x8*>(&br.q.a[off]);
          da = *reinterpret_cast<const bf16x8*>(&br.d.a[off]);
        } else {
          const int row = 32 * qb + l32;
          const int off = row * D + 8 * ((2 * ks + hh) ^ (row & Rows::SW));
          qa = *reinterpret_cast<const bf16x8*>(&br.q[off]);
          da = *reinterpret_cast<const bf16x8*>(&br.d[off]);
        }
        s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], s[qb], 0, 0, 0);
        dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf[ks], dp[qb], 0, 0, 0);
      }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
      s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, kf[DK], s[qb], 0, 0, 0);
    if constexpr (RB == 1) {   // every wave is done with this tile's rows
      __syncthreads();
      if (more) dma_rows(it + 1);
    }

    // element (qb, r) is query q0 + 32 qb + 8 (r / 4) + 4 hh + r % 4 and key
    // my_k; a tile that every key of the wave sees whole needs no mask
    const bool full = (!CAUSAL || q0 >= key0 + 32 * wave + 31) &&
                      key0 + 32 * wave + 32 <= N;   // wave-uniform
    bf16x8 pb[2][2], zb[2][2];
    auto weights = [&](const bool masked) __attribute__((always_inline)) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int qi = 32 * qb + 8 * j + 4 * hh;
          const f32x4 vac = *reinterpret_cast<const f32x4*>(&b.ac[qi]);
          const f32x4 vacl = *reinterpret_cast<const f32x4*>(&b.acl[qi]);
          const f32x4 vl2 = *reinterpret_cast<const f32x4*>(&b.l2[qi]);
          const f32x4 vdl = *reinterpret_cast<const f32x4*>(&b.dl[qi]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * j + i;
            const bool vis = !masked || (k_ok && (!CAUSAL || my_k <= q0 + qi + i));
            const float e = __builtin_amdgcn_exp2f(fmaf(s[qb][r], vac[i], -vl2[i]));
            const float p = vis ? e : 0.0f;
            const float dz = p * (dp[qb][r] - vdl[i]);
            a_sum = fmaf(vac[i], dz, a_sum);
            pb[qb][r >> 3][r & 7] = static_cast<__bf16>(p);
            zb[qb][r >> 3][r & 7] = static_cast<__bf16>(dz * vacl[i]);   // dZ c alpha
          }
        }
    };
    if (full) weights(false); else weights(true);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int off = (32 * db + l32) * TrTile<DO>::P + 32 * qb + 16 * hf + 8 * hh;
          const u32x4 da4 = *reinterpret_cast<const u32x4*>(&b.dt.a[off]);
          dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, da4),
                                                            pb[qb][hf], dva[db], 0, 0, 0);
          const u32x4 qa4 = *reinterpret_cast<const u32x4*>(&b.qt.a[off]);
          dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qa4),
                                                            zb[qb][hf], dka[db], 0, 0, 0);
        }

    if (HAS_BIAS && it % t_count == t_count - 1) {   // last tile of head h
      const float a_key = (a_sum + __shfl_xor(a_sum, 32, 64)) * a_unit;   // A[h, my_k]
      ds_sum = fmaf(gain[h], a_key, ds_sum);
      // dgain partial: sum over this wave's 32 keys of s * A (a -inf score has A = 0)
      float g_part = (k_ok && hh == 0 && s_key != -INFINITY) ? s_key * a_key : 0.0f;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) g_part += __shfl_xor(g_part, m, 64);
      if (lane == 0 && dof == 0) part_dg[(slot * 4 + wave) * G + (h - kvh * G)] = g_part;
      a_sum = 0.0f;
    }
    if (more) {
      store_rows(rows[RB == 2 ? ((it + 1) & 1) : 0]);
      store_tr(trs[(it + 1) & 1]);
      dma_wait();
    }
    __syncthreads();
  }

  const int key_local = 32 * wave + l32;
  if (HAS_BIAS && hh == 0 && dof == 0) part_ds[slot * kKeysPerWg + key_local] = ds_sum;
  if (split) {
    // dK^T, dV^T accumulator entries of this lane: dims dof + 32 db + 8 j + 4 hh .. +3
    float* pk = part_kv + ((slot * 2) * kKeysPerWg + key_local) * D + dof + 4 * hh;
    float* pv = pk + static_cast<size_t>(kKeysPerWg) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<f32x4*>(pk + 32 * db + 8 * j) =
            f32x4{dka[db][4 * j], dka[db][4 * j + 1], dka[db][4 * j + 2], dka[db][4 * j + 3]};
        *reinterpret_cast<f32x4*>(pv + 32 * db + 8 * j) =
            f32x4{dva[db][4 * j], dva[db][4 * j + 1], dva[db][4 * j + 2], dva[db][4 * j + 3]};
      }
  } else if (k_ok) {
    const int64_t off = static_cast<int64_t>(my_k) * Hkv * D + static_cast<int64_t>(kvh) * D + dof;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 wk, wv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wk[i] = static_cast<__bf16>(dka[db][4 * j + i]);
          wv[i] = static_cast<__bf16>(dva[db][4 * j + i]);
        }
        *reinterpret_cast<bf16x4*>(dk + off + 32 * db + 8 * j + 4 * hh) = wk;
        *reinterpret_cast<bf16x4*>(dv + off + 32 * db + 8 * j + 4 * hh) = wv;
      }
  }
}

// Chunks of a split key block (causal: key block kb's first query tile is
// 2 kb; chunk count ceil(tiles / qchunk)).
__device__ __forceinline__ int kv_chunks(int kb, int nq, int qchunk, bool causal) {
  const int tiles = nq - (causal ? kb * (kKeysPerWg / kTile) : 0);
  return (tiles + qchunk - 1) / qchunk;
}

// dK, dV of split key blocks: the chunks' fp32 partials summed in chunk
// order, stored as bf16.  One thread per (key, KV head, 4 dims).
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_kv_reduce_kernel(
    const float* __restrict__ part_kv, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    int32_t N, int32_t Hkv, int32_t nkb, int32_t qchunk, int causal) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_key = static_cast<int64_t>(Hkv) * (D / 4);
  if (i >= static_cast<int64_t>(N) * per_key) return;
  const int key = static_cast<int>(i / per_key);
  const int kvh = static_cast<int>((i % per_key) / (D / 4));
  const int d4 = static_cast<int>(i % (D / 4));
  const int kb = key / kKeysPerWg, kl = key % kKeysPerWg;
  const int nq = (N + kTile - 1) / kTile;
  const int nc = kv_chunks(kb, nq, qchunk, causal != 0);
  if (nc <= 1) return;   // written directly by the key block's only workgroup
  // (bandwidth-bound: occupancy hides the load latency, so the loop stays a
  // plain one with few registers)
  f32x4 sk = f32x4{0.f, 0.f, 0.f, 0.f}, sv = sk;
  for (int c = 0; c < nc; ++c) {
    const size_t slot = (static_cast<size_t>(c) * nkb + kb) * Hkv + kvh;
    const float* pk = part_kv + ((slot * 2) * kKeysPerWg + kl) * D + 4 * d4;
    sk += *reinterpret_cast<const f32x4*>(pk);
    sv += *reinterpret_cast<const f32x4*>(pk + static_cast<size_t>(kKeysPerWg) * D);
  }
  const int64_t off = static_cast<int64_t>(key) * Hkv * D + static_cast<int64_t>(kvh) * D + 4 * d4;
  bf16x4 wk, wv;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    wk[e] = static_cast<__bf16>(sk[e]);
    wv[e] = static_cast<__bf16>(sv[e]);
  }
  *reinterpret_cast<bf16x4*>(dk + off) = wk;
  *reinterpret_cast<bf16x4*>(dv + off) = wv;
}

// dscore[c] = sum over KV heads and chunks of part_ds (workgroups below
// n_ds_blocks, one thread per key); dgain[h] = sum over key blocks, chunks
// and waves of part_dg (one workgroup per head: strided partial sums, then a
// tree in LDS).  Fixed order throughout: deterministic.
__global__ __launch_bounds__(256) void attn_bwd_reduce_kernel(const float* __restrict__ part_ds,
                                                              const float* __restrict__ part_dg,
                                                              float* __restrict__ dscore,
                                                              float* __restrict__ dgain,
                                                              int32_t N, int32_t Hq, int32_t Hkv,
                                                              int32_t nkb, int32_t qchunk,
                                                              int causal, int32_t n_ds_blocks) {
  const int nq = (N + kTile - 1) / kTile;
  if (static_cast<int>(blockIdx.x) < n_ds_blocks) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= N) return;
    const int kb = static_cast<int>(i) / kKeysPerWg, kl = static_cast<int>(i) % kKeysPerWg;
    const int nc = kv_chunks(kb, nq, qchunk, causal != 0);   // <= kMaxKvChunks
    float acc = 0.0f;
    for (int h = 0; h < Hkv; ++h) {
      // a head's chunk partials read together, then added in chunk order
      float v[kMaxKvChunks];
#pragma unroll
      for (int c = 0; c < kMaxKvChunks; ++c)
        v[c] = c < nc ? part_ds[((static_cast<size_t>(c) * nkb + kb) * Hkv + h) * kKeysPerWg + kl]
                      : 0.0f;
#pragma unroll
      for (int c = 0; c < kMaxKvChunks; ++c)
        if (c < nc) acc += v[c];
    }
    dscore[i] = acc;
    return;
  }
  const int h = static_cast<int>(blockIdx.x) - n_ds_blocks;
  const int G = Hq / Hkv, kvh = h / G, hl = h % G;
  // entries (key block, chunk, wave) in key-block-major order; thread t sums
  // entries t, t + 256, ...
  const int per_kb = 4 * ((nq + qchunk - 1) / qchunk);   // upper bound of waves x chunks
  float acc = 0.0f;
  for (int e = threadIdx.x; e < nkb * per_kb; e += 256) {
    const int kb = e / per_kb, c = (e % per_kb) / 4, w = e % 4;
    if (c < kv_chunks(kb, nq, qchunk, causal != 0)) {
      const size_t slot = (static_cast<size_t>(c) * nkb + kb) * Hkv + kvh;
      acc += part_dg[(slot * 4 + w) * G + hl];
    }
  }
  __shared__ float red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int m = 128; m >= 1; m >>= 1) {
    if (static_cast<int>(threadIdx.x) < m) red[threadIdx.x] += red[threadIdx.x + m];
    __syncthreads();
  }
  if (threadIdx.x == 0) dgain[h] = red[0];
}

// dK/dV query chunks: enough (query chunk, key block, KV head) workgroups to
// give every CU about three, at most 8 chunks per key block.
struct BwdWorkspace {
  int32_t nkb, nchunk, qchunk;
  size_t delta, lse2, part_ds, part_dg, part_kv, bytes;   // float offsets, total bytes
};
BwdWorkspace bwd_workspace(int64_t N, int64_t Hq, int64_t Hkv, int64_t D) {
  BwdWorkspace w;
  w.nkb = static_cast<int32_t>((N + kKeysPerWg - 1) / kKeysPerWg);
  const int64_t nq = (N + kTile - 1) / kTile;
  const int64_t pairs = std::max<int64_t>(int64_t{1}, w.nkb * Hkv);
  const int64_t want =
      std::min<int64_t>(kMaxKvChunks, std::max<int64_t>(1, (768 + pairs - 1) / pairs));
  w.qchunk = static_cast<int32_t>(std::max<int64_t>(1, (nq + want - 1) / want));
  w.nchunk = static_cast<int32_t>(std::max<int64_t>(1, (nq + w.qchunk - 1) / w.qchunk));
  const size_t slots = static_cast<size_t>(w.nchunk) * w.nkb * Hkv;
  w.delta = 0;
  w.lse2 = static_cast<size_t>(Hq * N);
  w.part_ds = w.lse2 + static_cast<size_t>(Hq * N);
  w.part_dg = w.part_ds + slots * kKeysPerWg;
  w.part_kv = w.part_dg + slots * 4 * static_cast<size_t>(Hq / Hkv);
  const size_t kv = w.nchunk > 1 ? slots * 2 * kKeysPerWg * static_cast<size_t>(D) : 0;
  w.bytes = (w.part_kv + kv) * sizeof(float);
  return w;
}

struct BwdArgs {
  const uint16_t *q, *k, *v, *out, *dout;
  const float *ks, *gain, *qs, *lse;
  float scale;
  uint16_t *dq, *dk, *dv;
  float *dscore, *dgain;
  float* ws;
  int32_t N, Hq, Hkv;
  bool causal;
  hipStream_t s;
};

// Head dim 256: each gradient kernel runs twice, once per 128-dim half of
// its output (the accumulators of all 256 dims do not fit the registers).
template <int D, int HPW, bool CAUSAL, bool B, bool QS>
void launch_bwd(const BwdArgs& a, const BwdWorkspace& w) {
  constexpr int DO = D > 128 ? 128 : D;
  constexpr int PB = 32 * (4 / HPW);
  const int32_t npb = (a.N + PB - 1) / PB, nhg = a.Hq / HPW;
  const int32_t nkb = w.nkb;
  float* delta = a.ws + w.delta;
  float* lse2 = a.ws + w.lse2;
  float* pds = a.ws + w.part_ds;
  float* pdg = a.ws + w.part_dg;
  float* pkv = a.ws + w.part_kv;
  const int64_t rows = static_cast<int64_t>(a.N) * a.Hq;
  attn_bwd_pre_kernel<D><<<dim3(static_cast<uint32_t>((rows + 255) / 256)), dim3(256), 0, a.s>>>(
      a.out, a.dout, a.lse, delta, lse2, a.N, a.Hq);
  for (int dof = 0; dof < D; dof += DO)
    attn_bwd_dkdv_kernel<D, DO, CAUSAL, B, QS>
        <<<dim3(static_cast<uint32_t>(w.nchunk * nkb * a.Hkv)), dim3(256), 0, a.s>>>(
            a.q, a.k, a.v, a.ks, a.gain, a.qs, a.scale, a.dout, lse2, delta, a.dk, a.dv, pkv,
            pds, pdg, a.N, a.Hq, a.Hkv, nkb, w.qchunk, dof);
  if (w.nchunk > 1) {
    const int64_t n = static_cast<int64_t>(a.N) * a.Hkv * (D / 4);
    attn_bwd_kv_reduce_kernel<D><<<dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0,
                                   a.s>>>(pkv, a.dk, a.dv, a.N, a.Hkv, nkb, w.qchunk,
                                          CAUSAL ? 1 : 0);
  }
  for (int dof = 0; dof < D; dof += DO)
    attn_bwd_dq_kernel<D, DO, HPW, CAUSAL, B, QS>
        <<<dim3(static_cast<uint32_t>(npb * nhg)), dim3(256), 0, a.s>>>(
            a.q, a.k, a.v, a.ks, a.gain, a.qs, a.scale, a.dout, lse2, delta, a.dq, a.N, a.Hq,
            a.Hkv, npb, nhg, dof);
  if (B) {
    const int32_t nds = (a.N + 255) / 256;
    attn_bwd_reduce_kernel<<<dim3(static_cast<uint32_t>(nds + a.Hq)), dim3(256), 0, a.s>>>(
        pds, pdg, a.dscore, a.dgain, a.N, a.Hq, a.Hkv, nkb, w.qchunk, CAUSAL ? 1 : 0, nds);
  }
}

template <int D, int HPW>
void launch_bwd_d(const BwdArgs& a, const BwdWorkspace& w) {
  const bool b = a.ks != nullptr, qs = a.qs != nullptr;
#define TG_BWD(C, B, Q) launch_bwd<D, HPW, C, B, Q>(a, w)
  if (a.causal) {
    if (b) { if (qs) TG_BWD(true, true, true); else TG_BWD(true, true, false); }
    else { if (qs) TG_BWD(true, false, true); else TG_BWD(true, false, false); }
  } else {
    if (b) { if (qs) TG_BWD(false, true, true); else TG_BWD(false, true, false); }
    else { if (qs) TG_BWD(false, false, true); else TG_BWD(false, false, false); }
  }
#undef TG_BWD
}

}  // namespace
}  // namespace tg

extern "C" size_t tg_bias_attn_bwd_workspace_size(int64_t N, int64_t Hq, int64_t Hkv,
                                                  int64_t D) {
  if (N < 0 || N > tg::kMaxTokens || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 ||
      N * Hq > tg::kMaxTokens || (D != 64 && D != 128 && D != 256))
    return 0;
  return tg::bwd_workspace(N, Hq, Hkv, D).bytes;
}

extern "C" tg_status tg_bias_attn_bwd(tg_dtype dt, int64_t N, int64_t Hq, int64_t Hkv, int64_t D,
                                      const void* q, const void* k, const void* v,
                                      const float* key_score, const float* gain,
                                      const float* q_scale, float softmax_scale, int causal,
                                      const void* out, const void* dout, const float* lse,
                                      void* dq, void* dk, void* dv, float* dscore, float* dgain,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  using namespace tg;
  if (dt != TG_DTYPE_F32 && dt != TG_DTYPE_BF16)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_bias_attn_bwd: unknown dtype %d", (int)dt);
  if (N < 0 || N > kMaxTokens || Hq < 1 || Hkv < 1 || Hq > 65536 || Hkv > 65536)
    return fail(TG_ERR_INVALID_ARGUMENT,
                "tg_bias_attn_bwd: need 0 <= N <= 2^31-1 and 1 <= Hkv, Hq (N=%lld Hq=%lld Hkv=%lld)",
                (long long)N, (long long)Hq, (long long)Hkv);
  if (Hq % Hkv != 0)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_bias_attn_bwd: Hq %% Hkv != 0 (%lld, %lld)",
                (long long)Hq, (long long)Hkv);
  if (dt != TG_DTYPE_BF16)
    return fail(TG_ERR_UNSUPPORTED, "tg_bias_attn_bwd: bf16 only");
  if (D != 64 && D != 128 && D != 256)
    return fail(TG_ERR_UNSUPPORTED,
                "tg_bias_attn_bwd: head dim must be 64, 128 or 256 (D=%lld)", (long long)D);
  if (N * Hq > kMaxTokens || N * Hq * D * 2 > kMaxTokens)
    return fail(TG_ERR_UNSUPPORTED,
                "tg_bias_attn_bwd: N * Hq * D * 2 must be < 2^31 (32-bit offsets)");
  const BwdWorkspace w = bwd_workspace(N, Hq, Hkv, D);
  if (w.bytes > 0 && (workspace == nullptr || workspace_bytes < w.bytes))
    return fail(TG_ERR_WORKSPACE, "tg_bias_attn_bwd: workspace of %zu bytes, need %zu",
                workspace == nullptr ? (size_t)0 : workspace_bytes, w.bytes);
  if (workspace != nullptr && !aligned(workspace, 16))
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_bias_attn_bwd: workspace must be 16-byte aligned");
  if (N == 0) {
    clear_error();
    return TG_OK;
  }
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_bias_attn_bwd: NULL q/k/v/out/dout/lse/dq/dk/dv");
  if (key_score && (!gain || !dscore || !dgain))
    return fail(TG_ERR_INVALID_ARGUMENT,
                "tg_bias_attn_bwd: key_score given without gain, dscore or dgain");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_bias_attn_bwd: tensors must be 16-byte aligned");
  BwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<const uint16_t*>(out);
  a.dout = static_cast<const uint16_t*>(dout);
  a.ks = key_score;
  a.gain = gain;
  a.qs = q_scale;
  a.lse = lse;
  a.scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf(static_cast<float>(D));
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.dscore = dscore;
  a.dgain = dgain;
  a.ws = static_cast<float*>(workspace);
  a.N = static_cast<int32_t>(N);
  a.Hq = static_cast<int32_t>(Hq);
  a.Hkv = static_cast<int32_t>(Hkv);
  a.causal = causal != 0;
  a.s = as_stream(stream);
  const int64_t G = Hq / Hkv;
  const int hpw = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  if (D == 256) {
    if (hpw == 4) launch_bwd_d<256, 4>(a, w);
    else if (hpw == 2) launch_bwd_d<256, 2>(a, w);
    else launch_bwd_d<256, 1>(a, w);
  } else if (D == 128) {
    if (hpw == 4) launch_bwd_d<128, 4>(a, w);
    else if (hpw == 2) launch_bwd_d<128, 2>(a, w);
    else launch_bwd_d<128, 1>(a, w);
  } else {
    if (hpw == 4) launch_bwd_d<64, 4>(a, w);
    else if (hpw == 2) launch_bwd_d<64, 2>(a, w);
    else launch_bwd_d<64, 1>(a, w);
  }
  return check_launch("tg_bias_attn_bwd");
}
