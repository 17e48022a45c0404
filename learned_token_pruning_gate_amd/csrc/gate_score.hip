// gate_score.hip -- [a1] the gate's scorer: RMSNorm of each prunable token's
// residual row followed by an MLP d -> h (SiLU) -> 1.
//
// TokenGate pages: ai.info summary "Key Contributions" item 1 (a scoring MLP
// over the RMSNorm-normalised post-attention residual scores the prunable
// tokens), the techbycountry explainer "how the gate works" and the README
// mirror "How it works".
//
// bf16 path (gfx950).  The gate reads every prunable residual row once
// (n_P * d * 2 bytes) and performs 2 * n_P * d * h flops: at h = 256 that
// is 256 flop per byte, just under the MI355X bf16 ridge, so the kernel is
// built to stream the residual at HBM rate while the MFMA pipes keep up:
//   * RMSNorm is folded into a per-row scale applied after the projection:
//     W1 (gamma * x / rms) = (W1 (gamma * x)) / rms, so the row's sum of
//     squares is accumulated from the same registers that stage the tile;
//   * a workgroup owns TM rows and all h outputs; the TM x 64 residual tile
//     of each k-stage goes HBM -> registers (two stages in flight, loaded
//     non-temporally so the stream does not evict W1 from L2) -> padded LDS
//     (double buffered, one barrier per stage) and is read by the four waves
//     as MFMA A operands;
//   * each wave owns h/4 output columns and streams its slice of W1 (which
//     stays resident in each XCD's L2) straight into registers as MFMA B
//     operands, one stage ahead;
//   * v_mfma_f32_16x16x32_bf16 accumulates z in fp32; the epilogue applies
//     1/rms, b1, SiLU and w2 per element and reduces over h inside 16-lane
//     rows and then across the four waves through LDS.
//
// f32 path: one wave per row on the vector ALUs (fp32 throughout).
#include "tg_common.hpp"

namespace tg {
namespace {

constexpr int kKS = 64;                 // k elements per stage
#ifndef TG_GATE_TM
#define TG_GATE_TM 64                   // residual rows per workgroup
#endif
constexpr int kPitch = kKS + 8;         // LDS row pitch in bf16 (144 bytes)

#ifndef TG_GATE_MINWG
#define TG_GATE_MINWG 2                 // workgroups per CU the registers are sized for
#endif

// FAST: d is a multiple of 2 * kKS, so every stage is full; per-lane load
// offsets are fixed and the stage advance is the instruction's scalar offset.
template <int TM, int NT, bool HAS_GAMMA, bool FAST>
__global__ __launch_bounds__(256, TG_GATE_MINWG) void gate_bf16_kernel(
    const uint16_t* __restrict__ resid, int64_t ld_x, const uint8_t* __restrict__ prunable,
    const float* __restrict__ gamma, float eps, const uint16_t* __restrict__ w1,
    const float* __restrict__ b1, const float* __restrict__ w2, float b2,
    float* __restrict__ scores, int32_t T, int32_t d) {
  constexpr int RPT = TM / 32;          // staged rows per thread
  constexpr int MT = TM / 16;           // 16-row MFMA tiles per wave
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][TM * kPitch];
  extern __shared__ __attribute__((aligned(16))) float s_gamma[];   // [d] when HAS_GAMMA
  __shared__ float s_rs[TM];
  __shared__ float s_part[4][TM];
  __shared__ int s_any;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * TM;

  // staging role: row (tid/8) + 32 i, 16-byte chunk tid % 8 of the stage.
  // Loads go through buffer resources: an offset past the end reads zeros,
  // so rows that are not prunable (or past T) and the k tail need no branch.
  const int chunk = tid & 7;
  constexpr uint32_t kOff = 0x80000000u;   // beyond every resource below
  bool live[RPT];
  uint32_t xoff[RPT];                      // byte offset of the row's chunk, or kOff
  int any = 0;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = (tid >> 3) + 32 * i;
    live[i] = (row0 + r < T) && prunable[row0 + r] != 0;
    any |= live[i];
    xoff[i] = live[i] ? static_cast<uint32_t>(r) * static_cast<uint32_t>(ld_x) * 2u + chunk * 16u
                      : kOff;
  }
  const int64_t rows_here = T - row0 < TM ? T - row0 : TM;
  const __amdgpu_buffer_rsrc_t x_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(resid + row0 * ld_x), 0,
      static_cast<int>(static_cast<uint32_t>(((rows_here - 1) * ld_x + d) * 2)), 0x00020000);
  const __amdgpu_buffer_rsrc_t w_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(w1), 0, static_cast<int>(static_cast<uint32_t>(NT * 64 * d * 2)),
      0x00020000);
  if (HAS_GAMMA) {   // RMSNorm weight staged once; read from LDS per stage
    for (int i = tid; i < d; i += 256) s_gamma[i] = gamma[i];
    __syncthreads();
  }
  if (tid == 0) s_any = 0;
  __syncthreads();
  if (any) s_any = 1;
  __syncthreads();
  if (!s_any) {  // no prunable row in this tile
    if (tid < TM && row0 + tid < T) scores[row0 + tid] = 0.0f;
    return;
  }

  // compute role: wave owns columns [wave*16*NT, (wave+1)*16*NT)
  const int hbase = wave * 16 * NT;
  const int lrow = lane & 15;            // A row / B column inside a 16x16 tile
  const int lk = (lane >> 4) * 8;        // k offset of this lane's 8 elements
  uint32_t woff[NT];                     // byte offset of this lane's W1 row at k = lk
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    woff[nt] = (static_cast<uint32_t>(hbase + nt * 16 + lrow) * static_cast<uint32_t>(d) + lk) * 2u;

  const int nstages = (d + kKS - 1) / kKS;
  float ss[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) ss[i] = 0.0f;

  // two register sets: stage s+2 is in flight while stage s+1 is stored
  u32x4 xr[2][RPT];
  auto load_x = [&](int s, u32x4 (&dst)[RPT]) {
    if (FAST) {
#pragma unroll
      for (int i = 0; i < RPT; ++i)   // streamed once (non-temporal)
        dst[i] = __builtin_amdgcn_raw_buffer_load_b128(x_rs, xoff[i], s * kKS * 2, 2);
    } else {
      const bool kin = s * kKS + chunk * 8 < d;
#pragma unroll
      for (int i = 0; i < RPT; ++i)
        dst[i] = __builtin_amdgcn_raw_buffer_load_b128(
            x_rs, kin ? xoff[i] + static_cast<uint32_t>(s) * kKS * 2u : kOff, 0, 2);
    }
  };
  auto store_x = [&](int s, int buf, const u32x4 (&src)[RPT]) {
    float g[8];
    if (HAS_GAMMA) {
      const int k = s * kKS + chunk * 8;   // rows past d are zero, any gamma works
      const f32x4 g0 = *reinterpret_cast<const f32x4*>(&s_gamma[k < d ? k : 0]);
      const f32x4 g1 = *reinterpret_cast<const f32x4*>(&s_gamma[(k < d ? k : 0) + 4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        g[e] = g0[e];
        g[4 + e] = g1[e];
      }
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      u32x4 v = src[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(v[e] << 16);
        const float hi = __uint_as_float(v[e] & 0xffff0000u);
        ss[i] = fmaf(lo, lo, ss[i]);
        ss[i] = fmaf(hi, hi, ss[i]);
        if (HAS_GAMMA) {
          __bf16 blo = static_cast<__bf16>(lo * g[2 * e]);
          __bf16 bhi = static_cast<__bf16>(hi * g[2 * e + 1]);
          v[e] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, blo)) |
                 (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, bhi)) << 16);
        }
      }
      const int r = (tid >> 3) + 32 * i;
      *reinterpret_cast<u32x4*>(&xs[buf][r * kPitch + chunk * 8]) = v;
    }
  };

  // W1 fragments stay integer vectors until they reach the MFMA (bf16 vector
  // values would pick up extra register operations right after the load)
  u32x4 wc[NT][2], wn[NT][2];
  auto load_w = [&](int s, u32x4 (&w)[NT][2]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      if (FAST) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          w[nt][kk] = __builtin_amdgcn_raw_buffer_load_b128(w_rs, woff[nt] + kk * 64,
                                                            s * kKS * 2, 0);
      } else {
        const bool kin = s * kKS + kk * 32 + lk < d;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          w[nt][kk] = __builtin_amdgcn_raw_buffer_load_b128(
              w_rs, kin ? woff[nt] + static_cast<uint32_t>(s * kKS + kk * 32) * 2u : kOff, 0,
              0);
      }
    }
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_x(0, xr[0]);
  if (!FAST || nstages > 1) load_x(1, xr[1]);
  load_w(0, wc);
  store_x(0, 0, xr[0]);
  __syncthreads();

  // One stage: prefetch x(s+2) and W1(s+1), multiply stage s out of LDS
  // buffer s&1 with W1(s), then stage x(s+1) into the other buffer.  Every
  // stage runs unconditionally: loads past d read zeros, which leave the
  // accumulators and sums of squares unchanged, and straight-line loads let
  // the compiler wait for exactly the data each step needs.
  // PREF: issue this stage's prefetches (the FAST epilogue stages do not).
  auto stage = [&](int s, const u32x4 (&wcur)[NT][2], u32x4 (&wnext)[NT][2], bool pref_x,
                   bool pref_w, bool stage_next) {
    const int buf = s & 1;
    if (pref_x) load_x(s + 2, xr[buf]);
    if (pref_w) load_w(s + 1, wnext);
    // keep the prefetches issued here: the scheduler would otherwise sink them
    // next to their uses and serialise the pipeline
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(&xs[buf][(mt * 16 + lrow) * kPitch + kk * 32 + lk]));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a, __builtin_bit_cast(bf16x8, wcur[nt][kk]), acc[mt][nt], 0, 0, 0);
      }
    }
    if (stage_next) store_x(s + 1, buf ^ 1, xr[buf ^ 1]);
    __syncthreads();
  };
  if (FAST) {
    // steady state: stages 0 .. nstages-3 with every prefetch in range, then
    // two epilogue stages without prefetch (nstages is even and >= 2)
    for (int s = 0; s + 2 < nstages; s += 2) {
      stage(s, wc, wn, true, true, true);
      stage(s + 1, wn, wc, s + 3 < nstages, true, true);
    }
    stage(nstages - 2, wc, wn, false, true, true);
    stage(nstages - 1, wn, wc, false, false, false);
  } else {
    for (int s = 0; s < nstages; s += 2) {   // an odd count runs one all-zero stage
      stage(s, wc, wn, true, true, true);
      stage(s + 1, wn, wc, true, true, true);
    }
  }

  // per-row 1/rms: reduce the sum of squares over the 8 lanes of a row
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    float v = ss[i];
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    v += __shfl_xor(v, 4, 64);
    if (chunk == 0) s_rs[(tid >> 3) + 32 * i] = 1.0f / sqrtf(v / static_cast<float>(d) + eps);
  }
  __syncthreads();

  // epilogue: z = acc/rms + b1; partial score over this wave's columns
  float part[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) part[mt][r] = 0.0f;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = hbase + nt * 16 + lrow;
    const float bb = b1 ? b1[n] : 0.0f;
    const float ww = w2[n];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = mt * 16 + (lane >> 4) * 4 + r;
        const float z = fmaf(acc[mt][nt][r], s_rs[tok], bb);
        part[mt][r] = fmaf(ww, z / (1.0f + expf(-z)), part[mt][r]);
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = part[mt][r];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      v += __shfl_xor(v, 8, 64);
      if (lrow == 0) s_part[wave][mt * 16 + (lane >> 4) * 4 + r] = v;
    }
  }
  __syncthreads();
  if (tid < TM) {
    const int64_t t = row0 + tid;
    if (t < T) {
      const float s = b2 + ((s_part[0][tid] + s_part[1][tid]) + (s_part[2][tid] + s_part[3][tid]));
      scores[t] = prunable[t] ? s : 0.0f;
    }
  }
}

// fp32 path: one wave per row.  u = gamma*x/rms is formed on the fly;
// lane j accumulates z_j over the row (x broadcast from L1), then the wave
// reduces w2 . SiLU(z) across lanes.
__global__ __launch_bounds__(256) void gate_f32_kernel(
    const float* __restrict__ resid, int64_t ld_x, const uint8_t* __restrict__ prunable,
    const float* __restrict__ gamma, float eps, const float* __restrict__ w1,
    const float* __restrict__ b1, const float* __restrict__ w2, float b2,
    float* __restrict__ scores, int32_t T, int32_t d, int32_t h) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  if (!prunable[t]) {
    if (lane == 0) scores[t] = 0.0f;
    return;
  }
  const float* x = resid + t * ld_x;
  float ss = 0.0f;
  for (int i = lane; i < d; i += 64) ss = fmaf(x[i], x[i], ss);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const float inv_rms = 1.0f / sqrtf(ss / static_cast<float>(d) + eps);
  float part = 0.0f;
  for (int j = lane; j < h; j += 64) {
    const float* wr = w1 + static_cast<int64_t>(j) * d;
    float z = 0.0f;
    for (int i = 0; i < d; ++i) {
      const float u = gamma ? gamma[i] * (x[i] * inv_rms) : x[i] * inv_rms;
      z = fmaf(wr[i], u, z);
    }
    if (b1) z += b1[j];
    part = fmaf(w2[j], z / (1.0f + expf(-z)), part);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
  if (lane == 0) scores[t] = b2 + part;
}

template <int TM, int NT, bool FAST>
void launch_bf16_f(bool has_gamma, int64_t T, dim3 grid, hipStream_t s, const uint16_t* x,
                   int64_t ld, const uint8_t* p, const float* g, float eps, const uint16_t* w1,
                   const float* b1, const float* w2, float b2, float* out, int32_t d) {
  if (has_gamma)
    gate_bf16_kernel<TM, NT, true, FAST><<<grid, dim3(256), static_cast<size_t>(d) * 4, s>>>(
        x, ld, p, g, eps, w1, b1, w2, b2, out, static_cast<int32_t>(T), d);
  else
    gate_bf16_kernel<TM, NT, false, FAST><<<grid, dim3(256), 0, s>>>(
        x, ld, p, g, eps, w1, b1, w2, b2, out, static_cast<int32_t>(T), d);
}

template <int TM, int NT>
void launch_bf16(bool has_gamma, int64_t T, dim3 grid, hipStream_t s, const uint16_t* x,
                 int64_t ld, const uint8_t* p, const float* g, float eps, const uint16_t* w1,
                 const float* b1, const float* w2, float b2, float* out, int32_t d) {
  if (d % (2 * kKS) == 0)
    launch_bf16_f<TM, NT, true>(has_gamma, T, grid, s, x, ld, p, g, eps, w1, b1, w2, b2, out, d);
  else
    launch_bf16_f<TM, NT, false>(has_gamma, T, grid, s, x, ld, p, g, eps, w1, b1, w2, b2, out, d);
}

}  // namespace
}  // namespace tg

extern "C" tg_status tg_gate_score(tg_dtype dt, int64_t T, int64_t d, int64_t h,
                                   const void* resid, int64_t resid_row_stride,
                                   const uint8_t* prunable, const float* rms_weight, float eps,
                                   const void* w1, const float* b1, const float* w2, float b2,
                                   float* scores, void* stream) {
  using namespace tg;
  if (dt != TG_DTYPE_F32 && dt != TG_DTYPE_BF16)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_gate_score: unknown dtype %d", (int)dt);
  if (T < 0 || T > kMaxTokens || d < 1 || h < 1 || d > kMaxTokens || h > kMaxTokens)
    return fail(TG_ERR_INVALID_ARGUMENT,
                "tg_gate_score: need 0 <= T <= 2^31-1, d >= 1, h >= 1 (T=%lld d=%lld h=%lld)",
                (long long)T, (long long)d, (long long)h);
  if (!(eps >= 0.0f))
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_gate_score: eps must be >= 0");
  if (T == 0) {
    clear_error();
    return TG_OK;
  }
  if (!resid || !prunable || !w1 || !w2 || !scores)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_gate_score: NULL resid/prunable/w1/w2/scores");
  if (resid_row_stride < d)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_gate_score: resid_row_stride %lld < d %lld",
                (long long)resid_row_stride, (long long)d);
  hipStream_t s = as_stream(stream);
  if (dt == TG_DTYPE_F32) {
    if (!aligned(resid, 4) || !aligned(w1, 4))
      return fail(TG_ERR_INVALID_ARGUMENT, "tg_gate_score: misaligned f32 pointer");
    const int64_t blocks = (T + 3) / 4;
    gate_f32_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s>>>(
        static_cast<const float*>(resid), resid_row_stride, prunable, rms_weight, eps,
        static_cast<const float*>(w1), b1, w2, b2, scores, static_cast<int32_t>(T),
        static_cast<int32_t>(d), static_cast<int32_t>(h));
    return check_launch("tg_gate_score");
  }
  if (d % 8 != 0)
    return fail(TG_ERR_UNSUPPORTED, "tg_gate_score: bf16 path needs d %% 8 == 0 (d=%lld)",
                (long long)d);
  if (h % 64 != 0 || h > 256)
    return fail(TG_ERR_UNSUPPORTED,
                "tg_gate_score: bf16 path needs h in {64, 128, 192, 256} (h=%lld)",
                (long long)h);
  if (rms_weight != nullptr && d > 16384)
    return fail(TG_ERR_UNSUPPORTED,
                "tg_gate_score: bf16 path with an RMSNorm weight needs d <= 16384 (LDS-staged)");
  if (static_cast<int64_t>(TG_GATE_TM) * resid_row_stride * 2 > kMaxTokens || h * d * 2 > kMaxTokens)
    return fail(TG_ERR_UNSUPPORTED,
                "tg_gate_score: bf16 path addresses a 64-row tile and W1 with 31-bit offsets");
  if (!aligned(resid, 16) || !aligned(w1, 16) || (resid_row_stride % 8) != 0)
    return fail(TG_ERR_INVALID_ARGUMENT,
                "tg_gate_score: bf16 resid/w1 must be 16-byte aligned, row stride %% 8 == 0");
  const auto* x = static_cast<const uint16_t*>(resid);
  const auto* w = static_cast<const uint16_t*>(w1);
  const int32_t d32 = static_cast<int32_t>(d);
  const bool g = rms_weight != nullptr;
  constexpr int TM = TG_GATE_TM;
  const dim3 grid(static_cast<uint32_t>((T + TM - 1) / TM));
  switch (h / 64) {
    case 1: launch_bf16<TM, 1>(g, T, grid, s, x, resid_row_stride, prunable, rms_weight, eps, w, b1, w2, b2, scores, d32); break;
    case 2: launch_bf16<TM, 2>(g, T, grid, s, x, resid_row_stride, prunable, rms_weight, eps, w, b1, w2, b2, scores, d32); break;
    case 3: launch_bf16<TM, 3>(g, T, grid, s, x, resid_row_stride, prunable, rms_weight, eps, w, b1, w2, b2, scores, d32); break;
    default: launch_bf16<TM, 4>(g, T, grid, s, x, resid_row_stride, prunable, rms_weight, eps, w, b1, w2, b2, scores, d32); break;
  }
  return check_launch("tg_gate_score");
}
