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
constexpr int kTM = 64;                 // residual rows per workgroup (register-staged kernel)
constexpr int kPitch = kKS + 8;         // LDS row pitch in bf16 (144 bytes)

constexpr int kMinWG = 2;               // workgroups per CU its registers are sized for

// FAST: d is a multiple of 2 * kKS, so every stage is full; per-lane load
// offsets are fixed and the stage advance is the instruction's scalar offset.
template <int TM, int NT, bool HAS_GAMMA, bool FAST>
__global__ __launch_bounds__(256, kMinWG) void gate_bf16_kernel(
    const uint16_t* __restrict__ resid, int64_t ld_x, const uint8_t* __restrict__ prunable,
    const float* __restrict__ gamma, float eps, const uint16_t* __restrict__ w1,
    const float* __restrict__ b1, const float* __restrict__ w2, float b2,
    float* __restrict__ scores, int32_t T, int32_t d, const int32_t* __restrict__ t_dyn) {
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
  if (t_dyn != nullptr) {   // the prompt's length, read at run time (T is the capacity)
    T = min(T, max(*t_dyn, 0));
    if (row0 >= T) return;
  }

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
  // FAST: stages are walked in a rotated order per workgroup (see the DMA
  // kernel: power-of-two row strides put one k slice in few L2 channels).
  const int rot = FAST ? static_cast<int>((blockIdx.x >> 3) % static_cast<uint32_t>(nstages)) : 0;
  auto phys = [&](int s) { const int k = s + rot; return k >= nstages ? k - nstages : k; };
  auto load_x = [&](int s, u32x4 (&dst)[RPT]) {
    if (FAST) {
      const int ps = phys(s);
#pragma unroll
      for (int i = 0; i < RPT; ++i)   // streamed once (non-temporal)
        dst[i] = __builtin_amdgcn_raw_buffer_load_b128(x_rs, xoff[i], ps * kKS * 2, 2);
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
      const int k = (FAST ? phys(s) : s) * kKS + chunk * 8;   // past d: x is zero
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
        const int ps = phys(s);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          w[nt][kk] = __builtin_amdgcn_raw_buffer_load_b128(w_rs, woff[nt] + kk * 64,
                                                            ps * kKS * 2, 0);
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

// ---------------------------------------------------------------------------
// Streaming pipeline (no RMSNorm weight, d % 64 == 0, d >= 128).  Measured on
// gfx950, the register/LDS kernel above is bound by on-chip traffic rather
// than by HBM: every workgroup re-reads all of W1 from L2, and routing both
// operands through LDS puts more bytes through the LDS port than the MFMA
// pipes can use.  This kernel gives each operand the path that moves it once:
//   * the residual tile (64 rows, shared by every wave) goes HBM -> LDS with
//     gfx950's direct-to-LDS loads, 1 KiB MFMA A fragments in lane order,
//     into a ring of DEPTH+1 64-k stages, DEPTH of them in flight;
//   * each wave owns NTW 16-column tiles of h and streams only its own W1
//     B fragments straight into registers, DEPTH stages ahead, never through
//     LDS.  W1 is read either row-major ([h, d]) or in the packed layout that
//     tg_gate_pack_w1 writes, where one stage's fragments are one contiguous
//     block (row-major fragments gather 16 rows 4 KiB apart);
//   * LDS traffic per stage is the tile written once and read by each wave:
//     (1 + NW) * 8 KiB, against 16 MFMAs per wave.
// The compiler does not track the direct loads, so waits are explicit.  The
// A fragments are read one stage ahead: during stage s a wave waits for its
// own loads of stage s+1 (s_waitcnt vmcnt), one barrier makes every wave's
// stage s+1 visible (and frees the slot of stage s-1), and the wave reads
// stage s+1's fragments before issuing stage s's MFMAs, whose fragments it
// read in stage s-1.  The row's sum of squares comes from the A fragments.
// ---------------------------------------------------------------------------
__device__ __forceinline__ constexpr int vmcnt_imm(int n) {
  return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14);   // lgkmcnt/expcnt: no wait
}
constexpr int kLgkm0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);    // lgkmcnt(0) only

constexpr int kDepth = 4;               // k-stages in flight in the streaming kernel

template <int RT>
struct XSlot {
  u32x4 b[8 * RT][64];   // (row tile mt, k half kk) -> block mt*2+kk, lane order
};

// Packed W1 (tg_gate_pack_w1): for stage ks = k / 64, column tile ht = n / 16
// and k half kk, a 1 KiB block whose lane l holds W1[16 ht + l % 16]
// [64 ks + 32 kk + 8 (l / 16) + e], e = 0..7.  Block (ks, ht, kk) starts at
// element ((ks * (h / 16) + ht) * 2 + kk) * 512.
__host__ __device__ constexpr int64_t packed_block(int64_t ks, int64_t ht, int64_t kk, int64_t h) {
  return ((ks * (h / 16) + ht) * 2 + kk) * 512;
}

// SiLU(z) = z / (1 + e^-z) from the hardware base-2 exponential and
// reciprocal (each within a few ulp): e^-z = 2^(-z log2 e).  Large |z| stays
// finite: 2^+big = inf gives z * 0 = -0, 2^-big = 0 gives z.
__device__ __forceinline__ float silu_fast(float z) {
  constexpr float kLog2e = 1.4426950408889634f;
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// NST > 0 fixes the number of 64-k stages (d = 64 * NST) at compile time; the
// stages are then fully unrolled.  Either way every ring index is a
// compile-time constant, so the slots are distinct LDS objects and the W1
// register sets distinct registers: the compiler never merges their waits.
// RT: 64-row tiles per workgroup.  Each workgroup streams all of W1 through
// its CU once, so RT = 2 (128 rows) halves W1's traffic per row and RT = 4
// (256 rows) quarters it, with 2 or 4 times the matrix work per stage and
// barrier; their A fragments are read in the stage that uses them rather
// than one stage ahead, which would not fit the registers.  At RT = 4 a
// stage's residual slot is 32 KiB and the accumulators take 128 registers,
// so two stages are in flight (three slots), not four.
// OCC = 2: two 64-row workgroups share each CU (at most 128 registers per
// lane), each with two stages in flight and its A fragments read in the
// stage that uses them; one workgroup's barrier and load waits then overlap
// the other's matrix work.
template <int NTW, int NW, int NST, bool PACKED, int RT = 1, int OCC = 1>
__global__ __launch_bounds__(NW * 64, OCC) void gate_bf16_stream_kernel(
    const uint16_t* __restrict__ resid, int64_t ld_x, const uint8_t* __restrict__ prunable,
    float eps, const uint16_t* __restrict__ w1, const float* __restrict__ b1,
    const float* __restrict__ w2, float b2, float* __restrict__ scores, int32_t T, int32_t d,
    int32_t h, const int32_t* __restrict__ t_dyn) {
  constexpr int TM = 64 * RT;
  constexpr int MT = 4 * RT;                   // 16-row tiles
  constexpr int DEPTH = (RT == 4 || OCC == 2) ? 2 : kDepth;
  constexpr int R = DEPTH + 1;                 // ring length
  constexpr int XPW = 8 * RT / NW;             // residual blocks each wave loads per stage
  constexpr int PER_STAGE = XPW + 2 * NTW;     // vector-memory instructions per wave per stage
  constexpr bool AHEAD = RT == 1 && OCC == 1;  // A fragments read one stage ahead
  // sum of squares: with 8 waves over 4 row tiles, wave w takes row tile
  // w & 3, k half w >> 2; otherwise wave w takes row tile w, both halves
  constexpr bool SS_HALVES = NW == 8 && RT == 1;
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(RT == 1 || ((RT == 2 || RT == 4) && NW == 8), "128/256-row tiles with 8 waves");
  static_assert(OCC == 1 || (OCC == 2 && RT == 1 && NW == 8), "two workgroups per CU: 64 rows, 8 waves");
  static_assert(DEPTH >= 2 && R <= 8 && PER_STAGE * (DEPTH - 1) <= 63, "ring shape");
  using XS = XSlot<RT>;
  __shared__ __attribute__((aligned(16))) XS xs0, xs1, xs2, xs3, xs4, xs5, xs6, xs7;
  __shared__ float s_ss[2][TM];
  __shared__ float s_rs[TM];
  __shared__ float s_part[NW][TM];
  __shared__ int s_any;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lrow = lane & 15;
  const int lgrp = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * TM;
  if (t_dyn != nullptr) {   // the prompt's length, read at run time (T is the capacity)
    T = min(T, max(*t_dyn, 0));
    if (row0 >= T) return;
  }

  if (tid == 0) s_any = 0;
  __syncthreads();
  if (tid < TM && row0 + tid < T && prunable[row0 + tid]) s_any = 1;
  __syncthreads();
  if (!s_any) {
    if (tid < TM && row0 + tid < T) scores[row0 + tid] = 0.0f;
    return;
  }

  // residual blocks wave*XPW + i: row tile (block >> 1), k half (block & 1).
  // Rows past T re-read row T-1 (valid memory); their scores are never stored.
  static_assert(XPW <= 4, "residual blocks per wave: xsrc holds four");
  const uint16_t* xsrc[4];   // XPW <= 4 (a fixed size: the direct-load builtin rejects a dependent type)
#pragma unroll
  for (int i = 0; i < XPW; ++i) {
    const int blk = wave * XPW + i;
    const int64_t r = row0 + 16 * (blk >> 1) + lrow;
    xsrc[i] = resid + (r < T ? r : T - 1) * ld_x + 32 * (blk & 1) + 8 * lgrp;
  }
  // W1 through a buffer resource (offsets are 32-bit; the host checks h*d*2)
  const __amdgpu_buffer_rsrc_t w_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(w1), 0, static_cast<int>(static_cast<uint32_t>(h) * d * 2u),
      0x00020000);
  const int ht0 = wave * NTW;   // this wave's first 16-column tile
  uint32_t woff;                // byte offset of this lane's fragment of (stage 0, ht0, kk 0)
  if (PACKED)
    woff = static_cast<uint32_t>(packed_block(0, ht0, 0, h)) * 2u + lane * 16u;
  else
    woff = (static_cast<uint32_t>(16 * ht0 + lrow) * static_cast<uint32_t>(d) + 8 * lgrp) * 2u;
  // byte step between the wave's fragments (nt, kk) and between stages
  const uint32_t w_nt = PACKED ? 2048u : 32u * static_cast<uint32_t>(d);
  const uint32_t w_kk = PACKED ? 1024u : 64u;
  const uint32_t w_ks = PACKED ? static_cast<uint32_t>(h) * 128u : 128u;

  const int nstages = NST > 0 ? NST : d / kKS;
  // Each workgroup walks the k stages in a rotated order, so the workgroups
  // of an XCD (block ids 8 apart) read different parts of W1 at a time.
  const int rot = static_cast<int>((blockIdx.x >> 3) % static_cast<uint32_t>(nstages));

  u32x4 wr[R][NTW][2];   // W1 fragments, one set per ring slot
  auto issue = [&](int st, XS& sl, u32x4 (&w)[NTW][2]) {
    int ks = st + rot;
    ks = ks >= nstages ? ks - nstages : ks;
#pragma unroll
    for (int i = 0; i < XPW; ++i)
      __builtin_amdgcn_global_load_lds(xsrc[i] + ks * kKS,
                                       (__attribute__((address_space(3))) void*)&sl.b[wave * XPW + i][0],
                                       16, 0, 0);
    const uint32_t so = static_cast<uint32_t>(ks) * w_ks;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        w[nt][kk] = __builtin_amdgcn_raw_buffer_load_b128(w_rs, woff + nt * w_nt + kk * w_kk, so, 0);
  };
  auto wait_own = [&](int ahead) {   // own loads of a stage done; `ahead` later stages may be in flight
    switch (ahead) {
      case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
      case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_STAGE)); break;
      case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PER_STAGE)); break;
      case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * PER_STAGE)); break;
      case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * PER_STAGE)); break;
      case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5 * PER_STAGE)); break;
      default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(6 * PER_STAGE)); break;
    }
  };

  f32x4 acc[MT][NTW];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) acc[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Row sums of squares on the matrix cores: an A fragment times itself
  // (as B) puts sum_k x_r,k^2 on the diagonal of the 16x16 product.  The
  // products of bf16 values are exact in fp32, as on the vector ALUs.  With 8
  // waves, wave w takes row tile w & 3 and k half w >> 2 of every stage; with
  // 4 waves, wave w takes row tile w and both k halves.
  // (256-row tiles: wave w takes row tiles w and w + 8.)
  constexpr int SST = SS_HALVES ? 1 : MT / NW;   // sum-of-squares row tiles per wave
  f32x4 acc_ss[SST];
#pragma unroll
  for (int j = 0; j < SST; ++j) acc_ss[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int ss_tile = SS_HALVES ? (wave & 3) : wave;
  const int ss_half = SS_HALVES ? (wave >> 2) : 0;

  // One stage ahead: stage s's A fragments (and this wave's sum-of-squares
  // fragment) sit in registers, read during stage s-1, so the LDS latency of
  // a stage's reads and the barrier before them overlap the previous stage's
  // MFMAs instead of preceding this stage's.
  u32x4 av[2][4];
  u32x4 mine[2];   // the sum-of-squares fragments (one or both k halves)
  constexpr int NSS = SS_HALVES ? 1 : 2;
  auto read_frags = [&](const XS& sl, u32x4 (&a)[2][4], u32x4 (&mn)[2]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int m = 0; m < 4; ++m) a[kk][m] = sl.b[m * 2 + kk][lane];
#pragma unroll
    for (int i = 0; i < NSS; ++i) mn[i] = sl.b[ss_tile * 2 + (SS_HALVES ? ss_half : i)][lane];
  };
  auto stage = [&](int s, const XS& sl_cur, const XS& sl_next, const u32x4 (&wc)[NTW][2],
                   XS& nsl, u32x4 (&wn)[NTW][2]) {
    const int last = nstages - 1;
    if constexpr (!AHEAD) {
      // this wave's loads of stage s are done (later stages may be in
      // flight); after the barrier every wave's stage s has landed and stage
      // s-1's slot is free for stage s + DEPTH
      (void)sl_next;
      wait_own(s + DEPTH - 1 <= last ? DEPTH - 1 : last - s);
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_s_barrier();
      if (s + DEPTH <= last) issue(s + DEPTH, nsl, wn);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < SST; ++j)
#pragma unroll
        for (int i = 0; i < NSS; ++i) {
          const u32x4 mn = sl_cur.b[(ss_tile + j * NW) * 2 + (SS_HALVES ? ss_half : i)][lane];
          acc_ss[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, mn),
                                                              __builtin_bit_cast(bf16x8, mn),
                                                              acc_ss[j], 0, 0, 0);
        }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const u32x4 a = sl_cur.b[m * 2 + kk][lane];
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt)
            acc[m][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, wc[nt][kk]),
                acc[m][nt], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      return;
    }
    u32x4 an[2][4];
    u32x4 mn[2];
    if (s < last) {
      // this wave's loads of stage s+1 are done (later stages may still be in
      // flight) and its reads of stage s have returned; after the barrier
      // every wave's stage s+1 has landed, and stage s-1's slot is free
      wait_own(s + DEPTH - 1 <= last ? DEPTH - 2 : last - s - 1);
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_s_barrier();
      read_frags(sl_next, an, mn);
    }
    if (s + DEPTH <= last) issue(s + DEPTH, nsl, wn);
    // keep the reads and the prefetch issued here, ahead of this stage's MFMAs
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NSS; ++i)
      acc_ss[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, mine[i]),
                                                          __builtin_bit_cast(bf16x8, mine[i]),
                                                          acc_ss[0], 0, 0, 0);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
          if constexpr (AHEAD)
            acc[m][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, av[kk][m]), __builtin_bit_cast(bf16x8, wc[nt][kk]),
                acc[m][nt], 0, 0, 0);
    }
    // every MFMA of this stage is issued before the next stage's barrier: a
    // wave waiting there has its matrix work queued behind it
    __builtin_amdgcn_sched_barrier(0);
    if (s < last) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int m = 0; m < 4; ++m) av[kk][m] = an[kk][m];
#pragma unroll
      for (int i = 0; i < 2; ++i) mine[i] = mn[i];
    }
  };
  // slot j of the ring: LDS object xs<j>, register set wr[j]
#define TG_SLOT(X)                                                                  \
  ((X) == 0 ? xs0 : (X) == 1 ? xs1 : (X) == 2 ? xs2 : (X) == 3 ? xs3 : (X) == 4 ? xs4 \
   : (X) == 5 ? xs5 : (X) == 6 ? xs6 : xs7)
#define TG_STAGE_SLOT(S, J)                                                    \
  stage((S), TG_SLOT(J), TG_SLOT((J + 1) % R), wr[J], TG_SLOT((J + DEPTH) % R), \
        wr[(J + DEPTH) % R])
  auto run = [&](int s, int j) {   // j == s % R, a constant after unrolling
    switch (j) {
      case 0: TG_STAGE_SLOT(s, 0); break;
      case 1: TG_STAGE_SLOT(s, 1); break;
      case 2: TG_STAGE_SLOT(s, 2); break;
      case 3: if constexpr (R > 3) TG_STAGE_SLOT(s, 3); break;
      case 4: if constexpr (R > 4) TG_STAGE_SLOT(s, 4); break;
      case 5: if constexpr (R > 5) TG_STAGE_SLOT(s, 5); break;
      case 6: if constexpr (R > 6) TG_STAGE_SLOT(s, 6); break;
      default: if constexpr (R > 7) TG_STAGE_SLOT(s, 7); break;
    }
  };
#undef TG_STAGE_SLOT
#undef TG_SLOT
  // prologue: stages 0 .. DEPTH-1 in flight (nstages >= 2; later ones guarded),
  // then stage 0's fragments into registers
  issue(0, xs0, wr[0]);
  issue(1, xs1, wr[1]);
  if constexpr (DEPTH > 2) if (2 < nstages) issue(2, xs2, wr[2 % R]);
  if constexpr (DEPTH > 3) if (3 < nstages) issue(3, xs3, wr[3 % R]);
  if constexpr (DEPTH > 4) if (4 < nstages) issue(4, xs4, wr[4 % R]);
  if constexpr (DEPTH > 5) if (5 < nstages) issue(5, xs5, wr[5 % R]);
  if constexpr (DEPTH > 6) if (6 < nstages) issue(6, xs6, wr[6 % R]);
  if constexpr (AHEAD) {
    wait_own(nstages - 1 < DEPTH - 1 ? nstages - 1 : DEPTH - 1);
    __builtin_amdgcn_s_barrier();
    read_frags(xs0, av, mine);
  }
  if constexpr (NST > 0) {
#pragma unroll
    for (int s = 0; s < NST; ++s) run(s, s % R);
  } else {
    for (int s0 = 0; s0 < nstages; s0 += R) {
#pragma unroll
      for (int j = 0; j < R; ++j)
        if (s0 + j < nstages) run(s0 + j, j);
    }
  }

  // lane l holds rows 4 (l >> 4) + r, column l & 15 of the product: the
  // diagonal entry of row i is lane 16 (i >> 2) + i, register i & 3
  if (((lane & 15) >> 2) == lgrp) {
    const int r = lane & 3;
#pragma unroll
    for (int j = 0; j < SST; ++j) {
      const f32x4 a = acc_ss[j];
      const float v = r == 0 ? a[0] : r == 1 ? a[1] : r == 2 ? a[2] : a[3];
      s_ss[ss_half][(ss_tile + j * NW) * 16 + (lane & 15)] = v;
    }
  }
  if (!SS_HALVES && tid < TM) s_ss[1][tid] = 0.0f;
  __syncthreads();
  if (tid < TM) s_rs[tid] = 1.0f / sqrtf((s_ss[0][tid] + s_ss[1][tid]) / static_cast<float>(d) + eps);
  __syncthreads();

  float part[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) part[m][r] = 0.0f;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int n = (ht0 + nt) * 16 + lrow;
    const float bb = b1 ? b1[n] : 0.0f;
    const float ww = w2[n];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float z = fmaf(acc[m][nt][r], s_rs[m * 16 + lgrp * 4 + r], bb);
        part[m][r] = fmaf(ww, silu_fast(z), part[m][r]);
      }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = part[m][r];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      v += __shfl_xor(v, 8, 64);
      if (lrow == 0) s_part[wave][m * 16 + lgrp * 4 + r] = v;
    }
  __syncthreads();
  if (tid < TM) {
    const int64_t t = row0 + tid;
    if (t < T) {
      float sc = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; w += 2) sc += s_part[w][tid] + s_part[w + 1][tid];
      scores[t] = prunable[t] ? b2 + sc : 0.0f;
    }
  }
}

// tg_gate_pack_w1: one thread per 16-byte fragment of the packed layout.
__global__ void gate_pack_w1_kernel(const uint16_t* __restrict__ w1, uint16_t* __restrict__ out,
                                    int32_t h, int32_t d) {
  const int64_t f = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;   // fragment
  const int64_t nfrag = static_cast<int64_t>(h) * d / 8;
  if (f >= nfrag) return;
  const int l = static_cast<int>(f & 63);
  const int64_t blk = f >> 6;                 // ((ks * (h/16) + ht) * 2 + kk)
  const int kk = static_cast<int>(blk & 1);
  const int64_t ht = (blk >> 1) % (h / 16);
  const int64_t ks = (blk >> 1) / (h / 16);
  const int64_t row = 16 * ht + (l & 15);
  const int64_t col = 64 * ks + 32 * kk + 8 * (l >> 4);
  *reinterpret_cast<u32x4*>(out + f * 8) = *reinterpret_cast<const u32x4*>(w1 + row * d + col);
}

// ---------------------------------------------------------------------------
// fp32 path: one wave per row.  u = gamma*x/rms is formed on the fly;
// lane j accumulates z_j over the row (x broadcast from L1), then the wave
// reduces w2 . SiLU(z) across lanes.
__global__ __launch_bounds__(256) void gate_f32_kernel(
    const float* __restrict__ resid, int64_t ld_x, const uint8_t* __restrict__ prunable,
    const float* __restrict__ gamma, float eps, const float* __restrict__ w1,
    const float* __restrict__ b1, const float* __restrict__ w2, float b2,
    float* __restrict__ scores, int32_t T, int32_t d, int32_t h,
    const int32_t* __restrict__ t_dyn) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t_dyn != nullptr) T = min(T, max(*t_dyn, 0));   // run-time length (T: capacity)
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
                   const float* b1, const float* w2, float b2, float* out, int32_t d,
                   const int32_t* t_dyn) {
  if (has_gamma)
    gate_bf16_kernel<TM, NT, true, FAST><<<grid, dim3(256), static_cast<size_t>(d) * 4, s>>>(
        x, ld, p, g, eps, w1, b1, w2, b2, out, static_cast<int32_t>(T), d, t_dyn);
  else
    gate_bf16_kernel<TM, NT, false, FAST><<<grid, dim3(256), 0, s>>>(
        x, ld, p, g, eps, w1, b1, w2, b2, out, static_cast<int32_t>(T), d, t_dyn);
}

template <int TM, int NT>
void launch_bf16(bool has_gamma, int64_t T, dim3 grid, hipStream_t s, const uint16_t* x,
                 int64_t ld, const uint8_t* p, const float* g, float eps, const uint16_t* w1,
                 const float* b1, const float* w2, float b2, float* out, int32_t d,
                 const int32_t* t_dyn) {
  if (d % (2 * kKS) == 0)
    launch_bf16_f<TM, NT, true>(has_gamma, T, grid, s, x, ld, p, g, eps, w1, b1, w2, b2, out, d,
                                t_dyn);
  else
    launch_bf16_f<TM, NT, false>(has_gamma, T, grid, s, x, ld, p, g, eps, w1, b1, w2, b2, out,
                                 d, t_dyn);
}

// Streaming kernel dispatch: h = 16 * NTW * NW.  At h = 256 a prompt long
// enough for two rounds of 256-row (or 128-row) workgroups on every CU takes
// those tiles (a quarter or half of the W1 traffic per row); shorter ones
// keep 64-row tiles, so that every CU still gets a workgroup, two at a time
// when there are at least two per CU (32k tokens: 5-8% faster than one).
void launch_stream(bool packed, int64_t T, int64_t h, int32_t d, hipStream_t s,
                   const uint16_t* x, int64_t ld, const uint8_t* p, float eps,
                   const uint16_t* w, const float* b1, const float* w2, float b2, float* out,
                   const int32_t* t_dyn) {
  const int32_t T32 = static_cast<int32_t>(T), h32 = static_cast<int32_t>(h);
  const int64_t cus = device_cu_count();
  const bool rows256 = h == 256 && (T + 255) / 256 >= 2 * cus;
  const bool rows128 = h == 256 && (T + 127) / 128 >= 2 * cus;
  const bool two64 = h == 256 && (T + 63) / 64 >= 2 * cus;
#define TG_GATE_STREAM(NTW, NW, NST, RT, OCC)                                                \
  do {                                                                                      \
    const dim3 grid(static_cast<uint32_t>((T + 64 * RT - 1) / (64 * RT)));                  \
    if (packed)                                                                             \
      gate_bf16_stream_kernel<NTW, NW, NST, true, RT, OCC><<<grid, dim3(NW * 64), 0, s>>>(  \
          x, ld, p, eps, w, b1, w2, b2, out, T32, d, h32, t_dyn);                           \
    else                                                                                    \
      gate_bf16_stream_kernel<NTW, NW, NST, false, RT, OCC><<<grid, dim3(NW * 64), 0, s>>>( \
          x, ld, p, eps, w, b1, w2, b2, out, T32, d, h32, t_dyn);                           \
  } while (0)
  if (h == 256 && d == 2048) {   // Qwen3-1.7B hidden size, h = 256
    // two 64-row workgroups per CU also below the 256-row threshold: at
    // 65536 tokens they measured 81.5 us against 92.7 us for 128-row tiles
    if (rows256) TG_GATE_STREAM(2, 8, 32, 4, 1);
    else if (two64) TG_GATE_STREAM(2, 8, 32, 1, 2);
    else TG_GATE_STREAM(2, 8, 32, 1, 1);
  } else if (h == 256) {
    if (rows256) TG_GATE_STREAM(2, 8, 0, 4, 1);
    else if (rows128) TG_GATE_STREAM(2, 8, 0, 2, 1);
    else if (two64) TG_GATE_STREAM(2, 8, 0, 1, 2);
    else TG_GATE_STREAM(2, 8, 0, 1, 1);
  } else if (h == 192) TG_GATE_STREAM(3, 4, 0, 1, 1);
  else if (h == 128) TG_GATE_STREAM(2, 4, 0, 1, 1);
  else TG_GATE_STREAM(1, 4, 0, 1, 1);
#undef TG_GATE_STREAM
}

}  // namespace

tg_status gate_score_call(const char* fn, tg_dtype dt, int64_t T, int64_t d, int64_t h,
                          const void* resid, int64_t resid_row_stride, const uint8_t* prunable,
                          const float* rms_weight, float eps, const void* w1, bool packed,
                          const float* b1, const float* w2, float b2, float* scores,
                          void* stream, const int32_t* t_dyn) {
  if (dt != TG_DTYPE_F32 && dt != TG_DTYPE_BF16)
    return fail(TG_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", fn, (int)dt);
  if (T < 0 || T > kMaxTokens || d < 1 || h < 1 || d > kMaxTokens || h > kMaxTokens)
    return fail(TG_ERR_INVALID_ARGUMENT,
                "%s: need 0 <= T <= 2^31-1, d >= 1, h >= 1 (T=%lld d=%lld h=%lld)", fn,
                (long long)T, (long long)d, (long long)h);
  if (!(eps >= 0.0f)) return fail(TG_ERR_INVALID_ARGUMENT, "%s: eps must be >= 0", fn);
  if (packed) {
    if (dt != TG_DTYPE_BF16)
      return fail(TG_ERR_UNSUPPORTED, "%s: packed W1 is a bf16 layout", fn);
    if (d % kKS != 0 || d < 2 * kKS || h % 64 != 0 || h > 256)
      return fail(TG_ERR_UNSUPPORTED,
                  "%s: packed W1 needs d %% 64 == 0, d >= 128, h in {64, 128, 192, 256} "
                  "(d=%lld h=%lld)", fn, (long long)d, (long long)h);
    if (rms_weight != nullptr)
      return fail(TG_ERR_UNSUPPORTED,
                  "%s: packed W1 takes no RMSNorm weight (pass NULL for a unit weight)", fn);
  }
  if (T == 0) {
    clear_error();
    return TG_OK;
  }
  if (!resid || !prunable || !w1 || !w2 || !scores)
    return fail(TG_ERR_INVALID_ARGUMENT, "%s: NULL resid/prunable/w1/w2/scores", fn);
  if (resid_row_stride < d)
    return fail(TG_ERR_INVALID_ARGUMENT, "%s: resid_row_stride %lld < d %lld", fn,
                (long long)resid_row_stride, (long long)d);
  hipStream_t s = as_stream(stream);
  if (dt == TG_DTYPE_F32) {
    if (!aligned(resid, 4) || !aligned(w1, 4))
      return fail(TG_ERR_INVALID_ARGUMENT, "%s: misaligned f32 pointer", fn);
    const int64_t blocks = (T + 3) / 4;
    gate_f32_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s>>>(
        static_cast<const float*>(resid), resid_row_stride, prunable, rms_weight, eps,
        static_cast<const float*>(w1), b1, w2, b2, scores, static_cast<int32_t>(T),
        static_cast<int32_t>(d), static_cast<int32_t>(h), t_dyn);
    return check_launch(fn);
  }
  if (d % 8 != 0)
    return fail(TG_ERR_UNSUPPORTED, "%s: bf16 path needs d %% 8 == 0 (d=%lld)", fn, (long long)d);
  if (h % 64 != 0 || h > 256)
    return fail(TG_ERR_UNSUPPORTED, "%s: bf16 path needs h in {64, 128, 192, 256} (h=%lld)", fn,
                (long long)h);
  if (rms_weight != nullptr && d > 16384)
    return fail(TG_ERR_UNSUPPORTED,
                "%s: bf16 path with an RMSNorm weight needs d <= 16384 (LDS-staged)", fn);
  if (static_cast<int64_t>(kTM) * resid_row_stride * 2 > kMaxTokens || h * d * 2 > kMaxTokens)
    return fail(TG_ERR_UNSUPPORTED,
                "%s: bf16 path addresses a 64-row tile and W1 with 31-bit offsets", fn);
  if (!aligned(resid, 16) || !aligned(w1, 16) || (resid_row_stride % 8) != 0)
    return fail(TG_ERR_INVALID_ARGUMENT,
                "%s: bf16 resid/w1 must be 16-byte aligned, row stride %% 8 == 0", fn);
  const auto* x = static_cast<const uint16_t*>(resid);
  const auto* w = static_cast<const uint16_t*>(w1);
  const int32_t d32 = static_cast<int32_t>(d);
  if (packed) {
    launch_stream(true, T, h, d32, s, x, resid_row_stride, prunable, eps, w, b1, w2, b2, scores,
                  t_dyn);
    return check_launch(fn);
  }
  if (rms_weight == nullptr && d % kKS == 0 && d >= 2 * kKS) {
    launch_stream(false, T, h, d32, s, x, resid_row_stride, prunable, eps, w, b1, w2, b2, scores,
                  t_dyn);
    return check_launch(fn);
  }
  const bool g = rms_weight != nullptr;
  constexpr int TM = kTM;
  const dim3 grid(static_cast<uint32_t>((T + TM - 1) / TM));
  switch (h / 64) {
    case 1: launch_bf16<TM, 1>(g, T, grid, s, x, resid_row_stride, prunable, rms_weight, eps, w, b1, w2, b2, scores, d32, t_dyn); break;
    case 2: launch_bf16<TM, 2>(g, T, grid, s, x, resid_row_stride, prunable, rms_weight, eps, w, b1, w2, b2, scores, d32, t_dyn); break;
    case 3: launch_bf16<TM, 3>(g, T, grid, s, x, resid_row_stride, prunable, rms_weight, eps, w, b1, w2, b2, scores, d32, t_dyn); break;
    default: launch_bf16<TM, 4>(g, T, grid, s, x, resid_row_stride, prunable, rms_weight, eps, w, b1, w2, b2, scores, d32, t_dyn); break;
  }
  return check_launch(fn);
}

}  // namespace tg

extern "C" tg_status tg_gate_score(tg_dtype dt, int64_t T, int64_t d, int64_t h,
                                   const void* resid, int64_t resid_row_stride,
                                   const uint8_t* prunable, const float* rms_weight, float eps,
                                   const void* w1, const float* b1, const float* w2, float b2,
                                   float* scores, void* stream) {
  return tg::gate_score_call("tg_gate_score", dt, T, d, h, resid, resid_row_stride, prunable,
                             rms_weight, eps, w1, false, b1, w2, b2, scores, stream, nullptr);
}

extern "C" tg_status tg_gate_score_packed(tg_dtype dt, int64_t T, int64_t d, int64_t h,
                                          const void* resid, int64_t resid_row_stride,
                                          const uint8_t* prunable, const float* rms_weight,
                                          float eps, const void* w1_packed, const float* b1,
                                          const float* w2, float b2, float* scores,
                                          void* stream) {
  return tg::gate_score_call("tg_gate_score_packed", dt, T, d, h, resid, resid_row_stride,
                             prunable, rms_weight, eps, w1_packed, true, b1, w2, b2, scores,
                             stream, nullptr);
}

extern "C" size_t tg_gate_w1_packed_bytes(tg_dtype dt, int64_t h, int64_t d) {
  if (dt != TG_DTYPE_BF16 || h < 64 || h > 256 || h % 64 != 0 || d < 128 || d % 64 != 0 ||
      d > tg::kMaxTokens)
    return 0;
  return static_cast<size_t>(h) * static_cast<size_t>(d) * 2u;
}

extern "C" tg_status tg_gate_pack_w1(tg_dtype dt, int64_t h, int64_t d, const void* w1,
                                     void* w1_packed, void* stream) {
  using namespace tg;
  const size_t bytes = tg_gate_w1_packed_bytes(dt, h, d);
  if (bytes == 0)
    return fail(TG_ERR_UNSUPPORTED,
                "tg_gate_pack_w1: needs bf16, d %% 64 == 0, d >= 128, h in {64, 128, 192, 256} "
                "(dt=%d h=%lld d=%lld)", (int)dt, (long long)h, (long long)d);
  if (static_cast<int64_t>(bytes) > kMaxTokens)
    return fail(TG_ERR_UNSUPPORTED, "tg_gate_pack_w1: W1 must stay below 2^31 bytes");
  if (!w1 || !w1_packed)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_gate_pack_w1: NULL w1/w1_packed");
  if (!aligned(w1, 16) || !aligned(w1_packed, 16))
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_gate_pack_w1: pointers must be 16-byte aligned");
  const int64_t nfrag = static_cast<int64_t>(bytes / 16);
  gate_pack_w1_kernel<<<dim3(static_cast<uint32_t>((nfrag + 255) / 256)), dim3(256), 0,
                        as_stream(stream)>>>(static_cast<const uint16_t*>(w1),
                                             static_cast<uint16_t*>(w1_packed),
                                             static_cast<int32_t>(h), static_cast<int32_t>(d));
  return check_launch("tg_gate_pack_w1");
}
