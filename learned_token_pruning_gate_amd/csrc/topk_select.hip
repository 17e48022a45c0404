// topk_select.hip -- [a2] radix top-K threshold over the prunable tokens'
// scores and [a3] order-preserving compaction of the kept set.
//
// TokenGate pages: ai.info summary "Key Contributions" item 1 and
// "Methodology in Plain English" -- the gate keeps its K best prunable
// tokens plus every non-prunable token; the README mirror's "Quick start"
// budget None keeps every prunable token.
//
// Design (gfx950).  Scores become order-preserving u32 keys (NaN lowest,
// -0 == +0).  Three histogram passes over digits of 11, 11 and 10 bits find
// the K-th largest key v*: every workgroup builds an LDS histogram of the
// keys that still match the resolved prefix and adds it to a global one;
// the last workgroup to arrive (device-scope counter, no grid barrier)
// picks the digit whose bucket holds the K-th key and updates the prefix.
// A pass whose bucket is taken whole resolves early and the later passes
// exit at once.  Then one compaction kernel computes, per token,
//   a = !prunable || key > v*,   b = prunable && key == v*,
// and with exclusive prefix counts A, B (in token order) writes token t to
// slot A + min(B, need) when a, or when b and B < need (lower index wins
// ties).  The prefix counts across workgroups come from a single-pass
// decoupled look-back whose workgroup order is a ticket taken at start, so
// a workgroup only ever waits on workgroups that are already running.
//
// Workspace: global histograms, pass counters, the resolved state and the
// look-back descriptors.  It must start all-zero; the last workgroup of each
// pass clears what that pass used, so every call ends with it all-zero.  The
// first histogram pass also resets the compaction's ticket and descriptors.
#include "tg_common.hpp"

namespace tg {
namespace {

constexpr int kThreads = 256;
constexpr int kItems = 4;                        // consecutive tokens per thread
constexpr int kChunk = kThreads * kItems;        // tokens per workgroup sweep
constexpr int kMaxBlocks = 4096;

struct Control {
  uint32_t done[4];     // arrival counters: 3 histogram passes + compaction
  uint32_t ticket;      // compaction workgroup order
  uint32_t prefix;      // resolved high bits of v* (low bits zero)
  uint32_t mask;        // which bits of the key are resolved
  uint32_t need;        // prunable keys equal to prefix (under mask) to keep
  uint32_t resolved;    // selection fully determined
  uint32_t n_prunable;
  uint32_t pad[6];
};

constexpr size_t kHistOff[3] = {0, 2048 * 4, 4096 * 4};
constexpr size_t kCtrlOff = (4096 + 1024) * 4;
constexpr size_t kFlagOff = kCtrlOff + 256;

__host__ __device__ inline int64_t blocks_for(int64_t T, int64_t* per_block) {
  int64_t pb = (T + kMaxBlocks - 1) / kMaxBlocks;
  pb = ((pb + kChunk - 1) / kChunk) * kChunk;
  if (pb < kChunk) pb = kChunk;
  if (per_block) *per_block = pb;
  return T == 0 ? 1 : (T + pb - 1) / pb;
}

// fp32 score -> u32 key whose unsigned order is the numeric order; NaN maps
// below -inf and -0 maps to +0.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (s != s) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive block-wide sum scan (256 threads) of one u32 per thread.
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, uint32_t* s_wave,
                                                         uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  if (lane == 63) s_wave[wave] = v;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    const uint32_t x = s_wave[w];
    if (w < wave) base += x;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return base + v;
}

// ---------------------------------------------------------------------------
// Histogram pass PASS over digit bits [SHIFT, SHIFT + BITS).
// ---------------------------------------------------------------------------
template <int PASS>
__global__ __launch_bounds__(kThreads) void radix_hist_kernel(
    const float* __restrict__ scores, const uint8_t* __restrict__ prunable, int32_t T,
    int64_t per_block, uint32_t K, uint32_t n_compact_blocks, uint8_t* __restrict__ ws) {
  constexpr int BITS = PASS == 2 ? 10 : 11;
  constexpr int NB = 1 << BITS;
  constexpr int SHIFT = PASS == 0 ? 21 : (PASS == 1 ? 10 : 0);
  constexpr int BPT = NB / kThreads;  // bins per thread in the resolve step
  __shared__ uint32_t h[NB];
  __shared__ uint32_t s_wave[kThreads / 64];
  __shared__ int s_last;

  Control* ctl = reinterpret_cast<Control*>(ws + kCtrlOff);
  uint32_t* ghist = reinterpret_cast<uint32_t*>(ws + kHistOff[PASS]);
  if (PASS == 0 && blockIdx.x == 0) {
    // The compaction kernel's ticket and look-back descriptors are reset here
    // on every call (the compaction runs later on the same stream), so even a
    // workspace that was not zeroed can never make it wait on a descriptor
    // that nobody writes.
    uint64_t* flags = reinterpret_cast<uint64_t*>(ws + kFlagOff);
    for (uint32_t j = threadIdx.x; j < n_compact_blocks; j += kThreads) flags[j] = 0;
    if (threadIdx.x == 0) {
      ctl->ticket = 0;
      ctl->done[3] = 0;
    }
  }
  uint32_t prefix = 0, mask = 0;
  if (PASS > 0) {
    if (ctl->resolved) return;  // same value in every workgroup
    prefix = ctl->prefix;
    mask = ctl->mask;
  }
  for (int b = threadIdx.x; b < NB; b += kThreads) h[b] = 0;
  __syncthreads();

  const int64_t begin = static_cast<int64_t>(blockIdx.x) * per_block;
  const int64_t end = begin + per_block < T ? begin + per_block : T;
  for (int64_t base = begin; base < end; base += kChunk) {
    const int64_t t0 = base + static_cast<int64_t>(threadIdx.x) * kItems;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int64_t t = t0 + i;
      if (t < end && prunable[t]) {
        const uint32_t key = score_key(scores[t]);
        if ((key & mask) == prefix) atomicAdd(&h[(key >> SHIFT) & (NB - 1)], 1u);
      }
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < NB; b += kThreads)
    if (h[b]) atomicAdd(&ghist[b], h[b]);
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = atomicAdd(&ctl->done[PASS], 1u) == gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;

  // ---- last workgroup: resolve this digit --------------------------------
  __threadfence();
  for (int b = threadIdx.x; b < NB; b += kThreads) {
    h[b] = ld_agent(&ghist[b]);
    ghist[b] = 0;  // leave the workspace clean for the next call
  }
  __syncthreads();
  // Every thread reads the previous pass's need before the scan's barriers;
  // the resolving thread overwrites it afterwards.
  uint32_t need = PASS == 0 ? 0 : ctl->need;
  // thread i owns bins NB-1-i*BPT down to NB-(i+1)*BPT (descending keys)
  uint32_t mine = 0;
  const int top = NB - 1 - threadIdx.x * BPT;
#pragma unroll
  for (int j = 0; j < BPT; ++j) mine += h[top - j];
  uint32_t total = 0;
  const uint32_t incl = block_inclusive_scan(mine, s_wave, &total);
  const uint32_t above_me = incl - mine;  // keys in bins above mine

  if (PASS == 0) {
    // total = |P| (every prunable key matches the empty prefix)
    if (threadIdx.x == 0) {
      ctl->n_prunable = total;
      ctl->done[PASS] = 0;
      if (K >= total || K == 0) {  // keep all / keep none of the prunable tokens
        ctl->prefix = 0;
        ctl->mask = 0;
        ctl->need = K >= total ? total : 0;
        ctl->resolved = 1;
      }
    }
    if (K >= total || K == 0) return;
    need = K;
  } else if (threadIdx.x == 0) {
    ctl->done[PASS] = 0;
  }
  // the thread whose bins contain the need-th largest key resolves the digit
  if (above_me < need && need <= above_me + mine) {
    uint32_t cum = above_me;
    for (int j = 0; j < BPT; ++j) {
      const int b = top - j;
      const uint32_t c = h[b];
      if (cum + c >= need) {
        const uint32_t rest = need - cum;  // keys of bucket b still to keep
        ctl->prefix = prefix | (static_cast<uint32_t>(b) << SHIFT);
        ctl->mask = mask | (static_cast<uint32_t>(NB - 1) << SHIFT);
        ctl->need = rest;
        ctl->resolved = (rest == c || PASS == 2) ? 1u : 0u;
        break;
      }
      cum += c;
    }
  }
}

// ---------------------------------------------------------------------------
// Order-preserving compaction with a ticket-ordered decoupled look-back.
// ---------------------------------------------------------------------------
constexpr uint64_t kFlagAgg = 1ull << 62;
constexpr uint64_t kFlagIncl = 2ull << 62;
constexpr uint64_t kMask31 = (1ull << 31) - 1;

__device__ __forceinline__ uint64_t pack_desc(uint64_t flag, uint32_t a, uint32_t b) {
  return flag | (static_cast<uint64_t>(a) << 31) | static_cast<uint64_t>(b);
}

__global__ __launch_bounds__(kThreads) void compact_kernel(
    const float* __restrict__ scores, const uint8_t* __restrict__ prunable, int32_t T,
    int64_t per_block, uint8_t* __restrict__ ws, int32_t* __restrict__ kept_idx,
    int64_t capacity, int32_t* __restrict__ n_kept) {
  __shared__ uint32_t s_wave[kThreads / 64];
  __shared__ uint32_t s_ticket;
  __shared__ uint32_t s_pre_a, s_pre_b;
  __shared__ int s_last;

  Control* ctl = reinterpret_cast<Control*>(ws + kCtrlOff);
  uint64_t* flags = reinterpret_cast<uint64_t*>(ws + kFlagOff);
  const uint32_t prefix = ctl->prefix, mask = ctl->mask, need = ctl->need;

  if (threadIdx.x == 0) s_ticket = atomicAdd(&ctl->ticket, 1u);
  __syncthreads();
  const uint32_t w = s_ticket;
  const int64_t begin = static_cast<int64_t>(w) * per_block;
  const int64_t end = begin + per_block < T ? begin + per_block : T;

  // (1) this workgroup's counts of a and b
  uint32_t ca = 0, cb = 0;
  for (int64_t base = begin; base < end; base += kChunk) {
    const int64_t t0 = base + static_cast<int64_t>(threadIdx.x) * kItems;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int64_t t = t0 + i;
      if (t < end) {
        if (!prunable[t]) {
          ++ca;
        } else {
          const uint32_t km = score_key(scores[t]) & mask;
          ca += km > prefix;
          cb += km == prefix;
        }
      }
    }
  }
  uint32_t tot_a = 0, tot_b = 0;
  block_inclusive_scan(ca, s_wave, &tot_a);
  block_inclusive_scan(cb, s_wave, &tot_b);

  // (2) exclusive prefix over earlier workgroups
  if (threadIdx.x == 0) {
    uint32_t pa = 0, pb = 0;
    if (w == 0) {
      st_agent(&flags[0], pack_desc(kFlagIncl, tot_a, tot_b));
    } else {
      st_agent(&flags[w], pack_desc(kFlagAgg, tot_a, tot_b));
      int64_t j = static_cast<int64_t>(w) - 1;
      while (true) {
        const uint64_t dsc = ld_agent(&flags[j]);
        const uint64_t f = dsc & (3ull << 62);
        if (f == 0) {
          __builtin_amdgcn_s_sleep(1);
          continue;
        }
        pa += static_cast<uint32_t>((dsc >> 31) & kMask31);
        pb += static_cast<uint32_t>(dsc & kMask31);
        if (f == kFlagIncl) break;
        --j;
      }
      st_agent(&flags[w], pack_desc(kFlagIncl, pa + tot_a, pb + tot_b));
    }
    s_pre_a = pa;
    s_pre_b = pb;
    if (w == gridDim.x - 1) {
      const uint32_t B = pb + tot_b;
      n_kept[0] = static_cast<int32_t>(pa + tot_a + (B < need ? B : need));
    }
  }
  __syncthreads();
  uint32_t run_a = s_pre_a, run_b = s_pre_b;

  // (3) scatter kept token indices in order
  for (int64_t base = begin; base < end; base += kChunk) {
    const int64_t t0 = base + static_cast<int64_t>(threadIdx.x) * kItems;
    uint8_t fa[kItems], fb[kItems];
    uint32_t la = 0, lb = 0;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int64_t t = t0 + i;
      fa[i] = fb[i] = 0;
      if (t < end) {
        if (!prunable[t]) {
          fa[i] = 1;
        } else {
          const uint32_t km = score_key(scores[t]) & mask;
          fa[i] = km > prefix;
          fb[i] = km == prefix;
        }
      }
      la += fa[i];
      lb += fb[i];
    }
    uint32_t chunk_a = 0, chunk_b = 0;
    uint32_t xa = block_inclusive_scan(la, s_wave, &chunk_a) - la + run_a;
    uint32_t xb = block_inclusive_scan(lb, s_wave, &chunk_b) - lb + run_b;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const bool keep = fa[i] || (fb[i] && xb < need);
      if (keep) {
        const int64_t slot = static_cast<int64_t>(xa) + (xb < need ? xb : need);
        if (slot < capacity) kept_idx[slot] = static_cast<int32_t>(t0 + i);
      }
      xa += fa[i];
      xb += fb[i];
    }
    run_a += chunk_a;
    run_b += chunk_b;
  }

  // (4) the last workgroup to finish clears the look-back state
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomicAdd(&ctl->done[3], 1u) == gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (uint32_t j = threadIdx.x; j < gridDim.x; j += kThreads) flags[j] = 0;
  if (threadIdx.x == 0) {
    ctl->ticket = 0;
    ctl->done[3] = 0;
    ctl->prefix = 0;
    ctl->mask = 0;
    ctl->need = 0;
    ctl->resolved = 0;
    ctl->n_prunable = 0;
  }
}

__global__ void write_zero_kernel(int32_t* p) { p[0] = 0; }

// ---------------------------------------------------------------------------
// Single-workgroup path (T <= kLdsTokens): the whole selection in one launch.
// Every token's key is staged once in LDS as key + 1 (0 marks a non-prunable
// token; the largest key, +inf's, still fits), then the same three digit
// passes and the same ordered compaction run out of LDS, with block-wide
// scans instead of cross-workgroup counters.  The workspace is not touched.
// ---------------------------------------------------------------------------
constexpr int kLdsTokens = 32768;
constexpr int kOneThreads = 1024;

// Inclusive sum scan of one u32 per lane over the 64 lanes of a wave: four
// row shifts (within rows of 16 lanes), then the row broadcasts 15 and 31
// carry each row's total into the rows above it.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  int x = static_cast<int>(v);
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return static_cast<uint32_t>(x);
}

// Inclusive scan of a pair of u32 over the 1024 threads of the workgroup.
__device__ __forceinline__ void wg_inclusive_scan2(uint32_t& a, uint32_t& b, uint32_t* s_wave,
                                                   uint32_t& tot_a, uint32_t& tot_b) {
  constexpr int NW = kOneThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  a = wave_inclusive_scan(a);
  b = wave_inclusive_scan(b);
  if (lane == 63) {
    s_wave[wave] = a;
    s_wave[NW + wave] = b;
  }
  __syncthreads();
  uint32_t ba = 0, bb = 0, ta = 0, tb = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t xa = s_wave[w], xb = s_wave[NW + w];
    ba += w < wave ? xa : 0u;
    bb += w < wave ? xb : 0u;
    ta += xa;
    tb += xb;
  }
  a += ba;
  b += bb;
  tot_a = ta;
  tot_b = tb;
}

// MAXT: the most tokens the launch may stage.  At MAXT <= 16384 the keys
// leave room for NCOPY copies of the first digit's histogram, bin-major (the
// copies of a bin in adjacent banks), lane l adding to copy l % NCOPY: the
// first digit (sign, exponent and two mantissa bits) puts most scores in a
// few bins, and the copies cut the same-address conflicts of the LDS atomics.
template <int MAXT>
__global__ __launch_bounds__(kOneThreads) void select_one_wg_kernel(
    const float* __restrict__ scores, const uint8_t* __restrict__ prunable, int32_t T,
    uint32_t K, int32_t* __restrict__ kept_idx, int64_t capacity,
    int32_t* __restrict__ n_kept) {
  constexpr int NCOPY = MAXT <= 16384 ? 8 : 1;
  __shared__ __attribute__((aligned(16))) uint32_t keys[MAXT];
  // the digit histograms and the resolved state, double-buffered by pass:
  // the next pass's histogram is cleared while wave 0 scans this one's
  __shared__ uint32_t hist2[2][2048];
  __shared__ __attribute__((aligned(16))) uint32_t histc[NCOPY > 1 ? 2048 * NCOPY : 4];
  __shared__ uint32_t s_wave[2 * (kOneThreads / 64)];
  __shared__ uint32_t s_state2[2][4];   // prefix, mask, need, resolved
  const int tid = threadIdx.x;
  const int lane = tid & 63;

  for (int b = tid; b < 2048; b += kOneThreads) hist2[0][b] = 0;
  if constexpr (NCOPY > 1)
#pragma unroll
    for (int b = 4 * tid; b < 2048 * NCOPY; b += 4 * kOneThreads)
      *reinterpret_cast<u32x4*>(&histc[b]) = u32x4{0, 0, 0, 0};
  // staging: each thread takes 16 consecutive tokens per round with 16-byte
  // buffer loads (all issued before any is used); past T they read zeros,
  // i.e. non-prunable (the thread holding the tail reads its bytes singly)
  const __amdgpu_buffer_rsrc_t p_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(prunable), 0, T, 0x00020000);
  const __amdgpu_buffer_rsrc_t s_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(scores), 0, T * 4, 0x00020000);
  for (int base = 0; base < T; base += kOneThreads * 16) {
    const int t0 = base + tid * 16;
    if (t0 < T) {
      u32x4 pm = __builtin_amdgcn_raw_buffer_load_b128(p_rs, t0, 0, 0);
      u32x4 sv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sv[j] = __builtin_amdgcn_raw_buffer_load_b128(s_rs, (t0 + 4 * j) * 4, 0, 0);
      if (t0 + 16 > T) {   // the range check is per dword: fetch the tail bytewise
        pm = u32x4{0, 0, 0, 0};
        for (int e = 0; t0 + e < T; ++e)
          pm[e >> 2] |= static_cast<uint32_t>(prunable[t0 + e] != 0) << (8 * (e & 3));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 kv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool p = ((pm[j] >> (8 * e)) & 0xffu) != 0;
          kv[e] = p ? score_key(__uint_as_float(sv[j][e])) + 1u : 0u;
        }
        // t0 + 15 < MAXT: t0 is a multiple of 16 below T <= MAXT
        *reinterpret_cast<u32x4*>(&keys[t0 + 4 * j]) = kv;
      }
    }
  }
  __syncthreads();

  // threshold: up to three digit passes; wave 0 resolves each digit
  uint32_t prefix = 0, mask = 0, need = K;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int bits = pass == 2 ? 10 : 11;
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t nb = 1u << bits;
    uint32_t* hist = hist2[pass & 1];
    uint32_t* s_state = s_state2[pass & 1];
    // thread tid takes keys 4 tid + 4096 i .. + 3 with 16-byte LDS reads
    // (staged keys past T, up to the next multiple of 16, are 0: skipped)
#pragma unroll
    for (int i = 0; i < MAXT / (4 * kOneThreads); ++i) {
      const int t = 4 * tid + 4 * kOneThreads * i;
      if (t < T) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(&keys[t]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t k = kv[e];
          if (k != 0 && (k & mask) == prefix) {
            const uint32_t bin = (k >> shift) & (nb - 1);
            if (NCOPY > 1 && pass == 0)
              atomicAdd(&histc[bin * NCOPY + (lane & (NCOPY - 1))], 1u);
            else
              atomicAdd(&hist[bin], 1u);
          }
        }
      }
    }
    __syncthreads();
    if (NCOPY > 1 && pass == 0) {   // fold the copies into hist
      for (int b = tid; b < 2048; b += kOneThreads) {
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < NCOPY; j += 4) {
          const u32x4 v4 = *reinterpret_cast<const u32x4*>(&histc[b * NCOPY + j]);
          c += v4[0] + v4[1] + v4[2] + v4[3];
        }
        hist[b] = c;
      }
      __syncthreads();
    }
    if (tid >= 64 && pass < 2) {   // the next pass's histogram (used two passes ago)
      const uint32_t nb_next = pass == 1 ? 1024u : 2048u;
      for (uint32_t b = tid - 64; b < nb_next; b += kOneThreads - 64) hist2[(pass + 1) & 1][b] = 0;
    }
    if (tid < 64) {
      // lane l owns bins nb-1-l*bpl down to nb-(l+1)*bpl (descending keys),
      // kept in registers for the search below
      const int bpl = static_cast<int>(nb) / 64;
      const int top = static_cast<int>(nb) - 1 - lane * bpl;
      uint32_t cnt[32];
      uint32_t mine = 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        cnt[j] = j < bpl ? hist[top - j] : 0u;
        mine += cnt[j];
      }
      const uint32_t incl = wave_inclusive_scan(mine);
      const uint32_t total = __shfl(incl, 63, 64);
      uint32_t nd = need;
      if (pass == 0) {   // total = |P|: every prunable key matches the empty prefix
        if (K >= total || K == 0) {
          if (lane == 0) {
            s_state[0] = 0;
            s_state[1] = 0;
            s_state[2] = K >= total ? total : 0u;
            s_state[3] = 1;
          }
          nd = 0;   // no lane resolves a digit
        }
      }
      const uint32_t above = incl - mine;
      if (nd != 0 && above < nd && nd <= above + mine) {
        // the one bin where the running count first reaches nd
        uint32_t cum = above;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const uint32_t c = cnt[j];
          if (cum < nd && cum + c >= nd) {
            s_state[0] = prefix | (static_cast<uint32_t>(top - j) << shift);
            s_state[1] = mask | ((nb - 1) << shift);
            s_state[2] = nd - cum;
            s_state[3] = (nd - cum == c || pass == 2) ? 1u : 0u;
          }
          cum += c;
        }
      }
    }
    __syncthreads();
    prefix = s_state[0];
    mask = s_state[1];
    need = s_state[2];
    const bool resolved = s_state[3] != 0;
    // no second barrier: the next pass writes the other histogram and state
    if (resolved) break;   // uniform across the workgroup
  }

  // ordered compaction: thread tid owns the contiguous tokens
  // [tid * C, tid * C + C), C a multiple of 4; one workgroup scan of the
  // counts (a, b) gives every thread its output slots
  const int C = ((T + kOneThreads - 1) / kOneThreads + 3) & ~3;
  const int c0 = tid * C;
  uint32_t ca = 0, cb = 0;
  for (int i = 0; i < C; i += 4) {
    if (c0 + i < T) {
      const u32x4 kv = *reinterpret_cast<const u32x4*>(&keys[c0 + i]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t k = kv[e];
        const bool in = c0 + i + e < T;
        const uint32_t km = k & mask;
        ca += in && (k == 0 || km > prefix);
        cb += in && k != 0 && km == prefix;
      }
    }
  }
  uint32_t xa = ca, xb = cb, tot_a = 0, tot_b = 0;
  wg_inclusive_scan2(xa, xb, s_wave, tot_a, tot_b);
  xa -= ca;   // exclusive prefixes
  xb -= cb;
  for (int i = 0; i < C; i += 4) {
    if (c0 + i < T) {
      const u32x4 kv = *reinterpret_cast<const u32x4*>(&keys[c0 + i]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = c0 + i + e;
        const uint32_t k = kv[e];
        const uint32_t km = k & mask;
        const bool fa = t < T && (k == 0 || km > prefix);
        const bool fb = t < T && k != 0 && km == prefix;
        if (fa || (fb && xb < need)) {
          const int64_t slot = static_cast<int64_t>(xa) + (xb < need ? xb : need);
          if (slot < capacity) kept_idx[slot] = t;
        }
        xa += fa;
        xb += fb;
      }
    }
  }
  if (tid == 0) n_kept[0] = static_cast<int32_t>(tot_a + (tot_b < need ? tot_b : need));
}

}  // namespace
}  // namespace tg

extern "C" size_t tg_topk_workspace_size(int64_t T) {
  using namespace tg;
  if (T < 0) T = 0;
  const int64_t G = blocks_for(T, nullptr);
  const size_t bytes = kFlagOff + static_cast<size_t>(G) * sizeof(uint64_t);
  return (bytes + 255) & ~static_cast<size_t>(255);
}

extern "C" tg_status tg_topk_select(int64_t T, const float* scores, const uint8_t* prunable,
                                    int64_t K, int32_t* kept_idx, int64_t kept_capacity,
                                    int32_t* n_kept, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  using namespace tg;
  if (T < 0 || T > kMaxTokens)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_topk_select: need 0 <= T <= 2^31-1 (T=%lld)",
                (long long)T);
  if (K < 0)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_topk_select: K must be >= 0 (K=%lld)",
                (long long)K);
  if (kept_capacity < 0)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_topk_select: kept_capacity < 0");
  if (n_kept == nullptr)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_topk_select: n_kept is NULL");
  hipStream_t s = as_stream(stream);
  if (T == 0) {
    write_zero_kernel<<<1, 1, 0, s>>>(n_kept);
    return check_launch("tg_topk_select");
  }
  if (scores == nullptr || prunable == nullptr)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_topk_select: scores/prunable is NULL");
  if (kept_idx == nullptr && kept_capacity > 0)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_topk_select: kept_idx is NULL");
  if (!aligned(scores, 4) || !aligned(kept_idx, 4) || !aligned(n_kept, 4))
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_topk_select: misaligned pointer");
  const size_t need_bytes = tg_topk_workspace_size(T);
  if (workspace == nullptr || workspace_bytes < need_bytes)
    return fail(TG_ERR_WORKSPACE, "tg_topk_select: workspace needs %zu bytes, got %zu",
                need_bytes, workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (!aligned(workspace, 256))
    return fail(TG_ERR_WORKSPACE, "tg_topk_select: workspace must be 256-byte aligned");

  const uint32_t Kc = static_cast<uint32_t>(K < T ? K : T);
  if (T <= kLdsTokens && aligned(prunable, 16)) {
    if (T <= kLdsTokens / 2)
      select_one_wg_kernel<kLdsTokens / 2><<<dim3(1), dim3(kOneThreads), 0, s>>>(
          scores, prunable, static_cast<int32_t>(T), Kc, kept_idx, kept_capacity, n_kept);
    else
      select_one_wg_kernel<kLdsTokens><<<dim3(1), dim3(kOneThreads), 0, s>>>(
          scores, prunable, static_cast<int32_t>(T), Kc, kept_idx, kept_capacity, n_kept);
    return check_launch("tg_topk_select");
  }
  int64_t per_block = 0;
  const int64_t G = blocks_for(T, &per_block);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const int32_t T32 = static_cast<int32_t>(T);
  radix_hist_kernel<0><<<dim3(G), dim3(kThreads), 0, s>>>(scores, prunable, T32, per_block,
                                                           Kc, static_cast<uint32_t>(G), ws);
  radix_hist_kernel<1><<<dim3(G), dim3(kThreads), 0, s>>>(scores, prunable, T32, per_block,
                                                           Kc, static_cast<uint32_t>(G), ws);
  radix_hist_kernel<2><<<dim3(G), dim3(kThreads), 0, s>>>(scores, prunable, T32, per_block,
                                                           Kc, static_cast<uint32_t>(G), ws);
  compact_kernel<<<dim3(G), dim3(kThreads), 0, s>>>(scores, prunable, T32, per_block, ws,
                                                     kept_idx, kept_capacity, n_kept);
  return check_launch("tg_topk_select");
}
