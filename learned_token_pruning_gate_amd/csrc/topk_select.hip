// topk_select.hip -- [a2] radix top-K threshold over the prunable tokens'
// scores and [a3] order-preserving compaction of the kept set.
//
// TokenGate pages: ai.info summary "Key Contributions" item 1 and
// "Methodology in Plain English" -- the gate keeps its K best prunable
// tokens plus every non-prunable token; the README mirror's "Quick start"
// budget None keeps every prunable token.
//
// Design (gfx950).  Scores become order-preserving u32 keys (NaN lowest,
// -0 == +0).  Three paths by prompt length: T <= 24576, one workgroup with
// every key in LDS; T <= 524288 (the grid path below), one launch of up to
// 32 workgroups that meet at grid barriers; longer prompts, the four
// launches described here.  Three histogram passes over digits of 11, 11
// and 10 bits find the K-th largest key v*: every workgroup builds an LDS
// histogram of the
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
// look-back descriptors (or, on the grid path, its barrier counters and
// per-workgroup counts in the descriptors' place).  It must start all-zero;
// the last workgroup of each pass (of the grid launch) clears what it used,
// so every call ends with it all-zero.  The first histogram pass also resets
// the compaction's ticket and descriptors.
#include <cstdlib>
#include <mutex>

#include "tg_common.hpp"

// Scratch of tg_topk_select_noalloc: the select workspace as a file-scope
// device array, one copy on each GPU the library runs on, held until the
// process ends.  Host code never passes this name to a kernel (on the host
// it is only a stand-in for the symbol); it uses the device address that
// hipGetSymbolAddress returns for the current device.  The workspace of the
// largest T (4096 look-back descriptors) is 53.5 KiB; 64 KiB covers every T.
static __device__ __align__(256) uint8_t scratch[64 * 1024];

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

// Tokens per workgroup: at least two sweeps (2048 tokens), so that the
// digit passes' global histogram atomics and the compaction's look-back
// chain serve half as many workgroups (measured at 128k tokens: the select
// took 52 us with 1024-token workgroups, 40 us with these and the windowed
// look-back); at most kMaxBlocks workgroups.
constexpr int64_t kMinPerBlock = 2 * kChunk;

__host__ __device__ inline int64_t blocks_for(int64_t T, int64_t* per_block) {
  int64_t pb = (T + kMaxBlocks - 1) / kMaxBlocks;
  pb = ((pb + kChunk - 1) / kChunk) * kChunk;
  if (pb < kMinPerBlock) pb = kMinPerBlock;
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

// A thread's 4 consecutive tokens l0 .. l0 + 3 of its workgroup's range
// [begin, begin + nloc): the prunable bytes as one word and the scores as
// one 16-byte load, through buffer resources based at the range (reads past
// it return 0), so that both are in flight together.  The range check is
// per dword, so the thread whose 4 tokens straddle the range's end reads its
// prunable bytes singly (tail_fix).
struct Tok4 {
  uint32_t p;   // byte e: token l0 + e is prunable (nonzero) or not
  u32x4 s;      // score bits of the 4 tokens
};
__device__ __forceinline__ Tok4 load_tok4(__amdgpu_buffer_rsrc_t p_rs,
                                          __amdgpu_buffer_rsrc_t s_rs, int32_t l0) {
  Tok4 r;
  r.p = __builtin_amdgcn_raw_buffer_load_b32(p_rs, l0, 0, 0);
  r.s = __builtin_amdgcn_raw_buffer_load_b128(s_rs, 4 * l0, 0, 0);
  return r;
}
__device__ __forceinline__ uint32_t tail_fix(uint32_t p, const uint8_t* __restrict__ pb,
                                             int32_t l0, int32_t nloc) {
  if (l0 + 4 <= nloc) return p;
  uint32_t q = 0;
  for (int e = 0; e < 4; ++e)
    if (l0 + e < nloc) q |= static_cast<uint32_t>(pb[l0 + e] != 0) << (8 * e);
  return q;
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
    int64_t per_block, uint32_t K, uint32_t n_compact_blocks, uint8_t* __restrict__ ws,
    const int32_t* __restrict__ t_dyn) {
  constexpr int BITS = PASS == 2 ? 10 : 11;
  if (t_dyn != nullptr) T = min(T, max(*t_dyn, 0));   // run-time length (T: capacity)
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
  const int32_t nloc = end > begin ? static_cast<int32_t>(end - begin) : 0;
  const __amdgpu_buffer_rsrc_t p_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(prunable + begin), 0, nloc, 0x00020000);
  const __amdgpu_buffer_rsrc_t s_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(scores + begin), 0, 4 * nloc, 0x00020000);
  // two sweeps' loads in flight per round trip
  for (int32_t lb = 0; lb < nloc; lb += 2 * kChunk) {
    Tok4 tk[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      tk[j] = load_tok4(p_rs, s_rs, lb + j * kChunk + kItems * static_cast<int32_t>(threadIdx.x));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int32_t l0 = lb + j * kChunk + kItems * static_cast<int32_t>(threadIdx.x);
      const uint32_t pw = tail_fix(tk[j].p, prunable + begin, l0, nloc);
#pragma unroll
      for (int i = 0; i < kItems; ++i) {
        if ((pw >> (8 * i)) & 0xffu) {
          const uint32_t key = score_key(__uint_as_float(tk[j].s[i]));
          if ((key & mask) == prefix) atomicAdd(&h[(key >> SHIFT) & (NB - 1)], 1u);
        }
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
    int64_t capacity, int32_t* __restrict__ n_kept, const int32_t* __restrict__ t_dyn) {
  if (t_dyn != nullptr) T = min(T, max(*t_dyn, 0));   // run-time length (T: capacity)
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
  const int32_t nloc = end > begin ? static_cast<int32_t>(end - begin) : 0;
  const __amdgpu_buffer_rsrc_t p_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(prunable + begin), 0, nloc, 0x00020000);
  const __amdgpu_buffer_rsrc_t s_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(scores + begin), 0, 4 * nloc, 0x00020000);
  // token l0 + i of a sweep: kept always (a), or tied at the threshold (b)
  auto classify = [&](const Tok4& tk, uint32_t pw, int32_t l0, int i, uint32_t& fa,
                      uint32_t& fb) {
    fa = fb = 0;
    if (l0 + i < nloc) {
      if (((pw >> (8 * i)) & 0xffu) == 0) {
        fa = 1;
      } else {
        const uint32_t km = score_key(__uint_as_float(tk.s[i])) & mask;
        fa = km > prefix;
        fb = km == prefix;
      }
    }
  };

  // (1) this workgroup's counts of a and b (two sweeps' loads per round trip)
  uint32_t ca = 0, cb = 0;
  for (int32_t lb = 0; lb < nloc; lb += 2 * kChunk) {
    Tok4 tk[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      tk[j] = load_tok4(p_rs, s_rs, lb + j * kChunk + kItems * static_cast<int32_t>(threadIdx.x));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int32_t l0 = lb + j * kChunk + kItems * static_cast<int32_t>(threadIdx.x);
      const uint32_t pw = tail_fix(tk[j].p, prunable + begin, l0, nloc);
#pragma unroll
      for (int i = 0; i < kItems; ++i) {
        uint32_t fa, fb;
        classify(tk[j], pw, l0, i, fa, fb);
        ca += fa;
        cb += fb;
      }
    }
  }
  uint32_t tot_a = 0, tot_b = 0;
  block_inclusive_scan(ca, s_wave, &tot_a);
  block_inclusive_scan(cb, s_wave, &tot_b);

  // (2) exclusive prefix over earlier workgroups.  Wave 0 reads a window of
  // 64 predecessors' descriptors per round trip (lane i: workgroup top - i):
  // the nearest inclusive one ends the walk, and every aggregate before it
  // is added; a nearer predecessor that has not published yet makes the
  // wave read the window again.
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    uint32_t pa = 0, pb = 0;
    if (w == 0) {
      if (lane == 0) st_agent(&flags[0], pack_desc(kFlagIncl, tot_a, tot_b));
    } else {
      if (lane == 0) st_agent(&flags[w], pack_desc(kFlagAgg, tot_a, tot_b));
      int64_t top = static_cast<int64_t>(w) - 1;
      while (true) {
        const int64_t j = top - lane;
        // before the first workgroup: an inclusive descriptor of zero counts
        const uint64_t dsc = j >= 0 ? ld_agent(&flags[j]) : pack_desc(kFlagIncl, 0, 0);
        const uint64_t f = dsc & (3ull << 62);
        const uint64_t incl = __ballot(f == kFlagIncl);
        const uint64_t zero = __ballot(f == 0);
        const int first_incl = incl ? __builtin_ctzll(incl) : 64;
        const int first_zero = zero ? __builtin_ctzll(zero) : 64;
        if (first_zero < first_incl) {
          __builtin_amdgcn_s_sleep(1);
          continue;
        }
        uint32_t wa = lane <= first_incl ? static_cast<uint32_t>((dsc >> 31) & kMask31) : 0u;
        uint32_t wb = lane <= first_incl ? static_cast<uint32_t>(dsc & kMask31) : 0u;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          wa += __shfl_xor(wa, off, 64);
          wb += __shfl_xor(wb, off, 64);
        }
        pa += wa;
        pb += wb;
        if (first_incl < 64) break;
        top -= 64;
      }
      if (lane == 0) st_agent(&flags[w], pack_desc(kFlagIncl, pa + tot_a, pb + tot_b));
    }
    if (lane == 0) {
      s_pre_a = pa;
      s_pre_b = pb;
      if (w == gridDim.x - 1) {
        const uint32_t B = pb + tot_b;
        n_kept[0] = static_cast<int32_t>(pa + tot_a + (B < need ? B : need));
      }
    }
  }
  __syncthreads();
  uint32_t run_a = s_pre_a, run_b = s_pre_b;

  // (3) scatter kept token indices in order
  for (int32_t base = 0; base < nloc; base += kChunk) {
    const int32_t l0 = base + kItems * static_cast<int32_t>(threadIdx.x);
    const int64_t t0 = begin + l0;
    const Tok4 tk = load_tok4(p_rs, s_rs, l0);
    const uint32_t pw = tail_fix(tk.p, prunable + begin, l0, nloc);
    uint32_t fa[kItems], fb[kItems];
    uint32_t la = 0, lb = 0;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      classify(tk, pw, l0, i, fa[i], fb[i]);
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
    int32_t* __restrict__ n_kept, const int32_t* __restrict__ t_dyn) {
  constexpr int NCOPY = MAXT <= 16384 ? 8 : 1;
  if (t_dyn != nullptr) T = min(T, max(*t_dyn, 0));   // run-time length (T: capacity)
  __shared__ __attribute__((aligned(16))) uint32_t keys[MAXT];
  // the digit histograms and the resolved state, double-buffered by pass:
  // the next pass's histogram is cleared while wave 0 scans this one's
  __shared__ uint32_t hist2[2][2048];
  __shared__ __attribute__((aligned(16))) uint32_t histc[NCOPY > 1 ? 2048 * NCOPY : 4];
  __shared__ uint32_t s_wave[2 * (kOneThreads / 64)];
  __shared__ uint32_t s_state2[2][4];   // prefix, mask, need, resolved
  __shared__ uint32_t s_np[kOneThreads / 64];   // prunable tokens per wave
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
  uint32_t np = 0;   // this thread's prunable tokens
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
          np += p;
        }
        // t0 + 15 < MAXT: t0 is a multiple of 16 below T <= MAXT
        *reinterpret_cast<u32x4*>(&keys[t0 + 4 * j]) = kv;
      }
    }
  }
  // |P| is summed only when K could reach it (K >= T / 2, or K == 0)
  const bool count_p = K == 0 || 2 * static_cast<int64_t>(K) >= T;
  if (count_p) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) np += __shfl_xor(np, off, 64);
    if (lane == 0) s_np[tid >> 6] = np;
  }
  __syncthreads();
  uint32_t n_p = 0xffffffffu;   // |P|, or "unknown"
  if (count_p) {
    n_p = 0;
#pragma unroll
    for (int w = 0; w < kOneThreads / 64; ++w) n_p += s_np[w];
  }

  // threshold: up to three digit passes; wave 0 resolves each digit.  Keep
  // all or none of the prunable tokens (K >= |P| or K == 0): no digit to
  // resolve (prefix and mask 0 make every prunable token tie at the
  // threshold, and need says how many of them stay).  Otherwise the first
  // pass finds |P| and still decides this case.
  const bool all_or_none = count_p && (K >= n_p || K == 0);
  uint32_t prefix = 0, mask = 0, need = all_or_none ? (K >= n_p ? n_p : 0u) : K;
  if (!all_or_none) {
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
        for (uint32_t b = tid - 64; b < nb_next; b += kOneThreads - 64)
          hist2[(pass + 1) & 1][b] = 0;
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

// ---------------------------------------------------------------------------
// Grid path (kGridMinT < T <= kGridMaxT): the whole selection in one launch
// of G <= kGridMaxWG workgroups that are resident together (at most one per
// CU, far fewer than the CUs).  Each stages its range of `per` tokens in LDS
// once, as the single-workgroup kernel does; the digit passes then add the
// workgroups' LDS histograms into global ones and meet at a grid barrier,
// after which every workgroup reads the global histogram and resolves the
// digit itself (the same result everywhere, so every workgroup takes the
// same branches and barriers).  The compaction publishes each workgroup's
// (a, b) counts, meets at a last barrier and adds its predecessors' counts.
// A barrier is a counter per barrier: each workgroup adds 1 after its
// writes, then waits for G.  The wait is bounded (kSpinLimit polls); one that
// gives up marks the call failed, which its last workgroup reports as
// n_kept = -1, so a workgroup that never ran could not hang the device.
// The last workgroup to finish clears every counter and histogram.
// ---------------------------------------------------------------------------
constexpr int kGridThreads = 1024;
constexpr int kGridMaxWG = 32;
constexpr int kGridPer = 4096;                                    // tokens per workgroup, up to ...
constexpr int kGridPerMax = 16384;                                // ... this (64 KiB of keys)
constexpr int64_t kGridMinT = 24576;   // below it the single workgroup is faster (20k: 14.9 vs 16.9 us)
constexpr int64_t kGridMaxT = static_cast<int64_t>(kGridMaxWG) * kGridPerMax;
constexpr uint32_t kSpinLimit = 1u << 22;

// Grid path control, at kFlagOff (the compaction descriptors' space, which
// the grid path does not use): all-zero between calls.
struct GridCtl {
  uint32_t arrive[5];    // barrier counters: digit passes 0..2, |P|, compaction
  uint32_t exit_count;   // workgroups done
  uint32_t n_p;          // sum of the workgroups' prunable counts
  uint32_t timeout;      // some barrier wait gave up
  uint64_t slot[kGridMaxWG];   // workgroup g's (a count << 32) | b count
};

// Everything one workgroup hands to another goes through device-coherent
// operations: atomics (performed at the device's coherence point, as the
// cross-workgroup sums here rely on) and agent-scope loads and stores, which
// bypass the non-coherent caches.  So a barrier needs no cache write-back:
// every wave waits until its own memory operations have completed (a
// workgroup-scope release), then thread 0 arrives and waits for all G.
// `want` is G in every call but the forced-timeout check (below), and
// `limit` the poll bound.
__device__ __forceinline__ void grid_barrier(uint32_t* count, uint32_t want, uint32_t limit,
                                             uint32_t* timeout) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);   // vmcnt, expcnt and lgkmcnt all 0
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t polls = 0;
    while (ld_agent(count) < want) {
      __builtin_amdgcn_s_sleep(1);
      if (++polls > limit) {
        atomicOr(timeout, 1u);
        break;
      }
    }
  }
  __syncthreads();
}

template <int MAXT>
__global__ __launch_bounds__(kGridThreads) void select_grid_kernel(
    const float* __restrict__ scores, const uint8_t* __restrict__ prunable, int32_t T,
    int32_t per, uint32_t K, int32_t* __restrict__ kept_idx, int64_t capacity,
    int32_t* __restrict__ n_kept, uint8_t* __restrict__ ws, const int32_t* __restrict__ t_dyn,
    uint32_t extra, uint32_t limit) {
  constexpr int NCOPY = MAXT <= kGridPer ? 8 : 2;
  constexpr int NW = kGridThreads / 64;
  if (t_dyn != nullptr) T = min(T, max(*t_dyn, 0));   // run-time length (T: capacity)
  __shared__ __attribute__((aligned(16))) uint32_t keys[MAXT];
  __shared__ uint32_t hist[2048];
  __shared__ __attribute__((aligned(16))) uint32_t histc[2048 * NCOPY];
  __shared__ uint32_t s_wave[2 * NW];
  __shared__ uint32_t s_state[4];   // prefix, mask, need, resolved
  __shared__ uint32_t s_np[NW];
  __shared__ uint32_t s_pre[2];
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const uint32_t G = gridDim.x;
  const uint32_t want = G + extra;   // arrivals a barrier waits for
  const uint32_t g = blockIdx.x;
  GridCtl* ctl = reinterpret_cast<GridCtl*>(ws + kFlagOff);

  // this workgroup's tokens [begin, begin + nloc); per is a multiple of 16,
  // so the 16-byte loads below stay aligned
  const int64_t begin = static_cast<int64_t>(g) * per;
  const int32_t nloc = static_cast<int32_t>(
      begin >= T ? 0 : (T - begin < per ? T - begin : static_cast<int64_t>(per)));
  const __amdgpu_buffer_rsrc_t p_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(prunable + begin), 0, nloc, 0x00020000);
  const __amdgpu_buffer_rsrc_t s_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(scores + begin), 0, nloc * 4, 0x00020000);
  uint32_t np = 0;
  for (int base = 0; base < nloc; base += kGridThreads * 16) {
    const int t0 = base + tid * 16;
    if (t0 < nloc) {
      u32x4 pm = __builtin_amdgcn_raw_buffer_load_b128(p_rs, t0, 0, 0);
      u32x4 sv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sv[j] = __builtin_amdgcn_raw_buffer_load_b128(s_rs, (t0 + 4 * j) * 4, 0, 0);
      if (t0 + 16 > nloc) {   // the range check is per dword: fetch the tail bytewise
        pm = u32x4{0, 0, 0, 0};
        for (int e = 0; t0 + e < nloc; ++e)
          pm[e >> 2] |= static_cast<uint32_t>(prunable[begin + t0 + e] != 0) << (8 * (e & 3));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 kv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool p = ((pm[j] >> (8 * e)) & 0xffu) != 0;
          kv[e] = p ? score_key(__uint_as_float(sv[j][e])) + 1u : 0u;
          np += p;
        }
        *reinterpret_cast<u32x4*>(&keys[t0 + 4 * j]) = kv;   // t0 + 15 < per <= MAXT
      }
    }
  }

  // |P| over all workgroups, when K could reach it (K >= T / 2, or K == 0)
  const bool count_p = K == 0 || 2 * static_cast<int64_t>(K) >= T;
  uint32_t n_p = 0xffffffffu;   // |P|, or "unknown"
  if (count_p) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) np += __shfl_xor(np, off, 64);
    if (lane == 0) s_np[tid >> 6] = np;
    __syncthreads();
    if (tid == 0) {
      uint32_t c = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) c += s_np[w];
      if (c) atomicAdd(&ctl->n_p, c);
    }
    grid_barrier(&ctl->arrive[3], want, limit, &ctl->timeout);
    n_p = ld_agent(&ctl->n_p);
  }

  const bool all_or_none = count_p && (K >= n_p || K == 0);
  uint32_t prefix = 0, mask = 0, need = all_or_none ? (K >= n_p ? n_p : 0u) : K;
  if (!all_or_none) {
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int bits = pass == 2 ? 10 : 11;
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const uint32_t nb = 1u << bits;
      uint32_t* ghist = reinterpret_cast<uint32_t*>(ws + kHistOff[pass]);
      for (int b = tid; b < 2048; b += kGridThreads) hist[b] = 0;
      if (pass == 0)
#pragma unroll
        for (int b = 4 * tid; b < 2048 * NCOPY; b += 4 * kGridThreads)
          *reinterpret_cast<u32x4*>(&histc[b]) = u32x4{0, 0, 0, 0};
      __syncthreads();
#pragma unroll
      for (int i = 0; i < MAXT / (4 * kGridThreads); ++i) {
        const int t = 4 * tid + 4 * kGridThreads * i;
        if (t < nloc) {
          const u32x4 kv = *reinterpret_cast<const u32x4*>(&keys[t]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t k = kv[e];
            if (k != 0 && (k & mask) == prefix) {
              const uint32_t bin = (k >> shift) & (nb - 1);
              if (pass == 0)
                atomicAdd(&histc[bin * NCOPY + (lane & (NCOPY - 1))], 1u);
              else
                atomicAdd(&hist[bin], 1u);
            }
          }
        }
      }
      __syncthreads();
      // fold the first digit's copies, and add the nonzero bins to the
      // global histogram
      for (uint32_t b = tid; b < nb; b += kGridThreads) {
        uint32_t c;
        if (pass == 0) {
          c = 0;
#pragma unroll
          for (int j = 0; j < NCOPY; j += 2) {
            const u32x2 v2 = *reinterpret_cast<const u32x2*>(&histc[b * NCOPY + j]);
            c += v2[0] + v2[1];
          }
        } else {
          c = hist[b];
        }
        if (c) atomicAdd(&ghist[b], c);
      }
      grid_barrier(&ctl->arrive[pass], want, limit, &ctl->timeout);
      for (uint32_t b = tid; b < nb; b += kGridThreads) hist[b] = ld_agent(&ghist[b]);
      __syncthreads();
      if (tid < 64) {
        // the single-workgroup kernel's resolve: lane l owns bins
        // nb-1-l*bpl down to nb-(l+1)*bpl (descending keys)
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
        if (lane == 0) s_state[3] = 0;
        if (pass == 0) {   // total = |P|: every prunable key matches the empty prefix
          if (K >= total || K == 0) {
            if (lane == 0) {
              s_state[0] = 0;
              s_state[1] = 0;
              s_state[2] = K >= total ? total : 0u;
              s_state[3] = 1;
            }
            nd = 0;
          }
        }
        const uint32_t above = incl - mine;
        if (nd != 0 && above < nd && nd <= above + mine) {
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
      __syncthreads();   // every thread has read the state before the next pass
      if (resolved) break;   // the same in every workgroup
    }
  }

  // ordered compaction: thread tid owns the contiguous tokens
  // [tid * C, tid * C + C) of the range, C a multiple of 4
  const int C = ((nloc + kGridThreads - 1) / kGridThreads + 3) & ~3;
  const int c0 = tid * C;
  uint32_t ca = 0, cb = 0;
  for (int i = 0; i < C; i += 4) {
    if (c0 + i < nloc) {
      const u32x4 kv = *reinterpret_cast<const u32x4*>(&keys[c0 + i]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t k = kv[e];
        const bool in = c0 + i + e < nloc;
        const uint32_t km = k & mask;
        ca += in && (k == 0 || km > prefix);
        cb += in && k != 0 && km == prefix;
      }
    }
  }
  uint32_t xa = ca, xb = cb, tot_a = 0, tot_b = 0;
  wg_inclusive_scan2(xa, xb, s_wave, tot_a, tot_b);
  if (tid == 0) st_agent(&ctl->slot[g], (static_cast<uint64_t>(tot_a) << 32) | tot_b);
  grid_barrier(&ctl->arrive[4], want, limit, &ctl->timeout);
  if (tid < 64) {   // the counts of the workgroups before this one (G <= 64)
    const uint64_t v = lane < static_cast<int>(g) ? ld_agent(&ctl->slot[lane]) : 0ull;
    uint32_t pa = static_cast<uint32_t>(v >> 32), pb = static_cast<uint32_t>(v);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      pa += __shfl_xor(pa, off, 64);
      pb += __shfl_xor(pb, off, 64);
    }
    if (lane == 0) {
      s_pre[0] = pa;
      s_pre[1] = pb;
    }
  }
  __syncthreads();
  xa = xa - ca + s_pre[0];   // exclusive prefixes over the whole prompt
  xb = xb - cb + s_pre[1];
  for (int i = 0; i < C; i += 4) {
    if (c0 + i < nloc) {
      const u32x4 kv = *reinterpret_cast<const u32x4*>(&keys[c0 + i]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = c0 + i + e;
        const uint32_t k = kv[e];
        const uint32_t km = k & mask;
        const bool fa = t < nloc && (k == 0 || km > prefix);
        const bool fb = t < nloc && k != 0 && km == prefix;
        if (fa || (fb && xb < need)) {
          const int64_t slot = static_cast<int64_t>(xa) + (xb < need ? xb : need);
          if (slot < capacity) kept_idx[slot] = static_cast<int32_t>(begin + t);
        }
        xa += fa;
        xb += fb;
      }
    }
  }

  // the last workgroup to finish writes the kept count and clears the
  // control words and histograms (every workgroup has passed every barrier
  // and read every histogram by then)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&ctl->exit_count, 1u) == G - 1;
  __syncthreads();
  if (!s_last) return;
  if (tid == 0) {
    // the totals over every workgroup's slot (the last to finish may be any)
    uint64_t all_a = 0, all_b = 0;
    for (uint32_t j = 0; j < G; ++j) {
      const uint64_t v = ld_agent(&ctl->slot[j]);
      all_a += v >> 32;
      all_b += static_cast<uint32_t>(v);
    }
    const bool failed = ld_agent(&ctl->timeout) != 0;
    n_kept[0] = failed ? -1
                       : static_cast<int32_t>(all_a + (all_b < need ? all_b : static_cast<uint64_t>(need)));
    for (int j = 0; j < 5; ++j) st_agent(&ctl->arrive[j], 0u);
    st_agent(&ctl->n_p, 0u);
    st_agent(&ctl->timeout, 0u);
    st_agent(&ctl->exit_count, 0u);
  }
  for (int j = tid; j < kGridMaxWG; j += kGridThreads) st_agent(&ctl->slot[j], static_cast<uint64_t>(0));
  for (int b = tid; b < 2048 + 2048 + 1024; b += kGridThreads)
    st_agent(reinterpret_cast<uint32_t*>(ws + kHistOff[0]) + b, 0u);
}

}  // namespace
}  // namespace tg

extern "C" size_t tg_topk_workspace_size(int64_t T) {
  using namespace tg;
  if (T < 0) T = 0;
  const int64_t G = blocks_for(T, nullptr);
  size_t bytes = kFlagOff + static_cast<size_t>(G) * sizeof(uint64_t);
  if (bytes < kFlagOff + sizeof(GridCtl)) bytes = kFlagOff + sizeof(GridCtl);   // grid path
  return (bytes + 255) & ~static_cast<size_t>(255);
}

namespace tg {
namespace {

__global__ void zero_bytes_kernel(uint8_t* __restrict__ p, int32_t n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Device address of `scratch` on the current device, looked up (and the
// array cleared on `s`) on the first call on each device.
tg_status static_scratch(hipStream_t s, uint8_t** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(TG_ERR_LAUNCH, "tg_topk_select_noalloc: no usable current device (%s)",
                hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(TG_ERR_LAUNCH, "tg_topk_select_noalloc: hipGetSymbolAddress failed: %s",
                  hipGetErrorString(e));
    // the selection needs an all-zero workspace: clear it once, with a kernel
    zero_bytes_kernel<<<dim3(sizeof(scratch) / 256), dim3(256), 0, s>>>(
        static_cast<uint8_t*>(p), static_cast<int32_t>(sizeof(scratch)));
    const tg_status st = check_launch("tg_topk_select_noalloc");
    if (st != TG_OK) return st;
    ptr[dev] = p;
  }
  *out = static_cast<uint8_t*>(ptr[dev]);
  return TG_OK;
}

// Host-side checks of tg_topk_select's arguments (all but the workspace).
tg_status select_check(const char* fn, int64_t T, const float* scores, const uint8_t* prunable,
                       int64_t K, const int32_t* kept_idx, int64_t kept_capacity,
                       const int32_t* n_kept) {
  if (T < 0 || T > kMaxTokens)
    return fail(TG_ERR_INVALID_ARGUMENT, "%s: need 0 <= T <= 2^31-1 (T=%lld)", fn,
                (long long)T);
  if (K < 0)
    return fail(TG_ERR_INVALID_ARGUMENT, "%s: K must be >= 0 (K=%lld)", fn, (long long)K);
  if (kept_capacity < 0) return fail(TG_ERR_INVALID_ARGUMENT, "%s: kept_capacity < 0", fn);
  if (n_kept == nullptr) return fail(TG_ERR_INVALID_ARGUMENT, "%s: n_kept is NULL", fn);
  if (T == 0) return TG_OK;
  if (scores == nullptr || prunable == nullptr)
    return fail(TG_ERR_INVALID_ARGUMENT, "%s: scores/prunable is NULL", fn);
  if (kept_idx == nullptr && kept_capacity > 0)
    return fail(TG_ERR_INVALID_ARGUMENT, "%s: kept_idx is NULL", fn);
  if (!aligned(scores, 4) || !aligned(kept_idx, 4) || !aligned(n_kept, 4))
    return fail(TG_ERR_INVALID_ARGUMENT, "%s: misaligned pointer", fn);
  return TG_OK;
}

// The launches of a checked call; ws holds at least tg_topk_workspace_size(T)
// bytes, 256-byte aligned, all zero.
tg_status select_launch(const char* fn, int64_t T, const float* scores,
                        const uint8_t* prunable, int64_t K, int32_t* kept_idx,
                        int64_t kept_capacity, int32_t* n_kept, uint8_t* ws, hipStream_t s,
                        const int32_t* t_dyn) {
  if (T == 0) {
    write_zero_kernel<<<1, 1, 0, s>>>(n_kept);
    return check_launch(fn);
  }
  const uint32_t Kc = static_cast<uint32_t>(K < T ? K : T);
  if (T > kGridMinT && T <= kGridMaxT && aligned(prunable, 16)) {
    // one launch, G workgroups resident together (G <= kGridMaxWG, far
    // below the CU count; each takes at most one CU)
    const int64_t G = std::min<int64_t>(kGridMaxWG, (T + kGridPer - 1) / kGridPer);
    const int64_t per = ((T + G - 1) / G + 15) / 16 * 16;
    const int32_t T32 = static_cast<int32_t>(T);
    // TG_TEST_SELECT_TIMEOUT=1 (read once) makes every barrier wait for one
    // arrival more than there are workgroups, with a short poll bound: the
    // waits give up and the call reports n_kept = -1.  The failure path is
    // tested this way, with every workgroup still exiting normally.
    static const bool force_timeout = [] {
      const char* e = std::getenv("TG_TEST_SELECT_TIMEOUT");
      return e != nullptr && e[0] == '1';
    }();
    const uint32_t extra = force_timeout ? 1u : 0u;
    const uint32_t limit = force_timeout ? 256u : kSpinLimit;
    if (per <= kGridPer)
      select_grid_kernel<kGridPer><<<dim3(G), dim3(kGridThreads), 0, s>>>(
          scores, prunable, T32, static_cast<int32_t>(per), Kc, kept_idx, kept_capacity, n_kept,
          ws, t_dyn, extra, limit);
    else
      select_grid_kernel<kGridPerMax><<<dim3(G), dim3(kGridThreads), 0, s>>>(
          scores, prunable, T32, static_cast<int32_t>(per), Kc, kept_idx, kept_capacity, n_kept,
          ws, t_dyn, extra, limit);
    return check_launch(fn);
  }
  if (T <= kLdsTokens && aligned(prunable, 16)) {
    if (T <= kLdsTokens / 2)
      select_one_wg_kernel<kLdsTokens / 2><<<dim3(1), dim3(kOneThreads), 0, s>>>(
          scores, prunable, static_cast<int32_t>(T), Kc, kept_idx, kept_capacity, n_kept, t_dyn);
    else
      select_one_wg_kernel<kLdsTokens><<<dim3(1), dim3(kOneThreads), 0, s>>>(
          scores, prunable, static_cast<int32_t>(T), Kc, kept_idx, kept_capacity, n_kept, t_dyn);
    return check_launch(fn);
  }
  int64_t per_block = 0;
  const int64_t G = blocks_for(T, &per_block);
  const int32_t T32 = static_cast<int32_t>(T);
  radix_hist_kernel<0><<<dim3(G), dim3(kThreads), 0, s>>>(scores, prunable, T32, per_block,
                                                           Kc, static_cast<uint32_t>(G), ws, t_dyn);
  radix_hist_kernel<1><<<dim3(G), dim3(kThreads), 0, s>>>(scores, prunable, T32, per_block,
                                                           Kc, static_cast<uint32_t>(G), ws, t_dyn);
  radix_hist_kernel<2><<<dim3(G), dim3(kThreads), 0, s>>>(scores, prunable, T32, per_block,
                                                           Kc, static_cast<uint32_t>(G), ws, t_dyn);
  compact_kernel<<<dim3(G), dim3(kThreads), 0, s>>>(scores, prunable, T32, per_block, ws,
                                                     kept_idx, kept_capacity, n_kept, t_dyn);
  return check_launch(fn);
}

}  // namespace
}  // namespace tg

namespace tg {

tg_status topk_select_call(int64_t T, const float* scores, const uint8_t* prunable, int64_t K,
                           int32_t* kept_idx, int64_t kept_capacity, int32_t* n_kept,
                           void* workspace, size_t workspace_bytes, void* stream,
                           const int32_t* t_dyn) {
  tg_status st = select_check("tg_topk_select", T, scores, prunable, K, kept_idx,
                              kept_capacity, n_kept);
  if (st != TG_OK) return st;
  if (T > 0) {
    const size_t need_bytes = tg_topk_workspace_size(T);
    if (workspace == nullptr || workspace_bytes < need_bytes)
      return fail(TG_ERR_WORKSPACE, "tg_topk_select: workspace needs %zu bytes, got %zu",
                  need_bytes, workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (!aligned(workspace, 256))
      return fail(TG_ERR_WORKSPACE, "tg_topk_select: workspace must be 256-byte aligned");
  }
  return select_launch("tg_topk_select", T, scores, prunable, K, kept_idx, kept_capacity,
                       n_kept, static_cast<uint8_t*>(workspace), as_stream(stream), t_dyn);
}

}  // namespace tg

extern "C" tg_status tg_topk_select(int64_t T, const float* scores, const uint8_t* prunable,
                                    int64_t K, int32_t* kept_idx, int64_t kept_capacity,
                                    int32_t* n_kept, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  return tg::topk_select_call(T, scores, prunable, K, kept_idx, kept_capacity, n_kept,
                              workspace, workspace_bytes, stream, nullptr);
}

extern "C" tg_status tg_topk_select_noalloc(int64_t T, const float* scores,
                                            const uint8_t* prunable, int64_t K,
                                            int32_t* kept_idx, int64_t kept_capacity,
                                            int32_t* n_kept, void* stream) {
  using namespace tg;
  const char* fn = "tg_topk_select_noalloc";
  tg_status st = select_check(fn, T, scores, prunable, K, kept_idx, kept_capacity, n_kept);
  if (st != TG_OK) return st;
  const size_t need = tg_topk_workspace_size(T);
  if (need > sizeof(scratch))
    return fail(TG_ERR_UNSUPPORTED,
                "%s: T=%lld needs %zu bytes of scratch, the static array holds %zu", fn,
                (long long)T, need, sizeof(scratch));
  hipStream_t s = as_stream(stream);
  uint8_t* ws = nullptr;
  st = static_scratch(s, &ws);
  if (st != TG_OK) return st;
  return select_launch(fn, T, scores, prunable, K, kept_idx, kept_capacity, n_kept, ws, s,
                       nullptr);
}
