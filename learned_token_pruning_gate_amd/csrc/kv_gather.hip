// kv_gather.hip -- the lower layers' KV cache gathered to the kept tokens.
//
// TokenGate pages: ai.info summary "Key Contributions" item 1 (the layers
// above the gate never hold KV entries for pruned tokens) and "Methodology in
// Plain English" (the lower layers ran on every token); the serving recipe
// compacts the lower layers' cache to the kept tokens as well, so the whole
// KV cache of the prompt holds only kept tokens.  Same kept_idx as the
// residual gather; a pure copy, bound by HBM bandwidth, normally enqueued on
// a second stream while the upper layers' attention runs.
//
// One 64-lane wave per (layer, kept token) moves its K and V rows with
// 16-byte loads and stores, four independent loads in flight per lane.
#include "tg_common.hpp"

namespace tg {
namespace {

constexpr int kPairsPerBlock = 4;   // one wave per (layer, kept token)

// One 64-lane wave moves the K row and the V row of one (layer, kept token):
// the index is read once and both rows' 16-byte loads are in flight together.
__global__ __launch_bounds__(256) void kv_gather_kernel(
    const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
    const int32_t* __restrict__ kept_idx, uint8_t* __restrict__ ko, uint8_t* __restrict__ vo,
    int64_t nvec, int32_t L, int32_t T, int32_t N, const int32_t* __restrict__ n_dyn) {
  const int lane = threadIdx.x & 63;
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * kPairsPerBlock + (threadIdx.x >> 6);
  if (pair >= static_cast<int64_t>(L) * N) return;
  const int64_t l = pair / N, r = pair - l * N;
  // with a run-time kept count (N: capacity), rows at or past it are zero
  const int32_t t = (n_dyn == nullptr || r < *n_dyn) ? kept_idx[r] : -1;
  const bool valid = t >= 0 && t < T;   // an out-of-range index yields zero rows
  const int64_t row_bytes = nvec * 16;
  const int64_t so = (l * T + (valid ? t : 0)) * row_bytes, dof = pair * row_bytes;
  const u32x4* ks = kc ? reinterpret_cast<const u32x4*>(kc + so) : nullptr;
  const u32x4* vs = vc ? reinterpret_cast<const u32x4*>(vc + so) : nullptr;
  u32x4* kd = ko ? reinterpret_cast<u32x4*>(ko + dof) : nullptr;
  u32x4* vd = vo ? reinterpret_cast<u32x4*>(vo + dof) : nullptr;
  const u32x4 z = u32x4{0, 0, 0, 0};
  for (int64_t i = lane; i < nvec; i += 128) {
    const bool two = i + 64 < nvec;
    const u32x4 k0 = (ks && valid) ? ks[i] : z;
    const u32x4 v0 = (vs && valid) ? vs[i] : z;
    const u32x4 k1 = (ks && valid && two) ? ks[i + 64] : z;
    const u32x4 v1 = (vs && valid && two) ? vs[i + 64] : z;
    if (kd) kd[i] = k0;
    if (vd) vd[i] = v0;
    if (two) {
      if (kd) kd[i + 64] = k1;
      if (vd) vd[i + 64] = v1;
    }
  }
}

}  // namespace

tg_status kv_gather_call(tg_dtype dt, int64_t L, int64_t T, int64_t N, int64_t Hkv, int64_t D,
                         const void* k_cache, const void* v_cache, const int32_t* kept_idx,
                         void* k_kept, void* v_kept, void* stream, const int32_t* n_dyn) {
  if (dt != TG_DTYPE_F32 && dt != TG_DTYPE_BF16)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_kv_gather: unknown dtype %d", (int)dt);
  if (L < 0 || T < 0 || N < 0 || Hkv < 1 || D < 1 || T > kMaxTokens || N > kMaxTokens ||
      L > 65536)
    return fail(TG_ERR_INVALID_ARGUMENT,
                "tg_kv_gather: need L, T, N >= 0 and Hkv, D >= 1 (L=%lld T=%lld N=%lld)",
                (long long)L, (long long)T, (long long)N);
  const int64_t row_bytes = Hkv * D * (dt == TG_DTYPE_BF16 ? 2 : 4);
  if (row_bytes % 16 != 0)
    return fail(TG_ERR_UNSUPPORTED, "tg_kv_gather: Hkv * D * element size must be a multiple "
                                    "of 16 bytes (%lld)", (long long)row_bytes);
  if (L == 0 || N == 0 || (k_cache == nullptr && v_cache == nullptr && k_kept == nullptr &&
                            v_kept == nullptr)) {
    clear_error();
    return TG_OK;
  }
  if (kept_idx == nullptr)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_kv_gather: kept_idx is NULL");
  if ((k_cache == nullptr) != (k_kept == nullptr) || (v_cache == nullptr) != (v_kept == nullptr))
    return fail(TG_ERR_INVALID_ARGUMENT,
                "tg_kv_gather: a cache and its output must both be given or both be NULL");
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(k_kept, 16) ||
      !aligned(v_kept, 16))
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_kv_gather: caches and outputs must be 16-byte aligned");
  const int64_t blocks = (L * N + kPairsPerBlock - 1) / kPairsPerBlock;
  if (blocks > 0x7fffffffLL)
    return fail(TG_ERR_UNSUPPORTED, "tg_kv_gather: too many rows");
  kv_gather_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, as_stream(stream)>>>(
      static_cast<const uint8_t*>(k_cache), static_cast<const uint8_t*>(v_cache), kept_idx,
      static_cast<uint8_t*>(k_kept), static_cast<uint8_t*>(v_kept), row_bytes / 16,
      static_cast<int32_t>(L), static_cast<int32_t>(T), static_cast<int32_t>(N), n_dyn);
  return check_launch("tg_kv_gather");
}

}  // namespace tg

extern "C" tg_status tg_kv_gather(tg_dtype dt, int64_t L, int64_t T, int64_t N, int64_t Hkv,
                                  int64_t D, const void* k_cache, const void* v_cache,
                                  const int32_t* kept_idx, void* k_kept, void* v_kept,
                                  void* stream) {
  return tg::kv_gather_call(dt, L, T, N, Hkv, D, k_cache, v_cache, kept_idx, k_kept, v_kept,
                            stream, nullptr);
}
