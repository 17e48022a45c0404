// compact_gather.hip -- [a4] gather of residual rows, original positions and
// gate scores into kept order.
//
// TokenGate pages: ai.info summary "Key Contributions" item 1 and the README
// mirror "How it works" -- the layers above the gate run only on the kept
// tokens, so their residual rows are compacted in original order.
//
// A pure copy, bound by HBM bandwidth: one 64-lane wave moves one row with
// 16-byte vector loads and stores (a 4 KiB bf16 row of d = 2048 is four
// coalesced 1 KiB sweeps); a 256-thread workgroup handles four rows.  The
// per-row index, position and score are handled by lane 0 of the wave.
#include "tg_common.hpp"

namespace tg {
namespace {

constexpr int kRowsPerBlock = 4;  // one wave per row

template <typename V>
__global__ __launch_bounds__(256) void gather_rows_kernel(
    const uint8_t* __restrict__ src, int64_t src_stride_bytes,
    const float* __restrict__ scores, const int32_t* __restrict__ kept_idx,
    uint8_t* __restrict__ dst, int64_t dst_stride_bytes, int64_t row_vecs,
    int32_t T, int32_t N, int32_t* __restrict__ pos_kept,
    float* __restrict__ score_kept, const int32_t* __restrict__ n_dyn) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + wave;
  if (r >= N) return;
  // with a run-time kept count (N is then the capacity), rows at or past it
  // are written as padding: zero row, position -1, score 0
  const bool live = n_dyn == nullptr || r < *n_dyn;
  const int32_t t = live ? kept_idx[r] : -1;
  const bool valid = (t >= 0) && (t < T);
  if (lane == 0) {
    if (pos_kept) pos_kept[r] = valid ? t : -1;
    if (score_kept) score_kept[r] = valid ? scores[t] : 0.0f;
  }
  if (dst == nullptr) return;
  V* d = reinterpret_cast<V*>(dst + r * dst_stride_bytes);
  if (!valid) {
    for (int64_t i = lane; i < row_vecs; i += 64) d[i] = V{};
    return;
  }
  const V* s = reinterpret_cast<const V*>(src + static_cast<int64_t>(t) * src_stride_bytes);
  // Issue up to four independent loads per lane before storing.
  int64_t i = lane;
  for (; i + 192 < row_vecs; i += 256) {
    V a = s[i], b = s[i + 64], c = s[i + 128], e = s[i + 192];
    d[i] = a;
    d[i + 64] = b;
    d[i + 128] = c;
    d[i + 192] = e;
  }
  for (; i < row_vecs; i += 64) d[i] = s[i];
}

struct alignas(16) Vec16 {
  uint32_t w[4];
};
struct alignas(4) Vec4 {
  uint32_t w;
};
struct alignas(2) Vec2 {
  uint16_t w;
};

template <typename V>
tg_status launch(const void* resid, int64_t src_stride_bytes, const float* scores,
                 const int32_t* kept_idx, void* resid_kept, int64_t dst_stride_bytes,
                 int64_t row_bytes, int64_t T, int64_t N, int32_t* pos_kept,
                 float* score_kept, hipStream_t stream, const int32_t* n_dyn) {
  const int64_t blocks = (N + kRowsPerBlock - 1) / kRowsPerBlock;
  gather_rows_kernel<V><<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream>>>(
      static_cast<const uint8_t*>(resid), src_stride_bytes, scores, kept_idx,
      static_cast<uint8_t*>(resid_kept), dst_stride_bytes,
      row_bytes / static_cast<int64_t>(sizeof(V)), static_cast<int32_t>(T),
      static_cast<int32_t>(N), pos_kept, score_kept, n_dyn);
  return check_launch("tg_compact_gather");
}

}  // namespace

tg_status compact_gather_call(tg_dtype dt, int64_t T, int64_t N, int64_t d, const void* resid,
                              int64_t resid_row_stride, const float* scores,
                              const int32_t* kept_idx, void* resid_kept,
                              int64_t kept_row_stride, int32_t* pos_kept, float* score_kept,
                              void* stream, const int32_t* n_dyn) {
  if (dt != TG_DTYPE_F32 && dt != TG_DTYPE_BF16)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_compact_gather: unknown dtype %d", (int)dt);
  if (T < 0 || T > kMaxTokens || N < 0 || N > kMaxTokens || d < 1)
    return fail(TG_ERR_INVALID_ARGUMENT,
                "tg_compact_gather: need 0 <= T, N <= 2^31-1 and d >= 1 (T=%lld N=%lld d=%lld)",
                (long long)T, (long long)N, (long long)d);
  if (N == 0) {
    clear_error();
    return TG_OK;
  }
  if (kept_idx == nullptr)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_compact_gather: kept_idx is NULL");
  if (score_kept != nullptr && scores == nullptr)
    return fail(TG_ERR_INVALID_ARGUMENT, "tg_compact_gather: score_kept needs scores");
  const int64_t esize = dt == TG_DTYPE_BF16 ? 2 : 4;
  const int64_t row_bytes = d * esize;
  int64_t sstride = 0, dstride = 0;
  if (resid_kept != nullptr) {
    if (resid == nullptr)
      return fail(TG_ERR_INVALID_ARGUMENT, "tg_compact_gather: resid is NULL");
    if (resid_row_stride < d || kept_row_stride < d)
      return fail(TG_ERR_INVALID_ARGUMENT,
                  "tg_compact_gather: row strides must be >= d (%lld, %lld < %lld)",
                  (long long)resid_row_stride, (long long)kept_row_stride, (long long)d);
    sstride = resid_row_stride * esize;
    dstride = kept_row_stride * esize;
    if (!aligned(resid, esize) || !aligned(resid_kept, esize))
      return fail(TG_ERR_INVALID_ARGUMENT, "tg_compact_gather: misaligned resid pointers");
  }
  hipStream_t s = as_stream(stream);
  const bool v16 = resid_kept == nullptr ||
                   (row_bytes % 16 == 0 && sstride % 16 == 0 && dstride % 16 == 0 &&
                    aligned(resid, 16) && aligned(resid_kept, 16));
  if (v16)
    return launch<Vec16>(resid, sstride, scores, kept_idx, resid_kept, dstride, row_bytes,
                         T, N, pos_kept, score_kept, s, n_dyn);
  const bool v4 = row_bytes % 4 == 0 && sstride % 4 == 0 && dstride % 4 == 0 &&
                  aligned(resid, 4) && aligned(resid_kept, 4);
  if (v4)
    return launch<Vec4>(resid, sstride, scores, kept_idx, resid_kept, dstride, row_bytes,
                        T, N, pos_kept, score_kept, s, n_dyn);
  return launch<Vec2>(resid, sstride, scores, kept_idx, resid_kept, dstride, row_bytes, T,
                      N, pos_kept, score_kept, s, n_dyn);
}

}  // namespace tg

extern "C" tg_status tg_compact_gather(tg_dtype dt, int64_t T, int64_t N, int64_t d,
                                       const void* resid, int64_t resid_row_stride,
                                       const float* scores, const int32_t* kept_idx,
                                       void* resid_kept, int64_t kept_row_stride,
                                       int32_t* pos_kept, float* score_kept,
                                       void* stream) {
  return tg::compact_gather_call(dt, T, N, d, resid, resid_row_stride, scores, kept_idx,
                                 resid_kept, kept_row_stride, pos_kept, score_kept, stream,
                                 nullptr);
}
