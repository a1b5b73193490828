// Row gather (FastKV summary page, sections 2A-2B: the propagated tokens'
// hidden rows become the shortened sequence; the retained K/V entries of
// each KV head become the compressed cache).
//
// Byte-generic: a row is row_bytes (a multiple of 16) copied as 16-byte
// lanes.  Consecutive threads cover consecutive 16-byte pieces of a row and
// then consecutive rows, so row loads and all stores are coalesced.  Stores
// are non-temporal: the compacted tensors are not read again by this pass.
#include "kvsel_internal.hpp"

namespace kvsel {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void copy16(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                       bool valid) {
  uint4 v = valid ? *src : make_uint4(0u, 0u, 0u, 0u);
  __builtin_nontemporal_store(v.x, &dst->x);
  __builtin_nontemporal_store(v.y, &dst->y);
  __builtin_nontemporal_store(v.z, &dst->z);
  __builtin_nontemporal_store(v.w, &dst->w);
}

// Output row rh (launch-local, = s_local * heads + h) -> source row, or -1.
__device__ __forceinline__ int64_t source_row(int rh, int heads, const int32_t* __restrict__ idx,
                                              int per_head, int64_t L, const SelBatch& sb,
                                              int64_t* out_row) {
  const int h = rh % heads;
  const int64_t s = static_cast<int64_t>(sb.out[0]) + rh / heads;   // global output position
  const int sq = find_segment(sb.out, sb.count, s);
  const int32_t pos = idx[(per_head ? static_cast<int64_t>(h) : 0) * L + s];
  *out_row = s * heads + h;
  if (pos < 0 || pos >= sb.len[sq]) return -1;
  return (static_cast<int64_t>(sb.off[sq]) + pos) * heads + h;
}

__global__ __launch_bounds__(kThreads) void k_gather(const uint4* __restrict__ src, int heads, int cpr,
                                                     const int32_t* __restrict__ idx, int per_head,
                                                     int64_t L, SelBatch sb, uint4* __restrict__ dst,
                                                     int rows_out) {
  if (cpr <= kThreads) {
    const int rpi = kThreads / cpr;              // rows per block iteration
    const int rl = threadIdx.x / cpr;
    const int c = threadIdx.x - rl * cpr;
    if (rl >= rpi) return;
    for (int rh = blockIdx.x * rpi + rl; rh < rows_out; rh += gridDim.x * rpi) {
      int64_t orow;
      const int64_t srow = source_row(rh, heads, idx, per_head, L, sb, &orow);
      copy16(src + (srow < 0 ? 0 : srow) * cpr + c, dst + orow * cpr + c, srow >= 0);
    }
  } else {
    for (int rh = blockIdx.x; rh < rows_out; rh += gridDim.x) {
      int64_t orow;
      const int64_t srow = source_row(rh, heads, idx, per_head, L, sb, &orow);
      for (int c = threadIdx.x; c < cpr; c += kThreads)
        copy16(src + (srow < 0 ? 0 : srow) * cpr + c, dst + orow * cpr + c, srow >= 0);
    }
  }
}

}  // namespace

hipError_t launch_gather(const void* src, int heads, int row_bytes, const int32_t* idx,
                         int idx_per_head, int64_t L, const SelBatch& sb, void* dst,
                         hipStream_t stream) {
  const int cpr = row_bytes / 16;
  const int64_t rows_out = (static_cast<int64_t>(sb.out[sb.count]) - sb.out[0]) * heads;
  if (rows_out <= 0) return hipSuccess;
  const int rpi = cpr <= kThreads ? kThreads / cpr : 1;
  int64_t blocks = (rows_out + rpi - 1) / rpi;
  const int64_t cap = 256 * 16;   // fills 256 CUs; the kernel strides beyond
  if (blocks > cap) blocks = cap;
  k_gather<<<static_cast<unsigned>(blocks), kThreads, 0, stream>>>(
      static_cast<const uint4*>(src), heads, cpr, idx, idx_per_head, L, sb,
      static_cast<uint4*>(dst), static_cast<int>(rows_out));
  return hipGetLastError();
}

}  // namespace kvsel
