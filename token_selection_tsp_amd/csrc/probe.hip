// Streaming-read probe: the memory-system reference rates that the score,
// top-k and gather kernels are priced against (a plain read of a large
// buffer, a read in the key cache's [T, h_kv, d] layout one head at a time,
// and a re-read of a buffer that fits the last-level cache).  Not a step of
// the selection path: a measurement aid, so the ceilings quoted for the
// kernels can be re-measured from the library itself.
//
// Work-group (x, h) reads rows [x*rpw, (x+1)*rpw) of head h: row r of head h
// is the row_bytes bytes at r*stride + h*row_bytes.  Consecutive threads take
// consecutive 16-byte pieces of that range (whole cache lines per wave), each
// thread keeps eight loads in flight, and the XOR of everything it read goes
// to one word per work-group so that no load can be dropped.
#include "kvsel_internal.hpp"

namespace kvsel {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeInFlight = 8;

__global__ __launch_bounds__(kProbeThreads) void k_probe_read(const char* __restrict__ base, int64_t rows,
                                                              int row_shift, int row_bytes, int64_t stride,
                                                              int64_t rpw, uint32_t* __restrict__ out) {
  const int h = blockIdx.y;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * rpw;
  const int64_t r1 = r0 + rpw < rows ? r0 + rpw : rows;
  const int64_t np = r0 < r1 ? (r1 - r0) << (row_shift - 4) : 0;   // 16-byte pieces
  const int pmask = (row_bytes >> 4) - 1;
  const char* hb = base + static_cast<int64_t>(h) * row_bytes;
  uint4 acc = make_uint4(0u, 0u, 0u, 0u);
  for (int64_t p0 = threadIdx.x; p0 < np; p0 += kProbeThreads * kProbeInFlight) {
    uint4 v[kProbeInFlight];
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) {
      const int64_t p = p0 + static_cast<int64_t>(u) * kProbeThreads;
      const int64_t pc = p < np ? p : np - 1;   // clamped: every load stays inside the range
      const int64_t r = r0 + (pc >> (row_shift - 4));
      v[u] = *reinterpret_cast<const uint4*>(hb + r * stride + ((pc & pmask) << 4));
    }
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) {
      acc.x ^= v[u].x; acc.y ^= v[u].y; acc.z ^= v[u].z; acc.w ^= v[u].w;
    }
  }
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  __shared__ uint32_t red[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int i = 0; i < kProbeThreads / 64; ++i) t ^= red[i];
    out[static_cast<size_t>(h) * gridDim.x + blockIdx.x] = t;
  }
}

}  // namespace

hipError_t launch_probe_read(const void* src, int64_t rows, int heads, int row_bytes, int64_t stride,
                             int wgs, uint32_t* out, hipStream_t stream) {
  const int64_t rpw = (rows + wgs - 1) / wgs;
  k_probe_read<<<dim3(wgs, heads), kProbeThreads, 0, stream>>>(static_cast<const char*>(src), rows,
                                                                __builtin_ctz(static_cast<unsigned>(row_bytes)),
                                                                row_bytes, stride, rpw, out);
  return hipGetLastError();
}

}  // namespace kvsel
