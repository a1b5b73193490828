// Row gather (FastKV summary page, sections 2A-2B: the propagated tokens'
// hidden rows become the shortened sequence; the retained K/V entries of
// each KV head become the compressed cache).
//
// Byte-generic: a row is row_bytes (a multiple of 16) copied as 16-byte
// pieces.  One launch serves up to kGatherMaxJobs gathers (K, V and the
// hidden rows of a selection pass): each job gets a share of the
// work-groups in proportion to its bytes.  A job's output rows are cut into
// tiles of rows_per_tile rows (about 32 KB); for each tile a work-group
// first resolves every row's source (one index load per row, all at once,
// into LDS), then streams the tile's pieces with consecutive threads on
// consecutive pieces and kUnroll pieces per thread in flight.  Row loads
// and stores are non-temporal (each byte is touched once), which a plain
// 1 GiB copy on MI355X measures ~10% faster than cached accesses.
//
// Paged variant (the compressed K/V written straight into a decode cache
// kept in fixed-size blocks): the destination of selected row s of a
// sequence is slot s % block_size of block block_table[s / block_size];
// rows whose block number is outside [0, num_blocks) are not written.
#include "kvsel_internal.hpp"

namespace kvsel {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr int kMaxBlocks = 256 * 32;   // blocks stride beyond
constexpr int kTilePieces = 2048;      // 16-byte pieces per tile (32 KB)

template <bool PAGED>
__global__ __launch_bounds__(kThreads) void k_gather(GatherLaunch a) {
  __shared__ int64_t s_src[kGatherMaxTileRows], s_dst[kGatherMaxTileRows];
  int j = 0;
  while (j + 1 < a.njobs && static_cast<int>(blockIdx.x) >= a.job[j + 1].block0) ++j;
  const GatherJob& jb = a.job[j];
  const int nblocks = (j + 1 < a.njobs ? a.job[j + 1].block0 : static_cast<int>(gridDim.x)) - jb.block0;
  const int rt = jb.rows_per_tile;
  const int64_t ntiles = (jb.rows_out + rt - 1) / rt;
  const u32x4* src = static_cast<const u32x4*>(jb.src);
  u32x4* dst = static_cast<u32x4*>(jb.dst);
  for (int64_t tile = blockIdx.x - jb.block0; tile < ntiles; tile += nblocks) {
    const int64_t r0 = tile * rt;
    const int nrows = static_cast<int>(min(static_cast<int64_t>(rt), jb.rows_out - r0));
    // sources of the tile's rows: output row rh = s_local * heads + h
    for (int t = threadIdx.x; t < nrows; t += kThreads) {
      const int rh = static_cast<int>(r0) + t;                   // rows_out < 2^31
      const int q = rh / jb.heads;
      const int h = rh - q * jb.heads;
      const int64_t s = static_cast<int64_t>(jb.out[0]) + q;    // global output position
      const int sq = find_segment(jb.out, a.count, s);
      const int32_t pos = jb.idx[(jb.per_head ? static_cast<int64_t>(h) : 0) * jb.L + s];
      if constexpr (PAGED) {
        const int sl = static_cast<int>(s - jb.out[sq]);          // sequence-local position
        const int32_t blk = jb.block_table[static_cast<int64_t>(sq) * jb.max_blocks + sl / jb.block_size];
        s_dst[t] = (blk < 0 || blk >= jb.num_blocks)
                       ? -1
                       : ((static_cast<int64_t>(blk) * jb.block_size + sl % jb.block_size) * jb.heads + h) *
                             jb.cpr;
      } else {
        s_dst[t] = (s * jb.heads + h) * jb.cpr;
      }
      s_src[t] = (pos < 0 || pos >= a.len[sq]) ? -1 : ((static_cast<int64_t>(a.off[sq]) + pos) * jb.heads + h) * jb.cpr;
    }
    __syncthreads();
    const int pieces = nrows * jb.cpr;
    for (int p0 = threadIdx.x; p0 < pieces; p0 += kThreads * kUnroll) {
      u32x4 v[kUnroll];
      int64_t d[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int p = min(p0 + u * kThreads, pieces - 1);
        const int row = jb.cpr_shift >= 0 ? (p >> jb.cpr_shift) : p / jb.cpr;
        const int c = p - row * jb.cpr;
        const int64_t so = s_src[row];
        const int64_t dr = s_dst[row];
        d[u] = (PAGED && dr < 0) ? -1 : dr + c;
        v[u] = so >= 0 ? __builtin_nontemporal_load(src + so + c) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (p0 + u * kThreads < pieces && (!PAGED || d[u] >= 0)) __builtin_nontemporal_store(v[u], dst + d[u]);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_gather(GatherLaunch& a, hipStream_t stream) {
  // rows per tile: about 32 KB of pieces (on MI355X a sweep of tile size,
  // work-group cap and pieces in flight put 16-32 KB tiles ~5% ahead of
  // 64 KB ones for the K/V/hidden gathers of a 128K-token pass);
  // work-groups in proportion to each job's bytes, at least one per job
  int64_t total = 0;
  for (int j = 0; j < a.njobs; ++j) {
    GatherJob& jb = a.job[j];
    int rt = kTilePieces / jb.cpr;
    jb.rows_per_tile = rt < 1 ? 1 : (rt > kGatherMaxTileRows ? kGatherMaxTileRows : rt);
    total += jb.rows_out * jb.cpr;
  }
  if (total <= 0) return hipSuccess;
  int64_t want = (total + kTilePieces - 1) / kTilePieces;   // about one tile per work-group
  if (want > kMaxBlocks) want = kMaxBlocks;
  int blocks = 0;
  for (int j = 0; j < a.njobs; ++j) {
    a.job[j].block0 = blocks;
    const int64_t pj = a.job[j].rows_out * a.job[j].cpr;
    int64_t bj = pj > 0 ? (pj * want + total - 1) / total : 0;
    if (pj > 0 && bj < 1) bj = 1;
    blocks += static_cast<int>(bj);
  }
  if (a.paged)
    k_gather<true><<<blocks, kThreads, 0, stream>>>(a);
  else
    k_gather<false><<<blocks, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace kvsel
