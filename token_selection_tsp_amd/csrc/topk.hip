// Top-k plus the window (FastKV summary page, section 2A: the selected subset
// is propagated together with the window tokens; section 2B / StructKV
// section 2C: one call per decoupled budget).
//
// Exact selection of the k largest candidates of every (row, sequence), ties
// to the lower position, written in ascending order and followed by the
// window.  Values become order-preserving 32-bit keys (-0 folded onto +0);
// everything after that is integer, so the result is exact and
// deterministic.  Four launches, each spread over the whole GPU:
//  0. bracket (one work-group per row and sequence): 4096 evenly spaced keys
//     are sampled; one histogram over their key range locates two sample
//     ranks a few standard deviations either side of the expected rank of
//     the k-th largest, and the outer edges of their bins bound where it
//     must lie.  Rows whose candidates all fit the list take every key.
//  1. collect (one work-group per 4096-key chunk): count the chunk's keys
//     above the bracket and append the keys inside it, with their positions,
//     to the row's candidate list (space reserved once per work-group).
//  2. threshold (one work-group per row and sequence): the k-th largest key
//     tau is found exactly among the candidates by radix select over the
//     shrinking key range in LDS, and with it how many keys equal to tau are
//     kept; then every chunk's output offset follows from the per-chunk
//     counts in index order.  If the bracket missed (or the list overflowed)
//     the same select runs over the whole row -- slower, still exact.
//  3. write (one work-group per chunk): keys above tau plus the first kept
//     keys equal to tau, compacted in index order at the chunk's offset; the
//     first chunk also writes the window.
#include "kvsel_internal.hpp"

namespace kvsel {
namespace {

constexpr int kBig = 1024;                    // threads of the per-row kernels
constexpr int kSmall = 256;                   // threads of the per-chunk kernels
constexpr int kPerThread = kTopkChunk / kSmall;
constexpr int kBins = 2048;
constexpr int kSample = 4096;

// per (row, sequence) state words
enum { kLo = 0, kHi, kCount, kTau, kTakeEq, kMode, kAbove, kStateWords = 8 };
enum { kModeSelect = 0, kModeNone = 1, kModeAll = 2 };
// per (row, chunk) words
enum { kAboveC = 0, kCandC, kOutPos, kEqBefore, kChunkWords = 4 };

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;                       // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // larger float -> larger key
}

// Exclusive prefix sum over the work-group in thread order; *total gets the sum.
template <int NT>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
  constexpr int W = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const uint32_t s = sh[i];
    pre += (i < wave) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return pre + x - v;
}

struct SelectShared {
  uint32_t hist[kBins];
  uint32_t sh[kBig / 64];
  uint32_t sel_lo, sel_krem;
};

// The krem-th largest key (1-based) among those in [lo, hi] that visit()
// yields (visit(f) calls f(key) for every key).  Returns the key; *krem_out
// = its rank among the keys equal to it, i.e. how many of them are kept.
// Radix over the shrinking key range, at most 2048 bins per pass.
template <typename Visit>
__device__ uint32_t select_kth(Visit visit, uint32_t lo, uint32_t hi, uint32_t krem,
                               SelectShared& S, uint32_t* krem_out) {
  const int tid = threadIdx.x;
  while (lo < hi) {
    const uint32_t span = hi - lo;
    const int bits = 32 - __clz(span);
    const int shift = bits > 11 ? bits - 11 : 0;
    const int nbins = static_cast<int>(span >> shift) + 1;
    for (int b = tid; b < nbins; b += kBig) S.hist[b] = 0u;
    __syncthreads();
    visit([&](uint32_t u) {
      if (u >= lo && u <= hi) atomicAdd(&S.hist[(u - lo) >> shift], 1u);
    });
    __syncthreads();
    // thread t owns bins top-2t and top-2t-1 (descending); its exclusive
    // prefix counts the keys in all higher bins
    const int b1 = nbins - 1 - 2 * tid;
    const int b0 = b1 - 1;
    const uint32_t h1 = b1 >= 0 ? S.hist[b1] : 0u;
    const uint32_t h0 = b0 >= 0 ? S.hist[b0] : 0u;
    uint32_t tot;
    const uint32_t above = block_scan<kBig>(h1 + h0, S.sh, &tot);
    if (b1 >= 0 && above < krem && above + h1 >= krem) {
      S.sel_lo = lo + (static_cast<uint32_t>(b1) << shift);
      S.sel_krem = krem - above;
    } else if (b0 >= 0 && above + h1 < krem && above + h1 + h0 >= krem) {
      S.sel_lo = lo + (static_cast<uint32_t>(b0) << shift);
      S.sel_krem = krem - above - h1;
    }
    __syncthreads();
    const uint32_t nlo = S.sel_lo;
    const uint64_t top = static_cast<uint64_t>(nlo) + ((1ull << shift) - 1ull);
    hi = top < hi ? static_cast<uint32_t>(top) : hi;
    lo = nlo;
    krem = S.sel_krem;
    __syncthreads();
  }
  *krem_out = krem;
  return lo;
}

struct Ctx {    // one (row, sequence)
  const float* x;
  int n, nc, keep, w;
  uint32_t* st;
  uint32_t* chunks;   // this sequence's first chunk record
  uint32_t* list;     // candidate list: (key, position) pairs
  int nchunks, cap;
};

__device__ __forceinline__ Ctx ctx_of(const float* keys, int64_t T, const SelBatch& sb, const TopkWork& wk,
                                      int sq, int row, int w) {
  Ctx c;
  c.n = sb.len[sq];
  c.nc = c.n - w;
  c.keep = sb.keep[sq];
  c.w = w;
  c.x = keys + static_cast<size_t>(row) * T + sb.off[sq];
  c.st = wk.state + (static_cast<size_t>(row) * sb.count + sq) * kStateWords;
  c.chunks = wk.chunk + (static_cast<size_t>(row) * wk.chunks_total + sb.chunk0[sq]) * kChunkWords;
  c.list = wk.list + (static_cast<size_t>(row) * wk.list_total + sb.list0[sq]) * 2;
  c.nchunks = sb.chunk0[sq + 1] - sb.chunk0[sq];
  c.cap = sb.list0[sq + 1] - sb.list0[sq];
  return c;
}

// ---- 0: bracket ----------------------------------------------------------------
__global__ __launch_bounds__(kBig) void k_topk_bracket(const float* __restrict__ keys, int64_t T,
                                                       SelBatch sb, int w, TopkWork wk) {
  __shared__ SelectShared S;
  __shared__ uint32_t s_min[kBig / 64], s_max[kBig / 64];
  const Ctx c = ctx_of(keys, T, sb, wk, blockIdx.x, blockIdx.y, w);
  const int tid = threadIdx.x;
  uint32_t lo = 0u, hi = 0xFFFFFFFFu, mode = kModeSelect;
  if (c.keep == 0) {
    mode = kModeNone;
  } else if (c.keep >= c.nc) {
    mode = kModeAll;
  } else if (c.nc > c.cap) {
    // The list cannot hold every key: bracket the k-th largest with a sample
    // of evenly spaced keys.  One histogram of the sample over its key range
    // locates the sample ranks r_hi < r < r_lo (a generous margin either
    // side of the expected rank r of the k-th largest); the bracket is the
    // outer edges of their bins.
    const int stride = c.nc / kSample;   // >= 1 since nc > cap >= kSample
    uint32_t u[kSample / kBig];
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
    for (int e = 0; e < kSample / kBig; ++e) {
      u[e] = order_key(c.x[(e * kBig + tid) * stride]);
      mn = min(mn, u[e]);
      mx = max(mx, u[e]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      mn = min(mn, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mn), o)));
      mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), o)));
    }
    if ((tid & 63) == 0) { s_min[tid >> 6] = mn; s_max[tid >> 6] = mx; }
    for (int b = tid; b < kBins; b += kBig) S.hist[b] = 0u;
    __syncthreads();
    mn = s_min[0]; mx = s_max[0];
#pragma unroll
    for (int i = 1; i < kBig / 64; ++i) { mn = min(mn, s_min[i]); mx = max(mx, s_max[i]); }
    const uint32_t span = mx - mn;
    const int bits = span ? 32 - __clz(span) : 0;
    const int shift = bits > 11 ? bits - 11 : 0;
    const int nbins = static_cast<int>(span >> shift) + 1;
#pragma unroll
    for (int e = 0; e < kSample / kBig; ++e) atomicAdd(&S.hist[(u[e] - mn) >> shift], 1u);
    __syncthreads();
    const double r = static_cast<double>(c.keep) * kSample / c.nc;   // expected sample rank
    const double margin = 4.0 * sqrt(fmax(r * (1.0 - r / kSample), 0.0)) + 8.0;
    const int r_hi = static_cast<int>(floor(r - margin));          // 0-based, descending
    const int r_lo = static_cast<int>(ceil(r + margin));
    // thread t owns bins top-2t, top-2t-1; `above` counts the higher bins
    const int b1 = nbins - 1 - 2 * tid;
    const int b0 = b1 - 1;
    const uint32_t h1 = b1 >= 0 ? S.hist[b1] : 0u;
    const uint32_t h0 = b0 >= 0 ? S.hist[b0] : 0u;
    uint32_t tot;
    const uint32_t above = block_scan<kBig>(h1 + h0, S.sh, &tot);
    auto owns = [&](int rank, int b, uint32_t before, uint32_t h) {
      return b >= 0 && rank >= 0 && static_cast<uint32_t>(rank) >= before &&
             static_cast<uint32_t>(rank) < before + h;
    };
    // bin edges: bin b covers keys mn + (b << shift) .. mn + ((b + 1) << shift) - 1
    auto top_of = [&](int b) {
      const uint64_t t = static_cast<uint64_t>(mn) + ((static_cast<uint64_t>(b) + 1) << shift) - 1;
      return t > 0xFFFFFFFFull ? 0xFFFFFFFFu : static_cast<uint32_t>(t);
    };
    if (owns(r_hi, b1, above, h1)) S.sel_lo = top_of(b1);
    if (owns(r_hi, b0, above + h1, h0)) S.sel_lo = top_of(b0);
    if (owns(r_lo, b1, above, h1)) S.sel_krem = mn + (static_cast<uint32_t>(b1) << shift);
    if (owns(r_lo, b0, above + h1, h0)) S.sel_krem = mn + (static_cast<uint32_t>(b0) << shift);
    __syncthreads();
    if (r_hi >= 0) hi = S.sel_lo;
    if (r_lo < kSample) lo = S.sel_krem;
  }
  if (tid == 0) {
    c.st[kLo] = lo;
    c.st[kHi] = hi;
    c.st[kCount] = 0u;
    c.st[kMode] = mode;
  }
}

// ---- 1: collect ----------------------------------------------------------------
__global__ __launch_bounds__(kSmall) void k_topk_collect(const float* __restrict__ keys, int64_t T,
                                                         SelBatch sb, int w, TopkWork wk) {
  __shared__ uint32_t sh[kSmall / 64];
  __shared__ uint32_t s_base;
  const int sq = find_segment(sb.chunk0, sb.count, static_cast<int>(blockIdx.x));
  const int cc = blockIdx.x - sb.chunk0[sq];
  const Ctx c = ctx_of(keys, T, sb, wk, sq, blockIdx.y, w);
  if (c.st[kMode] != kModeSelect) return;
  const uint32_t lo = c.st[kLo], hi = c.st[kHi];
  const int tid = threadIdx.x;
  const int j0 = cc * kTopkChunk;
  uint32_t u[kPerThread];
  int j[kPerThread];
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    j[e] = j0 + e * kSmall + tid;
    u[e] = order_key(c.x[min(j[e], c.nc - 1)]);
  }
  uint32_t above = 0, inside = 0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const bool ok = j[e] < c.nc;
    above += (ok && u[e] > hi) ? 1u : 0u;
    inside += (ok && u[e] >= lo && u[e] <= hi) ? 1u : 0u;
  }
  uint32_t tot_in, tot_above;
  const uint32_t pre = block_scan<kSmall>(inside, sh, &tot_in);
  block_scan<kSmall>(above, sh, &tot_above);
  if (tid == 0) {
    s_base = tot_in ? atomicAdd(&c.st[kCount], tot_in) : 0u;
    uint32_t* rec = c.chunks + static_cast<size_t>(cc) * kChunkWords;
    rec[kAboveC] = tot_above;
    rec[kCandC] = tot_in;
  }
  __syncthreads();
  uint32_t pos = s_base + pre;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    if (j[e] < c.nc && u[e] >= lo && u[e] <= hi) {
      if (pos < static_cast<uint32_t>(c.cap)) {
        c.list[2 * static_cast<size_t>(pos)] = u[e];
        c.list[2 * static_cast<size_t>(pos) + 1] = static_cast<uint32_t>(j[e]);
      }
      ++pos;
    }
  }
}

// ---- 2: threshold and chunk offsets --------------------------------------------
__global__ __launch_bounds__(kBig) void k_topk_threshold(const float* __restrict__ keys, int64_t T,
                                                         SelBatch sb, int w, TopkWork wk) {
  __shared__ SelectShared S;
  __shared__ uint32_t cand[kTopkCap];
  __shared__ uint32_t gt_c[kTopkMaxChunks], eq_c[kTopkMaxChunks];
  const Ctx c = ctx_of(keys, T, sb, wk, blockIdx.x, blockIdx.y, w);
  if (c.st[kMode] != kModeSelect) return;
  const int tid = threadIdx.x;
  const uint32_t keep = static_cast<uint32_t>(c.keep);
  const uint32_t lo = c.st[kLo], hi = c.st[kHi];
  const uint32_t count = c.st[kCount];
  // keys above the bracket over the whole row
  uint32_t above_mine = 0;
  for (int i = tid; i < c.nchunks; i += kBig) above_mine += c.chunks[static_cast<size_t>(i) * kChunkWords + kAboveC];
  uint32_t above;
  block_scan<kBig>(above_mine, S.sh, &above);
  const bool listed = count <= static_cast<uint32_t>(c.cap) && count <= static_cast<uint32_t>(kTopkCap);
  const bool bracketed = listed && above < keep && keep <= above + count;
  for (int i = tid; i < c.nchunks; i += kBig) { gt_c[i] = 0u; eq_c[i] = 0u; }

  uint32_t tau, take_eq;
  if (bracketed) {
    // the whole list in one batch of loads; positions stay in registers
    constexpr int E = kTopkCap / kBig;
    const uint2* lst = reinterpret_cast<const uint2*>(c.list);
    uint2 ent[E];
#pragma unroll
    for (int e = 0; e < E; ++e) ent[e] = lst[min(static_cast<uint32_t>(e * kBig + tid), count - 1u)];
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (static_cast<uint32_t>(e * kBig + tid) < count) cand[e * kBig + tid] = ent[e].x;
    __syncthreads();
    auto vis = [&](auto f) {
      for (uint32_t i = tid; i < count; i += kBig) f(cand[i]);
    };
    tau = select_kth(vis, lo, hi, keep - above, S, &take_eq);
    // per-chunk keys above / equal to tau: the chunk's keys above the bracket
    // plus its candidates above tau
    for (int i = tid; i < c.nchunks; i += kBig) gt_c[i] = c.chunks[static_cast<size_t>(i) * kChunkWords + kAboveC];
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (static_cast<uint32_t>(e * kBig + tid) < count) {
        const uint32_t ch = ent[e].y / kTopkChunk;
        if (ent[e].x > tau) atomicAdd(&gt_c[ch], 1u);
        else if (ent[e].x == tau) atomicAdd(&eq_c[ch], 1u);
      }
    }
  } else {
    // the bracket missed: exact select over the whole row, then recount
    __syncthreads();
    auto vis = [&](auto f) {
      for (int j = tid; j < c.nc; j += kBig) f(order_key(c.x[j]));
    };
    tau = select_kth(vis, 0u, 0xFFFFFFFFu, keep, S, &take_eq);
    for (int j = tid; j < c.nc; j += kBig) {
      const uint32_t u = order_key(c.x[j]);
      if (u > tau) atomicAdd(&gt_c[j / kTopkChunk], 1u);
      else if (u == tau) atomicAdd(&eq_c[j / kTopkChunk], 1u);
    }
  }
  __syncthreads();
  // chunk offsets in index order: equal keys are kept first-come
  uint32_t eq_run = 0, out_run = 0;
  for (int base = 0; base < c.nchunks; base += kBig) {
    const int i = base + tid;
    const uint32_t g = i < c.nchunks ? gt_c[i] : 0u;
    const uint32_t q = i < c.nchunks ? eq_c[i] : 0u;
    uint32_t eq_tot;
    const uint32_t eq_pre = eq_run + block_scan<kBig>(q, S.sh, &eq_tot);
    const uint32_t rem = take_eq > eq_pre ? take_eq - eq_pre : 0u;
    const uint32_t sel = g + min(q, rem);
    uint32_t sel_tot;
    const uint32_t out_pre = out_run + block_scan<kBig>(sel, S.sh, &sel_tot);
    if (i < c.nchunks) {
      uint32_t* rec = c.chunks + static_cast<size_t>(i) * kChunkWords;
      rec[kOutPos] = out_pre;
      rec[kEqBefore] = eq_pre;
    }
    eq_run += eq_tot;
    out_run += sel_tot;
  }
  if (tid == 0) {
    c.st[kTau] = tau;
    c.st[kTakeEq] = take_eq;
  }
}

// ---- 3: write ------------------------------------------------------------------
__global__ __launch_bounds__(kSmall) void k_topk_write(const float* __restrict__ keys, int64_t T,
                                                       SelBatch sb, int w, TopkWork wk,
                                                       int32_t* __restrict__ idx, int64_t L) {
  __shared__ uint32_t sh[kSmall / 64];
  const int sq = find_segment(sb.chunk0, sb.count, static_cast<int>(blockIdx.x));
  const int cc = blockIdx.x - sb.chunk0[sq];
  const int row = blockIdx.y;
  const Ctx c = ctx_of(keys, T, sb, wk, sq, row, w);
  int32_t* out = idx + static_cast<size_t>(row) * L + sb.out[sq];
  const int tid = threadIdx.x;
  const uint32_t mode = c.st[kMode];
  if (cc == 0)
    for (int t = tid; t < w; t += kSmall) out[c.keep + t] = c.nc + t;
  const int j0 = cc * kTopkChunk;
  if (mode == kModeNone) return;
  if (mode == kModeAll) {
    for (int j = j0 + tid; j < min(c.nc, j0 + kTopkChunk); j += kSmall) out[j] = j;
    return;
  }
  const uint32_t tau = c.st[kTau];
  const uint32_t* rec = c.chunks + static_cast<size_t>(cc) * kChunkWords;
  const uint32_t out_pos = rec[kOutPos];
  const uint32_t eq_before = rec[kEqBefore];
  const uint32_t take_eq = c.st[kTakeEq];
  const uint32_t rem = take_eq > eq_before ? take_eq - eq_before : 0u;
  // thread t owns kPerThread consecutive keys, so its scan prefix is in index order
  const int a = j0 + tid * kPerThread;
  uint32_t u[kPerThread];
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) u[e] = order_key(c.x[min(a + e, c.nc - 1)]);
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const bool ok = a + e < c.nc;
    gt += (ok && u[e] > tau) ? 1u : 0u;
    eq += (ok && u[e] == tau) ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t pre = block_scan<kSmall>((gt << 16) | eq, sh, &tot);   // < 2^16 each per chunk
  const uint32_t gt_pre = pre >> 16, eq_pre = pre & 0xFFFFu;
  uint32_t pos = out_pos + gt_pre + min(eq_pre, rem);
  uint32_t eq_left = rem > eq_pre ? rem - eq_pre : 0u;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    if (a + e < c.nc) {
      bool k = u[e] > tau;
      if (u[e] == tau && eq_left > 0) { k = true; --eq_left; }
      if (k) out[pos++] = a + e;
    }
  }
}

}  // namespace

size_t topk_workspace_bytes(int rows, int count, int chunks_total, int64_t list_total) {
  const size_t st = static_cast<size_t>(rows) * count * kStateWords * 4;
  const size_t ch = static_cast<size_t>(rows) * chunks_total * kChunkWords * 4;
  const size_t li = static_cast<size_t>(rows) * list_total * 8;
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  return up(st) + up(ch) + up(li);
}

hipError_t launch_topk(const float* keys, int64_t T, int rows, int w, const SelBatch& sb,
                       int32_t* idx, int64_t L, void* ws, hipStream_t stream) {
  const int chunks_total = sb.chunk0[sb.count];
  const int64_t list_total = sb.list0[sb.count];
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  TopkWork wk;
  char* p = static_cast<char*>(ws);
  wk.state = reinterpret_cast<uint32_t*>(p);
  p += up(static_cast<size_t>(rows) * sb.count * kStateWords * 4);
  wk.chunk = reinterpret_cast<uint32_t*>(p);
  p += up(static_cast<size_t>(rows) * chunks_total * kChunkWords * 4);
  wk.list = reinterpret_cast<uint32_t*>(p);
  wk.chunks_total = chunks_total;
  wk.list_total = list_total;
  k_topk_bracket<<<dim3(sb.count, rows), kBig, 0, stream>>>(keys, T, sb, w, wk);
  k_topk_collect<<<dim3(chunks_total, rows), kSmall, 0, stream>>>(keys, T, sb, w, wk);
  k_topk_threshold<<<dim3(sb.count, rows), kBig, 0, stream>>>(keys, T, sb, w, wk);
  k_topk_write<<<dim3(chunks_total, rows), kSmall, 0, stream>>>(keys, T, sb, w, wk, idx, L);
  return hipGetLastError();
}

}  // namespace kvsel
