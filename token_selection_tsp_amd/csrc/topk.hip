// Top-k plus the window (FastKV summary page, section 2A: the selected subset
// is propagated together with the window tokens; section 2B / StructKV
// section 2C: the KV-retention budget and the propagation budget are
// independent, so one launch pair can serve both).
//
// Exact selection of the k largest candidates of every (row, sequence), ties
// to the lower position, written in ascending order and followed by the
// window.  Values become order-preserving 32-bit keys (-0 folded onto +0);
// everything after that is integer, so the result is exact and
// deterministic.  A launch takes one of two paths, both over every row of up
// to two budgets: for short rows, or many sequences, one launch with one
// work-group per (row, sequence) (k_topk_row, below); otherwise two
// launches:
//  1. collect (one work-group per 4096-key chunk).  Each work-group first
//     brackets the k-th largest key of its row by itself: evenly spaced keys
//     of the row are sampled and one histogram over their key range locates
//     two sample ranks a few standard deviations either side of the
//     expected rank; the bracket is the outer edges of their bins.  Every
//     work-group of a row computes the same bracket from the same sample, so
//     no launch is spent on it.  (Rows whose candidates all fit the select's
//     buffer take every key.)  Then it counts its chunk's keys above the
//     bracket and writes the keys inside it, with their positions, to the
//     chunk's own slot of the workspace.
//  2. finish (several work-groups per row and sequence, as many as fill the
//     GPU once).  Each finds the k-th
//     largest key tau exactly among the candidates by radix select over the
//     shrinking key range in LDS, and with it how many keys equal to tau are
//     kept; every chunk's output offset follows from per-chunk counts in
//     index order.  (If the bracket missed, the select runs over the whole
//     row: slower, still exact.)  The work-groups of a row compute the same
//     threshold (deterministically) and each writes its share of the chunks,
//     so no work-group waits for another.
#include "kvsel_internal.hpp"

namespace kvsel {
namespace {

constexpr int kBig = 1024;                    // threads of the finish kernel
constexpr int kSmall = 256;                   // threads of the collect kernel
constexpr int kPerThread = kTopkChunk / kSmall;
constexpr int kBins = 2048;
constexpr int kSample = 4096;
constexpr int kFinishWGs = 256;               // finish work-groups in all: one per compute unit
constexpr int kWriteBatch = 4;                // chunks a finish work-group loads at once
constexpr int kRowMaxKeys = 65536;            // longest row the one-work-group path takes
static_assert(kTopkCap >= 4 * (kSample / 4), "sampled rows need 4 adjacent keys per sample point");

// per (row, chunk) words, written by collect
enum { kAboveC = 0, kCandC };
static_assert(kTopkChunkWords == 2, "a chunk record holds its count above the bracket and its candidates");
enum { kModeSelect = 0, kModeNone = 1, kModeAll = 2 };

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;                       // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // larger float -> larger key
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (a few
// cycles each, against ~100 for an LDS-crossbar shuffle): shifts by 1, 2, 4
// and 8 within each row of 16 lanes (lanes shifted in from outside the row
// read 0), then row 0's total into row 1 and row 2's into row 3, then the
// total of rows 0-1 into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t x) {
  constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowShr + 1, 0xf, 0xf, true));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowShr + 2, 0xf, 0xf, true));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowShr + 4, 0xf, 0xf, true));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowShr + 8, 0xf, 0xf, true));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowBcast15, 0xa, 0xf, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowBcast31, 0xc, 0xf, false));
  return x;
}

// Exclusive prefix sum over the work-group in thread order; *total gets the sum.
template <int NT>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
  constexpr int W = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_scan_incl(v);
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

// block_scan without its closing barrier: for a caller that passes a
// work-group barrier before sh is written again.
template <int NT>
__device__ __forceinline__ uint32_t block_scan_open(uint32_t v, uint32_t* sh, uint32_t* total) {
  constexpr int W = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_scan_incl(v);
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const uint32_t s = sh[i];
    pre += (i < wave) ? s : 0u;
    tot += s;
  }
  *total = tot;
  return pre + x - v;
}

struct SelectShared {
  uint32_t hist[2][kBins];   // one per pass, alternating
  uint32_t sh[kBig / 64];
  uint32_t sel_lo[2], sel_krem[2];
};

// The krem-th largest key (1-based) among those in [lo, hi] that visit()
// yields (visit(f) calls f(key) for every key).  Returns the key; *krem_out
// = its rank among the keys equal to it, i.e. how many of them are kept.
// Radix over the shrinking key range, at most 2048 bins per pass.  Passes
// alternate between two histograms and two result slots, so a pass needs
// three work-group barriers: after the histogram (the next pass's histogram
// is cleared before it), inside the scan, and after the selected bin is
// written.  A histogram or slot is written again only two passes later,
// after its last reader has passed those barriers.
template <typename Visit>
__device__ uint32_t select_kth(Visit visit, uint32_t lo, uint32_t hi, uint32_t krem,
                               SelectShared& S, uint32_t* krem_out) {
  const int tid = threadIdx.x;
  if (lo < hi) {
    for (int b = tid; b < kBins; b += kBig) S.hist[0][b] = 0u;
    __syncthreads();
  }
  int cur = 0;
  while (lo < hi) {
    const uint32_t span = hi - lo;
    const int bits = 32 - __clz(span);
    const int shift = bits > 11 ? bits - 11 : 0;
    const int nbins = static_cast<int>(span >> shift) + 1;
    uint32_t* hist = S.hist[cur];
    visit([&](uint32_t u) {
      if (u >= lo && u <= hi) atomicAdd(&hist[(u - lo) >> shift], 1u);
    });
    for (int b = tid; b < kBins; b += kBig) S.hist[cur ^ 1][b] = 0u;
    __syncthreads();
    // thread t owns bins top-2t and top-2t-1 (descending); its exclusive
    // prefix counts the keys in all higher bins
    const int b1 = nbins - 1 - 2 * tid;
    const int b0 = b1 - 1;
    const uint32_t h1 = b1 >= 0 ? hist[b1] : 0u;
    const uint32_t h0 = b0 >= 0 ? hist[b0] : 0u;
    uint32_t tot;
    const uint32_t above = block_scan_open<kBig>(h1 + h0, S.sh, &tot);
    if (b1 >= 0 && above < krem && above + h1 >= krem) {
      S.sel_lo[cur] = lo + (static_cast<uint32_t>(b1) << shift);
      S.sel_krem[cur] = krem - above;
    } else if (b0 >= 0 && above + h1 < krem && above + h1 + h0 >= krem) {
      S.sel_lo[cur] = lo + (static_cast<uint32_t>(b0) << shift);
      S.sel_krem[cur] = krem - above - h1;
    }
    __syncthreads();
    const uint32_t nlo = S.sel_lo[cur];
    const uint64_t top = static_cast<uint64_t>(nlo) + ((1ull << shift) - 1ull);
    hi = top < hi ? static_cast<uint32_t>(top) : hi;
    lo = nlo;
    krem = S.sel_krem[cur];
    cur ^= 1;
  }
  *krem_out = krem;
  return lo;
}

struct Ctx {    // one (row, sequence)
  const float* x;
  int n, nc, keep, w;
  uint32_t* chunks;   // this sequence's first chunk record
  uint32_t* list;     // this sequence's first chunk slot: kTopkChunk (key, position) pairs per chunk
  int32_t* out;       // this (row, sequence)'s output
  int nchunks;
};

__device__ __forceinline__ Ctx ctx_of(const TopkLaunch& a, int sq, int r) {
  const int s = (a.nsets > 1 && r >= a.set[1].row0) ? 1 : 0;
  const TopkSet& st = a.set[s];
  const int lr = r - st.row0;
  Ctx c;
  c.n = a.len[sq];
  c.nc = c.n - a.w;
  c.keep = st.keep[sq];
  c.w = a.w;
  c.x = st.keys + static_cast<size_t>(lr) * a.T + a.off[sq];
  const size_t ch = static_cast<size_t>(r) * a.chunks_total + a.chunk0[sq];
  c.chunks = a.chunk + ch * kTopkChunkWords;
  c.list = a.list + ch * kTopkChunk * 2;
  c.out = st.idx + static_cast<size_t>(lr) * st.L + st.out[sq];
  c.nchunks = a.chunk0[sq + 1] - a.chunk0[sq];
  return c;
}

__device__ __forceinline__ int mode_of(const Ctx& c) {
  return c.keep == 0 ? kModeNone : (c.keep >= c.nc ? kModeAll : kModeSelect);
}

// ---- 1: bracket and collect ------------------------------------------------------
struct BracketShared {
  uint32_t hist[kBins];
  uint32_t sh[kSmall / 64];
  uint32_t mn[kSmall / 64], mx[kSmall / 64];
  uint32_t lo, hi;
};

// The bracket of one row from a sample of kSample keys: kSample/4 evenly
// spaced points, four adjacent keys at each (one cache line serves the four
// loads; every work-group of the row reads the sample, so its cache traffic
// counts).  Every work-group of the row computes the same bracket.  NT
// threads; the shared arrays are hist[kBins], sh and mn, mx [NT/64], and
// lo_s, hi_s.
template <int NT>
__device__ void bracket(const Ctx& c, uint32_t* hist, uint32_t* sh, uint32_t* mnv, uint32_t* mxv, uint32_t& lo_s,
                        uint32_t& hi_s, uint32_t* lo_out, uint32_t* hi_out) {
  constexpr int E = kSample / NT;
  constexpr int W = NT / 64;
  const int tid = threadIdx.x;
  const int stride = c.nc / (kSample / 4);   // >= 16: only rows longer than 16384 candidates are bracketed
  uint32_t u[E];
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int p = (e / 4) * NT + tid;   // sample point
    u[e] = order_key(c.x[static_cast<size_t>(p) * stride + (e % 4)]);
    mn = min(mn, u[e]);
    mx = max(mx, u[e]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = min(mn, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mn), o)));
    mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), o)));
  }
  if ((tid & 63) == 0) { mnv[tid >> 6] = mn; mxv[tid >> 6] = mx; }
  for (int b = tid; b < kBins; b += NT) hist[b] = 0u;
  __syncthreads();
  mn = mnv[0]; mx = mxv[0];
#pragma unroll
  for (int i = 1; i < W; ++i) { mn = min(mn, mnv[i]); mx = max(mx, mxv[i]); }
  const uint32_t span = mx - mn;
  const int bits = span ? 32 - __clz(span) : 0;
  const int shift = bits > 11 ? bits - 11 : 0;
  const int nbins = static_cast<int>(span >> shift) + 1;
#pragma unroll
  for (int e = 0; e < E; ++e) atomicAdd(&hist[(u[e] - mn) >> shift], 1u);
  __syncthreads();
  const double r = static_cast<double>(c.keep) * kSample / c.nc;   // expected sample rank
  // adjacent keys are not independent draws: a wider margin than 4 sigma
  const double margin = 5.0 * sqrt(fmax(r * (1.0 - r / kSample), 0.0)) + 8.0;
  const int r_hi = static_cast<int>(floor(r - margin));          // 0-based, descending
  const int r_lo = static_cast<int>(ceil(r + margin));
  // thread t owns bins top-OWN*t .. top-OWN*t-OWN+1 (descending); `before`
  // counts the sample keys in all higher bins
  constexpr int OWN = kBins / NT;
  uint32_t h[OWN], mine = 0;
#pragma unroll
  for (int i = 0; i < OWN; ++i) {
    const int b = nbins - 1 - (OWN * tid + i);
    h[i] = b >= 0 ? hist[b] : 0u;
    mine += h[i];
  }
  uint32_t tot;
  uint32_t before = block_scan<NT>(mine, sh, &tot);
  // bin b covers keys mn + (b << shift) .. mn + ((b + 1) << shift) - 1
#pragma unroll
  for (int i = 0; i < OWN; ++i) {
    const int b = nbins - 1 - (OWN * tid + i);
    if (b >= 0 && h[i] > 0) {
      if (r_hi >= 0 && static_cast<uint32_t>(r_hi) >= before && static_cast<uint32_t>(r_hi) < before + h[i]) {
        const uint64_t t = static_cast<uint64_t>(mn) + ((static_cast<uint64_t>(b) + 1) << shift) - 1;
        hi_s = t > 0xFFFFFFFFull ? 0xFFFFFFFFu : static_cast<uint32_t>(t);
      }
      if (r_lo < kSample && static_cast<uint32_t>(r_lo) >= before && static_cast<uint32_t>(r_lo) < before + h[i])
        lo_s = mn + (static_cast<uint32_t>(b) << shift);
    }
    before += h[i];
  }
  __syncthreads();
  *hi_out = r_hi >= 0 ? hi_s : 0xFFFFFFFFu;
  *lo_out = r_lo < kSample ? lo_s : 0u;
}

__global__ __launch_bounds__(kSmall) void k_topk_collect(TopkLaunch a) {
  __shared__ BracketShared B;
  const int sq = find_segment(a.chunk0, a.count, static_cast<int>(blockIdx.x));
  const int cc = blockIdx.x - a.chunk0[sq];
  const Ctx c = ctx_of(a, sq, blockIdx.y);
  const int tid = threadIdx.x;
  if (mode_of(c) != kModeSelect) return;
  // this chunk's keys first: their loads are in flight during the bracket
  const int j0 = cc * kTopkChunk;
  uint32_t u[kPerThread];
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) u[e] = order_key(c.x[min(j0 + e * kSmall + tid, c.nc - 1)]);
  uint32_t lo = 0u, hi = 0xFFFFFFFFu;
  if (c.nc > kTopkCap) bracket<kSmall>(c, B.hist, B.sh, B.mn, B.mx, B.lo, B.hi, &lo, &hi);
  uint32_t above = 0, inside = 0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const bool ok = j0 + e * kSmall + tid < c.nc;
    above += (ok && u[e] > hi) ? 1u : 0u;
    inside += (ok && u[e] >= lo && u[e] <= hi) ? 1u : 0u;
  }
  // both counts in one scan: each is at most kTopkChunk < 2^16 per chunk
  static_assert(kTopkChunk < (1 << 16), "packed counts");
  uint32_t tot;
  uint32_t pos = block_scan<kSmall>((above << 16) | inside, B.sh, &tot) & 0xFFFFu;
  const uint32_t tot_in = tot & 0xFFFFu, tot_above = tot >> 16;
  uint32_t* slot = c.list + static_cast<size_t>(cc) * kTopkChunk * 2;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int j = j0 + e * kSmall + tid;
    if (j < c.nc && u[e] >= lo && u[e] <= hi) {
      slot[2 * static_cast<size_t>(pos)] = u[e];
      slot[2 * static_cast<size_t>(pos) + 1] = static_cast<uint32_t>(j);
      ++pos;
    }
  }
  if (tid == 0) {
    uint32_t* rec = c.chunks + static_cast<size_t>(cc) * kTopkChunkWords;
    rec[kAboveC] = tot_above;
    rec[kCandC] = tot_in;
    if (cc == 0) {   // the row's bracket, for the finish kernel
      uint32_t* br = a.bracket + (static_cast<size_t>(blockIdx.y) * a.count + sq) * 2;
      br[0] = lo;
      br[1] = hi;
    }
  }
}

// ---- 2: finish --------------------------------------------------------------------
struct FinishShared {
  SelectShared S;
  uint32_t cand[kTopkCap];
  uint32_t gt_c[kTopkMaxChunks], eq_c[kTopkMaxChunks], coff[kTopkMaxChunks + 1];
  uint32_t above;
};

// Rows of up to kOneWave chunks do their per-chunk scans in one wave (DPP
// scans, no work-group barrier inside).
constexpr int kOneWave = 64;

constexpr int kPT = kTopkChunk / kBig;   // keys per thread and chunk in the finish kernel

// Keys of one batch of this work-group's chunks: c0, c0 + splits, ... (up
// to kWriteBatch chunks), four consecutive keys per thread and chunk.
__device__ __forceinline__ void load_batch(const Ctx& c, int c0, int splits,
                                           uint32_t (&u)[kWriteBatch][kPT]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < kWriteBatch; ++q) {
    const int a = (c0 + q * splits) * kTopkChunk + tid * kPT;
#pragma unroll
    for (int e = 0; e < kPT; ++e) u[q][e] = order_key(c.x[min(a + e, c.nc - 1)]);
  }
}

// Kept positions of one batch's chunks, in index order: each chunk is
// compacted with one packed scan of its (above, equal) counts.
__device__ void write_batch(const Ctx& c, int c0, int splits, uint32_t tau, const FinishShared& F,
                            uint32_t* sh, const uint32_t (&u)[kWriteBatch][kPT]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < kWriteBatch; ++q) {
    const int cc = c0 + q * splits;
    if (cc >= c.nchunks) break;   // uniform
    const int a = cc * kTopkChunk + tid * kPT;
    const uint32_t rem = F.eq_c[cc];
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < kPT; ++e) {
      const bool ok = a + e < c.nc;
      gt += (ok && u[q][e] > tau) ? 1u : 0u;
      eq += (ok && u[q][e] == tau) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t pre = block_scan<kBig>((gt << 16) | eq, sh, &tot);   // < 2^16 each per chunk
    const uint32_t gt_pre = pre >> 16, eq_pre = pre & 0xFFFFu;
    uint32_t pos = F.gt_c[cc] + gt_pre + min(eq_pre, rem);
    uint32_t eq_left = rem > eq_pre ? rem - eq_pre : 0u;
    // this thread's kept keys of the chunk go to pos .. pos + mine - 1: one
    // check that they stay inside the budget (always, when the offsets are
    // consistent) keeps every write in the row's output
    const uint32_t mine = gt + min(eq, eq_left);
    if (pos + mine <= static_cast<uint32_t>(c.keep)) {
#pragma unroll
      for (int e = 0; e < kPT; ++e) {
        if (a + e < c.nc) {
          bool k = u[q][e] > tau;
          if (u[q][e] == tau && eq_left > 0) { k = true; --eq_left; }
          if (k) c.out[pos++] = a + e;
        }
      }
    }
  }
}

// Kept positions of this work-group's chunks of a selecting row: chunks
// split, split + splits, ...; the first batch's keys were loaded at the
// start of the kernel (they do not depend on the threshold).
__device__ void write_chunks(const Ctx& c, int split, int splits, uint32_t tau, const FinishShared& F,
                             uint32_t* sh, const uint32_t (&first)[kWriteBatch][kPT]) {
  write_batch(c, split, splits, tau, F, sh, first);
  for (int c0 = split + splits * kWriteBatch; c0 < c.nchunks; c0 += splits * kWriteBatch) {
    uint32_t u[kWriteBatch][kPT];
    load_batch(c, c0, splits, u);
    write_batch(c, c0, splits, tau, F, sh, u);
  }
}

__global__ __launch_bounds__(kBig) void k_topk_finish(TopkLaunch a) {
  __shared__ FinishShared F;
  SelectShared& S = F.S;
  const int sq = blockIdx.x;
  const int r = blockIdx.y;
  const int split = blockIdx.z, splits = gridDim.z;
  const Ctx c = ctx_of(a, sq, r);
  const int tid = threadIdx.x;
  const int mode = mode_of(c);
  if (split == 0)
    for (int t = tid; t < c.w; t += kBig) c.out[c.keep + t] = c.nc + t;
  if (mode == kModeNone) return;
  if (mode == kModeAll) {
    for (int j = split * kBig + tid; j < c.nc; j += splits * kBig) c.out[j] = j;
    return;
  }
  const uint32_t keep = static_cast<uint32_t>(c.keep);
  // This work-group's first batch of chunk keys (for the final write) does
  // not wait for the threshold: its loads go out before the counts'.
  uint32_t first[kWriteBatch][kPT];
  load_batch(c, split, splits, first);
  const int lane = tid & 63, wave = tid >> 6;
  constexpr int NW = kBig / 64;
  const uint32_t* br = a.bracket + (static_cast<size_t>(r) * a.count + sq) * 2;
  const uint32_t lo = br[0], hi = br[1];
  // per-chunk counts -> candidate offsets
  uint32_t above = 0, total = 0;
  if (c.nchunks <= kOneWave) {
    if (wave == 0) {
      const uint32_t* rec = c.chunks + static_cast<size_t>(min(lane, c.nchunks - 1)) * kTopkChunkWords;
      const bool ok = lane < c.nchunks;
      const uint32_t av = ok ? rec[kAboveC] : 0u;
      const uint32_t nv = ok ? rec[kCandC] : 0u;
      const uint32_t a_incl = wave_scan_incl(av);
      const uint32_t n_incl = wave_scan_incl(nv);
      if (ok) { F.coff[lane] = n_incl - nv; F.gt_c[lane] = av; F.eq_c[lane] = 0u; }
      if (lane == 63) { F.coff[c.nchunks] = n_incl; F.above = a_incl; }
    }
    __syncthreads();
    total = F.coff[c.nchunks];
    above = F.above;
  } else {
    for (int base = 0; base < c.nchunks; base += kBig) {
      const int i = base + tid;
      const uint32_t* rec = c.chunks + static_cast<size_t>(i) * kTopkChunkWords;
      const uint32_t av = i < c.nchunks ? rec[kAboveC] : 0u;
      const uint32_t nv = i < c.nchunks ? rec[kCandC] : 0u;
      uint32_t a_tot, n_tot;
      block_scan<kBig>(av, S.sh, &a_tot);
      const uint32_t pre = total + block_scan<kBig>(nv, S.sh, &n_tot);
      if (i < c.nchunks) { F.coff[i] = pre; F.gt_c[i] = av; F.eq_c[i] = 0u; }
      above += a_tot;
      total += n_tot;
    }
    if (tid == 0) F.coff[c.nchunks] = total;
    __syncthreads();
  }
  const bool bracketed = total <= static_cast<uint32_t>(kTopkCap) && above < keep && keep <= above + total;
  uint32_t tau, take_eq;
  if (bracketed) {
    // wave wv gathers the candidates of chunks wv, wv + 16, ... into entries
    // coff[i] .. coff[i+1]-1 of the row (batches of 8 loads per lane)
    constexpr int BL = 8;
    for (int i = wave; i < c.nchunks; i += NW) {
      const uint32_t b0 = F.coff[i], n = F.coff[i + 1] - b0;
      const uint32_t* src = c.list + static_cast<size_t>(i) * kTopkChunk * 2;
      for (uint32_t t0 = 0; t0 < n; t0 += 64 * BL) {
        uint32_t v[BL];
#pragma unroll
        for (int q = 0; q < BL; ++q) {
          const uint32_t t = t0 + 64 * q + lane;
          v[q] = t < n ? src[2 * static_cast<size_t>(t)] : 0u;
        }
#pragma unroll
        for (int q = 0; q < BL; ++q) {
          const uint32_t t = t0 + 64 * q + lane;
          if (t < n) F.cand[b0 + t] = v[q];
        }
      }
    }
    __syncthreads();
    auto vis = [&](auto f) {
      for (uint32_t i = tid; i < total; i += kBig) f(F.cand[i]);
    };
    tau = select_kth(vis, lo, hi, keep - above, S, &take_eq);
    // candidates above / equal to tau, per chunk, by the wave that owns it
    for (int i = wave; i < c.nchunks; i += NW) {
      const uint32_t b0 = F.coff[i], n = F.coff[i + 1] - b0;
      uint32_t ngt = 0, neq = 0;   // wave-uniform counts
      for (uint32_t t0 = 0; t0 < n; t0 += 64) {
        const uint32_t t = t0 + lane;
        const uint32_t u = t < n ? F.cand[b0 + t] : 0u;
        ngt += static_cast<uint32_t>(__popcll(__ballot(t < n && u > tau)));
        neq += static_cast<uint32_t>(__popcll(__ballot(t < n && u == tau)));
      }
      if (lane == 0) { F.gt_c[i] += ngt; F.eq_c[i] = neq; }
    }
  } else {
    // the bracket missed: exact select over the whole row, then recount
    auto vis = [&](auto f) {
      for (int j = tid; j < c.nc; j += kBig) f(order_key(c.x[j]));
    };
    tau = select_kth(vis, 0u, 0xFFFFFFFFu, keep, S, &take_eq);
    for (int i = tid; i < c.nchunks; i += kBig) F.gt_c[i] = 0u;
    __syncthreads();
    for (int j = tid; j < c.nc; j += kBig) {
      const uint32_t u = order_key(c.x[j]);
      if (u > tau) atomicAdd(&F.gt_c[j / kTopkChunk], 1u);
      else if (u == tau) atomicAdd(&F.eq_c[j / kTopkChunk], 1u);
    }
  }
  __syncthreads();
  // chunk offsets in index order (equal keys are kept first-come): chunk i's
  // output offset goes to gt_c[i], the equal keys it may keep to eq_c[i]
  if (c.nchunks <= kOneWave) {
    if (wave == 0) {
      const bool ok = lane < c.nchunks;
      const uint32_t g = ok ? F.gt_c[lane] : 0u;
      const uint32_t q = ok ? F.eq_c[lane] : 0u;
      const uint32_t eq_pre = wave_scan_incl(q) - q;
      const uint32_t rem = take_eq > eq_pre ? take_eq - eq_pre : 0u;
      const uint32_t sel = g + min(q, rem);
      const uint32_t out_pre = wave_scan_incl(sel) - sel;
      if (ok) { F.gt_c[lane] = out_pre; F.eq_c[lane] = min(q, rem); }
    }
  } else {
    uint32_t eq_run = 0, out_run = 0;
    for (int base = 0; base < c.nchunks; base += kBig) {
      const int i = base + tid;
      const uint32_t g = i < c.nchunks ? F.gt_c[i] : 0u;
      const uint32_t q = i < c.nchunks ? F.eq_c[i] : 0u;
      uint32_t eq_tot;
      const uint32_t eq_pre = eq_run + block_scan<kBig>(q, S.sh, &eq_tot);
      const uint32_t rem = take_eq > eq_pre ? take_eq - eq_pre : 0u;
      const uint32_t sel = g + min(q, rem);
      uint32_t sel_tot;
      const uint32_t out_pre = out_run + block_scan<kBig>(sel, S.sh, &sel_tot);
      if (i < c.nchunks) { F.gt_c[i] = out_pre; F.eq_c[i] = min(q, rem); }
      eq_run += eq_tot;
      out_run += sel_tot;
    }
  }
  __syncthreads();
  write_chunks(c, split, splits, tau, F, S.sh, first);
}

// ---- one work-group per (row, sequence) ------------------------------------------
// Rows of up to kRowMaxKeys candidates run the whole selection in one
// launch, one 1024-thread work-group per (row, sequence), with no
// workspace: (1) for rows longer than kRowDirect the same sampled bracket
// as the collect kernel, (2) one pass over the row counts the keys above the
// bracket and appends those inside it to LDS, (3) the exact threshold by
// radix select over them (over the whole row, read again, if the bracket
// missed or the list overflowed), (4) a second pass writes the kept
// positions in index order.  The passes read the row as 16-byte slots of
// four keys, slot i holding keys s0 + 4i .. s0 + 4i + 3 with s0 in [-3, 0]
// chosen so that slots are 16-byte aligned; only whole slots inside the row
// are read that way, and the up to three keys before the first whole slot
// (head) and after the last (tail) are handled by thread 0.
constexpr int kRowThreads = kBig;                      // select_kth and block_scan<kBig> sizes
constexpr int kRowVec = 8;                             // most slots per thread per block (32768 keys)
constexpr int kRowCap = 32768;                         // listed keys held in LDS
constexpr int kRowDirect = 16384;                      // rows up to this long list every key
constexpr int kRowWaves = kRowThreads / 64;

struct RowShared {
  SelectShared S;
  uint32_t cand[kRowCap];
  uint32_t cnt[2][kRowVec * kRowWaves];   // per (slot step, wave) packed counts, double-buffered
  uint32_t tot_g[2], tot_q[2];
  uint32_t mn[kRowWaves], mx[kRowWaves];
  uint32_t n_in, n_above, lo, hi, in_mn, in_mx, head_g, head_q;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct RowGeom {     // the row's slots: whole slots [i0, i1), head keys [0, hs), tail keys [ts, nc)
  const float* xa;   // x + s0, 16-byte aligned
  int s0, i0, i1, hs, ts;   // nc <= kRowMaxKeys
};

__device__ __forceinline__ RowGeom row_geom(const float* x, int nc) {
  RowGeom g;
  const int s0 = -static_cast<int>((reinterpret_cast<uintptr_t>(x) >> 2) & 3u);
  g.s0 = s0;
  g.xa = x + s0;
  g.hs = s0 < 0 ? min(nc, s0 + 4) : 0;
  g.i0 = s0 < 0 ? 1 : 0;
  g.i1 = max(g.i0, (nc - s0) / 4);
  g.ts = max(g.hs, s0 + 4 * g.i1);
  return g;
}

// Keys of this thread's slots of block b (slot i0 + b*VEC*kRowThreads +
// e*kRowThreads + tid, e < VEC); the bit e of the result is set when that
// slot is a whole slot of the row (the others load a clamped slot and are
// ignored).
template <int VEC>
__device__ __forceinline__ uint32_t row_load(const RowGeom& g, int b, uint32_t (&u)[VEC][4]) {
  uint32_t ok = 0;
  f32x4 v[VEC];   // every load issued before any is used
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    const int i = g.i0 + (b * VEC + e) * kRowThreads + static_cast<int>(threadIdx.x);
    ok |= i < g.i1 ? (1u << e) : 0u;
    v[e] = reinterpret_cast<const f32x4*>(g.xa)[min(i, g.i1 - 1)];
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e)
#pragma unroll
    for (int j = 0; j < 4; ++j) u[e][j] = order_key(v[e][j]);
  return ok;
}

// One key of the ordered write (index j): above tau -> slot g + min(q, take);
// equal to tau -> slot g + q while q < take.  Stores stay below keep.
__device__ __forceinline__ void row_emit(int32_t* out, uint32_t u, uint32_t tau, uint32_t take, uint32_t keep,
                                         int j, uint32_t& g, uint32_t& q) {
  const bool gt = u > tau, eq = u == tau;
  const uint32_t at = g + (gt ? min(q, take) : q);
  if ((gt || (eq && q < take)) && at < keep) out[at] = j;
  g += gt ? 1u : 0u;
  q += eq ? 1u : 0u;
}

template <int VEC>
__global__ __launch_bounds__(kRowThreads) void k_topk_row(TopkLaunch a) {
  __shared__ RowShared R;
  const Ctx c = ctx_of(a, blockIdx.x, blockIdx.y);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int mode = mode_of(c);
  for (int t = tid; t < c.w; t += kRowThreads) c.out[c.keep + t] = c.nc + t;
  if (mode == kModeNone) return;
  if (mode == kModeAll) {
    for (int j = tid; j < c.nc; j += kRowThreads) c.out[j] = j;
    return;
  }
  const uint32_t keep = static_cast<uint32_t>(c.keep);
  const RowGeom g = row_geom(c.x, c.nc);
  const int nblocks = (g.i1 - g.i0 + VEC * kRowThreads - 1) / (VEC * kRowThreads);

  // (1) bracket; (2) keys above it counted, keys inside it listed (with
  // their range, which narrows the select's first pass)
  uint32_t lo = 0u, hi = 0xFFFFFFFFu;
  if (c.nc > kRowDirect) bracket<kRowThreads>(c, R.S.hist[0], R.S.sh, R.mn, R.mx, R.lo, R.hi, &lo, &hi);
  if (tid == 0) { R.n_in = 0u; R.n_above = 0u; R.in_mn = 0xFFFFFFFFu; R.in_mx = 0u; }
  __syncthreads();
  uint32_t above = 0, imn = 0xFFFFFFFFu, imx = 0u;
  for (int b = 0; b < nblocks; ++b) {
    uint32_t u[VEC][4];
    const uint32_t ok = row_load<VEC>(g, b, u);
    // bit 4e+j of inb: key j of slot e is listed (a lane bit mask, so the
    // list pass below reads bits rather than keeping 32 compare masks live)
    uint32_t inb = 0;
#pragma unroll
    for (int e = 0; e < VEC; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t v = (ok >> e) & 1u;
        above += v & (u[e][j] > hi ? 1u : 0u);
        const uint32_t in = v & (u[e][j] >= lo ? 1u : 0u) & (u[e][j] <= hi ? 1u : 0u);
        inb |= in << (4 * e + j);
        imn = min(imn, in ? u[e][j] : 0xFFFFFFFFu);
        imx = max(imx, in ? u[e][j] : 0u);
      }
    const uint32_t nin = __builtin_popcount(inb);
    const uint32_t incl = wave_scan_incl(nin);
    uint32_t base = 0;
    if (lane == 63 && incl > 0) base = atomicAdd(&R.n_in, incl);
    uint32_t pos = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(base), 63)) + incl - nin;
#pragma unroll
    for (int e = 0; e < VEC; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t in = (inb >> (4 * e + j)) & 1u;
        if (in && pos < static_cast<uint32_t>(kRowCap)) R.cand[pos] = u[e][j];
        pos += in;
      }
  }
  if (tid == 0) {   // head and tail keys
    for (int jj = 0; jj < g.hs + (c.nc - g.ts); ++jj) {
      const int j = jj < g.hs ? jj : g.ts + (jj - g.hs);
      const uint32_t u = order_key(c.x[j]);
      above += u > hi ? 1u : 0u;
      if (u >= lo && u <= hi) {
        const uint32_t p = atomicAdd(&R.n_in, 1u);
        if (p < static_cast<uint32_t>(kRowCap)) R.cand[p] = u;
        imn = min(imn, u);
        imx = max(imx, u);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    above += static_cast<uint32_t>(__shfl_xor(static_cast<int>(above), o));
    imn = min(imn, static_cast<uint32_t>(__shfl_xor(static_cast<int>(imn), o)));
    imx = max(imx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(imx), o)));
  }
  if (lane == 0) {
    if (above > 0) atomicAdd(&R.n_above, above);
    atomicMin(&R.in_mn, imn);
    atomicMax(&R.in_mx, imx);
  }
  __syncthreads();
  const uint32_t n_in = R.n_in, n_above = R.n_above;

  // (3) the threshold tau and how many keys equal to it are kept
  uint32_t tau, take;
  if (n_in <= static_cast<uint32_t>(kRowCap) && n_above < keep && keep <= n_above + n_in) {
    auto vis = [&](auto f) {
      for (uint32_t i = tid; i < n_in; i += kRowThreads) f(R.cand[i]);
    };
    tau = select_kth(vis, R.in_mn, R.in_mx, keep - n_above, R.S, &take);
  } else {   // the bracket missed or the list overflowed: the whole row, read again
    auto vis = [&](auto f) {
      for (int j = tid; j < c.nc; j += kRowThreads) f(order_key(c.x[j]));
    };
    tau = select_kth(vis, 0u, 0xFFFFFFFFu, keep, R.S, &take);
  }

  // (4) kept positions in index order: head keys (thread 0), then per block
  // the (above, equal) counts of every (slot step, wave) run of 256 keys
  // scanned in index order with carries across blocks, then tail keys
  if (tid == 0) {
    uint32_t gg = 0, qq = 0;
    for (int j = 0; j < g.hs; ++j) row_emit(c.out, order_key(c.x[j]), tau, take, keep, j, gg, qq);
    R.head_g = gg;
    R.head_q = qq;
  }
  __syncthreads();
  uint32_t carry_g = R.head_g, carry_q = R.head_q;
  for (int b = 0; b < nblocks; ++b) {
    uint32_t u[VEC][4];
    const uint32_t ok = row_load<VEC>(g, b, u);
    const int buf = b & 1;
    uint32_t lane_pre[VEC];
    uint32_t gtb = 0, eqb = 0;   // bit 4e+j: key j of slot e is above / equal to tau (whole slots only)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t v = (ok >> e) & 1u;
        gtb |= (v & (u[e][j] > tau ? 1u : 0u)) << (4 * e + j);
        eqb |= (v & (u[e][j] == tau ? 1u : 0u)) << (4 * e + j);
      }
      const uint32_t gt = __builtin_popcount((gtb >> (4 * e)) & 0xFu);
      const uint32_t eq = __builtin_popcount((eqb >> (4 * e)) & 0xFu);
      const uint32_t v = (gt << 16) | eq;   // < 2^16 each within a run
      const uint32_t incl = wave_scan_incl(v);
      lane_pre[e] = incl - v;
      if (lane == 63) R.cnt[buf][e * kRowWaves + wave] = incl;
    }
    __syncthreads();
    if (wave == 0) {   // exclusive prefix over the block's runs, in index order
      const uint32_t v0 = 2 * lane < VEC * kRowWaves ? R.cnt[buf][2 * lane] : 0u;
      const uint32_t v1 = 2 * lane + 1 < VEC * kRowWaves ? R.cnt[buf][2 * lane + 1] : 0u;
      const uint32_t incl = wave_scan_incl(v0 + v1);   // block totals < 2^16 each
      if (2 * lane < VEC * kRowWaves) R.cnt[buf][2 * lane] = incl - v0 - v1;
      if (2 * lane + 1 < VEC * kRowWaves) R.cnt[buf][2 * lane + 1] = incl - v1;
      if (lane == 63) { R.tot_g[buf] = incl >> 16; R.tot_q[buf] = incl & 0xFFFFu; }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const uint32_t pre = R.cnt[buf][e * kRowWaves + wave] + lane_pre[e];
      uint32_t gg = carry_g + (pre >> 16), qq = carry_q + (pre & 0xFFFFu);
      const int j0 = g.s0 + 4 * (g.i0 + (b * VEC + e) * kRowThreads + tid);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t gt = (gtb >> (4 * e + j)) & 1u, eq = (eqb >> (4 * e + j)) & 1u;
        const uint32_t at = gg + (gt ? min(qq, take) : qq);
        if ((gt | (eq & (qq < take ? 1u : 0u))) && at < keep) c.out[at] = j0 + j;
        gg += gt;
        qq += eq;
      }
    }
    carry_g += R.tot_g[buf];
    carry_q += R.tot_q[buf];
  }
  if (tid == 0)
    for (int j = g.ts; j < c.nc; ++j) row_emit(c.out, order_key(c.x[j]), tau, take, keep, j, carry_g, carry_q);
}

}  // namespace

// Which path a launch takes.  The one-work-group path costs about
// kRowUs + kRowUsPerKey per key of the longest row (one compute unit does a
// row's per-key work, twice); the two-launch path about kPairUs plus
// kPairUsPerSeq per sequence beyond the first (its per-chunk and per-row
// steps multiply with the sequences).  Measured on MI355X with 8 + 1 rows:
// 1K keys 8.8 against 15.3 us, 32K 22.5 against 17.3 us, 64K 35.8 against
// 18.1 us, eight sequences of 4K-32K 23.2 against 38.8 us.
namespace {
constexpr double kRowUs = 5.0, kRowUsPerKey = 0.00053, kPairUs = 15.0, kPairUsPerSeq = 2.5;
bool row_path_faster(int max_nc, int count) {
  if (max_nc > kRowMaxKeys) return false;
  return kRowUs + kRowUsPerKey * max_nc < kPairUs + kPairUsPerSeq * (count - 1);
}
}  // namespace

hipError_t launch_topk(TopkLaunch& a, void* ws, hipStream_t stream) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  char* p = static_cast<char*>(ws);
  a.bracket = reinterpret_cast<uint32_t*>(p);
  p += up(static_cast<size_t>(a.rows_total) * a.count * 2 * 4);
  a.chunk = reinterpret_cast<uint32_t*>(p);
  p += up(static_cast<size_t>(a.rows_total) * a.chunks_total * kTopkChunkWords * 4);
  a.list = reinterpret_cast<uint32_t*>(p);
  int max_nc = 0;
  for (int i = 0; i < a.count; ++i) max_nc = max(max_nc, a.len[i] - a.w);
  if (row_path_faster(max_nc, a.count)) {   // one work-group per (row, sequence), one launch
    // slots per thread per block: enough for the longest row in one block,
    // at most kRowVec (rows longer than that take several blocks)
    const int slots = (max_nc + 3) / 4 + 1;
    const dim3 grid(a.count, a.rows_total);
    if (slots <= kRowThreads) k_topk_row<1><<<grid, kRowThreads, 0, stream>>>(a);
    else if (slots <= 2 * kRowThreads) k_topk_row<2><<<grid, kRowThreads, 0, stream>>>(a);
    else if (slots <= 4 * kRowThreads) k_topk_row<4><<<grid, kRowThreads, 0, stream>>>(a);
    else k_topk_row<kRowVec><<<grid, kRowThreads, 0, stream>>>(a);
    return hipGetLastError();
  }
  k_topk_collect<<<dim3(a.chunks_total, a.rows_total), kSmall, 0, stream>>>(a);
  // as many work-groups per (row, sequence) as fill the GPU once, at most
  // one per chunk of the longest sequence
  int max_chunks = 1;
  for (int i = 0; i < a.count; ++i) max_chunks = max(max_chunks, a.chunk0[i + 1] - a.chunk0[i]);
  int splits = kFinishWGs / (a.rows_total * a.count);
  splits = splits < 1 ? 1 : (splits > max_chunks ? max_chunks : splits);
  k_topk_finish<<<dim3(a.count, a.rows_total, splits), kBig, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace kvsel
