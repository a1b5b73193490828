// Cross-layer accumulation, head sum and per-layer attention statistics.
//
// StructKV summary page, section 2A (global in-degree: attention summed
// from the input layer to the pivot) and section 2B (entropy, sparsity and
// variance monitored per layer); FastKV section 2A (one propagated set per
// sequence, scored by the sum over KV heads).
//
// One streaming pass over score (and c_in): each work-group owns 512 keys
// of one sequence and all KV heads, issues every head's loads at once (heads
// in blocks of 8), writes c_out and tok, and leaves per-head partial sums of
// the three statistics; a second small kernel adds the partials of each
// sequence in a fixed order.  Deterministic: fixed-order reductions, no
// atomics.
#include "kvsel_internal.hpp"

namespace kvsel {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kPer = kStatChunk / kThreads;   // keys per thread
constexpr int kHB = 8;                         // heads per block of loads

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(kThreads) void k_stats_partial(StatsLaunch a, SeqBatch sb) {
  __shared__ float red[kWaves][3 * kHB];
  const int x = blockIdx.x;
  const int sq = find_segment(sb.base, sb.count, x);
  const int chunk = x - sb.base[sq];
  const int n = sb.len[sq];
  const int64_t off = sb.off[sq];
  const int j0 = chunk * kStatChunk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool want_stats = a.stats != nullptr;
  const float inv_mass = static_cast<float>(1.0 / a.mass);
  const float inv_n = 1.0f / n;
  const double dn = static_cast<double>(n);

  int jj[kPer];
  bool ok[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    jj[e] = j0 + e * kThreads + threadIdx.x;
    ok[e] = jj[e] < n;
    jj[e] = ok[e] ? jj[e] : n - 1;     // clamped: loads stay in bounds and unconditional
  }
  float tok[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) tok[e] = 0.f;

  for (int g0 = 0; g0 < a.h_kv; g0 += kHB) {
    float sc[kHB][kPer], ci[kHB][kPer];
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) {
      const int g = min(g0 + hb, a.h_kv - 1);
      const size_t row = static_cast<size_t>(g) * a.T + off;
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        sc[hb][e] = a.score[row + jj[e]];
        ci[hb][e] = a.c_in ? a.c_in[row + jj[e]] : 0.f;
      }
    }
    float part[3 * kHB];
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) {
      const bool head = g0 + hb < a.h_kv;
      const size_t row = static_cast<size_t>(min(g0 + hb, a.h_kv - 1)) * a.T + off;
      float ent = 0.f, var = 0.f, spar = 0.f;
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        if (!(head && ok[e])) continue;
        const float s = sc[hb][e];
        const float v = ci[hb][e] + s;
        if (a.c_out) a.c_out[row + jj[e]] = v;
        tok[e] += v;
        const float p = s * inv_mass;
        ent -= p > 0.f ? p * logf(p) : 0.f;
        const float dp = p - inv_n;
        var += dp * dp;
        // p < 1/n decided exactly: s * n < mass (exact in double for n < 2^29)
        spar += (static_cast<double>(s) * dn < a.mass) ? 1.f : 0.f;
      }
      part[3 * hb] = ent;
      part[3 * hb + 1] = spar;
      part[3 * hb + 2] = var;
    }
    if (want_stats) {
#pragma unroll
      for (int i = 0; i < 3 * kHB; ++i) part[i] = wave_sum(part[i]);
      if (lane == 0) {
#pragma unroll
        for (int i = 0; i < 3 * kHB; ++i) red[wave][i] = part[i];
      }
      __syncthreads();
      const int i = threadIdx.x;
      if (i < 3 * kHB && g0 + i / 3 < a.h_kv) {
        double t = 0.0;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) t += red[wv][i];
        a.part[(static_cast<size_t>(x) * a.h_kv + g0) * 3 + i] = t;
      }
      __syncthreads();
    }
  }
  if (a.tok) {
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      if (ok[e]) a.tok[off + jj[e]] = tok[e];
  }
}

__global__ __launch_bounds__(kThreads) void k_stats_final(StatsLaunch a, SeqBatch sb) {
  __shared__ double red[kWaves][3];
  const int sq = blockIdx.x;
  const int c0 = sb.base[sq], c1 = sb.base[sq + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const double n = sb.len[sq];
  const int per = 3 * a.h_kv;   // values per chunk
  // each thread adds whole chunks (their 3*h_kv values are contiguous; the
  // loads are unrolled so they are all in flight together); value v of a
  // chunk belongs to statistic v % 3
  double acc[3] = {0.0, 0.0, 0.0};
  for (int c = c0 + static_cast<int>(threadIdx.x); c < c1; c += kThreads) {
    const double* p = a.part + static_cast<size_t>(c) * per;
#pragma unroll 8
    for (int v = 0; v < per; v += 3) {
      acc[0] += p[v];
      acc[1] += p[v + 1];
      acc[2] += p[v + 2];
    }
  }
#pragma unroll
  for (int q = 0; q < 3; ++q) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc[q] += __shfl_xor(acc[q], o);
  }
  if (lane == 0) { red[wave][0] = acc[0]; red[wave][1] = acc[1]; red[wave][2] = acc[2]; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double t[3] = {0.0, 0.0, 0.0};
    for (int wv = 0; wv < kWaves; ++wv)
      for (int q = 0; q < 3; ++q) t[q] += red[wv][q];
    float* o = a.stats + static_cast<size_t>(sb.first + sq) * 3;
    o[0] = static_cast<float>(t[0] / a.h_kv);
    o[1] = static_cast<float>(t[1] / (a.h_kv * n));
    o[2] = static_cast<float>(t[2] / (a.h_kv * n));
  }
}

}  // namespace

hipError_t launch_accumulate_stats(const StatsLaunch& a, const SeqBatch& sb, hipStream_t stream) {
  const int units = sb.base[sb.count];
  if (units > 0) k_stats_partial<<<units, kThreads, 0, stream>>>(a, sb);
  if (a.stats) k_stats_final<<<sb.count, kThreads, 0, stream>>>(a, sb);
  return hipGetLastError();
}

}  // namespace kvsel
