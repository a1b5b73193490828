// C ABI of libkvsel: host-side validation, workspace sizing, launch planning.
// Nothing here allocates device memory, copies host->device, or synchronises.
#include <cmath>
#include <cstdint>
#include <vector>

#include "../../include/kvsel.h"
#include "kvsel_internal.hpp"

#define KVSEL_API extern "C" __attribute__((visibility("default")))

namespace {

using kvsel::kMaxSeq;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validated view of a packed batch.
struct Batch {
  int B = 0;
  int64_t T = 0;
  std::vector<int32_t> off, len;
};

// cu_seqlens: cu[0] == 0, non-decreasing, total within int32.
bool read_batch(const kvsel_varlen* v, Batch* out) {
  if (v == nullptr || v->batch < 1 || v->cu_seqlens == nullptr) return false;
  const int32_t* cu = v->cu_seqlens;
  if (cu[0] != 0) return false;
  out->B = v->batch;
  out->off.resize(v->batch);
  out->len.resize(v->batch);
  for (int b = 0; b < v->batch; ++b) {
    if (cu[b + 1] < cu[b]) return false;
    out->off[b] = cu[b];
    out->len[b] = cu[b + 1] - cu[b];
  }
  out->T = cu[v->batch];
  return true;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t round_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Groups of at most kMaxSeq sequences with `units(b)` work units each.
template <typename F>
std::vector<kvsel::SeqBatch> plan_groups(const Batch& bt, F units) {
  std::vector<kvsel::SeqBatch> groups;
  for (int b0 = 0; b0 < bt.B; b0 += kMaxSeq) {
    kvsel::SeqBatch sb{};
    sb.count = std::min(kMaxSeq, bt.B - b0);
    sb.first = b0;
    sb.base[0] = 0;
    for (int i = 0; i < sb.count; ++i) {
      sb.off[i] = bt.off[b0 + i];
      sb.len[i] = bt.len[b0 + i];
      sb.base[i + 1] = sb.base[i] + static_cast<int32_t>(units(b0 + i));
    }
    groups.push_back(sb);
  }
  return groups;
}

int keep_of(int n, int w, int k) { return std::min(std::max(k, 0), n - w); }

// Selection layout: per-sequence output lengths min(n, k + w) and offsets,
// and the selection kernels' chunk prefixes.
bool selection_groups(const Batch& bt, const int32_t* k_host, int w,
                      std::vector<kvsel::SelBatch>* groups, int64_t* L) {
  int64_t pos = 0;
  for (int b0 = 0; b0 < bt.B; b0 += kMaxSeq) {
    kvsel::SelBatch sb{};
    sb.count = std::min(kMaxSeq, bt.B - b0);
    int64_t chunks = 0;
    for (int i = 0; i < sb.count; ++i) {
      const int b = b0 + i;
      if (k_host[b] < 0) return false;
      const int nc = bt.len[b] - w;
      sb.off[i] = bt.off[b];
      sb.len[i] = bt.len[b];
      sb.keep[i] = keep_of(bt.len[b], w, k_host[b]);
      sb.out[i] = static_cast<int32_t>(pos);
      sb.chunk0[i] = static_cast<int32_t>(chunks);
      pos += sb.keep[i] + w;
      chunks += std::max<int64_t>(1, ceil_div(nc, kvsel::kTopkChunk));
      if (pos > INT32_MAX || chunks > INT32_MAX) return false;
    }
    sb.out[sb.count] = static_cast<int32_t>(pos);
    sb.chunk0[sb.count] = static_cast<int32_t>(chunks);
    groups->push_back(sb);
  }
  *L = pos;
  return true;
}

bool selection_fits(const Batch& bt, int w) {
  for (int b = 0; b < bt.B; ++b)
    if (ceil_div(bt.len[b] - w, kvsel::kTopkChunk) > kvsel::kTopkMaxChunks) return false;
  return true;
}

size_t topk_ws(const std::vector<kvsel::SelBatch>& groups, int rows_total) {
  size_t need = 0;
  for (const auto& g : groups)
    need = std::max(need, kvsel::topk_workspace_bytes(rows_total, g.count, g.chunk0[g.count]));
  return need;
}

// One budget's rows of a top-k launch (the selection layout of group g).
void topk_set(const kvsel::SelBatch& g, const float* keys, int rows, int row0, int32_t* idx, int64_t L,
              kvsel::TopkSet* s) {
  s->keys = keys;
  s->idx = idx;
  s->L = L;
  s->rows = rows;
  s->row0 = row0;
  for (int i = 0; i < g.count; ++i) s->keep[i] = g.keep[i];
  for (int i = 0; i <= g.count; ++i) s->out[i] = g.out[i];
}

bool window_fits(const Batch& bt, int w) {
  if (w < 1) return false;
  for (int b = 0; b < bt.B; ++b)
    if (bt.len[b] < w) return false;
  return true;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// ---- window score planning -------------------------------------------------

struct ScorePlan {
  std::vector<kvsel::SeqBatch> groups;
  int chunk = kvsel::kScoreChunkMin;
  size_t part_bytes = 0;
};

// Keys per work-group.  One work-group fits per CU, so a pass of W
// work-groups runs in ceil(W / 256) rounds on MI355X's 256 CUs, and each
// round costs a fixed start and tail (the Q loads, the normaliser merge, the
// ring's first tiles: about 10 us measured per pass) plus the streaming of
// the longest chunk of the round (about 11 ns per key at the rate one
// work-group per CU reaches).  The chunk, a multiple of 128 keys (four key
// streams of whole tiles) in [kScoreChunkMin, kScoreChunkMax], is the one
// with the least estimated time; ties go to the smaller chunk.  At 128K keys
// and 8 KV heads that is 4096 keys: one round of 256 work-groups.
int score_chunk(const Batch& bt, int h_kv) {
  constexpr double kRoundStartUs = 10.0, kUsPerKey = 0.011;
  int longest = 0;
  for (int b = 0; b < bt.B; ++b) longest = std::max(longest, bt.len[b]);
  int best = kvsel::kScoreChunkMin;
  double best_t = 0.0;
  for (int chunk = kvsel::kScoreChunkMin; chunk <= kvsel::kScoreChunkMax; chunk += 128) {
    int64_t units = 0;
    for (int b = 0; b < bt.B; ++b) units += ceil_div(bt.len[b], chunk);
    const int64_t rounds = ceil_div(units * h_kv, 256);
    const double t = static_cast<double>(rounds) * (kRoundStartUs + kUsPerKey * std::min(chunk, longest));
    if (chunk == kvsel::kScoreChunkMin || t < best_t) {
      best = chunk;
      best_t = t;
    }
  }
  return best;
}

ScorePlan plan_score(const Batch& bt, int h_kv) {
  ScorePlan p;
  p.chunk = score_chunk(bt, h_kv);
  p.groups = plan_groups(bt, [&](int b) { return ceil_div(bt.len[b], p.chunk); });
  size_t max_units = 0;
  for (const auto& g : p.groups) max_units = std::max<size_t>(max_units, g.base[g.count]);
  p.part_bytes = round_up(max_units * h_kv * kvsel::kScoreRowsPerGroup * 2 * sizeof(float));
  return p;
}

bool score_args_ok(const Batch& bt, int h_q, int h_kv, int w) {
  if (h_q < 1 || h_kv < 1 || h_q % h_kv != 0) return false;
  if (!window_fits(bt, w)) return false;
  const int64_t rows = static_cast<int64_t>(w) * (h_q / h_kv);
  return rows <= (1 << 20);
}

// Bytes of the row-entropy partials: one float4 per work unit, KV head and
// window row (units of the largest launch group); then per launch group a
// counter per sequence and a double per (sequence, KV head).
size_t entropy_rows_bytes(const ScorePlan& p, int h_q, int h_kv, int w) {
  size_t max_units = 0;
  for (const auto& g : p.groups) max_units = std::max<size_t>(max_units, g.base[g.count]);
  return round_up(max_units * h_kv * static_cast<size_t>(w) * (h_q / h_kv) * 4 * sizeof(float));
}
size_t entropy_part_bytes(const ScorePlan& p, int h_q, int h_kv, int w) {
  return entropy_rows_bytes(p, h_q, h_kv, w) + round_up(kMaxSeq * sizeof(uint32_t)) +
         round_up(static_cast<size_t>(kMaxSeq) * h_kv * sizeof(double));
}

// Shared by the two-pass score calls: validation, then per launch group
// every row group, and the row entropies when asked.
// Argument checks shared by the two-pass score calls (host only).
int score_validate(const kvsel_varlen* v, Batch* bt, const void* q_win, const void* k, int32_t h_q,
                   int32_t h_kv, int32_t d, int32_t w, float scale, const float* score, const float* lse,
                   const float* row_ent, const float* mean_ent, bool want_ent) {
  if (!read_batch(v, bt) || !score_args_ok(*bt, h_q, h_kv, w)) return KVSEL_EINVAL;
  if (!(std::isfinite(scale) && scale > 0.f)) return KVSEL_EINVAL;
  if (q_win == nullptr || k == nullptr || score == nullptr) return KVSEL_EINVAL;
  if (want_ent && row_ent == nullptr) return KVSEL_EINVAL;
  for (const void* p : {static_cast<const void*>(q_win), k, static_cast<const void*>(score)})
    if (!aligned16(p)) return KVSEL_EINVAL;
  for (const void* p : {static_cast<const void*>(lse), static_cast<const void*>(row_ent),
                        static_cast<const void*>(mean_ent)})
    if (p && !aligned16(p)) return KVSEL_EINVAL;
  if (d != 64 && d != 128) return KVSEL_EUNSUPPORTED;
  return KVSEL_OK;
}

// The outputs of kvsel_accumulate_stats, when the score call also does its work.
struct StatsOut {
  const float* c_in;
  float* c_out;
  float* tok;
  float* stats;
};

// Bytes of the statistics epilogue's workspace: per unit and KV head the
// three statistics' sums (double), then the per-unit and per-sequence counts
// (units of the largest launch group).
size_t score_stats_units(const ScorePlan& p) {
  size_t max_units = 0;
  for (const auto& g : p.groups) max_units = std::max<size_t>(max_units, g.base[g.count]);
  return max_units;
}
size_t score_stats_bytes(const ScorePlan& p, int h_kv) {
  const size_t units = score_stats_units(p);
  return round_up(units * h_kv * 3 * sizeof(double)) + round_up((units + kMaxSeq) * sizeof(uint32_t));
}

int window_score_impl(const kvsel_varlen* v, const void* q_win, const void* k, int32_t h_q,
                      int32_t h_kv, int32_t d, int32_t w, float scale, float* score, float* lse,
                      float* row_ent, float* mean_ent, bool want_ent, void* ws, size_t ws_bytes,
                      void* stream, const StatsOut* so = nullptr) {
  Batch bt;
  const int st = score_validate(v, &bt, q_win, k, h_q, h_kv, d, w, scale, score, lse, row_ent, mean_ent,
                                want_ent);
  if (st != KVSEL_OK) return st;
  if (so != nullptr)
    for (const void* q : {static_cast<const void*>(so->c_in), static_cast<const void*>(so->c_out),
                          static_cast<const void*>(so->tok), static_cast<const void*>(so->stats)})
      if (q && !aligned16(q)) return KVSEL_EINVAL;
  const ScorePlan p = plan_score(bt, h_kv);
  const bool with_stats = so != nullptr && (so->c_out || so->tok || so->stats);
  const size_t ent_bytes = want_ent ? entropy_part_bytes(p, h_q, h_kv, w) : 0;
  const size_t st_bytes = with_stats ? score_stats_bytes(p, h_kv) : 0;
  if (ws == nullptr || !aligned16(ws) || ws_bytes < p.part_bytes + ent_bytes + st_bytes) return KVSEL_EWORKSPACE;
  if (bt.T == 0) return KVSEL_OK;

  kvsel::WindowScoreLaunch a{};
  a.q = q_win; a.k = k; a.h_q = h_q; a.h_kv = h_kv; a.d = d; a.w = w; a.T = bt.T;
  a.chunk = p.chunk;
  a.scale = scale; a.score = score; a.lse = lse;
  a.part = ws;
  if (want_ent) {
    char* e = static_cast<char*>(ws) + p.part_bytes;
    a.entpart = e;
    e += entropy_rows_bytes(p, h_q, h_kv, w);
    a.ent_ctr = reinterpret_cast<uint32_t*>(e);
    e += round_up(kMaxSeq * sizeof(uint32_t));
    a.ent_head = reinterpret_cast<double*>(e);
    a.row_ent = row_ent;
    a.mean_ent = mean_ent;
  }
  kvsel::ScoreStats sst{};
  if (with_stats) {
    char* e = static_cast<char*>(ws) + p.part_bytes;
    sst.c_in = so->c_in;
    sst.c_out = so->c_out;
    sst.tok = so->tok;
    sst.stats = so->stats;
    sst.part = reinterpret_cast<double*>(e);
    sst.ctr = reinterpret_cast<uint32_t*>(e + round_up(score_stats_units(p) * h_kv * 3 * sizeof(double)));
    sst.mass = static_cast<double>(w) * (h_q / h_kv);
    a.st = &sst;
  }
  const int R = w * (h_q / h_kv);
  for (const auto& g : p.groups) {
    for (int row0 = 0; row0 < R; row0 += kvsel::kScoreRowsPerGroup) {
      const int rows = std::min(kvsel::kScoreRowsPerGroup, R - row0);
      if (kvsel::launch_window_score(a, g, row0, rows, as_stream(stream)) != hipSuccess)
        return KVSEL_ELAUNCH;
    }
    if (want_ent && kvsel::launch_row_entropy(a, g, as_stream(stream)) != hipSuccess)
      return KVSEL_ELAUNCH;
  }
  return KVSEL_OK;
}

}  // namespace

KVSEL_API const char* kvsel_status_string(int status) {
  switch (status) {
    case KVSEL_OK: return "ok";
    case KVSEL_EINVAL: return "invalid argument";
    case KVSEL_EUNSUPPORTED: return "unsupported configuration";
    case KVSEL_EWORKSPACE: return "workspace missing or too small";
    case KVSEL_ELAUNCH: return "HIP launch failed";
    default: return "unknown status";
  }
}

KVSEL_API int kvsel_abi_version(void) { return KVSEL_ABI_VERSION; }

KVSEL_API int64_t kvsel_selected_length(const kvsel_varlen* v, const int32_t* k_host, int32_t w) {
  Batch bt;
  if (!read_batch(v, &bt) || k_host == nullptr || !window_fits(bt, w)) return -1;
  std::vector<kvsel::SelBatch> groups;
  int64_t L = 0;
  if (!selection_groups(bt, k_host, w, &groups, &L)) return -1;
  return L;
}

KVSEL_API size_t kvsel_window_score_workspace(const kvsel_varlen* v, int32_t h_q, int32_t h_kv,
                                              int32_t d, int32_t w) {
  Batch bt;
  if (!read_batch(v, &bt) || !score_args_ok(bt, h_q, h_kv, w) || (d != 64 && d != 128)) return 0;
  const ScorePlan p = plan_score(bt, h_kv);
  return p.part_bytes;
}

KVSEL_API int kvsel_window_score(const kvsel_varlen* v, const void* q_win, const void* k, int32_t h_q,
                                 int32_t h_kv, int32_t d, int32_t w, float scale, float* score,
                                 float* lse, void* ws, size_t ws_bytes, void* stream) {
  return window_score_impl(v, q_win, k, h_q, h_kv, d, w, scale, score, lse, nullptr, nullptr, false,
                           ws, ws_bytes, stream);
}

KVSEL_API int kvsel_window_score_noalloc(const kvsel_varlen* v, const void* q_win, const void* k,
                                         int32_t h_q, int32_t h_kv, int32_t d, int32_t w, float scale,
                                         float* score, float* lse, void* stream) {
  static_assert(KVSEL_NOALLOC_SCRATCH_BYTES == kvsel::kNoAllocScratchBytes, "header and library agree");
  Batch bt;
  const int st = score_validate(v, &bt, q_win, k, h_q, h_kv, d, w, scale, score, lse, nullptr, nullptr,
                                false);
  if (st != KVSEL_OK) return st;
  // the partials of the largest launch group must fit the fixed scratch;
  // pass A writes every partial pass B reads, so nothing needs clearing
  if (plan_score(bt, h_kv).part_bytes > kvsel::kNoAllocScratchBytes) return KVSEL_EWORKSPACE;
  if (bt.T == 0) return KVSEL_OK;
  void* ws = nullptr;
  if (kvsel::noalloc_scratch(&ws) != hipSuccess || ws == nullptr) return KVSEL_ELAUNCH;
  return window_score_impl(v, q_win, k, h_q, h_kv, d, w, scale, score, lse, nullptr, nullptr, false, ws,
                           kvsel::kNoAllocScratchBytes, stream);
}

KVSEL_API size_t kvsel_window_score_stats_workspace(const kvsel_varlen* v, int32_t h_q, int32_t h_kv, int32_t d,
                                                    int32_t w) {
  Batch bt;
  if (!read_batch(v, &bt) || !score_args_ok(bt, h_q, h_kv, w) || (d != 64 && d != 128)) return 0;
  const ScorePlan p = plan_score(bt, h_kv);
  return p.part_bytes + score_stats_bytes(p, h_kv);
}

KVSEL_API int kvsel_window_score_stats(const kvsel_varlen* v, const void* q_win, const void* k, int32_t h_q,
                                       int32_t h_kv, int32_t d, int32_t w, float scale, float* score, float* lse,
                                       const float* c_in, float* c_out, float* tok, float* stats, void* ws,
                                       size_t ws_bytes, void* stream) {
  const StatsOut so{c_in, c_out, tok, stats};
  return window_score_impl(v, q_win, k, h_q, h_kv, d, w, scale, score, lse, nullptr, nullptr, false, ws,
                           ws_bytes, stream, &so);
}

KVSEL_API size_t kvsel_window_score_entropy_workspace(const kvsel_varlen* v, int32_t h_q, int32_t h_kv,
                                                      int32_t d, int32_t w) {
  Batch bt;
  if (!read_batch(v, &bt) || !score_args_ok(bt, h_q, h_kv, w) || (d != 64 && d != 128)) return 0;
  const ScorePlan p = plan_score(bt, h_kv);
  return p.part_bytes + entropy_part_bytes(p, h_q, h_kv, w);
}

KVSEL_API int kvsel_window_score_entropy(const kvsel_varlen* v, const void* q_win, const void* k,
                                         int32_t h_q, int32_t h_kv, int32_t d, int32_t w, float scale,
                                         float* score, float* lse, float* row_ent, float* mean_ent,
                                         void* ws, size_t ws_bytes, void* stream) {
  return window_score_impl(v, q_win, k, h_q, h_kv, d, w, scale, score, lse, row_ent, mean_ent, true,
                           ws, ws_bytes, stream);
}

KVSEL_API int kvsel_window_score_lse(const kvsel_varlen* v, const void* q_win, const void* k, int32_t h_q,
                                     int32_t h_kv, int32_t d, int32_t w, float scale, const float* lse_in,
                                     float* score, void* stream) {
  Batch bt;
  if (!read_batch(v, &bt) || !score_args_ok(bt, h_q, h_kv, w)) return KVSEL_EINVAL;
  if (!(std::isfinite(scale) && scale > 0.f)) return KVSEL_EINVAL;
  if (q_win == nullptr || k == nullptr || score == nullptr || lse_in == nullptr) return KVSEL_EINVAL;
  if (!aligned16(q_win) || !aligned16(k) || !aligned16(score) || !aligned16(lse_in)) return KVSEL_EINVAL;
  if (d != 64 && d != 128) return KVSEL_EUNSUPPORTED;
  if (bt.T == 0) return KVSEL_OK;
  const ScorePlan p = plan_score(bt, h_kv);
  kvsel::WindowScoreLaunch a{};
  a.q = q_win; a.k = k; a.h_q = h_q; a.h_kv = h_kv; a.d = d; a.w = w; a.T = bt.T;
  a.chunk = p.chunk;
  a.scale = scale; a.score = score; a.lse_in = lse_in;
  const int R = w * (h_q / h_kv);
  for (int row0 = 0; row0 < R; row0 += kvsel::kScoreRowsPerGroup) {
    const int rows = std::min(kvsel::kScoreRowsPerGroup, R - row0);
    for (const auto& g : p.groups)
      if (kvsel::launch_window_score(a, g, row0, rows, as_stream(stream)) != hipSuccess)
        return KVSEL_ELAUNCH;
  }
  return KVSEL_OK;
}

KVSEL_API size_t kvsel_accumulate_stats_workspace(const kvsel_varlen* v, int32_t h_kv) {
  Batch bt;
  if (!read_batch(v, &bt) || h_kv < 1) return 0;
  const auto groups = plan_groups(bt, [&](int b) { return ceil_div(bt.len[b], kvsel::kStatChunk); });
  size_t max_units = 0;
  for (const auto& g : groups) max_units = std::max<size_t>(max_units, g.base[g.count]);
  return round_up(max_units * h_kv * 3 * sizeof(double));
}

KVSEL_API int kvsel_accumulate_stats(const kvsel_varlen* v, const float* score, int32_t h_kv,
                                     int32_t w, int32_t group, const float* c_in, float* c_out,
                                     float* tok, float* stats, void* ws, size_t ws_bytes,
                                     void* stream) {
  Batch bt;
  if (!read_batch(v, &bt) || h_kv < 1 || w < 1 || group < 1) return KVSEL_EINVAL;
  if (!window_fits(bt, w)) return KVSEL_EINVAL;   // every sequence holds the window (n >= w >= 1)
  if (score == nullptr || !aligned16(score)) return KVSEL_EINVAL;
  for (const void* p : {static_cast<const void*>(c_in), static_cast<const void*>(c_out),
                        static_cast<const void*>(tok), static_cast<const void*>(stats)})
    if (p && !aligned16(p)) return KVSEL_EINVAL;
  const size_t need = kvsel_accumulate_stats_workspace(v, h_kv);
  if (stats && (ws == nullptr || !aligned16(ws) || ws_bytes < need)) return KVSEL_EWORKSPACE;
  if (c_out == nullptr && tok == nullptr && stats == nullptr) return KVSEL_OK;
  const auto groups = plan_groups(bt, [&](int b) { return ceil_div(bt.len[b], kvsel::kStatChunk); });
  kvsel::StatsLaunch a{};
  a.score = score; a.c_in = c_in; a.c_out = c_out; a.tok = tok; a.stats = stats;
  a.part = static_cast<double*>(ws); a.h_kv = h_kv; a.T = bt.T;
  a.mass = static_cast<double>(w) * group;
  for (const auto& g : groups)
    if (kvsel::launch_accumulate_stats(a, g, as_stream(stream)) != hipSuccess) return KVSEL_ELAUNCH;
  return KVSEL_OK;
}

KVSEL_API size_t kvsel_topk_workspace(const kvsel_varlen* v, int32_t rows, int32_t w) {
  return kvsel_topk2_workspace(v, rows, 0, w);
}

KVSEL_API size_t kvsel_topk2_workspace(const kvsel_varlen* v, int32_t rows_a, int32_t rows_b, int32_t w) {
  Batch bt;
  if (!read_batch(v, &bt) || rows_a < 1 || rows_b < 0 || !window_fits(bt, w)) return 0;
  std::vector<int32_t> zero(bt.B, 0);
  std::vector<kvsel::SelBatch> groups;
  int64_t L = 0;
  if (!selection_groups(bt, zero.data(), w, &groups, &L)) return 0;
  return topk_ws(groups, rows_a + rows_b);
}

KVSEL_API int kvsel_topk(const kvsel_varlen* v, const float* keys, int32_t rows, int32_t w,
                         const int32_t* k_host, int32_t* idx, void* ws, size_t ws_bytes,
                         void* stream) {
  return kvsel_topk2(v, w, keys, rows, k_host, idx, nullptr, 0, nullptr, nullptr, ws, ws_bytes, stream);
}

KVSEL_API int kvsel_topk2(const kvsel_varlen* v, int32_t w, const float* keys_a, int32_t rows_a,
                          const int32_t* k_a, int32_t* idx_a, const float* keys_b, int32_t rows_b,
                          const int32_t* k_b, int32_t* idx_b, void* ws, size_t ws_bytes, void* stream) {
  Batch bt;
  if (!read_batch(v, &bt) || rows_a < 1 || rows_b < 0 || rows_a + rows_b > 65535) return KVSEL_EINVAL;
  if (!window_fits(bt, w) || k_a == nullptr) return KVSEL_EINVAL;
  if (keys_a == nullptr || idx_a == nullptr || !aligned16(keys_a) || !aligned16(idx_a)) return KVSEL_EINVAL;
  if (rows_b > 0 && (k_b == nullptr || keys_b == nullptr || idx_b == nullptr || !aligned16(keys_b) ||
                     !aligned16(idx_b)))
    return KVSEL_EINVAL;
  std::vector<kvsel::SelBatch> ga, gb;
  int64_t La = 0, Lb = 0;
  if (!selection_groups(bt, k_a, w, &ga, &La)) return KVSEL_EINVAL;
  if (rows_b > 0 && !selection_groups(bt, k_b, w, &gb, &Lb)) return KVSEL_EINVAL;
  if (!selection_fits(bt, w)) return KVSEL_EUNSUPPORTED;
  if (ws == nullptr || !aligned16(ws) || ws_bytes < topk_ws(ga, rows_a + rows_b)) return KVSEL_EWORKSPACE;
  for (size_t i = 0; i < ga.size(); ++i) {
    const kvsel::SelBatch& g = ga[i];
    kvsel::TopkLaunch a{};
    a.count = g.count;
    for (int s = 0; s < g.count; ++s) { a.off[s] = g.off[s]; a.len[s] = g.len[s]; }
    for (int s = 0; s <= g.count; ++s) a.chunk0[s] = g.chunk0[s];
    a.w = w;
    a.T = bt.T;
    a.nsets = rows_b > 0 ? 2 : 1;
    a.rows_total = rows_a + rows_b;
    a.chunks_total = g.chunk0[g.count];
    topk_set(g, keys_a, rows_a, 0, idx_a, La, &a.set[0]);
    if (rows_b > 0) topk_set(gb[i], keys_b, rows_b, rows_a, idx_b, Lb, &a.set[1]);
    if (kvsel::launch_topk(a, ws, as_stream(stream)) != hipSuccess) return KVSEL_ELAUNCH;
  }
  return KVSEL_OK;
}

KVSEL_API int kvsel_gather(const kvsel_varlen* v, const void* src, int32_t heads, int32_t row_bytes,
                           const int32_t* idx, int32_t idx_per_head, const int32_t* k_host,
                           int32_t w, void* dst, void* stream) {
  const kvsel_gather_job job{src, dst, idx, k_host, heads, row_bytes, idx_per_head, 0};
  return kvsel_gather_multi(v, w, 1, &job, stream);
}

namespace {

// Shared by the flat and the paged gathers; pages is null for the flat one.
int gather_impl(const kvsel_varlen* v, int32_t w, int32_t n_jobs, const kvsel_gather_job* jobs,
                const kvsel_paged_cache* pages, void* stream) {
  Batch bt;
  if (!read_batch(v, &bt) || jobs == nullptr || n_jobs < 1 || n_jobs > KVSEL_GATHER_MAX_JOBS)
    return KVSEL_EINVAL;
  if (!window_fits(bt, w)) return KVSEL_EINVAL;
  std::vector<std::vector<kvsel::SelBatch>> groups(n_jobs);
  std::vector<int64_t> L(n_jobs);
  for (int j = 0; j < n_jobs; ++j) {
    const kvsel_gather_job& jb = jobs[j];
    if (jb.heads < 1 || jb.k_host == nullptr) return KVSEL_EINVAL;
    if (jb.row_bytes <= 0 || jb.row_bytes % 16 != 0) return KVSEL_EINVAL;
    if (jb.idx_per_head != 0 && jb.idx_per_head != 1) return KVSEL_EINVAL;
    if (jb.src == nullptr || jb.idx == nullptr) return KVSEL_EINVAL;
    if (!aligned16(jb.src) || !aligned16(jb.idx)) return KVSEL_EINVAL;
    if (!selection_groups(bt, jb.k_host, w, &groups[j], &L[j])) return KVSEL_EINVAL;
    if (L[j] * jb.heads > INT32_MAX) return KVSEL_EUNSUPPORTED;
    if (pages == nullptr) {
      if (jb.dst == nullptr || !aligned16(jb.dst)) return KVSEL_EINVAL;
    } else {
      const kvsel_paged_cache& pc = pages[j];
      if (jb.dst != nullptr) return KVSEL_EINVAL;        // the cache is the destination
      if (pc.cache == nullptr || !aligned16(pc.cache)) return KVSEL_EINVAL;
      if (pc.block_table == nullptr || (reinterpret_cast<uintptr_t>(pc.block_table) & 3u) != 0)
        return KVSEL_EINVAL;
      if (pc.block_size < 1 || pc.max_blocks < 1 || pc.num_blocks < 1) return KVSEL_EINVAL;
      for (int b = 0; b < bt.B; ++b) {
        const int64_t Lb = std::min<int64_t>(bt.len[b], static_cast<int64_t>(std::max(jb.k_host[b], 0)) + w);
        if (ceil_div(Lb, pc.block_size) > pc.max_blocks) return KVSEL_EINVAL;
      }
      if (static_cast<int64_t>(pc.num_blocks) * pc.block_size * jb.heads > (int64_t{1} << 40))
        return KVSEL_EUNSUPPORTED;
    }
  }
  for (size_t gi = 0; gi < groups[0].size(); ++gi) {
    kvsel::GatherLaunch a{};
    const kvsel::SelBatch& g0 = groups[0][gi];
    a.count = g0.count;
    for (int s = 0; s < g0.count; ++s) { a.off[s] = g0.off[s]; a.len[s] = g0.len[s]; }
    a.njobs = n_jobs;
    a.paged = pages != nullptr ? 1 : 0;
    for (int j = 0; j < n_jobs; ++j) {
      const kvsel_gather_job& jb = jobs[j];
      const kvsel::SelBatch& g = groups[j][gi];
      kvsel::GatherJob& o = a.job[j];
      o.src = jb.src;
      o.dst = pages != nullptr ? pages[j].cache : jb.dst;
      o.idx = jb.idx;
      o.L = L[j];
      o.heads = jb.heads;
      o.cpr = jb.row_bytes / 16;
      o.cpr_shift = (o.cpr & (o.cpr - 1)) == 0 ? __builtin_ctz(static_cast<unsigned>(o.cpr)) : -1;
      o.per_head = (jb.idx_per_head && jb.heads > 1) ? 1 : 0;
      for (int s = 0; s <= g.count; ++s) o.out[s] = g.out[s];
      o.rows_out = static_cast<int64_t>(g.out[g.count] - g.out[0]) * jb.heads;
      if (pages != nullptr) {
        const kvsel_paged_cache& pc = pages[j];
        // the launch's sequences are gi * kMaxSeq onwards
        o.block_table = pc.block_table + static_cast<int64_t>(gi) * kMaxSeq * pc.max_blocks;
        o.block_size = pc.block_size;
        o.max_blocks = pc.max_blocks;
        o.num_blocks = pc.num_blocks;
      }
    }
    if (kvsel::launch_gather(a, as_stream(stream)) != hipSuccess) return KVSEL_ELAUNCH;
  }
  return KVSEL_OK;
}

}  // namespace

KVSEL_API int kvsel_gather_multi(const kvsel_varlen* v, int32_t w, int32_t n_jobs,
                                 const kvsel_gather_job* jobs, void* stream) {
  return gather_impl(v, w, n_jobs, jobs, nullptr, stream);
}

KVSEL_API int kvsel_gather_paged(const kvsel_varlen* v, int32_t w, int32_t n_jobs,
                                 const kvsel_gather_job* jobs, const kvsel_paged_cache* pages,
                                 void* stream) {
  if (pages == nullptr) return KVSEL_EINVAL;
  return gather_impl(v, w, n_jobs, jobs, pages, stream);
}

KVSEL_API int32_t kvsel_pivot_layer(const float* entropy, int32_t layers, int32_t stride) {
  if (entropy == nullptr || layers < 1 || stride < 1) return -1;
  for (int l = 0; l < layers; ++l)
    if (!std::isfinite(entropy[static_cast<int64_t>(l) * stride])) return -1;
  if (layers == 1) return 0;
  int best = 1;
  double best_drop = static_cast<double>(entropy[0]) - entropy[stride];
  for (int l = 2; l < layers; ++l) {
    const double drop = static_cast<double>(entropy[static_cast<int64_t>(l - 1) * stride]) -
                        entropy[static_cast<int64_t>(l) * stride];
    if (drop > best_drop) { best_drop = drop; best = l; }
  }
  return best;
}

KVSEL_API int32_t kvsel_pivot_layer_sparsity(const float* entropy, const float* sparsity, int32_t layers,
                                             int32_t stride) {
  if (entropy == nullptr || sparsity == nullptr || layers < 1 || stride < 1) return -1;
  auto at = [&](const float* a, int l) { return static_cast<double>(a[static_cast<int64_t>(l) * stride]); };
  for (int l = 0; l < layers; ++l)
    if (!std::isfinite(at(entropy, l)) || !std::isfinite(at(sparsity, l))) return -1;
  int best = -1;
  double best_drop = 0.0;
  for (int l = 1; l < layers; ++l) {
    if (!(at(sparsity, l) > at(sparsity, l - 1))) continue;
    const double drop = at(entropy, l - 1) - at(entropy, l);
    if (best < 0 || drop > best_drop) { best_drop = drop; best = l; }
  }
  return best >= 0 ? best : kvsel_pivot_layer(entropy, layers, stride);
}

KVSEL_API int kvsel_probe_read(const void* src, int64_t rows, int32_t heads, int32_t row_bytes,
                               int64_t stride_bytes, int32_t wgs_per_head, uint32_t* out, void* stream) {
  if (src == nullptr || out == nullptr || !aligned16(src) || !aligned16(out)) return KVSEL_EINVAL;
  if (rows < 1 || heads < 1 || heads > 65535 || wgs_per_head < 1) return KVSEL_EINVAL;
  if (row_bytes < 16 || (row_bytes & (row_bytes - 1)) != 0) return KVSEL_EINVAL;
  if (stride_bytes % 16 != 0 || stride_bytes < static_cast<int64_t>(heads) * row_bytes) return KVSEL_EINVAL;
  if (kvsel::launch_probe_read(src, rows, heads, row_bytes, stride_bytes, wgs_per_head, out,
                               as_stream(stream)) != hipSuccess)
    return KVSEL_ELAUNCH;
  return KVSEL_OK;
}
