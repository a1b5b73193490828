// Internal declarations shared by the libkvsel translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace kvsel {

// Sequences handled by one launch.  Their metadata rides in the kernel
// arguments (no host->device copies); bigger batches are split into
// several launches.
constexpr int kMaxSeq = 64;

// Launch metadata of up to kMaxSeq packed sequences.
struct SeqBatch {
  int32_t count;               // sequences in this launch
  int32_t first;               // batch index of the first one
  int32_t off[kMaxSeq];        // first packed row of each sequence
  int32_t len[kMaxSeq];        // its length
  int32_t base[kMaxSeq + 1];   // prefix of per-sequence work units (launch-local)
};

// Metadata for selection and gather launches.
struct SelBatch {
  int32_t count;
  int32_t off[kMaxSeq];        // first packed input row
  int32_t len[kMaxSeq];        // sequence length n
  int32_t keep[kMaxSeq];       // kept candidates min(k, n - w)
  int32_t out[kMaxSeq + 1];    // first output position (global), out[count] = end
  int32_t chunk0[kMaxSeq + 1]; // selection: prefix of 4096-key chunks (launch-local)
};

// Largest s in [0, count) with base[s] <= x (base ascending).
template <typename Arr>
__device__ __forceinline__ int find_segment(const Arr& base, int count, long long x) {
  int lo = 0, hi = count - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (base[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---- window score ---------------------------------------------------------
constexpr int kScoreRowsPerGroup = 128;   // softmax rows handled per kernel pass
constexpr int kScoreChunkMin = 512;       // keys per work-group: a multiple of 4 key streams x 32 keys
// Pass B keeps a work-group's column sums in LDS beside the four 32 KB rings
// and the exchange buffer: 128 + 1 + 30 KB of the CU's 160 KB.
constexpr int kScoreChunkMax = 7680;

// The head sum, running accumulation and per-sequence statistics of
// kvsel_accumulate_stats, done in pass B's epilogue (kvsel_window_score_stats).
struct ScoreStats {
  const float* c_in;      // [h_kv, T] or null
  float* c_out;           // [h_kv, T] or null (may alias c_in)
  float* tok;             // [T] or null
  float* stats;           // [B, 3] or null
  double* part;           // [units, h_kv, 3] per-unit sums of the three statistics
  uint32_t* ctr;          // [units] heads done per unit, then [kMaxSeq] units x heads done per sequence
  double mass;            // w * group
};

struct WindowScoreLaunch {
  const void* q;          // bf16 [B, w, h_q, d]
  const void* k;          // bf16 [T, h_kv, d]
  int32_t h_q, h_kv, d, w;
  int32_t chunk;          // keys per work-group
  int64_t T;
  float scale;
  float* score;           // [h_kv, T]
  float* lse;             // [B, h_q, w] or null
  const float* lse_in;    // [B, h_q, w] given normalisers (pass B only), or null
  void* part;             // partial (max, sum) per chunk and row
  void* entpart;          // row entropy: per-unit (m, l, tt, -) float4 [units, h_kv, w*G], or null
  float* row_ent;         // [B, h_q, w] row entropies (with entpart)
  float* mean_ent;        // [B] their mean per sequence, or null
  uint32_t* ent_ctr;      // [kMaxSeq] work-groups done per sequence (row entropy)
  double* ent_head;       // [kMaxSeq, h_kv] per-head sums of the row entropies
  const ScoreStats* st;   // head sum and statistics in pass B's epilogue, or null
};
hipError_t launch_window_score(const WindowScoreLaunch& a, const SeqBatch& sb, int row0,
                               int rows, hipStream_t stream);
// After every row group of sb's sequences: the row entropies from entpart.
hipError_t launch_row_entropy(const WindowScoreLaunch& a, const SeqBatch& sb, hipStream_t stream);

// ---- accumulate / stats ---------------------------------------------------
constexpr int kStatChunk = 512;           // keys per work-group

struct StatsLaunch {
  const float* score;
  const float* c_in;
  float* c_out;
  float* tok;
  float* stats;
  double* part;           // [units, h_kv, 3]
  int32_t h_kv;
  int64_t T;
  double mass;            // w * group
};
hipError_t launch_accumulate_stats(const StatsLaunch& a, const SeqBatch& sb, hipStream_t stream);

// ---- top-k ----------------------------------------------------------------
constexpr int kTopkChunk = 4096;       // keys per work item of the per-chunk steps
constexpr int kTopkCap = 16384;        // candidates the exact select holds in LDS per (row, sequence)
constexpr int kTopkMaxChunks = 2048;   // chunks per sequence (n <= 8M + w)

struct TopkSet {                       // one budget's rows
  const float* keys;                   // [rows, T]
  int32_t* idx;                        // [rows, L]
  int64_t L;
  int32_t rows;
  int32_t row0;                        // its first row in the launch's row numbering
  int32_t keep[kMaxSeq];               // kept candidates min(k, n - w)
  int32_t out[kMaxSeq + 1];            // first output position (global)
};

struct TopkLaunch {                    // up to two budgets over the same sequences
  int32_t count;
  int32_t off[kMaxSeq];
  int32_t len[kMaxSeq];
  int32_t chunk0[kMaxSeq + 1];         // prefix of 4096-key chunks (launch-local)
  int32_t w;
  int32_t nsets, rows_total, chunks_total;
  int64_t T;
  TopkSet set[2];
  uint32_t* bracket;                   // workspace: [rows_total][count][2]
  uint32_t* chunk;                     // workspace: [rows_total][chunks_total][2]
  uint32_t* list;                      // workspace: [rows_total][chunks_total][kTopkChunk][2]
};
constexpr int kTopkChunkWords = 2;     // per (row, chunk) record: keys above the bracket, candidates
// Workspace of one top-k launch: per (row, sequence) the bracket, per
// (row, chunk) the record, per (row, chunk) a list of up to kTopkChunk
// (key, position) candidates; each part 256-byte aligned.
inline size_t topk_workspace_bytes(int rows_total, int count, int chunks_total) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const size_t br = static_cast<size_t>(rows_total) * count * 2 * 4;
  const size_t ch = static_cast<size_t>(rows_total) * chunks_total * kTopkChunkWords * 4;
  const size_t li = static_cast<size_t>(rows_total) * chunks_total * kTopkChunk * 8;
  return up(br) + up(ch) + up(li);
}
hipError_t launch_topk(TopkLaunch& a, void* ws, hipStream_t stream);

// ---- gather ---------------------------------------------------------------
constexpr int kGatherMaxJobs = 4;
constexpr int kGatherMaxTileRows = 256;   // output rows a gather work-group resolves at once

struct GatherJob {
  const void* src;             // [T, heads, cpr * 16 bytes]
  void* dst;                   // [L, heads, cpr * 16 bytes]
  const int32_t* idx;          // [heads or 1, L]
  int64_t L;
  int64_t rows_out;            // output rows of this launch's sequences (x heads)
  int32_t heads, cpr, per_head;
  int32_t cpr_shift;           // log2(cpr) when cpr is a power of two, else -1
  int32_t rows_per_tile;       // output rows per work-group step
  int32_t block0;              // first work-group of this job
  int32_t out[kMaxSeq + 1];    // first output position (global) per sequence
  // paged destination (when the launch is paged): dst is [num_blocks,
  // block_size, heads, cpr * 16 bytes]; selected row s of launch sequence i
  // goes to block block_table[i * max_blocks + s / block_size]
  const int32_t* block_table;
  int32_t block_size, max_blocks, num_blocks;
};

struct GatherLaunch {
  int32_t count;
  int32_t off[kMaxSeq];
  int32_t len[kMaxSeq];
  int32_t njobs;
  int32_t paged;               // every job writes through a block table
  GatherJob job[kGatherMaxJobs];
};
hipError_t launch_gather(GatherLaunch& a, hipStream_t stream);

// ---- fixed scratch of the no-allocation entry point ------------------------
constexpr size_t kNoAllocScratchBytes = size_t{4} << 20;
// Device address of this device's copy of the scratch array (looked up once
// per device, with that device current, then cached).
hipError_t noalloc_scratch(void** out);

// ---- streaming-read probe (measurement aid) ------------------------------
hipError_t launch_probe_read(const void* src, int64_t rows, int heads, int row_bytes, int64_t stride,
                             int wgs, uint32_t* out, hipStream_t stream);

}  // namespace kvsel
