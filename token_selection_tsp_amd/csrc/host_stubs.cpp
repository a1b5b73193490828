// Host-only stand-ins for the kernel launches, for the sanitizer build of
// the C ABI (libkvsel_hostcheck.so): the argument validation, workspace
// sizing and launch planning in api.cpp run under AddressSanitizer and
// UndefinedBehaviorSanitizer on the host, with every launch replaced by a
// check of the launch description it would have received.  Nothing here
// is part of the GPU library.
#include <cstdio>
#include <cstdlib>

#include "kvsel_internal.hpp"

namespace kvsel {
namespace {

// A launch description the planner hands over must be consistent: the
// sequences of a launch group, their work-unit prefix and lengths.
void check_batch(const SeqBatch& sb) {
  if (sb.count < 1 || sb.count > kMaxSeq || sb.base[0] != 0) std::abort();
  for (int i = 0; i < sb.count; ++i)
    if (sb.base[i + 1] < sb.base[i] || sb.len[i] < 0 || sb.off[i] < 0) std::abort();
}

alignas(256) unsigned char g_scratch[kNoAllocScratchBytes];

}  // namespace

hipError_t launch_window_score(const WindowScoreLaunch& a, const SeqBatch& sb, int row0, int rows, hipStream_t) {
  check_batch(sb);
  if (rows < 1 || rows > kScoreRowsPerGroup || row0 < 0 || a.chunk < kScoreChunkMin || a.chunk > kScoreChunkMax ||
      a.chunk % 128 != 0 || (a.lse_in == nullptr && a.part == nullptr))
    std::abort();
  for (int i = 0; i < sb.count; ++i)
    if (sb.base[i + 1] - sb.base[i] != (sb.len[i] + a.chunk - 1) / a.chunk) std::abort();
  return hipSuccess;
}

hipError_t launch_row_entropy(const WindowScoreLaunch& a, const SeqBatch& sb, hipStream_t) {
  check_batch(sb);
  if (a.entpart == nullptr || a.row_ent == nullptr || a.ent_ctr == nullptr) std::abort();
  return hipSuccess;
}

hipError_t launch_accumulate_stats(const StatsLaunch& a, const SeqBatch& sb, hipStream_t) {
  check_batch(sb);
  if (a.stats != nullptr && a.part == nullptr) std::abort();
  return hipSuccess;
}

hipError_t launch_topk(TopkLaunch& a, void* ws, hipStream_t) {
  if (a.count < 1 || a.count > kMaxSeq || a.nsets < 1 || a.nsets > 2 || ws == nullptr) std::abort();
  for (int i = 0; i < a.count; ++i)
    if (a.chunk0[i + 1] < a.chunk0[i]) std::abort();
  return hipSuccess;
}

hipError_t launch_gather(GatherLaunch& a, hipStream_t) {
  if (a.count < 1 || a.count > kMaxSeq || a.njobs < 1 || a.njobs > kGatherMaxJobs) std::abort();
  return hipSuccess;
}

hipError_t launch_probe_read(const void* src, int64_t rows, int heads, int row_bytes, int64_t stride, int wgs,
                             uint32_t* out, hipStream_t) {
  if (src == nullptr || out == nullptr || rows < 1 || heads < 1 || wgs < 1 || row_bytes < 16 ||
      stride < static_cast<int64_t>(heads) * row_bytes)
    std::abort();
  return hipSuccess;
}

hipError_t noalloc_scratch(void** out) {
  *out = g_scratch;
  return hipSuccess;
}

}  // namespace kvsel
