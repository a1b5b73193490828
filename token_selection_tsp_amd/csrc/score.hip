// Window score: causal softmax of the last w queries over all keys, summed
// over the window rows and the query heads of each GQA group.
//
// FastKV summary page, section 2A (token importance from the attention of a
// window of recent tokens) and the FastKV abstract (GQA-aware compression).
//
// Design (CDNA4, gfx950):
//  * Per (sequence, KV head) the window gives R = w*G softmax rows that all
//    read the same keys, so S = Q_g K_g^T is a small dense contraction
//    (R x d x N) done on bf16 MFMA (v_mfma_f32_32x32x16_bf16), fp32 accumulate.
//  * Each row's normaliser is final only after its last key, so keys are
//    visited twice: pass A keeps an online (max, sum) per row per chunk of
//    keys; pass B first merges those partials into the log2 normaliser lse2
//    of each row, then recomputes the logits and adds 2^(x - lse2) down each
//    key's column.
//  * A work-group has four "lanes of keys" (pairs); each owns a run of
//    32-key tiles.  Tiles stream from HBM straight into the pair's LDS ring
//    with 16-byte direct-to-LDS loads (global_load_lds_dwordx4), several
//    tiles in flight without costing VGPRs.  Every load instruction covers
//    whole key rows (full cache lines); an XOR swizzle of the 16-byte chunks
//    within a row keeps the per-lane MFMA fragment reads (one ds_read_b128
//    per k-step) free of bank conflicts.
//  * Up to 64 rows, one wave per pair holds all Q fragments.  Above that the
//    pair is two waves (8 waves per work-group, 2 per SIMD), each with 64
//    rows, sharing every tile: accumulators then stay in VGPRs, so the
//    softmax arithmetic reads them directly.  The pairs hold the same rows;
//    the work-group loads them once into LDS and every wave takes its
//    fragments from there.
//  * Pass A uses the key fragments as the MFMA A operand (keys x rows
//    output: a row's statistics stay inside a lane); pass B uses them as the
//    B operand (rows x keys output: a key's column sum stays inside a lane
//    plus one cross-half swap, and the two waves of a pair add their
//    halves through LDS).
//  * The head-dim axis is permuted identically for Q and K: lane half h at
//    step s holds elements [h*d/2 + 8s, +8), so a lane reads a contiguous
//    half row over the steps.
//  * No floating-point atomics: every key column is finished by exactly
//    one lane.
//  * The row-entropy variant keeps one more online term per row in pass A
//    (StructKV summary page, section 2B: the attention entropy the pivot
//    search watches); k_row_entropy merges it over the chunks in order, and
//    the last work-group of a sequence (one integer counter) adds the
//    per-head sums for the sequence's mean.
#include "kvsel_internal.hpp"

#define KVSEL_AS_GLOBAL __attribute__((address_space(1)))
#define KVSEL_AS_LDS __attribute__((address_space(3)))

namespace kvsel {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPairs = 4;                 // key streams per work-group
constexpr int kTile = 32;
constexpr int kRingBytes = 32 * 1024;     // LDS ring per pair, pass B
constexpr int kRingBytesA = 32 * 1024;    // pass A (its row reduction reuses the ring)
constexpr bool kReverseB = true;          // pass B walks its tiles last to first
constexpr float kNegBig = -1.0e30f;       // "no key seen yet" (finite: keeps x - m finite)
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// D: head dim; RS: waves per pair (row split); NBW: 32-row blocks per wave.
template <int D, int RS, int NBW>
struct Cfg {
  static constexpr int kSteps = D / 16;               // 16-byte loads per lane per tile
  static constexpr int kTileBytes = kSteps * 1024;
  static constexpr int kDepth = kRingBytes / kTileBytes;
  static constexpr int kWaves = kPairs * RS;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRows = 32 * NBW * RS;         // rows covered by one work-group
};

// Row of the 32x32 MFMA result held in accumulator v by a lane of half `half`
// (the column is lane % 32).
__device__ __forceinline__ int acc_row(int v, int half) {
  return ((v >> 2) << 3) + (half << 2) + (v & 3);
}

__device__ __forceinline__ bf16x8 load8(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// IEEE-2019 maximum (NaN-propagating): lowers to v_maximum3_f32 with no
// operand canonicalisation, unlike fmaxf.  Logits are finite or -inf.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Wait until at most N vector-memory operations of this wave are pending.
// The direct-to-LDS loads are not tracked by the compiler, so the ring
// waits for them explicitly; vector-memory operations complete in order.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Work-group barrier without the memory fence __syncthreads() implies (a
// fence would also wait for the ring's in-flight loads).  LDS writes that
// must be seen across it are waited for explicitly first.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Key tiles move with direct-to-LDS loads.  Each instruction moves whole
// key rows (512/D keys, 1 KB, every byte of their cache lines), so the
// memory side sees full-line requests.  A row is D/8 chunks of 16 bytes;
// chunk c of tile key kk is stored at position c ^ (kk % (D/8)) of row kk,
// which spreads the later per-lane fragment reads over all LDS banks.
//
// For instruction s, lane l fills position p = l % (D/8) of tile key
// kk = (512/D)*s + l/(D/8), i.e. chunk p ^ (kk % (D/8)).  The chunk index
// repeats with period (D/8)/(512/D) in s, so each lane keeps that many byte
// offsets (relative to the tile's first key and step s's first key); the
// rest of the address is wave-uniform and lives in scalar registers.
template <int D>
struct DmaPlan {
  static constexpr int CPR = D / 8;            // 16-byte chunks per key row
  static constexpr int KPI = 64 / CPR;         // key rows per instruction
  static constexpr int PERIOD = CPR / KPI;     // distinct per-lane offsets
  uint32_t voff[PERIOD];                       // bytes from the step's first key row

  __device__ __forceinline__ void init(int lane, int h_kv) {
    const int p = lane % CPR, q = lane / CPR;
#pragma unroll
    for (int j = 0; j < PERIOD; ++j) {
      const int c = p ^ ((KPI * j + q) % CPR);
      voff[j] = static_cast<uint32_t>((q * h_kv * D + 8 * c) * 2);
    }
  }
};

// Copy keys t0 .. t0+31 of KV head g (rows clamped to n-1 only in a tail
// tile) into an LDS ring slot.
template <int D>
__device__ __forceinline__ void dma_tile(const DmaPlan<D>& plan, const __bf16* k, int64_t off, int n,
                                         int t0, int h_kv, int g, int lane, char* slot) {
  constexpr int CPR = DmaPlan<D>::CPR, KPI = DmaPlan<D>::KPI, PERIOD = DmaPlan<D>::PERIOD;
  if (t0 + kTile <= n) {
    // uniform tile base + per-step uniform stride + per-lane offset
    const char* base = reinterpret_cast<const char*>(k + ((off + t0) * h_kv + g) * D);
    const int64_t step = static_cast<int64_t>(KPI) * h_kv * D * 2;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      __builtin_amdgcn_global_load_lds((KVSEL_AS_GLOBAL void*)(base + s * step + plan.voff[s % PERIOD]),
                                       (KVSEL_AS_LDS void*)(slot + s * 1024), 16, 0, 0);
  } else {
    const int p = lane % CPR;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const int kk = KPI * s + lane / CPR;
      const int c = p ^ (kk % CPR);
      const int64_t row = off + min(t0 + kk, n - 1);
      const __bf16* src = k + (row * h_kv + g) * D + 8 * c;
      __builtin_amdgcn_global_load_lds((KVSEL_AS_GLOBAL void*)src, (KVSEL_AS_LDS void*)(slot + s * 1024),
                                       16, 0, 0);
    }
  }
}

// MFMA fragments of a tile: lane l takes key kl = l%32, head-dim chunk
// c = (l/32)*(D/16) + s at k-step s, stored at position c ^ (kl % (D/8)).
// Since s < D/16 occupies the low bits of c, that position is b ^ s with
// b = ((l/32)*(D/16)) ^ (kl % (D/8)) fixed per lane.
template <int D>
__device__ __forceinline__ void read_tile(bf16x8 (&kf)[D / 16], const char* slot, int lane) {
  constexpr int CPR = D / 8;
  const int kl = lane & 31;
  const char* rowp = slot + kl * (2 * D);
  const int b = ((lane >> 5) * (D / 16)) ^ (kl % CPR);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) kf[s] = *reinterpret_cast<const bf16x8*>(rowp + 16 * (b ^ s));
}

// Ring protocol for one pair.  Iteration t: the issuing wave waits for tile
// t, the pair meets at a barrier (tile t visible to both; both finished
// reading tile t-1), the issuer refills tile t-1's slot with tile t-1+P, and
// both read tile t.  REV walks the pair's tiles last to first (pass B: the
// keys pass A read last are the ones most likely still in the last-level
// cache).  The walk starts at tile `rot` of the pair's range and wraps, with
// rot spread over the pairs of a launch: if every pair starts at its first
// tile, all of a launch's key streams read addresses that agree modulo the
// chunk stride at the same moment, and on MI355X the work-groups of heads 1
// and 5 (byte offsets 256 and 1280 of each 2 KB key row at 8 KV heads) then
// ran 5-6 us longer than the rest of pass A.  Both passes use the same rot,
// so pass B still starts on pass A's last tile.
template <int D, int RS, bool REV, int RB>
struct Ring {
  static constexpr int S = D / 16;
  static constexpr int P = RB / (S * 1024);
  static constexpr int B = S * 1024;
  const __bf16* k;
  int64_t off;
  int n, kbeg, ntiles, h_kv, g, lane;
  bool issuer;
  char* ring;
  DmaPlan<D> plan;
  int rot = 0;   // first tile of the walk, 0 <= rot < ntiles

  __device__ __forceinline__ int key0(int t) const {
    int i = (REV ? ntiles - 1 - t : t) + rot;
    if (i >= ntiles) i -= ntiles;
    return kbeg + i * kTile;
  }
  __device__ __forceinline__ void start() {
    plan.init(lane, h_kv);
    if (issuer)
      for (int p = 0; p < P - 1 && p < ntiles; ++p)
        dma_tile<D>(plan, k, off, n, key0(p), h_kv, g, lane, ring + p * B);
  }
  // Tile t's fragments into kf and its first key into t0; false when this
  // pair has no tile t.  With two waves per pair every wave of the
  // work-group calls this the same number of times (the barrier count must
  // match), also past the end of its own tiles.
  __device__ __forceinline__ bool fetch(int t, bf16x8 (&kf)[S], int* t0) {
    const bool live = t < ntiles;
    if (issuer && live) {
      if (t + P - 2 < ntiles) wait_vmem<(P - 2) * S>(); else wait_vmem<0>();
    }
    if (RS > 1) { wait_lds(); barrier(); }
    if (!live) return false;
    const int refill = t - 1 + P;
    if (issuer && refill < ntiles)
      dma_tile<D>(plan, k, off, n, key0(refill), h_kv, g, lane, ring + (refill % P) * B);
    read_tile<D>(kf, ring + (t % P) * B, lane);
    wait_lds();
    *t0 = key0(t);
    return true;
  }
};

// First tile of a pair's walk: pairs of consecutive work-groups start 5
// tiles apart (mod the pair's tile count), the same in pass A and pass B.
__device__ __forceinline__ int walk_start(int ntiles, int x, int pair) {
  return ntiles > 0 ? ((x * kPairs + pair) * 5) % ntiles : 0;
}

// Q fragments through LDS, for the whole work-group at once: its kRows
// window rows (rows past `rows` are zero) are loaded once, chunk c (16
// bytes) of row r stored at chunk position c ^ (r % (D/8)) of LDS row r, and
// each wave then reads its lanes' fragments (row 32*rb + col, chunks
// half*(D/16) + s; the swizzle spreads every 16-lane read phase over all
// banks).  The key streams of a work-group hold the same rows, so this is
// one load of them per work-group where each stream loading its own copy
// would be four.  `stage` is LDS the ring has not started on (kRows * 2D
// bytes); the closing barrier frees it for the ring.
template <int D, int RS, int NBW>
__device__ __forceinline__ void load_q_lds(bf16x8 (&qf)[NBW][D / 16], const __bf16* q, int seq, int g, int G,
                                           int h_q, int w, int row0, int rows, int rb0, int col, int half,
                                           int tid, char* stage) {
  using C = Cfg<D, RS, NBW>;
  constexpr int CPR = D / 8;
  constexpr int kChunks = C::kRows * CPR;
  constexpr int kPer = (kChunks + C::kThreads - 1) / C::kThreads;
  bf16x8 v[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {   // loads first, all in flight
    const int qc = tid + k * C::kThreads;
    const int r = qc / CPR, cc = qc % CPR;
    const int rr = row0 + min(r, rows - 1);   // clamped: every load stays inside Q
    const int i = rr / G;
    const int hh = rr - i * G;
    v[k] = load8(q + ((static_cast<size_t>(seq) * w + i) * h_q + g * G + hh) * D + 8 * cc);
  }
  const bf16x8 zero = {};
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int qc = tid + k * C::kThreads;
    const int r = qc / CPR, cc = qc % CPR;
    if (qc < kChunks)
      *reinterpret_cast<bf16x8*>(stage + 16 * (r * CPR + (cc ^ (r % CPR)))) = r < rows ? v[k] : zero;
  }
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < NBW; ++rb) {
    const int r = 32 * (rb0 + rb) + col;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const int cc = half * (D / 16) + s;
      qf[rb][s] = *reinterpret_cast<const bf16x8*>(stage + 16 * (r * CPR + (cc ^ (r % CPR))));
    }
  }
  __syncthreads();
}

struct Unit {      // this work-group's (sequence, chunk) and one pair's key range
  int sq, n, kbeg, kend;
  int64_t off;
};

__device__ __forceinline__ Unit unit_of(const SeqBatch& sb, int x, int chunk_keys, int pair) {
  Unit u;
  u.sq = find_segment(sb.base, sb.count, x);
  const int chunk = x - sb.base[u.sq];
  u.n = sb.len[u.sq];
  u.off = sb.off[u.sq];
  const int per_pair = chunk_keys / kPairs;
  u.kbeg = chunk * chunk_keys + pair * per_pair;
  u.kend = min(u.n, u.kbeg + per_pair);
  return u;
}

// Scheduling pattern for a block of NM MFMAs issued with independent vector
// work: one MFMA, then NV vector instructions, repeated (the softmax of a
// 32-row block is ~57 vector instructions, a block's column sums ~40).
constexpr int kValuPerMfma = 7;
constexpr int kValuPerMfmaB = 5;
template <int NM, int NV>
__device__ __forceinline__ void interleave_mfma_valu() {
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
  }
}

// ---- pass A: online (max, sum) of 2^x per row ------------------------------------
// x = scale*log2(e) * <q, k>, the logit in log2 units.  The loop is software
// pipelined: tile t's MFMAs are issued into one accumulator set while the
// softmax arithmetic of tile t-1 runs on the other, so the matrix pipe and
// the vector/transcendental pipes work at the same time.

// Logits of one tile, keys x rows: acc[rb][v] holds key t0 + acc_row(v, half)
// of row rbase + 32*rb + col.
template <int D, int NBW>
__device__ __forceinline__ void a_mfma(f32x16 (&acc)[NBW], const bf16x8 (&kf)[D / 16],
                                       const bf16x8 (&qf)[NBW][D / 16]) {
#pragma unroll
  for (int rb = 0; rb < NBW; ++rb) {
    acc[rb] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) acc[rb] = mfma(kf[s], qf[rb][s], acc[rb]);
  }
}

// Logits of one 32-row block: keys x rows.
template <int D>
__device__ __forceinline__ void a_mfma1(f32x16& acc, const bf16x8 (&kf)[D / 16], const bf16x8 (&qf)[D / 16]) {
  acc = f32x16{};
#pragma unroll
  for (int s = 0; s < D / 16; ++s) acc = mfma(kf[s], qf[s], acc);
}

// Online (max m, sum l) of 2^x over this lane's keys of each row, x the
// logit in log2 units.  With ENT also tt = sum 2^(x-m) * (x-m), rescaled
// with l when m moves: at the end the row's entropy is
// ln2 * (log2 l - tt / l), a sum of two non-negative terms.  Hidden keys
// are -inf as without ENT (so m and l round identically); their x - m is
// clamped to a finite value in the tt term only, so it adds 0 * finite.
template <int NBW, bool MASK, bool ENT>
__device__ __forceinline__ void a_softmax(f32x16 (&acc)[NBW], float (&m)[NBW], float (&l)[NBW],
                                          float (&tt)[NBW], float c, int t0, int n, int w, int rbase,
                                          int G, int col, int half) {
#pragma unroll
  for (int rb = 0; rb < NBW; ++rb) {
    if (MASK) {
      const int vis = n - w + (rbase + 32 * rb + col) / G;   // last key this row sees
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kj = t0 + acc_row(v, half);
        acc[rb][v] = (kj < n && kj <= vis) ? acc[rb][v] : -INFINITY;
      }
    }
    float t[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) t[v] = vmax(acc[rb][v], acc[rb][v + 8]);
#pragma unroll
    for (int v = 0; v < 4; ++v) t[v] = vmax(t[v], t[v + 4]);
    const float tm = vmax(vmax(t[0], t[1]), vmax(t[2], t[3]));
    const float mn = vmax(m[rb], tm * c);
    float s4[4];
    if constexpr (ENT) {
      float t4[4];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float y = fmaf(acc[rb][v], c, -mn);
        const float e = fast_exp2(y);
        const float yt = MASK ? fmaxf(y, kNegBig) : y;   // -inf only for hidden keys
        if (v < 4) { s4[v] = e; t4[v] = e * yt; }
        else { s4[v & 3] += e; t4[v & 3] = fmaf(e, yt, t4[v & 3]); }
      }
      const float dm = m[rb] - mn;
      const float a = fast_exp2(dm);
      tt[rb] = a * fmaf(dm, l[rb], tt[rb]) + ((t4[0] + t4[1]) + (t4[2] + t4[3]));
      l[rb] = fmaf(l[rb], a, (s4[0] + s4[1]) + (s4[2] + s4[3]));
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) s4[v] = fast_exp2(fmaf(acc[rb][v], c, -mn));
#pragma unroll
      for (int v = 4; v < 16; ++v) s4[v & 3] += fast_exp2(fmaf(acc[rb][v], c, -mn));
      l[rb] = fmaf(l[rb], fast_exp2(m[rb] - mn), (s4[0] + s4[1]) + (s4[2] + s4[3]));
    }
    m[rb] = mn;
  }
}

// Merge of two (m, l, tt) states of the same row (tt as in a_softmax); m
// and l round exactly as in the plain merge.
__device__ __forceinline__ void ent_merge(float& m, float& l, float& tt, float mo, float lo, float to) {
  const float mm = fmaxf(m, mo);
  const float a = fast_exp2(m - mm), b = fast_exp2(mo - mm);
  tt = a * fmaf(m - mm, l, tt) + b * fmaf(mo - mm, lo, to);
  l = fmaf(l, a, lo * b);
  m = mm;
}

// With ENT the work-group also leaves each row's (m, l, tt) over its chunk
// in entpart[unit][g][row] (rtot rows per KV head); k_row_entropy merges
// them.
// Pass A over work unit x (a chunk of one sequence's keys) of KV head g, in
// the LDS ring given.
template <int D, int RS, int NBW, bool ENT>
__device__ __forceinline__ void pass_a_unit(
    char (*ring)[kRingBytesA], int tid, int x, int g, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const SeqBatch& sb, int chunk_keys, int h_q, int h_kv, int w, int row0, int rows, float c,
    float2* __restrict__ part, float4* __restrict__ entpart, int rtot, uint32_t* __restrict__ ent_ctr,
    uint32_t* __restrict__ st_ctr) {
  using C = Cfg<D, RS, NBW>;
  constexpr int S = D / 16;
  // after the tile loop the ring is free: the per-pair row statistics go there
  float2 (*red)[C::kRows] = reinterpret_cast<float2 (*)[C::kRows]>(&ring[0][0]);
  float (*redt)[C::kRows] = reinterpret_cast<float (*)[C::kRows]>(&ring[0][0] + sizeof(float2) * kPairs * C::kRows);
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int pair = __builtin_amdgcn_readfirstlane(wave % kPairs);    // wave-uniform
  const int split = __builtin_amdgcn_readfirstlane(wave / kPairs);
  const int half = lane >> 5;
  const int col = lane & 31;
  const Unit u = unit_of(sb, x, chunk_keys, pair);
  const int G = h_q / h_kv;
  const int rb0 = split * NBW;

  if (ENT && x == 0 && g == 0 && tid < kMaxSeq)
    ent_ctr[tid] = 0u;   // k_row_entropy's counters, before it runs
  if (st_ctr != nullptr) {   // pass B's epilogue counters, before it runs
    const int units = sb.base[sb.count];
    if (g == 0 && tid == 0) st_ctr[x] = 0u;
    if (x == 0 && g == 0 && tid < kMaxSeq) st_ctr[units + tid] = 0u;
  }

  bf16x8 qf[NBW][S];
  load_q_lds<D, RS, NBW>(qf, q, sb.first + u.sq, g, G, h_q, w, row0, rows, rb0, col, half, tid, &ring[0][0]);

  float m[NBW], l[NBW], tt[NBW];
#pragma unroll
  for (int rb = 0; rb < NBW; ++rb) { m[rb] = kNegBig; l[rb] = 0.f; tt[rb] = 0.f; }
  const int full_lim = u.n - w + 1;   // keys < full_lim are visible to every window row
  const int rbase = row0 + 32 * rb0;

  Ring<D, RS, false, kRingBytesA> rg{k, u.off, u.n, u.kbeg,
                        u.kend > u.kbeg ? (u.kend - u.kbeg + kTile - 1) / kTile : 0,
                        h_kv, g, lane, split == 0, ring[pair]};
  rg.rot = walk_start(rg.ntiles, x, pair);
  rg.start();
  const int tmax = RS > 1 ? chunk_keys / (kPairs * kTile) : rg.ntiles;   // uniform when RS > 1
  if constexpr (NBW == 2) {
    // Row-block pipeline: the MFMAs of (tile t, block 1) run while block 0
    // of tile t is reduced, and those of (t+1, block 0) while block 1 is.
    float m1[1], l1[1], m2[1], l2[1], t1[1], t2[1];
    m1[0] = m[0]; l1[0] = l[0]; m2[0] = m[1]; l2[0] = l[1]; t1[0] = tt[0]; t2[0] = tt[1];
    auto soft = [&](f32x16 (&acc)[1], float (&mm)[1], float (&ll)[1], float (&tl)[1], int t0, int rb) {
      if (t0 + kTile <= full_lim)
        a_softmax<1, false, ENT>(acc, mm, ll, tl, c, t0, u.n, w, rbase + 32 * rb, G, col, half);
      else
        a_softmax<1, true, ENT>(acc, mm, ll, tl, c, t0, u.n, w, rbase + 32 * rb, G, col, half);
    };
    bf16x8 kf[S];
    f32x16 acc_a[1], acc_b[1];
    // one half-step: the MFMAs of one block into acc_new and the softmax of
    // the other block (acc_old, tile starting at t0s), in one basic block so
    // the scheduler can interleave them (one MFMA, then a share of the
    // vector work, ...): the matrix pipe runs under the vector work of the
    // same wave
    auto both = [&](f32x16& acc_new, const bf16x8 (&qfb)[S], f32x16 (&acc_old)[1], float (&mm)[1],
                    float (&ll)[1], float (&tl)[1], int t0s, int rb) {
      if (t0s + kTile <= full_lim) {
        a_mfma1<D>(acc_new, kf, qfb);
        a_softmax<1, false, ENT>(acc_old, mm, ll, tl, c, t0s, u.n, w, rbase + 32 * rb, G, col, half);
        interleave_mfma_valu<S, kValuPerMfma + (ENT ? 2 : 0)>();
      } else {
        a_mfma1<D>(acc_new, kf, qfb);
        a_softmax<1, true, ENT>(acc_old, mm, ll, tl, c, t0s, u.n, w, rbase + 32 * rb, G, col, half);
        interleave_mfma_valu<S, kValuPerMfma + (ENT ? 2 : 0)>();
      }
    };
    int t0 = 0, t0n = 0;
    bool live = tmax > 0 && rg.fetch(0, kf, &t0);
    if (live) a_mfma1<D>(acc_a[0], kf, qf[0]);
    for (int t = 0; t < tmax; ++t) {
      if (live) both(acc_b[0], qf[1], acc_a, m1, l1, t1, t0, 0);
      bool live_n = false;
      if (t + 1 < tmax) {
        live_n = rg.fetch(t + 1, kf, &t0n);
      } else if (RS > 1) {
        wait_lds();
        barrier();
      }
      if (live_n && live) {
        both(acc_a[0], qf[0], acc_b, m2, l2, t2, t0, 1);
      } else {
        if (live_n) a_mfma1<D>(acc_a[0], kf, qf[0]);
        if (live) soft(acc_b, m2, l2, t2, t0, 1);
      }
      live = live_n;
      t0 = t0n;
    }
    m[0] = m1[0]; l[0] = l1[0]; m[1] = m2[0]; l[1] = l2[0]; tt[0] = t1[0]; tt[1] = t2[0];
  } else {
    // two accumulator sets, addressed statically: the loop is unrolled by two
    f32x16 acc0[NBW], acc1[NBW];
    int t0_prev = 0;
    auto step = [&](int t, f32x16 (&acc_new)[NBW], f32x16 (&acc_old)[NBW]) {
      bf16x8 kf[S];
      int t0 = 0;
      const bool live = t < tmax && rg.fetch(t, kf, &t0);
      if (live) a_mfma<D, NBW>(acc_new, kf, qf);
      if (t >= 1 && t - 1 < rg.ntiles) {
        if (t0_prev + kTile <= full_lim)
          a_softmax<NBW, false, ENT>(acc_old, m, l, tt, c, t0_prev, u.n, w, rbase, G, col, half);
        else
          a_softmax<NBW, true, ENT>(acc_old, m, l, tt, c, t0_prev, u.n, w, rbase, G, col, half);
      }
      t0_prev = t0;
    };
    for (int t = 0; t <= tmax; t += 2) {
      step(t, acc0, acc1);
      if (t + 1 <= tmax) step(t + 1, acc1, acc0);
    }
  }

  // the two lane halves saw different keys of the same row
#pragma unroll
  for (int rb = 0; rb < NBW; ++rb) {
    const float mo = __shfl_xor(m[rb], 32);
    const float lo = __shfl_xor(l[rb], 32);
    if constexpr (ENT) {
      const float to = __shfl_xor(tt[rb], 32);
      ent_merge(m[rb], l[rb], tt[rb], mo, lo, to);
    } else {
      const float mm = fmaxf(m[rb], mo);
      l[rb] = fmaf(l[rb], fast_exp2(m[rb] - mm), lo * fast_exp2(mo - mm));
      m[rb] = mm;
    }
  }
  __syncthreads();   // every wave is done with the ring
  if (half == 0) {
#pragma unroll
    for (int rb = 0; rb < NBW; ++rb) {
      red[pair][32 * (rb0 + rb) + col] = make_float2(m[rb], l[rb]);
      if constexpr (ENT) redt[pair][32 * (rb0 + rb) + col] = tt[rb];
    }
  }
  __syncthreads();
  if constexpr (ENT) {
    // the row's (m, l, tt) over the whole chunk: the four pairs in order
    for (int r = tid; r < C::kRows && r < rows; r += C::kThreads) {
      float mm = red[0][r].x, ll = red[0][r].y, tl = redt[0][r];
#pragma unroll
      for (int p = 1; p < kPairs; ++p) ent_merge(mm, ll, tl, red[p][r].x, red[p][r].y, redt[p][r]);
      entpart[(static_cast<size_t>(x) * h_kv + g) * rtot + row0 + r] = make_float4(mm, ll, tl, 0.f);
    }
  }
  for (int r = tid; r < C::kRows && r < rows; r += C::kThreads) {
    float mm = red[0][r].x;
#pragma unroll
    for (int p = 1; p < kPairs; ++p) mm = fmaxf(mm, red[p][r].x);
    float ll = 0.f;
#pragma unroll
    for (int p = 0; p < kPairs; ++p) ll += red[p][r].y * fast_exp2(red[p][r].x - mm);
    part[(static_cast<size_t>(x) * h_kv + g) * kScoreRowsPerGroup + r] = make_float2(mm, ll);
  }
}

template <int D, int RS, int NBW, bool ENT>
__global__ __launch_bounds__(64 * kPairs * RS) void k_score_pass_a(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, SeqBatch sb, int chunk_keys, int h_q,
    int h_kv, int w, int row0, int rows, float c, float2* __restrict__ part, float4* __restrict__ entpart,
    int rtot, uint32_t* __restrict__ ent_ctr, uint32_t* __restrict__ st_ctr) {
  __shared__ __attribute__((aligned(16))) char ring[kPairs][kRingBytesA];
  pass_a_unit<D, RS, NBW, ENT>(ring, threadIdx.x, blockIdx.x, blockIdx.y, q, k, sb, chunk_keys, h_q, h_kv, w, row0, rows,
                               c, part, entpart, rtot, ent_ctr, st_ctr);
}

// ---- pass B: column sums of 2^(x - lse2) ------------------------------------------
// Software pipelined like pass A.  Logits rows x keys: acc[rb][v] holds row
// rbase + 32*rb + acc_row(v, half) of key t0 + col.
template <int D, int NBW>
__device__ __forceinline__ void b_mfma(f32x16 (&acc)[NBW], const bf16x8 (&kf)[D / 16],
                                       const bf16x8 (&qf)[NBW][D / 16]) {
#pragma unroll
  for (int rb = 0; rb < NBW; ++rb) {
    acc[rb] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) acc[rb] = mfma(qf[rb][s], kf[s], acc[rb]);
  }
}

template <int D>
__device__ __forceinline__ void b_mfma1(f32x16& acc, const bf16x8 (&kf)[D / 16], const bf16x8 (&qf)[D / 16]) {
  acc = f32x16{};
#pragma unroll
  for (int s = 0; s < D / 16; ++s) acc = mfma(qf[s], kf[s], acc);
}

// Column sum of one 32-row block (rows rbase + acc_row(v, half)) for key t0 + col,
// this lane's half only.
template <bool MASK>
__device__ __forceinline__ float b_colsum1(const f32x16& acc, const float (&nl)[16], float c, int t0,
                                           int n, int w, int rbase, int G, int col, int half) {
  const int kj = t0 + col;
  float s4[4];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float x = fmaf(acc[v], c, nl[v]);
    if (MASK) {
      const int i = (rbase + acc_row(v, half)) / G;
      x = (kj < n && kj <= n - w + i) ? x : -INFINITY;
    }
    const float e = fast_exp2(x);
    if (v < 4) s4[v] = e; else s4[v & 3] += e;
  }
  return (s4[0] + s4[1]) + (s4[2] + s4[3]);
}

// This wave's column sum for key t0 + col (in both lane halves).
template <int NBW, bool MASK>
__device__ __forceinline__ float b_colsum(const f32x16 (&acc)[NBW], const float (&nl)[NBW][16], float c,
                                          int t0, int n, int w, int rbase, int G, int col, int half) {
  const int kj = t0 + col;
  float s4[4];
#pragma unroll
  for (int rb = 0; rb < NBW; ++rb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float x = fmaf(acc[rb][v], c, nl[rb][v]);
      if (MASK) {
        const int i = (rbase + 32 * rb + acc_row(v, half)) / G;
        x = (kj < n && kj <= n - w + i) ? x : -INFINITY;
      }
      const float e = fast_exp2(x);
      if (rb == 0 && v < 4) s4[v] = e; else s4[v & 3] += e;
    }
  float cs = (s4[0] + s4[1]) + (s4[2] + s4[3]);
  return cs + __shfl_xor(cs, 32);
}

// Device-scope relaxed accesses for values that another work-group of the
// same launch reads (the epilogue below): coherent across the XCDs' L2
// caches by themselves, with no cache-wide write-back or invalidate.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(double* p, double v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), __double_as_longlong(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double load_coherent(const double* p) {
  return __longlong_as_double(static_cast<long long>(__hip_atomic_load(
      reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
}

// Pass B's epilogue with the head sum and statistics (StructKV summary
// page, sections 2A-2B; FastKV section 2A): the unit's final score (its
// column sums, plus the earlier row groups' share) goes out, with c_out =
// c_in + score; the unit's sums of the three statistics' terms (fp32 terms
// as the stats kernel forms them, added in double) go to st.part.  The last
// of a unit's h_kv work-groups to finish (a per-unit count) writes the
// unit's head sum, adding the heads in order; the last of a sequence's
// units x heads work-groups writes its statistics, adding the units' sums
// in a fixed order.  Counts are zeroed by the same call's pass A.
template <int kThreads>
__device__ __forceinline__ void stats_epilogue(const ScoreStats& st, const float* obuf, float* score, int64_t T,
                                               int accumulate, int tid, int x, int g, int h_kv, const SeqBatch& sb,
                                               int sq, int n, int64_t off, int kchunk, int nk, char* scratch) {
  constexpr int kWaves = kThreads / 64;
  double* red = reinterpret_cast<double*>(scratch);   // [kWaves][3]
  int* flag = reinterpret_cast<int*>(scratch + sizeof(double) * 3 * kWaves);
  const size_t row = static_cast<size_t>(g) * T + off + kchunk;
  const bool coherent_x = st.tok != nullptr;   // the unit's last work-group reads every head's values
  const float inv_mass = static_cast<float>(1.0 / st.mass);
  const float inv_n = 1.0f / n;
  const double dn = static_cast<double>(n);
  double te = 0.0, ts = 0.0, tv = 0.0;
  for (int j = tid; j < nk; j += kThreads) {
    const float s = accumulate ? score[row + j] + obuf[j] : obuf[j];
    if (coherent_x) store_coherent(score + row + j, s); else score[row + j] = s;
    if (st.c_out != nullptr) {
      const float v = (st.c_in != nullptr ? st.c_in[row + j] : 0.f) + s;
      if (coherent_x) store_coherent(st.c_out + row + j, v); else st.c_out[row + j] = v;
    }
    if (st.stats != nullptr) {
      const float p = s * inv_mass;
      te -= p > 0.f ? static_cast<double>(p * logf(p)) : 0.0;
      const float dp = p - inv_n;
      tv += static_cast<double>(dp * dp);
      // p < 1/n decided exactly: s * n < mass (exact in double for n < 2^29)
      ts += (static_cast<double>(s) * dn < st.mass) ? 1.0 : 0.0;
    }
  }
  const int units = sb.base[sb.count];
  if (st.stats != nullptr) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      te += __shfl_xor(te, o);
      ts += __shfl_xor(ts, o);
      tv += __shfl_xor(tv, o);
    }
    if ((tid & 63) == 0) {
      red[3 * (tid >> 6)] = te;
      red[3 * (tid >> 6) + 1] = ts;
      red[3 * (tid >> 6) + 2] = tv;
    }
    __syncthreads();
    if (tid < 3) {
      double t = 0.0;
      for (int wv = 0; wv < kWaves; ++wv) t += red[3 * wv + tid];
      store_coherent(st.part + (static_cast<size_t>(x) * h_kv + g) * 3 + tid, t);
    }
  }
  wait_vmem<0>();    // this thread's coherent stores are complete ...
  __syncthreads();   // ... for every thread, before the counts
  if (tid == 0) {
    int f = 0;
    if (st.tok != nullptr &&
        __hip_atomic_fetch_add(&st.ctr[x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            static_cast<uint32_t>(h_kv - 1))
      f |= 1;
    if (st.stats != nullptr) {
      const uint32_t per_seq = static_cast<uint32_t>((sb.base[sq + 1] - sb.base[sq]) * h_kv);
      if (__hip_atomic_fetch_add(&st.ctr[units + sq], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
          per_seq - 1)
        f |= 2;
    }
    *flag = f;
  }
  __syncthreads();
  const int f = *flag;
  if (f & 1) {   // the unit's head sum: x summed over the heads in order, as kvsel_accumulate_stats does
    // Each thread takes JB keys at a time and loads HB heads' values of all
    // of them before adding any: the loads are then in flight together
    // instead of one round trip per value.
    constexpr int JB = 4, HB = 8;
    const size_t col = static_cast<size_t>(off + kchunk);
    const float* src = st.c_out != nullptr ? st.c_out : score;
    const bool add_cin = st.c_out == nullptr && st.c_in != nullptr;
    for (int j0 = tid; j0 < nk; j0 += JB * kThreads) {
      float t[JB];
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) t[jj] = 0.f;
      for (int g0 = 0; g0 < h_kv; g0 += HB) {
        float v[JB][HB];
#pragma unroll
        for (int jj = 0; jj < JB; ++jj)
#pragma unroll
          for (int hh = 0; hh < HB; ++hh) {
            const int j = min(j0 + jj * kThreads, nk - 1);      // clamped: loads stay in bounds
            const int gg = min(g0 + hh, h_kv - 1);
            v[jj][hh] = load_coherent(src + static_cast<size_t>(gg) * T + col + j);
          }
#pragma unroll
        for (int jj = 0; jj < JB; ++jj)
#pragma unroll
          for (int hh = 0; hh < HB; ++hh) {
            if (g0 + hh >= h_kv) continue;
            const size_t r = static_cast<size_t>(g0 + hh) * T + col + min(j0 + jj * kThreads, nk - 1);
            t[jj] += add_cin ? st.c_in[r] + v[jj][hh] : v[jj][hh];
          }
      }
#pragma unroll
      for (int jj = 0; jj < JB; ++jj)
        if (j0 + jj * kThreads < nk) st.tok[col + j0 + jj * kThreads] = t[jj];
    }
  }
  if ((f & 2) && tid < 64) {   // the sequence's statistics: its units' sums, one wave, fixed order
    const int c0 = sb.base[sq];
    const int terms = (sb.base[sq + 1] - c0) * h_kv;
    double e = 0.0, sp = 0.0, va = 0.0;
    for (int i = tid; i < terms; i += 64) {
      const double* pp = st.part + (static_cast<size_t>(c0) * h_kv + i) * 3;
      e += load_coherent(pp);
      sp += load_coherent(pp + 1);
      va += load_coherent(pp + 2);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      e += __shfl_xor(e, o);
      sp += __shfl_xor(sp, o);
      va += __shfl_xor(va, o);
    }
    if (tid == 0) {
      float* o = st.stats + static_cast<size_t>(sb.first + sq) * 3;
      o[0] = static_cast<float>(e / h_kv);
      o[1] = static_cast<float>(sp / (static_cast<double>(h_kv) * n));
      o[2] = static_cast<float>(va / (static_cast<double>(h_kv) * n));
    }
  }
}

// Pass B over work unit x of KV head g.  obuf (kScoreChunkMax floats) holds
// the unit's column sums, stored after the loop; before it, the merge of the
// normalisers (NSL x 128 partials, then 128 results).
template <int D, int RS, int NBW, bool STATS>
__device__ __forceinline__ void pass_b_unit(
    char (*ring)[kRingBytes], float (*xch)[2][32], float* obuf, int tid, int x, int g,
    const __bf16* __restrict__ q,
    const __bf16* __restrict__ k, const SeqBatch& sb, int chunk_keys, int h_q, int h_kv, int w, int row0,
    int rows, float c, const float2* __restrict__ part, const float* __restrict__ lse_in,
    float* __restrict__ lse, float* __restrict__ score, int64_t T, int accumulate, const ScoreStats& st) {
  constexpr int S = D / 16;
  constexpr int kThreads = 64 * kPairs * RS;
  constexpr int NSL = kThreads / kScoreRowsPerGroup;   // slices of the normaliser merge
  static_assert(kScoreChunkMax >= 3 * NSL * kScoreRowsPerGroup, "merge scratch fits obuf");
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int pair = __builtin_amdgcn_readfirstlane(wave % kPairs);    // wave-uniform
  const int split = __builtin_amdgcn_readfirstlane(wave / kPairs);
  const int half = lane >> 5;
  const int col = lane & 31;
  const Unit u = unit_of(sb, x, chunk_keys, pair);
  const int G = h_q / h_kv;
  const int rb0 = split * NBW;
  const int rbase = row0 + 32 * rb0;

  bf16x8 qf[NBW][S];
  load_q_lds<D, RS, NBW>(qf, q, sb.first + u.sq, g, G, h_q, w, row0, rows, rb0, col, half, tid, &ring[0][0]);

  // Normaliser of every row of this (sequence, KV head).  Given (lse_in, the
  // natural-log normalisers the layer's own attention computed): lse2 =
  // lse_in * log2(e).  Otherwise merge pass A's per-chunk (max, sum)
  // partials into lse2 = m + log2(l): NSL slices of threads split the
  // sequence's chunks (independent loads), then combine in a fixed order;
  // every work-group of the sequence computes the same bits, and the first
  // one publishes the natural-log value when asked.
  if (lse_in != nullptr) {
    float* lse2s = obuf + 2 * NSL * kScoreRowsPerGroup;
    const int r = tid;
    if (r < kScoreRowsPerGroup) {
      const int rr = row0 + min(r, rows - 1);
      const int i = rr / G;
      const int hh = rr - i * G;
      lse2s[r] = lse_in[(static_cast<size_t>(sb.first + u.sq) * h_q + g * G + hh) * w + i] * kLog2e;
    }
    __syncthreads();
  } else {
    float2* red = reinterpret_cast<float2*>(obuf);                      // [NSL][128]
    float* lse2s = obuf + 2 * NSL * kScoreRowsPerGroup;                  // [128]
    const int r = tid % kScoreRowsPerGroup, slice = tid / kScoreRowsPerGroup;
    const int c0 = sb.base[u.sq], c1 = sb.base[u.sq + 1];
    const float2* p = part + static_cast<size_t>(g) * kScoreRowsPerGroup + r;
    const size_t stride = static_cast<size_t>(h_kv) * kScoreRowsPerGroup;
    // batches of MB partials per thread, all loads of a batch in flight
    // (one batch covers NSL * MB chunks: a 128K-key sequence at 4096 keys
    // per chunk); padding entries are (-big, 0)
    constexpr int MB = 8;
    float m = kNegBig, l = 0.f;
    for (int b0 = c0 + slice; b0 < c1; b0 += NSL * MB) {
      float2 v[MB];
#pragma unroll
      for (int e = 0; e < MB; ++e) {
        const int cu = b0 + e * NSL;
        v[e] = cu < c1 ? p[cu * stride] : make_float2(kNegBig, 0.f);
      }
      float bm = m;
#pragma unroll
      for (int e = 0; e < MB; ++e) bm = fmaxf(bm, v[e].x);
      l *= exp2f(m - bm);
#pragma unroll
      for (int e = 0; e < MB; ++e) l += v[e].y * exp2f(v[e].x - bm);
      m = bm;
    }
    red[slice * kScoreRowsPerGroup + r] = make_float2(m, l);
    __syncthreads();
    if (slice == 0) {
      float mm = red[r].x;
#pragma unroll
      for (int s2 = 1; s2 < NSL; ++s2) mm = fmaxf(mm, red[s2 * kScoreRowsPerGroup + r].x);
      float ll = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < NSL; ++s2) ll += red[s2 * kScoreRowsPerGroup + r].y * exp2f(red[s2 * kScoreRowsPerGroup + r].x - mm);
      const float v = mm + log2f(ll);
      lse2s[r] = v;
      if (lse != nullptr && x == c0 && r < rows) {
        const int rr = row0 + r;
        const int i = rr / G;
        const int hh = rr - i * G;
        lse[(static_cast<size_t>(sb.first + u.sq) * h_q + g * G + hh) * w + i] = v * kLn2;
      }
    }
    __syncthreads();
  }
  // -lse2 of the rows this lane holds in the rows x keys layout; padding
  // rows get -inf so they add nothing
  float nl[NBW][16];
#pragma unroll
  for (int rb = 0; rb < NBW; ++rb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int rr = 32 * (rb0 + rb) + acc_row(v, half);
      nl[rb][v] = rr < rows ? -obuf[2 * NSL * kScoreRowsPerGroup + rr] : -INFINITY;
    }
  __syncthreads();   // obuf becomes the column-sum buffer

  const int full_lim = u.n - w + 1;
  // (the key tiles are requested only now: with loads of its own in flight
  // the compiler would put a wait for everything before the tile loop's
  // LDS reads)
  Ring<D, RS, kReverseB, kRingBytes> rg{k, u.off, u.n, u.kbeg,
                            u.kend > u.kbeg ? (u.kend - u.kbeg + kTile - 1) / kTile : 0,
                            h_kv, g, lane, split == 0, ring[pair]};
  rg.rot = walk_start(rg.ntiles, x, pair);
  rg.start();
  // Column sums collect in LDS and leave in one coalesced store at the end:
  // a global store inside the loop would count against the ring's vmcnt
  // waits (loads and stores share the counter).
  const int kchunk = u.kbeg - pair * (chunk_keys / kPairs);   // first key of the work-group
  auto emit = [&](int kj, float cs) {
    if (half == 0) obuf[kj - kchunk] = cs;
  };

  const int tmax = RS > 1 ? chunk_keys / (kPairs * kTile) : rg.ntiles;   // uniform when RS > 1
  // With two waves per pair, split 1 hands its half of tile s's column sums
  // over through xch[pair][s & 1] during iteration s+1 and split 0 adds them
  // during iteration s+2, after the barrier that separates the two.
  if constexpr (NBW == 2) {
    // Row-block pipeline as in pass A.  With two waves per pair, split 1
    // hands tile t's half over through xch[pair][t & 1] at the end of
    // iteration t; split 0 adds it in iteration t+1, after the barrier.
    const float (&nl0)[16] = nl[0];
    const float (&nl1)[16] = nl[1];
    auto part = [&](const f32x16& acc, const float (&nlr)[16], int t0, int rb) {
      return (t0 + kTile <= full_lim)
          ? b_colsum1<false>(acc, nlr, c, t0, u.n, w, rbase + 32 * rb, G, col, half)
          : b_colsum1<true>(acc, nlr, c, t0, u.n, w, rbase + 32 * rb, G, col, half);
    };
    bf16x8 kf[S];
    f32x16 acc_a, acc_b;
    // one half-step: the MFMAs of one block into acc_new and the column sums
    // of the other (acc_old), in one basic block so the scheduler can
    // interleave them (as in pass A)
    auto both = [&](f32x16& acc_new, const bf16x8 (&qfb)[S], const f32x16& acc_old,
                    const float (&nlr)[16], int t0s, int rb) {
      float r;
      if (t0s + kTile <= full_lim) {
        b_mfma1<D>(acc_new, kf, qfb);
        r = b_colsum1<false>(acc_old, nlr, c, t0s, u.n, w, rbase + 32 * rb, G, col, half);
        interleave_mfma_valu<S, kValuPerMfmaB>();
      } else {
        b_mfma1<D>(acc_new, kf, qfb);
        r = b_colsum1<true>(acc_old, nlr, c, t0s, u.n, w, rbase + 32 * rb, G, col, half);
        interleave_mfma_valu<S, kValuPerMfmaB>();
      }
      return r;
    };
    int t0 = 0, t0n = 0;
    float pend = 0.f;
    int pend_kj = 0;
    bool live = tmax > 0 && rg.fetch(0, kf, &t0);
    if (live) b_mfma1<D>(acc_a, kf, qf[0]);
    for (int t = 0; t < tmax; ++t) {
      float cs = 0.f;
      if (live) cs = both(acc_b, qf[1], acc_a, nl0, t0, 0);
      bool live_n = false;
      if (t + 1 < tmax) {
        live_n = rg.fetch(t + 1, kf, &t0n);
      } else if (RS > 1) {
        wait_lds();
        barrier();
      }
      if (RS > 1 && split == 0 && t >= 1 && t - 1 < rg.ntiles)
        emit(pend_kj, pend + xch[pair][(t - 1) & 1][col]);
      if (live_n && live) {
        cs += both(acc_a, qf[0], acc_b, nl1, t0, 1);
      } else {
        if (live_n) b_mfma1<D>(acc_a, kf, qf[0]);
        if (live) cs += part(acc_b, nl1, t0, 1);
      }
      if (live) {
        cs += __shfl_xor(cs, 32);
        if (RS == 1) {
          emit(t0 + col, cs);
        } else if (split == 1) {
          if (half == 0) xch[pair][t & 1][col] = cs;
        } else {
          pend = cs;
          pend_kj = t0 + col;
        }
      }
      live = live_n;
      t0 = t0n;
    }
    if (RS > 1) {
      wait_lds();
      barrier();
      if (split == 0 && tmax >= 1 && tmax - 1 < rg.ntiles)
        emit(pend_kj, pend + xch[pair][(tmax - 1) & 1][col]);
    }
  } else {
    // Two accumulator sets and two pending sums, addressed statically: the
    // loop is unrolled by two (set 0 / pend 0 belong to even tiles).
    f32x16 acc0[NBW], acc1[NBW];
    float pend0 = 0.f, pend1 = 0.f;
    int pkj0 = 0, pkj1 = 0;
    int t0_prev = 0;
    auto step = [&](int t, f32x16 (&acc_new)[NBW], f32x16 (&acc_old)[NBW], float& pend_new,
                    int& pkj_new, float& pend_old, int& pkj_old) {
      // acc_new / pend_new: tile t (and t-2); acc_old / pend_old: tile t-1
      bf16x8 kf[S];
      int t0 = 0;
      bool live = false;
      if (t < tmax) {
        live = rg.fetch(t, kf, &t0);
      } else if (RS > 1) {
        wait_lds();
        barrier();
      }
      if (RS > 1 && split == 0 && t >= 2 && t - 2 < rg.ntiles)
        emit(pkj_new, pend_new + xch[pair][t & 1][col]);
      if (live) b_mfma<D, NBW>(acc_new, kf, qf);
      if (t >= 1 && t - 1 < rg.ntiles) {
        const float cs = (t0_prev + kTile <= full_lim)
            ? b_colsum<NBW, false>(acc_old, nl, c, t0_prev, u.n, w, rbase, G, col, half)
            : b_colsum<NBW, true>(acc_old, nl, c, t0_prev, u.n, w, rbase, G, col, half);
        if (RS == 1) {
          emit(t0_prev + col, cs);
        } else if (split == 1) {
          if (half == 0) xch[pair][(t - 1) & 1][col] = cs;
        } else {
          pend_old = cs;
          pkj_old = t0_prev + col;
        }
      }
      t0_prev = t0;
    };
    for (int t = 0; t <= tmax; t += 2) {
      step(t, acc0, acc1, pend0, pkj0, pend1, pkj1);
      if (t + 1 <= tmax) step(t + 1, acc1, acc0, pend1, pkj1, pend0, pkj0);
    }
    if (RS > 1) {
      wait_lds();
      barrier();
      if (split == 0 && tmax >= 1 && tmax - 1 < rg.ntiles)
        emit(((tmax - 1) & 1) ? pkj1 : pkj0,
             (((tmax - 1) & 1) ? pend1 : pend0) + xch[pair][(tmax - 1) & 1][col]);
    }
  }
  __syncthreads();
  const int nk = min(chunk_keys, u.n - kchunk);
  if constexpr (STATS) {
    stats_epilogue<kThreads>(st, obuf, score, T, accumulate, tid, x, g, h_kv, sb, u.sq, u.n, u.off, kchunk, nk,
                             &ring[0][0]);
  } else {
    float* out = score + static_cast<size_t>(g) * T + u.off + kchunk;
    for (int j = tid; j < nk; j += kThreads)
      out[j] = accumulate ? out[j] + obuf[j] : obuf[j];
  }
}

template <int D, int RS, int NBW, bool STATS>
__global__ __launch_bounds__(64 * kPairs * RS) void k_score_pass_b(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, SeqBatch sb, int chunk_keys, int h_q,
    int h_kv, int w, int row0, int rows, float c, const float2* __restrict__ part,
    const float* __restrict__ lse_in, float* __restrict__ lse, float* __restrict__ score, int64_t T,
    int accumulate, ScoreStats st) {
  __shared__ __attribute__((aligned(16))) char ring[kPairs][kRingBytes];
  __shared__ float xch[kPairs][2][32];
  __shared__ __attribute__((aligned(16))) float obuf[kScoreChunkMax];
  pass_b_unit<D, RS, NBW, STATS>(ring, xch, obuf, threadIdx.x, blockIdx.x, blockIdx.y, q, k, sb, chunk_keys, h_q,
                                 h_kv, w, row0, rows, c, part, lse_in, lse, score, T, accumulate, st);
}

// Row entropies of one launch's sequences, one work-group per (sequence,
// KV head) and a thread per row: the row's (m, l, tt) partials merged over
// the sequence's work units in order, H = ln2 * (log2 l - tt / l), written
// to row_ent [B, h_q, w].  For mean_ent, each work-group leaves the sum of
// its rows' H (fixed order) in head_sum and counts itself in ctr[sequence]
// (zeroed by the same call's pass A); the sequence's last work-group adds
// the h_kv sums in head order.  The partials load 32 units at a time.
constexpr int kEntThreads = 256;
__global__ __launch_bounds__(kEntThreads) void k_row_entropy(SeqBatch sb, const float4* __restrict__ entpart,
                                                             int h_q, int h_kv, int w,
                                                             float* __restrict__ row_ent,
                                                             float* __restrict__ mean_ent,
                                                             uint32_t* __restrict__ ctr,
                                                             double* __restrict__ head_sum) {
  constexpr int MB = 32;   // a 128K-key sequence's units in one batch
  __shared__ double red[kEntThreads / 64];
  __shared__ int last;
  const int sq = blockIdx.x;
  const int g = blockIdx.y;
  const int G = h_q / h_kv;
  const int R = w * G;
  const int c0 = sb.base[sq], c1 = sb.base[sq + 1];
  const int b = sb.first + sq;
  const size_t stride = static_cast<size_t>(h_kv) * R;
  double tot = 0.0;
  for (int r = threadIdx.x; r < R; r += kEntThreads) {
    const float4* p = entpart + static_cast<size_t>(g) * R + r;
    // per batch: the running state moves to the batch's max once, then each
    // unit adds l_u 2^(m_u - M) to l and 2^(m_u - M) (tt_u + (m_u - M) l_u)
    // to tt, in unit order
    float m = kNegBig, l = 0.f, tl = 0.f;
    for (int cb = c0; cb < c1; cb += MB) {
      float4 v[MB];
#pragma unroll
      for (int e = 0; e < MB; ++e)
        v[e] = cb + e < c1 ? p[(cb + e) * stride] : make_float4(kNegBig, 0.f, 0.f, 0.f);
      float bm = m;
#pragma unroll
      for (int e = 0; e < MB; ++e) bm = fmaxf(bm, v[e].x);
      const float a = fast_exp2(m - bm);
      tl = a * fmaf(m - bm, l, tl);
      l *= a;
#pragma unroll
      for (int e = 0; e < MB; ++e) {
        const float dm = v[e].x - bm;
        const float f = fast_exp2(dm);
        l = fmaf(f, v[e].y, l);
        tl = fmaf(f, fmaf(dm, v[e].y, v[e].z), tl);
      }
      m = bm;
    }
    const float h = kLn2 * (log2f(l) - tl / l);
    const int i = r / G, hh = r - i * G;
    row_ent[(static_cast<size_t>(b) * h_q + g * G + hh) * w + i] = h;
    tot += h;
  }
  if (mean_ent == nullptr) return;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = tot;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int i = 0; i < kEntThreads / 64; ++i) t += red[i];
    head_sum[static_cast<size_t>(sq) * h_kv + g] = t;
    __threadfence();   // the sum is visible device-wide before the count
    const uint32_t done = __hip_atomic_fetch_add(&ctr[sq], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last = done + 1 == static_cast<uint32_t>(h_kv);
  }
  __syncthreads();
  if (last && threadIdx.x == 0) {
    __threadfence();
    double t = 0.0;
    for (int gg = 0; gg < h_kv; ++gg)
      t += __hip_atomic_load(&head_sum[static_cast<size_t>(sq) * h_kv + gg], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    mean_ent[b] = static_cast<float>(t / (static_cast<double>(h_kv) * R));
  }
}

template <int D, int RS, int NBW>
hipError_t run(const WindowScoreLaunch& a, const SeqBatch& sb, int row0, int rows, hipStream_t st) {
  using C = Cfg<D, RS, NBW>;
  const int units = sb.base[sb.count];
  const float c = a.scale * 1.44269504088896340736f;
  const __bf16* q = static_cast<const __bf16*>(a.q);
  const __bf16* k = static_cast<const __bf16*>(a.k);
  float2* part = static_cast<float2*>(a.part);
  dim3 grid(units, a.h_kv);
  const int rtot = a.w * (a.h_q / a.h_kv);
  float4* entpart = static_cast<float4*>(a.entpart);
  // the statistics epilogue runs in the last row group's pass B, on the
  // final score; that row group's pass A zeroes its counters
  const bool last_rows = row0 + rows >= rtot;
  const bool with_stats = a.st != nullptr && last_rows && a.lse_in == nullptr && entpart == nullptr;
  uint32_t* st_ctr = with_stats ? a.st->ctr : nullptr;
  if (a.lse_in == nullptr && entpart != nullptr)
    k_score_pass_a<D, RS, NBW, true><<<grid, C::kThreads, 0, st>>>(q, k, sb, a.chunk, a.h_q, a.h_kv, a.w,
                                                                   row0, rows, c, part, entpart, rtot,
                                                                   a.ent_ctr, nullptr);
  else if (a.lse_in == nullptr)
    k_score_pass_a<D, RS, NBW, false><<<grid, C::kThreads, 0, st>>>(q, k, sb, a.chunk, a.h_q, a.h_kv, a.w,
                                                                    row0, rows, c, part, nullptr, rtot,
                                                                    nullptr, st_ctr);
  if (with_stats)
    k_score_pass_b<D, RS, NBW, true><<<grid, C::kThreads, 0, st>>>(q, k, sb, a.chunk, a.h_q, a.h_kv, a.w,
                                                                   row0, rows, c, part, a.lse_in, a.lse, a.score,
                                                                   a.T, row0 > 0 ? 1 : 0, *a.st);
  else
    k_score_pass_b<D, RS, NBW, false><<<grid, C::kThreads, 0, st>>>(q, k, sb, a.chunk, a.h_q, a.h_kv, a.w,
                                                                    row0, rows, c, part, a.lse_in, a.lse, a.score,
                                                                    a.T, row0 > 0 ? 1 : 0, ScoreStats{});
  return hipGetLastError();
}

template <int D>
hipError_t run_d(const WindowScoreLaunch& a, const SeqBatch& sb, int row0, int rows, hipStream_t st) {
  switch ((rows + 31) / 32) {
    case 1: return run<D, 1, 1>(a, sb, row0, rows, st);
    case 2: return run<D, 1, 2>(a, sb, row0, rows, st);
    default: return run<D, 2, 2>(a, sb, row0, rows, st);
  }
}

}  // namespace

hipError_t launch_window_score(const WindowScoreLaunch& a, const SeqBatch& sb, int row0, int rows,
                               hipStream_t stream) {
  if (a.d == 64) return run_d<64>(a, sb, row0, rows, stream);
  return run_d<128>(a, sb, row0, rows, stream);
}

hipError_t launch_row_entropy(const WindowScoreLaunch& a, const SeqBatch& sb, hipStream_t stream) {
  k_row_entropy<<<dim3(sb.count, a.h_kv), kEntThreads, 0, stream>>>(
      sb, static_cast<const float4*>(a.entpart), a.h_q, a.h_kv, a.w, a.row_ent, a.mean_ent, a.ent_ctr,
      a.ent_head);
  return hipGetLastError();
}

}  // namespace kvsel
