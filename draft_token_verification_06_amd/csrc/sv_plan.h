// Launch plan and workspace layout shared by the C-ABI layer and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "sv_rowset.h"

namespace sv {

#ifndef SV_FIN_THREADS
#define SV_FIN_THREADS 1024
#endif
#ifndef SV_FIN_BATCH
#define SV_FIN_BATCH 2
#endif
constexpr int kFinThreads = SV_FIN_THREADS;  // sampling workgroup (one per sequence)
constexpr int kFinWaves = kFinThreads / 64;
constexpr int kFinBatch = SV_FIN_BATCH;      // chunks per pipelined batch
constexpr int kMaxVocab = 1 << 21;    // 2,097,152 tokens
// Chunks of a sampling pass: at most ceil((V + 3) / (4 kFinThreads)) (four
// slots per thread and up to 3 slots of head offset); 513 at 1024 threads.
constexpr int fin_chunks_max(int V) { return (V + 3 + kFinThreads * 4 - 1) / (kFinThreads * 4); }
constexpr int kFinMaxChunks = fin_chunks_max(kMaxVocab);
constexpr int kFinFillWorkgroups = 256;  // draw workgroups wanted per launch
constexpr int kMaxSegments = 64;      // row segments (split-row mode)
constexpr int64_t kFillWorkgroups = 16384;  // row workgroups per launch (256 CUs)
// A row splits into at most ceil(V / kMinSegment) segments: shorter segments
// leave each workgroup too few loads to cover its start-up and reduction.
constexpr int kMinSegment = 32768;

// Work item of the sampling pass of one sequence: draw from
//   w_k = p_k                       (BONUS)
//   w_k = max(0, p_k - cq * q_k)    (RESIDUAL; cq = 1 for a window or a node's
//                                    first residual, larger after several
//                                    rejected siblings)
// with p_k = 2^(t_k log2e - ct), q_k = 2^(d_k log2e - cd); the offsets carry
// the row maximum and the log of the row's normaliser.
enum : int { JOB_NONE = 0, JOB_BONUS = 1, JOB_RESIDUAL = 2 };

struct SampleJob {
  const void *t_row;
  const void *d_row;
  int32_t *out_slot;  // where the drawn token is stored
  float ct, cd;
  float v;            // sampling uniform
  int32_t mode;
  float cq;           // coefficient of q in the residual (>= 1)
  int32_t pad[5];
};
static_assert(sizeof(SampleJob) == 64, "SampleJob is one 64-byte record");

// Tree shape handed to the tree kernels by value.
constexpr int kTreeMaxDepth = 64;
struct TreeMeta {
  int32_t N;
  int32_t max_depth;
  uint64_t internal[kTreeMaxNodes / 64];  // bit v: node v has children
  int16_t parent[kTreeMaxNodes];
  int16_t rank[kTreeMaxNodes];
  int16_t first_child[kTreeMaxNodes];     // smallest child index, or -1
  int16_t next_sibling[kTreeMaxNodes];    // next larger index with the same parent, or -1
  uint8_t depth[kTreeMaxNodes];
};
static_assert(sizeof(TreeMeta) <= 2560, "tree metadata travels in the kernel arguments");

// LM-head fused path: vocabulary columns per GEMM block tile, threads per
// GEMM workgroup.
constexpr int kLmBN = 256;
constexpr int kLmGemmThreads = 512;

// A dispatch packet gives each grid dimension's size in work-items as a 32-bit
// count, so a launch of `blocks` workgroups of `threads` along one dimension
// must stay within it; the entry points reject calls whose grids would not.
constexpr int64_t kMaxGridItems = 0xFFFFFFFFll;
inline bool grid_fits(int64_t blocks, int64_t threads) { return blocks >= 1 && blocks <= kMaxGridItems / threads; }

struct RowPlan {
  int S;        // segments per row
  int seg_len;  // elements per segment (multiple of 8)
};

inline RowPlan plan_rows(int64_t rows_total, int32_t V) {
  int64_t S = 1;
  if (rows_total < kFillWorkgroups) S = (kFillWorkgroups + rows_total - 1) / rows_total;
  int64_t cap = (V + kMinSegment - 1) / kMinSegment;
  if (cap < 1) cap = 1;
  if (S > cap) S = cap;
  if (S > kMaxSegments) S = kMaxSegments;
  int64_t seg = (V + S - 1) / S;
  seg = (seg + 7) / 8 * 8;
  S = (V + seg - 1) / seg;
  return {static_cast<int>(S), static_cast<int>(seg)};
}

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace sections (byte offsets); rows_per_seq counts target + draft rows.
struct Layout {
  RowPlan plan;
  int rows_per_seq;
  int cmax;  // chunk sums per sequence in the split draw
  size_t part_off, jobs_off, spart_off, status_off, arrive_off, total;
};

// op: 0 window, 1 greedy, 2 tree (n = gamma or N).
inline Layout make_layout(int op, int64_t B, int32_t n, int32_t V) {
  Layout L{};
  if (op == 0) L.rows_per_seq = 2 * n + 1;
  else if (op == 1) L.rows_per_seq = n + 1;
  else L.rows_per_seq = 2 * n;
  L.plan = plan_rows(B * L.rows_per_seq, V);
  size_t off = 0;
  L.part_off = off;
  off = align256(off + sizeof(float) * 2 * static_cast<size_t>(B) * L.rows_per_seq * L.plan.S);
  L.jobs_off = off;
  off = align256(off + (op == 1 ? 0 : sizeof(SampleJob) * static_cast<size_t>(B)));
  L.cmax = (op == 1) ? 0 : fin_chunks_max(V);
  L.spart_off = off;
  off = align256(off + sizeof(float) * static_cast<size_t>(B) * L.cmax);
  L.status_off = off;  // early-exit window: per-sequence status
  off = align256(off + (op == 0 ? sizeof(int32_t) * static_cast<size_t>(B) : 0));
  L.arrive_off = off;  // split draw: per-sequence arrival counter
  off = align256(off + (op == 1 ? 0 : sizeof(int32_t) * static_cast<size_t>(B)));
  L.total = off;
  return L;
}

// Workspace of the LM-head fused window (byte offsets).  Rows: B(gamma+1)
// target rows then B gamma draft rows.
struct LmLayout {
  int NT;  // column tiles
  int cmax;
  size_t part_off, stats_off, gath_off, jobs_off, spart_off, arrive_off, rows_t_off, rows_d_off, total;
};

inline LmLayout make_lm_layout(int64_t B, int32_t gamma, int32_t V) {
  LmLayout L{};
  const int64_t Mt = B * (gamma + 1), Md = B * gamma, M = Mt + Md;
  L.NT = (V + kLmBN - 1) / kLmBN;
  L.cmax = fin_chunks_max(V);
  size_t off = 0;
  L.part_off = off;
  off = align256(off + sizeof(float) * 2 * static_cast<size_t>(M) * L.NT);
  L.stats_off = off;
  off = align256(off + sizeof(float) * 2 * static_cast<size_t>(M));
  L.gath_off = off;
  off = align256(off + sizeof(float) * static_cast<size_t>(M));
  L.jobs_off = off;
  off = align256(off + sizeof(SampleJob) * static_cast<size_t>(B));
  L.spart_off = off;
  off = align256(off + sizeof(float) * static_cast<size_t>(B) * L.cmax);
  L.arrive_off = off;
  off = align256(off + sizeof(int32_t) * static_cast<size_t>(B));
  L.rows_t_off = off;
  off = align256(off + sizeof(float) * static_cast<size_t>(Mt) * V);
  L.rows_d_off = off;
  off = align256(off + sizeof(float) * static_cast<size_t>(Md) * V);
  L.total = off;
  return L;
}

}  // namespace sv
