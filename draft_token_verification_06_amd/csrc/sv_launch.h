// Kernel argument blocks and launchers (host-callable, defined in sv_kernels.hip).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "sv_plan.h"

namespace sv {

struct WindowArgs {
  const char *t;
  int64_t t_stride_bytes;
  const char *d;
  int64_t d_stride_bytes;
  const int32_t *tokens;
  const int32_t *window_len;
  int32_t gamma, V, S;
  uint64_t seed, tag;
  const uint64_t *seq_ids;
  const int64_t *base_pos;
  const float2 *part;
  int32_t *n_accepted;
  int32_t *out_tokens;
  float *p_draft, *q_draft;
  SampleJob *jobs;
  int32_t stage_lo;   // early exit: first position of the last block (decided in the draw)
  int32_t *status;    // early exit: per-sequence status
};

struct GreedyArgs {
  const int32_t *tokens;
  const int32_t *window_len;
  int32_t gamma, V, S;
  const float2 *part;
  int32_t *n_accepted;
  int32_t *out_tokens;
};

struct TreeArgs {
  const char *t;
  const char *d;
  int64_t seq_bytes;
  const int32_t *tokens;
  int32_t V, S, R, mode;
  uint64_t seed, tag;
  const uint64_t *seq_ids;
  const int64_t *base_pos;
  const float2 *part;
  int32_t *n_accepted, *best_node, *out_tokens, *out_nodes;
  SampleJob *jobs;
  TreeMeta meta;
};

struct RollbackArgs {
  int32_t *buf_tokens;
  int32_t *buf_len;
  int32_t K, cap;
  const int32_t *verified;
  int64_t verified_stride;
  const int32_t *verified_len;
  int32_t len_offset;
};

// LM-head fused window.  GEMM rows g < M: hidden row g of A (row stride lda
// elements) against every row of W ([V][K], bf16).
struct LmGemmArgs {
  const uint16_t *A;
  int64_t lda;
  const uint16_t *W;
  int32_t M, V, K;
  int32_t RB, NT;             // row blocks, column tiles (set by the launcher)
  float2 *part;               // [M][NT] (max, sum-exp) per row and column tile
  float *gath;                // [M] logit at the row's draft token
  const int32_t *tokens;      // [B][gamma]
  int32_t gamma, rows_per_seq;
  float *out;                 // [M][V] float32 logits
};

struct LmDecideArgs {
  const float2 *stats_t, *stats_d;
  const float *gath_t, *gath_d;
  const int32_t *tokens;
  const int32_t *window_len;
  int32_t gamma, V;
  uint64_t seed, tag;
  const uint64_t *seq_ids;
  const int64_t *base_pos;
  int32_t *n_accepted, *out_tokens;
  float *p_draft, *q_draft;
  SampleJob *jobs;
  const float *rows_t, *rows_d;  // the GEMM's float32 logits, [B][gamma+1][V] / [B][gamma][V]
  int32_t *arrive;               // arrival counters of the draw, zeroed here
};

// Launches the GEMMs of two problems (target rows, draft rows) as one grid.
void launch_lm_gemm(LmGemmArgs A0, LmGemmArgs A1, hipStream_t st);
int64_t lm_gemm_blocks(int64_t M, int V);
void launch_lm_combine(const float2 *part, int NT, int M, float2 *stats, hipStream_t st);
void launch_lm_decide(const LmDecideArgs &A, int B, hipStream_t st);

// Workspace of the split draw (several workgroups per sequence): chunk sums
// spart [B][cmax] and one arrival counter per sequence, which the launch
// before the draw zeroes.
struct DrawScratch {
  float *spart;
  int cmax;
  int32_t *arrive;
};

void launch_window_finish(int dtype, const WindowArgs &A, int B, const DrawScratch &ds, hipStream_t st);
void launch_stage_decide(int dtype, const WindowArgs &A, int B, int lo, int hi, int32_t *status, hipStream_t st);
void launch_stage_finish(int dtype, const WindowArgs &A, int B, const DrawScratch &ds, hipStream_t st);
void launch_greedy_decide(const GreedyArgs &A, int B, hipStream_t st);
void launch_tree_decide(int dtype, const TreeArgs &A, int B, hipStream_t st);
void launch_tree_finish(int dtype, SampleJob *jobs, int B, int V, const DrawScratch &ds, hipStream_t st);
// Stochastic tree: the draw kernels decide each sequence themselves (no separate decision launch).
void launch_tree_decide_draw(int dtype, const TreeArgs &A, int B, const DrawScratch &ds, hipStream_t st);
void launch_tree_walk(int dtype, const TreeArgs &A, int B, hipStream_t st);
void launch_rollback(const RollbackArgs &A, int S, int stage, hipStream_t st);

}  // namespace sv
