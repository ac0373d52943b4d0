// C-ABI entry points of libspecverify.so: argument validation, workspace
// carving and kernel dispatch.  No allocation, no synchronisation; every
// launch goes to the caller's stream.
#include <algorithm>
#include <cstdint>
#include <cstring>

#include "sv.h"
#include "sv_launch.h"
#include "sv_plan.h"

using namespace sv;

namespace {

constexpr int kVersion = 10100;  // 1.1.0
constexpr int kWaveThreads = 64;  // threads of the one-wavefront launches (decisions, rollback)

// The row list of a launch holds a full window's rows and a tree's target rows
// plus its internal draft rows.
static_assert(kMaxLaunchRows >= 2 * SV_MAX_GAMMA + 1, "row list too short for a window");
static_assert(kMaxLaunchRows >= 2 * kTreeMaxNodes - 1, "row list too short for a tree");

int elem_bytes(int dtype) {
  switch (dtype) {
    case SV_DT_F32: return 4;
    case SV_DT_BF16:
    case SV_DT_F16: return 2;
    default: return 0;
  }
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_workspace(void *ws, size_t bytes, size_t need) {
  if (need == 0) return SV_EINVAL;
  if (!ws || !aligned(ws, 256) || bytes < need) return SV_EWORKSPACE;
  return SV_OK;
}

// The row-statistics grid (one workgroup per listed row and segment; a
// layout's rows_per_seq bounds the rows a launch lists) fits a dispatch.
bool rows_fit(int64_t B, const Layout &L) {
  return grid_fits(B * L.rows_per_seq * L.plan.S, kRowThreads);
}

int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SV_OK : SV_ELAUNCH;
}

// Builds the tree description; returns SV_OK or SV_ETREE.
int build_tree(const int32_t *parent, int32_t N, TreeMeta *meta) {
  if (!parent || N < 1 || N > kTreeMaxNodes) return SV_ETREE;
  if (parent[0] != -1) return SV_ETREE;
  std::memset(meta, 0, sizeof(*meta));
  meta->N = N;
  int count_at[kTreeMaxNodes + 1] = {0};
  count_at[0] = 1;
  meta->parent[0] = -1;
  int last_child[kTreeMaxNodes];
  for (int v = 0; v < kTreeMaxNodes; ++v) {
    meta->first_child[v] = -1;
    meta->next_sibling[v] = -1;
    last_child[v] = -1;
  }
  int max_depth = 0;
  for (int v = 1; v < N; ++v) {
    const int w = parent[v];
    if (w < 0 || w >= v) return SV_ETREE;
    const int d = meta->depth[w] + 1;
    if (d > kTreeMaxDepth) return SV_ETREE;
    meta->parent[v] = static_cast<int16_t>(w);
    meta->depth[v] = static_cast<uint8_t>(d);
    meta->rank[v] = static_cast<int16_t>(count_at[d]++);
    meta->internal[w >> 6] |= 1ull << (w & 63);
    if (last_child[w] < 0) meta->first_child[w] = static_cast<int16_t>(v);
    else meta->next_sibling[last_child[w]] = static_cast<int16_t>(v);
    last_child[w] = v;
    if (d > max_depth) max_depth = d;
  }
  meta->max_depth = max_depth;
  return SV_OK;
}

}  // namespace

extern "C" {

int sv_version(void) { return kVersion; }

const char *sv_strerror(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_EINVAL: return "invalid argument (size, null or misaligned pointer)";
    case SV_EDTYPE: return "unknown logits dtype";
    case SV_EWORKSPACE: return "workspace missing, not 256-byte aligned, or too small";
    case SV_ETREE: return "malformed tree (parent[0] != -1, parent[v] not in [0, v), too many nodes or too deep)";
    case SV_ELAUNCH: return "kernel launch failed";
    case SV_ESCRATCH: return "the call needs more workspace than the library's static scratch (SV_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

size_t sv_workspace_size(int op, int32_t B, int32_t n, int32_t V, int dtype) {
  if (elem_bytes(dtype) == 0 || B < 1 || V < 1 || V > kMaxVocab) return 0;
  if (op == SV_OP_WINDOW || op == SV_OP_GREEDY) {
    if (n < 1 || n > SV_MAX_GAMMA) return 0;
  } else if (op == SV_OP_TREE) {
    if (n < 1 || n > SV_TREE_MAX_NODES) return 0;
  } else if (op == SV_OP_LMHEAD) {
    if (n < 1 || n > SV_MAX_GAMMA || dtype != SV_DT_BF16) return 0;
    return make_lm_layout(B, n, V).total;
  } else {
    return 0;
  }
  return make_layout(op, B, n, V).total;
}

}  // extern "C"

namespace {

constexpr int kPartRows = 1, kPartFinish = 2, kEarlyExit = 4;

// parts: kPartRows = row statistics, kPartFinish = decide + draw; kEarlyExit:
// rows in position blocks, each followed by a decide, then the draw.
int window_impl(int parts, const void *target_logits, int64_t target_seq_stride,
                const void *draft_logits, int64_t draft_seq_stride, int dtype,
                const int32_t *draft_tokens, const int32_t *window_len,
                int32_t B, int32_t gamma, int32_t V,
                uint64_t seed, uint64_t tag, const uint64_t *seq_ids,
                const int64_t *base_pos,
                int32_t *n_accepted, int32_t *out_tokens,
                float *p_draft, float *q_draft,
                void *workspace, size_t workspace_bytes, hipStream_t stream) {
  const int eb = elem_bytes(dtype);
  if (eb == 0) return SV_EDTYPE;
  if (B < 1 || gamma < 1 || gamma > SV_MAX_GAMMA || V < 1 || V > kMaxVocab) return SV_EINVAL;
  if (!target_logits || !draft_logits || !draft_tokens || !n_accepted || !out_tokens) return SV_EINVAL;
  if (!aligned(target_logits, eb) || !aligned(draft_logits, eb)) return SV_EINVAL;
  const int64_t t_rows = static_cast<int64_t>(gamma + 1) * V;
  const int64_t d_rows = static_cast<int64_t>(gamma) * V;
  if (target_seq_stride == 0) target_seq_stride = t_rows;
  if (draft_seq_stride == 0) draft_seq_stride = d_rows;
  if (target_seq_stride < t_rows || draft_seq_stride < d_rows) return SV_EINVAL;
  const Layout L = make_layout(SV_OP_WINDOW, B, gamma, V);
  if (!rows_fit(B, L) || !grid_fits(B, kFinThreads)) return SV_EINVAL;
  const int ws = check_workspace(workspace, workspace_bytes, L.total);
  if (ws != SV_OK) return ws;

  char *wsb = static_cast<char *>(workspace);
  float2 *part = reinterpret_cast<float2 *>(wsb + L.part_off);
  SampleJob *jobs = reinterpret_cast<SampleJob *>(wsb + L.jobs_off);
  const DrawScratch ds{reinterpret_cast<float *>(wsb + L.spart_off), L.cmax,
                       reinterpret_cast<int32_t *>(wsb + L.arrive_off)};

  RowSet rs{};
  rs.t = static_cast<const char *>(target_logits);
  rs.t_stride_bytes = target_seq_stride * eb;
  rs.d = static_cast<const char *>(draft_logits);
  rs.d_stride_bytes = draft_seq_stride * eb;
  rs.arrive = ds.arrive;
  rs.B = B;
  rs.R_out = 2 * gamma + 1;
  rs.d_slot0 = gamma + 1;
  rs.window_len = window_len;
  rs.status = nullptr;
  rs.gamma = gamma;
  rs.V = V;
  rs.S = L.plan.S;
  rs.seg_len = L.plan.seg_len;
  WindowArgs A{};
  A.t = rs.t;
  A.t_stride_bytes = rs.t_stride_bytes;
  A.d = rs.d;
  A.d_stride_bytes = rs.d_stride_bytes;
  A.tokens = draft_tokens;
  A.window_len = window_len;
  A.gamma = gamma;
  A.V = V;
  A.S = L.plan.S;
  A.seed = seed;
  A.tag = tag;
  A.seq_ids = seq_ids;
  A.base_pos = base_pos;
  A.part = part;
  A.n_accepted = n_accepted;
  A.out_tokens = out_tokens;
  A.p_draft = p_draft;
  A.q_draft = q_draft;
  A.jobs = jobs;
  if ((parts & kPartRows) && !(parts & kEarlyExit)) {
    RowSet all = rs;
    all.add_target(0, gamma + 1);
    all.add_draft(0, gamma);
    launch_row_stats(dtype, false, all, part, stream);
  }
  if (!(parts & (kPartFinish | kEarlyExit))) return launch_status();
  if (!(parts & kEarlyExit)) {
    launch_window_finish(dtype, A, B, ds, stream);
    return launch_status();
  }
  // Position blocks of doubling width [0,1), [1,3), [3,7), ... up to the bonus
  // row gamma; a block that would leave at most half its width behind takes
  // the rest too (gamma = 8: [0,1), [1,3), [3,9)), which saves a stage's two
  // launches for a few extra rows.  Blocks stay within one wavefront (<= 48
  // positions).  A row workgroup of a sequence that is already done exits at
  // once.
  int32_t *status = reinterpret_cast<int32_t *>(wsb + L.status_off);
  for (int lo = 0, width = 1; lo <= gamma; lo += width, width *= 2) {
    int hi = std::min(gamma + 1, lo + width);
    if (gamma + 1 - hi <= width / 2) hi = gamma + 1;
    width = hi - lo;
    RowSet st = rs;
    st.add_target(lo, hi);
    st.add_draft(lo, std::min(hi, static_cast<int>(gamma)));
    st.status = lo == 0 ? nullptr : status;
    st.arrive = lo == 0 ? ds.arrive : nullptr;  // every sequence has workgroups in the first block
    launch_row_stats(dtype, false, st, part, stream);
    if (hi <= gamma) {
      launch_stage_decide(dtype, A, B, lo, hi, status, stream);
    } else {  // the last block is decided inside the draw
      WindowArgs Af = A;
      Af.stage_lo = lo;
      Af.status = status;
      launch_stage_finish(dtype, Af, B, ds, stream);
    }
  }
  return launch_status();
}

}  // namespace

extern "C" {

int sv_verify_window(const void *target_logits, int64_t target_seq_stride,
                     const void *draft_logits, int64_t draft_seq_stride, int dtype,
                     const int32_t *draft_tokens, const int32_t *window_len,
                     int32_t B, int32_t gamma, int32_t V,
                     uint64_t seed, uint64_t tag, const uint64_t *seq_ids,
                     const int64_t *base_pos,
                     int32_t *n_accepted, int32_t *out_tokens,
                     float *p_draft, float *q_draft,
                     void *workspace, size_t workspace_bytes, hipStream_t stream) {
  return window_impl(kPartRows | kPartFinish, target_logits, target_seq_stride, draft_logits, draft_seq_stride, dtype,
                     draft_tokens, window_len, B, gamma, V, seed, tag, seq_ids, base_pos,
                     n_accepted, out_tokens, p_draft, q_draft, workspace, workspace_bytes, stream);
}

int sv_verify_window_early_exit(const void *target_logits, int64_t target_seq_stride,
                                const void *draft_logits, int64_t draft_seq_stride, int dtype,
                                const int32_t *draft_tokens, const int32_t *window_len,
                                int32_t B, int32_t gamma, int32_t V,
                                uint64_t seed, uint64_t tag, const uint64_t *seq_ids,
                                const int64_t *base_pos,
                                int32_t *n_accepted, int32_t *out_tokens,
                                float *p_draft, float *q_draft,
                                void *workspace, size_t workspace_bytes, hipStream_t stream) {
  return window_impl(kEarlyExit, target_logits, target_seq_stride, draft_logits, draft_seq_stride, dtype,
                     draft_tokens, window_len, B, gamma, V, seed, tag, seq_ids, base_pos, n_accepted,
                     out_tokens, p_draft, q_draft, workspace, workspace_bytes, stream);
}

int sv_verify_window_part(int part, const void *target_logits, int64_t target_seq_stride,
                          const void *draft_logits, int64_t draft_seq_stride, int dtype,
                          const int32_t *draft_tokens, const int32_t *window_len,
                          int32_t B, int32_t gamma, int32_t V,
                          uint64_t seed, uint64_t tag, const uint64_t *seq_ids,
                          const int64_t *base_pos,
                          int32_t *n_accepted, int32_t *out_tokens,
                          float *p_draft, float *q_draft,
                          void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (part != SV_PART_ROW_STATS && part != SV_PART_DECIDE_SAMPLE) return SV_EINVAL;
  return window_impl(part == SV_PART_ROW_STATS ? kPartRows : kPartFinish, target_logits, target_seq_stride,
                     draft_logits, draft_seq_stride, dtype, draft_tokens, window_len, B, gamma, V,
                     seed, tag, seq_ids, base_pos, n_accepted, out_tokens, p_draft, q_draft,
                     workspace, workspace_bytes, stream);
}

int sv_verify_greedy(const void *target_logits, int64_t target_seq_stride, int dtype,
                     const int32_t *draft_tokens, const int32_t *window_len,
                     int32_t B, int32_t gamma, int32_t V,
                     int32_t *n_accepted, int32_t *out_tokens,
                     void *workspace, size_t workspace_bytes, hipStream_t stream) {
  const int eb = elem_bytes(dtype);
  if (eb == 0) return SV_EDTYPE;
  if (B < 1 || gamma < 1 || gamma > SV_MAX_GAMMA || V < 1 || V > kMaxVocab) return SV_EINVAL;
  if (!target_logits || !draft_tokens || !n_accepted || !out_tokens) return SV_EINVAL;
  if (!aligned(target_logits, eb)) return SV_EINVAL;
  const int64_t t_rows = static_cast<int64_t>(gamma + 1) * V;
  if (target_seq_stride == 0) target_seq_stride = t_rows;
  if (target_seq_stride < t_rows) return SV_EINVAL;
  const Layout L = make_layout(SV_OP_GREEDY, B, gamma, V);
  if (!rows_fit(B, L) || !grid_fits(B, kWaveThreads)) return SV_EINVAL;
  const int ws = check_workspace(workspace, workspace_bytes, L.total);
  if (ws != SV_OK) return ws;
  float2 *part = reinterpret_cast<float2 *>(static_cast<char *>(workspace) + L.part_off);

  RowSet rs{};
  rs.t = static_cast<const char *>(target_logits);
  rs.t_stride_bytes = target_seq_stride * eb;
  rs.d = nullptr;
  rs.B = B;
  rs.R_out = gamma + 1;
  rs.d_slot0 = gamma + 1;
  rs.window_len = window_len;
  rs.status = nullptr;
  rs.gamma = gamma;
  rs.V = V;
  rs.S = L.plan.S;
  rs.seg_len = L.plan.seg_len;
  rs.add_target(0, gamma + 1);
  launch_row_stats(dtype, true, rs, part, stream);

  GreedyArgs A{};
  A.tokens = draft_tokens;
  A.window_len = window_len;
  A.gamma = gamma;
  A.V = V;
  A.S = L.plan.S;
  A.part = part;
  A.n_accepted = n_accepted;
  A.out_tokens = out_tokens;
  launch_greedy_decide(A, B, stream);
  return launch_status();
}

int32_t sv_tree_max_depth(const int32_t *parent_host, int32_t N) {
  TreeMeta meta;
  const int st = build_tree(parent_host, N, &meta);
  return st == SV_OK ? meta.max_depth : st;
}

int sv_verify_tree(const void *target_logits, const void *draft_logits, int dtype,
                   const int32_t *node_tokens, const int32_t *parent_host,
                   int32_t B, int32_t N, int32_t V, int mode,
                   uint64_t seed, uint64_t tag, const uint64_t *seq_ids,
                   const int64_t *base_pos,
                   int32_t *n_accepted, int32_t *best_node,
                   int32_t *out_tokens, int32_t *out_nodes,
                   void *workspace, size_t workspace_bytes, hipStream_t stream) {
  const int eb = elem_bytes(dtype);
  if (eb == 0) return SV_EDTYPE;
  if (B < 1 || V < 1 || V > kMaxVocab) return SV_EINVAL;
  if (mode != SV_TREE_GREEDY && mode != SV_TREE_STOCHASTIC && mode != SV_TREE_MULTI_CANDIDATE) return SV_EINVAL;
  const bool sampled = mode != SV_TREE_GREEDY;
  TreeMeta meta;
  const int tst = build_tree(parent_host, N, &meta);
  if (tst != SV_OK) return tst;
  if (!target_logits || !node_tokens || !n_accepted || !best_node || !out_tokens) return SV_EINVAL;
  if (meta.max_depth > 0 && !out_nodes) return SV_EINVAL;
  if (sampled && !draft_logits) return SV_EINVAL;
  if (!aligned(target_logits, eb) || (draft_logits && !aligned(draft_logits, eb))) return SV_EINVAL;
  const Layout L = make_layout(SV_OP_TREE, B, N, V);
  if (!rows_fit(B, L) || !grid_fits(B, sampled ? kFinThreads : kTreeMaxNodes)) return SV_EINVAL;
  const int ws = check_workspace(workspace, workspace_bytes, L.total);
  if (ws != SV_OK) return ws;
  char *wsb = static_cast<char *>(workspace);
  float2 *part = reinterpret_cast<float2 *>(wsb + L.part_off);
  SampleJob *jobs = reinterpret_cast<SampleJob *>(wsb + L.jobs_off);

  const int64_t seq_bytes = static_cast<int64_t>(N) * V * eb;
  const DrawScratch ds{reinterpret_cast<float *>(wsb + L.spart_off), L.cmax,
                       reinterpret_cast<int32_t *>(wsb + L.arrive_off)};
  RowSet rs{};
  rs.t = static_cast<const char *>(target_logits);
  rs.t_stride_bytes = seq_bytes;
  rs.arrive = ds.arrive;
  rs.d = static_cast<const char *>(draft_logits);
  rs.d_stride_bytes = seq_bytes;
  rs.B = B;
  rs.R_out = 2 * N;
  rs.d_slot0 = N;
  rs.window_len = nullptr;
  rs.status = nullptr;
  rs.gamma = 0;
  rs.V = V;
  rs.S = L.plan.S;
  rs.seg_len = L.plan.seg_len;
  // Row results are laid out for 2N rows per sequence (draft row v at slot
  // N + v); only the rows the decision reads are listed: every target row,
  // and, when sampling, the draft rows of nodes with children.
  rs.add_target(0, N);
  if (sampled)
    for (int v = 0; v < N; ++v)
      if ((meta.internal[v >> 6] >> (v & 63)) & 1ull) rs.add_draft(v, v + 1);
  launch_row_stats(dtype, !sampled, rs, part, stream);
  const int R = 2 * N;

  TreeArgs A{};
  A.t = rs.t;
  A.d = rs.d;
  A.seq_bytes = seq_bytes;
  A.tokens = node_tokens;
  A.V = V;
  A.S = L.plan.S;
  A.R = R;
  A.mode = sampled ? 1 : 0;
  A.seed = seed;
  A.tag = tag;
  A.seq_ids = seq_ids;
  A.base_pos = base_pos;
  A.part = part;
  A.n_accepted = n_accepted;
  A.best_node = best_node;
  A.out_tokens = out_tokens;
  A.out_nodes = out_nodes;
  A.jobs = jobs;
  A.meta = meta;
  if (mode == SV_TREE_MULTI_CANDIDATE) {
    launch_tree_walk(dtype, A, B, stream);
    return launch_status();
  }
  if (mode == SV_TREE_STOCHASTIC)
    launch_tree_decide_draw(dtype, A, B, ds, stream);
  else
    launch_tree_decide(dtype, A, B, stream);
  return launch_status();
}

int sv_rollback(int32_t *buf_tokens, int32_t *buf_len, int32_t S, int32_t K,
                int32_t cap, int32_t stage,
                const int32_t *verified_tokens, int64_t verified_stride,
                const int32_t *verified_len, int32_t len_offset,
                hipStream_t stream) {
  if (S < 1 || K < 2 || cap < 1 || stage < 1 || stage >= K) return SV_EINVAL;
  if (stage > 65535) return SV_EINVAL;
  if (!buf_tokens || !buf_len || !verified_tokens || !verified_len) return SV_EINVAL;
  if (verified_stride < 0) return SV_EINVAL;
  if (!grid_fits(S, kWaveThreads)) return SV_EINVAL;
  RollbackArgs A{};
  A.buf_tokens = buf_tokens;
  A.buf_len = buf_len;
  A.K = K;
  A.cap = cap;
  A.verified = verified_tokens;
  A.verified_stride = verified_stride;
  A.verified_len = verified_len;
  A.len_offset = len_offset;
  launch_rollback(A, S, stage, stream);
  return launch_status();
}

int32_t sv_probe_blocks(size_t bytes) { return probe_blocks(bytes); }

int sv_probe_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream) {
  if (!src || !sink || bytes < 16 || bytes % 16 != 0 || bytes > (size_t(1) << 40) || !aligned(src, 16))
    return SV_EINVAL;
  launch_probe_read(src, bytes, sink, stream);
  return launch_status();
}

int sv_verify_window_lmhead(const void *hidden_target, const void *unembed_target, int32_t Ht,
                            const void *hidden_draft, const void *unembed_draft, int32_t Hd,
                            const int32_t *draft_tokens, const int32_t *window_len,
                            int32_t B, int32_t gamma, int32_t V,
                            uint64_t seed, uint64_t tag, const uint64_t *seq_ids,
                            const int64_t *base_pos,
                            int32_t *n_accepted, int32_t *out_tokens,
                            float *p_draft, float *q_draft,
                            void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (B < 1 || gamma < 1 || gamma > SV_MAX_GAMMA || V < 1 || V > kMaxVocab) return SV_EINVAL;
  if (Ht < SV_LMHEAD_K_STEP || Hd < SV_LMHEAD_K_STEP || Ht % SV_LMHEAD_K_STEP || Hd % SV_LMHEAD_K_STEP ||
      Ht > SV_LMHEAD_MAX_HIDDEN || Hd > SV_LMHEAD_MAX_HIDDEN)
    return SV_EINVAL;
  if (!hidden_target || !unembed_target || !hidden_draft || !unembed_draft || !draft_tokens || !n_accepted ||
      !out_tokens)
    return SV_EINVAL;
  if (!aligned(hidden_target, 16) || !aligned(unembed_target, 16) || !aligned(hidden_draft, 16) ||
      !aligned(unembed_draft, 16))
    return SV_EINVAL;
  const int64_t Mt = static_cast<int64_t>(B) * (gamma + 1), Md = static_cast<int64_t>(B) * gamma;
  // grids: the GEMM (both problems), the combine (four rows per workgroup of
  // 256), the decision (one wave per sequence) and the draw (1024 threads per
  // sequence)
  if (Mt + Md > (int64_t{1} << 30) || !grid_fits(lm_gemm_blocks(Mt, V) + lm_gemm_blocks(Md, V), kLmGemmThreads) ||
      !grid_fits((Mt + Md + 3) / 4, 256) || !grid_fits(B, kFinThreads))
    return SV_EINVAL;
  const LmLayout L = make_lm_layout(B, gamma, V);
  const int ws = check_workspace(workspace, workspace_bytes, L.total);
  if (ws != SV_OK) return ws;
  char *wsb = static_cast<char *>(workspace);
  float2 *part = reinterpret_cast<float2 *>(wsb + L.part_off);
  float2 *stats = reinterpret_cast<float2 *>(wsb + L.stats_off);
  float *gath = reinterpret_cast<float *>(wsb + L.gath_off);
  SampleJob *jobs = reinterpret_cast<SampleJob *>(wsb + L.jobs_off);
  const DrawScratch ds{reinterpret_cast<float *>(wsb + L.spart_off), L.cmax,
                       reinterpret_cast<int32_t *>(wsb + L.arrive_off)};
  float *rows_t = reinterpret_cast<float *>(wsb + L.rows_t_off);
  float *rows_d = reinterpret_cast<float *>(wsb + L.rows_d_off);

  // every target and draft row: float32 logits, statistics and the draft-token logits
  LmGemmArgs G{};
  G.A = static_cast<const uint16_t *>(hidden_target);
  G.lda = Ht;
  G.W = static_cast<const uint16_t *>(unembed_target);
  G.M = static_cast<int32_t>(Mt);
  G.V = V;
  G.K = Ht;
  G.part = part;
  G.gath = gath;
  G.tokens = draft_tokens;
  G.gamma = gamma;
  G.rows_per_seq = gamma + 1;
  G.out = rows_t;
  LmGemmArgs Gd = G;
  Gd.A = static_cast<const uint16_t *>(hidden_draft);
  Gd.lda = Hd;
  Gd.W = static_cast<const uint16_t *>(unembed_draft);
  Gd.M = static_cast<int32_t>(Md);
  Gd.K = Hd;
  Gd.part = part + Mt * L.NT;
  Gd.gath = gath + Mt;
  Gd.rows_per_seq = gamma;
  Gd.out = rows_d;
  launch_lm_gemm(G, Gd, stream);
  launch_lm_combine(part, L.NT, static_cast<int>(Mt + Md), stats, stream);

  LmDecideArgs D{};
  D.stats_t = stats;
  D.stats_d = stats + Mt;
  D.gath_t = gath;
  D.gath_d = gath + Mt;
  D.tokens = draft_tokens;
  D.window_len = window_len;
  D.gamma = gamma;
  D.V = V;
  D.seed = seed;
  D.tag = tag;
  D.seq_ids = seq_ids;
  D.base_pos = base_pos;
  D.n_accepted = n_accepted;
  D.out_tokens = out_tokens;
  D.p_draft = p_draft;
  D.q_draft = q_draft;
  D.jobs = jobs;
  D.rows_t = rows_t;
  D.rows_d = rows_d;
  D.arrive = ds.arrive;
  launch_lm_decide(D, B, stream);

  launch_tree_finish(SV_DT_F32, jobs, B, V, ds, stream);
  return launch_status();
}

}  // extern "C"
