/*
 * sv.h -- C ABI of the speculative-decoding verification library (libspecverify.so)
 *
 * What is computed (sources by page title and section):
 *   - Speculative-sampling verification of a window of gamma draft tokens: the
 *     rule the CLaSp review page cites as lossless ("Assumptions & free
 *     parameters") and the PipeSpec review page cites through the Leviathan et
 *     al. expected-token formula ("Assumptions & free parameters").  Draft i is
 *     accepted when u_i < min(1, p_i(x_i) / q_i(x_i)); the scan stops at the
 *     first rejection; the replacement token is drawn from the renormalised
 *     max(0, p_n - q_n), or, after a full window, a bonus token from p_len.
 *   - Greedy verification: keep the longest prefix of drafts equal to the
 *     target's argmax predictions and emit the argmax of the first unmatched
 *     row (PipeSpec review, "What carries the argument").
 *   - Verification of a tree-shaped speculative batch ("Accelerating LLM
 *     Inference with Staged Speculative Decoding", abstract).
 *   - Rollback of earlier stages' token buffers to the last verified token
 *     (PipeSpec review, "What carries the argument").
 *
 * Conventions shared by every call
 *   - Every pointer is caller-owned DEVICE memory unless its comment says HOST.
 *     The library allocates nothing and keeps no pointer after returning.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *     Nothing synchronises; outputs are valid once the stream reaches them.
 *   - Logits: dtype SV_DT_F32 / SV_DT_BF16 / SV_DT_F16, rows of V contiguous
 *     elements.  Rows of one sequence are contiguous; consecutive sequences
 *     are `*_seq_stride` ELEMENTS apart (0 = dense).  Pointers must be aligned
 *     to the element size.  Logits must be finite or -inf with at least one
 *     finite value per row; otherwise results are unspecified (no fault).
 *     Logits are used as given (temperature 1; greedy is temperature 0).
 *   - Uniforms: Philox4x64-10 with key (seed, tag) and counter
 *     (seq_id, pos, rank, 0); word 0 -> accept uniform, word 1 -> sampling
 *     uniform, each (word >> 40) * 2^-24.  seq_ids[b] (NULL => b) names the
 *     sequence; base_pos[b] (NULL => 0) is the absolute position of the last
 *     committed token, so draft i of a window sits at pos base_pos + 1 + i and
 *     a tree node at base_pos + depth; rank is a tree node's index among the
 *     nodes of its depth (0 for windows).  `tag` separates the stages of a
 *     hierarchy.
 *   - Host-detectable errors return a negative sv_status and enqueue nothing.
 *     Among them: sizes whose launches would not fit a dispatch, which counts
 *     each grid dimension in 32-bit work-items (SV_EINVAL).  The row pass
 *     takes 256 work-items per row segment, and rows are split into segments
 *     only while a launch has fewer than 16,384 rows, so B times the rows per
 *     sequence must stay below 2^24; calls that draw take 1024 work-items per
 *     sequence, so B <= 4,194,303.
 *     Per-sequence data errors (a token outside [0, V), a window_len outside
 *     [0, gamma]) are found on the device and mark that sequence with
 *     n_accepted[b] = -1 and an all -1 row of out_tokens.  A launch failure
 *     returns SV_ELAUNCH.  Nothing aborts or throws across this ABI.
 *   - Results are bitwise deterministic for identical inputs (fixed reduction
 *     order, no floating-point atomics).  Calls are reentrant; overlapping calls
 *     must not share a workspace.
 */
#ifndef SPECVERIFY_SV_H
#define SPECVERIFY_SV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SV_DT_F32 = 0, SV_DT_BF16 = 1, SV_DT_F16 = 2 } sv_dtype;

typedef enum {
  SV_OK = 0,
  SV_EINVAL = -1,     /* bad size, null required pointer, misaligned pointer   */
  SV_EDTYPE = -2,     /* unknown dtype                                         */
  SV_EWORKSPACE = -3, /* workspace missing, misaligned (256 B) or too small    */
  SV_ETREE = -4,      /* malformed parent array, too many nodes or too deep    */
  SV_ELAUNCH = -5,    /* a kernel launch failed                                */
  SV_ESCRATCH = -6    /* the call needs more than SV_SCRATCH_BYTES of scratch  */
} sv_status;

typedef enum { SV_OP_WINDOW = 0, SV_OP_GREEDY = 1, SV_OP_TREE = 2, SV_OP_LMHEAD = 3 } sv_op;

typedef enum { SV_TREE_GREEDY = 0, SV_TREE_STOCHASTIC = 1, SV_TREE_MULTI_CANDIDATE = 2 } sv_tree_mode;

#define SV_MAX_GAMMA 64
#define SV_TREE_MAX_NODES 256
#define SV_LMHEAD_K_STEP 64
#define SV_LMHEAD_MAX_HIDDEN 65536
#define SV_TREE_MAX_DEPTH 64
/* Device scratch of sv_verify_window_noalloc, per GPU (8 MiB). */
#define SV_SCRATCH_BYTES (8u << 20)

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int sv_version(void);

/* Static, human-readable text of a sv_status value. */
const char *sv_strerror(int status);

/* Bytes of device workspace the call `op` needs for B sequences with
 * n = gamma (window, greedy) or n = N tree nodes (tree), vocabulary V and
 * dtype.  Returns 0 for invalid arguments.  The workspace must be 256-byte
 * aligned; its contents on entry do not matter. */
size_t sv_workspace_size(int op, int32_t B, int32_t n, int32_t V, int dtype);

/* Stochastic window verification (speculative sampling).
 *   target_logits [B][gamma+1][V]: row i = target next-token logits after the
 *                 context extended by drafts 0..i-1; row gamma is the bonus row.
 *   draft_logits  [B][gamma][V]: the draft distribution each draft was drawn from.
 *   draft_tokens  [B][gamma] int32.
 *   window_len    [B] int32 in [0, gamma], drafts to verify per sequence, or
 *                 NULL (= gamma).  Rows past a sequence's window are not read.
 *   1 <= gamma <= SV_MAX_GAMMA, B >= 1, V >= 1.
 * Outputs:
 *   n_accepted [B]: accepted drafts n (or -1, see conventions).
 *   out_tokens [B][gamma+1]: drafts 0..n-1, then the corrected token (n < len)
 *              or the bonus token (n = len), then -1.
 *   p_draft, q_draft [B][gamma] float or NULL: p_i(x_i), q_i(x_i) for
 *              i < window_len (0 past it); meaningful for i <= n. */
int sv_verify_window(const void *target_logits, int64_t target_seq_stride,
                     const void *draft_logits, int64_t draft_seq_stride, int dtype,
                     const int32_t *draft_tokens, const int32_t *window_len,
                     int32_t B, int32_t gamma, int32_t V,
                     uint64_t seed, uint64_t tag, const uint64_t *seq_ids,
                     const int64_t *base_pos,
                     int32_t *n_accepted, int32_t *out_tokens,
                     float *p_draft, float *q_draft,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/* sv_verify_window for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, rule and outputs as sv_verify_window (bit-identical), minus
 * the workspace: the library keeps one SV_SCRATCH_BYTES device array per GPU
 * (a static device variable, held until the process ends) and uses it as the
 * workspace.  Its address is looked up once per device, on the first call
 * with that device current; the call allocates nothing.
 *   Limit: sv_workspace_size(SV_OP_WINDOW, B, gamma, V, dtype) must not
 *   exceed SV_SCRATCH_BYTES (B = 256, gamma = 8, V = 128256 needs 156 KiB);
 *   larger calls return SV_ESCRATCH and enqueue nothing.
 *   Every call on one GPU shares that array and no state survives between
 *   calls, so calls that overlap on one GPU (different streams, or host
 *   threads) race and must be serialised by the caller; calls in one stream
 *   are ordered.  Argument errors (SV_EDTYPE, SV_EINVAL) are reported first,
 *   then SV_ESCRATCH; SV_ELAUNCH if the array's address cannot be obtained. */
int sv_verify_window_noalloc(const void *target_logits, int64_t target_seq_stride,
                             const void *draft_logits, int64_t draft_seq_stride, int dtype,
                             const int32_t *draft_tokens, const int32_t *window_len,
                             int32_t B, int32_t gamma, int32_t V,
                             uint64_t seed, uint64_t tag, const uint64_t *seq_ids,
                             const int64_t *base_pos,
                             int32_t *n_accepted, int32_t *out_tokens,
                             float *p_draft, float *q_draft, hipStream_t stream);

/* sv_verify_window in two halves on the same workspace and arguments:
 *   part SV_PART_ROW_STATS     -- the streaming pass over every needed logits
 *                                 row (the call's HBM traffic);
 *   part SV_PART_DECIDE_SAMPLE -- accept decisions, first rejection and the
 *                                 residual / bonus draw.
 * Running ROW_STATS then DECIDE_SAMPLE on one stream equals one
 * sv_verify_window call bit for bit.  Lets a caller overlap the streaming pass
 * with other work or time it on its own.  DECIDE_SAMPLE reads what ROW_STATS
 * left in the workspace (row results, and the draw's zeroed arrival counters),
 * so it must follow a ROW_STATS on the same workspace and arguments; it may be
 * repeated after one. */
#define SV_PART_ROW_STATS 1
#define SV_PART_DECIDE_SAMPLE 2
int sv_verify_window_part(int part, const void *target_logits, int64_t target_seq_stride,
                          const void *draft_logits, int64_t draft_seq_stride, int dtype,
                          const int32_t *draft_tokens, const int32_t *window_len,
                          int32_t B, int32_t gamma, int32_t V,
                          uint64_t seed, uint64_t tag, const uint64_t *seq_ids,
                          const int64_t *base_pos,
                          int32_t *n_accepted, int32_t *out_tokens,
                          float *p_draft, float *q_draft,
                          void *workspace, size_t workspace_bytes, hipStream_t stream);

/* sv_verify_window that stops reading a sequence's rows at its first
 * rejection ("the scan stops at the first rejection"): target and draft rows
 * are reduced in position blocks of doubling width [0,1), [1,3), [3,7), ...,
 * where a block that would leave at most half its width behind takes the rest
 * (gamma = 8: [0,1), [1,3), [3,9)), each block followed by a decision; a
 * sequence that has rejected a draft (or used up its window) reads no further
 * rows.  Same arguments and workspace (SV_OP_WINDOW) as sv_verify_window;
 * n_accepted and out_tokens are bit-identical to it, as are p_draft/q_draft
 * for i <= n (they are 0 past n).  The row bytes read shrink from
 * B(2 gamma + 1)V to about B(2 E[n] + 2)V at the cost of 2 launches per block
 * (3 blocks at gamma = 8). */
int sv_verify_window_early_exit(const void *target_logits, int64_t target_seq_stride,
                                const void *draft_logits, int64_t draft_seq_stride, int dtype,
                                const int32_t *draft_tokens, const int32_t *window_len,
                                int32_t B, int32_t gamma, int32_t V,
                                uint64_t seed, uint64_t tag, const uint64_t *seq_ids,
                                const int64_t *base_pos,
                                int32_t *n_accepted, int32_t *out_tokens,
                                float *p_draft, float *q_draft,
                                void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Greedy window verification (temperature 0).  Same layouts as
 * sv_verify_window; only target rows 0..window_len are read.  n is the first
 * i < len with draft_tokens[i] != argmax(row i) (smallest index among equal
 * maxima; -0 equals +0), else len; out_tokens = drafts 0..n-1, argmax(row n),
 * then -1.  Bit-exact. */
int sv_verify_greedy(const void *target_logits, int64_t target_seq_stride, int dtype,
                     const int32_t *draft_tokens, const int32_t *window_len,
                     int32_t B, int32_t gamma, int32_t V,
                     int32_t *n_accepted, int32_t *out_tokens,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Depth of the deepest node of a tree given by HOST parent indices
 * (parent[0] = -1, 0 <= parent[v] < v), or SV_ETREE. */
int32_t sv_tree_max_depth(const int32_t *parent_host, int32_t N);

/* Token-tree verification.
 *   target_logits [B][N][V]: row v = target next-token logits after node v.
 *   draft_logits  [B][N][V]: row v = the draft distribution v's children were
 *                 drawn from; may be NULL in greedy mode; leaf rows are not read.
 *   node_tokens   [B][N] int32: token of node v (entry 0, the root, ignored).
 *   parent_host   HOST [N]: parent[0] = -1, 0 <= parent[v] < v (BFS or any
 *                 topological order); N <= SV_TREE_MAX_NODES, depth <=
 *                 SV_TREE_MAX_DEPTH; read during the call only.
 *   mode: SV_TREE_GREEDY, SV_TREE_STOCHASTIC or SV_TREE_MULTI_CANDIDATE.
 * GREEDY / STOCHASTIC: node v >= 1 is accepted when its parent is accepted
 * and its token passes the test against the parent's row (argmax equality, or
 * u_v q_w < p_w).  The deepest accepted node d (smallest index among equals)
 * ends the path.  With more than one child per node the STOCHASTIC rule does
 * not keep the target distribution.
 * MULTI_CANDIDATE: the multi-round scheme of SpecInfer (cited by title on the
 * PipeSpec and CLaSp review pages), which keeps the target distribution when
 * siblings are i.i.d. draws from their parent's draft row.  From the root,
 * the children of the current node w are tried in index order against a
 * residual r that starts at p_w: child v (token x) is accepted when
 * u_v q_w(x) < r(x); after a rejection r becomes the renormalised
 * max(0, r - q_w) (kept as it is if that has no mass).  An accepted child
 * becomes w; the walk ends at a leaf (bonus draw from p_w) or at a node whose
 * children were all rejected (draw from r).  d is the final node.  One
 * 1024-thread workgroup per sequence makes one pass over rows w of both
 * logits per rejection.
 * Uniforms: node v's test uses word 0 at (base_pos + depth(v), rank(v)); the
 * token drawn after d uses word 1 at (base_pos + depth(d) + 1, rank(d)).
 * Outputs (D = sv_tree_max_depth):
 *   n_accepted [B] = depth(d) (or -1); best_node [B] = d;
 *   out_tokens [B][D+1]: path tokens, then argmax(row d) (greedy), a bonus
 *              draw from p_d (d a leaf) or a draw from the residual at d,
 *              then -1;
 *   out_nodes  [B][D]: path node ids, then -1. */
int sv_verify_tree(const void *target_logits, const void *draft_logits, int dtype,
                   const int32_t *node_tokens, const int32_t *parent_host,
                   int32_t B, int32_t N, int32_t V, int mode,
                   uint64_t seed, uint64_t tag, const uint64_t *seq_ids,
                   const int64_t *base_pos,
                   int32_t *n_accepted, int32_t *best_node,
                   int32_t *out_tokens, int32_t *out_nodes,
                   void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Rollback of per-stage token buffers to a verified sequence.
 *   buf_tokens [S][K][cap] int32, buf_len [S][K] int32 (in/out).
 *   verified_tokens: stream s's verified sequence starts at
 *                 verified_tokens + s * verified_stride (int32 elements);
 *   verified_len [S]: its length is verified_len[s] + len_offset
 *                 (len_offset = 1 lets n_accepted of a verify call be passed);
 *                 the caller provides at least that many tokens per sequence
 *                 (a length in [0, cap] is read; the library cannot check the
 *                 width of the verified rows).
 *   stage in [1, K-1]: buffers 0..stage-1 are rolled back, others untouched.
 * For each j < stage with L the verified length: m = first t < min(len_j, L)
 * where buffer j differs from the verified sequence, else min(len_j, L); if
 * m < L the buffer's slots m..L-1 get the verified tokens and len_j = L,
 * otherwise the buffer (already holding the verified prefix) is kept.
 * A length outside [0, cap] (verified or buffer) leaves that buffer's tokens
 * untouched and sets its buf_len to -1.  The verified sequence must not
 * overlap a buffer being rolled back.  Bit-exact. */
int sv_rollback(int32_t *buf_tokens, int32_t *buf_len, int32_t S, int32_t K,
                int32_t cap, int32_t stage,
                const int32_t *verified_tokens, int64_t verified_stride,
                const int32_t *verified_len, int32_t len_offset,
                hipStream_t stream);

/* Diagnostic: stream `bytes` (a multiple of 16, 16-byte aligned, at most
 * 2^40) of device memory through the same nontemporal 16-byte loads the row
 * pass uses, one contiguous 256 KiB chunk per workgroup, and write one 32-bit
 * checksum per workgroup to `sink` [sv_probe_blocks(bytes)]; measures the read
 * bandwidth ceiling of the running GPU. */
int32_t sv_probe_blocks(size_t bytes);
int sv_probe_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);

/* Speculative-sampling window on logits produced from hidden states, with
 * the LM head fused into the verification: the same rule and outputs as
 * sv_verify_window, where the logits are
 *   target row i of sequence b = hidden_target[b][i] . unembed_target[k] for k < V,
 *   draft  row i of sequence b = hidden_draft[b][i]  . unembed_draft[k],
 * dot products of bf16 values accumulated in float32 on the matrix cores.
 * Each GEMM tile feeds the row statistics and the logits at the draft tokens
 * directly, so no pass reads the logits back to reduce them; the same tiles
 * write the float32 logits to the workspace, and the draw reads only target
 * row n and draft row n of each sequence there.  This is an extension beyond
 * the pages, which only say that draft and target models produce the
 * distributions.
 *   hidden_target [B][gamma+1][Ht] bf16, unembed_target [V][Ht] bf16,
 *   hidden_draft  [B][gamma][Hd]   bf16, unembed_draft  [V][Hd] bf16; dense,
 *   16-byte aligned; Ht, Hd multiples of SV_LMHEAD_K_STEP, at most
 *   SV_LMHEAD_MAX_HIDDEN.
 *   Other arguments and outputs as sv_verify_window; workspace of
 *   sv_workspace_size(SV_OP_LMHEAD, B, gamma, V, SV_DT_BF16) bytes (it holds
 *   the 2 gamma + 1 float32 logit rows of every sequence: 2.25 GB at B = 256,
 *   gamma = 8, V = 128256).
 * Errors: as sv_verify_window; SV_EINVAL for hidden sizes outside the rules. */
int sv_verify_window_lmhead(const void *hidden_target, const void *unembed_target, int32_t Ht,
                            const void *hidden_draft, const void *unembed_draft, int32_t Hd,
                            const int32_t *draft_tokens, const int32_t *window_len,
                            int32_t B, int32_t gamma, int32_t V,
                            uint64_t seed, uint64_t tag, const uint64_t *seq_ids,
                            const int64_t *base_pos,
                            int32_t *n_accepted, int32_t *out_tokens,
                            float *p_draft, float *q_draft,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_SV_H */
