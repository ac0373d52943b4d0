// HIP kernels of the verification library (gfx950), after the row
// statistics (sv_rows.hip):
//
// Decide: one wavefront (or one workgroup for trees) per sequence combines the
//   segment results, forms p(x) and q(x) at the draft tokens, draws the Philox
//   uniforms and finds the first rejection with a wavefront ballot --
//   window_decide (in wave 0 of the draw), k_stage_decide (early exit, one
//   block of positions), k_greedy_decide, k_tree_decide.
// Sampling (k_finish, one 1024-thread workgroup per sequence; k_finish_part,
//   several per sequence, for small batches): the one extra pass over the row
//   of the first rejection (or the bonus row) keeps chunk sums of the weights,
//   then searches the chunk holding tau = v * Z.  The job comes from the window
//   decision, from the last early-exit block's decision, or from the jobs array.
// k_tree_walk: the lossless multi-candidate tree walk, one workgroup per
//   sequence, one sampling pass per rejected sibling.
// Rollback, k_rollback: first divergence by ballot, then copy of the
//   verified tail.
#include <climits>

#include "sv_device.h"
#include "sv_launch.h"
#include "sv_plan.h"

namespace sv {

// Sum of v over the wave, valid in every lane, in a fixed order: within each
// row of 16 lanes by DPP moves (swap neighbours, swap pairs, rotate by 4, by
// 8), then the four row sums read from lanes 0, 16, 32 and 48 and added in
// that order.  Every lane must be active.  The DPP moves and lane reads cost a
// few cycles each, where a butterfly of lane shuffles goes through LDS six
// times; that latency sits on the critical path of the latency-bound draws.
template <int kCtrl>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, true));
}
__device__ __forceinline__ float lane_value(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}
__device__ __forceinline__ float wave_total(float v) {
  v += dpp_move<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_move<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_move<0x124>(v);  // row_ror 4
  v += dpp_move<0x128>(v);  // row_ror 8
  return ((lane_value(v, 0) + lane_value(v, 16)) + lane_value(v, 32)) + lane_value(v, 48);
}

// Inclusive prefix sum over the wave in lane order, every lane active: within
// rows of 16 lanes by DPP row shifts by 1, 2, 4 and 8 (a lane shifted in from
// outside its row reads 0), then the rows after the first add the running
// total of the rows before them: lane 15 of rows 0 and 2 into rows 1 and 3,
// then lane 31 into rows 2 and 3.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_rows(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, kRowMask, 0xF, false));
}
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  x += dpp_move<0x111>(x);    // row_shr 1
  x += dpp_move<0x112>(x);    // row_shr 2
  x += dpp_move<0x114>(x);    // row_shr 4
  x += dpp_move<0x118>(x);    // row_shr 8
  x += dpp_rows<0x142, 0xA>(x);  // row_bcast 15, into rows 1 and 3
  x += dpp_rows<0x143, 0xC>(x);  // row_bcast 31, into rows 2 and 3
  return x;
}
// The value of lane l - 1 in lane l, 0 in lane 0 (DPP wave_shr 1).
__device__ __forceinline__ float wave_shift_up1(float x) { return dpp_move<0x138>(x); }

// Largest int over the wave, read from lane 0 (every lane active): DPP within
// rows of 16 lanes, then the four row maxima.
template <int kCtrl>
__device__ __forceinline__ int dpp_move_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, kCtrl, 0xF, 0xF, true);
}
__device__ __forceinline__ int wave_max_int(int v) {
  v = max(v, dpp_move_i<0xB1>(v));
  v = max(v, dpp_move_i<0x4E>(v));
  v = max(v, dpp_move_i<0x124>(v));
  v = max(v, dpp_move_i<0x128>(v));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Residual mass max(0, p - cq q) below which a draw counts it as none and
// draws from p.  Weights are formed as 2^(x log2e - c) with offsets c of
// magnitude ~10-60 rounded to float32, so two rows holding the same logits
// can differ by ~1e-6 in every weight when their offsets round differently
// (the row pass reduces rows at different 16-byte alignments in different
// orders); mass below 2^-16 cannot be told apart from that rounding.
constexpr float kNoResidualMass = 0x1p-16f;

// Combine the S segment results of one row, in segment order.  The loads go
// out kSegBatch at a time ahead of their combines, so a row costs
// ceil(S / kSegBatch) round trips, not S.
constexpr int kSegBatch = 8;

__device__ __forceinline__ MaxSum row_maxsum(const float2 *p, int S) {
  MaxSum r{kNegInf, 0.0f};
  for (int k0 = 0; k0 < S; k0 += kSegBatch) {
    float2 q[kSegBatch];
#pragma unroll
    for (int j = 0; j < kSegBatch; ++j)
      if (k0 + j < S) q[j] = p[k0 + j];
#pragma unroll
    for (int j = 0; j < kSegBatch; ++j)
      if (k0 + j < S) r = k0 + j == 0 ? MaxSum{q[j].x, q[j].y} : combine(r, MaxSum{q[j].x, q[j].y});
  }
  return r;
}

// The results of several rows (a target row and its draft row, or two such
// pairs) at once, each combined in segment order as row_maxsum does: every
// row's loads go out before any is combined, so the set costs one row's round
// trips.  Each pointer must address S readable results whatever its flag: the
// loads are not predicated per lane (a lane-predicated load waits for its
// data on its own), and a row whose flag is false keeps the value it came
// with.
template <int kRows>
__device__ __forceinline__ void row_maxsum_rows(const float2 *const (&p)[kRows], const bool (&use)[kRows], int S,
                                                MaxSum (&r)[kRows]) {
  for (int k0 = 0; k0 < S; k0 += kSegBatch) {
    float2 q[kRows][kSegBatch];
#pragma unroll
    for (int j = 0; j < kSegBatch; ++j)
      if (k0 + j < S) {
#pragma unroll
        for (int t = 0; t < kRows; ++t) q[t][j] = p[t][k0 + j];
      }
#pragma unroll
    for (int j = 0; j < kSegBatch; ++j)
#pragma unroll
      for (int t = 0; t < kRows; ++t)
        if (use[t] && k0 + j < S)
          r[t] = k0 + j == 0 ? MaxSum{q[t][j].x, q[t][j].y} : combine(r[t], MaxSum{q[t][j].x, q[t][j].y});
  }
}
__device__ __forceinline__ void row_maxsum_pair(const float2 *pa, bool la, const float2 *pb, bool lb, int S,
                                                MaxSum &ra, MaxSum &rb) {
  const float2 *const p[2] = {pa, pb};
  const bool use[2] = {la, lb};
  MaxSum r[2] = {ra, rb};
  row_maxsum_rows<2>(p, use, S, r);
  ra = r[0];
  rb = r[1];
}

__device__ __forceinline__ MaxIdx row_argmax(const float2 *p, int S) {
  MaxIdx r{kNegInf, 0};
  for (int k0 = 0; k0 < S; k0 += kSegBatch) {
    float2 q[kSegBatch];
#pragma unroll
    for (int j = 0; j < kSegBatch; ++j)
      if (k0 + j < S) q[j] = p[k0 + j];
#pragma unroll
    for (int j = 0; j < kSegBatch; ++j)
      if (k0 + j < S) {
        const MaxIdx c{q[j].x, __float_as_int(q[j].y)};
        r = k0 + j == 0 ? c : combine(r, c);
      }
  }
  return r;
}

// p = exp(x - m) / s at one gathered logit.
__device__ __forceinline__ float prob_at(float x, MaxSum st) {
  return exp_shift(x, st.m * kLog2e) / st.s;
}

// Exponent offset c with p_k = 2^(x_k log2e - c): c = m log2e + log2(s).
__device__ __forceinline__ float norm_offset(MaxSum st) { return st.m * kLog2e + log2f(st.s); }

// ---------------------------------------------------------------------------
// Decide: stochastic window (wave 0 of the calling workgroup)
// ---------------------------------------------------------------------------
// Lane i examines draft i: p_i(x_i), q_i(x_i) from the row results, the
// accept uniform of (seq, base_pos + 1 + i), accept iff u * q < p; the first
// rejection is the first zero of the ballot.  Returns the sampling job of the
// sequence in *job (JOB_NONE when the sequence is marked invalid).  When
// `write` is set this workgroup also writes the sequence's outputs.
template <int DT>
__device__ void window_decide(const WindowArgs &A, int b, int i, bool write, SampleJob *job) {
  using E = Elt<DT>;
  const int R = 2 * A.gamma + 1;
  int32_t *out = A.out_tokens + static_cast<int64_t>(b) * (A.gamma + 1);
  const int len = A.window_len ? A.window_len[b] : A.gamma;
  const int xi = i < A.gamma ? A.tokens[static_cast<int64_t>(b) * A.gamma + i] : 0;
  // The row results of target row i (i <= gamma) and draft row i (i < gamma)
  // are loaded before the window is checked, whatever its length (rows past
  // it, and those of a sequence found invalid, hold stale values that are not
  // used), so they travel with the token loads; only the two logit gathers
  // wait for the token.
  const float2 *prow = A.part + static_cast<int64_t>(b) * R * A.S;
  MaxSum st{0.0f, 1.0f}, sd{0.0f, 1.0f};
  row_maxsum_pair(prow + min(i, A.gamma) * A.S, i <= A.gamma, prow + (A.gamma + 1 + min(i, A.gamma - 1)) * A.S,
                  i < A.gamma, A.S, st, sd);
  const uint64_t seq = A.seq_ids ? A.seq_ids[b] : static_cast<uint64_t>(b);
  const int64_t base = A.base_pos ? A.base_pos[b] : 0;
  const bool bad_len = len < 0 || len > A.gamma;
  const bool bad_tok = !bad_len && i < len && (xi < 0 || xi >= A.V);
  if (__any(bad_len || bad_tok)) {
    if (write) {
      for (int k = i; k <= A.gamma; k += kWave) out[k] = -1;
      for (int k = i; k < A.gamma; k += kWave) {
        if (A.p_draft) A.p_draft[static_cast<int64_t>(b) * A.gamma + k] = 0.0f;
        if (A.q_draft) A.q_draft[static_cast<int64_t>(b) * A.gamma + k] = 0.0f;
      }
      if (i == 0) A.n_accepted[b] = -1;
    }
    if (i == 0) job->mode = JOB_NONE;
    return;
  }
  const int x = i < len ? xi : 0;
  const char *trow0 = A.t + b * A.t_stride_bytes;
  const char *drow0 = A.d + b * A.d_stride_bytes;
  const int64_t row_bytes = static_cast<int64_t>(A.V) * E::kBytes;
  // the two logits at the draft token go out before the uniforms are
  // computed, from every lane (lanes past the window read token 0 of row
  // min(i, gamma - 1) and do not use it), so the Philox rounds run while
  // they are in flight
  const int ig = min(i, A.gamma - 1);
  const uint32_t traw = E::raw(trow0 + ig * row_bytes, x);
  const uint32_t draw = E::raw(drow0 + ig * row_bytes, x);
  __builtin_amdgcn_sched_barrier(0);  // keeps the two loads ahead of the rounds
  const U64x4 w = philox4x64_10({seq, static_cast<uint64_t>(base + 1 + i), 0, 0}, A.seed, A.tag);
  const float vi = uniform24(w.c1);
  float P = 0.0f, Q = 0.0f;
  bool acc = false;
  if (i < len) {
    P = prob_at(E::dec(traw), st);
    Q = prob_at(E::dec(draw), sd);
    acc = uniform24(w.c0) * Q < P;
  }
  const uint64_t inv = ~static_cast<uint64_t>(__ballot(acc));
  int n = inv ? __builtin_ctzll(inv) : kWave;
  n = min(n, len);

  if (write) {
    if (i < A.gamma) {
      const int64_t o = static_cast<int64_t>(b) * A.gamma + i;
      if (A.p_draft) A.p_draft[o] = P;
      if (A.q_draft) A.q_draft[o] = Q;
    }
    for (int k = i; k <= A.gamma; k += kWave)
      if (k != n) out[k] = k < n ? x : -1;
  }
  // statistics and sampling uniform of row n, from lane n
  // n is the same in every lane: lane reads, not shuffles through LDS
  const int ln = n & (kWave - 1);
  MaxSum tn{lane_value(st.m, ln), lane_value(st.s, ln)};
  const MaxSum dn{lane_value(sd.m, ln), lane_value(sd.s, ln)};
  float v = lane_value(vi, ln);
  if (i == 0) {
    if (n >= kWave) {  // gamma = 64 with every draft accepted: row 64 has no lane
      tn = row_maxsum(prow + n * A.S, A.S);
      const U64x4 w = philox4x64_10({seq, static_cast<uint64_t>(base + 1 + n), 0, 0}, A.seed, A.tag);
      v = uniform24(w.c1);
    }
    SampleJob jb{};
    jb.t_row = trow0 + n * row_bytes;
    jb.ct = norm_offset(tn);
    if (n < len) {
      jb.mode = JOB_RESIDUAL;
      jb.cq = 1.0f;
      jb.d_row = drow0 + n * row_bytes;
      jb.cd = norm_offset(dn);
    } else {
      jb.mode = JOB_BONUS;
      jb.d_row = nullptr;
      jb.cd = 0.0f;
    }
    jb.v = v;
    jb.out_slot = out + n;
    *job = jb;
    if (write) A.n_accepted[b] = n;
  }
}

// ---------------------------------------------------------------------------
// Decide: early-exit window, positions [lo, hi) of every sequence still
// verifying (one wavefront per sequence, lane i <-> position lo + i)
// ---------------------------------------------------------------------------
// The first block (lo = 0) validates the sequence and sets its status; a
// sequence is done at its first rejection (residual job on that row) or once
// its window is exhausted (bonus job on row len), and then writes its outputs.
// Row results, uniforms and the job are the ones sv_verify_window computes.
// The job goes to *job_out; write_out gates the window outputs, write_status
// the status word (the last block, decided inside the draw, leaves it alone).
template <int DT>
__device__ __forceinline__ void stage_decide(const WindowArgs &A, int b, int i, int lo, int hi, int32_t *status,
                                             bool write_out, bool write_status, SampleJob *job_out) {
  using E = Elt<DT>;
  const int p = lo + i;
  const int R = 2 * A.gamma + 1;
  int32_t *out = A.out_tokens + static_cast<int64_t>(b) * (A.gamma + 1);
  // Status, window length, token, ids and this block's row results go out
  // together (the row results of a finished sequence are stale and unused):
  // one round trip, then the two logit gathers.
  const int32_t stat = lo > 0 ? status[b] : kSeqVerifying;
  const int len = A.window_len ? A.window_len[b] : A.gamma;
  const int xp = p < A.gamma ? A.tokens[static_cast<int64_t>(b) * A.gamma + p] : 0;
  const uint64_t seq = A.seq_ids ? A.seq_ids[b] : static_cast<uint64_t>(b);
  const int64_t base = A.base_pos ? A.base_pos[b] : 0;
  const float2 *prow = A.part + static_cast<int64_t>(b) * R * A.S;
  MaxSum st{0.0f, 1.0f}, sd{0.0f, 1.0f};
  row_maxsum_pair(prow + min(p, hi - 1) * A.S, p < hi, prow + (A.gamma + 1 + min(p, A.gamma - 1)) * A.S,
                  p < hi && p < A.gamma, A.S, st, sd);
  if (stat != kSeqVerifying) return;
  if (lo == 0) {
    const bool bad_len = len < 0 || len > A.gamma;
    const bool bad_tok = !bad_len && p < len && (xp < 0 || xp >= A.V);
    if (__any(bad_len || bad_tok)) {
      if (write_out) {
        for (int k = i; k <= A.gamma; k += kWave) out[k] = -1;
        for (int k = i; k < A.gamma; k += kWave) {
          if (A.p_draft) A.p_draft[static_cast<int64_t>(b) * A.gamma + k] = 0.0f;
          if (A.q_draft) A.q_draft[static_cast<int64_t>(b) * A.gamma + k] = 0.0f;
        }
      }
      if (i == 0) {
        if (write_out) A.n_accepted[b] = -1;
        job_out->mode = JOB_NONE;
        if (write_status) status[b] = -1;
      }
      return;
    }
  }
  const char *trow0 = A.t + b * A.t_stride_bytes;
  const char *drow0 = A.d + b * A.d_stride_bytes;
  const int64_t row_bytes = static_cast<int64_t>(A.V) * E::kBytes;
  const int cnt = min(hi, len) - lo;  // positions examined in this block
  // token logits first, from every lane (see window_decide), then the uniforms
  const int pg = min(p, A.gamma - 1);
  const int xg = i < cnt ? xp : 0;
  const uint32_t traw = E::raw(trow0 + pg * row_bytes, xg);
  const uint32_t draw = E::raw(drow0 + pg * row_bytes, xg);
  __builtin_amdgcn_sched_barrier(0);
  const U64x4 w = philox4x64_10({seq, static_cast<uint64_t>(base + 1 + p), 0, 0}, A.seed, A.tag);
  const float vi = uniform24(w.c1);
  float P = 0.0f, Q = 0.0f;
  bool acc = false;
  if (i < cnt) {
    P = prob_at(E::dec(traw), st);
    Q = prob_at(E::dec(draw), sd);
    acc = uniform24(w.c0) * Q < P;
  }
  const uint64_t inv = ~static_cast<uint64_t>(__ballot(acc));
  const int k = inv ? __builtin_ctzll(inv) : kWave;  // leading accepts in this block
  const bool rejected = k < cnt;
  const bool done = rejected || len < hi;
  const int n = rejected ? lo + k : len;  // meaningful when done
  if (write_out && i < cnt && (!done || p <= n)) {
    const int64_t o = static_cast<int64_t>(b) * A.gamma + p;
    if (A.p_draft) A.p_draft[o] = P;
    if (A.q_draft) A.q_draft[o] = Q;
  }
  if (!done) {
    if (i == 0 && lo == 0 && write_status) status[b] = kSeqVerifying;
    return;
  }
  if (write_out) {
    for (int q = n + i; q < A.gamma; q += kWave) {  // never examined: past n or past the window
      if (q == n && n < len) continue;
      if (A.p_draft) A.p_draft[static_cast<int64_t>(b) * A.gamma + q] = 0.0f;
      if (A.q_draft) A.q_draft[static_cast<int64_t>(b) * A.gamma + q] = 0.0f;
    }
    for (int q = i; q <= A.gamma; q += kWave)
      if (q != n) out[q] = q < n ? A.tokens[static_cast<int64_t>(b) * A.gamma + q] : -1;
  }
  const int src = (n - lo) & (kWave - 1);
  const MaxSum tn{lane_value(st.m, src), lane_value(st.s, src)};  // src is wave-uniform
  const MaxSum dn{lane_value(sd.m, src), lane_value(sd.s, src)};
  const float v = lane_value(vi, src);
  if (i == 0) {
    SampleJob jb{};
    jb.t_row = trow0 + n * row_bytes;
    jb.ct = norm_offset(tn);
    if (rejected) {
      jb.mode = JOB_RESIDUAL;
      jb.cq = 1.0f;
      jb.d_row = drow0 + n * row_bytes;
      jb.cd = norm_offset(dn);
    } else {
      jb.mode = JOB_BONUS;
      jb.d_row = nullptr;
      jb.cd = 0.0f;
    }
    jb.v = v;
    jb.out_slot = out + n;
    *job_out = jb;
    if (write_out) A.n_accepted[b] = n;
    if (write_status) status[b] = n;
  }
}

template <int DT>
__global__ void __launch_bounds__(kWave) k_stage_decide(WindowArgs A, int lo, int hi, int32_t *__restrict__ status) {
  const int b = blockIdx.x;
  stage_decide<DT>(A, b, threadIdx.x, lo, hi, status, true, true, A.jobs + b);
}

// ---------------------------------------------------------------------------
// Decide: greedy window
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kWave) k_greedy_decide(GreedyArgs A) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const int R = A.gamma + 1;
  int32_t *out = A.out_tokens + static_cast<int64_t>(b) * (A.gamma + 1);
  const int len = A.window_len ? A.window_len[b] : A.gamma;
  const int xi = i < A.gamma ? A.tokens[static_cast<int64_t>(b) * A.gamma + i] : 0;
  // the row results travel with the token loads (rows past the window hold
  // stale values and are not used)
  const float2 *prow = A.part + static_cast<int64_t>(b) * R * A.S;
  const int am_row = i <= A.gamma ? row_argmax(prow + i * A.S, A.S).i : 0;
  const bool bad_len = len < 0 || len > A.gamma;
  const bool bad_tok = !bad_len && i < len && (xi < 0 || xi >= A.V);
  if (__any(bad_len || bad_tok)) {
    for (int k = i; k <= A.gamma; k += kWave) out[k] = -1;
    if (i == 0) A.n_accepted[b] = -1;
    return;
  }
  const int x = i < len ? xi : 0;
  const int am = i <= len ? am_row : 0;
  const uint64_t mask = __ballot(i < len && x != am);
  const int n = mask ? __builtin_ctzll(mask) : len;
  int y = __builtin_amdgcn_readlane(am, n & (kWave - 1));  // n is wave-uniform
  for (int k = i; k <= A.gamma; k += kWave)
    if (k != n) out[k] = k < n ? x : -1;
  if (i == 0) {
    if (n >= kWave) y = row_argmax(prow + n * A.S, A.S).i;
    A.n_accepted[b] = n;
    out[n] = y;
  }
}

// ---------------------------------------------------------------------------
// Decide: token tree (one thread per node, N <= 256)
// ---------------------------------------------------------------------------
// The tree decision of sequence b by the calling workgroup: thread v < N
// examines node v; threads past kTreeMaxNodes only join the barriers.  When
// `write` is set the outputs are written.  The sampling job (stochastic mode)
// goes to *job, which may be null in greedy mode; an invalid token gives
// job->mode = JOB_NONE.
template <int DT>
__device__ void tree_decide(const TreeArgs &A, int b, int v, bool write, SampleJob *job_out) {
  using E = Elt<DT>;
  const int N = A.meta.N;
  const int D = A.meta.max_depth;
  int32_t *out_t = A.out_tokens + static_cast<int64_t>(b) * (D + 1);
  int32_t *out_n = A.out_nodes + static_cast<int64_t>(b) * D;
  const int32_t *toks = A.tokens + static_cast<int64_t>(b) * N;
  const int tok = (v >= 1 && v < N) ? toks[v] : 0;
  // the parent row's results and the ids travel with the token loads
  const float2 *prow = A.part + static_cast<int64_t>(b) * A.R * A.S;
  const uint64_t seq = A.seq_ids ? A.seq_ids[b] : static_cast<uint64_t>(b);
  const int64_t base = A.base_pos ? A.base_pos[b] : 0;
  int am = -1;
  MaxSum st{0.0f, 1.0f}, sd{0.0f, 1.0f};
  const bool node = v >= 1 && v < N;
  const int pw = node ? A.meta.parent[v] : 0;  // row 0 stands in for threads without a node
  if (A.mode == 0) {
    const int a = row_argmax(prow + pw * A.S, A.S).i;  // unpredicated load (row 0 stands in)
    am = node ? a : -1;
  } else {
    row_maxsum_pair(prow + pw * A.S, node, prow + (N + pw) * A.S, node, A.S, st, sd);
  }
  const bool bad = v >= 1 && v < N && (tok < 0 || tok >= A.V);
  if (__syncthreads_or(bad)) {
    if (write) {
      for (int k = v; k <= D; k += kTreeMaxNodes) out_t[k] = -1;
      for (int k = v; k < D; k += kTreeMaxNodes) out_n[k] = -1;
      if (v == 0) {
        A.n_accepted[b] = -1;
        A.best_node[b] = -1;
      }
    }
    if (v == 0 && job_out) job_out->mode = JOB_NONE;
    return;
  }
  const int64_t row_bytes = static_cast<int64_t>(A.V) * E::kBytes;
  const char *t0 = A.t + b * A.seq_bytes;
  const char *d0 = A.d ? A.d + b * A.seq_bytes : nullptr;

  __shared__ unsigned char s_acc[kTreeMaxNodes];
  __shared__ int s_parent[kTreeMaxNodes];
  __shared__ int s_path[kTreeMaxDepth + 1];
  __shared__ int s_best, s_key;
  if (v < N) {
    bool acc = true;
    if (v >= 1) {
      const int w = A.meta.parent[v];
      if (A.mode == 0) {
        acc = tok == am;
      } else {
        const float P = prob_at(E::one(t0 + w * row_bytes, tok), st);
        const float Q = prob_at(E::one(d0 + w * row_bytes, tok), sd);
        const U64x4 r = philox4x64_10(
            {seq, static_cast<uint64_t>(base + A.meta.depth[v]), static_cast<uint64_t>(A.meta.rank[v]), 0},
            A.seed, A.tag);
        acc = uniform24(r.c0) * Q < P;
      }
    }
    s_acc[v] = acc;
    s_parent[v] = A.meta.parent[v];
  }
  if (v == 0) s_key = 0;
  __syncthreads();
  // A node is accepted when its own test and every ancestor's passed; the
  // deepest accepted node wins, ties to the smallest index (key depth, -index).
  {
    int key = -1;
    if (v < N) {
      bool ok = s_acc[v];
      for (int u = s_parent[v]; ok && u > 0; u = s_parent[u]) ok = s_acc[u];
      if (ok) key = (static_cast<int>(A.meta.depth[v]) << 16) | (0xFFFF - v);
    }
    key = wave_max_int(key);
    if ((v & (kWave - 1)) == 0 && key >= 0) atomicMax(&s_key, key);  // one LDS atomic per wave
  }
  __syncthreads();
  if (v == 0) {
    const int best = 0xFFFF - (s_key & 0xFFFF);
    int w = best;
    for (int k = A.meta.depth[best] - 1; k >= 0; --k) {
      s_path[k] = w;
      w = s_parent[w];
    }
    s_best = best;
  }
  __syncthreads();
  const int best = s_best;
  const int nd = A.meta.depth[best];
  if (write) {
    for (int k = v; k < D; k += kTreeMaxNodes) out_n[k] = k < nd ? s_path[k] : -1;
    for (int k = v; k <= D; k += kTreeMaxNodes)
      if (k != nd) out_t[k] = k < nd ? toks[s_path[k]] : -1;
  }
  if (v == 0) {
    if (write) {
      A.n_accepted[b] = nd;
      A.best_node[b] = best;
    }
    if (A.mode == 0) {
      if (write) out_t[nd] = row_argmax(prow + best * A.S, A.S).i;
    } else {
      SampleJob job{};
      job.t_row = t0 + best * row_bytes;
      job.ct = norm_offset(row_maxsum(prow + best * A.S, A.S));
      if ((A.meta.internal[best >> 6] >> (best & 63)) & 1ull) {
        job.mode = JOB_RESIDUAL;
        job.cq = 1.0f;
        job.d_row = d0 + best * row_bytes;
        job.cd = norm_offset(row_maxsum(prow + (N + best) * A.S, A.S));
      } else {
        job.mode = JOB_BONUS;
        job.d_row = nullptr;
        job.cd = 0.0f;
      }
      const U64x4 r = philox4x64_10(
          {seq, static_cast<uint64_t>(base + nd + 1), static_cast<uint64_t>(A.meta.rank[best]), 0},
          A.seed, A.tag);
      job.v = uniform24(r.c1);
      job.out_slot = out_t + nd;
      *job_out = job;
    }
  }
}

// Standalone decision, one 256-thread workgroup per sequence (greedy trees).
template <int DT>
__global__ void __launch_bounds__(kTreeMaxNodes) k_tree_decide(TreeArgs A) {
  const int b = blockIdx.x;
  tree_decide<DT>(A, b, threadIdx.x, true, A.jobs ? A.jobs + b : nullptr);
}

// ---------------------------------------------------------------------------
// Sampling pass: one 1024-thread workgroup per sequence
// ---------------------------------------------------------------------------
// Weight of token k: p_k (bonus) or max(0, p_k - cq q_k) (residual), with
// p_k = 2^(t_k log2e - ct), q_k = 2^(d_k log2e - cd).
// p_k <= 1 and cq >= 0, so the clamp to [0, 1] is the max (one instruction);
// with cq = 1 the fused multiply-add rounds exactly like p - q.
__device__ __forceinline__ float bonus_weight(const SampleJob &job, float t) {
  return exp2_fast(__builtin_fmaf(t, kLog2e, -job.ct));
}
__device__ __forceinline__ float residual_weight(const SampleJob &job, float t, float d) {
  const float p = bonus_weight(job, t);
  const float q = exp2_fast(__builtin_fmaf(d, kLog2e, -job.cd));
  return __builtin_amdgcn_fmed3f(__builtin_fmaf(-job.cq, q, p), 0.0f, 1.0f);
}
__device__ __forceinline__ float weight_of(const SampleJob &job, float t, float d) {
  return job.mode != JOB_RESIDUAL ? bonus_weight(job, t) : residual_weight(job, t, d);
}

// Geometry of a sampling pass.  Vector geometry (kVec): the row is covered by
// the 16-byte blocks that hold it, counted from the block holding element 0;
// h = the offset of element 0 in its block, in elements (0 for aligned rows).
// Both rows of a residual job must share h.  Element k of the row is slot
// (k + h) % EPV of block (k + h) / EPV, so chunk c, thread t holds the EPV
// elements [c CH + t EPV - h, ... + EPV) (CH = kFinThreads EPV); slots outside
// [0, V) weigh 0.  A 16-byte aligned block never straddles a page, so loading
// one that holds at least one element of the row is safe; blocks holding none
// are not loaded.  Element geometry (!kVec, rows at different offsets): thread
// t holds 4 elements [c CH + 4t, ... + 4), loaded one by one.
__device__ __forceinline__ int job_shift(const SampleJob &job, int elem_bytes) {
  const int ta = static_cast<int>(reinterpret_cast<uintptr_t>(job.t_row) & 15);
  if (job.mode == JOB_RESIDUAL && static_cast<int>(reinterpret_cast<uintptr_t>(job.d_row) & 15) != ta) return -1;
  return ta / elem_bytes;
}

template <int DT, bool kVec>
struct FinGeom {
  static constexpr int E = kVec ? Elt<DT>::kEPV : 4;
  static constexpr int CH = kFinThreads * E;
};

template <int DT, bool kVec>
__device__ __forceinline__ int finish_chunks(int V, int h) {
  return (V + h + FinGeom<DT, kVec>::CH - 1) / FinGeom<DT, kVec>::CH;
}

// First element index of thread tid's slots in chunk c.
template <int DT, bool kVec>
__device__ __forceinline__ int slot0(int c, int tid, int h) {
  return c * FinGeom<DT, kVec>::CH + tid * FinGeom<DT, kVec>::E - h;
}

// Block `i` (16 bytes) of a row whose element 0 sits h elements into its block.
template <int DT>
__device__ __forceinline__ const uint4 *row_blocks(const void *row, int h) {
  return reinterpret_cast<const uint4 *>(static_cast<const char *>(row) - h * Elt<DT>::kBytes);
}

// Weights of thread tid's slots of chunk c (0 outside [0, V)).
template <int DT, bool kVec>
__device__ __forceinline__ void thread_weights(const SampleJob &job, int V, int c, int tid, int h, float *w) {
  using E = Elt<DT>;
  using G = FinGeom<DT, kVec>;
  const int k0 = slot0<DT, kVec>(c, tid, h);
  const bool resid = job.mode == JOB_RESIDUAL;
  if (kVec) {
    if (k0 >= V) {
#pragma unroll
      for (int e = 0; e < G::E; ++e) w[e] = 0.0f;
      return;
    }
    const int64_t blk = static_cast<int64_t>(c) * kFinThreads + tid;
    const uint4 rt = load_vec(row_blocks<DT>(job.t_row, h) + blk);
    const uint4 rd = resid ? load_vec(row_blocks<DT>(job.d_row, h) + blk) : make_uint4(0, 0, 0, 0);
    float xt[Elt<DT>::kEPV], xd[Elt<DT>::kEPV];
    E::vec(rt, xt);
    E::vec(rd, xd);
    const bool whole = k0 >= 0 && k0 + G::E <= V;
#pragma unroll
    for (int e = 0; e < G::E; ++e) {
      const float x = weight_of(job, xt[e], xd[e]);
      w[e] = (whole || (k0 + e >= 0 && k0 + e < V)) ? x : 0.0f;
    }
  } else {
#pragma unroll
    for (int e = 0; e < G::E; ++e) {
      const int k = k0 + e;
      w[e] = k < V ? weight_of(job, E::one(job.t_row, k), resid ? E::one(job.d_row, k) : 0.0f) : 0.0f;
    }
  }
}

// Sum of thread tid's weights of chunk c, then the wave sum into wp.
template <int DT, bool kVec>
__device__ __forceinline__ void chunk_sum_guarded(const SampleJob &job, int V, int c, int h, float *wp, int tid) {
  using G = FinGeom<DT, kVec>;
  float w[G::E];
  thread_weights<DT, kVec>(job, V, c, tid, h, w);
  float t = 0.0f;
#pragma unroll
  for (int e = 0; e < G::E; ++e) t += w[e];
  t = wave_total(t);
  if ((tid & (kWave - 1)) == 0) wp[c * kFinWaves + tid / kWave] = t;
}

// Weights of kFinBatch chunks already loaded as 16-byte vectors; wave sums to wp.
template <int DT>
__device__ __forceinline__ void batch_sums(const SampleJob &job, const uint4 *rt, const uint4 *rd, int c0,
                                           float *wp, int tid) {
  using E = Elt<DT>;
  constexpr int EPV = E::kEPV;
  // the job is the same for the whole workgroup: one scalar branch here, not
  // a per-element select between the two weights
  const bool resid = __builtin_amdgcn_readfirstlane(job.mode) == JOB_RESIDUAL;
#pragma unroll
  for (int u = 0; u < kFinBatch; ++u) {
    float xt[EPV];
    E::vec(rt[u], xt);
    float t = 0.0f;
    if (resid) {
      float xd[EPV];
      E::vec(rd[u], xd);
#pragma unroll
      for (int e = 0; e < EPV; ++e) t += residual_weight(job, xt[e], xd[e]);
    } else {
#pragma unroll
      for (int e = 0; e < EPV; ++e) t += bonus_weight(job, xt[e]);
    }
    t = wave_total(t);
    if ((tid & (kWave - 1)) == 0) wp[(c0 + u) * kFinWaves + tid / kWave] = t;
  }
}

template <bool kCached>
__device__ __forceinline__ uint4 load_pass(const uint4 *p) {
  if constexpr (kCached) return load_vec(p);
  else return load_stream(p);
}

// Streams chunks [c_begin, c_end) of the job's row(s) once;
// wp[c * kFinWaves + wave] = wave sum of chunk c.  Vector geometry: chunks
// whose slots all lie in [0, V) go in batches of kFinBatch, the next batch's
// loads in flight while the current one is reduced; the head chunk (h > 0)
// and the row's end are masked per slot.  The batches use nontemporal loads;
// kCached selects ordinary cached ones instead, for the tree walk, whose
// passes read the same row pair once per rejected sibling and find it in L2
// from the second pass on.
template <int DT, bool kVec, bool kCached = false>
__device__ __forceinline__ void stream_chunk_sums(const SampleJob &job, int V, int c_begin, int c_end, int h,
                                                  float *wp, int tid) {
  int c = c_begin;
  if (kVec) {
    constexpr int CH = FinGeom<DT, true>::CH;
    if (h > 0 && c == 0 && c < c_end) {
      chunk_sum_guarded<DT, true>(job, V, 0, h, wp, tid);
      c = 1;
    }
    const int full = min(c_end, (V + h) / CH);  // chunks with every slot inside the row
    const bool resid = job.mode == JOB_RESIDUAL;
    const uint4 *tv = row_blocks<DT>(job.t_row, h) + tid;
    const uint4 *dv = row_blocks<DT>(job.d_row, h) + tid;
    const uint4 zero = make_uint4(0, 0, 0, 0);
    if (full - c >= kFinBatch) {
      uint4 at[kFinBatch], ad[kFinBatch], bt[kFinBatch], bd[kFinBatch];
#pragma unroll
      for (int u = 0; u < kFinBatch; ++u) {
        at[u] = load_pass<kCached>(tv + (c + u) * kFinThreads);
        ad[u] = resid ? load_pass<kCached>(dv + (c + u) * kFinThreads) : zero;
      }
      for (; c + 2 * kFinBatch <= full; c += kFinBatch) {
#pragma unroll
        for (int u = 0; u < kFinBatch; ++u) {
          bt[u] = load_pass<kCached>(tv + (c + kFinBatch + u) * kFinThreads);
          bd[u] = resid ? load_pass<kCached>(dv + (c + kFinBatch + u) * kFinThreads) : zero;
        }
        batch_sums<DT>(job, at, ad, c, wp, tid);
#pragma unroll
        for (int u = 0; u < kFinBatch; ++u) {
          at[u] = bt[u];
          ad[u] = bd[u];
        }
      }
      batch_sums<DT>(job, at, ad, c, wp, tid);
      c += kFinBatch;
    }
  }
  for (; c < c_end; ++c) chunk_sum_guarded<DT, kVec>(job, V, c, h, wp, tid);
}

// cs[c] = sum over waves of wp[c][wave], in wave order, for c in [c_begin, c_end).
__device__ __forceinline__ void chunk_totals(const float *wp, int c_begin, int c_end, float *cs, int tid) {
  for (int c = c_begin + tid; c < c_end; c += kFinThreads) {
    float t = wp[c * kFinWaves];
#pragma unroll
    for (int w = 1; w < kFinWaves; ++w) t += wp[c * kFinWaves + w];
    cs[c] = t;
  }
}

// Inverse CDF from the chunk sums cs[0..C): wave 0 forms their inclusive
// prefix sums (a wave scan over 64 chunks at a time, carried in chunk order),
// Z = the last one, tau = v * Z, and the chunk holding tau is the first whose
// prefix exceeds it; then the first k of that chunk whose running sum exceeds
// tau (w_k > 0).  If rounding leaves no such chunk, the last chunk with mass;
// if it leaves no such k, the chunk's last k with w_k > 0.  Returns -1 (every
// thread) when the weights have no mass: none at all, or a residual whose
// mass is below kNoResidualMass.  cs must be visible to the whole workgroup.
template <int DT, bool kVec>
__device__ int draw_from_sums(const SampleJob &job, int V, int C, int h, const float *cs, int tid) {
  using G = FinGeom<DT, kVec>;
  __shared__ float s_base, s_tau;
  __shared__ int s_chunk, s_cand, s_last;
  __shared__ float s_wave_tot[kFinWaves];
  __shared__ float s_pref[kFinMaxChunks];
  if (tid < kWave) {
    const int lane = tid;
    float carry = 0.0f;
    int last_mass = -1;
    for (int c0 = 0; c0 < C; c0 += kWave) {
      const int c = c0 + lane;
      const float x = c < C ? cs[c] : 0.0f;
      float incl = wave_inclusive_scan(x);
      incl += carry;
      if (c < C) s_pref[c] = incl;
      const uint64_t mass = __ballot(c < C && x > 0.0f);
      if (mass) last_mass = c0 + 63 - __builtin_clzll(mass);
      carry = lane_value(incl, kWave - 1);
    }
    const float Z = carry;
    const float tau = job.v * Z;
    int chunk = -1;
    for (int c0 = 0; c0 < C && chunk < 0; c0 += kWave) {
      const int c = c0 + lane;
      const uint64_t hit = __ballot(c < C && s_pref[c] > tau);
      if (hit) chunk = c0 + __builtin_ctzll(hit);
    }
    if (chunk < 0) chunk = last_mass;  // rounding left tau at or past the total (-1: no mass)
    if (!(Z > 0.0f) || (job.mode == JOB_RESIDUAL && Z < kNoResidualMass)) chunk = -1;
    if (lane == 0) {
      s_chunk = chunk;
      s_base = chunk > 0 ? s_pref[chunk - 1] : 0.0f;
      s_tau = tau;
      s_cand = INT_MAX;
      s_last = -1;
    }
  }
  __syncthreads();
  const int chunk = s_chunk;
  if (chunk < 0) return -1;
  float w[G::E];
  thread_weights<DT, kVec>(job, V, chunk, tid, h, w);
  float ts = 0.0f;
#pragma unroll
  for (int e = 0; e < G::E; ++e) ts += w[e];
  const int wave = tid / kWave, lane = tid & (kWave - 1);
  const float incl = wave_inclusive_scan(ts);
  const float excl = wave_shift_up1(incl);  // 0 in lane 0
  if (lane == kWave - 1) s_wave_tot[wave] = incl;
  __syncthreads();
  float wave_off = 0.0f;
  for (int k = 0; k < wave; ++k) wave_off += s_wave_tot[k];
  float run = s_base + (wave_off + excl);
  const float tau = s_tau;
  const int k0 = slot0<DT, kVec>(chunk, tid, h);
  int cand = INT_MAX, last = -1;
#pragma unroll
  for (int e = 0; e < G::E; ++e) {
    run += w[e];
    if (cand == INT_MAX && run > tau && w[e] > 0.0f) cand = k0 + e;
    if (w[e] > 0.0f) last = k0 + e;
  }
  // Slots grow with the thread index, so a wave's first candidate is its
  // lowest lane with one and its last mass its highest such lane: one LDS
  // atomic per wave (1024 on one word serialise for microseconds).
  const uint64_t has_cand = __ballot(cand != INT_MAX);
  const uint64_t has_last = __ballot(last >= 0);
  if (has_cand && lane == __builtin_ctzll(has_cand)) atomicMin(&s_cand, cand);
  if (has_last && lane == 63 - __builtin_clzll(has_last)) atomicMax(&s_last, last);
  __syncthreads();
  int y = s_cand != INT_MAX ? s_cand : s_last;
  if (y < 0) y = max(0, chunk * G::CH - h);  // the chunk had mass but rounding hid it from every slot
  return y;
}

// A residual job drawn as a bonus from the target row: what a draw with no
// residual mass falls back to (the rejected draft had p = q = 0 and the two
// rows are identical, or identical to within the rounding of their
// normalisers).
__device__ __forceinline__ SampleJob as_bonus(SampleJob job) {
  job.mode = JOB_BONUS;
  job.d_row = nullptr;
  job.cd = 0.0f;
  job.cq = 0.0f;
  return job;
}

// Sampling pass of one job over chunks [0, C) and the draw, by the whole
// workgroup; chunk sums in s_cs.  Returns -1 when the weights have no mass.
template <int DT>
__device__ __forceinline__ int sample_pass(const SampleJob &job, int V, float *s_wp, float *s_cs, int tid) {
  const int h = job_shift(job, Elt<DT>::kBytes);
  if (h >= 0) {
    const int C = finish_chunks<DT, true>(V, h);
    stream_chunk_sums<DT, true>(job, V, 0, C, h, s_wp, tid);
    __syncthreads();
    chunk_totals(s_wp, 0, C, s_cs, tid);
    __syncthreads();
    return draw_from_sums<DT, true>(job, V, C, h, s_cs, tid);
  }
  const int C = finish_chunks<DT, false>(V, 0);
  stream_chunk_sums<DT, false>(job, V, 0, C, 0, s_wp, tid);
  __syncthreads();
  chunk_totals(s_wp, 0, C, s_cs, tid);
  __syncthreads();
  return draw_from_sums<DT, false>(job, V, C, 0, s_cs, tid);
}

// The draw of one job; a residual without mass is drawn from p instead.
template <int DT>
__device__ __forceinline__ int sample_job(const SampleJob &job, int V, float *s_wp, float *s_cs, int tid) {
  const int y = sample_pass<DT>(job, V, s_wp, s_cs, tid);
  if (y >= 0) return y;
  __syncthreads();  // s_cs and the draw's LDS are reused
  return sample_pass<DT>(as_bonus(job), V, s_wp, s_cs, tid);
}

// Where the draw's job comes from: the jobs array (an early-exit sequence
// decided in an earlier block, or the LM-head path), the window decision
// (wave 0), the early-exit decision of the last position block
// [A.stage_lo, gamma] (wave 0, for sequences still verifying), or the
// stochastic tree decision (the first kTreeMaxNodes threads; A is then a
// TreeArgs).  `write` gates the outputs.
enum : int { SRC_JOBS = 0, SRC_WINDOW = 1, SRC_STAGE = 2, SRC_TREE = 3 };

// Job of sequence b into s_job; returns whether it was decided here.
template <int DT, int kSrc, typename Args>
__device__ __forceinline__ bool load_job(const Args &A, const SampleJob *jobs, int b, bool write,
                                         SampleJob *s_job, int tid) {
  bool decided = false;
  if constexpr (kSrc == SRC_TREE) {
    tree_decide<DT>(A, b, tid, write, s_job);  // every thread joins its barriers
    decided = true;
  } else if constexpr (kSrc == SRC_WINDOW) {
    if (tid < kWave) window_decide<DT>(A, b, tid, write, s_job);
    decided = true;
  } else if constexpr (kSrc == SRC_STAGE) {
    if (A.status[b] == kSeqVerifying) {
      if (tid < kWave) stage_decide<DT>(A, b, tid, A.stage_lo, A.gamma + 1, A.status, write, false, s_job);
      decided = true;
    } else if (tid == 0) {
      *s_job = jobs[b];
    }
  } else if (tid == 0) {
    *s_job = jobs[b];
  }
  __syncthreads();
  return decided;
}

// One workgroup per sequence (large batches): decide, one pass over the
// row(s) with chunk sums in LDS, draw.
template <int DT, int kSrc, typename Args = WindowArgs>
__global__ void __launch_bounds__(kFinThreads) k_finish(Args A, const SampleJob *__restrict__ jobs, int V) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ SampleJob s_job;
  __shared__ float s_wp[kFinMaxChunks * kFinWaves];
  __shared__ float s_cs[kFinMaxChunks];
  load_job<DT, kSrc>(A, jobs, b, true, &s_job, tid);
  const SampleJob job = s_job;
  if (job.mode == JOB_NONE) return;
  const int y = sample_job<DT>(job, V, s_wp, s_cs, tid);
  if (tid == 0) *job.out_slot = y;
}

// Small batches, grid (B, G): workgroup g decides (redundantly, it is cheap)
// and sums its share of the chunks into spart[b][c]; the g = 0 workgroup
// writes the window outputs and the job.  The last of the G workgroups of a
// sequence to finish (a device-scope arrival counter; the launch before this
// one zeroed it) reads all chunk sums and draws.  No workgroup waits for
// another: the others just exit.
template <int DT, int kSrc, typename Args = WindowArgs>
__global__ void __launch_bounds__(kFinThreads) k_finish_part(Args A, SampleJob *__restrict__ jobs, int V,
                                                            float *__restrict__ spart, int cmax,
                                                            int32_t *__restrict__ arrive) {
  const int b = blockIdx.x;
  const int g = blockIdx.y;
  const int G = gridDim.y;
  const int tid = threadIdx.x;
  __shared__ SampleJob s_job;
  __shared__ float s_wp[kFinMaxChunks * kFinWaves];
  __shared__ float s_cs[kFinMaxChunks];
  __shared__ int s_last;
  static_assert(kFinMaxChunks <= kFinThreads, "one chunk sum per thread in the draw");
  const bool decided = load_job<DT, kSrc>(A, jobs, b, g == 0, &s_job, tid);
  const SampleJob job = s_job;
  if (decided && g == 0 && tid == 0) jobs[b] = job;
  if (job.mode == JOB_NONE) return;
  const int h = job_shift(job, Elt<DT>::kBytes);
  const bool vec = h >= 0;
  const int C = vec ? finish_chunks<DT, true>(V, h) : finish_chunks<DT, false>(V, 0);
  const int c0 = static_cast<int>(static_cast<int64_t>(C) * g / G);
  const int c1 = static_cast<int>(static_cast<int64_t>(C) * (g + 1) / G);
  if (vec) stream_chunk_sums<DT, true>(job, V, c0, c1, h, s_wp, tid);
  else stream_chunk_sums<DT, false>(job, V, c0, c1, 0, s_wp, tid);
  __syncthreads();
  chunk_totals(s_wp, c0, c1, s_cs, tid);
  __syncthreads();
  // Hand-off without cache-wide write-backs: the chunk sums are stored and
  // read back as device-scope atomics (written through to, and read from, the
  // level the XCDs share), and every writer waits for its stores to complete
  // before the workgroup's arrival is counted.
  float *sp = spart + static_cast<int64_t>(b) * cmax;
  for (int c = c0 + tid; c < c1; c += kFinThreads)
    __hip_atomic_store(sp + c, s_cs[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(arrive + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old + 1) % G == 0;
  }
  __syncthreads();
  if (!s_last) return;
  if (tid < C) s_cs[tid] = __hip_atomic_load(sp + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  int y = vec ? draw_from_sums<DT, true>(job, V, C, h, s_cs, tid)
              : draw_from_sums<DT, false>(job, V, C, 0, s_cs, tid);
  if (y < 0) {  // no residual mass: this workgroup draws from p alone
    __syncthreads();
    y = sample_pass<DT>(as_bonus(job), V, s_wp, s_cs, tid);
  }
  if (tid == 0) *job.out_slot = y;
}

// ---------------------------------------------------------------------------
// Token tree, lossless multi-candidate walk (one 1024-thread workgroup per
// sequence)
// ---------------------------------------------------------------------------
// SpecInfer's multi-round scheme (cited by title on the PipeSpec and CLaSp
// review pages): from the root, the children of the current node w are tried
// in index order against the residual r of w.  After j rejections at w,
// r = max(0, p - c q) / Z with c = 0, Z = 1 at first and, per rejection,
// c <- c + Z, Z <- sum_k max(0, p_k - c q_k) (p, q: rows w of the target and
// draft).  This closed form equals renormalising max(0, r - q) after every
// rejection.  Child token x is accepted iff u * q(x) * Z < p(x) - c q(x),
// which with c = 0, Z = 1 is the window's u * q < p.  An accepted child
// becomes w and r restarts at its p.  A leaf ends the walk with a bonus draw
// from p_w; a node whose children were all rejected ends it with a draw from
// r, using the chunk sums of the pass that produced Z.  A rejection whose new
// residual has no mass (r equal to q) keeps the previous r.
//
// Set-up, one thread per node v: p_w(x_v), q_w(x_v) and u_v against the
// parent w, the exponent offsets of rows v, the draw uniform after v, and the
// child links, all into LDS.  Then thread 0 walks through LDS alone; every
// thread joins the streaming passes (one per rejection, over rows w of both
// logits) and the final draw.
enum : int { WALK_PASS = 0, WALK_PASS_DRAW = 1, WALK_DRAW = 2 };

template <int DT>
__global__ void __launch_bounds__(kFinThreads) k_tree_walk(TreeArgs A) {
  using E = Elt<DT>;
  static_assert(kFinThreads >= kTreeMaxNodes, "one thread per node in the set-up");
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int N = A.meta.N;
  const int D = A.meta.max_depth;
  const int V = A.V;
  int32_t *out_t = A.out_tokens + static_cast<int64_t>(b) * (D + 1);
  int32_t *out_n = A.out_nodes + static_cast<int64_t>(b) * D;
  const int32_t *toks = A.tokens + static_cast<int64_t>(b) * N;
  const int tok = (tid >= 1 && tid < N) ? toks[tid] : 0;
  const bool bad = tid >= 1 && tid < N && (tok < 0 || tok >= V);
  if (__syncthreads_or(bad)) {
    for (int k = tid; k <= D; k += kFinThreads) out_t[k] = -1;
    for (int k = tid; k < D; k += kFinThreads) out_n[k] = -1;
    if (tid == 0) {
      A.n_accepted[b] = -1;
      A.best_node[b] = -1;
    }
    return;
  }
  const float2 *prow = A.part + static_cast<int64_t>(b) * A.R * A.S;
  const int64_t row_bytes = static_cast<int64_t>(V) * E::kBytes;
  const char *t0 = A.t + b * A.seq_bytes;
  const char *d0 = A.d + b * A.seq_bytes;
  const uint64_t seq = A.seq_ids ? A.seq_ids[b] : static_cast<uint64_t>(b);
  const int64_t base = A.base_pos ? A.base_pos[b] : 0;

  __shared__ SampleJob s_job;
  __shared__ float s_wp[kFinMaxChunks * kFinWaves];
  __shared__ float s_cs[kFinMaxChunks];
  __shared__ float s_P[kTreeMaxNodes], s_Q[kTreeMaxNodes], s_u[kTreeMaxNodes];
  __shared__ float s_ct[kTreeMaxNodes], s_cd[kTreeMaxNodes], s_v[kTreeMaxNodes];
  __shared__ int s_first[kTreeMaxNodes], s_next[kTreeMaxNodes], s_tok[kTreeMaxNodes];
  __shared__ int s_path[kTreeMaxDepth];
  __shared__ int s_cmd, s_nd, s_w;

  if (tid < N) {
    const int v = tid;
    const int first = A.meta.first_child[v];
    const int depth = A.meta.depth[v];
    const int rank = A.meta.rank[v];
    // the token's logits in the parent's rows (the root reads token 0 of row
    // 0 and does not use it), then the results of rows v and of the parent's
    // rows w, all four as one batch; the Philox rounds run while they land
    const int w = v >= 1 ? A.meta.parent[v] : 0;
    const uint32_t traw = E::raw(t0 + w * row_bytes, tok);
    const uint32_t draw = E::raw(d0 + w * row_bytes, tok);
    const float2 *const rows4[4] = {prow + v * A.S, prow + (N + v) * A.S, prow + w * A.S, prow + (N + w) * A.S};
    const bool use4[4] = {true, first >= 0, v >= 1, v >= 1};
    MaxSum r4[4] = {{0.0f, 1.0f}, {0.0f, 1.0f}, {0.0f, 1.0f}, {0.0f, 1.0f}};
    row_maxsum_rows<4>(rows4, use4, A.S, r4);
    const MaxSum st = r4[2], sd = r4[3];
    s_ct[v] = norm_offset(r4[0]);
    s_cd[v] = first >= 0 ? norm_offset(r4[1]) : 0.0f;
    s_v[v] = uniform24(
        philox4x64_10({seq, static_cast<uint64_t>(base + depth + 1), static_cast<uint64_t>(rank), 0}, A.seed, A.tag)
            .c1);
    if (v >= 1) {
      s_P[v] = prob_at(E::dec(traw), st);
      s_Q[v] = prob_at(E::dec(draw), sd);
      s_u[v] = uniform24(
          philox4x64_10({seq, static_cast<uint64_t>(base + depth), static_cast<uint64_t>(rank), 0}, A.seed, A.tag)
              .c0);
    }
    s_first[v] = first;
    s_next[v] = A.meta.next_sibling[v];
    s_tok[v] = tok;
  }
  __syncthreads();

  // walk state, meaningful in thread 0 only
  int w = 0, nd = 0, cand = s_first[0], pend_chunks = 0;
  float c = 0.0f, Z = 1.0f, c_try = 0.0f;
  bool pending = false, sums_ok = false;
  for (;;) {
    if (tid == 0) {
      if (pending) {  // s_cs holds the chunk sums of max(0, p - c_try q)
        float z = 0.0f;
        for (int k = 0; k < pend_chunks; ++k) z += s_cs[k];
        sums_ok = z >= kNoResidualMass;
        if (sums_ok) {
          c = c_try;
          Z = z;
        }
        pending = false;
      }
      SampleJob jb{};
      int cmd = -1;
      while (cmd < 0) {
        jb.t_row = t0 + w * row_bytes;
        jb.ct = s_ct[w];
        if (cand >= 0) {
          const float P = s_P[cand], Q = s_Q[cand];
          if (s_u[cand] * Q * Z < __builtin_fmaf(-c, Q, P)) {
            s_path[nd++] = cand;
            w = cand;
            cand = s_first[w];
            c = 0.0f;
            Z = 1.0f;
            sums_ok = false;
            continue;
          }
          c_try = c + Z;
          jb.mode = JOB_RESIDUAL;
          jb.d_row = d0 + w * row_bytes;
          jb.cd = s_cd[w];
          jb.cq = c_try;
          pending = true;
          cand = s_next[cand];
          cmd = WALK_PASS;
        } else {
          if (s_first[w] >= 0 && c > 0.0f) {
            jb.mode = JOB_RESIDUAL;
            jb.d_row = d0 + w * row_bytes;
            jb.cd = s_cd[w];
            jb.cq = c;
          } else {  // a leaf, or no rejection left residual mass: draw from p
            jb.mode = JOB_BONUS;
            jb.d_row = nullptr;
            jb.cd = 0.0f;
            jb.cq = 0.0f;
          }
          jb.v = s_v[w];
          jb.out_slot = out_t + nd;
          cmd = (jb.mode == JOB_RESIDUAL && sums_ok) ? WALK_DRAW : WALK_PASS_DRAW;
        }
      }
      const int hj = job_shift(jb, E::kBytes);
      pend_chunks = hj >= 0 ? finish_chunks<DT, true>(V, hj) : finish_chunks<DT, false>(V, 0);
      s_job = jb;
      s_cmd = cmd;
      s_nd = nd;
      s_w = w;
    }
    __syncthreads();
    const SampleJob job = s_job;
    const int cmd = s_cmd;
    const int h = job_shift(job, E::kBytes);
    const bool vec = h >= 0;
    const int C = vec ? finish_chunks<DT, true>(V, h) : finish_chunks<DT, false>(V, 0);
    if (cmd != WALK_DRAW) {
      if (vec) stream_chunk_sums<DT, true, true>(job, V, 0, C, h, s_wp, tid);
      else stream_chunk_sums<DT, false, true>(job, V, 0, C, 0, s_wp, tid);
      __syncthreads();
      chunk_totals(s_wp, 0, C, s_cs, tid);
      __syncthreads();
    }
    if (cmd == WALK_PASS) continue;
    int y = vec ? draw_from_sums<DT, true>(job, V, C, h, s_cs, tid)
                : draw_from_sums<DT, false>(job, V, C, 0, s_cs, tid);
    if (y < 0) {  // rounding left the residual without mass: draw from p_w
      __syncthreads();
      y = sample_pass<DT>(as_bonus(job), V, s_wp, s_cs, tid);
    }
    const int n = s_nd;
    for (int k = tid; k < D; k += kFinThreads) out_n[k] = k < n ? s_path[k] : -1;
    for (int k = tid; k <= D; k += kFinThreads) out_t[k] = k < n ? s_tok[s_path[k]] : (k == n ? y : -1);
    if (tid == 0) {
      A.n_accepted[b] = n;
      A.best_node[b] = s_w;
    }
    return;
  }
}

// ---------------------------------------------------------------------------
// Rollback
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kWave) k_rollback(RollbackArgs A) {
  const int s = blockIdx.x;
  const int j = blockIdx.y;
  const int lane = threadIdx.x;
  int32_t *len_j = A.buf_len + static_cast<int64_t>(s) * A.K + j;
  const int L = A.verified_len[s] + A.len_offset;
  const int lj = *len_j;
  if (L < 0 || L > A.cap || lj < 0 || lj > A.cap) {
    if (lane == 0) *len_j = -1;
    return;
  }
  int32_t *buf = A.buf_tokens + (static_cast<int64_t>(s) * A.K + j) * A.cap;
  const int32_t *ver = A.verified + static_cast<int64_t>(s) * A.verified_stride;
  const int lim = min(lj, L);
  int m = lim;
  for (int t0 = 0; t0 < lim; t0 += kWave) {
    const int t = t0 + lane;
    const uint64_t diff = __ballot(t < lim && buf[t] != ver[t]);
    if (diff) {
      m = t0 + __builtin_ctzll(diff);
      break;
    }
  }
  if (m < L) {
    for (int t = m + lane; t < L; t += kWave) buf[t] = ver[t];
    if (lane == 0) *len_j = L;
  }
}

// ---------------------------------------------------------------------------
// Launchers (host side)
// ---------------------------------------------------------------------------
// Workgroups per sequence for the draw: enough to give every CU work, at
// most one per chunk of the vector geometry.
static int finish_split(int B, int V, int dtype) {
  const int epv = dtype == DT_F32 ? 4 : 8;
  const int chunks = (V + kFinThreads * epv - 1) / (kFinThreads * epv);
  int G = (kFinFillWorkgroups + B - 1) / B;
  if (G > chunks) G = chunks;
  return G < 1 ? 1 : G;
}

template <int DT, int kSrc, typename Args = WindowArgs>
static void launch_finish_t(const Args &A, SampleJob *jobs, int B, int V, const DrawScratch &ds, hipStream_t st) {
  const int G = finish_split(B, V, DT);
  if (G == 1) {
    hipLaunchKernelGGL((k_finish<DT, kSrc, Args>), dim3(B), dim3(kFinThreads), 0, st, A, jobs, V);
  } else {
    hipLaunchKernelGGL((k_finish_part<DT, kSrc, Args>), dim3(B, G), dim3(kFinThreads), 0, st, A, jobs, V, ds.spart,
                       ds.cmax, ds.arrive);
  }
}

template <int kSrc>
static void launch_finish(int dtype, const WindowArgs &A, SampleJob *jobs, int B, int V, const DrawScratch &ds,
                          hipStream_t st) {
  switch (dtype) {
    case DT_BF16: launch_finish_t<DT_BF16, kSrc>(A, jobs, B, V, ds, st); break;
    case DT_F16: launch_finish_t<DT_F16, kSrc>(A, jobs, B, V, ds, st); break;
    default: launch_finish_t<DT_F32, kSrc>(A, jobs, B, V, ds, st); break;
  }
}

void launch_window_finish(int dtype, const WindowArgs &A, int B, const DrawScratch &ds, hipStream_t st) {
  launch_finish<SRC_WINDOW>(dtype, A, A.jobs, B, A.V, ds, st);
}

void launch_stage_finish(int dtype, const WindowArgs &A, int B, const DrawScratch &ds, hipStream_t st) {
  launch_finish<SRC_STAGE>(dtype, A, A.jobs, B, A.V, ds, st);
}

void launch_stage_decide(int dtype, const WindowArgs &A, int B, int lo, int hi, int32_t *status, hipStream_t st) {
  switch (dtype) {
    case DT_BF16: hipLaunchKernelGGL(k_stage_decide<DT_BF16>, dim3(B), dim3(kWave), 0, st, A, lo, hi, status); break;
    case DT_F16: hipLaunchKernelGGL(k_stage_decide<DT_F16>, dim3(B), dim3(kWave), 0, st, A, lo, hi, status); break;
    default: hipLaunchKernelGGL(k_stage_decide<DT_F32>, dim3(B), dim3(kWave), 0, st, A, lo, hi, status); break;
  }
}

void launch_greedy_decide(const GreedyArgs &A, int B, hipStream_t st) {
  hipLaunchKernelGGL(k_greedy_decide, dim3(B), dim3(kWave), 0, st, A);
}

void launch_tree_decide(int dtype, const TreeArgs &A, int B, hipStream_t st) {
  switch (dtype) {
    case DT_BF16: hipLaunchKernelGGL(k_tree_decide<DT_BF16>, dim3(B), dim3(kTreeMaxNodes), 0, st, A); break;
    case DT_F16: hipLaunchKernelGGL(k_tree_decide<DT_F16>, dim3(B), dim3(kTreeMaxNodes), 0, st, A); break;
    default: hipLaunchKernelGGL(k_tree_decide<DT_F32>, dim3(B), dim3(kTreeMaxNodes), 0, st, A); break;
  }
}

void launch_tree_finish(int dtype, SampleJob *jobs, int B, int V, const DrawScratch &ds, hipStream_t st) {
  const WindowArgs none{};
  launch_finish<SRC_JOBS>(dtype, none, jobs, B, V, ds, st);
}

void launch_tree_decide_draw(int dtype, const TreeArgs &A, int B, const DrawScratch &ds, hipStream_t st) {
  switch (dtype) {
    case DT_BF16: launch_finish_t<DT_BF16, SRC_TREE, TreeArgs>(A, A.jobs, B, A.V, ds, st); break;
    case DT_F16: launch_finish_t<DT_F16, SRC_TREE, TreeArgs>(A, A.jobs, B, A.V, ds, st); break;
    default: launch_finish_t<DT_F32, SRC_TREE, TreeArgs>(A, A.jobs, B, A.V, ds, st); break;
  }
}

void launch_tree_walk(int dtype, const TreeArgs &A, int B, hipStream_t st) {
  switch (dtype) {
    case DT_BF16: hipLaunchKernelGGL(k_tree_walk<DT_BF16>, dim3(B), dim3(kFinThreads), 0, st, A); break;
    case DT_F16: hipLaunchKernelGGL(k_tree_walk<DT_F16>, dim3(B), dim3(kFinThreads), 0, st, A); break;
    default: hipLaunchKernelGGL(k_tree_walk<DT_F32>, dim3(B), dim3(kFinThreads), 0, st, A); break;
  }
}

void launch_rollback(const RollbackArgs &A, int S, int stage, hipStream_t st) {
  hipLaunchKernelGGL(k_rollback, dim3(S, stage), dim3(kWave), 0, st, A);
}

}  // namespace sv
