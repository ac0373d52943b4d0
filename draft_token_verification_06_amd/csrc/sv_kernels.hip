// HIP kernels of the verification library (gfx950).
//
// Pass 1, k_row_stats: each workgroup streams one segment of one vocabulary
//   row from HBM with 16-byte loads and reduces it to (max, sum 2^((x-max)
//   log2e)) or to (max, first index of the max).  Per-thread batches of
//   kUnroll vectors are kept in registers: the batch maximum is taken first so
//   that every element costs exactly one exponential, then wave butterflies and
//   one LDS step finish the workgroup in a fixed order.
// Decide, k_window_decide / k_greedy_decide / k_tree_decide: one wavefront (or
//   one workgroup for trees) per sequence combines the segment results, forms
//   p(x) and q(x) at the draft tokens, draws the Philox uniforms, and finds the
//   first rejection with a wavefront ballot.
// Sampling, k_sample_partial + k_sample_select: the one extra pass over the
//   row of the first rejection (or the bonus row): chunk sums of the weights,
//   then an inverse-CDF search inside the chunk holding tau = v * Z.
// Rollback, k_rollback: first divergence by ballot, then copy of the
//   verified tail.
#include <climits>

#include "sv_device.h"
#include "sv_launch.h"
#include "sv_plan.h"

namespace sv {

constexpr int kUnroll = 4;  // 16-byte loads in flight per thread

// ---------------------------------------------------------------------------
// Pass 1: row statistics
// ---------------------------------------------------------------------------

template <int DT, bool kArgmax>
struct RowAcc;

template <int DT>
struct RowAcc<DT, false> {
  float m = kNegInf, s = 0.0f;
  __device__ __forceinline__ void batch(const float *x, int n, int) {
    float bm = x[0];
#pragma unroll
    for (int k = 1; k < kUnroll * Elt<DT>::kEPV; ++k) bm = fmaxf(bm, x[k]);
    if (bm > m) {
      s *= exp_shift(m, bm * kLog2e);
      m = bm;
    }
    if (m != kNegInf) {
      const float ml = m * kLog2e;
      float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < kUnroll * Elt<DT>::kEPV; ++k) acc[k & 3] += exp_shift(x[k], ml);
      s += (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
    (void)n;
  }
  __device__ __forceinline__ void one(float x, int) {
    if (x > m) {
      s = s * exp_shift(m, x * kLog2e) + 1.0f;
      m = x;
    } else if (m != kNegInf) {
      s += exp_shift(x, m * kLog2e);
    }
  }
  __device__ __forceinline__ float2 result(float *lds_m, float *lds_s, int tid) {
    MaxSum v = wave_reduce(MaxSum{m, s});
    const int w = tid / kWave;
    if ((tid & (kWave - 1)) == 0) {
      lds_m[w] = v.m;
      lds_s[w] = v.s;
    }
    __syncthreads();
    MaxSum r{lds_m[0], lds_s[0]};
#pragma unroll
    for (int k = 1; k < kRowThreads / kWave; ++k) r = combine(r, MaxSum{lds_m[k], lds_s[k]});
    return make_float2(r.m, r.s);
  }
};

template <int DT>
struct RowAcc<DT, true> {
  float m = kNegInf;
  int i = INT_MAX;
  // x holds kUnroll vectors; vector u starts at element index base + u * stride.
  __device__ __forceinline__ void batch(const float *x, int base, int stride) {
    constexpr int EPV = Elt<DT>::kEPV;
    float bm = x[0];
#pragma unroll
    for (int k = 1; k < kUnroll * EPV; ++k) bm = fmaxf(bm, x[k]);
    if (bm > m) {
      int found = INT_MAX;
#pragma unroll
      for (int k = kUnroll * EPV - 1; k >= 0; --k)
        if (x[k] == bm) found = base + (k / EPV) * stride + (k % EPV);
      m = bm;
      i = found;
    }
  }
  __device__ __forceinline__ void one(float x, int k) {
    if (x > m || (x == m && k < i)) {
      m = x;
      i = k;
    }
  }
  __device__ __forceinline__ float2 result(float *lds_m, float *lds_s, int tid) {
    MaxIdx v = wave_reduce(MaxIdx{m, i});
    const int w = tid / kWave;
    if ((tid & (kWave - 1)) == 0) {
      lds_m[w] = v.m;
      lds_s[w] = __int_as_float(v.i);
    }
    __syncthreads();
    MaxIdx r{lds_m[0], __float_as_int(lds_s[0])};
#pragma unroll
    for (int k = 1; k < kRowThreads / kWave; ++k)
      r = combine(r, MaxIdx{lds_m[k], __float_as_int(lds_s[k])});
    return make_float2(r.m, __int_as_float(r.i));
  }
};

template <int DT, bool kArgmax>
__global__ void __launch_bounds__(kRowThreads) k_row_stats(RowSet rs, float2 *__restrict__ part) {
  using E = Elt<DT>;
  constexpr int EPV = E::kEPV;
  const int R = rs.rows_t + rs.rows_d;
  const int64_t blk = blockIdx.x;
  const int seg = static_cast<int>(blk % rs.S);
  const int64_t rj = blk / rs.S;
  const int j = static_cast<int>(rj % R);
  const int64_t b = rj / R;

  int len = rs.gamma;
  if (rs.window_len) {
    len = rs.window_len[b];
    if (len < 0 || len > rs.gamma) return;
  }
  const char *row;
  if (j < rs.rows_t) {
    if (rs.window_len && j > len) return;
    row = rs.t + b * rs.t_stride_bytes + static_cast<int64_t>(j) * rs.V * E::kBytes;
  } else {
    const int jd = j - rs.rows_t;
    if (rs.window_len && jd >= len) return;
    if (!((rs.dmask[jd >> 6] >> (jd & 63)) & 1ull)) return;
    row = rs.d + b * rs.d_stride_bytes + static_cast<int64_t>(jd) * rs.V * E::kBytes;
  }

  const int lo = seg * rs.seg_len;
  const int hi = min(rs.V, lo + rs.seg_len);
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row + static_cast<int64_t>(lo) * E::kBytes);
  const int mis = static_cast<int>(addr & 15);
  const int head = min(mis ? (16 - mis) / E::kBytes : 0, hi - lo);
  const int a = lo + head;
  const int nvec = (hi - a) / EPV;
  const int tail = a + nvec * EPV;
  const uint4 *vp = reinterpret_cast<const uint4 *>(row + static_cast<int64_t>(a) * E::kBytes);
  const int tid = threadIdx.x;

  RowAcc<DT, kArgmax> acc;
  const uint4 neg = make_uint4(E::kNegInfPair, E::kNegInfPair, E::kNegInfPair, E::kNegInfPair);
  for (int v0 = 0; v0 < nvec; v0 += kUnroll * kRowThreads) {
    uint4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int vi = v0 + u * kRowThreads + tid;
      r[u] = vi < nvec ? vp[vi] : neg;
    }
    float x[kUnroll * EPV];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) E::vec(r[u], x + u * EPV);
    acc.batch(x, a + (v0 + tid) * EPV, kRowThreads * EPV);
  }
  for (int k = lo + tid; k < a; k += kRowThreads) acc.one(E::one(row, k), k);
  for (int k = tail + tid; k < hi; k += kRowThreads) acc.one(E::one(row, k), k);

  __shared__ float lds_m[kRowThreads / kWave], lds_s[kRowThreads / kWave];
  const float2 res = acc.result(lds_m, lds_s, tid);
  if (tid == 0) part[blk] = res;
}

// Combine the S segment results of one row, in segment order.
__device__ __forceinline__ MaxSum row_maxsum(const float2 *p, int S) {
  MaxSum r{p[0].x, p[0].y};
  for (int k = 1; k < S; ++k) r = combine(r, MaxSum{p[k].x, p[k].y});
  return r;
}

__device__ __forceinline__ MaxIdx row_argmax(const float2 *p, int S) {
  MaxIdx r{p[0].x, __float_as_int(p[0].y)};
  for (int k = 1; k < S; ++k) r = combine(r, MaxIdx{p[k].x, __float_as_int(p[k].y)});
  return r;
}

// p = exp(x - m) / s at one gathered logit.
__device__ __forceinline__ float prob_at(float x, MaxSum st) {
  return exp_shift(x, st.m * kLog2e) / st.s;
}

// ---------------------------------------------------------------------------
// Decide: stochastic window
// ---------------------------------------------------------------------------
template <int DT>
__global__ void __launch_bounds__(kWave) k_window_decide(WindowArgs A) {
  using E = Elt<DT>;
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const int R = 2 * A.gamma + 1;
  int32_t *out = A.out_tokens + static_cast<int64_t>(b) * (A.gamma + 1);
  const int len = A.window_len ? A.window_len[b] : A.gamma;
  const bool bad_len = len < 0 || len > A.gamma;
  int x = 0;
  if (!bad_len && i < len) x = A.tokens[static_cast<int64_t>(b) * A.gamma + i];
  const bool bad_tok = !bad_len && i < len && (x < 0 || x >= A.V);
  if (__any(bad_len || bad_tok)) {
    for (int k = i; k <= A.gamma; k += kWave) out[k] = -1;
    if (A.p_draft)
      for (int k = i; k < A.gamma; k += kWave) A.p_draft[static_cast<int64_t>(b) * A.gamma + k] = 0.0f;
    if (A.q_draft)
      for (int k = i; k < A.gamma; k += kWave) A.q_draft[static_cast<int64_t>(b) * A.gamma + k] = 0.0f;
    if (i == 0) {
      A.n_accepted[b] = -1;
      A.jobs[b].mode = JOB_NONE;
    }
    return;
  }

  const float2 *prow = A.part + static_cast<int64_t>(b) * R * A.S;
  const char *trow0 = A.t + b * A.t_stride_bytes;
  const char *drow0 = A.d + b * A.d_stride_bytes;
  const int64_t row_bytes = static_cast<int64_t>(A.V) * E::kBytes;
  const uint64_t seq = A.seq_ids ? A.seq_ids[b] : static_cast<uint64_t>(b);
  const int64_t base = A.base_pos ? A.base_pos[b] : 0;

  float P = 0.0f, Q = 0.0f;
  bool acc = false;
  if (i < len) {
    const MaxSum st = row_maxsum(prow + i * A.S, A.S);
    const MaxSum sd = row_maxsum(prow + (A.gamma + 1 + i) * A.S, A.S);
    P = prob_at(E::one(trow0 + i * row_bytes, x), st);
    Q = prob_at(E::one(drow0 + i * row_bytes, x), sd);
    const U64x4 w = philox4x64_10({seq, static_cast<uint64_t>(base + 1 + i), 0, 0}, A.seed, A.tag);
    acc = uniform24(w.c0) * Q < P;
  }
  const uint64_t inv = ~static_cast<uint64_t>(__ballot(acc));
  int n = inv ? __builtin_ctzll(inv) : kWave;
  n = min(n, len);

  if (i < A.gamma) {
    const int64_t o = static_cast<int64_t>(b) * A.gamma + i;
    if (A.p_draft) A.p_draft[o] = P;
    if (A.q_draft) A.q_draft[o] = Q;
  }
  for (int k = i; k <= A.gamma; k += kWave)
    if (k != n) out[k] = k < n ? x : -1;
  if (i == 0) {
    A.n_accepted[b] = n;
    SampleJob job{};
    const MaxSum st = row_maxsum(prow + n * A.S, A.S);
    job.t_row = trow0 + n * row_bytes;
    job.mt_l2e = st.m * kLog2e;
    job.inv_st = 1.0f / st.s;
    if (n < len) {
      const MaxSum sd = row_maxsum(prow + (A.gamma + 1 + n) * A.S, A.S);
      job.mode = JOB_RESIDUAL;
      job.d_row = drow0 + n * row_bytes;
      job.md_l2e = sd.m * kLog2e;
      job.inv_sd = 1.0f / sd.s;
    } else {
      job.mode = JOB_BONUS;
      job.d_row = nullptr;
      job.md_l2e = 0.0f;
      job.inv_sd = 0.0f;
    }
    const U64x4 w = philox4x64_10({seq, static_cast<uint64_t>(base + 1 + n), 0, 0}, A.seed, A.tag);
    job.v = uniform24(w.c1);
    job.out_slot = out + n;
    A.jobs[b] = job;
  }
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
  const bool bad_len = len < 0 || len > A.gamma;
  int x = 0;
  if (!bad_len && i < len) x = A.tokens[static_cast<int64_t>(b) * A.gamma + i];
  const bool bad_tok = !bad_len && i < len && (x < 0 || x >= A.V);
  if (__any(bad_len || bad_tok)) {
    for (int k = i; k <= A.gamma; k += kWave) out[k] = -1;
    if (i == 0) A.n_accepted[b] = -1;
    return;
  }
  const float2 *prow = A.part + static_cast<int64_t>(b) * R * A.S;
  bool mismatch = false;
  if (i < len) mismatch = x != row_argmax(prow + i * A.S, A.S).i;
  const uint64_t mask = __ballot(mismatch);
  const int n = mask ? __builtin_ctzll(mask) : len;
  for (int k = i; k <= A.gamma; k += kWave)
    if (k != n) out[k] = k < n ? x : -1;
  if (i == 0) {
    A.n_accepted[b] = n;
    out[n] = row_argmax(prow + n * A.S, A.S).i;
  }
}

// ---------------------------------------------------------------------------
// Decide: token tree (one thread per node, N <= 256)
// ---------------------------------------------------------------------------
template <int DT>
__global__ void __launch_bounds__(kTreeMaxNodes) k_tree_decide(TreeArgs A) {
  using E = Elt<DT>;
  const int b = blockIdx.x;
  const int v = threadIdx.x;
  const int N = A.meta.N;
  const int D = A.meta.max_depth;
  int32_t *out_t = A.out_tokens + static_cast<int64_t>(b) * (D + 1);
  int32_t *out_n = A.out_nodes + static_cast<int64_t>(b) * D;
  const int32_t *toks = A.tokens + static_cast<int64_t>(b) * N;
  const int tok = (v >= 1 && v < N) ? toks[v] : 0;
  const bool bad = v >= 1 && v < N && (tok < 0 || tok >= A.V);
  if (__syncthreads_or(bad)) {
    for (int k = v; k <= D; k += kTreeMaxNodes) out_t[k] = -1;
    for (int k = v; k < D; k += kTreeMaxNodes) out_n[k] = -1;
    if (v == 0) {
      A.n_accepted[b] = -1;
      A.best_node[b] = -1;
      if (A.jobs) A.jobs[b].mode = JOB_NONE;
    }
    return;
  }
  const float2 *prow = A.part + static_cast<int64_t>(b) * A.R * A.S;
  const int64_t row_bytes = static_cast<int64_t>(A.V) * E::kBytes;
  const char *t0 = A.t + b * A.seq_bytes;
  const char *d0 = A.d ? A.d + b * A.seq_bytes : nullptr;
  const uint64_t seq = A.seq_ids ? A.seq_ids[b] : static_cast<uint64_t>(b);
  const int64_t base = A.base_pos ? A.base_pos[b] : 0;

  __shared__ unsigned char s_acc[kTreeMaxNodes];
  __shared__ int s_path[kTreeMaxDepth + 1];
  __shared__ int s_best;
  if (v < N) {
    bool acc = true;
    if (v >= 1) {
      const int w = A.meta.parent[v];
      if (A.mode == 0) {
        acc = tok == row_argmax(prow + w * A.S, A.S).i;
      } else {
        const MaxSum st = row_maxsum(prow + w * A.S, A.S);
        const MaxSum sd = row_maxsum(prow + (N + w) * A.S, A.S);
        const float P = prob_at(E::one(t0 + w * row_bytes, tok), st);
        const float Q = prob_at(E::one(d0 + w * row_bytes, tok), sd);
        const U64x4 r = philox4x64_10(
            {seq, static_cast<uint64_t>(base + A.meta.depth[v]), static_cast<uint64_t>(A.meta.rank[v]), 0},
            A.seed, A.tag);
        acc = uniform24(r.c0) * Q < P;
      }
    }
    s_acc[v] = acc;
  }
  __syncthreads();
  if (v == 0) {
    // accepted = own test and parent accepted; nodes come after their parents
    int best = 0;
    for (int u = 1; u < N; ++u) {
      s_acc[u] = s_acc[u] && s_acc[A.meta.parent[u]];
      if (s_acc[u] && A.meta.depth[u] > A.meta.depth[best]) best = u;
    }
    int w = best;
    for (int k = A.meta.depth[best] - 1; k >= 0; --k) {
      s_path[k] = w;
      w = A.meta.parent[w];
    }
    s_best = best;
  }
  __syncthreads();
  const int best = s_best;
  const int nd = A.meta.depth[best];
  for (int k = v; k < D; k += kTreeMaxNodes) out_n[k] = k < nd ? s_path[k] : -1;
  for (int k = v; k <= D; k += kTreeMaxNodes)
    if (k != nd) out_t[k] = k < nd ? toks[s_path[k]] : -1;
  if (v == 0) {
    A.n_accepted[b] = nd;
    A.best_node[b] = best;
    if (A.mode == 0) {
      out_t[nd] = row_argmax(prow + best * A.S, A.S).i;
    } else {
      SampleJob job{};
      const MaxSum st = row_maxsum(prow + best * A.S, A.S);
      job.t_row = t0 + best * row_bytes;
      job.mt_l2e = st.m * kLog2e;
      job.inv_st = 1.0f / st.s;
      if ((A.meta.internal[best >> 6] >> (best & 63)) & 1ull) {
        const MaxSum sd = row_maxsum(prow + (N + best) * A.S, A.S);
        job.mode = JOB_RESIDUAL;
        job.d_row = d0 + best * row_bytes;
        job.md_l2e = sd.m * kLog2e;
        job.inv_sd = 1.0f / sd.s;
      } else {
        job.mode = JOB_BONUS;
        job.d_row = nullptr;
        job.md_l2e = 0.0f;
        job.inv_sd = 0.0f;
      }
      const U64x4 r = philox4x64_10(
          {seq, static_cast<uint64_t>(base + nd + 1), static_cast<uint64_t>(A.meta.rank[best]), 0},
          A.seed, A.tag);
      job.v = uniform24(r.c1);
      job.out_slot = out_t + nd;
      A.jobs[b] = job;
    }
  }
}

// ---------------------------------------------------------------------------
// Sampling pass
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float sample_weight(const SampleJob &job, int k) {
  using E = Elt<DT>;
  const float p = exp_shift(E::one(job.t_row, k), job.mt_l2e) * job.inv_st;
  if (job.mode != JOB_RESIDUAL) return p;
  const float q = exp_shift(E::one(job.d_row, k), job.md_l2e) * job.inv_sd;
  return fmaxf(0.0f, p - q);
}

template <int DT>
__global__ void __launch_bounds__(kSampleThreads) k_sample_partial(const SampleJob *__restrict__ jobs,
                                                                   int V, int C, float *__restrict__ spart) {
  const int c = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const SampleJob job = jobs[b];
  float acc = 0.0f;
  if (job.mode != JOB_NONE) {
    const int lo = c * kSampleChunk;
    const int hi = min(V, lo + kSampleChunk);
    for (int k = lo + tid; k < hi; k += kSampleThreads) acc += sample_weight<DT>(job, k);
  }
  acc = wave_sum(acc);
  __shared__ float lds[kSampleThreads / kWave];
  if ((tid & (kWave - 1)) == 0) lds[tid / kWave] = acc;
  __syncthreads();
  if (tid == 0) {
    float s = lds[0];
#pragma unroll
    for (int k = 1; k < kSampleThreads / kWave; ++k) s += lds[k];
    spart[static_cast<int64_t>(b) * C + c] = s;
  }
}

template <int DT>
__global__ void __launch_bounds__(kSampleThreads) k_sample_select(const SampleJob *__restrict__ jobs,
                                                                  int V, int C, const float *__restrict__ spart) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const SampleJob job = jobs[b];
  if (job.mode == JOB_NONE) return;
  __shared__ float s_base, s_tau;
  __shared__ int s_chunk;
  __shared__ float s_wsum[kSampleThreads / kWave];
  __shared__ int s_cand, s_last;
  if (tid == 0) {
    const float *sp = spart + static_cast<int64_t>(b) * C;
    float Z = 0.0f;
    for (int c = 0; c < C; ++c) Z += sp[c];
    const float tau = job.v * Z;
    int chunk = -1;
    float run = 0.0f, base = 0.0f;
    for (int c = 0; c < C; ++c) {
      const float nxt = run + sp[c];
      if (nxt > tau) {
        chunk = c;
        base = run;
        break;
      }
      run = nxt;
    }
    if (chunk < 0) {  // rounding left tau at or past the total: last chunk with mass
      run = 0.0f;
      for (int c = 0; c < C; ++c) {
        if (sp[c] > 0.0f) {
          chunk = c;
          base = run;
        }
        run += sp[c];
      }
      if (chunk < 0) chunk = 0;
    }
    s_chunk = chunk;
    s_base = base;
    s_tau = tau;
    s_cand = INT_MAX;
    s_last = -1;
  }
  __syncthreads();
  const int lo = s_chunk * kSampleChunk;
  const int hi = min(V, lo + kSampleChunk);
  const int k0 = lo + tid * kSamplePerThread;
  float w[kSamplePerThread];
  float ts = 0.0f;
#pragma unroll
  for (int e = 0; e < kSamplePerThread; ++e) {
    w[e] = (k0 + e < hi) ? sample_weight<DT>(job, k0 + e) : 0.0f;
    ts += w[e];
  }
  // exclusive prefix of the per-thread sums, in thread order
  const int lane = tid & (kWave - 1);
  float incl = ts;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  float excl = __shfl_up(incl, 1);
  if (lane == 0) excl = 0.0f;
  if (lane == kWave - 1) s_wsum[tid / kWave] = incl;
  __syncthreads();
  float wave_off = 0.0f;
  for (int k = 0; k < tid / kWave; ++k) wave_off += s_wsum[k];
  float run = s_base + (wave_off + excl);
  const float tau = s_tau;
  int cand = INT_MAX, last = -1;
#pragma unroll
  for (int e = 0; e < kSamplePerThread; ++e) {
    if (k0 + e < hi) {
      run += w[e];
      if (cand == INT_MAX && run > tau && w[e] > 0.0f) cand = k0 + e;
      if (w[e] > 0.0f) last = k0 + e;
    }
  }
  if (cand != INT_MAX) atomicMin(&s_cand, cand);
  if (last >= 0) atomicMax(&s_last, last);
  __syncthreads();
  if (tid == 0) {
    int y = s_cand != INT_MAX ? s_cand : s_last;
    if (y < 0) y = lo;  // no mass anywhere: only reachable with invalid logits
    *job.out_slot = y;
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
// Read-bandwidth probe
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kRowThreads) k_probe_read(const uint4 *__restrict__ src, int64_t nvec,
                                                            uint32_t *__restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kRowThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kRowThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < nvec; i += kUnroll * stride) {
    uint4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) r[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  }
  for (; i < nvec; i += stride) {
    const uint4 r = src[i];
    acc ^= r.x ^ r.y ^ r.z ^ r.w;
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ uint32_t lds[kRowThreads / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) lds[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int k = 0; k < kRowThreads / kWave; ++k) r ^= lds[k];
    sink[blockIdx.x] = r;
  }
}

// ---------------------------------------------------------------------------
// Launchers (host side)
// ---------------------------------------------------------------------------
template <bool kArgmax>
static void launch_row_stats_t(int dtype, const RowSet &rs, int64_t blocks, float2 *part, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(blocks)), block(kRowThreads);
  switch (dtype) {
    case DT_BF16: hipLaunchKernelGGL((k_row_stats<DT_BF16, kArgmax>), grid, block, 0, st, rs, part); break;
    case DT_F16: hipLaunchKernelGGL((k_row_stats<DT_F16, kArgmax>), grid, block, 0, st, rs, part); break;
    default: hipLaunchKernelGGL((k_row_stats<DT_F32, kArgmax>), grid, block, 0, st, rs, part); break;
  }
}

void launch_row_stats(int dtype, bool argmax, const RowSet &rs, int64_t blocks, float2 *part, hipStream_t st) {
  if (argmax) launch_row_stats_t<true>(dtype, rs, blocks, part, st);
  else launch_row_stats_t<false>(dtype, rs, blocks, part, st);
}

void launch_window_decide(int dtype, const WindowArgs &A, int B, hipStream_t st) {
  switch (dtype) {
    case DT_BF16: hipLaunchKernelGGL(k_window_decide<DT_BF16>, dim3(B), dim3(kWave), 0, st, A); break;
    case DT_F16: hipLaunchKernelGGL(k_window_decide<DT_F16>, dim3(B), dim3(kWave), 0, st, A); break;
    default: hipLaunchKernelGGL(k_window_decide<DT_F32>, dim3(B), dim3(kWave), 0, st, A); break;
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

void launch_sample(int dtype, const SampleJob *jobs, int B, int V, int C, float *spart, hipStream_t st) {
  const dim3 g1(C, B), g2(B), blk(kSampleThreads);
  switch (dtype) {
    case DT_BF16:
      hipLaunchKernelGGL(k_sample_partial<DT_BF16>, g1, blk, 0, st, jobs, V, C, spart);
      hipLaunchKernelGGL(k_sample_select<DT_BF16>, g2, blk, 0, st, jobs, V, C, spart);
      break;
    case DT_F16:
      hipLaunchKernelGGL(k_sample_partial<DT_F16>, g1, blk, 0, st, jobs, V, C, spart);
      hipLaunchKernelGGL(k_sample_select<DT_F16>, g2, blk, 0, st, jobs, V, C, spart);
      break;
    default:
      hipLaunchKernelGGL(k_sample_partial<DT_F32>, g1, blk, 0, st, jobs, V, C, spart);
      hipLaunchKernelGGL(k_sample_select<DT_F32>, g2, blk, 0, st, jobs, V, C, spart);
      break;
  }
}

void launch_rollback(const RollbackArgs &A, int S, int stage, hipStream_t st) {
  hipLaunchKernelGGL(k_rollback, dim3(S, stage), dim3(kWave), 0, st, A);
}

int probe_blocks(size_t bytes) {
  const int64_t nvec = static_cast<int64_t>(bytes / 16);
  int64_t blocks = (nvec + kRowThreads - 1) / kRowThreads;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  return static_cast<int>(blocks);
}

void launch_probe_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t st) {
  const int blocks = probe_blocks(bytes);
  hipLaunchKernelGGL(k_probe_read, dim3(blocks), dim3(kRowThreads), 0, st,
                     reinterpret_cast<const uint4 *>(src), static_cast<int64_t>(bytes / 16), sink);
}

}  // namespace sv
