// Row statistics of the verification library (gfx950), and the read probe
// that measures the same loads' ceiling.
//
// k_row_stats: each workgroup streams one segment of one vocabulary row from
//   HBM with 16-byte loads and reduces it to (max, sum 2^((x-max) log2e)) or
//   to (max, first index of the max).  Per-thread batches of kUnroll vectors
//   are kept in registers: the batch maximum is taken first so that every
//   element costs exactly one exponential, then DPP moves within each wave
//   and one LDS step finish the workgroup in a fixed order.
// k_probe_read: the same nontemporal loads over one contiguous buffer.
#include "sv_device.h"
#include "sv_rowset.h"

namespace sv {

#ifndef SV_ROW_UNROLL
#define SV_ROW_UNROLL 8
#endif
// 16-byte loads per thread per batch; the next batch is loaded while the
// current one is reduced, so 2 * kUnroll loads are in flight per thread.
constexpr int kUnroll = SV_ROW_UNROLL;

// ---------------------------------------------------------------------------
// Pass 1: row statistics
// ---------------------------------------------------------------------------

template <int DT, bool kArgmax, int U = kUnroll>
struct RowAcc;

template <int DT, int U>
struct RowAcc<DT, false, U> {
  float m = kNegInf, s = 0.0f;
  __device__ __forceinline__ void batch(const float *x, int n, int) {
    float bm = x[0];
#pragma unroll
    for (int k = 1; k < U * Elt<DT>::kEPV; ++k) bm = fmaxf(bm, x[k]);
    if (bm > m) {
      s *= rescale(m, bm);
      m = bm;
    }
    if (m != kNegInf) {
      const float ml = m * kLog2e;
      float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < U * Elt<DT>::kEPV; ++k) acc[k & 3] += exp_shift(x[k], ml);
      s += (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
    (void)n;
  }
  __device__ __forceinline__ void one(float x, int) {
    if (x > m) {
      s = s * rescale(m, x) + 1.0f;
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

template <int DT, int U>
struct RowAcc<DT, true, U> {
  float m = kNegInf;
  int i = INT_MAX;
  // x holds U vectors; vector u starts at element index base + u * stride.
  __device__ __forceinline__ void batch(const float *x, int base, int stride) {
    constexpr int EPV = Elt<DT>::kEPV;
    float bm = x[0];
#pragma unroll
    for (int k = 1; k < U * EPV; ++k) bm = fmaxf(bm, x[k]);
    if (bm > m) {
      int found = INT_MAX;
#pragma unroll
      for (int k = U * EPV - 1; k >= 0; --k)
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

// Streams elements [lo, hi) of one row into a per-thread accumulator: a
// scalar head up to the first 16-byte boundary, a body of 16-byte vectors,
// a scalar tail.  Body vectors go in batches of U per thread (thread tid takes
// vectors tid, tid + NT, ...); over full batches the next batch's loads are in
// flight while the current batch is reduced, and a guarded remainder batch
// fills its gaps with -inf.
template <int DT, int NT, int U, typename Acc>
__device__ __forceinline__ void stream_segment(const char *row, int lo, int hi, int tid, Acc &acc) {
  using E = Elt<DT>;
  constexpr int EPV = E::kEPV;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row + static_cast<int64_t>(lo) * E::kBytes);
  const int mis = static_cast<int>(addr & 15);
  const int head = min(mis ? (16 - mis) / E::kBytes : 0, hi - lo);
  const int a = lo + head;
  const int nvec = (hi - a) / EPV;
  const int tail = a + nvec * EPV;
  const uint4 *vp = reinterpret_cast<const uint4 *>(row + static_cast<int64_t>(a) * E::kBytes);
  constexpr int kStep = U * NT;
  const int nfull = nvec / kStep;
  if (nfull > 0) {
    uint4 cur[U], nxt[U];
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = load_stream(vp + u * NT + tid);
    for (int it = 0; it < nfull - 1; ++it) {
      const uint4 *q = vp + (it + 1) * kStep + tid;
#pragma unroll
      for (int u = 0; u < U; ++u) nxt[u] = load_stream(q + u * NT);
      float x[U * EPV];
#pragma unroll
      for (int u = 0; u < U; ++u) E::vec(cur[u], x + u * EPV);
      acc.batch(x, a + (it * kStep + tid) * EPV, NT * EPV);
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    }
    float x[U * EPV];
#pragma unroll
    for (int u = 0; u < U; ++u) E::vec(cur[u], x + u * EPV);
    acc.batch(x, a + ((nfull - 1) * kStep + tid) * EPV, NT * EPV);
  }
  if (nfull * kStep < nvec) {
    const uint4 neg = make_uint4(E::kNegInfPair, E::kNegInfPair, E::kNegInfPair, E::kNegInfPair);
    uint4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int vi = nfull * kStep + u * NT + tid;
      r[u] = vi < nvec ? load_stream(vp + vi) : neg;
    }
    float x[U * EPV];
#pragma unroll
    for (int u = 0; u < U; ++u) E::vec(r[u], x + u * EPV);
    acc.batch(x, a + (nfull * kStep + tid) * EPV, NT * EPV);
  }
  for (int k = lo + tid; k < a; k += NT) acc.one(E::one(row, k), k);
  for (int k = tail + tid; k < hi; k += NT) acc.one(E::one(row, k), k);
}

template <int DT, bool kArgmax>
__global__ void __launch_bounds__(kRowThreads) k_row_stats(RowSet rs, float2 *__restrict__ part) {
  using E = Elt<DT>;
  const uint32_t blk = blockIdx.x;  // B * R * S < 2^31 (checked on the host)
  const int seg = static_cast<int>(blk % static_cast<uint32_t>(rs.S));
  const uint32_t rj = blk / static_cast<uint32_t>(rs.S);
  const int j = static_cast<int>(rj % static_cast<uint32_t>(rs.R));
  const int64_t b = rj / static_cast<uint32_t>(rs.R);

  // The arrival counters of the draw that follows start from zero.
  if (rs.arrive && j == 0 && seg == 0 && threadIdx.x == 0) rs.arrive[b] = 0;
  if (rs.status && rs.status[b] != kSeqVerifying) return;
  int len = rs.gamma;
  if (rs.window_len) {
    len = rs.window_len[b];
    if (len < 0 || len > rs.gamma) return;
  }
  const int e = rs.row[j];
  const int i = e & ~kDraftRow;
  const char *row;
  int slot;
  if (!(e & kDraftRow)) {
    if (rs.window_len && i > len) return;
    row = rs.t + b * rs.t_stride_bytes + static_cast<int64_t>(i) * rs.V * E::kBytes;
    slot = i;
  } else {
    if (rs.window_len && i >= len) return;
    row = rs.d + b * rs.d_stride_bytes + static_cast<int64_t>(i) * rs.V * E::kBytes;
    slot = rs.d_slot0 + i;
  }

  const int lo = seg * rs.seg_len;
  const int hi = min(rs.V, lo + rs.seg_len);
  const int tid = threadIdx.x;
  RowAcc<DT, kArgmax> acc;
  stream_segment<DT, kRowThreads, kUnroll>(row, lo, hi, tid, acc);

  __shared__ float lds_m[kRowThreads / kWave], lds_s[kRowThreads / kWave];
  float2 res = acc.result(lds_m, lds_s, tid);
  // A segment with no value above -inf has its first index as the first
  // maximum, so a row of -inf values has argmax 0.
  if constexpr (kArgmax)
    if (__float_as_int(res.y) == INT_MAX) res.y = __int_as_float(lo);
  if (tid == 0) part[(b * rs.R_out + slot) * rs.S + seg] = res;
}

// ---------------------------------------------------------------------------
// Read-bandwidth probe: each workgroup streams one contiguous chunk with the
// same nontemporal 16-byte loads as the row pass, kUnroll loads per thread in
// flight, and folds the words into a checksum.
// ---------------------------------------------------------------------------
constexpr int64_t kProbeChunk = 16384;  // 16-byte vectors per workgroup (256 KiB)

__global__ void __launch_bounds__(kRowThreads) k_probe_read(const uint4 *__restrict__ src, int64_t nvec,
                                                            uint32_t *__restrict__ sink) {
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * kProbeChunk;
  const int64_t n = min(kProbeChunk, nvec - lo);
  const uint4 *p = src + lo;
  uint32_t acc = 0;
  int64_t v0 = 0;
  for (; v0 + kUnroll * kRowThreads <= n; v0 += kUnroll * kRowThreads) {
    uint4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) r[u] = load_stream(p + v0 + u * kRowThreads + threadIdx.x);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  }
  for (int64_t i = v0 + threadIdx.x; i < n; i += kRowThreads) {
    const uint4 r = load_stream(p + i);
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
static void launch_row_stats_t(int dtype, const RowSet &rs, float2 *part, hipStream_t st) {
  const int64_t blocks = static_cast<int64_t>(rs.B) * rs.R * rs.S;
  if (blocks < 1) return;
  const dim3 grid(static_cast<unsigned>(blocks)), block(kRowThreads);
  switch (dtype) {
    case DT_BF16: hipLaunchKernelGGL((k_row_stats<DT_BF16, kArgmax>), grid, block, 0, st, rs, part); break;
    case DT_F16: hipLaunchKernelGGL((k_row_stats<DT_F16, kArgmax>), grid, block, 0, st, rs, part); break;
    default: hipLaunchKernelGGL((k_row_stats<DT_F32, kArgmax>), grid, block, 0, st, rs, part); break;
  }
}

void launch_row_stats(int dtype, bool argmax, const RowSet &rs, float2 *part, hipStream_t st) {
  if (argmax) launch_row_stats_t<true>(dtype, rs, part, st);
  else launch_row_stats_t<false>(dtype, rs, part, st);
}

int probe_blocks(size_t bytes) {
  const int64_t nvec = static_cast<int64_t>(bytes / 16);
  return static_cast<int>((nvec + kProbeChunk - 1) / kProbeChunk);
}

void launch_probe_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t st) {
  const int blocks = probe_blocks(bytes);
  hipLaunchKernelGGL(k_probe_read, dim3(blocks), dim3(kRowThreads), 0, st,
                     reinterpret_cast<const uint4 *>(src), static_cast<int64_t>(bytes / 16), sink);
}

}  // namespace sv
