// LM head fused with verification (gfx950): logits = hidden x unembedding^T
// on the matrix cores, consumed tile by tile by the row statistics, so no
// pass reads the logits back to reduce them.  The same epilogue writes the
// float32 logits out with nontemporal stores, and the sampling pass reads
// only the rows a draw needs, target row n and draft row n of each sequence.
// The writes lengthen the launch in proportion to their bytes, by less than
// a second GEMM over the drawn rows would take.
//
// GEMM: C[M x V] = A[M x K] * W[V x K]^T, bf16 inputs, float32 accumulation in
// v_mfma_f32_32x32x16_bf16.  Block tile 256 x 256, K step 64, 8 waves of 64 x
// 128 (4 along M, 2 along V), double-buffered LDS, one barrier per K step; a
// tile's global loads are issued a whole K step before they are stored to LDS.
// The K loop's issue order is fixed by hand: every MFMA is followed by its
// share of LDS reads, LDS stores and global loads, so the two waves of a SIMD
// keep the matrix core fed while the LDS traffic (the binding resource at
// this wave tile) flows.
// Operand layout of the 32x32x16 instruction (checked on the device): lane l
// supplies A[l % 32][8 (l / 32) + j] and W-row (l % 32) at the same k, j < 8;
// accumulator register r of lane l is C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sv_device.h"
#include "sv_launch.h"
#include "sv_plan.h"

namespace sv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;                   // rows per block
constexpr int kBN = kLmBN;                 // 2 waves along V, 128 columns each
constexpr int kBK = 64;                    // K step: four MFMA sub-steps of 16
constexpr int kWaveM = 64;                 // rows per wave: kBM / kWaveM waves along M
constexpr int kMT = kWaveM / 32;           // 32-row accumulator tiles per wave
constexpr int kWavesM = kBM / kWaveM;
constexpr int kGemmThreads = 64 * kWavesM * 2;
static_assert(kGemmThreads == kLmGemmThreads, "the host checks grids against kLmGemmThreads");
constexpr int kChunksK = kBK / 8;          // 16-byte chunks per row and K step
constexpr int kLoadsA = kBM * kChunksK / kGemmThreads;
constexpr int kLoadsW = kBN * kChunksK / kGemmThreads;
constexpr int kLdsRow = kBK + 8;  // bf16 per LDS row: 16 bytes of padding spread the banks
constexpr int kStageElems = (kBM + kBN) * kLdsRow;
static_assert(kBN == 256, "the wave layout covers 256 columns");

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Block -> tile map: blocks are handed to the 8 XCDs round-robin, so blocks
// L, L + 8, ... share an XCD; those get the row blocks of one column tile in
// turn, and the unembedding tile is read from HBM once per XCD's L2.
__device__ __forceinline__ bool lm_tile(int L, int RB, int NT, int *rb, int *ct) {
  const int xcd = L & 7, slot = L >> 3;
  *ct = xcd + 8 * (slot / RB);
  *rb = slot % RB;
  return *ct < NT;
}

// Lane exchanges within a wave: a DPP move (kCtrl: quad permutation or row
// rotation, within rows of 16 lanes) and lane l ^ 16 within each half-wave.
template <int kCtrl>
__device__ __forceinline__ float lm_dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, true));
}
// Larger of two floats that are never NaN here, without canonicalising
// operands that come from lane exchanges.
__device__ __forceinline__ float lm_max(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float lm_swap16(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}

// One 256 x 256 output tile of problem P; L is the block's index within P.
__device__ __forceinline__ void lm_gemm_tile(const LmGemmArgs &P, int L) {
  __shared__ uint4 lds_raw[2 * kStageElems * sizeof(uint16_t) / sizeof(uint4)];
  uint16_t *lds = reinterpret_cast<uint16_t *>(lds_raw);
  __shared__ float2 s_red[2][kBM];
  __shared__ int s_tok[kBM];
  __shared__ float s_gath[kBM + 64];
  int rb, ct;
  if (!lm_tile(L, P.RB, P.NT, &rb, &ct)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % kWavesM, wn = wave / kWavesM;
  const int half = lane >> 5, c32 = lane & 31;
  const int row0 = rb * kBM, col0 = ct * kBN;

  // this thread's A and W chunks of every K step (chunk q = tid + threads * j)
  const uint4 *asrc[kLoadsA], *wsrc[kLoadsW];
  int aoff[kLoadsA], woff[kLoadsW];
#pragma unroll
  for (int j = 0; j < kLoadsA; ++j) {
    const int q = tid + kGemmThreads * j;
    const int r = q / kChunksK, ch = q % kChunksK;
    const int gr = row0 + r;
    const int64_t arow = gr < P.M ? gr : 0;
    asrc[j] = reinterpret_cast<const uint4 *>(P.A + arow * P.lda + ch * 8);
    aoff[j] = r * kLdsRow + ch * 8;
  }
#pragma unroll
  for (int j = 0; j < kLoadsW; ++j) {
    const int q = tid + kGemmThreads * j;
    const int r = q / kChunksK, ch = q % kChunksK;
    const int gc = col0 + r;
    wsrc[j] = reinterpret_cast<const uint4 *>(P.W + static_cast<int64_t>(gc < P.V ? gc : 0) * P.K + ch * 8);
    woff[j] = kBM * kLdsRow + r * kLdsRow + ch * 8;
  }
  if (tid < kBM) {
    const int g = row0 + tid;
    int x = -1;
    if (g < P.M) {
      const int b = g / P.rows_per_seq, i = g - b * P.rows_per_seq;
      if (i < P.gamma) x = P.tokens[static_cast<int64_t>(b) * P.gamma + i];
    }
    s_tok[tid] = x;
  }

  f32x16_t acc[kMT][4];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mt][nt][e] = 0.0f;

  // Rows past M (A) or V (W) load row 0, in bounds; their products land in
  // accumulator rows that are never stored and columns the epilogues mask.
  uint4 ra[kLoadsA], rw[kLoadsW];
  bf16x8_t a[2][kMT], w[2][4];  // operand fragments of two sub-steps
  const int nk = P.K / kBK;
  // Load item j of a tile (j < kLoadsA: A chunk, else W chunk) at K offset
  // k0 into the staging registers, store it to LDS stage st, and read
  // fragment f of sub-step ks of stage st (f = 0: A tile 0, 1..4: W tiles
  // 0..3, 5..: A tiles 1..) into slot.
#define SV_LM_LOAD1(j, k0)                                            \
  {                                                                   \
    if ((j) < kLoadsA)                                                \
      ra[j] = load_vec(asrc[j] + (k0) / 8);                           \
    else                                                              \
      rw[(j) - kLoadsA] = load_vec(wsrc[(j) - kLoadsA] + (k0) / 8);   \
  }
#define SV_LM_STORE1(j, st)                                                                       \
  {                                                                                               \
    if ((j) < kLoadsA)                                                                            \
      *reinterpret_cast<uint4 *>(lds + (st) * kStageElems + aoff[j]) = ra[j];                     \
    else                                                                                          \
      *reinterpret_cast<uint4 *>(lds + (st) * kStageElems + woff[(j) - kLoadsA]) = rw[(j) - kLoadsA]; \
  }
#define SV_LM_FRAG(slot, st, ks, f)                                                                        \
  {                                                                                                        \
    const uint16_t *sa_ = lds + (st) * kStageElems + (wm * kWaveM + c32) * kLdsRow + 8 * half + (ks) * 16; \
    const uint16_t *sw_ =                                                                                  \
        lds + (st) * kStageElems + kBM * kLdsRow + (wn * 128 + c32) * kLdsRow + 8 * half + (ks) * 16;      \
    if ((f) == 0)                                                                                          \
      a[slot][0] = as_bf16x8(*reinterpret_cast<const uint4 *>(sa_));                                       \
    else if ((f) <= 4)                                                                                     \
      w[slot][(f) - 1] = as_bf16x8(*reinterpret_cast<const uint4 *>(sw_ + ((f) - 1) * 32 * kLdsRow));      \
    else                                                                                                   \
      a[slot][(f) - 4] = as_bf16x8(*reinterpret_cast<const uint4 *>(sa_ + ((f) - 4) * 32 * kLdsRow));      \
  }
  // One sub-step: the MFMAs of slot cur, in a fixed issue order.  The reads
  // of the next sub-step's fragments (stage st_r, sub-step ks_r, into slot
  // nxt) go out two after each of the first MFMAs; with tile set, each MFMA
  // is also followed by its share of the tile hand-over: store an item of the
  // tile fetched a step earlier to stage st_w, then fetch the same item two
  // steps ahead (K offset k0).  The fences keep the scheduler from moving
  // anything across them.
#define SV_LM_SUBSTEP(cur, nxt, st_r, ks_r, tile, st_w, k0)                                                   \
  _Pragma("unroll") for (int i_ = 0; i_ < kSubMfma; ++i_) {                                                   \
    acc[i_ / 4][i_ % 4] =                                                                                     \
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][i_ / 4], w[cur][i_ % 4], acc[i_ / 4][i_ % 4], 0, 0, 0); \
    _Pragma("unroll") for (int f_ = 2 * i_; f_ < 2 * i_ + 2; ++f_) if (f_ < kSubFrags)                        \
        SV_LM_FRAG(nxt, st_r, ks_r, f_)                                                                       \
    if (tile)                                                                                                 \
      _Pragma("unroll") for (int j_ = i_ * kTileItems / kSubMfma; j_ < (i_ + 1) * kTileItems / kSubMfma; ++j_) { \
        SV_LM_STORE1(j_, st_w)                                                                                \
        SV_LM_LOAD1(j_, k0)                                                                                   \
      }                                                                                                       \
    __builtin_amdgcn_sched_barrier(0);                                                                        \
  }
  constexpr int kSubMfma = kMT * 4, kSubFrags = kMT + 4, kTileItems = kLoadsA + kLoadsW;
  static_assert(kSubFrags <= 2 * kSubMfma && kTileItems <= 2 * kSubMfma, "a sub-step carries the hand-over");

  // Prologue: tile 0 to stage 0, tile 1 in the registers, the first fragments.
#pragma unroll
  for (int j = 0; j < kTileItems; ++j) SV_LM_LOAD1(j, 0)
#pragma unroll
  for (int j = 0; j < kTileItems; ++j) SV_LM_STORE1(j, 0)
#pragma unroll
  for (int j = 0; j < kTileItems; ++j) SV_LM_LOAD1(j, (nk > 1 ? kBK : 0))
  __syncthreads();
#pragma unroll
  for (int f = 0; f < kSubFrags; ++f) SV_LM_FRAG(0, 0, 0, f)
  __builtin_amdgcn_sched_barrier(0);
  // K step kt multiplies stage st = kt & 1 in four sub-steps of 16.  Sub-step
  // 1 stores the tile of step kt + 1 (fetched during step kt - 1) to stage
  // st ^ 1 and fetches the tile of step kt + 2.  One barrier, after sub-step
  // 2, separates every wave's last read of stage st and its stores to stage
  // st ^ 1 from the reads of stage st ^ 1 and, one step later, from the
  // stores that overwrite stage st; sub-step 3 multiplies from registers and
  // meanwhile reads the next stage's first fragments.  The last steps store
  // and fetch tiles nobody reads (K offsets clamped in range), so the loop
  // body has no branches.
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    const int kf = min(kt + 2, nk - 1) * kBK;
    SV_LM_SUBSTEP(0, 1, st, 1, false, 0, 0)
    SV_LM_SUBSTEP(1, 0, st, 2, true, st ^ 1, kf)
    SV_LM_SUBSTEP(0, 1, st, 3, false, 0, 0)
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    SV_LM_SUBSTEP(1, 0, st ^ 1, 0, false, 0, 0)
  }
#undef SV_LM_SUBSTEP
#undef SV_LM_FRAG
#undef SV_LM_STORE1
#undef SV_LM_LOAD1

  // Row statistics of this wave's 128 columns: max, then sum of exp(x - max)
  // (the same 2^(x log2e - m log2e) form as the streaming row pass), across
  // the 32 lanes of each half-wave: within each row of 16 lanes by DPP
  // (swap neighbours, swap pairs, rotate by 4 and by 8), then across the two
  // rows of the half by a swizzle.  Lane j of a half keeps the result of the
  // half's j-th row (and row j + 32 with four row tiles), so the loop has no
  // branches and one LDS store per lane ends it.  The lane holding a row's
  // draft-token column leaves that logit in s_gath (other lanes write a
  // scratch slot of their own).  Each lane also writes its logits of rows
  // below M: 32 consecutive columns per half-wave and store.
  const bool full = col0 + kBN <= P.V;
  const int cbase = col0 + wn * 128 + c32;
  constexpr int kKeep = kMT / 2;
  float keep_m[kKeep], keep_s[kKeep];
#pragma unroll
  for (int q = 0; q < kKeep; ++q) {
    keep_m[q] = kNegInf;
    keep_s[q] = 0.0f;
  }
  auto rows = [&](auto masked) {
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = wm * kWaveM + mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      float v[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        v[nt] = (!decltype(masked)::value || cbase + nt * 32 < P.V) ? acc[mt][nt][r] : kNegInf;
      if (row0 + rl < P.M) {
        float *orow = P.out + static_cast<int64_t>(row0 + rl) * P.V + cbase;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          if (!decltype(masked)::value || cbase + nt * 32 < P.V) __builtin_nontemporal_store(acc[mt][nt][r], orow + nt * 32);
      }
      float m = lm_max(lm_max(v[0], v[1]), lm_max(v[2], v[3]));
      m = lm_max(m, lm_dpp<0xB1>(m));
      m = lm_max(m, lm_dpp<0x4E>(m));
      m = lm_max(m, lm_dpp<0x124>(m));
      m = lm_max(m, lm_dpp<0x128>(m));
      m = lm_max(m, lm_swap16(m));
      const float ml = m != kNegInf ? m * kLog2e : 0.0f;
      float s = 0.0f;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) s += exp_shift(v[nt], ml);
      s += lm_dpp<0xB1>(s);
      s += lm_dpp<0x4E>(s);
      s += lm_dpp<0x124>(s);
      s += lm_dpp<0x128>(s);
      s += lm_swap16(s);
      const int j = mt * 16 + r;
      keep_m[j / 32] = c32 == j % 32 ? m : keep_m[j / 32];
      keep_s[j / 32] = c32 == j % 32 ? s : keep_s[j / 32];
      const int d = s_tok[rl] - cbase;
      float g = acc[mt][0][r];
      g = d == 32 ? acc[mt][1][r] : g;
      g = d == 64 ? acc[mt][2][r] : g;
      g = d == 96 ? acc[mt][3][r] : g;
      const bool hit = d >= 0 && d < 128 && (d & 31) == 0;
      s_gath[hit ? rl : kBM + lane] = g;
    }
  };
  if (full)  // every column of the tile lies inside the vocabulary
    rows(std::false_type{});
  else
    rows(std::true_type{});
#pragma unroll
  for (int q = 0; q < kKeep; ++q) {
    const int j = 32 * q + c32, mt = j / 16, r = j % 16;
    s_red[wn][wm * kWaveM + mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3)] = make_float2(keep_m[q], keep_s[q]);
  }
  __syncthreads();
  if (tid < kBM && row0 + tid < P.M) {
    const float2 p0 = s_red[0][tid], p1 = s_red[1][tid];
    const MaxSum c = combine(MaxSum{p0.x, p0.y}, MaxSum{p1.x, p1.y});
    P.part[static_cast<int64_t>(row0 + tid) * P.NT + ct] = make_float2(c.m, c.s);
    const int x = s_tok[tid];
    if (x >= col0 && x < col0 + kBN) P.gath[row0 + tid] = s_gath[tid];
  }
}

// Two GEMM problems in one launch (target and draft rows, the same column
// tiles): blocks [0, blocks0) take P0, the rest P1, so the last rounds run
// the tiles with fewer K steps when the draft's hidden width is smaller.
// blocks0 is a multiple of 8, so both problems keep the XCD-aware tile map.
__global__ void __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(kGemmThreads / 256)))
k_lm_gemm(LmGemmArgs P0, LmGemmArgs P1) {
  const int blocks0 = 8 * ((P0.NT + 7) / 8) * P0.RB;
  const int L = blockIdx.x;
  if (L < blocks0)
    lm_gemm_tile(P0, L);
  else
    lm_gemm_tile(P1, L - blocks0);
}

// Per row, the column-tile partials in a fixed order: lane-strided, then the
// wave reduction.  One wave per row.
__global__ void __launch_bounds__(256) k_lm_combine(const float2 *__restrict__ part, int NT, int M,
                                                    float2 *__restrict__ stats) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  MaxSum a{kNegInf, 0.0f};
  const float2 *p = part + static_cast<int64_t>(row) * NT;
  for (int c = lane; c < NT; c += kWave) {
    const float2 q = p[c];
    a = combine(a, MaxSum{q.x, q.y});
  }
  a = wave_reduce(a);
  if (lane == 0) stats[row] = make_float2(a.m, a.s);
}

__device__ __forceinline__ float lm_prob(float x, float2 st) {
  return exp_shift(x, st.x * kLog2e) / st.y;
}
__device__ __forceinline__ float lm_offset(float2 st) { return st.x * kLog2e + log2f(st.y); }

// Window decision from the fused statistics (one wave per sequence, lane i =
// position i): p_i(x_i), q_i(x_i) from the row statistics and the logits at the
// draft tokens; accept iff u q < p; the first rejection ends the window.
// Writes the window outputs and the sampling job, which points at target row
// n and draft row n of the logits the GEMM wrote.
__global__ void __launch_bounds__(kWave) k_lm_decide(LmDecideArgs A) {
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  if (i == 0) A.arrive[b] = 0;  // arrival counter of this sequence's draw
  const int g = A.gamma;
  int32_t *out = A.out_tokens + static_cast<int64_t>(b) * (g + 1);
  const int len = A.window_len ? A.window_len[b] : g;
  const int x = i < g ? A.tokens[static_cast<int64_t>(b) * g + i] : 0;
  // the ids and the statistics and token logits of rows i go out with the
  // token loads, before the window is checked (values of an invalid
  // sequence, or past its window, are not used)
  const uint64_t seq = A.seq_ids ? A.seq_ids[b] : static_cast<uint64_t>(b);
  const int64_t base = A.base_pos ? A.base_pos[b] : 0;
  const int64_t rt = static_cast<int64_t>(b) * (g + 1), rd = static_cast<int64_t>(b) * g;
  float2 sti{0.0f, 1.0f}, sdi{0.0f, 1.0f};
  float gti = 0.0f, gdi = 0.0f;
  if (i < g) {
    sti = A.stats_t[rt + i];
    gti = A.gath_t[rt + i];
    sdi = A.stats_d[rd + i];
    gdi = A.gath_d[rd + i];
  }
  const bool bad_len = len < 0 || len > g;
  const bool bad_tok = !bad_len && i < len && (x < 0 || x >= A.V);
  if (__any(bad_len || bad_tok)) {
    for (int k = i; k <= g; k += kWave) out[k] = -1;
    for (int k = i; k < g; k += kWave) {
      if (A.p_draft) A.p_draft[static_cast<int64_t>(b) * g + k] = 0.0f;
      if (A.q_draft) A.q_draft[static_cast<int64_t>(b) * g + k] = 0.0f;
    }
    if (i == 0) {
      A.n_accepted[b] = -1;
      A.jobs[b].mode = JOB_NONE;
    }
    return;
  }
  const U64x4 w = philox4x64_10({seq, static_cast<uint64_t>(base + 1 + i), 0, 0}, A.seed, A.tag);
  float P = 0.0f, Q = 0.0f;
  bool acc = false;
  if (i < len) {
    P = lm_prob(gti, sti);
    Q = lm_prob(gdi, sdi);
    acc = uniform24(w.c0) * Q < P;
  }
  const uint64_t inv = ~static_cast<uint64_t>(__ballot(acc));
  int n = inv ? __builtin_ctzll(inv) : kWave;
  n = min(n, len);
  if (i < g) {
    if (A.p_draft) A.p_draft[rd + i] = P;
    if (A.q_draft) A.q_draft[rd + i] = Q;
  }
  for (int k = i; k <= g; k += kWave)
    if (k != n) out[k] = k < n ? A.tokens[rd + k] : -1;
  float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(uniform24(w.c1)), n & (kWave - 1)));
  if (i == 0) {
    if (n >= kWave) {  // gamma = 64 with every draft accepted: position 64 has no lane
      const U64x4 w2 = philox4x64_10({seq, static_cast<uint64_t>(base + 1 + n), 0, 0}, A.seed, A.tag);
      v = uniform24(w2.c1);
    }
    SampleJob jb{};
    jb.t_row = A.rows_t + (rt + n) * A.V;
    jb.ct = lm_offset(A.stats_t[rt + n]);
    if (n < len) {
      jb.mode = JOB_RESIDUAL;
      jb.d_row = A.rows_d + (rd + n) * A.V;
      jb.cd = lm_offset(A.stats_d[rd + n]);
      jb.cq = 1.0f;
    } else {
      jb.mode = JOB_BONUS;
      jb.d_row = nullptr;
    }
    jb.v = v;
    jb.out_slot = out + n;
    A.jobs[b] = jb;
    A.n_accepted[b] = n;
  }
}

int64_t lm_gemm_blocks(int64_t M, int V) {
  const int64_t RB = (M + kBM - 1) / kBM, NT = (V + kBN - 1) / kBN;
  return 8 * ((NT + 7) / 8) * RB;
}

void launch_lm_gemm(LmGemmArgs A0, LmGemmArgs A1, hipStream_t st) {
  A0.RB = (A0.M + kBM - 1) / kBM;
  A0.NT = (A0.V + kBN - 1) / kBN;
  A1.RB = (A1.M + kBM - 1) / kBM;
  A1.NT = (A1.V + kBN - 1) / kBN;
  const int64_t blocks = lm_gemm_blocks(A0.M, A0.V) + lm_gemm_blocks(A1.M, A1.V);
  hipLaunchKernelGGL(k_lm_gemm, dim3(static_cast<unsigned>(blocks)), dim3(kGemmThreads), 0, st, A0, A1);
}

void launch_lm_combine(const float2 *part, int NT, int M, float2 *stats, hipStream_t st) {
  hipLaunchKernelGGL(k_lm_combine, dim3((M + 3) / 4), dim3(256), 0, st, part, NT, M, stats);
}

void launch_lm_decide(const LmDecideArgs &A, int B, hipStream_t st) {
  hipLaunchKernelGGL(k_lm_decide, dim3(B), dim3(kWave), 0, st, A);
}

}  // namespace sv
