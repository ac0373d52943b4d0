// Device helpers of the verification kernels (gfx950, wave64).
//
// Logit decoding, the Philox4x64-10 uniform stream, and the fixed-order
// (max, sum-exp) / (max, first-index) combines used by every reduction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

// Pointers known to address global memory (address space 1): loads through
// them compile to global_load rather than flat_load, also when the pointer
// value was read from LDS.
#define SV_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ const SV_GLOBAL T *as_global(const T *p) {
  return reinterpret_cast<const SV_GLOBAL T *>(reinterpret_cast<uintptr_t>(p));
}
template <typename T>
__device__ __forceinline__ const SV_GLOBAL T *as_global(const void *p) {
  return reinterpret_cast<const SV_GLOBAL T *>(reinterpret_cast<uintptr_t>(p));
}

// 16-byte streaming load with the nontemporal hint: logits are read once per
// pass, and the hint lifts sustained HBM read bandwidth on gfx950.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4 *p) {
  const u32x4_t v = __builtin_nontemporal_load(as_global<u32x4_t>(static_cast<const void *>(p)));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 load_vec(const void *p) {
  const u32x4_t v = *as_global<u32x4_t>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------
// Logit decoding.  A 16-byte vector holds EPV elements; decoding is exact.
// ---------------------------------------------------------------------------
template <int DT> struct Elt;

template <> struct Elt<DT_BF16> {
  static constexpr int kBytes = 2;
  static constexpr int kEPV = 8;
  static constexpr uint32_t kNegInfPair = 0xFF80FF80u;  // two bf16 -inf
  // raw(): the element's bits, dec(): their value; one() = dec(raw()).
  __device__ static __forceinline__ uint32_t raw(const void *row, int64_t i) { return as_global<uint16_t>(row)[i]; }
  __device__ static __forceinline__ float dec(uint32_t r) { return __uint_as_float(r << 16); }
  __device__ static __forceinline__ float one(const void *row, int64_t i) { return dec(raw(row, i)); }
  __device__ static __forceinline__ void vec(const uint4 &r, float *x) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(w[k] << 16);
      x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  }
};

template <> struct Elt<DT_F16> {
  static constexpr int kBytes = 2;
  static constexpr int kEPV = 8;
  static constexpr uint32_t kNegInfPair = 0xFC00FC00u;  // two f16 -inf
  __device__ static __forceinline__ float h2f(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
  }
  __device__ static __forceinline__ uint32_t raw(const void *row, int64_t i) { return as_global<uint16_t>(row)[i]; }
  __device__ static __forceinline__ float dec(uint32_t r) { return h2f(r); }
  __device__ static __forceinline__ float one(const void *row, int64_t i) { return dec(raw(row, i)); }
  __device__ static __forceinline__ void vec(const uint4 &r, float *x) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = h2f(w[k] & 0xFFFFu);
      x[2 * k + 1] = h2f(w[k] >> 16);
    }
  }
};

template <> struct Elt<DT_F32> {
  static constexpr int kBytes = 4;
  static constexpr int kEPV = 4;
  static constexpr uint32_t kNegInfPair = 0xFF800000u;  // one f32 -inf
  __device__ static __forceinline__ uint32_t raw(const void *row, int64_t i) { return as_global<uint32_t>(row)[i]; }
  __device__ static __forceinline__ float dec(uint32_t r) { return __uint_as_float(r); }
  __device__ static __forceinline__ float one(const void *row, int64_t i) { return dec(raw(row, i)); }
  __device__ static __forceinline__ void vec(const uint4 &r, float *x) {
    x[0] = __uint_as_float(r.x);
    x[1] = __uint_as_float(r.y);
    x[2] = __uint_as_float(r.z);
    x[3] = __uint_as_float(r.w);
  }
};


// 2^x on the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// exp(x - m) evaluated as 2^(x*log2e - m*log2e); every kernel uses this one
// form so numerators and normalisers carry the same rounding of m*log2e.
__device__ __forceinline__ float exp_shift(float x, float m_log2e) {
  return exp2_fast(__builtin_fmaf(x, kLog2e, -m_log2e));
}

// ---------------------------------------------------------------------------
// Combines of per-lane results (row maximum with the sum of exponentials, or
// maximum with its first index).  The comparisons are exact; the wave
// reductions below apply them in a fixed order.
// ---------------------------------------------------------------------------
struct MaxSum {
  float m, s;
};

// Rescale factor 2^((from - to) log2e) = exp(from - to) for from <= to.  It is
// taken from the difference of the two maxima, so the side that already holds
// the maximum is multiplied by exactly 1 and repeated combines add no bias.
__device__ __forceinline__ float rescale(float from, float to) { return exp2_fast((from - to) * kLog2e); }

__device__ __forceinline__ MaxSum combine(MaxSum a, MaxSum b) {
  const float m = fmaxf(a.m, b.m);
  if (m == kNegInf) return {kNegInf, 0.0f};
  return {m, a.s * rescale(a.m, m) + b.s * rescale(b.m, m)};
}

struct MaxIdx {
  float m;
  int i;
};

__device__ __forceinline__ MaxIdx combine(MaxIdx a, MaxIdx b) {
  return (b.m > a.m || (b.m == a.m && b.i < a.i)) ? b : a;
}

// Wave reductions: within each row of 16 lanes by DPP moves (swap neighbours,
// swap pairs, rotate by 4, by 8), then the four row results, read from lanes
// 0, 16, 32 and 48, combined in that order; every lane gets the result.  Every
// lane must be active.  DPP moves and lane reads take a few cycles where a
// butterfly of lane shuffles goes through LDS once per step.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, true));
}
template <int kCtrl>
__device__ __forceinline__ int dpp_i32(int x) {
  return __builtin_amdgcn_update_dpp(0, x, kCtrl, 0xF, 0xF, true);
}
__device__ __forceinline__ float read_lane_f32(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

template <int kCtrl>
__device__ __forceinline__ MaxSum dpp_step(MaxSum v) {
  return combine(v, MaxSum{dpp_f32<kCtrl>(v.m), dpp_f32<kCtrl>(v.s)});
}
__device__ __forceinline__ MaxSum wave_reduce(MaxSum v) {
  v = dpp_step<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_step<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_step<0x124>(v);  // row_ror 4
  v = dpp_step<0x128>(v);  // row_ror 8
  const MaxSum r0{read_lane_f32(v.m, 0), read_lane_f32(v.s, 0)};
  const MaxSum r1{read_lane_f32(v.m, 16), read_lane_f32(v.s, 16)};
  const MaxSum r2{read_lane_f32(v.m, 32), read_lane_f32(v.s, 32)};
  const MaxSum r3{read_lane_f32(v.m, 48), read_lane_f32(v.s, 48)};
  return combine(combine(r0, r1), combine(r2, r3));
}

template <int kCtrl>
__device__ __forceinline__ MaxIdx dpp_step(MaxIdx v) {
  return combine(v, MaxIdx{dpp_f32<kCtrl>(v.m), dpp_i32<kCtrl>(v.i)});
}
__device__ __forceinline__ MaxIdx wave_reduce(MaxIdx v) {
  v = dpp_step<0xB1>(v);
  v = dpp_step<0x4E>(v);
  v = dpp_step<0x124>(v);
  v = dpp_step<0x128>(v);
  const MaxIdx r0{read_lane_f32(v.m, 0), __builtin_amdgcn_readlane(v.i, 0)};
  const MaxIdx r1{read_lane_f32(v.m, 16), __builtin_amdgcn_readlane(v.i, 16)};
  const MaxIdx r2{read_lane_f32(v.m, 32), __builtin_amdgcn_readlane(v.i, 32)};
  const MaxIdx r3{read_lane_f32(v.m, 48), __builtin_amdgcn_readlane(v.i, 48)};
  return combine(combine(r0, r1), combine(r2, r3));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// ---------------------------------------------------------------------------
// Philox4x64-10 (Salmon et al., SC'11): two 64x64->128 multiplies per round,
// Weyl key schedule, 10 rounds.
// ---------------------------------------------------------------------------
struct U64x4 {
  uint64_t c0, c1, c2, c3;
};

__device__ __forceinline__ U64x4 philox4x64_10(U64x4 c, uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(M0, c.c0), lo0 = M0 * c.c0;
    const uint64_t hi1 = __umul64hi(M1, c.c2), lo1 = M1 * c.c2;
    c = {hi1 ^ c.c1 ^ k0, lo1, hi0 ^ c.c3 ^ k1, lo0};
    k0 += W0;
    k1 += W1;
  }
  return c;
}

// Top 24 bits of a word on the 2^-24 grid: exact in float32.
__device__ __forceinline__ float uniform24(uint64_t w) {
  return static_cast<float>(static_cast<uint32_t>(w >> 40)) * 0x1p-24f;
}

}  // namespace sv
