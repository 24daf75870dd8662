// device.hpp - gfx950 device helpers for the SMC-SD verify / resample / KV kernels.
//
// Wave64 throughout: reductions and scans use 64-lane shuffles, then LDS across the
// waves of a workgroup.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/smcsd.h"

namespace smcsd {

constexpr int kWave = 64;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr double kLn2 = 0.693147180559945309417232121458176568;
constexpr double kLog2e = 1.442695040888963407359924681001892137;

// ---------------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11).  Each of the ten rounds takes
// the 64-bit products of counter words 0 and 2 with the two round multipliers; the
// new counter is (hi(w2*M1) ^ w1 ^ k0, lo(w2*M1), hi(w0*M0) ^ w3 ^ k1, lo(w0*M0)).
// The key advances by the two Weyl increments after every round.
// ---------------------------------------------------------------------------------
// Each 64-bit product is one v_mad_u64_u32 (both halves at once) instead of a mul_lo and
// a mul_hi.
__device__ __forceinline__ void philox_block(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)c[0] * 0xD2511F53u;
    const uint64_t p1 = (uint64_t)c[2] * 0xCD9E8D57u;
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    c[0] = hi1 ^ c[1] ^ k0;
    c[1] = lo1;
    c[2] = hi0 ^ c[3] ^ k1;
    c[3] = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

// Counter layout: (stream index, step low, step high, tag); key: (seed low, seed high).
// The uniform keeps the top 24 bits of one output word: exact in fp32 and fp64.
__device__ __forceinline__ double philox_uniform(uint64_t seed, uint32_t index, uint64_t step,
                                                 uint32_t tag, int word) {
  uint32_t c[4] = {index, (uint32_t)step, (uint32_t)(step >> 32), tag};
  philox_block(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  const uint32_t w = word == 0 ? c[0] : word == 1 ? c[1] : word == 2 ? c[2] : c[3];
  return (double)(w >> 8) * (1.0 / 16777216.0);
}

// ---------------------------------------------------------------------------------
// element access
// ---------------------------------------------------------------------------------
template <int DT> struct Elt;
template <> struct Elt<SMCSD_DTYPE_F32> {
  static constexpr int kBytes = 4;
  static constexpr int kPerVec = 4;  // elements per 16-byte vector
  __device__ __forceinline__ static float load(const char *row, int64_t v) {
    return reinterpret_cast<const float *>(row)[v];
  }
  __device__ __forceinline__ static void unpack(const uint4 &w, float *x) {
    x[0] = __uint_as_float(w.x);
    x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z);
    x[3] = __uint_as_float(w.w);
  }
};
template <> struct Elt<SMCSD_DTYPE_BF16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
  __device__ __forceinline__ static float load(const char *row, int64_t v) {
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(row)[v] << 16);
  }
  // bf16 is the upper half of an fp32: widening is a shift or a mask.
  __device__ __forceinline__ static void unpack(const uint4 &w, float *x) {
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xFFFF0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xFFFF0000u);
    x[4] = __uint_as_float(w.z << 16);
    x[5] = __uint_as_float(w.z & 0xFFFF0000u);
    x[6] = __uint_as_float(w.w << 16);
    x[7] = __uint_as_float(w.w & 0xFFFF0000u);
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte streaming load that does not keep the line in the caches (the logits are read
// once per step; a read-only stream measured ~7.0 TB/s this way versus ~6.3 TB/s with
// ordinary loads on the MI355X).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4 *p) {
  const u32x4_t r = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(r.x, r.y, r.z, r.w);
}

// The same streaming load through a buffer resource: the resource holds a wave-uniform
// base and size, the lane supplies a 32-bit byte offset and the instruction a uniform one,
// so a group of loads needs no per-lane 64-bit address arithmetic.  Offsets past the
// resource's size would read zeros (no fault); callers keep every offset inside it.
constexpr int kBufRsrcWord3 = 0x00020000;  // raw (untyped) buffer, 32-bit data format
constexpr int kBufNonTemporal = 2;         // cache-policy operand: nt
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, kBufRsrcWord3);
}
__device__ __forceinline__ uint4 load_stream(__amdgpu_buffer_rsrc_t rs, int lane_off, int uni_off) {
  const u32x4_t r = __builtin_amdgcn_raw_buffer_load_b128(rs, lane_off, uni_off, kBufNonTemporal);
  return make_uint4(r.x, r.y, r.z, r.w);
}

// -inf in every element of a 16-byte vector (fills the lanes past a row's end)
template <int DT> struct NegInfVec;
template <> struct NegInfVec<SMCSD_DTYPE_F32> {
  __device__ __forceinline__ static uint4 get() {
    return make_uint4(0xFF800000u, 0xFF800000u, 0xFF800000u, 0xFF800000u);
  }
};
template <> struct NegInfVec<SMCSD_DTYPE_BF16> {
  __device__ __forceinline__ static uint4 get() {
    return make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u);
  }
};

// ---------------------------------------------------------------------------------
// Online log-sum-exp state over raw logits x with scale c = log2(e) / T:
//   m  = running max of x,   mc = m * c (rounded once, reused everywhere),
//   s  = sum 2^(x*c - mc).
// -inf logits add exactly 0; a NaN or +inf logit turns s into NaN, which the
// consumers report as NAN_INPUT.  mc is 0 while m is -inf.
// ---------------------------------------------------------------------------------
struct Lse {
  float m, mc, s;
};

__device__ __forceinline__ Lse lse_init() { return Lse{kNegInf, 0.0f, 0.0f}; }

template <int NV>
__device__ __forceinline__ void lse_update(Lse &st, const float (&x)[NV], float c) {
  float vmax = x[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) vmax = fmaxf(vmax, x[i]);
  if (vmax > st.m) {
    const float mcn = __fmul_rn(vmax, c);
    st.s = (st.m == kNegInf) ? st.s * 0.0f : st.s * fast_exp2(st.mc - mcn);
    st.m = vmax;
    st.mc = mcn;
  }
  float e[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) e[i] = fast_exp2(fmaf(x[i], c, -st.mc));
  // pairwise tree keeps the dependency chain short
#pragma unroll
  for (int w = 1; w < NV; w *= 2)
#pragma unroll
    for (int i = 0; i + w < NV; i += 2 * w) e[i] += e[i + w];
  st.s += e[0];
}

// lse_update over NV elements that also hands back gs[q], the sum of 2^(x*c - mc) over the
// q-th run of G consecutive elements, relative to the updated mc.  The pairwise tree first
// sums each run, then the runs: the same tree, and total, as lse_update.
template <int NV, int G>
__device__ __forceinline__ void lse_update_g(Lse &st, const float (&x)[NV], float c,
                                             float (&gs)[NV / G]) {
  float vmax = x[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) vmax = fmaxf(vmax, x[i]);
  if (vmax > st.m) {
    const float mcn = __fmul_rn(vmax, c);
    st.s = (st.m == kNegInf) ? st.s * 0.0f : st.s * fast_exp2(st.mc - mcn);
    st.m = vmax;
    st.mc = mcn;
  }
#pragma unroll
  for (int q = 0; q < NV / G; ++q) {
    float e[G];
#pragma unroll
    for (int i = 0; i < G; ++i) e[i] = fast_exp2(fmaf(x[q * G + i], c, -st.mc));
#pragma unroll
    for (int w = 1; w < G; w *= 2)
#pragma unroll
      for (int i = 0; i + w < G; i += 2 * w) e[i] += e[i + w];
    gs[q] = e[0];
  }
  float t[NV / G];
#pragma unroll
  for (int q = 0; q < NV / G; ++q) t[q] = gs[q];
#pragma unroll
  for (int w = 1; w < NV / G; w *= 2)
#pragma unroll
    for (int q = 0; q + w < NV / G; q += 2 * w) t[q] += t[q + w];
  st.s += t[0];
}

__device__ __forceinline__ Lse lse_combine(const Lse &a, const Lse &b, float c) {
  const float M = fmaxf(a.m, b.m);
  if (M == kNegInf) return Lse{kNegInf, 0.0f, a.s + b.s};
  const float Mc = __fmul_rn(M, c);
  const float ta = (a.m == kNegInf) ? a.s * 0.0f : a.s * fast_exp2(a.mc - Mc);
  const float tb = (b.m == kNegInf) ? b.s * 0.0f : b.s * fast_exp2(b.mc - Mc);
  return Lse{M, Mc, ta + tb};
}

__device__ __forceinline__ Lse lse_shfl_xor(const Lse &a, int mask) {
  return Lse{__shfl_xor(a.m, mask, kWave), __shfl_xor(a.mc, mask, kWave),
             __shfl_xor(a.s, mask, kWave)};
}

// Workgroup reduction of the online state; the result is valid in thread 0.
template <int BLOCK>
__device__ __forceinline__ Lse lse_block_reduce(Lse st, float c, Lse *lds) {
#pragma unroll
  for (int mask = 1; mask < kWave; mask <<= 1) st = lse_combine(st, lse_shfl_xor(st, mask), c);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  if (lane == 0) lds[wave] = st;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < BLOCK / kWave; ++w) st = lse_combine(st, lds[w], c);
  }
  return st;
}

// ---------------------------------------------------------------------------------
// scans and sums
// ---------------------------------------------------------------------------------
// fp64 values moved across lanes by DPP, as two 32-bit halves; lanes whose source is
// outside the pattern, or whose row is not in ROW_MASK, read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_d(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)b, CTRL, ROW_MASK, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(b >> 32), CTRL, ROW_MASK, 0xf, true);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}
// Inclusive scan over the 64 lanes: shifts of 1, 2, 4 and 8 lanes within each row of 16,
// then the last lane of row 0 (and of row 2) added to row 1 (and row 3), then lane 31 added
// to rows 2 and 3.
__device__ __forceinline__ double wave_inclusive_scan(double v) {
  v += dpp_d<0x111, 0xf>(v);  // row_shr:1
  v += dpp_d<0x112, 0xf>(v);  // row_shr:2
  v += dpp_d<0x114, 0xf>(v);  // row_shr:4
  v += dpp_d<0x118, 0xf>(v);  // row_shr:8
  v += dpp_d<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_d<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}
// The same scan for 32-bit integers: one DPP move per step (integer sums are exact, so the
// result does not depend on the order of the additions).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, true);
}
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += dpp_i<0x111, 0xf>(v);  // row_shr:1
  v += dpp_i<0x112, 0xf>(v);  // row_shr:2
  v += dpp_i<0x114, 0xf>(v);  // row_shr:4
  v += dpp_i<0x118, 0xf>(v);  // row_shr:8
  v += dpp_i<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_i<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}
// The sum over the 64 lanes, in every lane: the scan's last lane, read as a uniform value.
__device__ __forceinline__ double wave_sum(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(wave_inclusive_scan(v));
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, kWave - 1);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), kWave - 1);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// 32-bit values moved across lanes by DPP.  dpp_f: lanes whose source is outside the
// pattern, or whose row is not in ROW_MASK, read 0 (for sums); dpp_f_keep: they read
// their own value (for maxima).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, true));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f_keep(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
// The sum (max) over the 64 lanes, in every lane: the DPP scan pattern above, then the
// last lane read as a uniform value.  A fixed order, so the same bits every time.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f<0x111, 0xf>(v);
  v += dpp_f<0x112, 0xf>(v);
  v += dpp_f<0x114, 0xf>(v);
  v += dpp_f<0x118, 0xf>(v);
  v += dpp_f<0x142, 0xa>(v);
  v += dpp_f<0x143, 0xc>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f_keep<0x111, 0xf>(v));
  v = fmaxf(v, dpp_f_keep<0x112, 0xf>(v));
  v = fmaxf(v, dpp_f_keep<0x114, 0xf>(v));
  v = fmaxf(v, dpp_f_keep<0x118, 0xf>(v));
  v = fmaxf(v, dpp_f_keep<0x142, 0xa>(v));
  v = fmaxf(v, dpp_f_keep<0x143, 0xc>(v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

// Workgroup reduction of the online state with NS sums that share its reference, in two
// phases: the workgroup's max first, then every thread's s and sums rescaled once to that
// max and added with DPP wave sums (no cross-lane permutes, no per-step rescaling).
// Results valid in thread 0: the state, and the sums relative to its mc.  lds holds
// (BLOCK / 64) * (NS + 2) floats and must not be reused before the next barrier.
template <int BLOCK, int NS>
__device__ __forceinline__ Lse lse_block_reduce_sums(Lse st, float *v, float c, float *lds) {
  constexpr int W = BLOCK / kWave;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const float wm = wave_max_f32(st.m);
  if (lane == 0) lds[wave] = wm;
  __syncthreads();
  float M = lds[0];
#pragma unroll
  for (int w = 1; w < W; ++w) M = fmaxf(M, lds[w]);
  const float Mc = M == kNegInf ? 0.0f : __fmul_rn(M, c);
  const bool inf = st.m == kNegInf;
  const float f = inf ? 0.0f : fast_exp2(st.mc - Mc);
  const float s = wave_sum_f32(inf ? st.s * 0.0f : st.s * f);
  float t[NS > 0 ? NS : 1];
#pragma unroll
  for (int q = 0; q < NS; ++q) t[q] = wave_sum_f32(inf ? v[q] * 0.0f : v[q] * f);
  float *l2 = lds + W;
  if (lane == 0) {
    l2[wave * (NS + 1)] = s;
#pragma unroll
    for (int q = 0; q < NS; ++q) l2[wave * (NS + 1) + 1 + q] = t[q];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float S = l2[0];
#pragma unroll
    for (int q = 0; q < NS; ++q) v[q] = l2[1 + q];
#pragma unroll
    for (int w = 1; w < W; ++w) {
      S += l2[w * (NS + 1)];
#pragma unroll
      for (int q = 0; q < NS; ++q) v[q] += l2[w * (NS + 1) + 1 + q];
    }
    st = Lse{M, Mc, S};
  }
  return st;
}

template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const T o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

// Exclusive scan across the workgroup; *total receives the sum.  lds holds
// BLOCK / 64 elements.  Every thread must call it.
template <typename T, int BLOCK>
__device__ __forceinline__ T block_exclusive_scan(T v, T *lds, T *total) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const T inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) lds[wave] = inc;
  __syncthreads();
  T base = T(0), tot = T(0);
#pragma unroll
  for (int w = 0; w < BLOCK / kWave; ++w) {
    const T x = lds[w];
    if (w < wave) base += x;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

template <typename T, int BLOCK>
__device__ __forceinline__ T block_sum(T v, T *lds) {
  T tot;
  block_exclusive_scan<T, BLOCK>(v, lds, &tot);
  return tot;
}

}  // namespace smcsd
