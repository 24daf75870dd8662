// resample.hpp - one prompt's ESS, resampling decision and systematic ancestors (gfx950),
// as device functions shared by the resample kernels and the fused resample + KV kernel,
// so both entry points compute the same bits.
//
// The Resample step of an SMC-SD round (SMC explainers, methodology "core flow"): the
// effective sample size is computed every round and, below the threshold, particles are
// resampled by weight - high-weight particles duplicated, low-weight ones dropped.
// Readings: ESS = (sum w)^2 / sum w^2 with w = exp(lw - max lw) in fp64, clamped to
// [1, N]; resample iff ESS < tau*N; systematic resampling with one Philox offset per
// prompt (tag 2); ancestors[i] = first j with C_j / C_{N-1} > (i + u0) / N (N-1 if none);
// log-weights reset to 0 afterwards.  A prompt whose weights are all zero or NaN keeps
// identity ancestors, gets ess = 0 and sets DEGENERATE_WEIGHTS.
#pragma once

#include "device.hpp"
#include "internal.hpp"

namespace smcsd {

constexpr int kResBlock = 256;

// By one wave, N <= kWave: everything in registers and lane shuffles.  Every lane of the
// wave calls it with x = lwb[lane] already loaded (any value for lanes >= N, which idle), so
// a caller can issue that load early.  Outputs of prompt b: ab[N] ancestors, *essb, *resb
// and the status flag (only when out), the reset of lwb (only when reset); sa (nullable)
// gets the ancestors too.  Returns the decision (every lane).  Several workgroups may
// resample one prompt (the same bits in each) when one of them writes the outputs and none
// resets lwb while another may still read it.
__device__ __forceinline__ int resample_prompt_wave(float x_in, float *__restrict__ lwb, int N,
                                                    float tau, uint64_t seed, int b, uint64_t step,
                                                    int32_t *__restrict__ ab, float *essb,
                                                    int32_t *resb, int32_t *status, int32_t *sa,
                                                    bool out, bool reset) {
  const int lane = threadIdx.x % kWave;
  const bool act = lane < N;
  const float x = act ? x_in : kNegInf;
  const bool bad = __ballot(act && isnan(x)) != 0ull;
  const float m = wave_max_f32(act && !isnan(x) ? x : kNegInf);  // in every lane
  if (bad || !isfinite(m)) {
    if (act) {
      if (out) ab[lane] = lane;
      if (sa) sa[lane] = lane;
    }
    if (lane == 0 && out) {
      *essb = 0.0f;
      *resb = 0;
      atomicOr(status, SMCSD_ST_DEGENERATE_WEIGHTS);
    }
    return 0;
  }
  const double w = act ? exp((double)x - (double)m) : 0.0;
  const double s1 = wave_sum(w), s2 = wave_sum(w * w);
  double e = s1 * s1 / s2;
  if (e < 1.0) e = 1.0;
  if (e > (double)N) e = (double)N;
  const bool doit = e < (double)tau * (double)N;
  if (lane == 0 && out) {
    *essb = (float)e;
    *resb = doit;
  }
  if (!doit) {
    if (act) {
      if (out) ab[lane] = lane;
      if (sa) sa[lane] = lane;
    }
    return 0;
  }
  const double cum = wave_inclusive_scan(w);  // inclusive prefix over the lanes
  const double tot = __shfl(cum, N - 1, kWave);
  const double cn = cum / tot;  // C_j, each lane's divided once (the search compares these)
  const double u0 = philox_uniform(seed, (uint32_t)b, step, 2u, 0);
  const double pos = ((double)lane + u0) / (double)N;
  // number of j with C_j <= pos (C non-decreasing) = first j with C_j > pos
  int idx = 0;
#pragma unroll
  for (int stp = kWave / 2; stp >= 1; stp >>= 1) {
    const int cand = idx + stp - 1;
    const double cv = __shfl(cn, min(cand, N - 1), kWave);
    if (cand < N && !(cv > pos)) idx += stp;
  }
  if (act) {
    const int a = idx < N ? idx : N - 1;
    if (out) ab[lane] = a;
    if (sa) sa[lane] = a;
    if (reset) lwb[lane] = 0.0f;
  }
  return 1;
}

// LDS of resample_prompt_block
struct ResampleLds {
  double w[kMaxN];
  double dred[kResBlock / kWave];
  float fred[kResBlock / kWave];
  int ired[kResBlock / kWave];
  int decision;
};

// By a whole kResBlock-thread workgroup (every thread calls it), N <= kMaxN: the weights
// staged in LDS in fp64, the inclusive prefix by contiguous per-thread segments plus a
// workgroup scan, every particle's ancestor by binary search over the prefix.  Same
// outputs, flags and return value as resample_prompt_wave.
__device__ __forceinline__ int resample_prompt_block(float *__restrict__ lwb, int N, float tau,
                                                     uint64_t seed, int b, uint64_t step,
                                                     int32_t *__restrict__ ab, float *essb,
                                                     int32_t *resb, int32_t *status, int32_t *sa,
                                                     ResampleLds &L, bool out, bool reset) {
  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;

  // max over the prompt's log-weights (NaN detected separately)
  float m = kNegInf;
  int bad = 0;
  for (int n = tid; n < N; n += kResBlock) {
    const float x = lwb[n];
    if (isnan(x)) bad = 1;
    else m = fmaxf(m, x);
  }
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    m = fmaxf(m, __shfl_xor(m, d, kWave));
    bad |= __shfl_xor(bad, d, kWave);
  }
  if (lane == 0) {
    L.fred[wave] = m;
    L.ired[wave] = bad;
  }
  __syncthreads();
  m = L.fred[0];
  bad = L.ired[0];
  for (int i = 1; i < kResBlock / kWave; ++i) {
    m = fmaxf(m, L.fred[i]);
    bad |= L.ired[i];
  }
  __syncthreads();

  if (bad || !isfinite(m)) {
    for (int n = tid; n < N; n += kResBlock) {
      if (out) ab[n] = n;
      if (sa) sa[n] = n;
    }
    if (tid == 0 && out) {
      *essb = 0.0f;
      *resb = 0;
      atomicOr(status, SMCSD_ST_DEGENERATE_WEIGHTS);
    }
    return 0;
  }

  double s1 = 0.0, s2 = 0.0;
  for (int n = tid; n < N; n += kResBlock) {
    const double x = exp((double)lwb[n] - (double)m);
    L.w[n] = x;
    s1 += x;
    s2 += x * x;
  }
  s1 = block_sum<double, kResBlock>(s1, L.dred);
  s2 = block_sum<double, kResBlock>(s2, L.dred);
  double e = s1 * s1 / s2;
  if (e < 1.0) e = 1.0;
  if (e > (double)N) e = (double)N;
  if (tid == 0) {
    L.decision = e < (double)tau * (double)N;
    if (out) {
      *essb = (float)e;
      *resb = L.decision;
    }
  }
  __syncthreads();
  if (!L.decision) {
    for (int n = tid; n < N; n += kResBlock) {
      if (out) ab[n] = n;
      if (sa) sa[n] = n;
    }
    return 0;
  }

  // inclusive prefix of w in place: contiguous segments, then a workgroup scan
  const int per = (N + kResBlock - 1) / kResBlock;
  const int j0 = min(N, tid * per), j1 = min(N, j0 + per);
  double acc = 0.0;
  for (int j = j0; j < j1; ++j) acc += L.w[j];
  double total;
  const double off = block_exclusive_scan<double, kResBlock>(acc, L.dred, &total);
  double run = off;
  for (int j = j0; j < j1; ++j) {
    run += L.w[j];
    L.w[j] = run;
  }
  __syncthreads();
  const double tot = L.w[N - 1];  // the prefix's last entry
  __syncthreads();                // read by every thread before its owner rescales it
  // C_j = prefix_j / tot, each entry divided once by the thread that wrote it (the search
  // compares these)
  for (int j = j0; j < j1; ++j) L.w[j] = L.w[j] / tot;
  __syncthreads();
  const double u0 = philox_uniform(seed, (uint32_t)b, step, 2u, 0);
  for (int i = tid; i < N; i += kResBlock) {
    const double pos = ((double)i + u0) / (double)N;
    int lo = 0, hi = N;  // first j with C_j > pos, N if none
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (L.w[mid] > pos) hi = mid;
      else lo = mid + 1;
    }
    const int a = lo < N ? lo : N - 1;
    if (out) ab[i] = a;
    if (sa) sa[i] = a;
  }
  if (reset)
    for (int n = tid; n < N; n += kResBlock) lwb[n] = 0.0f;
  return 1;
}

}  // namespace smcsd
