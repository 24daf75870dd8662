// resample.hip - ESS and systematic resampling, one workgroup per prompt (gfx950).
//
// The Resample step of an SMC-SD round (SMC explainers, methodology "core flow"): the
// effective sample size is computed every round and, below the threshold, particles are
// resampled by weight - high-weight particles duplicated, low-weight ones dropped.
// Readings: ESS = (sum w)^2 / sum w^2 with w = exp(lw - max lw) in fp64, clamped to
// [1, N]; resample iff ESS < tau*N; systematic resampling with one Philox offset per
// prompt; log-weights reset to 0 afterwards.
//
// The N weights of a prompt are staged in LDS in fp64; the inclusive prefix sum uses
// contiguous per-thread segments plus a workgroup scan, and every particle finds its
// ancestor by binary search over the prefix.
#include "device.hpp"
#include "internal.hpp"

namespace smcsd {

constexpr int kResBlock = 256;

__global__ __launch_bounds__(kResBlock) void k_resample(float *__restrict__ lw, int N, float tau,
                                                        uint64_t seed, uint64_t step,
                                                        int32_t *__restrict__ anc,
                                                        float *__restrict__ ess,
                                                        int32_t *__restrict__ resampled,
                                                        int32_t *status) {
  __shared__ double w[kMaxN];
  __shared__ double dred[kResBlock / kWave];
  __shared__ float fred[kResBlock / kWave];
  __shared__ int ired[kResBlock / kWave];
  __shared__ int sDo;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  float *lwb = lw + (int64_t)b * N;
  int32_t *ab = anc + (int64_t)b * N;

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
    fred[wave] = m;
    ired[wave] = bad;
  }
  __syncthreads();
  m = fred[0];
  bad = ired[0];
  for (int i = 1; i < kResBlock / kWave; ++i) {
    m = fmaxf(m, fred[i]);
    bad |= ired[i];
  }
  __syncthreads();

  if (bad || !isfinite(m)) {
    for (int n = tid; n < N; n += kResBlock) ab[n] = n;
    if (tid == 0) {
      ess[b] = 0.0f;
      resampled[b] = 0;
      atomicOr(status, SMCSD_ST_DEGENERATE_WEIGHTS);
    }
    return;
  }

  double s1 = 0.0, s2 = 0.0;
  for (int n = tid; n < N; n += kResBlock) {
    const double x = exp((double)lwb[n] - (double)m);
    w[n] = x;
    s1 += x;
    s2 += x * x;
  }
  s1 = block_sum<double, kResBlock>(s1, dred);
  s2 = block_sum<double, kResBlock>(s2, dred);
  double e = s1 * s1 / s2;
  if (e < 1.0) e = 1.0;
  if (e > (double)N) e = (double)N;
  if (tid == 0) {
    ess[b] = (float)e;
    sDo = e < (double)tau * (double)N;
    resampled[b] = sDo;
  }
  __syncthreads();
  if (!sDo) {
    for (int n = tid; n < N; n += kResBlock) ab[n] = n;
    return;
  }

  // inclusive prefix of w in place: contiguous segments, then a workgroup scan
  const int per = (N + kResBlock - 1) / kResBlock;
  const int j0 = min(N, tid * per), j1 = min(N, j0 + per);
  double acc = 0.0;
  for (int j = j0; j < j1; ++j) acc += w[j];
  double total;
  const double off = block_exclusive_scan<double, kResBlock>(acc, dred, &total);
  double run = off;
  for (int j = j0; j < j1; ++j) {
    run += w[j];
    w[j] = run;
  }
  __syncthreads();
  const double tot = w[N - 1];  // C_{N-1} = 1 exactly
  const double u0 = philox_uniform(seed, (uint32_t)b, step, 2u, 0);
  for (int i = tid; i < N; i += kResBlock) {
    const double pos = ((double)i + u0) / (double)N;
    int lo = 0, hi = N;  // first j with w[j]/tot > pos, N if none
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (w[mid] / tot > pos) hi = mid;
      else lo = mid + 1;
    }
    ab[i] = lo < N ? lo : N - 1;
  }
  for (int n = tid; n < N; n += kResBlock) lwb[n] = 0.0f;
}

// Up to 64 particles: one wave per prompt, four prompts per workgroup, everything in
// registers and lane shuffles (no workgroup barriers).  Same arithmetic as k_resample:
// fp64 weights relative to the max, ESS clamped to [1, N], strict threshold, systematic
// positions (i + u0) / N against the normalised inclusive prefix.
constexpr int kResWaves = 4;

__global__ __launch_bounds__(kWave * kResWaves) void k_resample_wave(
    float *__restrict__ lw, int B, int N, float tau, uint64_t seed, uint64_t step,
    int32_t *__restrict__ anc, float *__restrict__ ess, int32_t *__restrict__ resampled,
    int32_t *status) {
  const int lane = threadIdx.x % kWave;
  const int b = blockIdx.x * kResWaves + threadIdx.x / kWave;
  if (b >= B) return;  // a whole wave: no barrier below
  float *lwb = lw + (int64_t)b * N;
  int32_t *ab = anc + (int64_t)b * N;
  const bool act = lane < N;
  const float x = act ? lwb[lane] : kNegInf;
  int bad = act && isnan(x);
  float m = act && !isnan(x) ? x : kNegInf;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    m = fmaxf(m, __shfl_xor(m, d, kWave));
    bad |= __shfl_xor(bad, d, kWave);
  }
  if (bad || !isfinite(m)) {
    if (act) ab[lane] = lane;
    if (lane == 0) {
      ess[b] = 0.0f;
      resampled[b] = 0;
      atomicOr(status, SMCSD_ST_DEGENERATE_WEIGHTS);
    }
    return;
  }
  const double w = act ? exp((double)x - (double)m) : 0.0;
  double s1 = w, s2 = w * w;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    s1 += __shfl_xor(s1, d, kWave);
    s2 += __shfl_xor(s2, d, kWave);
  }
  double e = s1 * s1 / s2;
  if (e < 1.0) e = 1.0;
  if (e > (double)N) e = (double)N;
  const bool doit = e < (double)tau * (double)N;
  if (lane == 0) {
    ess[b] = (float)e;
    resampled[b] = doit;
  }
  if (!doit) {
    if (act) ab[lane] = lane;
    return;
  }
  double cum = w;  // inclusive prefix over the lanes
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const double o = __shfl_up(cum, d, kWave);
    if (lane >= d) cum += o;
  }
  const double tot = __shfl(cum, N - 1, kWave);
  const double u0 = philox_uniform(seed, (uint32_t)b, step, 2u, 0);
  const double pos = ((double)lane + u0) / (double)N;
  // number of j with C_j <= pos (C non-decreasing) = first j with C_j > pos
  int idx = 0;
#pragma unroll
  for (int stp = kWave / 2; stp >= 1; stp >>= 1) {
    const int cand = idx + stp - 1;
    const double cv = __shfl(cum, min(cand, N - 1), kWave);
    if (cand < N && !(cv / tot > pos)) idx += stp;
  }
  if (act) {
    ab[lane] = idx < N ? idx : N - 1;
    lwb[lane] = 0.0f;
  }
}

hipError_t launch_resample(float *lw, int B, int N, float tau, uint64_t seed, uint64_t step,
                           int32_t *anc, float *ess, int32_t *resampled, int32_t *status,
                           hipStream_t stream) {
  if (N <= kWave)
    hipLaunchKernelGGL(k_resample_wave, dim3((B + kResWaves - 1) / kResWaves),
                       dim3(kWave * kResWaves), 0, stream, lw, B, N, tau, seed, step, anc, ess,
                       resampled, status);
  else
    hipLaunchKernelGGL(k_resample, dim3(B), dim3(kResBlock), 0, stream, lw, N, tau, seed, step,
                       anc, ess, resampled, status);
  return hipGetLastError();
}

}  // namespace smcsd
