// resample.hip - ESS and systematic resampling, one workgroup (or one wave) per prompt
// (gfx950).  The per-prompt arithmetic is in resample.hpp, shared with the fused
// resample + KV kernel.
#include "resample.hpp"

namespace smcsd {

template <bool STRIDE>
__global__ __launch_bounds__(kResBlock) void k_resample(float *__restrict__ lw, int B, int N, float tau,
                                                        uint64_t seed, uint64_t step,
                                                        int32_t *__restrict__ anc,
                                                        float *__restrict__ ess,
                                                        int32_t *__restrict__ resampled,
                                                        int32_t *status) {
  __shared__ ResampleLds L;
  for (int b = blockIdx.x; b < B; b += gridDim.x) {  // a grid smaller than B strides over it
    resample_prompt_block(lw + (int64_t)b * N, N, tau, seed, b, step, anc + (int64_t)b * N,
                          ess + b, resampled + b, status, nullptr, L, true, true);
    if (!STRIDE) break;  // the grid covers the batch: no loop kept
    __syncthreads();     // the next prompt reuses the LDS
  }
}

// Up to 64 particles: one wave per prompt, four prompts per workgroup, no workgroup
// barriers.
constexpr int kResWaves = 4;

template <bool STRIDE>
__global__ __launch_bounds__(kWave * kResWaves) void k_resample_wave(
    float *__restrict__ lw, int B, int N, float tau, uint64_t seed, uint64_t step,
    int32_t *__restrict__ anc, float *__restrict__ ess, int32_t *__restrict__ resampled,
    int32_t *status) {
  const int lane = threadIdx.x % kWave;
  // one prompt per wave, no workgroup barrier; a grid smaller than B strides over it
  for (int b = blockIdx.x * kResWaves + threadIdx.x / kWave; b < B; b += gridDim.x * kResWaves) {
    float *lwb = lw + (int64_t)b * N;
    const float x = lane < N ? lwb[lane] : 0.0f;
    resample_prompt_wave(x, lwb, N, tau, seed, b, step, anc + (int64_t)b * N, ess + b,
                         resampled + b, status, nullptr, true, true);
    if (!STRIDE) break;
  }
}

hipError_t launch_resample(float *lw, int B, int N, float tau, uint64_t seed, uint64_t step,
                           int32_t *anc, float *ess, int32_t *resampled, int32_t *status,
                           hipStream_t stream) {
  // the looping forms only where the grid cap leaves fewer workgroups (or waves) than
  // prompts: the loop costs registers
  if (N <= kWave) {
    const int64_t items = ((int64_t)B + kResWaves - 1) / kResWaves;
    const unsigned g = grid_blocks(items, kWave * kResWaves);
    hipLaunchKernelGGL((int64_t)g < items ? k_resample_wave<true> : k_resample_wave<false>, dim3(g),
                       dim3(kWave * kResWaves), 0, stream, lw, B, N, tau, seed, step, anc, ess,
                       resampled, status);
  } else {
    const unsigned g = grid_blocks(B, kResBlock);
    hipLaunchKernelGGL((int64_t)g < B ? k_resample<true> : k_resample<false>, dim3(g), dim3(kResBlock),
                       0, stream, lw, B, N, tau, seed, step, anc, ess, resampled, status);
  }
  return hipGetLastError();
}

}  // namespace smcsd
