// kvcheck.hip - a debugging check of the refcounted block-table state (gfx950).
//
// The pointer exchange keeps three structures consistent (SMC explainers, "system
// optimisation design": KV blocks shared by pointer, freed by reference count): every
// block's refcount equals the number of table slots that name it, the free stack holds
// each unreferenced block exactly once, and no referenced block is on it.  This check
// recounts all three from scratch, independently of the exchange kernels, and counts the
// violations of each kind.  Five small launches, integer work only; meant for tests and
// debug runs, not for the timed path.
#include "../../include/smcsd.h"
#include "internal.hpp"

namespace smcsd {

namespace {

constexpr int kChkBlock = 256;

// counters: [refs per block x P][free-stack occurrences per block x P]; violations [5]
__global__ __launch_bounds__(kChkBlock) void k_kvc_clear(int32_t *__restrict__ refs,
                                                         int32_t *__restrict__ occ, int64_t P,
                                                         int32_t *__restrict__ viol) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < P; i += stride) {
    refs[i] = 0;
    occ[i] = 0;
  }
  if (blockIdx.x == 0 && threadIdx.x < SMCSD_KV_CHECK_KINDS) viol[threadIdx.x] = 0;
}

// every allocated slot: count a reference to its block; an id outside [0, P) other than
// the -1 of an unfilled slot is violation 1
__global__ __launch_bounds__(kChkBlock) void k_kvc_tables(const int32_t *__restrict__ T, int64_t S,
                                                          int M_cap, int slots, int64_t P,
                                                          int32_t *__restrict__ refs,
                                                          int32_t *__restrict__ viol) {
  const int64_t n = S * slots;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int bad = 0;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) {
    const int64_t g = e / slots, s = e - g * slots;
    const int32_t b = T[g * M_cap + s];
    if (b >= 0 && b < P) atomicAdd(&refs[b], 1);
    else if (b != -1) ++bad;
  }
  if (bad) atomicAdd(&viol[1], bad);
}

// every free-stack entry below the top: count its block; an entry outside [0, P), and a
// top outside [0, P], is violation 2 (the top is clamped to [0, P])
__global__ __launch_bounds__(kChkBlock) void k_kvc_free(const int32_t *__restrict__ fl,
                                                        const int32_t *__restrict__ free_top,
                                                        int64_t P, int32_t *__restrict__ occ,
                                                        int32_t *__restrict__ viol) {
  const int32_t top_raw = *free_top;
  const int64_t top = top_raw < 0 ? 0 : (top_raw > P ? P : top_raw);
  if (blockIdx.x == 0 && threadIdx.x == 0 && (top_raw < 0 || top_raw > P)) atomicAdd(&viol[2], 1);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < top; i += stride) {
    const int32_t b = fl[i];
    if (b >= 0 && b < P) atomicAdd(&occ[b], 1);
    else ++bad;
  }
  if (bad) atomicAdd(&viol[2], bad);
}

// every block: 0 refcount != references; 2 extra occurrences on the free stack; 3 on the
// free stack with a positive refcount; 4 refcount <= 0 and not on the free stack (leaked)
__global__ __launch_bounds__(kChkBlock) void k_kvc_compare(const int32_t *__restrict__ rc,
                                                           const int32_t *__restrict__ refs,
                                                           const int32_t *__restrict__ occ,
                                                           int64_t P, int32_t *__restrict__ viol) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int v0 = 0, v2 = 0, v3 = 0, v4 = 0;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < P; b += stride) {
    const int32_t r = rc[b], o = occ[b];
    v0 += r != refs[b];
    v2 += o > 1 ? o - 1 : 0;
    v3 += o > 0 && r > 0;
    v4 += o == 0 && r <= 0;
  }
  if (v0) atomicAdd(&viol[0], v0);
  if (v2) atomicAdd(&viol[2], v2);
  if (v3) atomicAdd(&viol[3], v3);
  if (v4) atomicAdd(&viol[4], v4);
}

// the status bit, once every count is in
__global__ void k_kvc_flag(const int32_t *__restrict__ viol, int32_t *status) {
  int any = 0;
  for (int k = 0; k < SMCSD_KV_CHECK_KINDS; ++k) any |= viol[k];
  if (any) atomicOr(status, SMCSD_ST_KV_INCONSISTENT);
}

}  // namespace

size_t kv_check_ws_bytes(int64_t P) { return 2 * align256(sizeof(int32_t) * (size_t)P); }

hipError_t launch_kv_check(const int32_t *T, int64_t S, int M_cap, int slots,
                           const int32_t *rc, const int32_t *fl, const int32_t *free_top,
                           int64_t P, int32_t *viol, int32_t *status, char *ws,
                           hipStream_t stream) {
  int32_t *refs = reinterpret_cast<int32_t *>(ws);
  int32_t *occ = reinterpret_cast<int32_t *>(ws + align256(sizeof(int32_t) * (size_t)P));
  const unsigned gp = grid_blocks(P, kChkBlock);
  hipLaunchKernelGGL(k_kvc_clear, dim3(gp), dim3(kChkBlock), 0, stream, refs, occ, P, viol);
  if (S > 0 && slots > 0)
    hipLaunchKernelGGL(k_kvc_tables, dim3(grid_blocks(S * slots, kChkBlock)), dim3(kChkBlock), 0,
                       stream, T, S, M_cap, slots, P, refs, viol);
  hipLaunchKernelGGL(k_kvc_free, dim3(gp), dim3(kChkBlock), 0, stream, fl, free_top, P, occ, viol);
  hipLaunchKernelGGL(k_kvc_compare, dim3(gp), dim3(kChkBlock), 0, stream, rc, refs, occ, P, viol);
  hipLaunchKernelGGL(k_kvc_flag, dim3(1), dim3(1), 0, stream, viol, status);
  return hipGetLastError();
}

}  // namespace smcsd
