// kv.hip - KV cache pointer exchange with reference counts (gfx950).
//
// After resampling, the KV cache follows the particles by exchanging block pointers and
// updating reference counts; prefixes stay shared across particles and no KV data is
// copied (SMC explainers, "system optimisation design": KV cache; Spanish page, cache
// management).  Integer work only, one launch per call, bit-deterministic although it
// uses atomics:
//   * within a column tile of a prompt's tables, all refcount increments are performed
//     (waited for, then a barrier) before any decrement, so a block that stays
//     referenced never reaches 0, and the one decrement that brings a count to 0 marks
//     the block freed exactly once (a block lives in one column of one prompt);
//   * freed blocks go to a bitmap and are pushed in descending id order; pops are
//     assigned by prefix sums over the sequences in ascending order.
//
// One workgroup per prompt does the exchange, the table gather (staged through LDS in
// column tiles) and the copy-on-write decision for its partial tail.  The last
// workgroup to finish (a device-scope counter with release/acquire fences) performs the
// global part: push the freed blocks, pop fresh blocks for the reservation and the
// copy-on-write list, update the stack top, and reset the counter for the next call.
//
// Each workgroup runs this code about once per call, so its instruction fetches are
// cold: the kernel is written as short loops (no wide unrolling, 32-bit indices, one
// shared scan routine) because code size, not data, sets its latency.
#include "device.hpp"
#include "internal.hpp"

namespace smcsd {

constexpr int kKvBlock = 256;
constexpr int kKvTileInts = 8192;  // 32 KiB of table staged per tile
constexpr int kPushBatch = 16;

// Wait until every memory operation this wave issued (atomics included) has completed.
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Exclusive scan over the 256 threads of the workgroup; *total gets the sum.
__device__ __forceinline__ int kv_scan(int v, int *lds, int *total) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  int inc = v;
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  if (lane == kWave - 1) lds[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < kKvBlock / kWave; ++w) {
    if (w < wave) base += lds[w];
    tot += lds[w];
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

__global__ __launch_bounds__(kKvBlock) void k_kv(
    const int32_t *__restrict__ anc, const int32_t *__restrict__ resampled, int B, int N,
    int32_t *__restrict__ T, int M_cap, int nb_old, int nb_new, int tail_slot, int tail_mod,
    int32_t *__restrict__ rc, int P, int32_t *__restrict__ free_list,
    int32_t *__restrict__ free_top, uint32_t *__restrict__ bitmap, int32_t *__restrict__ needs_cow,
    int32_t *__restrict__ cow_excl, int32_t *__restrict__ scal, int32_t *__restrict__ done,
    int32_t *__restrict__ cow_count, int32_t *status) {
  __shared__ int32_t a[kMaxN], cnt[kMaxN], tail_old[kMaxN], tail_new[kMaxN];
  __shared__ int32_t tile[kKvTileInts];
  __shared__ int red[kKvBlock / kWave];
  __shared__ int sFlags, sValid, sLast;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int row0 = b * N;
  const int tail_partial = tail_mod != 0;
  if (tid == 0) {
    sFlags = 0;
    sValid = 1;
  }
  const int res = resampled[b] != 0;
  for (int i = tid; i < N; i += kKvBlock) {
    cnt[i] = 0;
    const int32_t x = res ? anc[row0 + i] : i;
    a[i] = (x < 0 || x >= N) ? -1 : x;
  }
  __syncthreads();
  for (int i = tid; i < N; i += kKvBlock)
    if (a[i] < 0) sValid = 0;
  __syncthreads();
  const int do_exchange = res && sValid;
  if (res && !sValid && tid == 0) sFlags |= SMCSD_ST_BAD_INPUT;

  // ---- phase 1: exchange (prompts that resampled)
  if (do_exchange) {
    for (int i = tid; i < N; i += kKvBlock) atomicAdd(&cnt[a[i]], 1);
    __syncthreads();
    const int W = max(1, min(nb_old, kKvTileInts / N));
    for (int s0 = 0; s0 < nb_old; s0 += W) {
      const int w = min(W, nb_old - s0), nw = N * w;
#pragma unroll 4
      for (int e = tid; e < nw; e += kKvBlock) {
        const int j = e / w, s = e - j * w;
        tile[j * W + s] = T[(row0 + j) * M_cap + s0 + s];
      }
      __syncthreads();
      // refcount delta of each run of equal blocks down a column: sum of (c_j - 1);
      // pass sign = +1 applies the increments, sign = -1 the decrements
#pragma unroll 1
      for (int sign = 1; sign >= -1; sign -= 2) {
#pragma unroll 1
        for (int e = tid; e < nw; e += kKvBlock) {
          const int j = e / w, s = e - j * w;
          const int32_t blk = tile[j * W + s];
          if (j > 0 && tile[(j - 1) * W + s] == blk) continue;  // not the head of its run
          int delta = 0;
          for (int jj = j; jj < N && tile[jj * W + s] == blk; ++jj) delta += cnt[jj] - 1;
          if (delta * sign <= 0) continue;
          if (blk < 0 || blk >= P) {
            atomicOr(&sFlags, SMCSD_ST_BAD_INPUT);
            continue;
          }
          const int old = atomicAdd(&rc[blk], delta);
          if (old + delta == 0) atomicOr(&bitmap[blk >> 5], 1u << (blk & 31));
        }
        wait_memory();  // increments performed before any decrement
        __syncthreads();
      }
      if (tail_partial && tail_slot >= s0 && tail_slot < s0 + w)
        for (int j = tid; j < N; j += kKvBlock) tail_old[j] = tile[j * W + (tail_slot - s0)];
#pragma unroll 4
      for (int e = tid; e < nw; e += kKvBlock) {
        const int i = e / w, s = e - i * w;
        T[(row0 + i) * M_cap + s0 + s] = tile[a[i] * W + s];
      }
      __syncthreads();
    }
    if (tail_partial)
      for (int i = tid; i < N; i += kKvBlock) tail_new[i] = tail_old[a[i]];
  } else if (tail_partial) {
    for (int i = tid; i < N; i += kKvBlock) tail_new[i] = T[(row0 + i) * M_cap + tail_slot];
  }
  __syncthreads();

  // copy-on-write decision: the partial tail is also held by a higher-index sequence of
  // this prompt (the highest holder keeps the block)
  for (int i = tid; i < N; i += kKvBlock) {
    int need = 0;
    if (tail_partial) {
      const int32_t blk = tail_new[i];
      if (blk >= P) atomicOr(&sFlags, SMCSD_ST_BAD_INPUT);
      if (blk >= 0 && blk < P)
        for (int h = i + 1; h < N && !need; ++h) need = tail_new[h] == blk;
    }
    needs_cow[row0 + i] = need;
  }
  __syncthreads();
  if (tid == 0 && sFlags) atomicOr(status, sFlags);

  // ---- the last workgroup to arrive pushes the freed blocks and lays out the pops
  __threadfence();
  __syncthreads();
  if (tid == 0) sLast = atomicAdd(done, 1) == B - 1;
  __syncthreads();
  if (!sLast) return;
  __threadfence();
  if (tid == 0) sFlags = 0;
  const int top = *free_top;

  // push: the freed block of ascending rank r goes to stack position top + F - 1 - r;
  // each thread owns a contiguous run of bitmap words
  const int nwords = (P + 31) / 32;
  const int wper = (nwords + kKvBlock - 1) / kKvBlock;
  const int w0 = min(nwords, tid * wper), w1 = min(nwords, w0 + wper);
  int nbits = 0;
#pragma unroll 4
  for (int w = w0; w < w1; ++w) nbits += __popc(bitmap[w]);
  int F;
  int r = kv_scan(nbits, red, &F);
  for (int wb = w0; wb < w1; wb += kPushBatch) {
    uint32_t v[kPushBatch];
#pragma unroll
    for (int i = 0; i < kPushBatch; ++i) v[i] = bitmap[min(wb + i, w1 - 1)];
    asm volatile("" ::: "memory");  // the batch's loads go out before any of its stores
#pragma unroll
    for (int i = 0; i < kPushBatch; ++i) {
      uint32_t bits = wb + i < w1 ? v[i] : 0u;
      if (!bits) continue;
      bitmap[wb + i] = 0u;
      for (; bits; bits &= bits - 1, ++r) {
        const int64_t pos = (int64_t)top + F - 1 - r;
        if (pos >= 0 && pos < P) free_list[pos] = (wb + i) * 32 + __ffs(bits) - 1;
        else atomicOr(&sFlags, SMCSD_ST_BAD_INPUT);
      }
    }
  }

  // pop layout: sequence g owns pop indices [g*nfresh + cow_excl[g], ... + cow_g + nfresh)
  const int S = B * N;
  const int nfresh = nb_new - nb_old;
  const int sper = (S + kKvBlock - 1) / kKvBlock;
  const int g0 = min(S, tid * sper), g1 = min(S, g0 + sper);
  int mycow = 0;
#pragma unroll 4
  for (int g = g0; g < g1; ++g) mycow += needs_cow[g];
  int C;
  int ci = kv_scan(mycow, red, &C);
  const int64_t avail = (int64_t)top + F;
  int ok_cow = 0;  // copy-on-writes whose pop falls inside the stack
  for (int g = g0; g < g1; ++g) {
    const int f = needs_cow[g];
    cow_excl[g] = ci;
    ok_cow += f && (int64_t)g * nfresh + ci < avail;
    ci += f;
  }
  int ncow_ok;
  kv_scan(ok_cow, red, &ncow_ok);
  if (tid == 0) {
    scal[0] = top;
    scal[1] = F;
    const int64_t nt = avail - ((int64_t)S * nfresh + C);
    *free_top = (int32_t)(nt > 0 ? nt : 0);
    *cow_count = ncow_ok;
    *done = 0;
  }
  __syncthreads();
  if (tid == 0 && sFlags) atomicOr(status, sFlags);
}

// Pops, one thread per sequence: a sequence's copy-on-write (tail slot) pops first, then
// its fresh slots; pop k takes the stack entry at avail - 1 - k.
__global__ __launch_bounds__(kKvBlock) void k_kv_pop(
    int S, int32_t *__restrict__ T, int M_cap, int nb_old, int nb_new, int tail_slot,
    int tail_mod, int32_t *__restrict__ rc, int P, const int32_t *__restrict__ free_list,
    const int32_t *__restrict__ needs_cow, const int32_t *__restrict__ cow_excl,
    const int32_t *__restrict__ scal, int32_t *__restrict__ cow, int32_t *status) {
  const int g = blockIdx.x * kKvBlock + threadIdx.x;
  if (g >= S) return;
  const int nfresh = nb_new - nb_old;
  const int64_t avail = (int64_t)scal[0] + scal[1];
  const int f = needs_cow[g], ce = cow_excl[g];
  int64_t k = (int64_t)g * nfresh + ce;
  int flags = 0;
  for (int st = f ? -1 : 0; st < nfresh; ++st, ++k) {
    if (k >= avail) {
      flags |= SMCSD_ST_NOSPACE;
      continue;
    }
    const int64_t pos = avail - 1 - k;
    const int32_t d = pos < P ? free_list[pos] : -1;
    const int32_t o = st < 0 ? T[(int64_t)g * M_cap + tail_slot] : 0;
    if (d < 0 || d >= P || o < 0 || o >= P) {
      flags |= SMCSD_ST_BAD_INPUT;
      continue;
    }
    if (st < 0) {
      atomicSub(&rc[o], 1);
      cow[3 * ce + 0] = o;
      cow[3 * ce + 1] = d;
      cow[3 * ce + 2] = tail_mod;
    }
    rc[d] = 1;
    T[(int64_t)g * M_cap + (st < 0 ? tail_slot : nb_old + st)] = d;
  }
  if (flags) atomicOr(status, flags);
}

hipError_t launch_kv(const int32_t *anc, const int32_t *resampled, int B, int N, int32_t *tables,
                     int M_cap, int bs, int64_t L, int R, int32_t *rc, int32_t *free_list,
                     int32_t *free_top, int64_t P, int32_t *cow, int32_t *cow_count,
                     int32_t *status, char *ws, hipStream_t stream) {
  const int S = B * N;
  const KvWs w = kv_ws_layout(B, S, P);
  uint32_t *bitmap = reinterpret_cast<uint32_t *>(ws + w.bitmap);
  int32_t *needs_cow = reinterpret_cast<int32_t *>(ws + w.cow_flags);
  int32_t *cow_excl = reinterpret_cast<int32_t *>(ws + w.cow_excl);
  int32_t *done = reinterpret_cast<int32_t *>(ws + w.done);
  int32_t *scal = reinterpret_cast<int32_t *>(ws + w.scal);
  const int nb_old = (int)ceil_div(L, bs);
  const int nb_new = (int)ceil_div(L + R, bs);
  const int tail_slot = (int)(L / bs), tail_mod = (int)(L % bs);
  hipLaunchKernelGGL(k_kv, dim3(B), dim3(kKvBlock), 0, stream, anc, resampled, B, N, tables, M_cap,
                     nb_old, nb_new, tail_slot, tail_mod, rc, (int)P, free_list, free_top, bitmap,
                     needs_cow, cow_excl, scal, done, cow_count, status);
  hipLaunchKernelGGL(k_kv_pop, dim3((S + kKvBlock - 1) / kKvBlock), dim3(kKvBlock), 0, stream, S,
                     tables, M_cap, nb_old, nb_new, tail_slot, tail_mod, rc, (int)P, free_list,
                     needs_cow, cow_excl, scal, cow, status);
  return hipGetLastError();
}

}  // namespace smcsd
