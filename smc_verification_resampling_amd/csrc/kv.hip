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
#include "device.hpp"
#include "internal.hpp"

namespace smcsd {

constexpr int kKvBlock = 256;
constexpr int kKvTileInts = 8192;  // 32 KiB of table staged per tile

// Wait until every memory operation this wave issued (atomics included) has completed.
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0); }

__global__ __launch_bounds__(kKvBlock) void k_kv(
    const int32_t *__restrict__ anc, const int32_t *__restrict__ resampled, int B, int N,
    int32_t *__restrict__ T, int M_cap, int nb_old, int nb_new, int tail_slot, int tail_mod,
    int32_t *__restrict__ rc, int64_t P, int32_t *__restrict__ free_list,
    int32_t *__restrict__ free_top, uint32_t *__restrict__ bitmap, int32_t *__restrict__ needs_cow,
    int32_t *__restrict__ cow_per_prompt, int32_t *__restrict__ done, int32_t *__restrict__ cow,
    int32_t *__restrict__ cow_count, int32_t *status) {
  __shared__ int32_t a[kMaxN], cnt[kMaxN], tail_old[kMaxN], tail_new[kMaxN];
  __shared__ int32_t tile[kKvTileInts];
  __shared__ int64_t red64[kKvBlock / kWave];
  __shared__ int sFlags, sValid, sLast;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int64_t row0 = (int64_t)b * N;
  const int tail_partial = tail_mod != 0;
  if (tid == 0) {
    sFlags = 0;
    sValid = 1;
  }
  const int res = resampled[b] != 0;
  for (int i = tid; i < N; i += kKvBlock) {
    cnt[i] = 0;
    int32_t x = i;
    if (res) {
      x = anc[row0 + i];
      if (x < 0 || x >= N) x = -1;
    }
    a[i] = x;
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
      const int w = min(W, nb_old - s0);
      for (int e = tid; e < N * w; e += kKvBlock) {
        const int j = e / w, s = e - j * w;
        tile[j * W + s] = T[(row0 + j) * M_cap + s0 + s];
      }
      __syncthreads();
      // refcount delta of each run of equal blocks down a column: sum of (c_j - 1)
      for (int sign = 1; sign >= -1; sign -= 2) {
        for (int e = tid; e < N * w; e += kKvBlock) {
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
          if (sign > 0) {
            atomicAdd(&rc[blk], delta);
          } else {
            const int old = atomicAdd(&rc[blk], delta);
            if (old + delta == 0) atomicOr(&bitmap[blk >> 5], 1u << (blk & 31));
          }
        }
        wait_memory();  // increments performed before any decrement
        __syncthreads();
      }
      if (tail_partial && tail_slot >= s0 && tail_slot < s0 + w)
        for (int j = tid; j < N; j += kKvBlock) tail_old[j] = tile[j * W + (tail_slot - s0)];
      for (int e = tid; e < N * w; e += kKvBlock) {
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
  int64_t mine = 0;
  for (int i = tid; i < N; i += kKvBlock) {
    int need = 0;
    if (tail_partial) {
      const int32_t blk = tail_new[i];
      if (blk >= P) atomicOr(&sFlags, SMCSD_ST_BAD_INPUT);
      if (blk >= 0 && blk < P)
        for (int h = i + 1; h < N; ++h)
          if (tail_new[h] == blk) {
            need = 1;
            break;
          }
    }
    needs_cow[row0 + i] = need;
    mine += need;
  }
  const int64_t ncow_prompt = block_sum<int64_t, kKvBlock>(mine, red64);
  if (tid == 0) {
    cow_per_prompt[b] = (int32_t)ncow_prompt;
    if (sFlags) atomicOr(status, sFlags);
  }

  // ---- the last workgroup to arrive does the global push / pop
  __threadfence();
  __syncthreads();
  if (tid == 0) sLast = atomicAdd(done, 1) == B - 1;
  __syncthreads();
  if (!sLast) return;
  __threadfence();
  if (tid == 0) sFlags = 0;
  const int64_t top = *free_top;

  // push: ascending rank r of a freed block goes to stack position top + F - 1 - r
  const int64_t nwords = (P + 31) / 32;
  const int64_t wper = (nwords + kKvBlock - 1) / kKvBlock;
  const int64_t w0 = min(nwords, (int64_t)tid * wper), w1 = min(nwords, w0 + wper);
  int64_t cntb = 0;
  for (int64_t w = w0; w < w1; ++w) cntb += __popc(bitmap[w]);
  int64_t F;
  int64_t r = block_exclusive_scan<int64_t, kKvBlock>(cntb, red64, &F);
  for (int64_t w = w0; w < w1; ++w) {
    uint32_t bits = bitmap[w];
    if (!bits) continue;
    bitmap[w] = 0u;
    while (bits) {
      const int bit = __ffs(bits) - 1;
      bits &= bits - 1;
      const int64_t pos = top + F - 1 - r;
      if (pos >= 0 && pos < P) free_list[pos] = (int32_t)(w * 32 + bit);
      else atomicOr(&sFlags, SMCSD_ST_BAD_INPUT);
      ++r;
    }
  }
  __syncthreads();

  // pops in ascending (sequence, slot) order: copy-on-write tail first, then fresh slots
  const int S = B * N;
  const int64_t avail = top + F;
  const int nfresh = nb_new - nb_old;
  const int sper = (S + kKvBlock - 1) / kKvBlock;
  const int g0 = min(S, tid * sper), g1 = min(S, g0 + sper);
  int64_t nalloc = 0, ncw = 0;
  for (int g = g0; g < g1; ++g) {
    nalloc += needs_cow[g] + nfresh;
    ncw += needs_cow[g];
  }
  int64_t A, C;
  int64_t k = block_exclusive_scan<int64_t, kKvBlock>(nalloc, red64, &A);
  int64_t ci = block_exclusive_scan<int64_t, kKvBlock>(ncw, red64, &C);
  int64_t cow_done = 0;
  for (int g = g0; g < g1; ++g) {
    int32_t *Tg = T + (int64_t)g * M_cap;
    if (needs_cow[g]) {
      if (k < avail && avail - 1 - k < P) {
        const int32_t d = free_list[avail - 1 - k];
        const int32_t o = Tg[tail_slot];
        if (d >= 0 && d < P && o >= 0 && o < P) {
          atomicSub(&rc[o], 1);
          rc[d] = 1;
          Tg[tail_slot] = d;
          cow[3 * ci + 0] = o;
          cow[3 * ci + 1] = d;
          cow[3 * ci + 2] = tail_mod;
          ++ci;
          ++cow_done;
        } else {
          atomicOr(&sFlags, SMCSD_ST_BAD_INPUT);
        }
      } else {
        atomicOr(&sFlags, SMCSD_ST_NOSPACE);
      }
      ++k;
    }
    for (int s = nb_old; s < nb_new; ++s) {
      if (k < avail && avail - 1 - k < P) {
        const int32_t d = free_list[avail - 1 - k];
        if (d >= 0 && d < P) {
          rc[d] = 1;
          Tg[s] = d;
        } else {
          atomicOr(&sFlags, SMCSD_ST_BAD_INPUT);
        }
      } else {
        atomicOr(&sFlags, SMCSD_ST_NOSPACE);
      }
      ++k;
    }
  }
  const int64_t cdone = block_sum<int64_t, kKvBlock>(cow_done, red64);
  if (tid == 0) {
    const int64_t nt = avail - A;
    *free_top = (int32_t)(nt > 0 ? nt : 0);
    *cow_count = (int32_t)cdone;
    *done = 0;
    if (sFlags) atomicOr(status, sFlags);
  }
}

hipError_t launch_kv(const int32_t *anc, const int32_t *resampled, int B, int N, int32_t *tables,
                     int M_cap, int bs, int64_t L, int R, int32_t *rc, int32_t *free_list,
                     int32_t *free_top, int64_t P, int32_t *cow, int32_t *cow_count,
                     int32_t *status, char *ws, hipStream_t stream) {
  const KvWs w = kv_ws_layout(B, (int64_t)B * N, P);
  uint32_t *bitmap = reinterpret_cast<uint32_t *>(ws + w.bitmap);
  int32_t *needs_cow = reinterpret_cast<int32_t *>(ws + w.cow_flags);
  int32_t *cow_per_prompt = reinterpret_cast<int32_t *>(ws + w.cow_per_prompt);
  int32_t *done = reinterpret_cast<int32_t *>(ws + w.done);
  const int nb_old = (int)ceil_div(L, bs);
  const int nb_new = (int)ceil_div(L + R, bs);
  hipLaunchKernelGGL(k_kv, dim3(B), dim3(kKvBlock), 0, stream, anc, resampled, B, N, tables, M_cap,
                     nb_old, nb_new, (int)(L / bs), (int)(L % bs), rc, P, free_list, free_top,
                     bitmap, needs_cow, cow_per_prompt, done, cow, cow_count, status);
  return hipGetLastError();
}

}  // namespace smcsd
