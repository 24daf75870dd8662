// kv.hip - KV cache pointer exchange with reference counts (gfx950).
//
// After resampling, the KV cache follows the particles by exchanging block pointers and
// updating reference counts; prefixes stay shared across particles and no KV data is
// copied (SMC explainers, "system optimisation design": KV cache; Spanish page, cache
// management).  Integer work only, two launches per call, bit-deterministic although it
// uses atomics:
//   * k_kv, one workgroup per prompt: the exchange over column tiles of the prompt's
//     tables staged in LDS.  Columns whose entries are all equal (shared prefixes) keep
//     their blocks and counts and are skipped.  Down each other column, a run of equal
//     blocks gets one refcount update, sum over the run of (c_j - 1); all increments are
//     performed (waited for, then a barrier) before any decrement, so a block that stays
//     referenced never reaches 0, and the decrement that brings a count to 0 marks the
//     block in a freed bitmap exactly once (a block lives in one column of one prompt).
//     Then the gathered tables and the copy-on-write decision for the partial tail.  The
//     last workgroup to finish (a device-scope counter with release / acquire fences)
//     counts the freed blocks per group of bitmap words, lays out every sequence's pops
//     and sets the new stack top.
//   * k_kv_pop, one thread per bitmap word and one per sequence: a freed block's rank in
//     ascending id order fixes its stack position (pushed in descending id order) and,
//     if that pop is requested, the table slot it fills; sequences take their remaining
//     pops from the old stack and write their copy-on-write records.
#include "device.hpp"
#include "internal.hpp"
#include "kv_layout.hpp"

namespace smcsd {

constexpr int kKvBlock = 256;
constexpr int kKvTileInts = 8192;  // table entries staged per column tile (32 KiB)
constexpr int kStage = 16;         // table loads in flight per thread while staging
constexpr int kNegBatch = 4;       // decrements in flight per thread
constexpr int kHash = 2 * kMaxN;   // open-addressing table of the tail blocks (load <= 1/2)

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

__device__ __forceinline__ int tail_hash(int32_t blk) {
  return (int)(((uint32_t)blk * 0x9E3779B1u) >> 21) & (kHash - 1);
}

__global__ __launch_bounds__(kKvBlock) void k_kv(
    const int32_t *__restrict__ anc, const int32_t *__restrict__ resampled, int B, int N,
    int32_t *__restrict__ T, int M_cap, int nb_old, int nb_new, int tail_slot, int tail_mod,
    int32_t *__restrict__ rc, int P, int32_t *__restrict__ free_top,
    uint32_t *__restrict__ bitmap, int32_t *__restrict__ cow_src, int32_t *__restrict__ cow_excl,
    int32_t *__restrict__ gbase, int32_t *__restrict__ popmap, int32_t *__restrict__ scal,
    int32_t *__restrict__ done, int32_t *__restrict__ cow_count, int32_t *status) {
  __shared__ int32_t a[kMaxN], cnt[kMaxN], tail_old[kMaxN], tail_new[kMaxN];
  __shared__ int32_t tile[kKvTileInts];
  __shared__ uint8_t colu[kKvTileInts];  // column of the tile holds one block in every row
  __shared__ int2 negl[kKvTileInts];     // (block, decrement); later the tail hash table
  __shared__ int gcnt[kKvBlock];
  __shared__ int red[kKvBlock / kWave];
  __shared__ int sFlags, sValid, sLast, sNeg;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int row0 = b * N;
  const int tail_partial = tail_mod != 0;
  if (tid == 0) {
    sFlags = 0;
    sValid = 1;
  }
  // the ancestor row is read whether or not the prompt resampled, so both loads overlap
  const int res = resampled[b] != 0;
  for (int i = tid; i < N; i += kKvBlock) {
    a[i] = anc[row0 + i];
    cnt[i] = 0;
  }
  __syncthreads();
  for (int i = tid; i < N; i += kKvBlock) {
    const int32_t x = res ? a[i] : i;
    const int ok = x >= 0 && x < N;
    a[i] = ok ? x : -1;
    if (!ok) sValid = 0;
  }
  __syncthreads();
  const int do_exchange = res && sValid;
  if (res && !sValid && tid == 0) sFlags |= SMCSD_ST_BAD_INPUT;

  // ---- phase 1: exchange (prompts that resampled)
  if (do_exchange) {
    for (int i = tid; i < N; i += kKvBlock) atomicAdd(&cnt[a[i]], 1);
    const int W = max(1, min(nb_old, kKvTileInts / N));
    for (int s0 = 0; s0 < nb_old; s0 += W) {
      const int w = min(W, nb_old - s0), nw = N * w;
      for (int e0 = tid; e0 < nw; e0 += kKvBlock * kStage) {
        int32_t v[kStage];
#pragma unroll
        for (int k = 0; k < kStage; ++k) {
          const int e = min(e0 + k * kKvBlock, nw - 1);
          const int j = e / w, s = e - j * w;
          v[k] = T[(row0 + j) * M_cap + s0 + s];
        }
#pragma unroll
        for (int k = 0; k < kStage; ++k) {
          const int e = e0 + k * kKvBlock;
          const int j = e / w, s = e - j * w;
          if (e < nw) tile[j * W + s] = v[k];
        }
      }
      for (int s = tid; s < w; s += kKvBlock) colu[s] = 1;
      if (tid == 0) sNeg = 0;
      __syncthreads();
      for (int e = tid; e < nw; e += kKvBlock) {
        const int j = e / w, s = e - j * w;
        if (j > 0 && tile[j * W + s] != tile[(j - 1) * W + s]) colu[s] = 0;
      }
      __syncthreads();
      // a uniform column keeps its block: the sum of (c_j - 1) over all rows is 0
      for (int e = tid; e < nw; e += kKvBlock) {
        const int j = e / w, s = e - j * w;
        if (colu[s]) continue;
        const int32_t blk = tile[j * W + s];
        if (j > 0 && tile[(j - 1) * W + s] == blk) continue;  // not the head of its run
        int delta = 0;
        for (int jj = j; jj < N && tile[jj * W + s] == blk; ++jj) delta += cnt[jj] - 1;
        if (delta == 0) continue;
        if (blk < 0 || blk >= P) {
          atomicOr(&sFlags, SMCSD_ST_BAD_INPUT);
          continue;
        }
        if (delta > 0) atomicAdd(&rc[blk], delta);
        else negl[atomicAdd(&sNeg, 1)] = make_int2(blk, delta);
      }
      wait_memory();  // increments performed before any decrement
      __syncthreads();
      const int nneg = sNeg;
      for (int l0 = tid; l0 < nneg; l0 += kKvBlock * kNegBatch) {
        int2 q[kNegBatch];
        int old[kNegBatch];
#pragma unroll
        for (int k = 0; k < kNegBatch; ++k) {
          const int l = l0 + k * kKvBlock;
          q[k] = l < nneg ? negl[l] : make_int2(0, 0);
        }
#pragma unroll
        for (int k = 0; k < kNegBatch; ++k) old[k] = q[k].y ? atomicAdd(&rc[q[k].x], q[k].y) : 1;
#pragma unroll
        for (int k = 0; k < kNegBatch; ++k)
          if (q[k].y && old[k] + q[k].y == 0) atomicOr(&bitmap[q[k].x >> 5], 1u << (q[k].x & 31));
      }
      if (tail_partial && tail_slot >= s0 && tail_slot < s0 + w)
        for (int j = tid; j < N; j += kKvBlock) tail_old[j] = tile[j * W + (tail_slot - s0)];
      for (int e = tid; e < nw; e += kKvBlock) {
        const int i = e / w, s = e - i * w;
        const int32_t v = tile[a[i] * W + s];
        if (v != tile[i * W + s]) T[(row0 + i) * M_cap + s0 + s] = v;
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
  // this prompt (the highest holder keeps the block).  The highest holder of each tail
  // block comes from an LDS hash table keyed by block id.
  int32_t *hkey = reinterpret_cast<int32_t *>(negl);
  int32_t *hmax = hkey + kHash;
  if (tail_partial) {
    for (int h = tid; h < kHash; h += kKvBlock) {
      hkey[h] = -1;
      hmax[h] = -1;
    }
    __syncthreads();
    for (int i = tid; i < N; i += kKvBlock) {
      const int32_t blk = tail_new[i];
      if (blk >= P) atomicOr(&sFlags, SMCSD_ST_BAD_INPUT);
      if (blk < 0 || blk >= P) continue;
      int h = tail_hash(blk);
      for (;;) {  // at most N keys in 2N slots: an empty slot always exists
        const int32_t prev = atomicCAS(&hkey[h], -1, blk);
        if (prev == -1 || prev == blk) break;
        h = (h + 1) & (kHash - 1);
      }
      atomicMax(&hmax[h], i);
    }
    __syncthreads();
  }
  for (int i = tid; i < N; i += kKvBlock) {
    int32_t src = 0;
    if (tail_partial) {
      const int32_t blk = tail_new[i];
      if (blk >= 0 && blk < P) {
        int h = tail_hash(blk);
        while (hkey[h] != blk) h = (h + 1) & (kHash - 1);
        if (hmax[h] > i) src = blk + 1;
      }
    }
    cow_src[row0 + i] = src;
  }
  __syncthreads();
  if (tid == 0 && sFlags) atomicOr(status, sFlags);

  // ---- the last workgroup to arrive ranks the freed blocks and lays out the pops
  __threadfence();
  __syncthreads();
  if (tid == 0) sLast = atomicAdd(done, 1) == B - 1;
  __syncthreads();
  if (!sLast) return;
  __threadfence();
  const int top = *free_top;
  const int S = B * N;
  const int nfresh = nb_new - nb_old;
  const int sper = (S + kKvBlock - 1) / kKvBlock;
  const int g0 = min(S, tid * sper), g1 = min(S, g0 + sper);
  int mycow = 0;
  for (int g = g0; g < g1; ++g) mycow += cow_src[g] != 0;

  // freed blocks per group of kKvGroupWords bitmap words: wave w sums the groups
  // congruent to w mod 4, one 16-byte load per lane per group (the bitmap region is
  // padded to 64 words, so a load that starts below nwords stays inside it)
  const int nwords = (P + 31) / 32;
  const int ngroups = (nwords + kKvGroupWords - 1) / kKvGroupWords;
  const int lane = tid % kWave, wave = tid / kWave;
  const uint4 *bm4 = reinterpret_cast<const uint4 *>(bitmap);
  int F = 0;
  for (int r0 = 0; r0 < ngroups; r0 += kKvBlock) {
    const int ng = min(kKvBlock, ngroups - r0);
    for (int k0 = wave; k0 < ng; k0 += 8 * (kKvBlock / kWave)) {
      int c[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int gi = k0 + k * (kKvBlock / kWave);
        const int w4 = (r0 + gi) * kKvGroupWords + lane * 4;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (gi < ng && w4 < nwords) v = bm4[w4 / 4];
        c[k] = __popc(v.x) + __popc(v.y) + __popc(v.z) + __popc(v.w);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        int x = c[k];
        for (int m = kWave / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
        const int gi = k0 + k * (kKvBlock / kWave);
        if (lane == 0 && gi < ng) gcnt[gi] = x;
      }
    }
    __syncthreads();
    int tot;
    const int ex = kv_scan(tid < ng ? gcnt[tid] : 0, red, &tot);
    if (tid < ng) gbase[r0 + tid] = F + ex;
    F += tot;
  }

  // pop layout: sequence g owns pop indices [g*nfresh + cow_excl[g], ... + cow_g + nfresh);
  // pop k < F takes the freed block of ascending rank k, recorded in popmap for the pop
  // kernel, and pop k >= F the old stack entry at top + F - 1 - k
  int C;
  int ci = kv_scan(mycow, red, &C);
  const int64_t avail = (int64_t)top + F;
  int ok_cow = 0;  // copy-on-writes whose pop falls inside the stack
  for (int g = g0; g < g1; ++g) {
    const int f = cow_src[g] != 0;
    cow_excl[g] = ci;
    const int64_t k0 = (int64_t)g * nfresh + ci;
    ok_cow += f && k0 < avail;
    for (int64_t k = k0; k < k0 + f + nfresh && k < F; ++k) popmap[k] = g;
    ci += f;
  }
  int ncow_ok;
  kv_scan(ok_cow, red, &ncow_ok);
  if (tid == 0) {
    const int64_t npops = (int64_t)S * nfresh + C;
    scal[0] = top;
    scal[1] = F;
    scal[2] = (int32_t)min(npops, (int64_t)INT32_MAX);
    const int64_t nt = avail - npops;
    *free_top = (int32_t)(nt > 0 ? nt : 0);
    *cow_count = ncow_ok;
    *done = 0;
  }
}

// Workgroups [0, ngroups): one thread per freed-bitmap word; the rest: one thread per
// sequence.  A sequence's copy-on-write (tail slot) pops first, then its fresh slots.
__global__ __launch_bounds__(kKvBlock) void k_kv_pop(
    int S, int ngroups, int nwords, int32_t *__restrict__ T, int M_cap, int nb_old, int nb_new,
    int tail_slot, int tail_mod, int32_t *__restrict__ rc, int P, int32_t *__restrict__ free_list,
    uint32_t *__restrict__ bitmap, const int32_t *__restrict__ cow_src,
    const int32_t *__restrict__ cow_excl, const int32_t *__restrict__ gbase,
    const int32_t *__restrict__ popmap, const int32_t *__restrict__ scal,
    int32_t *__restrict__ cow, int32_t *status) {
  __shared__ int red[kKvBlock / kWave];
  const int tid = threadIdx.x;
  const int nfresh = nb_new - nb_old;
  const int F = scal[1], npops = scal[2];
  const int64_t avail = (int64_t)scal[0] + F;
  int flags = 0;
  if ((int)blockIdx.x < ngroups) {
    // the freed block of ascending rank r goes to stack position top + F - 1 - r (pushed
    // in descending id order); if pop r is requested it also fills that pop's slot
    const int gi = blockIdx.x;
    const int w = gi * kKvGroupWords + tid;
    uint32_t bits = w < nwords ? bitmap[w] : 0u;
    const int base = gbase[gi];
    int tot;
    int r = base + kv_scan(__popc(bits), red, &tot);
    if (bits) bitmap[w] = 0u;
    for (; bits; bits &= bits - 1, ++r) {
      const int32_t d = w * 32 + __ffs(bits) - 1;
      const int64_t pos = avail - 1 - r;
      if (pos >= 0 && pos < P) free_list[pos] = d;
      else flags |= SMCSD_ST_BAD_INPUT;
      if (r < npops) {
        const int g = popmap[r];
        const int f = cow_src[g] != 0, ce = cow_excl[g];
        const int st = (int)(r - ((int64_t)g * nfresh + ce)) - f;
        rc[d] = 1;
        T[(int64_t)g * M_cap + (st < 0 ? tail_slot : nb_old + st)] = d;
        if (st < 0) cow[3 * ce + 1] = d;
      }
    }
  } else {
    const int g = (blockIdx.x - ngroups) * kKvBlock + tid;
    if (g < S) {
      const int32_t cs = cow_src[g];
      const int ce = cow_excl[g];
      int64_t k = (int64_t)g * nfresh + ce;
      for (int st = cs ? -1 : 0; st < nfresh; ++st, ++k) {
        if (k >= avail) {
          flags |= SMCSD_ST_NOSPACE;
          continue;
        }
        int32_t d = -1;
        if (k >= F) {  // from the old stack
          const int64_t pos = avail - 1 - k;
          d = pos < P ? free_list[pos] : -1;
          if (d < 0 || d >= P) {
            flags |= SMCSD_ST_BAD_INPUT;
            continue;
          }
        }
        if (st < 0) {
          atomicSub(&rc[cs - 1], 1);
          cow[3 * ce + 0] = cs - 1;
          cow[3 * ce + 2] = tail_mod;
        }
        if (d >= 0) {
          rc[d] = 1;
          T[(int64_t)g * M_cap + (st < 0 ? tail_slot : nb_old + st)] = d;
          if (st < 0) cow[3 * ce + 1] = d;
        }
      }
    }
  }
  if (flags) atomicOr(status, flags);
}

hipError_t launch_kv(const int32_t *anc, const int32_t *resampled, int B, int N, int32_t *tables,
                     int M_cap, int bs, int64_t L, int R, int32_t *rc, int32_t *free_list,
                     int32_t *free_top, int64_t P, int32_t *cow, int32_t *cow_count,
                     int32_t *status, char *ws, hipStream_t stream) {
  const int S = B * N;
  const KvWs w = kv_ws_layout(S, P);
  uint32_t *bitmap = reinterpret_cast<uint32_t *>(ws + w.bitmap);
  int32_t *cow_src = reinterpret_cast<int32_t *>(ws + w.cow_src);
  int32_t *cow_excl = reinterpret_cast<int32_t *>(ws + w.cow_excl);
  int32_t *gbase = reinterpret_cast<int32_t *>(ws + w.gbase);
  int32_t *popmap = reinterpret_cast<int32_t *>(ws + w.popmap);
  int32_t *done = reinterpret_cast<int32_t *>(ws + w.done);
  int32_t *scal = reinterpret_cast<int32_t *>(ws + w.scal);
  const int nb_old = (int)ceil_div(L, bs);
  const int nb_new = (int)ceil_div(L + R, bs);
  const int tail_slot = (int)(L / bs), tail_mod = (int)(L % bs);
  const int nwords = (int)ceil_div(P, 32);
  const int ngroups = (int)ceil_div(nwords, kKvGroupWords);
  hipLaunchKernelGGL(k_kv, dim3(B), dim3(kKvBlock), 0, stream, anc, resampled, B, N, tables, M_cap,
                     nb_old, nb_new, tail_slot, tail_mod, rc, (int)P, free_top, bitmap, cow_src,
                     cow_excl, gbase, popmap, scal, done, cow_count, status);
  hipLaunchKernelGGL(k_kv_pop, dim3(ngroups + (S + kKvBlock - 1) / kKvBlock), dim3(kKvBlock), 0,
                     stream, S, ngroups, nwords, tables, M_cap, nb_old, nb_new, tail_slot, tail_mod,
                     rc, (int)P, free_list, bitmap, cow_src, cow_excl, gbase, popmap, scal, cow,
                     status);
  return hipGetLastError();
}

}  // namespace smcsd
