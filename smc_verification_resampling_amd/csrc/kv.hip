// kv.hip - KV cache pointer exchange with reference counts (gfx950).
//
// After resampling, the KV cache follows the particles by exchanging block pointers and
// updating reference counts; prefixes stay shared across particles and no KV data is
// copied (SMC explainers, "system optimisation design": KV cache; Spanish page, cache
// management).  Integer work only, two launches per call, bit-deterministic although it
// uses atomics:
//   * k_kv, one workgroup per prompt: the exchange over column tiles of the prompt's
//     tables staged in LDS.  Down each column (one thread per column and 16-row segment)
//     a run of equal blocks gets one refcount change, sum over the run of (c_j - 1); all
//     increments are performed (waited for, then a barrier) before any decrement, so a
//     block that stays referenced never reaches 0, and the decrement that brings a count
//     to 0 marks the block in a freed bitmap and counts it in its group of 8192 ids,
//     exactly once.  With at most 16 particles one thread holds a whole column; it issues
//     the column's increments and then its decrements with no wait, since one thread's
//     atomics on an address take effect in program order.  Then the gathered tables and
//     the copy-on-write decision for the partial tail.
//   * k_kv_pop_fast (up to 8192 sequences), one thread per bitmap word and one per
//     sequence: every workgroup first forms the group-count prefix and the copy-on-write
//     prefix itself; a freed block's rank in ascending id order fixes its stack position
//     (pushed in descending id order) and, if that pop is requested, the table slot it
//     fills; sequences take their remaining pops from the old stack.
//   * with more sequences, the last k_kv workgroup to finish (a device-scope counter with
//     release / acquire fences) lays out the pops for k_kv_pop instead.
// The bitmap and group counts alternate between two buffers by call parity, so a call
// clears the pair its predecessor used while nobody reads it.
#include "device.hpp"
#include "internal.hpp"
#include "kv_layout.hpp"
#include "resample.hpp"

namespace smcsd {

constexpr int kKvBlock = kKvThreads;
constexpr int kKvTileInts = kKvTileEntries;  // table entries staged per column tile (32 KiB)
constexpr int kStage = 16;         // table loads in flight per thread while staging
constexpr int kNegBatch = 4;       // decrements in flight per thread
constexpr int kHash = 2 * kMaxN;   // open-addressing table of the tail blocks (load <= 1/2)
constexpr int kSeg = 16;           // table rows one thread walks down a column
// first-tile entries each prefetching thread loads up front (enough for three waves)
constexpr int kPre = (kKvTileInts + kKvBlock - kWave - 1) / (kKvBlock - kWave);

// Wait until every memory operation this wave issued (atomics included) has completed.
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Exclusive scan over the 256 threads of the workgroup; *total gets the sum.
__device__ __forceinline__ int kv_scan(int v, int *lds, int *total) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int inc = wave_inclusive_scan(v);
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

// Three scans over the workgroup in one pass: returns the exclusive prefix of v.z and
// writes the totals of v.x, v.y, v.z.  lds holds 3 * (kKvBlock / kWave) ints and must not
// be reused before the next barrier.
__device__ __forceinline__ int kv_scan3(int3 v, int *lds, int3 *total) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int3 inc = make_int3(wave_inclusive_scan(v.x), wave_inclusive_scan(v.y),
                             wave_inclusive_scan(v.z));
  constexpr int kW = kKvBlock / kWave;
  if (lane == kWave - 1) {
    lds[wave] = inc.x;
    lds[kW + wave] = inc.y;
    lds[2 * kW + wave] = inc.z;
  }
  __syncthreads();
  int3 tot = make_int3(0, 0, 0);
  int base = 0;
  for (int w = 0; w < kW; ++w) {
    tot.x += lds[w];
    tot.y += lds[kW + w];
    const int z = lds[2 * kW + w];
    if (w < wave) base += z;
    tot.z += z;
  }
  *total = tot;
  return base + inc.z - v.z;
}

__device__ __forceinline__ int tail_hash(int32_t blk) {
  return (int)(((uint32_t)blk * 0x9E3779B1u) >> 21) & (kHash - 1);
}

struct KvBufs {
  uint32_t *bitmap2;  // two bitmaps of nwp words
  int32_t *gcount2;   // two arrays of ngp group counts
  int nwords, ngroups, nwp, ngp;
  int32_t *cow_src, *cow_excl, *gbase, *popmap, *done, *ctr, *scal;
};

static_assert(kKvBlock == kResBlock, "the fused resample runs on the KV workgroup");

// Log-weights of resampled prompts that the pop kernel resets (lw == nullptr: none), when
// the fused resample ran in several workgroups per prompt.
struct LwReset {
  float *lw;
  const int32_t *res;
  int N;
};

// fr.lw != nullptr: the Resample step is fused in - each workgroup first resamples its
// prompt (the same device code as smcsd_resample, so the same bits) and takes the
// ancestors from LDS; anc / resampled are then unused.
// parts > 1: a prompt's old table columns are split over `parts` workgroups (blockIdx.x =
// prompt * parts + part), `span` columns each; a block id sits in one column only, so the
// refcount changes of different columns are independent.  The workgroup whose columns hold
// the partial tail (part 0 when there is none) makes the prompt's copy-on-write decision;
// with tail_alone that is the last part, which holds the tail column only, so the decision
// runs beside the other parts' columns instead of after a full part's.
// With the resample fused in, every part resamples the prompt (the same bits), part 0
// writes the ancestors, ESS and decision, and the log-weights of resampled prompts are
// reset by the pop kernel, after every part has read them.
__global__ __launch_bounds__(kKvBlock) void k_kv(
    const int32_t *__restrict__ anc, const int32_t *__restrict__ resampled, FusedResample fr,
    int B, int N, int parts, int span, int tail_alone, int32_t *__restrict__ T, int M_cap,
    int nb_old,
    int nb_new, int tail_slot, int tail_mod, int32_t *__restrict__ rc, int P,
    int32_t *__restrict__ free_top, KvBufs wb, int fast, int32_t *__restrict__ cow_count,
    int32_t *status) {
  __shared__ int32_t a[kMaxN], cnt[kMaxN], tail_old[kMaxN], tail_new[kMaxN];
  __shared__ int32_t tile[kKvTileInts];
  __shared__ uint8_t colu[kKvTileInts];  // column of the tile holds one block in every row
  __shared__ int2 negl[kKvTileInts];     // (block, decrement); later the tail hash table
  __shared__ int red[kKvBlock / kWave];
  __shared__ int sFlags, sValid, sLast, sNeg;
  const int b = blockIdx.x / parts, part = blockIdx.x - b * parts, tid = threadIdx.x;
  const int row0 = b * N;
  const int tail_partial = tail_mod != 0;
  const bool tail_part = tail_alone && part == parts - 1;
  const int body_end = tail_alone ? nb_old - 1 : nb_old;
  const int c_begin = tail_part ? nb_old - 1 : min(body_end, part * span);
  const int c_end = tail_part ? nb_old : min(body_end, c_begin + span);
  const bool tail_owner =
      tail_partial ? tail_slot >= c_begin && tail_slot < c_end : part == 0;
  int32_t *__restrict__ cow_src = wb.cow_src;
  if (tid == 0) {
    sFlags = 0;
    sValid = 1;
  }
  // the call counter is only read here (the pop kernel advances it); its parity selects
  // this call's bitmap and group counts
  const int C = *wb.ctr;
  uint32_t *__restrict__ bitmap = wb.bitmap2 + (C & 1) * wb.nwp;
  int32_t *__restrict__ gcount = wb.gcount2 + (C & 1) * wb.ngp;
  if (blockIdx.x == 0 && tid == 0) {
    wb.scal[0] = *free_top;
    wb.scal[3] = C;
  }
  // the ancestor row and the first column tile of the old tables are read whether or not
  // the prompt resampled, so all of this workgroup's first loads overlap.  With the fused
  // one-wave resample, wave 0 loads only the prompt's log-weights and the other waves take
  // its share of the tile: the load counter is per wave, so wave 0's resample then waits
  // for its own load alone while the tile is still arriving.
  const bool split = fr.lw && N <= kWave;
  const float lw0 = split && tid < N ? fr.lw[row0 + tid] : 0.0f;
  const int pthr = split ? kKvBlock - kWave : kKvBlock;  // threads that prefetch
  const int pid = split ? tid - kWave : tid;              // this one's index among them
  const int W = max(1, min(c_end - c_begin, kKvTileInts / N));
  const int w0 = min(W, c_end - c_begin), nw0 = N * w0;
  int32_t pre[kPre];
  {
    // entry e = pid + k * pthr sits at row j = e / w0, column s = e % w0: two divisions up
    // front, then a carry per step instead of a division per entry
    const int wd = max(w0, 1);  // w0 = 0 (no columns): nothing is loaded
    const int dj = pthr / wd, ds = pthr - dj * wd;
    int j = pid >= 0 ? pid / wd : 0;
    int s = pid >= 0 ? pid - j * wd : 0;
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      const int e = pid + k * pthr;
      pre[k] = 0;
      if (pid >= 0 && e < nw0) pre[k] = T[(row0 + j) * M_cap + c_begin + s];
      j += dj;
      s += ds;
      if (s >= wd) {
        s -= wd;
        ++j;
      }
    }
  }
  // with the one-wave resample, waves 1-3 stage the first tile in LDS as soon as their
  // loads are in, while wave 0 resamples (the resample does not touch the tile)
  if (split && pid >= 0) {
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      const int e = pid + k * pthr;
      if (e < nw0) tile[e] = pre[k];
    }
  }
  int res;
  if (fr.lw) {
    __shared__ ResampleLds sResL;
    __shared__ int sRes;
    if (N <= kWave) {
      if (tid < kWave) {
        const int d = resample_prompt_wave(lw0, fr.lw + row0, N, fr.tau, fr.seed, b, fr.step,
                                           fr.anc + row0, fr.ess + b, fr.res + b, status, a,
                                           part == 0, parts == 1);
        if (tid == 0) sRes = d;
      }
    } else {
      const int d = resample_prompt_block(fr.lw + row0, N, fr.tau, fr.seed, b, fr.step,
                                          fr.anc + row0, fr.ess + b, fr.res + b, status, a, sResL,
                                          part == 0, parts == 1);
      if (tid == 0) sRes = d;
    }
    for (int i = tid; i < N; i += kKvBlock) cnt[i] = 0;
    __syncthreads();
    res = sRes;
  } else {
    res = resampled[b] != 0;
    for (int i = tid; i < N; i += kKvBlock) {
      a[i] = anc[row0 + i];
      cnt[i] = 0;
    }
    __syncthreads();
  }
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
    const int nseg = (N + kSeg - 1) / kSeg;
    for (int s0 = c_begin; s0 < c_end; s0 += W) {
      const int w = min(W, c_end - s0), nw = N * w;
      if (s0 == c_begin && !split) {
        // the first tile is W columns wide (W = min(c_end - c_begin, kKvTileInts / N) = w),
        // so entry e = j * w + s sits at tile[e]: no division on this path
#pragma unroll
        for (int k = 0; k < kPre; ++k) {
          const int e = pid + k * pthr;
          if (pid >= 0 && e < nw) tile[e] = pre[k];
        }
      }
      for (int e0 = tid; s0 > c_begin && e0 < nw; e0 += kKvBlock * kStage) {
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
      if (tid == 0) sNeg = 0;
      if (nseg > 1)
        for (int s = tid; s < w; s += kKvBlock) colu[s] = 1;
      __syncthreads();
      if (nseg > 1) {
        // columns of more than one segment: flag the uniform ones (a block shared by every
        // row keeps its count, the sum of (c_j - 1) over all rows being 0)
        for (int e = tid; e < nw; e += kKvBlock) {
          const int j = e / w, s = e - j * w;
          if (j > 0 && tile[j * W + s] != tile[(j - 1) * W + s]) colu[s] = 0;
        }
        __syncthreads();
      }
      // one thread per (column, segment of kSeg rows): each run of equal blocks down the
      // segment gets one refcount change, the sum of (c_j - 1) over the run.  Increments
      // are issued at once; decrements are listed for after them (a run split over
      // segments gets one change per piece: every piece that increments still lands
      // before every piece that decrements).
      for (int it = tid; it < w * nseg; it += kKvBlock) {
        const int sg = it / w, s = it - sg * w;
        const int j0 = sg * kSeg, j1 = min(N, j0 + kSeg);
        int32_t v[kSeg];
        int d[kSeg];
#pragma unroll
        for (int k = 0; k < kSeg; ++k) {
          const int j = min(j0 + k, N - 1);
          v[k] = tile[j * W + s];
          d[k] = cnt[j] - 1;
        }
        if (tail_partial && s0 + s == tail_slot) {
#pragma unroll
          for (int k = 0; k < kSeg; ++k)
            if (j0 + k < j1) tail_old[j0 + k] = v[k];
        }
        // a block id outside [0, P) in an allocated slot (one a NOSPACE call left at -1, or a
        // corrupt table) is flagged wherever it sits, and changes no count
        bool oob = false;
#pragma unroll
        for (int k = 0; k < kSeg; ++k) oob |= j0 + k < j1 && (v[k] < 0 || v[k] >= P);
        if (oob) atomicOr(&sFlags, SMCSD_ST_BAD_INPUT);
        if (nseg > 1 && colu[s]) continue;
        if (nseg == 1) {
          // the whole column is in this thread, and a thread's atomics on one address take
          // effect in program order: its increments, then at once its decrements, leave no
          // block at a transient 0 and need no wait between them.  accs[k] is the change of
          // the run that ends at row k (0 elsewhere).
          int accs[kSeg], olds[kSeg];
          int run = 0;
#pragma unroll
          for (int k = 0; k < kSeg; ++k) {
            run += k < N ? d[k] : 0;
            const bool end = k < N && (k == N - 1 || (k + 1 < kSeg && v[k + 1] != v[k]));
            accs[k] = end ? run : 0;
            if (end) run = 0;
            if (v[k] < 0 || v[k] >= P) accs[k] = 0;
          }
#pragma unroll
          for (int k = 0; k < kSeg; ++k)
            if (accs[k] > 0) atomicAdd(&rc[v[k]], accs[k]);
#pragma unroll
          for (int k = 0; k < kSeg; ++k) olds[k] = accs[k] < 0 ? atomicAdd(&rc[v[k]], accs[k]) : 1;
#pragma unroll
          for (int k = 0; k < kSeg; ++k)
            if (accs[k] < 0 && olds[k] + accs[k] == 0) {
              atomicOr(&bitmap[v[k] >> 5], 1u << (v[k] & 31));
              atomicAdd(&gcount[v[k] / kKvGroupBlocks], 1);
            }
          continue;
        }
        int32_t blk = v[0];
        int acc = 0;
        auto flush = [&]() {
          if (acc == 0 || blk < 0 || blk >= P) return;  // out-of-range ids flagged above
          if (acc > 0) atomicAdd(&rc[blk], acc);
          else negl[atomicAdd(&sNeg, 1)] = make_int2(blk, acc);
        };
#pragma unroll
        for (int k = 0; k < kSeg; ++k) {
          if (j0 + k < j1) {
            if (v[k] != blk) {
              flush();
              blk = v[k];
              acc = 0;
            }
            acc += d[k];
          }
        }
        flush();
      }
      if (nseg > 1) wait_memory();  // increments performed before any decrement
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
          if (q[k].y && old[k] + q[k].y == 0) {
            atomicOr(&bitmap[q[k].x >> 5], 1u << (q[k].x & 31));
            atomicAdd(&gcount[q[k].x / kKvGroupBlocks], 1);
          }
      }
      // the new tables (stores issued after the refcount waits, so nothing waits on them
      // before the kernel ends)
      for (int it = tid; it < w * nseg; it += kKvBlock) {
        const int sg = it / w, s = it - sg * w;
        const int j0 = sg * kSeg, j1 = min(N, j0 + kSeg);
#pragma unroll
        for (int k = 0; k < kSeg; ++k) {
          const int i = j0 + k;
          if (i < j1) {
            const int32_t nv = tile[a[i] * W + s];
            if (nv != tile[i * W + s]) T[(row0 + i) * M_cap + s0 + s] = nv;
          }
        }
      }
      __syncthreads();
    }
    if (tail_partial && tail_owner)
      for (int i = tid; i < N; i += kKvBlock) tail_new[i] = tail_old[a[i]];
  } else if (tail_partial && tail_owner) {
    for (int i = tid; i < N; i += kKvBlock) tail_new[i] = T[(row0 + i) * M_cap + tail_slot];
  }
  __syncthreads();

  // copy-on-write decision: the partial tail is also held by a higher-index sequence of
  // this prompt (the highest holder keeps the block).  The highest holder of each tail
  // block comes from an LDS hash table keyed by block id.
  int32_t *hkey = reinterpret_cast<int32_t *>(negl);
  int32_t *hmax = hkey + kHash;
  if (tail_partial && tail_owner) {
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
  for (int i = tid; tail_owner && i < N; i += kKvBlock) {
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

  if (fast) return;

  // ---- many sequences: the last workgroup to arrive forms the group rank bases and lays
  // out the pops for k_kv_pop
  __threadfence();
  __syncthreads();
  if (tid == 0) sLast = atomicAdd(wb.done, 1) == (int)gridDim.x - 1;
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
  int F = 0;
  for (int r0 = 0; r0 < wb.ngroups; r0 += kKvBlock) {
    const int q = r0 + tid;
    int tot;
    const int ex = kv_scan(q < wb.ngroups ? gcount[q] : 0, red, &tot);
    if (q < wb.ngroups) wb.gbase[q] = F + ex;
    F += tot;
  }

  // pop layout: sequence g owns pop indices [g*nfresh + cow_excl[g], ... + cow_g + nfresh);
  // pop k < F takes the freed block of ascending rank k, recorded in popmap for the pop
  // kernel, and pop k >= F the old stack entry at top + F - 1 - k
  int Ctot;
  int ci = kv_scan(mycow, red, &Ctot);
  const int64_t avail = (int64_t)top + F;
  int ok_cow = 0;  // copy-on-writes whose pop falls inside the stack
  for (int g = g0; g < g1; ++g) {
    const int f = cow_src[g] != 0;
    wb.cow_excl[g] = ci;
    const int64_t k0 = (int64_t)g * nfresh + ci;
    ok_cow += f && k0 < avail;
    for (int64_t k = k0; k < k0 + f + nfresh && k < F; ++k) wb.popmap[k] = g;
    ci += f;
  }
  int ncow_ok;
  kv_scan(ok_cow, red, &ncow_ok);
  if (tid == 0) {
    const int64_t npops = (int64_t)S * nfresh + Ctot;
    wb.scal[1] = F;
    wb.scal[2] = (int32_t)min(npops, (int64_t)INT32_MAX);
    const int64_t nt = avail - npops;
    *free_top = (int32_t)(nt > 0 ? nt : 0);
    *cow_count = ncow_ok;
    *wb.done = 0;
  }
}

// Clear the bitmap and group counts of the other parity (used by the previous call) and,
// from workgroup 0, advance the call counter.
__device__ __forceinline__ void kv_clear_other(const KvBufs &wb, int C) {
  uint32_t *ob = wb.bitmap2 + ((C + 1) & 1) * wb.nwp;
  int32_t *og = wb.gcount2 + ((C + 1) & 1) * wb.ngp;
  const int stride = gridDim.x * kKvBlock;
  for (int i = blockIdx.x * kKvBlock + threadIdx.x; i < wb.nwords; i += stride) ob[i] = 0u;
  for (int i = blockIdx.x * kKvBlock + threadIdx.x; i < wb.ngroups; i += stride) og[i] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) *wb.ctr = C + 1;
}

// Pops of one sequence (one thread per sequence): its copy-on-write (tail slot) pops
// first, then its fresh slots; pop k takes the freed block of rank k when k < F (written
// by the bitmap-word threads) and otherwise the old stack entry at top + F - 1 - k.
__device__ __forceinline__ int kv_sequence_pops(int g, int32_t cs, int ce, int nfresh, int F,
                                                int64_t avail, int32_t *__restrict__ T, int M_cap,
                                                int nb_old, int tail_slot, int tail_mod,
                                                int32_t *__restrict__ rc, int P,
                                                const int32_t *__restrict__ free_list,
                                                int32_t *__restrict__ cow) {
  int flags = 0;
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
        // a corrupt stack entry: flagged; a copy-on-write is listed with destination -1
        // and nothing else changes
        flags |= SMCSD_ST_BAD_INPUT;
        if (st < 0) {
          cow[3 * ce + 0] = cs - 1;
          cow[3 * ce + 1] = -1;
          cow[3 * ce + 2] = tail_mod;
        }
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
  return flags;
}

// A freed block d of ascending rank r: stack position top + F - 1 - r (pushed in
// descending id order); if pop r is requested (r < npops) it also fills that pop's slot
// of sequence g, whose pops start at start_g and begin with a copy-on-write when f = 1.
__device__ __forceinline__ void kv_place_freed(int32_t d, int64_t r, int64_t avail, int P,
                                               int32_t *__restrict__ free_list, int &flags) {
  const int64_t pos = avail - 1 - r;
  if (pos >= 0 && pos < P) free_list[pos] = d;
  else flags |= SMCSD_ST_BAD_INPUT;
}
__device__ __forceinline__ void kv_fill_pop(int32_t d, int g, int st, int ce, int32_t *__restrict__ T,
                                            int M_cap, int nb_old, int tail_slot,
                                            int32_t *__restrict__ rc, int32_t *__restrict__ cow) {
  rc[d] = 1;
  T[(int64_t)g * M_cap + (st < 0 ? tail_slot : nb_old + st)] = d;
  if (st < 0) cow[3 * ce + 1] = d;
}

// Many-sequence path.  Workgroups [0, ngroups): one thread per word of this call's bitmap;
// the rest: one thread per sequence.  Uses the layout the last k_kv workgroup wrote.
__global__ __launch_bounds__(kKvBlock) void k_kv_pop(
    int S, int32_t *__restrict__ T, int M_cap, int nb_old, int nb_new, int tail_slot,
    int tail_mod, int32_t *__restrict__ rc, int P, int32_t *__restrict__ free_list, KvBufs wb,
    int32_t *__restrict__ cow, int32_t *status, LwReset lr) {
  __shared__ int32_t sList[kKvGroupBlocks];  // this group's freed block ids, ascending
  __shared__ int red[kKvBlock / kWave];
  const int tid = threadIdx.x;
  const int nfresh = nb_new - nb_old;
  const int C = wb.scal[3];
  const int F = wb.scal[1], npops = wb.scal[2];
  const int64_t avail = (int64_t)wb.scal[0] + F;
  const uint32_t *bitmap = wb.bitmap2 + (C & 1) * wb.nwp;
  int flags = 0;
  if ((int)blockIdx.x < wb.ngroups) {
    const int gi = blockIdx.x;
    const int w = gi * kKvGroupWords + tid;
    uint32_t bits = w < wb.nwords ? bitmap[w] : 0u;
    const int base = wb.gbase[gi];
    int tot;
    int j = kv_scan(__popc(bits), red, &tot);
    for (; bits; bits &= bits - 1, ++j) sList[j] = w * 32 + __ffs(bits) - 1;
    __syncthreads();
    for (int i = tid; i < tot; i += kKvBlock) {
      const int32_t d = sList[i];
      const int64_t r = (int64_t)base + i;
      kv_place_freed(d, r, avail, P, free_list, flags);
      if (r < npops) {
        const int g = wb.popmap[r];
        const int f = wb.cow_src[g] != 0, ce = wb.cow_excl[g];
        const int st = (int)(r - ((int64_t)g * nfresh + ce)) - f;
        if (st >= -f && st < nfresh) kv_fill_pop(d, g, st, ce, T, M_cap, nb_old, tail_slot, rc, cow);
      }
    }
  } else {
    const int g = (blockIdx.x - wb.ngroups) * kKvBlock + tid;
    if (g < S) {
      flags |= kv_sequence_pops(g, wb.cow_src[g], wb.cow_excl[g], nfresh, F, avail, T, M_cap,
                                nb_old, tail_slot, tail_mod, rc, P, free_list, cow);
      if (lr.lw && lr.res[g / lr.N]) lr.lw[g] = 0.0f;
    }
  }
  kv_clear_other(wb, C);
  if (flags) atomicOr(status, flags);
}

// One-pass path (S <= kKvFastSeqMax, ngroups <= kKvFastGroupMax): every workgroup forms the
// group-count prefix and the copy-on-write prefix itself, then workgroups [0, ngroups)
// place the freed blocks of their bitmap words and the rest make the sequences' pops.
constexpr int kGPer = kKvFastGroupMax / kKvBlock;
constexpr int kSPer = kKvFastSeqMax / kKvBlock;

__global__ __launch_bounds__(kKvBlock) void k_kv_pop_fast(
    int S, int32_t *__restrict__ T, int M_cap, int nb_old, int nb_new, int tail_slot,
    int tail_mod, int32_t *__restrict__ rc, int P, int32_t *__restrict__ free_list,
    int32_t *__restrict__ free_top, KvBufs wb, int32_t *__restrict__ cow,
    int32_t *__restrict__ cow_count, int32_t *status, LwReset lr) {
  __shared__ int32_t sSrc[kKvFastSeqMax];  // copy-on-write source + 1 per sequence
  __shared__ int32_t sEx[kKvFastSeqMax];   // exclusive prefix of the copy-on-write flags
  __shared__ int32_t sList[kKvGroupBlocks];  // this group's freed block ids, ascending
  __shared__ int red[kKvBlock / kWave];
  __shared__ int red3[3 * (kKvBlock / kWave)];
  const int tid = threadIdx.x;
  const int gi = blockIdx.x;
  const bool word_wg = gi < wb.ngroups;
  const int nfresh = nb_new - nb_old;

  // one round of loads: scalars, this group's word in both bitmaps, both parities of the
  // group counts, this thread's run of copy-on-write sources
  const int C = wb.scal[3], top = wb.scal[0];
  const int w = gi * kKvGroupWords + tid;
  uint32_t wb0 = 0u, wb1 = 0u;
  if (word_wg && w < wb.nwords) {
    wb0 = wb.bitmap2[w];
    wb1 = wb.bitmap2[wb.nwp + w];
  }
  int gc0[kGPer], gc1[kGPer];
#pragma unroll
  for (int k = 0; k < kGPer; ++k) {
    const int q = tid + k * kKvBlock;
    gc0[k] = q < wb.ngroups ? wb.gcount2[q] : 0;
    gc1[k] = q < wb.ngroups ? wb.gcount2[wb.ngp + q] : 0;
  }
  const int sper = (S + kKvBlock - 1) / kKvBlock;
  const int g0 = min(S, tid * sper), g1 = min(S, g0 + sper);
  int cs[kSPer];
#pragma unroll
  for (int k = 0; k < kSPer; ++k) cs[k] = g0 + k < g1 ? wb.cow_src[g0 + k] : 0;

  const int par = C & 1;
  const uint32_t bits0 = par ? wb1 : wb0;
  int Fpart = 0, below = 0, mycow = 0;
#pragma unroll
  for (int k = 0; k < kGPer; ++k) {
    const int v = par ? gc1[k] : gc0[k];
    Fpart += v;
    if (tid + k * kKvBlock < gi) below += v;
  }
#pragma unroll
  for (int k = 0; k < kSPer; ++k) mycow += cs[k] != 0;
  int3 tot3;
  int ci = kv_scan3(make_int3(Fpart, below, mycow), red3, &tot3);
  const int F = tot3.x, base = tot3.y, Ctot = tot3.z;
#pragma unroll
  for (int k = 0; k < kSPer; ++k) {
    if (g0 + k < g1) {
      sSrc[g0 + k] = cs[k];
      sEx[g0 + k] = ci;
    }
    ci += cs[k] != 0;
  }
  const int64_t avail = (int64_t)top + F;
  const int64_t npops = (int64_t)S * nfresh + Ctot;
  __syncthreads();

  int flags = 0;
  if (word_wg) {
    // the group's freed ids in ascending order into LDS (freed blocks cluster in low ids,
    // so a word can hold many), then one thread per freed block
    uint32_t bits = bits0;
    int tot;
    int j = kv_scan(__popc(bits), red, &tot);
    for (; bits; bits &= bits - 1, ++j) sList[j] = w * 32 + __ffs(bits) - 1;
    __syncthreads();
    for (int i = tid; i < tot; i += kKvBlock) {
      const int32_t d = sList[i];
      const int64_t r = (int64_t)base + i;
      kv_place_freed(d, r, avail, P, free_list, flags);
      if (r < npops) {
        // the owner of pop r: the last sequence whose first pop index is <= r
        int lo = 0, hi = S - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if ((int64_t)mid * nfresh + sEx[mid] <= r) lo = mid;
          else hi = mid - 1;
        }
        const int ce = sEx[lo], f = sSrc[lo] != 0;
        const int st = (int)(r - ((int64_t)lo * nfresh + ce)) - f;
        if (st >= -f && st < nfresh) kv_fill_pop(d, lo, st, ce, T, M_cap, nb_old, tail_slot, rc, cow);
      }
    }
    if (gi == 0) {
      // copy-on-writes whose pop falls inside the stack, and the new top
      int ok = 0;
      for (int g = g0; g < g1; ++g) ok += sSrc[g] != 0 && (int64_t)g * nfresh + sEx[g] < avail;
      int ncow_ok;
      kv_scan(ok, red, &ncow_ok);
      if (tid == 0) {
        const int64_t nt = avail - npops;
        *free_top = (int32_t)(nt > 0 ? nt : 0);
        *cow_count = ncow_ok;
      }
    }
  } else {
    const int g = (gi - wb.ngroups) * kKvBlock + tid;
    if (g < S) {
      flags |= kv_sequence_pops(g, sSrc[g], sEx[g], nfresh, F, avail, T, M_cap, nb_old,
                                tail_slot, tail_mod, rc, P, free_list, cow);
      if (lr.lw && lr.res[g / lr.N]) lr.lw[g] = 0.0f;
    }
  }
  kv_clear_other(wb, C);
  if (flags) atomicOr(status, flags);
}

hipError_t launch_kv(const int32_t *anc, const int32_t *resampled, const FusedResample &fr, int B,
                     int N, int32_t *tables, int M_cap, int bs, int64_t L, int R, int32_t *rc,
                     int32_t *free_list, int32_t *free_top, int64_t P, int32_t *cow,
                     int32_t *cow_count, int32_t *status, char *ws, hipStream_t stream) {
  const int S = B * N;
  const KvWs w = kv_ws_layout(S, P);
  KvBufs wb;
  wb.bitmap2 = reinterpret_cast<uint32_t *>(ws + w.bitmap);
  wb.gcount2 = reinterpret_cast<int32_t *>(ws + w.gcount);
  wb.nwords = (int)w.nwords;
  wb.ngroups = (int)w.ngroups;
  wb.nwp = (int)w.nwp;
  wb.ngp = (int)w.ngp;
  wb.cow_src = reinterpret_cast<int32_t *>(ws + w.cow_src);
  wb.cow_excl = reinterpret_cast<int32_t *>(ws + w.cow_excl);
  wb.gbase = reinterpret_cast<int32_t *>(ws + w.gbase);
  wb.popmap = reinterpret_cast<int32_t *>(ws + w.popmap);
  wb.done = reinterpret_cast<int32_t *>(ws + w.done);
  wb.ctr = reinterpret_cast<int32_t *>(ws + w.ctr);
  wb.scal = reinterpret_cast<int32_t *>(ws + w.scal);
  const int nb_old = (int)ceil_div(L, bs);
  const int nb_new = (int)ceil_div(L + R, bs);
  const int tail_slot = (int)(L / bs), tail_mod = (int)(L % bs);
  const int fast = S <= kKvFastSeqMax && w.ngroups <= kKvFastGroupMax;
  const unsigned grid2 = (unsigned)(w.ngroups + (S + kKvBlock - 1) / kKvBlock);
  // prompts split over column parts (kv_split); with the resample fused in, each part
  // resamples the prompt and the pop kernel resets the log-weights
  const KvSplit ks = kv_split(N, nb_old, tail_mod);
  const int tail_alone = ks.tail_alone, span = ks.span, parts = ks.parts;
  const LwReset lr = fr.lw && parts > 1 ? LwReset{fr.lw, fr.res, N} : LwReset{nullptr, nullptr, 1};
  hipLaunchKernelGGL(k_kv, dim3((unsigned)((int64_t)B * parts)), dim3(kKvBlock), 0, stream, anc,
                     resampled, fr, B, N, parts, span, tail_alone, tables, M_cap, nb_old, nb_new,
                     tail_slot, tail_mod, rc, (int)P, free_top, wb, fast, cow_count, status);
  if (fast)
    hipLaunchKernelGGL(k_kv_pop_fast, dim3(grid2), dim3(kKvBlock), 0, stream, S, tables, M_cap,
                       nb_old, nb_new, tail_slot, tail_mod, rc, (int)P, free_list, free_top, wb, cow,
                       cow_count, status, lr);
  else
    hipLaunchKernelGGL(k_kv_pop, dim3(grid2), dim3(kKvBlock), 0, stream, S, tables, M_cap, nb_old,
                       nb_new, tail_slot, tail_mod, rc, (int)P, free_list, wb, cow, status, lr);
  return hipGetLastError();
}

}  // namespace smcsd
