// verify.hip - Score / Bonus / Reweight of an SMC-SD round, and the SpS verify, on gfx950.
//
// The verify step is a bandwidth-bound reduction over B*N*(2K+1) rows of V logits
// (SMC explainers, methodology: verification as fixed-size vectorised operations; the
// target scores all drafted positions in one batched pass and adds a bonus token).
// No MFMA: nothing here is a contraction.
//
// Kernels
//   k_lse_partials   grid = tiles, 256 threads: big tiles of at most 32768 entries for the
//                    non-bonus rows (a row's big tiles of equal size in the plain verify)
//                    and 32 KiB tiles for the bonus row (position K).  One streaming
//                    pass with 16-byte nontemporal loads; per lane an online (max, sum of
//                    2^(x*c - max*c)); a workgroup reduction; one (max, sum) pair per tile.
//                    Bonus tiles also write the sums of their 8 slabs (one slab = the 256
//                    vectors loaded together), reduced in two phases (the workgroup max,
//                    then DPP wave sums of the rescaled values), so the bonus draw re-reads
//                    one slab instead of a whole chunk.
//   k_smc_finalize   grid = sequences.  Combines the chunk pairs in fp64 into each row's
//                    normaliser, gathers the draft-token log-probabilities, draws the bonus
//                    token by inverse CDF (selects the slab from the slab sums of all the
//                    row's chunks in one scan, re-reads only that slab; the draw starts from
//                    the bonus row's own normaliser, not waiting for the other rows') and
//                    updates the log-weight.
//   race mode        the bonus row's tiles also run an exponential race (exponential-races
//                    summary page, key design) over their elements and keep the winner;
//                    the finalize takes the best of the tiles' winners and reads only the
//                    winner's logit: no slab sums and no re-read, for one Philox block per
//                    four vocabulary entries and two logarithms per entry.
//   k_sps_resid      SpS: acceptance tests from the gathered log-probabilities (in every
//                    workgroup, or from k_sps_decide for rows of many chunks), one pass over
//                    the residual max(0, p - q) (or p_K) of the single row pair that is
//                    needed with per-slab sums, and its inverse CDF by the sequence's last
//                    workgroup, which re-reads one slab.
#include <algorithm>
#include <climits>

#include "device.hpp"
#include "internal.hpp"

namespace smcsd {

struct RowMap {
  const char *tgt, *drf;
  int64_t row_bytes;  // bytes between consecutive rows
  int seq_step;
  int K;
  __device__ __forceinline__ const char *row(int g, int slot) const {
    const int64_t src = (int64_t)g * seq_step;
    if (slot <= K) return tgt + (src * (K + 1) + slot) * row_bytes;
    return drf + (src * K + (slot - K - 1)) * row_bytes;
  }
};

// One chunk pair (m, s) re-expressed relative to the row's Mc, in fp64.  -inf chunks add
// 0 (their s is 0, or NaN if the chunk held a NaN, which then propagates).
__device__ __forceinline__ double chunk_term(float2 p, float c, float Mc) {
  if (p.x == kNegInf) return (double)p.y * 0.0;
  return (double)p.y * (double)fast_exp2(__fmul_rn(p.x, c) - Mc);
}

// ---------------------------------------------------------------------------------
// Exponential race (bonus row in race mode)
// ---------------------------------------------------------------------------------
// Token v's clock: word v mod 4 of the Philox block with counter (g, step low, step high,
// kTagRace | (v div 4) << 8); u_v = (floor(w / 2^9) + 1/2) * 2^-23 is exact in fp32 and
// lies in (0, 1); E_v = -ln u_v.  The key x_v*c - log2(-log2 u_v) equals
// log2(e) * (z_v - ln E_v) less a constant shared by every v, so the largest key is the
// race's winner, argmin E_v / p_v.  Both logarithms see normal arguments only
// (u_v >= 2^-24, -log2 u_v >= 2^-24 * log2(e)).  Equal keys go to the smaller id; a -inf
// logit has key -inf and a NaN logit a NaN key, which never wins (the row's LSE reports
// the NaN).
constexpr uint32_t kTagRace = 6u;

struct RaceBest {
  float key;
  int idx;
};

__device__ __forceinline__ RaceBest race_init() { return RaceBest{kNegInf, INT_MAX}; }

// Merge of two candidates (largest key, then smallest id), branch-free.
__device__ __forceinline__ void race_take(RaceBest &b, float key, int idx) {
  const bool take = (key > b.key) | ((key == b.key) & (idx < b.idx));
  b.key = take ? key : b.key;
  b.idx = take ? idx : b.idx;
}

// A thread's own elements arrive in increasing id order: a strictly larger key wins and
// an equal key keeps the earlier (smaller) id.
__device__ __forceinline__ void race_next(RaceBest &b, float key, int idx) {
  const bool take = key > b.key;
  b.key = take ? key : b.key;
  b.idx = take ? idx : b.idx;
}

__device__ __forceinline__ float race_key(float x, float c, uint32_t w) {
  const float u = fmaf((float)(w >> 9), 0x1p-23f, 0x1p-24f);
  const float e2 = -__builtin_amdgcn_logf(u);
  return fmaf(x, c, -__builtin_amdgcn_logf(e2));
}

__device__ __forceinline__ void race_block(uint64_t seed, int g, uint64_t step, int v4,
                                           uint32_t w[4]) {
  w[0] = (uint32_t)g;
  w[1] = (uint32_t)step;
  w[2] = (uint32_t)(step >> 32);
  w[3] = kTagRace | ((uint32_t)v4 << 8);
  philox_block(w, (uint32_t)seed, (uint32_t)(seed >> 32));
}

// One element v on its own (head, tail, or a vector that does not start at a multiple of 4);
// every call of a thread has a larger v than its previous calls
__device__ __forceinline__ void race_one(RaceBest &b, float x, float c, uint64_t seed, int g,
                                         uint64_t step, int v) {
  uint32_t w[4];
  race_block(seed, g, step, v >> 2, w);
  const int j = v & 3;
  const uint32_t wj = j == 0 ? w[0] : j == 1 ? w[1] : j == 2 ? w[2] : w[3];
  race_next(b, race_key(x, c, wj), v);
}

// The elements of one 16-byte vector starting at v, a multiple of 4 (unpacked here from the
// raw vector: the raw form is half the registers of the widened one for bf16)
template <int DT>
__device__ __forceinline__ void race_vec(RaceBest &b, const uint4 &raw, float c, uint64_t seed, int g,
                                         uint64_t step, int v) {
  constexpr int NV = Elt<DT>::kPerVec;
  float x[NV];
  Elt<DT>::unpack(raw, x);
#pragma unroll
  for (int q = 0; q < NV / 4; ++q) {
    uint32_t w[4];
    race_block(seed, g, step, (v >> 2) + q, w);
#pragma unroll
    for (int j = 0; j < 4; ++j) race_next(b, race_key(x[4 * q + j], c, w[j]), v + 4 * q + j);
  }
}

// Workgroup argmax of (key, -idx); the result is valid in thread 0.
template <int BLOCK>
__device__ __forceinline__ RaceBest race_block_reduce(RaceBest b, RaceBest *lds) {
#pragma unroll
  for (int mask = 1; mask < kWave; mask <<= 1)
    race_take(b, __shfl_xor(b.key, mask, kWave), __shfl_xor(b.idx, mask, kWave));
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  if (lane == 0) lds[wave] = b;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < BLOCK / kWave; ++w) race_take(b, lds[w].key, lds[w].idx);
  }
  return b;
}

// ---------------------------------------------------------------------------------
// Streaming LSE pass
// ---------------------------------------------------------------------------------
// Elements of one slab: the kStreamBlock vectors a workgroup loads in one unrolled step.
template <int DT>
constexpr int kSlabElems = kStreamBlock * Elt<DT>::kPerVec;
static_assert(kChunkElemsBf16 == kSlabs * kSlabElems<SMCSD_DTYPE_BF16> &&
                  kChunkElemsF32 == kSlabs * kSlabElems<SMCSD_DTYPE_F32>,
              "a tile is one unrolled step: vector group u of every thread is slab u");

// Slab of element v of a tile whose vector body starts at a0 (head elements go to slab 0,
// tail elements to the slab their index falls in, capped at the last).
template <int DT>
__device__ __forceinline__ int slab_of(int64_t v, int64_t a0) {
  return v < a0 ? 0 : (int)min((int64_t)kSlabs - 1, (v - a0) / kSlabElems<DT>);
}

// Tiles: the rows other than the bonus row (nb_per_seq per sequence: the K target rows,
// then the K draft rows unless the draft's log q is given) in chunks_big big tiles each,
// of big_elems elements (the last takes the rest), and the bonus rows in chunks of
// chunk_elems (one unrolled step each), in the order described at the tile loop.  Tile indices below ntiles_big are big
// tiles, the rest bonus tiles.  Partials of row (g, slot) start at
// part[(g * R + slot) * chunks].
// RACE: the bonus tiles write the winner of their race to race[g * chunks + ch] as
// (key bits, id) instead of slab sums.
// Bonus tiles held back to the end of the LSE pass (inverse-CDF mode): about half of one
// full set of resident workgroups (5 per CU on 256 CUs); measured at C3 and C5 against
// 0, 160, 320, 1280 and 2560.
constexpr int kTailBonusTiles = 640;

template <int DT, bool RACE>
__global__ __launch_bounds__(kStreamBlock) void k_lse_partials(RowMap rm, int nseq, int V,
                                                                int chunk_elems, int chunks,
                                                                int chunks_big, int big_elems,
                                                                int nb_per_seq, float c,
                                                                float2 *__restrict__ part,
                                                                float *__restrict__ sub,
                                                                int64_t ntiles, uint64_t seed,
                                                                uint64_t step,
                                                                int2 *__restrict__ race,
                                                                int32_t *__restrict__ zero_seq) {
  using E = Elt<DT>;
  constexpr int EPV = E::kPerVec;
  __shared__ Lse lds[kStreamBlock / kWave];
  __shared__ RaceBest sRace[kStreamBlock / kWave];
  __shared__ RaceBest sRaceT[RACE ? kStreamBlock : 1];
  __shared__ float sRed[(kStreamBlock / kWave) * (2 + kSlabs)];
  __shared__ float sSlabT[kStreamBlock][kSlabs + 1];  // per-thread slab sums (bonus tiles)
  const int K = rm.K;
  const int R = 2 * K + 1;
  const int tid = threadIdx.x;
  const int64_t ntiles_big = ntiles - (int64_t)nseq * chunks;
  // Tile order: the bonus rows' one-step tiles spread evenly among the big tiles (tile t
  // is a bonus tile when floor(t * nB1 / n1) steps up at t), except the last M, which run
  // at the very end: small tiles even out the kernel's tail.  In race mode the bonus tiles
  // are ALU-heavy and none is held back, so all their arithmetic overlaps the streaming.
  const int64_t nB = ntiles - ntiles_big;
  const int64_t M = min(nB, (int64_t)(RACE ? 0 : kTailBonusTiles));
  const int64_t n1 = ntiles - M, nB1 = nB - M;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    // zero_seq (SpS: the draw's arrival counters) gets one zero per sequence (ntiles >= nseq)
    if (zero_seq && t < nseq && tid == 0) zero_seq[t] = 0;
    int64_t tt;
    bool isb;
    if (t < n1) {
      const int64_t kb = t * nB1 / n1, kb1 = (t + 1) * nB1 / n1;
      isb = kb1 > kb;
      tt = isb ? ntiles_big + kb : t - kb;
    } else {
      isb = true;
      tt = ntiles_big + nB1 + (t - n1);
    }
    int g, slot, ch;
    int64_t ce;
    if (isb) {
      const int64_t tb = tt - ntiles_big;
      g = (int)(tb / chunks);
      ch = (int)(tb - (int64_t)g * chunks);
      slot = K;
      ce = chunk_elems;
    } else {
      // nb_per_seq = 2K (target rows 0..K-1, then draft rows) or K (target rows only)
      const int64_t u = tt;
      const int64_t r = u / chunks_big;
      ch = (int)(u - r * chunks_big);
      g = (int)(r / nb_per_seq);
      const int j = (int)(r - (int64_t)g * nb_per_seq);
      slot = j < K ? j : j + 1;
      ce = big_elems;
    }
    const char *row = rm.row(g, slot);
    const int64_t e0 = (int64_t)ch * ce;
    const int64_t e1 = min((int64_t)V, e0 + ce);
    const uintptr_t addr0 = (uintptr_t)(row + e0 * E::kBytes);
    int64_t head = (int64_t)((16 - (addr0 & 15)) & 15) / E::kBytes;
    if (head > e1 - e0) head = e1 - e0;
    const int64_t a0 = e0 + head;
    const int64_t nvec = (e1 - a0) / EPV;
    const int64_t a1 = a0 + nvec * EPV;

    Lse st = lse_init();
    const bool bonus = slot == K;
    RaceBest rb = race_init();
    float xh = kNegInf, xt = kNegInf;
    if (tid < head) {
      xh = E::load(row, e0 + tid);
      const float x[1] = {xh};
      lse_update<1>(st, x, c);
      if (RACE && bonus) race_one(rb, xh, c, seed, g, step, (int)(e0 + tid));
    }
    if (tid < e1 - a1) {
      xt = E::load(row, a1 + tid);
      const float x[1] = {xt};
      lse_update<1>(st, x, c);
    }
    // body: kStreamUnroll 16-byte vectors per lane in flight, then one max / rescale for
    // the whole group of kStreamUnroll*EPV elements.  A bonus tile is one such group.
    if (!RACE && bonus) {
#pragma unroll
      for (int u = 0; u < kSlabs; ++u) sSlabT[tid][u] = 0.0f;
    }
    const uint4 *vp = reinterpret_cast<const uint4 *>(row + a0 * E::kBytes);
    constexpr int64_t kGroupVecs = (int64_t)kStreamBlock * kStreamUnroll;
    for (int64_t v0 = 0; v0 < nvec; v0 += kGroupVecs) {
      uint4 buf[kStreamUnroll];
      if (v0 + kGroupVecs <= nvec) {
        // a whole group: no per-load bounds test or -inf fill, and buffer loads whose
        // offsets (lane, then load) stay inside the group's kGroupVecs * 16 bytes
        const __amdgpu_buffer_rsrc_t rs = stream_rsrc(vp + v0, (int)(kGroupVecs * 16));
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) buf[u] = load_stream(rs, tid * 16, u * kStreamBlock * 16);
      } else {
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
          const int64_t v = v0 + u * kStreamBlock + tid;
          buf[u] = v < nvec ? load_stream(vp + v) : NegInfVec<DT>::get();
        }
      }
      if (RACE && bonus && (a0 & 3) == 0) {
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
          const int64_t v = v0 + u * kStreamBlock + tid;
          if (v < nvec) race_vec<DT>(rb, buf[u], c, seed, g, step, (int)(a0 + v * EPV));
        }
        sRaceT[tid] = rb;  // parked: no race registers held across the LSE update
      }

      float x[kStreamUnroll * EPV];
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) E::unpack(buf[u], x + u * EPV);
      float gs[kSlabs];
      lse_update_g<kStreamUnroll * EPV, EPV>(st, x, c, gs);
      // bonus tiles park this thread's slab sums in LDS (no registers held across the
      // workgroup reduction)
      if (!RACE && bonus) {
#pragma unroll
        for (int u = 0; u < kSlabs; ++u) sSlabT[tid][u] = gs[u];
      }
    }
    if (RACE && bonus && (a0 & 3) == 0 && nvec > 0) rb = sRaceT[tid];
    if (RACE && bonus && (a0 & 3) != 0) {
      // vectors that do not start at a multiple of 4 (a row start that is not 16-byte
      // aligned): the body's elements one at a time, read again
      for (int v = (int)a0 + tid; v < (int)a1; v += kStreamBlock) race_one(rb, E::load(row, v), c, seed, g, step, v);
    }
    // the tail last (a thread races its elements in increasing id order), read again
    // rather than held in a register across the body
    if (RACE && bonus && tid < e1 - a1) race_one(rb, E::load(row, a1 + tid), c, seed, g, step, (int)(a1 + tid));
    if (RACE && bonus) {
      st = lse_block_reduce<kStreamBlock>(st, c, lds);
      rb = race_block_reduce<kStreamBlock>(rb, sRace);
      if (tid == 0) {
        part[((int64_t)g * R + slot) * chunks + ch] = make_float2(st.m, st.s);
        race[(int64_t)g * chunks + ch] = make_int2(__float_as_int(rb.key), rb.idx);
      }
    } else if (!bonus) {
      st = lse_block_reduce<kStreamBlock>(st, c, lds);
      if (tid == 0) part[((int64_t)g * R + slot) * chunks + ch] = make_float2(st.m, st.s);
    } else {
      // slab sums relative to this thread's m*c (its head and tail elements included),
      // carried through the same workgroup reduction as s
      float slab[kSlabs];
#pragma unroll
      for (int u = 0; u < kSlabs; ++u) slab[u] = sSlabT[tid][u];
      if (tid < head) slab[0] += fast_exp2(fmaf(xh, c, -st.mc));
      if (tid < e1 - a1) {
        const float t = fast_exp2(fmaf(xt, c, -st.mc));
        const int ts = slab_of<DT>(a1 + tid, a0);
#pragma unroll
        for (int u = 0; u < kSlabs; ++u)
          if (u == ts) slab[u] += t;
      }
      st = lse_block_reduce_sums<kStreamBlock, kSlabs>(st, slab, c, sRed);
      if (tid == 0) {
        part[((int64_t)g * R + slot) * chunks + ch] = make_float2(st.m, st.s);
        float *o = sub + ((int64_t)g * chunks + ch) * kSlabs;
#pragma unroll
        for (int u = 0; u < kSlabs; ++u) o[u] = slab[u];
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------
// Row normalisers from the chunk pairs (thread r handles row slot r).
// L2 = log2 of sum_v 2^(x_v * c) = Mc + log2(S).
// ---------------------------------------------------------------------------------
struct RowNorm {
  float Mc;
  double S, L2;
  int flags;
};

// p points to LDS or to global memory; a caller passes a pointer of one known kind (not a
// select between the two), so the loads are LDS or global loads, not flat ones, and the
// unrolled loops keep several in flight.
// The row's reference Mc (its max times c) and S = sum of its chunk terms; returns the max.
__device__ __forceinline__ float row_mc_s(const float2 *p, int chunks, float c, float &Mc,
                                          double &S) {
  float M = kNegInf;
#pragma unroll 8
  for (int i = 0; i < chunks; ++i) M = fmaxf(M, p[i].x);
  Mc = M == kNegInf ? 0.0f : __fmul_rn(M, c);
  S = 0.0;
#pragma unroll 8
  for (int i = 0; i < chunks; ++i) S += chunk_term(p[i], c, Mc);
  return M;
}

__device__ __forceinline__ RowNorm row_norm(const float2 *p, int chunks, float c) {
  RowNorm r{};
  const float M = row_mc_s(p, chunks, c, r.Mc, r.S);
  r.L2 = (double)r.Mc + log2(r.S);
  r.flags = 0;
  if (isnan(r.S) || isinf(r.S)) r.flags |= SMCSD_ST_NAN_INPUT;
  else if (M == kNegInf) r.flags |= SMCSD_ST_EMPTY_ROW;
  return r;
}

// Inverse CDF inside one range [e0, e1) of a row (a chunk or a slab): the first v whose running sum
// base + sum_{w<=v} val(w) exceeds target.  The chunk is cut into units of 8 consecutive
// elements; thread t loads units [t*UPT, (t+1)*UPT) once and keeps them in registers.
// Unit sums are fp32 (fn.reduce), running sums fp64.  One workgroup exclusive scan finds
// the owning thread, which walks its own units element by element (fn.val_from_raw, the
// same fp32 values the unit sums used).  Rounding can leave no crossing where the oracle's
// margin is at rounding level; then the last element with a positive value before the
// crossing point is returned.  Every thread must call it; every thread gets the index
// (-1 if there is none) and *logit the pick's logit (fn.logit).  UPT * 8 * BLOCK must
// cover the range.
// Workgroup size of the SMC finalize, one workgroup per sequence (hundreds at a time).
constexpr int kSmcFinalBlock = 256;

// 8-element units per thread when a BLOCK-thread workgroup re-reads one chunk
template <int DT, int BLOCK>
constexpr int kUnitsPerThread = (DT == SMCSD_DTYPE_BF16 ? kChunkElemsBf16 : kChunkElemsF32) / 8 /
                                BLOCK;
static_assert(kChunkElemsF32 % (8 * kSmcFinalBlock) == 0,
              "a chunk must split evenly into the workgroup's units");

template <int BLOCK, int UPT, typename Fn>
__device__ __forceinline__ int chunk_inverse_cdf(int64_t e0, int64_t e1, double base,
                                                 double target, const Fn &fn, double *scan_lds,
                                                 int *misc, float *logit) {
  const int tid = threadIdx.x;
  const int nunits = (int)((e1 - e0 + 7) / 8);
  typename Fn::Raw raw[UPT];
  float us[UPT];
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = min(tid * UPT + i, nunits - 1);  // clamped: every load is in bounds
    const int64_t a = e0 + 8 * (int64_t)u;
    fn.load(a, min(e1, a + 8), raw[i]);
  }
  if (tid == 0) {
    misc[0] = INT_MAX;  // owner thread
    misc[1] = -1;       // last unit with a positive sum
    misc[2] = -1;       // result
  }
  double loc = 0.0;
  int lastu = -1;
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = tid * UPT + i;
    us[i] = u < nunits ? fn.reduce(raw[i]) : 0.0f;
    loc += (double)us[i];
    if (us[i] > 0.0f) lastu = u;
  }
  double tot;
  const double start = base + block_exclusive_scan<double, BLOCK>(loc, scan_lds, &tot);
  // one LDS atomic per wave: the first crossing lane, the wave's last positive unit
  const int lane = tid % kWave;
  const unsigned long long cross = __ballot(tid * UPT < nunits && start + loc > target);
  int lu = lastu;
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) lu = max(lu, __shfl_xor(lu, m, kWave));
  if (lane == 0) {
    if (cross) atomicMin(&misc[0], tid + __ffsll(cross) - 1);
    if (lu >= 0) atomicMax(&misc[1], lu);
  }
  __syncthreads();
  const int owner = misc[0], last_all = misc[1];
  const int who = owner != INT_MAX ? owner : (last_all >= 0 ? last_all / UPT : -1);
  if (tid == who) {
    int pick_i = -1, pick_j = -1;
    if (owner != INT_MAX) {
      double run = start;
      int lastpos_i = -1, lastpos_j = -1;  // last positive element inside the crossing unit
      int lastu_i = -1;                     // last own unit with a positive sum before it
      bool crossed = false;
#pragma unroll
      for (int i = 0; i < UPT; ++i) {
        if (crossed || tid * UPT + i >= nunits) continue;
        if (run + (double)us[i] > target) {
          crossed = true;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if (pick_i >= 0) continue;
            const float y = fn.val_from_raw(raw[i], j);
            if (y > 0.0f) {
              lastpos_i = i;
              lastpos_j = j;
            }
            run += (double)y;
            if (run > target) {
              pick_i = i;
              pick_j = j;
            }
          }
        } else {
          run += (double)us[i];
          if (us[i] > 0.0f) lastu_i = i;
        }
      }
      if (pick_i < 0 && lastpos_i >= 0) {
        pick_i = lastpos_i;
        pick_j = lastpos_j;
      }
      if (pick_i < 0 && lastu_i >= 0) pick_i = lastu_i;
    } else {
      pick_i = last_all - tid * UPT;
    }
    if (pick_i >= 0 && pick_j < 0) {
      // last positive element of unit pick_i
#pragma unroll
      for (int i = 0; i < UPT; ++i)
        if (i == pick_i)
#pragma unroll
          for (int j = 7; j >= 0; --j)
            if (pick_j < 0 && fn.val_from_raw(raw[i], j) > 0.0f) pick_j = j;
    }
    if (pick_i >= 0 && pick_j >= 0) {
      float x = 0.0f;
#pragma unroll
      for (int i = 0; i < UPT; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (i == pick_i && j == pick_j) x = fn.logit(raw[i], j);
      misc[2] = (int)(e0 + 8 * (int64_t)(tid * UPT + pick_i) + pick_j);
      *logit = x;
    }
  }
  __syncthreads();
  const int res = misc[2];
  __syncthreads();
  return res;
}

// Bonus-row element value 2^(x*c - Mc) over 8-element units.  The unit load is eight
// unrolled scalar loads at clamped in-bounds indices: branch-free, any row alignment.
template <int DT>
struct ExpRow {
  const char *row;
  float c, Mc;
  bool vec;  // the row starts 16-byte aligned: whole units are read as 16-byte vectors
  struct Raw {
    float x[8];
  };
  __device__ __forceinline__ void load(int64_t a, int64_t b, Raw &r) const {
    using E = Elt<DT>;
    if (vec && a + 8 <= b) {
      const uint4 *p = reinterpret_cast<const uint4 *>(row + a * E::kBytes);
#pragma unroll
      for (int q = 0; q < 8 / E::kPerVec; ++q) E::unpack(p[q], r.x + q * E::kPerVec);
      return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = E::load(row, min(a + i, b - 1));
      r.x[i] = a + i < b ? x : kNegInf;
    }
  }
  __device__ __forceinline__ float val_from_raw(const Raw &r, int i) const {
    return fast_exp2(fmaf(r.x[i], c, -Mc));
  }
  __device__ __forceinline__ float logit(const Raw &r, int i) const { return r.x[i]; }
  __device__ __forceinline__ float reduce(const Raw &r) const {
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = val_from_raw(r, i);
    return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
  }
};

// ---------------------------------------------------------------------------------
// SMC finalize: one workgroup per sequence
// ---------------------------------------------------------------------------------
constexpr int kMaxPartLds = 1024;  // chunk pairs of one sequence staged in LDS (else read in place)
constexpr int kMaxSubLds = 1024;   // bonus slab sums of one sequence staged in LDS
// units per thread for the finalize's one-slab re-read: a slab plus a head or tail of
// fewer than 8 elements each
constexpr int kSmcUnits = 2;
static_assert(kSlabElems<SMCSD_DTYPE_BF16> + 16 <= 8 * kSmcFinalBlock * kSmcUnits &&
                  kSlabElems<SMCSD_DTYPE_F32> + 16 <= 8 * kSmcFinalBlock * kSmcUnits,
              "the finalize workgroup must cover one slab");

template <int DT, bool RACE, bool STRIDE>
__global__ __launch_bounds__(kSmcFinalBlock) void k_smc_finalize(
    RowMap rm, int nseq, const int32_t *__restrict__ draft_tokens, int V, int chunk_elems, int chunks,
    int chunks_big, float c, float alpha, uint64_t seed, uint64_t step, uint32_t bonus_tag,
    const float2 *__restrict__ part, const float *__restrict__ logq_in,
    const float *__restrict__ sub, const int2 *__restrict__ race, float *__restrict__ lw,
    int32_t *__restrict__ out_tokens,
    int32_t *__restrict__ out_num,
    float *__restrict__ out_logp, float *__restrict__ out_logq, float *__restrict__ out_lse,
    int32_t *status) {
  using E = Elt<DT>;
  const int K = rm.K, R = 2 * K + 1;
  const int tid = threadIdx.x;
  __shared__ double sL2[2 * kMaxK + 1];
  __shared__ double sLogp[kMaxK + 1], sLogq[kMaxK + 1];
  __shared__ int32_t sTok[kMaxK + 1];
  __shared__ float2 sPart[kMaxPartLds];
  __shared__ float sSub[kMaxSubLds];
  __shared__ double sScan[kSmcFinalBlock / kWave];
  __shared__ int sMisc[4];
  __shared__ int64_t sLo, sHi;
  __shared__ double sBase;
  __shared__ float sPickLogit;
  __shared__ int sFlags;
  // one sequence per workgroup; a grid smaller than the batch strides over it
  for (int g = blockIdx.x; g < nseq; g += gridDim.x) {
  if (tid == 0) sFlags = 0;
  const float lw_old = tid == 0 && lw ? lw[g] : 0.0f;  // loaded early: used only at the end

  // One round of loads, all issued before any is used: the draft tokens (and a given log
  // q), this sequence's chunk pairs and slab sums into registers, the draft-token logits
  // as soon as the tokens are in, then the LDS staging.  The token and logit loads are
  // made by every lane at clamped, valid addresses (no divergent branch around a load, so
  // each use waits for its own load only); the register staging has uniform bounds.
  constexpr int kPartPer = kMaxPartLds / kSmcFinalBlock;
  constexpr int kSubPer = kMaxSubLds / kSmcFinalBlock;
  const int64_t src = (int64_t)g * rm.seq_step;
  const bool tok_lane = tid < 2 * K;
  const int kk = tok_lane ? (tid < K ? tid : tid - K) : 0;
  const int slot = tid < K ? kk : K + 1 + kk;
  int32_t x = 0;
  float lq_given = 0.0f;
  if (K > 0) {
    x = draft_tokens[src * K + kk];
    if (logq_in) lq_given = logq_in[src * K + kk];
  }
  const int npart = R * chunks;
  const bool part_in_lds = npart <= kMaxPartLds;
  const float2 *gpart = part + (int64_t)g * npart;
  float2 pr[kPartPer];
  if (part_in_lds) {
#pragma unroll
    for (int j = 0; j < kPartPer; ++j)
      if (j * kSmcFinalBlock < npart) pr[j] = gpart[min(tid + j * kSmcFinalBlock, npart - 1)];
  }
  const int nsub = chunks * kSlabs;
  const bool sub_in_lds = nsub <= kMaxSubLds;
  const float *gsub = sub + (int64_t)g * nsub;
  float sr[kSubPer];
  if (!RACE && sub_in_lds) {
#pragma unroll
    for (int j = 0; j < kSubPer; ++j)
      if (j * kSmcFinalBlock < nsub) sr[j] = gsub[min(tid + j * kSmcFinalBlock, nsub - 1)];
  }
  const bool xv_lane = tid < (logq_in ? K : 2 * K) && x >= 0 && x < V;
  const float xv_raw = E::load(rm.row(g, xv_lane ? slot : 0), xv_lane ? x : 0);
  if (part_in_lds) {
#pragma unroll
    for (int j = 0; j < kPartPer; ++j)
      if (tid + j * kSmcFinalBlock < npart) sPart[tid + j * kSmcFinalBlock] = pr[j];
  }
  if (!RACE && sub_in_lds) {
#pragma unroll
    for (int j = 0; j < kSubPer; ++j)
      if (tid + j * kSmcFinalBlock < nsub) sSub[tid + j * kSmcFinalBlock] = sr[j];
  }
  __syncthreads();
  const float xv = xv_lane ? xv_raw : 0.0f;

  // The bonus draw needs only the bonus row's Mc_K and S_K: every wave forms them itself
  // (the same loop, so the same bits; a wave's instructions cost the same whatever its
  // active lanes), so they are uniform with no barrier, and wave 0 goes straight on to the
  // slab pick while waves 1 and 2 combine every row's chunk pairs in fp64, log2 included
  // (the draft rows only when their log q is not given), for the log-probabilities.
  float McK;
  double SK;
  if (part_in_lds) row_mc_s(sPart + K * chunks, chunks, c, McK, SK);
  else row_mc_s(gpart + K * chunks, chunks, c, McK, SK);
  if (tid >= kWave && tid < kWave + (logq_in ? K + 1 : R)) {
    const int r = tid - kWave;
    const int n = r == K ? chunks : chunks_big;
    const RowNorm rn = part_in_lds ? row_norm(sPart + r * chunks, n, c)
                                   : row_norm(gpart + r * chunks, n, c);
    sL2[r] = rn.L2;
    if (rn.flags) atomicOr(&sFlags, rn.flags);
  }

  // Bonus: u = U(seed; g, step, BONUS); first v whose running sum of 2^(x*c - Mc_K)
  // exceeds u * S_K (the unnormalised CDF; the common factor 2^Mc_K cancels).
  const double u = philox_uniform(seed, (uint32_t)g, step, bonus_tag, 0);
  const double target = u * SK;
  const char *brow = rm.row(g, K);
  int bonus = -1;
  float race_logit = 0.0f;
  if (RACE) {
    // race mode: the best of the tiles' winners (largest key, then smallest id); only
    // thread 0 uses the result
    if (isfinite(SK) && SK > 0.0 && tid < kWave) {
      RaceBest b = race_init();
      for (int i = tid; i < chunks; i += kWave) {
        const int2 r = race[(int64_t)g * chunks + i];
        race_take(b, __int_as_float(r.x), r.y);
      }
#pragma unroll
      for (int mask = 1; mask < kWave; mask <<= 1)
        race_take(b, __shfl_xor(b.key, mask, kWave), __shfl_xor(b.idx, mask, kWave));
      if (tid == 0 && b.key > kNegInf && b.idx >= 0 && b.idx < V) {
        bonus = b.idx;
        race_logit = E::load(brow, b.idx);
      }
    }
  } else if (isfinite(SK) && SK > 0.0) {
    if (tid < kWave) {
      // wave 0: the slab whose running sum first exceeds the target, over all slabs of the
      // row in order (chunk-major), by lane prefix sums and a ballot per 64 slabs; a slab's
      // term is its sum rescaled from its chunk's reference to the row's.  If rounding
      // leaves no crossing, the last slab with a positive term.
      const int lane = tid;
      const int nsl = chunks * kSlabs;
      double base = 0.0, base_last = 0.0;
      int sel = -1, last = -1;
      // sb / pk both in LDS or both in global memory (never a select between the two)
      auto scan = [&](const float *sb, const float2 *pk) {
        for (int j0 = 0; j0 < nsl && sel < 0; j0 += kWave) {
          const int j = j0 + lane;
          double t = 0.0;
          if (j < nsl) {
            const float2 p = pk[j / kSlabs];
            if (p.x != kNegInf) t = (double)sb[j] * (double)fast_exp2(__fmul_rn(p.x, c) - McK);
          }
          const double inc = wave_inclusive_scan(t);
          const unsigned long long hit = __ballot(j < nsl && base + inc > target);
          const unsigned long long pos = __ballot(j < nsl && t > 0.0);
          if (pos) {
            const int f = 63 - __clzll(pos);
            last = j0 + f;
            base_last = base + __shfl(inc - t, f, kWave);
          }
          if (hit) {
            const int f = __ffsll(hit) - 1;
            sel = j0 + f;
            base += __shfl(inc - t, f, kWave);
          } else {
            base += __shfl(inc, kWave - 1, kWave);
          }
        }
      };
      if (part_in_lds && sub_in_lds) scan(sSub, sPart + K * chunks);
      else scan(gsub, gpart + K * chunks);
      if (sel < 0) {
        sel = last >= 0 ? last : nsl - 1;
        base = last >= 0 ? base_last : base;
      }
      const int ch = sel / kSlabs, sl = sel - ch * kSlabs;
      // slab bounds: the vector body starts at the first 16-byte aligned element
      const int64_t e0 = (int64_t)ch * chunk_elems;
      const int64_t e1 = min((int64_t)V, e0 + (int64_t)chunk_elems);
      const uintptr_t addr0 = reinterpret_cast<uintptr_t>(brow + e0 * E::kBytes);
      const int64_t a0 = e0 + min((int64_t)(((16 - (addr0 & 15)) & 15) / E::kBytes), e1 - e0);
      if (lane == 0) {
        sLo = sl == 0 ? e0 : min(e1, a0 + (int64_t)sl * kSlabElems<DT>);
        sHi = sl == kSlabs - 1 ? e1 : min(e1, a0 + (int64_t)(sl + 1) * kSlabElems<DT>);
        sBase = base;
      }
    }
    __syncthreads();
    const int64_t lo = sLo, hi = sHi;
    if (hi > lo) {
      const ExpRow<DT> fn{brow, c, McK,
                          (reinterpret_cast<uintptr_t>(brow + lo * E::kBytes) & 15) == 0};
      bonus = chunk_inverse_cdf<kSmcFinalBlock, kSmcUnits>(lo, hi, sBase, target, fn, sScan, sMisc,
                                                           &sPickLogit);
    }
  }

  __syncthreads();  // every row's normaliser is in
  if (tid < 2 * K) {
    const int k = tid < K ? tid : tid - K;
    double lp = __builtin_nan("");
    if (x < 0 || x >= V) atomicOr(&sFlags, SMCSD_ST_BAD_INPUT);
    else if (logq_in && tid >= K) lp = (double)lq_given;
    else lp = ((double)xv * (double)c - sL2[slot]) * kLn2;
    if (tid < K) {
      sLogp[k] = lp;
      sTok[k] = x;
    } else {
      sLogq[k] = lp;
    }
  }

  double lpK = __builtin_nan("");
  if (bonus >= 0) lpK = ((double)(RACE ? race_logit : sPickLogit) * (double)c - sL2[K]) * kLn2;
  int32_t *tok = out_tokens + (int64_t)g * (K + 1);
  if (tid < K) {
    tok[tid] = sTok[tid];
    if (out_logp) out_logp[(int64_t)g * (K + 1) + tid] = (float)sLogp[tid];
    if (out_logq) out_logq[(int64_t)g * K + tid] = (float)sLogq[tid];
  }
  if (out_lse && tid < R)
    out_lse[(int64_t)g * R + tid] = logq_in && tid > K ? __builtin_nanf("") : (float)(sL2[tid] * kLn2);
  if (tid == 0) {
    double incr = 0.0;
    for (int k = 0; k < K; ++k) incr += (double)alpha * sLogp[k] - sLogq[k];
    incr += ((double)alpha - 1.0) * lpK;
    if (lw) lw[g] = (float)((double)lw_old + incr);
    tok[K] = bonus;
    if (out_num) out_num[g] = K + 1;
    if (out_logp) out_logp[(int64_t)g * (K + 1) + K] = (float)lpK;
    if (sFlags) atomicOr(status, sFlags);
  }
  if (!STRIDE) break;  // the grid covers the batch: one sequence, no loop kept
  __syncthreads();      // the next sequence reuses the LDS
  }
}

// ---------------------------------------------------------------------------------
// SpS
// ---------------------------------------------------------------------------------
// Per row: the element probability is 2^(x*c - Mc) * inv (inv = 1/S); from lse_in the
// pair is (LSE*log2(e), 1).  ws_norm[g] = {Mc_p, inv_p, Mc_q, inv_q} for row pair k*.
template <int DT, bool STRIDE>
__global__ __launch_bounds__(kWave) void k_sps_decide(
    RowMap rm, int nseq, const int32_t *__restrict__ draft_tokens, int V, int chunks, int chunks_big, float c,
    uint64_t seed, uint64_t step, const float2 *__restrict__ part, const float *__restrict__ lse_in,
    int32_t *__restrict__ ws_kstar, float4 *__restrict__ ws_norm, int32_t *__restrict__ out_tokens,
    int32_t *__restrict__ out_num, float *__restrict__ out_logp, float *__restrict__ out_logq,
    float *__restrict__ out_lse, int32_t *status) {
  using E = Elt<DT>;
  const int K = rm.K, R = 2 * K + 1;
  const int tid = threadIdx.x;
  __shared__ double sL2[2 * kMaxK + 1], sS[2 * kMaxK + 1];
  __shared__ float sMc[2 * kMaxK + 1];
  __shared__ double sLogp[kMaxK + 1], sLogq[kMaxK + 1];
  __shared__ int32_t sTok[kMaxK + 1];
  __shared__ int sFlags;
  for (int g = blockIdx.x; g < nseq; g += gridDim.x) {
  const int64_t src = (int64_t)g * rm.seq_step;
  if (tid == 0) sFlags = 0;
  __syncthreads();
  for (int r = tid; r < R; r += kWave) {
    if (lse_in) {
      const double L2 = (double)lse_in[src * R + r] * kLog2e;
      sL2[r] = L2;
      sS[r] = 1.0;
      sMc[r] = (float)L2;
      if (isnan(L2) || L2 == __builtin_inf()) atomicOr(&sFlags, SMCSD_ST_NAN_INPUT);
      else if (L2 == -__builtin_inf()) atomicOr(&sFlags, SMCSD_ST_EMPTY_ROW);
    } else {
      const RowNorm rn = row_norm(part + ((int64_t)g * R + r) * chunks, r == K ? chunks : chunks_big, c);
      sL2[r] = rn.L2;
      sS[r] = rn.S;
      sMc[r] = rn.Mc;
      if (rn.flags) atomicOr(&sFlags, rn.flags);
    }
  }
  __syncthreads();
  for (int j = tid; j < 2 * K; j += kWave) {
    const int k = j < K ? j : j - K;
    const int slot = j < K ? k : K + 1 + k;
    const int32_t x = draft_tokens[src * K + k];
    double lp = __builtin_nan("");
    if (x < 0 || x >= V) atomicOr(&sFlags, SMCSD_ST_BAD_INPUT);
    else lp = ((double)E::load(rm.row(g, slot), x) * (double)c - sL2[slot]) * kLn2;
    if (j < K) {
      sLogp[k] = lp;
      sTok[k] = x;
    } else {
      sLogq[k] = lp;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int kstar = K;
    for (int k = 0; k < K; ++k) {
      const double ratio = exp(sLogp[k] - sLogq[k]);
      const double r = philox_uniform(seed, (uint32_t)g, step, 3u | ((uint32_t)(k / 4) << 8), k % 4);
      if (!(r < ratio)) {
        kstar = k;
        break;
      }
    }
    ws_kstar[g] = kstar;
    const int qs = K + 1 + kstar;
    ws_norm[g] = make_float4(sMc[kstar], (float)(1.0 / sS[kstar]), kstar < K ? sMc[qs] : 0.0f,
                             kstar < K ? (float)(1.0 / sS[qs]) : 0.0f);
    int32_t *tok = out_tokens + (int64_t)g * (K + 1);
    for (int k = 0; k <= K; ++k) tok[k] = k < kstar ? sTok[k] : -1;
    if (out_num) out_num[g] = kstar + 1;
    if (out_logp)
      for (int k = 0; k < K; ++k) out_logp[(int64_t)g * (K + 1) + k] = (float)sLogp[k];
    if (out_logq)
      for (int k = 0; k < K; ++k) out_logq[(int64_t)g * K + k] = (float)sLogq[k];
    if (out_lse)
      for (int r = 0; r < R; ++r) out_lse[(int64_t)g * R + r] = (float)(sL2[r] * kLn2);
    if (sFlags) atomicOr(status, sFlags);
  }
  if (!STRIDE) break;
  __syncthreads();  // the next sequence reuses the LDS
  }
}

// Residual (or target) row values for the SpS draw: the same fp32 expression in the
// residual pass and in the re-read, so a slab's re-read values are the ones it summed.
template <int DT>
struct ResidRow {
  const char *prow, *qrow;
  float c, Mcp, invp, Mcq, invq;
  bool use_rho;
  bool vec;  // both rows start 16-byte aligned: whole units are read as 16-byte vectors
  struct Raw {
    float p[8], q[8];
  };
  __device__ __forceinline__ float pval(float xp) const {
    return fast_exp2(fmaf(xp, c, -Mcp)) * invp;
  }
  __device__ __forceinline__ float rho(float p, float xq) const {
    return fmaxf(p - fast_exp2(fmaf(xq, c, -Mcq)) * invq, 0.0f);
  }
  __device__ __forceinline__ float val_from(float xp, float xq) const {
    const float p = pval(xp);
    return use_rho ? rho(p, xq) : p;
  }
  __device__ __forceinline__ void load(int64_t a, int64_t b, Raw &r) const {
    using E = Elt<DT>;
    if (vec && a + 8 <= b) {
      const uint4 *pp = reinterpret_cast<const uint4 *>(prow + a * E::kBytes);
      const uint4 *pq = reinterpret_cast<const uint4 *>((use_rho ? qrow : prow) + a * E::kBytes);
#pragma unroll
      for (int k = 0; k < 8 / E::kPerVec; ++k) {
        E::unpack(pp[k], r.p + k * E::kPerVec);
        if (use_rho) E::unpack(pq[k], r.q + k * E::kPerVec);
      }
      if (!use_rho)
#pragma unroll
        for (int i = 0; i < 8; ++i) r.q[i] = 0.0f;
      return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t v = min(a + i, b - 1);
      const float xp = E::load(prow, v);
      r.p[i] = a + i < b ? xp : kNegInf;
      r.q[i] = use_rho ? E::load(qrow, v) : 0.0f;
    }
  }
  __device__ __forceinline__ float val_from_raw(const Raw &r, int i) const {
    return val_from(r.p[i], r.q[i]);
  }
  __device__ __forceinline__ float logit(const Raw &r, int i) const { return r.p[i]; }
  __device__ __forceinline__ float reduce(const Raw &r) const {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += val_from(r.p[i], r.q[i]);
    return s;
  }
};

// SpS after the LSE pass: k_sps_resid, one workgroup of kStreamBlock threads per
// (sequence, vocabulary chunk).
//   * the decision.  FUSED (rows of at most kSpsFusedChunksMax chunk pairs): every
//     workgroup forms it from the chunk pairs - the row normalisers (wave 0), the draft
//     tokens' logits (wave 1), then one lane per draft position tests r_k < p/q and a
//     ballot gives the first rejection k* (K when all pass); the chunk-0 workgroup writes
//     the per-sequence outputs.  Otherwise k_sps_decide has written k* and the norms.
//   * the residual pass over this chunk of row pair k* (the target row alone when k* = K):
//     wave w sums slab w, a contiguous quarter of the chunk, of max(0, p - q) and of p.
//   * the last workgroup of the sequence to finish (an arrival counter per sequence, which
//     the LSE pass zeroes) draws the token: the slab where the running sum of the slab
//     sums crosses u * total, then one re-read of that slab and its inverse CDF.  The slab
//     sums travel as agent-scope atomic stores and loads, ordered by waiting for the
//     stores before the counter increment: device-scope fences instead (an L2 write-back
//     in every workgroup and an invalidate in the last) made the kernel 3x slower on the
//     MI355X (16 sequences, V = 128256 fp32: 49.7 us against 15.3 us), and a separate draw
//     kernel cost one more launch (11.5 + 4.8 us of kernels, 10 us more per call).
constexpr int kSpsSlabs = kStreamBlock / kWave;
template <int DT>
constexpr int kSpsSlabElems =
    (DT == SMCSD_DTYPE_BF16 ? kChunkElemsBf16 : kChunkElemsF32) / kSpsSlabs;
template <int DT>
constexpr int kSpsVecsPerLane = kSpsSlabElems<DT> / Elt<DT>::kPerVec / kWave;
static_assert(kSpsSlabs == kSpsSlabsWs, "the workspace holds one slab sum pair per wave");
static_assert(kSpsVecsPerLane<SMCSD_DTYPE_F32> * Elt<SMCSD_DTYPE_F32>::kPerVec * kWave ==
                      kSpsSlabElems<SMCSD_DTYPE_F32> &&
                  kSpsVecsPerLane<SMCSD_DTYPE_BF16> * Elt<SMCSD_DTYPE_BF16>::kPerVec * kWave ==
                      kSpsSlabElems<SMCSD_DTYPE_BF16>,
              "a slab is whole vectors of every lane of one wave");
static_assert(kSpsSlabElems<SMCSD_DTYPE_F32> % (8 * kStreamBlock) == 0 &&
                  kSpsSlabElems<SMCSD_DTYPE_BF16> % (8 * kStreamBlock) == 0,
              "a slab splits evenly into the re-read's units");

__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) v |= __shfl_xor(v, m, kWave);
  return v;
}

// Elements [a, a + kPerVec) of a row as one 16-byte word (bf16: element 2i in the low half
// of word i); with the row unaligned or the vector crossing b, element loads at indices
// clamped to b - 1 (those at or beyond b are then garbage the caller masks).
template <int DT>
__device__ __forceinline__ uint4 load_vec_any(const char *row, int64_t a, int64_t b, bool vec) {
  using E = Elt<DT>;
  if (vec && a + E::kPerVec <= b) return *reinterpret_cast<const uint4 *>(row + a * E::kBytes);
  uint32_t w[4];
  if (DT == SMCSD_DTYPE_F32) {
    const uint32_t *r = reinterpret_cast<const uint32_t *>(row);
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = r[min(a + i, b - 1)];
  } else {
    const uint16_t *r = reinterpret_cast<const uint16_t *>(row);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)r[min(a + 2 * i, b - 1)] | ((uint32_t)r[min(a + 2 * i + 1, b - 1)] << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

struct SpsDecision {
  double L2[2 * kMaxK + 1], S[2 * kMaxK + 1];
  float Mc[2 * kMaxK + 1];
  double lp[kMaxK], lq[kMaxK];
  float x[2 * kMaxK];  // the draft tokens' logits: target rows, then draft rows
  int32_t tok[kMaxK];
  int fl[2];
  float4 nm;
  int kstar, flags;
};

constexpr int kSpsFusedChunksMax = 32;

// The SpS decision of sequence g into D (every thread calls it; ends with a barrier).
template <int DT>
__device__ __forceinline__ void sps_decide(const RowMap &rm, int g, const int32_t *__restrict__ draft_tokens,
                                           int V, int chunks, int chunks_big, float c, uint64_t seed,
                                           uint64_t step, const float2 *__restrict__ part,
                                           const float *__restrict__ lse_in, SpsDecision &D) {
  const int K = rm.K, R = 2 * K + 1;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int64_t src = (int64_t)g * rm.seq_step;
  if (tid < kWave) {
    int fl = 0;
    for (int r = lane; r < R; r += kWave) {
      if (lse_in) {
        const double L2 = (double)lse_in[src * R + r] * kLog2e;
        D.L2[r] = L2;
        D.S[r] = 1.0;
        D.Mc[r] = (float)L2;
        if (isnan(L2) || L2 == __builtin_inf()) fl |= SMCSD_ST_NAN_INPUT;
        else if (L2 == -__builtin_inf()) fl |= SMCSD_ST_EMPTY_ROW;
      } else {
        const RowNorm rn = row_norm(part + ((int64_t)g * R + r) * chunks, r == K ? chunks : chunks_big, c);
        D.L2[r] = rn.L2;
        D.S[r] = rn.S;
        D.Mc[r] = rn.Mc;
        fl |= rn.flags;
      }
    }
    fl = wave_or(fl);
    if (lane == 0) D.fl[0] = fl;
  } else if (tid < 2 * kWave) {
    int fl = 0;
    if (lane < 2 * K) {
      const int k = lane < K ? lane : lane - K;
      const int slot = lane < K ? k : K + 1 + k;
      const int32_t x = draft_tokens[src * K + k];
      float xv = __builtin_nanf("");
      if (x < 0 || x >= V) fl = SMCSD_ST_BAD_INPUT;
      else xv = Elt<DT>::load(rm.row(g, slot), x);
      D.x[lane] = xv;
      if (lane < K) D.tok[k] = x;
    }
    fl = wave_or(fl);
    if (lane == 0) D.fl[1] = fl;
  }
  __syncthreads();
  if (tid < kWave) {
    bool rej = false;
    if (lane < K) {
      const double lp = ((double)D.x[lane] * (double)c - D.L2[lane]) * kLn2;
      const double lq = ((double)D.x[K + lane] * (double)c - D.L2[K + 1 + lane]) * kLn2;
      D.lp[lane] = lp;
      D.lq[lane] = lq;
      const double ratio = exp(lp - lq);
      const double r = philox_uniform(seed, (uint32_t)g, step, 3u | ((uint32_t)(lane / 4) << 8), lane % 4);
      rej = !(r < ratio);
    }
    const unsigned long long m = __ballot(rej);
    if (lane == 0) {
      const int kstar = m ? __ffsll(m) - 1 : K;
      const int qs = K + 1 + kstar;
      D.kstar = kstar;
      D.nm = make_float4(D.Mc[kstar], (float)(1.0 / D.S[kstar]), kstar < K ? D.Mc[qs] : 0.0f,
                         kstar < K ? (float)(1.0 / D.S[qs]) : 0.0f);
      D.flags = D.fl[0] | D.fl[1];
    }
  }
  __syncthreads();
}

// One slab-sum pair, published by one workgroup and read by another of the same launch:
// agent-scope atomic store and load (written through to, and read from, the point where
// the chip's L2 caches are coherent), so no L2 write-back or invalidate is needed.
__device__ __forceinline__ void slab_store(float2 *p, float2 v) {
  const unsigned long long b =
      (unsigned long long)__float_as_uint(v.x) | ((unsigned long long)__float_as_uint(v.y) << 32);
  __hip_atomic_store(reinterpret_cast<unsigned long long *>(p), b, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 slab_load(const float2 *p) {
  const unsigned long long b = __hip_atomic_load(reinterpret_cast<const unsigned long long *>(p),
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32)));
}

struct SpsDrawLds {
  double scan[kStreamBlock / kWave];
  int misc[4];
  float pick_logit;
  double tot, base;
  int use, sl;
};

// The SpS token of sequence g (every thread of a kStreamBlock workgroup calls it): the slab
// where the running sum of the slab sums crosses u * total, then the inverse CDF inside it.
template <int DT>
__device__ __forceinline__ void sps_draw(int g, int K, int kstar, float4 nm, const char *prow,
                                         const char *qrow, bool vec, int V, int chunk_elems,
                                         int chunks, float c, uint64_t seed, uint64_t step,
                                         const float2 *__restrict__ slab, SpsDrawLds &L,
                                         int32_t *__restrict__ out_tokens,
                                         float *__restrict__ out_logp, int32_t *status) {
  constexpr int Q = kSpsSlabElems<DT>;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int nsl = chunks * kSpsSlabs;
  const float2 *p2 = slab + (int64_t)g * nsl;
  const double u = philox_uniform(seed, (uint32_t)g, step, 4u, 0);
  if (tid < kWave) {
    // one lane per slab: the residual and target totals, then the first slab whose running
    // sum exceeds u * total (scan within 64 slabs, then block by block, the same order in
    // both passes: the running sum ends exactly at the total, and u < 1)
    double rt = 0.0, pt = 0.0;
    for (int j0 = 0; j0 < nsl; j0 += kWave) {
      const int j = j0 + lane;
      const float2 v = j < nsl ? slab_load(p2 + j) : make_float2(0.0f, 0.0f);
      rt += wave_sum((double)v.x);
      pt += wave_sum((double)v.y);
    }
    const bool use_rho = qrow != nullptr && rt > 0.0;
    const double total = use_rho ? rt : pt;
    const double target = u * total;
    double base = 0.0;
    int sl = -1;
    if (isfinite(total) && total > 0.0) {
      int lastpos = -1;
      double lastval = 0.0;
      for (int j0 = 0; j0 < nsl && sl < 0; j0 += kWave) {
        const int j = j0 + lane;
        const float2 v = j < nsl ? slab_load(p2 + j) : make_float2(0.0f, 0.0f);
        const double x = use_rho ? (double)v.x : (double)v.y;
        const double inc = wave_inclusive_scan(x);
        const unsigned long long hit = __ballot(j < nsl && base + inc > target);
        const unsigned long long pos = __ballot(x > 0.0);
        if (pos) {
          const int f = 63 - __clzll(pos);
          lastpos = j0 + f;
          lastval = __shfl(x, f, kWave);
        }
        if (hit) {
          const int f = __ffsll(hit) - 1;
          sl = j0 + f;
          base += __shfl(inc - x, f, kWave);
        } else {
          base += __shfl(inc, kWave - 1, kWave);
        }
      }
      if (sl < 0) {  // not reached (see above): the last slab with a positive sum
        sl = lastpos;
        base = total - lastval;
      }
    }
    if (lane == 0) {
      L.tot = total;
      L.use = use_rho;
      L.sl = sl;
      L.base = base;
    }
  }
  __syncthreads();
  const double total = L.tot;
  int tok = -1;
  if (isfinite(total) && total > 0.0 && L.sl >= 0) {
    const int sl = L.sl;
    const int64_t a0 = (int64_t)(sl / kSpsSlabs) * chunk_elems + (int64_t)(sl % kSpsSlabs) * Q;
    const int64_t a1 = min((int64_t)V, a0 + (int64_t)Q);
    const ResidRow<DT> fd{prow, qrow, c, nm.x, nm.y, nm.z, nm.w, L.use != 0, vec};
    tok = chunk_inverse_cdf<kStreamBlock, Q / 8 / kStreamBlock>(a0, a1, L.base, u * total, fd,
                                                                L.scan, L.misc, &L.pick_logit);
  }
  if (tid == 0) {
    out_tokens[(int64_t)g * (K + 1) + kstar] = tok;
    if (out_logp) {
      // log p of the drawn token: (x*c - L2)*ln2 with L2 = Mc + log2(1/inv)
      double lp = __builtin_nan("");
      if (tok >= 0)
        lp = ((double)L.pick_logit * (double)c - ((double)nm.x - log2((double)nm.y))) * kLn2;
      out_logp[(int64_t)g * (K + 1) + K] = (float)lp;
    }
    if (tok < 0) atomicOr(status, isnan(total) ? SMCSD_ST_NAN_INPUT : SMCSD_ST_EMPTY_ROW);
  }
}

template <int DT, bool FUSED, bool STRIDE>
__global__ __launch_bounds__(kStreamBlock) void k_sps_resid(
    RowMap rm, int nseq, const int32_t *__restrict__ draft_tokens, int V, int chunk_elems,
    int chunks, int chunks_big, float c, uint64_t seed, uint64_t step,
    const float2 *__restrict__ part, const float *__restrict__ lse_in,
    const int32_t *__restrict__ ws_kstar, const float4 *__restrict__ ws_norm,
    float2 *__restrict__ slab, int32_t *__restrict__ arrivals, int32_t *__restrict__ out_tokens,
    int32_t *__restrict__ out_num, float *__restrict__ out_logp, float *__restrict__ out_logq,
    float *__restrict__ out_lse, int32_t *status) {
  using E = Elt<DT>;
  constexpr int EPV = E::kPerVec, NV = kSpsVecsPerLane<DT>, Q = kSpsSlabElems<DT>;
  __shared__ SpsDecision D;
  __shared__ SpsDrawLds DL;
  __shared__ int sLast;
  const int K = rm.K, R = 2 * K + 1;
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int64_t ntiles = (int64_t)nseq * chunks;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int g = (int)(t / chunks);
    const int ch = (int)(t - (int64_t)g * chunks);
    int kstar;
    float4 nm;
    if (FUSED) {
      sps_decide<DT>(rm, g, draft_tokens, V, chunks, chunks_big, c, seed, step, part, lse_in, D);
      kstar = D.kstar;
      nm = D.nm;
      if (ch == 0 && tid < kWave) {
        // the per-sequence outputs; the token at k* is the draw's
        int32_t *tok = out_tokens + (int64_t)g * (K + 1);
        if (lane <= K && lane != kstar) tok[lane] = lane < kstar ? D.tok[lane] : -1;
        if (lane < K) {
          if (out_logp) out_logp[(int64_t)g * (K + 1) + lane] = (float)D.lp[lane];
          if (out_logq) out_logq[(int64_t)g * K + lane] = (float)D.lq[lane];
        }
        if (out_lse)
          for (int r = lane; r < R; r += kWave) out_lse[(int64_t)g * R + r] = (float)(D.L2[r] * kLn2);
        if (lane == 0) {
          if (out_num) out_num[g] = kstar + 1;
          if (D.flags) atomicOr(status, D.flags);
        }
      }
    } else {
      kstar = ws_kstar[g];
      nm = ws_norm[g];
    }
    const char *prow = rm.row(g, kstar);
    const char *qrow = kstar < K ? rm.row(g, K + 1 + kstar) : nullptr;
    const bool vec = ((uintptr_t)prow % 16 == 0) && ((uintptr_t)qrow % 16 == 0);
    const ResidRow<DT> fn{prow, qrow, c, nm.x, nm.y, nm.z, nm.w, qrow != nullptr, vec};

    // residual pass: slab wv of this chunk, NV vectors per lane per row
    const int64_t e0 = (int64_t)ch * chunk_elems;
    const int64_t e1 = min((int64_t)V, e0 + (int64_t)chunk_elems);
    const int64_t s0 = e0 + (int64_t)wv * Q;
    const int64_t s1 = min(e1, s0 + (int64_t)Q);
    float srho = 0.0f, sp = 0.0f;
    auto accum = [&](const uint4 &wp, const uint4 &wq, int64_t a) {
      float xp[EPV], xq[EPV];
      E::unpack(wp, xp);
      E::unpack(wq, xq);
#pragma unroll
      for (int i = 0; i < EPV; ++i) {
        if (a + i < s1) {
          const float p = fn.pval(xp[i]);
          sp += p;
          if (qrow) srho += fn.rho(p, xq[i]);
        }
      }
    };
    if (vec && s1 - s0 == Q) {
      // a whole slab of aligned rows: every 16-byte load issued before the first use
      uint4 rp[NV], rq[NV];
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int64_t a = s0 + (int64_t)(lane + u * kWave) * EPV;
        rp[u] = *reinterpret_cast<const uint4 *>(prow + a * E::kBytes);
        rq[u] = qrow ? *reinterpret_cast<const uint4 *>(qrow + a * E::kBytes) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < NV; ++u) accum(rp[u], rq[u], s0 + (int64_t)(lane + u * kWave) * EPV);
    } else if (s0 < s1) {
      // a partial slab or unaligned rows: element loads at clamped indices
      for (int u = 0; u < NV; ++u) {
        const int64_t a = s0 + (int64_t)(lane + u * kWave) * EPV;
        const uint4 wp = load_vec_any<DT>(prow, a, s1, vec);
        const uint4 wq = qrow ? load_vec_any<DT>(qrow, a, s1, vec) : make_uint4(0, 0, 0, 0);
        accum(wp, wq, a);
      }
    }
    srho = wave_sum_f32(srho);
    sp = wave_sum_f32(sp);
    if (lane == 0) slab_store(slab + t * kSpsSlabs + wv, make_float2(srho, sp));
    // arrival: every wave's slab store has completed (waited for) before the workgroup's
    // counter increment is issued, so the workgroup that sees the count reach `chunks`
    // reads every slab of the sequence; it draws the token
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) sLast = atomicAdd(&arrivals[g], 1) == chunks - 1;
    __syncthreads();
    if (sLast)
      sps_draw<DT>(g, K, kstar, nm, prow, qrow, vec, V, chunk_elems, chunks, c, seed, step, slab,
                   DL, out_tokens, out_logp, status);
    if (!STRIDE) break;
    __syncthreads();  // the next tile reuses the LDS
  }
}

__global__ void k_zero_i32(int32_t *__restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// ---------------------------------------------------------------------------------
// Philox check kernel
// ---------------------------------------------------------------------------------
__global__ void k_philox(const uint32_t *__restrict__ ctr, const uint32_t *__restrict__ key, int n,
                         uint32_t *__restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint32_t c[4] = {ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3]};
  philox_block(c, key[2 * i], key[2 * i + 1]);
  out[4 * i] = c[0];
  out[4 * i + 1] = c[1];
  out[4 * i + 2] = c[2];
  out[4 * i + 3] = c[3];
}

// ---------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------
// Occupancy of the inverse-CDF LSE pass.  Its registers allow 5 workgroups (20 waves) per
// CU; measured on the MI355X, 4 stream faster whenever rows span several tiles (B = 32,
// N = 16, K = 4, V = 128256 bf16: verify call 186 -> 183 us; B = 8, N = 128, K = 5,
// V = 152064: 517 -> 506 us; B = 16, N = 64, K = 8, fp32: 1325 -> 1316 us), while 3 per CU
// is no better than 5 and 2 is 20 % slower.  The race mode (ALU-heavy bonus tiles) and a
// launch of bonus tiles only (K = 0: the draft sampler) are faster at 5 and keep it.  The
// limit is set through LDS: the launch asks for dynamic LDS, which the kernel never
// touches, so that each workgroup holds just over a fifth of the CU's 160 KiB.
constexpr size_t kLdsPerCu = 160 * 1024;
constexpr int kLseWgPerCu = 4;

struct LdsPad {
  hipError_t err;
  size_t bytes;
};

// Taken once per element type (a thread-safe static): the kernel's static LDS is fixed at
// build time.
template <int DT>
static hipError_t lse_occupancy_pad(size_t *pad) {
  static const LdsPad p = [] {
    hipFuncAttributes fa{};
    const hipError_t e =
        hipFuncGetAttributes(&fa, reinterpret_cast<const void *>(&k_lse_partials<DT, false>));
    if (e != hipSuccess) return LdsPad{e, 0};
    const size_t per_wg = kLdsPerCu / (kLseWgPerCu + 1) + 1;
    return LdsPad{hipSuccess, per_wg > fa.sharedSizeBytes ? per_wg - fa.sharedSizeBytes : 0};
  }();
  *pad = p.bytes;
  return p.err;
}

template <int DT>
static hipError_t launch_verify_t(const VerifyArgs &a) {
  const int esz = Elt<DT>::kBytes;
  const int ce = chunk_elems(DT);
  const int chunks = (int)ceil_div(a.V, ce);
  const int K = a.K;
  RowMap rm{static_cast<const char *>(a.tgt), static_cast<const char *>(a.drf),
            a.row_stride * esz, a.seq_step, K};
  const VerifyWs w = verify_ws_layout(a.nseq, K, a.V, a.mode);
  float2 *part = reinterpret_cast<float2 *>(a.ws + w.part);
  float *sub = reinterpret_cast<float *>(a.ws + w.sub);
  int2 *race = reinterpret_cast<int2 *>(a.ws + w.race);
  // In the plain verify (inverse-CDF bonus or SpS, target and draft rows read) a row's big
  // tiles share it equally (whole 16-byte vectors each; the last takes the rest, never
  // nothing: the rounding adds under chunks_big * 8 elements, far below a tile); in race
  // mode and with the draft's log q given they are full tiles and a shorter remainder.
  // Chosen by measurement per mode (no model of why it differs).
  const int chunks_big = (int)ceil_div(a.V, big_tile_elems(esz, a.mode == SMCSD_MODE_SMC_RACE));
  const bool balance = a.mode != SMCSD_MODE_SMC_RACE && !a.logq_in;
  const int big_elems = balance ? (int)(ceil_div(ceil_div(a.V, chunks_big), 16 / esz) * (16 / esz))
                                : big_tile_elems(esz, a.mode == SMCSD_MODE_SMC_RACE);
  const int nb_per_seq = a.logq_in ? K : 2 * K;
  const int64_t ntiles = (int64_t)a.nseq * (chunks + (int64_t)nb_per_seq * chunks_big);
  const unsigned grid = grid_blocks(ntiles, kStreamBlock);
  size_t pad = 0;
  if (K > 0 && a.mode != SMCSD_MODE_SMC_RACE) {
    const hipError_t e = lse_occupancy_pad<DT>(&pad);
    if (e != hipSuccess) return e;
  }

  if (a.mode == SMCSD_MODE_SMC || a.mode == SMCSD_MODE_SMC_RACE) {
    const bool rc = a.mode == SMCSD_MODE_SMC_RACE;
    if (rc)
      hipLaunchKernelGGL((k_lse_partials<DT, true>), dim3(grid), dim3(kStreamBlock), 0, a.stream, rm,
                         a.nseq, a.V, ce, chunks, chunks_big, big_elems, nb_per_seq, a.c, part, sub, ntiles,
                         a.seed, a.step, race, nullptr);
    else
      hipLaunchKernelGGL((k_lse_partials<DT, false>), dim3(grid), dim3(kStreamBlock), pad, a.stream,
                         rm, a.nseq, a.V, ce, chunks, chunks_big, big_elems, nb_per_seq, a.c, part, sub, ntiles,
                         a.seed, a.step, race, nullptr);
    // one workgroup per sequence; the looping form only where the grid cap leaves fewer
    // workgroups than sequences (its loop costs registers: 157 VGPRs against 59)
    const unsigned gf = grid_blocks(a.nseq, kSmcFinalBlock);
    const bool stride = (int64_t)gf < a.nseq;
    auto fin = rc ? (stride ? k_smc_finalize<DT, true, true> : k_smc_finalize<DT, true, false>)
                  : (stride ? k_smc_finalize<DT, false, true> : k_smc_finalize<DT, false, false>);
    hipLaunchKernelGGL(fin, dim3(gf), dim3(kSmcFinalBlock), 0, a.stream, rm, a.nseq,
                       a.draft_tokens, a.V, ce, chunks, chunks_big, a.c, a.alpha, a.seed, a.step,
                       a.bonus_tag, part, a.logq_in, sub, race, a.log_weights, a.out_tokens,
                       a.out_num_tokens, a.out_logp, a.out_logq, a.out_lse, a.status);
    return hipGetLastError();
  }
  int32_t *kstar = reinterpret_cast<int32_t *>(a.ws + w.kstar);
  float4 *norm = reinterpret_cast<float4 *>(a.ws + w.l2);
  float2 *slab = reinterpret_cast<float2 *>(a.ws + w.part2);
  int32_t *arrivals = reinterpret_cast<int32_t *>(a.ws + w.arrivals);
  if (!a.lse_in)
    hipLaunchKernelGGL((k_lse_partials<DT, false>), dim3(grid), dim3(kStreamBlock), pad, a.stream, rm,
                       a.nseq, a.V, ce, chunks, chunks_big, big_elems, nb_per_seq, a.c, part, sub, ntiles,
                       a.seed, a.step, race, arrivals);
  else
    hipLaunchKernelGGL(k_zero_i32, dim3(grid_blocks(a.nseq, kStreamBlock)), dim3(kStreamBlock), 0,
                       a.stream, arrivals, a.nseq);
  // the decision inside every residual workgroup while a row has few chunk pairs, else a
  // decide kernel first
  const bool fused = chunks <= kSpsFusedChunksMax;
  if (!fused) {
    const unsigned gd = grid_blocks(a.nseq, kWave);
    hipLaunchKernelGGL(((int64_t)gd < a.nseq ? k_sps_decide<DT, true> : k_sps_decide<DT, false>),
                       dim3(gd), dim3(kWave), 0, a.stream, rm, a.nseq, a.draft_tokens, a.V, chunks,
                       chunks_big, a.c, a.seed, a.step, part, a.lse_in, kstar, norm, a.out_tokens,
                       a.out_num_tokens, a.out_logp, a.out_logq, a.out_lse, a.status);
  }
  const int64_t ntiles2 = (int64_t)a.nseq * chunks;
  const unsigned grid2 = grid_blocks(ntiles2, kStreamBlock);
  const bool stride2 = (int64_t)grid2 < ntiles2;
  auto resid = fused ? (stride2 ? k_sps_resid<DT, true, true> : k_sps_resid<DT, true, false>)
                     : (stride2 ? k_sps_resid<DT, false, true> : k_sps_resid<DT, false, false>);
  hipLaunchKernelGGL(resid, dim3(grid2), dim3(kStreamBlock), 0, a.stream, rm, a.nseq,
                     a.draft_tokens, a.V, ce, chunks, chunks_big, a.c, a.seed, a.step, part,
                     a.lse_in, kstar, norm, slab, arrivals, a.out_tokens, a.out_num_tokens,
                     a.out_logp, a.out_logq, a.out_lse, a.status);
  return hipGetLastError();
}

hipError_t launch_verify(const VerifyArgs &a) {
  if (a.dtype == SMCSD_DTYPE_BF16) return launch_verify_t<SMCSD_DTYPE_BF16>(a);
  return launch_verify_t<SMCSD_DTYPE_F32>(a);
}

hipError_t launch_philox(const uint32_t *ctr, const uint32_t *key, int n, uint32_t *out,
                         hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_philox, dim3((n + 255) / 256), dim3(256), 0, stream, ctr, key, n, out);
  return hipGetLastError();
}

}  // namespace smcsd
