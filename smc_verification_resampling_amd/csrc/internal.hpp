// internal.hpp - launch geometry and workspace layout shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <algorithm>
#include <stdint.h>

namespace smcsd {

// Streaming LSE pass: one workgroup reduces one tile = (row, chunk of the vocabulary).
constexpr int kStreamBlock = 256;
constexpr int kStreamUnroll = 8;
// elements per tile: 32 KiB of logits for both dtypes
constexpr int kChunkElemsBf16 = 16384;
constexpr int kChunkElemsF32 = 8192;
constexpr int kChunkElemsMin = kChunkElemsF32;  // workspace is sized for the smaller tile
// Rows other than the bonus row are cut into big tiles: fewer workgroup reductions per
// byte.  Their partials use the first ceil(V / big tile) slots.  Inverse-CDF and SpS
// passes: kBigTileElems elements (64 KiB of bf16, 128 KiB of fp32: about four tiles per row
// of a 128K vocabulary).  Measured on the MI355X with that pass at 4 workgroups per CU:
// bf16 rows stream fastest in 64 KiB tiles (B = 32, N = 16, K = 4, V = 128256: 4,955
// against 4,923 steps/s for 128 KiB; 256 KiB 4,760), fp32 rows in 128 KiB tiles
// (B = 16, N = 64, K = 8: 719 against 712 steps/s for 64 KiB).  Race mode keeps 128 KiB
// for both dtypes: its ALU-heavy bonus tiles, spread among the big tiles, ran 7 % slower
// among 64 KiB bf16 tiles (4,541 against 4,894 steps/s at the B = 32 shape).
// In the plain verify (target and draft rows read, inverse-CDF bonus or SpS) these are
// upper bounds: a row's ceil(V / bound) big tiles share its V elements equally (rounded
// up to whole 16-byte vectors).  A plain read of 8.93 GB in the fp32 rows of a 128K
// vocabulary took 1,275-1,278 us in three 128 KiB tiles and a 117 KiB remainder per row
// and 1,247-1,250 us in four equal tiles (aligned 128 KiB tiles: 1,241-1,244 us); in the
// LSE pass equal tiles gave 5,014-5,023 against 4,984-4,994 steps/s at B = 32, N = 16,
// K = 4, V = 128256 bf16, and 738.6-740.9 against 737.0-739.6 at B = 16, N = 64, K = 8
// fp32 (two boxes, two reps each).  Race mode and the verify with the draft's log q given
// keep full tiles and a remainder: equal tiles cost them 0.9 % and 1.1 % at the B = 32
// shape (4,917 against 4,962 and 7,848 against 7,933 steps/s, same box).
constexpr int kBigTileElems = 32768;
constexpr int kRaceBigTileBytes = 128 * 1024;
constexpr int big_tile_elems(int elt_bytes, bool race) {
  return race ? kRaceBigTileBytes / elt_bytes : kBigTileElems;
}
static_assert(kBigTileElems % kChunkElemsBf16 == 0 && kBigTileElems % kChunkElemsF32 == 0 &&
                  (kRaceBigTileBytes / 2) % kChunkElemsBf16 == 0 &&
                  (kRaceBigTileBytes / 4) % kChunkElemsF32 == 0,
              "a big tile is a whole number of unrolled steps for both dtypes");

constexpr int kMaxK = 32;
constexpr int kMaxN = 1024;
constexpr int kMaxV = 1 << 24;  // largest vocabulary taken (and tested); ids fit every index type used

// A dispatch's size in work-items is a 32-bit field of the launch packet: a grid of more
// than 2^32 - 1 threads does not launch as asked.  Kernels whose item count can exceed
// that stride over their items with a grid of at most this many workgroups (still far more
// than the 256 compute units hold at once).
constexpr int64_t kMaxGridBlocks = 1 << 22;
inline unsigned grid_blocks(int64_t items, int threads_per_block) {
  const int64_t cap = std::min<int64_t>(kMaxGridBlocks, (int64_t)0xFFFFFFFF / threads_per_block);
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(items, cap));
}

inline int chunk_elems(int dtype) { return dtype == 1 ? kChunkElemsBf16 : kChunkElemsF32; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// A tile of the bonus row also sums its kSlabs slabs (one slab = the kStreamBlock vectors a
// workgroup loads together) so that the bonus draw re-reads one slab, not the whole chunk.
constexpr int kSlabs = kStreamUnroll;
// Residual slabs per chunk of the SpS draw (one per wave of a kStreamBlock workgroup).
constexpr int kSpsSlabsWs = kStreamBlock / 64;

// Verify workspace: [row partials float2 x nseq*(2K+1)*chunks][bonus slab sums float x nseq*chunks*kSlabs]
//                   [bonus race winners int2 x nseq*chunks]
//                   [kstar int32 x nseq][L2 pair double2 x nseq]
//                   [residual slab sums float2 x nseq*chunks*kSpsSlabsWs][arrival counters int32 x nseq]
struct VerifyWs {
  size_t part, sub, race, kstar, l2, part2, arrivals, total;
};
inline VerifyWs verify_ws_layout(int64_t nseq, int K, int V, int mode) {
  VerifyWs w{};
  const int64_t chunks = ceil_div(V, kChunkElemsMin);
  size_t off = 0;
  w.part = off;
  off += align256(sizeof(float) * 2 * (size_t)(nseq * (2 * K + 1) * chunks));
  w.sub = off;
  off += align256(sizeof(float) * (size_t)(nseq * chunks * kSlabs));
  w.race = off;
  off += align256(sizeof(int32_t) * 2 * (size_t)(nseq * chunks));
  if (mode == 1) {
    w.kstar = off;
    off += align256(sizeof(int32_t) * (size_t)nseq);
    w.l2 = off;
    off += align256(sizeof(double) * 2 * (size_t)nseq);
    w.part2 = off;
    off += align256(sizeof(float) * 2 * (size_t)(nseq * chunks * kSpsSlabsWs));
    w.arrivals = off;
    off += align256(sizeof(int32_t) * (size_t)nseq);
  }
  w.total = off;
  return w;
}

struct VerifyArgs {
  const void *tgt, *drf;
  int dtype;
  int64_t row_stride;
  int seq_step;
  const int32_t *draft_tokens;
  int nseq, K, V;
  float c;      // log2(e) / T, rounded once on the host
  float alpha;
  int mode;
  uint64_t seed, step;
  const float *lse_in;
  const float *logq_in;
  uint32_t bonus_tag;  // RNG tag of the row-K draw: 1 (bonus token) or 5 | pos << 8 (draft)
  float *log_weights;
  int32_t *out_tokens, *out_num_tokens;
  float *out_logp, *out_logq, *out_lse;
  int32_t *status;
  char *ws;
  hipStream_t stream;
};

hipError_t launch_verify(const VerifyArgs &a);

hipError_t launch_resample(float *lw, int B, int N, float tau, uint64_t seed, uint64_t step,
                           int32_t *anc, float *ess, int32_t *resampled, int32_t *status,
                           hipStream_t stream);

// The Resample step run inside the KV exchange kernel (lw == nullptr: not fused; the
// ancestors and decisions then come from anc / resampled).
struct FusedResample {
  float *lw;
  float tau;
  uint64_t seed, step;
  int32_t *anc;
  float *ess;
  int32_t *res;
};

hipError_t launch_kv(const int32_t *anc, const int32_t *resampled, const FusedResample &fr, int B,
                     int N, int32_t *tables, int M_cap, int bs, int64_t L, int R, int32_t *rc,
                     int32_t *free_list, int32_t *free_top, int64_t P, int32_t *cow,
                     int32_t *cow_count, int32_t *status, char *ws, hipStream_t stream);

// The block-table state check (kvcheck.hip): workspace bytes and launches.
size_t kv_check_ws_bytes(int64_t P);
hipError_t launch_kv_check(const int32_t *T, int64_t S, int M_cap, int slots,
                           const int32_t *rc, const int32_t *fl, const int32_t *free_top,
                           int64_t P, int32_t *viol, int32_t *status, char *ws,
                           hipStream_t stream);

hipError_t launch_stream_read(const void *p, int64_t bytes, uint32_t *tile_xor,
                              hipStream_t stream);
hipError_t launch_philox(const uint32_t *ctr, const uint32_t *key, int n, uint32_t *out,
                         hipStream_t stream);

}  // namespace smcsd
