// kv_layout.hpp - workspace layout of the KV pointer exchange (shared by kv.hip and capi.hip).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "internal.hpp"

namespace smcsd {

constexpr int kKvThreads = 256;                  // threads of every KV workgroup
constexpr int kKvTileEntries = 8192;             // table entries of one column tile (32 KiB)
constexpr int kKvGroupWords = 256;               // freed-bitmap words per pop-kernel workgroup
constexpr int kKvGroupBlocks = 32 * kKvGroupWords;  // blocks per group (8192)
// One-pass pop kernel (no last-workgroup step) limits: every workgroup holds the whole
// copy-on-write prefix in LDS and reads every group count.
constexpr int kKvFastSeqMax = 8192;
constexpr int kKvFastGroupMax = 4096;

// Two freed-block bitmaps and two per-group freed counts, used alternately by successive
// calls (parity of the call counter): a call sets bits in one pair and clears the other
// pair, which the previous call used.
//   [bitmap x2: uint32 x nwp each][group counts x2: int32 x ngp each]
//   [copy-on-write source + 1 (0 = none) int32 x S]
//   [copy-on-write exclusive prefix int32 x S][group rank bases int32 x ngroups]
//   [pop index -> sequence int32 x P]            (these three: many-sequence path only)
//   [arrival counter][call counter][scalars x 8]
// The whole workspace must be zero before the first call; calls keep it consistent.
struct KvWs {
  size_t bitmap, gcount, cow_src, cow_excl, gbase, popmap, done, ctr, scal, total;
  int64_t nwords, ngroups, nwp, ngp;
};
inline KvWs kv_ws_layout(int64_t S, int64_t P) {
  KvWs w{};
  w.nwords = ceil_div(P, 32);
  w.ngroups = ceil_div(w.nwords, kKvGroupWords);
  w.nwp = ceil_div(w.nwords, 64) * 64;
  w.ngp = ceil_div(w.ngroups, 64) * 64;
  size_t off = 0;
  w.bitmap = off;
  off += align256(sizeof(uint32_t) * 2 * (size_t)w.nwp);
  w.gcount = off;
  off += align256(sizeof(int32_t) * 2 * (size_t)w.ngp);
  w.cow_src = off;
  off += align256(sizeof(int32_t) * (size_t)S);
  w.cow_excl = off;
  off += align256(sizeof(int32_t) * (size_t)S);
  w.gbase = off;
  off += align256(sizeof(int32_t) * (size_t)w.ngroups);
  w.popmap = off;
  off += align256(sizeof(int32_t) * (size_t)P);
  w.done = off;
  off += align256(sizeof(int32_t));
  w.ctr = off;
  off += align256(sizeof(int32_t));
  w.scal = off;
  off += align256(sizeof(int32_t) * 8);
  w.total = off;
  return w;
}

// Workgroups of the exchange kernel per prompt.  A prompt whose old table spans more than
// one column tile (N * nb_old > kKvTileEntries) is split over workgroups of a quarter tile's
// columns each, and with a partial tail the tail column gets a part of its own (its
// workgroup also makes the copy-on-write decision).  Measured on the MI355X: B = 8,
// N = 128 with ~330 blocks per sequence spent 91 us in one workgroup per prompt, 31 us
// with one per tile and 26 us with one per quarter tile.
struct KvSplit {
  int parts, span, tail_alone;
};
inline KvSplit kv_split(int N, int nb_old, int tail_mod) {
  const int wcap = std::max(1, kKvTileEntries / N);
  const bool split = (int64_t)N * nb_old > kKvTileEntries;  // then nb_old > 8
  KvSplit k;
  k.tail_alone = split && tail_mod != 0;
  k.span = split ? std::max(1, wcap / 4) : std::max(nb_old, 1);
  k.parts = split ? (int)ceil_div(nb_old - k.tail_alone, k.span) + k.tail_alone : 1;
  return k;
}

}  // namespace smcsd
