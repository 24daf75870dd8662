// kv_layout.hpp - workspace layout of the KV pointer exchange (shared by kv.hip and capi.hip).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "internal.hpp"

namespace smcsd {

constexpr int kKvGroupWords = 256;  // freed-bitmap words per pop-kernel workgroup

// [freed bitmap uint32 x ceil(P/32), padded to 64 words]
// [copy-on-write source + 1 (0 = none) int32 x S] [copy-on-write exclusive prefix int32 x S]
// [bitmap group rank bases int32 x ceil(words/256)] [pop index -> sequence int32 x P]
// [arrival counter] [top, F, pops requested]
// The bitmap and the counter must be zero before a call and are zero after it.
struct KvWs {
  size_t bitmap, cow_src, cow_excl, gbase, popmap, done, scal, total;
};
inline KvWs kv_ws_layout(int64_t S, int64_t P) {
  KvWs w{};
  const int64_t nwords = ceil_div(P, 32);
  size_t off = 0;
  w.bitmap = off;
  off += align256(sizeof(uint32_t) * (size_t)nwords);
  w.cow_src = off;
  off += align256(sizeof(int32_t) * (size_t)S);
  w.cow_excl = off;
  off += align256(sizeof(int32_t) * (size_t)S);
  w.gbase = off;
  off += align256(sizeof(int32_t) * (size_t)ceil_div(nwords, kKvGroupWords));
  w.popmap = off;
  off += align256(sizeof(int32_t) * (size_t)P);
  w.done = off;
  off += align256(sizeof(int32_t));
  w.scal = off;
  off += align256(sizeof(int32_t) * 4);
  w.total = off;
  return w;
}

}  // namespace smcsd
