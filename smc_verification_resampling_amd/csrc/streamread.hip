// streamread.hip - a measurement aid (gfx950): every 16-byte word of a buffer read once.
//
// The verify's LSE pass is one streaming read of the logits with a few VALU operations per
// element: decoding is bound by memory bandwidth, not arithmetic (SMC explainers, problem
// statement).  Its speed of light is therefore the rate at which the chip streams reads
// from HBM, which on a real part sits below the 8 TB/s of the data sheet.  This kernel
// reads with the LSE pass's instruction (16-byte nontemporal buffer loads; all 32 loads of
// a thread's share of a tile are in flight at once) and does no arithmetic beyond an XOR
// fold, so its rate is that achievable ceiling, measured on the same GPU beside the verify
// call.  One workgroup per contiguous 128 KiB tile: on the MI355X that order streamed
// fastest among those measured (32 to 256 KiB tiles, tiles split into interleaved pieces,
// a grid-stride sweep of the whole buffer).
// Each workgroup writes the XOR of its tile's 32-bit words to its own output word, so the
// loads cannot be dropped and every tile's bounds can be checked against the host.  No
// atomics: an atomic XOR from every workgroup into one word serialised at the memory side
// and held the workgroups' slots, and cost a quarter of the read rate on random data (but
// nothing on data whose tiles XOR to zero).  One launch per call.
#include "../../include/smcsd.h"
#include "device.hpp"
#include "internal.hpp"

namespace smcsd {

namespace {

constexpr int kReadBlock = 256;
constexpr int kReadUnroll = 8;
constexpr int kReadTileBytes = SMCSD_STREAM_READ_TILE_BYTES;
constexpr int kReadStepBytes = kReadBlock * 16 * kReadUnroll;  // 8 loads per thread
constexpr int kReadSteps = kReadTileBytes / kReadStepBytes;
static_assert(kReadSteps * kReadStepBytes == kReadTileBytes, "a tile is whole steps");

__device__ __forceinline__ uint32_t fold(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Workgroup b reads bytes [b * tile, min(bytes, (b + 1) * tile)) and writes their XOR to
// tile_xor[b].  Full tiles issue their loads with no bounds test; the last, partial tile
// (bytes is a multiple of 16) tests each load against its end, so no load leaves the buffer.
__global__ __launch_bounds__(kReadBlock) void k_stream_read(const char *__restrict__ p,
                                                            int64_t bytes,
                                                            uint32_t *__restrict__ tile_xor) {
  const int64_t t0 = (int64_t)blockIdx.x * kReadTileBytes;
  const int64_t left = bytes - t0;
  const int nb = left < kReadTileBytes ? (int)left : kReadTileBytes;
  const __amdgpu_buffer_rsrc_t rs = stream_rsrc(p + t0, nb);
  const int lane_off = threadIdx.x * 16;
  uint32_t acc = 0;
  if (nb == kReadTileBytes) {
#pragma unroll
    for (int s = 0; s < kReadSteps; ++s) {
      uint4 v[kReadUnroll];
#pragma unroll
      for (int k = 0; k < kReadUnroll; ++k)
        v[k] = load_stream(rs, lane_off, s * kReadStepBytes + k * kReadBlock * 16);
#pragma unroll
      for (int k = 0; k < kReadUnroll; ++k) acc ^= fold(v[k]);
    }
  } else {
    for (int s = 0; s < kReadSteps; ++s) {
      uint4 v[kReadUnroll];
#pragma unroll
      for (int k = 0; k < kReadUnroll; ++k) {
        const int off = s * kReadStepBytes + k * kReadBlock * 16;
        v[k] = lane_off + off < nb ? load_stream(rs, lane_off, off) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int k = 0; k < kReadUnroll; ++k) acc ^= fold(v[k]);
    }
  }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, kWave);
  __shared__ uint32_t red[kReadBlock / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int w = 0; w < kReadBlock / kWave; ++w) x ^= red[w];
    tile_xor[blockIdx.x] = x;
  }
}

}  // namespace

hipError_t launch_stream_read(const void *p, int64_t bytes, uint32_t *tile_xor,
                              hipStream_t stream) {
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)((bytes + kReadTileBytes - 1) / kReadTileBytes)),
                     dim3(kReadBlock), 0, stream, static_cast<const char *>(p), bytes, tile_xor);
  return hipGetLastError();
}

}  // namespace smcsd
