// Read-bandwidth probes: the memory side of paged decode with none of its arithmetic.
//
// A paged KV read fetches whole (block, kv head) tiles -- S * D contiguous elements of K, the
// same of V -- from blocks that lie anywhere in the pool (Qualiteg, "About PagedAttention for
// LLM serving", item 1-2: blocks need not be contiguous; vAttention section 3.1: the attention
// kernel must read non-contiguous KV-cache blocks). What HBM delivers to a kernel that only
// loads such tiles is the ceiling a decode kernel can approach; a streaming read of one
// contiguous buffer is the ceiling of any read at all. Both probes fold what they load into a
// value that is stored only if it equals a fixed pattern, so no load can be dropped.
#include <stdint.h>

#include "host_errors.hpp"
#include "kernels.hpp"

namespace pkv {
namespace {

constexpr int kProbeThreads = 256;                      // 4 waves; 16 bytes per lane per load
constexpr int kPieceBytes = kProbeThreads * 16;         // one coalesced 4 KiB load per workgroup
constexpr int kStreamUnroll = 8;                        // 4 KiB pieces in flight per workgroup
constexpr int64_t kStreamChunk = (int64_t)kPieceBytes * kStreamUnroll;  // 32 KiB
constexpr int kGatherUnroll = 8;                        // tiles in flight per workgroup
constexpr uint32_t kNeverPattern = 0x9E3779B9u;

__device__ __forceinline__ void keep(uint32_t x, uint32_t* sink) {
  if (x == kNeverPattern) sink[0] = x;  // depends on every load; in practice never taken
}

// Workgroup w reads 32 KiB chunks w, w + grid, ...: eight coalesced 4 KiB loads per chunk.
template <bool NT>
__global__ void __launch_bounds__(kProbeThreads)
stream_read_kernel(const char* __restrict__ buf, int64_t chunks, uint32_t* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t c = blockIdx.x; c < chunks; c += gridDim.x) {
    const char* p = buf + c * kStreamChunk + threadIdx.x * 16;
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = load_kv<NT, u32x4>(p + u * kPieceBytes);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u];
  }
  keep(acc.x ^ acc.y ^ acc.z ^ acc.w, sink);
}

// Workgroup w reads listed tiles w * U .. w * U + U - 1, then the same U tiles one grid
// further on, ...; a tile of PIECES * 4 KiB is PIECES coalesced loads. A tile whose byte range
// is not inside [0, base_bytes) or whose offset is not 16-byte aligned is skipped.
template <bool NT, int PIECES>
__global__ void __launch_bounds__(kProbeThreads)
tile_gather_kernel(const char* __restrict__ base, int64_t base_bytes,
                   const int64_t* __restrict__ offsets, int32_t num_tiles, uint32_t* sink) {
  constexpr int64_t kTile = (int64_t)PIECES * kPieceBytes;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t t0 = (int64_t)blockIdx.x * kGatherUnroll; t0 < num_tiles;
       t0 += (int64_t)gridDim.x * kGatherUnroll) {
    int64_t off[kGatherUnroll];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int64_t o = t0 + u < num_tiles ? offsets[t0 + u] : -1;
      off[u] = (o >= 0 && (o & 15) == 0 && o <= base_bytes - kTile) ? o : -1;
    }
    u32x4 v[kGatherUnroll][PIECES];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u)
#pragma unroll
      for (int pc = 0; pc < PIECES; ++pc)
        v[u][pc] = off[u] >= 0
                       ? load_kv<NT, u32x4>(base + off[u] + pc * kPieceBytes + threadIdx.x * 16)
                       : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u)
#pragma unroll
      for (int pc = 0; pc < PIECES; ++pc) acc ^= v[u][pc];
  }
  keep(acc.x ^ acc.y ^ acc.z ^ acc.w, sink);
}

bool aligned(const void* p, uintptr_t a) { return p && ((uintptr_t)p % a) == 0; }

pkv_status launch_status(const char* fn) {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PKV_OK : hip_failure(e, fn);
}

}  // namespace
}  // namespace pkv

extern "C" {

pkv_status pkv_probe_stream_read(const void* buf, size_t bytes, int32_t nontemporal,
                                 int32_t workgroups, uint32_t* sink, void* stream) {
  const char* fn = "pkv_probe_stream_read";
  using namespace pkv;
  if (bytes == 0 || bytes % kStreamChunk || workgroups <= 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: bytes %zu (a positive multiple of %lld) "
                "workgroups %d", fn, bytes, (long long)kStreamChunk, workgroups);
  if (!aligned(buf, 16) || !aligned(sink, 4))
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: a pointer is null or misaligned", fn);
  const int64_t chunks = (int64_t)(bytes / kStreamChunk);
  const int grid = (int)(chunks < workgroups ? chunks : workgroups);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (nontemporal)
    stream_read_kernel<true><<<grid, kProbeThreads, 0, s>>>((const char*)buf, chunks, sink);
  else
    stream_read_kernel<false><<<grid, kProbeThreads, 0, s>>>((const char*)buf, chunks, sink);
  return launch_status(fn);
}

pkv_status pkv_probe_tile_gather(const void* base, size_t base_bytes,
                                 const int64_t* tile_offsets, int32_t num_tiles,
                                 int32_t tile_bytes, int32_t nontemporal, int32_t workgroups,
                                 uint32_t* sink, void* stream) {
  const char* fn = "pkv_probe_tile_gather";
  using namespace pkv;
  if (num_tiles < 0 || workgroups <= 0 || base_bytes > (size_t)INT64_MAX)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: num_tiles %d workgroups %d", fn, num_tiles,
                workgroups);
  if (tile_bytes != kPieceBytes && tile_bytes != 2 * kPieceBytes)
    return fail(PKV_ERR_UNSUPPORTED, "%s: tile_bytes %d (supported: 4096, 8192)", fn,
                tile_bytes);
  if (num_tiles == 0) return PKV_OK;
  if (!aligned(base, 16) || !aligned(tile_offsets, 8) || !aligned(sink, 4))
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: a pointer is null or misaligned", fn);
  const int64_t rounds = ((int64_t)num_tiles + kGatherUnroll - 1) / kGatherUnroll;
  const int grid = (int)(rounds < workgroups ? rounds : workgroups);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const char* b = (const char*)base;
  const int64_t nb = (int64_t)base_bytes;
  if (tile_bytes == kPieceBytes) {
    if (nontemporal)
      tile_gather_kernel<true, 1><<<grid, kProbeThreads, 0, s>>>(b, nb, tile_offsets, num_tiles, sink);
    else
      tile_gather_kernel<false, 1><<<grid, kProbeThreads, 0, s>>>(b, nb, tile_offsets, num_tiles, sink);
  } else {
    if (nontemporal)
      tile_gather_kernel<true, 2><<<grid, kProbeThreads, 0, s>>>(b, nb, tile_offsets, num_tiles, sink);
    else
      tile_gather_kernel<false, 2><<<grid, kProbeThreads, 0, s>>>(b, nb, tile_offsets, num_tiles, sink);
  }
  return launch_status(fn);
}

}  // extern "C"
