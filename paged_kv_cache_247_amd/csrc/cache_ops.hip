// Cache maintenance kernels: writing each step's new K/V rows into their slots, and
// copy-on-write of whole blocks.
//
// A slot is block_id * S + position: the new token's K/V go to that position of that block
// (the cache grows by one position per generated token; Qualiteg, "About PagedAttention for LLM
// serving", the past_key_values loop of "Deepening Our Understanding ..." and item 1-2 on
// blocks). Requests that share a prefix share its blocks (Hacker News discussion of
// PagedAttention, replies on shared prefixes); a block is copied before a sequence writes into
// a shared one.
#include <limits.h>

#include "kernels.hpp"

namespace pkv {
namespace {

// One workgroup per new token. K: the token's rows are 16-byte vector stores into the [S][D]
// tiles. V goes to column pos % VS of column group pos / VS, each group a [D][VS] tile
// (VS = min(S, 32)): one element per (head, dim) row. When the token's aligned piece of kPiece
// positions (32 bytes of 16-bit elements: a whole memory sector, one row of a block of 16) is
// filled by kPiece consecutive tokens with consecutive slots -- the new tokens of a prompt --
// the k-th of them stores whole pieces of the k-th sixteenth of the (head, dim) rows, gathering
// each row's kPiece elements from all of them, so every token does the same work and every
// row is written once in full. Otherwise (the newest token of each of many sequences, the ends
// of a prompt) the token stores its own element of every row.
constexpr int kCacheThreads = 128;
constexpr int kPiece = 16;

template <Dt DT, int D, int S>
__global__ void __launch_bounds__(kCacheThreads) reshape_and_cache_kernel(const CacheWriteParams a) {
  using T = typename Elt<DT>::T;
  constexpr int EB = Elt<DT>::bytes;
  constexpr int VEC = 16 / EB;
  constexpr int VS = S < 32 ? S : 32;
  static_assert(VS % kPiece == 0, "a piece of positions stays within one column group");
  const int t = blockIdx.x;
  const int Hkv = a.num_kv_heads;
  const int64_t sl = a.slot_mapping[t];
  if (sl < 0 || sl >= (int64_t)a.num_blocks * S) return;
  const int64_t blk = sl / S;
  const int pos = (int)(sl % S);

  const char* key = reinterpret_cast<const char*>(a.key) + (size_t)t * Hkv * D * EB;
  char* kc = reinterpret_cast<char*>(a.k_cache);
  for (int v = threadIdx.x; v < Hkv * D / VEC; v += kCacheThreads) {
    const int h = (v * VEC) / D;
    const int d = (v * VEC) % D;
    const u32x4 x = *reinterpret_cast<const u32x4*>(key + ((size_t)h * D + d) * EB);
    *reinterpret_cast<u32x4*>(kc + (((blk * Hkv + h) * S + pos) * D + d) * EB) = x;
  }

  // Is the piece filled by tokens t - k .. t - k + kPiece - 1 with consecutive slots?
  const int k = pos % kPiece;
  const int t0 = t - k;
  bool full = t0 >= 0 && t0 + kPiece <= a.num_tokens;
  int64_t w[kPiece];
#pragma unroll
  for (int q = 0; q < kPiece; ++q) w[q] = full ? a.slot_mapping[t0 + q] : -1;
#pragma unroll
  for (int q = 0; q < kPiece; ++q) full = full && w[q] == sl - k + q;
  T* piece = reinterpret_cast<T*>(a.v_cache) + (size_t)blk * Hkv * S * D +
             (size_t)(pos / VS) * VS * D + (pos - k) % VS;
  if (full) {
    const T* val = reinterpret_cast<const T*>(a.value) + (size_t)t0 * Hkv * D;
    const int R = Hkv * D / kPiece;  // rows of this token's share
    for (int x = threadIdx.x; x < R; x += kCacheThreads) {
      const int e = k * R + x;
      __attribute__((aligned(16))) T row[kPiece];
#pragma unroll
      for (int q = 0; q < kPiece; ++q) row[q] = val[(size_t)q * Hkv * D + e];
      T* dst = piece + (size_t)(e / D) * S * D + (size_t)(e % D) * VS;
#pragma unroll
      for (int q = 0; q < kPiece * EB / 16; ++q)
        reinterpret_cast<u32x4*>(dst)[q] = reinterpret_cast<const u32x4*>(row)[q];
    }
  } else {
    const T* val = reinterpret_cast<const T*>(a.value) + (size_t)t * Hkv * D;
    for (int e = threadIdx.x; e < Hkv * D; e += kCacheThreads)
      piece[(size_t)(e / D) * S * D + (size_t)(e % D) * VS + k] = val[e];
  }
}

// A block of one pool is one contiguous tile. Workgroup (pair, piece) of (layer, pool) copies
// 4 KiB of it, one 16-byte vector per thread, so that a copy of a few blocks still spreads
// over the GPU and each thread waits for memory once.
constexpr int kCopyThreads = 256;
constexpr int kCopyPiece = kCopyThreads * 16;  // bytes per workgroup

__global__ void __launch_bounds__(kCopyThreads) copy_blocks_kernel(const CopyParams a) {
  const int pair = blockIdx.x / a.pieces;
  const int piece = blockIdx.x - pair * a.pieces;
  const int layer = blockIdx.y;
  const int64_t src = a.block_mapping[2 * pair];
  const int64_t dst = a.block_mapping[2 * pair + 1];
  if (src < 0 || dst < 0 || src >= a.num_blocks || dst >= a.num_blocks || src == dst) return;
  char* base = reinterpret_cast<char*>(blockIdx.z == 0 ? a.k[layer] : a.v[layer]);
  const u32x4* s = reinterpret_cast<const u32x4*>(base + src * a.tile_bytes);
  u32x4* d = reinterpret_cast<u32x4*>(base + dst * a.tile_bytes);
  const int64_t e = (int64_t)piece * kCopyThreads + threadIdx.x;
  if (e < a.tile_bytes / 16) d[e] = s[e];
}

// Conversion of a V pool between token rows [N, Hkv, S, D] and column groups. In both layouts
// column group c of a (block, kv head) tile holds positions c*VS .. c*VS + VS - 1 in the same
// VS*D elements, as [VS][D] rows or as a [D][VS] tile; so each workgroup transposes whole
// groups through LDS, reading and writing 16-byte vectors in HBM order. The LDS rows of
// positions are padded by one dword, so that the strided reads and writes along a head-dim
// index spread over the banks.
constexpr int kLayoutThreads = 256;
constexpr int kLayoutGrid = 4096;  // workgroups; each loops over groups
constexpr int kLayoutRowDwords = 128 + 1;  // f32 rows of D = 128, padded

template <typename U, bool TO_COLUMNS>
__global__ void __launch_bounds__(kLayoutThreads) v_layout_kernel(const VLayoutParams a) {
  constexpr int VEC = 16 / (int)sizeof(U);  // elements per 16-byte vector
  constexpr int UW = 4 / (int)sizeof(U);    // elements per dword
  __shared__ uint32_t lds[32 * kLayoutRowDwords];
  U* const lu = reinterpret_cast<U*>(lds);
  const int D = a.head_dim;
  const int VS = a.group;
  const int RW = D / UW;                // dwords of one position row
  const int LW = RW + 1;                // dwords of its padded LDS row
  const int nvec = VS * D / VEC;        // 16-byte vectors of a group
  for (int64_t grp = blockIdx.x; grp < a.num_groups; grp += gridDim.x) {
    const size_t off = (size_t)grp * VS * D * sizeof(U);
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.src) + off);
    u32x4* dst = reinterpret_cast<u32x4*>(static_cast<char*>(a.dst) + off);
    if constexpr (TO_COLUMNS) {
      for (int v = threadIdx.x; v < nvec; v += kLayoutThreads) {
        const u32x4 x = src[v];
        const int t = (4 * v) / RW;  // RW is a multiple of 4: a vector stays in its row
        uint32_t* r = lds + t * LW + (4 * v) % RW;
        r[0] = x[0]; r[1] = x[1]; r[2] = x[2]; r[3] = x[3];
      }
      __syncthreads();
      for (int v = threadIdx.x; v < nvec; v += kLayoutThreads) {
        const int d = (v * VEC) / VS;  // VS is a multiple of VEC: a vector stays in its row
        const int t0 = (v * VEC) % VS;
        __attribute__((aligned(16))) U col[VEC];
#pragma unroll
        for (int j = 0; j < VEC; ++j) col[j] = lu[(t0 + j) * LW * UW + d];
        dst[v] = *reinterpret_cast<const u32x4*>(col);
      }
    } else {
      for (int v = threadIdx.x; v < nvec; v += kLayoutThreads) {
        const int d = (v * VEC) / VS;
        const int t0 = (v * VEC) % VS;
        __attribute__((aligned(16))) U col[VEC];
        *reinterpret_cast<u32x4*>(col) = src[v];
#pragma unroll
        for (int j = 0; j < VEC; ++j) lu[(t0 + j) * LW * UW + d] = col[j];
      }
      __syncthreads();
      for (int v = threadIdx.x; v < nvec; v += kLayoutThreads) {
        const uint32_t* r = lds + ((4 * v) / RW) * LW + (4 * v) % RW;
        dst[v] = u32x4{r[0], r[1], r[2], r[3]};
      }
    }
    __syncthreads();  // the next group reuses the LDS rows
  }
}

template <Dt DT, int D>
hipError_t write_d(int block_size, const CacheWriteParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)p.num_tokens);
  constexpr int TH = kCacheThreads;
  switch (block_size) {
    case 16: reshape_and_cache_kernel<DT, D, 16><<<grid, TH, 0, stream>>>(p); break;
    case 32: reshape_and_cache_kernel<DT, D, 32><<<grid, TH, 0, stream>>>(p); break;
    case 64: reshape_and_cache_kernel<DT, D, 64><<<grid, TH, 0, stream>>>(p); break;
    case 128: reshape_and_cache_kernel<DT, D, 128><<<grid, TH, 0, stream>>>(p); break;
    case 256: reshape_and_cache_kernel<DT, D, 256><<<grid, TH, 0, stream>>>(p); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

template <Dt DT>
hipError_t write_t(int head_dim, int block_size, const CacheWriteParams& p, hipStream_t stream) {
  switch (head_dim) {
    case 64: return write_d<DT, 64>(block_size, p, stream);
    case 128: return write_d<DT, 128>(block_size, p, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

hipError_t launch_reshape_and_cache(Dt dt, int head_dim, int block_size,
                                    const CacheWriteParams& p, hipStream_t stream) {
  switch (dt) {
    case Dt::F32: return write_t<Dt::F32>(head_dim, block_size, p, stream);
    case Dt::F16: return write_t<Dt::F16>(head_dim, block_size, p, stream);
    case Dt::BF16: return write_t<Dt::BF16>(head_dim, block_size, p, stream);
  }
  return hipErrorNotSupported;
}

hipError_t launch_copy_blocks(int num_layers, const CopyParams& p, hipStream_t stream) {
  CopyParams q = p;
  q.pieces = (int32_t)((p.tile_bytes + kCopyPiece - 1) / kCopyPiece);
  if ((int64_t)p.num_pairs * q.pieces > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(p.num_pairs * q.pieces), (unsigned)num_layers, 2);
  copy_blocks_kernel<<<grid, kCopyThreads, 0, stream>>>(q);
  return hipGetLastError();
}

hipError_t launch_v_layout(Dt dt, bool to_columns, const VLayoutParams& p, hipStream_t stream) {
  if (p.head_dim > 128 || p.group > 32 || p.num_groups <= 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(p.num_groups < kLayoutGrid ? p.num_groups : kLayoutGrid));
  if (dt == Dt::F32) {
    if (to_columns) v_layout_kernel<uint32_t, true><<<grid, kLayoutThreads, 0, stream>>>(p);
    else v_layout_kernel<uint32_t, false><<<grid, kLayoutThreads, 0, stream>>>(p);
  } else {
    if (to_columns) v_layout_kernel<uint16_t, true><<<grid, kLayoutThreads, 0, stream>>>(p);
    else v_layout_kernel<uint16_t, false><<<grid, kLayoutThreads, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace pkv
