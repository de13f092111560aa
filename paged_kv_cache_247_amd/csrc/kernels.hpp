// Internal launcher interface between the C ABI (api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace pkv {

// Arguments of one decode launch. A work unit is (sequence i, kv head g, range p) where range
// p covers positions [p * range_tokens, (p + 1) * range_tokens) of the sequence; single-pass
// mode uses one range of max_blocks_per_seq * block_size positions.
struct DecodeParams {
  void* out;
  const void* q;
  void* k_cache;  // written only by the fused newest-token write
  void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* work_items;  // NULL = all units in index order; else unit = i * num_ranges + p
  // NULL, or [num_units][4] sequences (-1 = none) sharing the blocks of range 0: each unit is
  // such a group (MFMA kernel, partials only), written to partition 0 of every member
  const int32_t* group_members;
  const void* new_key;        // NULL, or [B, Hkv, D]: position L-1 of each sequence, fused write
  const void* new_value;
  float* max_logits;
  float* exp_sums;
  float* tmp_out;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  int32_t range_tokens;
  int32_t num_ranges;
  int32_t num_units;  // grid units (work items, or num_seqs * num_ranges)
  float scale_log2e;
};

struct ReduceParams {
  void* out;
  const float* max_logits;
  const float* exp_sums;
  const float* tmp_out;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t partition_size;
  int32_t max_num_partitions;
};

constexpr int kMaxLayersPerLaunch = 32;

struct CopyParams {
  void* k[kMaxLayersPerLaunch];
  void* v[kMaxLayersPerLaunch];
  const int64_t* block_mapping;
  int32_t num_pairs;
  int32_t num_blocks;
  int64_t tile_bytes;  // Hkv * S * D * elt: one block of one pool
  int32_t pieces;      // workgroups per tile (set by the launcher)
};

struct CacheWriteParams {
  const void* key;
  const void* value;
  void* k_cache;
  void* v_cache;
  const int64_t* slot_mapping;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t num_blocks;
};

// Conversion of a V pool between token rows [N, Hkv, S, D] and the column-group layout.
struct VLayoutParams {
  const void* src;
  void* dst;
  int64_t num_groups;  // N * Hkv * S / VS column groups
  int32_t head_dim;
  int32_t group;       // VS = min(S, 32) positions per column group
};

// Each returns hipSuccess or the launch error; hipErrorNotSupported if no instantiation
// matches (the C ABI validates shapes before calling, so that is a library bug).
// nt: non-temporal K/V loads (else cached loads, for shared prefixes).
//
// The decode kernels are built once per block size (decode_valu.hip and decode_mfma.hip are
// compiled with -DPKV_BLOCK_SIZE=S, one object each), so each S is its own explicit
// instantiation and no other translation unit instantiates them.
template <int S>
hipError_t launch_decode_valu_bs(Dt dt, int head_dim, int group, bool partial, bool nt,
                                 const DecodeParams& p, hipStream_t stream);
template <int S>
hipError_t launch_decode_mfma_bs(Dt dt, int head_dim, bool partial, bool nt,
                                 const DecodeParams& p, hipStream_t stream);
// Groups sharing a prefix (grp) and the step's other units (rest, with a work list) in one
// launch of the MFMA kernel, both as partials with cached loads.
template <int S>
hipError_t launch_decode_mfma_shared_bs(Dt dt, int head_dim, const DecodeParams& grp,
                                        const DecodeParams& rest, hipStream_t stream);
#define PKV_DECODE_BLOCK_SIZE(S)                                                              \
  extern template hipError_t launch_decode_valu_bs<S>(Dt, int, int, bool, bool,              \
                                                      const DecodeParams&, hipStream_t);     \
  extern template hipError_t launch_decode_mfma_bs<S>(Dt, int, bool, bool,                   \
                                                      const DecodeParams&, hipStream_t);     \
  extern template hipError_t launch_decode_mfma_shared_bs<S>(                                \
      Dt, int, const DecodeParams&, const DecodeParams&, hipStream_t);
PKV_DECODE_BLOCK_SIZE(16)
PKV_DECODE_BLOCK_SIZE(32)
PKV_DECODE_BLOCK_SIZE(64)
PKV_DECODE_BLOCK_SIZE(128)
PKV_DECODE_BLOCK_SIZE(256)
#undef PKV_DECODE_BLOCK_SIZE

inline hipError_t launch_decode_valu(Dt dt, int head_dim, int block_size, int group,
                                     bool partial, bool nt, const DecodeParams& p,
                                     hipStream_t stream) {
  switch (block_size) {
    case 16: return launch_decode_valu_bs<16>(dt, head_dim, group, partial, nt, p, stream);
    case 32: return launch_decode_valu_bs<32>(dt, head_dim, group, partial, nt, p, stream);
    case 64: return launch_decode_valu_bs<64>(dt, head_dim, group, partial, nt, p, stream);
    case 128: return launch_decode_valu_bs<128>(dt, head_dim, group, partial, nt, p, stream);
    case 256: return launch_decode_valu_bs<256>(dt, head_dim, group, partial, nt, p, stream);
    default: return hipErrorNotSupported;
  }
}

inline hipError_t launch_decode_mfma(Dt dt, int head_dim, int block_size, bool partial,
                                     bool nt, const DecodeParams& p, hipStream_t stream) {
  switch (block_size) {
    case 16: return launch_decode_mfma_bs<16>(dt, head_dim, partial, nt, p, stream);
    case 32: return launch_decode_mfma_bs<32>(dt, head_dim, partial, nt, p, stream);
    case 64: return launch_decode_mfma_bs<64>(dt, head_dim, partial, nt, p, stream);
    case 128: return launch_decode_mfma_bs<128>(dt, head_dim, partial, nt, p, stream);
    case 256: return launch_decode_mfma_bs<256>(dt, head_dim, partial, nt, p, stream);
    default: return hipErrorNotSupported;
  }
}

inline hipError_t launch_decode_mfma_shared(Dt dt, int head_dim, int block_size,
                                            const DecodeParams& grp, const DecodeParams& rest,
                                            hipStream_t stream) {
  switch (block_size) {
    case 16: return launch_decode_mfma_shared_bs<16>(dt, head_dim, grp, rest, stream);
    case 32: return launch_decode_mfma_shared_bs<32>(dt, head_dim, grp, rest, stream);
    case 64: return launch_decode_mfma_shared_bs<64>(dt, head_dim, grp, rest, stream);
    case 128: return launch_decode_mfma_shared_bs<128>(dt, head_dim, grp, rest, stream);
    case 256: return launch_decode_mfma_shared_bs<256>(dt, head_dim, grp, rest, stream);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_reduce(Dt dt, int head_dim, const ReduceParams& p, hipStream_t stream);
hipError_t launch_reshape_and_cache(Dt dt, int head_dim, int block_size,
                                    const CacheWriteParams& p, hipStream_t stream);
hipError_t launch_copy_blocks(int num_layers, const CopyParams& p, hipStream_t stream);
hipError_t launch_v_layout(Dt dt, bool to_columns, const VLayoutParams& p, hipStream_t stream);

}  // namespace pkv
