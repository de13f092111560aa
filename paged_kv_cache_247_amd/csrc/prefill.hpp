// Internal interface of the paged prefill kernel (chunked-query causal attention over the
// paged KV cache) between the C ABI (api.cpp) and its translation unit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace pkv {

// Rows (query token x head of a kv-head group) of one workgroup: 4 waves of 32 rows. A work
// unit is (sequence i, kv head g, tile t of 128 / G query tokens).
constexpr int kPrefillWaves = 4;
constexpr int kPrefillRows = kPrefillWaves * 32;

struct PrefillParams {
  void* out;                  // [T, H, D]
  const void* q;              // [T, H, D]
  const void* k_cache;        // [N, Hkv, S, D]
  const void* v_cache;        // [N, Hkv, (S / VS) D, VS], VS = min(S, 32)
  const int32_t* block_tables;  // [B, MB]
  const int32_t* context_lens;  // [B]
  const int32_t* query_start;   // [B + 1]
  const int32_t* work_items;    // NULL = units in index order; else unit = i * num_tiles + t
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  int32_t num_tiles;   // tiles of the longest query chunk
  int32_t num_units;   // grid units (work items, or num_seqs * num_tiles)
  float scale_log2e;
};

hipError_t launch_prefill(Dt dt, int head_dim, int block_size, const PrefillParams& p,
                          hipStream_t stream);

}  // namespace pkv
