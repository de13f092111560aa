// Split-context decode and its merge with the partition workspace in library-owned device
// memory, for callers that cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). The computation is exactly pkv_paged_attention_decode in
// split-context mode followed by pkv_paged_attention_reduce; only where the workspace lives
// differs.
#include <mutex>

#include "host_errors.hpp"
#include "pagedkv.h"

namespace {

// The partition workspace: max_logits | exp_sums | tmp_out, each part starting on a 256-byte
// boundary. Every device the library runs on holds its own copy until the process ends.
static __device__ __align__(256) unsigned char scratch[PKV_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once known

// The device address of `scratch` on the current device. Host code must never pass the
// array's own name to a kernel or a copy: on the host it is only a stand-in for the symbol.
pkv_status scratch_address(const char* fn, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return pkv::hip_failure(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "%s: device %d (at most %d devices)", fn, dev,
                     kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return pkv::hip_failure(e, "hipGetSymbolAddress(scratch)");
    if (!p) return pkv::fail(PKV_ERR_HIP, "%s: no device address for the workspace", fn);
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PKV_OK;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" pkv_status pkv_paged_attention_decode_static(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* work_items, int32_t num_work_items, int32_t max_context_len,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, float scale, pkv_dtype dtype,
    int32_t partition_size, void* stream) {
  const char* fn = "pkv_paged_attention_decode_static";
  const int dt = pkv::enum_arg(dtype);
  if (dt != PKV_F32 && dt != PKV_F16 && dt != PKV_BF16)
    return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "%s: bad dtype %d", fn, dt);
  if (partition_size <= 0)
    return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "%s: partition_size %d (split-context only)", fn,
                     partition_size);
  if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || max_context_len < 0)
    return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "%s: num_seqs %d num_heads %d head_dim %d "
                     "max_context_len %d", fn, num_seqs, num_heads, head_dim, max_context_len);
  const size_t np = ((size_t)max_context_len + partition_size - 1) / partition_size;
  const unsigned __int128 rows128 = (unsigned __int128)num_seqs * (unsigned)num_heads * np;
  const unsigned __int128 need128 =
      2 * (rows128 * sizeof(float) + 255) + rows128 * (unsigned)head_dim * sizeof(float);
  if (need128 > PKV_STATIC_WORKSPACE_BYTES)
    return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "%s: %d sequences x %d heads x %zu partitions "
                     "need more than the %zu bytes of the static workspace", fn, num_seqs,
                     num_heads, np, (size_t)PKV_STATIC_WORKSPACE_BYTES);
  const size_t rows = (size_t)rows128;
  const size_t part = round256(rows * sizeof(float));
  void* base = nullptr;
  pkv_status st = scratch_address(fn, &base);
  if (st != PKV_OK) return st;
  float* max_logits = static_cast<float*>(base);
  float* exp_sums = reinterpret_cast<float*>(static_cast<char*>(base) + part);
  float* tmp_out = reinterpret_cast<float*>(static_cast<char*>(base) + 2 * part);
  // Partitions past a sequence's last one are neither written nor read, so nothing in the
  // workspace has to start at zero.
  st = pkv_paged_attention_decode(nullptr, q, k_cache, v_cache, block_tables,
                                  max_blocks_per_seq, context_lens, work_items, num_work_items,
                                  max_context_len, num_seqs, num_heads, num_kv_heads, head_dim,
                                  block_size, num_blocks, scale, dtype, partition_size,
                                  max_logits, exp_sums, tmp_out, stream);
  if (st != PKV_OK) return st;
  return pkv_paged_attention_reduce(out, max_logits, exp_sums, tmp_out, context_lens, num_seqs,
                                    num_heads, head_dim, partition_size, (int32_t)np, dtype,
                                    stream);
}
