// The C ABI of pagedkv.h: host-side validation of every scalar and pointer, kernel-family
// choice, grid sizing and launch on the caller's stream. Nothing here allocates.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <hip/hip_runtime.h>

#include "host_errors.hpp"
#include "kernels.hpp"
#include "pagedkv.h"
#include "prefill.hpp"

namespace {
thread_local int t_last_hip = 0;
thread_local char t_msg[256] = "";
}  // namespace

namespace pkv {

pkv_status fail(pkv_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(t_msg, sizeof t_msg, fmt, ap);
  va_end(ap);
  return s;
}

pkv_status hip_failure(hipError_t e, const char* what) {
  t_last_hip = (int)e;
  return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace pkv

namespace {

using pkv::fail;

pkv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  if (e == hipErrorNotSupported)
    return fail(PKV_ERR_UNSUPPORTED, "%s: no kernel instantiation for this shape", what);
  return pkv::hip_failure(e, what);
}

bool aligned(const void* p, uintptr_t a) { return p && ((uintptr_t)p % a) == 0; }

// Enum arguments are checked as the ints the caller passed (pkv::enum_arg) before they are
// used as enums.
bool valid_dtype(int d) { return d == PKV_F32 || d == PKV_F16 || d == PKV_BF16; }

pkv::Dt to_dt(int d) { return static_cast<pkv::Dt>(d); }

// Shape checks shared by every entry point.
pkv_status check_tile(const char* fn, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int dtype) {
  if (!valid_dtype(dtype)) return fail(PKV_ERR_INVALID_ARGUMENT, "%s: bad dtype %d", fn, dtype);
  if (num_kv_heads <= 0) return fail(PKV_ERR_INVALID_ARGUMENT, "%s: num_kv_heads %d", fn, num_kv_heads);
  if (head_dim <= 0 || block_size <= 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: head_dim %d block_size %d", fn, head_dim, block_size);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "%s: head_dim %d (supported: 64, 128)", fn, head_dim);
  if (block_size != 16 && block_size != 32 && block_size != 64 && block_size != 128 &&
      block_size != 256)
    return fail(PKV_ERR_UNSUPPORTED, "%s: block_size %d (supported: 16, 32, 64, 128, 256)", fn,
                block_size);
  return PKV_OK;
}

pkv_status decode_impl(const pkv_decode_options* opt, void* out, const void* q, void* k_cache,
                       void* v_cache, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                       const int32_t* work_items, int32_t num_work_items,
                       int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t num_blocks, float scale, int dtype,
                       int32_t partition_size, float* max_logits, float* exp_sums,
                       float* tmp_out, void* stream, const int32_t* groups = nullptr,
                       int32_t num_groups = 0) {
  const char* fn = groups ? "pkv_paged_attention_decode_shared" : "pkv_paged_attention_decode";
  pkv_status st = check_tile(fn, num_kv_heads, head_dim, block_size, dtype);
  if (st != PKV_OK) return st;
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARGUMENT, "%s: num_seqs %d", fn, num_seqs);
  if (num_heads <= 0 || num_heads % num_kv_heads)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: num_heads %d not a positive multiple of num_kv_heads %d",
                fn, num_heads, num_kv_heads);
  const int G = num_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(PKV_ERR_UNSUPPORTED, "%s: query group %d (supported: 1, 2, 4, 8, 16)", fn, G);
  if (num_blocks <= 0 || max_blocks_per_seq <= 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: num_blocks %d max_blocks_per_seq %d", fn,
                num_blocks, max_blocks_per_seq);
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: max_blocks_per_seq %d x block_size %d positions "
                "exceed int32", fn, max_blocks_per_seq, block_size);
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: max_context_len %d outside [0, %lld]", fn,
                max_context_len, (long long)max_blocks_per_seq * block_size);
  if (!isfinite(scale)) return fail(PKV_ERR_INVALID_ARGUMENT, "%s: scale is not finite", fn);
  if (partition_size < 0 || (partition_size > 0 && partition_size % block_size))
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: partition_size %d is not 0 or a multiple of %d",
                fn, partition_size, block_size);
  const bool partial = partition_size > 0;
  if (partial) {
    if (!aligned(max_logits, 4) || !aligned(exp_sums, 4) || !aligned(tmp_out, 16))
      return fail(PKV_ERR_INVALID_ARGUMENT, "%s: partition workspace pointers null or misaligned", fn);
  } else if (max_logits || exp_sums || tmp_out) {
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: workspace pointers must be NULL in single-pass mode", fn);
  }
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      (!partial && !aligned(out, 16)) || (block_tables && !aligned(block_tables, 4)) ||
      !aligned(context_lens, 4) || (work_items && !aligned(work_items, 4)))
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: a tensor pointer is null or misaligned", fn);
  if (!block_tables && (int64_t)num_seqs * max_blocks_per_seq > num_blocks)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: without block tables the pool needs num_seqs * "
                "max_blocks_per_seq = %lld blocks, it has %d", fn,
                (long long)num_seqs * max_blocks_per_seq, num_blocks);
  static const pkv_decode_options defaults = {PKV_KERNEL_AUTO, 0u, nullptr, nullptr};
  if (!opt) opt = &defaults;
  if (opt->flags & ~(uint32_t)PKV_DECODE_CACHED_KV)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: unknown option flags 0x%x", fn, opt->flags);
  if ((opt->new_key == nullptr) != (opt->new_value == nullptr) ||
      (opt->new_key && (!aligned(opt->new_key, 16) || !aligned(opt->new_value, 16))))
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: new_key/new_value must both be NULL or both set "
                "and 16-byte aligned", fn);
  bool mfma;
  const int kernel = pkv::enum_arg(opt->kernel);
  switch (kernel) {
    case PKV_KERNEL_AUTO: mfma = dtype != PKV_F32 && G >= 4; break;
    case PKV_KERNEL_VALU: mfma = false; break;
    case PKV_KERNEL_MFMA: mfma = true; break;
    default: return fail(PKV_ERR_INVALID_ARGUMENT, "%s: bad kernel family %d", fn, kernel);
  }
  if (mfma && dtype == PKV_F32)
    return fail(PKV_ERR_UNSUPPORTED, "%s: the MFMA kernel takes fp16/bf16 only", fn);
  if (!mfma && G > 8)
    return fail(PKV_ERR_UNSUPPORTED, "%s: the VALU kernel takes query groups up to 8", fn);
  if (!mfma && !block_tables)
    return fail(PKV_ERR_UNSUPPORTED, "%s: the table-free contiguous layout runs on the MFMA kernel only", fn);
  if (groups) {
    if (!partial || !block_tables || !mfma || (opt->new_key && !work_items))
      return fail(PKV_ERR_INVALID_ARGUMENT, "%s: groups take partitions, block tables, the MFMA "
                  "kernel, and new rows only with a work list", fn);
    if (num_groups < 0 || !aligned(groups, 16))
      return fail(PKV_ERR_INVALID_ARGUMENT, "%s: groups pointer misaligned or num_groups %d", fn,
                  num_groups);
    if (num_seqs == 0) return PKV_OK;  // no member can be named: nothing to write
  }

  const int64_t ranges = partial ? ((int64_t)max_context_len + partition_size - 1) / partition_size : 1;
  if (work_items && num_work_items < 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: num_work_items %d", fn, num_work_items);
  const int64_t listed = work_items ? (int64_t)num_work_items : 0;
  const int64_t units = groups ? (int64_t)num_groups + listed
                       : work_items ? listed : (int64_t)num_seqs * ranges;
  if ((int64_t)num_seqs * ranges > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: %lld units", fn, (long long)num_seqs * ranges);
  const int64_t grid = units * num_kv_heads;  // the MFMA kernel pads units to a multiple of 8
  if ((units + 15) / 8 * 8 * num_kv_heads > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: grid of %lld workgroups", fn, (long long)grid);
  if (grid == 0) return PKV_OK;
  // No (sequence, range) unit exists (no sequences, or split mode with no positions): nothing
  // to write, and a work list could name none -- the kernels clamp work items into that range
  // (and groups would have no partition record to write).
  if ((int64_t)num_seqs * ranges == 0) return PKV_OK;

  pkv::DecodeParams p;
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.work_items = work_items;
  p.group_members = groups;
  p.num_units = (int32_t)(groups ? num_groups : units);
  p.new_key = opt->new_key;
  p.new_value = opt->new_value;
  p.max_logits = max_logits;
  p.exp_sums = exp_sums;
  p.tmp_out = tmp_out;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.range_tokens = partial ? partition_size : max_blocks_per_seq * block_size;
  p.num_ranges = (int32_t)ranges;
  p.scale_log2e = scale * pkv::kLog2e;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (groups && listed > 0) {
    // The groups and the listed units in one launch; the groups write no new rows.
    pkv::DecodeParams rest = p;
    rest.group_members = nullptr;
    rest.num_units = (int32_t)listed;
    p.work_items = nullptr;
    p.new_key = p.new_value = nullptr;
    return hip_status(pkv::launch_decode_mfma_shared(to_dt(dtype), head_dim, block_size, p,
                                                     rest, s), fn);
  }
  p.work_items = groups ? nullptr : work_items;
  p.new_key = groups ? nullptr : opt->new_key;
  p.new_value = groups ? nullptr : opt->new_value;
  const bool nt = !(opt->flags & PKV_DECODE_CACHED_KV);
  const hipError_t e =
      mfma ? pkv::launch_decode_mfma(to_dt(dtype), head_dim, block_size, partial, nt, p, s)
           : pkv::launch_decode_valu(to_dt(dtype), head_dim, block_size, G, partial, nt, p, s);
  return hip_status(e, fn);
}

pkv_status v_layout(const char* fn, bool to_columns, const void* src, void* dst,
                    int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int dtype, void* stream) {
  pkv_status st = check_tile(fn, num_kv_heads, head_dim, block_size, dtype);
  if (st != PKV_OK) return st;
  if (num_blocks < 0) return fail(PKV_ERR_INVALID_ARGUMENT, "%s: num_blocks %d", fn, num_blocks);
  if (num_blocks == 0) return PKV_OK;
  if (!aligned(src, 16) || !aligned(dst, 16))
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: a pointer is null or misaligned", fn);
  static const int eb[3] = {4, 2, 2};
  const int64_t bytes = (int64_t)num_blocks * num_kv_heads * block_size * head_dim * eb[dtype];
  const uintptr_t s = (uintptr_t)src, d = (uintptr_t)dst;
  if (s != d && s < d + bytes && d < s + bytes)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: source and destination overlap but differ", fn);
  pkv::VLayoutParams p;
  p.src = src;
  p.dst = dst;
  p.group = block_size < 32 ? block_size : 32;
  p.num_groups = (int64_t)num_blocks * num_kv_heads * (block_size / p.group);
  p.head_dim = head_dim;
  return hip_status(pkv::launch_v_layout(to_dt(dtype), to_columns, p,
                                         reinterpret_cast<hipStream_t>(stream)), fn);
}

}  // namespace

extern "C" {

pkv_status pkv_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                 void* v_cache, const int64_t* slot_mapping,
                                 int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, pkv_dtype dtype,
                                 void* stream) {
  const char* fn = "pkv_reshape_and_cache";
  pkv_status st = check_tile(fn, num_kv_heads, head_dim, block_size, pkv::enum_arg(dtype));
  if (st != PKV_OK) return st;
  if (num_tokens < 0 || num_blocks <= 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: num_tokens %d num_blocks %d", fn, num_tokens, num_blocks);
  if (num_tokens == 0) return PKV_OK;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(slot_mapping, 8))
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: a pointer is null or misaligned", fn);
  pkv::CacheWriteParams p;
  p.key = key;
  p.value = value;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.slot_mapping = slot_mapping;
  p.num_tokens = num_tokens;
  p.num_kv_heads = num_kv_heads;
  p.num_blocks = num_blocks;
  return hip_status(pkv::launch_reshape_and_cache(to_dt(dtype), head_dim, block_size, p,
                                                  reinterpret_cast<hipStream_t>(stream)), fn);
}

pkv_status pkv_paged_attention_decode(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* work_items, int32_t num_work_items, int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    pkv_dtype dtype, int32_t partition_size, float* max_logits, float* exp_sums,
    float* tmp_out, void* stream) {
  // Without new rows the kernels never write the pools.
  return decode_impl(nullptr, out, q, const_cast<void*>(k_cache), const_cast<void*>(v_cache),
                     block_tables, max_blocks_per_seq, context_lens, work_items,
                     num_work_items, max_context_len, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, scale, pkv::enum_arg(dtype), partition_size, max_logits, exp_sums, tmp_out,
                     stream);
}

pkv_status pkv_paged_attention_decode_ex(
    const pkv_decode_options* options, void* out, const void* q, void* k_cache, void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* work_items, int32_t num_work_items, int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    pkv_dtype dtype, int32_t partition_size, float* max_logits, float* exp_sums,
    float* tmp_out, void* stream) {
  return decode_impl(options, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                     context_lens, work_items, num_work_items, max_context_len, num_seqs,
                     num_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, scale, pkv::enum_arg(dtype),
                     partition_size, max_logits, exp_sums, tmp_out, stream);
}

pkv_status pkv_paged_attention_decode_shared(
    const void* q, void* k_cache, void* v_cache, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, const int32_t* groups,
    int32_t num_groups, const int32_t* work_items, int32_t num_work_items,
    const void* new_key, const void* new_value, int32_t max_context_len, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, float scale, pkv_dtype dtype, int32_t partition_size,
    float* max_logits, float* exp_sums, float* tmp_out, void* stream) {
  if (!groups)
    return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_paged_attention_decode_shared: groups is NULL");
  const pkv_decode_options mfma = {PKV_KERNEL_MFMA, 0u, new_key, new_value};
  return decode_impl(&mfma, nullptr, q, k_cache, v_cache,
                     block_tables, max_blocks_per_seq, context_lens, work_items, num_work_items,
                     max_context_len, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, scale, pkv::enum_arg(dtype), partition_size, max_logits, exp_sums, tmp_out,
                     stream, groups, num_groups);
}

pkv_status pkv_paged_attention_decode_grouped(
    void* out, const void* q, void* k_cache, void* v_cache, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, const int32_t* groups,
    int32_t num_groups, int32_t shared_len, const void* new_key, const void* new_value,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, float scale, pkv_dtype dtype, void* stream) {
  const char* fn = "pkv_paged_attention_decode_grouped";
  const int dt = pkv::enum_arg(dtype);
  pkv_status st = check_tile(fn, num_kv_heads, head_dim, block_size, dt);
  if (st != PKV_OK) return st;
  if (dt == PKV_F32) return fail(PKV_ERR_UNSUPPORTED, "%s: the matrix-core kernel takes fp16/bf16 only", fn);
  if (num_seqs < 0 || num_groups < 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: num_seqs %d num_groups %d", fn, num_seqs, num_groups);
  if (num_heads <= 0 || num_heads % num_kv_heads)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: num_heads %d not a positive multiple of num_kv_heads %d",
                fn, num_heads, num_kv_heads);
  const int G = num_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(PKV_ERR_UNSUPPORTED, "%s: query group %d (supported: 1, 2, 4, 8, 16)", fn, G);
  if (num_blocks <= 0 || max_blocks_per_seq <= 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: num_blocks %d max_blocks_per_seq %d", fn,
                num_blocks, max_blocks_per_seq);
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: max_blocks_per_seq %d x block_size %d positions "
                "exceed int32", fn, max_blocks_per_seq, block_size);
  if (shared_len < 0 || shared_len % block_size || shared_len > max_blocks_per_seq * block_size)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: shared_len %d is not a multiple of %d in [0, %d]",
                fn, shared_len, block_size, max_blocks_per_seq * block_size);
  if (!isfinite(scale)) return fail(PKV_ERR_INVALID_ARGUMENT, "%s: scale is not finite", fn);
  if ((new_key == nullptr) != (new_value == nullptr) ||
      (new_key && (!aligned(new_key, 16) || !aligned(new_value, 16))))
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: new_key/new_value must both be NULL or both set "
                "and 16-byte aligned", fn);
  if ((int64_t)num_groups * num_kv_heads > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: grid of %lld workgroups", fn,
                (long long)num_groups * num_kv_heads);
  if (num_groups == 0 || num_seqs == 0) return PKV_OK;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(groups, 16))
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: a tensor pointer is null or misaligned", fn);
  pkv::DecodeParams p = {};
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.work_items = nullptr;
  p.group_members = groups;
  p.new_key = new_key;
  p.new_value = new_value;
  p.max_logits = p.exp_sums = p.tmp_out = nullptr;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.range_tokens = shared_len;
  p.num_ranges = 1;
  p.num_units = num_groups;
  p.scale_log2e = scale * pkv::kLog2e;
  return hip_status(pkv::launch_decode_mfma(to_dt(dt), head_dim, block_size, false, false, p,
                                            reinterpret_cast<hipStream_t>(stream)), fn);
}

pkv_status pkv_paged_attention_reduce(void* out, const float* max_logits,
                                      const float* exp_sums, const float* tmp_out,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_heads, int32_t head_dim,
                                      int32_t partition_size, int32_t max_num_partitions,
                                      pkv_dtype dtype, void* stream) {
  const char* fn = "pkv_paged_attention_reduce";
  const int dt = pkv::enum_arg(dtype);
  if (!valid_dtype(dt)) return fail(PKV_ERR_INVALID_ARGUMENT, "%s: bad dtype %d", fn, dt);
  if (num_seqs < 0 || num_heads <= 0 || partition_size <= 0 || max_num_partitions < 0)
    return fail(PKV_ERR_INVALID_ARGUMENT,
                "%s: num_seqs %d num_heads %d partition_size %d max_num_partitions %d", fn,
                num_seqs, num_heads, partition_size, max_num_partitions);
  if (head_dim != 64 && head_dim != 128)
    return fail(head_dim > 0 ? PKV_ERR_UNSUPPORTED : PKV_ERR_INVALID_ARGUMENT,
                "%s: head_dim %d (supported: 64, 128)", fn, head_dim);
  if ((int64_t)num_seqs * num_heads > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: too many rows", fn);
  if (num_seqs == 0) return PKV_OK;
  if (!aligned(out, 16) || !aligned(context_lens, 4) ||
      (max_num_partitions > 0 &&
       (!aligned(max_logits, 4) || !aligned(exp_sums, 4) || !aligned(tmp_out, 16))))
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: a pointer is null or misaligned", fn);
  pkv::ReduceParams p;
  p.out = out;
  p.max_logits = max_logits;
  p.exp_sums = exp_sums;
  p.tmp_out = tmp_out;
  p.context_lens = context_lens;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.partition_size = partition_size;
  p.max_num_partitions = max_num_partitions;
  return hip_status(pkv::launch_reduce(to_dt(dt), head_dim, p, reinterpret_cast<hipStream_t>(stream)), fn);
}

int32_t pkv_prefill_tile_tokens(int32_t num_heads, int32_t num_kv_heads) {
  if (num_kv_heads <= 0 || num_heads <= 0 || num_heads % num_kv_heads) return 0;
  const int G = num_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return 0;
  return pkv::kPrefillRows / G;
}

pkv_status pkv_paged_attention_prefill(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                                       const int32_t* query_start, int32_t max_query_len,
                                       const int32_t* work_items, int32_t num_work_items,
                                       int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t num_blocks, float scale,
                                       pkv_dtype dtype, void* stream) {
  const char* fn = "pkv_paged_attention_prefill";
  pkv_status st = check_tile(fn, num_kv_heads, head_dim, block_size, pkv::enum_arg(dtype));
  if (st != PKV_OK) return st;
  if (dtype == PKV_F32)
    return fail(PKV_ERR_UNSUPPORTED, "%s: fp32 inputs (the matrix-core kernel takes fp16/bf16)", fn);
  if (num_seqs < 0 || num_tokens < 0 || max_query_len < 0 || num_work_items < 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: num_seqs %d num_tokens %d max_query_len %d", fn,
                num_seqs, num_tokens, max_query_len);
  if (num_heads <= 0 || num_heads % num_kv_heads)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: num_heads %d not a positive multiple of num_kv_heads %d",
                fn, num_heads, num_kv_heads);
  const int32_t tile = pkv_prefill_tile_tokens(num_heads, num_kv_heads);
  if (tile == 0)
    return fail(PKV_ERR_UNSUPPORTED, "%s: query group %d (supported: 1, 2, 4, 8, 16)", fn,
                num_heads / num_kv_heads);
  if (num_blocks <= 0 || max_blocks_per_seq <= 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: num_blocks %d max_blocks_per_seq %d", fn,
                num_blocks, max_blocks_per_seq);
  if (!isfinite(scale)) return fail(PKV_ERR_INVALID_ARGUMENT, "%s: scale is not finite", fn);
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(query_start, 4) ||
      (work_items && !aligned(work_items, 4)))
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: a tensor pointer is null or misaligned", fn);
  const int64_t tiles = ((int64_t)max_query_len + tile - 1) / tile;
  const int64_t units = work_items ? num_work_items : (int64_t)num_seqs * tiles;
  if ((int64_t)num_seqs * tiles > INT32_MAX || units * num_kv_heads > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: too many work units", fn);
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0 || units == 0) return PKV_OK;
  pkv::PrefillParams p;
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.query_start = query_start;
  p.work_items = work_items;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.num_tiles = (int32_t)tiles;
  p.num_units = (int32_t)units;
  p.scale_log2e = scale * pkv::kLog2e;
  return hip_status(pkv::launch_prefill(to_dt(dtype), head_dim, block_size, p,
                                        reinterpret_cast<hipStream_t>(stream)), fn);
}

pkv_status pkv_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                           const int64_t* block_mapping, int32_t num_pairs,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, pkv_dtype dtype, void* stream) {
  const char* fn = "pkv_copy_blocks";
  pkv_status st = check_tile(fn, num_kv_heads, head_dim, block_size, pkv::enum_arg(dtype));
  if (st != PKV_OK) return st;
  if (num_layers < 0 || num_pairs < 0 || num_blocks <= 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: num_layers %d num_pairs %d num_blocks %d", fn,
                num_layers, num_pairs, num_blocks);
  if (num_layers == 0 || num_pairs == 0) return PKV_OK;
  if (!k_caches || !v_caches || !aligned(block_mapping, 8))
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: null pointer array or misaligned mapping", fn);
  for (int l = 0; l < num_layers; ++l)
    if (!aligned(k_caches[l], 16) || !aligned(v_caches[l], 16))
      return fail(PKV_ERR_INVALID_ARGUMENT, "%s: layer %d pool pointer null or misaligned", fn, l);
  static const int eb[3] = {4, 2, 2};
  pkv::CopyParams p;
  p.block_mapping = block_mapping;
  p.num_pairs = num_pairs;
  p.num_blocks = num_blocks;
  p.tile_bytes = (int64_t)num_kv_heads * block_size * head_dim * eb[(int)dtype];
  for (int l0 = 0; l0 < num_layers; l0 += pkv::kMaxLayersPerLaunch) {
    const int n = num_layers - l0 < pkv::kMaxLayersPerLaunch ? num_layers - l0 : pkv::kMaxLayersPerLaunch;
    for (int l = 0; l < n; ++l) {
      p.k[l] = k_caches[l0 + l];
      p.v[l] = v_caches[l0 + l];
    }
    st = hip_status(pkv::launch_copy_blocks(n, p, reinterpret_cast<hipStream_t>(stream)), fn);
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

pkv_status pkv_v_cache_from_rows(const void* v_rows, void* v_cache, int32_t num_blocks,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 pkv_dtype dtype, void* stream) {
  return v_layout("pkv_v_cache_from_rows", true, v_rows, v_cache, num_blocks, num_kv_heads,
                  head_dim, block_size, pkv::enum_arg(dtype), stream);
}

pkv_status pkv_v_cache_to_rows(const void* v_cache, void* v_rows, int32_t num_blocks,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               pkv_dtype dtype, void* stream) {
  return v_layout("pkv_v_cache_to_rows", false, v_cache, v_rows, num_blocks, num_kv_heads,
                  head_dim, block_size, pkv::enum_arg(dtype), stream);
}

size_t pkv_partition_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                     int32_t max_context_len, int32_t partition_size) {
  if (partition_size <= 0 || num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 ||
      max_context_len <= 0)
    return 0;
  const size_t np = ((size_t)max_context_len + partition_size - 1) / partition_size;
  const unsigned __int128 bytes =
      (unsigned __int128)4 * (size_t)num_seqs * (size_t)num_heads * np * ((size_t)head_dim + 2);
  return bytes > SIZE_MAX ? SIZE_MAX : (size_t)bytes;
}

const char* pkv_status_string(pkv_status s) {
  switch (pkv::enum_arg(s)) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARGUMENT: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_NO_BLOCKS: return "out of blocks";
  }
  return "unknown status";
}

int pkv_last_hip_error(void) { return t_last_hip; }

const char* pkv_last_error_message(void) { return t_msg; }

int pkv_abi_version(void) { return 6; }

}  // extern "C"
