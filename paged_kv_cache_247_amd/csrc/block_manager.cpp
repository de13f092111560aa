// Host block manager (pkv_bm_* in pagedkv.h): reference-counted physical blocks, per-sequence
// block lists, sharing by fork, copy-on-write on append, swap out/in to a host pool; and
// pkv_swap_blocks, the copies a swap needs. Pure host bookkeeping: the caller runs the copies
// (pkv_copy_blocks, pkv_swap_blocks) on its stream before the blocks are written or reused.
#include <stdint.h>

#include <new>
#include <unordered_map>
#include <vector>

#include <hip/hip_runtime.h>

#include "host_errors.hpp"
#include "pagedkv.h"

namespace {

struct Seq {
  std::vector<int32_t> blocks;  // device block ids, or host block ids while swapped out
  int32_t tokens = 0;
  bool on_host = false;
};

}  // namespace

struct pkv_block_manager {
  int32_t block_size = 0;
  std::vector<int32_t> ref;        // references to each device block
  std::vector<int32_t> free_dev;   // stack of free device blocks (lowest id on top)
  std::vector<int32_t> free_host;  // stack of free host blocks
  std::unordered_map<int64_t, Seq> seqs;
};

namespace {

using pkv::fail;

std::vector<int32_t> id_stack(int32_t n) {
  std::vector<int32_t> v((size_t)n);
  for (int32_t i = 0; i < n; ++i) v[(size_t)i] = n - 1 - i;
  return v;
}

Seq* find(pkv_block_manager* bm, int64_t seq) {
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? nullptr : &it->second;
}

void release_device(pkv_block_manager* bm, int32_t b) {
  if (--bm->ref[(size_t)b] == 0) bm->free_dev.push_back(b);
}

// Host allocations (the sequence map, block lists) happen before any change to the books, so
// running out of host memory leaves them as they were; no exception leaves the C ABI. The free
// lists never grow past their size at creation, so returning blocks allocates nothing.
pkv_status out_of_memory(const char* fn) {
  return fail(PKV_ERR_INVALID_ARGUMENT, "%s: out of host memory", fn);
}

}  // namespace

extern "C" {

pkv_status pkv_bm_create(int32_t num_blocks, int32_t num_host_blocks, int32_t block_size,
                         pkv_block_manager** out) {
  if (!out) return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_create: out is NULL");
  *out = nullptr;
  if (num_blocks < 0 || num_host_blocks < 0 || block_size <= 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_create: num_blocks %d num_host_blocks %d block_size %d",
                num_blocks, num_host_blocks, block_size);
  pkv_block_manager* bm = new (std::nothrow) pkv_block_manager;
  if (!bm) return out_of_memory("pkv_bm_create");
  try {
    bm->block_size = block_size;
    bm->ref.assign((size_t)num_blocks, 0);
    bm->free_dev = id_stack(num_blocks);
    bm->free_host = id_stack(num_host_blocks);
  } catch (const std::bad_alloc&) {
    delete bm;
    return out_of_memory("pkv_bm_create");
  }
  *out = bm;
  return PKV_OK;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int32_t pkv_bm_free_blocks(const pkv_block_manager* bm) {
  return bm ? (int32_t)bm->free_dev.size() : 0;
}

int32_t pkv_bm_free_host_blocks(const pkv_block_manager* bm) {
  return bm ? (int32_t)bm->free_host.size() : 0;
}

pkv_status pkv_bm_add(pkv_block_manager* bm, int64_t seq, int32_t num_tokens) {
  if (!bm || seq < 0 || num_tokens < 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_add: bad manager, sequence or count");
  if (find(bm, seq)) return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_add: sequence %lld exists", (long long)seq);
  const size_t nb = ((size_t)num_tokens + bm->block_size - 1) / bm->block_size;
  if (nb > bm->free_dev.size())
    return fail(PKV_ERR_NO_BLOCKS, "pkv_bm_add: %zu blocks needed, %zu free", nb, bm->free_dev.size());
  Seq* s;
  try {
    s = &bm->seqs.emplace(seq, Seq{}).first->second;
    s->blocks.reserve(nb);
  } catch (const std::bad_alloc&) {
    bm->seqs.erase(seq);
    return out_of_memory("pkv_bm_add");
  }
  s->tokens = num_tokens;
  for (size_t k = 0; k < nb; ++k) {
    const int32_t b = bm->free_dev.back();
    bm->free_dev.pop_back();
    bm->ref[(size_t)b] = 1;
    s->blocks.push_back(b);
  }
  return PKV_OK;
}

pkv_status pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm || child < 0) return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_fork: bad manager or child");
  Seq* p = find(bm, parent);
  if (!p || p->on_host)
    return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_fork: parent %lld unknown or swapped out", (long long)parent);
  if (find(bm, child)) return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_fork: child %lld exists", (long long)child);
  try {
    Seq c = *p;
    p = nullptr;  // the map may rehash below
    const Seq& k = bm->seqs.emplace(child, std::move(c)).first->second;
    for (int32_t b : k.blocks) ++bm->ref[(size_t)b];
  } catch (const std::bad_alloc&) {
    return out_of_memory("pkv_bm_fork");
  }
  return PKV_OK;
}

pkv_status pkv_bm_append(pkv_block_manager* bm, int64_t seq, int64_t* slot, int32_t* copy_src,
                         int32_t* copy_dst) {
  if (!bm || !slot || !copy_src || !copy_dst)
    return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_append: NULL argument");
  Seq* s = find(bm, seq);
  if (!s || s->on_host)
    return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_append: sequence %lld unknown or swapped out", (long long)seq);
  *copy_src = *copy_dst = -1;
  const int32_t S = bm->block_size;
  const int32_t pos = s->tokens;
  try {
    s->blocks.reserve(s->blocks.size() + 1);
  } catch (const std::bad_alloc&) {
    return out_of_memory("pkv_bm_append");
  }
  if (pos % S == 0) {  // the token opens a new block
    if (bm->free_dev.empty()) return fail(PKV_ERR_NO_BLOCKS, "pkv_bm_append: no free block");
    const int32_t b = bm->free_dev.back();
    bm->free_dev.pop_back();
    bm->ref[(size_t)b] = 1;
    s->blocks.push_back(b);
  } else if (bm->ref[(size_t)s->blocks.back()] > 1) {  // shared last block: copy on write
    if (bm->free_dev.empty()) return fail(PKV_ERR_NO_BLOCKS, "pkv_bm_append: no free block for a copy");
    const int32_t b = bm->free_dev.back();
    bm->free_dev.pop_back();
    bm->ref[(size_t)b] = 1;
    *copy_src = s->blocks.back();
    *copy_dst = b;
    --bm->ref[(size_t)s->blocks.back()];
    s->blocks.back() = b;
  }
  *slot = (int64_t)s->blocks.back() * S + pos % S;
  s->tokens = pos + 1;
  return PKV_OK;
}

pkv_status pkv_bm_free(pkv_block_manager* bm, int64_t seq) {
  if (!bm) return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_free: manager is NULL");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_free: sequence %lld unknown", (long long)seq);
  for (int32_t b : it->second.blocks) {
    if (it->second.on_host) bm->free_host.push_back(b);
    else release_device(bm, b);
  }
  bm->seqs.erase(it);
  return PKV_OK;
}

int32_t pkv_bm_num_tokens(const pkv_block_manager* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : it->second.tokens;
}

int32_t pkv_bm_ref_count(const pkv_block_manager* bm, int32_t block) {
  if (!bm || block < 0 || (size_t)block >= bm->ref.size()) return -1;
  return bm->ref[(size_t)block];
}

pkv_status pkv_bm_tables(const pkv_block_manager* bm, const int64_t* seqs, int32_t n,
                         int32_t max_blocks, int32_t* tables, int32_t* context_lens) {
  if (!bm || n < 0 || max_blocks < 0 || (n > 0 && (!seqs || !tables || !context_lens)))
    return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_tables: bad arguments");
  for (int32_t k = 0; k < n; ++k) {
    auto it = bm->seqs.find(seqs[k]);
    if (it == bm->seqs.end() || it->second.on_host)
      return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_tables: sequence %lld unknown or swapped out",
                  (long long)seqs[k]);
    const Seq& s = it->second;
    if ((int64_t)s.blocks.size() > max_blocks)
      return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_tables: sequence %lld holds %zu blocks > %d",
                  (long long)seqs[k], s.blocks.size(), max_blocks);
    int32_t* row = tables + (size_t)k * max_blocks;
    for (int32_t j = 0; j < max_blocks; ++j)
      row[j] = (size_t)j < s.blocks.size() ? s.blocks[(size_t)j] : -1;
    context_lens[k] = s.tokens;
  }
  return PKV_OK;
}

pkv_status pkv_bm_swap_out(pkv_block_manager* bm, int64_t seq, int32_t* pairs, int32_t max_pairs,
                           int32_t* num_pairs) {
  if (!bm || !num_pairs || (max_pairs > 0 && !pairs))
    return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_swap_out: NULL argument");
  Seq* s = find(bm, seq);
  if (!s || s->on_host)
    return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_swap_out: sequence %lld unknown or swapped out", (long long)seq);
  const size_t nb = s->blocks.size();
  if ((size_t)max_pairs < nb)
    return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_swap_out: room for %d pairs, %zu needed", max_pairs, nb);
  if (nb > bm->free_host.size())
    return fail(PKV_ERR_NO_BLOCKS, "pkv_bm_swap_out: %zu host blocks needed, %zu free", nb, bm->free_host.size());
  for (size_t k = 0; k < nb; ++k) {
    const int32_t h = bm->free_host.back();
    bm->free_host.pop_back();
    pairs[2 * k] = s->blocks[k];
    pairs[2 * k + 1] = h;
    release_device(bm, s->blocks[k]);
    s->blocks[k] = h;
  }
  s->on_host = true;
  *num_pairs = (int32_t)nb;
  return PKV_OK;
}

pkv_status pkv_bm_swap_in(pkv_block_manager* bm, int64_t seq, int32_t* pairs, int32_t max_pairs,
                          int32_t* num_pairs) {
  if (!bm || !num_pairs || (max_pairs > 0 && !pairs))
    return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_swap_in: NULL argument");
  Seq* s = find(bm, seq);
  if (!s || !s->on_host)
    return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_swap_in: sequence %lld unknown or not swapped out", (long long)seq);
  const size_t nb = s->blocks.size();
  if ((size_t)max_pairs < nb)
    return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_bm_swap_in: room for %d pairs, %zu needed", max_pairs, nb);
  if (nb > bm->free_dev.size())
    return fail(PKV_ERR_NO_BLOCKS, "pkv_bm_swap_in: %zu blocks needed, %zu free", nb, bm->free_dev.size());
  for (size_t k = 0; k < nb; ++k) {
    const int32_t d = bm->free_dev.back();
    bm->free_dev.pop_back();
    bm->ref[(size_t)d] = 1;
    pairs[2 * k] = s->blocks[k];
    pairs[2 * k + 1] = d;
    bm->free_host.push_back(s->blocks[k]);
    s->blocks[k] = d;
  }
  s->on_host = false;
  *num_pairs = (int32_t)nb;
  return PKV_OK;
}

pkv_status pkv_swap_blocks(const void* src_k, const void* src_v, int32_t num_src_blocks,
                           void* dst_k, void* dst_v, int32_t num_dst_blocks,
                           const int32_t* pairs, int32_t num_pairs, size_t block_bytes,
                           int32_t to_device, void* stream) {
  if (num_pairs < 0 || (num_pairs > 0 && (!src_k || !src_v || !dst_k || !dst_v || !pairs)) ||
      block_bytes == 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_swap_blocks: bad arguments");
  for (int32_t k = 0; k < num_pairs; ++k)
    if (pairs[2 * k] < 0 || pairs[2 * k] >= num_src_blocks || pairs[2 * k + 1] < 0 ||
        pairs[2 * k + 1] >= num_dst_blocks)
      return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_swap_blocks: pair %d (%d, %d) outside the pools", k,
                  pairs[2 * k], pairs[2 * k + 1]);
  const hipMemcpyKind kind = to_device ? hipMemcpyHostToDevice : hipMemcpyDeviceToHost;
  const void* src[2] = {src_k, src_v};
  void* dst[2] = {dst_k, dst_v};
  for (int32_t k = 0; k < num_pairs; ++k) {
    for (int kv = 0; kv < 2; ++kv) {
      const hipError_t e = hipMemcpyAsync(
          static_cast<char*>(dst[kv]) + (size_t)pairs[2 * k + 1] * block_bytes,
          static_cast<const char*>(src[kv]) + (size_t)pairs[2 * k] * block_bytes, block_bytes,
          kind, static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return pkv::hip_failure(e, "pkv_swap_blocks: hipMemcpyAsync");
    }
  }
  return PKV_OK;
}

}  // extern "C"
