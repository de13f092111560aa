// Virtually contiguous KV pool on HIP virtual memory (pkv_vmm_pool_* in pagedkv.h): address
// space for every sequence's maximum length reserved up front, physical pages mapped as the
// sequence grows. This is the allocator that the table-free decode reads through; the
// decode kernels themselves are unchanged.
#include <stdint.h>
#include <string.h>

#include <new>
#include <vector>

#include <hip/hip_runtime.h>

#include "host_errors.hpp"
#include "pagedkv.h"

struct pkv_vmm_pool {
  int device = 0;
  int32_t num_seqs = 0;
  int32_t block_size = 0;      // positions per block
  int32_t blocks_per_seq = 0;  // MB of the table-free decode addressing
  size_t block_bytes = 0;      // one block of all kv heads, in each of K and V
  size_t page_bytes = 0;
  size_t seq_bytes = 0;        // one sequence's region in each of K and V
  void* base[2] = {nullptr, nullptr};  // K, V
  // pages[kv][seq]: handles of the pages mapped, in order, from the start of the region
  std::vector<std::vector<hipMemGenericAllocationHandle_t>> pages[2];
  size_t mapped = 0;
};

namespace {

using pkv::fail;

size_t elt_size(int dtype) { return dtype == PKV_F32 ? 4 : 2; }

hipMemAllocationProp device_prop(int device) {
  hipMemAllocationProp prop;
  memset(&prop, 0, sizeof prop);
  prop.type = hipMemAllocationTypePinned;
  prop.location.type = hipMemLocationTypeDevice;
  prop.location.id = device;
  return prop;
}

size_t gcd(size_t a, size_t b) {
  while (b) {
    const size_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

char* region(const pkv_vmm_pool* p, int kv, int32_t seq) {
  return static_cast<char*>(p->base[kv]) + (size_t)seq * p->seq_bytes;
}

// Unmaps and releases the pages of one sequence's region past the first `keep`.
pkv_status drop_pages(pkv_vmm_pool* p, int kv, int32_t seq, size_t keep) {
  auto& v = p->pages[kv][seq];
  while (v.size() > keep) {
    char* at = region(p, kv, seq) + (v.size() - 1) * p->page_bytes;
    hipError_t e = hipMemUnmap(at, p->page_bytes);
    if (e != hipSuccess) return pkv::hip_failure(e, "pkv_vmm_pool: hipMemUnmap");
    e = hipMemRelease(v.back());
    if (e != hipSuccess) return pkv::hip_failure(e, "pkv_vmm_pool: hipMemRelease");
    v.pop_back();
    p->mapped -= p->page_bytes;
  }
  return PKV_OK;
}

// Maps pages until one sequence's region has `want` of them, each readable and writable by
// the pool's device. A failure leaves the pages mapped so far in place (they are released
// with the sequence or the pool).
pkv_status add_pages(pkv_vmm_pool* p, int kv, int32_t seq, size_t want) {
  auto& v = p->pages[kv][seq];
  const hipMemAllocationProp prop = device_prop(p->device);
  hipMemAccessDesc access;
  memset(&access, 0, sizeof access);
  access.location.type = hipMemLocationTypeDevice;
  access.location.id = p->device;
  access.flags = hipMemAccessFlagsProtReadWrite;
  try {
    v.reserve(want);  // the only host allocation here, before any page exists
  } catch (const std::bad_alloc&) {
    return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_vmm_pool_map: out of host memory");
  }
  while (v.size() < want) {
    hipMemGenericAllocationHandle_t h;
    hipError_t e = hipMemCreate(&h, p->page_bytes, &prop, 0);
    if (e != hipSuccess) return pkv::hip_failure(e, "pkv_vmm_pool_map: hipMemCreate");
    char* at = region(p, kv, seq) + v.size() * p->page_bytes;
    e = hipMemMap(at, p->page_bytes, 0, h, 0);
    if (e != hipSuccess) {
      (void)hipMemRelease(h);
      return pkv::hip_failure(e, "pkv_vmm_pool_map: hipMemMap");
    }
    e = hipMemSetAccess(at, p->page_bytes, &access, 1);
    if (e != hipSuccess) {
      (void)hipMemUnmap(at, p->page_bytes);
      (void)hipMemRelease(h);
      return pkv::hip_failure(e, "pkv_vmm_pool_map: hipMemSetAccess");
    }
    v.push_back(h);
    p->mapped += p->page_bytes;
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_vmm_pool_create(int32_t num_seqs, int32_t max_context_len, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, pkv_dtype dtype,
                               size_t page_bytes, pkv_vmm_pool** pool) {
  const char* fn = "pkv_vmm_pool_create";
  if (!pool) return fail(PKV_ERR_INVALID_ARGUMENT, "%s: pool is NULL", fn);
  *pool = nullptr;
  const int dt = pkv::enum_arg(dtype);
  if (num_seqs <= 0 || max_context_len <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || (dt != PKV_F32 && dt != PKV_F16 && dt != PKV_BF16))
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: bad shape or dtype", fn);
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return pkv::hip_failure(e, "pkv_vmm_pool_create: hipGetDevice");
  const hipMemAllocationProp prop = device_prop(device);
  size_t min_gran = 0, rec_gran = 0;
  e = hipMemGetAllocationGranularity(&min_gran, &prop, hipMemAllocationGranularityMinimum);
  if (e != hipSuccess) return pkv::hip_failure(e, "pkv_vmm_pool_create: granularity");
  e = hipMemGetAllocationGranularity(&rec_gran, &prop, hipMemAllocationGranularityRecommended);
  if (e != hipSuccess) return pkv::hip_failure(e, "pkv_vmm_pool_create: granularity");
  if (min_gran == 0) return fail(PKV_ERR_UNSUPPORTED, "%s: no virtual memory support", fn);
  const size_t page = page_bytes ? page_bytes : (rec_gran ? rec_gran : min_gran);
  if (page % min_gran)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: page_bytes %zu is not a multiple of %zu", fn,
                page, min_gran);
  const size_t block_bytes = (size_t)num_kv_heads * block_size * head_dim * elt_size(dt);
  // Blocks per sequence: enough for max_context_len, rounded up so that every region is a
  // whole number of pages (a multiple of page / gcd(page, block_bytes) blocks).
  const size_t unit = page / gcd(page, block_bytes);
  size_t mb = ((size_t)max_context_len + block_size - 1) / block_size;
  mb = (mb + unit - 1) / unit * unit;
  if (mb * (size_t)num_seqs > (size_t)INT32_MAX)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: more than 2^31 blocks", fn);
  pkv_vmm_pool* p = new (std::nothrow) pkv_vmm_pool;
  if (!p) return fail(PKV_ERR_INVALID_ARGUMENT, "%s: out of host memory", fn);
  p->device = device;
  p->num_seqs = num_seqs;
  p->block_size = block_size;
  p->blocks_per_seq = (int32_t)mb;
  p->block_bytes = block_bytes;
  p->page_bytes = page;
  p->seq_bytes = mb * block_bytes;
  try {
    for (int kv = 0; kv < 2; ++kv) p->pages[kv].assign(num_seqs, {});
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: out of host memory", fn);
  }
  const size_t total = p->seq_bytes * (size_t)num_seqs;
  for (int kv = 0; kv < 2; ++kv) {
    e = hipMemAddressReserve(&p->base[kv], total, page, nullptr, 0);
    if (e != hipSuccess) {
      p->base[kv] = nullptr;
      const pkv_status st = pkv::hip_failure(e, "pkv_vmm_pool_create: hipMemAddressReserve");
      pkv_vmm_pool_destroy(p);
      return st;
    }
  }
  *pool = p;
  return PKV_OK;
}

pkv_status pkv_vmm_pool_map(pkv_vmm_pool* p, int32_t seq, int32_t num_positions) {
  if (!p || seq < 0 || seq >= p->num_seqs || num_positions < 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_vmm_pool_map: bad pool, sequence or count");
  const size_t blocks = ((size_t)num_positions + p->block_size - 1) / p->block_size;
  if (blocks > (size_t)p->blocks_per_seq)
    return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_vmm_pool_map: %d positions exceed the %d-block region",
                num_positions, p->blocks_per_seq);
  const size_t want = (blocks * p->block_bytes + p->page_bytes - 1) / p->page_bytes;
  for (int kv = 0; kv < 2; ++kv) {
    const pkv_status st = add_pages(p, kv, seq, want);
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

pkv_status pkv_vmm_pool_unmap(pkv_vmm_pool* p, int32_t seq) {
  if (!p || seq < 0 || seq >= p->num_seqs)
    return fail(PKV_ERR_INVALID_ARGUMENT, "pkv_vmm_pool_unmap: bad pool or sequence");
  for (int kv = 0; kv < 2; ++kv) {
    const pkv_status st = drop_pages(p, kv, seq, 0);
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

void pkv_vmm_pool_destroy(pkv_vmm_pool* p) {
  if (!p) return;
  for (int kv = 0; kv < 2; ++kv) {
    for (int32_t s = 0; s < (int32_t)p->pages[kv].size(); ++s) drop_pages(p, kv, s, 0);
    if (p->base[kv]) (void)hipMemAddressFree(p->base[kv], p->seq_bytes * (size_t)p->num_seqs);
  }
  delete p;
}

pkv_status pkv_vmm_pool_copy(pkv_vmm_pool* p, int32_t seq, int32_t num_blocks, void* k,
                             void* v, int32_t to_pool, void* stream) {
  const char* fn = "pkv_vmm_pool_copy";
  if (!p || seq < 0 || seq >= p->num_seqs || num_blocks < 0 || !k || !v)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%s: bad pool, sequence, count or pointer", fn);
  const size_t bytes = (size_t)num_blocks * p->block_bytes;
  for (int kv = 0; kv < 2; ++kv)
    if (bytes > p->pages[kv][seq].size() * p->page_bytes)
      return fail(PKV_ERR_INVALID_ARGUMENT, "%s: %d blocks of sequence %d are not all mapped", fn,
                  num_blocks, seq);
  if (bytes == 0) return PKV_OK;
  void* user[2] = {k, v};
  for (int kv = 0; kv < 2; ++kv) {
    char* pool_at = region(p, kv, seq);
    const hipError_t e =
        to_pool ? hipMemcpyAsync(pool_at, user[kv], bytes, hipMemcpyDeviceToDevice,
                                 static_cast<hipStream_t>(stream))
                : hipMemcpyAsync(user[kv], pool_at, bytes, hipMemcpyDeviceToDevice,
                                 static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return pkv::hip_failure(e, "pkv_vmm_pool_copy: hipMemcpyAsync");
  }
  return PKV_OK;
}

void* pkv_vmm_pool_k(const pkv_vmm_pool* p) { return p ? p->base[0] : nullptr; }
void* pkv_vmm_pool_v(const pkv_vmm_pool* p) { return p ? p->base[1] : nullptr; }
int32_t pkv_vmm_pool_blocks_per_seq(const pkv_vmm_pool* p) { return p ? p->blocks_per_seq : 0; }
size_t pkv_vmm_pool_page_bytes(const pkv_vmm_pool* p) { return p ? p->page_bytes : 0; }
size_t pkv_vmm_pool_mapped_bytes(const pkv_vmm_pool* p) { return p ? p->mapped : 0; }

}  // extern "C"
