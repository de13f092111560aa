// Randomised exercise of the virtual-memory pool (pkv_vmm_pool_* in vmm.cpp) on the CPU, built
// with AddressSanitizer and UndefinedBehaviorSanitizer by test_host_sanitized.py. The HIP virtual
// memory calls the pool makes are replaced by a host model of an address space: reservations,
// physical allocations and mappings are kept in tables, and every call is checked against them
// (a mapping must lie inside a reservation and overlap no other, only whole mappings are
// unmapped, a copy touches mapped and accessible pages only, a reservation is freed only when
// nothing in it is mapped). Calls can be made to fail on request, so that the pool's error
// paths run too. After every pool call the bytes the pool reports as mapped must equal what the
// model holds, and after every destroy nothing may be left reserved, mapped or allocated.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "pagedkv.h"

struct ihipMemGenericAllocationHandle {
  size_t size;
  int mapped;
};

namespace {

struct Mapping {
  size_t size;
  hipMemGenericAllocationHandle_t h;
  bool access;
};

size_t g_min_gran = 4096, g_rec_gran = 2 << 20;
uintptr_t g_next_va = (uintptr_t)1 << 44;
std::map<uintptr_t, size_t> g_reserved;   // base -> bytes
std::map<uintptr_t, Mapping> g_mapped;    // address -> mapping
std::set<hipMemGenericAllocationHandle_t> g_handles;
int g_fail_in = -1;  // the g_fail_in-th fallible call from now fails (-1: none)
bool g_fired = false;  // an injected failure happened
int g_violations = 0;

#define CHECK(cond, ...)                         \
  do {                                           \
    if (!(cond)) {                               \
      printf("model violation: " __VA_ARGS__);   \
      printf("\n");                              \
      ++g_violations;                            \
    }                                            \
  } while (0)

bool inject() {
  if (g_fail_in < 0) return false;
  if (g_fail_in-- == 0) return g_fired = true;
  return false;
}

bool in_reservation(uintptr_t a, size_t n) {
  auto it = g_reserved.upper_bound(a);
  if (it == g_reserved.begin()) return false;
  --it;
  return a >= it->first && a + n <= it->first + it->second;
}

// Bytes of [a, a + n) covered by accessible mappings.
bool covered(uintptr_t a, size_t n) {
  while (n > 0) {
    auto it = g_mapped.upper_bound(a);
    if (it == g_mapped.begin()) return false;
    --it;
    if (a >= it->first + it->second.size || !it->second.access) return false;
    const size_t take = std::min(n, (size_t)(it->first + it->second.size - a));
    a += take;
    n -= take;
  }
  return true;
}

size_t mapped_in(uintptr_t base, size_t bytes) {
  size_t s = 0;
  for (auto& m : g_mapped)
    if (m.first >= base && m.first < base + bytes) s += m.second.size;
  return s;
}

}  // namespace

extern "C" {

hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}

hipError_t hipMemGetAllocationGranularity(size_t* g, const hipMemAllocationProp* prop,
                                          hipMemAllocationGranularity_flags option) {
  CHECK(prop && prop->location.id == 0, "granularity query for another device");
  *g = option == hipMemAllocationGranularityMinimum ? g_min_gran : g_rec_gran;
  return hipSuccess;
}

hipError_t hipMemAddressReserve(void** ptr, size_t size, size_t alignment, void*,
                                unsigned long long) {
  if (inject()) return hipErrorOutOfMemory;
  CHECK(size > 0 && alignment > 0 && size % g_min_gran == 0, "reserve of %zu bytes", size);
  const size_t al = alignment ? alignment : g_min_gran;
  g_next_va = (g_next_va + al - 1) / al * al;
  *ptr = (void*)g_next_va;
  g_reserved[g_next_va] = size;
  g_next_va += size + al;  // a gap between reservations
  return hipSuccess;
}

hipError_t hipMemAddressFree(void* p, size_t size) {
  auto it = g_reserved.find((uintptr_t)p);
  CHECK(it != g_reserved.end() && it->second == size, "free of an unreserved range");
  if (it == g_reserved.end()) return hipErrorInvalidValue;
  CHECK(mapped_in(it->first, it->second) == 0, "free of a range with mappings");
  g_reserved.erase(it);
  return hipSuccess;
}

hipError_t hipMemCreate(hipMemGenericAllocationHandle_t* h, size_t size,
                        const hipMemAllocationProp* prop, unsigned long long) {
  if (inject()) return hipErrorOutOfMemory;
  CHECK(prop && prop->type == hipMemAllocationTypePinned &&
            prop->location.type == hipMemLocationTypeDevice && size % g_min_gran == 0 && size,
        "create of %zu bytes", size);
  *h = new ihipMemGenericAllocationHandle{size, 0};
  g_handles.insert(*h);
  return hipSuccess;
}

hipError_t hipMemRelease(hipMemGenericAllocationHandle_t h) {
  CHECK(g_handles.count(h), "release of an unknown handle");
  if (!g_handles.count(h)) return hipErrorInvalidValue;
  CHECK(!h->mapped, "release of a mapped handle");
  g_handles.erase(h);
  delete h;
  return hipSuccess;
}

hipError_t hipMemMap(void* p, size_t size, size_t offset, hipMemGenericAllocationHandle_t h,
                     unsigned long long) {
  if (inject()) return hipErrorOutOfMemory;
  const uintptr_t a = (uintptr_t)p;
  CHECK(g_handles.count(h) && !h->mapped && h->size == size && offset == 0,
        "map of a bad handle");
  CHECK(a % g_min_gran == 0 && in_reservation(a, size), "map outside a reservation");
  auto next = g_mapped.lower_bound(a);
  CHECK(next == g_mapped.end() || next->first >= a + size, "overlapping map");
  if (next != g_mapped.begin()) {
    auto prev = std::prev(next);
    CHECK(prev->first + prev->second.size <= a, "overlapping map");
  }
  g_mapped[a] = {size, h, false};
  h->mapped = 1;
  return hipSuccess;
}

hipError_t hipMemSetAccess(void* p, size_t size, const hipMemAccessDesc* desc, size_t count) {
  if (inject()) return hipErrorOutOfMemory;
  auto it = g_mapped.find((uintptr_t)p);
  CHECK(it != g_mapped.end() && it->second.size == size, "access on an unmapped range");
  CHECK(desc && count == 1 && desc->flags == hipMemAccessFlagsProtReadWrite, "access flags");
  if (it != g_mapped.end()) it->second.access = true;
  return hipSuccess;
}

hipError_t hipMemUnmap(void* p, size_t size) {
  auto it = g_mapped.find((uintptr_t)p);
  CHECK(it != g_mapped.end() && it->second.size == size, "unmap of a range that is not a mapping");
  if (it == g_mapped.end()) return hipErrorInvalidValue;
  it->second.h->mapped = 0;
  g_mapped.erase(it);
  return hipSuccess;
}

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind kind,
                          hipStream_t) {
  CHECK(kind == hipMemcpyDeviceToDevice, "copy kind");
  const uintptr_t d = (uintptr_t)dst, s = (uintptr_t)src;
  const bool dp = in_reservation(d, 1), sp = in_reservation(s, 1);
  CHECK(dp != sp, "a copy must have exactly one side in the pool");
  const uintptr_t pool = dp ? d : s;
  CHECK(covered(pool, bytes), "copy touches unmapped pool bytes");
  return hipSuccess;
}

}  // extern "C"

int main() {
  std::mt19937 rng(11);
  const pkv_dtype dts[3] = {PKV_F32, PKV_F16, PKV_BF16};
  int created = 0, failed_calls = 0;
  for (int trial = 0; trial < 400; ++trial) {
    g_min_gran = (rng() % 2) ? 4096 : 65536;
    g_rec_gran = (rng() % 2) ? g_min_gran : (size_t)2 << 20;
    const int B = 1 + rng() % 6, maxlen = 1 + rng() % 3000, Hkv = 1 + rng() % 8;
    const int D = (rng() % 2) ? 64 : 128, S = 16 << (rng() % 3);
    const pkv_dtype dt = dts[rng() % 3];
    const size_t page = (rng() % 3) ? 0 : g_min_gran * (1 + rng() % 16);
    if (rng() % 10 == 0) g_fail_in = 0;  // the reservation itself fails
    pkv_vmm_pool* p = nullptr;
    pkv_status st = pkv_vmm_pool_create(B, maxlen, Hkv, D, S, dt, page, &p);
    g_fail_in = -1;
    if (st != PKV_OK) {
      CHECK(p == nullptr && g_reserved.empty() && g_handles.empty(), "failed create left state");
      ++failed_calls;
      continue;
    }
    ++created;
    const size_t pg = pkv_vmm_pool_page_bytes(p);
    const int MB = pkv_vmm_pool_blocks_per_seq(p);
    const size_t block = (size_t)Hkv * S * D * (dt == PKV_F32 ? 4 : 2);
    CHECK((size_t)MB * S >= (size_t)maxlen, "region holds fewer than max_context_len positions");
    CHECK((size_t)MB * block % pg == 0, "region is not whole pages");
    CHECK(pg % g_min_gran == 0 && (page == 0 || pg == page), "page size");
    std::vector<size_t> pages[2] = {std::vector<size_t>(B, 0), std::vector<size_t>(B, 0)};
    const uintptr_t kb = (uintptr_t)pkv_vmm_pool_k(p), vb = (uintptr_t)pkv_vmm_pool_v(p);
    const size_t region = (size_t)MB * block * B;
    for (int op = 0; op < 200; ++op) {
      const int kind = rng() % 10, seq = (int)(rng() % (B + 1)) - (rng() % 8 == 0);
      const bool valid_seq = seq >= 0 && seq < B;
      if (kind < 5) {  // map
        const int n = (rng() % 12 == 0) ? MB * S + 1 + rng() % 50 : rng() % (MB * S + 1);
        if (rng() % 6 == 0) g_fail_in = rng() % 8;
        g_fired = false;
        st = pkv_vmm_pool_map(p, seq, n);
        g_fail_in = -1;
        const size_t blocks = ((size_t)n + S - 1) / S;
        if (!valid_seq || blocks > (size_t)MB) {
          CHECK(st == PKV_ERR_INVALID_ARGUMENT, "map(%d, %d) accepted", seq, n);
        } else if (st == PKV_OK) {
          for (int kv = 0; kv < 2; ++kv)
            pages[kv][seq] = std::max(pages[kv][seq], (blocks * block + pg - 1) / pg);
        } else {
          CHECK(g_fired && st == PKV_ERR_HIP, "map failed without an injected failure");
          ++failed_calls;
          // the pages mapped before the failure stay mapped (released with the sequence)
          pages[0][seq] = mapped_in(kb + (size_t)seq * MB * block, (size_t)MB * block) / pg;
          pages[1][seq] = mapped_in(vb + (size_t)seq * MB * block, (size_t)MB * block) / pg;
        }
      } else if (kind < 7) {  // unmap
        st = pkv_vmm_pool_unmap(p, seq);
        CHECK((st == PKV_OK) == valid_seq, "unmap(%d) status %d", seq, (int)st);
        if (valid_seq) pages[0][seq] = pages[1][seq] = 0;
      } else {  // copy in or out
        const int nb = (int)(rng() % (MB + 2)) - (rng() % 10 == 0);
        char dummy[16];
        st = pkv_vmm_pool_copy(p, seq, nb, dummy, dummy + 8, rng() % 2, nullptr);
        const size_t kmapped = valid_seq ? mapped_in(kb + (size_t)seq * MB * block,
                                                     (size_t)MB * block) : 0;
        const size_t vmapped = valid_seq ? mapped_in(vb + (size_t)seq * MB * block,
                                                     (size_t)MB * block) : 0;
        const bool ok = valid_seq && nb >= 0 && (size_t)nb * block <= std::min(kmapped, vmapped);
        CHECK((st == PKV_OK) == ok, "copy(%d, %d) status %d", seq, nb, (int)st);
      }
      size_t total = 0;
      for (int s = 0; s < B; ++s) total += (pages[0][s] + pages[1][s]) * pg;
      CHECK(pkv_vmm_pool_mapped_bytes(p) == total, "pool reports %zu mapped bytes, model %zu",
            pkv_vmm_pool_mapped_bytes(p), total);
      CHECK(mapped_in(kb, region) + mapped_in(vb, region) == total,
            "address space holds %zu mapped bytes, model %zu",
            mapped_in(kb, region) + mapped_in(vb, region), total);
    }
    pkv_vmm_pool_destroy(p);
    CHECK(g_reserved.empty() && g_mapped.empty() && g_handles.empty(),
          "destroy left %zu reservations, %zu mappings, %zu allocations", g_reserved.size(),
          g_mapped.size(), g_handles.size());
  }
  // invalid arguments: nothing reserved, nothing allocated
  pkv_vmm_pool* p = nullptr;
  CHECK(pkv_vmm_pool_create(0, 64, 8, 128, 16, PKV_BF16, 0, &p) == PKV_ERR_INVALID_ARGUMENT, "");
  CHECK(pkv_vmm_pool_create(4, 64, 8, 128, 16, (pkv_dtype)7, 0, &p) == PKV_ERR_INVALID_ARGUMENT, "");
  g_min_gran = 65536;
  CHECK(pkv_vmm_pool_create(4, 64, 8, 128, 16, PKV_BF16, 4096, &p) == PKV_ERR_INVALID_ARGUMENT,
        "page smaller than the granularity accepted");
  CHECK(pkv_vmm_pool_create(1 << 20, 1 << 30, 8, 128, 16, PKV_BF16, 0, &p) == PKV_ERR_INVALID_ARGUMENT,
        "more than 2^31 blocks accepted");
  CHECK(p == nullptr && g_reserved.empty() && g_handles.empty(), "invalid create left state");
  printf("pools %d, refused or failed calls %d, violations %d\n", created, failed_calls,
         g_violations);
  if (g_violations == 0 && created > 100 && failed_calls > 10) {
    printf("vmm fuzz ok\n");
    return 0;
  }
  return 1;
}
