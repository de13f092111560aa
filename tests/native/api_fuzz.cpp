// Randomised exercise of the C ABI's host side (api.cpp: argument validation, kernel-family
// choice, grid sizing) on the CPU, built with AddressSanitizer and UndefinedBehaviorSanitizer
// for the host by test_host_sanitized.py. The kernel launchers are replaced by stubs that record
// each launch and check what the validated call hands to the kernels: a positive unit count
// whose grid fits in 32 bits, the block size and head dimension of a real instantiation, the
// workspace exactly in split-context mode, the work list's length, and so on. Arguments are
// drawn from valid values, edge values and invalid ones (negative, zero, huge, null, misaligned,
// enum values outside their enumerators). A call that returns an error must have launched
// nothing and left a message; a call that succeeds must have launched at most once.
#include <climits>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "kernels.hpp"
#include "pagedkv.h"
#include "prefill.hpp"

namespace {

int g_launches = 0;
int g_violations = 0;

#define CHECK(cond, ...)                         \
  do {                                           \
    if (!(cond)) {                               \
      printf("violation: " __VA_ARGS__);         \
      printf("\n");                              \
      ++g_violations;                            \
    }                                            \
  } while (0)

bool valid_dt(pkv::Dt dt) {
  const int v = static_cast<int>(dt);
  return v == 0 || v == 1 || v == 2;
}

void check_decode(const char* what, pkv::Dt dt, int head_dim, int S, const pkv::DecodeParams& p,
                  bool partial, bool may_be_empty = false) {
  CHECK(valid_dt(dt) && (head_dim == 64 || head_dim == 128), "%s: dtype/head_dim", what);
  CHECK(S == 16 || S == 32 || S == 64 || S == 128 || S == 256, "%s: block size %d", what, S);
  CHECK((p.num_units > 0 || (may_be_empty && p.num_units == 0)) && p.num_seqs > 0 &&
            p.num_kv_heads > 0 && p.num_heads > 0,
        "%s: empty launch (units %d seqs %d)", what, p.num_units, p.num_seqs);
  CHECK(((int64_t)p.num_units + 15) / 8 * 8 * p.num_kv_heads <= INT32_MAX, "%s: grid", what);
  const int G = p.num_heads / p.num_kv_heads;
  CHECK(p.num_heads % p.num_kv_heads == 0 && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16),
        "%s: group %d", what, G);
  CHECK(p.num_blocks > 0 && p.max_blocks_per_seq > 0 && p.range_tokens > 0 && p.num_ranges > 0,
        "%s: sizes", what);
  CHECK((int64_t)p.num_seqs * p.num_ranges <= INT32_MAX, "%s: unit space", what);
  CHECK(p.q && p.k_cache && p.v_cache && p.context_lens, "%s: null tensor", what);
  CHECK(partial == (p.max_logits != nullptr) && partial == (p.exp_sums != nullptr) &&
            partial == (p.tmp_out != nullptr) && (partial || p.out),
        "%s: workspace in the wrong mode", what);
  CHECK(!partial || p.range_tokens % S == 0, "%s: partition not whole blocks", what);
  CHECK(p.work_items || p.group_members || p.num_units == p.num_seqs * p.num_ranges,
        "%s: units %d without a work list", what, p.num_units);
  CHECK((p.new_key == nullptr) == (p.new_value == nullptr), "%s: new rows", what);
  CHECK(!p.block_tables ? (int64_t)p.num_seqs * p.max_blocks_per_seq <= p.num_blocks : true,
        "%s: table-free pool too small", what);
}

}  // namespace

namespace pkv {

template <int S>
hipError_t launch_decode_valu_bs(Dt dt, int head_dim, int group, bool partial, bool,
                                 const DecodeParams& p, hipStream_t) {
  ++g_launches;
  check_decode("valu", dt, head_dim, S, p, partial);
  CHECK(group <= 8 && group == p.num_heads / p.num_kv_heads && p.block_tables,
        "valu: group %d or table-free", group);
  CHECK(!p.group_members, "valu: groups");
  return hipSuccess;
}

template <int S>
hipError_t launch_decode_mfma_bs(Dt dt, int head_dim, bool partial, bool, const DecodeParams& p,
                                 hipStream_t) {
  ++g_launches;
  check_decode("mfma", dt, head_dim, S, p, partial);
  CHECK(dt != Dt::F32, "mfma: fp32");
  CHECK(!p.group_members || (partial && p.block_tables && !p.work_items && !p.new_key),
        "mfma: grouped launch");
  return hipSuccess;
}

template <int S>
hipError_t launch_decode_mfma_shared_bs(Dt dt, int head_dim, const DecodeParams& grp,
                                        const DecodeParams& rest, hipStream_t) {
  ++g_launches;
  // no groups at all is allowed here: every piece of the grid is then a listed unit
  check_decode("shared groups", dt, head_dim, S, grp, true, true);
  check_decode("shared rest", dt, head_dim, S, rest, true);
  CHECK(grp.group_members && !grp.work_items && !grp.new_key, "shared: group part");
  CHECK(!rest.group_members && rest.work_items, "shared: listed part");
  return hipSuccess;
}

#define STUB_BS(S)                                                                             \
  template hipError_t launch_decode_valu_bs<S>(Dt, int, int, bool, bool, const DecodeParams&, \
                                               hipStream_t);                                  \
  template hipError_t launch_decode_mfma_bs<S>(Dt, int, bool, bool, const DecodeParams&,      \
                                               hipStream_t);                                  \
  template hipError_t launch_decode_mfma_shared_bs<S>(Dt, int, const DecodeParams&,           \
                                                      const DecodeParams&, hipStream_t);
STUB_BS(16)
STUB_BS(32)
STUB_BS(64)
STUB_BS(128)
STUB_BS(256)
#undef STUB_BS

hipError_t launch_reduce(Dt dt, int head_dim, const ReduceParams& p, hipStream_t) {
  ++g_launches;
  CHECK(valid_dt(dt) && (head_dim == 64 || head_dim == 128), "reduce: dtype/head_dim");
  CHECK(p.num_seqs > 0 && p.num_heads > 0 && p.partition_size > 0 && p.max_num_partitions >= 0,
        "reduce: sizes");
  CHECK((int64_t)p.num_seqs * p.num_heads <= INT32_MAX, "reduce: grid");
  CHECK(p.out && p.context_lens && (p.max_num_partitions == 0 ||
                                    (p.max_logits && p.exp_sums && p.tmp_out)),
        "reduce: pointers");
  return hipSuccess;
}

hipError_t launch_reshape_and_cache(Dt dt, int head_dim, int block_size,
                                    const CacheWriteParams& p, hipStream_t) {
  ++g_launches;
  CHECK(valid_dt(dt) && (head_dim == 64 || head_dim == 128), "cache write: dtype/head_dim");
  CHECK(block_size == 16 || block_size == 32 || block_size == 64 || block_size == 128 ||
            block_size == 256, "cache write: block size");
  CHECK(p.num_tokens > 0 && p.num_kv_heads > 0 && p.num_blocks > 0, "cache write: sizes");
  CHECK(p.key && p.value && p.k_cache && p.v_cache && p.slot_mapping, "cache write: pointers");
  return hipSuccess;
}

hipError_t launch_copy_blocks(int num_layers, const CopyParams& p, hipStream_t) {
  ++g_launches;
  CHECK(num_layers >= 1 && num_layers <= kMaxLayersPerLaunch, "copy: %d layers", num_layers);
  for (int l = 0; l < num_layers && l < kMaxLayersPerLaunch; ++l)
    CHECK(p.k[l] && p.v[l], "copy: layer %d null", l);
  CHECK(p.num_pairs > 0 && p.num_blocks > 0 && p.tile_bytes > 0 && p.block_mapping,
        "copy: sizes");
  return hipSuccess;
}

hipError_t launch_v_layout(Dt dt, bool, const VLayoutParams& p, hipStream_t) {
  ++g_launches;
  CHECK(valid_dt(dt) && (p.head_dim == 64 || p.head_dim == 128), "v layout: dtype/head_dim");
  CHECK(p.group == 16 || p.group == 32, "v layout: group %d", p.group);
  CHECK(p.num_groups > 0 && p.src && p.dst, "v layout: sizes");
  const int64_t bytes = p.num_groups * p.group * p.head_dim * (dt == Dt::F32 ? 4 : 2);
  const uintptr_t s = (uintptr_t)p.src, d = (uintptr_t)p.dst;
  CHECK(s == d || s + bytes <= d || d + bytes <= s, "v layout: overlapping pools");
  return hipSuccess;
}

hipError_t launch_prefill(Dt dt, int head_dim, int block_size, const PrefillParams& p,
                          hipStream_t) {
  ++g_launches;
  CHECK((dt == Dt::F16 || dt == Dt::BF16) && (head_dim == 64 || head_dim == 128),
        "prefill: dtype/head_dim");
  CHECK(block_size == 16 || block_size == 32 || block_size == 64 || block_size == 128 ||
            block_size == 256, "prefill: block size");
  CHECK(p.num_units > 0 && p.num_tiles > 0 && p.num_seqs > 0 && p.num_kv_heads > 0,
        "prefill: sizes");
  CHECK((int64_t)p.num_units * p.num_kv_heads <= INT32_MAX, "prefill: grid");
  CHECK(p.work_items || (int64_t)p.num_units == (int64_t)p.num_seqs * p.num_tiles,
        "prefill: units without a work list");
  CHECK(p.out && p.q && p.k_cache && p.v_cache && p.block_tables && p.context_lens &&
            p.query_start, "prefill: pointers");
  return hipSuccess;
}

}  // namespace pkv

namespace {

std::mt19937 rng(5);

int32_t pick_int(std::initializer_list<int32_t> good) {
  static const int32_t edge[] = {0, -1, 1, 2, 3, 7, 15, 16, 17, 31, 32, 48, 63, 64, 65, 96, 127,
                                 128, 129, 255, 256, 512, 1000, 4096, 65536, 1 << 20,
                                 INT32_MAX / 2, INT32_MAX - 1, INT32_MAX, INT32_MIN, -16};
  if (rng() % 3 == 0) return edge[rng() % (sizeof edge / sizeof edge[0])];
  return good.begin()[rng() % good.size()];
}

// Device-like addresses: aligned, misaligned or null. Never dereferenced by the host code.
void* pick_ptr(int align = 16) {
  const uint32_t r = rng() % 20;
  if (r == 0) return nullptr;
  if (r == 1) return (void*)(uintptr_t)(0x100000 + 2);
  if (r == 2) return (void*)(uintptr_t)(0x100000 + 4);
  if (r == 3) return (void*)(uintptr_t)(0x100000 + 8);
  return (void*)(uintptr_t)(0x100000 + align * (rng() % 1024));
}

template <class E>
E pick_enum(int lo, int hi) {
  int v = (rng() % 8 == 0) ? (int)(rng() % 20) - 5 : lo + (int)(rng() % (hi - lo + 1));
  E e;
  static_assert(sizeof(E) == sizeof(int), "C enum");
  memcpy(&e, &v, sizeof v);  // a C caller may pass any int
  return e;
}

void after(const char* fn, pkv_status st, int launches_before, int max_launches = 1) {
  const int n = g_launches - launches_before;
  if (st != PKV_OK) {
    CHECK(n == 0, "%s: failed with status %d after %d launches", fn, (int)st, n);
    CHECK(pkv_last_error_message() && pkv_last_error_message()[0], "%s: no message", fn);
    CHECK(st == PKV_ERR_INVALID_ARGUMENT || st == PKV_ERR_UNSUPPORTED, "%s: status %d", fn,
          (int)st);
  } else {
    CHECK(n <= max_launches, "%s: %d launches", fn, n);
  }
}

}  // namespace

int main() {
  int ok = 0, refused = 0;
  for (int it = 0; it < 60000; ++it) {
    const int before = g_launches;
    const int which = rng() % 8;
    pkv_status st;
    const char* fn = "";
    const int32_t B = pick_int({1, 2, 4, 9, 128}), H = pick_int({4, 8, 32, 64}),
                  Hkv = pick_int({1, 2, 4, 8, 32}), D = pick_int({64, 128}),
                  S = pick_int({16, 32, 64, 128, 256}), N = pick_int({32, 1024, 32768}),
                  MB = pick_int({4, 64, 256, 1024}), maxlen = pick_int({0, 1, 64, 4096, 32768}),
                  P = pick_int({0, 32, 512, 2048}), nitems = pick_int({0, 3, 128, 4096});
    const float scale = (rng() % 20 == 0) ? 1.0f / 0.0f : 0.088f;
    const pkv_dtype dt = pick_enum<pkv_dtype>(0, 2);
    void* items = (rng() % 2) ? pick_ptr(4) : nullptr;
    void *ml = nullptr, *es = nullptr, *to = nullptr;
    if (P > 0 || rng() % 8 == 0) {
      ml = pick_ptr(4);
      es = pick_ptr(4);
      to = pick_ptr(16);
    }
    if (which == 0 || which == 1) {
      const uint32_t flags = (rng() % 10 == 0) ? 4u : (uint32_t)(rng() % 2);
      pkv_decode_options opt = {pick_enum<pkv_kernel>(0, 2), flags,
                                (rng() % 3 == 0) ? pick_ptr() : nullptr, nullptr};
      if (opt.new_key && rng() % 5) opt.new_value = pick_ptr();
      void* bt = (rng() % 6 == 0) ? nullptr : pick_ptr(4);
      fn = "decode_ex";
      st = pkv_paged_attention_decode_ex(which ? &opt : nullptr, pick_ptr(), pick_ptr(), pick_ptr(),
                                         pick_ptr(), (const int32_t*)bt, MB,
                                         (const int32_t*)pick_ptr(4), (const int32_t*)items,
                                         nitems, maxlen, B, H, Hkv, D, S, N, scale, dt, P,
                                         (float*)ml, (float*)es, (float*)to, nullptr);
    } else if (which == 2) {
      fn = "decode_shared";
      const int32_t ng = pick_int({0, 1, 64});
      void* nk = (rng() % 3 == 0) ? pick_ptr() : nullptr;
      void* nv = nk && rng() % 5 ? pick_ptr() : nullptr;
      st = pkv_paged_attention_decode_shared(
          pick_ptr(), pick_ptr(), pick_ptr(), (const int32_t*)pick_ptr(4), MB,
          (const int32_t*)pick_ptr(4), (const int32_t*)((rng() % 10) ? pick_ptr(16) : nullptr),
          ng, (const int32_t*)items, nitems, nk, nv, maxlen, B, H, Hkv, D, S, N, scale, dt, P,
          (float*)ml, (float*)es, (float*)to, nullptr);
    } else if (which == 3) {
      fn = "reduce";
      st = pkv_paged_attention_reduce(pick_ptr(), (const float*)ml, (const float*)es,
                                      (const float*)to, (const int32_t*)pick_ptr(4), B, H, D, P,
                                      pick_int({0, 1, 61, 64}), dt, nullptr);
    } else if (which == 4) {
      fn = "reshape_and_cache";
      st = pkv_reshape_and_cache(pick_ptr(), pick_ptr(), pick_ptr(), pick_ptr(),
                                 (const int64_t*)pick_ptr(8), pick_int({0, 1, 128}), Hkv, D, S,
                                 N, dt, nullptr);
    } else if (which == 5) {
      fn = "copy_blocks";
      const int layers = (int)(rng() % 70) - (rng() % 10 == 0);
      std::vector<void*> ks(layers > 0 ? layers : 1), vs(layers > 0 ? layers : 1);
      for (auto& k : ks) k = pick_ptr();
      for (auto& v : vs) v = pick_ptr();
      if (rng() % 2)  // mostly well-formed layer arrays
        for (int l = 0; l < (int)ks.size(); ++l) ks[l] = vs[l] = (void*)(uintptr_t)(0x100000 + 16 * l);
      st = pkv_copy_blocks(rng() % 20 ? ks.data() : nullptr, vs.data(), layers,
                           (const int64_t*)pick_ptr(8), pick_int({0, 1, 64}), Hkv, D, S, N, dt,
                           nullptr);
      after(fn, st, before, layers / 32 + 1);
      (st == PKV_OK ? ok : refused)++;
      continue;
    } else if (which == 6) {
      fn = "v_layout";
      void* src = pick_ptr();
      const int r = (int)(rng() % 4);  // the same pool, a near one (overlapping) or a far one
      void* dst = r == 0 ? src : (void*)((uintptr_t)src + (r == 1 ? 4096 : ((uintptr_t)1 << 40)));
      if (rng() % 2)
        st = pkv_v_cache_from_rows(src, dst, pick_int({-1, 0, 1, 32768}), Hkv, D, S, dt, nullptr);
      else
        st = pkv_v_cache_to_rows(src, dst, pick_int({-1, 0, 1, 32768}), Hkv, D, S, dt, nullptr);
    } else {
      fn = "prefill";
      st = pkv_paged_attention_prefill(pick_ptr(), pick_ptr(), pick_ptr(), pick_ptr(),
                                       (const int32_t*)pick_ptr(4), MB,
                                       (const int32_t*)pick_ptr(4), (const int32_t*)pick_ptr(4),
                                       pick_int({0, 1, 512, 4096}), (const int32_t*)items,
                                       nitems, B, pick_int({0, 100, 8192}), H, Hkv, D, S, N,
                                       scale, dt, nullptr);
    }
    after(fn, st, before);
    (st == PKV_OK ? ok : refused)++;
  }
  // status strings take any int
  for (int v = -3; v < 8; ++v) {
    pkv_status s;
    memcpy(&s, &v, sizeof v);
    CHECK(pkv_status_string(s) != nullptr, "status string %d", v);
  }
  CHECK(pkv_partition_workspace_bytes(INT32_MAX, INT32_MAX, 128, INT32_MAX, 1) == SIZE_MAX,
        "workspace size of the largest shape saturates");
  CHECK(pkv_partition_workspace_bytes(32, 64, 128, 30785, 512) == (size_t)4 * 32 * 64 * 61 * 130,
        "workspace size");
  printf("calls accepted %d, refused %d, launches %d, violations %d\n", ok, refused, g_launches,
         g_violations);
  if (g_violations == 0 && ok > 1000 && refused > 1000 && g_launches > 500) {
    printf("api fuzz ok\n");
    return 0;
  }
  return 1;
}
