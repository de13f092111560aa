// Randomised exercise of the host block manager (pkv_bm_*) against a shadow model of its books,
// built with AddressSanitizer and UndefinedBehaviorSanitizer on the CPU by test_block_manager_sanitized.py:
// every operation (add, append, fork, free, swap out, swap in, tables) is followed by a check that
// token counts, reference counts and free counts match the model, including the refused calls.
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>
#include "pagedkv.h"
struct Sh { int tokens; bool host; };
int main() {
  std::mt19937 rng(7);
  for (int trial = 0; trial < 100; ++trial) {
    const int N = 1 + rng() % 40, NH = rng() % 30, S = (rng() % 2) ? 16 : 32;
    pkv_block_manager* bm = nullptr;
    if (pkv_bm_create(N, NH, S, &bm) != PKV_OK) { printf("create failed\n"); return 1; }
    std::map<long long, Sh> live;
    long long next = 0;
    std::vector<int32_t> pairs(2 * 1024);
    for (int op = 0; op < 2000; ++op) {
      const int kind = rng() % 7;
      auto pick = [&](bool host) -> long long {
        std::vector<long long> c;
        for (auto& kv : live) if (kv.second.host == host) c.push_back(kv.first);
        return c.empty() ? -1 : c[rng() % c.size()];
      };
      if (kind == 0) {
        int n = rng() % (3 * S);
        if (pkv_bm_add(bm, next, n) == PKV_OK) live[next] = {n, false};
        ++next;
      } else if (kind == 1) {
        long long s = pick(false); if (s < 0) continue;
        int64_t slot; int32_t a, b;
        if (pkv_bm_append(bm, s, &slot, &a, &b) == PKV_OK) live[s].tokens++;
      } else if (kind == 2) {
        long long s = pick(false); if (s < 0) continue;
        if (pkv_bm_fork(bm, s, next) == PKV_OK) live[next] = live[s];
        ++next;
      } else if (kind == 3) {
        long long s = pick(rng() % 2); if (s < 0) continue;
        if (pkv_bm_free(bm, s) != PKV_OK) { printf("free failed\n"); return 1; }
        live.erase(s);
      } else if (kind == 4) {
        long long s = pick(false); if (s < 0) continue;
        int32_t n;
        if (pkv_bm_swap_out(bm, s, pairs.data(), 1024, &n) == PKV_OK) live[s].host = true;
      } else if (kind == 5) {
        long long s = pick(true); if (s < 0) continue;
        int32_t n;
        if (pkv_bm_swap_in(bm, s, pairs.data(), 1024, &n) == PKV_OK) live[s].host = false;
      } else {
        std::vector<int64_t> ids;
        for (auto& kv : live) if (!kv.second.host) ids.push_back(kv.first);
        const int MBk = 1 + rng() % 12;
        std::vector<int32_t> t(ids.size() * MBk + 1), l(ids.size() + 1);
        pkv_bm_tables(bm, ids.data(), (int32_t)ids.size(), MBk, t.data(), l.data());
      }
      // books: token counts agree; references = holders; free counts consistent
      std::vector<int> holders(N, 0);
      int host_used = 0;
      for (auto& kv : live) {
        if (pkv_bm_num_tokens(bm, kv.first) != kv.second.tokens) { printf("tokens differ\n"); return 1; }
        const int nb = (kv.second.tokens + S - 1) / S;
        if (kv.second.host) { host_used += nb; continue; }
        std::vector<int32_t> row(64), len(1);
        int64_t id = kv.first;
        if (pkv_bm_tables(bm, &id, 1, 64, row.data(), len.data()) != PKV_OK) { printf("tables\n"); return 1; }
        for (int j = 0; j < nb; ++j) holders[row[j]]++;
      }
      int free_count = 0;
      for (int b = 0; b < N; ++b) {
        if (pkv_bm_ref_count(bm, b) != holders[b]) { printf("ref differs block %d\n", b); return 1; }
        free_count += holders[b] == 0;
      }
      if (pkv_bm_free_blocks(bm) != free_count || pkv_bm_free_host_blocks(bm) != NH - host_used) {
        printf("free counts differ\n"); return 1;
      }
    }
    pkv_bm_destroy(bm);
  }
  printf("fuzz ok\n");
  return 0;
}
