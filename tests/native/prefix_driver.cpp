// Test driver for the prefix cache: reads an op trace on stdin, applies it
// through the C interface and prints one result line and one state line per
// op.  Built with AddressSanitizer and UndefinedBehaviorSanitizer by the CPU
// test-suite, which compares its output with the prefix-cache oracle.
#include <cstdio>
#include <iostream>
#include <map>
#include <sstream>
#include <string>
#include <vector>

#include "pkv.h"

int main() {
  pkv_allocator* a = nullptr;
  std::map<int, std::vector<int32_t>> rows;
  const int32_t kCap = 1024;
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string op;
    in >> op;
    if (op == "create") {
      int32_t nb, bs;
      in >> nb >> bs;
      std::vector<int32_t> order(nb);
      for (auto& x : order) in >> x;
      int st = pkv_allocator_create(nb, bs, order.data(), &a);
      if (st == 0) st = pkv_prefix_cache_enable(a);
      std::printf("%d\n", st);
      continue;
    }
    std::vector<int32_t> toks;
    if (op == "match" || op == "register") {
      int sid, cap, n;
      in >> sid >> cap >> n;
      toks.resize(n > 0 ? n : 1);
      for (int i = 0; i < n; ++i) in >> toks[i];
      if (op == "match") {
        std::vector<int32_t> row(kCap, -1);
        int32_t got = -1;
        int st = pkv_prefix_match(a, toks.data(), n, row.data(), cap, &got);
        if (st == 0) {
          row.resize(got);
          rows[sid] = row;
          std::printf("ok");
          for (int32_t b : row) std::printf(" %d", b);
          std::printf("\n");
        } else {
          std::printf("err %d\n", st);
        }
      } else {
        std::vector<int32_t>& row = rows[sid];
        int32_t added = -1;
        // for register the second number is first_block
        int st = pkv_prefix_register(a, toks.data(), n, row.data(), static_cast<int32_t>(row.size()), cap, &added);
        if (st == 0) std::printf("ok %d\n", added); else std::printf("err %d\n", st);
      }
    } else if (op == "reserve") {
      int sid, cur, n;
      in >> sid >> cur >> n;
      std::vector<int32_t>& row = rows[sid];
      std::vector<int32_t> buf(kCap, -1);
      for (size_t i = 0; i < row.size(); ++i) buf[i] = row[i];
      int32_t nb = static_cast<int32_t>(row.size());
      std::vector<int64_t> slots(n > 0 ? n : 1);
      int32_t pair[2] = {-1, -1}, ncow = 0;
      int st = pkv_seq_reserve(a, buf.data(), kCap, &nb, cur, n, slots.data(), pair, &ncow);
      if (st == 0) {
        row.assign(buf.begin(), buf.begin() + nb);
        std::printf("ok");
        for (int i = 0; i < n; ++i) std::printf(" %lld", static_cast<long long>(slots[i]));
        std::printf("\n");
      } else {
        std::printf("err %d\n", st);
      }
    } else if (op == "release") {
      int sid;
      in >> sid;
      std::vector<int32_t>& row = rows[sid];
      int st = pkv_seq_release(a, row.empty() ? nullptr : row.data(), static_cast<int32_t>(row.size()));
      if (st == 0) rows.erase(sid);
      std::printf(st == 0 ? "ok\n" : "err %d\n", st);
    }
    const int32_t nb = pkv_num_blocks(a);
    std::vector<int32_t> buf(nb > 0 ? nb : 1);
    int n = pkv_free_list(a, buf.data(), nb);
    std::printf("free");
    for (int i = 0; i < n; ++i) std::printf(" %d", buf[i]);
    n = pkv_prefix_lru(a, buf.data(), nb);
    std::printf(" | lru");
    for (int i = 0; i < n; ++i) std::printf(" %d", buf[i]);
    std::printf(" | cached %d | ref", pkv_prefix_cached_blocks(a));
    for (int32_t b = 0; b < nb; ++b) std::printf(" %d", pkv_block_refcount(a, b));
    std::printf("\n");
  }
  pkv_allocator_destroy(a);
  return 0;
}
