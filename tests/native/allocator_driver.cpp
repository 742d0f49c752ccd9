// Test driver for the host allocator: reads an op trace on stdin, applies it
// through the C interface and prints one result line per op.  Built with
// AddressSanitizer and UndefinedBehaviorSanitizer by the CPU test-suite.
#include <cstdio>
#include <cstring>
#include <iostream>
#include <map>
#include <sstream>
#include <string>
#include <vector>

#include "pkv.h"

int main() {
  pkv_allocator* a = nullptr;
  std::map<int, std::vector<int32_t>> rows;  // sequence id -> row (capacity-sized)
  std::map<int, int32_t> nblk;
  const int32_t kCap = 4096;
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
      std::printf("%d\n", st);
    } else if (op == "alloc") {
      int32_t b = -1;
      int st = pkv_block_alloc(a, &b);
      std::printf(st == 0 ? "ok %d\n" : "err %d\n", st == 0 ? b : st);
    } else if (op == "incref" || op == "decref") {
      int32_t b;
      in >> b;
      int st = op == "incref" ? pkv_block_incref(a, b) : pkv_block_decref(a, b);
      std::printf(st == 0 ? "ok\n" : "err %d\n", st);
    } else if (op == "fork") {
      int src, dst;
      in >> src >> dst;
      std::vector<int32_t> row(kCap, -1);
      int st = pkv_seq_fork(a, rows[src].data(), nblk[src], row.data());
      if (st == 0) {
        rows[dst] = row;
        nblk[dst] = nblk[src];
        std::printf("ok\n");
      } else {
        std::printf("err %d\n", st);
      }
    } else if (op == "reserve") {
      int sid, cur, n;
      in >> sid >> cur >> n;
      if (!rows.count(sid)) {
        rows[sid] = std::vector<int32_t>(kCap, -1);
        nblk[sid] = 0;
      }
      std::vector<int64_t> slots(n > 0 ? n : 1);
      int32_t pair[2] = {-1, -1}, ncow = 0;
      int st = pkv_seq_reserve(a, rows[sid].data(), kCap, &nblk[sid], cur, n, slots.data(), pair, &ncow);
      if (st != 0) {
        std::printf("err %d\n", st);
        continue;
      }
      std::printf("ok");
      for (int i = 0; i < n; ++i) std::printf(" %lld", static_cast<long long>(slots[i]));
      std::printf(" |");
      if (ncow) std::printf(" %d %d", pair[0], pair[1]);
      std::printf(" |");
      for (int j = 0; j < nblk[sid]; ++j) std::printf(" %d", rows[sid][j]);
      std::printf("\n");
    } else if (op == "release") {
      int sid;
      in >> sid;
      int st = pkv_seq_release(a, rows[sid].data(), nblk[sid]);
      if (st == 0) {
        rows.erase(sid);
        nblk.erase(sid);
        std::printf("ok\n");
      } else {
        std::printf("err %d\n", st);
      }
    } else if (op == "state") {
      int32_t nb = pkv_num_blocks(a);
      std::vector<int32_t> fl(nb > 0 ? nb : 1);
      int n = pkv_free_list(a, fl.data(), nb);
      std::printf("free");
      for (int i = 0; i < n; ++i) std::printf(" %d", fl[i]);
      std::printf(" | ref");
      for (int32_t b = 0; b < nb; ++b) std::printf(" %d", pkv_block_refcount(a, b));
      std::printf("\n");
    }
  }
  pkv_allocator_destroy(a);
  return 0;
}
