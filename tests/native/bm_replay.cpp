// bm_replay.cpp -- replays a stream of block-manager operations read from
// stdin against the library's host block manager (pa_bm_* in include/pa.h)
// and prints one line per operation.  Test infrastructure: built together
// with pa_block_manager.cpp under AddressSanitizer and UndefinedBehavior-
// Sanitizer by tests/test_block_manager_sanitized.py, which writes the
// stream and compares every printed line with the prefix-cache oracle.
//
// Input, one operation per line (all integers):
//   create NB BS CACHING N o_0 .. o_{N-1}   (N = 0: default free order)
//   add N t_0 .. t_{N-1}      -> "seq cached" | "err STATUS"
//   append SEQ TOKEN          -> "slot src dst" | "err STATUS"
//   fork SEQ                  -> "seq" | "err STATUS"
//   free SEQ                  -> "ok" | "err STATUS"
//   table SEQ                 -> "n b_0 .. b_{n-1}" (n = -1: unknown)
//   length SEQ                -> "L"
//   counts                    -> "free cached"
//   destroy                   -> "ok"
// A create with invalid arguments prints "null".

#include <cstdint>
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "pa.h"

int main() {
  pa_block_manager* m = nullptr;
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string op;
    if (!(in >> op)) continue;
    std::ostringstream out;
    if (op == "create") {
      int32_t nb = 0, bs = 0, caching = 0, n = 0;
      in >> nb >> bs >> caching >> n;
      std::vector<int32_t> order(n > 0 ? n : 0);
      for (auto& o : order) in >> o;
      if (m) pa_bm_destroy(m);
      m = pa_bm_create(nb, bs, caching, n > 0 ? order.data() : nullptr);
      out << (m ? "ok" : "null");
    } else if (op == "add") {
      int32_t n = 0;
      in >> n;
      std::vector<int32_t> t(n > 0 ? n : 0);
      for (auto& x : t) in >> x;
      int32_t seq = -1, cached = -1;
      const pa_status st = pa_bm_add(m, t.empty() ? nullptr : t.data(), n, &seq, &cached);
      if (st == PA_OK) out << seq << ' ' << cached;
      else out << "err " << st;
    } else if (op == "append") {
      int32_t seq = 0, token = 0, slot = -1, src = -1, dst = -1;
      in >> seq >> token;
      const pa_status st = pa_bm_append(m, seq, token, &slot, &src, &dst);
      if (st == PA_OK) out << slot << ' ' << src << ' ' << dst;
      else out << "err " << st;
    } else if (op == "fork") {
      int32_t seq = 0, nseq = -1;
      in >> seq;
      const pa_status st = pa_bm_fork(m, seq, &nseq);
      if (st == PA_OK) out << nseq;
      else out << "err " << st;
    } else if (op == "free") {
      int32_t seq = 0;
      in >> seq;
      const pa_status st = pa_bm_free(m, seq);
      if (st == PA_OK) out << "ok";
      else out << "err " << st;
    } else if (op == "table") {
      int32_t seq = 0;
      in >> seq;
      const int32_t n = pa_bm_table(m, seq, nullptr, 0);
      out << n;
      if (n > 0) {
        // one entry short first: the call must stop at the capacity
        std::vector<int32_t> buf(n, -7);
        pa_bm_table(m, seq, buf.data(), n - 1);
        if (buf[n - 1] != -7) out << " overflow";
        pa_bm_table(m, seq, buf.data(), n);
        for (int32_t b : buf) out << ' ' << b;
      }
    } else if (op == "length") {
      int32_t seq = 0;
      in >> seq;
      out << pa_bm_length(m, seq);
    } else if (op == "counts") {
      out << pa_bm_free_blocks(m) << ' ' << pa_bm_cached_blocks(m);
    } else if (op == "destroy") {
      pa_bm_destroy(m);
      m = nullptr;
      out << "ok";
    } else {
      out << "bad op";
    }
    std::cout << out.str() << '\n';
  }
  if (m) pa_bm_destroy(m);
  std::cout.flush();
  return 0;
}
