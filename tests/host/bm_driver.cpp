// Host-only driver of the block manager for the sanitizer tests: reads one
// allocator operation per line from stdin and prints its result, so that a
// test can replay the same script on the oracle and compare line by line.
//
//   N <num_blocks> <block_size> [<free order ...>]   pool (first line)
//   C                        seq_create             -> <seq>
//   K <n> <ids ...>          seq_create_cached      -> <rc> <seq> <cached> <slots ...>
//   A <seq> <n>              alloc, no token ids    -> <rc> <cow src> <cow dst> <slots ...>
//   T <seq> <n> <ids ...>    alloc with token ids   -> the same
//   F <seq>                  fork                   -> <rc> <child>
//   X <seq>                  free                   -> <rc>
//   S                        state                  -> refcounts / free queue / counters lines
// rc: 0 ok, 1 invalid argument, 2 no blocks, 3 bad sequence.
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "block_manager.hpp"

namespace {

int rc_of(pa::BmStatus s) { return static_cast<int>(s); }

std::vector<int32_t> read_ints(std::istringstream& in, int64_t n) {
  std::vector<int32_t> v(static_cast<size_t>(n > 0 ? n : 0));
  for (auto& x : v) in >> x;
  return v;
}

void print_ints(const char* tag, const std::vector<int32_t>& v) {
  std::printf("%s", tag);
  for (int32_t x : v) std::printf(" %d", x);
  std::printf("\n");
}

}  // namespace

int main() {
  std::string line;
  if (!std::getline(std::cin, line)) return 2;
  std::istringstream head(line);
  char op;
  int32_t nb = 0, bs = 0;
  head >> op >> nb >> bs;
  if (op != 'N' || nb < 1 || bs < 1) return 2;
  pa::BlockManager bm(nb, bs);
  std::vector<int32_t> order;
  for (int32_t x; head >> x;) order.push_back(x);
  if (!order.empty() && bm.set_free_order(order.data(), static_cast<int32_t>(order.size())) != pa::BmStatus::kOk)
    return 2;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    if (!(in >> op)) continue;
    if (op == 'C') {
      std::printf("%d\n", bm.seq_create());
    } else if (op == 'K') {
      int32_t n;
      in >> n;
      const std::vector<int32_t> ids = read_ints(in, n);
      std::vector<int32_t> slots(static_cast<size_t>(n > 0 ? n : 1));
      int32_t seq = -1, cached = -1;
      const int rc = rc_of(bm.seq_create_cached(ids.data(), n, &seq, &cached, slots.data()));
      std::printf("%d %d %d", rc, rc == 0 ? seq : -1, rc == 0 ? cached : -1);
      if (rc == 0)
        for (int32_t i = 0; i < n - cached; ++i) std::printf(" %d", slots[i]);
      std::printf("\n");
    } else if (op == 'A' || op == 'T') {
      int32_t seq, n;
      in >> seq >> n;
      std::vector<int32_t> ids;
      if (op == 'T') ids = read_ints(in, n);
      std::vector<int32_t> slots(static_cast<size_t>(n > 0 ? n : 1));
      int32_t src = -1, dst = -1;
      const int rc = rc_of(bm.alloc(seq, n, slots.data(), &src, &dst, op == 'T' ? ids.data() : nullptr));
      std::printf("%d %d %d", rc, src, dst);
      if (rc == 0)
        for (int32_t i = 0; i < n; ++i) std::printf(" %d", slots[i]);
      std::printf("\n");
    } else if (op == 'F') {
      int32_t seq, child = -1;
      in >> seq;
      const int rc = rc_of(bm.fork(seq, &child));
      std::printf("%d %d\n", rc, rc == 0 ? child : -1);
    } else if (op == 'X') {
      int32_t seq;
      in >> seq;
      std::printf("%d\n", rc_of(bm.free_seq(seq)));
    } else if (op == 'S') {
      print_ints("R", bm.refcounts());
      std::vector<int32_t> q(static_cast<size_t>(bm.free_count()));
      bm.free_queue(q.data());
      print_ints("Q", q);
      std::printf("S %lld %lld %lld %lld %lld %lld %lld %lld %lld\n",
                  static_cast<long long>(bm.free_count()), static_cast<long long>(bm.shared_blocks()),
                  static_cast<long long>(bm.live_seqs()), static_cast<long long>(bm.cow_copies()),
                  static_cast<long long>(bm.alloc_failures()), static_cast<long long>(bm.cache_hits()),
                  static_cast<long long>(bm.cache_misses()), static_cast<long long>(bm.cache_evictions()),
                  static_cast<long long>(bm.cached_blocks()));
    } else {
      return 2;
    }
  }
  return 0;
}
