// Op-log replayer for the library's host core (csrc/pa_host.cpp), built with
// g++ under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py.  Test infrastructure only: it links the
// product's host core, not the oracle, and reads one op log from stdin:
//
//   desc <block_size> <n_kv_heads> <head_dim> <kv_dtype> <group> <num_blocks>
//        <num_sink_blocks> <sink_blocks_per_seq> <window_tokens>
//   body <n> <ids...>          (initial free order; n = 0: identity)
//   sink <n> <ids...>
//   then one op per line: create | reserve s n | fork p | release s |
//   truncate s n | alloc arena | incref id | free id | clone id | settle s |
//   plookup n ids... | pregister s n ids... | pevict k
//
// It prints one line per op ("ok ..." with the op's results, or "err <status>")
// and then the final state: every block's refcount, both free stacks (next
// pop first), the clone count, the prefix-cache counters and every live
// sequence's length and table.
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "pa_host.hpp"

namespace {

std::vector<int32_t> read_ints(std::istringstream& in, int n) {
  std::vector<int32_t> v(size_t(n > 0 ? n : 0));
  for (auto& x : v) in >> x;
  return v;
}

void print_list(const char* tag, const std::vector<int32_t>& v) {
  std::cout << tag;
  for (int32_t x : v) std::cout << ' ' << x;
  std::cout << '\n';
}

}  // namespace

int main() {
  std::string line, word;
  pa::Desc d{};
  std::vector<int32_t> body, sink;
  std::vector<std::string> ops;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    if (!(in >> word)) continue;
    if (word == "desc") {
      in >> d.block_size >> d.n_kv_heads >> d.head_dim >> d.kv_dtype >> d.group_size >>
          d.num_blocks >> d.num_sink_blocks >> d.sink_blocks_per_seq >> d.window_tokens;
    } else if (word == "body" || word == "sink") {
      int n = 0;
      in >> n;
      (word == "body" ? body : sink) = read_ints(in, n);
    } else {
      ops.push_back(line);
    }
  }
  try {
    pa::validate_desc(d);
  } catch (const pa::Error& e) {
    std::cout << "desc err " << int(e.code) << '\n';
    return 0;
  }
  pa::PoolCore core(d, body.empty() ? nullptr : body.data(), sink.empty() ? nullptr : sink.data());
  int32_t max_sid = -1;  // sequence ids are handed out 0, 1, 2, ...
  for (const std::string& op : ops) {
    std::istringstream in(op);
    in >> word;
    try {
      std::ostringstream res;
      if (word == "create") {
        max_sid = core.seq_create();
        res << max_sid;
      } else if (word == "reserve") {
        int32_t s = 0, n = 0;
        in >> s >> n;
        std::vector<std::pair<int32_t, int32_t>> clones;
        for (int32_t slot : core.seq_reserve(s, n, &clones)) res << slot << ' ';
      } else if (word == "fork") {
        int32_t p = 0;
        in >> p;
        max_sid = core.seq_fork(p);
        res << max_sid;
      } else if (word == "release") {
        int32_t s = 0;
        in >> s;
        core.seq_release(s);
      } else if (word == "truncate") {
        int32_t s = 0, n = 0;
        in >> s >> n;
        core.seq_truncate(s, n);
      } else if (word == "alloc") {
        int32_t a = 0;
        in >> a;
        res << core.alloc(a);
      } else if (word == "incref") {
        int32_t id = 0;
        in >> id;
        core.incref(id);
      } else if (word == "free") {
        int32_t id = 0;
        in >> id;
        core.free_block(id);
      } else if (word == "clone") {
        int32_t id = 0;
        in >> id;
        res << core.cow_clone(id);
      } else if (word == "settle") {
        int32_t s = 0;
        in >> s;
        std::vector<std::pair<int32_t, int32_t>> moves;
        res << core.seq_settle(s, &moves);
      } else if (word == "plookup") {
        int n = 0;
        in >> n;
        const std::vector<int32_t> ids = read_ints(in, n);
        int32_t sid = -1;
        const int32_t cached = core.prefix_lookup(ids.empty() ? nullptr : ids.data(), n, &sid);
        if (sid >= 0) max_sid = sid;
        res << sid << ' ' << cached;
      } else if (word == "pregister") {
        int32_t s = 0;
        int n = 0;
        in >> s >> n;
        const std::vector<int32_t> ids = read_ints(in, n);
        res << core.prefix_register(s, ids.empty() ? nullptr : ids.data(), n);
      } else if (word == "pevict") {
        int32_t k = 0;
        in >> k;
        res << core.prefix_evict(k);
      } else {
        std::cerr << "unknown op " << word << '\n';
        return 2;
      }
      std::cout << "ok " << res.str() << '\n';
    } catch (const pa::Error& e) {
      std::cout << "err " << int(e.code) << '\n';
    }
  }
  std::vector<int32_t> refs;
  for (int32_t id = 0; id < core.total_blocks(); ++id) refs.push_back(core.refcount(id));
  print_list("ref", refs);
  print_list("free0", core.free_list(pa::kBody));
  print_list("free1", core.free_list(pa::kSink));
  std::cout << "clones " << core.num_clones() << '\n';
  std::cout << "prefix " << core.prefix_entries() << ' ' << core.prefix_hit_blocks() << ' '
            << core.prefix_asked_blocks() << '\n';
  for (int32_t sid = 0; sid <= max_sid; ++sid) {
    try {
      const pa::Seq& s = core.seq(sid);
      std::cout << "seq " << sid << ' ' << s.length;
      for (int32_t b : s.table) std::cout << ' ' << b;
      std::cout << '\n';
    } catch (const pa::Error&) {
      std::cout << "seq " << sid << " released\n";
    }
  }
  return 0;
}
