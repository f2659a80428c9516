// Host core of libpa (see pa_host.hpp for sources).
#include "pa_host.hpp"

#include <algorithm>
#include <limits>
#include <unordered_map>

namespace pa {

namespace {
[[noreturn]] void fail(Status s, const std::string& m) { throw Error{s, m}; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
}  // namespace

bool is_raw(int32_t dt) { return dt == kF32 || dt == kF16 || dt == kBF16; }

int32_t elem_bytes(int32_t dt) { return dt == kF32 ? 4 : 2; }

void validate_desc(const Desc& d) {
  if (d.block_size != kBlock) {
    if (d.block_size != 8 && d.block_size != 32) fail(kUnsupported, "block_size must be 8, 16 or 32");
    if ((d.kv_dtype != kF16 && d.kv_dtype != kBF16) || d.head_dim != 128 || d.num_sink_blocks > 0 ||
        d.window_tokens > 0)
      fail(kUnsupported, "block sizes 8 and 32 need a raw F16/BF16 pool with head_dim 128, no sink arena");
  }
  if (d.n_kv_heads < 1 || d.n_kv_heads > 1024) fail(kInvalidArg, "n_kv_heads out of range");
  if (d.head_dim < 32 || d.head_dim > 256 || d.head_dim % 32)
    fail(kInvalidArg, "head_dim must be a multiple of 32 in [32, 256]");
  if (d.num_blocks < 0 || d.num_sink_blocks < 0) fail(kInvalidArg, "negative block count");
  if (int64_t(d.num_blocks) + d.num_sink_blocks > (int64_t(1) << 26))
    fail(kInvalidArg, "too many blocks (slot ids must fit in int32)");
  if (d.kv_dtype == kInt4) {
    if (d.group_size < 32 || d.group_size % 32 || d.head_dim % d.group_size)
      fail(kInvalidArg, "INT4 group_size must be a multiple of 32 dividing head_dim");
  } else if (d.kv_dtype == kFp8) {
    if (d.head_dim % 64) fail(kInvalidArg, "FP8 needs head_dim multiple of 64");
  } else if (!is_raw(d.kv_dtype)) {
    fail(kInvalidArg, "unknown kv_dtype");
  }
  if ((d.num_sink_blocks > 0) != (d.sink_blocks_per_seq > 0) || d.sink_blocks_per_seq < 0)
    fail(kInvalidArg, "num_sink_blocks and sink_blocks_per_seq go together");
  if (d.num_sink_blocks > 0 && is_raw(d.kv_dtype))
    fail(kUnsupported, "a sink arena needs an INT4 or FP8 body");
  if (d.window_tokens < 0) fail(kInvalidArg, "negative window_tokens");
  if (d.window_tokens > 0 && d.num_sink_blocks == 0)
    fail(kInvalidArg, "a window needs the FP16 (sink) arena");
}

Layout compute_layout(const Desc& d) {
  validate_desc(d);
  Layout L;
  for (int i = 0; i < kNumArr; ++i) {
    L.offset[i] = std::numeric_limits<size_t>::max();
    L.slab[i] = 0;
    L.nblocks[i] = 0;
  }
  const size_t D = size_t(d.head_dim), B = size_t(d.block_size);
  struct Item { int id; size_t slab; int32_t n; };
  std::vector<Item> items;
  if (is_raw(d.kv_dtype)) {
    size_t e = size_t(elem_bytes(d.kv_dtype));
    items = {{kArrK, B * D * e, d.num_blocks}, {kArrV, B * D * e, d.num_blocks}};
  } else if (d.kv_dtype == kInt4) {
    size_t ng = D / size_t(d.group_size);
    items = {{kArrK, B * D / 2, d.num_blocks},  {kArrV, B * D / 2, d.num_blocks},
             {kArrKS, B * ng * 2, d.num_blocks}, {kArrKZ, B * ng * 2, d.num_blocks},
             {kArrVS, B * ng * 2, d.num_blocks}, {kArrVZ, B * ng * 2, d.num_blocks}};
  } else {
    items = {{kArrK, B * D, d.num_blocks}, {kArrV, B * D, d.num_blocks},
             {kArrKS, B * 2, d.num_blocks}, {kArrVS, B * 2, d.num_blocks}};
  }
  if (d.num_sink_blocks > 0) {
    items.push_back({kArrSK, B * D * 2, d.num_sink_blocks});
    items.push_back({kArrSV, B * D * 2, d.num_sink_blocks});
  }
  size_t off = 0;
  for (const Item& it : items) {
    off = align256(off);
    L.offset[it.id] = off;
    L.slab[it.id] = it.slab;
    L.nblocks[it.id] = it.n;
    off += it.slab * size_t(d.n_kv_heads) * size_t(it.n);
  }
  L.total = align256(off);
  return L;
}

// ---------------------------------------------------------------------------
PoolCore::PoolCore(const Desc& d, const int32_t* body_order, const int32_t* sink_order) : d_(d) {
  validate_desc(d);
  ref_.assign(size_t(total_blocks()), 0);
  const int32_t n[2] = {d.num_blocks, d.num_sink_blocks};
  const int32_t* order[2] = {body_order, sink_order};
  const int32_t base[2] = {0, d.num_blocks};
  for (int a = 0; a < 2; ++a) {
    std::vector<char> seen(size_t(n[a]), 0);
    std::vector<int32_t>& st = stack_[a];
    st.resize(size_t(n[a]));
    for (int32_t i = 0; i < n[a]; ++i) {
      int32_t x = order[a] ? order[a][i] : i;
      if (x < 0 || x >= n[a] || seen[size_t(x)]) fail(kInvalidArg, "free order is not a permutation");
      seen[size_t(x)] = 1;
      st[size_t(n[a] - 1 - i)] = base[a] + x;  // first element on top
    }
  }
}

void PoolCore::check_id(int32_t id) const {
  if (id < 0 || id >= total_blocks()) fail(kBadId, "block id " + std::to_string(id) + " out of range");
}

int32_t PoolCore::arena_of(int32_t id) const {
  check_id(id);
  return id >= d_.num_blocks ? kSink : kBody;
}

int32_t PoolCore::alloc(int32_t arena) {
  if (arena != kBody && arena != kSink) fail(kInvalidArg, "arena must be 0 (body) or 1 (sink)");
  std::vector<int32_t>& st = stack_[arena];
  if (st.empty()) fail(kOutOfBlocks, arena == kBody ? "body arena empty" : "sink arena empty");
  int32_t id = st.back();
  st.pop_back();
  ref_[size_t(id)] = 1;
  return id;
}

void PoolCore::incref(int32_t id) {
  check_id(id);
  if (ref_[size_t(id)] == 0) fail(kRefcount, "incref of free block " + std::to_string(id));
  ++ref_[size_t(id)];
}

void PoolCore::free_block(int32_t id) {
  check_id(id);
  if (ref_[size_t(id)] == 0) fail(kRefcount, "free of free block " + std::to_string(id));
  if (--ref_[size_t(id)] == 0) stack_[arena_of(id)].push_back(id);
}

int32_t PoolCore::cow_clone(int32_t src) {
  check_id(src);
  if (ref_[size_t(src)] == 0) fail(kRefcount, "clone of free block " + std::to_string(src));
  int32_t dst = alloc(arena_of(src));
  free_block(src);
  ++clones_;
  return dst;
}

int32_t PoolCore::refcount(int32_t id) const {
  check_id(id);
  return ref_[size_t(id)];
}

int32_t PoolCore::num_free(int32_t arena) const {
  if (arena != kBody && arena != kSink) fail(kInvalidArg, "arena must be 0 or 1");
  return int32_t(stack_[arena].size());
}

std::vector<int32_t> PoolCore::free_list(int32_t arena) const {
  if (arena != kBody && arena != kSink) fail(kInvalidArg, "arena must be 0 or 1");
  return std::vector<int32_t>(stack_[arena].rbegin(), stack_[arena].rend());
}

int64_t PoolCore::n_out(int64_t length) const {
  if (d_.window_tokens == 0) return std::numeric_limits<int64_t>::max();
  return std::max<int64_t>(0, (length - d_.window_tokens) / kBlock);
}

// FP16 arena for the sink blocks and for every block not entirely older than
// the window at `length` (the reserve's final length), body otherwise.
int32_t PoolCore::arena_for_logical(int32_t j, int64_t length) const {
  return (j < d_.sink_blocks_per_seq || j >= n_out(length)) ? kSink : kBody;
}

Seq& PoolCore::seq_mut(int32_t id) {
  if (id < 0 || size_t(id) >= seqs_.size() || !seqs_[size_t(id)].live)
    fail(kBadId, "unknown sequence " + std::to_string(id));
  return seqs_[size_t(id)];
}

const Seq& PoolCore::seq(int32_t id) const {
  if (id < 0 || size_t(id) >= seqs_.size() || !seqs_[size_t(id)].live)
    fail(kBadId, "unknown sequence " + std::to_string(id));
  return seqs_[size_t(id)];
}

int32_t PoolCore::seq_create() {
  if (seqs_.size() >= size_t(std::numeric_limits<int32_t>::max())) fail(kInvalidArg, "too many sequences");
  seqs_.emplace_back();
  seqs_.back().live = true;
  return int32_t(seqs_.size() - 1);
}

// A call that drops (or copies) references of blocks[from..] must find at
// least as many references as it uses, or it changes nothing.
void PoolCore::check_drop(const std::vector<int32_t>& blocks, size_t from) const {
  std::unordered_map<int32_t, int32_t> uses;
  for (size_t i = from; i < blocks.size(); ++i) ++uses[blocks[i]];
  for (const auto& kv : uses)
    if (ref_[size_t(kv.first)] < kv.second)
      fail(kRefcount, "block " + std::to_string(kv.first) + " has fewer refs than uses");
}

int32_t PoolCore::seq_fork(int32_t parent) {
  const Seq& p = seq(parent);
  check_drop(p.table, 0);
  std::vector<int32_t> table = p.table;
  int32_t len = p.length;
  int32_t child = seq_create();
  for (int32_t b : table) ++ref_[size_t(b)];
  Seq& c = seqs_[size_t(child)];
  c.table = std::move(table);
  c.length = len;
  return child;
}

std::vector<int32_t> PoolCore::seq_reserve(int32_t sid, int32_t n,
                                           std::vector<std::pair<int32_t, int32_t>>* clones) {
  Seq& s = seq_mut(sid);
  if (n < 0) fail(kInvalidArg, "negative token count");
  if (int64_t(s.length) + n > int64_t(std::numeric_limits<int32_t>::max() / 2))
    fail(kInvalidArg, "sequence too long");
  std::vector<int32_t> slots;
  if (n == 0) return slots;
  int32_t need[2] = {0, 0};
  const int32_t bs = d_.block_size;
  const bool clone = (s.length % bs != 0) && ref_[size_t(s.table.back())] > 1;
  if (clone) ++need[arena_of(s.table.back())];
  const int32_t first_new = int32_t(s.table.size());
  const int32_t last = int32_t((int64_t(s.length) + n + bs - 1) / bs);
  const int64_t final_len = int64_t(s.length) + n;
  for (int32_t j = first_new; j < last; ++j) ++need[arena_for_logical(j, final_len)];
  for (int a = 0; a < 2; ++a)
    if (size_t(need[a]) > stack_[a].size())
      fail(kOutOfBlocks, std::string(a == kBody ? "body" : "sink") + " arena needs " +
                             std::to_string(need[a]) + " blocks, has " +
                             std::to_string(stack_[a].size()));
  if (clone) {
    int32_t src = s.table.back();
    int32_t dst = cow_clone(src);
    s.table.back() = dst;
    if (clones) clones->emplace_back(src, dst);
  }
  for (int32_t j = first_new; j < last; ++j) s.table.push_back(alloc(arena_for_logical(j, final_len)));
  slots.resize(size_t(n));
  for (int32_t i = 0; i < n; ++i) {
    int32_t p = s.length + i;
    slots[size_t(i)] = s.table[size_t(p / bs)] * bs + p % bs;
  }
  s.length += n;
  return slots;
}

int32_t PoolCore::seq_settle(int32_t sid, std::vector<std::pair<int32_t, int32_t>>* moves) {
  Seq& s = seq_mut(sid);
  const int64_t end = std::min<int64_t>(n_out(s.length), int64_t(s.table.size()));
  std::vector<int32_t> todo;
  for (int64_t j = d_.sink_blocks_per_seq; j < end; ++j)
    if (arena_of(s.table[size_t(j)]) == kSink) todo.push_back(int32_t(j));
  if (todo.size() > stack_[kBody].size())
    fail(kOutOfBlocks, "body arena needs " + std::to_string(todo.size()) + " blocks, has " +
                           std::to_string(stack_[kBody].size()));
  for (int32_t j : todo) {
    const int32_t src = s.table[size_t(j)];
    const int32_t dst = alloc(kBody);
    s.table[size_t(j)] = dst;
    free_block(src);
    if (moves) moves->emplace_back(src, dst);
  }
  return int32_t(todo.size());
}

void PoolCore::seq_truncate(int32_t sid, int32_t new_len) {
  Seq& s = seq_mut(sid);
  if (new_len < 0 || new_len > s.length) fail(kInvalidArg, "truncate beyond length");
  size_t keep = size_t((new_len + d_.block_size - 1) / d_.block_size);
  check_drop(s.table, keep);
  while (s.table.size() > keep) {
    free_block(s.table.back());
    s.table.pop_back();
  }
  s.length = new_len;
}

void PoolCore::seq_release(int32_t sid) {
  Seq& s = seq_mut(sid);
  check_drop(s.table, 0);
  for (auto it = s.table.rbegin(); it != s.table.rend(); ++it) free_block(*it);
  s.table.clear();
  s.table.shrink_to_fit();
  s.length = 0;
  s.live = false;
}

// ---- block-hash prefix cache (Primer chapter 8, section 8.3: hash the prompt
// in block-sized pieces; a hit points the new request's table at the cached
// block and skips its prefill; a miss is prefilled and its block registered.
// The 3-minute page, "Compartilhamento e compromissos": shared prefixes map to
// the same physical blocks) -----------------------------------------------------

uint64_t PoolCore::block_hash(uint64_t prev, const int32_t* ids16) {
  constexpr uint64_t kPrime = 0x100000001b3ull;
  uint64_t h = 0xcbf29ce484222325ull;
  for (int i = 0; i < 8; ++i) {
    h ^= (prev >> (8 * i)) & 0xFFu;
    h *= kPrime;
  }
  for (int t = 0; t < kBlock; ++t) {
    const uint32_t v = uint32_t(ids16[t]);
    for (int i = 0; i < 4; ++i) {
      h ^= (v >> (8 * i)) & 0xFFu;
      h *= kPrime;
    }
  }
  return h;
}

namespace {
void need_prefix_pool(const Desc& d) {
  if (d.window_tokens > 0)
    fail(kUnsupported, "the prefix cache needs a pool without a local window (blocks would move)");
  if (d.block_size != kBlock) fail(kUnsupported, "the prefix cache keys 16-token blocks");
}
}  // namespace

int32_t PoolCore::prefix_lookup(const int32_t* ids, int32_t n, int32_t* out_seq) {
  need_prefix_pool(d_);
  if (n < 0) fail(kInvalidArg, "negative token count");
  if (n > 0 && !ids) fail(kInvalidArg, "null token ids");
  const int32_t sid = seq_create();
  Seq& s = seqs_[size_t(sid)];
  uint64_t h = 0xcbf29ce484222325ull;
  int32_t parent = -1;
  const int32_t nb = n / kBlock;
  for (int32_t j = 0; j < nb; ++j) {
    h = block_hash(h, ids + size_t(j) * kBlock);
    auto it = pcache_.find(h);
    if (it == pcache_.end()) break;
    PEntry& e = it->second;
    if (e.parent != parent || !std::equal(e.ids, e.ids + kBlock, ids + size_t(j) * kBlock)) break;
    incref(e.block);
    s.table.push_back(e.block);
    e.stamp = ++pclock_;
    parent = e.block;
  }
  const int32_t hits = int32_t(s.table.size());
  s.length = hits * kBlock;
  p_asked_ += nb;
  p_hits_ += hits;
  if (out_seq) *out_seq = sid;
  return hits * kBlock;
}

int32_t PoolCore::prefix_register(int32_t sid, const int32_t* ids, int32_t n) {
  need_prefix_pool(d_);
  const Seq& s = seq(sid);
  if (n < 0) fail(kInvalidArg, "negative token count");
  if (n > 0 && !ids) fail(kInvalidArg, "null token ids");
  const int32_t nb = std::min(n, s.length) / kBlock;
  uint64_t h = 0xcbf29ce484222325ull, ph = 0;
  int32_t parent = -1, added = 0;
  for (int32_t j = 0; j < nb; ++j) {
    h = block_hash(h, ids + size_t(j) * kBlock);
    const int32_t blk = s.table[size_t(j)];
    auto it = pcache_.find(h);
    if (it != pcache_.end()) {
      PEntry& e = it->second;
      // the position is cached under another block (or another chain): stop
      if (e.block != blk || e.parent != parent) break;
      e.stamp = ++pclock_;
    } else {
      incref(blk);
      PEntry e{};
      e.block = blk;
      e.parent = parent;
      e.parent_hash = ph;
      std::copy(ids + size_t(j) * kBlock, ids + size_t(j + 1) * kBlock, e.ids);
      e.stamp = ++pclock_;
      e.children = 0;
      pcache_.emplace(h, e);
      if (j > 0) ++pcache_.at(ph).children;
      ++added;
    }
    parent = blk;
    ph = h;
  }
  return added;
}

int32_t PoolCore::prefix_evict(int32_t max_blocks) {
  if (max_blocks < 0) fail(kInvalidArg, "negative max_blocks");
  int32_t done = 0;
  while (done < max_blocks) {
    // the least recently used leaf whose block only the cache holds
    auto best = pcache_.end();
    for (auto it = pcache_.begin(); it != pcache_.end(); ++it) {
      const PEntry& e = it->second;
      if (e.children == 0 && ref_[size_t(e.block)] == 1 && (best == pcache_.end() || e.stamp < best->second.stamp))
        best = it;
    }
    if (best == pcache_.end()) break;
    const PEntry e = best->second;
    pcache_.erase(best);
    if (e.parent >= 0) --pcache_.at(e.parent_hash).children;
    free_block(e.block);
    ++done;
  }
  return done;
}

}  // namespace pa
