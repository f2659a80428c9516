// Host core of libpa: pool descriptor checks, pool memory layout, the LIFO
// block allocator with refcounts, and per-sequence block tables.  Pure C++17,
// no HIP: it builds with g++ as well as hipcc.
//
// Sources: "The 8GB VRAM Breakthrough ..." section 3 (flat pool of 16-token
// blocks, block tables, copy-on-write of a partially filled shared block) and
// section 4 (FP16 sink blocks beside a compressed body); "A Ideia de 60 Anos
// Que Domou a Memoria da GPU", "o codigo" (pool = stack of free ids + one
// refcount per block: rent pops, return pushes when the count reaches zero)
// and "a ideia roubada" (a new block only when the previous one is full).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <unordered_map>
#include <utility>
#include <vector>

namespace pa {

enum Status : int32_t {
  kOk = 0,
  kInvalidArg = 1,
  kOutOfBlocks = 2,
  kRefcount = 3,
  kBadId = 4,
  kUnsupported = 5,
  kHip = 6,
};

enum Dtype : int32_t { kF32 = 0, kF16 = 1, kBF16 = 2, kInt4 = 3, kFp8 = 4 };
enum Arena : int32_t { kBody = 0, kSink = 1 };
enum ArrayId : int32_t { kArrK = 0, kArrV, kArrKS, kArrKZ, kArrVS, kArrVZ, kArrSK, kArrSV, kNumArr };

constexpr int32_t kBlock = 16;

// Thrown inside the library, turned into a status at the C boundary.
struct Error {
  Status code;
  std::string msg;
};

struct Desc {
  int32_t block_size, n_kv_heads, head_dim, kv_dtype, group_size, num_blocks, num_sink_blocks,
      sink_blocks_per_seq, window_tokens;
};

struct Layout {
  size_t total = 0;
  size_t offset[kNumArr];
  size_t slab[kNumArr];
  int32_t nblocks[kNumArr];  // slabs per head in the array (arena size)
};

bool is_raw(int32_t dt);
int32_t elem_bytes(int32_t dt);  // raw dtypes only
void validate_desc(const Desc& d);
Layout compute_layout(const Desc& d);

struct Seq {
  std::vector<int32_t> table;
  int32_t length = 0;
  bool live = false;
};

class PoolCore {
 public:
  PoolCore(const Desc& d, const int32_t* body_order, const int32_t* sink_order);

  const Desc& desc() const { return d_; }
  int32_t total_blocks() const { return d_.num_blocks + d_.num_sink_blocks; }
  int32_t arena_of(int32_t id) const;

  int32_t alloc(int32_t arena);
  void incref(int32_t id);
  void free_block(int32_t id);
  // Pops a block of src's arena, drops one ref of src; the caller copies data.
  int32_t cow_clone(int32_t src);
  int32_t refcount(int32_t id) const;
  int32_t num_free(int32_t arena) const;
  std::vector<int32_t> free_list(int32_t arena) const;  // next pop first
  int64_t num_clones() const { return clones_; }

  int32_t seq_create();
  int32_t seq_fork(int32_t parent);
  // Appends n slots; clones (src, dst) performed are appended to *clones.
  std::vector<int32_t> seq_reserve(int32_t seq, int32_t n,
                                   std::vector<std::pair<int32_t, int32_t>>* clones);
  // Moves the sequence's FP16 blocks that have left the window into the body
  // (pairs (FP16 source, body target) appended to *moves); all-or-nothing.
  int32_t seq_settle(int32_t seq, std::vector<std::pair<int32_t, int32_t>>* moves);
  void seq_truncate(int32_t seq, int32_t new_len);
  void seq_release(int32_t seq);
  const Seq& seq(int32_t id) const;

  // ---- block-hash prefix cache ----------------------------------------------
  // A full block of a prompt is keyed by the chained hash of the prompt's
  // token ids up to and including it: h_j = FNV-1a-64(h_{j-1} as 8 bytes LE,
  // then the block's 16 ids as int32 LE), h_{-1} = the FNV-1a offset basis.
  static uint64_t block_hash(uint64_t prev, const int32_t* ids16);
  // New sequence mapped onto the cached blocks of the longest cached prefix
  // of whole blocks (each entry checked on its ids and on its parent block);
  // returns the cached tokens (a multiple of 16).
  int32_t prefix_lookup(const int32_t* ids, int32_t n, int32_t* out_seq);
  // Enters the sequence's full blocks (up to n ids) not yet cached; the cache
  // holds one reference per entry.  Stops at the first block whose chain
  // position is cached under another block.  Returns the entries added.
  int32_t prefix_register(int32_t seq, const int32_t* ids, int32_t n);
  // Drops up to max_blocks entries, least recently used first, among those
  // with no cached child whose block only the cache holds; returns how many.
  int32_t prefix_evict(int32_t max_blocks);
  int32_t prefix_entries() const { return int32_t(pcache_.size()); }
  int64_t prefix_hit_blocks() const { return p_hits_; }
  int64_t prefix_asked_blocks() const { return p_asked_; }

 private:
  Seq& seq_mut(int32_t id);
  void check_id(int32_t id) const;
  void check_drop(const std::vector<int32_t>& blocks, size_t from) const;
  int64_t n_out(int64_t length) const;  // logical blocks entirely older than the window
  int32_t arena_for_logical(int32_t j, int64_t length) const;

  struct PEntry {
    int32_t block, parent;  // parent: the cached block of position j - 1, -1 at j = 0
    uint64_t parent_hash;
    int32_t ids[kBlock];
    uint64_t stamp;   // last use (lookup hit or register)
    int32_t children; // cached entries whose parent this is
  };
  std::unordered_map<uint64_t, PEntry> pcache_;
  uint64_t pclock_ = 0;
  int64_t p_hits_ = 0, p_asked_ = 0;

  Desc d_;
  std::vector<int32_t> ref_;
  std::vector<int32_t> stack_[2];  // back() is the top
  std::vector<Seq> seqs_;
  int64_t clones_ = 0;
};

}  // namespace pa
