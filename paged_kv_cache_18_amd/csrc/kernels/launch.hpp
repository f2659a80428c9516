// Interface between the C ABI (pa_capi.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../pa_host.hpp"

namespace pa {

// Device view of a pool: base pointer plus the arrays of include/pa.h.
struct PoolDev {
  uint8_t* base;
  int32_t n_kv_heads, head_dim, kv_dtype, group_size, num_blocks, num_sink_blocks;
  int32_t sink_per_seq;  // logical blocks 0..sink_per_seq-1 live in the sink arena
  int32_t window_tokens;  // > 0: the blocks of the last window_tokens tokens may also be FP16
  int32_t block_size;     // tokens per block: 16; 8 or 32 (raw 16-bit, D 128)
  size_t off[kNumArr];
  size_t slab[kNumArr];
};

// Window migration (FP16 sink-arena block -> body block), up to
// kMigrateMax pairs per launch.
constexpr int kMigrateMax = 16;
struct MigrateJob {
  int32_t src[kMigrateMax], dst[kMigrateMax];
  int32_t n;
};
hipError_t launch_migrate(const PoolDev& p, const MigrateJob& job, hipStream_t s);

hipError_t launch_append(const PoolDev& p, const void* k, const void* v, int32_t in_dtype,
                         const int32_t* slots, int32_t n_tokens, hipStream_t s);

// Token lens[b] - 1 of every sequence b, from rows b of k / v, into the slot
// its table row gives (a decode step's append, slots from the tables).
hipError_t launch_append_last(const PoolDev& p, const void* k, const void* v, int32_t in_dtype,
                              const int32_t* tables, const int32_t* lens, int32_t batch,
                              int32_t max_blocks, int32_t max_len, hipStream_t s);

hipError_t launch_block_copy(const PoolDev& p, int32_t src, int32_t dst, hipStream_t s);

enum DecodeKernel : int32_t { kKernGeneric = 0, kKernMfma16 = 1, kKernQuant = 2 };

struct DecodeArgs {
  PoolDev pool;
  const void* q;
  const int32_t* tables;
  const int32_t* lens;
  int32_t batch, n_q_heads, q_dtype, max_blocks_per_seq, max_seq_len;
  int32_t n_query;        // queries per sequence: 1 (decode), gamma + 1 (verify) or a prefill chunk
  // matrix-core kernels: column slices per (sequence, KV head) -- segments
  // (b, h * col_slices + s) of 32 (query, head) columns each; 1 = one
  // segment of all n_query * G columns
  int32_t col_slices;
  int32_t slice_cols;    // (query, head) columns of a column slice when col_slices > 1
  float scale_log2;      // softmax scale * log2(e): scores live in the log2 domain
  void* out;
  float* ws_o;           // [batch][n_q_heads][max_splits][head_dim] partial sums
  float* ws_ml;          // [batch][n_q_heads][max_splits][2] (max, sum), log2 domain
  // matrix-core kernels: the unit queue, then one arrival counter per unit
  // (the first unit of a segment that spans several), ctr_stride words
  // apart; zero between calls
  unsigned* counters;
  int ctr_stride;
  // matrix-core kernels with the merge launch: per segment (first unit, with
  // bit 31 set when its first piece is in the unit's second slot; pieces)
  int32_t* jobs;
  int32_t split_blocks;  // logical blocks per split
  int32_t max_splits;
  int32_t kernel;        // DecodeKernel
  int32_t prio;          // matrix-core kernels: 1 = progress-based wave priority
  int32_t unit_blocks;   // matrix-core kernels: blocks per queued unit (0: none)
  int32_t static_permille;  // share of a region its owner streams, in 1/1000
  int32_t defer_merge;   // matrix-core kernels: 1 = leave split segments to the merge launch
  // matrix-core decode kernels: a decode step that appends its new token
  // first -- token lens[b] - 1 of every sequence b, K and V from row b of
  // [batch][n_kv_heads][head_dim] inputs of dtype app_dt, into the slot its
  // table gives -- or nullptr
  const void* app_k;
  const void* app_v;
  int32_t app_dt;
};

hipError_t launch_decode_split(const DecodeArgs& a, hipStream_t s);
// Resident workgroups per compute unit of the split kernel `kernel` for a pool
// of kv_dtype (from the runtime's occupancy calculator; cached).
// nct: 0 for decode, else the verify step's column tiles (1 or 2).
int decode_split_occupancy(int32_t kernel, int32_t kv_dtype, int nct, int32_t group_size);
hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t s);
// Merge launch of the matrix-core kernels (defer_merge = 1).
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t s);

// Chunked-prefill attention of 16-bit pools of 16-token blocks (n_query
// queries per sequence, causal): one workgroup per (sequence, KV head, group
// of 128 (query, head) columns), no workspace.
hipError_t launch_prefill_tile(const DecodeArgs& a, hipStream_t s);

// Zero `bytes` (a multiple of 16) at p with plain vector stores.
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

// Streaming read of `bytes` (a multiple of 16) at src with `grid` workgroups.
hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, int grid, hipStream_t s);

// Plain read of every slab a decode of the batch reads (through the tables);
// sink[0] ^= the XOR of every 32-bit word read.  Head dim 128: 16-bit pools
// of 8-, 16- or 32-token blocks, INT4 and FP8 pools (with their FP16 sinks).
bool paged_read_supported(const PoolDev& p);
hipError_t launch_paged_read(const PoolDev& p, const int32_t* tables, const int32_t* lens, int32_t batch,
                             int32_t max_blocks, int32_t max_seq_len, void* sink, int grid, hipStream_t s);

}  // namespace pa
