// KV append with fused quantize-on-write (the per-token work, shared with the
// decode step that appends its own new token, is in append_common.hpp), the
// window migration and the copy-on-write block copy.
//
// "The 8GB VRAM Breakthrough ...", section 5 (flowchart): a token-position
// router sends sink tokens to the FP16 block pool and the body through a
// fused quantizer into the compressed pool.  Section 3 ("Copy-on-Write (CoW)
// Prefix Sharing"): before a sequence writes into a partially filled shared
// block, a fresh block receives a copy.
#pragma clang fp contract(off)

#include "append_common.hpp"

namespace pa {

namespace {

constexpr int kWaves = 4;  // waves per workgroup

// One wave per (token, kv head, K-or-V): wave index gw = 2 (token H + head)
// + kind, below 2^31 (the launch checks).
template <int MP>
__global__ __launch_bounds__(kWaves * 64) void append_kv_kernel(PoolDev p, const void* kin,
                                                                const void* vin, int in_dt,
                                                                const int32_t* slots, int n) {
  const int lane = threadIdx.x & 63;
  const int gw = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * kWaves + int(threadIdx.x >> 6));
  const int H = p.n_kv_heads;
  const int kind = gw & 1;  // 0 = K, 1 = V
  const int th = gw >> 1;
  const int tok = th / H, h = th % H;
  if (tok >= n) return;
  // the slot is loaded alongside the token's values (append_one issues their
  // loads before it looks at the block id): one memory round trip, not two
  const int slot = slots[tok];
  const int bs = p.block_size;
  app::append_one<MP>(p, kin, vin, in_dt, size_t(tok), h, kind, slot < 0 ? -1 : slot / bs,
                      slot < 0 ? 0 : slot % bs, lane);
}

// A decode step's new tokens: token lens[b] - 1 of every sequence b (rows b
// of kin / vin), into the slot its table row gives; one wave per (sequence,
// kv head, K-or-V).  Sequences of length 0 write nothing.
template <int MP>
__global__ __launch_bounds__(kWaves * 64) void append_last_kernel(PoolDev p, const void* kin,
                                                                  const void* vin, int in_dt,
                                                                  const int32_t* tables,
                                                                  const int32_t* lens, int batch,
                                                                  int max_blocks, int max_len) {
  const int lane = threadIdx.x & 63;
  const int gw = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * kWaves + int(threadIdx.x >> 6));
  const int H = p.n_kv_heads;
  const int kind = gw & 1, th = gw >> 1;
  const int b = th / H, h = th % H;
  if (b >= batch) return;
  const int L = min(max(lens[b], 0), max_len);
  const int bs = p.block_size;
  const int id = L > 0 ? tables[size_t(b) * max_blocks + (L - 1) / bs] : -1;
  app::append_one<MP>(p, kin, vin, in_dt, size_t(b), h, kind, id, L > 0 ? (L - 1) % bs : 0, lane);
}

// Copy-on-write: every array's slabs of block `src` (all heads) to `dst`.
struct CopyJob {
  size_t src[kNumArr], dst[kNumArr], bytes[kNumArr];
  int n;
};

__global__ __launch_bounds__(256) void block_copy_kernel(uint8_t* base, CopyJob job) {
  const int a = blockIdx.y;
  if (a >= job.n) return;
  const size_t units = job.bytes[a] / 16;
  const uint4* s = reinterpret_cast<const uint4*>(base + job.src[a]);
  uint4* d = reinterpret_cast<uint4*>(base + job.dst[a]);
  for (size_t u = size_t(blockIdx.x) * blockDim.x + threadIdx.x; u < units;
       u += size_t(gridDim.x) * blockDim.x)
    d[u] = s[u];
}

constexpr int kMigrateMP = 2;  // dimension pairs per lane: head_dim <= 256

// Window migration: the 16 FP16 tokens of sink-arena block src[i] (every
// head, K and V) quantized into body block dst[i]; one wave per (pair, token,
// head, K-or-V).
__global__ __launch_bounds__(kWaves * 64) void migrate_kernel(PoolDev p, MigrateJob job) {
  const int lane = threadIdx.x & 63;
  const long gw = (long(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int H = p.n_kv_heads, D = p.head_dim, N = p.num_blocks;
  const int kind = int(gw & 1);
  long r = gw >> 1;
  const int h = int(r % H);
  r /= H;
  const int t = int(r % 16);
  const long pi = r / 16;
  if (pi >= job.n) return;
  const int src = job.src[pi], dst = job.dst[pi];
  if (src < N || src >= N + p.num_sink_blocks || dst < 0 || dst >= N) return;
  const int arr = kind ? kArrSV : kArrSK;
  const uint16_t* slab = reinterpret_cast<const uint16_t*>(
      p.base + p.off[arr] + (size_t(src - N) * H + h) * p.slab[arr]);
  float x[kMigrateMP][2];
  bool has[kMigrateMP];
#pragma unroll
  for (int m = 0; m < kMigrateMP; ++m) {
    const int k = lane + 64 * m;
    has[m] = 2 * k < D;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int d = 2 * k + e;
      x[m][e] = has[m] ? f16_bits_to_f32(slab[kind ? raw_v_elem(t, d, D) : raw_k_elem(t, d)]) : 0.f;
    }
  }
  app::quantize_store<kMigrateMP>(p, dst, t, h, kind, x, has, lane);
}

}  // namespace

hipError_t launch_migrate(const PoolDev& p, const MigrateJob& job, hipStream_t s) {
  if (job.n <= 0) return hipSuccess;
  const long waves = long(job.n) * 16 * p.n_kv_heads * 2;
  const unsigned grid = unsigned((waves + kWaves - 1) / kWaves);
  hipLaunchKernelGGL(migrate_kernel, dim3(grid), dim3(kWaves * 64), 0, s, p, job);
  return hipGetLastError();
}

hipError_t launch_append(const PoolDev& p, const void* k, const void* v, int32_t in_dtype,
                         const int32_t* slots, int32_t n_tokens, hipStream_t s) {
  if (n_tokens <= 0) return hipSuccess;
  const long waves = long(n_tokens) * p.n_kv_heads * 2;
  if (waves >= (1L << 31)) return hipErrorInvalidValue;  // the kernel indexes waves in 32 bits
  const unsigned grid = unsigned((waves + kWaves - 1) / kWaves);
  if (p.head_dim <= 128)
    hipLaunchKernelGGL(append_kv_kernel<1>, dim3(grid), dim3(kWaves * 64), 0, s, p, k, v, in_dtype,
                       slots, n_tokens);
  else
    hipLaunchKernelGGL(append_kv_kernel<2>, dim3(grid), dim3(kWaves * 64), 0, s, p, k, v, in_dtype,
                       slots, n_tokens);
  return hipGetLastError();
}

hipError_t launch_append_last(const PoolDev& p, const void* k, const void* v, int32_t in_dtype,
                              const int32_t* tables, const int32_t* lens, int32_t batch,
                              int32_t max_blocks, int32_t max_len, hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  const long waves = long(batch) * p.n_kv_heads * 2;
  if (waves >= (1L << 31)) return hipErrorInvalidValue;
  const unsigned grid = unsigned((waves + kWaves - 1) / kWaves);
  if (p.head_dim <= 128)
    hipLaunchKernelGGL(append_last_kernel<1>, dim3(grid), dim3(kWaves * 64), 0, s, p, k, v, in_dtype,
                       tables, lens, batch, max_blocks, max_len);
  else
    hipLaunchKernelGGL(append_last_kernel<2>, dim3(grid), dim3(kWaves * 64), 0, s, p, k, v, in_dtype,
                       tables, lens, batch, max_blocks, max_len);
  return hipGetLastError();
}

hipError_t launch_block_copy(const PoolDev& p, int32_t src, int32_t dst, hipStream_t s) {
  CopyJob job{};
  const int N = p.num_blocks, H = p.n_kv_heads;
  const bool sink = src >= N;
  const int ls = sink ? src - N : src, ld = sink ? dst - N : dst;
  for (int a = 0; a < kNumArr; ++a) {
    const bool sink_arr = (a == kArrSK || a == kArrSV);
    if (p.slab[a] == 0 || sink_arr != sink) continue;
    const size_t per = p.slab[a] * size_t(H);
    job.src[job.n] = p.off[a] + size_t(ls) * per;
    job.dst[job.n] = p.off[a] + size_t(ld) * per;
    job.bytes[job.n] = per;
    ++job.n;
  }
  if (job.n == 0) return hipSuccess;
  hipLaunchKernelGGL(block_copy_kernel, dim3(8, job.n), dim3(256), 0, s, p.base, job);
  return hipGetLastError();
}

}  // namespace pa
