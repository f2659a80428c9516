// Streaming-read kernel: the achievable HBM read rate on this GPU, measured
// beside the decode (a measurement aid, not a step of the method).  Each
// workgroup reads contiguous 32 KiB spans in a grid-stride loop (eight
// 16-byte loads in flight per lane) and folds them into one word that decides
// a (practically never taken) store to sink[0], so the loads cannot be
// dropped.  The paged read: the same kind of plain read over exactly the
// slabs a decode of a batch reads, through its block tables (the paged
// access pattern without the arithmetic).  Also the plain zero fill that
// clears the allocation-free decode's static scratch counters.
#include <algorithm>

#include "launch.hpp"

namespace pa {

namespace {

typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));

constexpr int kUnroll = 8;  // 16-byte loads in flight per lane

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                          uint32_t* sink) {
  // each trip a workgroup reads one contiguous 32 KiB span
  const size_t span = size_t(256) * kUnroll;
  size_t i = size_t(blockIdx.x) * span + threadIdx.x;
  const size_t stride = size_t(gridDim.x) * span;
  uint32_t acc = 0;
  for (; i + 256 * (kUnroll - 1) < n16; i += stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + 256 * u];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][3];
  }
  for (; i < n16; i += 256) acc ^= src[i][0];  // the last partial span
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// Every (sequence b, logical block j < its block count, KV head h) of the
// batch, two units per wave and trip in a grid-stride loop (heads fastest):
// the slabs of block tables[b][j] for head h in every array of its arena,
// 16 bytes per lane and load, all of a trip's loads issued before any is
// used.  RK: 1 KiB rounds of a K or V slab; NM: metadata arrays of a
// quantized body (scales, zeros: one round, the lanes inside the slab);
// quantized pools also hold FP16 sink-arena blocks (4 rounds of K and V, D =
// 128).  Table entries and lengths are read through the scalar cache one
// unit ahead.  Each workgroup folds the words it read by XOR into sink[0]
// with one atomic XOR: the result is the XOR of every word read.
typedef __attribute__((address_space(4))) const int32_t const_i32;

template <int RK, int NM>
__global__ __launch_bounds__(256) void paged_read_kernel(PoolDev p, const int32_t* __restrict__ tables,
                                                         const int32_t* __restrict__ lens, int batch,
                                                         int max_blocks, int max_seq_len, uint32_t* sink) {
  constexpr int kMeta[4] = {kArrKS, NM == 4 ? kArrKZ : kArrVS, kArrVS, kArrVZ};
  constexpr int kSinkRounds = 4;
  const int lane = threadIdx.x & 63;
  const int H = p.n_kv_heads, BS = p.block_size, N = p.num_blocks, NS = p.num_sink_blocks;
  const int units = batch * max_blocks * H;  // < 2^31 (checked on the host)
  const int nw = int(gridDim.x) * 4;
  const int per_seq = max_blocks * H;
  uint32_t acc = 0;
  auto fetch_info = [&](int u, int& id, int& L, int& j, int& h) {
    const int uu = u < units ? u : units - 1;
    const int b = uu / per_seq, r = uu - b * per_seq;
    j = r / H;
    h = r - j * H;
    L = *(const_i32*)(lens + b);
    id = *(const_i32*)(tables + size_t(b) * max_blocks + j);
  };
  auto ld = [&](int arr, size_t sid, uint32_t at, u32x4& v, bool& ok) {
    const uint32_t slab = uint32_t(p.slab[arr]);
    const uint32_t o = at + uint32_t(lane) * 16;
    ok = o < slab;
    v = *reinterpret_cast<const u32x4*>(p.base + p.off[arr] + sid * slab + (ok ? o : 0u));
  };
  // two units per trip (u and u + nw): all their loads in flight together
  int u = int(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int id0 = 0, L0 = 0, j0 = 0, h0 = 0, id1 = 0, L1 = 0, j1 = 0, h1 = 0;
  if (u < units) {
    fetch_info(u, id0, L0, j0, h0);
    fetch_info(u + nw, id1, L1, j1, h1);
  }
  constexpr int NB = 2 * RK + NM;  // loads of a body block
  constexpr int NK = 2 * kSinkRounds;
  constexpr int NV = NB > NK ? NB : NK;
  // one unit's loads into v (its kind decided on the scalar unit)
  auto issue = [&](int uu, int id, int L, int j, int h, u32x4 (&v)[NV], bool (&ok)[NV]) {
#pragma unroll
    for (int k = 0; k < NV; ++k) ok[k] = false;
    const int Lc = min(max(L, 0), max_seq_len);
    const bool live = uu < units && j * BS < Lc;
    if (live && id >= 0 && id < N) {
      const size_t sid = size_t(id) * H + h;
#pragma unroll
      for (int r = 0; r < RK; ++r) {
        ld(kArrK, sid, 1024u * r, v[r], ok[r]);
        ld(kArrV, sid, 1024u * r, v[RK + r], ok[RK + r]);
      }
#pragma unroll
      for (int m = 0; m < NM; ++m) ld(kMeta[m], sid, 0u, v[2 * RK + m], ok[2 * RK + m]);
    } else if (NM > 0 && live && id >= N && id < N + NS) {
      const size_t sid = size_t(id - N) * H + h;
#pragma unroll
      for (int r = 0; r < kSinkRounds; ++r) {
        ld(kArrSK, sid, 1024u * r, v[r], ok[r]);
        ld(kArrSV, sid, 1024u * r, v[kSinkRounds + r], ok[kSinkRounds + r]);
      }
    }
  };
  for (; u < units; u += 2 * nw) {
    u32x4 va[NV], vb[NV];
    bool oa[NV], ob[NV];
    issue(u, id0, L0, j0, h0, va, oa);
    issue(u + nw, id1, L1, j1, h1, vb, ob);
    fetch_info(u + 2 * nw, id0, L0, j0, h0);  // the next trip's entries, in flight meanwhile
    fetch_info(u + 3 * nw, id1, L1, j1, h1);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (oa[k]) acc ^= va[k][0] ^ va[k][1] ^ va[k][2] ^ va[k][3];
      if (ob[k]) acc ^= vb[k][0] ^ vb[k][1] ^ vb[k][2] ^ vb[k][3];
    }
  }
  // the workgroup's XOR: one atomic per workgroup
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (int(threadIdx.x) < o) red[threadIdx.x] ^= red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0 && red[0] != 0u) atomicXor(sink, red[0]);
}

// Plain zero fill, 16 bytes per thread and trip.
__global__ __launch_bounds__(256) void zero_kernel(u32x4* __restrict__ dst, size_t n16) {
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += size_t(gridDim.x) * 256)
    dst[i] = u32x4{0u, 0u, 0u, 0u};
}

}  // namespace

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const unsigned grid = unsigned(std::min<size_t>((n16 + 255) / 256, 1024));
  hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, s, static_cast<u32x4*>(p), n16);
  return hipGetLastError();
}

bool paged_read_supported(const PoolDev& p) {
  if (p.head_dim != 128) return false;
  if (p.kv_dtype == kInt4 || p.kv_dtype == kFp8) return true;
  return p.slab[kArrK] == 2048 || p.slab[kArrK] == 4096 || p.slab[kArrK] == 8192;
}

hipError_t launch_paged_read(const PoolDev& p, const int32_t* tables, const int32_t* lens, int32_t batch,
                             int32_t max_blocks, int32_t max_seq_len, void* sink, int grid, hipStream_t s) {
  uint32_t* sk = static_cast<uint32_t*>(sink);
  const dim3 g{unsigned(grid)}, b{256u};
  if (p.kv_dtype == kInt4)  // 1 KiB code slabs; scales and zeros of K and V
    hipLaunchKernelGGL((paged_read_kernel<1, 4>), g, b, 0, s, p, tables, lens, batch, max_blocks, max_seq_len, sk);
  else if (p.kv_dtype == kFp8)  // 2 KiB code slabs; the K and V scales
    hipLaunchKernelGGL((paged_read_kernel<2, 2>), g, b, 0, s, p, tables, lens, batch, max_blocks, max_seq_len, sk);
  else if (p.slab[kArrK] == 2048)
    hipLaunchKernelGGL((paged_read_kernel<2, 0>), g, b, 0, s, p, tables, lens, batch, max_blocks, max_seq_len, sk);
  else if (p.slab[kArrK] == 4096)
    hipLaunchKernelGGL((paged_read_kernel<4, 0>), g, b, 0, s, p, tables, lens, batch, max_blocks, max_seq_len, sk);
  else
    hipLaunchKernelGGL((paged_read_kernel<8, 0>), g, b, 0, s, p, tables, lens, batch, max_blocks, max_seq_len, sk);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, int grid, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(unsigned(grid)), dim3(256), 0, s,
                     static_cast<const u32x4*>(src), bytes / 16, static_cast<uint32_t*>(sink));
  return hipGetLastError();
}

}  // namespace pa
