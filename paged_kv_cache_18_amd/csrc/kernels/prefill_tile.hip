// Chunked-prefill attention on the matrix cores, for 16-bit pools of 16-token
// blocks and head_dim 128.
//
// "The 8GB VRAM Breakthrough ...", section 5 ("Notice two critical details",
// item 1, "Chunked Prefill"): a long prompt is prefilled in 512-token
// chunks; each chunk's queries attend, causally, over everything the
// sequence has cached so far (earlier chunks plus the chunk itself, appended
// through the block table first).  Query qi of a chunk of n_query sits at
// position L - n_query + qi and sees tokens 0 .. L - n_query + qi.
//
// A chunk has many queries per KV block (n_query x G columns per KV head), so
// the work is a dense product and the design point differs from decode: a
// workgroup of eight waves owns 128 (query, head) columns of one (sequence,
// KV head) -- one 16-column tile per wave -- and streams every block that its
// columns can see through LDS once for all eight.  Each wave moves an eighth
// of the block (one 1 KiB chunk of K or of V, 16 bytes per lane) from HBM
// straight into a three-slot LDS ring (global_load_lds_dwordx4: no register
// staging); after a barrier every wave reads the whole K and V^T of the block
// in matrix-core operand order.  Two blocks are in flight while one is
// consumed.  Small waves (one tile) keep four of them per SIMD to hide each
// other's matrix-core and softmax latencies.  No split: a workgroup sees all
// of its columns' tokens and writes the normalized rows itself.
//
// Per block and wave the arithmetic is the decode kernel's (decode_mfma.hip):
// S^T = K Q^T with v_mfma_f32_16x16x32 per tile, the causal mask per column,
// the online softmax in the log2 domain with a lazily moved reference, the
// weights split into a 16-bit high part and residual, and O^T += V^T P^T per
// 16-dim row tile with both parts in one v_mfma_f32_16x16x32.
#include "decode_common.hpp"

namespace pa {

namespace {

using namespace dec;

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane
// (global_load_lds_dwordx4).  The builtin exists only for the device pass;
// the host pass compiles the kernel for its launch stub alone.
__device__ inline void load_lds16(const void* src, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
#endif
}

constexpr int kPrefillWaves = 8;
constexpr int kPrefillCols = 16 * kPrefillWaves;  // (query, head) columns per workgroup
constexpr int kSlotElems = 2 * 16 * kD;  // one block's K and V slabs

template <typename T>
__global__ __launch_bounds__(kPrefillWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void prefill_tile_kernel(
    DecodeArgs a, int ngrp) {
  typedef typename Mfma<T>::v8 v8;
  typedef typename Mfma<T>::v4 v4;
  __shared__ __attribute__((aligned(16))) T ring[3][kSlotElems];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 4, c = lane & 15;
  const PoolDev& p = a.pool;
  const int H = p.n_kv_heads, Hq = a.n_q_heads, G = Hq / H, nq = a.n_query, N = p.num_blocks;
  const int ncols = nq * G;

  // workgroup -> (sequence b, KV head h, column group grp).  Workgroups go to
  // the 8 XCDs round robin; the groups of one (b, h) are placed on one XCD so
  // that its blocks come from that XCD's L2 after the first group reads them.
  const int id = int(blockIdx.x), nbh = a.batch * H;
  int bh, grp;
  if (nbh % 8 == 0) {
    const int k = id / 8;
    bh = id % 8 + 8 * (k / ngrp);
    grp = k % ngrp;
  } else {
    bh = id / ngrp;
    grp = id % ngrp;
  }
  const int b = bh / H, h = bh % H;
  const int L = seq_len(a, b);
  const int32_t* trow = a.tables + size_t(b) * a.max_blocks_per_seq;
  const T* kbase = reinterpret_cast<const T*>(p.base + p.off[kArrK]);
  const T* vbase = reinterpret_cast<const T*>(p.base + p.off[kArrV]);
  const float sl2 = a.scale_log2;
  T* out = static_cast<T*>(a.out);

  // this wave's column col0 + c: query col / G, head h*G + col % G
  const int col0 = grp * kPrefillCols + 16 * w;
  const int col = col0 + c;
  const bool colok = col < ncols;
  const int qi = colok ? col / G : 0, gi = colok ? col % G : 0;
  const size_t orow = (size_t(b) * nq + qi) * Hq + size_t(h) * G + gi;
  const int lim = colok ? L - nq + qi : -1;
  v8 qf[4];
  {
    const T* qp = static_cast<const T*>(a.q) + orow * kD + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[kk] = colok ? *reinterpret_cast<const v8*>(qp + 32 * kk) : v8{};
  }
  // tokens the group's last column sees bound the blocks streamed
  const int last = min(ncols, (grp + 1) * kPrefillCols) - 1;
  const int seen = max(0, min(L, L - nq + last / G + 1));
  const int nblk = (seen + 15) >> 4;
  const bool active = col0 < ncols;  // wave-uniform: the wave has a column to compute

  f32x4 o[kNT];
#pragma unroll
  for (int T_ = 0; T_ < kNT; ++T_) o[T_] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -__builtin_inff(), l_run = 0.f;

  // this wave's eighth of block j into LDS slot `slot`: K chunk w (waves
  // 0..3) or V chunk w - 4 (waves 4..7), lane l's 16 bytes at l * 16 of the
  // chunk; a slot holds K then V, so chunk w lands at w * 512 elements.  One
  // load, always issued, so the wait counts below are fixed.  Past the last
  // block it re-reads that block into a slot nobody reads.
  const T* cbase = w < 4 ? kbase : vbase;
  auto load = [&](int j, int slot) {
    const int id_ = table_entry(trow + min(j, nblk - 1));
    const size_t slab = (size_t(id_ >= 0 && id_ < N ? id_ : 0) * H + h) * (16 * kD);
    load_lds16(cbase + slab + size_t(w & 3) * 512 + size_t(lane) * 8, &ring[slot][w * 512]);
  };

  // block j from LDS slot `slot`: S^T, causal mask, online softmax, O^T += V^T P^T
  auto consume = [&](int slot, int j) {
    if (!active) return;
    v8 kf[4], vf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kf[kk] = *reinterpret_cast<const v8*>(&ring[slot][kk * 512 + lane * 8]);
#pragma unroll
    for (int u = 0; u < 4; ++u) vf[u] = *reinterpret_cast<const v8*>(&ring[slot][2048 + u * 512 + lane * 8]);
    const int valid = min(16, L - 16 * j);
    if (valid < 16) {
      // unwritten tail slots may hold any bits (NaN too): zero them so a zero
      // weight never meets one; each dword holds two tokens
      const int t0 = 4 * g;
      const uint32_t m01 = (t0 + 0 < valid ? 0x0000FFFFu : 0u) | (t0 + 1 < valid ? 0xFFFF0000u : 0u);
      const uint32_t m23 = (t0 + 2 < valid ? 0x0000FFFFu : 0u) | (t0 + 3 < valid ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        u32x4 dw = __builtin_bit_cast(u32x4, vf[u]);
        dw[0] &= m01;
        dw[1] &= m23;
        dw[2] &= m01;
        dw[3] &= m23;
        vf[u] = __builtin_bit_cast(v8, dw);
      }
    }
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) sc = Mfma<T>::qk(kf[kk], qf[kk], sc);
    float x[4];
    bool vis[4];
    float bm = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 16 * j + 4 * g + i;
      vis[i] = 4 * g + i < valid && tok <= lim;
      x[i] = vis[i] ? sc[i] * sl2 : -__builtin_inff();
      bm = fmaxf(bm, x[i]);
    }
    bm = rows_max(bm);
    // the reference moves only when a block's max passes it by more than 8
    // (weights stay <= 2^8); numerator and denominator share it
    const bool move = bm > m_ref + 8.f;
    if (__any(move)) {
      const float m_new = move ? bm : m_ref;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      l_run *= alpha;
#pragma unroll
      for (int T_ = 0; T_ < kNT; ++T_) o[T_] *= alpha;
      m_ref = m_new;
    }
    v4 phi, plo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pw = vis[i] ? __builtin_amdgcn_exp2f(x[i] - m_ref) : 0.f;
      l_run += pw;
      phi[i] = T(pw);
      plo[i] = T(pw - float(phi[i]));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const v4 vt = {vf[u][4 * par + 0], vf[u][4 * par + 1], vf[u][4 * par + 2], vf[u][4 * par + 3]};
        o[2 * u + par] = Mfma<T>::pv2(vt, phi, plo, o[2 * u + par]);
      }
    }
  };

  if (nblk > 0) {
    // block j lives in slot j % 3.  At the top of step j this wave's loads of
    // blocks j and j + 1 are outstanding (one each): waiting down to one
    // leaves block j + 1 in flight; the barrier then publishes every wave's
    // eighth of block j and frees the slot of block j - 1 for block j + 2.
    load(0, 0);
    load(1, 1);
    for (int j = 0; j < nblk; ++j) {
      asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
      __syncthreads();
      load(j + 2, (j + 2) % 3);
      consume(j % 3, j);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // normalized row: lane (g, c) holds dims 32g + 8i + T of its column
  const float l = rows_sum(l_run);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (colok) {
    T* op = out + orow * kD + 32 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v8 v;
#pragma unroll
      for (int T_ = 0; T_ < kNT; ++T_) v[T_] = T(o[T_][i] * inv);
      *reinterpret_cast<v8*>(op + 8 * i) = v;
    }
  }
}

}  // namespace

int prefill_tile_groups(int32_t n_query, int32_t n_q_heads, int32_t n_kv_heads) {
  return (n_query * (n_q_heads / n_kv_heads) + kPrefillCols - 1) / kPrefillCols;
}

hipError_t launch_prefill_tile(const DecodeArgs& a, hipStream_t s) {
  const int ngrp = prefill_tile_groups(a.n_query, a.n_q_heads, a.pool.n_kv_heads);
  const dim3 grid(unsigned(a.batch) * unsigned(a.pool.n_kv_heads) * unsigned(ngrp)), block(kPrefillWaves * 64);
  if (a.q_dtype == kBF16)
    hipLaunchKernelGGL(prefill_tile_kernel<__bf16>, grid, block, 0, s, a, ngrp);
  else
    hipLaunchKernelGGL(prefill_tile_kernel<_Float16>, grid, block, 0, s, a, ngrp);
  return hipGetLastError();
}

}  // namespace pa
