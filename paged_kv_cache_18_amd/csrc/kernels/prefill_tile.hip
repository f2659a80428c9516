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
// workgroup of eight waves owns 256 (query, head) columns of one (sequence,
// KV head) -- 32 per wave, in two groups of four waves -- and streams every
// block its columns can see through LDS once for all eight, two blocks (32
// tokens) per step.  Each wave moves 2 KiB of the step (16 bytes per lane per
// load) from HBM straight into a four-slot LDS ring (global_load_lds_dwordx4:
// no register staging), two steps ahead.  No split: a workgroup sees all of
// its columns' tokens and writes the normalized rows itself.
//
// The two groups run in ping-pong, one wave of each on every SIMD: a group's
// products phase (P.V of one step, S^T of the next, operands already in
// registers) runs while the other group's softmax phase runs the
// exponentials and reads from LDS the operands of its own next products.  On
// this GPU a 32x32x16 product holds the SIMD's vector issue for about half
// of its 32 cycles, so the split keeps the matrix core fed while the vector
// work fills the other half.
//
// Per step and wave, on v_mfma_f32_32x32x16 (32 tokens x 32 columns):
//   S^T = K Q^T, 8 products over the 128 dimensions.  A = K: lane l reads the
//     16-byte chunk of token l % 32, dimensions 8 (l / 32) + 16 kk, which the
//     pool's K layout stores whole; B = Q^T from registers.  The result gives
//     lane l column l % 32 and 16 tokens, 8 (i / 4) + 4 (l / 32) + i % 4, so a
//     column's max or sum is 16 values in the lane plus one swap with lane
//     l ^ 32.
//   The causal mask (only for steps that reach past the wave's first column's
//     limit), the online softmax in the log2 domain with a lazily moved
//     reference, the weights split into a 16-bit high part and residual.
//   O^T += V^T P^T per 32-dimension tile, block by block, high part then
//     residual.  The score layout is the B operand as it stands: slot
//     8 (l / 32) + e of block t's product is the lane's score i = 8t + e, i.e.
//     token 16t + 8 (e / 4) + 4 (l / 32) + e % 4, and A = V^T takes the same
//     token order: lane (h = l / 32, m = l % 32) reads tokens 4h..4h+3 and
//     8+4h..8+4h+3 of dimension 8 (m / 2) + 2u + m % 2 (tile u), two 8-byte
//     pieces of the pool's V layout; each 16 consecutive lanes read 128
//     consecutive bytes.
#include "decode_common.hpp"

#include <type_traits>

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

typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

// c + A B on 32x32x16: lane l holds A[l % 32][8 (l / 32) .. + 7] and
// B[8 (l / 32) .. + 7][l % 32]; element i of the result is
// C[8 (i / 4) + 4 (l / 32) + i % 4][l % 32].
template <typename T>
struct Mma32;
template <>
struct Mma32<__bf16> {
  typedef __bf16 v8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
  static __device__ inline f32x16 run(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mma32<_Float16> {
  typedef _Float16 v8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
  static __device__ inline f32x16 run(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// the two values of lanes l and l ^ 32 (one swap of the wave's halves)
__device__ inline float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// p0, p1 (weights of two consecutive B-operand slots e, e + 1) as a 16-bit
// high part and the residual: p = hi + lo up to the residual's rounding.
// bf16: hi is p with the low 16 bits cut (the upper halves of both words
// in one byte permute), lo = p - hi exact in fp32, then rounded.
template <typename T, typename V8>
__device__ inline void split2(float p0, float p1, V8& hi, V8& lo, int e) {
  if constexpr (std::is_same<T, __bf16>::value) {
    const uint32_t h0 = __float_as_uint(p0) & 0xFFFF0000u, h1 = __float_as_uint(p1) & 0xFFFF0000u;
    const uint32_t hp = __builtin_amdgcn_perm(h1, h0, 0x07060302u);
    hi[e] = __builtin_bit_cast(__bf16, uint16_t(hp));
    hi[e + 1] = __builtin_bit_cast(__bf16, uint16_t(hp >> 16));
    lo[e] = T(p0 - __uint_as_float(h0));
    lo[e + 1] = T(p1 - __uint_as_float(h1));
  } else {
    const T a = T(p0), b = T(p1);
    hi[e] = a;
    hi[e + 1] = b;
    lo[e] = T(p0 - float(a));
    lo[e + 1] = T(p1 - float(b));
  }
}

constexpr int kGroupWaves = 4;                      // waves of one column group
constexpr int kPrefillWaves = 2 * kGroupWaves;       // two groups in ping-pong
constexpr int kWaveCols = 32;
constexpr int kGroupCols = kWaveCols * kGroupWaves;  // 128
constexpr int kPrefillCols = 2 * kGroupCols;         // (query, head) columns per workgroup
constexpr int kSlab = 16 * kD;                       // elements of one block's K or V slab
constexpr int kStepElems = 4 * kSlab;                // K of both blocks, then V of both
constexpr int kSlots = 4;

template <typename T>
__global__ __launch_bounds__(kPrefillWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void prefill_tile_kernel(
    DecodeArgs a, int ngrp) {
  typedef typename Mma32<T>::v8 v8;
  __shared__ __attribute__((aligned(16))) T ring[kSlots][kStepElems];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int gw = w / kGroupWaves;                                   // column group: 0 or 1
  const int hh = lane >> 5, n = lane & 31;
  const PoolDev& p = a.pool;
  const int H = p.n_kv_heads, Hq = a.n_q_heads, G = Hq / H, nq = a.n_query, N = p.num_blocks;
  const int ncols = nq * G;

  // workgroup -> (sequence b, KV head h, column tile grp).  Workgroups go to
  // the 8 XCDs round robin; the tiles of one (b, h) are placed on one XCD so
  // that its blocks come from that XCD's L2 after the first tile reads them.
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
  T* out = static_cast<T*>(a.out);

  // this lane's column col0 + n: query col / G, head h*G + col % G
  const int col0 = grp * kPrefillCols + kWaveCols * w;
  const int col = col0 + n;
  const bool colok = col < ncols;
  const int qi = colok ? col / G : 0, gi = colok ? col % G : 0;
  const size_t orow = (size_t(b) * nq + qi) * Hq + size_t(h) * G + gi;
  const int lim = colok ? L - nq + qi : -1;
  // x = s * scale; a negative scale runs as |scale| on -q (exact), so the
  // max of the raw scores scales to the max of x.  A zero scale runs as the
  // smallest normal float: every visible weight is still exp2(0) = 1 exactly,
  // and a masked score stays -inf instead of becoming -inf * 0 = NaN.
  const float sl2 = fmaxf(fabsf(a.scale_log2), __FLT_MIN__);
  const uint32_t qflip = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  v8 qf[8];
  {
    const T* qp = static_cast<const T*>(a.q) + orow * kD + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4 d = colok ? *reinterpret_cast<const u32x4*>(qp + 16 * kk) : u32x4{0u, 0u, 0u, 0u};
      d ^= qflip;
      qf[kk] = __builtin_bit_cast(v8, d);
    }
  }
  // tokens the workgroup's last column sees bound the blocks streamed
  const int last = min(ncols, (grp + 1) * kPrefillCols) - 1;
  const int seen = max(0, min(L, L - nq + last / G + 1));
  const int nblk = (seen + 15) >> 4;
  const int nstep = (nblk + 1) >> 1;
  // wave-uniform: the wave has a column to compute; its first column sees the
  // fewest tokens (a step wholly within that limit needs no mask and holds no
  // token at or past L)
  const bool active = col0 < ncols;
  const int minlim = L - nq + col0 / G;

  f32x16 o[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) o[u] = f32x16{};
  float m_ref = -__builtin_inff(), l_run = 0.f;

  // Step s_ (blocks 2 s_ and 2 s_ + 1) into LDS slot s_ % 4: 16 chunks of
  // 1 KiB (K of block 0, K of block 1, V of block 0, V of block 1, four each);
  // wave w moves chunks 2w and 2w + 1, lane l's 16 bytes at l * 16 of each.
  // Always issued, so the wait counts below are fixed: past the last block
  // it re-reads that block (masked where it is read).  The table entry is
  // read one step ahead, so the wait for that scalar load is off the path.
  // (Scalar work is kept short here: eight waves share the compute unit's
  // one scalar unit, and this runs every step.)
  const int cw = 2 * w;                      // first chunk of this wave
  const int cblk = (cw >> 2) & 1;            // its block within the step
  const T* wbase = (cw < 8 ? kbase : vbase) + size_t(h) * kSlab + (cw & 3) * 512;
  const uint32_t slab_stride = uint32_t(H) * kSlab;  // elements per block id
  const uint32_t loff = uint32_t(lane) * 8;
  const int jmax = max(nblk - 1, 0);
  auto entry = [&](int s_) { return table_entry(trow + min(2 * s_ + cblk, jmax)); };
  auto load = [&](int id_, int s_) {
    const uint32_t idv = uint32_t(id_) < uint32_t(N) ? uint32_t(id_) : 0u;
    const T* src = wbase + uint64_t(idv) * slab_stride + loff;
    T* dst = &ring[s_ & (kSlots - 1)][cw * 512];
    load_lds16(src, dst);
    load_lds16(src + 512, dst + 512);
  };

  // LDS element offsets of this lane's operand chunks within a slot
  const int kl = (n >> 4) * kSlab + (hh * 16 + (n & 15)) * 8;
  const int vl = 2 * kSlab + ((hh * 16 + (n >> 1)) * 2 + (n & 1)) * 4;

  // S^T of step s_: 8 products over the dimensions
  auto qk = [&](int s_) {
    const T* base = ring[s_ % kSlots];
    f32x16 sc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      sc = Mma32<T>::run(*reinterpret_cast<const v8*>(base + kl + kk * 256), qf[kk], sc);
    return sc;
  };

  // V of step s_ for block t, tile u: two 8-byte pieces
  auto vread = [&](const T* base, int t, int u) {
    const T* vp = base + vl + t * kSlab + u * 512;
    typedef T v4 __attribute__((__vector_size__(4 * sizeof(T))));
    const v4 p0 = *reinterpret_cast<const v4*>(vp);
    const v4 p1 = *reinterpret_cast<const v4*>(vp + 256);
    return v8{p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
  };

  // The operands of one products phase: V of step sv (both blocks, four
  // tiles) and K of step sk, read from LDS in the wave's softmax phase before
  // (the other group's matrix-core products run meanwhile).
  struct Ops {
    v8 vf[2][4];
    v8 kf[8];
  };
  auto fetch = [&](int sv, int sk, Ops& op) {
    const T* vb = ring[sv % kSlots];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 4; ++u) op.vf[t][u] = vread(vb, t, u);
    if (sk >= 0) {
      const T* kb = ring[sk % kSlots];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) op.kf[kk] = *reinterpret_cast<const v8*>(kb + kl + kk * 256);
    }
  };

  // O^T += V^T P^T (block by block, high part then residual) and, with QK,
  // S^T of the next step, from operands in registers; the S^T products go
  // between P.V ones, so no product waits on the one before.
  auto prod = [&](const Ops& op, bool with_qk, const v8 (&phi)[2], const v8 (&plo)[2]) {
    f32x16 acc = f32x16{};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = i >> 3, u = i & 3, lo = (i >> 2) & 1;
      o[u] = Mma32<T>::run(op.vf[t][u], lo ? plo[t] : phi[t], o[u]);
      if (with_qk && (i & 1)) acc = Mma32<T>::run(op.kf[i >> 1], qf[i >> 1], acc);
    }
    return acc;
  };

  // softmax of step s_ (scores sc) into the weights phi + plo.  masked: the
  // step reaches past the limit of the wave's first column (the causal
  // diagonal, the last step).
  auto soft = [&](const f32x16& sc, int s_, bool masked, v8 (&phi)[2], v8 (&plo)[2]) {
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = sc[i];
    if (masked) {
      const int t0 = 32 * s_ + 4 * hh;  // token of score i: t0 + 8 (i / 4) + i % 4
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = t0 + 8 * (i >> 2) + (i & 3) <= lim ? x[i] : -__builtin_inff();
    }
    // NaN-propagating maximum (v_maximum3_f32): no input quieting, and no
    // score is NaN here (a token past L is masked to -inf first)
    float bm = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[0], x[1]), x[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2)
      bm = __builtin_elementwise_maximum(__builtin_elementwise_maximum(bm, x[i]), x[i + 1]);
    bm = halves_max(__builtin_elementwise_maximum(bm, x[15])) * sl2;
    // the reference moves only when a step's max passes it by more than 8
    // (weights stay <= 2^8); numerator and denominator share it.  A column
    // that does not move keeps its sums as they are (alpha 1: with nothing
    // seen yet, m_ref - m_ref would be -inf - -inf).
    const bool move = bm > m_ref + 8.f;
    if (__any(move)) {
      const float alpha = move ? __builtin_amdgcn_exp2f(m_ref - bm) : 1.f;
      m_ref = move ? bm : m_ref;
      l_run *= alpha;
#pragma unroll
      for (int u = 0; u < 4; ++u) o[u] *= alpha;
    }
    // a column with nothing seen yet has m_ref = -inf and only masked
    // scores: against the most negative float they still weigh exp2(-inf) = 0
    const float mu = __builtin_elementwise_maximum(m_ref, -__FLT_MAX__);
    float ps[16];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], sl2, -mu));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i + 1], sl2, -mu));
      ps[i] = p0;
      ps[i + 1] = p1;
      split2<T>(p0, p1, phi[i >> 3], plo[i >> 3], i & 7);
    }
#pragma unroll
    for (int st = 1; st < 16; st *= 2)
#pragma unroll
      for (int i = 0; i < 16; i += 2 * st) ps[i] += ps[i + st];
    l_run += ps[0];
    // the weights are made here, in the softmax phase: without this the
    // compiler sinks their arithmetic past the barrier into the products
    // phase that reads them
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      u32x4 a0 = __builtin_bit_cast(u32x4, phi[t]), a1 = __builtin_bit_cast(u32x4, plo[t]);
      asm volatile("" : "+v"(a0), "+v"(a1));
      phi[t] = __builtin_bit_cast(v8, a0);
      plo[t] = __builtin_bit_cast(v8, a1);
    }
    asm volatile("" : "+v"(l_run));
  };

  // V of the last step's tokens at or past L is zeroed in LDS by the waves
  // that load it, once it has landed: unwritten slots may hold any bits (NaN
  // too), and a zero weight must not meet one.  In chunk u of a V slab lane
  // (g, r) = (l / 16, l % 16) holds tokens 4g..4g+3 (two dims, two tokens per
  // dword).
  auto zero_tail = [&](int s_) {
    if (cw < 8) return;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      u32x4* q = reinterpret_cast<u32x4*>(&ring[s_ % kSlots][(cw + k) * 512 + lane * 8]);
      const int tk = 32 * s_ + 16 * cblk + 4 * (lane >> 4);
      const uint32_t m01 = (tk < L ? 0x0000FFFFu : 0u) | (tk + 1 < L ? 0xFFFF0000u : 0u);
      const uint32_t m23 = (tk + 2 < L ? 0x0000FFFFu : 0u) | (tk + 3 < L ? 0xFFFF0000u : 0u);
      *q &= u32x4{m01, m23, m01, m23};
    }
  };

  // Ping-pong of the two column groups (one wave of each on every SIMD),
  // phase by phase with a barrier between phases.  Each group runs, phase
  // after phase, the products of step s (P.V of step s - 1, S^T of step s,
  // operands in registers) and then the softmax of step s, during which it
  // also reads from LDS the operands of its next products (V of step s, K of
  // step s + 1); group 1 starts one phase later.  So while one group's wave
  // keeps the SIMD's matrix core busy, the other's runs its exponentials and
  // its LDS reads.  Workgroup phase 2j holds group 0's products of step j and
  // group 1's softmax of step j - 1.  Step j must have landed by phase
  // 2j - 1 (group 0 reads K of step j in its softmax phase 2j - 1): it is
  // issued at phase 2j - 4 (two steps ahead, into the slot of step j - 4,
  // whose last reader ran in phase 2j - 6), and before the barrier of phase
  // 2j - 1 each wave waits for its own loads down to the two of step j + 1.
  // Both groups pass 2 nstep + 2 barriers.
  int ph = 0;
  int nid = entry(2);
  // The barrier is the bare s_barrier: a workgroup fence would also wait for
  // every load in flight (the prefetch of the next two steps).  Before it
  // each wave waits for its own LDS accesses (a slot's readers are done
  // before the slot is loaded again; the tail fix-up is written) and, at odd
  // phases, for its loads of the step the next phase starts.
  auto boundary = [&]() {
    if (ph & 1)
      asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)" ::: "memory");
    else
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if ((ph & 1) == 0) {
      const int j = ph >> 1;
      load(nid, j + 2);
      if (j == nstep - 1) zero_tail(j);
    }
    // the next entry is read at the start of this wave's softmax phase
    if (((ph - gw) & 1) == 1) nid = entry((ph >> 1) + 3);
    ++ph;
  };
  load(entry(0), 0);
  load(entry(1), 1);
  asm volatile("s_waitcnt vmcnt(2)" ::: "memory");  // step 0, published by the first barrier
  if (nstep > 0) {
    if (!active) {
      for (int k = 0; k < 2 * nstep + 2; ++k) boundary();
    } else {
      v8 phi[2], plo[2];
      Ops op;
      if (gw == 1) boundary();
      boundary();
      f32x16 sc = qk(0);
      for (int s_ = 0; s_ < nstep - 1; ++s_) {
        boundary();
        fetch(s_, s_ + 1, op);
        soft(sc, s_, 32 * s_ + 31 > minlim, phi, plo);
        boundary();
        sc = prod(op, true, phi, plo);
      }
      boundary();
      fetch(nstep - 1, -1, op);
      soft(sc, nstep - 1, true, phi, plo);
      boundary();
      prod(op, false, phi, plo);
      if (gw == 0) boundary();
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // normalized column: lane (hh, n) holds, of tile u, element i = row
  // m = 8 (i / 4) + 4hh + i % 4, dimension 8 (m / 2) + 2u + m % 2 -- for each
  // of its eight rows r = m / 2 = 4q + 2hh + jj (q = i / 4, jj = (i % 4) / 2)
  // the 8 dimensions 8r .. 8r + 7
  const float l = halves_sum(l_run);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (colok) {
    T* op = out + orow * kD;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        v8 v;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int par = 0; par < 2; ++par) v[2 * u + par] = T(o[u][4 * q + 2 * jj + par] * inv);
        *reinterpret_cast<v8*>(op + 8 * (4 * q + 2 * hh + jj)) = v;
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
