// Shared pieces of the matrix-core decode split kernels (decode_mfma.hip for
// 16-bit pools, decode_quant.hip for INT4/FP8 pools): the flattened work
// list and its units, the per-piece iteration, and the 4-wave merge.
//
// Work list: the blocks of every (sequence b, KV head h) segment laid end to
// end, h major, then b, then logical block j, so every KV head (segment index
// hv, with column slices) has a list of the same TB blocks.  Normally each
// head's list is cut into q = grid / heads regions of C blocks (a region never
// holds two heads); otherwise (grid not a multiple of the heads, or a queue or
// fixed region size asked for) the whole list is cut into regions of C
// blocks.  One region per workgroup of the persistent grid; which workgroup
// owns which region is the kernel's choice (see Units).  The first Cs blocks of a
// region are its owner's; the rest are cut into units of U blocks that any
// workgroup takes, in order, from a queue once it has streamed its own prefix
// (compute units and XCDs do not stream at the same rate, so equal shares
// would not finish together).  The cut is fixed by the shapes alone; only who
// streams a unit varies.  A segment inside one unit is finished in place
// (normalized, written to out); a segment crossing units leaves a partial
// (max, sum, weighted sum) in the unit's slot 0 (its first piece there) or
// slot 1 (a later one), and the workgroup that writes the segment's last
// partial (counted on an arrival counter) merges them all, in unit order: one
// launch does the whole decode and the result does not depend on the timing.
#pragma once

#include "common.hpp"

namespace pa {
namespace dec {

constexpr int kD = 128;       // head_dim of the matrix-core kernels
constexpr int kNT = kD / 16;  // 16-dim output tiles (tile T row r = dim 8r + T)
constexpr int kWaves = 4;     // wavefronts per workgroup

typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

template <typename T>
struct Mfma;
// pv(a, b, c): c + A B on 16x16x16 (A = a: lane (g, r) holds A[r][4g..4g+3];
// B = b: lane (g, c) holds B[4g..4g+3][c]).  pv2(a, hi, lo, c) = pv(a, hi,
// pv(a, lo, c)) up to fp32 rounding in one 16x16x32 product: lane group g
// covers k = 8g..8g+7 there, and k = 8g + e is paired with token 4g + (e & 3)
// of part e / 4 -- A = (a, a), B = (hi, lo), so no value moves across lanes.

template <>
struct Mfma<__bf16> {
  typedef __bf16 v8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
  typedef __bf16 v4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
  static __device__ inline f32x4 qk(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ inline f32x4 pv(v4 a, v4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  // a (hi + lo) in one 16x16x32 product (see pv2 below)
  static __device__ inline f32x4 pv2(v4 a, v4 hi, v4 lo, f32x4 c) {
    return qk(v8{a[0], a[1], a[2], a[3], a[0], a[1], a[2], a[3]},
              v8{hi[0], hi[1], hi[2], hi[3], lo[0], lo[1], lo[2], lo[3]}, c);
  }
};

template <>
struct Mfma<_Float16> {
  typedef _Float16 v8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
  typedef _Float16 v4 __attribute__((__vector_size__(4 * sizeof(_Float16))));
  static __device__ inline f32x4 qk(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ inline f32x4 pv(v4 a, v4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  static __device__ inline f32x4 pv2(v4 a, v4 hi, v4 lo, f32x4 c) {
    return qk(v8{a[0], a[1], a[2], a[3], a[0], a[1], a[2], a[3]},
              v8{hi[0], hi[1], hi[2], hi[3], lo[0], lo[1], lo[2], lo[3]}, c);
  }
};

// Workgroup barrier for data exchanged through LDS only: waits for this
// wave's LDS operations (not for its vector-memory loads, which stay in
// flight across it), and keeps LDS accesses on their side of it.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A block-table entry at a wave-uniform index, read through the scalar
// (constant) cache: the tables are read-only for the whole call.  A plain
// load becomes a vector load here (the kernels store to other buffers), and
// its result needs a wait on the vector-memory counter, which also waits for
// the K/V blocks already in flight.
typedef __attribute__((address_space(4))) const int32_t const_i32;
__device__ inline int table_entry(const int32_t* p) { return *(const_i32*)p; }

// Max / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48)
// with the gfx950 row-swap instructions: plain vector ALU, so no LDS round
// trip (whose counter wait would also wait for pending scalar loads).  Each
// swap returns the lane's own value and its partner row's, in some order.
__device__ inline float rows_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float rows_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline int seq_len(const DecodeArgs& a, int b) {
  return min(max(a.lens[b], 0), a.max_seq_len);
}

__device__ inline int seq_blocks(const DecodeArgs& a, int b) { return (seq_len(a, b) + 15) >> 4; }

// Segments per sequence: one per KV head and column slice.
__device__ inline int seg_heads(const DecodeArgs& a) { return a.pool.n_kv_heads * max(a.col_slices, 1); }

// LDS of a workgroup: per wave and output column (max, sum, acc) of the
// current piece, reused as scratch by the segment merge.
// Sequence lengths, and the running sums of their list positions, kept in
// LDS by setup_units for the first kLenCap sequences (later ones are read
// from memory where needed).
constexpr int kLenCap = 512;

// CAP output columns; NV stash slots (one per wave, or per wave of a pair
// when the waves split the column tiles).
template <int CAP, int NV = kWaves>
struct SharedT {
  static constexpr int kSlots = NV;
  int len[kLenCap];
  int pre[kLenCap];  // blocks of sequences 0..b: the place after b in every head's list
  float m[NV][CAP];
  float l[NV][CAP];
  alignas(16) float o[NV][CAP][kD + 1];
  int b, fb;
  int units[10];
  int next;
  int last;
};
using Shared = SharedT<16>;

// Length (tokens) and blocks of sequence b, from the LDS copy where it has one.
template <class SH>
__device__ inline int len_of(const DecodeArgs& a, const SH& sh, int b) {
  return b < kLenCap ? sh.len[b] : seq_len(a, b);
}
template <class SH>
__device__ inline int blocks_of(const DecodeArgs& a, const SH& sh, int b) {
  return (len_of(a, sh, b) + 15) >> 4;
}

// Output columns of a segment (b, hv), hv = h*nsl + s (KV head h, column
// slice s of SW columns): its column col is the (query, head) column
// gc = s*SW + col = qi*G + gi, query qi of the sequence's n_query (1 for
// decode) and query head h*G + gi, stored at row (b*n_query + qi)*Hq + h*G + gi
// of out ([batch][n_query][Hq][D]).  The last slice may hold fewer columns.
struct OutMap {
  int G, Hq, nq, nsl, SW;
  __device__ int ncol() const { return SW; }
  __device__ int cols(int hv) const { return min(SW, nq * G - (hv % nsl) * SW); }
  __device__ int gcol(int hv, int col) const { return (hv % nsl) * SW + col; }
  __device__ size_t row(int b, int hv, int col) const {
    const int gc = gcol(hv, col);
    return (size_t(b) * nq + gc / G) * Hq + (hv / nsl) * G + gc % G;
  }
};

__device__ inline OutMap out_map(const DecodeArgs& a) {
  const int G = a.n_q_heads / a.pool.n_kv_heads, nq = max(a.n_query, 1), nsl = max(a.col_slices, 1);
  return OutMap{G, a.n_q_heads, nq, nsl, nsl > 1 ? a.slice_cols : nq * G};
}

// The cut of the work list (see the top of this file).  Unit ids grow with
// position: region r holds units r*(1+m) (its prefix) .. r*(1+m)+m; with the
// per-head cut (n = TB > 0, no queue: m = 0) unit h*q + k is region k of
// head h's list.
//
// Owners.  Workgroups go to the 8 XCDs round robin.  owned_by_head gives
// region k of head h to workgroup k*heads + h, so with 8 heads each XCD
// streams one head's slabs of every block (the 16-bit kernel: 2 % shorter on
// the ragged Llama-3-8B-shaped batch than with unit = workgroup).  The
// identity (owned) gives the regions over the same blocks of different heads
// to workgroups h*q + k, on one XCD when q is a multiple of 8, where the
// quantized kernel's scale and zero rows of several heads, which share cache
// lines, are fetched once.
struct Units {
  int W;   // blocks in the list
  int R;   // regions (= the grid)
  int C;   // blocks per region
  int Cs;  // owner's prefix of a region, >= 1
  int U;   // blocks per queued unit
  int m;   // queued units per region
  int n;   // list length of the per-head cut (= TB), 0 = one cut of the whole list
  int TB;  // blocks of one head's list: W = TB * heads
  int hs;  // heads (segment indices) of the per-head cut, else 0
  int q;   // regions per head (per-head cut)
  __device__ int per() const { return 1 + m; }
  __device__ int owned(int bid) const { return bid * per(); }
  __device__ int owned_by_head(int bid) const { return hs > 0 ? (bid % hs) * q + bid / hs : bid * per(); }
  __device__ int total() const { return R * per(); }
  __device__ int unit_of(int p) const {
    if (n > 0) {
      const int s = p / n;
      return s * q + (p - s * n) / C;
    }
    const int r = p / C, o = p - r * C;
    return r * per() + (o < Cs ? 0 : 1 + (o - Cs) / U);
  }
  __device__ int start(int u) const {
    if (n > 0) {
      const int s = u / q;
      return min(W, s * n + min((u - s * q) * C, n));
    }
    const int r = u / per(), k = u - r * per();
    return r * C + (k == 0 ? 0 : Cs + (k - 1) * U);
  }
  __device__ int end(int u) const {
    if (n > 0) {
      const int s = u / q;
      return min(W, s * n + min((u - s * q + 1) * C, n));
    }
    const int r = u / per(), k = u - r * per();
    return min(W, r * C + (k == 0 ? Cs : min(C, Cs + k * U)));
  }
  // q-th unit of the queue: the first queued unit of every region, then the
  // second, ...
  __device__ int queued(int q) const { return (q % R) * per() + 1 + q / R; }
};

// The cut of a list of TB blocks per segment (wave-uniform arithmetic).
__device__ inline Units cut_of(const DecodeArgs& a, int TB) {
  const int W = TB * seg_heads(a);
  const int R = a.max_splits;  // the split kernel's grid
  int C, Cs, U = 1, m = 0, n = 0, q = 0, hs = 0;
  if (a.split_blocks > 0) {
    C = Cs = a.split_blocks;
  } else {
    C = max(1, (W + R - 1) / R);
    Cs = C;
    if (a.unit_blocks > 0 && a.static_permille < 1000) {
      U = a.unit_blocks;
      Cs = max(1, int(int64_t(C) * max(a.static_permille, 0) / 1000));
      m = (C - Cs + U - 1) / U;
    } else if (R % seg_heads(a) == 0 && TB > 0) {
      hs = seg_heads(a);
      n = TB;
      q = R / hs;
      C = Cs = (TB + q - 1) / q;
    }
  }
  return Units{W, R, C, Cs, U, m, n, TB, hs, q};
}

// Wave 0 reads the lengths (one load per sequence, kept in LDS for the
// first kLenCap) and sizes the cut from them; every thread gets both.
template <class SH>
__device__ inline Units setup_units(const DecodeArgs& a, SH& sh, int w, int lane) {
  if (w == 0) {
    int W = 0;
    for (int base = 0; base < a.batch; base += 64) {
      const int bb = base + lane;
      const int L = bb < a.batch ? seq_len(a, bb) : 0;
      const int sz = (L + 15) >> 4;
      int incl = sz;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      if (bb < min(a.batch, kLenCap)) {
        sh.len[bb] = L;
        sh.pre[bb] = W + incl;
      }
      W += __shfl(incl, 63, 64);
    }
    const Units u = cut_of(a, W);
    if (lane == 0) {
      sh.units[0] = u.W;
      sh.units[1] = u.R;
      sh.units[2] = u.C;
      sh.units[3] = u.Cs;
      sh.units[4] = u.U;
      sh.units[5] = u.m;
      sh.units[6] = u.n;
      sh.units[7] = u.q;
      sh.units[8] = u.TB;
      sh.units[9] = u.hs;
    }
  }
  __syncthreads();
  return Units{sh.units[0], sh.units[1], sh.units[2], sh.units[3], sh.units[4], sh.units[5], sh.units[6], sh.units[8], sh.units[9], sh.units[7]};
}

// ---- The cut with the lengths in registers (batches of at most 64) ----------
// Every wave reads the lengths itself, lane b holding sequence b, and keeps
// the running sum of their block counts in a register: the cut, the
// sequence holding a position and each piece's bounds then come from
// cross-lane reads of registers, with no LDS traffic and no workgroup barrier
// ahead of the first block loads.  A launch takes this form when the batch
// fits one wave and no queue is asked for (every workgroup streams exactly
// its own region).
constexpr int kRegLens = 64;

struct RegLens {
  int len;   // lane b: the length of sequence b (0 past the batch)
  int incl;  // lane b: blocks of sequences 0..b
  __device__ int len_of(int b) const { return __builtin_amdgcn_readlane(len, b & 63); }
  __device__ int blocks_of(int b) const { return (len_of(b) + 15) >> 4; }
};

// Inclusive running sum over the 64 lanes: shifts inside each row of 16
// lanes, then each row's total carried into the rows above it.
__device__ inline int wave_incl_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}

__device__ inline RegLens reg_lens(const DecodeArgs& a, int lane) {
  RegLens r;
  r.len = lane < a.batch ? seq_len(a, lane) : 0;
  r.incl = wave_incl_sum((r.len + 15) >> 4);
  return r;
}

__device__ inline Units reg_units(const DecodeArgs& a, const RegLens& rl) {
  return cut_of(a, __builtin_amdgcn_readlane(rl.incl, 63));
}

// The sequence b holding position p0 and the place fb of its first block in
// its head's list, from the running sums.
__device__ inline void reg_locate(const Units& um, const RegLens& rl, int p0, int& b, int& fb) {
  const int r0 = p0 % um.TB;
  const unsigned long long hit = __ballot(rl.incl > r0);  // lanes past the batch hold TB
  b = hit ? __builtin_ctzll(hit) : 64;
  fb = b > 0 ? __builtin_amdgcn_readlane(rl.incl, (b - 1) & 63) : 0;
}

// The sequence b holding position p0 and the place fb of its first block in
// its head's list (p0 = h * TB + fb + j).  Every wave reads them from the running sums in LDS where the batch fits
// there; otherwise wave 0 scans the lengths and every thread gets them.
template <class SH>
__device__ inline void locate(const DecodeArgs& a, SH& sh, const Units& um, int w, int lane, int p0, int& b,
                              int& fb) {
  const int B = a.batch;
  const int r0 = p0 % um.TB;
  if (B <= kLenCap) {
    b = B;
    fb = 0;
    for (int base = 0; base < B; base += 64) {
      const int bb = base + lane;
      const unsigned long long hit = __ballot(bb < B && sh.pre[bb] > r0);
      if (hit) {
        b = base + __builtin_ctzll(hit);
        fb = b > 0 ? __builtin_amdgcn_readfirstlane(sh.pre[b - 1]) : 0;
        break;
      }
    }
    return;
  }
  if (w == 0) {
    int run = 0, f = 0, fbi = B;
    for (int base = 0; base < B; base += 64) {
      const int bb = base + lane;
      const int sz = bb < B ? blocks_of(a, sh, bb) : 0;
      int incl = sz;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      const unsigned long long hit = __ballot(run + incl > r0);
      if (hit) {
        const int fl = __builtin_ctzll(hit);
        fbi = base + fl;
        f = run + __shfl(incl - sz, fl, 64);
        break;
      }
      run += __shfl(incl, 63, 64);
    }
    if (lane == 0) {
      sh.b = fbi;
      sh.fb = f;
    }
  }
  __syncthreads();
  b = sh.b;
  fb = sh.fb;
}

// Arrival counters: word 0 is the unit queue, unit u's counter is word
// (1 + u) (times the stride).
__device__ inline unsigned* unit_counter(const DecodeArgs& a, int u) {
  return a.counters + size_t(1 + u) * a.ctr_stride;
}

// The next unit this workgroup streams: its own prefix first (start = its
// region's prefix id), then units from the queue; -1 when the queue is empty.
// Every workgroup ends with exactly one refused take, so the take that sees
// count R*m + R - 1 is the call's last and resets the queue to 0.
template <class SH>
__device__ inline int next_unit(const DecodeArgs& a, SH& sh, const Units& um) {
  if (um.m == 0) return -1;
  if (threadIdx.x == 0) {
    const unsigned nq = unsigned(um.R) * unsigned(um.m);
    int u = -1;
    while (true) {
      const unsigned q = __hip_atomic_fetch_add(a.counters, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (q + 1 == nq + unsigned(um.R)) __hip_atomic_store(a.counters, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (q >= nq) break;
      const int cand = um.queued(int(q));
      if (um.start(cand) < um.end(cand)) {
        u = cand;
        break;
      }
    }
    sh.next = u;
  }
  __syncthreads();
  const int u = sh.next;
  __syncthreads();
  return u;
}


// Zero the output rows of empty sequences (no piece covers them); workgroup
// c takes sequences c, c + grid, ...  blocks(b): the block count of sequence b.
template <typename TO, class BK>
__device__ inline void zero_empty_rows(const DecodeArgs& a, BK blocks) {
  const int Hq = a.n_q_heads, nq = max(a.n_query, 1);
  TO* out = static_cast<TO*>(a.out);
  for (int b = blockIdx.x; b < a.batch; b += gridDim.x)
    if (blocks(b) == 0)
      for (int i = threadIdx.x; i < nq * Hq * kD; i += kWaves * 64)
        out[size_t(b) * nq * Hq * kD + i] = TO(0.f);
}

// The next piece [jbeg, jend) of segment (b, h) starting at position pos;
// advances (b, fb) past finished or empty sequences, back to the first
// sequence where pos enters the next head's list.  False when done.
template <class BK>
__device__ inline bool next_piece(const DecodeArgs& a, BK blocks, const Units& um, int pos, int pos1,
                                  int& b, int& fb, int& h, int& jbeg, int& jend, int& nb) {
  while (pos < pos1) {
    const int hv = pos / um.TB, r = pos - hv * um.TB;
    if (r < fb) {
      b = 0;
      fb = 0;
    }
    if (b >= a.batch) return false;
    nb = blocks(b);
    if (r >= fb + nb) {
      fb += nb;
      ++b;
      continue;
    }
    h = hv;
    jbeg = r - fb;
    jend = min(nb, jbeg + (pos1 - pos));
    return true;
  }
  return false;
}

// A decode step that appends its own new token (a.app_k set; 16-bit pools
// of head_dim 128 with inputs of the pool's dtype).  Token L - 1 of
// sequence b, KV head h, is written by the wave that will read the segment's
// last block (tile nb - 1, in the piece holding it): the wave loads the
// token's K and V words (lane l: dims 2l, 2l + 1) before its pipeline's
// first loads, and stores them into the slot its table row gives right
// before it issues the load of that block.  A wave's own memory operations
// are performed in order, so its load of the block sees the stores; no
// other wave reads the block.  Column slices of one head: the first slice's wave
// writes.
struct NewToken {
  uint32_t k = 0, v = 0;  // the lane's two K and two V values
  bool on = false;
};

__device__ inline NewToken new_token_load(const DecodeArgs& a, int lane, int b, int hv, int nsl,
                                          int jw, int nst, int jend, int nb, int L) {
  NewToken nt;
  nt.on = a.app_k != nullptr && jend == nb && nb > 0 && L >= 1 && hv % nsl == 0 && nb - 1 >= jw &&
          (nb - 1 - jw) % nst == 0;
  if (nt.on) {
    const size_t row = (size_t(b) * a.pool.n_kv_heads + hv / nsl) * kD + 2 * lane;
    nt.k = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.app_k) + row);
    nt.v = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.app_v) + row);
  }
  return nt;
}

__device__ inline void new_token_store(const DecodeArgs& a, const NewToken& nt, int lane, int hv,
                                       int nsl, int L, const int32_t* trow) {
  if (!nt.on) return;
  const PoolDev& p = a.pool;
  const int H = p.n_kv_heads, h = hv / nsl, bs = p.block_size;
  const int id = table_entry(trow + (L - 1) / bs), t = (L - 1) % bs;
  if (id < 0 || id >= p.num_blocks) return;
  const size_t sid = size_t(id) * H + h;
  uint16_t* ks = reinterpret_cast<uint16_t*>(p.base + p.off[kArrK] + sid * p.slab[kArrK]);
  uint16_t* vs = reinterpret_cast<uint16_t*>(p.base + p.off[kArrV] + sid * p.slab[kArrV]);
  *reinterpret_cast<uint32_t*>(ks + raw_k_elem(t, 2 * lane, bs)) = nt.k;
  vs[raw_v_elem(t, 2 * lane, kD, bs)] = uint16_t(nt.v & 0xFFFFu);
  vs[raw_v_elem(t, 2 * lane + 1, kD, bs)] = uint16_t(nt.v >> 16);
}

// Wave issue priority from the share of its chunk a workgroup still has to
// stream (done of C blocks): bands above 1/2, 1/4 and 1/16 remaining.  With
// equal chunks, the workgroups a compute unit holds would otherwise progress
// in dispatch order (older waves win issue arbitration) and the youngest
// would finish last; this lets the ones behind catch up.
//
// ELDER (the 16-bit kernel): the grid's first half, dispatched first, runs
// one band lower at equal progress, so that the second half's workgroup on
// the same compute unit keeps pace from the start (the quantized kernel
// measured slower with it).
template <bool ELDER = false>
__device__ inline void prio_from_progress(const DecodeArgs& a, int done, int C) {
  if (!a.prio) return;
  const int r = max(C - done, 0);
  if constexpr (ELDER) {
    if (int(blockIdx.x) < int(gridDim.x) / 2) {
      if (2 * r > C)
        __builtin_amdgcn_s_setprio(2);
      else if (4 * r > C)
        __builtin_amdgcn_s_setprio(1);
      else
        __builtin_amdgcn_s_setprio(0);
      return;
    }
  }
  if (2 * r > C)
    __builtin_amdgcn_s_setprio(3);
  else if (4 * r > C)
    __builtin_amdgcn_s_setprio(2);
  else if (16 * r > C)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// Partials cross workgroups (and the XCDs' separate L2 caches) through
// agent-scope relaxed atomic stores and loads: these write through to, and
// read from, the level every XCD shares, so no L2 write-back or invalidate
// (what an agent-scope fence costs, for every line of the cache) is needed.
// The writer waits for its stores to complete before it counts its arrival;
// the reader loads only after the arrival that completes the segment.
__device__ inline void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Count this workgroup's arrival on the counter of unit c0, the first unit of
// a segment of np pieces (a unit starts at most one segment that runs past its
// end, so c0 names the segment); true for the arrival that completes the
// segment, which resets the counter to 0 for the next call.
__device__ inline bool arrive(const DecodeArgs& a, int c0, int np) {
  unsigned* ctr = unit_counter(a, c0);
  const unsigned old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool last = old + 1 == unsigned(np);
  if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return last;
}

// The merge launch's job for segment (b, hs), which starts at position S of
// the list and has nb blocks: its first unit (bit 31: its first piece is in
// that unit's second slot) and its piece count.  Written, every call, by the
// workgroup of the segment's first piece; read after the split launch ends.
__device__ inline void write_job(const DecodeArgs& a, const Units& um, int b, int hs, int S, int nb) {
  const int c0 = um.unit_of(S), np = um.unit_of(S + nb - 1) - c0 + 1;
  int32_t* j = a.jobs + 2 * (size_t(b) * seg_heads(a) + hs);
  j[0] = int32_t(unsigned(c0) | (S != um.start(c0) ? 0x80000000u : 0u));
  j[1] = np;
}

// Buffer resource word 3 for plain dword-addressed buffers on gfx950, and the
// cache-policy bit of a buffer load that reads at agent scope (sc1).
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kSc1 = 16;

// Merge the np partials of segment (b, h), which starts at position S of the
// list, and write out.  Its first unit c0 holds its piece in slot 1 unless
// the segment starts the unit, every later unit in slot 0.  Thread (pg, col)
// folds pieces pg, pg + P, ... of one 16-byte output column with a running
// log-sum-exp (m, l, acc), kMergeBatch pieces in flight; each batch's (max,
// sum) pairs are loaded once (one per thread, issued with the partial sums)
// and shared through LDS.  The P piece groups of a column are then folded in
// order through LDS:
//   m = max m_i, l = sum l_i 2^(m_i - m), o = sum o_i 2^(m_i - m) / l.
// The order is fixed, so the result does not depend on arrival order.
constexpr int kMergeBatch = 12;  // 16 spills at three waves per SIMD

struct Lse {
  float m, l;
  f32x4 o;
  __device__ void add(float mi, float li, f32x4 oi) {
    if (mi == -__builtin_inff()) return;  // a piece of no token
    const float mn = fmaxf(m, mi);
    const float sa = exp2f(m - mn), sb = exp2f(mi - mn);
    o = o * sa + oi * sb;
    l = l * sa + li * sb;
    m = mn;
  }
  // N pieces at once: their common maximum first, then every piece's weight
  // on its own (no chain of rescales); a piece of max -inf (no token) adds
  // nothing.
  template <int N>
  __device__ void add_all(const float (&mi)[N], const float (&li)[N], const f32x4 (&oi)[N]) {
    float mn = m;
#pragma unroll
    for (int u = 0; u < N; ++u) mn = fmaxf(mn, mi[u]);
    if (mn == -__builtin_inff()) return;  // nothing seen yet
    const float sa = m == -__builtin_inff() ? 0.f : exp2f(m - mn);
    float ln = l * sa;
    f32x4 on = o * sa;
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const bool none = mi[u] == -__builtin_inff();
      const float w = exp2f(mi[u] - mn);
      ln += none ? 0.f : li[u] * w;
      on += none ? f32x4{0.f, 0.f, 0.f, 0.f} : oi[u] * w;
    }
    m = mn;
    l = ln;
    o = on;
  }
};

// c0: the segment's first unit; split_first: its first piece sits in that
// unit's second slot; rows: the partial rows the workspace holds (bounds of
// the buffer loads).
// ALL: each batch's pieces at once with a common maximum (Lse::add_all; the
// merge launch), else one at a time (Lse::add; the split kernels, whose
// registers the batched form crowds).
// WIDE (the split kernels): slices of 9-24 columns with up to 4 pieces take
// one memory round trip.
template <typename TO, class SH, bool ALL = false, bool WIDE = false>
__device__ inline void merge_segment(const DecodeArgs& a, SH& sh, const OutMap& om, int b, int h,
                                     int c0, bool split_first, int np, unsigned rows, int col0,
                                     int ncol) {
  const int NC = om.ncol();
  auto row_of = [&](int i) -> unsigned {  // workspace row of column 0 of piece i
    return unsigned((c0 + i) * 2 + ((i == 0 && split_first) ? 1 : 0)) * unsigned(NC);
  };
  const __amdgpu_buffer_rsrc_t ro =
      __builtin_amdgcn_make_buffer_rsrc(a.ws_o, (short)0, int(rows * kD * 4), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rml =
      __builtin_amdgcn_make_buffer_rsrc(a.ws_ml, (short)0, int(rows * 8), kRsrcWord3);
  constexpr int kCols = kD / 4;           // float4 columns of one output column
  float* red = &sh.o[0][0][0];            // [256][6]: m, l, o of each thread
  float2* mls = reinterpret_cast<float2*>(red + 256 * 6);  // [span][nh] (max, sum) of a batch
  static_assert(256 * 6 + 2 * 256 <= sizeof(sh.o) / sizeof(float), "LDS reuse");
  TO* out = static_cast<TO*>(a.out);
  const int tid = threadIdx.x;
  const int F = ncol * kCols;  // float4 columns of the slice
  if (WIDE && !ALL && F > 256 && F <= 3 * 256 && np <= 4) {
    // Wide slice, few pieces (a verify step's 17-24 columns): each thread
    // takes up to three float4 columns, one per trip of 256, and all their
    // pieces' loads are in flight at once (one memory round trip instead of
    // one per trip); pieces are added in order, as in the trips below.
    const int pt = min(tid, np * ncol - 1);
    const u32x2 pair = __builtin_amdgcn_raw_buffer_load_b64(
        rml, (row_of(pt / ncol) + col0 + pt % ncol) * 8u, 0, kSc1);
    u32x4 ov[12];
#pragma unroll
    for (int u = 0; u < 12; ++u) {
      const int i = min(u % 4, np - 1);                            // past the end: a re-read
      const int cc = col0 * kCols + min(tid + 256 * (u / 4), F - 1);  // never used
      ov[u] = __builtin_amdgcn_raw_buffer_load_b128(
          ro, row_of(i) * kD * 4u + unsigned(cc / kCols) * kD * 4u + unsigned(cc % kCols) * 16u, 0, kSc1);
    }
    if (tid < np * ncol) mls[tid] = float2{__uint_as_float(pair[0]), __uint_as_float(pair[1])};
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int c = tid + 256 * k;
      if (c >= F) break;
      const int hc = col0 + c / kCols;
      Lse r{-__builtin_inff(), 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < np) {
          const float2 ml = mls[i * ncol + hc - col0];
          const u32x4 v = ov[4 * k + i];
          r.add(ml.x, ml.y, f32x4{__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                                  __uint_as_float(v[3])});
        }
      }
      if (hc < om.cols(h)) {  // the last column slice may be short
        const float inv = r.l > 0.f ? 1.f / r.l : 0.f;
        TO* o = out + om.row(b, h, hc) * kD + (c % kCols) * 4;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) o[e2] = TO(r.o[e2] * inv);
      }
    }
    __syncthreads();  // mls is LDS the caller reuses
    return;
  }
  // float4 columns [col0, col0 + 32*ncol) in trips of at most 256
  for (int base = col0 * kCols; base < (col0 + ncol) * kCols; base += 256) {
    const int Ft = min(256, (col0 + ncol) * kCols - base);
    const int P = 256 / Ft;               // piece groups
    const int pg = tid / Ft, cc = base + tid % Ft;
    const int h0 = base / kCols, nh = Ft / kCols;
    const int span = kMergeBatch * P;     // pieces per batch (span * nh <= 96 pairs)
    const int hc = cc / kCols;
    const unsigned cb = unsigned(hc) * kD * 4u + unsigned(cc % kCols) * 16u;
    Lse r{-__builtin_inff(), 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
    for (int q0 = 0; q0 < np; q0 += span) {
      // one (max, sum) pair per thread, issued with this thread's partial sums
      // (unconditionally: a load under a branch makes the compiler wait for it
      // before the loads that follow)
      const int pt = min(tid, span * nh - 1);
      const u32x2 pair = __builtin_amdgcn_raw_buffer_load_b64(
          rml, (row_of(min(q0 + pt / nh, np - 1)) + h0 + pt % nh) * 8u, 0, kSc1);
      u32x4 ov[kMergeBatch];
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const int i = min(q0 + u * P + pg, np - 1);  // past the end: a re-read, never used
        ov[u] = __builtin_amdgcn_raw_buffer_load_b128(ro, row_of(i) * kD * 4u + cb, 0, kSc1);
      }
      if (tid < span * nh) mls[tid] = float2{__uint_as_float(pair[0]), __uint_as_float(pair[1])};
      __syncthreads();
      if (pg < P) {
        if constexpr (ALL) {
          float mb[kMergeBatch], lb[kMergeBatch];
          f32x4 ob[kMergeBatch];
#pragma unroll
          for (int u = 0; u < kMergeBatch; ++u) {
            const float2 ml = mls[min((u * P + pg) * nh + hc - h0, span * nh - 1)];
            mb[u] = q0 + u * P + pg < np ? ml.x : -__builtin_inff();  // past the end: no piece
            lb[u] = ml.y;
            ob[u] = f32x4{__uint_as_float(ov[u][0]), __uint_as_float(ov[u][1]), __uint_as_float(ov[u][2]),
                          __uint_as_float(ov[u][3])};
          }
          r.add_all(mb, lb, ob);
        } else {
#pragma unroll
          for (int u = 0; u < kMergeBatch; ++u) {
            const int i = q0 + u * P + pg;
            if (i < np) {
              const float2 ml = mls[(u * P + pg) * nh + hc - h0];
              r.add(ml.x, ml.y, f32x4{__uint_as_float(ov[u][0]), __uint_as_float(ov[u][1]),
                                      __uint_as_float(ov[u][2]), __uint_as_float(ov[u][3])});
            }
          }
        }
      }
      __syncthreads();  // mls is rewritten by the next batch
    }
    if (P > 1) {
      float* e = red + tid * 6;
      e[0] = r.m;
      e[1] = r.l;
      e[2] = r.o[0];
      e[3] = r.o[1];
      e[4] = r.o[2];
      e[5] = r.o[3];
      __syncthreads();
      if (tid < Ft) {
        r = Lse{-__builtin_inff(), 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
        if constexpr (ALL) {
          for (int g0 = 0; g0 < P; g0 += 4) {  // the P piece groups, four at a time
            float mg[4], lg[4];
            f32x4 og[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const float* q = red + (min(g0 + k, P - 1) * Ft + tid) * 6;
              mg[k] = g0 + k < P ? q[0] : -__builtin_inff();
              lg[k] = q[1];
              og[k] = f32x4{q[2], q[3], q[4], q[5]};
            }
            r.add_all(mg, lg, og);
          }
        } else {
          for (int g2 = 0; g2 < P; ++g2) {
            const float* q = red + (g2 * Ft + tid) * 6;
            r.add(q[0], q[1], f32x4{q[2], q[3], q[4], q[5]});
          }
        }
      }
      __syncthreads();  // red is rewritten by the next trip
    }
    if (pg == 0 && hc < om.cols(h)) {  // the last column slice may be short
      const float inv = r.l > 0.f ? 1.f / r.l : 0.f;
      TO* o = out + om.row(b, h, hc) * kD + (cc % kCols) * 4;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) o[e2] = TO(r.o[e2] * inv);
    }
  }
}

// A wave's (max, sum, acc) of its share of a piece for the 16 columns of one
// tile into LDS (column col0 + c for lane (g, c)); l_run must already be
// summed over the lane groups.
template <class SH>
__device__ inline void stash_piece(SH& sh, int w, int g, int col, const f32x4 (&o)[kNT], float m_ref,
                                   float l_run) {
  if (g == 0) {
    sh.m[w][col] = m_ref;
    sh.l[w][col] = l_run;
  }
#pragma unroll
  for (int T_ = 0; T_ < kNT; ++T_)
#pragma unroll
    for (int i = 0; i < 4; ++i) sh.o[w][col][kNT * (4 * g + i) + T_] = o[T_][i];
}

// Merge the 4 waves' stashed piece through LDS and write it: normalized to
// `out` (type TO) when it is a whole segment, else as a partial in slot
// `slot` of unit `unit`, counted on the segment's arrival counter; the
// completing arrival merges the segment (unless the merge launch will).  S =
// the segment's start position, nb its blocks.  Ends with a barrier (LDS is
// reused by the next piece).  Its barriers wait on LDS only, so loads a wave
// issued for its next piece keep flying through the merge; the one exchange
// through memory (a partial read by the completing arrival) waits for this
// workgroup's stores explicitly before the arrival counts.
template <typename TO, class SH>
__device__ inline void finish_piece(const DecodeArgs& a, SH& sh, const OutMap& om, bool complete,
                                    int slot, int unit, int b, int h, int S, int nb,
                                    const Units& um) {
  const int NC = om.ncol();
  lds_barrier();
  TO* out = static_cast<TO*>(a.out);
  // Four consecutive dimensions per thread: one weight computation and one
  // 16-byte partial store serve four outputs.
  const __amdgpu_buffer_rsrc_t rws = __builtin_amdgcn_make_buffer_rsrc(
      a.ws_o, (short)0, int(unsigned(um.total()) * 2u * unsigned(NC) * kD * 4u), kRsrcWord3);
  for (int i4 = threadIdx.x; i4 < NC * (kD / 4); i4 += kWaves * 64) {
    const int hc = i4 / (kD / 4), d0 = (i4 % (kD / 4)) * 4;
    float mv[SH::kSlots], lv[SH::kSlots], ov[SH::kSlots][4];
#pragma unroll
    for (int v = 0; v < SH::kSlots; ++v) {
      mv[v] = sh.m[v][hc];
      lv[v] = sh.l[v][hc];
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[v][e] = sh.o[v][hc][d0 + e];
    }
    float M = -__builtin_inff();
#pragma unroll
    for (int v = 0; v < SH::kSlots; ++v) M = fmaxf(M, mv[v]);
    float lsum = 0.f, osum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < SH::kSlots; ++v) {
      // a slot whose wave saw no block (or no visible token) adds nothing
      // (selected, not branched around: its terms are computed and dropped)
      const bool none = mv[v] == -__builtin_inff();
      const float wt = exp2f(mv[v] - M);
      lsum += none ? 0.f : lv[v] * wt;
#pragma unroll
      for (int e = 0; e < 4; ++e) osum[e] += none ? 0.f : ov[v][e] * wt;
    }
    if (complete) {
      if (hc < om.cols(h)) {
        TO* o = out + om.row(b, h, hc) * kD + d0;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = TO(lsum > 0.f ? osum[e] / lsum : 0.f);
      }
    } else {
      const unsigned row = (unsigned(unit) * 2u + unsigned(slot)) * unsigned(NC) + unsigned(hc);
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4{__float_as_uint(osum[0]), __float_as_uint(osum[1]), __float_as_uint(osum[2]),
                __float_as_uint(osum[3])},
          rws, (row * kD + unsigned(d0)) * 4u, 0, kSc1);
      if (d0 == 0) {
        st_agent(&a.ws_ml[size_t(row) * 2], M);
        st_agent(&a.ws_ml[size_t(row) * 2 + 1], lsum);
      }
    }
  }
  if (!complete && !a.defer_merge) {
    const int c0 = um.unit_of(S);
    const int np = um.unit_of(S + nb - 1) - c0 + 1;
    wait_stores();  // this workgroup's partial is complete before its arrival counts
    lds_barrier();
    if (threadIdx.x == 0) sh.last = arrive(a, c0, np) ? 1 : 0;
    lds_barrier();
    if (sh.last)
      merge_segment<TO, SH, false, true>(a, sh, om, b, h, c0, S != um.start(c0), np,
                        unsigned(um.total()) * 2u * unsigned(NC), 0, NC);
  }
  lds_barrier();
}

}  // namespace dec
}  // namespace pa
