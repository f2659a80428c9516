// Shared pieces of the matrix-core decode split kernels (decode_mfma.hip for
// 16-bit pools, decode_quant.hip for INT4/FP8 pools): the flattened,
// evenly chunked work list, the per-piece iteration, and the 4-wave merge.
//
// Work list: the blocks of every (sequence b, KV head h) segment laid end to
// end (b major, then h, then logical block j).  Workgroup c owns positions
// [c*C, (c+1)*C).  A segment inside one chunk is finished in place
// (normalized, written to out); a segment crossing chunk boundaries leaves a
// partial (max, sum, weighted sum) in the chunk's slot 0 (its first piece) or
// slot 1 (its last piece), merged later by the combine kernel.
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
};

__device__ inline int seq_len(const DecodeArgs& a, int b) {
  return min(max(a.lens[b], 0), a.max_seq_len);
}

__device__ inline int seq_blocks(const DecodeArgs& a, int b) { return (seq_len(a, b) + 15) >> 4; }

// Start of sequence b's segments in the flattened list: Hkv * sum_{b'<b} nb_b'.
__device__ inline int seq_start(const DecodeArgs& a, int b, int lane) {
  int acc = 0;
  for (int base = 0; base < b; base += 64) {
    const int bb = base + lane;
    acc += bb < b ? seq_blocks(a, bb) : 0;
  }
  return wave_sum_int(acc) * a.pool.n_kv_heads;
}

// Total blocks of the flattened list (one wavefront, result in every lane).
__device__ inline int total_work(const DecodeArgs& a, int lane) {
  int tot = 0;
  for (int base = 0; base < a.batch; base += 64)
    tot += base + lane < a.batch ? seq_blocks(a, base + lane) * a.pool.n_kv_heads : 0;
  return wave_sum_int(tot);
}

// Chunk size: fixed (a.split_blocks > 0) or the work shared evenly by the grid.
__device__ inline int chunk_size(const DecodeArgs& a, int lane, int grid) {
  if (a.split_blocks > 0) return a.split_blocks;
  return max(1, (total_work(a, lane) + grid - 1) / grid);
}

struct Shared {
  float m[kWaves][16];
  float l[kWaves][16];
  float o[kWaves][16][kD + 1];
  int b, fb, c;
};

// Wave 0 finds the sequence holding this workgroup's first position.  Returns
// false (for every thread) when the chunk lies past the end of the work.
__device__ inline bool locate_chunk(const DecodeArgs& a, Shared& sh, int w, int lane, int& b,
                                    int& fb, int& pos0, int& pos1) {
  const int H = a.pool.n_kv_heads, B = a.batch;
  if (w == 0) {
    const int C = chunk_size(a, lane, int(gridDim.x));
    const int p0 = int(blockIdx.x) * C;
    int run = 0, f = 0, fbi = -1;
    for (int base = 0; base < B; base += 64) {
      const int bb = base + lane;
      const int sz = bb < B ? seq_blocks(a, bb) * H : 0;
      int incl = sz;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      const unsigned long long hit = __ballot(run + incl > p0);
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
      sh.c = C;
    }
  }
  __syncthreads();
  b = sh.b;
  fb = sh.fb;
  pos0 = int(blockIdx.x) * sh.c;
  pos1 = pos0 + sh.c;
  return b >= 0;
}

// The next piece [jbeg, jend) of segment (b, h) starting at position pos;
// advances (b, fb) past finished or empty sequences.  False when done.
__device__ inline bool next_piece(const DecodeArgs& a, int pos, int pos1, int& b, int& fb, int& h,
                                  int& jbeg, int& jend, int& nb) {
  const int H = a.pool.n_kv_heads;
  while (pos < pos1 && b < a.batch) {
    nb = seq_blocks(a, b);
    if (pos >= fb + nb * H) {
      fb += nb * H;
      ++b;
      continue;
    }
    h = (pos - fb) / nb;
    jbeg = (pos - fb) % nb;
    jend = min(nb, jbeg + (pos1 - pos));
    return true;
  }
  return false;
}

// Merge the 4 waves' (max, sum, acc) of one piece through LDS and write the
// piece: normalized to `out` (type TO) when it is a whole segment, else as a
// partial in the workgroup's slot.  l_run must already be summed over the
// lane groups.  Ends with a barrier (LDS is reused by the next piece).
template <typename TO>
__device__ inline void merge_piece(const DecodeArgs& a, Shared& sh, int w, int g, int c,
                                   const f32x4 (&o)[kNT], float m_ref, float l_run, bool complete,
                                   int slot, int b, int h) {
  const int Hq = a.n_q_heads, G = Hq / a.pool.n_kv_heads;
  if (g == 0) {
    sh.m[w][c] = m_ref;
    sh.l[w][c] = l_run;
  }
#pragma unroll
  for (int T_ = 0; T_ < kNT; ++T_)
#pragma unroll
    for (int i = 0; i < 4; ++i) sh.o[w][c][kNT * (4 * g + i) + T_] = o[T_][i];
  __syncthreads();
  TO* out = static_cast<TO*>(a.out);
  for (int idx = threadIdx.x; idx < G * kD; idx += kWaves * 64) {
    const int hc = idx / kD, d = idx % kD;
    float M = -__builtin_inff();
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, sh.m[v][hc]);
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      if (sh.m[v][hc] == -__builtin_inff()) continue;  // wave saw no block
      const float wt = exp2f(sh.m[v][hc] - M);
      lsum += sh.l[v][hc] * wt;
      osum += sh.o[v][hc][d] * wt;
    }
    if (complete) {
      out[(size_t(b) * Hq + h * G + hc) * kD + d] = TO(lsum > 0.f ? osum / lsum : 0.f);
    } else {
      const size_t row = (size_t(blockIdx.x) * 2 + slot) * G + hc;
      a.ws_o[row * kD + d] = osum;
      if (d == 0) {
        a.ws_ml[row * 2] = M;
        a.ws_ml[row * 2 + 1] = lsum;
      }
    }
  }
  __syncthreads();
}

}  // namespace dec
}  // namespace pa
