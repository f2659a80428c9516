// Matrix-core decode split kernel for 16-bit (bf16 / fp16) pools, head_dim 128,
// and its combine kernel.
//
// What it computes is decode attention through block tables ("The 8GB VRAM
// Breakthrough ...", section 3: the kernel reads each sequence's block table
// on the fly and gathers K for Q K^T and V for the softmax-weighted sum;
// blocks are contiguous inside, so only the fetch changes -- "PagedAttention
// aplica memoria virtual ao cache KV de LLMs").  The pages' kernel was written
// for a consumer GPU in CUDA/Triton; this one is laid out for CDNA4.
//
// Work decomposition.  The blocks of every (sequence b, KV head h) segment are
// laid end to end in one list (b major, then h, then logical block j), and
// workgroup c owns the chunk [c*C, (c+1)*C) of it, whatever the sequence
// lengths.  By default the grid is one workgroup per resident slot of the
// GPU and C = ceil(W / grid) for the W blocks of this call (read from the
// lengths on the device), so every workgroup streams the same number of
// blocks and all finish together; a fixed C can be requested instead.  A segment that lies inside one chunk
// is finished there (normalized and written to out).  A segment crossing chunk
// boundaries leaves one partial (max, sum, weighted sum) per chunk it touches;
// a chunk holds at most two such pieces (its first and its last), so the
// workspace is two slots per workgroup.  The combine kernel merges them.
//
// Inside a workgroup (4 wavefronts) a piece's blocks go round-robin to the
// waves.  All G = Hq/Hkv query heads of the KV head are packed into one
// 16-column tile, so every K/V block is read from HBM exactly once.
//
// Per 16-token block, per wavefront (lane l = 16*g + c):
//  * the table entry is a wave-uniform scalar load;
//  * K: four 16-byte loads, unit kk of lane l = 1 KiB-contiguous chunk
//    kk*1024 + 16*l of the slab = K[token c][dims 32kk+8g .. +7];
//  * S^T = K Q^T with four v_mfma_f32_16x16x32 (A = K rows = tokens,
//    B = Q^T columns = the packed query heads); lane (g, c) receives
//    S[head c][tokens 4g .. 4g+3];
//  * online softmax in the log2 domain: block max over the 16 tokens (in-lane,
//    then across the four lane groups); the running sum and accumulators are
//    rescaled only when the block max passes the reference by more than 2^8;
//  * P is split into a 16-bit high part and a 16-bit residual so the PV product
//    keeps ~16 significant bits of each weight;
//  * V: four 16-byte loads, unit u of lane l = V[tokens 4g..4g+3][dims 8c+2u,
//    8c+2u+1]; O^T += V^T P^T with v_mfma_f32_16x16x16 per 16-dim tile T
//    (rows = dims 8r+T), so lane (g, c) owns output head c: the softmax
//    rescale is a per-lane scalar.
// The loads of a wave's next block are issued before its current block is
// consumed (two register buffers).  After each piece the 4 waves merge
// (max, sum, acc) through LDS.
#include "common.hpp"

namespace pa {

namespace {

constexpr int kD = 128;        // head_dim handled here
constexpr int kNT = kD / 16;   // 16-dim output tiles
constexpr int kWaves = 4;

typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));

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

__device__ inline int seq_blocks(const DecodeArgs& a, int b) {
  const int L = min(max(a.lens[b], 0), a.max_seq_len);
  return (L + 15) >> 4;
}

// Start of sequence b's segments in the flattened list: Hkv * sum_{b'<b} nb_b'.
__device__ inline int seq_start(const DecodeArgs& a, int b, int lane) {
  int acc = 0;
  for (int base = 0; base < b; base += 64) {
    const int bb = base + lane;
    acc += bb < b ? seq_blocks(a, bb) : 0;
  }
  return wave_sum_int(acc) * a.pool.n_kv_heads;
}

template <typename T>
__global__ __launch_bounds__(kWaves * 64) void decode_split_mfma16(DecodeArgs a) {
  typedef typename Mfma<T>::v8 v8;
  typedef typename Mfma<T>::v4 v4;
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];
  __shared__ float sm_o[kWaves][16][kD + 1];
  __shared__ int sh_b, sh_fb, sh_c;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 4, c = lane & 15;
  const PoolDev& p = a.pool;
  const int H = p.n_kv_heads, Hq = a.n_q_heads, G = Hq / H, B = a.batch;
  T* out = static_cast<T*>(a.out);
  // ---- locate the chunk: wave 0 scans the per-sequence sizes ---------------------
  // With a.split_blocks == 0 the chunk size is derived from the total work W
  // so that the grid (one workgroup per resident slot) shares it evenly.
  if (w == 0) {
    int C = a.split_blocks;
    if (C <= 0) {
      int tot = 0;
      for (int base = 0; base < B; base += 64)
        tot += base + lane < B ? seq_blocks(a, base + lane) * H : 0;
      tot = wave_sum_int(tot);
      C = max(1, (tot + int(gridDim.x) - 1) / int(gridDim.x));
    }
    const int pos0 = int(blockIdx.x) * C;
    int run = 0, fb = 0, fbi = -1;
    for (int base = 0; base < B; base += 64) {
      const int bb = base + lane;
      const int sz = bb < B ? seq_blocks(a, bb) * H : 0;
      int incl = sz;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      const unsigned long long hit = __ballot(run + incl > pos0);
      if (hit) {
        const int fl = __builtin_ctzll(hit);
        fbi = base + fl;
        fb = run + __shfl(incl - sz, fl, 64);
        break;
      }
      run += __shfl(incl, 63, 64);
    }
    if (lane == 0) {
      sh_b = fbi;
      sh_fb = fb;
      sh_c = C;
    }
  }
  __syncthreads();
  int b = sh_b, fb = sh_fb;
  const int C = sh_c;
  const int pos0 = int(blockIdx.x) * C, pos1 = pos0 + C;
  if (b < 0) return;  // chunk past the end of the work

  const T* kbase = reinterpret_cast<const T*>(p.base + p.off[kArrK]);
  const T* vbase = reinterpret_cast<const T*>(p.base + p.off[kArrV]);
  const float sl2 = a.scale_log2;
  const int nbk = p.num_blocks;

  // per-piece state, captured by the lambdas below
  int h = 0, L = 0;
  const int32_t* trow = a.tables;
  v8 qf[4];
  f32x4 o[kNT];
  // Running statistics per lane (= per packed head c): m_ref is the reference
  // the weights are taken against, l_run the running sum of weights.
  float m_ref = -__builtin_inff(), l_run = 0.f;

  // K/V of one block into registers (8 x 16-byte loads, 1 KiB contiguous per
  // load across the wave).  The loads are issued unconditionally -- an
  // out-of-range table entry reads block 0 and is never consumed -- so no
  // branch separates a load from its use and the wait counters stay exact.
  auto fetch = [&](int id, v8(&kf)[4], v8(&vf)[4]) {
    const int safe = (id < 0 || id >= nbk) ? 0 : id;
    const size_t slab = (size_t(safe) * H + h) * (16 * kD);
    const T* ks = kbase + slab;
    const T* vs = vbase + slab;
#pragma unroll
    for (int u = 0; u < 4; ++u) kf[u] = *reinterpret_cast<const v8*>(ks + (u * 64 + lane) * 8);
#pragma unroll
    for (int u = 0; u < 4; ++u) vf[u] = *reinterpret_cast<const v8*>(vs + (u * 64 + lane) * 8);
  };
  auto ok = [&](int id) { return id >= 0 && id < nbk; };

  // One block: S^T = K Q^T, online softmax, O^T += V^T P^T.  `valid` tokens
  // of the block count (0 for a skipped table entry: every weight is zero).
  // It always runs, so every load is waited on along every path.
  auto consume = [&](int valid, const v8(&kf)[4], v8(&vf)[4]) {
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) sc = Mfma<T>::qk(kf[kk], qf[kk], sc);
    float x[4];
    float bm = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = (4 * g + i < valid) ? sc[i] * sl2 : -__builtin_inff();
      bm = fmaxf(bm, x[i]);
    }
    bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    // The reference only moves when a block's max exceeds it by more than 8
    // (weights stay <= 2^8, far inside fp32 and the two-part 16-bit split),
    // so the accumulators are rarely rescaled.  The result is unchanged:
    // numerator and denominator share the reference.
    const bool move = bm > m_ref + 8.f;
    if (__any(move)) {
      const float m_new = move ? bm : m_ref;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      l_run *= alpha;
#pragma unroll
      for (int T_ = 0; T_ < kNT; ++T_) o[T_] *= alpha;
      m_ref = m_new;
    }
    float pw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pw[i] = (4 * g + i < valid) ? __builtin_amdgcn_exp2f(x[i] - m_ref) : 0.f;
      l_run += pw[i];
    }
    if (valid < 16) {
      // Unwritten tail slots may hold anything (even NaN bit patterns): zero
      // them so a zero weight cannot meet a NaN.  Each dword holds two tokens.
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
    v4 phi, plo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      phi[i] = T(pw[i]);
      plo[i] = T(pw[i] - float(phi[i]));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        v4 vt = {vf[u][4 * par + 0], vf[u][4 * par + 1], vf[u][4 * par + 2], vf[u][4 * par + 3]};
        o[2 * u + par] = Mfma<T>::pv(vt, phi, o[2 * u + par]);
        o[2 * u + par] = Mfma<T>::pv(vt, plo, o[2 * u + par]);
      }
    }
  };

  int pos = pos0;
  bool first = true;
  while (pos < pos1 && b < B) {
    const int nb = seq_blocks(a, b);
    if (pos >= fb + nb * H) {  // past sequence b (also skips empty ones)
      fb += nb * H;
      ++b;
      continue;
    }
    h = (pos - fb) / nb;
    const int jbeg = (pos - fb) % nb;
    const int jend = min(nb, jbeg + (pos1 - pos));
    L = min(max(a.lens[b], 0), a.max_seq_len);
    trow = a.tables + size_t(b) * a.max_blocks_per_seq;
    {
      // Q^T fragment: lane (g, c) holds Q[h*G + c][32kk + 8g .. +7], zero for c >= G.
      const T* qp = static_cast<const T*>(a.q) + (size_t(b) * Hq + h * G + c) * kD + 8 * g;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qf[kk] = c < G ? *reinterpret_cast<const v8*>(qp + 32 * kk) : v8{};
    }
#pragma unroll
    for (int T_ = 0; T_ < kNT; ++T_) o[T_] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_ref = -__builtin_inff();
    l_run = 0.f;

    // Software pipeline over this wave's blocks jw+4k, k = 0..n-1: the loads
    // of block k+1 are in flight while block k is consumed.  Two register
    // buffers alternate (pairs of blocks per trip, one exit), so no copies and
    // no full waits.  The prefetch past the last block re-reads it (an L2 hit).
    const int jw = jbeg + w;
    const int n = jw < jend ? (jend - jw + kWaves - 1) / kWaves : 0;
    auto id_of = [&](int k) { return trow[jw + kWaves * k]; };
    auto valid_of = [&](int k, int id) { return ok(id) ? L - 16 * (jw + kWaves * k) : 0; };
    v8 ka[4], va[4], kb[4], vb[4];
    if (n > 0) {
      int ida = id_of(0);
      fetch(ida, ka, va);
      int k = 0;
      for (; k + 1 < n; k += 2) {
        const int idb = id_of(k + 1);
        fetch(idb, kb, vb);
        consume(valid_of(k, ida), ka, va);
        const int kn = min(k + 2, n - 1);
        const int idn = id_of(kn);
        fetch(idn, ka, va);
        consume(valid_of(k + 1, idb), kb, vb);
        ida = idn;
      }
      if (k < n) consume(valid_of(k, ida), ka, va);
    }

    // ---- merge the 4 waves of this piece -------------------------------------
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    if (g == 0) {
      sm_m[w][c] = m_ref;
      sm_l[w][c] = l_run;
    }
#pragma unroll
    for (int T_ = 0; T_ < kNT; ++T_)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_o[w][c][kNT * (4 * g + i) + T_] = o[T_][i];
    __syncthreads();
    const bool complete = jbeg == 0 && jend == nb;
    const int slot = first ? 0 : 1;
    for (int idx = threadIdx.x; idx < G * kD; idx += kWaves * 64) {
      const int hc = idx / kD, d = idx % kD;
      float M = -__builtin_inff();
#pragma unroll
      for (int v = 0; v < kWaves; ++v) M = fmaxf(M, sm_m[v][hc]);
      float lsum = 0.f, osum = 0.f;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        if (sm_m[v][hc] == -__builtin_inff()) continue;  // wave saw no block
        const float wt = exp2f(sm_m[v][hc] - M);
        lsum += sm_l[v][hc] * wt;
        osum += sm_o[v][hc][d] * wt;
      }
      if (complete) {
        out[(size_t(b) * Hq + h * G + hc) * kD + d] = T(lsum > 0.f ? osum / lsum : 0.f);
      } else {
        const size_t row = (size_t(blockIdx.x) * 2 + slot) * G + hc;
        a.ws_o[row * kD + d] = osum;
        if (d == 0) {
          a.ws_ml[row * 2] = M;
          a.ws_ml[row * 2 + 1] = lsum;
        }
      }
    }
    __syncthreads();  // LDS is reused by the next piece
    pos += jend - jbeg;
    first = false;
  }
}

// Merge the pieces of one (sequence b, query head hq) left by the split
// kernel: chunks c0..c1 touch the segment; chunk c0 holds it in slot 1 unless
// the segment starts its chunk, every later chunk in slot 0.
//   m = max m_i, l = sum l_i 2^(m_i - m), o = sum o_i 2^(m_i - m) / l.
// Rows of empty sequences are zeroed here.
constexpr int kCombineChunk = 256;

template <typename T>
__global__ __launch_bounds__(64) void decode_combine_mfma16(DecodeArgs a) {
  __shared__ float wsh[kCombineChunk];
  const int hq = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int H = a.pool.n_kv_heads, Hq = a.n_q_heads, G = Hq / H, h = hq / G, hc = hq % G;
  T* out = static_cast<T*>(a.out) + (size_t(b) * Hq + hq) * kD;
  const int nb = seq_blocks(a, b);
  if (nb == 0) {
    for (int d = lane; d < kD; d += 64) out[d] = T(0.f);
    return;
  }
  int C = a.split_blocks;
  if (C <= 0) {  // the split kernel's derived chunk size
    int tot = 0;
    for (int base = 0; base < a.batch; base += 64)
      tot += base + lane < a.batch ? seq_blocks(a, base + lane) * H : 0;
    tot = wave_sum_int(tot);
    C = max(1, (tot + a.max_splits - 1) / a.max_splits);
  }
  const int S = seq_start(a, b, lane) + h * nb, E = S + nb;
  const int c0 = S / C, c1 = (E - 1) / C;
  if (c0 == c1) return;  // finished inside one chunk
  const int np = c1 - c0 + 1;
  auto row_of = [&](int i) {
    const int slot = (i == 0 && S != c0 * C) ? 1 : 0;
    return (size_t(c0 + i) * 2 + slot) * G + hc;
  };
  const float ninf = -__builtin_inff();
  float M = ninf;
  for (int i = lane; i < np; i += 64) M = fmaxf(M, a.ws_ml[row_of(i) * 2]);
  M = wave_max(M);
  float lsum = 0.f;
  for (int i = lane; i < np; i += 64) {
    const size_t r = row_of(i);
    const float m = a.ws_ml[r * 2];
    if (m != ninf) lsum += a.ws_ml[r * 2 + 1] * exp2f(m - M);
  }
  lsum = wave_sum(lsum);
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  float acc0 = 0.f, acc1 = 0.f;
  for (int q0 = 0; q0 < np; q0 += kCombineChunk) {
    const int qn = min(kCombineChunk, np - q0);
    __syncthreads();
    for (int i = lane; i < qn; i += 64) {
      const float m = a.ws_ml[row_of(q0 + i) * 2];
      wsh[i] = m != ninf ? exp2f(m - M) * inv : 0.f;
    }
    __syncthreads();
    int i = 0;
    for (; i + 4 <= qn; i += 4) {  // independent loads in flight
      const float* s0 = a.ws_o + row_of(q0 + i + 0) * kD;
      const float* s1 = a.ws_o + row_of(q0 + i + 1) * kD;
      const float* s2 = a.ws_o + row_of(q0 + i + 2) * kD;
      const float* s3 = a.ws_o + row_of(q0 + i + 3) * kD;
      const float x0 = s0[lane], x1 = s1[lane], x2 = s2[lane], x3 = s3[lane];
      const float y0 = s0[lane + 64], y1 = s1[lane + 64], y2 = s2[lane + 64], y3 = s3[lane + 64];
      acc0 += (x0 * wsh[i] + x1 * wsh[i + 1]) + (x2 * wsh[i + 2] + x3 * wsh[i + 3]);
      acc1 += (y0 * wsh[i] + y1 * wsh[i + 1]) + (y2 * wsh[i + 2] + y3 * wsh[i + 3]);
    }
    for (; i < qn; ++i) {
      const float* src = a.ws_o + row_of(q0 + i) * kD;
      acc0 += src[lane] * wsh[i];
      acc1 += src[lane + 64] * wsh[i];
    }
  }
  out[lane] = T(acc0);
  out[lane + 64] = T(acc1);
}

}  // namespace

hipError_t launch_decode_split_mfma16(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(unsigned(a.max_splits));
  if (a.pool.kv_dtype == kBF16)
    hipLaunchKernelGGL(decode_split_mfma16<__bf16>, grid, dim3(kWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL(decode_split_mfma16<_Float16>, grid, dim3(kWaves * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_combine_mfma16(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(unsigned(a.n_q_heads), unsigned(a.batch));
  if (a.pool.kv_dtype == kBF16)
    hipLaunchKernelGGL(decode_combine_mfma16<__bf16>, grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(decode_combine_mfma16<_Float16>, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
