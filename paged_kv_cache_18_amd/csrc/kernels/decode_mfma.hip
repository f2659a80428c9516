// Matrix-core decode split kernel for 16-bit (bf16 / fp16) pools, head_dim 128.
//
// What it computes is decode attention through block tables ("The 8GB VRAM
// Breakthrough ...", section 3: the kernel reads each sequence's block table
// on the fly and gathers K for Q K^T and V for the softmax-weighted sum;
// blocks are contiguous inside, so only the fetch changes -- "PagedAttention
// aplica memoria virtual ao cache KV de LLMs").  The pages' kernel was written
// for a consumer GPU in CUDA/Triton; this one is laid out for CDNA4.
//
// Work decomposition: one workgroup of 4 wavefronts per (sequence b, KV head
// h, split of the logical blocks); wave w takes blocks j0+w, j0+w+4, ...  All
// G = Hq/Hkv query heads of the KV head are packed into one 16-column tile, so
// every K/V block is read from HBM exactly once.
//
// Per 16-token block, per wavefront (lane l = 16*g + c):
//  * the table entry is a wave-uniform scalar load;
//  * K: four 16-byte loads, unit kk of lane l = 1 KiB-contiguous chunk
//    kk*1024 + 16*l of the slab = K[token c][dims 32kk+8g .. +7];
//  * S^T = K Q^T with four v_mfma_f32_16x16x32 (A = K rows = tokens,
//    B = Q^T columns = the packed query heads); lane (g, c) receives
//    S[head c][tokens 4g .. 4g+3];
//  * online softmax in the log2 domain: block max over the 16 tokens (in-lane,
//    then across the four lane groups), rescale of the running sum and of the
//    accumulators;
//  * P is split into a 16-bit high part and a 16-bit residual so the PV product
//    keeps ~16 significant bits of each weight;
//  * V: four 16-byte loads, unit u of lane l = V[tokens 4g..4g+3][dims 8c+2u,
//    8c+2u+1]; O^T += V^T P^T with v_mfma_f32_16x16x16 per 16-dim tile T
//    (rows = dims 8r+T), so lane (g, c) owns output head c: the softmax
//    rescale is a per-lane scalar.
// At the end the 4 waves merge (max, sum, acc) through LDS; a single-split
// sequence is normalized and written to out, otherwise the split's partials go
// to the workspace for the combine kernel.
#include "common.hpp"

namespace pa {

namespace {

constexpr int kD = 128;        // head_dim handled here
constexpr int kNT = kD / 16;   // 16-dim output tiles
constexpr int kWaves = 4;

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

template <typename T>
__global__ __launch_bounds__(kWaves * 64) void decode_split_mfma16(DecodeArgs a) {
  typedef typename Mfma<T>::v8 v8;
  typedef typename Mfma<T>::v4 v4;
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];
  __shared__ float sm_o[kWaves][16][kD + 1];

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 4, c = lane & 15;
  const PoolDev& p = a.pool;
  const int H = p.n_kv_heads, Hq = a.n_q_heads, G = Hq / H;
  const int L = min(max(a.lens[b], 0), a.max_seq_len);
  const int nb = (L + 15) >> 4, S = a.split_blocks;
  const int j0 = split * S;
  T* out = static_cast<T*>(a.out);
  if (j0 >= nb) {
    if (split == 0)  // empty sequence: zero rows
      for (int i = threadIdx.x; i < G * kD; i += kWaves * 64)
        out[(size_t(b) * Hq + h * G) * kD + i] = T(0.f);
    return;
  }
  const int j1 = min(nb, j0 + S), nsplit = (nb + S - 1) / S;

  // Q^T fragment: lane (g, c) holds Q[h*G + c][32kk + 8g .. +7], zero for c >= G.
  v8 qf[4];
  {
    const T* qp = static_cast<const T*>(a.q) + (size_t(b) * Hq + h * G + c) * kD + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (c < G)
        qf[kk] = *reinterpret_cast<const v8*>(qp + 32 * kk);
      else
        qf[kk] = v8{};
    }
  }

  f32x4 o[kNT];
#pragma unroll
  for (int T_ = 0; T_ < kNT; ++T_) o[T_] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff(), l_run = 0.f;

  const T* kbase = reinterpret_cast<const T*>(p.base + p.off[kArrK]);
  const T* vbase = reinterpret_cast<const T*>(p.base + p.off[kArrV]);
  const int32_t* trow = a.tables + size_t(b) * a.max_blocks_per_seq;
  const float sl2 = a.scale_log2;

  for (int j = j0 + w; j < j1; j += kWaves) {
    const int id = trow[j];  // uniform address: scalar load
    if (id < 0 || id >= p.num_blocks) continue;
    const size_t slab = (size_t(id) * H + h) * (16 * kD);
    const T* ks = kbase + slab;
    const T* vs = vbase + slab;
    v8 kf[4], vf[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) kf[u] = *reinterpret_cast<const v8*>(ks + (u * 64 + lane) * 8);
#pragma unroll
    for (int u = 0; u < 4; ++u) vf[u] = *reinterpret_cast<const v8*>(vs + (u * 64 + lane) * 8);

    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) s = Mfma<T>::qk(kf[kk], qf[kk], s);

    const int valid = L - 16 * j;  // >= 1
    float x[4];
    float bm = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = (4 * g + i < valid) ? s[i] * sl2 : -__builtin_inff();
      bm = fmaxf(bm, x[i]);
    }
    bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    const float m_new = fmaxf(m_run, bm);
    const float alpha = exp2f(m_run - m_new);
    float pw[4], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pw[i] = exp2f(x[i] - m_new);
      psum += pw[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int T_ = 0; T_ < kNT; ++T_) o[T_] *= alpha;

    if (valid < 16) {  // unwritten tail slots may hold anything: zero them
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (4 * g + (e & 3) >= valid) vf[u][e] = T(0.f);
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
  }

  // ---- merge the 4 waves ----------------------------------------------------------
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (g == 0) {
    sm_m[w][c] = m_run;
    sm_l[w][c] = l_run;
  }
#pragma unroll
  for (int T_ = 0; T_ < kNT; ++T_)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_o[w][c][kNT * (4 * g + i) + T_] = o[T_][i];
  __syncthreads();

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
    const size_t hq = size_t(b) * Hq + h * G + hc;
    if (nsplit == 1) {
      out[hq * kD + d] = T(lsum > 0.f ? osum / lsum : 0.f);
    } else {
      const size_t wrow = hq * a.max_splits + split;
      a.ws_o[wrow * kD + d] = osum;
      if (d == 0) {
        a.ws_ml[wrow * 2] = M;
        a.ws_ml[wrow * 2 + 1] = lsum;
      }
    }
  }
}

}  // namespace

hipError_t launch_decode_split_mfma16(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(unsigned(a.max_splits), unsigned(a.pool.n_kv_heads), unsigned(a.batch));
  if (a.pool.kv_dtype == kBF16)
    hipLaunchKernelGGL(decode_split_mfma16<__bf16>, grid, dim3(kWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL(decode_split_mfma16<_Float16>, grid, dim3(kWaves * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
