// Generic decode split kernel (vector ALU, any storage dtype) and the split-K
// combine kernel.
//
// Decode attention through block tables: "The 8GB VRAM Breakthrough ...",
// section 3 ("How Logical-to-Physical Block Tables Work": the kernel reads the
// table on the fly and gathers K for the Q K^T dot product and V for the
// softmax-weighted sum); INT4/FP8 values are dequantized in registers, never
// written back (section 5, "On-the-Fly Register Dequantization").
//
// The generic kernel handles every dtype, head_dim and GQA ratio, one query
// head per wavefront, one token at a time, and the verify step's several
// queries per sequence (each attending to the cache up to its own token).  It is the path for fp32 pools and
// for shapes the matrix-core kernel does not take.  Both kernels share the
// split/workspace contract: scores live in the log2 domain (scale folded with
// log2 e), split s of sequence b writes (max, sum) and the unnormalized sum of
// weighted values; a sequence with one split is normalized and written to
// `out` directly.
#include "common.hpp"

namespace pa {

namespace {

constexpr int kMaxDimPerLane = 4;  // head_dim <= 256

// Tokens query qi of sequence b attends to: a verify step's n_query new tokens
// are the last of the sequence's L cached tokens, and query qi sees the cache
// up to and including its own token (causal among the new ones); decode is
// n_query = 1 (all L tokens).
__device__ inline int query_len(const DecodeArgs& a, int b, int qi) {
  const int L = min(max(a.lens[b], 0), a.max_seq_len);
  return max(0, L - max(a.n_query, 1) + 1 + qi);
}

__device__ inline void store_out(void* out, size_t i, float x, int dt) {
  if (dt == kF32)
    static_cast<float*>(out)[i] = x;
  else if (dt == kF16)
    static_cast<uint16_t*>(out)[i] = f32_to_f16_bits(x);
  else
    static_cast<uint16_t*>(out)[i] = f32_to_bf16_bits(x);
}

// Value of element (t, d) of K (kind 0) or V (kind 1) in block `id`, head `h`.
__device__ inline float read_elem(const PoolDev& p, int id, int h, int t, int d, int kind) {
  const int H = p.n_kv_heads, D = p.head_dim;
  if (id >= p.num_blocks) {  // FP16 sink arena
    const int arr = kind ? kArrSV : kArrSK;
    const uint16_t* s = reinterpret_cast<const uint16_t*>(
        p.base + p.off[arr] + (size_t(id - p.num_blocks) * H + h) * p.slab[arr]);
    return f16_bits_to_f32(s[kind ? raw_v_elem(t, d, D) : raw_k_elem(t, d)]);
  }
  const int arr = kind ? kArrV : kArrK;
  const size_t sid = size_t(id) * H + h;
  const uint8_t* slab = p.base + p.off[arr] + sid * p.slab[arr];
  const int dt = p.kv_dtype;
  if (is_raw_dev(dt)) {
    const int i = kind ? raw_v_elem(t, d, D) : raw_k_elem(t, d);
    return load_as_f32(slab, size_t(i), dt);
  }
  if (dt == kInt4) {
    const int k = d >> 1;
    const uint32_t byte = slab[kind ? int4_v_byte(t, k, D) : int4_k_byte(t, k, D)];
    const uint32_t q = (byte >> ((d & 1) * 4)) & 15u;
    const int ng = D / p.group_size, gi = d / p.group_size;
    const int sarr = kind ? kArrVS : kArrKS, zarr = kind ? kArrVZ : kArrKZ;
    const uint16_t* sc = reinterpret_cast<const uint16_t*>(p.base + p.off[sarr] + sid * p.slab[sarr]);
    const uint16_t* zp = reinterpret_cast<const uint16_t*>(p.base + p.off[zarr] + sid * p.slab[zarr]);
    return (float(q) - f16_bits_to_f32(zp[t * ng + gi])) * f16_bits_to_f32(sc[t * ng + gi]);
  }
  // FP8
  const uint32_t c = slab[kind ? fp8_v_byte(t, d, D) : fp8_k_byte(t, d)];
  const int sarr = kind ? kArrVS : kArrKS;
  const uint16_t* sc = reinterpret_cast<const uint16_t*>(p.base + p.off[sarr] + sid * p.slab[sarr]);
  return e4m3_decode(c) * f16_bits_to_f32(sc[t]);
}

__global__ __launch_bounds__(64) void decode_split_generic(DecodeArgs a) {
  const int split = blockIdx.x, hq = blockIdx.y, r = blockIdx.z, lane = threadIdx.x;
  const PoolDev& p = a.pool;
  const int D = p.head_dim, Hq = a.n_q_heads, G = Hq / p.n_kv_heads, h = hq / G;
  const int nq = max(a.n_query, 1), b = r / nq;
  const int L = query_len(a, b, r % nq);
  const int nb = (L + 15) >> 4, S = a.split_blocks;
  const int j0 = split * S;
  const size_t orow = (size_t(r) * Hq + hq) * D;
  if (j0 >= nb) {
    if (split == 0)
      for (int d = lane; d < D; d += 64) store_out(a.out, orow + d, 0.f, a.q_dtype);
    return;
  }
  const int j1 = min(nb, j0 + S), nsplit = (nb + S - 1) / S;
  float qv[kMaxDimPerLane], acc[kMaxDimPerLane];
#pragma unroll
  for (int m = 0; m < kMaxDimPerLane; ++m) {
    const int d = lane + 64 * m;
    qv[m] = d < D ? load_as_f32(a.q, orow + d, a.q_dtype) : 0.f;
    acc[m] = 0.f;
  }
  float m_run = -__builtin_inff(), l_run = 0.f;
  const int total = p.num_blocks + p.num_sink_blocks;
  for (int j = j0; j < j1; ++j) {
    const int id = a.tables[size_t(b) * a.max_blocks_per_seq + j];
    if (id < 0 || id >= total) continue;
    const int nt = min(16, L - 16 * j);
    for (int t = 0; t < nt; ++t) {
      float part = 0.f;
#pragma unroll
      for (int m = 0; m < kMaxDimPerLane; ++m) {
        const int d = lane + 64 * m;
        if (d < D) part += qv[m] * read_elem(p, id, h, t, d, 0);
      }
      const float s = wave_sum(part) * a.scale_log2;
      const float m_new = fmaxf(m_run, s);
      const float alpha = exp2f(m_run - m_new);
      const float w = exp2f(s - m_new);
      l_run = l_run * alpha + w;
#pragma unroll
      for (int m = 0; m < kMaxDimPerLane; ++m) {
        const int d = lane + 64 * m;
        if (d < D) acc[m] = acc[m] * alpha + w * read_elem(p, id, h, t, d, 1);
      }
      m_run = m_new;
    }
  }
  if (nsplit == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int m = 0; m < kMaxDimPerLane; ++m) {
      const int d = lane + 64 * m;
      if (d < D) store_out(a.out, orow + d, acc[m] * inv, a.q_dtype);
    }
    return;
  }
  const size_t wrow = (size_t(r) * Hq + hq) * a.max_splits + split;
#pragma unroll
  for (int m = 0; m < kMaxDimPerLane; ++m) {
    const int d = lane + 64 * m;
    if (d < D) a.ws_o[wrow * D + d] = acc[m];
  }
  if (lane == 0) {
    a.ws_ml[wrow * 2] = m_run;
    a.ws_ml[wrow * 2 + 1] = l_run;
  }
}

// Merge the splits of one (sequence, query head): m = max m_i,
// l = sum l_i 2^(m_i - m), o = sum o_i 2^(m_i - m) / l.  The statistics of all
// splits are read in parallel (one split per lane), the normalized weights go
// through LDS, and each lane sums its dimensions over the splits with
// independent loads.
constexpr int kCombineChunk = 256;

__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a) {
  __shared__ float wsh[kCombineChunk];
  const int hq = blockIdx.x, r = blockIdx.y, lane = threadIdx.x;
  const int D = a.pool.head_dim, Hq = a.n_q_heads, S = a.split_blocks;
  const int nq = max(a.n_query, 1);
  const int L = query_len(a, r / nq, r % nq);
  const int nsplit = (((L + 15) >> 4) + S - 1) / S;
  if (nsplit <= 1) return;
  const size_t row = (size_t(r) * Hq + hq) * a.max_splits;
  const float* ml = a.ws_ml + row * 2;
  const float ninf = -__builtin_inff();
  float M = ninf;
  for (int i = lane; i < nsplit; i += 64) M = fmaxf(M, ml[2 * i]);
  M = wave_max(M);
  // a split whose blocks were all skipped has max -inf and weight 0
  float lsum = 0.f;
  for (int i = lane; i < nsplit; i += 64)
    if (ml[2 * i] != ninf) lsum += ml[2 * i + 1] * exp2f(ml[2 * i] - M);
  lsum = wave_sum(lsum);
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  float acc[kMaxDimPerLane] = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nsplit; c0 += kCombineChunk) {
    const int cn = min(kCombineChunk, nsplit - c0);
    __syncthreads();
    for (int i = lane; i < cn; i += 64) {
      const float m = ml[2 * (c0 + i)];
      wsh[i] = m != ninf ? exp2f(m - M) * inv : 0.f;
    }
    __syncthreads();
    const float* base = a.ws_o + (row + c0) * D;
#pragma unroll
    for (int k = 0; k < kMaxDimPerLane; ++k) {
      const int d = lane + 64 * k;
      if (d >= D) break;
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
      int i = 0;
      for (; i + 4 <= cn; i += 4) {
        s0 += base[size_t(i + 0) * D + d] * wsh[i + 0];
        s1 += base[size_t(i + 1) * D + d] * wsh[i + 1];
        s2 += base[size_t(i + 2) * D + d] * wsh[i + 2];
        s3 += base[size_t(i + 3) * D + d] * wsh[i + 3];
      }
      for (; i < cn; ++i) s0 += base[size_t(i) * D + d] * wsh[i];
      acc[k] += (s0 + s1) + (s2 + s3);
    }
  }
#pragma unroll
  for (int k = 0; k < kMaxDimPerLane; ++k) {
    const int d = lane + 64 * k;
    if (d < D) store_out(a.out, (size_t(r) * Hq + hq) * D + d, acc[k], a.q_dtype);
  }
}

}  // namespace

hipError_t launch_decode_split_mfma16(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_split_quant(const DecodeArgs& a, hipStream_t s);

int occupancy_mfma16(int32_t kv_dtype, int nct);
int occupancy_quant(int32_t kv_dtype, int32_t group_size, int nct);

int decode_split_occupancy(int32_t kernel, int32_t kv_dtype, int nct, int32_t group_size) {
  if (kernel == kKernMfma16) return occupancy_mfma16(kv_dtype, nct);
  if (kernel == kKernQuant) return occupancy_quant(kv_dtype, group_size, nct);
  return 1;
}

hipError_t launch_decode_split(const DecodeArgs& a, hipStream_t s) {
  if (a.batch <= 0) return hipSuccess;
  if (a.kernel == kKernMfma16) return a.max_splits > 0 ? launch_decode_split_mfma16(a, s) : hipSuccess;
  if (a.kernel == kKernQuant) return a.max_splits > 0 ? launch_decode_split_quant(a, s) : hipSuccess;
  dim3 grid(unsigned(a.max_splits), unsigned(a.n_q_heads), unsigned(a.batch) * unsigned(max(a.n_query, 1)));
  hipLaunchKernelGGL(decode_split_generic, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t s) {
  if (a.batch <= 0) return hipSuccess;
  // the matrix-core kernels merge split segments themselves, or leave them to
  // the merge launch
  if (a.kernel == kKernMfma16 || a.kernel == kKernQuant)
    return a.defer_merge ? launch_decode_merge(a, s) : hipSuccess;
  if (a.max_splits <= 1) return hipSuccess;
  dim3 grid(unsigned(a.n_q_heads), unsigned(a.batch) * unsigned(max(a.n_query, 1)));
  hipLaunchKernelGGL(decode_combine_kernel, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
