// KV append with fused quantize-on-write, and the copy-on-write block copy.
//
// "The 8GB VRAM Breakthrough ...", section 5 (flowchart): a token-position
// router sends sink tokens to the FP16 block pool and the body through a
// fused quantizer (per-group asymmetric INT4, or FP8) into the compressed
// pool.  Section 4 fixes the formats: FP8 E4M3 with a per-head dynamic scale;
// INT4 codes q in [0, 15] with fp16 scale s and zero z, x = (q - z) * s.
// Section 3 ("Copy-on-Write (CoW) Prefix Sharing"): before a sequence writes
// into a partially filled shared block, a fresh block receives a copy.
//
// The quantize rule (include/pa.h, "Numerics") is computed with one IEEE
// fp32 operation per step, rounded to nearest even, so every code, scale and
// zero is reproducible bit for bit.
#pragma clang fp contract(off)

#include "common.hpp"

namespace pa {

namespace {

constexpr int kWaves = 4;  // waves per workgroup

// Min / max over the 64 lanes of a wave (all lanes active), every lane gets
// the result: DPP moves inside each 16-lane row (quad swaps, then the half-row
// and row mirrors), then the gfx950 row swaps across the four rows -- all in
// registers, no LDS round trip.  Exact in any order.
template <int CTRL>
__device__ inline float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <bool MAX>
__device__ inline float wave_extreme(float x) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); };
  x = op(x, dpp_move<0xB1>(x));   // quad [1,0,3,2]
  x = op(x, dpp_move<0x4E>(x));   // quad [2,3,0,1]
  x = op(x, dpp_move<0x141>(x));  // row half mirror
  x = op(x, dpp_move<0x140>(x));  // row mirror
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Quantize one (token t, kv head h, K-or-V) vector of a body block `id` and
// store codes, scales and zeros: lane l holds dims 2k, 2k+1 for
// k = l + 64*m (valid where has[m]).  Inputs are first rounded to fp16.
template <int MP>
__device__ inline void quantize_store(const PoolDev& p, int id, int t, int h, int kind,
                                      float (&x)[MP][2], const bool (&has)[MP], int lane) {
  const int H = p.n_kv_heads, D = p.head_dim;
#pragma unroll
  for (int m = 0; m < MP; ++m) {
    x[m][0] = f16_bits_to_f32(f32_to_f16_bits(x[m][0]));
    x[m][1] = f16_bits_to_f32(f32_to_f16_bits(x[m][1]));
  }
  const size_t slab_id = size_t(id) * H + h;

  if (p.kv_dtype == kFp8) {
    float amax = 0.f;
#pragma unroll
    for (int m = 0; m < MP; ++m)
      if (has[m]) amax = fmaxf(amax, fmaxf(fabsf(x[m][0]), fabsf(x[m][1])));
    amax = wave_extreme<true>(amax);
    uint16_t sb = f32_to_f16_bits(__fdiv_rn(amax, 448.0f));
    float s = f16_bits_to_f32(sb);
    if (s == 0.f) {
      s = 1.f;
      sb = 0x3C00;
    }
    const int arr = kind ? kArrV : kArrK;
    uint8_t* codes = p.base + p.off[arr] + slab_id * p.slab[arr];
#pragma unroll
    for (int m = 0; m < MP; ++m) {
      if (!has[m]) continue;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int d = 2 * (lane + 64 * m) + e;
        float y = __fdiv_rn(x[m][e], s);
        y = fminf(fmaxf(y, -448.0f), 448.0f);
        codes[kind ? fp8_v_byte(t, d, D) : fp8_k_byte(t, d)] = uint8_t(e4m3_encode(y));
      }
    }
    if (lane == 0) {
      const int sarr = kind ? kArrVS : kArrKS;
      reinterpret_cast<uint16_t*>(p.base + p.off[sarr] + slab_id * p.slab[sarr])[t] = sb;
    }
    return;
  }

  // INT4, groups of gs dims: per group min/max, then s, z, codes.
  const int gs = p.group_size, ng = D / gs;
  const int arr = kind ? kArrV : kArrK;
  uint8_t* codes = p.base + p.off[arr] + slab_id * p.slab[arr];
  const int sarr = kind ? kArrVS : kArrKS, zarr = kind ? kArrVZ : kArrKZ;
  uint16_t* sc = reinterpret_cast<uint16_t*>(p.base + p.off[sarr] + slab_id * p.slab[sarr]);
  uint16_t* zp = reinterpret_cast<uint16_t*>(p.base + p.off[zarr] + slab_id * p.slab[zarr]);
  for (int gi = 0; gi < ng; ++gi) {
    float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
    for (int m = 0; m < MP; ++m) {
      const int k = lane + 64 * m;
      if (has[m] && (2 * k) / gs == gi) {
        mn = fminf(mn, fminf(x[m][0], x[m][1]));
        mx = fmaxf(mx, fmaxf(x[m][0], x[m][1]));
      }
    }
    mn = wave_extreme<false>(mn);
    mx = wave_extreme<true>(mx);
    uint16_t sb = f32_to_f16_bits(__fdiv_rn(__fsub_rn(mx, mn), 15.0f));
    float s = f16_bits_to_f32(sb);
    if (s == 0.f) {
      s = 1.f;
      sb = 0x3C00;
    }
    uint16_t zb = f32_to_f16_bits(__fdiv_rn(-mn, s));
    float z = f16_bits_to_f32(zb);
    if (__builtin_isinf(z)) {
      zb = z > 0.f ? uint16_t(0x7BFF) : uint16_t(0xFBFF);  // +-65504
      z = f16_bits_to_f32(zb);
    }
#pragma unroll
    for (int m = 0; m < MP; ++m) {
      const int k = lane + 64 * m;
      if (!(has[m] && (2 * k) / gs == gi)) continue;
      uint32_t q[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float r = rintf(__fadd_rn(__fdiv_rn(x[m][e], s), z));
        q[e] = uint32_t(fminf(fmaxf(r, 0.f), 15.f));
      }
      codes[kind ? int4_v_byte(t, k, D) : int4_k_byte(t, k, D)] = uint8_t(q[0] | (q[1] << 4));
      if (2 * k == gi * gs) {
        sc[t * ng + gi] = sb;
        zp[t * ng + gi] = zb;
      }
    }
  }
}

// One wave per (token, kv head, K-or-V).  Lane `l` holds the dimension pairs
// k = l + 64*m (dims 2k, 2k+1): the two nibbles of a packed INT4 byte always
// come from one lane, and a byte never mixes two tokens.
template <int MP>
__global__ __launch_bounds__(kWaves * 64) void append_kv_kernel(PoolDev p, const void* kin,
                                                                const void* vin, int in_dt,
                                                                const int32_t* slots, int n) {
  const int lane = threadIdx.x & 63;
  const long gw = (long(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int H = p.n_kv_heads, D = p.head_dim, N = p.num_blocks;
  const int kind = int(gw & 1);  // 0 = K, 1 = V
  const long th = gw >> 1;
  const long tok = th / H;
  const int h = int(th % H);
  if (tok >= n) return;
  // the token's values and its slot are loaded together (the values do not
  // depend on the slot: one memory round trip instead of two)
  const void* src = kind ? vin : kin;
  const size_t base = (size_t(tok) * H + h) * D;
  const int npairs = D >> 1;
  float x[MP][2];
  bool has[MP];
#pragma unroll
  for (int m = 0; m < MP; ++m) {
    const int k = lane + 64 * m;
    has[m] = k < npairs;
    x[m][0] = has[m] ? load_as_f32(src, base + 2 * k, in_dt) : 0.f;
    x[m][1] = has[m] ? load_as_f32(src, base + 2 * k + 1, in_dt) : 0.f;
  }
  const int slot = slots[tok];
  if (slot < 0) return;
  const int bs = p.block_size;  // 16; 8 or 32 for raw 16-bit pools
  const int id = slot / bs, t = slot % bs;
  if (id >= N + p.num_sink_blocks) return;

  // ---- FP16 sink arena and raw bodies: plain stores --------------------------
  const bool sink = id >= N;
  if (sink || is_raw_dev(p.kv_dtype)) {
    const int arr = sink ? (kind ? kArrSV : kArrSK) : (kind ? kArrV : kArrK);
    const int dt = sink ? int(kF16) : p.kv_dtype;
    uint8_t* slab = p.base + p.off[arr] + (size_t(sink ? id - N : id) * H + h) * p.slab[arr];
#pragma unroll
    for (int m = 0; m < MP; ++m) {
      if (!has[m]) continue;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int d = 2 * (lane + 64 * m) + e;
        const int idx = kind ? raw_v_elem(t, d, D, bs) : raw_k_elem(t, d, bs);
        if (dt == kF32)
          reinterpret_cast<float*>(slab)[idx] = x[m][e];
        else if (dt == kF16)
          reinterpret_cast<uint16_t*>(slab)[idx] = f32_to_f16_bits(x[m][e]);
        else
          reinterpret_cast<uint16_t*>(slab)[idx] = f32_to_bf16_bits(x[m][e]);
      }
    }
    return;
  }

  quantize_store<MP>(p, id, t, h, kind, x, has, lane);
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
  quantize_store<kMigrateMP>(p, dst, t, h, kind, x, has, lane);
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
  const unsigned grid = unsigned((waves + kWaves - 1) / kWaves);
  if (p.head_dim <= 128)
    hipLaunchKernelGGL(append_kv_kernel<1>, dim3(grid), dim3(kWaves * 64), 0, s, p, k, v, in_dtype,
                       slots, n_tokens);
  else
    hipLaunchKernelGGL(append_kv_kernel<2>, dim3(grid), dim3(kWaves * 64), 0, s, p, k, v, in_dtype,
                       slots, n_tokens);
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
