// Writing one token's K or V vector of one head into its slot: the body of
// the append (append.hip) and of the decode step that appends its new token
// itself (the matrix-core split kernels).
//
// "The 8GB VRAM Breakthrough ...", section 5 (flowchart): a token-position
// router sends sink tokens to the FP16 block pool and the body through a
// fused quantizer (per-group asymmetric INT4, or FP8) into the compressed
// pool.  Section 4 fixes the formats: FP8 E4M3 with a per-head dynamic scale;
// INT4 codes q in [0, 15] with fp16 scale s and zero z, x = (q - z) * s.
//
// The quantize rule (include/pa.h, "Numerics") is computed with one IEEE
// fp32 operation per step, rounded to nearest even (no contraction), so
// every code, scale and zero is reproducible bit for bit.
#pragma once

#include "common.hpp"

namespace pa {
namespace app {

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
#pragma clang fp contract(off)
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

// A pair of consecutive input elements (2i, 2i + 1) of dtype dt as floats:
// one 4-byte load for 16-bit inputs, one 8-byte load for fp32.
__device__ inline void load_pair(const void* p, size_t i, int dt, float (&x)[2]) {
  if (dt == kF32) {
    const float2 v = *reinterpret_cast<const float2*>(static_cast<const float*>(p) + 2 * i);
    x[0] = v.x;
    x[1] = v.y;
    return;
  }
  const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p) + 2 * i);
  const uint16_t lo = uint16_t(w & 0xFFFFu), hi = uint16_t(w >> 16);
  x[0] = dt == kF16 ? f16_bits_to_f32(lo) : bf16_bits_to_f32(lo);
  x[1] = dt == kF16 ? f16_bits_to_f32(hi) : bf16_bits_to_f32(hi);
}

// One wave writes token t of block `id` (a body or, from num_blocks on,
// FP16 sink-arena block), head h, K (kind 0) or V (kind 1), from row `row`
// of the [rows][H][D] input of dtype in_dt.  Lane l holds the dimension pairs
// k = l + 64*m (dims 2k, 2k+1): the two nibbles of a packed INT4 byte always
// come from one lane, a byte never mixes two tokens, and the pair is adjacent
// in the raw K layout (one store).  MP = 1 for head_dim <= 128, 2 to 256.
template <int MP>
__device__ inline void append_one(const PoolDev& p, const void* kin, const void* vin, int in_dt,
                                  size_t row, int h, int kind, int id, int t, int lane) {
  const int H = p.n_kv_heads, D = p.head_dim, N = p.num_blocks;
  const void* src = kind ? vin : kin;
  const size_t base = (row * H + h) * D;
  const int npairs = D >> 1;
  float x[MP][2];
  bool has[MP];
#pragma unroll
  for (int m = 0; m < MP; ++m) {
    const int k = lane + 64 * m;
    has[m] = k < npairs;
    x[m][0] = x[m][1] = 0.f;
    if (has[m]) load_pair(src, base / 2 + k, in_dt, x[m]);
  }
  if (id < 0 || id >= N + p.num_sink_blocks) return;
  const int bs = p.block_size;  // 16; 8 or 32 for raw 16-bit pools

  // ---- FP16 sink arena and raw bodies: plain stores --------------------------
  const bool sink = id >= N;
  if (sink || is_raw_dev(p.kv_dtype)) {
    const int arr = sink ? (kind ? kArrSV : kArrSK) : (kind ? kArrV : kArrK);
    const int dt = sink ? int(kF16) : p.kv_dtype;
    uint8_t* slab = p.base + p.off[arr] + (size_t(sink ? id - N : id) * H + h) * p.slab[arr];
#pragma unroll
    for (int m = 0; m < MP; ++m) {
      if (!has[m]) continue;
      const int d = 2 * (lane + 64 * m);
      if (kind == 0) {  // dims d, d + 1 adjacent: one store
        const int idx = raw_k_elem(t, d, bs);
        if (dt == kF32) {
          *reinterpret_cast<float2*>(reinterpret_cast<float*>(slab) + idx) = float2{x[m][0], x[m][1]};
        } else {
          const uint32_t w = dt == kF16 ? uint32_t(f32_to_f16_bits(x[m][0])) | (uint32_t(f32_to_f16_bits(x[m][1])) << 16)
                                        : uint32_t(f32_to_bf16_bits(x[m][0])) | (uint32_t(f32_to_bf16_bits(x[m][1])) << 16);
          *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(slab) + idx) = w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int idx = raw_v_elem(t, d + e, D, bs);
          if (dt == kF32)
            reinterpret_cast<float*>(slab)[idx] = x[m][e];
          else if (dt == kF16)
            reinterpret_cast<uint16_t*>(slab)[idx] = f32_to_f16_bits(x[m][e]);
          else
            reinterpret_cast<uint16_t*>(slab)[idx] = f32_to_bf16_bits(x[m][e]);
        }
      }
    }
    return;
  }

  quantize_store<MP>(p, id, t, h, kind, x, has, lane);
}

}  // namespace app
}  // namespace pa
