// Matrix-core decode split kernel for mixed-precision pools: FP16 sink blocks
// plus an asymmetric INT4 (one group per token and head) or FP8 E4M3 body,
// head_dim 128, fp16 queries.
//
// "The 8GB VRAM Breakthrough ...", section 5 ("On-the-Fly Register
// Dequantization"): the kernel loads the packed codes and their (scale, zero)
// and dequantizes in registers, never writing an FP16 copy back; section 4
// fixes the formats (INT4 x = (q - z) * s; FP8 E4M3 times a per-head scale);
// section 5's flowchart routes the sink tokens to an FP16 pool.
//
// The dequantization is folded out of the dot products so that the
// matrix-core operands stay exact:
//   INT4  S[t] = s_t * (sum_d q_d c_td - z_t * sum_d q_d)
//         O[d] = sum_t c_td (s_t p_t) - sum_t z_t s_t p_t
//   FP8   S[t] = s_t * sum_d q_d e(c_td),  O[d] = sum_t e(c_td) (s_t p_t)
// The codes enter the fp16 matrix cores exactly: an INT4 nibble n becomes the
// fp16 value n (0x6400|n is 1024+n, then an exact packed-fp16 subtract); an
// E4M3 code goes through the hardware FP8->fp16 conversion with scale 1
// (every E4M3 value is an fp16 value).  The weights
// s_t p_t are split into an fp16 high part and residual (~22 bits).  The
// softmax reference tracks the exact running max here, so every weight is
// <= 1 and s_t p_t stays inside the fp16 range.
//
// Scheduling (flattened, evenly chunked work list; 4 waves per workgroup;
// merge) is shared with the 16-bit kernel (decode_common.hpp).  The small
// quantized blocks (2,176 B for INT4, 4,160 B for FP8 per (block, head)) are
// prefetched NB-1 blocks ahead per wave.
#include <cstdlib>

#include "decode_common.hpp"

namespace pa {

namespace {

using namespace dec;

typedef _Float16 h8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef _Float16 h4 __attribute__((__vector_size__(4 * sizeof(_Float16))));
typedef _Float16 h2 __attribute__((__vector_size__(2 * sizeof(_Float16))));

// Nibbles at bits shift..shift+3 and shift+16..shift+19 of x -> fp16 pair.
__device__ inline uint32_t nib2h(uint32_t x, int shift) {
  const uint32_t t = ((x >> shift) & 0x000F000Fu) | 0x64006400u;  // 1024 + n
  h2 v = __builtin_bit_cast(h2, t) - h2{_Float16(1024.f), _Float16(1024.f)};
  return __builtin_bit_cast(uint32_t, v);
}

// E4M3 codes in bytes 0,1 (HI = false) or 2,3 (HI = true) of y -> fp16 pair,
// exactly (the hardware conversion with scale 1 reproduces the OCP table for
// every finite code; NaN codes give NaN).
template <bool HI>
__device__ inline uint32_t fp8pair(uint32_t y) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(y, 1.0f, HI));
}

__device__ inline float h_lo(uint32_t w) { return f16_bits_to_f32(uint16_t(w & 0xFFFFu)); }
__device__ inline float h_hi(uint32_t w) { return f16_bits_to_f32(uint16_t(w >> 16)); }

struct BufI4 {
  u32x4 kc, vc;          // K codes (dims 32kk+8g+0..7 per dword kk), V codes (dword j: tokens 4g+i, dims 8r+2j, +1)
  u32x2 ks, kz, vs, vz;  // fp16 scale/zero of tokens 4g..4g+3
};

struct BufF8 {
  u32x4 kc0, kc1, vc0, vc1;  // K units s = 0, 1; V units u = 0, 1
  u32x2 ks, vs;
};

template <int KIND>
struct Quant;

template <>
struct Quant<kInt4> {
  typedef BufI4 Buf;
};

template <>
struct Quant<kFp8> {
  typedef BufF8 Buf;
};

// NB = register buffers per wave (NB-1 blocks prefetched ahead).
template <int KIND, int NB>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(NB == 2 ? 3 : 2))) void decode_split_quant(DecodeArgs a) {
  typedef typename Quant<KIND>::Buf Buf;
  typedef Mfma<_Float16> MF;
  __shared__ Shared sh;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 4, c = lane & 15;
  const PoolDev& p = a.pool;
  const int H = p.n_kv_heads, Hq = a.n_q_heads, G = Hq / H, N = p.num_blocks;
  const int SP = p.sink_per_seq;
  zero_empty_rows<_Float16>(a);
  const Units um = setup_units(a, sh, w, lane);
  int b = 0, fb = 0;

  const float sl2 = a.scale_log2;
  const uint8_t* base = p.base;
  const int32_t* trow = a.tables;
  int h = 0, L = 0;
  h8 qp[4];            // Q^T fragments in the code's element order
  float qsum = 0.f;    // sum of the head's query (INT4 zero-point term)
  f32x4 o[kNT];
  float m_ref = -__builtin_inff(), l_run = 0.f, corr = 0.f;

  auto ok = [&](int id) { return id >= 0 && id < N; };

  // softmax update for one block's 4 scores per lane; returns the weights
  auto softmax = [&](const float (&x)[4], int valid, float (&pw)[4]) {
    float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    const bool move = bm > m_ref;
    if (__any(move)) {
      const float m_new = move ? bm : m_ref;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      l_run *= alpha;
      corr *= alpha;
#pragma unroll
      for (int T_ = 0; T_ < kNT; ++T_) o[T_] *= alpha;
      m_ref = m_new;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pw[i] = (4 * g + i < valid) ? __builtin_amdgcn_exp2f(x[i] - m_ref) : 0.f;
      l_run += pw[i];
    }
  };

  // ---- body blocks ------------------------------------------------------------
  auto fetch = [&](int id, Buf& bf) {
    const size_t sid = size_t(ok(id) ? id : 0) * H + h;  // unconditional load
    const uint8_t* kc = base + p.off[kArrK] + sid * p.slab[kArrK];
    const uint8_t* vc = base + p.off[kArrV] + sid * p.slab[kArrV];
    const uint8_t* ks = base + p.off[kArrKS] + sid * p.slab[kArrKS] + 8 * g;
    const uint8_t* vs = base + p.off[kArrVS] + sid * p.slab[kArrVS] + 8 * g;
    if constexpr (KIND == kInt4) {
      bf.kc = *reinterpret_cast<const u32x4*>(kc + lane * 16);
      bf.vc = *reinterpret_cast<const u32x4*>(vc + lane * 16);
      bf.ks = *reinterpret_cast<const u32x2*>(ks);
      bf.kz = *reinterpret_cast<const u32x2*>(base + p.off[kArrKZ] + sid * p.slab[kArrKZ] + 8 * g);
      bf.vs = *reinterpret_cast<const u32x2*>(vs);
      bf.vz = *reinterpret_cast<const u32x2*>(base + p.off[kArrVZ] + sid * p.slab[kArrVZ] + 8 * g);
    } else {
      bf.kc0 = *reinterpret_cast<const u32x4*>(kc + lane * 16);
      bf.kc1 = *reinterpret_cast<const u32x4*>(kc + 1024 + lane * 16);
      bf.vc0 = *reinterpret_cast<const u32x4*>(vc + lane * 16);
      bf.vc1 = *reinterpret_cast<const u32x4*>(vc + 1024 + lane * 16);
      bf.ks = *reinterpret_cast<const u32x2*>(ks);
      bf.vs = *reinterpret_cast<const u32x2*>(vs);
    }
  };

  auto consume = [&](int valid, const Buf& bf) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float ksc[4], vsc[4];
    ksc[0] = h_lo(bf.ks[0]); ksc[1] = h_hi(bf.ks[0]); ksc[2] = h_lo(bf.ks[1]); ksc[3] = h_hi(bf.ks[1]);
    vsc[0] = h_lo(bf.vs[0]); vsc[1] = h_hi(bf.vs[0]); vsc[2] = h_lo(bf.vs[1]); vsc[3] = h_hi(bf.vs[1]);
    float x[4];
    if constexpr (KIND == kInt4) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint32_t cw = bf.kc[kk];
        const u32x4 av = {nib2h(cw, 0), nib2h(cw, 4), nib2h(cw, 8), nib2h(cw, 12)};
        acc = MF::qk(__builtin_bit_cast(h8, av), qp[kk], acc);
      }
      float kzv[4];
      kzv[0] = h_lo(bf.kz[0]); kzv[1] = h_hi(bf.kz[0]); kzv[2] = h_lo(bf.kz[1]); kzv[3] = h_hi(bf.kz[1]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        x[i] = (4 * g + i < valid) ? ksc[i] * (acc[i] - kzv[i] * qsum) * sl2 : -__builtin_inff();
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x4 u = kk < 2 ? bf.kc0 : bf.kc1;
        const uint32_t x0 = u[(kk & 1) * 2], x1 = u[(kk & 1) * 2 + 1];
        const u32x4 av = {fp8pair<false>(x0), fp8pair<true>(x0), fp8pair<false>(x1), fp8pair<true>(x1)};
        acc = MF::qk(__builtin_bit_cast(h8, av), qp[kk], acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        x[i] = (4 * g + i < valid) ? ksc[i] * acc[i] * sl2 : -__builtin_inff();
    }
    float pw[4];
    softmax(x, valid, pw);
    // weights times the V scale; tail tokens' metadata may be garbage: select
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = (4 * g + i < valid) ? vsc[i] * pw[i] : 0.f;
    // FP8: zero the bytes of tail tokens (unwritten slots may hold NaN codes)
    const int t0 = 4 * g;
    const uint32_t vmask = (t0 + 0 < valid ? 0x000000FFu : 0u) | (t0 + 1 < valid ? 0x0000FF00u : 0u) |
                           (t0 + 2 < valid ? 0x00FF0000u : 0u) | (t0 + 3 < valid ? 0xFF000000u : 0u);
    if constexpr (KIND == kInt4) {
      float vzv[4];
      vzv[0] = h_lo(bf.vz[0]); vzv[1] = h_hi(bf.vz[0]); vzv[2] = h_lo(bf.vz[1]); vzv[3] = h_hi(bf.vz[1]);
#pragma unroll
      for (int i = 0; i < 4; ++i) corr += (4 * g + i < valid) ? vzv[i] * pv[i] : 0.f;
    }
    // B operand in the token order of the code pairs: INT4 (t0, t2), (t1, t3);
    // FP8 natural
    h4 bhi, blo;
    const int ord[4] = {0, KIND == kInt4 ? 2 : 1, KIND == kInt4 ? 1 : 2, 3};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bhi[e] = _Float16(pv[ord[e]]);
      blo[e] = _Float16(pv[ord[e]] - float(bhi[e]));
    }
#pragma unroll
    for (int T_ = 0; T_ < kNT; ++T_) {
      uint32_t lo, hi;
      if constexpr (KIND == kInt4) {
        const uint32_t cw = bf.vc[T_ >> 1];
        const int par = T_ & 1;
        lo = nib2h(cw, 4 * par);      // tokens (t0, t2)
        hi = nib2h(cw, 8 + 4 * par);  // tokens (t1, t3)
      } else {
        const uint32_t cw = (T_ < 4 ? bf.vc0[T_] : bf.vc1[T_ - 4]) & vmask;
        lo = fp8pair<false>(cw);  // tokens (t0, t1)
        hi = fp8pair<true>(cw);   // tokens (t2, t3)
      }
      const u32x2 av = {lo, hi};
      const h4 at = __builtin_bit_cast(h4, av);
      o[T_] = MF::pv(at, bhi, o[T_]);
      o[T_] = MF::pv(at, blo, o[T_]);
    }
  };

  // ---- FP16 sink blocks (raw layout, natural element order) ----------------------
  auto consume_sink = [&](int id, int valid) {
    const size_t sid = size_t(id - N) * H + h;
    const _Float16* ks = reinterpret_cast<const _Float16*>(base + p.off[kArrSK] + sid * p.slab[kArrSK]);
    const _Float16* vs = reinterpret_cast<const _Float16*>(base + p.off[kArrSV] + sid * p.slab[kArrSV]);
    const _Float16* qn = static_cast<const _Float16*>(a.q) + (size_t(b) * Hq + h * G + c) * kD + 8 * g;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const h8 kf = *reinterpret_cast<const h8*>(ks + (kk * 64 + lane) * 8);
      const h8 qf = c < G ? *reinterpret_cast<const h8*>(qn + 32 * kk) : h8{};
      acc = MF::qk(kf, qf, acc);
    }
    float x[4], pw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (4 * g + i < valid) ? acc[i] * sl2 : -__builtin_inff();
    softmax(x, valid, pw);
    h4 bhi, blo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pe = pw[i];
      bhi[i] = _Float16(pe);
      blo[i] = _Float16(pe - float(bhi[i]));
    }
    const int t0 = 4 * g;
    const uint32_t m01 = (t0 + 0 < valid ? 0x0000FFFFu : 0u) | (t0 + 1 < valid ? 0xFFFF0000u : 0u);
    const uint32_t m23 = (t0 + 2 < valid ? 0x0000FFFFu : 0u) | (t0 + 3 < valid ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      u32x4 dw = *reinterpret_cast<const u32x4*>(vs + (u * 64 + lane) * 8);
      dw[0] &= m01;  // unwritten tail slots may hold any bits
      dw[1] &= m23;
      dw[2] &= m01;
      dw[3] &= m23;
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const u32x2 av = {dw[2 * par], dw[2 * par + 1]};
        const h4 at = __builtin_bit_cast(h4, av);
        o[2 * u + par] = MF::pv(at, bhi, o[2 * u + par]);
        o[2 * u + par] = MF::pv(at, blo, o[2 * u + par]);
      }
    }
  };

  const int own_unit = int(blockIdx.x) * um.per();
  for (int unit = own_unit; unit >= 0; unit = next_unit(a, sh, um)) {
  const int pos0 = um.start(unit), pos1 = um.end(unit);
  if (pos0 >= pos1) continue;  // a region past the end of the work
  locate(a, sh, w, lane, pos0, b, fb);
  // progress-based priority in the owner's prefix; queued units run at the
  // base priority, behind the workgroups still streaming their own prefix
  const int prio_span = unit == own_unit ? pos1 - pos0 : 0;
  int pos = pos0;
  bool first = true;
  int jbeg = 0, jend = 0, nb = 0;
  while (next_piece(a, pos, pos1, b, fb, h, jbeg, jend, nb)) {
    L = seq_len(a, b);
    trow = a.tables + size_t(b) * a.max_blocks_per_seq;
    {
      // Q^T fragment of head c (dims 32kk + 8g + 0..7), permuted into the order
      // in which the code conversion delivers the K elements
      const _Float16* qn = static_cast<const _Float16*>(a.q) + (size_t(b) * Hq + h * G + c) * kD + 8 * g;
      float part = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const h8 q = c < G ? *reinterpret_cast<const h8*>(qn + 32 * kk) : h8{};
#pragma unroll
        for (int e = 0; e < 8; ++e) part += float(q[e]);
        if constexpr (KIND == kInt4)
          qp[kk] = h8{q[0], q[4], q[1], q[5], q[2], q[6], q[3], q[7]};
        else
          qp[kk] = q;
      }
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);
      qsum = part;
    }
#pragma unroll
    for (int T_ = 0; T_ < kNT; ++T_) o[T_] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_ref = -__builtin_inff();
    l_run = 0.f;
    corr = 0.f;

    // sink blocks of the piece (logical blocks < SP), one at a time
    const int send = min(jend, SP);
    for (int j = jbeg + w; j < send; j += kWaves) {
      const int id = trow[j];
      if (id >= N && id < N + p.num_sink_blocks) consume_sink(id, L - 16 * j);
    }

    // body blocks, software-pipelined NB-1 blocks ahead with NB register
    // buffers; loads are unconditional so no branch separates them from
    // their waits (past the end the last block is re-read: an L2 hit)
    const int jw = max(jbeg, SP) + w;
    const int n = jw < jend ? (jend - jw + kWaves - 1) / kWaves : 0;
    if (n > 0) {
      auto id_of = [&](int k) { return trow[jw + kWaves * min(k, n - 1)]; };
      auto valid_of = [&](int k, int id) { return ok(id) ? L - 16 * (jw + kWaves * k) : 0; };
      Buf buf[NB];
      int ids[NB];
#pragma unroll
      for (int s = 0; s < NB - 1; ++s) {
        ids[s] = id_of(s);
        fetch(ids[s], buf[s]);
      }
      int k = 0;
      for (; k + NB <= n; k += NB) {
        prio_from_progress(a, pos - pos0 + kWaves * k, prio_span);
#pragma unroll
        for (int s = 0; s < NB; ++s) {
          const int nxt = (s + NB - 1) % NB;
          ids[nxt] = id_of(k + s + NB - 1);
          fetch(ids[nxt], buf[nxt]);
          consume(valid_of(k + s, ids[s]), buf[s]);
        }
      }
#pragma unroll
      for (int s = 0; s < NB - 1; ++s)
        if (k + s < n) consume(valid_of(k + s, ids[s]), buf[s]);
    }

    // ---- finish the piece: zero-point correction, FP8 scale, merge ----------------
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    if constexpr (KIND == kInt4) {
      corr += __shfl_xor(corr, 16, 64);
      corr += __shfl_xor(corr, 32, 64);
#pragma unroll
      for (int T_ = 0; T_ < kNT; ++T_) o[T_] -= corr;
    }
    stash_piece(sh, w, g, c, o, m_ref, l_run);
    finish_piece<_Float16>(a, sh, out_map(a), jbeg == 0 && jend == nb, first ? 0 : 1, unit, b, h,
                      fb + h * nb, nb, um);
    pos += jend - jbeg;
    first = false;
  }
  }
}

}  // namespace

// Prefetch depth: PA_QUANT_NB = 2 (default, 3 waves per SIMD), 3, 4 or 6
// (2 waves per SIMD).
int quant_nb() {
  static int nb = 0;
  if (nb == 0) {
    const char* e = std::getenv("PA_QUANT_NB");
    const int v = e ? std::atoi(e) : 2;
    nb = (v == 3 || v == 4 || v == 6) ? v : 2;
  }
  return nb;
}

template <int KIND, int NB>
int occ_of() {
  int n = 0;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_split_quant<KIND, NB>,
                                                                     kWaves * 64, 0);
  return (e == hipSuccess && n > 0) ? n : 2;
}

template <int KIND>
int occ_kind() {
  switch (quant_nb()) {
    case 3: return occ_of<KIND, 3>();
    case 4: return occ_of<KIND, 4>();
    case 6: return occ_of<KIND, 6>();
    default: return occ_of<KIND, 2>();
  }
}

template <int KIND>
void launch_kind(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(unsigned(a.max_splits)), block(kWaves * 64);
  switch (quant_nb()) {
    case 3: hipLaunchKernelGGL((decode_split_quant<KIND, 3>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_split_quant<KIND, 4>), grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((decode_split_quant<KIND, 6>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((decode_split_quant<KIND, 2>), grid, block, 0, s, a); break;
  }
}

int occupancy_quant(int32_t kv_dtype) {
  static int cache[2] = {0, 0};
  const int i = kv_dtype == kInt4 ? 0 : 1;
  if (cache[i] == 0) cache[i] = i == 0 ? occ_kind<kInt4>() : occ_kind<kFp8>();
  return cache[i];
}

hipError_t launch_decode_split_quant(const DecodeArgs& a, hipStream_t s) {
  if (a.pool.kv_dtype == kInt4)
    launch_kind<kInt4>(a, s);
  else
    launch_kind<kFp8>(a, s);
  return hipGetLastError();
}

}  // namespace pa
