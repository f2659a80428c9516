// Matrix-core decode split kernel for mixed-precision pools: FP16 sink and
// window blocks plus an asymmetric INT4 (groups of 128 or 64 dims per token
// and head) or FP8 E4M3 body, head_dim 128, fp16 queries.
//
// "The 8GB VRAM Breakthrough ...", section 5 ("On-the-Fly Register
// Dequantization"): the kernel loads the packed codes and their (scale, zero)
// and dequantizes in registers, never writing an FP16 copy back; section 4
// fixes the formats (INT4 x = (q - z) * s; FP8 E4M3 times a per-head scale);
// section 5's flowchart routes the sink tokens to an FP16 pool.
//
// The dequantization is folded out of the dot products so that the
// matrix-core operands stay exact:
//   INT4  S[t] = sum_k s_tk * (sum_{d in k} q_d c_td - z_tk * sum_{d in k} q_d)
//         O[d] = sum_t c_td (s_tk p_t) - sum_t z_tk s_tk p_t   (k = group of d)
//   FP8   S[t] = s_t * sum_d q_d e(c_td),  O[d] = sum_t e(c_td) (s_t p_t)
// The codes enter the fp16 matrix cores exactly: an INT4 nibble n at bits 0..3
// of a half is the fp16 subnormal n * 2^-24, at bits 4..7 the subnormal
// 16n * 2^-24 (one AND per two codes; the matrix cores take subnormal fp16
// operands exactly), and the powers of two are taken out again after the
// products; an E4M3 code goes through the hardware FP8->fp16 conversion with
// scale 1 (every E4M3 value is an fp16 value).  The weights
// s_t p_t are split into an fp16 high part and residual (~22 bits).  The
// softmax reference moves only when a block's max passes it by more than 2
// (log2 units), so every weight is <= 4; the largest scales -- INT4
// fp16(131,008 / 15) = 8,736 for fp16 inputs, FP8 65,504 / 448 -- times 4
// stay inside the fp16 range.
//
// Scheduling (flattened, evenly chunked work list; 4 waves per workgroup;
// merge) is shared with the 16-bit kernel (decode_common.hpp).  The small
// quantized blocks (2,176 B for INT4, 4,160 B for FP8 per (block, head)) are
// prefetched NB-1 blocks ahead per wave.
#include <cstdlib>
#include <type_traits>

#include "append_common.hpp"
#include "decode_common.hpp"

namespace pa {

namespace {

using namespace dec;

typedef _Float16 h8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef _Float16 h4 __attribute__((__vector_size__(4 * sizeof(_Float16))));
typedef _Float16 h2 __attribute__((__vector_size__(2 * sizeof(_Float16))));

// INT4 codes to exact fp16 subnormals.  sub4(x): the half pairs of the
// nibbles at bits (0, 16) and (8, 24) at scale 1 -- n reads as n * 2^-24 --
// and at bits (4, 20) and (12, 28) at scale 16 -- n reads as 16n * 2^-24:
// {n0 n4, 16 n1 16 n5, n2 n6, 16 n3 16 n7} (times 2^-24) for nibbles n0..n7.
__device__ inline u32x4 sub4(uint32_t x) {
  const uint32_t y = x >> 8;
  return u32x4{x & 0x000F000Fu, x & 0x00F000F0u, y & 0x000F000Fu, y & 0x00F000F0u};
}
constexpr float kSub = 16777216.f;  // 2^24: a nibble's subnormal is n / kSub

// IEEE maximum (a NaN operand gives NaN) without the canonicalizing moves
// fmaxf brings; the operands are scores, or -inf for tokens a column does
// not see
__device__ inline float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ inline float rows_vmax(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// One (block, head) slab of a pool array as a buffer: its loads take the
// slab's address from scalar registers and a 32-bit lane offset from a
// vector register (no vector address arithmetic), and a load past the slab
// reads zeros.
typedef __amdgpu_buffer_rsrc_t Slab;
__device__ inline Slab slab_rsrc(const uint8_t* p, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, int(bytes), kRsrcWord3);
}
__device__ inline u32x4 sload4(Slab r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0); }
__device__ inline u32x2 sload2(Slab r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0); }

// Keep v in a register where it is computed: a select of it then stays a
// select instead of becoming a branch around its computation.
__device__ inline float pin(float v) {
  asm volatile("" : "+v"(v));
  return v;
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

// NG = scale groups per token and head (head_dim / group size: 1 or 2).
template <int NG>
struct BufI4 {
  u32x4 kc, vc;  // K codes (dims 32kk+8g+0..7 per dword kk), V codes (dword j: tokens 4g+i, dims 8r+2j, +1)
  // fp16 (scale, zero) of tokens 4g..4g+3, token-major (token i, group k at half i*NG+k)
  uint32_t ks[2 * NG], kz[2 * NG], vs[2 * NG], vz[2 * NG];
};

struct BufF8 {
  u32x4 kc0, kc1, vc0, vc1;  // K units s = 0, 1; V units u = 0, 1
  uint32_t ks[2], vs[2];
};

// One FP16 block of the sink/window arena for one head: K in the matrix-core
// operand order, V^T in 4 dwordx4 per lane.
struct Buf16 {
  h8 k[4];
  u32x4 v[4];
};

template <int KIND, int NG>
struct Quant;

template <int NG>
struct Quant<kInt4, NG> {
  typedef BufI4<NG> Buf;
};

template <>
struct Quant<kFp8, 1> {
  typedef BufF8 Buf;
};

// NW consecutive dwords at offset off of slab r (NW = 2: 8-byte aligned; 4,
// 8: 16-byte aligned)
template <int NW>
__device__ inline void load_words(Slab r, uint32_t off, uint32_t (&d)[NW]) {
  if constexpr (NW == 2) {
    const u32x2 v = sload2(r, off);
    d[0] = v[0];
    d[1] = v[1];
  } else {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const u32x4 v = sload4(r, off + 16 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) d[4 * i + e] = v[e];
    }
  }
}

// fp16 number idx of a dword array (idx a compile-time constant after unrolling)
template <int NW>
__device__ inline float half_at(const uint32_t (&m)[NW], int idx) {
  return (idx & 1) ? h_hi(m[idx >> 1]) : h_lo(m[idx >> 1]);
}

// f16(half HI of w) * a + c as one fp32 fma (one rounding); the compiler
// makes it one mixed-precision fma that reads the fp16 operand in place.
// Written as arithmetic, not inline assembly: the compiler then inserts the
// wait a read of a transcendental result needs (as inline assembly the fma
// read an exp2 result one instruction after it and took the old value).
template <bool HI>
__device__ inline float fma_h(uint32_t w, float a, float c) {
  const h2 v = __builtin_bit_cast(h2, w);
  return __builtin_fmaf(float(v[HI ? 1 : 0]), a, c);
}

// (scale or zero of token i in group `sel`, a per-lane group index < NG) * a
// + c.  NG = 1: token i is half i & 1 of word i / 2; NG = 2: word i holds
// groups (0, 1) of token i, rotated so that group sel is its low half.
template <int NG>
__device__ inline float fma_meta(const uint32_t (&m)[2 * NG], int i, int sel, float a, float c) {
  if constexpr (NG == 1) {
    return (i & 1) ? fma_h<true>(m[i >> 1], a, c) : fma_h<false>(m[i >> 1], a, c);
  } else {
    static_assert(NG == 2, "one or two scale groups");
    return fma_h<false>(__builtin_amdgcn_alignbit(m[i], m[i], uint32_t(sel) * 16u), a, c);
  }
}

// RNE fp16 pair of (a, b) as one word
__device__ inline uint32_t pk_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, h2{_Float16(a), _Float16(b)});
}

// NB = register buffers per wave (NB-1 blocks prefetched ahead).  NCT column
// tiles of 16; CAUSAL: a verify step or prefill chunk (n_query queries per
// sequence, each seeing the cache up to its own position).
//
// Columns.  A tile's 16 matrix-core columns hold S = 16 / NG logical columns
// once per scale group: column c is logical column c % S of group c / S (NG
// = 1: every column its own).  Logical column l of tile t is the segment's
// (query, head) column t*S + l -- for decode the query head, for a verify
// step query gc / G of head gc % G -- so the B operand computes every query
// head of the KV head (and every query of the step) against one fetch of
// the block.  The V weights of column c are scaled by group c / S.  Output
// tile row r holds dim 8r + T, which lies in group (8r) / group_size =
// g * NG / 4 for the rows 4g..4g+3 a lane holds: lane (g, c) keeps its
// column when c / S is that group.  The copies of a logical column compute
// identical scores, so identical softmax statistics.  On the K side each
// group has its own accumulator (dims 32kk.. lie in group kk * NG / 4).
// The codes of a block are converted to fp16 once and serve every tile.
//
// FP16 blocks (sink and window): a settled table row reads sink blocks, then
// body blocks, then the FP16 blocks of the window (ids >= num_blocks).  The
// body loop runs over every non-sink block of the piece and gives FP16 ids no
// weight; the window's run at the end of the piece is found by a backward
// scan of the table (issued before the body loop, read after it) and
// streamed, with the piece's sink blocks, by a second pipelined loop.  FP16
// ids the body loop met before that run (a table between a multi-block
// reserve and its settle: FP16 runs between body runs) are streamed after
// it, one block at a time, by the wave that met them.
//
// RL: a batch of at most 64 sequences with no queue, whose lengths every wave
// keeps in registers (see RegLens).  AP: a decode step that appends its new
// token (a.app_k set; decode only).
template <int KIND, int NB, int NG, int NCT, bool CAUSAL, bool RL = false, bool AP = false>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(NB == 2 && NCT == 1 ? 3 : 2))) void decode_split_quant(DecodeArgs a) {
  typedef typename Quant<KIND, NG>::Buf Buf;
  typedef Mfma<_Float16> MF;
  constexpr int S = 16 / NG;  // logical columns per tile
  __shared__ SharedT<S * NCT> sh;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 4, c = lane & 15;
  const PoolDev& p = a.pool;
  const int H = p.n_kv_heads, Hq = a.n_q_heads, G = Hq / H, N = p.num_blocks;
  const int SP = p.sink_per_seq, NS = p.num_sink_blocks;
  const int gsel = c / S;                       // scale group of column c
  const int lcol = c % S;                       // its logical column within a tile
  const bool keep = gsel == g * NG / 4;         // this lane's output rows lie in that group
  const OutMap om = out_map(a);
  const int nq = om.nq, nsl = om.nsl;
  const RegLens rl = [&] {
    if constexpr (RL) return reg_lens(a, lane);
    else return RegLens{0, 0};
  }();
  const Units um = [&] {
    if constexpr (RL) return reg_units(a, rl);
    else return setup_units(a, sh, w, lane);
  }();
  auto blocks_at = [&](int bb) {
    if constexpr (RL) return rl.blocks_of(bb);
    else return blocks_of(a, sh, bb);
  };
  zero_empty_rows<_Float16>(a, blocks_at);
  int b = 0, fb = 0;

  const float sl2 = a.scale_log2;
  const float slq = KIND == kInt4 ? sl2 * kSub : sl2;  // the body's score factor
  // -1 that the compiler does not see as a constant: pv - hi stays one
  // mixed-precision fma reading hi in place (as a subtraction it would
  // convert hi on its own first)
  const float neg1 = pin(-1.f);
  const uint8_t* base = p.base;
  const int32_t* trow = a.tables;
  int hv = 0, h = 0, L = 0;  // segment hv = h * nsl + column slice
  h8 qp[NCT][4];             // Q^T fragments in the code's element order
  float qs[NCT][NG];         // per-group sums of the column's query (INT4 zero-point terms)
  f32x4 o[NCT][kNT];
  float m_ref[NCT], l_run[NCT], corr[NCT];
  int lim[NCT];              // CAUSAL: last position the lane's column of tile t may see

  auto ok = [&](int id) { return id >= 0 && id < N; };
  auto ok16 = [&](int id) { return id >= N && id < N + NS; };

  // visibility of the lane's 4 tokens of logical block jl for tile t
  auto visible = [&](int t, int valid, int jl, int i) {
    bool v = 4 * g + i < valid;
    if constexpr (CAUSAL) v = v && 16 * jl + 4 * g + i <= lim[t];
    return v;
  };

  // softmax update of tile t for one block's 4 scores per lane; returns the
  // weights (0 for tokens the column does not see)
  auto softmax = [&](int t, const float (&x)[4], const bool (&vis)[4], float (&pw)[4]) {
    float bm = vmax(vmax(x[0], x[1]), vmax(x[2], x[3]));
    bm = rows_vmax(bm);
    const bool move = bm > m_ref[t] + 2.f;
    if (__any(move)) {
      // a lane whose reference stays keeps its sums (factor 1): a column
      // that has seen no token yet keeps m_ref = -inf, where exp2(-inf -
      // -inf) would be NaN -- and a causal column can see nothing in one
      // block and something in a later one (the FP16 blocks come last)
      const float alpha = move ? __builtin_amdgcn_exp2f(m_ref[t] - bm) : 1.f;
      l_run[t] *= alpha;
      corr[t] *= alpha;
#pragma unroll
      for (int T_ = 0; T_ < kNT; ++T_) o[t][T_] *= alpha;
      m_ref[t] = move ? bm : m_ref[t];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pw[i] = vis[i] ? __builtin_amdgcn_exp2f(x[i] - m_ref[t]) : 0.f;
      l_run[t] += pw[i];
    }
  };

  // ---- body blocks ------------------------------------------------------------
  // slab addresses in scalar registers; the lane offsets are 32-bit vector
  // values computed once
  const uint32_t lo16 = uint32_t(lane) * 16u, lo_meta = uint32_t(8 * NG * g);
  auto fetch = [&](int id, Buf& bf) {
    const size_t sid = size_t(ok(id) ? id : 0) * H + h;  // unconditional load
    auto at = [&](int arr) { return slab_rsrc(base + p.off[arr] + sid * p.slab[arr], p.slab[arr]); };
    if constexpr (KIND == kInt4) {
      bf.kc = sload4(at(kArrK), lo16);
      bf.vc = sload4(at(kArrV), lo16);
      load_words(at(kArrKS), lo_meta, bf.ks);
      load_words(at(kArrKZ), lo_meta, bf.kz);
      load_words(at(kArrVS), lo_meta, bf.vs);
      load_words(at(kArrVZ), lo_meta, bf.vz);
    } else {
      const Slab kc = at(kArrK), vc = at(kArrV);
      bf.kc0 = sload4(kc, lo16);
      bf.kc1 = sload4(kc, 1024 + lo16);
      bf.vc0 = sload4(vc, lo16);
      bf.vc1 = sload4(vc, 1024 + lo16);
      load_words(at(kArrKS), lo_meta, bf.ks);
      load_words(at(kArrVS), lo_meta, bf.vs);
    }
  };

  // jl: the block's logical index (causal limits).  full (a std::bool_constant):
  // every token of the block is visible -- a whole block of a decode step --
  // so no token needs a select.
  auto consume = [&](auto full, int valid, int jl, const Buf& bf) {
    constexpr bool FULL = decltype(full)::value;
    // K codes as exact fp16 operand fragments, shared by the tiles
    u32x4 kav[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if constexpr (KIND == kInt4) {
        kav[kk] = sub4(bf.kc[kk]);
      } else {
        const u32x4 u = kk < 2 ? bf.kc0 : bf.kc1;
        const uint32_t x0 = u[(kk & 1) * 2], x1 = u[(kk & 1) * 2 + 1];
        kav[kk] = u32x4{fp8pair<false>(x0), fp8pair<true>(x0), fp8pair<false>(x1), fp8pair<true>(x1)};
      }
    }
    // B operands of the P V products, per tile
    h4 bhi[NCT], blo[NCT];
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
      bool vis[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) vis[i] = FULL || visible(t, valid, jl, i);
      float x[4];
      if constexpr (KIND == kInt4) {
        // acc = 2^-24 sum_d q_d c_d per group (the query carries the 1/16 of
        // the scale-16 codes), qs = 2^-24 sum_d q_d, slq = 2^24 sl2
        f32x4 acc[NG];
#pragma unroll
        for (int k = 0; k < NG; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          acc[kk * NG / 4] = MF::qk(__builtin_bit_cast(h8, kav[kk]), qp[t][kk], acc[kk * NG / 4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float sc = 0.f;
#pragma unroll
          for (int k = 0; k < NG; ++k)
            sc += half_at(bf.ks, i * NG + k) * (acc[k][i] - half_at(bf.kz, i * NG + k) * qs[t][k]);
          const float xs = pin(sc * slq);
          x[i] = vis[i] ? xs : -__builtin_inff();
        }
      } else {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc = MF::qk(__builtin_bit_cast(h8, kav[kk]), qp[t][kk], acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float xs = pin(half_at(bf.ks, i) * acc[i] * slq);
          x[i] = vis[i] ? xs : -__builtin_inff();
        }
      }
      float pw[4];
      softmax(t, x, vis, pw);
      // weights times the V scale of this column's group; tail tokens'
      // metadata may be garbage: select
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float w_ = pin(fma_meta<NG>(bf.vs, i, gsel, pw[i], 0.f));
        pv[i] = vis[i] ? w_ : 0.f;
      }
      if constexpr (KIND == kInt4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (FULL) {
            corr[t] = fma_meta<NG>(bf.vz, i, gsel, pv[i], corr[t]);
          } else {
            const float z_ = pin(fma_meta<NG>(bf.vz, i, gsel, pv[i], 0.f));
            corr[t] += vis[i] ? z_ : 0.f;
          }
        }
      }
      // B operand in the token order of the code pairs: INT4 (t0, t2),
      // (t1, t3); FP8 natural.  hi = fp16(pv), lo = fp16(pv - hi) (pv - hi
      // is exact in fp32)
      const int ord[4] = {0, KIND == kInt4 ? 2 : 1, KIND == kInt4 ? 1 : 2, 3};
      const uint32_t h01 = pk_f16(pv[ord[0]], pv[ord[1]]), h23 = pk_f16(pv[ord[2]], pv[ord[3]]);
      const uint32_t l01 = pk_f16(fma_h<false>(h01, neg1, pv[ord[0]]), fma_h<true>(h01, neg1, pv[ord[1]]));
      const uint32_t l23 = pk_f16(fma_h<false>(h23, neg1, pv[ord[2]]), fma_h<true>(h23, neg1, pv[ord[3]]));
      bhi[t] = __builtin_bit_cast(h4, u32x2{h01, h23});
      blo[t] = __builtin_bit_cast(h4, u32x2{l01, l23});
    }
    // FP8: zero the bytes of tail tokens (unwritten slots may hold NaN codes)
    const int t0 = 4 * g;
    const uint32_t vmask = FULL ? ~0u
                                : (t0 + 0 < valid ? 0x000000FFu : 0u) | (t0 + 1 < valid ? 0x0000FF00u : 0u) |
                                      (t0 + 2 < valid ? 0x00FF0000u : 0u) | (t0 + 3 < valid ? 0xFF000000u : 0u);
#pragma unroll
    for (int T_ = 0; T_ < kNT; ++T_) {
      uint32_t lo, hi;
      if constexpr (KIND == kInt4) {
        // output tile T holds dim 8r + T: even tiles take the scale-1 codes,
        // odd tiles the scale-16 ones
        const u32x4 nv = sub4(bf.vc[T_ >> 1]);
        const int par = T_ & 1;
        lo = nv[par];      // bits 4par: tokens (t0, t2)
        hi = nv[2 + par];  // bits 8 + 4par: tokens (t1, t3)
      } else {
        const uint32_t cw = (T_ < 4 ? bf.vc0[T_] : bf.vc1[T_ - 4]) & vmask;
        lo = fp8pair<false>(cw);  // tokens (t0, t1)
        hi = fp8pair<true>(cw);   // tokens (t2, t3)
      }
      const u32x2 av = {lo, hi};
      const h4 at = __builtin_bit_cast(h4, av);
#pragma unroll
      for (int t = 0; t < NCT; ++t) o[t][T_] = MF::pv2(at, bhi[t], blo[t], o[t][T_]);
    }
  };
  // ---- FP16 blocks of the sink/window arena (raw fp16 in operand order) ----------
  auto fetch16 = [&](int id, Buf16& bf) {
    const size_t sid = size_t(ok16(id) ? id - N : 0) * H + h;  // unconditional load
    const _Float16* ks = reinterpret_cast<const _Float16*>(base + p.off[kArrSK] + sid * p.slab[kArrSK]);
    const _Float16* vs = reinterpret_cast<const _Float16*>(base + p.off[kArrSV] + sid * p.slab[kArrSV]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) bf.k[kk] = *reinterpret_cast<const h8*>(ks + (kk * 64 + lane) * 8);
#pragma unroll
    for (int u = 0; u < 4; ++u) bf.v[u] = *reinterpret_cast<const u32x4*>(vs + (u * 64 + lane) * 8);
  };

  // qf: the query fragments in natural element order, per tile
  auto consume16 = [&](int valid, int jl, const Buf16& bf, const h8 (&qf)[NCT][4]) {
    h4 bhi[NCT], blo[NCT];
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = MF::qk(bf.k[kk], qf[t][kk], acc);
      bool vis[4];
      float x[4], pw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vis[i] = visible(t, valid, jl, i);
        x[i] = vis[i] ? acc[i] * sl2 : -__builtin_inff();
      }
      softmax(t, x, vis, pw);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bhi[t][i] = _Float16(pw[i]);
        blo[t][i] = _Float16(pw[i] - float(bhi[t][i]));
      }
    }
    const int t0 = 4 * g;
    const uint32_t m01 = (t0 + 0 < valid ? 0x0000FFFFu : 0u) | (t0 + 1 < valid ? 0xFFFF0000u : 0u);
    const uint32_t m23 = (t0 + 2 < valid ? 0x0000FFFFu : 0u) | (t0 + 3 < valid ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      u32x4 dw = bf.v[u];
      dw[0] &= m01;  // unwritten tail slots may hold any bits
      dw[1] &= m23;
      dw[2] &= m01;
      dw[3] &= m23;
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const u32x2 av = {dw[2 * par], dw[2 * par + 1]};
        const h4 at = __builtin_bit_cast(h4, av);
#pragma unroll
        for (int t = 0; t < NCT; ++t) o[t][2 * u + par] = MF::pv2(at, bhi[t], blo[t], o[t][2 * u + par]);
      }
    }
  };

  const int own_unit = um.owned(int(blockIdx.x));
  for (int unit = own_unit; unit >= 0; unit = RL ? -1 : next_unit(a, sh, um)) {
  const int pos0 = um.start(unit), pos1 = um.end(unit);
  if (pos0 >= pos1) continue;  // a region past the end of the work
  if constexpr (RL) reg_locate(um, rl, pos0, b, fb);
  else locate(a, sh, um, w, lane, pos0, b, fb);
  // progress-based priority in the owner's prefix; queued units run at the
  // base priority, behind the workgroups still streaming their own prefix
  const int prio_span = unit == own_unit ? pos1 - pos0 : 0;
  int pos = pos0;
  bool first = true;
  int jbeg = 0, jend = 0, nb = 0;
  while (next_piece(a, blocks_at, um, pos, pos1, b, fb, hv, jbeg, jend, nb)) {
    if constexpr (RL) L = rl.len_of(b);
    else L = len_of(a, sh, b);
    trow = a.tables + size_t(b) * a.max_blocks_per_seq;
    h = hv / nsl;
    // a decode step that appends its new token (a.app_k set): the workgroup
    // whose piece ends the segment writes token L - 1 of head h -- wave 0 its
    // K, wave 1 its V, quantized where the block is a body block -- before any
    // of its waves loads a block; the barrier orders those stores before the
    // other waves' loads (no other workgroup reads the segment's last block)
    if constexpr (AP && !CAUSAL) {
      if (jend == nb && nb > 0 && L >= 1) {
        if (w < 2)
          app::append_one<1>(p, a.app_k, a.app_v, a.app_dt, size_t(b), h, w, table_entry(trow + (L - 1) / 16),
                             (L - 1) % 16, lane);
        __syncthreads();
      }
    }
    const int ncol = om.cols(hv);
    const int lo = max(jbeg, SP);  // first non-sink block of the piece
    // the table's last 64 entries of the piece, for the window scan below
    int tid = p.window_tokens > 0 ? trow[max(jend - 1 - lane, 0)] : 0;
    // Q^T fragments of the lane's logical column in every tile (dims
    // 32kk + 8g + 0..7): loaded here, and permuted into the order in which
    // the code conversion delivers the K elements (and summed per group)
    // once the body's first blocks are in flight
    auto load_q = [&](h8 (&dst)[NCT][4]) {
#pragma unroll
      for (int t = 0; t < NCT; ++t) {
        const int lc = t * S + lcol;
        const _Float16* qn = static_cast<const _Float16*>(a.q) + om.row(b, hv, min(lc, ncol - 1)) * kD + 8 * g;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          dst[t][kk] = lc < ncol ? *reinterpret_cast<const h8*>(qn + 32 * kk) : h8{};
      }
    };
    h8 qraw[NCT][4];
    load_q(qraw);
#pragma unroll
    for (int t = 0; t < NCT; ++t) lim[t] = L - nq + om.gcol(hv, min(t * S + lcol, ncol - 1)) / G;
    auto prep_q = [&]() {
#pragma unroll
      for (int t = 0; t < NCT; ++t) {
#pragma unroll
        for (int k = 0; k < NG; ++k) qs[t][k] = 0.f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const h8 q = qraw[t][kk];
#pragma unroll
          for (int e = 0; e < 8; ++e) qs[t][kk * NG / 4] += float(q[e]);
          // INT4: the order of sub4's halves, the scale-16 codes' dims / 16
          // (exact down to |q| = 2^-10; below, one rounding of a subnormal)
          const _Float16 r = _Float16(0.0625f);
          if constexpr (KIND == kInt4)
            qp[t][kk] = h8{q[0], q[4], q[1] * r, q[5] * r, q[2], q[6], q[3] * r, q[7] * r};
          else
            qp[t][kk] = q;
        }
#pragma unroll
        for (int k = 0; k < NG; ++k) qs[t][k] = rows_sum(qs[t][k]) * (KIND == kInt4 ? 1.f / kSub : 1.f);
      }
    };
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
#pragma unroll
      for (int T_ = 0; T_ < kNT; ++T_) o[t][T_] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_ref[t] = -__builtin_inff();
      l_run[t] = 0.f;
      corr[t] = 0.f;
    }

    // body blocks, software-pipelined NB-1 blocks ahead with NB register
    // buffers; loads are unconditional so no branch separates them from
    // their waits (past the end the last block is re-read: an L2 hit)
    const int jw = lo + w;
    const int n = jw < jend ? (jend - jw + kWaves - 1) / kWaves : 0;
    // the first position of this wave at which the body loop met an FP16 id
    // (given no weight there; see the FP16 blocks below)
    int first16 = jend;
    if (n > 0) {
      auto id_of = [&](int k) { return table_entry(trow + jw + kWaves * min(k, n - 1)); };
      auto valid_of = [&](int k, int id) { return ok(id) ? L - 16 * (jw + kWaves * k) : 0; };
      Buf buf[NB];
      int ids[NB];
#pragma unroll
      for (int s = 0; s < NB - 1; ++s) {
        ids[s] = id_of(s);
        fetch(ids[s], buf[s]);
      }
      // table entries are read one block ahead of the fetch that needs them
      int nid = id_of(NB - 1);
      __builtin_amdgcn_sched_barrier(0);
      prep_q();
      int k = 0;
      // Whole blocks -- every token written and seen by every column -- take
      // the instance without per-token selects; an FP16 or out-of-range entry
      // among them is skipped with a scalar branch (it gets no weight).  In
      // a decode step every block but a sequence's partial last one is whole;
      // in a verify step of at most 16 queries every block but the one or two
      // its queries' positions reach into.  Either way a wave holds at most
      // one other block, its last, which is left to the blocks after the
      // loops.  A longer prefill chunk takes the general instance throughout.
      auto step = [&](auto full, int s) {
        const int nxt = (s + NB - 1) % NB;
        ids[nxt] = nid;
        nid = id_of(k + s + NB);
        fetch(ids[nxt], buf[nxt]);
        // no instruction of the block's product may move above the next
        // block's loads (it would wait for data still in flight)
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(full)::value) {
          if (ok(ids[s])) consume(full, 16, jw + kWaves * (k + s), buf[s]);
        } else {
          consume(full, valid_of(k + s, ids[s]), jw + kWaves * (k + s), buf[s]);
        }
        if (ok16(ids[s])) first16 = min(first16, jw + kWaves * (k + s));
      };
      const int seen = CAUSAL ? L - nq + 1 : L;  // positions every column sees
      const int nl = (!CAUSAL || nq <= 16) ? (16 * (jw + kWaves * (n - 1) + 1) <= seen ? n : n - 1) : 0;
      for (; k + NB <= nl; k += NB) {
        prio_from_progress(a, pos - pos0 + kWaves * k, prio_span);
#pragma unroll
        for (int s = 0; s < NB; ++s) step(std::true_type{}, s);
      }
      if constexpr (CAUSAL) {
        for (; k + NB <= n; k += NB) {
          prio_from_progress(a, pos - pos0 + kWaves * k, prio_span);
#pragma unroll
          for (int s = 0; s < NB; ++s) step(std::false_type{}, s);
        }
      }
      // the rest: at most NB blocks, the first NB - 1 of them fetched (the
      // last one, block k + NB - 1 = nid, only after a block kept out of the
      // whole-block loop)
#pragma unroll
      for (int s = 0; s < NB; ++s)
        if (k + s < n) {
          if (s == NB - 1) {
            ids[s] = nid;
            fetch(nid, buf[s]);
          }
          consume(std::false_type{}, valid_of(k + s, ids[s]), jw + kWaves * (k + s), buf[s]);
          if (ok16(ids[s])) first16 = min(first16, jw + kWaves * (k + s));
        }
    } else {
      prep_q();
    }
    // INT4: the body read the codes at 2^-24 (even output tiles) and 16 *
    // 2^-24 (odd ones): the sums back to scale, less the zero-point term
    // (the FP16 blocks below add to the scaled sums)
    if constexpr (KIND == kInt4) {
#pragma unroll
      for (int t = 0; t < NCT; ++t) {
        const float cz = rows_sum(corr[t]);
        corr[t] = 0.f;
#pragma unroll
        for (int T_ = 0; T_ < kNT; ++T_) o[t][T_] = o[t][T_] * ((T_ & 1) ? kSub / 16.f : kSub) - cz;
      }
    }

    // the window's FP16 run [jt, jend): count FP16 ids backward from jend - 1
    int jt = jend;
    if (p.window_tokens > 0 && lo < jend) {
      for (int top = jend;;) {
        const int j = top - 1 - lane;
        const uint64_t fp = __ballot(j >= lo && ok16(tid));
        const int run = fp == ~uint64_t(0) ? 64 : __builtin_ctzll(~fp);
        jt = top - run;
        if (run < 64 || jt <= lo) break;
        top = jt;
        tid = trow[max(top - 1 - lane, 0)];
      }
    }

    // FP16 blocks: the piece's sink blocks [jbeg, min(jend, SP)) and the
    // window run [jt, jend), pipelined one block ahead
    const int ns = max(0, min(jend, SP) - jbeg);
    const int nf = ns + (jend - jt);
    const int n16 = w < nf ? (nf - w + kWaves - 1) / kWaves : 0;
    // the query fragments in natural element order, for the FP16 blocks (the
    // INT4 body permuted and scaled its copy: loaded again)
    h8 qf[NCT][4];
    if constexpr (KIND == kInt4) {
      if (n16 > 0 || first16 < jt) load_q(qf);
    } else {
#pragma unroll
      for (int t = 0; t < NCT; ++t)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qf[t][kk] = qp[t][kk];
    }
    if (n16 > 0) {
      auto j16 = [&](int k) {
        const int i = w + kWaves * min(k, n16 - 1);
        return i < ns ? jbeg + i : jt + (i - ns);
      };
      auto valid16 = [&](int k, int id) { return ok16(id) ? L - 16 * j16(k) : 0; };
      Buf16 bb[2];
      int ids[2];
      ids[0] = table_entry(trow + j16(0));
      fetch16(ids[0], bb[0]);
      int k = 0;
      for (; k + 2 <= n16; k += 2) {
        ids[1] = table_entry(trow + j16(k + 1));
        fetch16(ids[1], bb[1]);
        consume16(valid16(k, ids[0]), j16(k), bb[0], qf);
        ids[0] = table_entry(trow + j16(k + 2));
        fetch16(ids[0], bb[0]);
        consume16(valid16(k + 1, ids[1]), j16(k + 1), bb[1], qf);
      }
      if (k < n16) consume16(valid16(k, ids[0]), j16(k), bb[0], qf);
    }
    // FP16 blocks before the window's run: a table read between a reserve of
    // several blocks and its settle holds the old window's FP16 blocks
    // between body runs (and a failed settle leaves them there).  The body
    // loop gave them no weight; this wave streams the ones at its own
    // positions in [first16, jt) here, one at a time (a settled table never
    // takes this path).
    for (int j = first16; j < jt; j += kWaves) {
      const int id = table_entry(trow + j);
      if (ok16(id)) {
        Buf16 one;
        fetch16(id, one);
        consume16(L - 16 * j, j, one, qf);
      }
    }

    // ---- finish the piece: merge -------------------------------------------------------
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
      l_run[t] = rows_sum(l_run[t]);
      if (keep) stash_piece(sh, w, g, t * S + lcol, o[t], m_ref[t], l_run[t]);
    }
    if (a.defer_merge && jbeg == 0 && threadIdx.x == 0) write_job(a, um, b, hv, hv * um.TB + fb, nb);
    finish_piece<_Float16>(a, sh, om, jbeg == 0 && jend == nb, first ? 0 : 1, unit, b, hv,
                           hv * um.TB + fb, nb, um);
    pos += jend - jbeg;
    first = false;
  }
  }
}

}  // namespace

// Prefetch depth: PA_QUANT_NB = 2 (3 waves per SIMD), 3, 4 or 6 (2 waves per
// SIMD).  Default 3: two blocks in flight per wave at two waves per SIMD
// measured faster than one at three for INT4 (both group sizes) and FP8.
// (Read at every launch, as the other tuning variables are.)
template <int NG>
int quant_nb() {
  const char* e = std::getenv("PA_QUANT_NB");
  const int v = e ? std::atoi(e) : 0;
  return (v == 2 || v == 3 || v == 4 || v == 6) ? v : 3;
}

// Verify steps and prefill chunks: prefetch depth 3 with one column tile,
// 2 with two (their accumulators take the registers of a buffer).
template <int NCT>
constexpr int kVerifyNB = NCT == 1 ? 3 : 2;

template <int KIND, int NB, int NG, int NCT, bool CAUSAL>
int occ_of() {
  int n = 0;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &n, decode_split_quant<KIND, NB, NG, NCT, CAUSAL>, kWaves * 64, 0);
  return (e == hipSuccess && n > 0) ? n : 2;
}

// nct: 0 = decode, else the verify kernel with that many column tiles
template <int KIND, int NG>
int occ_kind(int nct) {
  if (nct == 1) return occ_of<KIND, kVerifyNB<1>, NG, 1, true>();
  if (nct == 2) return occ_of<KIND, kVerifyNB<2>, NG, 2, true>();
  switch (quant_nb<NG>()) {
    case 3: return occ_of<KIND, 3, NG, 1, false>();
    case 4: return occ_of<KIND, 4, NG, 1, false>();
    case 6: return occ_of<KIND, 6, NG, 1, false>();
    default: return occ_of<KIND, 2, NG, 1, false>();
  }
}

// The register-lengths form (RL) for batches of at most 64 sequences with no
// queue, at the default prefetch depths; the general form otherwise.
inline bool reg_lens_ok(const DecodeArgs& a) {
  return a.batch <= kRegLens && !(a.unit_blocks > 0 && a.static_permille < 1000);
}

template <int KIND, int NG>
void launch_kind(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(unsigned(a.max_splits)), block(kWaves * 64);
  const bool rl = reg_lens_ok(a);
  if (a.n_query > 1) {  // verify step / prefill chunk: logical columns of a segment
    const int cols = a.col_slices > 1 ? a.slice_cols : a.n_query * (a.n_q_heads / a.pool.n_kv_heads);
    if (cols * NG <= 16) {
      if (rl)
        hipLaunchKernelGGL((decode_split_quant<KIND, kVerifyNB<1>, NG, 1, true, true>), grid, block, 0, s, a);
      else
        hipLaunchKernelGGL((decode_split_quant<KIND, kVerifyNB<1>, NG, 1, true>), grid, block, 0, s, a);
    } else {
      if (rl)
        hipLaunchKernelGGL((decode_split_quant<KIND, kVerifyNB<2>, NG, 2, true, true>), grid, block, 0, s, a);
      else
        hipLaunchKernelGGL((decode_split_quant<KIND, kVerifyNB<2>, NG, 2, true>), grid, block, 0, s, a);
    }
    return;
  }
  if (a.app_k != nullptr) {  // a decode step: the default depth writes the new tokens itself
    if (quant_nb<NG>() == 3) {
      if (rl)
        hipLaunchKernelGGL((decode_split_quant<KIND, 3, NG, 1, false, true, true>), grid, block, 0, s, a);
      else
        hipLaunchKernelGGL((decode_split_quant<KIND, 3, NG, 1, false, false, true>), grid, block, 0, s, a);
      return;
    }
    if (launch_append_last(a.pool, a.app_k, a.app_v, a.app_dt, a.tables, a.lens, a.batch,
                           a.max_blocks_per_seq, a.max_seq_len, s) != hipSuccess)
      return;  // the caller's hipGetLastError reports it
  }
  switch (quant_nb<NG>()) {
    case 3:
      if (rl)
        hipLaunchKernelGGL((decode_split_quant<KIND, 3, NG, 1, false, true>), grid, block, 0, s, a);
      else
        hipLaunchKernelGGL((decode_split_quant<KIND, 3, NG, 1, false>), grid, block, 0, s, a);
      break;
    case 4: hipLaunchKernelGGL((decode_split_quant<KIND, 4, NG, 1, false>), grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((decode_split_quant<KIND, 6, NG, 1, false>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((decode_split_quant<KIND, 2, NG, 1, false>), grid, block, 0, s, a); break;
  }
}

// INT4 scale groups per token and head (1 or 2 here); FP8 has one scale per token
int groups_of(int32_t kv_dtype, int32_t group_size) {
  return kv_dtype == kInt4 && group_size > 0 ? kD / group_size : 1;
}

// nct: 0 for decode, else the verify kernel's column tiles (1 or 2).
int occupancy_quant(int32_t kv_dtype, int32_t group_size, int nct) {
  static int cache[3][3][7] = {};  // [INT4 NG = 1, INT4 NG = 2, FP8][nct][prefetch depth]
  const int ng = groups_of(kv_dtype, group_size);
  const int i = kv_dtype == kInt4 ? (ng == 1 ? 0 : 1) : 2;
  const int nb = nct == 1 ? kVerifyNB<1> : nct == 2 ? kVerifyNB<2> : i == 1 ? quant_nb<2>() : quant_nb<1>();
  int& c = cache[i][nct][nb];
  if (c == 0) {
    switch (i) {
      case 0: c = occ_kind<kInt4, 1>(nct); break;
      case 1: c = occ_kind<kInt4, 2>(nct); break;
      default: c = occ_kind<kFp8, 1>(nct); break;
    }
  }
  return c;
}

hipError_t launch_decode_split_quant(const DecodeArgs& a, hipStream_t s) {
  if (a.pool.kv_dtype == kInt4) {
    switch (groups_of(kInt4, a.pool.group_size)) {
      case 1: launch_kind<kInt4, 1>(a, s); break;
      case 2: launch_kind<kInt4, 2>(a, s); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    launch_kind<kFp8, 1>(a, s);
  }
  return hipGetLastError();
}

}  // namespace pa
