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
// The codes enter the fp16 matrix cores exactly: an INT4 nibble n becomes the
// fp16 value n (0x6400|n is 1024+n, then an exact packed-fp16 subtract); an
// E4M3 code goes through the hardware FP8->fp16 conversion with scale 1
// (every E4M3 value is an fp16 value).  The weights
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

#include "decode_common.hpp"

namespace pa {

namespace {

using namespace dec;

typedef _Float16 h8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef _Float16 h4 __attribute__((__vector_size__(4 * sizeof(_Float16))));
typedef _Float16 h2 __attribute__((__vector_size__(2 * sizeof(_Float16))));

// INT4 codes to exact fp16 values.  A nibble n placed in the low mantissa
// bits under 0x6400 reads as 1024 + n; one bit-select and one packed
// subtract give n.  A nibble at mantissa bits 4..7 reads as 1024 + 16n, and
// one packed fma, x/16 - 64, gives n (both steps exact in fp16).
// nib4(x): the fp16 pairs of the nibbles at bits (s, s + 16), s = 0, 4, 8, 12.
__device__ inline uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
  return r;
}
__device__ inline uint32_t nib_lo(uint32_t x) {  // bits 0..3 and 16..19
  const h2 v = __builtin_bit_cast(h2, and_or(x, 0x000F000Fu, 0x64006400u));
  return __builtin_bit_cast(uint32_t, v - h2{_Float16(1024.f), _Float16(1024.f)});
}
__device__ inline uint32_t nib_hi(uint32_t x) {  // bits 4..7 and 20..23
  const h2 v = __builtin_bit_cast(h2, and_or(x, 0x00F000F0u, 0x64006400u));
  return __builtin_bit_cast(
      uint32_t, __builtin_elementwise_fma(v, h2{_Float16(0.0625f), _Float16(0.0625f)},
                                          h2{_Float16(-64.f), _Float16(-64.f)}));
}
__device__ inline u32x4 nib4(uint32_t x) {
  const uint32_t y = x >> 8;
  return u32x4{nib_lo(x), nib_hi(x), nib_lo(y), nib_hi(y)};
}

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

// NW consecutive dwords at p (NW = 2: 8-byte aligned; 4, 8: 16-byte aligned)
template <int NW>
__device__ inline void load_words(const uint8_t* p, uint32_t (&d)[NW]) {
  if constexpr (NW == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    d[0] = v[0];
    d[1] = v[1];
  } else {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(p + 16 * i);
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

// Scale/zero of token i in group `sel` (a per-lane group index < NG).
template <int NG>
__device__ inline float half_sel(const uint32_t (&m)[2 * NG], int i, int sel) {
  float v = half_at(m, i * NG);
#pragma unroll
  for (int k = 1; k < NG; ++k) v = sel == k ? half_at(m, i * NG + k) : v;
  return v;
}

// NB = register buffers per wave (NB-1 blocks prefetched ahead).
//
// Groups (NG > 1, INT4 only; the launch guarantees NG * G <= 16): the
// matrix-core B operand has 16 columns and a KV head serves G query heads, so
// column c computes head c % G with the V weights scaled by group c / G.
// Output tile row r holds dim 8r + T, which lies in group (8r) / group_size =
// g * NG / 4 for the rows 4g..4g+3 a lane holds: lane (g, c) keeps column
// c - (g * NG / 4) * G.  The scores of the copies are identical, so are their
// softmax statistics.  On the K side each group has its own accumulator
// (dims 32kk.. lie in group kk * NG / 4).
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
template <int KIND, int NB, int NG>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(NB == 2 ? 3 : 2))) void decode_split_quant(DecodeArgs a) {
  typedef typename Quant<KIND, NG>::Buf Buf;
  typedef Mfma<_Float16> MF;
  __shared__ Shared sh;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 4, c = lane & 15;
  const PoolDev& p = a.pool;
  const int H = p.n_kv_heads, Hq = a.n_q_heads, G = Hq / H, N = p.num_blocks;
  const int SP = p.sink_per_seq, NS = p.num_sink_blocks;
  const int qcol = c < NG * G ? (NG == 1 ? c : c % G) : -1;  // query head (within the group) of column c
  const int gsel = NG == 1 ? 0 : min(c / G, NG - 1);  // scale group of column c
  const int keep = c - (NG == 1 ? 0 : (g * NG / 4) * G);  // column this lane writes
  const Units um = setup_units(a, sh, w, lane);
  zero_empty_rows<_Float16>(a, sh);
  int b = 0, fb = 0;

  const float sl2 = a.scale_log2;
  const uint8_t* base = p.base;
  const int32_t* trow = a.tables;
  int h = 0, L = 0;
  h8 qp[4];         // Q^T fragments in the code's element order
  float qs[NG];     // per-group sums of the head's query (INT4 zero-point terms)
  f32x4 o[kNT];
  float m_ref = -__builtin_inff(), l_run = 0.f, corr = 0.f;

  auto ok = [&](int id) { return id >= 0 && id < N; };
  auto ok16 = [&](int id) { return id >= N && id < N + NS; };

  // softmax update for one block's 4 scores per lane; returns the weights
  auto softmax = [&](const float (&x)[4], int valid, float (&pw)[4]) {
    float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    bm = rows_max(bm);
    const bool move = bm > m_ref + 2.f;
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
    const uint8_t* ks = base + p.off[kArrKS] + sid * p.slab[kArrKS] + 8 * NG * g;
    const uint8_t* vs = base + p.off[kArrVS] + sid * p.slab[kArrVS] + 8 * NG * g;
    if constexpr (KIND == kInt4) {
      bf.kc = *reinterpret_cast<const u32x4*>(kc + lane * 16);
      bf.vc = *reinterpret_cast<const u32x4*>(vc + lane * 16);
      load_words(ks, bf.ks);
      load_words(base + p.off[kArrKZ] + sid * p.slab[kArrKZ] + 8 * NG * g, bf.kz);
      load_words(vs, bf.vs);
      load_words(base + p.off[kArrVZ] + sid * p.slab[kArrVZ] + 8 * NG * g, bf.vz);
    } else {
      bf.kc0 = *reinterpret_cast<const u32x4*>(kc + lane * 16);
      bf.kc1 = *reinterpret_cast<const u32x4*>(kc + 1024 + lane * 16);
      bf.vc0 = *reinterpret_cast<const u32x4*>(vc + lane * 16);
      bf.vc1 = *reinterpret_cast<const u32x4*>(vc + 1024 + lane * 16);
      load_words(ks, bf.ks);
      load_words(vs, bf.vs);
    }
  };

  auto consume = [&](int valid, const Buf& bf) {
    float x[4];
    if constexpr (KIND == kInt4) {
      f32x4 acc[NG];
#pragma unroll
      for (int k = 0; k < NG; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint32_t cw = bf.kc[kk];
        const u32x4 av = nib4(cw);
        acc[kk * NG / 4] = MF::qk(__builtin_bit_cast(h8, av), qp[kk], acc[kk * NG / 4]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sc = 0.f;
#pragma unroll
        for (int k = 0; k < NG; ++k)
          sc += half_at(bf.ks, i * NG + k) * (acc[k][i] - half_at(bf.kz, i * NG + k) * qs[k]);
        const float xs = pin(sc * sl2);
        x[i] = (4 * g + i < valid) ? xs : -__builtin_inff();
      }
    } else {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x4 u = kk < 2 ? bf.kc0 : bf.kc1;
        const uint32_t x0 = u[(kk & 1) * 2], x1 = u[(kk & 1) * 2 + 1];
        const u32x4 av = {fp8pair<false>(x0), fp8pair<true>(x0), fp8pair<false>(x1), fp8pair<true>(x1)};
        acc = MF::qk(__builtin_bit_cast(h8, av), qp[kk], acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float xs = pin(half_at(bf.ks, i) * acc[i] * sl2);
        x[i] = (4 * g + i < valid) ? xs : -__builtin_inff();
      }
    }
    float pw[4];
    softmax(x, valid, pw);
    // weights times the V scale of this column's group; tail tokens' metadata
    // may be garbage: select
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float w_ = pin(half_sel<NG>(bf.vs, i, gsel) * pw[i]);
      pv[i] = (4 * g + i < valid) ? w_ : 0.f;
    }
    // FP8: zero the bytes of tail tokens (unwritten slots may hold NaN codes)
    const int t0 = 4 * g;
    const uint32_t vmask = (t0 + 0 < valid ? 0x000000FFu : 0u) | (t0 + 1 < valid ? 0x0000FF00u : 0u) |
                           (t0 + 2 < valid ? 0x00FF0000u : 0u) | (t0 + 3 < valid ? 0xFF000000u : 0u);
    if constexpr (KIND == kInt4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float z_ = pin(half_sel<NG>(bf.vz, i, gsel) * pv[i]);
        corr += (4 * g + i < valid) ? z_ : 0.f;
      }
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
        const u32x4 nv = nib4(bf.vc[T_ >> 1]);
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
      o[T_] = MF::pv2(at, bhi, blo, o[T_]);
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

  // qf: the query fragments in natural element order
  auto consume16 = [&](int valid, const Buf16& bf, const h8 (&qf)[4]) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = MF::qk(bf.k[kk], qf[kk], acc);
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
      u32x4 dw = bf.v[u];
      dw[0] &= m01;  // unwritten tail slots may hold any bits
      dw[1] &= m23;
      dw[2] &= m01;
      dw[3] &= m23;
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const u32x2 av = {dw[2 * par], dw[2 * par + 1]};
        const h4 at = __builtin_bit_cast(h4, av);
        o[2 * u + par] = MF::pv2(at, bhi, blo, o[2 * u + par]);
      }
    }
  };

  const int own_unit = um.owned(int(blockIdx.x));
  for (int unit = own_unit; unit >= 0; unit = next_unit(a, sh, um)) {
  const int pos0 = um.start(unit), pos1 = um.end(unit);
  if (pos0 >= pos1) continue;  // a region past the end of the work
  locate(a, sh, um, w, lane, pos0, b, fb);
  // progress-based priority in the owner's prefix; queued units run at the
  // base priority, behind the workgroups still streaming their own prefix
  const int prio_span = unit == own_unit ? pos1 - pos0 : 0;
  int pos = pos0;
  bool first = true;
  int jbeg = 0, jend = 0, nb = 0;
  while (next_piece(a, sh, um, pos, pos1, b, fb, h, jbeg, jend, nb)) {
    L = len_of(a, sh, b);
    trow = a.tables + size_t(b) * a.max_blocks_per_seq;
    const int lo = max(jbeg, SP);  // first non-sink block of the piece
    // the table's last 64 entries of the piece, for the window scan below
    int tid = p.window_tokens > 0 ? trow[max(jend - 1 - lane, 0)] : 0;
    // Q^T fragment of head qcol (dims 32kk + 8g + 0..7): loaded here, and
    // permuted into the order in which the code conversion delivers the K
    // elements (and summed per group) once the body's first blocks are in
    // flight
    h8 qraw[4];
    {
      const _Float16* qn =
          static_cast<const _Float16*>(a.q) + (size_t(b) * Hq + h * G + max(qcol, 0)) * kD + 8 * g;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        qraw[kk] = qcol >= 0 ? *reinterpret_cast<const h8*>(qn + 32 * kk) : h8{};
    }
    auto prep_q = [&]() {
#pragma unroll
      for (int k = 0; k < NG; ++k) qs[k] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const h8 q = qraw[kk];
#pragma unroll
        for (int e = 0; e < 8; ++e) qs[kk * NG / 4] += float(q[e]);
        if constexpr (KIND == kInt4)
          qp[kk] = h8{q[0], q[4], q[1], q[5], q[2], q[6], q[3], q[7]};
        else
          qp[kk] = q;
      }
#pragma unroll
      for (int k = 0; k < NG; ++k) qs[k] = rows_sum(qs[k]);
    };
#pragma unroll
    for (int T_ = 0; T_ < kNT; ++T_) o[T_] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_ref = -__builtin_inff();
    l_run = 0.f;
    corr = 0.f;

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
      for (; k + NB <= n; k += NB) {
        prio_from_progress(a, pos - pos0 + kWaves * k, prio_span);
#pragma unroll
        for (int s = 0; s < NB; ++s) {
          const int nxt = (s + NB - 1) % NB;
          ids[nxt] = nid;
          nid = id_of(k + s + NB);
          fetch(ids[nxt], buf[nxt]);
          // no instruction of the block's product may move above the next
          // block's loads (it would wait for data still in flight)
          __builtin_amdgcn_sched_barrier(0);
          consume(valid_of(k + s, ids[s]), buf[s]);
          if (ok16(ids[s])) first16 = min(first16, jw + kWaves * (k + s));
        }
      }
#pragma unroll
      for (int s = 0; s < NB - 1; ++s)
        if (k + s < n) {
          consume(valid_of(k + s, ids[s]), buf[s]);
          if (ok16(ids[s])) first16 = min(first16, jw + kWaves * (k + s));
        }
    } else {
      prep_q();
    }
    // the query fragments in natural element order, for the FP16 blocks
    h8 qf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const h8 q = qp[kk];
      if constexpr (KIND == kInt4)
        qf[kk] = h8{q[0], q[2], q[4], q[6], q[1], q[3], q[5], q[7]};
      else
        qf[kk] = q;
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
        consume16(valid16(k, ids[0]), bb[0], qf);
        ids[0] = table_entry(trow + j16(k + 2));
        fetch16(ids[0], bb[0]);
        consume16(valid16(k + 1, ids[1]), bb[1], qf);
      }
      if (k < n16) consume16(valid16(k, ids[0]), bb[0], qf);
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
        consume16(L - 16 * j, one, qf);
      }
    }

    // ---- finish the piece: zero-point correction, merge ------------------------------
    l_run = rows_sum(l_run);
    if constexpr (KIND == kInt4) {
      corr = rows_sum(corr);
#pragma unroll
      for (int T_ = 0; T_ < kNT; ++T_) o[T_] -= corr;
    }
    if (keep >= 0) stash_piece(sh, w, g, keep, o, m_ref, l_run);
    if (a.defer_merge && jbeg == 0 && threadIdx.x == 0) write_job(a, um, b, h, h * um.TB + fb, nb);
    finish_piece<_Float16>(a, sh, out_map(a), jbeg == 0 && jend == nb, first ? 0 : 1, unit, b, h,
                      h * um.TB + fb, nb, um);
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

template <int KIND, int NB, int NG>
int occ_of() {
  int n = 0;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_split_quant<KIND, NB, NG>,
                                                                     kWaves * 64, 0);
  return (e == hipSuccess && n > 0) ? n : 2;
}

template <int KIND, int NG>
int occ_kind() {
  switch (quant_nb<NG>()) {
    case 3: return occ_of<KIND, 3, NG>();
    case 4: return occ_of<KIND, 4, NG>();
    case 6: return occ_of<KIND, 6, NG>();
    default: return occ_of<KIND, 2, NG>();
  }
}

template <int KIND, int NG>
void launch_kind(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(unsigned(a.max_splits)), block(kWaves * 64);
  switch (quant_nb<NG>()) {
    case 3: hipLaunchKernelGGL((decode_split_quant<KIND, 3, NG>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_split_quant<KIND, 4, NG>), grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((decode_split_quant<KIND, 6, NG>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((decode_split_quant<KIND, 2, NG>), grid, block, 0, s, a); break;
  }
}

// INT4 scale groups per token and head (1 or 2 here); FP8 has one scale per token
int groups_of(int32_t kv_dtype, int32_t group_size) {
  return kv_dtype == kInt4 && group_size > 0 ? kD / group_size : 1;
}

int occupancy_quant(int32_t kv_dtype, int32_t group_size) {
  static int cache[3][7] = {};  // [INT4 NG = 1, INT4 NG = 2, FP8][prefetch depth]
  const int ng = groups_of(kv_dtype, group_size);
  const int i = kv_dtype == kInt4 ? (ng == 1 ? 0 : 1) : 2;
  const int nb = i == 1 ? quant_nb<2>() : quant_nb<1>();
  int& c = cache[i][nb];
  if (c == 0) {
    switch (i) {
      case 0: c = occ_kind<kInt4, 1>(); break;
      case 1: c = occ_kind<kInt4, 2>(); break;
      default: c = occ_kind<kFp8, 1>(); break;
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
