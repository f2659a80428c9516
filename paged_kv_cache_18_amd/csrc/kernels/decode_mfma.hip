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
// Work decomposition (decode_common.hpp).  The blocks of every (sequence b,
// KV head h) segment are laid end to end in one list, KV head major (h, then
// b, then logical block j), so every head's list holds the same TB blocks.
// By default the grid is one workgroup per resident slot of the GPU (at most
// two per compute unit) and each head's list is cut into q = grid / heads
// regions of C = ceil(TB / q) blocks (sized on the device from the lengths),
// so every workgroup streams the same number of blocks; a fixed C can be
// requested instead.  Region k of head h goes to workgroup k*heads + h
// (Units::owned_by_head): workgroups are dealt to the 8 XCDs round robin, so
// with 8 KV heads each XCD streams one head's slabs of every block.  A
// segment that lies inside one region is finished there (normalized and
// written to out).  A segment crossing region boundaries leaves one partial
// (max, sum, weighted sum) per region it touches; a region holds at most two
// such pieces (its first and its last), so the workspace is two slots per
// workgroup; the workgroup that completes a segment merges its partials.
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
//    8c+2u+1]; O^T += V^T P^T per 16-dim tile T (rows = dims 8r+T), both
//    parts of P in one v_mfma_f32_16x16x32 (V^T twice along k; two
//    v_mfma_f32_16x16x16 per part with two column tiles), so lane (g, c) owns
//    output head c: the softmax rescale is a per-lane scalar.
// The loads of a wave's next block are issued before its current block is
// consumed (two register buffers).  After each piece the 4 waves merge
// (max, sum, acc) through LDS; segments split across chunks are merged by the
// workgroup that completes them (decode_common.hpp).
#include <cstdlib>
#include <type_traits>

#include "decode_common.hpp"

namespace pa {

namespace {

using namespace dec;

// NB register buffers per wave: NB - 1 blocks in flight while one is
// consumed.  The kernel runs at two workgroups (two waves per SIMD) per
// compute unit -- three measured slower -- so it may hold up to 256 registers
// (NB = 2 needs about 170); deeper pipelines spill.
//
// NCT column tiles of 16 and CAUSAL: decode packs the G query heads of a KV
// head into one tile; the verify step packs n_query x G (query, head) columns
// into one or two tiles and masks, per column, the tokens after its own
// query's position (causal among the step's new tokens).
// BS: tokens per pool block (16; 8 or 32).  The kernel always works on
// 16-token tiles: tile jt is block jt (16), 16-token slab jt % 2 of block
// jt / 2 (32: tile id 2 * block + slab), or blocks 2jt and 2jt + 1 (8: lanes
// of tokens 8..15 read the second).
struct TileId {
  int a, b;  // 8-token blocks: the two block ids
};

//
// SPLIT (two column tiles only): waves 0, 1 compute tile 0 and waves 2, 3
// tile 1, each pair taking the piece's blocks alternately, so a wave carries
// one tile's registers and every block is read by two waves of the workgroup
// (the second from L2).  A pair stashes into two slots (wave w into slot
// w & 1, its tile's columns), which halves the LDS of the merge.
//
// RL: a batch of at most 64 sequences with no queue, whose lengths every wave
// keeps in registers (see RegLens).
template <typename T, int NB, int NCT, bool CAUSAL, int BS, bool SPLIT = false, bool RL = false>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void decode_split_mfma16(
    DecodeArgs a) {
  typedef typename Mfma<T>::v8 v8;
  typedef typename Mfma<T>::v4 v4;
  static_assert(!SPLIT || NCT == 2, "tile split needs two tiles");
  constexpr int NT = SPLIT ? 1 : NCT;  // tiles a wave computes
  __shared__ SharedT<16 * NCT, SPLIT ? 2 : kWaves> sh;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int t0 = SPLIT ? w >> 1 : 0;       // this wave's first tile
  const int nst = SPLIT ? 2 : kWaves;      // waves sharing a tile's blocks
  const int ws = SPLIT ? w & 1 : w;        // this wave's place among them
  const int g = lane >> 4, c = lane & 15;
  const PoolDev& p = a.pool;
  const int H = p.n_kv_heads, Hq = a.n_q_heads, G = Hq / H;
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
  zero_empty_rows<T>(a, blocks_at);
  int b = 0, fb = 0;

  const T* kbase = reinterpret_cast<const T*>(p.base + p.off[kArrK]);
  const T* vbase = reinterpret_cast<const T*>(p.base + p.off[kArrV]);
  const float sl2 = a.scale_log2;
  const int nbk = p.num_blocks;

  // per-piece state, captured by the lambdas below: segment hv = h*nsl + s
  // (KV head h, column slice s)
  int hv = 0, h = 0, L = 0;
  const int32_t* trow = a.tables;
  v8 qf[NT][4];
  f32x4 o[NT][kNT];
  // Running statistics per lane and tile (= per packed column): m_ref is the
  // reference the weights are taken against, l_run the running sum of weights.
  float m_ref[NT], l_run[NT];
  int lim[NT];  // CAUSAL: last position column 16(t0 + t) + c may see

  // K/V of one block into registers (8 x 16-byte loads, 1 KiB contiguous per
  // load across the wave).  The loads are issued unconditionally -- an
  // out-of-range table entry reads block 0 and is never consumed -- so no
  // branch separates a load from its use and the wait counters stay exact.
  // a tile's table entries: the block id (16), 2 * block id + slab (32), or
  // the two block ids (8)
  typedef typename std::conditional<BS == 8, TileId, int>::type Tid;
  auto fetch = [&](Tid tid, v8(&kf)[4], v8(&vf)[4]) {
    TileId ti;
    if constexpr (BS == 16) ti = TileId{tid, 0};
    else if constexpr (BS == 32) ti = TileId{tid >> 1, tid & 1};
    else ti = tid;
    const int safe = (ti.a < 0 || ti.a >= nbk) ? 0 : ti.a;
    const size_t slab = (size_t(safe) * H + h) * (BS * kD);
    if constexpr (BS == 16) {
      const T* ks = kbase + slab;
      const T* vs = vbase + slab;
#pragma unroll
      for (int u = 0; u < 4; ++u) kf[u] = *reinterpret_cast<const v8*>(ks + (u * 64 + lane) * 8);
#pragma unroll
      for (int u = 0; u < 4; ++u) vf[u] = *reinterpret_cast<const v8*>(vs + (u * 64 + lane) * 8);
    } else if constexpr (BS == 32) {  // half ti.b: a 16-token slab at 16*b tokens into the block
      const T* ks = kbase + slab + ti.b * (16 * kD);
      const T* vs = vbase + slab + ti.b * (16 * kD);
#pragma unroll
      for (int u = 0; u < 4; ++u) kf[u] = *reinterpret_cast<const v8*>(ks + (u * 64 + lane) * 8);
#pragma unroll
      for (int u = 0; u < 4; ++u) vf[u] = *reinterpret_cast<const v8*>(vs + (u * 64 + lane) * 8);
    } else {  // BS 8: tokens 0..7 from block a, 8..15 from block b
      const int sb = (ti.b < 0 || ti.b >= nbk) ? safe : ti.b;
      const size_t slab_b = (size_t(sb) * H + h) * (BS * kD);
      const T* ks = kbase + (c < 8 ? slab : slab_b) + ((g * BS + (c & 7)) * 8);
      const T* vs = vbase + (g < 2 ? slab : slab_b) + (((g & 1) * 16 + c) * 8);
#pragma unroll
      for (int u = 0; u < 4; ++u) kf[u] = *reinterpret_cast<const v8*>(ks + u * 4 * BS * 8);
#pragma unroll
      for (int u = 0; u < 4; ++u) vf[u] = *reinterpret_cast<const v8*>(vs + u * 2 * 16 * 8);
    }
  };
  auto ok = [&](int id) { return id >= 0 && id < nbk; };

  // One block (logical index jl): S^T = K Q^T, online softmax, O^T += V^T
  // P^T.  `valid` tokens of the block count (0 for a skipped table entry:
  // every weight is zero).  It always runs, so every load is waited on along
  // every path.
  auto consume = [&](int valid, int jl, const v8(&kf)[4], v8(&vf)[4]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) sc = Mfma<T>::qk(kf[kk], qf[t][kk], sc);
      float x[4];
      bool vis[4];
      float bm = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vis[i] = 4 * g + i < valid;
        if constexpr (CAUSAL) vis[i] = vis[i] && 16 * jl + 4 * g + i <= lim[t];
        x[i] = vis[i] ? sc[i] * sl2 : -__builtin_inff();
        bm = fmaxf(bm, x[i]);
      }
      bm = rows_max(bm);
      // The reference only moves when a block's max exceeds it by more than 8
      // (weights stay <= 2^8, far inside fp32 and the two-part 16-bit split),
      // so the accumulators are rarely rescaled.  The result is unchanged:
      // numerator and denominator share the reference.
      const bool move = bm > m_ref[t] + 8.f;
      if (__any(move)) {
        // factor 1 where the reference stays (no NaN from -inf - -inf for
        // a column that has seen no token yet)
        const float alpha = move ? __builtin_amdgcn_exp2f(m_ref[t] - bm) : 1.f;
        l_run[t] *= alpha;
#pragma unroll
        for (int T_ = 0; T_ < kNT; ++T_) o[t][T_] *= alpha;
        m_ref[t] = move ? bm : m_ref[t];
      }
      if (t == 0 && valid < 16) {
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
        const float pw = vis[i] ? __builtin_amdgcn_exp2f(x[i] - m_ref[t]) : 0.f;
        l_run[t] += pw;
        phi[i] = T(pw);
        plo[i] = T(pw - float(phi[i]));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int par = 0; par < 2; ++par) {
          v4 vt = {vf[u][4 * par + 0], vf[u][4 * par + 1], vf[u][4 * par + 2], vf[u][4 * par + 3]};
          if constexpr (NT == 1) {
            o[t][2 * u + par] = Mfma<T>::pv2(vt, phi, plo, o[t][2 * u + par]);
          } else {  // two tiles: the doubled operands would spill (measured 8 % slower)
            o[t][2 * u + par] = Mfma<T>::pv(vt, phi, o[t][2 * u + par]);
            o[t][2 * u + par] = Mfma<T>::pv(vt, plo, o[t][2 * u + par]);
          }
        }
      }
    }
  };

  const int own_unit = um.owned_by_head(int(blockIdx.x));
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
    const int ncol = om.cols(hv);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // Q^T fragment: lane (g, c) of tile t0 + t holds the segment's column
      // col = 16(t0 + t) + c, i.e. Q[query gc / G][head h*G + gc % G][32kk + 8g .. +7]
      // for gc = s*32 + col in column slice s; zero past the last column
      const int col = 16 * (t0 + t) + c, qi = om.gcol(hv, col) / G;
      const T* qp = static_cast<const T*>(a.q) + om.row(b, hv, min(col, ncol - 1)) * kD + 8 * g;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        qf[t][kk] = col < ncol ? *reinterpret_cast<const v8*>(qp + 32 * kk) : v8{};
      lim[t] = L - nq + qi;
#pragma unroll
      for (int T_ = 0; T_ < kNT; ++T_) o[t][T_] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_ref[t] = -__builtin_inff();
      l_run[t] = 0.f;
    }

    // Software pipeline over this wave's blocks jw + nst*k, k = 0..n-1: the loads
    // of blocks k+1 .. k+NB-1 are in flight while block k is consumed.  The
    // buffers rotate inside a fully unrolled trip of NB blocks (no copies, no
    // full waits); loads are unconditional, and past the last block they
    // re-read it (an L2 hit, never consumed).
    const int jw = jbeg + ws;
    const int n = jw < jend ? (jend - jw + nst - 1) / nst : 0;
    // a decode step's new token: its words are loaded ahead of the blocks
    const NewToken ntok = CAUSAL ? NewToken{} : new_token_load(a, lane, b, hv, nsl, jw, nst, jend, nb, L);
    auto id_of = [&](int k) -> Tid {
      const int jt = jw + nst * min(k, n - 1);
      if constexpr (BS == 16) {
        return table_entry(trow + jt);
      } else if constexpr (BS == 32) {
        return 2 * table_entry(trow + (jt >> 1)) + (jt & 1);
      } else {  // BS 8: the second block exists only if the sequence reaches it
        const int last = (L + BS - 1) / BS - 1;
        return TileId{table_entry(trow + 2 * jt), table_entry(trow + min(2 * jt + 1, last))};
      }
    };
    auto valid_of = [&](int k, Tid tid) {
      if constexpr (BS == 16) {
        return ok(tid) ? L - 16 * (jw + nst * k) : 0;
      } else if constexpr (BS == 32) {
        return ok(tid >> 1) ? L - 16 * (jw + nst * k) : 0;
      } else {
        const int v = L - 16 * (jw + nst * k);
        if (!ok(tid.a)) return 0;
        if constexpr (BS == 8) return ok(tid.b) ? v : min(v, 8);
        return v;
      }
    };
    if (n > 0) {
      v8 kb[NB][4], vb[NB][4];
      Tid ids[NB];
      // the new token goes in before the load of its block: ahead of the
      // first loads when they include it (this wave holds fewer than NB
      // blocks of the piece), else just before that load -- a wave's loads
      // and stores complete in order, so its waits for the loads issued
      // after the stores also wait for the stores: as late as possible, they
      // hold up nothing but the last block
      if constexpr (!CAUSAL)
        if (n < NB) new_token_store(a, ntok, lane, hv, nsl, L, trow);
#pragma unroll
      for (int s = 0; s < NB - 1; ++s) {
        ids[s] = id_of(s);
        fetch(ids[s], kb[s], vb[s]);
      }
      // table entries are read one block ahead of the fetch that needs them
      Tid nid = id_of(NB - 1);
      int k = 0;
      for (; k + NB <= n; k += NB) {
        prio_from_progress<true>(a, pos - pos0 + nst * k, prio_span);
#pragma unroll
        for (int s = 0; s < NB; ++s) {
          const int nxt = (s + NB - 1) % NB;
          ids[nxt] = nid;
          nid = id_of(k + s + NB);
          if constexpr (!CAUSAL)
            if (k + s == n - NB) new_token_store(a, ntok, lane, hv, nsl, L, trow);
          fetch(ids[nxt], kb[nxt], vb[nxt]);
          // no instruction of the block's product may move above the next
          // block's loads (it would wait for data still in flight)
          __builtin_amdgcn_sched_barrier(0);
          consume(valid_of(k + s, ids[s]), jw + nst * (k + s), kb[s], vb[s]);
        }
      }
#pragma unroll
      for (int s = 0; s < NB - 1; ++s)
        if (k + s < n) consume(valid_of(k + s, ids[s]), jw + nst * (k + s), kb[s], vb[s]);
    }

    // ---- merge the 4 waves of this piece, write it -----------------------------
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      l_run[t] += __shfl_xor(l_run[t], 16, 64);
      l_run[t] += __shfl_xor(l_run[t], 32, 64);
      stash_piece(sh, ws, g, 16 * (t0 + t) + c, o[t], m_ref[t], l_run[t]);
    }
    if (a.defer_merge && jbeg == 0 && threadIdx.x == 0) write_job(a, um, b, hv, hv * um.TB + fb, nb);
    finish_piece<T>(a, sh, om, jbeg == 0 && jend == nb, first ? 0 : 1, unit, b, hv, hv * um.TB + fb,
                    nb, um);
    pos += jend - jbeg;
    first = false;
  }
  }
}

// Two-tile verify steps split the tiles over the waves (PA_VERIFY_SPLIT=0:
// every wave computes both).  Read at every launch.
bool verify_split() {
  const char* e = std::getenv("PA_VERIFY_SPLIT");
  return !(e && std::atoi(e) == 0);
}

// Prefetch depth (PA_MFMA_NB = 2, 3 or 4; default 2).  Read at every launch,
// as the other tuning variables are.
int mfma_nb() {
  const char* e = std::getenv("PA_MFMA_NB");
  const int v = e ? std::atoi(e) : 2;
  return (v == 3 || v == 4) ? v : 2;
}

template <typename T, int BS>
hipError_t launch_bs(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(unsigned(a.max_splits)), block(kWaves * 64);
  // the register-lengths form for batches of at most 64 sequences with no
  // queue, at the default prefetch depth and tile split
  const bool rl = a.batch <= kRegLens && !(a.unit_blocks > 0 && a.static_permille < 1000);
  if (a.n_query > 1) {  // verify / prefill chunk: one or two column tiles, causal
    const int ncol = a.n_query * (a.n_q_heads / a.pool.n_kv_heads);  // > 32: slices of 32
    if (ncol <= 16) {
      if (rl)
        hipLaunchKernelGGL((decode_split_mfma16<T, 2, 1, true, BS, false, true>), grid, block, 0, s, a);
      else
        hipLaunchKernelGGL((decode_split_mfma16<T, 2, 1, true, BS>), grid, block, 0, s, a);
    } else if (verify_split()) {
      if (rl)
        hipLaunchKernelGGL((decode_split_mfma16<T, 2, 2, true, BS, true, true>), grid, block, 0, s, a);
      else
        hipLaunchKernelGGL((decode_split_mfma16<T, 2, 2, true, BS, true>), grid, block, 0, s, a);
    } else {
      hipLaunchKernelGGL((decode_split_mfma16<T, 2, 2, true, BS>), grid, block, 0, s, a);
    }
    return hipGetLastError();
  }
  if constexpr (BS == 16) {
    switch (mfma_nb()) {
      case 3: hipLaunchKernelGGL((decode_split_mfma16<T, 3, 1, false, 16>), grid, block, 0, s, a); break;
      case 4: hipLaunchKernelGGL((decode_split_mfma16<T, 4, 1, false, 16>), grid, block, 0, s, a); break;
      default:
        if (rl)
          hipLaunchKernelGGL((decode_split_mfma16<T, 2, 1, false, 16, false, true>), grid, block, 0, s, a);
        else
          hipLaunchKernelGGL((decode_split_mfma16<T, 2, 1, false, 16>), grid, block, 0, s, a);
        break;
    }
  } else {
    if (rl)
      hipLaunchKernelGGL((decode_split_mfma16<T, 2, 1, false, BS, false, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((decode_split_mfma16<T, 2, 1, false, BS>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_nb(const DecodeArgs& a, hipStream_t s) {
  switch (a.pool.block_size) {
    case 8: return launch_bs<T, 8>(a, s);
    case 32: return launch_bs<T, 32>(a, s);
    default: return launch_bs<T, 16>(a, s);
  }
}

template <typename T>
int occupancy_nb(int nct) {
  int n = 0;
  hipError_t e;
  if (nct == 2 && verify_split())
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_split_mfma16<T, 2, 2, true, 16, true>, kWaves * 64, 0);
  else if (nct == 2)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_split_mfma16<T, 2, 2, true, 16>, kWaves * 64, 0);
  else if (nct == 1)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_split_mfma16<T, 2, 1, true, 16>, kWaves * 64, 0);
  else
    switch (mfma_nb()) {
      case 3: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_split_mfma16<T, 3, 1, false, 16>, kWaves * 64, 0); break;
      case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_split_mfma16<T, 4, 1, false, 16>, kWaves * 64, 0); break;
      default: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_split_mfma16<T, 2, 1, false, 16>, kWaves * 64, 0); break;
    }
  return (e == hipSuccess && n > 0) ? n : 2;
}

}  // namespace

hipError_t launch_decode_split_mfma16(const DecodeArgs& a, hipStream_t s) {
  return a.pool.kv_dtype == kBF16 ? launch_nb<__bf16>(a, s) : launch_nb<_Float16>(a, s);
}

// nct: 0 = decode, 1 or 2 = verify step with that many column tiles.
int occupancy_mfma16(int32_t kv_dtype, int nct) {
  static int cache[2][3][5] = {};  // [dtype][column tiles][prefetch depth, or tile split]
  const int i = kv_dtype == kBF16 ? 0 : 1;
  int& c = cache[i][nct][nct == 0 ? mfma_nb() : verify_split() ? 1 : 0];
  if (c == 0) c = i == 0 ? occupancy_nb<__bf16>(nct) : occupancy_nb<_Float16>(nct);
  return c;
}

}  // namespace pa
