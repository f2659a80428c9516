// Merge launch of the matrix-core decode: the log-sum-exp merge of every
// (sequence, KV head) segment that the split kernel left in pieces
// (defer_merge = 1; chosen when segments span many workgroups, so that one
// merge per segment would leave a long serial tail at the end of the split).
//
// One workgroup per (sequence b, KV head h, output column c: query head of the
// group, times the query of a verify step): it rebuilds the work-list cut from
// the lengths exactly as the split kernel did, finds the segment's pieces and
// folds the 32 16-byte columns of column c over them (decode_common.hpp,
// merge_segment), in list order.  A segment of
// one piece was written by the split kernel and is skipped.
#include "decode_common.hpp"

namespace pa {

namespace {

using namespace dec;

template <typename TO>
__global__ __launch_bounds__(kWaves * 64) void decode_merge_kernel(DecodeArgs a) {
  __shared__ Shared sh;
  const int H = seg_heads(a);
  const OutMap om = out_map(a);
  const int hc = int(blockIdx.x) % om.ncol(), bh = int(blockIdx.x) / om.ncol();
  const int b = bh / H, h = bh % H;
  if (hc >= om.cols(h)) return;  // past the last column of a short slice
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const Units um = setup_units(a, sh, w, lane);
  const int nb = blocks_of(a, sh, b);
  if (nb == 0) return;  // workgroup-uniform
  const int S = seq_start(a, sh, b, lane) + h * nb;  // every wave computes it
  const int np = um.unit_of(S + nb - 1) - um.unit_of(S) + 1;
  if (np <= 1) return;
  merge_segment<TO>(a, sh, om, b, h, S, np, um, hc, 1);
}

}  // namespace

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t s) {
  const int nsl = max(a.col_slices, 1);
  const int ncol = nsl > 1 ? 32 : max(a.n_query, 1) * (a.n_q_heads / a.pool.n_kv_heads);
  const dim3 grid(unsigned(a.batch) * unsigned(a.pool.n_kv_heads * nsl) * unsigned(ncol));
  if (a.q_dtype == kBF16)
    hipLaunchKernelGGL(decode_merge_kernel<__bf16>, grid, dim3(kWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL(decode_merge_kernel<_Float16>, grid, dim3(kWaves * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
