// Merge launch of the matrix-core decode: the log-sum-exp merge of every
// (sequence, KV head) segment that the split kernel left in pieces
// (defer_merge = 1; chosen when segments span many workgroups, so that one
// merge per segment would leave a long serial tail at the end of the split).
//
// One workgroup per (sequence b, KV head h, output column c: query head of the
// group, times the query of a verify step): it reads the segment's job (first
// unit, first slot, piece count) that the split kernel wrote and folds the 32
// 16-byte columns of column c over the pieces (decode_common.hpp,
// merge_segment), in list order.  A segment of one piece was written by the
// split kernel and is skipped, as is an empty sequence (no job was written).
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
  const int32_t* job = a.jobs + 2 * (size_t(b) * H + h);
  const int j0 = job[0], np = job[1];
  if (seq_len(a, b) == 0 || np <= 1) return;  // workgroup-uniform
  const unsigned rows = unsigned((a.ws_ml - a.ws_o) / kD);  // partial rows of the workspace
  merge_segment<TO, Shared, true>(a, sh, om, b, h, j0 & 0x7FFFFFFF, j0 < 0, np, rows, hc, 1);
}

}  // namespace

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t s) {
  const int nsl = max(a.col_slices, 1);
  const int ncol = nsl > 1 ? a.slice_cols : max(a.n_query, 1) * (a.n_q_heads / a.pool.n_kv_heads);
  const dim3 grid(unsigned(a.batch) * unsigned(a.pool.n_kv_heads * nsl) * unsigned(ncol));
  if (a.q_dtype == kBF16)
    hipLaunchKernelGGL(decode_merge_kernel<__bf16>, grid, dim3(kWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL(decode_merge_kernel<_Float16>, grid, dim3(kWaves * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
