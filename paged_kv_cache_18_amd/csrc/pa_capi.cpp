// C ABI of libpa (declarations and contract: include/pa.h).
//
// Every entry point validates its arguments before touching any state, turns
// internal errors into a pa_status, and records a thread-local message.  Device
// work goes to the kernels behind kernels/launch.hpp on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <mutex>
#include <new>
#include <string>

#include "../../include/pa.h"
#include "kernels/launch.hpp"
#include "pa_host.hpp"

struct pa_pool {
  pa::PoolCore core;
  pa::Layout layout;
  uint8_t* dev;
  size_t dev_bytes;
  pa_pool(const pa::Desc& d, const int32_t* bo, const int32_t* so)
      : core(d, bo, so), layout(pa::compute_layout(d)), dev(nullptr), dev_bytes(0) {}
};

namespace {

thread_local std::string g_err;

[[noreturn]] void fail(pa::Status s, const std::string& m) { throw pa::Error{s, m}; }

template <class F>
pa_status guard(F&& f) {
  try {
    f();
    return PA_OK;
  } catch (const pa::Error& e) {
    g_err = e.msg;
    return e.code;
  } catch (const std::bad_alloc&) {
    g_err = "host out of memory";
    return PA_ERR_INVALID_ARG;
  } catch (...) {
    g_err = "internal error";
    return PA_ERR_INVALID_ARG;
  }
}

void need(const void* p, const char* what) {
  if (!p) fail(pa::kInvalidArg, std::string(what) + " is NULL");
}

pa::Desc to_desc(const pa_pool_desc* d) {
  need(d, "desc");
  return pa::Desc{d->block_size, d->n_kv_heads,      d->head_dim,
                  d->kv_dtype,   d->group_size,      d->num_blocks,
                  d->num_sink_blocks, d->sink_blocks_per_seq, d->window_tokens};
}

void check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) fail(pa::kHip, std::string(what) + ": " + hipGetErrorString(e));
}

pa::PoolDev dev_view(const pa_pool* p) {
  pa::PoolDev v{};
  const pa::Desc& d = p->core.desc();
  v.base = p->dev;
  v.n_kv_heads = d.n_kv_heads;
  v.head_dim = d.head_dim;
  v.kv_dtype = d.kv_dtype;
  v.group_size = d.kv_dtype == pa::kInt4 ? d.group_size : d.head_dim;
  v.num_blocks = d.num_blocks;
  v.num_sink_blocks = d.num_sink_blocks;
  v.sink_per_seq = d.sink_blocks_per_seq;
  v.window_tokens = d.window_tokens;
  v.block_size = d.block_size;
  for (int i = 0; i < pa::kNumArr; ++i) {
    v.off[i] = p->layout.offset[i];
    v.slab[i] = p->layout.slab[i];
  }
  return v;
}

void need_device(const pa_pool* p) {
  need(p, "pool");
  if (!p->dev) fail(pa::kInvalidArg, "metadata-only pool has no device memory");
}

void enqueue_copy(pa_pool* p, int32_t src, int32_t dst, void* stream) {
  if (!p->dev) return;
  check_hip(pa::launch_block_copy(dev_view(p), src, dst, static_cast<hipStream_t>(stream)),
            "block copy launch");
}

// ---- decode planning ---------------------------------------------------------------
int env_int(const char* name, int dflt) {
  const char* s = std::getenv(name);
  if (!s || !*s) return dflt;
  return std::atoi(s);
}

int32_t plan_split_blocks(int32_t batch, int32_t hkv, int32_t max_seq_len) {
  const int forced = env_int("PA_SPLIT_BLOCKS", 0);  // tuning knob
  if (forced > 0) return forced;
  const int64_t nb = (int64_t(max_seq_len) + 15) / 16;
  const int64_t pairs = int64_t(batch) * hkv;
  int32_t s = 16;
  // enough splits to fill 256 compute units several times over, no more
  while (s < (1 << 20) && pairs * ((nb + s - 1) / s) > 4096) s *= 2;
  return s;
}

// Compute units of the current device (cached per device).
int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

struct Plan {
  int32_t split_blocks, max_splits, kernel;
  int32_t unit_blocks, static_permille;  // the cut of the matrix-core kernels
  int32_t defer_merge;                   // split segments merged by a second launch
  int32_t col_slices;                    // matrix-core kernels: column slices per (seq, kv head)
  int32_t slice_cols;                    // (query, head) columns of a slice
  size_t ws_bytes;      // bytes the call needs
  size_t ws_o_offset;   // byte offset of the partial sums
  size_t ws_ml_offset;  // float index (from ws_o) of the (max, sum) pairs
  size_t ws_jobs_offset;  // byte offset of the merge launch's per-segment jobs (0: none)
};

// The workspace starts with kCtrCap counters of the matrix-core kernels (the
// unit queue, then one arrival counter per unit), kCtrStride 32-bit words
// apart (one per 128-byte line), at the same place for every call and shape:
// a zero-filled workspace stays valid because every call leaves them at zero
// and nothing else is written there.
constexpr int32_t kCtrCap = 8192;
constexpr int32_t kCtrStride = 32;
constexpr size_t kCtrBytes = size_t(kCtrCap) * kCtrStride * sizeof(unsigned);
// Default cut of the matrix-core kernels' work list: each workgroup streams
// this share (per mille) of its region, the rest is queued in units of
// kUnitBlocks blocks.  Queued units balance the finish times of compute units
// and XCDs, but a unit starts with an empty load pipeline, so at ~6 us of
// loaded HBM latency they cost more than they win; off by default
// (PA_STATIC_PERMILLE / PA_UNIT_BLOCKS turn them on).
constexpr int32_t kStaticPermille = 1000;
constexpr int32_t kUnitBlocks = 16;
// Average pieces per segment above which split segments are merged by a
// second launch instead of inside the split kernel.
constexpr int32_t kFuseMaxPieces = 16;
// Split-kernel workgroups per compute unit at most: two larger regions per
// CU measured as fast or faster than the three that fit (fewer piece ends;
// the long-context batch 2 %, the shared-prefix batch 17 % and the split-tile
// verify step 6 % faster).
constexpr int kDecodePerCu = 2;

// Upper bound of the flattened work list (blocks of all (sequence, kv head)
// segments) from the shapes alone.
int64_t flat_upper(int32_t batch, int32_t hkv, int32_t max_seq_len) {
  return int64_t(batch) * hkv * ((int64_t(max_seq_len) + 15) / 16);
}

// n_query: queries per sequence (1 = decode; the verify step's gamma + 1).
Plan make_plan(const pa_pool* p, int32_t batch, int32_t n_q_heads, int32_t max_seq_len,
               int32_t q_dtype, int32_t n_query = 1) {
  const pa::Desc& d = p->core.desc();
  Plan pl{};
  const int32_t G = n_q_heads / d.n_kv_heads;
  const int32_t ncol = n_query * G;  // output columns per (sequence, kv head)
  const bool mfma_ok = (d.kv_dtype == pa::kBF16 || d.kv_dtype == pa::kF16) &&
                       q_dtype == d.kv_dtype && d.head_dim == 128 && G <= 16 && d.num_sink_blocks == 0;
  // INT4 groups of 128 or 64 dims: the matrix-core B operand's 16 columns
  // hold every logical column once per group (16 / groups of them per tile);
  // decode needs one tile for the G query heads, a verify step or prefill
  // chunk takes two tiles and slices beyond them
  const int32_t ngroups = d.kv_dtype == pa::kInt4 ? d.head_dim / d.group_size : 1;
  const bool quant_ok = (d.kv_dtype == pa::kInt4 || d.kv_dtype == pa::kFp8) && q_dtype == pa::kF16 &&
                        d.head_dim == 128 && ngroups <= 2 && (n_query > 1 || ngroups * G <= 16);
  // more (query, head) columns than a segment takes (a long verify step, a
  // prefill chunk): slices of that many columns, each its own segment of the
  // work list -- 32 for 16-bit pools and INT4 groups of 128 / FP8 (two
  // tiles), 8 for INT4 groups of 64 (one tile: the two-tile kernel of that
  // group size holds more registers than a SIMD gives it, and its spills cost
  // more than the extra pass over the cache a third slice makes -- the
  // 6-query verify of 65,536 tokens: 73 us against 88)
  int32_t slice = mfma_ok ? 32 : ngroups == 2 ? 8 : 32;
  if (!mfma_ok) {  // tuning knob: quantized slice width, 1 .. 32 / groups
    const int q = env_int("PA_QUANT_SLICE", 0);
    if (q > 0) slice = std::min(q, 32 / ngroups);
  }
  const int32_t nsl = n_query > 1 && ncol > slice ? (ncol + slice - 1) / slice : 1;
  const int32_t seg_cols = nsl > 1 ? slice : ncol;
  const char* force = std::getenv("PA_DECODE_KERNEL");  // "generic" forces the VALU kernel
  const bool generic = force && std::strcmp(force, "generic") == 0;
  pl.kernel = generic ? pa::kKernGeneric
              : mfma_ok ? pa::kKernMfma16
              : quant_ok ? pa::kKernQuant
                         : pa::kKernGeneric;
  if (d.block_size != 16 && pl.kernel != pa::kKernMfma16)
    fail(pa::kUnsupported, "block sizes 8 and 32 are decoded by the matrix-core kernel only");
  const int64_t nb = (int64_t(max_seq_len) + 15) / 16;
  if (pl.kernel != pa::kKernGeneric) {
    // Fixed chunks of the flattened list; two partial slots per workgroup.
    pl.col_slices = nsl;
    pl.slice_cols = slice;
    const int64_t w = flat_upper(batch, d.n_kv_heads, max_seq_len) * pl.col_slices;
    if (w >= (int64_t(1) << 31) - 4096) fail(pa::kInvalidArg, "batch * n_kv_heads * blocks too large");
    int32_t c = env_int("PA_SPLIT_BLOCKS", 0);  // fixed chunk size (tuning/tests)
    int64_t units = 0;                          // units of the cut, at most
    if (c > 0) {
      c = int32_t(std::max<int64_t>(c, (w + kCtrCap - 2) / (kCtrCap - 1)));  // < kCtrCap units
      pl.split_blocks = c;
      pl.max_splits = int32_t(std::max<int64_t>(1, (w + c - 1) / c));
      units = pl.max_splits;
    } else {
      // persistent grid: one 4-wave workgroup per resident slot (from the
      // occupancy calculator); the chunk size is derived on the device from
      // the actual lengths
      pl.split_blocks = 0;
      int per_cu = env_int("PA_WG_PER_CU", 0);  // tuning knob; default: resident slots
      if (per_cu <= 0) {
        per_cu = pa::decode_split_occupancy(pl.kernel, d.kv_dtype,
                                            n_query == 1 ? 0 : seg_cols * ngroups <= 16 ? 1 : 2,
                                            d.group_size);
        per_cu = std::min(per_cu, kDecodePerCu);
      }
      pl.max_splits = int32_t(std::max<int64_t>(
          1, std::min<int64_t>({w, int64_t(cu_count()) * per_cu, int64_t(kCtrCap / 2)})));
      // queued units: the owner streams static_permille/1000 of its region,
      // the rest goes to the queue in units of unit_blocks (doubled until the
      // units fit the counters)
      const int64_t r = pl.max_splits, cmax = (w + r - 1) / r;
      pl.static_permille = std::clamp(env_int("PA_STATIC_PERMILLE", kStaticPermille), 0, 1000);
      int64_t u = std::max(1, env_int("PA_UNIT_BLOCKS", kUnitBlocks));
      if (pl.static_permille < 1000) {
        while (1 + r * (1 + (cmax + u - 1) / u) > kCtrCap) u *= 2;
        pl.unit_blocks = int32_t(u);
        units = r * (1 + (cmax + u - 1) / u);
      } else {
        pl.unit_blocks = 0;
        units = r;
      }
    }
    // Merging a segment is one round of loads per kMergeBatch pieces per
    // thread, done by the workgroup that completes it; when segments span
    // many workgroups on average those rounds form a serial tail, and a
    // second launch with one workgroup per (segment, query head) is shorter.
    const int64_t segs = std::max<int64_t>(1, int64_t(batch) * d.n_kv_heads * pl.col_slices);
    const int fuse_max = env_int("PA_FUSE_MAX_PIECES", kFuseMaxPieces);
    pl.defer_merge = units / segs + 1 > fuse_max ? 1 : 0;
    const size_t rows = size_t(units) * 2 * size_t(pl.col_slices > 1 ? seg_cols : ncol);
    pl.ws_o_offset = kCtrBytes;
    pl.ws_ml_offset = rows * size_t(d.head_dim);
    pl.ws_jobs_offset = kCtrBytes + rows * (size_t(d.head_dim) + 2) * sizeof(float);
    pl.ws_bytes = pl.ws_jobs_offset + size_t(segs) * 2 * sizeof(int32_t);
    return pl;
  }
  pl.split_blocks = plan_split_blocks(batch, d.n_kv_heads, max_seq_len);
  pl.max_splits = int32_t(std::max<int64_t>(1, (nb + pl.split_blocks - 1) / pl.split_blocks));
  const size_t rows = size_t(batch) * size_t(n_query) * size_t(n_q_heads) * size_t(pl.max_splits);
  pl.ws_o_offset = kCtrBytes;  // partials never overwrite the counters
  pl.ws_ml_offset = rows * size_t(d.head_dim);
  pl.ws_bytes = pl.max_splits > 1 ? kCtrBytes + rows * (size_t(d.head_dim) + 2) * sizeof(float) : 0;
  return pl;
}

void check_shapes(const pa_pool* p, int32_t batch, int32_t n_q_heads, int32_t max_seq_len) {
  need(p, "pool");
  const pa::Desc& d = p->core.desc();
  if (batch < 0 || batch > 65535) fail(pa::kInvalidArg, "batch must be in [0, 65535]");
  if (n_q_heads < 1 || n_q_heads % d.n_kv_heads) fail(pa::kInvalidArg, "n_q_heads must be a multiple of n_kv_heads");
  if (n_q_heads > 65535) fail(pa::kInvalidArg, "n_q_heads too large");
  if (max_seq_len < 0) fail(pa::kInvalidArg, "negative max_seq_len");
}

enum Phase { kBoth = 3, kSplit = 1, kCombine = 2 };

constexpr int32_t kMaxQueries = 4096;  // verify step / prefill chunk: queries per sequence, at most

// Prefill chunks of 16-bit pools of 16-token blocks go to the tile kernel
// (PA_PREFILL_TILE=0 keeps them on the split kernel, for comparison).
bool prefill_tile(const pa_pool* pool, const Plan& pl) {
  return pl.kernel == pa::kKernMfma16 && pool->core.desc().block_size == 16 &&
         env_int("PA_PREFILL_TILE", 1) != 0;
}

void* noalloc_scratch(hipStream_t s);

// noalloc: take the workspace from the library's static scratch array
// (pa_decode_attention_noalloc) instead of ws / ws_bytes.
// The step's append (pa_decode_step): K / V rows of the new tokens.
struct NewTokens {
  const void* k = nullptr;
  const void* v = nullptr;
  int32_t dtype = 0;
};

pa_status decode(int phase, const void* q, const pa_pool* pool, const int32_t* tables,
                 const int32_t* lens, int32_t batch, int32_t n_q_heads, int32_t q_dtype,
                 int32_t max_blocks, int32_t max_seq_len, float scale, void* out, void* ws,
                 size_t ws_bytes, void* stream, int32_t n_query = 1, bool prefill = false,
                 bool noalloc = false, NewTokens nt = {}) {
  return guard([&] {
    need_device(pool);
    if (nt.k || nt.v) {
      need(nt.k, "k_new");
      need(nt.v, "v_new");
      if (!pa::is_raw(nt.dtype)) fail(pa::kInvalidArg, "in_dtype must be F32, F16 or BF16");
    }
    check_shapes(pool, batch, n_q_heads, max_seq_len);
    if (n_query < 1 || n_query > kMaxQueries) fail(pa::kInvalidArg, "n_query must be in [1, 4096]");
    const pa::Desc& d = pool->core.desc();
    if (pa::is_raw(d.kv_dtype)) {
      if (q_dtype != d.kv_dtype) fail(pa::kInvalidArg, "q_dtype must equal the pool's kv_dtype");
    } else if (q_dtype != pa::kF16) {
      fail(pa::kInvalidArg, "INT4/FP8 pools take fp16 queries");
    }
    if (max_blocks < 1) fail(pa::kInvalidArg, "max_blocks_per_seq must be >= 1");
    if (int64_t(max_seq_len) > int64_t(max_blocks) * d.block_size)
      fail(pa::kInvalidArg, "max_seq_len exceeds block_size * max_blocks_per_seq");
    if (!std::isfinite(scale)) fail(pa::kInvalidArg, "scale must be finite");
    if (batch == 0) return;
    need(q, "q");
    need(tables, "block_tables_dev");
    need(lens, "seq_lens_dev");
    need(out, "out");
    const Plan pl = make_plan(pool, batch, n_q_heads, max_seq_len, q_dtype, n_query);
    const bool tile = prefill && prefill_tile(pool, pl);
    if (pl.kernel == pa::kKernGeneric && int64_t(batch) * n_query > 65535)
      fail(pa::kUnsupported, "batch * n_query above 65535 on the generic kernel");
    if (noalloc && !tile && pl.ws_bytes > 0) {
      if (pl.ws_bytes > PA_NOALLOC_SCRATCH_BYTES)
        fail(pa::kInvalidArg, "these shapes need " + std::to_string(pl.ws_bytes) +
                                  " bytes of workspace, above the static scratch of " +
                                  std::to_string(size_t(PA_NOALLOC_SCRATCH_BYTES)) +
                                  " bytes: use pa_decode_attention with a workspace");
      ws = noalloc_scratch(static_cast<hipStream_t>(stream));
      ws_bytes = PA_NOALLOC_SCRATCH_BYTES;
    }
    if (!tile && pl.ws_bytes > 0) {
      need(ws, "workspace");
      if (ws_bytes < pl.ws_bytes)
        fail(pa::kInvalidArg, "workspace too small: need " + std::to_string(pl.ws_bytes) + " bytes");
      if (reinterpret_cast<uintptr_t>(ws) % 256) fail(pa::kInvalidArg, "workspace must be 256-byte aligned");
    }
    pa::DecodeArgs a{};
    a.pool = dev_view(pool);
    a.q = q;
    a.tables = tables;
    a.lens = lens;
    a.batch = batch;
    a.n_q_heads = n_q_heads;
    a.q_dtype = q_dtype;
    a.max_blocks_per_seq = max_blocks;
    a.max_seq_len = max_seq_len;
    a.n_query = n_query;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.out = out;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (tile) {
      if (phase & kSplit) check_hip(pa::launch_prefill_tile(a, s), "prefill launch");
      return;
    }
    if (pl.ws_bytes) {
      a.ws_o = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + pl.ws_o_offset);
      a.ws_ml = a.ws_o + pl.ws_ml_offset;
      a.counters = static_cast<unsigned*>(ws);
      a.ctr_stride = kCtrStride;
      if (pl.ws_jobs_offset)
        a.jobs = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + pl.ws_jobs_offset);
    }
    a.prio = env_int("PA_PRIO", 1) != 0 ? 1 : 0;  // tuning knob
    a.unit_blocks = pl.unit_blocks;
    a.static_permille = pl.static_permille;
    a.defer_merge = pl.defer_merge;
    a.col_slices = std::max(pl.col_slices, 1);
    a.slice_cols = pl.slice_cols;
    a.split_blocks = pl.split_blocks;
    a.max_splits = pl.max_splits;
    a.kernel = pl.kernel;
    if (nt.k && (phase & kSplit)) {
      // the matrix-core kernels write the new tokens themselves (16-bit pools:
      // inputs of the pool's dtype; INT4/FP8 pools quantize them); otherwise a
      // launch of their own goes first
      if ((pl.kernel == pa::kKernMfma16 && nt.dtype == d.kv_dtype) || pl.kernel == pa::kKernQuant) {
        a.app_k = nt.k;
        a.app_v = nt.v;
        a.app_dt = nt.dtype;
      } else {
        check_hip(pa::launch_append_last(a.pool, nt.k, nt.v, nt.dtype, tables, lens, batch, max_blocks,
                                         max_seq_len, s),
                  "append launch");
      }
    }
    if (phase & kSplit) check_hip(pa::launch_decode_split(a, s), "decode split launch");
    if (phase & kCombine) check_hip(pa::launch_decode_combine(a, s), "decode combine launch");
  });
}

// ---- static scratch of the allocation-free decode ---------------------------------
// One copy per GPU (each device that loads the library's code object holds
// its own), kept until the process ends.  Host code never passes the array's
// name to a kernel or a copy: in host code it is a stand-in, not a device
// address.  The device address comes from hipGetSymbolAddress, once per
// device with that device current, and is kept per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

// The current device's scratch address; the first call on a device looks it
// up and clears the counter area (the only part a call expects at zero, and
// which every call leaves at zero) with a fill kernel on `s`.
void* noalloc_scratch(hipStream_t s) {
  int dev = -1;
  check_hip(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) fail(pa::kUnsupported, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p || reinterpret_cast<uintptr_t>(p) % 256) fail(pa::kHip, "scratch address not 256-byte aligned");
    check_hip(pa::launch_zero(p, kCtrBytes, s), "scratch clear launch");
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

static_assert(kCtrBytes <= PA_NOALLOC_SCRATCH_BYTES, "the counters fit the static scratch");

}  // namespace

extern "C" {

pa_status pa_pool_bytes(const pa_pool_desc* desc, size_t* bytes) {
  return guard([&] {
    need(bytes, "bytes");
    *bytes = pa::compute_layout(to_desc(desc)).total;
  });
}

pa_status pa_pool_create(const pa_pool_desc* desc, void* dev_mem, size_t dev_bytes,
                         const int32_t* body_free_order, const int32_t* sink_free_order,
                         pa_pool** out) {
  return guard([&] {
    need(out, "out");
    pa::Desc d = to_desc(desc);
    pa::Layout L = pa::compute_layout(d);
    if (dev_mem) {
      if (dev_bytes < L.total)
        fail(pa::kInvalidArg, "pool memory too small: need " + std::to_string(L.total) + " bytes");
      if (reinterpret_cast<uintptr_t>(dev_mem) % 256) fail(pa::kInvalidArg, "pool memory must be 256-byte aligned");
    } else if (dev_bytes != 0) {
      fail(pa::kInvalidArg, "dev_bytes must be 0 for a metadata-only pool");
    }
    pa_pool* p = new pa_pool(d, body_free_order, sink_free_order);
    p->dev = static_cast<uint8_t*>(dev_mem);
    p->dev_bytes = dev_bytes;
    *out = p;
  });
}

pa_status pa_pool_destroy(pa_pool* pool) {
  return guard([&] {
    need(pool, "pool");
    delete pool;
  });
}

pa_status pa_pool_layout(const pa_pool* pool, pa_layout* out) {
  return guard([&] {
    need(pool, "pool");
    need(out, "out");
    out->total_bytes = pool->layout.total;
    for (int i = 0; i < PA_NUM_ARR; ++i) {
      out->offset[i] = pool->layout.offset[i];
      out->slab_bytes[i] = pool->layout.slab[i];
    }
  });
}

pa_status pa_alloc_block(pa_pool* pool, int32_t arena, int32_t* out_id) {
  return guard([&] {
    need(pool, "pool");
    need(out_id, "out_id");
    *out_id = pool->core.alloc(arena);
  });
}

pa_status pa_incref(pa_pool* pool, int32_t id) {
  return guard([&] {
    need(pool, "pool");
    pool->core.incref(id);
  });
}

pa_status pa_free_block(pa_pool* pool, int32_t id) {
  return guard([&] {
    need(pool, "pool");
    pool->core.free_block(id);
  });
}

pa_status pa_cow_clone(pa_pool* pool, int32_t src, int32_t* out_dst, void* stream) {
  return guard([&] {
    need(pool, "pool");
    need(out_dst, "out_dst");
    int32_t dst = pool->core.cow_clone(src);
    *out_dst = dst;
    enqueue_copy(pool, src, dst, stream);
  });
}

pa_status pa_refcount(const pa_pool* pool, int32_t id, int32_t* out) {
  return guard([&] {
    need(pool, "pool");
    need(out, "out");
    *out = pool->core.refcount(id);
  });
}

pa_status pa_num_free(const pa_pool* pool, int32_t arena, int32_t* out) {
  return guard([&] {
    need(pool, "pool");
    need(out, "out");
    *out = pool->core.num_free(arena);
  });
}

pa_status pa_free_list(const pa_pool* pool, int32_t arena, int32_t* out, int32_t cap, int32_t* n) {
  return guard([&] {
    need(pool, "pool");
    need(n, "n");
    if (cap < 0) fail(pa::kInvalidArg, "negative cap");
    std::vector<int32_t> f = pool->core.free_list(arena);
    const int32_t m = std::min<int32_t>(cap, int32_t(f.size()));
    if (m > 0) need(out, "out");
    for (int32_t i = 0; i < m; ++i) out[i] = f[size_t(i)];
    *n = m;
  });
}

pa_status pa_num_clones(const pa_pool* pool, int64_t* out) {
  return guard([&] {
    need(pool, "pool");
    need(out, "out");
    *out = pool->core.num_clones();
  });
}

pa_status pa_seq_create(pa_pool* pool, int32_t* out_seq) {
  return guard([&] {
    need(pool, "pool");
    need(out_seq, "out_seq");
    *out_seq = pool->core.seq_create();
  });
}

pa_status pa_seq_fork(pa_pool* pool, int32_t parent, int32_t* out_child) {
  return guard([&] {
    need(pool, "pool");
    need(out_child, "out_child");
    *out_child = pool->core.seq_fork(parent);
  });
}

pa_status pa_seq_reserve(pa_pool* pool, int32_t seq, int32_t n_tokens, int32_t* slots_out,
                         void* stream) {
  return guard([&] {
    need(pool, "pool");
    if (n_tokens > 0) need(slots_out, "slots_out");
    std::vector<std::pair<int32_t, int32_t>> clones;
    std::vector<int32_t> slots = pool->core.seq_reserve(seq, n_tokens, &clones);
    if (!slots.empty()) std::memcpy(slots_out, slots.data(), slots.size() * sizeof(int32_t));
    for (const auto& c : clones) enqueue_copy(pool, c.first, c.second, stream);
  });
}

pa_status pa_seq_settle(pa_pool* pool, int32_t seq, void* stream, int32_t* n_moved) {
  return guard([&] {
    need(pool, "pool");
    std::vector<std::pair<int32_t, int32_t>> moves;
    const int32_t n = pool->core.seq_settle(seq, &moves);
    if (n_moved) *n_moved = n;
    if (!pool->dev) return;  // metadata-only pool
    const pa::PoolDev p = dev_view(pool);
    for (size_t i = 0; i < moves.size(); i += pa::kMigrateMax) {
      pa::MigrateJob job{};
      job.n = int32_t(std::min<size_t>(pa::kMigrateMax, moves.size() - i));
      for (int32_t k = 0; k < job.n; ++k) {
        job.src[k] = moves[i + size_t(k)].first;
        job.dst[k] = moves[i + size_t(k)].second;
      }
      check_hip(pa::launch_migrate(p, job, static_cast<hipStream_t>(stream)), "migrate launch");
    }
  });
}

pa_status pa_prefix_lookup(pa_pool* pool, const int32_t* ids, int32_t n, int32_t* out_seq,
                           int32_t* n_cached) {
  return guard([&] {
    need(pool, "pool");
    need(out_seq, "out_seq");
    need(n_cached, "n_cached_tokens");
    int32_t sid = -1;
    *n_cached = pool->core.prefix_lookup(ids, n, &sid);
    *out_seq = sid;
  });
}

pa_status pa_prefix_register(pa_pool* pool, int32_t seq, const int32_t* ids, int32_t n,
                             int32_t* n_added) {
  return guard([&] {
    need(pool, "pool");
    const int32_t k = pool->core.prefix_register(seq, ids, n);
    if (n_added) *n_added = k;
  });
}

pa_status pa_prefix_evict(pa_pool* pool, int32_t max_blocks, int32_t* n_evicted) {
  return guard([&] {
    need(pool, "pool");
    const int32_t k = pool->core.prefix_evict(max_blocks);
    if (n_evicted) *n_evicted = k;
  });
}

pa_status pa_prefix_stats(const pa_pool* pool, int32_t* n_entries, int64_t* hit_blocks,
                          int64_t* asked_blocks) {
  return guard([&] {
    need(pool, "pool");
    if (n_entries) *n_entries = pool->core.prefix_entries();
    if (hit_blocks) *hit_blocks = pool->core.prefix_hit_blocks();
    if (asked_blocks) *asked_blocks = pool->core.prefix_asked_blocks();
  });
}

pa_status pa_prefix_block_hashes(const int32_t* ids, int32_t n, uint64_t* out) {
  return guard([&] {
    if (n < 0) fail(pa::kInvalidArg, "negative token count");
    if (n >= pa::kBlock) {
      need(ids, "token_ids");
      need(out, "hashes_out");
    }
    uint64_t h = 0xcbf29ce484222325ull;
    for (int32_t j = 0; j < n / pa::kBlock; ++j) {
      h = pa::PoolCore::block_hash(h, ids + size_t(j) * pa::kBlock);
      out[j] = h;
    }
  });
}

pa_status pa_seq_truncate(pa_pool* pool, int32_t seq, int32_t new_len) {
  return guard([&] {
    need(pool, "pool");
    pool->core.seq_truncate(seq, new_len);
  });
}

pa_status pa_seq_release(pa_pool* pool, int32_t seq) {
  return guard([&] {
    need(pool, "pool");
    pool->core.seq_release(seq);
  });
}

pa_status pa_seq_info(const pa_pool* pool, int32_t seq, int32_t* len, int32_t* n_blocks) {
  return guard([&] {
    need(pool, "pool");
    const pa::Seq& s = pool->core.seq(seq);
    if (len) *len = s.length;
    if (n_blocks) *n_blocks = int32_t(s.table.size());
  });
}

pa_status pa_block_tables(const pa_pool* pool, const int32_t* seqs, int32_t n, int32_t max_blocks,
                          int32_t* tables_out, int32_t* lens_out) {
  return guard([&] {
    need(pool, "pool");
    if (n < 0 || max_blocks < 0) fail(pa::kInvalidArg, "negative size");
    if (n == 0) return;
    need(seqs, "seqs");
    need(tables_out, "tables_out");
    for (int32_t i = 0; i < n; ++i) {
      const pa::Seq& s = pool->core.seq(seqs[i]);
      if (int64_t(s.table.size()) > max_blocks)
        fail(pa::kInvalidArg, "sequence " + std::to_string(seqs[i]) + " has more blocks than max_blocks");
    }
    for (int32_t i = 0; i < n; ++i) {
      const pa::Seq& s = pool->core.seq(seqs[i]);
      int32_t* row = tables_out + size_t(i) * size_t(max_blocks);
      for (int32_t j = 0; j < max_blocks; ++j)
        row[j] = size_t(j) < s.table.size() ? s.table[size_t(j)] : -1;
      if (lens_out) lens_out[i] = s.length;
    }
  });
}

pa_status pa_append_kv(pa_pool* pool, const void* k, const void* v, int32_t in_dtype,
                       const int32_t* slots_dev, int32_t n_tokens, void* stream) {
  return guard([&] {
    need_device(pool);
    if (!pa::is_raw(in_dtype)) fail(pa::kInvalidArg, "in_dtype must be F32, F16 or BF16");
    if (n_tokens < 0) fail(pa::kInvalidArg, "negative n_tokens");
    if (n_tokens == 0) return;
    need(k, "k");
    need(v, "v");
    need(slots_dev, "slots_dev");
    check_hip(pa::launch_append(dev_view(pool), k, v, in_dtype, slots_dev, n_tokens,
                                static_cast<hipStream_t>(stream)),
              "append launch");
  });
}

pa_status pa_decode_workspace_bytes(const pa_pool* pool, int32_t batch, int32_t n_q_heads,
                                    int32_t max_seq_len, size_t* bytes) {
  return guard([&] {
    check_shapes(pool, batch, n_q_heads, max_seq_len);
    need(bytes, "bytes");
    const pa::Desc& d = pool->core.desc();
    const int32_t qdt = pa::is_raw(d.kv_dtype) ? d.kv_dtype : int32_t(pa::kF16);
    *bytes = make_plan(pool, batch, n_q_heads, max_seq_len, qdt).ws_bytes;
  });
}

pa_status pa_decode_split_blocks(const pa_pool* pool, int32_t batch, int32_t n_q_heads,
                                 int32_t max_seq_len, int32_t* out) {
  return guard([&] {
    check_shapes(pool, batch, n_q_heads, max_seq_len);
    need(out, "out");
    const pa::Desc& d = pool->core.desc();
    const int32_t qdt = pa::is_raw(d.kv_dtype) ? d.kv_dtype : int32_t(pa::kF16);
    const Plan pl = make_plan(pool, batch, n_q_heads, max_seq_len, qdt);
    *out = pl.split_blocks > 0 ? pl.split_blocks : -pl.max_splits;
  });
}

pa_status pa_decode_attention(const void* q, const pa_pool* pool, const int32_t* tables,
                              const int32_t* lens, int32_t batch, int32_t n_q_heads, int32_t q_dtype,
                              int32_t max_blocks, int32_t max_seq_len, float scale, void* out,
                              void* ws, size_t ws_bytes, void* stream) {
  return decode(kBoth, q, pool, tables, lens, batch, n_q_heads, q_dtype, max_blocks, max_seq_len,
                scale, out, ws, ws_bytes, stream);
}

pa_status pa_decode_attention_noalloc(const void* q, const pa_pool* pool, const int32_t* tables,
                                      const int32_t* lens, int32_t batch, int32_t n_q_heads,
                                      int32_t q_dtype, int32_t max_blocks, int32_t max_seq_len,
                                      float scale, void* out, void* stream) {
  return decode(kBoth, q, pool, tables, lens, batch, n_q_heads, q_dtype, max_blocks, max_seq_len,
                scale, out, nullptr, 0, stream, 1, false, true);
}

pa_status pa_decode_split(const void* q, const pa_pool* pool, const int32_t* tables,
                          const int32_t* lens, int32_t batch, int32_t n_q_heads, int32_t q_dtype,
                          int32_t max_blocks, int32_t max_seq_len, float scale, void* out, void* ws,
                          size_t ws_bytes, void* stream) {
  return decode(kSplit, q, pool, tables, lens, batch, n_q_heads, q_dtype, max_blocks, max_seq_len,
                scale, out, ws, ws_bytes, stream);
}

pa_status pa_decode_combine(const void* q, const pa_pool* pool, const int32_t* tables,
                            const int32_t* lens, int32_t batch, int32_t n_q_heads, int32_t q_dtype,
                            int32_t max_blocks, int32_t max_seq_len, float scale, void* out,
                            void* ws, size_t ws_bytes, void* stream) {
  return decode(kCombine, q, pool, tables, lens, batch, n_q_heads, q_dtype, max_blocks,
                max_seq_len, scale, out, ws, ws_bytes, stream);
}

pa_status pa_decode_step(const void* q, const void* k_new, const void* v_new, int32_t in_dtype,
                         pa_pool* pool, const int32_t* tables, const int32_t* lens, int32_t batch,
                         int32_t n_q_heads, int32_t q_dtype, int32_t max_blocks,
                         int32_t max_seq_len, float scale, void* out, void* ws, size_t ws_bytes,
                         void* stream) {
  return decode(kBoth, q, pool, tables, lens, batch, n_q_heads, q_dtype, max_blocks, max_seq_len,
                scale, out, ws, ws_bytes, stream, 1, false, false, NewTokens{k_new, v_new, in_dtype});
}

pa_status pa_decode_step_split(const void* q, const void* k_new, const void* v_new,
                               int32_t in_dtype, pa_pool* pool, const int32_t* tables,
                               const int32_t* lens, int32_t batch, int32_t n_q_heads,
                               int32_t q_dtype, int32_t max_blocks, int32_t max_seq_len,
                               float scale, void* out, void* ws, size_t ws_bytes, void* stream) {
  return decode(kSplit, q, pool, tables, lens, batch, n_q_heads, q_dtype, max_blocks, max_seq_len,
                scale, out, ws, ws_bytes, stream, 1, false, false, NewTokens{k_new, v_new, in_dtype});
}

pa_status pa_verify_workspace_bytes(const pa_pool* pool, int32_t batch, int32_t n_q_heads,
                                    int32_t n_query, int32_t max_seq_len, size_t* bytes) {
  return guard([&] {
    check_shapes(pool, batch, n_q_heads, max_seq_len);
    need(bytes, "bytes");
    if (n_query < 1 || n_query > kMaxQueries) fail(pa::kInvalidArg, "n_query must be in [1, 4096]");
    const pa::Desc& d = pool->core.desc();
    const int32_t qdt = pa::is_raw(d.kv_dtype) ? d.kv_dtype : int32_t(pa::kF16);
    *bytes = make_plan(pool, batch, n_q_heads, max_seq_len, qdt, n_query).ws_bytes;
  });
}

pa_status pa_verify_attention(const void* q, const pa_pool* pool, const int32_t* tables,
                              const int32_t* lens, int32_t batch, int32_t n_q_heads,
                              int32_t n_query, int32_t q_dtype, int32_t max_blocks,
                              int32_t max_seq_len, float scale, void* out, void* ws,
                              size_t ws_bytes, void* stream) {
  return decode(kBoth, q, pool, tables, lens, batch, n_q_heads, q_dtype, max_blocks, max_seq_len,
                scale, out, ws, ws_bytes, stream, n_query);
}

pa_status pa_verify_split(const void* q, const pa_pool* pool, const int32_t* tables,
                          const int32_t* lens, int32_t batch, int32_t n_q_heads, int32_t n_query,
                          int32_t q_dtype, int32_t max_blocks, int32_t max_seq_len, float scale,
                          void* out, void* ws, size_t ws_bytes, void* stream) {
  return decode(kSplit, q, pool, tables, lens, batch, n_q_heads, q_dtype, max_blocks, max_seq_len,
                scale, out, ws, ws_bytes, stream, n_query);
}

pa_status pa_verify_combine(const void* q, const pa_pool* pool, const int32_t* tables,
                            const int32_t* lens, int32_t batch, int32_t n_q_heads, int32_t n_query,
                            int32_t q_dtype, int32_t max_blocks, int32_t max_seq_len, float scale,
                            void* out, void* ws, size_t ws_bytes, void* stream) {
  return decode(kCombine, q, pool, tables, lens, batch, n_q_heads, q_dtype, max_blocks, max_seq_len,
                scale, out, ws, ws_bytes, stream, n_query);
}

pa_status pa_prefill_workspace_bytes(const pa_pool* pool, int32_t batch, int32_t n_q_heads,
                                     int32_t chunk, int32_t max_seq_len, size_t* bytes) {
  return guard([&] {
    check_shapes(pool, batch, n_q_heads, max_seq_len);
    need(bytes, "bytes");
    if (chunk < 1 || chunk > kMaxQueries) fail(pa::kInvalidArg, "chunk must be in [1, 4096]");
    const pa::Desc& d = pool->core.desc();
    const int32_t qdt = pa::is_raw(d.kv_dtype) ? d.kv_dtype : int32_t(pa::kF16);
    const Plan pl = make_plan(pool, batch, n_q_heads, max_seq_len, qdt, chunk);
    *bytes = prefill_tile(pool, pl) ? 0 : pl.ws_bytes;
  });
}

pa_status pa_prefill_attention(const void* q, const pa_pool* pool, const int32_t* tables,
                               const int32_t* lens, int32_t batch, int32_t n_q_heads,
                               int32_t chunk, int32_t q_dtype, int32_t max_blocks,
                               int32_t max_seq_len, float scale, void* out, void* ws,
                               size_t ws_bytes, void* stream) {
  return decode(kBoth, q, pool, tables, lens, batch, n_q_heads, q_dtype, max_blocks, max_seq_len,
                scale, out, ws, ws_bytes, stream, chunk, true);
}

pa_status pa_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
  return guard([&] {
    need(src, "src");
    need(sink, "sink");
    if (bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16)
      fail(pa::kInvalidArg, "src must be 16-byte aligned and bytes a multiple of 16");
    if (bytes == 0) return;
    check_hip(pa::launch_stream_read(src, bytes, sink, cu_count() * 8, static_cast<hipStream_t>(stream)),
              "stream read launch");
  });
}

pa_status pa_paged_read(const pa_pool* pool, const int32_t* tables, const int32_t* lens, int32_t batch,
                        int32_t max_blocks, int32_t max_seq_len, void* sink, void* stream) {
  return guard([&] {
    need_device(pool);
    const pa::Desc& d = pool->core.desc();
    if (batch < 0 || batch > 65535) fail(pa::kInvalidArg, "batch must be in [0, 65535]");
    if (max_seq_len < 0) fail(pa::kInvalidArg, "negative max_seq_len");
    if (max_blocks < 1) fail(pa::kInvalidArg, "max_blocks_per_seq must be >= 1");
    if (int64_t(max_seq_len) > int64_t(max_blocks) * d.block_size)
      fail(pa::kInvalidArg, "max_seq_len exceeds block_size * max_blocks_per_seq");
    if (batch == 0) return;
    need(tables, "block_tables_dev");
    need(lens, "seq_lens_dev");
    need(sink, "sink");
    if (!pa::paged_read_supported(dev_view(pool)))
      fail(pa::kUnsupported, "the paged read covers head_dim 128 pools (16-bit, INT4, FP8)");
    if (int64_t(batch) * max_blocks * d.n_kv_heads >= (int64_t(1) << 31))
      fail(pa::kUnsupported, "batch * max_blocks_per_seq * n_kv_heads too large for the paged read");
    check_hip(pa::launch_paged_read(dev_view(pool), tables, lens, batch, max_blocks, max_seq_len, sink,
                                    cu_count() * 2, static_cast<hipStream_t>(stream)),
              "paged read launch");
  });
}

const char* pa_last_error(void) { return g_err.c_str(); }

}  // extern "C"
