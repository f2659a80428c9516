"""Thin ctypes binding of libpa (include/pa.h), same names as the C calls.

Argument marshalling only: every computation happens in the library.  Device
buffers are passed as integers (device pointers) or as objects with a
``data_ptr()`` method (torch tensors); streams as integers (hipStream_t
handles, e.g. ``torch.cuda.current_stream().cuda_stream``) or None for the
default stream.  A non-OK status raises ``PaError`` carrying the status and
``pa_last_error()``.  The library is loaded on first use; if it has not been
built the call raises: there is no CPU fallback.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_OUT_OF_BLOCKS, PA_ERR_REFCOUNT = 0, 1, 2, 3
PA_ERR_BAD_ID, PA_ERR_UNSUPPORTED, PA_ERR_HIP = 4, 5, 6
STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "OUT_OF_BLOCKS", 3: "REFCOUNT", 4: "BAD_ID",
                5: "UNSUPPORTED", 6: "HIP"}
PA_F32, PA_F16, PA_BF16, PA_INT4_ASYM, PA_FP8_E4M3 = 0, 1, 2, 3, 4
DTYPES = {"f32": PA_F32, "f16": PA_F16, "bf16": PA_BF16, "int4": PA_INT4_ASYM, "fp8": PA_FP8_E4M3}
PA_ARENA_BODY, PA_ARENA_SINK = 0, 1
ARRAYS = ["K", "V", "KS", "KZ", "VS", "VZ", "SK", "SV"]
NUM_ARR = 8
SIZE_MAX = (1 << 64) - 1

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

i32, i64, sz, vp, f32 = C.c_int32, C.c_int64, C.c_size_t, C.c_void_p, C.c_float
P32 = C.POINTER(C.c_int32)


class pa_pool_desc(C.Structure):
    _fields_ = [("block_size", i32), ("n_kv_heads", i32), ("head_dim", i32), ("kv_dtype", i32),
                ("group_size", i32), ("num_blocks", i32), ("num_sink_blocks", i32),
                ("sink_blocks_per_seq", i32), ("window_tokens", i32)]


class pa_layout(C.Structure):
    _fields_ = [("total_bytes", sz), ("offset", sz * NUM_ARR), ("slab_bytes", sz * NUM_ARR)]


class PaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status
        self.code = STATUS_NAMES.get(status, str(status))


_lib = None

_DECODE_ARGS = [vp, vp, P32, P32, i32, i32, i32, i32, i32, f32, vp, vp, sz, vp]
_PROTOS = {
    "pa_pool_bytes": [C.POINTER(pa_pool_desc), C.POINTER(sz)],
    "pa_pool_create": [C.POINTER(pa_pool_desc), vp, sz, P32, P32, C.POINTER(vp)],
    "pa_pool_destroy": [vp],
    "pa_pool_layout": [vp, C.POINTER(pa_layout)],
    "pa_alloc_block": [vp, i32, P32],
    "pa_incref": [vp, i32],
    "pa_free_block": [vp, i32],
    "pa_cow_clone": [vp, i32, P32, vp],
    "pa_refcount": [vp, i32, P32],
    "pa_num_free": [vp, i32, P32],
    "pa_free_list": [vp, i32, P32, i32, P32],
    "pa_num_clones": [vp, C.POINTER(i64)],
    "pa_seq_create": [vp, P32],
    "pa_seq_fork": [vp, i32, P32],
    "pa_seq_reserve": [vp, i32, i32, P32, vp],
    "pa_seq_truncate": [vp, i32, i32],
    "pa_prefix_lookup": [vp, P32, i32, C.POINTER(i32), C.POINTER(i32)],
    "pa_prefix_register": [vp, i32, P32, i32, C.POINTER(i32)],
    "pa_prefix_evict": [vp, i32, C.POINTER(i32)],
    "pa_prefix_stats": [vp, C.POINTER(i32), C.POINTER(i64), C.POINTER(i64)],
    "pa_prefix_block_hashes": [P32, i32, C.POINTER(C.c_uint64)],
    "pa_seq_release": [vp, i32],
    "pa_seq_info": [vp, i32, P32, P32],
    "pa_block_tables": [vp, P32, i32, i32, P32, P32],
    "pa_append_kv": [vp, vp, vp, i32, P32, i32, vp],
    "pa_decode_workspace_bytes": [vp, i32, i32, i32, C.POINTER(sz)],
    "pa_decode_split_blocks": [vp, i32, i32, i32, P32],
    "pa_stream_read": [vp, sz, vp, vp],
    "pa_paged_read": [vp, P32, P32, i32, i32, i32, vp, vp],
    "pa_seq_settle": [vp, i32, vp, P32],
    "pa_decode_attention": _DECODE_ARGS,
    "pa_decode_attention_noalloc": [vp, vp, P32, P32, i32, i32, i32, i32, i32, f32, vp, vp],
    "pa_verify_workspace_bytes": [vp, i32, i32, i32, i32, C.POINTER(sz)],
    "pa_verify_attention": [vp, vp, P32, P32, i32, i32, i32, i32, i32, i32, f32, vp, vp, sz, vp],
    "pa_verify_split": [vp, vp, P32, P32, i32, i32, i32, i32, i32, i32, f32, vp, vp, sz, vp],
    "pa_verify_combine": [vp, vp, P32, P32, i32, i32, i32, i32, i32, i32, f32, vp, vp, sz, vp],
    "pa_prefill_workspace_bytes": [vp, i32, i32, i32, i32, C.POINTER(sz)],
    "pa_prefill_attention": [vp, vp, P32, P32, i32, i32, i32, i32, i32, i32, f32, vp, vp, sz, vp],
    "pa_decode_split": _DECODE_ARGS,
    "pa_decode_combine": _DECODE_ARGS,
    "pa_decode_step": [vp, vp, vp, i32] + _DECODE_ARGS[1:],
    "pa_decode_step_split": [vp, vp, vp, i32] + _DECODE_ARGS[1:],
}
EXPORTS = sorted(list(_PROTOS) + ["pa_last_error"])


def lib():
    """Load libpa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_kv_cache_18_amd.build` (no CPU fallback exists)")
        L = C.CDLL(LIB_PATH)
        for name, args in _PROTOS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = i32
        L.pa_last_error.argtypes = []
        L.pa_last_error.restype = C.c_char_p
        _lib = L
    return _lib


def _check(st):
    if st != PA_OK:
        raise PaError(st, lib().pa_last_error().decode())


def _ptr(x):
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return C.c_void_p(x.data_ptr())
    return C.c_void_p(int(x))


def _i32ptr(x):
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return C.cast(C.c_void_p(x.data_ptr()), P32)
    return C.cast(C.c_void_p(int(x)), P32)


def _host_i32(arr):
    a = np.ascontiguousarray(np.asarray(arr, dtype=np.int32))
    return a, a.ctypes.data_as(P32)


def make_desc(n_kv_heads, head_dim, kv_dtype, num_blocks, group_size=0, num_sink_blocks=0,
              sink_blocks_per_seq=0, block_size=16, window_tokens=0):
    kv = DTYPES[kv_dtype] if isinstance(kv_dtype, str) else int(kv_dtype)
    return pa_pool_desc(block_size, n_kv_heads, head_dim, kv, group_size, num_blocks,
                        num_sink_blocks, sink_blocks_per_seq, window_tokens)


# ---- pool ---------------------------------------------------------------------------
def pa_pool_bytes(desc):
    out = sz()
    _check(lib().pa_pool_bytes(C.byref(desc), C.byref(out)))
    return out.value


def pa_pool_create(desc, dev_mem, dev_bytes, body_free_order=None, sink_free_order=None):
    keep = []
    bo = so = None
    if body_free_order is not None:
        a, bo = _host_i32(body_free_order)
        keep.append(a)
    if sink_free_order is not None:
        a, so = _host_i32(sink_free_order)
        keep.append(a)
    out = vp()
    _check(lib().pa_pool_create(C.byref(desc), _ptr(dev_mem), dev_bytes,
                                bo, so, C.byref(out)))
    return out.value


def pa_pool_destroy(pool):
    _check(lib().pa_pool_destroy(pool))


def pa_pool_layout(pool):
    out = pa_layout()
    _check(lib().pa_pool_layout(pool, C.byref(out)))
    offs = {ARRAYS[i]: out.offset[i] for i in range(NUM_ARR) if out.offset[i] != SIZE_MAX}
    slabs = {ARRAYS[i]: out.slab_bytes[i] for i in range(NUM_ARR) if out.offset[i] != SIZE_MAX}
    return {"total_bytes": out.total_bytes, "offset": offs, "slab_bytes": slabs}


# ---- blocks -------------------------------------------------------------------------
def pa_alloc_block(pool, arena=PA_ARENA_BODY):
    out = i32()
    _check(lib().pa_alloc_block(pool, arena, C.byref(out)))
    return out.value


def pa_incref(pool, bid):
    _check(lib().pa_incref(pool, bid))


def pa_free_block(pool, bid):
    _check(lib().pa_free_block(pool, bid))


def pa_cow_clone(pool, src, stream=None):
    out = i32()
    _check(lib().pa_cow_clone(pool, src, C.byref(out), _ptr(stream)))
    return out.value


def pa_refcount(pool, bid):
    out = i32()
    _check(lib().pa_refcount(pool, bid, C.byref(out)))
    return out.value


def pa_num_free(pool, arena=PA_ARENA_BODY):
    out = i32()
    _check(lib().pa_num_free(pool, arena, C.byref(out)))
    return out.value


def pa_free_list(pool, arena=PA_ARENA_BODY):
    n = pa_num_free(pool, arena)
    buf = np.zeros(max(n, 1), dtype=np.int32)
    got = i32()
    _check(lib().pa_free_list(pool, arena, buf.ctypes.data_as(P32), n, C.byref(got)))
    return buf[:got.value].tolist()


def pa_num_clones(pool):
    out = i64()
    _check(lib().pa_num_clones(pool, C.byref(out)))
    return out.value


# ---- sequences ------------------------------------------------------------------------
def pa_seq_create(pool):
    out = i32()
    _check(lib().pa_seq_create(pool, C.byref(out)))
    return out.value


def pa_seq_fork(pool, parent):
    out = i32()
    _check(lib().pa_seq_fork(pool, parent, C.byref(out)))
    return out.value


def pa_seq_reserve(pool, seq, n_tokens, stream=None):
    buf = np.zeros(max(n_tokens, 1), dtype=np.int32)
    _check(lib().pa_seq_reserve(pool, seq, n_tokens, buf.ctypes.data_as(P32), _ptr(stream)))
    return buf[:n_tokens]


def pa_seq_truncate(pool, seq, new_len):
    _check(lib().pa_seq_truncate(pool, seq, new_len))


# ---- block-hash prefix cache --------------------------------------------------------
def _ids(token_ids):
    a = np.ascontiguousarray(np.asarray(token_ids, dtype=np.int32))
    return a, a.ctypes.data_as(P32)


def pa_prefix_lookup(pool, token_ids):
    """New sequence on the longest cached prefix; returns (seq, cached tokens)."""
    a, p = _ids(token_ids)
    sid, n = i32(), i32()
    _check(lib().pa_prefix_lookup(pool, p, a.size, C.byref(sid), C.byref(n)))
    return sid.value, n.value


def pa_prefix_register(pool, seq, token_ids):
    a, p = _ids(token_ids)
    n = i32()
    _check(lib().pa_prefix_register(pool, seq, p, a.size, C.byref(n)))
    return n.value


def pa_prefix_evict(pool, max_blocks):
    n = i32()
    _check(lib().pa_prefix_evict(pool, max_blocks, C.byref(n)))
    return n.value


def pa_prefix_stats(pool):
    e, h, a = i32(), i64(), i64()
    _check(lib().pa_prefix_stats(pool, C.byref(e), C.byref(h), C.byref(a)))
    return e.value, h.value, a.value


def pa_prefix_block_hashes(token_ids):
    a, p = _ids(token_ids)
    out = np.zeros(max(a.size // 16, 1), dtype=np.uint64)
    _check(lib().pa_prefix_block_hashes(p, a.size, out.ctypes.data_as(C.POINTER(C.c_uint64))))
    return out[:a.size // 16]


def pa_seq_release(pool, seq):
    _check(lib().pa_seq_release(pool, seq))


def pa_seq_info(pool, seq):
    ln, nb = i32(), i32()
    _check(lib().pa_seq_info(pool, seq, C.byref(ln), C.byref(nb)))
    return ln.value, nb.value


def pa_block_tables(pool, seqs, max_blocks):
    s, sp = _host_i32(seqs)
    n = len(s)
    tables = np.zeros((max(n, 1), max(max_blocks, 1)), dtype=np.int32)
    lens = np.zeros(max(n, 1), dtype=np.int32)
    _check(lib().pa_block_tables(pool, sp, n, max_blocks, tables.ctypes.data_as(P32),
                                 lens.ctypes.data_as(P32)))
    return tables[:n, :max_blocks], lens[:n]


# ---- device work -------------------------------------------------------------------------
def pa_append_kv(pool, k, v, in_dtype, slots_dev, n_tokens, stream=None):
    dt = DTYPES[in_dtype] if isinstance(in_dtype, str) else int(in_dtype)
    _check(lib().pa_append_kv(pool, _ptr(k), _ptr(v), dt, _i32ptr(slots_dev), n_tokens, _ptr(stream)))


def pa_decode_workspace_bytes(pool, batch, n_q_heads, max_seq_len):
    out = sz()
    _check(lib().pa_decode_workspace_bytes(pool, batch, n_q_heads, max_seq_len, C.byref(out)))
    return out.value


def pa_decode_split_blocks(pool, batch, n_q_heads, max_seq_len):
    out = i32()
    _check(lib().pa_decode_split_blocks(pool, batch, n_q_heads, max_seq_len, C.byref(out)))
    return out.value


def _decode(fn, q, pool, tables_dev, lens_dev, batch, n_q_heads, q_dtype, max_blocks, max_seq_len,
            scale, out, workspace, workspace_bytes, stream):
    dt = DTYPES[q_dtype] if isinstance(q_dtype, str) else int(q_dtype)
    _check(fn(_ptr(q), pool, _i32ptr(tables_dev), _i32ptr(lens_dev), batch, n_q_heads, dt,
              max_blocks, max_seq_len, scale, _ptr(out), _ptr(workspace), workspace_bytes,
              _ptr(stream)))


def pa_decode_attention(q, pool, tables_dev, lens_dev, batch, n_q_heads, q_dtype, max_blocks,
                        max_seq_len, scale, out, workspace, workspace_bytes, stream=None):
    _decode(lib().pa_decode_attention, q, pool, tables_dev, lens_dev, batch, n_q_heads, q_dtype,
            max_blocks, max_seq_len, scale, out, workspace, workspace_bytes, stream)


# bytes of the library's static scratch (include/pa.h, PA_NOALLOC_SCRATCH_BYTES)
PA_NOALLOC_SCRATCH_BYTES = 32 << 20


def pa_decode_attention_noalloc(q, pool, tables_dev, lens_dev, batch, n_q_heads, q_dtype,
                                max_blocks, max_seq_len, scale, out, stream=None):
    dt = DTYPES[q_dtype] if isinstance(q_dtype, str) else int(q_dtype)
    _check(lib().pa_decode_attention_noalloc(_ptr(q), pool, _i32ptr(tables_dev), _i32ptr(lens_dev),
                                             batch, n_q_heads, dt, max_blocks, max_seq_len, scale,
                                             _ptr(out), _ptr(stream)))


def _step(fn, q, k_new, v_new, in_dtype, pool, tables_dev, lens_dev, batch, n_q_heads, q_dtype,
          max_blocks, max_seq_len, scale, out, workspace, workspace_bytes, stream):
    dt = DTYPES[q_dtype] if isinstance(q_dtype, str) else int(q_dtype)
    idt = DTYPES[in_dtype] if isinstance(in_dtype, str) else int(in_dtype)
    _check(fn(_ptr(q), _ptr(k_new), _ptr(v_new), idt, pool, _i32ptr(tables_dev), _i32ptr(lens_dev),
              batch, n_q_heads, dt, max_blocks, max_seq_len, scale, _ptr(out), _ptr(workspace),
              workspace_bytes, _ptr(stream)))


def pa_decode_step(q, k_new, v_new, in_dtype, pool, tables_dev, lens_dev, batch, n_q_heads, q_dtype,
                   max_blocks, max_seq_len, scale, out, workspace, workspace_bytes, stream=None):
    _step(lib().pa_decode_step, q, k_new, v_new, in_dtype, pool, tables_dev, lens_dev, batch,
          n_q_heads, q_dtype, max_blocks, max_seq_len, scale, out, workspace, workspace_bytes, stream)


def pa_decode_step_split(q, k_new, v_new, in_dtype, pool, tables_dev, lens_dev, batch, n_q_heads,
                         q_dtype, max_blocks, max_seq_len, scale, out, workspace, workspace_bytes,
                         stream=None):
    _step(lib().pa_decode_step_split, q, k_new, v_new, in_dtype, pool, tables_dev, lens_dev, batch,
          n_q_heads, q_dtype, max_blocks, max_seq_len, scale, out, workspace, workspace_bytes, stream)


def pa_decode_split(q, pool, tables_dev, lens_dev, batch, n_q_heads, q_dtype, max_blocks,
                    max_seq_len, scale, out, workspace, workspace_bytes, stream=None):
    _decode(lib().pa_decode_split, q, pool, tables_dev, lens_dev, batch, n_q_heads, q_dtype,
            max_blocks, max_seq_len, scale, out, workspace, workspace_bytes, stream)


def pa_decode_combine(q, pool, tables_dev, lens_dev, batch, n_q_heads, q_dtype, max_blocks,
                      max_seq_len, scale, out, workspace, workspace_bytes, stream=None):
    _decode(lib().pa_decode_combine, q, pool, tables_dev, lens_dev, batch, n_q_heads, q_dtype,
            max_blocks, max_seq_len, scale, out, workspace, workspace_bytes, stream)


def pa_seq_settle(pool, seq, stream=None):
    """Move the sequence's FP16 blocks that left the window into the body;
    returns how many moved."""
    out = i32()
    _check(lib().pa_seq_settle(pool, seq, _ptr(stream), C.byref(out)))
    return out.value


def pa_verify_workspace_bytes(pool, batch, n_q_heads, n_query, max_seq_len):
    out = sz()
    _check(lib().pa_verify_workspace_bytes(pool, batch, n_q_heads, n_query, max_seq_len,
                                           C.byref(out)))
    return out.value


def _verify(fn, q, pool, tables_dev, lens_dev, batch, n_q_heads, n_query, q_dtype, max_blocks,
            max_seq_len, scale, out, workspace, workspace_bytes, stream):
    dt = DTYPES[q_dtype] if isinstance(q_dtype, str) else int(q_dtype)
    _check(fn(_ptr(q), pool, _i32ptr(tables_dev), _i32ptr(lens_dev), batch, n_q_heads, n_query, dt,
              max_blocks, max_seq_len, scale, _ptr(out), _ptr(workspace), workspace_bytes,
              _ptr(stream)))


def pa_verify_attention(q, pool, tables_dev, lens_dev, batch, n_q_heads, n_query, q_dtype,
                        max_blocks, max_seq_len, scale, out, workspace, workspace_bytes,
                        stream=None):
    _verify(lib().pa_verify_attention, q, pool, tables_dev, lens_dev, batch, n_q_heads, n_query,
            q_dtype, max_blocks, max_seq_len, scale, out, workspace, workspace_bytes, stream)


def pa_verify_split(q, pool, tables_dev, lens_dev, batch, n_q_heads, n_query, q_dtype, max_blocks,
                    max_seq_len, scale, out, workspace, workspace_bytes, stream=None):
    _verify(lib().pa_verify_split, q, pool, tables_dev, lens_dev, batch, n_q_heads, n_query,
            q_dtype, max_blocks, max_seq_len, scale, out, workspace, workspace_bytes, stream)


def pa_verify_combine(q, pool, tables_dev, lens_dev, batch, n_q_heads, n_query, q_dtype, max_blocks,
                      max_seq_len, scale, out, workspace, workspace_bytes, stream=None):
    _verify(lib().pa_verify_combine, q, pool, tables_dev, lens_dev, batch, n_q_heads, n_query,
            q_dtype, max_blocks, max_seq_len, scale, out, workspace, workspace_bytes, stream)


def pa_prefill_workspace_bytes(pool, batch, n_q_heads, chunk, max_seq_len):
    out = sz()
    _check(lib().pa_prefill_workspace_bytes(pool, batch, n_q_heads, chunk, max_seq_len,
                                            C.byref(out)))
    return out.value


def pa_prefill_attention(q, pool, tables_dev, lens_dev, batch, n_q_heads, chunk, q_dtype,
                         max_blocks, max_seq_len, scale, out, workspace, workspace_bytes,
                         stream=None):
    dt = DTYPES[q_dtype] if isinstance(q_dtype, str) else int(q_dtype)
    _check(lib().pa_prefill_attention(_ptr(q), pool, _i32ptr(tables_dev), _i32ptr(lens_dev), batch,
                                      n_q_heads, chunk, dt, max_blocks, max_seq_len, scale,
                                      _ptr(out), _ptr(workspace), workspace_bytes, _ptr(stream)))


def pa_stream_read(src, nbytes, sink, stream=None):
    """Measurement aid: stream-read nbytes of device memory at src."""
    _check(lib().pa_stream_read(_ptr(src), nbytes, _ptr(sink), _ptr(stream)))


def pa_paged_read(pool, tables_dev, lens_dev, batch, max_blocks, max_seq_len, sink, stream=None):
    """Measurement aid: read every slab a decode of this batch reads, with no
    arithmetic; sink[0] ^= the XOR of every 32-bit word read."""
    _check(lib().pa_paged_read(pool, _i32ptr(tables_dev), _i32ptr(lens_dev), batch, max_blocks,
                               max_seq_len, _ptr(sink), _ptr(stream)))


def pa_last_error():
    return lib().pa_last_error().decode()
