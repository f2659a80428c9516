"""Drive a workload through libpa: pool memory, op-log replay, K/V upload,
block tables, decode.  Orchestration only; every step of the path runs in the
library (allocator in C++, append/quantize and decode in HIP kernels).

PyTorch provides device memory and the stream.  With ``device=None`` the pool
is metadata-only (no device memory): the allocator, sequences and tables work,
nothing is written.
"""

from __future__ import annotations

import numpy as np

from . import binding as B

_TORCH_DT = {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}


def torch_dtype(name):
    import torch
    return getattr(torch, _TORCH_DT[name])


class PagedKV:
    def __init__(self, wl, device="cuda", body_free_order=None):
        self.wl = wl
        self.device = device
        self.desc = B.make_desc(wl.n_kv_heads, wl.head_dim, wl.kv_dtype, wl.num_blocks,
                                group_size=wl.group_size, num_sink_blocks=wl.num_sink_blocks,
                                sink_blocks_per_seq=wl.sink_blocks_per_seq,
                                window_tokens=wl.window_tokens, block_size=wl.block_size)
        self.pool_bytes = B.pa_pool_bytes(self.desc)
        order = wl.body_free_order if body_free_order is None else body_free_order
        if device is None:
            self.mem = None
            self.pool = B.pa_pool_create(self.desc, None, 0, order, wl.sink_free_order)
        else:
            import torch
            self.mem = torch.empty(self.pool_bytes, dtype=torch.uint8, device=device)
            self.pool = B.pa_pool_create(self.desc, self.mem, self.pool_bytes, order,
                                         wl.sink_free_order)
        self.results = []
        self._tok_cache = {}

    def close(self):
        if self.pool:
            B.pa_pool_destroy(self.pool)
            self.pool = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def stream(self):
        if self.device is None:
            return None
        import torch
        return torch.cuda.current_stream().cuda_stream

    def _tokens(self, sid):
        if sid not in self._tok_cache:
            self._tok_cache = {sid: self.wl.seq_tokens(sid)}  # keep one sequence cached
        return self._tok_cache[sid]

    def write_tokens(self, sid, start, slots):
        """Upload tokens [start, start+len(slots)) of sid and append them."""
        import torch
        n = len(slots)
        if n == 0:
            return
        K, V = self._tokens(sid)
        dt = torch_dtype(self.wl.in_dtype)
        k = torch.from_numpy(np.ascontiguousarray(K[start:start + n])).to(dt).to(self.device)
        v = torch.from_numpy(np.ascontiguousarray(V[start:start + n])).to(dt).to(self.device)
        s = torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int32)).to(self.device)
        B.pa_append_kv(self.pool, k, v, self.wl.in_dtype, s, n, self.stream())

    def replay(self, ops=None, write=True):
        """Run the op log through the library; returns per-op results (or the
        error code a refused op raised)."""
        ops = self.wl.ops if ops is None else ops
        out = []
        for op in ops:
            kind, args = op[0], op[1:]
            try:
                if kind == "create":
                    r = B.pa_seq_create(self.pool)
                elif kind == "reserve":
                    sid, n = args
                    start, _ = B.pa_seq_info(self.pool, sid)
                    r = [int(x) for x in B.pa_seq_reserve(self.pool, sid, n, self.stream())]
                    if write and self.mem is not None:
                        self.write_tokens(sid, start, r)
                elif kind == "fork":
                    r = B.pa_seq_fork(self.pool, *args)
                elif kind == "release":
                    r = B.pa_seq_release(self.pool, *args)
                elif kind == "truncate":
                    r = B.pa_seq_truncate(self.pool, *args)
                elif kind == "alloc":
                    r = B.pa_alloc_block(self.pool, *args)
                elif kind == "incref":
                    r = B.pa_incref(self.pool, *args)
                elif kind == "free":
                    r = B.pa_free_block(self.pool, *args)
                elif kind == "clone":
                    r = B.pa_cow_clone(self.pool, args[0], self.stream())
                elif kind == "settle":
                    r = B.pa_seq_settle(self.pool, args[0], self.stream())
                elif kind == "prefix_lookup":
                    r = B.pa_prefix_lookup(self.pool, args[0])
                elif kind == "prefix_register":
                    r = B.pa_prefix_register(self.pool, args[0], args[1])
                elif kind == "prefix_evict":
                    r = B.pa_prefix_evict(self.pool, args[0])
                else:
                    raise ValueError(kind)
            except B.PaError as e:
                r = ("error", e.code)
            out.append(r)
        self.results = out
        return out

    def tables(self, seqs=None, max_blocks=None):
        seqs = self.wl.decode_seqs if seqs is None else seqs
        if max_blocks is None:
            max_blocks = max([B.pa_seq_info(self.pool, s)[1] for s in seqs] + [1])
        return B.pa_block_tables(self.pool, seqs, max_blocks)

    def device_tables(self, seqs=None, max_blocks=None):
        import torch
        t, l = self.tables(seqs, max_blocks)
        return (torch.from_numpy(np.ascontiguousarray(t)).to(self.device),
                torch.from_numpy(np.ascontiguousarray(l)).to(self.device), t, l)

    def decode(self, q, tables_dev, lens_dev, max_seq_len, out=None, workspace=None,
               phase="both"):
        import torch
        b, hq, d = q.shape
        if out is None:
            out = torch.empty_like(q)
        need = B.pa_decode_workspace_bytes(self.pool, b, hq, max_seq_len)
        if workspace is None:
            workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=self.device)
        fn = {"both": B.pa_decode_attention, "split": B.pa_decode_split,
              "combine": B.pa_decode_combine}[phase]
        fn(q, self.pool, tables_dev, lens_dev, b, hq, self.wl.q_dtype, tables_dev.shape[1],
           max_seq_len, self.wl.scale, out, workspace, workspace.numel(), self.stream())
        return out

    def pool_host_bytes(self):
        return self.mem.cpu().numpy()
