"""The allocation-free decode entry point (GPU, through the C ABI).

pa_decode_attention_noalloc runs the kernels of pa_decode_attention with its
workspace in the library's static device array: on the same inputs its rows
must be bit-identical to pa_decode_attention's (same kernels, same cut of the
work list) and within the oracle's bar.  Two or more calls run back to back
on one GPU, each later one smaller, so a call that depended on what the
previous call left in the shared array would show it.
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_18_amd import binding as B
from paged_kv_cache_18_amd import workloads as W
from paged_kv_cache_18_amd.session import PagedKV

from _ref import TORCH_DT, assert_close, expected

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _inputs(wl):
    kv = PagedKV(wl, DEV)
    kv.replay()
    tdev, ldev, t, l = kv.device_tables()
    q = torch.from_numpy(wl.q()).to(TORCH_DT[wl.q_dtype]).to(DEV)
    return kv, tdev, ldev, q, int(max(l.max(), 1))


def _both(wl):
    """(rows of pa_decode_attention, rows of the no-alloc call) as float64."""
    kv, tdev, ldev, q, ml = _inputs(wl)
    bq, hq, d = q.shape
    need = B.pa_decode_workspace_bytes(kv.pool, bq, hq, ml)
    assert need <= B.PA_NOALLOC_SCRATCH_BYTES
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=DEV)
    ref = torch.empty_like(q)
    B.pa_decode_attention(q, kv.pool, tdev, ldev, bq, hq, wl.q_dtype, tdev.shape[1], ml, wl.scale,
                          ref, ws, ws.numel(), kv.stream())
    out = torch.full((bq + 1, hq, d), 7.0, dtype=q.dtype, device=DEV)
    B.pa_decode_attention_noalloc(q, kv.pool, tdev, ldev, bq, hq, wl.q_dtype, tdev.shape[1], ml,
                                  wl.scale, out[:bq], kv.stream())
    torch.cuda.synchronize()
    assert torch.all(out[bq] == 7.0), "write past out"
    res = ref.double().cpu().numpy(), out[:bq].double().cpu().numpy()
    kv.close()
    return res


# each entry: a sequence of workloads run back to back, every later one smaller
SEQUENCES = {
    "bf16": [W.from_lengths([900, 33, 2000, 1, 517, 0, 3000], 32, 8, 128, "bf16", seed=201),
             W.from_lengths([40, 3], 32, 8, 128, "bf16", seed=202)],
    "int4-fp8": [W.from_lengths([3000, 17, 700], 32, 8, 128, "int4", seed=203, group=128, sink=True,
                                outliers=True),
                 W.from_lengths([300, 16], 32, 8, 128, "fp8", seed=204, sink=True)],
    "generic-f32": [W.from_lengths([300, 45, 1000], 4, 4, 64, "f32", seed=205),
                    W.from_lengths([25, 47], 4, 4, 64, "f32", seed=206)],
}


@pytest.mark.parametrize("name", sorted(SEQUENCES))
def test_noalloc_matches_workspace_entry_point(name):
    for i, wl in enumerate(SEQUENCES[name]):
        print(f"[gpu] noalloc {name} call {i}: lens {wl.extra['lengths']} kv={wl.kv_dtype}", flush=True)
        ref, got = _both(wl)
        assert np.array_equal(got, ref), f"{name} call {i}: rows differ from pa_decode_attention"
        odt = "f32" if wl.q_dtype == "f32" else wl.q_dtype
        assert_close(got, expected(wl), odt, f"noalloc {name} call {i}")


def test_noalloc_merge_launch_mode(monkeypatch):
    """Segments merged by the second launch (many pieces per segment): the
    merge jobs and partials live in the static array too."""
    monkeypatch.setenv("PA_FUSE_MAX_PIECES", "1")
    for i, wl in enumerate([W.from_lengths([5000, 1, 2500], 32, 8, 128, "bf16", seed=207),
                            W.from_lengths([700, 20], 32, 8, 128, "bf16", seed=208)]):
        print(f"[gpu] noalloc merge launch call {i}", flush=True)
        ref, got = _both(wl)
        assert np.array_equal(got, ref), f"merge launch call {i}"
        assert_close(got, expected(wl), "bf16", f"noalloc merge launch call {i}")


def test_noalloc_refuses_shapes_above_the_scratch():
    """A shape whose workspace exceeds the static array is refused before any
    device work (the generic kernel's per-sequence splits of one very long
    fp32 sequence with 16 query heads)."""
    wl = W.from_lengths([40], 16, 1, 128, "f32", seed=209)
    kv, tdev, ldev, q, _ = _inputs(wl)
    ml = 1 << 20
    need = B.pa_decode_workspace_bytes(kv.pool, 1, 16, ml)
    assert need > B.PA_NOALLOC_SCRATCH_BYTES
    tables = torch.full((1, ml // 16), -1, dtype=torch.int32, device=DEV)
    tables[0, :tdev.shape[1]] = tdev[0]
    out = torch.full_like(q, 7.0)
    with pytest.raises(B.PaError) as e:
        B.pa_decode_attention_noalloc(q, kv.pool, tables, ldev, 1, 16, "f32", ml // 16, ml,
                                      wl.scale, out, kv.stream())
    assert e.value.code == "INVALID_ARG" and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    kv.close()
