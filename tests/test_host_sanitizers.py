"""The library's host core (csrc/pa_host.cpp: LIFO allocator, refcounts,
copy-on-write, sequences, window settle, prefix cache) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

The refcount guards and the all-or-nothing refusals are this build's own
additions to the pool sketch of "A Ideia de 60 Anos Que Domou a Memoria da
GPU" ("o codigo": rent pops, return pushes at a zero count), so they are
exercised here with every kind of op log the ABI tests use (random logs full
of refused calls, speculative steps with rollback, window settles, prefix
cache traffic, the workloads).  tests/host_replay.cpp replays a log through
the core built with g++ -fsanitize=address,undefined (no HIP involved); the
run must end cleanly (any sanitizer report aborts it) and its per-op results
and final state must equal what the library returns through its C ABI for
the same log (which tests/test_lib_host.py pins against the oracle).
"""

import os
import random
import shutil
import subprocess

import numpy as np
import pytest

from paged_kv_cache_18_amd import binding as B
from paged_kv_cache_18_amd import workloads as W
from paged_kv_cache_18_amd.session import PagedKV

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "paged_kv_cache_18_amd", "csrc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=1:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


@pytest.fixture(scope="module")
def replayer(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("san") / "host_replay")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-I", CSRC,
           os.path.join(HERE, "host_replay.cpp"), os.path.join(CSRC, "pa_host.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def _log_text(wl, ops):
    d = B.make_desc(wl.n_kv_heads, wl.head_dim, wl.kv_dtype, wl.num_blocks,
                    group_size=wl.group_size, num_sink_blocks=wl.num_sink_blocks,
                    sink_blocks_per_seq=wl.sink_blocks_per_seq, window_tokens=wl.window_tokens,
                    block_size=wl.block_size)
    lines = [f"desc {d.block_size} {d.n_kv_heads} {d.head_dim} {d.kv_dtype} {d.group_size} "
             f"{d.num_blocks} {d.num_sink_blocks} {d.sink_blocks_per_seq} {d.window_tokens}"]
    for tag, order in (("body", wl.body_free_order), ("sink", wl.sink_free_order)):
        order = [] if order is None else [int(x) for x in order]
        lines.append(f"{tag} {len(order)} " + " ".join(map(str, order)))
    for op in ops:
        k, a = op[0], op[1:]
        if k == "prefix_lookup":
            lines.append(f"plookup {len(a[0])} " + " ".join(map(str, a[0])))
        elif k == "prefix_register":
            lines.append(f"pregister {a[0]} {len(a[1])} " + " ".join(map(str, a[1])))
        elif k == "prefix_evict":
            lines.append(f"pevict {a[0]}")
        else:
            lines.append(" ".join([k] + [str(int(x)) for x in a]))
    return "\n".join(lines) + "\n"


CODES = {v: k for k, v in B.STATUS_NAMES.items()}


def _lib_lines(wl, ops):
    """The same log through the library's C ABI, printed in the replayer's format."""
    kv = PagedKV(wl, device=None)
    res = kv.replay(ops, write=False)
    out = []
    for r in res:
        if isinstance(r, tuple) and len(r) == 2 and r[0] == "error":
            out.append(f"err {CODES[r[1]]}")
        elif r is None:
            out.append("ok")
        elif isinstance(r, (list, tuple, np.ndarray)):
            out.append("ok " + " ".join(str(int(x)) for x in r))
        else:
            out.append(f"ok {int(r)}")
    n_total = wl.num_blocks + wl.num_sink_blocks
    out.append("ref " + " ".join(str(B.pa_refcount(kv.pool, i)) for i in range(n_total)))
    out.append("free0 " + " ".join(map(str, B.pa_free_list(kv.pool, B.PA_ARENA_BODY))))
    out.append("free1 " + " ".join(map(str, B.pa_free_list(kv.pool, B.PA_ARENA_SINK))))
    out.append(f"clones {B.pa_num_clones(kv.pool)}")
    e, h, a = B.pa_prefix_stats(kv.pool)
    out.append(f"prefix {e} {h} {a}")
    for sid in range(max(_created(res, ops), default=-1) + 1):
        try:
            ln, nb = B.pa_seq_info(kv.pool, sid)
        except B.PaError:
            out.append(f"seq {sid} released")
            continue
        t, _ = B.pa_block_tables(kv.pool, [sid], max(nb, 1))
        out.append(f"seq {sid} {ln}" + "".join(f" {int(x)}" for x in t[0, :nb]))
    kv.close()
    return out


def _created(res, ops):
    """Sequence ids handed out by the log (create, fork, prefix lookup)."""
    ids = []
    for r, op in zip(res, ops):
        if isinstance(r, tuple) and r and r[0] == "error":
            continue
        if op[0] in ("create", "fork"):
            ids.append(int(r))
        elif op[0] == "prefix_lookup":
            ids.append(int(r[0]))
    return ids


def _check(replayer, wl, ops):
    r = subprocess.run([replayer], input=_log_text(wl, ops), capture_output=True, text=True,
                       env=dict(os.environ, **SAN_ENV), timeout=120)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    got = [" ".join(ln.split()) for ln in r.stdout.splitlines()]
    want = [" ".join(ln.split()) for ln in _lib_lines(wl, ops)]
    assert got == want


def _random_ops(rnd, n, n_blocks, sink):
    ops, nseq = [], 0
    for _ in range(n):
        k = rnd.randrange(9)
        if k == 0 or nseq == 0:
            ops.append(("create",))
            nseq += 1
        elif k == 1:
            ops.append(("reserve", rnd.randrange(nseq + 1), rnd.randrange(-1, 40)))
        elif k == 2:
            ops.append(("fork", rnd.randrange(nseq + 1)))
            nseq += 1
        elif k == 3:
            ops.append(("release", rnd.randrange(nseq + 1)))
        elif k == 4:
            ops.append(("truncate", rnd.randrange(nseq + 1), rnd.randrange(-1, 30)))
        elif k == 5:
            ops.append(("alloc", rnd.choice([0, 1] if sink else [0, 0, 2])))
        elif k == 6:
            ops.append(("free", rnd.randrange(-1, n_blocks + 1)))
        elif k == 7:
            ops.append(("incref", rnd.randrange(-1, n_blocks + 1)))
        else:
            ops.append(("clone", rnd.randrange(-1, n_blocks + 1)))
    return ops


@pytest.mark.parametrize("seed", range(16))
def test_random_logs_under_sanitizers(replayer, seed):
    """Random logs, most ops refused (bad ids, double frees, refcount
    underflow, exhausted arenas): every refusal leaves the state unchanged."""
    rnd = random.Random(300 + seed)
    sink = seed % 3 == 0
    nb, ns = 10, (3 if sink else 0)
    wl = W.tiny()
    wl.num_blocks = nb
    wl.body_free_order = np.array(rnd.sample(range(nb), nb))
    if sink:
        wl.kv_dtype, wl.group_size = "int4", 64
        wl.num_sink_blocks, wl.sink_blocks_per_seq = ns, 1
        wl.sink_free_order = np.array(rnd.sample(range(ns), ns))
    _check(replayer, wl, _random_ops(rnd, 200, nb + ns, sink))


@pytest.mark.parametrize("seed", range(4))
def test_speculative_and_window_logs_under_sanitizers(replayer, seed):
    """Speculative steps (reserve gamma + 1, truncate the rejected tail) and
    window pools (reserve routing, settle, forks, truncation)."""
    rnd = random.Random(400 + seed)
    wl = W.window_batch([rnd.randrange(1, 90) for _ in range(3)], steps=3, window=32)
    ops = list(wl.ops)
    nseq = 3
    for _ in range(120):
        k = rnd.randrange(6)
        s_ = rnd.randrange(nseq + 1)
        if k == 0:
            ops.append(("reserve", s_, rnd.choice([1, 1, 2, 6, 15, 33, 200])))
        elif k == 1:
            ops.append(("settle", s_))
        elif k == 2:
            ops.append(("fork", s_))
            nseq += 1
        elif k == 3:
            ops.append(("truncate", s_, rnd.randrange(0, 120)))
        elif k == 4:
            ops.append(("reserve", s_, 6))
            ops.append(("truncate", s_, rnd.randrange(0, 200)))
        else:
            ops.append(("release", s_))
    _check(replayer, wl, ops)


@pytest.mark.parametrize("seed", range(4))
def test_prefix_cache_logs_under_sanitizers(replayer, seed):
    """Lookups, prefills, registrations, releases and evictions over a few
    prompt families."""
    rnd = random.Random(500 + seed)
    nb = 48
    wl = W.tiny()
    wl.num_blocks = nb
    wl.body_free_order = np.array(rnd.sample(range(nb), nb))
    kv = PagedKV(wl, device=None)        # drives the log so reserves fit the lookups
    bases = [[rnd.randrange(50) for _ in range(rnd.randrange(16, 90))] for _ in range(3)]
    live, ops = {}, []
    for _ in range(200):
        k = rnd.randrange(6)
        if k <= 1 or not live:
            ids = rnd.choice(bases)[:rnd.randrange(0, 90)] + [rnd.randrange(50)
                                                              for _ in range(rnd.randrange(0, 30))]
            op = ("prefix_lookup", ids)
        elif k == 2:
            sid = rnd.choice(list(live))
            op = ("reserve", sid, len(live[sid]) - B.pa_seq_info(kv.pool, sid)[0])
        elif k == 3:
            sid = rnd.choice(list(live))
            op = ("prefix_register", sid, live[sid])
        elif k == 4:
            sid = rnd.choice(list(live))
            op = ("release", sid)
        else:
            op = ("prefix_evict", rnd.randrange(0, 6))
        r = kv.replay([op], write=False)[0]
        ops.append(op)
        if op[0] == "prefix_lookup":
            live[r[0]] = op[1]
        elif op[0] == "release" and not (isinstance(r, tuple) and r[0] == "error"):
            del live[op[1]]
    kv.close()
    _check(replayer, wl, ops)


@pytest.mark.parametrize("name,kw", [
    ("llama3-8b", {"batch": 16, "min_len": 1, "max_len": 700}),
    ("shared-prefix-partial", {"n_children": 8, "max_suffix": 60}),
    ("mixed-window", {"length": 300, "steps": 40}),
    ("llama3-8b-bs8", {"batch": 16, "min_len": 1, "max_len": 300}),
])
def test_workload_logs_under_sanitizers(replayer, name, kw):
    wl = W.by_name(name, **kw)
    _check(replayer, wl, list(wl.ops))
