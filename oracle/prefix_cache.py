"""Oracle block-hash prefix cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (Primer chapter 8, section 8.3, "O prefix caching e a
alavanca de maior impacto que o PagedAttention desbloqueia"; 3-minute page,
"Compartilhamento e compromissos"): the prompt is hashed in block-sized
pieces; a piece whose hash is in the global cache of already-computed blocks
is mapped into the new request's block table and its prefill skipped; a
missing piece is prefilled and the resulting block registered.  Requests that
share a prefix thus point at the same physical blocks.

Readings where the pages are silent:

* Key of full block j: FNV-1a 64 over (key of block j-1 as 8 little-endian
  bytes, then the block's 16 token ids as int32 little-endian), the key of
  block -1 being the FNV-1a offset basis -- a chain, so a key names the whole
  prefix.  Only full blocks are cached.
* An entry also keeps its 16 ids and its parent block and is used only when
  both match the request (no false hit on a hash collision).
* The cache holds one reference per entry.  Registration walks the
  sequence's full blocks in order and stops at the first position cached
  under another block.
* Eviction: least recently used first (a hit or a registration is a use),
  among entries with no cached child whose block only the cache holds.
* Pools with a local window are refused: their blocks move between arenas.

FNV-1a 64 is written from its published definition: offset basis
14695981039346656037, prime 1099511628211; per byte, xor then multiply
modulo 2**64.
"""

from __future__ import annotations

from .allocator import PoolError, replay

FNV_OFFSET = 14695981039346656037
FNV_PRIME = 1099511628211
BLOCK = 16


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) % (1 << 64)
    return h


def block_keys(ids) -> list[int]:
    """Chained keys of the full blocks of a token-id sequence."""
    ids = [int(x) for x in ids]
    keys, prev = [], FNV_OFFSET
    for j in range(len(ids) // BLOCK):
        data = prev.to_bytes(8, "little") + b"".join(
            (t % (1 << 32)).to_bytes(4, "little") for t in ids[BLOCK * j:BLOCK * (j + 1)])
        prev = fnv1a64(data)
        keys.append(prev)
    return keys


class PrefixCache:
    """The cache over an oracle Pool (shares its refcounts and sequences)."""

    def __init__(self, pool):
        self.pool = pool
        self.entries: dict[int, dict] = {}
        self.clock = 0
        self.hits = 0
        self.asked = 0

    def _need_pool(self):
        if self.pool.window:
            raise PoolError("UNSUPPORTED", "prefix cache on a pool with a window")

    def lookup(self, ids):
        """New sequence on the longest cached prefix: (sid, cached tokens)."""
        self._need_pool()
        ids = [int(x) for x in ids]
        sid = self.pool.seq_create()
        seq = self.pool.seqs[sid]
        parent = -1
        keys = block_keys(ids)
        for j, key in enumerate(keys):
            e = self.entries.get(key)
            if e is None or e["parent"] != parent or e["ids"] != ids[BLOCK * j:BLOCK * (j + 1)]:
                break
            self.pool.incref(e["block"])
            seq.table.append(e["block"])
            self.clock += 1
            e["stamp"] = self.clock
            parent = e["block"]
        seq.length = BLOCK * len(seq.table)
        self.asked += len(keys)
        self.hits += len(seq.table)
        return sid, seq.length

    def register(self, sid, ids):
        self._need_pool()
        ids = [int(x) for x in ids]
        table, length = self.pool.seq_table(sid), self.pool.seq_len(sid)
        nb = min(len(ids), length) // BLOCK
        keys = block_keys(ids[:BLOCK * nb])
        parent, pkey, added = -1, None, 0
        for j, key in enumerate(keys):
            blk = table[j]
            e = self.entries.get(key)
            if e is not None:
                if e["block"] != blk or e["parent"] != parent:
                    break
                self.clock += 1
                e["stamp"] = self.clock
            else:
                self.pool.incref(blk)
                self.clock += 1
                self.entries[key] = {"block": blk, "parent": parent, "parent_key": pkey,
                                     "ids": ids[BLOCK * j:BLOCK * (j + 1)], "stamp": self.clock,
                                     "children": 0}
                if j > 0:
                    self.entries[pkey]["children"] += 1
                added += 1
            parent, pkey = blk, key
        return added

    def evict(self, max_blocks):
        if max_blocks < 0:
            raise PoolError("INVALID_ARG", "negative max_blocks")
        done = 0
        while done < max_blocks:
            cands = [(e["stamp"], k) for k, e in self.entries.items()
                     if e["children"] == 0 and self.pool.refcount(e["block"]) == 1]
            if not cands:
                break
            _, key = min(cands)
            e = self.entries.pop(key)
            if e["parent"] >= 0:
                self.entries[e["parent_key"]]["children"] -= 1
            self.pool.free(e["block"])
            done += 1
        return done

    def stats(self):
        return len(self.entries), self.hits, self.asked


def replay_with_cache(pool, cache, ops):
    """replay() with the prefix-cache ops: ("prefix_lookup", ids),
    ("prefix_register", sid, ids), ("prefix_evict", n)."""
    out = []
    for op in ops:
        kind, args = op[0], op[1:]
        if not kind.startswith("prefix_"):
            out += replay(pool, [op])
            continue
        try:
            if kind == "prefix_lookup":
                r = cache.lookup(args[0])
            elif kind == "prefix_register":
                r = cache.register(*args)
            elif kind == "prefix_evict":
                r = cache.evict(*args)
            else:
                raise ValueError(kind)
        except PoolError as e:
            r = ("error", e.code)
        out.append(r)
    return out
