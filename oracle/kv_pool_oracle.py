"""Reference model of a paged KV block pool with zero-copy forks (plain Python).

TEST INFRASTRUCTURE ONLY, like the rest of this package.

Source: "HPD-Parsing: Hierarchical Parallel Document Parsing" notes:
prerequisites "KV cache and shared-prefix reuse" (paged KV blocks; a forked
branch shares its parent's prefix blocks without copying them) and
Algorithm 1 (on a <FORK> the child is spawned with a zero-copy pointer to the
parent's KV; when branches finish their KV is released by reference count).
"PaDoc" summary, "Inference": branches reuse the complete KV blocks of the
shared prefix; only their own suffix needs new memory.

Readings where the pages are silent (listed in the design notes):
  * a sequence is a root (its own tokens only) or a fork: a read-only view of
    the first n tokens of a root's blocks plus tokens of its own;
  * forks are taken from roots (HPD forks content branches off the layout
    stream: one level);
  * free blocks are handed out lowest id first; an append that does not fit
    fails whole and changes nothing;
  * a block is free again when no sequence references it; releasing a root
    keeps the blocks its live forks still view;
  * sequence ids count up from 0 and are never reused.
"""
from __future__ import annotations


class PoolError(Exception):
    pass


class KVPool:
    def __init__(self, n_blocks: int, block_size: int):
        if n_blocks < 0 or block_size < 1:
            raise PoolError("bad pool size")
        self.n_blocks, self.bs = n_blocks, block_size
        self.ref = [0] * n_blocks
        self.seqs = {}  # id -> dict(view=[blocks], view_len, own=[blocks], own_len, root)
        self.next_id = 0

    def free_blocks(self) -> int:
        return sum(1 for r in self.ref if r == 0)

    def _take(self, k):
        free = [b for b in range(self.n_blocks) if self.ref[b] == 0][:k]
        if len(free) < k:
            raise PoolError("out of blocks")
        for b in free:
            self.ref[b] = 1
        return free

    def new_seq(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.seqs[sid] = dict(view=[], view_len=0, own=[], own_len=0, root=True)
        return sid

    def fork(self, parent: int, n_tokens: int) -> int:
        p = self.seqs.get(parent)
        if p is None or not p["root"]:
            raise PoolError("forks are taken from live roots")
        if not 0 <= n_tokens <= p["own_len"]:
            raise PoolError("fork point outside the parent")
        view = p["own"][:(n_tokens + self.bs - 1) // self.bs]
        for b in view:
            self.ref[b] += 1
        sid = self.next_id
        self.next_id += 1
        self.seqs[sid] = dict(view=list(view), view_len=n_tokens, own=[], own_len=0, root=False)
        return sid

    def append(self, sid: int, n_tokens: int):
        """Room for n_tokens more own tokens; returns their physical slots
        (block * block_size + offset)."""
        s = self.seqs.get(sid)
        if s is None or n_tokens < 0:
            raise PoolError("bad append")
        new_len = s["own_len"] + n_tokens
        need = (new_len + self.bs - 1) // self.bs - len(s["own"])
        s["own"] += self._take(need) if need > 0 else []
        slots = [s["own"][t // self.bs] * self.bs + t % self.bs for t in range(s["own_len"], new_len)]
        s["own_len"] = new_len
        return slots

    def release(self, sid: int):
        s = self.seqs.pop(sid, None)
        if s is None:
            raise PoolError("unknown sequence")
        for b in s["view"] + s["own"]:
            self.ref[b] -= 1

    def table(self, sid: int):
        s = self.seqs[sid]
        return list(s["view"]), s["view_len"], list(s["own"]), s["own_len"]


def gather(cache, blocks, n_tokens: int, block_size: int):
    """Logical tokens [0, n_tokens) of a paged sequence: token t lives in
    cache row blocks[t // block_size] * block_size + t % block_size (cache
    rows are [n_blocks * block_size, ...])."""
    rows = [blocks[t // block_size] * block_size + t % block_size for t in range(n_tokens)]
    return cache[rows]
