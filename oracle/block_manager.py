"""Reference model of the paged-KV block manager (plain Python, slow, obvious).

TEST INFRASTRUCTURE ONLY: used by the test suite to check the library's host
block manager and block copies; the library never imports it.

What it models (the pages' description of paging):
- ai-maas.com vLLM article, 先看浪费在哪里: KV memory is handed out in fixed
  blocks on demand as a sequence grows, instead of reserving max_len tokens
  per request up front, and returned when the sequence ends;
- ipipp.com vLLM/PagedAttention article, section 二: 16-token blocks, one
  block table per sequence mapping logical to physical blocks, blocks shared
  between sequences (parallel sampling, beam search) with a reference count,
  and a shared block copied before a sequence writes into it (copy-on-write).

Automatic prefix caching (bytelighting wiki "vLLM", paragraph on APC; the
ai-maas.com article's note that repeated prefixes are computed once and
shared): blocks are identified by their content along a chain.  Here a
registered block is keyed exactly by (the registration of its registered
predecessor, its 16 token ids); a hit on prompt block j needs the key built
from the block matched for j - 1.  Registered blocks without references are
evictable, oldest release first.

Conventions the pages leave open (the same ones the library documents):
- free blocks form a stack that starts as [num_blocks-1, ..., 1, 0]; a block
  goes back on top when its last reference (and its last pending copy) goes,
  and a freed sequence releases its blocks in table order;
- a write into a shared block is needed only when the sequence's last block is
  partly filled; a full last block is left shared and a new block is taken;
- a copy stays pending, holding both of its blocks, until it is taken; taken
  batches stop before a copy that reads a block an earlier copy in the batch
  writes;
- prefix caching: a prompt reuses at most (n - 1) // 16 blocks, so its last
  token is always computed; a block is registered when a sequence with known
  token ids fills it, unless the same content after the same registered
  predecessor is registered; a sequence that appended tokens without ids
  registers nothing more; eviction happens only when no never-registered
  block is free, and a freed sequence releases its blocks deepest first.
"""
from __future__ import annotations

from typing import Dict, List, Tuple

BLOCK = 16


class OutOfBlocks(Exception):
    pass


class RefBlockManager:
    def __init__(self, num_blocks: int, max_blocks_per_seq: int):
        self.num_blocks = num_blocks
        self.max_blocks_per_seq = max_blocks_per_seq
        self.free = list(range(num_blocks - 1, -1, -1))  # top of the stack = end of the list
        self.refs = [0] * num_blocks
        self.pins = [0] * num_blocks
        self.seqs: Dict[int, Tuple[List[int], int]] = {}  # seq -> (blocks, length)
        self.copies: List[Tuple[int, int]] = []
        # prefix caching
        self.caching = False
        self.registered: Dict[tuple, int] = {}   # (predecessor registration or None, tokens) -> block
        self.reg_of: Dict[int, Tuple[int, tuple]] = {}  # block -> (its registration id, its key)
        self.next_reg = 0
        self.lru: List[int] = []                 # evictable registered blocks, oldest release first
        self.track: Dict[int, dict] = {}         # seq -> {"on": ids known, "tail": [...], "par": registration}
        self.lookups = self.hits = self.evictions = 0

    # -- block bookkeeping ---------------------------------------------------
    def _free_count(self) -> int:
        return len(self.free) + len(self.lru)

    def _unregister(self, b: int) -> None:
        _, key = self.reg_of.pop(b)
        del self.registered[key]

    def _take(self) -> int:
        if self.free:
            b = self.free.pop()
        else:  # evict the registered block released longest ago
            b = self.lru.pop(0)
            self._unregister(b)
            self.evictions += 1
        self.refs[b] = 1
        return b

    def _maybe_free(self, b: int) -> None:
        if self.refs[b] == 0 and self.pins[b] == 0:
            if self.caching and b in self.reg_of:
                self.lru.append(b)
            else:
                self.free.append(b)

    def _alive(self, reg) -> bool:
        return any(r == reg for r, _ in self.reg_of.values())

    def _register(self, seq: int, j: int, tokens) -> None:
        """Block j of seq just filled with tokens."""
        t = self.track[seq]
        if j == 0:
            par = None
        else:
            par = t["par"]
            if par is None or not self._alive(par):
                t["par"] = None
                return
        key = (par, tuple(int(x) for x in tokens))
        if key in self.registered:
            t["par"] = self.reg_of[self.registered[key]][0]
            return
        b = self.seqs[seq][0][j]
        self.next_reg += 1
        self.registered[key] = b
        self.reg_of[b] = (self.next_reg, key)
        t["par"] = self.next_reg

    def _feed(self, seq: int, start: int, tokens) -> None:
        """Token ids of positions start.. of seq; register blocks as they fill."""
        t = self.track[seq]
        for i, tok in enumerate(tokens):
            t["tail"].append(int(tok))
            if len(t["tail"]) == BLOCK:
                self._register(seq, (start + i) // BLOCK, t["tail"])
                t["tail"] = []

    def enable_prefix_caching(self) -> None:
        if self.seqs or self.copies:
            raise KeyError("not empty")
        self.caching = True

    def _drop_ref(self, b: int) -> None:
        self.refs[b] -= 1
        self._maybe_free(b)

    # -- sequence operations -------------------------------------------------
    def add(self, seq: int) -> None:
        if seq in self.seqs:
            raise KeyError(seq)
        self.seqs[seq] = ([], 0)
        self.track[seq] = {"on": self.caching, "tail": [], "par": None}

    def add_prompt(self, seq: int, tokens) -> Tuple[List[int], int]:
        """(slots of the tokens to compute, tokens reused) for a new sequence with its prompt."""
        if not self.caching or seq in self.seqs:
            raise KeyError(seq)
        tokens = [int(x) for x in tokens]
        n = len(tokens)
        nb = -(-n // BLOCK)
        if nb > self.max_blocks_per_seq:
            raise OutOfBlocks()
        eligible = (n - 1) // BLOCK if n > 0 else 0
        hits, prev = [], None
        for j in range(eligible):
            key = (prev, tuple(tokens[j * BLOCK:(j + 1) * BLOCK]))
            if key not in self.registered:
                break
            b = self.registered[key]
            hits.append(b)
            prev = self.reg_of[b][0]
        in_lru = sum(1 for b in hits if b in self.lru)
        if nb - len(hits) > self._free_count() - in_lru:
            raise OutOfBlocks()
        self.lookups += eligible
        self.hits += len(hits)
        for b in hits:
            if self.refs[b] == 0 and b in self.lru:
                self.lru.remove(b)
            self.refs[b] += 1
        blocks = list(hits)
        while len(blocks) < nb:
            blocks.append(self._take())
        cached = len(hits) * BLOCK
        self.seqs[seq] = (blocks, n)
        self.track[seq] = {"on": True, "tail": [], "par": prev}
        self._feed(seq, cached, tokens[cached:])
        return [blocks[p // BLOCK] * BLOCK + p % BLOCK for p in range(cached, n)], cached

    def cache_stats(self):
        return (len(self.registered), len(self.lru), self.lookups, self.hits, self.evictions)

    def fork(self, parent: int, child: int) -> None:
        if parent == child or child in self.seqs or parent not in self.seqs:
            raise KeyError(child)
        blocks, length = self.seqs[parent]
        for b in blocks:
            self.refs[b] += 1
        self.seqs[child] = (list(blocks), length)
        t = self.track[parent]
        self.track[child] = {"on": t["on"], "tail": list(t["tail"]), "par": t["par"]}

    def append(self, seq: int, n: int, tokens=None) -> List[int]:
        """Slots (block * 16 + offset) of n new tokens at the end of seq (their ids, if known, in tokens)."""
        if n < 0 or seq not in self.seqs:
            raise KeyError(seq)
        blocks, length = self.seqs[seq]
        new_len = length + n
        new_blocks = -(-new_len // BLOCK)
        if new_blocks > self.max_blocks_per_seq:
            raise OutOfBlocks()
        copy_last = n > 0 and length % BLOCK != 0 and self.refs[blocks[-1]] > 1
        if (new_blocks - len(blocks)) + (1 if copy_last else 0) > self._free_count():
            raise OutOfBlocks()
        blocks = list(blocks)
        if copy_last:
            src = blocks[-1]
            dst = self._take()
            self.pins[src] += 1
            self.pins[dst] += 1
            self._drop_ref(src)
            blocks[-1] = dst
            self.copies.append((src, dst))
        while len(blocks) < new_blocks:
            blocks.append(self._take())
        self.seqs[seq] = (blocks, new_len)
        t = self.track[seq]
        if self.caching and t["on"] and n > 0:
            if tokens is None:
                t["on"] = False
            else:
                self._feed(seq, length, tokens)
        return [blocks[p // BLOCK] * BLOCK + p % BLOCK for p in range(length, new_len)]

    def release(self, seq: int) -> None:
        blocks, _ = self.seqs.pop(seq)
        del self.track[seq]
        for b in (reversed(blocks) if self.caching else blocks):
            self._drop_ref(b)

    def table(self, seqs: List[int], max_blocks: int):
        rows, lens = [], []
        for s in seqs:
            blocks, length = self.seqs[s]
            if len(blocks) > max_blocks:
                raise KeyError(s)
            rows.append(blocks + [-1] * (max_blocks - len(blocks)))
            lens.append(length)
        return rows, lens

    def take_copies(self, max_copies: int) -> List[Tuple[int, int]]:
        batch: List[Tuple[int, int]] = []
        while len(batch) < max_copies and len(batch) < len(self.copies):
            src, dst = self.copies[len(batch)]
            if any(d == src for _, d in batch):
                break
            batch.append((src, dst))
        del self.copies[: len(batch)]
        for src, dst in batch:
            self.pins[src] -= 1
            self._maybe_free(src)
            self.pins[dst] -= 1
            self._maybe_free(dst)
        return batch

    def stats(self) -> Tuple[int, int, int, int, int]:
        """(free blocks, used blocks, live sequences, tokens held with a shared block counted once, pending copies)"""
        fill: Dict[int, int] = {}
        for blocks, length in self.seqs.values():
            for j, b in enumerate(blocks):
                fill[b] = max(fill.get(b, 0), min(BLOCK, length - j * BLOCK))
        return (self._free_count(), self.num_blocks - self._free_count(), len(self.seqs), sum(fill.values()),
                len(self.copies))


def kv_utilisation(lens, max_len: int) -> Tuple[float, float]:
    """(contiguous reservation, paging): the share of reserved KV slots that hold a token when every sequence
    reserves max_len slots, and when it holds ceil(L / 16) blocks of 16."""
    total = sum(int(x) for x in lens)
    reserved = len(lens) * max_len
    paged = sum(-(-int(x) // BLOCK) * BLOCK for x in lens)
    return total / reserved, total / paged
