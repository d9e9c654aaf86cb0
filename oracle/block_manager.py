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

Conventions the pages leave open (the same ones the library documents):
- free blocks form a stack that starts as [num_blocks-1, ..., 1, 0]; a block
  goes back on top when its last reference (and its last pending copy) goes,
  and a freed sequence releases its blocks in table order;
- a write into a shared block is needed only when the sequence's last block is
  partly filled; a full last block is left shared and a new block is taken;
- a copy stays pending, holding both of its blocks, until it is taken; taken
  batches stop before a copy that reads a block an earlier copy in the batch
  writes.
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

    # -- block bookkeeping ---------------------------------------------------
    def _take(self) -> int:
        b = self.free.pop()
        self.refs[b] = 1
        return b

    def _maybe_free(self, b: int) -> None:
        if self.refs[b] == 0 and self.pins[b] == 0:
            self.free.append(b)

    def _drop_ref(self, b: int) -> None:
        self.refs[b] -= 1
        self._maybe_free(b)

    # -- sequence operations -------------------------------------------------
    def add(self, seq: int) -> None:
        if seq in self.seqs:
            raise KeyError(seq)
        self.seqs[seq] = ([], 0)

    def fork(self, parent: int, child: int) -> None:
        if parent == child or child in self.seqs or parent not in self.seqs:
            raise KeyError(child)
        blocks, length = self.seqs[parent]
        for b in blocks:
            self.refs[b] += 1
        self.seqs[child] = (list(blocks), length)

    def append(self, seq: int, n: int) -> List[int]:
        """Slots (block * 16 + offset) of n new tokens at the end of seq."""
        if n < 0 or seq not in self.seqs:
            raise KeyError(seq)
        blocks, length = self.seqs[seq]
        new_len = length + n
        new_blocks = -(-new_len // BLOCK)
        if new_blocks > self.max_blocks_per_seq:
            raise OutOfBlocks()
        copy_last = n > 0 and length % BLOCK != 0 and self.refs[blocks[-1]] > 1
        if (new_blocks - len(blocks)) + (1 if copy_last else 0) > len(self.free):
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
        return [blocks[p // BLOCK] * BLOCK + p % BLOCK for p in range(length, new_len)]

    def release(self, seq: int) -> None:
        blocks, _ = self.seqs.pop(seq)
        for b in blocks:
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
        return (len(self.free), self.num_blocks - len(self.free), len(self.seqs), sum(fill.values()), len(self.copies))


def kv_utilisation(lens, max_len: int) -> Tuple[float, float]:
    """(contiguous reservation, paging): the share of reserved KV slots that hold a token when every sequence
    reserves max_len slots, and when it holds ceil(L / 16) blocks of 16."""
    total = sum(int(x) for x in lens)
    reserved = len(lens) * max_len
    paged = sum(-(-int(x) // BLOCK) * BLOCK for x in lens)
    return total / reserved, total / paged
