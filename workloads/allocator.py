"""Host-side block allocator used to build block tables for the workloads.

Restates the block manager of "How LLM Inference Engines Work" (section
"PagedAttention: Virtual Memory for KV Caches", the simplified block
manager): a stack of free block ids; ``allocate`` pops one block for a
sequence and reports failure (instead of raising) when none is left;
``free`` drops one reference per block and returns a block to the free
list when its count reaches zero.  ``share`` adds the prefix sharing of
"AI Inference Serving at Scale" section 3 and "vLLM & High-Throughput
Serving" section 2: a second sequence's table points at the same physical
blocks, whose reference count goes up.

``fork_for_append`` is the host half of copy-on-write ("AI Inference
Serving at Scale" section 3; "vLLM & High-Throughput Serving", copy-on-write
prefix caching): before a sequence writes a token into a block other
sequences still reference, it gets a fresh block in that table slot, the
shared block loses one reference, and the (old, new) pair is returned for
the device copy (``pa_copy_blocks``).

Physical ids come out in the order of the initial free list, so seeding
that order with a permutation gives the shuffled pools of the workloads.
"""

from __future__ import annotations

from dataclasses import dataclass, field


@dataclass
class Sequence:
    """A sequence's logical-to-physical block list (its block-table row)."""

    request_id: str
    blocks: list[int] = field(default_factory=list)


class BlockManager:
    """Free list plus reference counts over a fixed pool of blocks."""

    def __init__(self, num_blocks: int, block_size: int, order=None):
        self.block_size = int(block_size)
        self.num_blocks = int(num_blocks)
        ids = list(range(num_blocks)) if order is None else [int(i) for i in order]
        if sorted(ids) != list(range(num_blocks)):
            raise ValueError("free-list order must be a permutation of the pool")
        # popped from the end: reverse so the first id of ``order`` is used first
        self._free = ids[::-1]
        self._refs: dict[int, int] = {}

    @property
    def free_blocks(self) -> int:
        return len(self._free)

    def ref_count(self, block_id: int) -> int:
        return self._refs.get(block_id, 0)

    def allocate(self, seq: Sequence) -> bool:
        """Give ``seq`` one more block; False when the pool is exhausted."""
        if not self._free:
            return False
        blk = self._free.pop()
        self._refs[blk] = 1
        seq.blocks.append(blk)
        return True

    def allocate_tokens(self, seq: Sequence, num_tokens: int) -> bool:
        """Allocate blocks until ``seq`` can hold ``num_tokens`` tokens."""
        need = -(-int(num_tokens) // self.block_size)
        while len(seq.blocks) < need:
            if not self.allocate(seq):
                return False
        return True

    def share(self, src: Sequence, dst: Sequence, num_blocks: int) -> None:
        """Point ``dst`` at the first ``num_blocks`` blocks of ``src``."""
        for blk in src.blocks[:num_blocks]:
            self._refs[blk] += 1
            dst.blocks.append(blk)

    def free(self, seq: Sequence) -> None:
        """Drop ``seq``'s references; recycle blocks nobody else holds."""
        for blk in seq.blocks:
            self._refs[blk] -= 1
            if self._refs[blk] == 0:
                del self._refs[blk]
                self._free.append(blk)
        seq.blocks = []

    def fork_for_append(self, seq: Sequence, position: int):
        """Make the block holding token ``position`` of ``seq`` private.

        Returns ``(src, dst)`` when the block was shared (the caller copies
        src to dst before writing), ``None`` when ``seq`` already owns it
        alone, and ``False`` when the pool has no free block for the copy
        (nothing is changed then).
        """
        i = int(position) // self.block_size
        blk = seq.blocks[i]
        if self._refs[blk] == 1:
            return None
        if not self._free:
            return False
        new = self._free.pop()
        self._refs[new] = 1
        self._refs[blk] -= 1
        seq.blocks[i] = new
        return blk, new
