"""Block-pool oracle: free list, reference counts, fork and copy-on-write.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it follows, by page and section:

* "19.2 KV Cache 系统化管理" §19.2.3, the ``PhysicalBlockPool`` class: the
  free list starts as the block ids in ascending order; ``allocate`` takes the
  id at the *end* of the list and sets its reference count to 1, and fails
  when the list is empty; ``release`` lowers the count by one and appends the
  id to the end of the free list when the count reaches zero.
* Same page and section, the ``BlockTable`` class: token number ``n`` of a
  request goes to logical block ``n // block_size`` at in-block slot
  ``n % block_size``; a new physical block is allocated when the logical
  block is not mapped yet; ``release_all`` releases the mapped blocks in
  logical order and clears the table.
* Same page, §19.2.2 (copy-on-write and prefix sharing): sharers point at the
  same physical block and its reference count equals the number of sharers;
  a write into a block whose count is above one allocates a new block,
  copies the old content, remaps the table entry and lowers the old block's
  count by one.
* "LLM 推理引擎的内存管理与调度" §4: the copy happens when a branch modifies a
  *shared tail block*; a fork shares every block of the parent.

Readings taken where the pages are silent (each is listed in the design doc):

* The initial free list may be any permutation of the block ids (the
  workloads draw one from a seed); it is still popped from the end.
* A slot is the flat index ``physical_block * block_size + offset``.
* ``append`` is all-or-nothing: when the free list cannot cover every block
  the call needs (the copy-on-write block plus the new blocks), it raises and
  nothing changes.  The pages' ``append_token`` also raises before it
  touches ``num_filled``.
* Copy-on-write copies the whole block (keys and values); the pair
  ``(old, new)`` is returned so that the device copy can run before the
  device write.

Prefix cache ("LLM 推理引擎的内存管理与调度" §5.1-5.2; "19.2 KV Cache 系统化管理"
§19.2.5): a full block is keyed by a chained hash ``h_i = H(h_{i-1},
tokens_i, extra)``; a new request looks its prompt's keys up block by block,
and every hit maps the cached block into its table with one more reference
(the prefill of that block is skipped); the first miss ends the match.
Cached blocks survive their requests: at reference count zero they become
evictable instead of free, and are reclaimed least recently released first
when the free list is empty.  Readings: H is 64-bit FNV-1a over the parent
key, a salt (the page's model / adapter / extra fields) and the token ids
(byte order below); the first block's parent key is 0; blocks released by
one call enter the eviction order in logical order; registering a key that
another block already holds keeps the first block.

Pins: the pages' worked example (10 tokens, block size 4, 16 blocks ->
blocks [15, 14, 13], 16/16 free after release), the lifecycle example of
§19.2.2 (7-token prompt in blocks 7 and 1, the 9th token opens block 3),
and the invariants ceil(len/bs) blocks per sequence, at most bs-1 unused
slots, reference count == number of sharers, every block free after
releasing everything -- checked by brute force against a set-based model.
"""

from __future__ import annotations

from collections import OrderedDict

FNV64_OFFSET = 0xCBF29CE484222325
FNV64_PRIME = 0x100000001B3


def fnv1a64(data: bytes, h: int = FNV64_OFFSET) -> int:
    """64-bit FNV-1a: for every byte, xor it in, then multiply by the FNV prime."""
    for byte in data:
        h ^= byte
        h = (h * FNV64_PRIME) & 0xFFFFFFFFFFFFFFFF
    return h


def prefix_hash(parent: int, tokens, salt: int = 0) -> int:
    """Key of one full block: FNV-1a over the parent key (8 bytes, little
    endian), the salt (8 bytes, little endian) and every token id (4 bytes,
    little endian, two's complement)."""
    data = int(parent).to_bytes(8, "little") + int(salt).to_bytes(8, "little")
    data += b"".join((int(t) & 0xFFFFFFFF).to_bytes(4, "little") for t in tokens)
    return fnv1a64(data)


class OracleNoFreeBlocks(RuntimeError):
    """The free list cannot supply the blocks an operation needs."""


class OracleBlockPool:
    """Host-side mirror of the physical block pool and per-request tables."""

    def __init__(self, num_blocks: int, block_size: int, initial_free=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        if initial_free is None:
            self.free_list = list(range(self.num_blocks))
        else:
            self.free_list = [int(x) for x in initial_free]
            if sorted(self.free_list) != list(range(self.num_blocks)):
                raise ValueError("initial_free must be a permutation of the block ids")
        self.ref_counts = [0] * self.num_blocks
        # prefix cache: key -> block, block -> key, evictable blocks (oldest first)
        self.cached: dict[int, int] = {}
        self.block_key: dict[int, int] = {}
        self.evictable: OrderedDict[int, None] = OrderedDict()
        # seq id -> [mapping(list of physical ids), num_filled]
        self.seqs: dict[int, list] = {}
        self._next_seq = 0

    # -- PhysicalBlockPool.allocate / release --------------------------------
    def _allocate(self) -> int:
        if self.free_list:
            block = self.free_list.pop()
        elif self.evictable:  # reclaim the least recently released cached block
            block, _ = self.evictable.popitem(last=False)
            del self.cached[self.block_key.pop(block)]
        else:
            raise OracleNoFreeBlocks("no free physical block")
        self.ref_counts[block] = 1
        return block

    def _release_block(self, block: int) -> None:
        self.ref_counts[block] -= 1
        if self.ref_counts[block] == 0:
            if block in self.block_key:
                self.evictable[block] = None
            else:
                self.free_list.append(block)

    def available(self) -> int:
        """Blocks an allocation can take: free ones and evictable cached ones."""
        return len(self.free_list) + len(self.evictable)

    # -- prefix cache --------------------------------------------------------
    def match_prefix(self, seq: int, keys) -> int:
        """Map the cached blocks of the longest matching key chain into the
        empty request ``seq``; returns the number of blocks hit."""
        mapping, filled = self.seqs[seq]
        if mapping or filled:
            raise ValueError("match_prefix needs an empty sequence")
        hits = 0
        for key in keys:
            block = self.cached.get(int(key))
            if block is None:
                break
            if self.ref_counts[block] == 0:
                del self.evictable[block]
            self.ref_counts[block] += 1
            mapping.append(block)
            hits += 1
        self.seqs[seq][1] = hits * self.block_size
        return hits

    def register_prefix(self, seq: int, keys) -> None:
        """Publish the first ``len(keys)`` (full) blocks of ``seq`` under ``keys``."""
        mapping, filled = self.seqs[seq]
        if len(keys) > filled // self.block_size:
            raise ValueError("only full blocks can be registered")
        for i, key in enumerate(keys):
            key, block = int(key), mapping[i]
            if block in self.block_key:
                if self.block_key[block] != key:
                    raise ValueError("block already cached under another key")
                continue
            if key in self.cached:
                continue  # another block holds this prefix already: the first one stays
            self.cached[key] = block
            self.block_key[block] = key

    # -- request lifecycle ---------------------------------------------------
    def new_seq(self) -> int:
        seq = self._next_seq
        self._next_seq += 1
        self.seqs[seq] = [[], 0]
        return seq

    def fork(self, parent: int) -> int:
        """A new request that shares every block of ``parent``."""
        mapping, filled = self.seqs[parent]
        for block in mapping:
            self.ref_counts[block] += 1
        child = self._next_seq
        self._next_seq += 1
        self.seqs[child] = [list(mapping), filled]
        return child

    def blocks_needed(self, seq: int, n_tokens: int) -> int:
        """Blocks that ``append(seq, n_tokens)`` would take from the free list."""
        mapping, filled = self.seqs[seq]
        if n_tokens <= 0:
            return 0
        bs = self.block_size
        need = 0
        first_block = filled // bs
        if first_block < len(mapping) and self.ref_counts[mapping[first_block]] > 1:
            need += 1  # copy-on-write of the shared, partly filled tail
        last_block = (filled + n_tokens - 1) // bs
        need += max(0, last_block + 1 - len(mapping))
        return need

    def append(self, seq: int, n_tokens: int):
        """Reserve slots for ``n_tokens`` new tokens of ``seq``.

        Returns ``(slots, cow_pairs)``: the flat slot of every new token in
        order, and the ``(old, new)`` block pairs whose content must be copied
        before the new tokens are written.
        """
        if n_tokens < 0:
            raise ValueError("n_tokens must be >= 0")
        if self.blocks_needed(seq, n_tokens) > self.available():
            raise OracleNoFreeBlocks("not enough free blocks for append")
        state = self.seqs[seq]
        mapping = state[0]
        bs = self.block_size
        slots = []
        cow = []
        for _ in range(n_tokens):
            filled = state[1]
            logical = filled // bs
            offset = filled % bs
            if logical >= len(mapping):
                mapping.append(self._allocate())
            elif self.ref_counts[mapping[logical]] > 1:
                old = mapping[logical]
                new = self._allocate()
                cow.append((old, new))
                self._release_block(old)
                mapping[logical] = new
            slots.append(mapping[logical] * bs + offset)
            state[1] = filled + 1
        return slots, cow

    def release(self, seq: int) -> None:
        """``BlockTable.release_all``: release blocks in logical order."""
        mapping, _ = self.seqs.pop(seq)
        for block in mapping:
            self._release_block(block)

    # -- queries -------------------------------------------------------------
    def seq_len(self, seq: int) -> int:
        return self.seqs[seq][1]

    def mapping(self, seq: int) -> list:
        return list(self.seqs[seq][0])

    def num_free(self) -> int:
        """Free plus evictable blocks (what allocations can still take)."""
        return self.available()

    def block_tables(self, seqs, max_blocks: int, fill: int = -1):
        """Rows of physical ids, one per sequence, padded with ``fill``."""
        rows = []
        for seq in seqs:
            mapping = self.seqs[seq][0]
            if len(mapping) > max_blocks:
                raise ValueError("sequence has more blocks than max_blocks")
            rows.append(list(mapping) + [fill] * (max_blocks - len(mapping)))
        return rows
