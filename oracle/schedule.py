"""Oracle for the host side of the path: token budget, block allocation and
the batch descriptor.  Plain Python, integer work only.

* Token budget: "Prefill Optimisation ...", section 2 ("Mechanics of chunked
  scheduling": decodes claim one token each, prefill gets the rest) and
  section 7 (``schedule_prompt``: slice a prompt by the remaining budget,
  refuse when no budget is left); "Chunked Prefill" blog note, section "From
  scratch" (decode-first fill, per-prefill chunk cap, skip instead of raise).
* Block alignment: "vLLM Chunked Prefill 如何改变 KV Cache 管理", section 2.3
  (with prefix caching on, a prompt that does not fit the budget is cut to
  ``(budget // block_size) * block_size`` tokens).
* Allocation: "Prefill Processing", section "Block Allocation" (allocate the
  delta between ``cdiv(computed + new, block_size)`` and the blocks held;
  table rows sized to ``cdiv(max_model_len, block_size)``, zero-filled) and
  "vLLM Chunked Prefill ..." section 2.1 (incremental growth per chunk).
* Shared prefix blocks carry a reference count ("Prefill Optimisation ...",
  section 3, "Three disjoint block buckets").
"""
from __future__ import annotations

from collections import deque


class BudgetExhausted(RuntimeError):
    """No prefill progress is possible under the budget."""


class OutOfBlocks(RuntimeError):
    """The pool cannot hold the blocks a step needs."""


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def schedule_prompt(max_batched_tokens: int, active_decodes: int, total_prompt_tokens: int,
                    block_size: int = 0, align_to_block: bool = False) -> list:
    """Chunk sizes of one prompt when ``active_decodes`` decodes hold their
    token each of every step.  With ``align_to_block`` a chunk that does not
    finish the prompt is cut down to whole blocks."""
    if max_batched_tokens <= 0:
        raise ValueError("max_batched_tokens must be positive")
    if total_prompt_tokens < 0 or active_decodes < 0:
        raise ValueError("counts must be non-negative")
    if align_to_block and block_size <= 0:
        raise ValueError("block_size must be positive")
    budget = max_batched_tokens - active_decodes
    if budget <= 0:
        raise BudgetExhausted(f"active_decodes ({active_decodes}) >= max_batched_tokens "
                              f"({max_batched_tokens})")
    chunks = []
    remaining = total_prompt_tokens
    while remaining > 0:
        take = min(remaining, budget)
        if align_to_block and take < remaining:
            take = (take // block_size) * block_size
            if take == 0:
                raise BudgetExhausted(f"budget {budget} is below one block of {block_size}")
        chunks.append(take)
        remaining -= take
    return chunks


class BlockPool:
    """Fixed pool of physical blocks: a FIFO free list (in the given order)
    and a reference count per block."""

    def __init__(self, num_blocks: int, free_order=None):
        order = range(num_blocks) if free_order is None else [int(x) for x in free_order]
        self.free = deque(order)
        self.ref = [0] * num_blocks

    def num_free(self) -> int:
        return len(self.free)

    def allocate(self, n: int) -> list:
        if n > len(self.free):
            raise OutOfBlocks(f"need {n} blocks, {len(self.free)} free")
        out = [self.free.popleft() for _ in range(n)]
        for blk in out:
            self.ref[blk] = 1
        return out

    def share(self, blocks) -> None:
        for blk in blocks:
            if self.ref[blk] <= 0:
                raise ValueError(f"block {blk} is not active")
            self.ref[blk] += 1

    def release(self, blocks) -> None:
        for blk in blocks:
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                self.free.append(blk)


class Request:
    def __init__(self, req_id: int, num_tokens: int, num_computed: int, blocks, is_decode: bool):
        self.req_id = req_id
        self.num_tokens = num_tokens        # tokens known so far (prompt, then + generated)
        self.num_computed = num_computed    # tokens whose KV is in the cache
        self.blocks = list(blocks)
        self.is_decode = is_decode


class Scheduler:
    """Decode-first token-budget scheduler over a ``BlockPool``."""

    def __init__(self, pool: BlockPool, block_size: int, max_batched_tokens: int,
                 max_blocks_per_seq: int, long_prefill_cap: int = 0,
                 align_to_block: bool = False):
        if block_size <= 0 or max_batched_tokens <= 0 or max_blocks_per_seq <= 0:
            raise ValueError("block_size, max_batched_tokens, max_blocks_per_seq must be positive")
        self.pool = pool
        self.block_size = block_size
        self.budget = max_batched_tokens
        self.max_blocks = max_blocks_per_seq
        self.cap = long_prefill_cap
        self.align = align_to_block
        self.reqs = []      # FCFS order

    def _find(self, req_id):
        for r in self.reqs:
            if r.req_id == req_id:
                return r
        raise KeyError(req_id)

    def add_request(self, req_id: int, num_prompt_tokens: int, prefix_blocks=()):
        """A new prompt; ``prefix_blocks`` are shared blocks of a prefix hit
        (looked up only before the first chunk), so ``len * block_size``
        tokens start out computed."""
        if num_prompt_tokens <= 0:
            raise ValueError("empty prompt")
        prefix_blocks = list(prefix_blocks)
        computed = len(prefix_blocks) * self.block_size
        if computed >= num_prompt_tokens:
            raise ValueError("prefix must leave at least one token to compute")
        if cdiv(num_prompt_tokens, self.block_size) > self.max_blocks:
            raise ValueError("prompt longer than a block-table row can map")
        self.pool.share(prefix_blocks)
        self.reqs.append(Request(req_id, num_prompt_tokens, computed, prefix_blocks, False))

    def add_partial(self, req_id: int, num_prompt_tokens: int, num_computed_tokens: int):
        """A prompt whose first ``num_computed_tokens`` are already cached in
        blocks it owns (taken from the pool now); prefill resumes there."""
        if num_computed_tokens < 0 or num_prompt_tokens <= num_computed_tokens:
            raise ValueError("need 0 <= computed < prompt")
        if cdiv(num_prompt_tokens, self.block_size) > self.max_blocks:
            raise ValueError("prompt longer than a block-table row can map")
        blocks = self.pool.allocate(cdiv(num_computed_tokens, self.block_size))
        self.reqs.append(Request(req_id, num_prompt_tokens, num_computed_tokens, blocks, False))

    def add_decode(self, req_id: int, context_len: int):
        """A running sequence with ``context_len`` tokens cached and one token to
        decode; its cache blocks are taken from the pool now."""
        if context_len <= 0:
            raise ValueError("empty context")
        if cdiv(context_len + 1, self.block_size) > self.max_blocks:
            raise ValueError("context longer than a block-table row can map")
        blocks = self.pool.allocate(cdiv(context_len, self.block_size))
        self.reqs.append(Request(req_id, context_len + 1, context_len, blocks, True))

    def step(self) -> dict:
        """Pick this step's tokens, grow the block tables, return the batch
        descriptor (decodes first, then prefills, each in arrival order)."""
        used = 0
        picked = []
        for r in self.reqs:
            if r.is_decode and used < self.budget:
                picked.append((r, 1))
                used += 1
        for r in self.reqs:
            if r.is_decode:
                continue
            if used >= self.budget:
                break
            remaining = r.num_tokens - r.num_computed
            take = min(remaining, self.budget - used)
            if self.cap > 0:
                take = min(take, self.cap)
            if self.align and take < remaining:
                take = (take // self.block_size) * self.block_size
            if take <= 0:
                continue
            picked.append((r, take))
            used += take
        need_new = []
        for r, take in picked:
            need = cdiv(r.num_computed + take, self.block_size)
            if need > self.max_blocks:
                raise ValueError(f"request {r.req_id} needs {need} blocks > row width {self.max_blocks}")
            need_new.append(need - len(r.blocks))
        if sum(need_new) > self.pool.num_free():
            raise OutOfBlocks(f"step needs {sum(need_new)} blocks, {self.pool.num_free()} free")
        for (r, _), k in zip(picked, need_new):
            r.blocks.extend(self.pool.allocate(k))
        cu = [0]
        cached, q_lens, req_ids, rows, slots = [], [], [], [], []
        for r, take in picked:
            req_ids.append(r.req_id)
            q_lens.append(take)
            cached.append(r.num_computed)
            cu.append(cu[-1] + take)
            rows.append(r.blocks + [0] * (self.max_blocks - len(r.blocks)))
            for t in range(take):
                p = r.num_computed + t
                slots.append(r.blocks[p // self.block_size] * self.block_size + p % self.block_size)
        self._last = picked
        return {"req_ids": req_ids, "q_lens": q_lens, "cu_seqlens_q": cu,
                "cached_seq_len": cached, "block_table": rows, "slot_mapping": slots,
                "num_tokens": used}

    def commit(self) -> None:
        """Advance every request of the last step; a finished prompt turns into
        a decode of the token its last chunk produced."""
        for r, take in self._last:
            r.num_computed += take
            if r.is_decode:
                r.num_tokens += 1
            elif r.num_computed == r.num_tokens:
                r.is_decode = True
                r.num_tokens += 1
        self._last = []

    def free_request(self, req_id: int) -> None:
        r = self._find(req_id)
        self.pool.release(r.blocks)
        self.reqs.remove(r)
