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
* Prefix caching (optional): the pool's blocks fall in three disjoint
  buckets, active (reference count > 0), reclaimable cached (count 0, still
  holding a known full block) and empty ("Prefill Optimisation ...", section
  3, "Cache granularity and eviction in preallocated pools"); the free count
  includes the reclaimable ones (same section, "Accounting considerations").
  Allocation takes empty blocks first and then evicts the least recently
  freed cached block, forgetting its identity (eviction is host metadata only).
  A request's prefix is looked up once, when it is first scheduled, and only
  over the blocks of that first chunk ("vLLM Chunked Prefill ...", section
  2.2 and the scenario of section 3.1); full blocks are registered under
  their exact chained identity (``oracle.prefix_cache``) as their tokens are
  computed.
"""
from __future__ import annotations

from collections import OrderedDict, deque

from . import prefix_cache as _pc


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
    room = max_batched_tokens - active_decodes      # prefill share of every step
    if room <= 0:
        raise BudgetExhausted("the decodes use the whole token budget")
    if total_prompt_tokens <= room:                 # fits in one step (or nothing to do)
        return [total_prompt_tokens] if total_prompt_tokens else []
    # every step but the last fills the room (cut to whole blocks when
    # aligning); the last takes what is left, which then fits the room
    full = (room // block_size) * block_size if align_to_block else room
    if full == 0:
        raise BudgetExhausted("the prefill share of a step is below one block")
    steps = cdiv(total_prompt_tokens - room, full)
    return [full] * steps + [total_prompt_tokens - steps * full]


class BlockPool:
    """Fixed pool of physical blocks: a FIFO list of empty blocks (in the
    given order), a reference count per block and, for prefix caching, the
    identity a block holds, the identity table and the reclaimable cached blocks
    in the order they were freed."""

    def __init__(self, num_blocks: int, free_order=None):
        order = range(num_blocks) if free_order is None else [int(x) for x in free_order]
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.identity = [None] * num_blocks
        self.table = {}
        self.lru = OrderedDict()

    def num_free(self) -> int:
        """Empty plus reclaimable blocks: what allocation can hand out."""
        return len(self.free) + len(self.lru)

    def num_empty(self) -> int:
        return len(self.free)

    def num_reclaimable(self) -> int:
        return len(self.lru)

    def num_active(self) -> int:
        return sum(1 for r in self.ref if r > 0)

    def allocate(self, n: int) -> list:
        if n > self.num_free():
            raise OutOfBlocks(f"need {n} blocks, {self.num_free()} free")
        out = []
        for _ in range(n):
            if self.free:
                blk = self.free.popleft()
            else:
                blk, _ = self.lru.popitem(last=False)     # least recently freed cached block
                del self.table[self.identity[blk]]
                self.identity[blk] = None
            self.ref[blk] = 1
            out.append(blk)
        return out

    def share(self, blocks) -> None:
        for blk in blocks:
            if self.ref[blk] <= 0:
                raise ValueError(f"block {blk} is not active")
            self.ref[blk] += 1

    def claim(self, blk: int) -> None:
        """A prefix hit: an active or a reclaimable cached block gains a user."""
        if self.ref[blk] == 0:
            del self.lru[blk]
        self.ref[blk] += 1

    def register(self, blk: int, ident: int) -> None:
        """Block ``blk`` now holds the full block ``ident`` (first holder wins)."""
        if ident not in self.table:
            self.table[ident] = blk
            self.identity[blk] = ident

    def lookup(self, idents) -> list:
        """Blocks of the leading run of known identities."""
        out = []
        for ident in idents:
            blk = self.table.get(ident)
            if blk is None:
                break
            out.append(blk)
        return out

    def release(self, blocks) -> None:
        """Drop one reference from each block.  Blocks left unused go back
        empty, in order; cached ones become reclaimable, the sequence's last
        block first, so that its leading blocks are evicted last."""
        unused = []
        for blk in blocks:
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                unused.append(blk)
        for blk in unused:
            if self.identity[blk] is None:
                self.free.append(blk)
        for blk in reversed(unused):
            if self.identity[blk] is not None:
                self.lru[blk] = None


class Request:
    def __init__(self, req_id: int, num_tokens: int, num_computed: int, blocks, is_decode: bool,
                 tokens=None, namespace: str = "default"):
        self.req_id = req_id
        self.num_tokens = num_tokens        # tokens known so far (prompt, then + generated)
        self.num_computed = num_computed    # tokens whose KV is in the cache
        self.blocks = list(blocks)
        self.is_decode = is_decode
        self.tokens = None if tokens is None else [int(t) for t in tokens]   # prompt token ids
        self.namespace = namespace
        self.ids = []                       # identities of its first full blocks
        self.looked_up = False


class Scheduler:
    """Decode-first token-budget scheduler over a ``BlockPool``."""

    def __init__(self, pool: BlockPool, block_size: int, max_batched_tokens: int,
                 max_blocks_per_seq: int, long_prefill_cap: int = 0,
                 align_to_block: bool = False, prefix_caching: bool = False,
                 max_long_partial_prefills: int = 0, preemption: bool = False):
        if block_size <= 0 or max_batched_tokens <= 0 or max_blocks_per_seq <= 0:
            raise ValueError("block_size, max_batched_tokens, max_blocks_per_seq must be positive")
        self.pool = pool
        self.block_size = block_size
        self.budget = max_batched_tokens
        self.max_blocks = max_blocks_per_seq
        self.cap = long_prefill_cap
        self.align = align_to_block
        self.prefix_caching = prefix_caching
        self.max_long = max_long_partial_prefills
        self.preemption = preemption
        self.preempted = []
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

    def add_request_tokens(self, req_id: int, tokens, namespace: str = "default"):
        """A new prompt given by its token ids.  With prefix caching on, its
        cached prefix is looked up when it is first scheduled, and its full
        blocks are registered as they are computed."""
        tokens = list(tokens)
        if not tokens:
            raise ValueError("empty prompt")
        if cdiv(len(tokens), self.block_size) > self.max_blocks:
            raise ValueError("prompt longer than a block-table row can map")
        self.reqs.append(Request(req_id, len(tokens), 0, [], False, tokens, namespace))

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

    def _take(self, remaining: int, used: int) -> int:
        """Tokens a prefill with ``remaining`` left gets when ``used`` of the
        budget is spoken for."""
        take = min(remaining, self.budget - used)
        if self.cap > 0:
            take = min(take, self.cap)
        if self.align and take < remaining:
            take = (take // self.block_size) * self.block_size
        return take

    def _plan(self, skip):
        """This step's picks: (request, tokens) pairs, prefix hits and new
        blocks per pick; requests in ``skip`` (preempted this step) wait."""
        used = 0
        picked = []
        hits = {}           # request -> blocks of its prefix hit (first scheduling only)
        for r in self.reqs:
            if r.is_decode and used < self.budget and id(r) not in skip:
                picked.append((r, 1))
                used += 1
        longs = 0
        for r in self.reqs:
            if r.is_decode or id(r) in skip:
                continue
            if used >= self.budget:
                break
            # long prompts (longer than the per-prefill cap) beyond the
            # allowed number per step wait; shorter ones behind them go on
            is_long = self.cap > 0 and r.num_tokens > self.cap
            if is_long and self.max_long > 0 and longs >= self.max_long:
                continue
            computed = r.num_computed
            hit = None
            if (self.prefix_caching and r.tokens is not None and not r.looked_up
                    and r.num_computed == 0):
                # the lookup covers the full blocks of the first chunk only,
                # and leaves at least the prompt's last token to compute
                first = self._take(r.num_tokens, used)
                limit = min(first, r.num_tokens - 1) // self.block_size
                hit = self.pool.lookup(_pc.prefix_identities(r.tokens[:limit * self.block_size],
                                                             self.block_size, r.namespace))
                computed = len(hit) * self.block_size
            take = self._take(r.num_tokens - computed, used)
            if take <= 0:
                continue
            if hit is not None:
                hits[id(r)] = hit
            picked.append((r, take))
            used += take
            longs += is_long
        need_new = []
        for r, take in picked:
            hit = hits.get(id(r))
            computed = r.num_computed if hit is None else len(hit) * self.block_size
            held = len(r.blocks) if hit is None else len(hit)
            need = cdiv(computed + take, self.block_size)
            if need > self.max_blocks:
                raise ValueError(f"request {r.req_id} needs {need} blocks > row width {self.max_blocks}")
            need_new.append(need - held)
        claimed = {b for h in hits.values() for b in h if self.pool.ref[b] == 0}
        fits = sum(need_new) <= self.pool.num_free() - len(claimed)
        return picked, hits, need_new, used, fits, sum(need_new), len(claimed)

    def _victim(self, skip):
        """First-come-first-served: the most recently arrived request that
        holds blocks ("vLLM Chunked Prefill ...", section 4)."""
        holders = [r for r in self.reqs if r.blocks and id(r) not in skip]
        return holders[-1] if holders else None

    def _preempt(self, r) -> None:
        """Release every block of ``r`` and send it back to position 0: it
        recomputes all its known tokens (and looks its prefix up again)."""
        self.pool.release(r.blocks)
        r.blocks = []
        r.num_computed = 0
        r.is_decode = False
        r.looked_up = False
        r.ids = []

    def step(self) -> dict:
        """Pick this step's tokens, grow the block tables, return the batch
        descriptor (decodes first, then prefills, each in arrival order).
        When the pool cannot hold the step: without preemption nothing
        changes and OutOfBlocks is raised; with it, the most recently
        arrived request holding blocks is preempted (all its blocks freed,
        its progress reset) and the step planned again, until it fits."""
        skip = set()
        self.preempted = []
        while True:
            picked, hits, need_new, used, fits, need, claimed = self._plan(skip)
            if fits:
                break
            victim = self._victim(skip) if self.preemption else None
            if victim is None:
                raise OutOfBlocks(f"step needs {need} blocks, "
                                  f"{self.pool.num_free() - claimed} free")
            self._preempt(victim)
            skip.add(id(victim))
            self.preempted.append(victim.req_id)
        for r, _ in picked:
            hit = hits.get(id(r))
            if hit is None:
                continue
            r.looked_up = True
            for b in hit:
                self.pool.claim(b)
            r.blocks = list(hit)
            r.num_computed = len(hit) * self.block_size
            r.ids = _pc.prefix_identities(r.tokens[:r.num_computed], self.block_size, r.namespace)
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
            if self.prefix_caching and r.tokens is not None:
                self._register(r)
            if r.is_decode:
                r.num_tokens += 1
            elif r.num_computed == r.num_tokens:
                r.is_decode = True
                r.num_tokens += 1
        self._last = []

    def _register(self, r) -> None:
        """Register the request's newly full prompt blocks under their identities."""
        bs = self.block_size
        full = min(r.num_computed, len(r.tokens)) // bs
        for j in range(len(r.ids), full):
            parent = r.ids[-1] if r.ids else _pc.scope_root(r.namespace)
            ident = _pc.next_identity(parent, r.tokens[j * bs:(j + 1) * bs])
            self.pool.register(r.blocks[j], ident)
            r.ids.append(ident)

    def free_request(self, req_id: int) -> None:
        r = self._find(req_id)
        self.pool.release(r.blocks)
        self.reqs.remove(r)
