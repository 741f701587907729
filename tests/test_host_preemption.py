"""Preemption and the long-prompt limit in the C++ host scheduler (product)
against the oracle: the pages' preemption numbers, the short-passes-long
step, and random engine runs under block pressure.  Integer work: every
descriptor, table, preemption list and pool count bit-exact."""
import numpy as np
import pytest

from chunked_prefill_paged_amd import HostScheduler, OutOfBlocks
from oracle import schedule as osch
from tests.golden_io import kv, rows
from tests.test_host_scheduler import _compare


def _case(name):
    for r in rows("allocation.txt"):
        if r[0] == name:
            return [int(x) for x in r[1:6]] + [kv(r[6])]
    raise KeyError(name)


class Pair:
    def __init__(self, nb, bs, budget, max_blocks, cap=0, align=False, order=None, caching=False,
                 max_long=0):
        self.max_blocks = max_blocks
        self.prod = HostScheduler(nb, bs, budget, max_blocks, cap, align, order,
                                  prefix_caching=caching, max_long_partial_prefills=max_long,
                                  preemption=True)
        self.pool = osch.BlockPool(nb, order)
        self.orc = osch.Scheduler(self.pool, bs, budget, max_blocks, cap, align,
                                  prefix_caching=caching, max_long_partial_prefills=max_long,
                                  preemption=True)

    def step(self):
        try:
            ob = self.orc.step()
        except osch.OutOfBlocks:
            with pytest.raises(OutOfBlocks):
                self.prod.step()
            assert self.prod.last_preempted() == self.orc.preempted
            self.check()
            return None
        pb = self.prod.step()
        _compare(pb, ob, self.max_blocks)
        assert self.prod.last_preempted() == self.orc.preempted
        self.check()
        return pb

    def commit(self):
        self.prod.commit()
        self.orc.commit()
        self.check()

    def free(self, rid):
        self.prod.free_request(rid)
        self.orc.free_request(rid)
        self.check()

    def check(self):
        assert self.prod.num_free_blocks() == self.pool.num_free()
        for r in self.orc.reqs:
            info = self.prod.request_info(r.req_id)
            assert info["num_computed"] == r.num_computed and info["is_decode"] == r.is_decode
            assert list(self.prod.request_blocks(r.req_id)) == r.blocks


def test_preempted_after_three_chunks_through_the_product():
    bs, _, chunk, prompt, max_len, want = _case("vllm_preempt_after3")
    width = -(-max_len // bs)
    p = Pair(32 + 3 * (chunk // bs) + 1, bs, chunk + 1, width)
    for s in (p.prod, p.orc):
        s.add_decode(1, 32 * bs)
        s.add_request(2, prompt)
    for _ in range(3):
        p.step()
        p.commit()
    assert p.prod.request_info(2)["num_computed"] == int(want["computed_before"])
    free_before = p.prod.num_free_blocks()
    b = p.step()
    assert p.prod.last_preempted() == [2]
    assert p.prod.num_free_blocks() - free_before == int(want["released"])
    assert p.prod.request_info(2)["num_computed"] == int(want["computed_after"])
    assert list(b["req_ids"]) == [1]


def test_short_prompt_passes_a_long_one_through_the_product():
    p = Pair(1000, 16, 2048, 512, cap=512, max_long=1)
    for s in (p.prod, p.orc):
        for rid, n in ((1, 4000), (2, 3000), (3, 100)):
            s.add_request(rid, n)
    b = p.step()
    assert list(b["req_ids"]) == [1, 3] and list(b["q_lens"]) == [512, 100]


@pytest.mark.parametrize("seed", range(12))
def test_random_runs_under_block_pressure_agree_with_oracle(seed):
    rng = np.random.default_rng(900 + seed)
    bs = int(2 ** rng.integers(2, 5))
    nb = int(rng.integers(40, 160))
    budget = int(rng.integers(16, 300))
    cap = int(rng.choice([0, 32, 64]))
    max_long = int(rng.choice([0, 1, 2]))
    caching = bool(rng.integers(0, 2))
    align = bool(rng.integers(0, 2))
    order = rng.permutation(nb).astype(np.int32)
    p = Pair(nb, bs, budget, 128, cap, align, order, caching, max_long)
    shared = [int(x) for x in rng.integers(0, 1 << 31, size=int(rng.integers(0, 120)))]
    next_id, preemptions = 0, 0
    for _ in range(90):
        a = rng.integers(0, 10)
        if a < 3:
            n = int(rng.integers(1, 300))
            if caching and rng.integers(0, 2):
                toks = shared + [int(x) for x in rng.integers(0, 1 << 31, size=n)]
                for s in (p.prod, p.orc):
                    s.add_request_tokens(next_id, toks)
            else:
                for s in (p.prod, p.orc):
                    s.add_request(next_id, n)
            next_id += 1
        elif a < 4 and p.orc.reqs:
            p.free(p.orc.reqs[int(rng.integers(0, len(p.orc.reqs)))].req_id)
        else:
            if p.step() is not None:
                preemptions += len(p.orc.preempted)
                p.commit()
        for r in list(p.orc.reqs):            # long decodes leave
            if r.is_decode and len(r.blocks) > 12:
                p.free(r.req_id)
