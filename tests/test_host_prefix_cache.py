"""Prefix caching in the C++ host scheduler (product) against the oracle:
the pages' scenarios and random engine runs with shared prompts, scopes,
frees and evictions.  Integer work: every descriptor, table and pool count
bit-exact."""
import numpy as np
import pytest

from chunked_prefill_paged_amd import HostScheduler, OutOfBlocks
from oracle import prefix_cache as opc
from oracle import schedule as osch
from tests.golden_io import ints, kv, rows
from tests.test_host_scheduler import _compare

GOLD = {r[0]: (int(r[1]), kv(r[2])) for r in rows("prefix_cache.txt")}


class Pair:
    def __init__(self, nb, bs, budget, max_blocks=4096, cap=0, align=False, order=None):
        self.max_blocks = max_blocks
        self.prod = HostScheduler(nb, bs, budget, max_blocks, cap, align, order, prefix_caching=True)
        self.pool = osch.BlockPool(nb, order)
        self.orc = osch.Scheduler(self.pool, bs, budget, max_blocks, cap, align, prefix_caching=True)

    def add(self, rid, tokens, ns="default"):
        self.prod.add_request_tokens(rid, tokens, ns)
        self.orc.add_request_tokens(rid, tokens, ns)

    def step(self):
        try:
            ob = self.orc.step()
        except osch.OutOfBlocks:
            with pytest.raises(OutOfBlocks):
                self.prod.step()
            return None
        pb = self.prod.step()
        _compare(pb, ob, self.max_blocks)
        self.check_pool()
        return pb

    def commit(self):
        self.prod.commit()
        self.orc.commit()
        self.check_pool()

    def free(self, rid):
        self.prod.free_request(rid)
        self.orc.free_request(rid)
        self.check_pool()

    def check_pool(self):
        st = self.prod.pool_stats()
        assert st == {"active": self.pool.num_active(), "reclaimable": self.pool.num_reclaimable(),
                      "empty": self.pool.num_empty()}
        assert self.prod.num_free_blocks() == self.pool.num_free()
        for r in self.orc.reqs:
            assert list(self.prod.request_blocks(r.req_id)) == r.blocks

    def run_prompt(self, rid):
        while not self.orc._find(rid).is_decode:
            assert self.step() is not None
            self.commit()


def test_pot_outcomes_through_the_product():
    bs, exp = GOLD["pot_test1"]
    p = Pair(1000, bs, 4096)
    base = list(range(1, 2501))
    p.add(1, base, "model_shared")
    p.run_prompt(1)
    p.free(1)
    assert p.prod.pool_stats()["reclaimable"] == int(exp["inserted"])
    query = base + list(range(5000, 5500))
    assert p.prod.prefix_match(query, "model_shared") == int(exp["cached"])
    p.add(2, query, "model_shared")
    b = p.step()
    assert list(b["cached_seq_len"]) == [int(exp["cached"])]
    assert list(b["q_lens"]) == [int(exp["fresh"])]
    p.commit()
    _, exp2 = GOLD["pot_test2"]
    seq = list(range(100, 164))
    p.add(3, seq, "model_shared")
    p.run_prompt(3)
    mutated = list(seq)
    mutated[5] = 999999
    assert p.prod.prefix_match(mutated, "model_shared") == int(exp2["cached"])
    _, exp3 = GOLD["pot_test3"]
    assert p.prod.prefix_match(base, "tenant_isolated") == int(exp3["cached"])


def test_kvm_first_chunk_only_through_the_product():
    bs, exp = GOLD["kvm_3_1"]
    p = Pair(2000, bs, 2048)
    system = [7 + (i * 7919) % 50000 for i in range(4096)]
    p.add(1, system + [60000 + i for i in range(256)])
    fresh = []
    while not p.orc._find(1).is_decode:
        before = len(p.prod.request_blocks(1))
        p.step()
        fresh.append(len(p.prod.request_blocks(1)) - before)
        p.commit()
    assert fresh == ints(exp["a_fresh"])
    a_blocks = list(p.prod.request_blocks(1))
    p.free(1)
    p.add(2, system + [70000 + i for i in range(512)])
    b = p.step()
    hit = int(exp["b_hit"])
    assert list(b["cached_seq_len"]) == [hit * bs]
    assert list(p.prod.request_blocks(2))[:hit] == a_blocks[:hit]
    computed = int(b["q_lens"][0])
    p.commit()
    while not p.orc._find(2).is_decode:
        computed += int(p.step()["q_lens"][0])
        p.commit()
    assert computed == int(exp["b_computed"])


def test_lru_trace_through_the_product():
    p = Pair(4, 4, 16)
    x = list(range(1, 9))
    p.add(10, x)
    p.run_prompt(10)
    p.free(10)
    p.add(11, list(range(100, 108)))
    p.run_prompt(11)
    p.free(11)
    p.add(12, [200, 201, 202])
    p.step()
    assert list(p.prod.request_blocks(12)) == [1]
    p.commit()
    p.add(13, x)
    b = p.step()
    assert int(b["cached_seq_len"][-1]) == 4
    assert list(p.prod.request_blocks(13)) == [0, 3]


@pytest.mark.parametrize("seed", range(12))
def test_random_prefix_cached_runs_agree_with_oracle(seed):
    """Prompts drawn as (shared system prompt, scope, private suffix), with
    decodes, frees and a pool small enough to evict: every step's descriptor,
    every table and the three bucket counts agree bit for bit."""
    rng = np.random.default_rng(500 + seed)
    bs = int(2 ** rng.integers(2, 5))
    nb = int(rng.integers(60, 300))
    budget = int(rng.integers(24, 400))
    cap = int(rng.choice([0, 0, 48]))
    align = bool(rng.integers(0, 2))
    order = rng.permutation(nb).astype(np.int32)
    p = Pair(nb, bs, budget, 256, cap, align, order)
    systems = [list(rng.integers(0, 1 << 32, size=int(rng.integers(0, 300)), dtype=np.uint64))
               for _ in range(4)]
    scopes = ["default", "tenant_a"]
    live, next_id = [], 0
    for _ in range(80):
        a = rng.integers(0, 10)
        if a < 3:
            sysp = systems[int(rng.integers(0, len(systems)))]
            suffix = list(rng.integers(0, 1 << 32, size=int(rng.integers(1, 200)), dtype=np.uint64))
            toks = [int(t) for t in sysp + suffix]
            ns = scopes[int(rng.integers(0, 2))]
            assert p.prod.prefix_match(toks, ns) == (
                len(p.pool.lookup(opc.prefix_identities(toks, bs, ns))) * bs)
            p.add(next_id, toks, ns)
            live.append(next_id)
            next_id += 1
        elif a < 4 and live:
            rid = live.pop(int(rng.integers(0, len(live))))
            p.free(rid)
        else:
            if p.step() is not None:
                p.commit()
        # finished prompts leave after a few decodes
        for r in list(p.orc.reqs):
            if r.is_decode and r.num_tokens - (r.tokens and len(r.tokens) or 0) > 3:
                p.free(r.req_id)
                live.remove(r.req_id)
