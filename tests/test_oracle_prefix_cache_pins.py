"""Pins of the prefix-cache oracle: the matching outcomes the pages print
(standalone cache and through the scheduler), the first-chunk-only lookup
scenario, bucket accounting, a hand-evaluated LRU trace, and planted
mistakes that each must fail a pin.  CPU only."""
import pytest

from oracle import prefix_cache as opc
from oracle import schedule as osch
from tests.golden_io import ints, kv, rows

GOLD = {r[0]: (int(r[1]), kv(r[2])) for r in rows("prefix_cache.txt")}


def test_pot_standalone_matching():
    bs, exp = GOLD["pot_test1"]
    cache = opc.KnownBlocks(bs)
    base = list(range(1, 2501))
    assert cache.add(base, "model_shared") == int(exp["inserted"])
    query = base + list(range(5000, 5500))
    hit = cache.hit_tokens(query, "model_shared")
    assert (hit, len(query) - hit) == (int(exp["cached"]), int(exp["fresh"]))
    bs, exp = GOLD["pot_test2"]
    seq = list(range(100, 164))
    cache.add(seq, "model_shared")
    mutated = list(seq)
    mutated[5] = 999999
    hit = cache.hit_tokens(mutated, "model_shared")
    assert (hit, len(mutated) - hit) == (int(exp["cached"]), int(exp["fresh"]))
    bs, exp = GOLD["pot_test3"]
    assert cache.hit_tokens(base, "tenant_isolated") == int(exp["cached"])


def test_one_changed_token_changes_every_later_identity():
    a = list(range(64))
    b = list(a)
    b[5] = 7777
    da, db = opc.prefix_identities(a, 16, "ns"), opc.prefix_identities(b, 16, "ns")
    assert len(da) == 4 and all(x != y for x, y in zip(da, db))
    assert opc.prefix_identities(a, 16, "ns") == da
    assert not set(opc.prefix_identities(a, 16, "other")) & set(da)
    # a change in the last block leaves the earlier identities alone
    c = list(a)
    c[63] = 1
    dc = opc.prefix_identities(c, 16, "ns")
    assert dc[:3] == da[:3] and dc[3] != da[3]
    # only full blocks have an identity
    assert len(opc.prefix_identities(a[:63], 16, "ns")) == 3


def _run(sched, rid):
    """Schedule and commit until request rid has finished its prompt; returns
    the fresh blocks it took per step."""
    fresh = []
    while True:
        before = len(sched._find(rid).blocks)
        sched.step()
        r = sched._find(rid)
        fresh.append(len(r.blocks) - before)
        sched.commit()
        if r.is_decode:
            return fresh


def _sched(num_blocks, bs, budget, max_blocks=4096):
    pool = osch.BlockPool(num_blocks)
    return pool, osch.Scheduler(pool, bs, budget, max_blocks, prefix_caching=True)


def test_pot_matching_through_the_scheduler():
    bs, exp = GOLD["pot_test1"]
    pool, s = _sched(1000, bs, 4096)
    base = list(range(1, 2501))
    s.add_request_tokens(1, base, "model_shared")
    _run(s, 1)
    assert len(pool.table) == int(exp["inserted"])
    s.free_request(1)
    s.add_request_tokens(2, base + list(range(5000, 5500)), "model_shared")
    b = s.step()
    assert b["cached_seq_len"] == [int(exp["cached"])] and b["q_lens"] == [int(exp["fresh"])]
    s.commit()
    s.free_request(2)
    _, exp3 = GOLD["pot_test3"]
    s.add_request_tokens(3, base, "tenant_isolated")
    assert s.step()["cached_seq_len"] == [int(exp3["cached"])]


def test_kvm_first_chunk_only_scenario():
    bs, exp = GOLD["kvm_3_1"]
    pool, s = _sched(2000, bs, 2048)
    system = [7 + (i * 7919) % 50000 for i in range(4096)]
    a = system + [60000 + i for i in range(256)]
    b = system + [70000 + i for i in range(512)]
    s.add_request_tokens("A", a)
    assert _run(s, "A") == ints(exp["a_fresh"])
    a_blocks = list(s._find("A").blocks)
    s.free_request("A")
    s.add_request_tokens("B", b)
    first = s.step()
    rb = s._find("B")
    hit = int(exp["b_hit"])
    assert first["cached_seq_len"] == [hit * bs]
    assert rb.blocks[:hit] == a_blocks[:hit]                 # A's first-chunk blocks
    assert not set(rb.blocks[hit:]) & set(a_blocks)          # nothing else of A's
    s.commit()
    computed = first["q_lens"][0]
    while not rb.is_decode:
        computed += s.step()["q_lens"][0]
        s.commit()
    assert computed == int(exp["b_computed"])
    # A's blocks for tokens 2048..4095 are still cached, unused by B
    assert all(pool.identity[x] is not None and pool.ref[x] == 0 for x in a_blocks[hit:256])


def test_three_buckets_partition_the_pool():
    pool, s = _sched(64, 4, 16)
    s.add_request_tokens(1, list(range(30)))
    s.add_request_tokens(2, list(range(100, 110)))
    for _ in range(3):
        s.step()
        s.commit()
        assert pool.num_active() + pool.num_reclaimable() + pool.num_empty() == 64
    s.free_request(1)
    assert pool.num_active() + pool.num_reclaimable() + pool.num_empty() == 64
    assert pool.num_reclaimable() == 7           # request 1's 7 full blocks (28 of 30 tokens)
    assert pool.num_free() == pool.num_empty() + pool.num_reclaimable()


def test_lru_eviction_trace():
    # pool of 4 blocks handed out 0,1,2,3; block_size 4; budget 16
    pool, s = _sched(4, 4, 16)
    x = list(range(1, 9))
    s.add_request_tokens("X", x)
    _run(s, "X")                      # X holds 0,1 (both full, registered)
    s.free_request("X")               # reclaimable, oldest first: 1, 0
    s.add_request_tokens("Y", list(range(100, 108)))
    _run(s, "Y")                      # Y takes the empty 2,3
    s.free_request("Y")               # reclaimable: 1, 0, 3, 2
    s.add_request_tokens("Z", [200, 201, 202])
    s.step()
    assert s._find("Z").blocks == [1]          # X's last block is evicted first
    s.commit()
    s.add_request_tokens("W", x)
    b = s.step()
    assert b["cached_seq_len"][-1] == 4        # X's first block still matches
    assert s._find("W").blocks == [0, 3]       # hit on 0, then the oldest left: 3


# --------------------------------------------------------------------------
# planted mistakes
# --------------------------------------------------------------------------
def _identity_without_parent(parent, block_tokens):
    # every block hangs off one root: content alone identifies it
    return _orig_next(-7, block_tokens)


def _root_without_scope(scope):
    return _orig_root("default")


_orig_next = opc.next_identity
_orig_root = opc.scope_root


def _release_mru(self, blocks):
    unused = []
    for blk in blocks:
        self.ref[blk] -= 1
        if self.ref[blk] == 0:
            unused.append(blk)
    for blk in unused:
        if self.identity[blk] is None:
            self.free.append(blk)
        else:
            self.lru[blk] = None
            self.lru.move_to_end(blk, last=False)      # newest first: evicted first


def test_block_content_at_another_position_does_not_match():
    # the chain, not the content alone, identifies a block: a query whose
    # first block equals a registered second block matches nothing
    cache = opc.KnownBlocks(4)
    cache.add([1, 2, 3, 4, 5, 6, 7, 8], "ns")
    assert cache.hit_tokens([5, 6, 7, 8, 9], "ns") == 0
    assert cache.hit_tokens([1, 2, 3, 4, 5, 6, 7, 8, 9], "ns") == 8


PINS = [test_one_changed_token_changes_every_later_identity,
        test_block_content_at_another_position_does_not_match,
        test_pot_standalone_matching, test_pot_matching_through_the_scheduler,
        test_kvm_first_chunk_only_scenario, test_three_buckets_partition_the_pool,
        test_lru_eviction_trace]


@pytest.mark.parametrize("name,target,attr,bad", [
    ("identity ignores the parent", opc, "next_identity", _identity_without_parent),
    ("identity ignores the scope", opc, "scope_root", _root_without_scope),
    ("most recently freed evicted first", osch.BlockPool, "release", _release_mru),
])
def test_planted_prefix_cache_mistake_is_caught(monkeypatch, name, target, attr, bad):
    monkeypatch.setattr(target, attr, bad)
    failures = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1, f"no pin caught: {name}"


def test_planted_lookup_beyond_the_first_chunk_is_caught(monkeypatch):
    orig = osch.Scheduler._take

    def _wide(self, remaining, used):
        # the lookup window (and only it) taken as the whole prompt
        import inspect
        caller = inspect.stack()[1]
        if "first = self._take" in (caller.code_context or [""])[0]:
            return remaining
        return orig(self, remaining, used)

    monkeypatch.setattr(osch.Scheduler, "_take", _wide)
    with pytest.raises(AssertionError):
        test_kvm_first_chunk_only_scenario()
