"""Pins of the host-side oracle (token budget, allocation, counters) against
the values the pages print (tests/golden/)."""
import pytest

from oracle import counters as oc
from oracle import schedule as osch
from tests.golden_io import ints, kv, rows


@pytest.mark.parametrize("row", rows("scheduler_traces.txt"), ids=lambda r: r[0])
def test_schedule_prompt_traces(row):
    name, budget, decodes, prompt, bs, align, whole, expected = row
    args = (int(budget), int(decodes), int(prompt), int(bs), bool(int(align)))
    if expected == "ERROR":
        with pytest.raises(osch.BudgetExhausted):
            osch.schedule_prompt(*args)
        return
    got = osch.schedule_prompt(*args)
    want = ints(expected)
    if int(whole):
        assert got == want
    else:
        assert got[:len(want)] == want
    assert sum(got) == int(prompt)


def test_cached_positions_follow_the_trace():
    traces = {r[0]: r for r in rows("scheduler_traces.txt")}
    for name, positions in rows("cached_positions.txt"):
        _, budget, decodes, prompt, bs, align, _, _ = traces[name]
        chunks = osch.schedule_prompt(int(budget), int(decodes), int(prompt))
        acc, got = 0, []
        for c in chunks:
            acc += c
            got.append(acc)
        assert got == ints(positions)


def test_alignment_only_when_the_rest_does_not_fit():
    # the last chunk (fits in the budget) is not cut; 508 -> 496 at bs16
    assert osch.schedule_prompt(512, 4, 2048, 16, True) == [496, 496, 496, 496, 64]
    assert osch.schedule_prompt(2048, 0, 1808, 16, True) == [1808]
    with pytest.raises(osch.BudgetExhausted):
        osch.schedule_prompt(20, 5, 100, 16, True)   # 15 tokens < one block


def test_invalid_arguments_are_refused():
    with pytest.raises(ValueError):
        osch.schedule_prompt(0, 0, 10)
    with pytest.raises(ValueError):
        osch.schedule_prompt(10, -1, 10)


def _alloc_case(name):
    for r in rows("allocation.txt"):
        if r[0] == name:
            return [int(x) for x in r[1:6]] + [kv(r[6])]
    raise KeyError(name)


def test_neuron_block_allocation_walkthrough():
    bs, prefix, chunk, prompt, max_len, want = _alloc_case("neuron_walkthrough")
    width = osch.cdiv(max_len, bs)
    assert width == int(want["row_width"])
    pool = osch.BlockPool(200)
    prefix_blocks = pool.allocate(prefix // bs)          # the cached prefix's owner
    s = osch.Scheduler(pool, bs, chunk, width)
    s.add_request(7, prompt, prefix_blocks)
    held, fresh = [], []
    for step in range(2):
        before = pool.num_free()
        batch = s.step()
        assert batch["q_lens"] == [chunk]
        fresh.append(before - pool.num_free())
        row = batch["block_table"][0]
        held.append(sum(1 for x in row[:len(s.reqs[0].blocks)]))
        if step == 0:
            assert len(row) - len(s.reqs[0].blocks) == int(want["null_after_step1"])
            assert all(x == 0 for x in row[len(s.reqs[0].blocks):])
        s.commit()
    assert held == ints(want["held"]) and fresh == ints(want["fresh"])
    assert pool.ref[prefix_blocks[0]] == 2                 # shared with the owner


def test_vllm_incremental_allocation():
    bs, _, chunk, prompt, max_len, want = _alloc_case("vllm_32k")
    pool = osch.BlockPool(4096)
    s = osch.Scheduler(pool, bs, chunk, osch.cdiv(max_len, bs))
    s.add_request(1, prompt)
    fresh = []
    while not s.reqs[0].is_decode:
        before = pool.num_free()
        s.step()
        fresh.append(before - pool.num_free())
        s.commit()
    assert len(fresh) == int(want["steps"])
    assert set(fresh) == {int(want["fresh_each"])} and sum(fresh) == int(want["total"])
    bs, _, chunk, prompt, max_len, want = _alloc_case("vllm_after3")
    pool = osch.BlockPool(4096)
    s = osch.Scheduler(pool, bs, chunk, osch.cdiv(max_len, bs))
    s.add_request(1, prompt)
    for _ in range(3):
        s.step()
        s.commit()
    assert len(s.reqs[0].blocks) == int(want["held_after3"])
    assert s.reqs[0].num_computed == int(want["computed_after3"])


def test_decode_first_budget_and_mixed_batch():
    # "Prefill Optimisation ...", section 2: decodes claim one token each and
    # the prefill chunk takes the rest (256 decodes + 1792 = 2048).
    pool = osch.BlockPool(60000)
    s = osch.Scheduler(pool, 16, 2048, 2048)
    for i in range(256):
        s.add_decode(i, 1024 + 16 * i)
    s.add_request(999, 32768)
    b = s.step()
    assert b["q_lens"] == [1] * 256 + [1792] and b["num_tokens"] == 2048
    assert b["cached_seq_len"][:3] == [1024, 1040, 1056] and b["cached_seq_len"][-1] == 0
    assert b["req_ids"][-1] == 999


def test_out_of_blocks_is_refused_without_side_effects():
    pool = osch.BlockPool(10)
    s = osch.Scheduler(pool, 16, 512, 64)
    s.add_request(1, 400)                          # needs 25 blocks
    with pytest.raises(osch.OutOfBlocks):
        s.step()
    assert pool.num_free() == 10 and s.reqs[0].blocks == []


def test_release_returns_blocks_after_last_reference():
    pool = osch.BlockPool(8)
    owner = pool.allocate(2)
    s = osch.Scheduler(pool, 4, 64, 16)
    s.add_request(1, 20, owner)
    pool.release(owner)                              # owner finishes; request still holds them
    assert pool.num_free() == 6
    s.free_request(1)
    assert pool.num_free() == 8


@pytest.mark.parametrize("name", ["section4", "exercise1"])
def test_pair_counts(name):
    r = {x[0]: kv(x[1]) for x in rows("pairs.txt")}[name]
    blocks = oc.full_prefix_blocks(int(r["prefix"]), int(r["block_size"]))
    cached = blocks * int(r["block_size"])
    fresh = int(r["prompt"]) - cached
    assert blocks == int(r["blocks"]) and cached == int(r["cached"]) and fresh == int(r["fresh"])
    assert fresh * cached == int(r["suffix_prefix"])
    assert oc.pairs(fresh, 0) == int(r["suffix_suffix"])
    assert oc.pairs(fresh, cached) == int(r["total"])
    assert oc.pairs(cached, 0) == int(r["skipped"])
    if "full" in r:
        assert oc.pairs(int(r["prompt"]), 0) == int(r["full"])


def test_quadratic_ratio_and_flops():
    r = {x[0]: kv(x[1]) for x in rows("pairs.txt")}["ratio_32k_4k"]
    ratio = oc.pairs(int(r["long"]), 0) / oc.pairs(int(r["short"]), 0)
    assert round(ratio) == int(r["ratio"])
    # 4 * L * H * pairs * d (2d for QK^T, 2d for PV per pair)
    assert oc.attention_flops(10, 32, 128) == 4 * 32 * 10 * 128
    # the 10k prompt at 2048: 50,005,000 pairs over its five chunks
    chunks = osch.schedule_prompt(2048, 0, 10000)
    c, total = 0, 0
    for n in chunks:
        total += oc.pairs(n, c)
        c += n
    assert total == oc.pairs(10000, 0) == 50005000


@pytest.mark.parametrize("name", ["section6", "exercise4"])
def test_kv_bytes(name):
    r = {x[0]: kv(x[1]) for x in rows("kv_bytes.txt")}[name]
    per_token = oc.kv_bytes_per_token(int(r["kv_heads"]), int(r["head_dim"]), int(r["elem_bytes"]),
                                      int(r["layers"]))
    assert per_token == int(r["per_token"])
    if "per_token_layer" in r:
        assert oc.kv_bytes_per_token(int(r["kv_heads"]), int(r["head_dim"]),
                                     int(r["elem_bytes"])) == int(r["per_token_layer"])
    assert per_token * int(r["tokens"]) == int(r["payload"])


def test_chunk_bytes_components():
    # one 2048-token chunk over 8192 cached at G=8, D=128, bf16: the cached KV
    # read alone is 8192 * 4096 bytes
    b0 = oc.chunk_bytes(2048, 0, 32, 8, 128, 2)
    b1 = oc.chunk_bytes(2048, 8192, 32, 8, 128, 2)
    assert b1 - b0 == 8192 * oc.kv_bytes_per_token(8, 128, 2)


def _check_chunk_bytes(fn):
    """Every term of the algorithmic bytes of a chunk, evaluated by hand for
    the 10k prompt's five chunks (G=8 KV heads, H=32, D=128, 2-byte
    elements): Q read 8192 B/token, new K and V read 4096 B/token and
    written to the cache 4096 B/token, cached K and V read 4096 B per cached
    token, O written 8192 B/token."""
    per_new = 8192 + 4096 + 4096 + 8192          # 24,576 B per active token
    per_cached = 4096
    hand = {(2048, 0): 50_331_648, (2048, 2048): 58_720_256, (2048, 4096): 67_108_864,
            (2048, 6144): 75_497_472, (1808, 8192): 77_987_840}
    for (n, c), total in hand.items():
        assert n * per_new + c * per_cached == total
        assert fn(n, c, 32, 8, 128, 2) == total
    # one token, nothing cached, H=1, G=1, D=1, 1-byte elements: Q, K, V,
    # the two cache writes and O are one byte each
    assert fn(1, 0, 1, 1, 1, 1) == 6
    # query heads touch only Q and O; KV heads only the K/V terms
    assert fn(10, 7, 3, 1, 1, 1) == 10 * 3 * 2 + 10 * 4 + 7 * 2
    assert fn(0, 7, 3, 1, 1, 1) == 14


def test_chunk_bytes_hand_evaluated():
    _check_chunk_bytes(oc.chunk_bytes)


@pytest.mark.parametrize("name,bad", [
    ("O write dropped", lambda n, c, H, G, D, e: oc.chunk_bytes(n, c, H, G, D, e) - n * H * D * e),
    ("cache write dropped", lambda n, c, H, G, D, e: oc.chunk_bytes(n, c, H, G, D, e) - 2 * n * G * D * e),
    ("cached V not counted", lambda n, c, H, G, D, e: oc.chunk_bytes(n, c, H, G, D, e) - c * G * D * e),
    ("Q sized by KV heads", lambda n, c, H, G, D, e: oc.chunk_bytes(n, c, H, G, D, e) - n * (H - G) * D * e),
])
def test_planted_chunk_bytes_mistake_is_caught(name, bad):
    with pytest.raises(AssertionError):
        _check_chunk_bytes(bad)
