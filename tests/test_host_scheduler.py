"""The C++ host scheduler (product) against the plain oracle scheduler and
the pages' printed traces.  Integer work: bit-exact."""
import numpy as np
import pytest

from chunked_prefill_paged_amd import BudgetExhausted, HostScheduler, OutOfBlocks, schedule_prompt
from oracle import schedule as osch
from tests.golden_io import ints, kv, rows


@pytest.mark.parametrize("row", rows("scheduler_traces.txt"), ids=lambda r: r[0])
def test_schedule_prompt_matches_pages(row):
    name, budget, decodes, prompt, bs, align, whole, expected = row
    args = (int(budget), int(decodes), int(prompt), int(bs), bool(int(align)))
    if expected == "ERROR":
        with pytest.raises(BudgetExhausted):
            schedule_prompt(*args)
        with pytest.raises(osch.BudgetExhausted):
            osch.schedule_prompt(*args)
        return
    got = schedule_prompt(*args)
    assert got == osch.schedule_prompt(*args)
    want = ints(expected)
    assert (got == want) if int(whole) else (got[:len(want)] == want)


@pytest.mark.parametrize("seed", range(12))
def test_schedule_prompt_random_agrees_with_oracle(seed):
    rng = np.random.default_rng(seed)
    for _ in range(50):
        budget = int(rng.integers(1, 3000))
        dec = int(rng.integers(0, budget + 2))
        prompt = int(rng.integers(0, 20000))
        bs = int(2 ** rng.integers(3, 8))
        align = bool(rng.integers(0, 2))
        try:
            want = osch.schedule_prompt(budget, dec, prompt, bs, align)
        except osch.BudgetExhausted:
            with pytest.raises(BudgetExhausted):
                schedule_prompt(budget, dec, prompt, bs, align)
            continue
        assert schedule_prompt(budget, dec, prompt, bs, align) == want


def _compare(batch, ob, max_blocks):
    assert list(batch["req_ids"]) == ob["req_ids"]
    assert list(batch["q_lens"]) == ob["q_lens"]
    assert list(batch["cu_seqlens_q"]) == ob["cu_seqlens_q"]
    assert list(batch["cached_seq_len"]) == ob["cached_seq_len"]
    assert batch["num_tokens"] == ob["num_tokens"]
    assert np.array_equal(batch["block_table"], np.array(ob["block_table"], dtype=np.int32)
                          .reshape(-1, max_blocks))
    assert list(batch["slot_mapping"]) == ob["slot_mapping"]


@pytest.mark.parametrize("seed", range(10))
def test_random_engine_runs_agree_with_oracle(seed):
    """Random mixes of prompts, prefix hits, decodes, steps and frees: every
    descriptor and the free count agree bit for bit."""
    rng = np.random.default_rng(100 + seed)
    bs = int(2 ** rng.integers(3, 6))
    nb = int(rng.integers(200, 600))
    budget = int(rng.integers(32, 700))
    max_blocks = 128
    cap = int(rng.choice([0, 0, 64, 200]))
    align = bool(rng.integers(0, 2))
    order = rng.permutation(nb).astype(np.int32)
    prod = HostScheduler(nb, bs, budget, max_blocks, cap, align, order)
    pool = osch.BlockPool(nb, order)
    orc = osch.Scheduler(pool, bs, budget, max_blocks, cap, align)
    live, next_id = [], 0
    for _ in range(60):
        action = rng.integers(0, 10)
        if action < 3:
            n = int(rng.integers(1, 1500))
            prefix = []
            if live and rng.integers(0, 2):
                donor = live[int(rng.integers(0, len(live)))]
                blocks = list(prod.request_blocks(donor))
                use = int(rng.integers(0, len(blocks) + 1))
                prefix = blocks[:use]
                if len(prefix) * bs >= n:
                    prefix = []
            try:
                osch_ok = True
                orc.add_request(next_id, n, prefix)
            except ValueError:
                osch_ok = False
            if osch_ok:
                prod.add_request(next_id, n, prefix)
                live.append(next_id)
            next_id += 1
        elif action < 4 and rng.integers(0, 2):
            n = int(rng.integers(2, 1200))
            done = int(rng.integers(0, n))
            try:
                orc.add_partial(next_id, n, done)
            except osch.OutOfBlocks:
                with pytest.raises(OutOfBlocks):
                    prod.add_partial(next_id, n, done)
                next_id += 1
                continue
            except ValueError:
                next_id += 1
                continue
            prod.add_partial(next_id, n, done)
            live.append(next_id)
            next_id += 1
        elif action < 4:
            ctx = int(rng.integers(1, 600))
            try:
                orc.add_decode(next_id, ctx)
            except osch.OutOfBlocks:
                with pytest.raises(OutOfBlocks):
                    prod.add_decode(next_id, ctx)
                next_id += 1
                continue
            prod.add_decode(next_id, ctx)
            live.append(next_id)
            next_id += 1
        elif action < 9:
            try:
                ob = orc.step()
            except osch.OutOfBlocks:
                with pytest.raises(OutOfBlocks):
                    prod.step()
                continue
            except ValueError:
                continue
            batch = prod.step()
            _compare(batch, ob, max_blocks)
            orc.commit()
            prod.commit()
        elif live:
            victim = live.pop(int(rng.integers(0, len(live))))
            orc.free_request(victim)
            prod.free_request(victim)
        assert prod.num_free_blocks() == pool.num_free()
        for blk in range(0, nb, 7):
            assert prod.refcount(blk) == pool.ref[blk]


def test_allocation_walkthrough_through_the_library():
    # "Prefill Processing", section "Block Allocation": 4096 cached tokens in
    # 32 shared blocks, 2048 per step at block_size 128 -> 48 then 64 blocks
    r = {x[0]: x for x in rows("allocation.txt")}["neuron_walkthrough"]
    bs, prefix, chunk, prompt, max_len = (int(x) for x in r[1:6])
    want = kv(r[6])
    width = -(-max_len // bs)
    assert width == int(want["row_width"])
    s = HostScheduler(200, bs, chunk, width)
    s.add_decode(1000, prefix)                 # the request that computed the prefix
    shared = s.request_blocks(1000)
    s.add_request(7, prompt, shared)
    s.free_request(1000)                       # it finishes; request 7 keeps the blocks
    assert s.refcount(int(shared[0])) == 1
    held, fresh = [], []
    for step in range(2):
        before = s.num_free_blocks()
        b = s.step()
        assert list(b["q_lens"]) == [chunk]
        fresh.append(before - s.num_free_blocks())
        held.append(s.request_info(7)["num_blocks"])
        if step == 0:
            assert int((b["block_table"][0][held[0]:] == 0).sum()) == int(want["null_after_step1"])
            assert list(b["block_table"][0][:32]) == list(shared)
        s.commit()
    assert held == ints(want["held"]) and fresh == ints(want["fresh"])


def test_incremental_allocation_32k():
    # "vLLM Chunked Prefill 如何改变 KV Cache 管理", sections 2.1 and 4
    r = {x[0]: x for x in rows("allocation.txt")}
    bs, _, chunk, prompt, max_len = (int(x) for x in r["vllm_32k"][1:6])
    want, want3 = kv(r["vllm_32k"][6]), kv(r["vllm_after3"][6])
    s = HostScheduler(4096, bs, chunk, -(-max_len // bs))
    s.add_request(1, prompt)
    fresh = []
    while not s.request_info(1)["is_decode"]:
        before = s.num_free_blocks()
        s.step()
        fresh.append(before - s.num_free_blocks())
        s.commit()
        if len(fresh) == 3:
            info = s.request_info(1)
            assert info["num_blocks"] == int(want3["held_after3"])
            assert info["num_computed"] == int(want3["computed_after3"])
    assert len(fresh) == int(want["steps"]) and set(fresh) == {int(want["fresh_each"])}
    assert sum(fresh) == int(want["total"])


def test_mixed_batch_of_config4_shape():
    # 256 decodes claim one token each; the 32k prompt at 30,720 cached gets 1792
    s = HostScheduler(40000, 16, 2048, 2048)
    for i in range(256):
        s.add_decode(i, 16 * (i + 1))
    s.add_request(999, 32768)
    b = s.step()
    assert list(b["q_lens"]) == [1] * 256 + [1792] and b["num_tokens"] == 2048
    assert list(b["cached_seq_len"][:2]) == [16, 32] and int(b["cached_seq_len"][-1]) == 0
