"""Pins of the oracle's preemption and long-prompt policies: the numbers the
pages print for a request preempted mid-prefill, a hand-evaluated
short-prompt-passes-long-prompt step, the all-or-nothing step without
preemption, and planted mistakes.  CPU only."""
import pytest

from oracle import schedule as osch
from tests.golden_io import kv, rows


def _case(name):
    for r in rows("allocation.txt"):
        if r[0] == name:
            return [int(x) for x in r[1:6]] + [kv(r[6])]
    raise KeyError(name)


def test_request_preempted_after_three_chunks():
    """'vLLM Chunked Prefill ...', section 4: preempted after 3 chunks, the
    request frees all its blocks and starts again from position 0."""
    bs, _, chunk, prompt, max_len, want = _case("vllm_preempt_after3")
    width = osch.cdiv(max_len, bs)
    # pool: an older decode C (32 blocks), then the 32k prompt A; room for
    # exactly A's first three chunks plus C's growth to 33 blocks
    nb = 32 + 3 * (chunk // bs) + 1
    pool = osch.BlockPool(nb)
    s = osch.Scheduler(pool, bs, chunk + 1, width, preemption=True)
    s.add_decode("C", 32 * bs)
    s.add_request("A", prompt)
    a = s._find("A")
    for _ in range(3):
        s.step()
        s.commit()
    assert a.num_computed == int(want["computed_before"]) and len(a.blocks) == int(want["released"])
    free_before = pool.num_free()
    batch = s.step()                         # A's 4th chunk does not fit: A is the newest holder
    assert s.preempted == ["A"]
    assert a.num_computed == int(want["computed_after"]) and a.blocks == []
    assert pool.num_free() - free_before == int(want["released"])    # C needed no new block
    assert batch["req_ids"] == ["C"]         # the step goes on without A
    s.commit()
    s.free_request("C")
    batch = s.step()                         # A resumes from position 0
    assert batch["req_ids"] == ["A"] and batch["cached_seq_len"] == [0]


def test_short_prompt_passes_a_long_one():
    """'vLLM Chunked Prefill ...', section 3.3: prompts longer than the
    threshold get at most that many tokens a step, and beyond the allowed
    number of long prompts a later long prompt waits while a short one
    behind it is scheduled.  Evaluated by hand for budget 2048, threshold
    512, one long prompt per step: L1 (4000) gets 512, L2 (3000) waits, S
    (100) gets 100."""
    pool = osch.BlockPool(1000)
    s = osch.Scheduler(pool, 16, 2048, 512, long_prefill_cap=512, max_long_partial_prefills=1)
    s.add_request("L1", 4000)
    s.add_request("L2", 3000)
    s.add_request("S", 100)
    b = s.step()
    assert b["req_ids"] == ["L1", "S"] and b["q_lens"] == [512, 100]
    # without the limit both long prompts get their 512
    pool2 = osch.BlockPool(1000)
    s2 = osch.Scheduler(pool2, 16, 2048, 512, long_prefill_cap=512)
    for rid, n in (("L1", 4000), ("L2", 3000), ("S", 100)):
        s2.add_request(rid, n)
    b2 = s2.step()
    assert b2["req_ids"] == ["L1", "L2", "S"] and b2["q_lens"] == [512, 512, 100]


def test_without_preemption_a_step_that_does_not_fit_changes_nothing():
    pool = osch.BlockPool(10)
    s = osch.Scheduler(pool, 16, 512, 64)
    s.add_decode("C", 100)                      # 7 blocks
    s.add_request("A", 400)                     # needs 25
    with pytest.raises(osch.OutOfBlocks):
        s.step()
    assert pool.num_free() == 3 and s._find("A").blocks == [] and s.preempted == []


# --------------------------------------------------------------------------
# planted mistakes
# --------------------------------------------------------------------------
def _preempt_keeps_progress(self, r):
    self.pool.release(r.blocks)
    r.blocks = []
    r.is_decode = False


PINS = [test_request_preempted_after_three_chunks, test_short_prompt_passes_a_long_one,
        test_without_preemption_a_step_that_does_not_fit_changes_nothing]


def test_planted_preemption_mistakes_are_caught(monkeypatch):
    monkeypatch.setattr(osch.Scheduler, "_preempt", _preempt_keeps_progress)
    with pytest.raises(AssertionError):
        test_request_preempted_after_three_chunks()


def test_planted_long_limit_ignored_is_caught(monkeypatch):
    orig = osch.Scheduler.__init__

    def init(self, *a, **k):
        orig(self, *a, **k)
        self.max_long = 0

    monkeypatch.setattr(osch.Scheduler, "__init__", init)
    with pytest.raises(AssertionError):
        test_short_prompt_passes_a_long_one()


def test_planted_oldest_victim_is_caught(monkeypatch):
    def oldest(self, skip):
        holders = [r for r in self.reqs if r.blocks and id(r) not in skip]
        return holders[0] if holders else None

    monkeypatch.setattr(osch.Scheduler, "_victim", oldest)
    with pytest.raises(AssertionError):
        test_request_preempted_after_three_chunks()
