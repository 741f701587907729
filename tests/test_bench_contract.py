"""bench.py's contract on the CPU: the refusal of more than one GPU, the exit
without a GPU, and the code digest that keys a recorded counter summary to
the kernel it was measured on (comment and whitespace edits keep it, code
edits void it)."""
import os
import shutil
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300,
                          env={**os.environ, "HIP_VISIBLE_DEVICES": ""})


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_no_gpu_exits_without_a_line():
    r = _run("--steps", "1", "--warmup", "1")
    if r.returncode == 0:
        pytest.skip("a GPU is visible here")
    assert r.stdout == ""


@pytest.fixture()
def tree(tmp_path, monkeypatch):
    """A copy of the kernel sources and the counter summary, with bench's
    root pointed at it."""
    for rel in bench.KERNEL_SOURCES + (bench.TRAFFIC_FILE,):
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def _edit(path, old, new):
    text = path.read_text()
    assert old in text
    path.write_text(text.replace(old, new, 1))


def test_comment_and_whitespace_edits_keep_the_digest(tree):
    src = tree / bench.KERNEL_SOURCES[0]
    before = bench.kernel_sources_sha256()
    _edit(src, "// ", "//   an added remark\n// ")
    _edit(src, "namespace cpa {", "namespace cpa { /* a block\n   remark */")
    _edit(src, "{\n", "{\n\n    \n")
    assert bench.kernel_sources_sha256() == before


def test_a_code_edit_changes_the_digest_and_voids_the_recorded_traffic(tree):
    summary = tree / bench.TRAFFIC_FILE                    # made current for the copied code
    lines = [f"source_sha256: {bench.kernel_sources_sha256()}" if ln.startswith("source_sha256:") else ln
             for ln in summary.read_text().splitlines()]
    summary.write_text("\n".join(lines) + "\n")
    assert bench.recorded_traffic() is not None
    src = tree / bench.KERNEL_SOURCES[0]
    before = bench.kernel_sources_sha256()
    _edit(src, "constexpr int kKeys = 64;", "constexpr int kKeys = 64 ;  // same value, other tokens\nint cpa_x;")
    assert bench.kernel_sources_sha256() != before
    assert bench.recorded_traffic() is None


def test_string_literals_are_part_of_the_digest(tree):
    """Inline asm text is code: a comment marker inside a string is kept and
    a change of the string changes the digest."""
    src = tree / bench.KERNEL_SOURCES[0]
    before = bench.kernel_sources_sha256()
    _edit(src, "s_nop 0", "s_nop 1")
    assert bench.kernel_sources_sha256() != before
    _edit(src, "s_nop 1", "s_nop 0 // not a comment")
    assert bench.kernel_sources_sha256() != before
