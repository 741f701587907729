"""Runs the host-scheduler tests against a library built from cpa_sched.cpp
alone (for example with AddressSanitizer and UndefinedBehaviorSanitizer):

    python tests/host_under_sanitizer.py LIBRARY [pytest args...]

The binding is pointed at LIBRARY; entry points it does not export (the
device side) are left out, and status names come from a table here.  Test
infrastructure only."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import ctypes  # noqa: E402

import pytest  # noqa: E402

from chunked_prefill_paged_amd import _lib  # noqa: E402

NAMES = {0: "ok", 1: "invalid argument", 2: "unsupported configuration", 3: "token budget exhausted",
         4: "out of KV-cache blocks", 5: "HIP error", 6: "workspace missing or too small",
         7: "unknown request"}


def main():
    path = os.path.abspath(sys.argv[1])
    probe = ctypes.CDLL(path)
    for name in list(_lib.SIGNATURES):
        if not hasattr(probe, name):
            del _lib.SIGNATURES[name]
    _lib.LIB_PATH = path
    _lib.status_string = lambda status: NAMES.get(status, "unknown status")
    files = [os.path.join(ROOT, "tests", f) for f in
             ("test_host_scheduler.py", "test_host_prefix_cache.py", "test_host_preemption.py")]
    return pytest.main(files + ["-q", "-p", "no:cacheprovider"] + sys.argv[2:])


if __name__ == "__main__":
    sys.exit(main())
