"""chunked_prefill_paged_amd: chunked-prefill / prefix-cached paged attention
for MI355X (gfx950).

The work happens in ``libchunked_prefill_attn.so`` (HIP kernels, C entry
points, host scheduler; see include/chunked_prefill_attn.h).  This package is
its thin Python binding.  Nothing falls back to Python or PyTorch compute: if
the library is missing, every entry point raises.
"""
from ._lib import BudgetExhausted, CpaError, OutOfBlocks, lib  # noqa: F401
from .attention import INLINE_DESC_INTS, AttnCall, cache_shapes  # noqa: F401
from .scheduler import HostScheduler, schedule_prompt  # noqa: F401
