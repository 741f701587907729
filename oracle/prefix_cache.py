"""Oracle for prefix-cache block identity and full-block prefix matching.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix ("Prefill Optimisation: Prefix Caching, Chunked Prefill,
and Disaggregation", section 3, "vLLM block hash chain", and the behaviour
its section 7 script prints):
* reuse is per full block; a partial last block is never shared;
* a block is the same block only if its own ordered token ids, its scope
  (a namespace that keeps tenants or models apart) and everything before it
  are the same, so one changed token changes the identity of its block and
  of every later block;
* a lookup walks the prompt's full blocks from the first and stops at the
  first block that is not known.

The pages build that identity with a cryptographic digest chained through
the parent's digest.  Here it is exact instead: every full block is a node
of one trie, reached from its scope's root by the token tuples of the
blocks before it, and its identity is the node's integer id.  Two blocks
share an identity exactly when scope and all tokens up to the block's end
agree, so no collision question arises.  Identities are only compared with
each other inside one process; the product's own digests are never
compared with them.
"""
from __future__ import annotations

# (parent node id, block token tuple) -> node id; a scope's root is keyed
# (-1, ("scope", name)).  The registry only grows; ids are process-local.
_nodes: dict = {}


def _intern(key) -> int:
    node = _nodes.get(key)
    if node is None:
        node = len(_nodes)
        _nodes[key] = node
    return node


def scope_root(scope: str) -> int:
    """Identity of the empty prefix under ``scope``."""
    return _intern((-1, ("scope", str(scope))))


def next_identity(parent: int, block_tokens) -> int:
    """Identity of the full block ``block_tokens`` that follows ``parent``."""
    return _intern((int(parent), tuple(int(t) for t in block_tokens)))


def prefix_identities(tokens, block_size: int, scope: str) -> list:
    """Identities of the full blocks of ``tokens``, first block first."""
    ids = []
    node = scope_root(scope)
    for start in range(0, len(tokens) - block_size + 1, block_size):
        node = next_identity(node, tokens[start:start + block_size])
        ids.append(node)
    return ids


class KnownBlocks:
    """A bare set of known full-block identities (no pool, no eviction):
    what a lookup against everything ever registered would reuse."""

    def __init__(self, block_size: int):
        if block_size <= 0:
            raise ValueError("block size must be positive")
        self.block_size = block_size
        self.ids = set()

    def add(self, tokens, scope: str = "default") -> int:
        """Make every full block of ``tokens`` known; returns their count."""
        ids = prefix_identities(list(tokens), self.block_size, scope)
        self.ids.update(ids)
        return len(ids)

    def hit_tokens(self, tokens, scope: str = "default") -> int:
        """Tokens covered by the leading run of known full blocks."""
        run = 0
        for ident in prefix_identities(list(tokens), self.block_size, scope):
            if ident not in self.ids:
                break
            run += 1
        return run * self.block_size
