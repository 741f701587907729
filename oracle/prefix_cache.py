"""Oracle for prefix-cache block identity: the parent-chained block hash and
full-block prefix matching.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Prefill Optimisation: Prefix Caching, Chunked Prefill, and
Disaggregation", section 3 ("vLLM block hash chain") and section 7 (the
pedagogical prefix cache):
* the cache is keyed per full block; a block's digest covers its parent
  block's digest, the scope (namespace) and the block's ordered token ids,
  so a change anywhere earlier changes every later digest;
* only full blocks are hashed and reused (tokens in multiples of the block
  size);
* matching walks the chain from the first block and stops at the first
  block whose digest is unknown.

The digest here follows the section 7 construction: SHA-256 over the
parent digest (hex text, "ROOT" for the first block) and the namespace, both
as UTF-8, then every token id as 4 unsigned big-endian bytes.
"""
from __future__ import annotations

import hashlib

ROOT = "ROOT"


def block_hash(parent: str, block_tokens, namespace: str) -> str:
    """Hex digest of one full block given its parent's digest."""
    h = hashlib.sha256()
    h.update(parent.encode("utf-8"))
    h.update(namespace.encode("utf-8"))
    for tok in block_tokens:
        h.update(int(tok).to_bytes(4, byteorder="big", signed=False))
    return h.hexdigest()


def chain(tokens, block_size: int, namespace: str) -> list:
    """Digests of the full blocks of ``tokens``, in order."""
    out, parent = [], ROOT
    for i in range(len(tokens) // block_size):
        parent = block_hash(parent, tokens[i * block_size:(i + 1) * block_size], namespace)
        out.append(parent)
    return out


class PrefixCache:
    """Set of known block digests (no pool): what ``match_prefix`` can reuse."""

    def __init__(self, block_size: int):
        if block_size <= 0:
            raise ValueError("block_size must be positive")
        self.block_size = block_size
        self.known = set()

    def insert_sequence(self, tokens, namespace: str = "default") -> int:
        """Register every full block of ``tokens``; returns how many."""
        digests = chain(list(tokens), self.block_size, namespace)
        self.known.update(digests)
        return len(digests)

    def match_prefix(self, tokens, namespace: str = "default"):
        """(cached tokens, fresh tokens): the longest run of known full
        blocks from the start, then the rest."""
        tokens = list(tokens)
        n = 0
        for d in chain(tokens, self.block_size, namespace):
            if d not in self.known:
                break
            n += 1
        split = n * self.block_size
        return tokens[:split], tokens[split:]
