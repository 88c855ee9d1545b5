"""Seeded synthetic request streams for the block manager.

Draws only: prompts (some starting with one of a few shared prefixes, so that
full prefix blocks repeat across requests), the tokens each request will
decode, and the random choices a test scheduler makes.  No block-manager
logic lives here.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class Request:
    prompt: np.ndarray         # int32 token ids
    decode_tokens: np.ndarray  # int32 ids appended one per decode step


def request_stream(seed: int, num_requests: int, block_size: int, *, vocab: int = 50,
                   num_prefixes: int = 3, share_prob: float = 0.6,
                   max_prefix_blocks: int = 3, max_suffix: int | None = None,
                   max_decode: int | None = None) -> list[Request]:
    """Prompts = optional shared prefix (whole blocks, sometimes plus a
    partial block) + a random suffix; a small vocabulary makes equal blocks
    under different prefixes common too."""
    rng = np.random.default_rng(seed)
    max_suffix = max_suffix or 3 * block_size
    max_decode = max_decode or 3 * block_size
    prefixes = []
    for _ in range(num_prefixes):
        n = int(rng.integers(1, max_prefix_blocks + 1)) * block_size
        if rng.random() < 0.3:
            n += int(rng.integers(1, block_size))
        prefixes.append(rng.integers(0, vocab, n).astype(np.int32))
    out = []
    for _ in range(num_requests):
        pre = prefixes[int(rng.integers(num_prefixes))] if rng.random() < share_prob else \
            np.zeros(0, np.int32)
        suffix = rng.integers(0, vocab, int(rng.integers(1, max_suffix + 1))).astype(np.int32)
        dec = rng.integers(0, vocab, int(rng.integers(1, max_decode + 1))).astype(np.int32)
        out.append(Request(np.concatenate([pre, suffix]).astype(np.int32), dec))
    return out
