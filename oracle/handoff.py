"""Sparse-attention hand-off: the top-k rows as physical cache slots, and
as the additive score mask the sparse attention applies.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Sources (web pages; cited by title and section):

* [HBM] "HBM index architecture design" (vLLM research notes), section 2.3:
  slot = block_table[req, pos // block_size] * block_size + pos % block_size
  (the same translation the write path uses, so the attention reads the
  keys the indexer scored).
* [RFC] "RFC: DeepseekV32 model support" (Ascend msmodeling), section 2.1.3,
  sparse MLA computation: after q k^T gives the score, a tensor of the
  score's shape holding 0 at the index_topk selected tokens and -inf
  elsewhere is added to the score (equivalent to keeping only those keys).

Readings where the pages are silent (listed in the design doc):
* the mask is fp32 [T, ld] over the same columns as the logits rows; every
  column of a row is written (0 for a selected token, -inf otherwise,
  including columns past the row's position);
* a -1 entry of a top-k row selects nothing and translates to slot -1, as
  does an index whose block-table entry is missing or negative.

Pins: tests/test_oracle_handoff.py -- the [HBM] 2.5 block row [3, 7, 12]
with the 2.3 formula worked by hand (the golden fixture shared with the
write path), the slot of every selected index equal to the slot the write
path stores that token at, and the mask's defining property: a softmax of
score + mask is zero exactly off the selected set and renormalises the
score over it.
"""

import numpy as np

from .indexer import PAGE_TOKENS, request_of_rows


def topk_to_slots(topk, block_table, query_start_loc):
    """Physical slot of every entry of the top-k rows [T, k] ([HBM] 2.3);
    -1 stays -1 and so does an index without a block-table page."""
    topk = np.asarray(topk, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    req = request_of_rows(query_start_loc, topk.shape[0])
    out = np.full(topk.shape, -1, dtype=np.int64)
    for t in range(topk.shape[0]):
        for j, idx in enumerate(topk[t]):
            if idx < 0 or idx // PAGE_TOKENS >= bt.shape[1]:
                continue
            page = int(bt[req[t], idx // PAGE_TOKENS])
            if page >= 0:
                out[t, j] = page * PAGE_TOKENS + idx % PAGE_TOKENS
    return out


def topk_mask(topk, ld):
    """fp32 [T, ld]: 0 at the columns a top-k row selects, -inf elsewhere
    ([RFC] 2.1.3)."""
    topk = np.asarray(topk, dtype=np.int64)
    mask = np.full((topk.shape[0], ld), -np.inf, dtype=np.float32)
    for t in range(topk.shape[0]):
        for idx in topk[t]:
            if 0 <= idx < ld:
                mask[t, idx] = 0.0
    return mask
