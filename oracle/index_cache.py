"""IndexCache F/S layer rule and the layer loop.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source: [IC] "vLLM IndexCache practical guide: cross-layer top-k index reuse
for DeepSeek-V3.2 (DSA)" (blog.gitcode.com):

* section 2 ("How It Works"): F (full) layers compute the top-k and store it
  in one model-wide shared int32 buffer; S (shared) layers do not call the
  indexer and use what the previous F layer wrote in the same forward pass;
  nothing is kept across requests or batches;
* section 3 (parameters): index_topk_freq defaults to 1 (every layer
  computes), index_topk_pattern defaults to null and overrides the frequency
  when set; index_skip_topk_offset defaults to 2 and a layer is skipped when
  max(layer_id - offset + 1, 0) % freq != 0, so layers 0 and 1 are always F;
* section 4 (usage): one pattern character per DSA layer, 'S' skips, a layer
  beyond the pattern's length falls back to F; the 61-layer example pattern;
* section 5 item 3: MTP/nextn layers (layer_id >= num_hidden_layers) ignore
  the pattern and always build the full indexer, and a layer must not start
  as S or it would read a never-written buffer; they compute the top-k at
  draft step 0 and a runtime switch (index_share_for_mtp_iteration) turns
  them into reusers for the later draft steps.

[KVB] "GLM-5.3 inference pipeline (12): paging budget, prefix hits and
eviction of the main KV and indexer caches", engineering-judgement section,
item 4 (MTP and speculative decoding): the reuse within an MTP iteration
holds only with that switch on and one draft token per position (eagle
topk 1); with several, every draft position ranks its own top-k.

Reading (listed in the design doc): ``mtp_reuse`` is that combined condition; a
pass may start with an S layer only when it is an MTP layer reusing at a
draft step > 0 -- the buffer then holds the rows draft step 0 wrote.

Pins: tests/test_oracle_index_cache.py against the guide's worked examples
(61 layers with freq 4 / offset 2; the printed 61-character pattern; freq 1;
past-the-pattern and MTP layers), fixtures under tests/golden/; the MTP
draft-step switch on the cases the two passages state (step 0 computes,
later steps reuse only with the switch, trunk layers unaffected, a reuse
pass leaves the buffer as step 0 wrote it).
"""

import numpy as np

from . import indexer


def is_skip(layer_id, pattern=None, freq=1, offset=2, num_hidden_layers=None,
            mtp_draft_step=0, mtp_reuse=False):
    """True if layer ``layer_id`` is an S layer (reuses the shared buffer)."""
    if freq < 1:
        raise ValueError("index_topk_freq must be >= 1")
    if pattern is not None and any(c not in "FS" for c in pattern):
        raise ValueError("index_topk_pattern may contain only 'F' and 'S'")
    if mtp_draft_step < 0:
        raise ValueError("mtp_draft_step must be >= 0")
    if num_hidden_layers is not None and layer_id >= num_hidden_layers:
        # MTP/nextn layer: built full; reuses only after draft step 0
        return bool(mtp_reuse) and mtp_draft_step > 0
    if pattern is not None:
        return layer_id < len(pattern) and pattern[layer_id] == "S"
    return max(layer_id - offset + 1, 0) % freq != 0


def skip_mask(num_layers, pattern=None, freq=1, offset=2,
              num_hidden_layers=None, first_layer=0, mtp_draft_step=0,
              mtp_reuse=False):
    """is_skip for layers first_layer .. first_layer + num_layers - 1."""
    return np.array([is_skip(first_layer + l, pattern, freq, offset,
                             num_hidden_layers, mtp_draft_step, mtp_reuse)
                     for l in range(num_layers)], dtype=bool)


def _is_mtp_reuse(layer_id, num_hidden_layers, mtp_draft_step, mtp_reuse):
    return (num_hidden_layers is not None and layer_id >= num_hidden_layers
            and bool(mtp_reuse) and mtp_draft_step > 0)


def run(layers, block_table, query_start_loc, positions, ld, k, buffer,
        pattern=None, freq=1, offset=2, num_hidden_layers=None,
        first_layer=0, mtp_draft_step=0, mtp_reuse=False):
    """Layer loop over one forward pass.

    ``layers[l]`` (layer id first_layer + l) is a dict with ``q`` (float32
    [T,H,128], bf16 values), ``weights`` (float32 [T,H]) and ``k_cache``
    (uint8 [pages, 8448]) for an F layer; it is ignored for an S layer.
    ``buffer`` (int32 [max_tokens, k]) is the shared buffer, copied, not
    modified.  Returns (is_skip, final buffer, snapshots) where snapshots[l]
    is the buffer after layer l.
    """
    L = len(layers)
    mask = skip_mask(L, pattern, freq, offset, num_hidden_layers, first_layer,
                     mtp_draft_step, mtp_reuse)
    if L > 0 and mask[0] and not _is_mtp_reuse(
            first_layer, num_hidden_layers, mtp_draft_step, mtp_reuse):
        raise ValueError("the first layer is S: it would read a buffer no "
                         "layer has written in this pass")
    T = len(positions)
    B = np.array(buffer, dtype=np.int32, copy=True)
    snaps = []
    for l in range(L):
        if not mask[l]:
            lay = layers[l]
            codes, s = indexer.quantize_q(lay["q"])
            lg = indexer.indexer_logits(codes, s, lay["weights"],
                                        lay["k_cache"], block_table,
                                        query_start_loc, positions, ld)
            indexer.write_buffer(B, indexer.indexer_topk(lg, positions, k))
        snaps.append(B[:T].copy())
    return mask, B, snaps
