"""Seeded synthetic inputs shaped like the indexer workloads on the pages.

This module only draws random numbers and lays bytes out; it holds none of
the indexer's arithmetic (no scoring, no top-k, no F/S rule) and imports
neither the HIP binding nor the CPU oracle, so both sides can consume exactly
the same inputs.

Recipe (numpy PCG64, one generator per batch, draws in this order):

1. per-request context lengths (where the workload draws them);
2. a permutation of the physical page pool; request r takes the next
   ceil(L_r / 64) pages of it as its block-table row (unused entries -1);
3. K: float32 N(0,1) [L_r, 128] per request in request order; an optional
   fraction of tokens (drawn without replacement) is multiplied by a boost;
4. q: float32 N(0,1) [T, H, 128], rounded to bf16 (round-to-nearest-even,
   torch's cast);
5. head weights: float32 N(0,1) / sqrt(H) [T, H].

The K cache is written the way the indexer-K write path stores it (GLM-5.3
KV/indexer cache budget article, sections on the SGLang buffer shape and on
eviction: per 64-token page, 64 x 128 FP8 e4m3fn key bytes, then 64 fp32
scales, 8448 bytes).  The FP8 encoding of K is torch's float32 ->
float8_e4m3fn cast (a library primitive) of K / scale with scale =
max|K| / 448 per token; it is input preparation, upstream of the hot path,
which starts from the cache bytes.  Tokens past a request's length inside its
last page are zero bytes.
"""

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import math
import os

import numpy as np
import torch

PAGE_TOKENS = 64
HEAD_DIM = 128
PAGE_KEY_BYTES = PAGE_TOKENS * HEAD_DIM
PAGE_BYTES = PAGE_KEY_BYTES + PAGE_TOKENS * 4
LD_ALIGN = 256

SEEDS = {"tiny": 0, "decode": 1, "prefill": 2, "index_cache": 3,
         "index_cache_pattern": 4, "long": 5}


@dataclass
class IndexerBatch:
    """One layer's inputs for the indexer (host memory)."""
    q_bf16: torch.Tensor          # bf16 [T, H, 128]
    weights: np.ndarray           # float32 [T, H]
    k_cache: np.ndarray           # uint8 [num_pages, 8448]
    block_table: np.ndarray       # int32 [R, max_pages]
    query_start_loc: np.ndarray   # int32 [R + 1]
    positions: np.ndarray         # int32 [T]
    k: int                        # index_topk
    ld: int                       # logits row stride (multiple of 256)
    contexts: list = field(default_factory=list)   # cached tokens per request
    name: str = ""

    @property
    def T(self):
        return int(self.positions.shape[0])

    @property
    def R(self):
        return int(self.block_table.shape[0])

    @property
    def H(self):
        return int(self.q_bf16.shape[1])

    @property
    def q_f32(self):
        """The bf16 q values as float32 (exact)."""
        return self.q_bf16.float().numpy()

    @property
    def visible_pairs(self):
        return int(np.sum(self.positions.astype(np.int64) + 1))


def round_up(x, a):
    return (x + a - 1) // a * a


def _quantize_tokens_fp8(k32):
    """float32 [N, 128] -> (codes uint8 [N, 128], scales float32 [N])."""
    amax = np.max(np.abs(k32), axis=1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    x = np.clip(k32 / safe[:, None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.numpy(), scale


def write_pages(k_cache, pages, k32):
    """Store tokens 0..N-1 of one request into its physical pages."""
    n = k32.shape[0]
    codes, scale = _quantize_tokens_fp8(k32)
    npg = (n + PAGE_TOKENS - 1) // PAGE_TOKENS
    pages = np.asarray(pages[:npg], dtype=np.int64)
    pad = npg * PAGE_TOKENS - n
    if pad:
        codes = np.concatenate([codes, np.zeros((pad, HEAD_DIM), np.uint8)])
        scale = np.concatenate([scale, np.zeros(pad, np.float32)])
    k_cache[pages, :PAGE_KEY_BYTES] = codes.reshape(npg, PAGE_KEY_BYTES)
    k_cache[pages, PAGE_KEY_BYTES:] = \
        scale.astype("<f4").view(np.uint8).reshape(npg, PAGE_TOKENS * 4)


def page_layout(rng, contexts, pool_pages=None, bt_width=None):
    """Draw the physical page of every logical page: a permutation of the
    pool, consumed request by request.  Returns (block_table, pool size)."""
    npages = [math.ceil(L / PAGE_TOKENS) for L in contexts]
    total = sum(npages)
    pool = total if pool_pages is None else pool_pages
    if pool < total:
        raise ValueError("page pool smaller than the pages needed")
    perm = rng.permutation(pool).astype(np.int32)
    width = max(npages + [1]) if bt_width is None else max(bt_width, 1)
    block_table = np.full((len(contexts), width), -1, dtype=np.int32)
    cur = 0
    for r, n in enumerate(npages):
        block_table[r, :n] = perm[cur: cur + n]
        cur += n
    return block_table, pool


def build_batch(rng, contexts, positions, H, k, pool_pages=None,
                boost_frac=0.0, boost=4.0, name="", bt_width=None,
                layout=None):
    """Generic builder.

    ``contexts[r]`` cached tokens for request r; ``positions[r]`` the list of
    query positions of request r (each < contexts[r]).  Rows are laid out
    request by request (query_start_loc).  ``layout`` = (block_table, pool)
    reuses a page layout drawn earlier instead of drawing one.
    """
    R = len(contexts)
    if layout is None:
        layout = page_layout(rng, contexts, pool_pages, bt_width)
    block_table, pool = layout
    k_cache = np.zeros((pool, PAGE_BYTES), dtype=np.uint8)
    for r, L in enumerate(contexts):
        pages = block_table[r, : math.ceil(L / PAGE_TOKENS)]
        k32 = rng.standard_normal((L, HEAD_DIM), dtype=np.float32)
        if boost_frac > 0:
            nb = int(round(boost_frac * L))
            idx = rng.choice(L, size=nb, replace=False)
            k32[idx] *= np.float32(boost)
        write_pages(k_cache, pages, k32)
    qsl = np.zeros(R + 1, dtype=np.int32)
    qsl[1:] = np.cumsum([len(p) for p in positions])
    pos = np.concatenate([np.asarray(p, dtype=np.int32) for p in positions]) \
        if R else np.zeros(0, np.int32)
    T = int(pos.shape[0])
    q32 = rng.standard_normal((T, H, HEAD_DIM), dtype=np.float32)
    q_bf16 = torch.from_numpy(q32).to(torch.bfloat16)
    w = (rng.standard_normal((T, H), dtype=np.float32)
         / np.float32(math.sqrt(H))).astype(np.float32)
    ld = round_up(max(int(pos.max()) + 1 if T else 1, 1), LD_ALIGN)
    return IndexerBatch(q_bf16=q_bf16, weights=w, k_cache=k_cache,
                        block_table=block_table.copy(), query_start_loc=qsl,
                        positions=pos, k=k, ld=ld, contexts=list(contexts),
                        name=name)


def tiny(seed=SEEDS["tiny"]):
    """1 request, 256 cached tokens (4 pages, permuted), 8 queries at
    positions 248..255, 4 heads, index_topk 32."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return build_batch(rng, [256], [list(range(248, 256))], H=4, k=32,
                       name="tiny")


def decode(seed=SEEDS["decode"], R=64, lo=1024, hi=8192, H=64, k=2048,
           pool_pages=16384):
    """R requests with contexts uniform in [lo, hi], one query each at the
    last position, pages drawn from a shuffled pool of 16384 pages."""
    rng = np.random.Generator(np.random.PCG64(seed))
    L = rng.integers(lo, hi, size=R, endpoint=True).tolist()
    return build_batch(rng, L, [[x - 1] for x in L], H=H, k=k,
                       pool_pages=pool_pages, name="decode",
                       bt_width=math.ceil(hi / PAGE_TOKENS))


def prefill(seed=SEEDS["prefill"], prefix=32768, chunk=8192, H=64, k=2048):
    """1 request: a cached prefix plus a chunk of new queries at positions
    prefix..prefix+chunk-1 (their own keys are in the cache), causal."""
    rng = np.random.Generator(np.random.PCG64(seed))
    L = prefix + chunk
    return build_batch(rng, [L], [list(range(prefix, L))], H=H, k=k,
                       name="prefill")


def long_context(seed=SEEDS["long"], context=1 << 20, rows=16, H=64, k=2048,
                 boost_frac=0.01):
    """1 request with a 1M-token cache (16384 shuffled pages), ``rows``
    consecutive decode queries at the tail; 1% of tokens boosted x4."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return build_batch(rng, [context], [list(range(context - rows, context))],
                       H=H, k=k, boost_frac=boost_frac, name="long")


def index_cache_pattern(num_layers=61, seed=SEEDS["index_cache_pattern"]):
    """A seeded random F/S pattern, first character forced to 'F'."""
    rng = np.random.Generator(np.random.PCG64(seed))
    chars = np.where(rng.random(num_layers) < 0.5, "F", "S")
    chars[0] = "F"
    return "".join(chars.tolist())


def index_cache_layers(full_layers, seed=SEEDS["index_cache"], R=32,
                       context=16384, H=64, k=2048, workers=None):
    """Independent per-layer inputs for the IndexCache stack.

    All layers share one batch of R decode requests (context tokens each, one
    query at the last position) and so one block table, drawn from ``seed``;
    every listed layer gets its own K cache, q and weights from its own PCG64
    stream spawned from ``seed``.  Layers are drawn on up to ``workers``
    threads (default: the usable cores, at most 16); each layer's bytes
    depend only on its own stream, so the result does not depend on the
    thread count.  Returns {layer: IndexerBatch}.
    """
    ss = np.random.SeedSequence(seed)
    n_streams = (max(full_layers) + 1) if full_layers else 0
    kids = ss.spawn(n_streams + 1)
    contexts = [context] * R
    layout = page_layout(np.random.Generator(np.random.PCG64(kids[0])),
                         contexts)

    def one(l):
        rng = np.random.Generator(np.random.PCG64(kids[l + 1]))
        return build_batch(rng, contexts, [[context - 1]] * R, H=H, k=k,
                           name=f"index_cache_layer{l}", layout=layout)

    if workers is None:
        workers = min(16, len(os.sched_getaffinity(0)))
    layers = list(full_layers)
    if workers <= 1 or len(layers) <= 1:
        return {l: one(l) for l in layers}
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return dict(zip(layers, ex.map(one, layers)))
