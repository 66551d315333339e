"""Seeded synthetic inputs for position-free paged prefill attention.

This module builds the *inputs* of one prefill step and nothing else: request
layouts made of block-aligned segments, the paged placement of every token,
the per-block descriptors, and N(0,1) values for Q, K and V. It holds none of
the method's arithmetic (no rotation, no mask evaluation, no softmax); both the
CPU oracle and the GPU path consume what it produces.

Request layouts follow the Block-Attention submission recipe of "MiniPIC:
Flexible Position-Independent Caching in <100LOC", §3.3.1: a system prompt
padded to a 16-token block boundary, documents that each start a new span
(SSep) and are padded to a block boundary, and a final task segment marked
PDep. §3.1.1 of the same page defines the three primitives (padding, SSep,
PDep). Padding tokens are ordinary tokens here: they get values and positions
like any other token.

Random draws use numpy's PCG64 in a fixed order: structure first, then K and V
for every unique context token (shared pool spans first), then Q.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

BLOCK = 16

# Per-block flag bits, as passed to the library.
FLAG_PDEP = 1
FLAG_GLOBAL = 2


# --------------------------------------------------------------------------
# bf16 storage helpers (bit manipulation only)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 with round-to-nearest-even; returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # u + 0x7FFF + lsb cannot wrap for any non-NaN input (largest: 0xFF800000 + 0x8000)
    t = (u >> 16) & np.uint32(1)
    t += u
    t += np.uint32(0x7FFF)
    t >>= 16
    r = t.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# Request structure
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Segment:
    """A run of context tokens that starts at a block boundary.

    kind:    'span'   - an SSep span (or the system prompt): attends within itself
             'pdep'   - a PDep segment: attends to everything before it
             'global' - a shared prefix whose blocks every later query may see
    length:  token count (already padded by the caller where padding applies)
    fresh:   True if its tokens are computed in this step (they are the query
             rows, and their K/V are written to the cache during the step);
             False if its K/V are already cached (written at set-up).
    pool:    index of a shared pool span; the segment then reuses that span's
             physical blocks and values (implies fresh=False).
    """
    kind: str
    length: int
    fresh: bool = True
    pool: Optional[int] = None


def pad_to_block(n: int) -> int:
    return ((n + BLOCK - 1) // BLOCK) * BLOCK


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                   # 'f32' or 'bf16'
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    rope_theta: float
    max_pos: int
    block_size: int
    # structure
    segments: List[List[Segment]]        # per request
    seg_start: List[List[int]]           # per request, ctx index of each segment start
    ctx_len: np.ndarray                  # [R] int32
    max_blocks_per_req: int
    block_table: np.ndarray              # [R, MB] int32 (physical block per logical block)
    logical_pos: np.ndarray              # [R, MB*16] int32
    span_id: np.ndarray                  # [R, MB] int32
    blk_flags: np.ndarray                # [R, MB] uint8
    q_indptr: np.ndarray                 # [R+1] int32
    q_ctx_idx: np.ndarray                # [total_q] int32
    # token data: unique tokens, each living in exactly one physical slot
    tok_slot: np.ndarray                 # [U] int64
    tok_of_ctx: List[np.ndarray]         # per request [L_r] -> unique token id
    num_blocks: int
    k_tok: np.ndarray                    # [U, Hkv, D] float32 or uint16 bits
    v_tok: np.ndarray                    # [U, Hkv, D]
    q: np.ndarray                        # [total_q, Hq, D] float32 or uint16 bits
    new_tok: np.ndarray                  # unique ids written during the step (query tokens, in q order)
    setup_tok: np.ndarray                # unique ids written at set-up (cached tokens)

    # ---- convenience views (no arithmetic beyond dtype decoding) ----
    @property
    def num_reqs(self) -> int:
        return len(self.segments)

    @property
    def total_q(self) -> int:
        return int(self.q_indptr[-1])

    @property
    def max_q_len(self) -> int:
        return int(np.max(np.diff(self.q_indptr))) if self.num_reqs else 0

    @property
    def max_ctx_len(self) -> int:
        return int(self.ctx_len.max()) if self.num_reqs else 0

    def as_f32(self, a: np.ndarray) -> np.ndarray:
        return bf16_bits_to_f32(a) if self.dtype == "bf16" else np.asarray(a, np.float32)

    def q_f64(self) -> np.ndarray:
        return self.as_f32(self.q).astype(np.float64)

    def request_dense(self, r: int):
        """Dense per-request K~, V (float64), positions and query rows.

        Values are gathered by token identity, never through the paged cache,
        so a paging bug on the GPU side cannot be mirrored here.
        """
        ids = self.tok_of_ctx[r]
        L = int(self.ctx_len[r])
        k = self.as_f32(self.k_tok[ids]).astype(np.float64)
        v = self.as_f32(self.v_tok[ids]).astype(np.float64)
        pos = self.logical_pos[r, :L].astype(np.int64)
        nb = (L + self.block_size - 1) // self.block_size
        span = self.span_id[r, :nb].astype(np.int64)
        flags = self.blk_flags[r, :nb].astype(np.int64)
        q0, q1 = int(self.q_indptr[r]), int(self.q_indptr[r + 1])
        q = self.as_f32(self.q[q0:q1]).astype(np.float64) if q1 > q0 else \
            np.zeros((0, self.num_q_heads, self.head_dim))
        qc = self.q_ctx_idx[q0:q1].astype(np.int64)
        return dict(q=q, q_ctx=qc, k=k, v=v, pos=pos, span_id=span, flags=flags)

    def pool_tokens_in_setup(self) -> np.ndarray:
        return self.setup_tok

    def query_segments(self, r: int):
        """(start, length, kind) of each segment of request r (host logic)."""
        return [(s0, seg.length, seg.kind) for s0, seg in zip(self.seg_start[r], self.segments[r])]


def build(name: str, requests: Sequence[Sequence[Segment]], *, pool_lengths: Sequence[int] = (),
          num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: str, rope_theta: float,
          max_pos: int, seed: int, rng: Optional[np.random.Generator] = None,
          positions: Optional[Sequence[np.ndarray]] = None,
          span_ids: Optional[Sequence[np.ndarray]] = None,
          extra_blocks: int = 0) -> Workload:
    """Lay out `requests` in a paged cache and draw values.

    `rng`, if given, must be the generator that already drew the structure so
    that the draw order stays structure → K/V → Q.
    """
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    R = len(requests)
    # --- allocate unique tokens: pool spans first, then per-request private segments
    block_owner = []          # allocation order of logical blocks (token-id base per block)
    tok_count = 0
    pool_base = []
    for plen in pool_lengths:
        pool_base.append(tok_count)
        nb = (plen + BLOCK - 1) // BLOCK
        for b in range(nb):
            block_owner.append(tok_count + b * BLOCK)
        tok_count += nb * BLOCK
    tok_of_ctx = []
    seg_starts = []
    seg_tok_base = []         # per request per segment: base unique id
    for r, segs in enumerate(requests):
        ids = []
        starts = []
        bases = []
        c = 0
        for si, seg in enumerate(segs):
            if c % BLOCK != 0:
                raise ValueError("every segment must start at a block boundary (pad the previous one)")
            starts.append(c)
            if seg.pool is not None:
                if pool_lengths[seg.pool] != seg.length:
                    raise ValueError("pool segment length mismatch")
                base = pool_base[seg.pool]
            else:
                base = tok_count
                nb = (seg.length + BLOCK - 1) // BLOCK
                for b in range(nb):
                    block_owner.append(tok_count + b * BLOCK)
                tok_count += nb * BLOCK
            bases.append(base)
            ids.append(np.arange(base, base + seg.length, dtype=np.int64))
            c += seg.length
        tok_of_ctx.append(np.concatenate(ids) if ids else np.zeros(0, np.int64))
        seg_starts.append(starts)
        seg_tok_base.append(bases)
    num_alloc_blocks = len(block_owner)
    num_blocks = num_alloc_blocks + extra_blocks
    # physical placement: a seeded permutation so that gathers are non-contiguous
    perm = rng.permutation(num_blocks)[:num_alloc_blocks]
    # unique token id -> physical slot
    tok_slot = np.full(tok_count, -1, dtype=np.int64)
    for ab, base in enumerate(block_owner):
        phys = int(perm[ab])
        tok_slot[base:base + BLOCK] = phys * BLOCK + np.arange(BLOCK)
    # --- per-request descriptors
    ctx_len = np.array([len(t) for t in tok_of_ctx], dtype=np.int32)
    MB = max(1, max(((int(L) + BLOCK - 1) // BLOCK for L in ctx_len), default=1))
    block_table = np.zeros((R, MB), np.int32)
    logical_pos = np.zeros((R, MB * BLOCK), np.int32)
    span_id = np.zeros((R, MB), np.int32)
    blk_flags = np.zeros((R, MB), np.uint8)
    q_ctx = []
    new_tok = []
    for r, segs in enumerate(requests):
        L = int(ctx_len[r])
        nb = (L + BLOCK - 1) // BLOCK
        ids = tok_of_ctx[r]
        for b in range(nb):
            block_table[r, b] = tok_slot[ids[b * BLOCK]] // BLOCK
        if positions is not None and positions[r] is not None:
            logical_pos[r, :L] = positions[r]
        else:
            logical_pos[r, :L] = np.arange(L, dtype=np.int32)
        for si, seg in enumerate(segs):
            s0 = seg_starts[r][si]
            b0 = s0 // BLOCK
            b1 = (s0 + seg.length + BLOCK - 1) // BLOCK
            sid = si if span_ids is None else int(span_ids[r][si])
            span_id[r, b0:b1] = sid
            if seg.kind == "pdep":
                blk_flags[r, b0:b1] |= FLAG_PDEP
            elif seg.kind == "global":
                blk_flags[r, b0:b1] |= FLAG_GLOBAL
            elif seg.kind != "span":
                raise ValueError(seg.kind)
            if seg.fresh and seg.pool is None:
                q_ctx.append((r, np.arange(s0, s0 + seg.length, dtype=np.int32)))
                new_tok.append(ids[s0:s0 + seg.length])
    q_indptr = np.zeros(R + 1, np.int32)
    per_r = [[] for _ in range(R)]
    for r, a in q_ctx:
        per_r[r].append(a)
    q_ctx_idx = []
    for r in range(R):
        a = np.concatenate(per_r[r]) if per_r[r] else np.zeros(0, np.int32)
        q_ctx_idx.append(a)
        q_indptr[r + 1] = q_indptr[r] + len(a)
    q_ctx_idx = np.concatenate(q_ctx_idx) if q_ctx_idx else np.zeros(0, np.int32)
    new_tok = np.concatenate([tok_of_ctx[r][qc] for r, qc in
                              zip(range(R), np.split(q_ctx_idx, q_indptr[1:-1]))]) \
        if len(q_ctx_idx) else np.zeros(0, np.int64)
    written = np.zeros(tok_count, bool)
    written[new_tok] = True
    setup_tok = np.nonzero(~written)[0]
    # --- values: K~ and V for every unique token, then Q
    shape = (tok_count, num_kv_heads, head_dim)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    q = rng.standard_normal((int(q_indptr[-1]), num_q_heads, head_dim), dtype=np.float32)
    if dtype == "bf16":
        k, v, q = f32_to_bf16_bits(k), f32_to_bf16_bits(v), f32_to_bf16_bits(q)
    elif dtype != "f32":
        raise ValueError(dtype)
    return Workload(name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, rope_theta=float(rope_theta), max_pos=int(max_pos),
                    block_size=BLOCK, segments=[list(s) for s in requests], seg_start=seg_starts,
                    ctx_len=ctx_len, max_blocks_per_req=MB, block_table=block_table,
                    logical_pos=logical_pos, span_id=span_id, blk_flags=blk_flags,
                    q_indptr=q_indptr, q_ctx_idx=q_ctx_idx, tok_slot=tok_slot,
                    tok_of_ctx=tok_of_ctx, num_blocks=num_blocks, k_tok=k, v_tok=v, q=q,
                    new_tok=new_tok, setup_tok=setup_tok)


# --------------------------------------------------------------------------
# The five benchmark workloads and smaller parity variants
# --------------------------------------------------------------------------

def _c1(seed=1, cached_spans=False):
    """Tiny fp32 case: 4 q heads, 2 KV heads, d 64; two 32-token SSep spans and a
    16-token PDep query; logical positions 0..79; theta 1e4."""
    segs = [Segment("span", 32, fresh=not cached_spans), Segment("span", 32, fresh=not cached_spans),
            Segment("pdep", 16)]
    return build("c1" + ("_cached" if cached_spans else ""), [segs], num_q_heads=4, num_kv_heads=2,
                 head_dim=64, dtype="f32", rope_theta=1e4, max_pos=128, seed=seed)


def _c2(seed=2):
    """Llama-3.1-8B attention shape in bf16: system prompt 512, ten 192-token SSep
    spans, 64-token PDep question, one request, every token computed now."""
    segs = [Segment("span", 512)] + [Segment("span", 192) for _ in range(10)] + [Segment("pdep", 64)]
    return build("c2", [segs], num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                 rope_theta=5e5, max_pos=32768, seed=seed)


def _c3(seed=3, num_reqs=16, pool=40, span_len=192, per_req=10, q_len=64, name="c3"):
    """16 concurrent requests drawing 10 of 40 cached 192-token spans in random
    order (the same physical blocks at different offsets) plus a 64-token PDep
    question each."""
    rng = np.random.Generator(np.random.PCG64(seed))
    reqs = []
    for _ in range(num_reqs):
        pick = rng.choice(pool, size=per_req, replace=False)
        segs = [Segment("span", span_len, fresh=False, pool=int(i)) for i in pick]
        segs.append(Segment("pdep", q_len))
        reqs.append(segs)
    return build(name, reqs, pool_lengths=[span_len] * pool, num_q_heads=32, num_kv_heads=8,
                 head_dim=128, dtype="bf16", rope_theta=5e5, max_pos=32768, seed=seed, rng=rng)


def _c3w(seed=3, name="c3w"):
    """The retrieval stand-in at the batch size of the pages' throughput table:
    64 requests, each 10 of 160 cached documents of 100 tokens (padded to 112)
    in random order plus a 64-token PDep question (the pool keeps c3's four
    uses per document)."""
    return _c3(seed, num_reqs=64, pool=160, span_len=pad_to_block(100), per_req=10, q_len=64, name=name)


def _c4(seed=4, n_spans=120, span_len=256, suffix=512, name="c4"):
    """Long context: 120 SSep spans of 256 tokens, a seeded half of them cached and
    the other half computed now, then a 512-token PDep suffix."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cached = np.zeros(n_spans, bool)
    cached[rng.choice(n_spans, size=n_spans // 2, replace=False)] = True
    segs = [Segment("span", span_len, fresh=not bool(c)) for c in cached]
    segs.append(Segment("pdep", suffix))
    return build(name, [segs], num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                 rope_theta=5e5, max_pos=32768, seed=seed, rng=rng)


def _c5(seed=5, num_reqs=8, n_spans=20, lo=128, hi=512, prefix=256, q_len=128, name="c5",
        num_q_heads=64):
    """70B single-layer shape: 64 q heads, 8 KV heads; 8 requests, each a shared
    cached 256-token prefix visible to every later query (Prompt-Cache style),
    20 fresh spans of U{128..512} tokens padded to 16, and a 128-token PDep
    question."""
    rng = np.random.Generator(np.random.PCG64(seed))
    reqs = []
    for _ in range(num_reqs):
        segs = [Segment("global", prefix, fresh=False, pool=0)]
        for n in rng.integers(lo, hi + 1, size=n_spans):
            segs.append(Segment("span", pad_to_block(int(n))))
        segs.append(Segment("pdep", q_len))
        reqs.append(segs)
    return build(name, reqs, pool_lengths=[prefix], num_q_heads=num_q_heads, num_kv_heads=8,
                 head_dim=128, dtype="bf16", rope_theta=5e5, max_pos=32768, seed=seed, rng=rng)


def _epic(name, seed, spans, recompute, head, tail, fresh_rest, **shape):
    """Spans whose first `recompute` tokens (block-rounded) are recomputed against
    all preceding context (a PDep segment) while the rest of the span keeps its
    span id, so the span's later queries still see its recomputed start."""
    rng = np.random.Generator(np.random.PCG64(seed))
    segs, ids = [], []
    if head:
        segs.append(Segment("span", head))
        ids.append(0)
    for i, n in enumerate(spans):
        sid = len(ids)
        segs += [Segment("pdep", recompute), Segment("span", n - recompute, fresh=fresh_rest)]
        ids += [sid, sid]
    segs.append(Segment("pdep", tail))
    ids.append(len(ids))
    return build(name, [segs], seed=seed, rng=rng, span_ids=[np.array(ids)], **shape)


_SHAPE_8B = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16", rope_theta=5e5, max_pos=32768)


def _e2(seed=2, name="e2"):
    """C2's layout with the first block of each span recomputed against the
    system prompt and earlier spans (EPIC / LegoLink); the rest of each span is
    computed as an SSep span that sees its recomputed start."""
    return _epic(name, seed, [192] * 10, 16, 512, 64, True, **_SHAPE_8B)


def _e4(seed=4, name="e4", n_spans=120):
    """C4's context with every span cached except its first block, which is
    recomputed against all preceding context; then the 512-token PDep suffix."""
    return _epic(name, seed, [256] * n_spans, 16, 0, 512, False, **_SHAPE_8B)


CONFIGS = {
    "e2": _e2,
    "e4": _e4,
    "c1": _c1,
    "c2": _c2,
    "c3": _c3,
    "c3w": _c3w,
    "c4": _c4,
    "c5": _c5,
}


def decode_view(w: Workload, seed: int = 0) -> Workload:
    """The decode step after a prefill batch: every request's last context
    token is its one query row.

    The query vector is the prefill batch's row for that token when the token
    was queried there, else a seeded N(0,1) draw. The token's K/V are the
    step's new entries; every other token is cached at set-up.
    """
    R = w.num_reqs
    q_ctx = (w.ctx_len.astype(np.int64) - 1).astype(np.int32)
    rows = np.full(R, -1, np.int64)
    for r in range(R):
        q0, q1 = int(w.q_indptr[r]), int(w.q_indptr[r + 1])
        hit = np.nonzero(w.q_ctx_idx[q0:q1] == q_ctx[r])[0]
        if len(hit):
            rows[r] = q0 + int(hit[0])
    q = np.empty((R,) + w.q.shape[1:], w.q.dtype)
    have = rows >= 0
    q[have] = w.q[rows[have]]
    if (~have).any():
        rng = np.random.Generator(np.random.PCG64(seed))
        x = rng.standard_normal((int((~have).sum()),) + w.q.shape[1:], dtype=np.float32)
        q[~have] = f32_to_bf16_bits(x) if w.dtype == "bf16" else x
    new_tok = np.array([w.tok_of_ctx[r][q_ctx[r]] for r in range(R)], np.int64)
    written = np.zeros(len(w.tok_slot), bool)
    written[new_tok] = True
    return dataclasses.replace(w, name=w.name.replace("c", "d", 1) if w.name.startswith("c") else w.name + "_decode",
                               q_indptr=np.arange(R + 1, dtype=np.int32), q_ctx_idx=q_ctx, q=q,
                               new_tok=new_tok, setup_tok=np.nonzero(~written)[0])


def make_config(name: str, seed: Optional[int] = None) -> Workload:
    """Benchmark workloads c1..c5, reduced variants used by parity tests, and
    d2..d5 (and d*_small): the decode step after the prefill of c2..c5."""
    if name.startswith("d") and name[1:2].isdigit():
        return decode_view(make_config("c" + name[1:], seed))
    small = {
        "c1_cached": lambda s: _c1(s or 1, cached_spans=True),
        # reduced copies of the big layouts: same structure, oracle-friendly size
        "c3_small": lambda s: _c3(s or 3, num_reqs=4, pool=8, per_req=4, q_len=48, name="c3_small"),
        "c4_small": lambda s: _c4(s or 4, n_spans=12, span_len=256, suffix=200, name="c4_small"),
        "c5_small": lambda s: _c5(s or 5, num_reqs=2, n_spans=4, prefix=64, q_len=40, name="c5_small"),
        "e4_small": lambda s: _e4(s or 4, name="e4_small", n_spans=12),
    }
    if name in small:
        return small[name](seed)
    fn = CONFIGS[name]
    return fn() if seed is None else fn(seed)


def custom(name: str, requests, *, num_q_heads=4, num_kv_heads=2, head_dim=64, dtype="f32",
           rope_theta=1e4, max_pos=4096, seed=0, **kw) -> Workload:
    """Free-form layouts for edge-case tests."""
    return build(name, requests, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                 head_dim=head_dim, dtype=dtype, rope_theta=rope_theta, max_pos=max_pos,
                 seed=seed, **kw)
