"""Host-side work accounting for a prefill batch (reporting only).

Counts the visible (query, key) pairs of a batch from its per-block
descriptors, walking runs of equal span id instead of evaluating a dense
mask: a query at context index c whose block is PDep sees c + 1 keys; any
other query sees the keys of its own run up to itself plus every key in a
GLOBAL block of an earlier run ("MiniPIC: Flexible Position-Independent
Caching in <100LOC", §3.1.1 and §3.3.1 for the meaning of the markers).

Algorithmic FLOPs of attention = 4 * d * Hq * pairs (one multiply-add for
QK^T and one for PV per pair and head dim element); exps, masking and the
rotation are not counted.
"""
import numpy as np

PDEP = 1
GLOBAL = 2


def visible_pairs(q_indptr, q_ctx_idx, ctx_len, span_id, blk_flags, block_size=16) -> int:
    q_indptr = np.asarray(q_indptr, np.int64)
    total = 0
    for r in range(len(q_indptr) - 1):
        qc = np.asarray(q_ctx_idx[q_indptr[r]:q_indptr[r + 1]], np.int64)
        if len(qc) == 0:
            continue
        L = int(ctx_len[r])
        nb = (L + block_size - 1) // block_size
        sp = np.asarray(span_id[r][:nb])
        fl = np.asarray(blk_flags[r][:nb]).astype(np.int64)
        # run start of every block
        starts = np.zeros(nb, np.int64)
        for b in range(1, nb):
            starts[b] = starts[b - 1] if sp[b] == sp[b - 1] else b
        # tokens in GLOBAL blocks strictly before each block
        tok_in_blk = np.minimum(block_size, L - np.arange(nb) * block_size)
        glob_tok = np.concatenate([[0], np.cumsum(np.where(fl & GLOBAL, tok_in_blk, 0))])
        bq = qc // block_size
        pdep = (fl[bq] & PDEP) != 0
        s0 = starts[bq]
        own = qc - s0 * block_size + 1
        total += int(np.where(pdep, qc + 1, own + glob_tok[s0]).sum())
    return total


def attention_flops(pairs: int, num_q_heads: int, head_dim: int) -> int:
    return 4 * head_dim * num_q_heads * int(pairs)


def workload_pairs(w) -> int:
    return visible_pairs(w.q_indptr, w.q_ctx_idx, w.ctx_len, w.span_id, w.blk_flags, w.block_size)


def decode_bytes(w) -> int:
    """Compulsory HBM bytes of one decode call (one query row per request):
    q and out rows and K and V of every key the query sees (once per KV head).
    The cos/sin rows are left out: a block of consecutive positions needs only
    one table row plus the per-offset angles, so their count depends on the
    method, not on the problem."""
    elem = 2 if w.dtype == "bf16" else 4
    bs = w.block_size
    total = 2 * int(w.total_q) * w.num_q_heads * w.head_dim * elem
    for r in range(int(w.num_reqs)):
        for c in np.asarray(w.q_ctx_idx[w.q_indptr[r]:w.q_indptr[r + 1]], np.int64):
            bq = int(c) // bs
            sp = np.asarray(w.span_id[r][:bq + 1])
            fl = np.asarray(w.blk_flags[r][:bq + 1]).astype(np.int64)
            vis = np.ones(bq + 1, bool) if fl[bq] & PDEP else ((fl & GLOBAL) != 0) | (sp == sp[bq])
            keys = int(vis.sum()) * bs - (bs - 1 - int(c) % bs)    # the query's own block up to itself
            total += keys * 2 * w.num_kv_heads * w.head_dim * elem
    return total
