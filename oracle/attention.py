"""Position-free paged prefill attention, plain float64 definition.

Oracle; test infrastructure only. "MiniPIC: Flexible Position-Independent
Caching in <100LOC":

* §3.2.1, score equation: score(t, j) = (R_t q_t)^T (R_pi(j) k~_j) / sqrt(d).
  The same section states that this equals re-rotating every cached key, so the
  oracle does exactly that: rotate every key of the request by its logical
  position, then run ordinary masked softmax attention.
* §3.2.2: baseline FlashAttention takes pre-rotated Q and K and computes
  softmax(Q_rot K_rot^T / sqrt(d)) V; V is unchanged by the method.

Readings where the pages leave a step open:
* Q arrives already rotated by its own logical position (the kernel listing of
  §3.2.2 consumes Q_rot); ``q_rotated=False`` rotates it here by pi(c).
* The query's position t is pi(c), the logical position of its own context
  index c.
* Grouped-query attention: query head h reads KV head h // (Hq / Hkv).
* softmax scale 1/sqrt(d) unless given.
"""
import numpy as np

from .mask import block_mask
from .rope import rotate


def prefill_attention(q, q_ctx, k, v, pos, span_id, flags, *, block_size: int, theta: float,
                      scale=None, q_rotated: bool = True, k_rotated: bool = False,
                      rows=None, chunk_bytes: int = 64 << 20):
    """Attention output for the query rows of one request.

    q:       [nq, Hq, d]   query rows (R_t q_t if q_rotated, else q_t)
    q_ctx:   [nq]          context index c of each query row
    k, v:    [L, Hkv, d]   K~ (unrotated unless k_rotated) and V of the request's context
    pos:     [L]           logical position pi(j) of each context token
    span_id, flags: [ceil(L/block_size)] per-block descriptors
    rows:    optional index array selecting a subset of the query rows
    returns  [len(rows) or nq, Hq, d] float64
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    q_ctx = np.asarray(q_ctx, np.int64)
    pos = np.asarray(pos, np.int64)
    if rows is not None:
        rows = np.asarray(rows, np.int64)
        q = q[rows]
        q_ctx = q_ctx[rows]
    nq, Hq, d = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    # position of each query: the logical position of its own context index
    if not q_rotated and nq:
        q = rotate(q, pos[q_ctx], theta)
    kr = k if k_rotated else rotate(k, pos, theta)
    out = np.zeros((nq, Hq, d), np.float64)
    if nq == 0 or L == 0:
        return out
    per_row = Hq * L * 8 * 3
    step = max(1, int(chunk_bytes // max(per_row, 1)))
    for r0 in range(0, nq, step):
        r1 = min(nq, r0 + step)
        m = block_mask(q_ctx[r0:r1], L, span_id, flags, block_size)       # [n, L]
        for g in range(Hkv):
            qg = q[r0:r1, g * G:(g + 1) * G, :]                             # [n, G, d]
            s = np.matmul(qg, kr[:, g, :].T) * scale                        # [n, G, L]
            s = np.where(m[:, None, :], s, -np.inf)
            mx = s.max(axis=-1, keepdims=True)
            p = np.exp(s - mx)
            p /= p.sum(axis=-1, keepdims=True)
            out[r0:r1, g * G:(g + 1) * G, :] = np.matmul(p, v[:, g, :])     # [n, G, d]
    return out


def workload_reference(w, r: int, rows=None, q_rotated: bool = True, k_rotated: bool = False,
                       q=None, k=None):
    """Oracle output for request r of a ``workload.Workload``.

    ``q`` / ``k`` optionally replace the request's query rows / keys (float64),
    e.g. for shift or reuse experiments.
    """
    dd = w.request_dense(r)
    return prefill_attention(dd["q"] if q is None else q, dd["q_ctx"], dd["k"] if k is None else k,
                             dd["v"], dd["pos"], dd["span_id"], dd["flags"],
                             block_size=w.block_size, theta=w.rope_theta,
                             q_rotated=q_rotated, k_rotated=k_rotated, rows=rows)


def visible_pair_count(w) -> int:
    """Number of visible (query, key) pairs per head over the whole batch."""
    total = 0
    for r in range(w.num_reqs):
        dd = w.request_dense(r)
        L = int(w.ctx_len[r])
        for r0 in range(0, len(dd["q_ctx"]), 512):
            m = block_mask(dd["q_ctx"][r0:r0 + 512], L, dd["span_id"], dd["flags"], w.block_size)
            total += int(m.sum())
    return total
