"""Dense attention mask from per-block span descriptors (oracle; test only).

"MiniPIC: Flexible Position-Independent Caching in <100LOC", §3.1.1: SSep
starts a span that is cacheable on its own, with a position-independent
attention mask; PDep marks a segment whose KV genuinely depends on all earlier
context; padding aligns spans so that markers start a block. §3.3.1 prefills
every document (and the system prompt) as its own request, so a span sees only
itself. The Prompt Cache style layout (§3.1.1, abstract) adds a shared prefix
that every later token may see; here it is a GLOBAL block flag.

Reading used (each block carries span_id and the PDEP / GLOBAL bits):

    visible(c, j) = j <= c  and  ( PDEP(block(c))
                                   or GLOBAL(block(j))
                                   or span_id(block(j)) == span_id(block(c)) )

Causality is by context index c, j (the order of tokens in the request), never
by logical position. The mask is block-granular except for the causal diagonal;
pad tokens are ordinary tokens.
"""
import numpy as np

PDEP = 1
GLOBAL = 2


def block_mask(q_ctx: np.ndarray, ctx_len: int, span_id: np.ndarray, flags: np.ndarray,
               block_size: int) -> np.ndarray:
    """Boolean [len(q_ctx), ctx_len] matrix of visible (query, key) pairs."""
    q_ctx = np.asarray(q_ctx, np.int64)
    j = np.arange(ctx_len, dtype=np.int64)
    bq = q_ctx // block_size
    bk = j // block_size
    span_id = np.asarray(span_id, np.int64)
    flags = np.asarray(flags, np.int64)
    causal = j[None, :] <= q_ctx[:, None]
    pdep_q = (flags[bq] & PDEP) != 0
    glob_k = (flags[bk] & GLOBAL) != 0
    same = span_id[bk][None, :] == span_id[bq][:, None]
    return causal & (pdep_q[:, None] | glob_k[None, :] | same)
