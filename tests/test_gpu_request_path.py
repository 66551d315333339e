"""End to end on the GPU: from marked token ids to attention outputs.

The request procedure of "MiniPIC: Flexible Position-Independent Caching in
<100LOC", §3.3.1 (documents marked with SSep and padded to a block boundary,
the task marked PDep), with the block hashes of §3.1.1:

  token ids -> minipic_describe_blocks (hashes, span ids, PDEP / GLOBAL bits)
            -> BlockCache.assign (physical blocks; cached blocks hit)
            -> minipic_slot_mapping (slots of the tokens that missed)
            -> minipic_write_kv (only those tokens)
            -> minipic_prefill_attn (the builder's span ids and flags)

Two requests in one batch share documents at different offsets (and the
second repeats one document); the second request's shared documents hit the
blocks the first one writes in the same step. Token values are drawn per
document (the same document has the same K/V wherever it appears, as the
position-free cache assumes) and per private segment, so the oracle's dense
per-request K/V come from the documents, never from the paged cache. Every
query row (each request's missed tokens) is compared with the oracle.
"""
import sys

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SSEP, PDEP, GLOB, PAD = 200001, 200002, 200003, 0
HQ, HKV, D, THETA = 32, 8, 128, 5e5


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _bf16(x):
    return torch.from_numpy(x).to(torch.bfloat16)


def _segment(rng, n, marker):
    body = rng.integers(1, 50000, size=n).tolist()
    if marker is not None:
        body[0] = marker
    return body + [PAD] * ((-len(body)) % 16)


@pytest.mark.parametrize("with_prefix", [False, True])
def test_marked_requests_through_the_whole_path(with_prefix):
    import position_independent_paged_amd as pip
    from position_independent_paged_amd.staging import DeviceBatch
    rng = np.random.default_rng(41 + with_prefix)
    docs = {k: _segment(rng, n, SSEP) for k, n in zip("abcd", (100, 180, 64, 37))}
    system = _segment(rng, 70, None)
    prefix = _segment(rng, 48, GLOB) if with_prefix else []
    tasks = [_segment(rng, 30, PDEP), _segment(rng, 45, PDEP)]
    layout = [["sys", "pre", "a", "b", "c", "t0"], ["sys", "pre", "c", "d", "a", "a", "t1"]]
    seg_tokens = dict(docs, sys=system, pre=prefix, t0=tasks[0], t1=tasks[1])
    # K~ / V per segment (a document's values do not depend on where it appears)
    seg_k = {k: rng.standard_normal((len(v), HKV, D), dtype=np.float32) for k, v in seg_tokens.items()}
    seg_v = {k: rng.standard_normal((len(v), HKV, D), dtype=np.float32) for k, v in seg_tokens.items()}
    # round to bf16 once: the oracle sees exactly the values the GPU stores
    seg_k = {k: _bf16(v).float().numpy() for k, v in seg_k.items()}
    seg_v = {k: _bf16(v).float().numpy() for k, v in seg_v.items()}

    num_blocks = 160
    cache = pip.BlockCache(num_blocks)
    reqs = []
    for segs in layout:
        toks = sum((seg_tokens[s] for s in segs), [])
        h, span, flags = pip.minipic_describe_blocks(toks, ssep=SSEP, pdep=PDEP, global_=GLOB, seed=3)
        bt, hit, nhit = cache.assign(h)
        slots, ctx_idx = pip.minipic_slot_mapping(bt, hit, len(toks))
        k = np.concatenate([seg_k[s] for s in segs])
        v = np.concatenate([seg_v[s] for s in segs])
        reqs.append(dict(toks=toks, span=span, flags=flags, bt=bt, hit=hit, slots=slots, ctx=ctx_idx, k=k, v=v))
        say(f"request {len(reqs) - 1}: {len(toks)} tokens, {len(bt)} blocks, {nhit} hit, "
            f"{len(slots)} tokens to compute")
    # the second request reuses the shared documents (and its repeated document) from the cache
    assert reqs[1]["hit"].sum() > 0 and len(reqs[1]["slots"]) < len(reqs[1]["toks"]) // 2

    R = len(reqs)
    MB = max(len(r["bt"]) for r in reqs)
    block_table = np.zeros((R, MB), np.int32)
    span_id = np.zeros((R, MB), np.int32)
    blk_flags = np.zeros((R, MB), np.uint8)
    logical_pos = np.zeros((R, MB * 16), np.int32)
    ctx_len = np.array([len(r["toks"]) for r in reqs], np.int32)
    for i, r in enumerate(reqs):
        nb = len(r["bt"])
        block_table[i, :nb], span_id[i, :nb], blk_flags[i, :nb] = r["bt"], r["span"], r["flags"]
        logical_pos[i, :len(r["toks"])] = np.arange(len(r["toks"]))
    # queries: each request's missed tokens (the ones computed now), Q already rotated
    q_ctx = [r["ctx"] for r in reqs]
    q_indptr = np.concatenate([[0], np.cumsum([len(c) for c in q_ctx])]).astype(np.int32)
    q = _bf16(rng.standard_normal((int(q_indptr[-1]), HQ, D), dtype=np.float32))

    dev = "cuda"
    kc = torch.full((num_blocks, HKV, 16, D), float("nan"), dtype=torch.bfloat16, device=dev)
    vc = torch.full((num_blocks, HKV, D, 16), float("nan"), dtype=torch.bfloat16, device=dev)
    new_k = torch.from_numpy(np.concatenate([r["k"][r["ctx"]] for r in reqs])).to(torch.bfloat16).to(dev)
    new_v = torch.from_numpy(np.concatenate([r["v"][r["ctx"]] for r in reqs])).to(torch.bfloat16).to(dev)
    slots = torch.from_numpy(np.concatenate([r["slots"] for r in reqs]).astype(np.int64)).to(dev)
    max_pos = 4096
    cos_sin = torch.empty((max_pos, D), dtype=torch.float32, device=dev)
    pip.minipic_rope_table(cos_sin, max_pos, D, THETA)
    batch = DeviceBatch(q_indptr=q_indptr, q_ctx_idx=np.concatenate(q_ctx), ctx_len=ctx_len,
                        block_table=block_table, logical_pos=logical_pos, span_id=span_id, blk_flags=blk_flags,
                        num_q_heads=HQ, num_kv_heads=HKV, head_dim=D, device=dev)
    ws = torch.zeros(pip.minipic_workspace_size(batch.struct, pip.MINIPIC_BF16), dtype=torch.uint8, device=dev)
    qd = q.to(dev)
    out = torch.zeros_like(qd)
    pip.minipic_write_kv(new_k, new_v, slots, kc, vc, num_kv_heads=HKV, head_dim=D, num_blocks=num_blocks)
    pip.minipic_prefill_attn(qd, kc, vc, num_blocks, batch.struct, cos_sin, max_pos, out, ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0
    got = out.float().cpu().numpy().astype(np.float64)
    qf = q.float().numpy().astype(np.float64)
    for i, r in enumerate(reqs):
        q0, q1 = int(q_indptr[i]), int(q_indptr[i + 1])
        L = len(r["toks"])
        want = oracle.prefill_attention(qf[q0:q1], r["ctx"], r["k"].astype(np.float64), r["v"].astype(np.float64),
                                        np.arange(L), r["span"].astype(np.int64), r["flags"].astype(np.int64),
                                        block_size=16, theta=THETA)
        err = np.abs(got[q0:q1] - want)
        rel = float(np.linalg.norm(got[q0:q1] - want) / np.linalg.norm(want))
        say(f"  request {i}: rows={q1 - q0} max_abs={err.max():.3e} rel_l2={rel:.3e}")
        assert np.isfinite(got[q0:q1]).all()
        assert err.max() <= 2e-2 and rel <= 1e-2
