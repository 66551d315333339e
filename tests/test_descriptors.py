"""Host descriptor builder and block cache (CPU only).

Pins the block-hash recurrence of "MiniPIC: Flexible Position-Independent
Caching in <100LOC", §3.1.1 (SSep blocks hash from the seed, PDep blocks from
the whole prefix, other blocks chain from their predecessor) by its
consequences, the segment semantics (span ids, PDEP / GLOBAL flags) against
the workload generator's descriptors, the marker contract, and the cache's
reuse of documents at any offset (the request procedure of §3.3.1).
"""
import numpy as np
import pytest

import workload
from workload import Segment
import position_independent_paged_amd as pip

SSEP, PDEP, GLOB, PAD = 100001, 100002, 100003, 0


def doc(rng, n, marker=SSEP):
    """A document of n tokens starting with `marker`, padded to a block boundary."""
    body = rng.integers(1, 50000, size=n - 1).tolist()
    toks = ([marker] if marker is not None else [rng.integers(1, 50000)]) + body
    return toks + [PAD] * ((-len(toks)) % 16)


def describe(tokens, seed=7):
    return pip.minipic_describe_blocks(tokens, ssep=SSEP, pdep=PDEP, global_=GLOB, seed=seed)


def test_ssep_document_hashes_do_not_depend_on_its_offset():
    rng = np.random.default_rng(0)
    d1, d2, d3 = doc(rng, 70), doc(rng, 40), doc(rng, 33)
    sys_a, sys_b = doc(rng, 50, marker=None), doc(rng, 90, marker=None)
    ha, _, _ = describe(sys_a + d1 + d2)
    hb, _, _ = describe(sys_b + d3 + d2 + d1)
    na, nb1, nb2, nb3 = len(sys_a) // 16, len(d1) // 16, len(d2) // 16, len(d3) // 16
    nsb = len(sys_b) // 16
    # every block of d1 and d2 (not only the SSep block) matches across the two prompts
    assert np.array_equal(ha[na:na + nb1], hb[nsb + nb3 + nb2:nsb + nb3 + nb2 + nb1])
    assert np.array_equal(ha[na + nb1:na + nb1 + nb2], hb[nsb + nb3:nsb + nb3 + nb2])
    # the system prompts differ
    assert ha[0] != hb[0]


def test_pdep_block_depends_on_the_whole_prefix():
    rng = np.random.default_rng(1)
    sys_, d1, d2 = doc(rng, 30, marker=None), doc(rng, 64), doc(rng, 48)
    task = doc(rng, 40, marker=PDEP)
    base, _, _ = describe(sys_ + d1 + d2 + task)
    nt = len(task) // 16
    # change one token inside d1 (after its marker): the SSep chain of d2 is
    # unaffected, the PDep task blocks all change
    d1x = list(d1)
    d1x[20] += 1
    h, _, _ = describe(sys_ + d1x + d2 + task)
    i1 = len(sys_) // 16
    i2 = i1 + len(d1) // 16
    assert np.array_equal(h[i2:i2 + len(d2) // 16], base[i2:i2 + len(d2) // 16])
    assert h[i1 + 1] != base[i1 + 1]
    assert np.all(h[-nt:] != base[-nt:])
    # swapping the two documents changes the task's hash (the prefix differs)
    hs, _, _ = describe(sys_ + d2 + d1 + task)
    assert np.all(hs[-nt:] != base[-nt:])
    # identical prefixes give identical hashes
    h2, _, _ = describe(sys_ + d1 + d2 + task)
    assert np.array_equal(h2, base)


def test_ordinary_blocks_chain_from_their_predecessor():
    rng = np.random.default_rng(2)
    toks = doc(rng, 64, marker=None)
    h, _, _ = describe(toks)
    t2 = list(toks)
    t2[3] += 1                       # block 0 changes -> every later block changes
    h2, _, _ = describe(t2)
    assert np.all(h2 != h)
    t3 = list(toks)
    t3[40] += 1                      # block 2 changes -> blocks 0, 1 keep their hashes
    h3, _, _ = describe(t3)
    assert np.array_equal(h3[:2], h[:2]) and np.all(h3[2:] != h[2:])
    # the seed h_0 enters every hash
    h4, _, _ = describe(toks, seed=8)
    assert np.all(h4 != h)


def test_segments_span_ids_and_flags():
    rng = np.random.default_rng(3)
    parts = [doc(rng, 20, marker=None), doc(rng, 48, marker=GLOB), doc(rng, 40), doc(rng, 16), doc(rng, 70, PDEP)]
    toks = sum(parts, [])
    _, span, flags = describe(toks)
    sizes = [len(p) // 16 for p in parts]
    want_span = np.repeat(np.arange(len(parts)), sizes)
    want_flags = np.repeat([0, pip.MINIPIC_BLK_GLOBAL, 0, 0, pip.MINIPIC_BLK_PDEP], sizes)
    assert np.array_equal(span, want_span)
    assert np.array_equal(flags, want_flags)


def test_marker_inside_a_block_breaks_the_contract():
    rng = np.random.default_rng(4)
    toks = doc(rng, 20, marker=None)[:20] + doc(rng, 30)       # SSep at position 20
    with pytest.raises(pip.MinipicError) as e:
        describe(toks)
    assert e.value.status == pip.MINIPIC_ERR_CONTRACT
    assert "position 20" in str(e.value)


@pytest.mark.parametrize("name", ["c2", "c3_small", "c4_small", "c5_small"])
def test_descriptors_match_the_generated_layouts(name):
    """Token sequences marked like the pages' request procedure give the
    generator's block structure: same span partition, same PDEP / GLOBAL bits.
    (The e2 / e4 layouts assign span ids directly: a recomputed PDep first
    block shares its span id with the rest of the document, which the marker
    segments cannot express.)"""
    w = workload.make_config(name)
    rng = np.random.default_rng(5)
    for r in range(w.num_reqs):
        toks = []
        for si, seg in enumerate(w.segments[r]):
            marker = {"span": SSEP, "pdep": PDEP, "global": GLOB}[seg.kind] if si > 0 else None
            body = rng.integers(1, 50000, size=seg.length).tolist()
            if marker is not None:
                body[0] = marker
            toks += body
        _, span, flags = describe(toks)
        nb = (int(w.ctx_len[r]) + 15) // 16
        want_flags = w.blk_flags[r, :nb]
        if w.segments[r][0].kind != "span":          # a leading PDep / GLOBAL segment has no marker here
            nf = (w.segments[r][0].length + 15) // 16
            want_flags = want_flags.copy()
            want_flags[:nf] = 0
        assert np.array_equal(flags, want_flags), (name, r)
        # same partition into segments (ids may be numbered differently)
        ws = w.span_id[r, :nb]
        assert np.array_equal(np.diff(span) != 0, np.diff(ws) != 0), (name, r)


def test_block_cache_reuses_documents_at_any_offset():
    rng = np.random.default_rng(6)
    sys_ = doc(rng, 40, marker=None)
    d1, d2 = doc(rng, 60), doc(rng, 100)
    task_a, task_b = doc(rng, 30, PDEP), doc(rng, 30, PDEP)
    cache = pip.BlockCache(64)
    a = sys_ + d1 + d2 + task_a
    ha, _, _ = describe(a)
    bt_a, hit_a, n_a = cache.assign(ha)
    assert n_a == 0 and len(set(bt_a.tolist())) == len(bt_a)
    b = sys_ + d2 + d1 + task_b
    hb, _, _ = describe(b)
    bt_b, hit_b, n_b = cache.assign(hb)
    ns, n1, n2, nt = len(sys_) // 16, len(d1) // 16, len(d2) // 16, len(task_b) // 16
    # the system prompt and both documents hit and share physical blocks; the task misses
    assert np.all(hit_b[:ns + n2 + n1] == 1) and np.all(hit_b[-nt:] == 0) and n_b == ns + n1 + n2
    assert np.array_equal(bt_b[:ns], bt_a[:ns])
    assert np.array_equal(bt_b[ns:ns + n2], bt_a[ns + n1:ns + n1 + n2])
    assert np.array_equal(bt_b[ns + n2:ns + n2 + n1], bt_a[ns:ns + n1])
    # only the task's tokens are computed and written
    slots, idx = pip.minipic_slot_mapping(bt_b, hit_b, len(b))
    assert np.array_equal(idx, np.arange(len(b) - len(task_b), len(b)))
    assert np.array_equal(slots, bt_b[idx // 16].astype(np.int64) * 16 + idx % 16)
    cache.close()


def test_same_document_twice_in_one_request():
    rng = np.random.default_rng(7)
    d = doc(rng, 32)
    h, _, _ = describe(d + d)
    cache = pip.BlockCache(8)
    bt, hit, n = cache.assign(h)
    assert np.array_equal(bt[:2], bt[2:]) and list(hit) == [0, 0, 1, 1] and n == 2


def test_block_cache_full_records_nothing():
    rng = np.random.default_rng(8)
    cache = pip.BlockCache(3)
    h, _, _ = describe(doc(rng, 64))                  # 4 blocks > 3
    with pytest.raises(pip.MinipicError) as e:
        cache.assign(h)
    assert e.value.status == pip.MINIPIC_ERR_CACHE_FULL
    h2, _, _ = describe(doc(rng, 48))                 # 3 blocks fit: nothing was taken before
    bt, hit, n = cache.assign(h2)
    assert n == 0 and sorted(bt.tolist()) == [0, 1, 2]


def test_document_after_a_shared_prefix_chains_from_it():
    """A span's tokens attend to every earlier GLOBAL block, so its K/V depend
    on that prefix: the same document after two different GLOBAL prefixes
    must not share cache blocks, after the same prefix it must, and without a
    GLOBAL segment the SSep rule (hash from h_0) is unchanged."""
    rng = np.random.default_rng(9)
    pre_a, pre_b = doc(rng, 64, marker=GLOB), doc(rng, 64, marker=GLOB)
    d = doc(rng, 80)
    task = doc(rng, 20, PDEP)
    npre, nd = len(pre_a) // 16, len(d) // 16
    ha, _, fa = describe(pre_a + d + task)
    hb, _, _ = describe(pre_b + d + task)
    hc, _, _ = describe(pre_a + doc(rng, 32) + d + task)      # same prefix, the document later
    h0, _, _ = describe(d)                                     # no prefix: SSep hashes from h_0
    doc_a, doc_b = ha[npre:npre + nd], hb[npre:npre + nd]
    assert np.all(doc_a != doc_b)
    assert np.array_equal(hc[npre + 2:npre + 2 + nd], doc_a)
    assert np.all(doc_a != h0)
    assert np.all(fa[:npre] == pip.MINIPIC_BLK_GLOBAL) and np.all(fa[npre:npre + nd] == 0)
    cache = pip.BlockCache(64)
    _, _, n1 = cache.assign(ha)
    _, hit_b, n2 = cache.assign(hb)
    assert n1 == 0 and n2 == 0 and not hit_b.any()
    _, hit_c, _ = cache.assign(hc)
    assert np.all(hit_c[:npre] == 1) and np.all(hit_c[npre + 2:npre + 2 + nd] == 1)
    cache.close()
