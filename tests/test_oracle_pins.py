"""Pins of the CPU oracle against facts that do not come from the oracle itself.

The pages print no worked numeric example, so the oracle is pinned by
closed forms of the rotation, a library attention routine on explicitly
rotated tensors, invariants the pages' mechanism implies, special cases and
brute force over every small segment layout ("MiniPIC: Flexible
Position-Independent Caching in <100LOC", §3.2.1 score equation and the
equivalence statement after it; §3.1.1; §3.3.1).
"""
import itertools
import math

import numpy as np
import pytest
import torch

import brute
import oracle
import workload
from oracle.mask import GLOBAL, PDEP

TOL = 1e-12


def seg_mask(q_ctx, L, segments):
    """Visibility from the segment description, via the brute-force rule."""
    return np.array([[brute.visible(int(c), j, segments) for j in range(L)] for c in q_ctx], bool)


def sdpa(qr, kr, v, mask):
    """torch's scaled_dot_product_attention in float64 on the CPU.

    qr: [nq, Hq, d]; kr, v: [L, Hkv, d]; mask [nq, L] (True = attend)."""
    nq, Hq, d = qr.shape
    Hkv = kr.shape[1]
    rep = Hq // Hkv
    q_t = torch.from_numpy(np.ascontiguousarray(qr.transpose(1, 0, 2)))               # [Hq, nq, d]
    k_t = torch.from_numpy(np.ascontiguousarray(np.repeat(kr, rep, axis=1).transpose(1, 0, 2)))
    v_t = torch.from_numpy(np.ascontiguousarray(np.repeat(v, rep, axis=1).transpose(1, 0, 2)))
    m_t = torch.from_numpy(mask)[None].expand(Hq, nq, kr.shape[0])
    o = torch.nn.functional.scaled_dot_product_attention(q_t, k_t, v_t, attn_mask=m_t)
    return o.numpy().transpose(1, 0, 2)


# --------------------------------------------------------------------------
# rotation
# --------------------------------------------------------------------------

def test_inv_freq_closed_forms():
    # base^(-2i/d): d=4, base 1e4 -> [1, 1e-2]; d=8 -> [1, 1e-1, 1e-2, 1e-3]
    np.testing.assert_allclose(oracle.inv_freq(4, 1e4), [1.0, 1e-2], rtol=1e-15)
    np.testing.assert_allclose(oracle.inv_freq(8, 1e4), [1.0, 1e-1, 1e-2, 1e-3], rtol=1e-14)
    # d=128, base 5e5: the last frequency is 5e5^(-126/128)
    f = oracle.inv_freq(128, 5e5)
    assert f[0] == 1.0 and len(f) == 64
    assert abs(f[-1] - 5e5 ** (-126 / 128)) < 1e-18


def test_rotate_d4_by_hand():
    # x = (1, 2, 3, 4), p = 1, base 1e4: pairs (x0, x2) at angle 1, (x1, x3) at angle 0.01
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    got = oracle.rotate(x, np.array([1]), 1e4)[0]
    c1, s1, c2, s2 = math.cos(1), math.sin(1), math.cos(0.01), math.sin(0.01)
    want = [1 * c1 - 3 * s1, 2 * c2 - 4 * s2, 3 * c1 + 1 * s1, 4 * c2 + 2 * s2]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)


def test_rotate_position_zero_is_identity():
    x = np.random.default_rng(0).standard_normal((7, 3, 64))
    assert np.array_equal(oracle.rotate(x, np.zeros(7, int), 5e5), x)


def test_rotate_preserves_norm_and_composes():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((9, 2, 128))
    p = rng.integers(0, 30000, 9)
    q = rng.integers(0, 2000, 9)
    rx = oracle.rotate(x, p, 5e5)
    np.testing.assert_allclose(np.linalg.norm(rx, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_allclose(oracle.rotate(rx, q, 5e5), oracle.rotate(x, p + q, 5e5), atol=1e-9)


def test_rotate_matches_complex_form():
    """RoFormer's complex form, evaluated by the brute-force helper."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 16))
    p = np.array([0, 1, 17, 4096, 30000])
    got = oracle.rotate(x, p, 1e4)
    want = np.array([brute.rot(list(x[i]), int(p[i]), 1e4) for i in range(5)])
    np.testing.assert_allclose(got, want, atol=1e-10)


def test_relative_position_identity():
    """(R_t q) . (R_pi k) = Re sum_i z_q conj(z_k) exp(i (t - pi) theta_i)."""
    rng = np.random.default_rng(3)
    d = 128
    qv = rng.standard_normal(d)
    kv = rng.standard_normal(d)
    th = 5e5 ** (-np.arange(d // 2) * 2.0 / d)
    zq = qv[:d // 2] + 1j * qv[d // 2:]
    zk = kv[:d // 2] + 1j * kv[d // 2:]
    for t, pi in [(0, 0), (5, 3), (3, 5), (31000, 12), (100, 4096)]:
        lhs = oracle.rotate(qv[None], np.array([t]), 5e5)[0] @ oracle.rotate(kv[None], np.array([pi]), 5e5)[0]
        rhs = np.real(np.sum(zq * np.conj(zk) * np.exp(1j * (t - pi) * th)))
        assert abs(lhs - rhs) < 1e-9 * max(1.0, abs(rhs))


# --------------------------------------------------------------------------
# mask
# --------------------------------------------------------------------------

def _descriptors(segments, L, bs):
    nb = (L + bs - 1) // bs
    span = np.zeros(nb, np.int64)
    flags = np.zeros(nb, np.int64)
    for sid, (s0, n, kind) in enumerate(segments):
        b0, b1 = s0 // bs, (s0 + n + bs - 1) // bs
        span[b0:b1] = sid
        if kind == "pdep":
            flags[b0:b1] |= PDEP
        if kind == "global":
            flags[b0:b1] |= GLOBAL
    return span, flags


def _layouts(nblocks, bs, tail):
    """Every split of `nblocks` blocks into segments and every kind per segment."""
    L = nblocks * bs - tail
    for cuts in itertools.product([0, 1], repeat=nblocks - 1):
        starts = [0] + [i + 1 for i, c in enumerate(cuts) if c]
        bounds = starts + [nblocks]
        for kinds in itertools.product(["span", "pdep", "global"], repeat=len(starts)):
            segs = []
            for i, kind in enumerate(kinds):
                s0 = bounds[i] * bs
                s1 = min(bounds[i + 1] * bs, L)
                segs.append((s0, s1 - s0, kind))
            yield L, segs


def test_block_mask_equals_segment_rule_exhaustive():
    for nblocks, bs, tail in [(1, 4, 1), (3, 2, 0), (4, 3, 2), (5, 2, 1)]:
        n = 0
        for L, segs in _layouts(nblocks, bs, tail):
            span, flags = _descriptors(segs, L, bs)
            q_ctx = np.arange(L)
            got = oracle.block_mask(q_ctx, L, span, flags, bs)
            assert np.array_equal(got, seg_mask(q_ctx, L, segs)), (segs,)
            n += 1
        assert n > 0


# --------------------------------------------------------------------------
# attention: brute force over every small layout
# --------------------------------------------------------------------------

@pytest.mark.parametrize("q_rotated", [True, False])
def test_attention_brute_force_all_layouts(q_rotated):
    rng = np.random.default_rng(4)
    nblocks, bs, tail = 4, 2, 1
    Hq, Hkv, d, base = 2, 1, 4, 10.0
    count = 0
    for L, segs in _layouts(nblocks, bs, tail):
        span, flags = _descriptors(segs, L, bs)
        q = rng.standard_normal((L, Hq, d))
        k = rng.standard_normal((L, Hkv, d))
        v = rng.standard_normal((L, Hkv, d))
        pos = rng.permutation(L) + 3          # non-monotone logical positions
        q_ctx = np.arange(L)
        got = oracle.prefill_attention(q, q_ctx, k, v, pos, span, flags, block_size=bs,
                                       theta=base, q_rotated=q_rotated)
        want = brute.attention(q.tolist(), q_ctx.tolist(), k.tolist(), v.tolist(), pos.tolist(),
                               segs, base, q_rotated)
        np.testing.assert_allclose(got, np.array(want), atol=1e-12, err_msg=str(segs))
        count += 1
    assert count == sum(math.comb(nblocks - 1, s - 1) * 3 ** s for s in range(1, nblocks + 1))


def test_attention_brute_force_gqa_and_wide_heads():
    rng = np.random.default_rng(5)
    segs = [(0, 8, "global"), (8, 6, "span"), (14, 4, "span"), (18, 5, "pdep")]
    L, bs = 23, 2
    span, flags = _descriptors(segs, L, bs)
    Hq, Hkv, d = 6, 2, 8
    q = rng.standard_normal((L, Hq, d))
    k = rng.standard_normal((L, Hkv, d))
    v = rng.standard_normal((L, Hkv, d))
    pos = np.arange(L) * 7 + 11
    q_ctx = np.array([0, 3, 8, 9, 13, 14, 17, 18, 22])
    got = oracle.prefill_attention(q[q_ctx], q_ctx, k, v, pos, span, flags, block_size=bs, theta=1e4,
                                   q_rotated=False)
    want = brute.attention(q[q_ctx].tolist(), q_ctx.tolist(), k.tolist(), v.tolist(), pos.tolist(),
                           segs, 1e4, False)
    np.testing.assert_allclose(got, np.array(want), atol=1e-12)


# --------------------------------------------------------------------------
# attention: library routine on explicitly rotated tensors (the equivalence
# statement of §3.2.1: in-kernel rotation equals re-rotating every cached key)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["c1", "c1_cached", "c3_small", "c5_small"])
def test_attention_equals_sdpa_on_prerotated(name):
    w = workload.make_config(name)
    for r in range(min(w.num_reqs, 2)):
        dd = w.request_dense(r)
        L = int(w.ctx_len[r])
        rows = np.arange(len(dd["q_ctx"]))
        if len(rows) > 300:
            rows = np.sort(np.random.default_rng(r).choice(len(rows), 300, replace=False))
        q_ctx = dd["q_ctx"][rows]
        kr = oracle.rotate(dd["k"], dd["pos"], w.rope_theta)
        mask = seg_mask(q_ctx, L, w.query_segments(r))
        want = sdpa(dd["q"][rows], kr, dd["v"], mask)
        got = oracle.workload_reference(w, r, rows=rows)
        np.testing.assert_allclose(got, want, atol=1e-11)
        # the same oracle on keys that were rotated beforehand
        got2 = oracle.workload_reference(w, r, rows=rows, k=kr, k_rotated=True)
        np.testing.assert_allclose(got2, want, atol=1e-11)


def test_gqa_equals_mha_with_repeated_kv():
    w = workload.make_config("c1")
    dd = w.request_dense(0)
    rep = w.num_q_heads // w.num_kv_heads
    a = oracle.workload_reference(w, 0)
    b = oracle.prefill_attention(dd["q"], dd["q_ctx"], np.repeat(dd["k"], rep, axis=1),
                                 np.repeat(dd["v"], rep, axis=1), dd["pos"], dd["span_id"],
                                 dd["flags"], block_size=16, theta=w.rope_theta)
    np.testing.assert_allclose(a, b, atol=TOL)


# --------------------------------------------------------------------------
# invariants the mechanism implies
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shift", [1, 17, 4096, 30000])
def test_shift_invariance(shift):
    """Scores depend on t - pi(j) only, so a common shift of every logical
    position leaves the output unchanged when Q is rotated by its own position."""
    w = workload.make_config("c1")
    dd = w.request_dense(0)
    args = (dd["q"], dd["q_ctx"], dd["k"], dd["v"])
    a = oracle.prefill_attention(*args, dd["pos"], dd["span_id"], dd["flags"], block_size=16,
                                 theta=w.rope_theta, q_rotated=False)
    b = oracle.prefill_attention(*args, dd["pos"] + shift, dd["span_id"], dd["flags"], block_size=16,
                                 theta=w.rope_theta, q_rotated=False)
    np.testing.assert_allclose(a, b, atol=1e-11)
    # with pre-rotated Q a shift of the keys alone must change the result
    c = oracle.prefill_attention(*args, dd["pos"] + shift, dd["span_id"], dd["flags"], block_size=16,
                                 theta=w.rope_theta, q_rotated=True)
    assert np.abs(c - oracle.prefill_attention(*args, dd["pos"], dd["span_id"], dd["flags"],
                                               block_size=16, theta=w.rope_theta)).max() > 1e-3


def test_same_span_at_two_offsets():
    """One cached span reused at different offsets by two requests (§3.3.1, last
    paragraph): a query inside the span gives the same output at both offsets,
    and each PDep row equals standard attention with that request's own
    positions."""
    w = workload.make_config("c3_small")
    # find a pool span used by requests 0 and 1 at different offsets
    found = None
    for i0, s0 in enumerate(w.segments[0]):
        for i1, s1 in enumerate(w.segments[1]):
            if s0.pool is not None and s0.pool == s1.pool and w.seg_start[0][i0] != w.seg_start[1][i1]:
                found = (w.seg_start[0][i0], w.seg_start[1][i1], s0.length)
    assert found is not None
    o0, o1, n = found
    d0, d1 = w.request_dense(0), w.request_dense(1)
    assert np.array_equal(d0["k"][o0:o0 + n], d1["k"][o1:o1 + n])
    rng = np.random.default_rng(6)
    qv = rng.standard_normal((n, w.num_q_heads, w.head_dim))
    outs = []
    for dd, off in [(d0, o0), (d1, o1)]:
        qc = np.arange(off, off + n)
        outs.append(oracle.prefill_attention(qv, qc, dd["k"], dd["v"], dd["pos"], dd["span_id"],
                                             dd["flags"], block_size=16, theta=w.rope_theta,
                                             q_rotated=False))
    np.testing.assert_allclose(outs[0], outs[1], atol=1e-11)
    # PDep rows: standard attention with explicit per-request rotation
    for r, dd in [(0, d0), (1, d1)]:
        kr = oracle.rotate(dd["k"], dd["pos"], w.rope_theta)
        want = sdpa(dd["q"], kr, dd["v"], seg_mask(dd["q_ctx"], int(w.ctx_len[r]), w.query_segments(r)))
        np.testing.assert_allclose(oracle.workload_reference(w, r), want, atol=1e-11)


# --------------------------------------------------------------------------
# special cases
# --------------------------------------------------------------------------

def test_first_token_of_span_sees_only_itself():
    w = workload.make_config("c1")
    dd = w.request_dense(0)
    out = oracle.workload_reference(w, 0)
    G = w.num_q_heads // w.num_kv_heads
    for c in (0, 32):                      # first token of each SSep span
        row = int(np.nonzero(dd["q_ctx"] == c)[0][0])
        for h in range(w.num_q_heads):
            assert np.array_equal(out[row, h], dd["v"][c, h // G])


def test_equal_positions_cancel_rope():
    rng = np.random.default_rng(7)
    L, Hq, Hkv, d = 40, 4, 2, 32
    q, k, v = (rng.standard_normal((L, h, d)) for h in (Hq, Hkv, Hkv))
    segs = [(0, 16, "span"), (16, 16, "span"), (32, 8, "pdep")]
    span, flags = _descriptors(segs, L, 16)
    pos = np.full(L, 1234)
    got = oracle.prefill_attention(q, np.arange(L), k, v, pos, span, flags, block_size=16,
                                   theta=1e4, q_rotated=False)
    want = sdpa(q, k, v, seg_mask(np.arange(L), L, segs))
    np.testing.assert_allclose(got, want, atol=1e-12)


@pytest.mark.parametrize("kind", ["one_span", "all_pdep"])
def test_reduces_to_causal_attention(kind):
    rng = np.random.default_rng(8)
    L, Hq, Hkv, d = 53, 4, 1, 16
    q, k, v = (rng.standard_normal((L, h, d)) for h in (Hq, Hkv, Hkv))
    nb = (L + 15) // 16
    span = np.zeros(nb, np.int64) if kind == "one_span" else np.arange(nb)
    flags = np.zeros(nb, np.int64) if kind == "one_span" else np.full(nb, PDEP)
    pos = np.arange(L) + 5
    got = oracle.prefill_attention(q, np.arange(L), k, v, pos, span, flags, block_size=16, theta=1e4,
                                   q_rotated=False)
    qr = oracle.rotate(q, pos, 1e4)
    kr = oracle.rotate(k, pos, 1e4)
    qt = torch.from_numpy(np.ascontiguousarray(qr.transpose(1, 0, 2)))
    kt = torch.from_numpy(np.ascontiguousarray(np.repeat(kr, Hq, 1).transpose(1, 0, 2)))
    vt = torch.from_numpy(np.ascontiguousarray(np.repeat(v, Hq, 1).transpose(1, 0, 2)))
    want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True).numpy()
    np.testing.assert_allclose(got, want.transpose(1, 0, 2), atol=1e-12)


def test_constant_v_gives_v():
    w = workload.make_config("c1")
    dd = w.request_dense(0)
    v = np.ones_like(dd["v"]) * 0.375
    out = oracle.prefill_attention(dd["q"], dd["q_ctx"], dd["k"], v, dd["pos"], dd["span_id"],
                                   dd["flags"], block_size=16, theta=w.rope_theta)
    np.testing.assert_allclose(out, 0.375, atol=1e-14)


def test_row_subset_equals_full():
    w = workload.make_config("c1")
    full = oracle.workload_reference(w, 0)
    rows = np.array([79, 3, 40, 64])
    np.testing.assert_allclose(oracle.workload_reference(w, 0, rows=rows), full[rows], atol=0)


def test_visible_pair_count_matches_segment_rule():
    w = workload.make_config("c3_small")
    total = 0
    for r in range(w.num_reqs):
        dd = w.request_dense(r)
        total += int(seg_mask(dd["q_ctx"], int(w.ctx_len[r]), w.query_segments(r)).sum())
    assert oracle.visible_pair_count(w) == total


def test_golden_snapshot_unchanged():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "c1_rows.json")) as f:
        doc = json.load(f)
    w = workload.make_config("c1")
    out = oracle.workload_reference(w, 0, rows=np.array(doc["rows"]))
    np.testing.assert_allclose(out[:, 0, :8], doc["out_head0_first8"], atol=1e-12)
    np.testing.assert_allclose(out.sum(axis=(1, 2)), doc["out_sum_per_row"], atol=1e-10)
