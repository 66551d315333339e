"""GPU checks of the boundary's contracts (needs an MI355X).

* Cache slots past a request's context hold no token: filled with NaN they
  must not reach any output (prefill bf16 / f32, decode).
* logical_pos entries past the context are not read for a result: -1 there,
  or a cos/sin table that ends right after the last position, sets no error.
* Every bit of the workspace error word, forced from the host through the
  batch arrays (the kernels clamp the offending index into bounds and record
  it; the call still completes).
* The span-id contract: a span id that reappears after another value is a
  different span; the call sets MINIPIC_EW_SPAN and attends by runs, which is
  the oracle's rule on span ids renumbered per run.
* A captured HIP graph of write_kv + prefill_attn replays bit-identically to
  the eager calls, with eager work in between.
* The planner's piece-doubling path (more split pieces than partial-result
  slots) gives the same result as the normal plan.
"""
import os
import sys

import numpy as np
import pytest

import oracle
import workload
from workload import Segment

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def stage(w, **kw):
    from position_independent_paged_amd.staging import DeviceWorkload
    return DeviceWorkload(w, **kw)


def out_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def check(name, got, want, dtype):
    err = np.abs(got - want)
    mx = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)) if err.size else 0.0
    say(f"  {name}: rows={got.shape[0]} max_abs={mx:.3e} rel_l2={rel:.3e}")
    assert np.isfinite(got).all(), name
    if dtype == "f32":
        assert mx <= 1e-4, (name, mx)
    else:
        assert mx <= 2e-2 and rel <= 1e-2, (name, mx, rel)


def oracle_all(w, span_id=None):
    """Oracle output of every query row of `w` (optionally with other span ids)."""
    outs = []
    for r in range(w.num_reqs):
        dd = w.request_dense(r)
        if len(dd["q_ctx"]) == 0:
            continue
        span = dd["span_id"] if span_id is None else np.asarray(span_id[r][:len(dd["span_id"])], np.int64)
        outs.append(oracle.prefill_attention(dd["q"], dd["q_ctx"], dd["k"], dd["v"], dd["pos"], span,
                                             dd["flags"], block_size=w.block_size, theta=w.rope_theta))
    return np.concatenate(outs)


# ---------------------------------------------------------------------------
# unwritten cache slots and positions past the context
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["c1", "c4_small", "c5_small", "e4_small"])
def test_nan_in_unwritten_slots_never_reaches_the_output(name):
    w = workload.make_config(name)
    ragged = [int(L) % 16 for L in w.ctx_len]
    say(f"NaN-filled cache {name}: ctx % 16 = {ragged}")
    dw = stage(w, cache_fill=float("nan"))
    dw.step()
    torch.cuda.synchronize()
    assert dw.error_word() == 0
    got = out_f64(dw.out)
    check(f"nan-cache/{name}", got, oracle_all(w), w.dtype)


@pytest.mark.parametrize("name", ["d2", "d5"])
def test_nan_in_unwritten_slots_decode(name):
    w = workload.make_config(name)
    # the decode query is the last context token: make its block ragged
    say(f"NaN-filled cache, decode {name}: ctx % 16 = {[int(L) % 16 for L in w.ctx_len]}")
    dw = stage(w, cache_fill=float("nan"))
    dw.write_new()
    dw.decode()
    torch.cuda.synchronize()
    assert dw.decode_error_word() == 0
    check(f"nan-cache/{name}", out_f64(dw.out), oracle_all(w), w.dtype)


def _ragged_custom(dtype, seed, tail_pos=-1):
    reqs = [[Segment("span", 48), Segment("span", 32), Segment("pdep", 21)],
            [Segment("global", 32, fresh=False, pool=0), Segment("span", 48), Segment("pdep", 9)]]
    w = workload.custom("ragged", reqs, pool_lengths=[32], num_q_heads=8, num_kv_heads=2, head_dim=128,
                        dtype=dtype, rope_theta=5e5, max_pos=4096, seed=seed)
    # positions past the context are -1 and the table ends right after the last position
    lp = w.logical_pos.copy()
    for r, L in enumerate(w.ctx_len):
        lp[r, int(L):] = tail_pos
    w.logical_pos = lp
    w.max_pos = int(max(int(L) for L in w.ctx_len))
    return w


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_positions_past_the_context_are_not_read(dtype):
    w = _ragged_custom(dtype, seed=21)
    say(f"positions past the context ({dtype}): ctx={list(w.ctx_len)} max_pos={w.max_pos}")
    dw = stage(w, cache_fill=float("nan"))
    dw.step()
    torch.cuda.synchronize()
    assert dw.error_word() == 0
    check(f"tail-pos/{dtype}", out_f64(dw.out), oracle_all(w), dtype)


def test_positions_past_the_context_are_not_read_decode():
    w = workload.decode_view(_ragged_custom("bf16", seed=22))
    say(f"positions past the context (decode): ctx={list(w.ctx_len)} max_pos={w.max_pos}")
    dw = stage(w, cache_fill=float("nan"))
    dw.write_new()
    dw.decode()
    torch.cuda.synchronize()
    assert dw.decode_error_word() == 0
    check("tail-pos/decode", out_f64(dw.out), oracle_all(w), "bf16")


# ---------------------------------------------------------------------------
# error word bits, forced from the host
# ---------------------------------------------------------------------------

def _corrupt(kind, dw, w):
    """Corrupt one device descriptor array of the staged batch (the host scalars
    stay valid) so that the `kind` check of the kernels fires."""
    b = dw.batch
    L0 = int(w.ctx_len[0])
    if kind == "block":
        b.block_table[0, 0] = w.num_blocks + 7
    elif kind == "pos":
        b.logical_pos[0, 5] = w.max_pos + 3
    elif kind == "qctx":
        b.q_ctx_idx[int(w.q_indptr[1]) - 1] = L0 + 40   # request 0's last query row, past its context
    elif kind == "ctx":
        b.ctx_len[0] = w.block_table.shape[1] * 16 + 5
    torch.cuda.synchronize()


_EW = {"block": 1, "pos": 2, "qctx": 4, "ctx": 8}


@pytest.mark.parametrize("kind", sorted(_EW))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_error_word_bits_prefill(kind, dtype):
    w = _ragged_custom(dtype, seed=23, tail_pos=0)
    w.max_pos = 4096
    say(f"error word prefill {dtype}: {kind}")
    dw = stage(w)
    _corrupt(kind, dw, w)
    dw.step()
    torch.cuda.synchronize()
    ew = dw.error_word()
    say(f"  error word {ew:#x}")
    assert ew & _EW[kind], (kind, ew)
    assert torch.isfinite(dw.out.float()).all()


@pytest.mark.parametrize("kind", sorted(_EW))
def test_error_word_bits_decode(kind):
    w0 = _ragged_custom("bf16", seed=24, tail_pos=0)
    w0.max_pos = 4096
    w = workload.decode_view(w0)
    say(f"error word decode: {kind}")
    dw = stage(w)
    _corrupt(kind, dw, w)
    dw.write_new()
    dw.decode()
    torch.cuda.synchronize()
    ew = dw.decode_error_word()
    say(f"  error word {ew:#x}")
    assert ew & _EW[kind], (kind, ew)
    assert torch.isfinite(dw.out.float()).all()


# ---------------------------------------------------------------------------
# span-id contract
# ---------------------------------------------------------------------------

def _reused_span_ids(dtype):
    # span id 0 names two runs (blocks 0-1 and 5-6): the second is a different span
    reqs = [[Segment("span", 32), Segment("span", 48), Segment("span", 32), Segment("span", 48),
             Segment("pdep", 23)]]
    ids = [np.array([0, 1, 0, 2, 3])]
    w = workload.custom("reuse", reqs, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype=dtype,
                        rope_theta=5e5, max_pos=4096, seed=31, span_ids=ids)
    runs = np.zeros_like(w.span_id)       # one id per run: what the library attends by
    for r in range(w.num_reqs):
        nb = (int(w.ctx_len[r]) + 15) // 16
        s = w.span_id[r, :nb]
        runs[r, :nb] = np.concatenate([[0], np.cumsum(s[1:] != s[:-1])])
    return w, runs


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_span_id_reused_after_another_span(dtype):
    w, runs = _reused_span_ids(dtype)
    say(f"span id reused ({dtype}): span_id={w.span_id[0].tolist()}")
    dw = stage(w)
    dw.step()
    torch.cuda.synchronize()
    assert dw.error_word() == 16
    check(f"span-runs/{dtype}", out_f64(dw.out), oracle_all(w, span_id=runs), dtype)


def test_span_id_reused_decode():
    w0, runs = _reused_span_ids("bf16")
    # decode query: a token of the second run of span id 0 (context index 90)
    import dataclasses
    w = workload.decode_view(w0)
    w = dataclasses.replace(w, q_ctx_idx=np.array([90], np.int32),
                            ctx_len=np.array([91], np.int32))
    w.tok_of_ctx = [w0.tok_of_ctx[0][:91]]
    w.new_tok = np.array([w0.tok_of_ctx[0][90]])
    written = np.zeros(len(w.tok_slot), bool)
    written[w.new_tok] = True
    w.setup_tok = np.nonzero(~written)[0]
    say(f"span id reused (decode): query at 90, span_id={w.span_id[0].tolist()}")
    dw = stage(w)
    dw.write_new()
    dw.decode()
    torch.cuda.synchronize()
    assert dw.decode_error_word() == 16
    check("span-runs/decode", out_f64(dw.out), oracle_all(w, span_id=runs), "bf16")


# ---------------------------------------------------------------------------
# HIP graph capture
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["c4_small", "c1"])
def test_graph_replay_matches_eager(name):
    w = workload.make_config(name)
    say(f"graph replay {name}")
    dw = stage(w)
    dw.step()
    torch.cuda.synchronize()
    ref = dw.out.clone()
    bits = torch.int16 if w.dtype == "bf16" else torch.int32
    other = torch.empty_like(dw.out)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dw.step()                       # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        dw.step()
    for i in range(4):
        dw.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dw.out.view(bits), ref.view(bits)), f"replay {i}"
        dw.attend(out=other)            # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(other.view(bits), ref.view(bits)), f"eager {i}"
    assert dw.error_word() == 0


# ---------------------------------------------------------------------------
# planner: more split pieces than partial-result slots
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["c4_small", "c5_small"])
def test_piece_doubling_path(name, monkeypatch):
    w = workload.make_config(name)
    dw = stage(w)
    dw.step()
    torch.cuda.synchronize()
    ref = dw.out.clone()
    info = dw.launch_info()
    monkeypatch.setenv("MINIPIC_SLOT_CAP", "8")
    info2 = dw.launch_info()
    say(f"piece doubling {name}: slots {info['partial_slots']} -> {info2['partial_slots']}")
    assert info2["partial_slots"] == 8 < info["partial_slots"]
    dw.out.zero_()
    dw.attend()
    torch.cuda.synchronize()
    assert dw.error_word() == 0
    got = out_f64(dw.out)
    check(f"doubling/{name}", got, oracle_all(w), w.dtype)
    # fewer, longer pieces: the same result up to the order of the fp32 sums
    assert np.abs(got - out_f64(ref)).max() <= (1e-5 if w.dtype == "f32" else 2e-2)


@pytest.mark.parametrize("name", ["d3_small", "d5_small"])
def test_graph_replay_matches_eager_decode(name):
    """Decode (split attention + merge) captured in a HIP graph: every replay,
    with eager calls between them, gives the eager output bit for bit."""
    w = workload.make_config(name)
    say(f"graph replay decode {name}")
    dw = stage(w)
    dw.write_new()
    dw.decode()
    torch.cuda.synchronize()
    ref = dw.out.clone()
    other = torch.empty_like(dw.out)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dw.decode()                     # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        dw.decode()
        dw.decode()
    for i in range(4):
        dw.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dw.out.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        dw.decode(out=other)            # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int16), ref.view(torch.int16)), f"eager {i}"
    assert dw.decode_error_word() == 0
