"""CPU-only checks of the library boundary and host logic (no GPU needed).

The library must load and export every entry point declared in
include/*.h; every invalid call must be rejected by host-side checks before
any HIP call is made.
"""
import glob
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workload
import position_independent_paged_amd as pip
from position_independent_paged_amd import metrics
from position_independent_paged_amd._binding import minipic_batch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        with open(h) as f:
            text = f.read()
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(minipic_\w+)\s*\(", text, re.M))
    return sorted(names)


def test_library_exports_every_header_symbol():
    lib = ctypes.CDLL(pip.LIB_PATH)
    names = header_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(pip.EXPORTS)


def test_version_and_status_strings():
    lib = pip.load_library()
    assert b"gfx950" in lib.minipic_version()
    assert lib.minipic_status_string(0) == b"ok"
    assert lib.minipic_status_string(-3) == b"workspace too small"


def _batch(**kw):
    d = dict(num_reqs=1, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, max_blocks_per_req=10,
             total_q=100, max_q_len=100, max_ctx_len=160, q_indptr=256, q_ctx_idx=256, ctx_len=256, block_table=256,
             logical_pos=256, span_id=256, blk_flags=256)
    d.update(kw)
    return minipic_batch(**d)


def _attn(b, dtype=1, ws_bytes=1 << 30, q=256, out=256, ws=256, table=256, max_pos=1024, flags=0, rope=True):
    lib = pip.load_library()
    fn = lib.minipic_prefill_attn if rope else lib.minipic_reference_prerotated
    return fn(q, 256, 256, 10, ctypes.byref(b), table, max_pos, 0.0, out, ws, ws_bytes, flags, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), -2),
    (dict(num_q_heads=12, num_kv_heads=8), -2),
    (dict(num_q_heads=48, num_kv_heads=4), -2),      # 12 heads per group
    (dict(block_size=32), -2),
    (dict(num_reqs=-1), -1),
    (dict(max_blocks_per_req=0), -1),
    (dict(max_ctx_len=161), -1),
    (dict(total_q=-5), -1),
    (dict(q_indptr=None), -1),
    (dict(max_q_len=0), -1),
    (dict(logical_pos=256 + 4), -1),                 # not 16-byte aligned
    (dict(num_q_heads=256, num_kv_heads=256), -2),   # work items hold the KV head in 8 bits
])
def test_attention_rejects_bad_batch(kw, code):
    assert _attn(_batch(**kw)) == code
    assert pip.load_library().minipic_last_error()


def test_attention_rejects_bad_buffers():
    b = _batch()
    assert _attn(b, dtype=7) == -2
    assert _attn(b, q=None) == -1
    assert _attn(b, table=None) == -1
    assert _attn(b, max_pos=0) == -1
    assert _attn(b, flags=0x10) == -1
    assert _attn(b, ws=None) == -1
    assert _attn(b, ws=256 + 4) == -1                 # misaligned
    assert _attn(b, ws_bytes=64) == -3
    # the kernels address the cos/sin table through a 32-bit buffer range
    assert _attn(b, max_pos=(1 << 22)) == -1          # 2^22 rows x 128 floats = 2^31 bytes
    assert b"2^31" in pip.load_library().minipic_last_error()
    assert _attn(b, max_pos=(1 << 22) - 1, ws_bytes=64) == -3
    # the pre-rotated variant does not need the table
    assert _attn(b, table=None, max_pos=0, ws_bytes=64, rope=False) == -3


def _plan(b, dtype=1, ws_bytes=1 << 30, ws=256, table=256, max_pos=1024, flags=0, num_blocks=10):
    return pip.load_library().minipic_prefill_plan(num_blocks, ctypes.byref(b), table, max_pos, ws, ws_bytes, flags,
                                                  dtype, None)


def _run(b, dtype=1, ws_bytes=1 << 30, q=256, out=256, ws=256, table=256, max_pos=1024, flags=0):
    return pip.load_library().minipic_prefill_run(q, 256, 256, 10, ctypes.byref(b), table, max_pos, 0.0, out, ws,
                                                 ws_bytes, flags, dtype, None)


def test_plan_and_run_validate_like_the_whole_call():
    # every check runs on the host before any HIP call, as for minipic_prefill_attn
    b = _batch()
    for fn in (_plan, _run):
        assert fn(_batch(head_dim=96)) == -2
        assert fn(_batch(num_reqs=-1)) == -1
        assert fn(b, dtype=7) == -2
        assert fn(b, table=None) == -1
        assert fn(b, max_pos=0) == -1
        assert fn(b, flags=0x10) == -1
        assert fn(b, ws=None) == -1
        assert fn(b, ws=256 + 4) == -1
        assert fn(b, ws_bytes=64) == -3
        assert fn(_batch(total_q=0, max_q_len=0)) == 0
    assert _plan(b, num_blocks=0) == -1
    assert _plan(b, num_blocks=-1) == -1
    # the plan takes no q, caches or output; the run does
    assert _run(b, q=None) == -1
    assert _run(b, out=None) == -1
    assert _plan(b, ws_bytes=64) == -3


def test_empty_batch_is_a_no_op():
    # nothing to compute: returns before any HIP call
    assert _attn(_batch(total_q=0, max_q_len=0)) == 0
    assert _attn(_batch(num_reqs=0, total_q=0, max_q_len=0)) == 0


def _decode(lib, b, dtype=pip.MINIPIC_BF16, flags=0, ws=1 << 20, cos=256, max_pos=64):
    return lib.minipic_decode_attn(256, 256, 256, 10, ctypes.byref(b), cos, max_pos, 0.0, 256, 256, ws,
                                   flags, dtype, None)


def test_decode_validation():
    """Every argument check runs before the first HIP call (testable without a GPU)."""
    lib = pip.load_library()
    one = dict(total_q=2, max_q_len=1, num_reqs=2)      # one query row per request
    assert _decode(lib, _batch(**one), dtype=pip.MINIPIC_F32) == -2
    assert _decode(lib, _batch(total_q=8, max_q_len=4, num_reqs=2)) == -1   # not one row per request
    assert b"one query row" in lib.minipic_last_error()
    assert _decode(lib, _batch(**one), flags=pip.MINIPIC_FLAG_ROTATE_Q) == -1
    assert _decode(lib, _batch(**one), cos=0) == -1
    assert _decode(lib, _batch(**one), max_pos=0) == -1
    assert _decode(lib, _batch(**one), max_pos=1 << 22) == -1
    assert _decode(lib, _batch(**one), ws=16) == -3
    assert _decode(lib, _batch(**one, head_dim=96)) == -2
    # the pre-rotated variant needs no table; an empty batch is a no-op
    b = _batch(**one)
    assert lib.minipic_decode_prerotated(256, 256, 256, 10, ctypes.byref(b), 0.0, 256, 256, 16, 0,
                                         pip.MINIPIC_BF16, None) == -3
    assert _decode(lib, _batch(num_reqs=0, total_q=0, max_q_len=0)) == 0


def test_decode_workspace_grows_with_the_batch():
    lib = pip.load_library()
    sizes = []
    for R, mb in [(1, 4), (1, 64), (4, 64), (64, 256)]:
        b = _batch(num_reqs=R, total_q=R, max_q_len=1, max_blocks_per_req=mb, max_ctx_len=16 * mb)
        n = ctypes.c_size_t(0)
        assert lib.minipic_decode_workspace_size(ctypes.byref(b), pip.MINIPIC_BF16, ctypes.byref(n)) == 0
        sizes.append(n.value)
    assert sizes == sorted(sizes) and sizes[0] >= 256
    # partial results of every (request, query head, split): at least Hq * (d + 2) floats per request
    assert sizes[-1] >= 64 * 8 * (128 + 2) * 4


def test_write_kv_validation():
    lib = pip.load_library()
    wk = lambda **kw: lib.minipic_write_kv(*[kw.get(k, v) for k, v in [
        ("k", 256), ("v", 256), ("slots", 256), ("n", 10), ("hkv", 8), ("d", 128), ("bs", 16), ("kc", 256),
        ("vc", 256), ("nb", 4), ("dtype", 1), ("stream", None)]])
    assert wk(bs=8) == -2
    assert wk(d=80) == -2
    assert wk(dtype=3) == -2
    assert wk(n=-1) == -1
    assert wk(hkv=0) == -1
    assert wk(k=None) == -1
    assert wk(n=0) == 0


def test_rope_table_validation():
    lib = pip.load_library()
    assert lib.minipic_rope_table(None, 10, 128, 1e4, None) == -1
    assert lib.minipic_rope_table(256, 0, 128, 1e4, None) == -1
    assert lib.minipic_rope_table(256, 10, 127, 1e4, None) == -1
    assert lib.minipic_rope_table(256, 10, 128, -1.0, None) == -1


def test_launch_plan_and_workspace():
    b = _batch(total_q=15872, max_q_len=15872, max_ctx_len=31232, max_blocks_per_req=1952)
    info = pip.minipic_get_launch_info(b, 1)
    assert info["tokens_per_tile"] == 64 and info["rows_per_tile"] == 256
    assert info["num_q_tiles"] == 248 and info["num_tiles"] == 248
    assert info["threads"] == 768          # 8 consumer + 4 producer waves
    ws = pip.minipic_workspace_size(b, 1)
    # per-tile key-block lists (16 B per block) and the partial-result slots (fp32 O, m, l per row)
    assert ws >= 248 * 1952 * 16 + info["partial_slots"] * 256 * (128 + 2) * 4
    assert info["partial_slots"] >= 64          # room to split every (tile, head) of the long suffix
    # a tiny batch gets a small workspace
    small = _batch(total_q=80, max_q_len=80, max_ctx_len=80, max_blocks_per_req=5, num_q_heads=4,
                   num_kv_heads=2, head_dim=64)
    si = pip.minipic_get_launch_info(small, 0)
    assert si["tokens_per_tile"] == 32 and si["num_q_tiles"] == 3
    assert pip.minipic_workspace_size(small, 0) < 8 << 20


def test_static_entry_rejects_on_the_host():
    """The allocation-free entry point refuses, before any HIP call, a batch whose workspace exceeds its array."""
    lib = pip.load_library()
    cap = pip.MINIPIC_STATIC_WORKSPACE_BYTES

    def call(b, err_word=None):
        return lib.minipic_prefill_attn_static(256, 256, 256, 10, ctypes.byref(b), 256, 1024, 0.0, 256, err_word, 0,
                                               pip.MINIPIC_BF16, None)
    big = _batch(total_q=65536, max_q_len=65536, max_ctx_len=131072, max_blocks_per_req=8192)
    assert pip.minipic_workspace_size(big, pip.MINIPIC_BF16) > cap
    assert call(big) == -3
    msg = lib.minipic_last_error()
    assert b"static workspace holds" in msg and str(cap).encode() in msg
    # every workload of the benchmark fits
    for name in ("c1", "c2", "c3", "c3w", "c4", "c5", "e4"):
        w = workload.make_config(name)
        assert metrics_workspace_bytes(w) <= cap, name
    assert call(_batch(), err_word=258) == -1          # err_word not 4-byte aligned
    assert call(_batch(num_kv_heads=3)) == -2         # the usual batch checks apply
    assert call(_batch(num_reqs=0)) == 0                          # nothing to do: no HIP call


def metrics_workspace_bytes(w):
    qi = np.asarray(w.q_indptr)
    b = _batch(num_reqs=w.num_reqs, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
               max_blocks_per_req=w.block_table.shape[1], total_q=int(qi[-1]), max_q_len=int(np.diff(qi).max()),
               max_ctx_len=int(w.ctx_len.max()))
    return pip.minipic_workspace_size(b, pip.MINIPIC_BF16 if w.dtype == "bf16" else pip.MINIPIC_F32)


@pytest.mark.parametrize("name", ["c1", "c1_cached", "c3_small", "c4_small", "c5_small", "c2"])
def test_pair_counter_matches_oracle_mask(name):
    w = workload.make_config(name)
    assert metrics.workload_pairs(w) == oracle.visible_pair_count(w)


def test_pair_counts_of_benchmark_layouts():
    # analytic counts of the layouts: c2 = sys 512 causal + 10 spans of 192 + PDep 64 over 2432..2495
    w = workload.make_config("c2")
    tri = lambda n: n * (n + 1) // 2
    want = tri(512) + 10 * tri(192) + sum(2432 + i + 1 for i in range(64))
    assert metrics.workload_pairs(w) == want
    w4 = workload.make_config("c4")
    want4 = 60 * tri(256) + sum(30720 + i + 1 for i in range(512))
    assert metrics.workload_pairs(w4) == want4
    # c3w: 64 requests, a 64-token PDep question over 10 documents of 112 tokens each
    w3w = workload.make_config("c3w")
    assert w3w.num_reqs == 64 and int(w3w.ctx_len.max()) == 10 * 112 + 64
    assert metrics.workload_pairs(w3w) == 64 * sum(1120 + i + 1 for i in range(64))


def test_generator_layout_invariants():
    w = workload.make_config("c3")
    # same pool span -> same physical blocks in two requests at different offsets
    seen = {}
    for r in range(w.num_reqs):
        for s0, seg in zip(w.seg_start[r], w.segments[r]):
            if seg.pool is None:
                continue
            blocks = tuple(w.block_table[r, s0 // 16:(s0 + seg.length) // 16])
            seen.setdefault(seg.pool, set()).add(blocks)
    assert all(len(v) == 1 for v in seen.values())
    # every physical block is used by one allocation only
    assert len(np.unique(w.tok_slot)) == len(w.tok_slot)
    # the draw is deterministic
    w2 = workload.make_config("c3")
    assert np.array_equal(w.q, w2.q) and np.array_equal(w.block_table, w2.block_table)


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38, np.inf], np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to even (1.0)
    b = workload.f32_to_bf16_bits(x)
    back = workload.bf16_bits_to_f32(b)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.015625 and back[3] == -2.5
    assert np.isinf(back[5])


def test_kernel_timing_rejects_reads_without_timed_calls():
    lib = pip.load_library()
    ms = (ctypes.c_float * 6)()
    n = ctypes.c_int32(-1)
    assert lib.minipic_set_kernel_timing(0) == 0
    assert lib.minipic_kernel_times(ms) == pip.MinipicError(-1, "").status
    assert lib.minipic_kernel_times_all(ms, 2, ctypes.byref(n)) == -1
    assert lib.minipic_set_kernel_timing(1) == 0
    assert lib.minipic_kernel_times_all(ms, 2, ctypes.byref(n)) == -1   # timing on, nothing timed yet
    assert lib.minipic_kernel_times_all(None, 2, ctypes.byref(n)) == -1
    assert lib.minipic_kernel_times_all(ms, -1, ctypes.byref(n)) == -1
    assert n.value == -1
    assert lib.minipic_set_kernel_timing(0) == 0
