"""GPU parity of libminipic.so against the CPU oracle (needs an MI355X).

Every call goes through the C ABI (ctypes binding). Tolerances: fp32
workloads max |err| <= 1e-4; bf16 workloads max |err| <= 2e-2 and relative
L2 error <= 1e-2, against the float64 oracle on the same inputs.
"""
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


def compare_workload(w, out, rows_per_req=None, seed=0, q_rotated=True, k_rotated=False):
    """Compare `out` [total_q, Hq, d] with the oracle, all rows or a sample per request."""
    rng = np.random.default_rng(seed)
    got_all, want_all = [], []
    for r in range(w.num_reqs):
        q0, q1 = int(w.q_indptr[r]), int(w.q_indptr[r + 1])
        if q1 == q0:
            continue
        rows = np.arange(q1 - q0)
        if rows_per_req is not None and len(rows) > rows_per_req:
            # always include the last rows (longest context) and a spread of the rest
            tail = rows[-min(64, rows_per_req // 2):]
            rest = rng.choice(rows[:-len(tail)], rows_per_req - len(tail), replace=False)
            rows = np.sort(np.concatenate([rest, tail]))
        want_all.append(oracle.workload_reference(w, r, rows=rows, q_rotated=q_rotated, k_rotated=k_rotated))
        got_all.append(out[q0 + rows])
    return np.concatenate(got_all), np.concatenate(want_all)


# ---------------------------------------------------------------------------
# tables and cache writes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,base,max_pos", [(64, 1e4, 128), (128, 5e5, 32768)])
def test_rope_table(d, base, max_pos):
    import position_independent_paged_amd as pip
    say(f"rope_table d={d} base={base} max_pos={max_pos}")
    cs = torch.empty((max_pos, d), dtype=torch.float32, device="cuda")
    pip.minipic_rope_table(cs, max_pos, d, base)
    torch.cuda.synchronize()
    ang = oracle.rope_angles(np.arange(max_pos), d, base)
    want = np.concatenate([np.cos(ang), np.sin(ang)], axis=1)
    got = cs.cpu().numpy().astype(np.float64)
    assert np.abs(got - want).max() <= 6e-8


@pytest.mark.parametrize("name", ["c1", "c3_small", "c5_small"])
def test_write_kv_bit_exact(name):
    w = workload.make_config(name)
    say(f"write_kv {name}")
    dw = stage(w)
    dw.write_new()
    torch.cuda.synchronize()
    bits = np.uint16 if w.dtype == "bf16" else np.uint32
    view = torch.int16 if w.dtype == "bf16" else torch.int32
    kc = dw.k_cache.view(view).cpu().numpy().view(bits)
    vc = dw.v_cache.view(view).cpu().numpy().view(bits)
    ktok = np.asarray(w.k_tok).view(bits)
    vtok = np.asarray(w.v_tok).view(bits)
    # host scatter of every token (set-up and new) into the documented layouts
    kref = np.zeros_like(kc)
    vref = np.zeros_like(vc)
    slots = w.tok_slot
    blk, off = slots // 16, slots % 16
    kref[blk, :, off, :] = ktok
    vref[blk, :, :, off] = vtok
    assert np.array_equal(kc, kref)
    assert np.array_equal(vc, vref)


def test_write_kv_scattered_and_skipped_slots():
    """Tokens that do not fill a block in order take the element-wise path;
    negative slots are skipped."""
    rng = np.random.default_rng(11)
    from position_independent_paged_amd import minipic_write_kv
    n, hkv, d, nb = 45, 2, 128, 8
    k = torch.from_numpy(rng.standard_normal((n, hkv, d), dtype=np.float32)).to(torch.bfloat16).cuda()
    v = torch.from_numpy(rng.standard_normal((n, hkv, d), dtype=np.float32)).to(torch.bfloat16).cuda()
    slots = rng.permutation(nb * 16)[:n].astype(np.int64)
    slots[[3, 17, 40]] = -1
    kc = torch.zeros((nb, hkv, 16, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros((nb, hkv, d, 16), dtype=torch.bfloat16, device="cuda")
    say("write_kv scattered")
    minipic_write_kv(k, v, torch.from_numpy(slots).cuda(), kc, vc, num_kv_heads=hkv, head_dim=d, num_blocks=nb)
    torch.cuda.synchronize()
    kr = torch.zeros_like(kc).cpu()
    vr = torch.zeros_like(vc).cpu()
    kh, vh = k.cpu(), v.cpu()
    for t, s in enumerate(slots):
        if s >= 0:
            kr[s // 16, :, s % 16, :] = kh[t]
            vr[s // 16, :, :, s % 16] = vh[t]
    assert torch.equal(kc.cpu().view(torch.int16), kr.view(torch.int16))
    assert torch.equal(vc.cpu().view(torch.int16), vr.view(torch.int16))


# ---------------------------------------------------------------------------
# attention parity
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["c1", "c1_cached", "c3_small", "c4_small", "c5_small", "c2", "c3", "c3w", "e2",
                                  "e4_small"])
def test_parity_all_rows(name):
    w = workload.make_config(name)
    say(f"parity {name}: dtype={w.dtype} R={w.num_reqs} total_q={w.total_q} max_ctx={w.max_ctx_len}")
    dw = stage(w)
    say(f"  plan {dw.launch_info()}")
    dw.step()
    torch.cuda.synchronize()
    assert dw.error_word() == 0
    got, want = compare_workload(w, out_f64(dw.out))
    check(name, got, want, w.dtype)


def check_full(name, got, want):
    """bf16 bar at full size: max abs <= 2e-2 and rel-L2 <= 1e-2 against the
    oracle. An output of magnitude 4 or more is stored in bf16 with a spacing
    of 2^-5, so its rounding alone can reach 1.6e-2; where the max abs bar is
    exceeded, the comparison is repeated against the oracle rounded to bf16 (the
    output type), which must then meet the same 2e-2."""
    err = np.abs(got - want)
    mx = float(err.max())
    rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    i = np.unravel_index(int(np.argmax(err)), err.shape)
    say(f"  {name}: rows={got.shape[0]} max_abs={mx:.3e} (|want| there {abs(want[i]):.3f}) rel_l2={rel:.3e}")
    assert np.isfinite(got).all(), name
    assert rel <= 1e-2, (name, rel)
    if mx > 2e-2:
        want_b = workload.bf16_bits_to_f32(workload.f32_to_bf16_bits(want.astype(np.float32))).astype(np.float64)
        mx_b = float(np.abs(got - want_b).max())
        say(f"  {name}: max_abs against the oracle rounded to bf16 = {mx_b:.3e}")
        assert mx_b <= 2e-2, (name, mx, mx_b)


def full_size_rows(w, r, rng, sample):
    """Rows of request r to compare: every PDep row, every row of one seeded
    span segment with queries, and a seeded sample of the rest."""
    q0, q1 = int(w.q_indptr[r]), int(w.q_indptr[r + 1])
    qc = w.q_ctx_idx[q0:q1]
    pdep = (w.blk_flags[r, qc // 16] & workload.FLAG_PDEP) != 0
    pick = pdep.copy()
    spans = [(s0, seg.length) for s0, seg in zip(w.seg_start[r], w.segments[r])
             if seg.kind == "span" and seg.fresh and seg.pool is None]
    if spans:
        s0, n = spans[int(rng.integers(len(spans)))]
        pick |= (qc >= s0) & (qc < s0 + n)
    rest = np.nonzero(~pick)[0]
    if len(rest):
        pick[rng.choice(rest, size=min(sample, len(rest)), replace=False)] = True
    return np.nonzero(pick)[0]


@pytest.mark.parametrize("name,sample", [("c4", 128), ("c5", 32), ("e4", 0)])
def test_parity_full_size(name, sample):
    """The full benchmark layouts in the configuration bench.py times: every
    PDep row (the long-context rows, split and merged), one whole span
    segment per request, and a sample of the other rows."""
    w = workload.make_config(name)
    say(f"parity(full size) {name}: total_q={w.total_q} max_ctx={w.max_ctx_len}")
    dw = stage(w)
    say(f"  plan {dw.launch_info()}")
    dw.step()
    torch.cuda.synchronize()
    assert dw.error_word() == 0
    out = out_f64(dw.out)
    rng = np.random.default_rng(1)
    got, want = [], []
    for r in range(w.num_reqs):
        rows = full_size_rows(w, r, rng, sample)
        q0 = int(w.q_indptr[r])
        want.append(oracle.workload_reference(w, r, rows=rows))
        got.append(out[q0 + rows])
    check_full(name, np.concatenate(got), np.concatenate(want))


def _sweep_layout(kind):
    if kind == "causal16k":
        return workload.custom("causal16k", [[Segment("pdep", 16384)]], num_q_heads=32, num_kv_heads=8,
                               head_dim=128, dtype="bf16", rope_theta=5e5, max_pos=32768, seed=16)
    return workload.custom("docs32", [[Segment("span", 1008) for _ in range(32)]], num_q_heads=32,
                           num_kv_heads=8, head_dim=128, dtype="bf16", rope_theta=5e5, max_pos=32768, seed=32)


@pytest.mark.parametrize("kind", ["causal16k", "docs32"])
def test_parity_sweep_sizes(kind):
    """Layouts of the preload sweeps at their own sizes: one 16K-token causal
    prompt (every row PDep, the last q tile included) and 32 documents of 1008
    tokens prefilled together as SSep spans."""
    w = _sweep_layout(kind)
    say(f"parity(sweep size) {kind}: total_q={w.total_q}")
    dw = stage(w)
    say(f"  plan {dw.launch_info()}")
    dw.step()
    torch.cuda.synchronize()
    assert dw.error_word() == 0
    rng = np.random.default_rng(2)
    n = int(w.total_q)
    rows = np.unique(np.concatenate([np.arange(n - 64, n), rng.choice(n - 64, size=96, replace=False)]))
    want = oracle.workload_reference(w, 0, rows=rows)
    check_full(kind, out_f64(dw.out)[rows], want)


@pytest.mark.parametrize("name", ["c1", "c3_small", "c5_small"])
def test_prerotated_kernel_parity(name):
    """The pre-rotated variant treats the cached keys as already rotated."""
    w = workload.make_config(name)
    say(f"prerotated {name}")
    dw = stage(w)
    dw.write_new()
    dw.attend_prerotated()
    torch.cuda.synchronize()
    got, want = compare_workload(w, out_f64(dw.out), k_rotated=True)
    check(name + "/prerot", got, want, w.dtype)


@pytest.mark.parametrize("name", ["c1", "c3_small"])
def test_rotate_q_flag(name):
    import position_independent_paged_amd as pip
    w = workload.make_config(name)
    say(f"rotate_q {name}")
    dw = stage(w, flags=pip.MINIPIC_FLAG_ROTATE_Q)
    dw.step()
    torch.cuda.synchronize()
    got, want = compare_workload(w, out_f64(dw.out), q_rotated=False)
    check(name + "/rotq", got, want, w.dtype)


def _variant(dtype, G, d, seed, positions_shift=0, nreq=2):
    Hkv = 2
    rng = np.random.default_rng(seed)
    reqs = []
    for r in range(nreq):
        segs = [Segment("global", 32, fresh=False, pool=0)] if r % 2 else []
        segs += [Segment("span", 16 * int(rng.integers(1, 9))) for _ in range(3)]
        segs += [Segment("span", 48, fresh=False, pool=1)]
        segs += [Segment("pdep", int(rng.integers(5, 70)))]
        reqs.append(segs)
    pos = None
    w0 = workload.custom("v", reqs, pool_lengths=[32, 48], num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=d,
                         dtype=dtype, rope_theta=1e4 if d == 64 else 5e5, max_pos=8192, seed=seed)
    if positions_shift:
        pos = [np.arange(int(L), dtype=np.int32) + positions_shift for L in w0.ctx_len]
        w0 = workload.custom("v", reqs, pool_lengths=[32, 48], num_q_heads=Hkv * G, num_kv_heads=Hkv,
                             head_dim=d, dtype=dtype, rope_theta=1e4 if d == 64 else 5e5, max_pos=8192,
                             seed=seed, positions=pos)
    return w0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
def test_parity_heads_and_dims(dtype, G, d):
    w = _variant(dtype, G, d, seed=G * 100 + d)
    say(f"variant dtype={dtype} G={G} d={d} total_q={w.total_q}")
    dw = stage(w)
    dw.step()
    torch.cuda.synchronize()
    assert dw.error_word() == 0
    got, want = compare_workload(w, out_f64(dw.out))
    check(f"{dtype}/G{G}/d{d}", got, want, dtype)


def test_shifted_positions():
    """Logical positions far from the context index (a span reused late in a
    long prompt); with Q rotated in-kernel by its own position the output
    matches the oracle, which depends only on position differences."""
    import position_independent_paged_amd as pip
    w = _variant("bf16", 4, 128, seed=5, positions_shift=6000)
    say("shifted positions")
    dw = stage(w, flags=pip.MINIPIC_FLAG_ROTATE_Q)
    dw.step()
    torch.cuda.synchronize()
    got, want = compare_workload(w, out_f64(dw.out), q_rotated=False)
    check("shift6000", got, want, "bf16")


@pytest.mark.parametrize("flags", ["rotate_q", "prerotated_q"])
def test_nonconsecutive_positions(flags):
    """Logical positions that do not run consecutively inside a block (every
    other block reversed, some far from the context index): those blocks take
    the per-key position look-up instead of the block's base position."""
    import position_independent_paged_amd as pip
    w0 = _variant("bf16", 4, 128, seed=11)
    pos = []
    for r, L in enumerate(w0.ctx_len):
        p_ = np.arange(int(L), dtype=np.int32)
        for b0 in range(0, int(L), 32):                     # reverse the positions of every other block
            blk = p_[b0:b0 + 16]
            p_[b0:b0 + len(blk)] = blk[::-1] + 3000 * (r + 1)
        pos.append(p_)
    w = workload.custom("v", w0.segments, pool_lengths=[32, 48], num_q_heads=8, num_kv_heads=2, head_dim=128,
                        dtype="bf16", rope_theta=5e5, max_pos=8192, seed=11, positions=pos)
    say(f"non-consecutive positions ({flags}) ctx={list(w.ctx_len)}")
    dw = stage(w, flags=pip.MINIPIC_FLAG_ROTATE_Q if flags == "rotate_q" else 0)
    dw.step()
    torch.cuda.synchronize()
    assert dw.error_word() == 0
    got, want = compare_workload(w, out_f64(dw.out), q_rotated=flags != "rotate_q")
    check(f"nonconsecutive/{flags}", got, want, "bf16")


def test_edge_layouts():
    """A request with no query rows, one single-token request, the same pool
    span twice in one request, queries that are not a suffix, and a ragged
    final block."""
    reqs = [
        [Segment("span", 64, fresh=False, pool=0)],                                   # no queries
        [Segment("pdep", 1)],                                                          # single token
        [Segment("span", 64, fresh=False, pool=0), Segment("span", 32), Segment("span", 64, fresh=False, pool=0),
         Segment("span", 48), Segment("pdep", 23)],                                    # same blocks twice
        [Segment("span", 16), Segment("span", 96, fresh=False), Segment("span", 80), Segment("pdep", 7)],
    ]
    for dtype in ("bf16", "f32"):
        w = workload.custom("edge", reqs, pool_lengths=[64], num_q_heads=8, num_kv_heads=2, head_dim=128,
                            dtype=dtype, rope_theta=5e5, max_pos=4096, seed=9)
        say(f"edge layouts {dtype} q_indptr={w.q_indptr.tolist()}")
        dw = stage(w)
        dw.step()
        torch.cuda.synchronize()
        assert dw.error_word() == 0
        got, want = compare_workload(w, out_f64(dw.out))
        check(f"edge/{dtype}", got, want, dtype)


def test_deterministic():
    w = workload.make_config("c4_small")
    say("determinism c4_small")
    dw = stage(w)
    dw.step()
    a = dw.out.clone()
    dw.attend()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), dw.out.view(torch.int16))


def test_kernel_timing_of_a_run_of_calls():
    """The timing record keeps every call made while timing is on and does not change the result."""
    from position_independent_paged_amd import (minipic_kernel_times, minipic_kernel_times_all,
                                                minipic_set_kernel_timing)
    w = workload.make_config("c3_small")
    say("kernel timing c3_small")
    dw = stage(w)
    dw.step()
    torch.cuda.synchronize()
    ref = dw.out.clone()
    minipic_set_kernel_timing(True)
    try:
        for _ in range(5):
            dw.attend()
        times = minipic_kernel_times_all(16)
        last = minipic_kernel_times()
    finally:
        minipic_set_kernel_timing(False)
    assert len(times) == 5
    for t in times:
        assert all(x > 0 for x in t), t
    assert last == times[-1]
    assert torch.equal(ref.view(torch.int16), dw.out.view(torch.int16))


def test_parity_context_beyond_one_planning_pass():
    """More than 2048 key blocks in one request: the planner's span-start search and its later passes
    read block descriptors past the first pass (loaded at kernel start); the PDep rows' lists run over
    nine staging passes of the attention kernel. Sampled span and PDep rows against the oracle."""
    segs = [Segment("global", 64, fresh=False, pool=0)]
    segs += [Segment("span", 240, fresh=False) for _ in range(140)]
    segs += [Segment("span", 256), Segment("span", 256), Segment("pdep", 64)]
    w = workload.custom("long", [segs], pool_lengths=[64], num_q_heads=8, num_kv_heads=2, head_dim=64,
                        dtype="bf16", rope_theta=5e5, max_pos=65536, seed=11)
    assert w.block_table.shape[1] > 2048
    say(f"parity long context: ctx={w.max_ctx_len} blocks={w.block_table.shape[1]} total_q={w.total_q}")
    dw = stage(w)
    say(f"  plan {dw.launch_info()}")
    dw.step()
    torch.cuda.synchronize()
    assert dw.error_word() == 0
    got, want = compare_workload(w, out_f64(dw.out), rows_per_req=160, seed=2)
    check("long", got, want, w.dtype)
