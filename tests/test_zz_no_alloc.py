"""The allocation-free prefill entry point against the allocating one (needs an MI355X).

minipic_prefill_attn_static runs the kernels of minipic_prefill_attn on the
library's own device array instead of a caller workspace. Calls in a row on
one stream share that array and find the previous call's contents in it, so
the checks run several different batches in a row, each later one smaller
than the first, and compare every output with the allocating entry point's
output for the same inputs, bit for bit (the same plan and kernels run on
both). The error word, which the static call writes to a word of the
caller's, is checked on a batch with an out-of-range block id.
"""
import sys

import numpy as np
import pytest

import oracle
import workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def stage(name):
    from position_independent_paged_amd.staging import DeviceWorkload
    w = workload.make_config(name)
    dw = DeviceWorkload(w)
    dw.write_new()
    return w, dw


def run_both(dw, err_word):
    """(allocating output, static output, allocating error word) for one staged batch."""
    import position_independent_paged_amd as pip
    dw.workspace.zero_()
    dw.attend()
    want = dw.out.clone()
    got = torch.full_like(dw.out, float("nan"))
    err_word.zero_()
    pip.minipic_prefill_attn_static(dw.q, dw.k_cache, dw.v_cache, dw.num_blocks, dw.batch.struct, dw.cos_sin,
                                    dw.max_pos, got, err_word, flags=dw.flags)
    torch.cuda.synchronize()
    return want, got, int(dw.workspace[:4].view(torch.int32).item())


def test_static_workspace_matches_the_allocating_entry_point():
    import position_independent_paged_amd as pip
    err_word = torch.zeros(1, dtype=torch.int32, device="cuda")
    # the first batch is the largest: the later ones find its partial results,
    # lists and counters in the array
    for i, name in enumerate(["c5_small", "c3_small", "c1"]):
        w, dw = stage(name)
        need = pip.minipic_workspace_size(dw.batch.struct, dw.dtype_code)
        say(f"call {i}: {name} ({w.dtype}, {int(w.q_indptr[-1])} query rows, workspace {need} bytes)")
        assert need <= pip.MINIPIC_STATIC_WORKSPACE_BYTES
        want, got, ew = run_both(dw, err_word)
        assert ew == 0 and int(err_word.item()) == 0
        assert torch.isfinite(got.float()).all(), name
        same = torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got.view(torch.int32),
                           want.view(torch.int16) if want.dtype == torch.bfloat16 else want.view(torch.int32))
        say(f"  bit-identical to minipic_prefill_attn: {same}")
        assert same, name
        if name == "c3_small":
            # and both agree with the oracle (bf16 tolerance of the parity tests)
            ref = []
            for r in range(w.num_reqs):
                dd = w.request_dense(r)
                ref.append(oracle.prefill_attention(dd["q"], dd["q_ctx"], dd["k"], dd["v"], dd["pos"], dd["span_id"],
                                                    dd["flags"], block_size=w.block_size, theta=w.rope_theta))
            ref = np.concatenate(ref)
            g = got.float().cpu().numpy().astype(np.float64)
            mx = float(np.abs(g - ref).max())
            rel = float(np.linalg.norm(g - ref) / np.linalg.norm(ref))
            say(f"  against the oracle: max_abs={mx:.3e} rel_l2={rel:.3e}")
            assert mx <= 2e-2 and rel <= 1e-2
        del dw


def test_static_error_word_goes_to_the_callers_word():
    import position_independent_paged_amd as pip
    w, dw = stage("c3_small")
    dw.batch.block_table[0, 0] = w.num_blocks + 7      # out of range: clamped and recorded
    torch.cuda.synchronize()
    err_word = torch.zeros(1, dtype=torch.int32, device="cuda")
    want, got, ew = run_both(dw, err_word)
    say(f"error words: allocating {ew:#x}, static {int(err_word.item()):#x}")
    assert ew & pip.MINIPIC_EW_BLOCK
    assert int(err_word.item()) == ew
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    # without a word of the caller's the bits are dropped and the call still completes
    out2 = torch.full_like(dw.out, float("nan"))
    pip.minipic_prefill_attn_static(dw.q, dw.k_cache, dw.v_cache, dw.num_blocks, dw.batch.struct, dw.cos_sin,
                                    dw.max_pos, out2, None, flags=dw.flags)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), want.view(torch.int16))


def test_static_rejects_a_batch_beyond_its_array():
    import position_independent_paged_amd as pip
    from position_independent_paged_amd._binding import minipic_batch
    big = minipic_batch(num_reqs=1, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                        max_blocks_per_req=8192, total_q=65536, max_q_len=65536, max_ctx_len=131072,
                        q_indptr=256, q_ctx_idx=256, ctx_len=256, block_table=256, logical_pos=256, span_id=256,
                        blk_flags=256)
    assert pip.minipic_workspace_size(big, pip.MINIPIC_BF16) > pip.MINIPIC_STATIC_WORKSPACE_BYTES
    q = torch.zeros(1, dtype=torch.bfloat16, device="cuda")
    cs = torch.zeros(1, dtype=torch.float32, device="cuda")
    with pytest.raises(pip.MinipicError, match="static workspace holds"):
        pip.minipic_prefill_attn_static(q, q, q, 10, big, cs, 1024, q, None)
