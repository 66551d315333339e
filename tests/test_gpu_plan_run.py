"""Plan once, run per layer (needs an MI355X).

minipic_prefill_plan launches only the planning kernels; minipic_prefill_run
launches the attention and merge kernels on the plan in the workspace and
leaves it ready for the next run. One plan serves several "layers" (different
q and caches over the same batch): every run must equal a whole
minipic_prefill_attn call on the same data bit for bit, and a run without a
plan of its own configuration must compute nothing and say so in the error
word.
"""
import sys

import pytest

import workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def stage(w):
    from position_independent_paged_amd.staging import DeviceWorkload
    return DeviceWorkload(w)


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _layers(dw, n):
    """n (q, k_cache, v_cache) sets over the same batch: the workload's own and
    exact power-of-two rescalings of it (with q rows rolled), so every layer's
    result differs."""
    out = [(dw.q, dw.k_cache, dw.v_cache)]
    for i in range(1, n):
        s = 2.0 ** -i
        out.append((torch.roll(dw.q, i, dims=0).contiguous(), (dw.k_cache * s).contiguous(),
                    (dw.v_cache * (1.0 / s)).contiguous()))
    return out


@pytest.mark.parametrize("name", ["c4_small", "c5_small", "c1"])
def test_one_plan_serves_many_runs(name):
    w = workload.make_config(name)
    say(f"plan once, run per layer: {name}")
    dw = stage(w)
    dw.write_new()
    layers = _layers(dw, 3)
    k0, v0 = dw.k_cache, dw.v_cache
    refs = []
    for q, k, v in layers:   # whole calls (each plans again)
        dw.k_cache, dw.v_cache = k, v
        out = torch.empty_like(dw.out)
        dw.attend(out=out, q=q)
        torch.cuda.synchronize()
        refs.append(out)
    dw.k_cache, dw.v_cache = k0, v0
    assert dw.error_word() == 0
    dw.plan()
    for rep in range(2):     # the plan serves every layer, twice over
        for i, (q, k, v) in enumerate(layers):
            out = torch.full_like(dw.out, float("nan"))
            dw.run(out=out, q=q, k_cache=k, v_cache=v)
            torch.cuda.synchronize()
            assert torch.equal(_bits(out), _bits(refs[i])), f"{name}: pass {rep}, layer {i}"
    assert dw.error_word() == 0
    assert not torch.equal(_bits(refs[0]), _bits(refs[1]))


def test_run_without_its_plan_computes_nothing():
    from position_independent_paged_amd import MINIPIC_EW_PLAN, MINIPIC_FLAG_ROTATE_Q
    w = workload.make_config("c4_small")
    dw = stage(w)
    dw.write_new()
    dw.workspace.zero_()                  # no plan at all
    out = torch.full_like(dw.out, 3.0)
    dw.run(out=out)
    torch.cuda.synchronize()
    assert dw.error_word() == MINIPIC_EW_PLAN
    assert bool((out == 3.0).all())
    dw.workspace[:4].zero_()
    dw.plan()                             # a plan of flags 0 ...
    dw.run(out=out, flags=MINIPIC_FLAG_ROTATE_Q)   # ... does not serve a run with other flags
    torch.cuda.synchronize()
    assert dw.error_word() == MINIPIC_EW_PLAN
    assert bool((out == 3.0).all())
    dw.workspace[:4].zero_()
    dw.run(out=out)                       # the plan is still there for its own configuration
    torch.cuda.synchronize()
    assert dw.error_word() == 0
    ref = torch.empty_like(dw.out)
    dw.attend(out=ref)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref))


def test_plan_beside_write_kv_on_a_second_stream():
    """The bench's step schedule: planning on a second stream while write_kv runs on
    the first, then the run on the first stream; every step equals a whole call."""
    w = workload.make_config("c4_small")
    dw = stage(w)
    dw.write_new()
    ref = torch.empty_like(dw.out)
    dw.attend(out=ref)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for rep in range(3):
        out = torch.full_like(dw.out, float("nan"))
        cur = torch.cuda.current_stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            dw.plan()
        dw.write_new()
        cur.wait_stream(side)
        dw.run(out=out)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref)), f"pass {rep}"
    assert dw.error_word() == 0
