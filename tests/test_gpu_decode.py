"""GPU parity of the decode entry points against the CPU oracle (needs an MI355X).

Decode is the prefill computation with one query row per request (the
request's last context token), so the oracle is the same function
(`oracle.workload_reference`) on the decode view of a workload. Every call
goes through the C ABI. Tolerance (bf16): max |err| <= 2e-2 and relative L2
error <= 1e-2 against the float64 oracle.
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


def stage(w):
    from position_independent_paged_amd.staging import DeviceWorkload
    return DeviceWorkload(w)


def oracle_rows(w, k_rotated=False):
    return np.concatenate([oracle.workload_reference(w, r, k_rotated=k_rotated) for r in range(w.num_reqs)])


def check(name, got, want):
    err = np.abs(got - want)
    mx = float(err.max())
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    say(f"  {name}: rows={got.shape[0]} max_abs={mx:.3e} rel_l2={rel:.3e}")
    assert np.isfinite(got).all(), name
    assert mx <= 2e-2 and rel <= 1e-2, (name, mx, rel)


def run_decode(w, prerotated=False):
    dw = stage(w)
    dw.write_new()
    if prerotated:
        dw.decode_prerotated()
    else:
        dw.decode()
    torch.cuda.synchronize()
    assert dw.decode_error_word() == 0
    return dw, dw.out.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", ["d3_small", "d4_small", "d5_small", "d2", "d3", "d4", "d5"])
def test_decode_parity(name):
    w = workload.make_config(name)
    say(f"decode {name}: R={w.num_reqs} Hq={w.num_q_heads} max_ctx={w.max_ctx_len}")
    _, got = run_decode(w)
    check(name, got, oracle_rows(w))


@pytest.mark.parametrize("name", ["d3_small", "d5_small"])
def test_decode_prerotated_parity(name):
    """The pre-rotated variant treats the cached keys as already rotated."""
    w = workload.make_config(name)
    say(f"decode prerotated {name}")
    _, got = run_decode(w, prerotated=True)
    check(name + "/prerot", got, oracle_rows(w, k_rotated=True))


def _decode_variant(G, d, seed, last_kind="pdep", global_prefix=True, nreq=3):
    """Requests of spans (one shared from a pool), an optional GLOBAL prefix
    and a last segment of `last_kind` whose last token decodes."""
    Hkv = 2
    rng = np.random.default_rng(seed)
    reqs = []
    for r in range(nreq):
        segs = [Segment("global", 32, fresh=False, pool=0)] if (global_prefix and r % 2 == 0) else []
        segs += [Segment("span", 16 * int(rng.integers(1, 12)), fresh=False) for _ in range(3)]
        segs += [Segment("span", 48, fresh=False, pool=1)]
        segs += [Segment(last_kind, int(rng.integers(1, 80)))]
        reqs.append(segs)
    w = workload.custom("v", reqs, pool_lengths=[32, 48], num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=d,
                        dtype="bf16", rope_theta=1e4 if d == 64 else 5e5, max_pos=8192, seed=seed)
    return workload.decode_view(w, seed=seed)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_heads_and_dims(G, d):
    w = _decode_variant(G, d, seed=G * 10 + d)
    say(f"decode variant G={G} d={d} ctx={list(w.ctx_len)}")
    _, got = run_decode(w)
    check(f"decode/G{G}/d{d}", got, oracle_rows(w))


@pytest.mark.parametrize("global_prefix", [False, True])
def test_decode_span_query(global_prefix):
    """A query inside an SSep span sees only its own span (and GLOBAL blocks)."""
    w = _decode_variant(4, 128, seed=7, last_kind="span", global_prefix=global_prefix)
    say(f"decode span query global={global_prefix} ctx={list(w.ctx_len)}")
    _, got = run_decode(w)
    check("decode/span", got, oracle_rows(w))


def test_decode_first_token_of_span():
    """A span of one token: the query sees only itself, so out = its value row."""
    reqs = [[Segment("span", 64, fresh=False), Segment("span", 1)]]
    w = workload.decode_view(workload.custom("one", reqs, num_q_heads=8, num_kv_heads=2, head_dim=128,
                                             dtype="bf16", rope_theta=5e5, max_pos=4096, seed=3))
    _, got = run_decode(w)
    v = w.as_f32(w.v_tok[w.tok_of_ctx[0][64]]).astype(np.float64)   # [Hkv, d]
    want = np.repeat(v, 4, axis=0)[None]
    check("decode/self", got, want)


def test_decode_deterministic():
    w = workload.make_config("d3_small")
    dw, a = run_decode(w)
    dw.decode()
    torch.cuda.synchronize()
    b = dw.out.float().cpu().numpy()
    assert np.array_equal(a.astype(np.float32), b)
