"""Parity of moe_layer_forward_replicated (hot-expert replication) with the oracle.

Routing, per-instance slots, counts, send counts, statistics and bucket rows
are compared bit for bit; outputs element by element on small shapes and on
every token of the skewed workload at full size with a replica plan drawn
from its own routed counts.
"""
import numpy as np
import pytest

import moe_inputs
import oracle
import routing_dispatch_expert_amd as moe
from tests.gpu_util import DeviceWeights, bits_to_f64, gpu_available, row_rel_err, say, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = {"bf16": 2e-2, "f32": 1e-4}


@pytest.fixture(autouse=True)
def _gpu():
    assert gpu_available(), "GPU tests need an MI355X; run them with -m gpu on a GPU host"
    moe.lib()


def _run(wl, dev_w, reps):
    b = None if wl.bias_vec is None else torch.from_numpy(wl.bias_vec).cuda()
    r = moe.forward_replicated(to_dev(wl.x, wl.dtype), to_dev(wl.wr, wl.dtype), *dev_w, wl.k, wl.cf,
                               torch.from_numpy(np.asarray(reps, np.int32)).cuda(), P=wl.P, router_bias=b,
                               want_buckets=True, want_src=True, max_ranks=wl.max_ranks)
    torch.cuda.synchronize()
    return r


def _check(wl, r, ref, reps, tokens):
    C = ref["C"]
    assert np.array_equal(r["topk_idx"].cpu().numpy(), ref["idx"])
    assert np.array_equal(r["slot"].cpu().numpy(), ref["slot"])
    assert np.array_equal(r["instance"].cpu().numpy(), ref["instance"])
    assert np.array_equal(r["src"].cpu().numpy().reshape(-1), ref["src"])
    assert np.array_equal(r["routed_count"].cpu().numpy(), ref["routed"])
    assert np.array_equal(r["kept_count"].cpu().numpy(), ref["kept"])
    st = ref["stats"]
    assert np.array_equal(r["send_count"].cpu().numpy(), st["send_count"])
    assert r["totals"].cpu().numpy().tolist() == [st["dropped"], st["fully_dropped_tokens"], st["padded_rows"],
                                                  st["offrank_bytes"]]
    got_b = to_host(r["buckets"], wl.dtype)
    for i in range(len(ref["kept"])):
        n = ref["kept"][i]
        rows = ref["src"][i * C: i * C + n] // wl.k
        assert np.array_equal(got_b[i, :n].view(np.uint8), wl.x[rows].view(np.uint8))
    got = to_host(r["out"], wl.dtype)[tokens]
    drop = np.all(ref["slot"][tokens] < 0, axis=1)
    assert np.array_equal(got[drop].view(np.uint8), wl.x[tokens][drop].view(np.uint8))
    err = row_rel_err(bits_to_f64(got, wl.dtype), ref["out64"])
    say(f"  out max rel err {err.max():.3e}; dropped {st['dropped']}")
    assert err.max() <= TOL[wl.dtype]


SMALL = [
    (dict(T=300, d=256, E=8, k=2, d_ff=320, cf=0.5), [3, 1, 1, 2, 1, 1, 1, 1]),
    (dict(T=257, d=128, E=16, k=4, d_ff=136, cf=0.6, P=4, bias="zipf1.2"), None),   # plan from the counts
    (dict(T=64, d=128, E=8, k=2, d_ff=256, cf=1.0, dtype="f32", x_std=1 / np.sqrt(128), wr_std=1 / np.sqrt(128)),
     [2, 2, 1, 1, 1, 1, 1, 3]),
    (dict(T=600, d=64, E=4, k=1, d_ff=64, cf=0.1, bias="hot0"), [9, 1, 1, 1]),      # one hot expert
    (dict(T=2048, d=256, E=4, k=2, d_ff=512, cf=0.5), [2, 2, 2, 2]),                # 256-row tiles
    # C = 400: 256-row tiles for GEMM 1, 128-row for GEMM 2 (two row-tile maps from the scan)
    (dict(T=1280, d=256, E=4, k=1, d_ff=256, cf=1.25), [2, 1, 1, 1]),
    (dict(T=300, d=256, E=32, k=4, d_ff=96, cf=1.0, P=8, max_ranks=2, bias="zipf1.2"), None),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_replicated_small_shapes_every_element(case):
    cfg, reps = SMALL[case]
    cfg = dict(cfg)
    cfg.setdefault("dtype", "bf16")
    wl = moe_inputs.custom(name=f"rep{case}", seed=3000 + case, **cfg)
    hw = wl.all_expert_weights()
    if reps is None:
        base = oracle.layer_forward(wl.x, wl.wr, lambda e: (hw[0][e], hw[1][e], hw[2][e]), wl.T, wl.d, wl.d_ff, wl.E,
                                    wl.k, wl.cf, wl.dtype, P=wl.P, bias=wl.bias_vec, tokens=np.arange(0),
                                    max_ranks=wl.max_ranks)
        reps = oracle.replica_plan(base["routed"], 8)
    say(f"replicated {case}: {cfg} replicas {list(reps)}")
    dw = tuple(to_dev(a, wl.dtype) for a in hw)
    r = _run(wl, dw, reps)
    ref = oracle.layer_forward(wl.x, wl.wr, lambda e: (hw[0][e], hw[1][e], hw[2][e]), wl.T, wl.d, wl.d_ff, wl.E,
                               wl.k, wl.cf, wl.dtype, P=wl.P, bias=wl.bias_vec, replicas=reps,
                               max_ranks=wl.max_ranks)
    _check(wl, r, ref, reps, np.arange(wl.T))


def test_one_replica_each_is_the_plain_layer():
    wl = moe_inputs.custom(T=500, d=256, E=16, k=4, d_ff=192, cf=0.8, seed=3100, P=4)
    dw = tuple(to_dev(a, wl.dtype) for a in wl.all_expert_weights())
    r = _run(wl, dw, np.ones(wl.E, np.int32))
    p = moe.forward(to_dev(wl.x, wl.dtype), to_dev(wl.wr, wl.dtype), *dw, wl.k, wl.cf, P=wl.P, want_buckets=True,
                    want_src=True)
    torch.cuda.synchronize()
    for key in ("out", "topk_idx", "slot", "src", "routed_count", "kept_count", "send_count", "totals", "buckets"):
        a, b = r[key], p[key]
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b), key
    assert torch.equal(r["instance"], r["topk_idx"])


def test_replicated_skewed_workload_full_size():
    wl = moe_inputs.workload("zipf_skew_drops")
    host, dev = DeviceWeights.get(wl)
    base = oracle.layer_forward(wl.x, wl.wr, lambda e: (host[0][e], host[1][e], host[2][e]), wl.T, wl.d, wl.d_ff,
                                wl.E, wl.k, wl.cf, wl.dtype, P=wl.P, bias=wl.bias_vec, tokens=np.arange(0))
    reps = oracle.replica_plan(base["routed"], 16)
    say(f"zipf_skew_drops with 16 extra replicas: {reps.tolist()}")
    r = _run(wl, dev, reps)
    tok = np.arange(wl.T)    # every token's output
    ref = oracle.layer_forward(wl.x, wl.wr, lambda e: (host[0][e], host[1][e], host[2][e]), wl.T, wl.d, wl.d_ff,
                               wl.E, wl.k, wl.cf, wl.dtype, P=wl.P, bias=wl.bias_vec, replicas=reps, tokens=tok)
    _check(wl, r, ref, reps, tok)
    say(f"  drops {base['stats']['dropped']} -> {ref['stats']['dropped']}")
    assert ref["stats"]["dropped"] < base["stats"]["dropped"]
