"""End-to-end parity of moe_layer_forward with the CPU oracle.

Small shapes are compared on every output element; the named workloads at
their full sizes are compared bit for bit on all routing outputs (indices,
counts, slots, drop masks, inverse map, statistics, every expert's
send-buffer rows) and on the layer output of every token (1024 tokens of the
two DeepSeek-V3-shaped prefill batches), plus every kept row of both expert
GEMMs (32 experts on the DeepSeek-V3 prefill shapes). Every output array is
followed by a canary region that must come back unchanged.
Layer output metric: per token max|got - ref| / max|ref|, at most 2e-2 for
bf16 and 1e-4 for fp32.
"""
import numpy as np
import pytest

import moe_inputs
import oracle
import routing_dispatch_expert_amd as moe
from tests.gpu_util import (DeviceWeights, Guarded, bits_to_f64, gpu_available, row_rel_err, say, to_dev,
                            to_host)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = {"bf16": 2e-2, "f32": 1e-4}


@pytest.fixture(autouse=True)
def _gpu():
    assert gpu_available(), "GPU tests need an MI355X; run them with -m gpu on a GPU host"
    moe.lib()


def run_layer(wl, wg, wu, wd, want_buckets=True):
    """moe_layer_forward with every output (and the buckets) in guarded buffers."""
    T, d, E, k, P = wl.T, wl.d, wl.E, wl.k, wl.P
    x = to_dev(wl.x, wl.dtype)
    C = moe.moe_capacity(T, E, k, wl.cf)
    g = Guarded()
    tdt = x.dtype
    r = {"C": C, "out": g.empty((T, d), tdt, "out"), "topk_idx": g.empty((T, k), torch.int32, "topk_idx"),
         "topk_w": g.empty((T, k), torch.float32, "topk_w"), "slot": g.empty((T, k), torch.int32, "slot"),
         "src": g.empty((E, C), torch.int32, "src"), "routed_count": g.empty((E,), torch.int32, "routed"),
         "kept_count": g.empty((E,), torch.int32, "kept"), "send_count": g.empty((P,), torch.int32, "send"),
         "totals": g.empty((4,), torch.int64, "totals")}
    if want_buckets:
        r["buckets"] = g.empty((E, C, d), tdt, "buckets")
    b = None if wl.bias_vec is None else torch.from_numpy(wl.bias_vec).cuda()
    n = moe.moe_workspace_size(T, d, wl.d_ff, E, k, wl.cf, P, wl.dtype)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    moe.moe_layer_forward(x, to_dev(wl.wr, wl.dtype), b, wg, wu, wd, T, d, wl.d_ff, E, k, wl.cf, P, wl.max_ranks,
                          wl.dtype, r["out"], r, ws, n)
    torch.cuda.synchronize()
    g.check()
    return r


def check_routing(wl, r, ref):
    C = ref["C"]
    assert r["C"] == C
    assert np.array_equal(r["topk_idx"].cpu().numpy(), ref["idx"]), "topk_idx"
    assert np.array_equal(r["slot"].cpu().numpy(), ref["slot"]), "slot"
    assert np.array_equal(r["src"].cpu().numpy().reshape(-1), ref["src"]), "src"
    assert np.array_equal(r["routed_count"].cpu().numpy(), ref["routed"]), "routed"
    assert np.array_equal(r["kept_count"].cpu().numpy(), ref["kept"]), "kept"
    st = ref["stats"]
    assert np.array_equal(r["send_count"].cpu().numpy(), st["send_count"]), "send_count"
    assert r["totals"].cpu().numpy().tolist() == [st["dropped"], st["fully_dropped_tokens"], st["padded_rows"],
                                                  st["offrank_bytes"]], "totals"
    # gates: the scores differ from the fp64 reference by accumulation error
    # only (well under 1e-4 at these shapes; the near-tie gap is 1e-3)
    w = r["topk_w"].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(w - ref["w"]) <= 2e-4 * ref["w"] + 1e-7), "topk_w"


def check_buckets(wl, r, ref, experts=None):
    """Kept bucket rows are bit copies of their tokens' rows (every expert
    unless a subset is given)."""
    got = to_host(r["buckets"], wl.dtype)
    C, k = ref["C"], wl.k
    src = ref["src"].reshape(-1, C)
    experts = range(wl.E) if experts is None else experts
    for e in experts:
        n = ref["kept"][e]
        rows = src[e, :n] // k
        assert np.array_equal(got[e, :n].view(np.uint8), wl.x[rows].view(np.uint8)), f"bucket rows of expert {e}"


def check_out(wl, r, ref):
    tok = ref["tokens"]
    got = to_host(r["out"], wl.dtype)[tok]
    slot = ref["slot"][tok]
    dropped = np.all(slot < 0, axis=1)
    assert np.array_equal(got[dropped].view(np.uint8), wl.x[tok][dropped].view(np.uint8)), "pass-through"
    err = row_rel_err(bits_to_f64(got, wl.dtype), ref["out64"])
    say(f"  out max rel err {err.max():.3e} over {tok.size} tokens ({dropped.sum()} fully dropped)")
    assert err.max() <= TOL[wl.dtype]
    return err.max()


# ------------------------------------------------------------- small shapes ---

SMALL = [
    dict(T=300, d=256, E=8, k=2, d_ff=320, cf=1.25),
    dict(T=257, d=128, E=16, k=4, d_ff=136, cf=0.6, P=4),
    dict(T=130, d=520, E=32, k=8, d_ff=72, cf=1.0, P=8, bias="zipf1.2"),
    dict(T=64, d=128, E=8, k=2, d_ff=256, cf=1.25, dtype="f32", x_std=1 / np.sqrt(128),
         wr_std=1 / np.sqrt(128)),
    dict(T=99, d=64, E=4, k=2, d_ff=96, cf=0.3, dtype="f32", x_std=0.125, wr_std=0.125),
    dict(T=1, d=64, E=8, k=2, d_ff=64, cf=1.0),
    dict(T=40, d=64, E=1, k=1, d_ff=64, cf=1.0),
    dict(T=500, d=64, E=4, k=1, d_ff=64, cf=0.1, bias="hot0"),
    dict(T=200, d=72, E=64, k=6, d_ff=40, cf=2.0),
    dict(T=1200, d=256, E=32, k=8, d_ff=256, cf=1.0),   # C = 300: 320-row tiles in both GEMMs
    # rank-limited routing: each token's experts on at most max_ranks of the P ranks
    dict(T=300, d=256, E=32, k=4, d_ff=96, cf=1.0, P=8, max_ranks=2),
    dict(T=130, d=1024, E=64, k=6, d_ff=72, cf=1.25, P=8, max_ranks=1, bias="zipf1.2"),
    dict(T=64, d=128, E=8, k=2, d_ff=64, cf=1.25, P=4, max_ranks=1, dtype="f32", x_std=1 / np.sqrt(128),
         wr_std=1 / np.sqrt(128)),
    # k E > 8192: the route kernel ranks each tile's copies with one wave instead of all sixteen
    dict(T=150, d=64, E=1024, k=16, d_ff=32, cf=2.0, P=4),
    # the most experts: the scan takes them 1024 at a time; k E = 8192 ranks with all waves
    dict(T=100, d=64, E=4096, k=2, d_ff=32, cf=4.0, P=8),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_layer_small_shapes_every_element(case):
    cfg = dict(SMALL[case])
    cfg.setdefault("dtype", "bf16")
    wl = moe_inputs.custom(name=f"small{case}", seed=1000 + case, **cfg)
    say(f"layer small {case}: {cfg}")
    hw = wl.all_expert_weights()
    dw = tuple(to_dev(a, wl.dtype) for a in hw)
    r = run_layer(wl, *dw)
    ref = oracle.layer_forward(wl.x, wl.wr, lambda e: (hw[0][e], hw[1][e], hw[2][e]), wl.T, wl.d, wl.d_ff,
                               wl.E, wl.k, wl.cf, wl.dtype, P=wl.P, bias=wl.bias_vec, max_ranks=wl.max_ranks)
    check_routing(wl, r, ref)
    check_buckets(wl, r, ref, range(wl.E))
    check_out(wl, r, ref)


def test_layer_is_deterministic():
    wl = moe_inputs.custom(T=2000, d=256, E=16, k=4, d_ff=256, cf=0.8, seed=77, P=4)
    dw = tuple(to_dev(a, wl.dtype) for a in wl.all_expert_weights())
    a = run_layer(wl, *dw)
    b = run_layer(wl, *dw)
    for key in ("out", "topk_idx", "topk_w", "slot", "src", "routed_count", "kept_count", "send_count", "totals",
                "buckets"):
        assert torch.equal(a[key].view(torch.uint8) if a[key].dtype == torch.bfloat16 else a[key],
                           b[key].view(torch.uint8) if b[key].dtype == torch.bfloat16 else b[key]), key


@pytest.mark.parametrize("T,E,d,one_pass", [(2000, 16, 256, True), (9000, 48, 256, True), (9000, 1024, 64, False)])
def test_stage_events_change_nothing(T, E, d, one_pass):
    # one kernel places and copies the rows (the slots stage is empty) when
    # each block can add up the earlier tiles' counts: every expert's column
    # (E (nt - 1) <= 65536) or, per token, its copies' experts (k (nt - 1) <=
    # 256); 140 tiles of 1024 experts, 4 copies a token, is neither
    wl = moe_inputs.custom(T=T, d=d, E=E, k=4, d_ff=d, cf=0.8, seed=78, P=4)
    dw = tuple(to_dev(a, wl.dtype) for a in wl.all_expert_weights())
    a = run_layer(wl, *dw)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(moe.STAGES))]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    moe.moe_set_stage_events([e.cuda_event for e in evs])
    try:
        b = run_layer(wl, *dw)
        ran = [moe.moe_stage_ran(i) for i in range(len(moe.STAGES))]
    finally:
        moe.moe_set_stage_events(None)
    want = [True] * len(moe.STAGES)
    want[moe.STAGES.index("slots")] = not one_pass
    assert ran == want
    for i in range(len(moe.STAGES)):
        if ran[i]:
            assert evs[2 * i].elapsed_time(evs[2 * i + 1]) >= 0
    for key in ("out", "topk_idx", "topk_w", "slot", "src", "routed_count", "kept_count", "send_count", "totals",
                "buckets"):
        assert torch.equal(a[key].view(torch.uint8) if a[key].dtype == torch.bfloat16 else a[key],
                           b[key].view(torch.uint8) if b[key].dtype == torch.bfloat16 else b[key]), key


# ---------------------------------------------------------- named workloads ---

def _sample_tokens(wl, ref_slot, n_rand, seed):
    rng = np.random.default_rng(seed)
    T = wl.T
    picks = set(range(min(4, T))) | set(range(max(0, T - 4), T))
    picks |= set(rng.choice(T, size=min(n_rand, T), replace=False).tolist())
    fully = np.nonzero(np.all(ref_slot < 0, axis=1))[0]
    partly = np.nonzero(np.any(ref_slot < 0, axis=1) & np.any(ref_slot >= 0, axis=1))[0]
    for group in (fully, partly):
        if group.size:
            picks |= set(rng.choice(group, size=min(4, group.size), replace=False).tolist())
    return np.array(sorted(picks))


def check_expert_gemms_full(wl, r, host, dev, n_experts=None):
    """The stage GEMMs at the workload's full size, on the layer's own buckets
    and kept counts (so with the same tile lists and split rounds as the
    layer): every kept row of h and y is written, no padding row is, nothing
    past either array is, and every kept row of every expert (of n_experts
    experts, the fullest and emptiest touched ones among them, when given)
    matches the oracle."""
    E, C, d, F = wl.E, r["C"], wl.d, wl.d_ff
    kept_dev = r["kept_count"]
    kept = kept_dev.cpu().numpy()
    bf = wl.dtype == "bf16"
    g = Guarded()

    def sentinel(shape, name):
        t = g.empty(shape, torch.bfloat16 if bf else torch.float32, name)
        if bf:
            t.view(torch.int16).fill_(0x1234)
        else:
            t.fill_(777.0)
        return t

    h, y = sentinel((E, C, F), "h"), sentinel((E, C, d), "y")
    ws_n = moe.moe_grouped_gemm_workspace_size(E, C)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    moe.moe_grouped_gemm(r["buckets"], kept_dev, *dev, E, C, d, F, wl.dtype, h, y, ws, ws_n)
    torch.cuda.synchronize()
    g.check()
    live = torch.arange(C, device="cuda")[None, :] < kept_dev[:, None].long()
    for name, t in (("h", h), ("y", y)):
        is_sent = (t.view(torch.int16) == 0x1234) if bf else (t == 777.0)
        assert not is_sent.any(-1)[live].any().item(), f"{name}: a kept row left (partly) unwritten"
        assert is_sent.all(-1)[~live].all().item(), f"{name}: a padding row written"
    touched = np.nonzero(kept > 0)[0]
    if n_experts is None or n_experts >= touched.size:
        experts = touched.tolist()
    else:
        rng = np.random.default_rng(wl.seed + 5)
        pick = {int(touched[np.argmax(kept[touched])]), int(touched[np.argmin(kept[touched])])}
        rest = [int(e) for e in touched if int(e) not in pick]
        pick |= set(rng.choice(rest, size=n_experts - len(pick), replace=False).tolist())
        experts = sorted(pick)
    tol_h, tol_y = (4e-3, 1e-2) if bf else (1e-5, 1e-5)
    src = r["src"].cpu().numpy()
    worst_h = worst_y = 0.0
    n_rows = 0
    for e in experts:
        n = int(kept[e])
        X = oracle.decode(wl.x[src[e, :n] // wl.k], wl.dtype)    # the tokens' rows, bit-checked in the buckets
        wg, wu, wd = (oracle.decode(a[e], wl.dtype) for a in host)
        got_h = bits_to_f64(to_host(h[e, :n], wl.dtype), wl.dtype)
        got_y = bits_to_f64(to_host(y[e, :n], wl.dtype), wl.dtype)
        eh = row_rel_err(got_h, oracle.expert_hidden(X, wg, wu)).max()
        ey = row_rel_err(got_y, oracle.expert_mlp(X, wg, wu, wd)).max()
        assert eh <= tol_h, f"h of expert {e}: {eh}"
        assert ey <= tol_y, f"y of expert {e}: {ey}"
        worst_h, worst_y, n_rows = max(worst_h, eh), max(worst_y, ey), n_rows + n
    say(f"  expert GEMMs at full size: all {int(kept.sum())} kept rows written; {n_rows} rows of "
        f"{len(experts)} experts match (h {worst_h:.2e}, y {worst_y:.2e})")


# tokens whose layer output the oracle computes (None: all of them), and the
# experts whose GEMM rows it computes in full (None: every touched expert)
WORKLOAD_TOKENS = {"tiny_f32": None, "mixtral_prefill": None, "deepseek_v3_prefill": 1024,
                   "deepseek_v3_node_limited": 1024, "deepseek_v3_decode": None, "zipf_skew_drops": None}
WORKLOAD_GEMM_EXPERTS = {"deepseek_v3_prefill": 32, "deepseek_v3_node_limited": 32}


@pytest.mark.parametrize("name", list(WORKLOAD_TOKENS))
def test_named_workload(name):
    wl = moe_inputs.workload(name)
    say(f"workload {name}: T={wl.T} d={wl.d} E={wl.E} k={wl.k} d_ff={wl.d_ff} cf={wl.cf} P={wl.P} "
        f"max_ranks={wl.max_ranks} {wl.dtype} (resampled {wl.resampled} near-tied tokens)")
    host, dev = DeviceWeights.get(wl)
    r = run_layer(wl, *dev)
    # routing, slots and statistics for every token (cheap in the oracle)
    ref_route = oracle.layer_forward(wl.x, wl.wr, lambda e: (host[0][e], host[1][e], host[2][e]), wl.T, wl.d,
                                     wl.d_ff, wl.E, wl.k, wl.cf, wl.dtype, P=wl.P, bias=wl.bias_vec,
                                     tokens=np.arange(0), max_ranks=wl.max_ranks)
    n = WORKLOAD_TOKENS[name]
    tokens = None if n is None else _sample_tokens(wl, ref_route["slot"], n, seed=wl.seed)
    ref = oracle.layer_forward(wl.x, wl.wr, lambda e: (host[0][e], host[1][e], host[2][e]), wl.T, wl.d, wl.d_ff,
                               wl.E, wl.k, wl.cf, wl.dtype, P=wl.P, bias=wl.bias_vec, tokens=tokens,
                               max_ranks=wl.max_ranks)
    check_routing(wl, r, ref)
    check_buckets(wl, r, ref)
    check_out(wl, r, ref)
    check_expert_gemms_full(wl, r, host, dev, WORKLOAD_GEMM_EXPERTS.get(name))
    if wl.max_ranks:
        ranks = r["topk_idx"].cpu().numpy() // (wl.E // wl.P)
        assert max(len(set(row)) for row in ranks.tolist()) <= wl.max_ranks
    st = ref["stats"]
    say(f"  dropped {st['dropped']} fully {st['fully_dropped_tokens']} padded {st['padded_rows']} "
        f"offrank MiB {st['offrank_bytes'] / 2**20:.1f}")
    if name == "deepseek_v3_decode":
        DeviceWeights.clear()
