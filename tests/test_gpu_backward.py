"""Parity of moe_layer_backward with the oracle's backward pass, through the C ABI.

Every gradient is compared element by element on small shapes that cover each
GEMM path (256- and 128-row tiles, the register-staged and decode kernels,
fp32), capacity drops, a router bias and a rank limit: dx per token, the three
expert-weight gradients per expert block, the router-weight gradient over the
whole tensor. The named workloads are checked
on sampled tokens and on sampled rows of the expert-weight gradients.
"""
import numpy as np
import pytest

import moe_inputs
import oracle
import routing_dispatch_expert_amd as moe
from tests.gpu_util import bits_to_f64, gpu_available, row_rel_err, say, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True)
def _gpu():
    assert gpu_available(), "GPU tests need an MI355X; run them with -m gpu on a GPU host"
    moe.lib()


BACK_CASES = [
    dict(T=300, d=256, E=8, k=2, d_ff=320, cf=1.25),                                   # 128-row tiles
    dict(T=257, d=128, E=16, k=4, d_ff=136, cf=0.6, P=4),                              # drops; K % 64 != 0
    dict(T=130, d=520, E=32, k=8, d_ff=72, cf=1.0, P=8, max_ranks=2, bias="zipf1.2"),  # rank limit, bias
    dict(T=64, d=128, E=8, k=2, d_ff=256, cf=1.25, dtype="f32", x_std=1 / np.sqrt(128), wr_std=1 / np.sqrt(128)),
    dict(T=16, d=256, E=32, k=4, d_ff=128, cf=2.0),                                    # decode-sized buckets
    dict(T=2048, d=256, E=4, k=2, d_ff=512, cf=1.25),                                  # 256-row tiles
    dict(T=1024, d=384, E=4, k=2, d_ff=192, cf=1.0),   # K-major weights, column tiles past N, stacked K
    dict(T=40, d=64, E=1, k=1, d_ff=64, cf=1.0),                                       # one expert: dense
    # 64 or more experts: the router weight gradient holds every expert in one block
    dict(T=200, d=136, E=64, k=6, d_ff=40, cf=2.0, bias="zipf1.2"),
    dict(T=100, d=64, E=96, k=4, d_ff=64, cf=1.0, dtype="f32", x_std=0.125, wr_std=0.125),
    dict(T=1200, d=256, E=32, k=8, d_ff=192, cf=1.0),  # C = 300: 320-row tiles for the GEMMs over d
    dict(T=1100, d=4096, E=4, k=2, d_ff=256, cf=1.25),  # C = 688, d >= 4096: 320-row tiles over d too
    # more than 1024 experts: the routed-count scan gives each thread several
    # experts; most experts get no copy
    dict(T=300, d=64, E=1500, k=4, d_ff=64, cf=2.0),
]


def _rel(got, ref):
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def _block_err(got, ref):
    """Per expert block (first axis): max|got - ref| / max|ref| within the block,
    the worst block returned. A block whose reference is exactly zero (an
    expert that kept no row) must come back exactly zero."""
    g, r = got.reshape(got.shape[0], -1), ref.reshape(ref.shape[0], -1)
    den, err = np.abs(r).max(1), np.abs(g - r).max(1)
    zero = den == 0
    assert np.all(err[zero] == 0), "a gradient block of an expert with no kept row is not zero"
    return float((err[~zero] / den[~zero]).max()) if np.any(~zero) else 0.0


@pytest.mark.parametrize("case", range(len(BACK_CASES)))
def test_backward_small_shapes_every_element(case):
    cfg = dict(BACK_CASES[case])
    cfg.setdefault("dtype", "bf16")
    wl = moe_inputs.custom(name=f"back{case}", seed=2000 + case, **cfg)
    say(f"backward {case}: {cfg}")
    dt = wl.dtype
    hw = wl.all_expert_weights()
    dout = wl.grad_out(1)
    ref = oracle.layer_backward(wl.x, wl.wr, lambda e: (hw[0][e], hw[1][e], hw[2][e]), dout, wl.T, wl.d, wl.d_ff,
                                wl.E, wl.k, wl.cf, dt, P=wl.P, bias=wl.bias_vec, max_ranks=wl.max_ranks)
    b = None if wl.bias_vec is None else torch.from_numpy(wl.bias_vec).cuda()
    r = moe.backward(to_dev(wl.x, dt), to_dev(wl.wr, dt), *(to_dev(a, dt) for a in hw), to_dev(dout, dt), wl.k, wl.cf,
                     P=wl.P, router_bias=b, max_ranks=wl.max_ranks)
    torch.cuda.synchronize()
    got = {key: bits_to_f64(to_host(r[name], dt), dt) for key, name in
           (("dx", "dx"), ("dwr", "dW_router"), ("dwg", "dW_gate"), ("dwu", "dW_up"), ("dwd", "dW_down"))}
    errs = {}
    errs["dx"] = float(row_rel_err(got["dx"], ref["dx"]).max())   # per token
    for key in ("dwg", "dwu", "dwd"):
        errs[key] = _block_err(got[key], ref[key])   # per expert
    errs["dwr"] = _rel(got["dwr"], ref["dwr"])
    if b is not None:
        errs["db"] = _rel(r["d_bias"].cpu().numpy().astype(np.float64), ref["db"])
    say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    tol = 2e-2 if dt == "bf16" else 1e-4
    for key, v in errs.items():
        assert v <= tol, (key, v)


# ------------------------------------------------ backward from kept state ---

# 128-, 256- and 320-row tiles, drops, a rank limit with a bias, fp32,
# decode-sized buckets; True where GEMM 1's LDS-DMA kernel writes g and u
# itself (256- and 320-row tiles, d % 128 == 0), so keeping them changes
# nothing in the forward
SAVED_CASES = [(0, False), (1, False), (2, False), (3, False), (4, False), (5, True), (6, True), (10, True),
               (11, True)]


@pytest.mark.parametrize("case,same_forward", SAVED_CASES)
def test_backward_from_kept_forward_state(case, same_forward):
    """A forward that keeps g, u and h: its output still matches the oracle
    (and equals the plain forward's bit for bit where GEMM 1 writes g and u
    itself), its g and u match the products of the bucket rows, and the
    backward that takes that state gives exactly the gradients of the one that
    recomputes it."""
    cfg = dict(BACK_CASES[case])
    cfg.setdefault("dtype", "bf16")
    wl = moe_inputs.custom(name=f"saved{case}", seed=2000 + case, **cfg)
    say(f"backward from kept state {case}: {cfg}")
    dt = wl.dtype
    hw = wl.all_expert_weights()
    x, wr = to_dev(wl.x, dt), to_dev(wl.wr, dt)
    dw = tuple(to_dev(a, dt) for a in hw)
    dout = to_dev(wl.grad_out(1), dt)
    b = None if wl.bias_vec is None else torch.from_numpy(wl.bias_vec).cuda()
    f = moe.forward(x, wr, *dw, wl.k, wl.cf, P=wl.P, router_bias=b, max_ranks=wl.max_ranks, keep_activations=True)
    plain = moe.forward(x, wr, *dw, wl.k, wl.cf, P=wl.P, router_bias=b, max_ranks=wl.max_ranks)
    torch.cuda.synchronize()
    if same_forward:
        assert torch.equal(f["out"].view(torch.uint8), plain["out"].view(torch.uint8))
    ref = oracle.layer_forward(wl.x, wl.wr, lambda e: (hw[0][e], hw[1][e], hw[2][e]), wl.T, wl.d, wl.d_ff, wl.E,
                               wl.k, wl.cf, dt, P=wl.P, bias=wl.bias_vec, max_ranks=wl.max_ranks)
    assert np.array_equal(f["topk_idx"].cpu().numpy(), ref["idx"])
    assert np.array_equal(f["slot"].cpu().numpy(), ref["slot"])
    tok = ref["tokens"]
    err = row_rel_err(bits_to_f64(to_host(f["out"], dt)[tok], dt), ref["out64"])
    tol = 2e-2 if dt == "bf16" else 1e-4
    assert err.max() <= tol, err.max()
    kept = f["kept_count"].cpu().numpy()
    X = bits_to_f64(to_host(f["buckets"], dt), dt)
    g, u = (bits_to_f64(to_host(f[n], dt), dt) for n in ("g", "u"))
    wg, wu = (bits_to_f64(a, dt) for a in hw[:2])
    for e in range(wl.E):
        n = int(kept[e])
        if n == 0:
            continue
        for got, w in ((g, wg), (u, wu)):
            assert row_rel_err(got[e, :n], X[e, :n] @ w[e].T).max() <= tol, e
    # rows past kept are not part of the kept state: NaN there must not reach any gradient
    for e in range(wl.E):
        for name in ("g", "u", "h"):
            f[name][e, int(kept[e]):] = float("nan")
    r0 = moe.backward(x, wr, *dw, dout, wl.k, wl.cf, P=wl.P, router_bias=b, max_ranks=wl.max_ranks,
                      want_d_bias=True)
    r1 = moe.backward(x, wr, *dw, dout, wl.k, wl.cf, P=wl.P, router_bias=b, max_ranks=wl.max_ranks,
                      want_d_bias=True, saved=f)
    torch.cuda.synchronize()
    for key in ("dx", "dW_router", "d_bias", "dW_gate", "dW_up", "dW_down"):
        assert torch.equal(r0[key].view(torch.uint8) if r0[key].dtype == torch.bfloat16 else r0[key],
                           r1[key].view(torch.uint8) if r1[key].dtype == torch.bfloat16 else r1[key]), key


# ---------------------------------------------------------- named workloads ---

FULL = ["mixtral_prefill", "zipf_skew_drops", "deepseek_v3_decode"]


@pytest.mark.parametrize("name", FULL)
def test_backward_named_workload_sampled(name):
    from tests.gpu_util import DeviceWeights
    wl = moe_inputs.workload(name)
    dt = wl.dtype
    say(f"backward workload {name}: T={wl.T} d={wl.d} E={wl.E} k={wl.k} d_ff={wl.d_ff}")
    host, dev = DeviceWeights.get(wl)
    dout = wl.grad_out(1)
    b = None if wl.bias_vec is None else torch.from_numpy(wl.bias_vec).cuda()
    r = moe.backward(to_dev(wl.x, dt), to_dev(wl.wr, dt), *dev, to_dev(dout, dt), wl.k, wl.cf, P=wl.P,
                     router_bias=b, max_ranks=wl.max_ranks, want_d_bias=True)
    torch.cuda.synchronize()
    del r["workspace"]
    torch.cuda.empty_cache()
    route = oracle.layer_forward(wl.x, wl.wr, lambda e: (host[0][e], host[1][e], host[2][e]), wl.T, wl.d, wl.d_ff,
                                 wl.E, wl.k, wl.cf, dt, P=wl.P, bias=wl.bias_vec, tokens=np.arange(0),
                                 max_ranks=wl.max_ranks)
    rng = np.random.default_rng(wl.seed + 17)
    T = wl.T
    tok = set(range(min(3, T))) | {T - 1} | set(rng.choice(T, size=min(8 if T > 64 else T, T), replace=False).tolist())
    fully = np.nonzero(np.all(route["slot"] < 0, axis=1))[0]
    if fully.size:
        tok |= set(rng.choice(fully, size=min(3, fully.size), replace=False).tolist())
    tok = sorted(tok)
    kept = route["kept"]
    touched = np.nonzero(kept > 0)[0]
    experts = sorted({int(touched[np.argmax(kept[touched])]), int(touched[np.argmin(kept[touched])]),
                      int(rng.choice(touched))})
    cols = [(e, int(f)) for e in experts for f in rng.choice(wl.d_ff, size=2, replace=False)]
    ref = oracle.layer_backward_sample(wl.x, wl.wr, lambda e: (host[0][e], host[1][e], host[2][e]), dout, wl.T,
                                       wl.d, wl.d_ff, wl.E, wl.k, wl.cf, dt, P=wl.P, bias=wl.bias_vec,
                                       max_ranks=wl.max_ranks, tokens=tok, cols=cols)
    dx = bits_to_f64(to_host(r["dx"], dt), dt)
    worst = 0.0
    for t in tok:
        e_ = _rel(dx[t], ref["dx"][t])
        worst = max(worst, e_)
        if np.all(route["slot"][t] < 0):  # fully dropped: dx = dout bit for bit
            assert np.array_equal(to_host(r["dx"], dt)[t].view(np.uint8), np.asarray(dout[t]).view(np.uint8))
    say(f"  dx over {len(tok)} tokens: max rel err {worst:.2e}")
    assert worst <= 2e-2
    # A weight-gradient row can be small because its dh is a near-cancelling sum
    # over d: dy is stored in bf16, so dh carries an absolute error of about
    # 2^-9 sqrt(sum_i (dy_i Wd_if)^2) whatever its size. Each sampled row is
    # therefore measured against the largest magnitude among the sampled rows
    # of the same gradient, not against its own.
    for key, name_ in (("dwd", "dW_down"), ("dwg", "dW_gate"), ("dwu", "dW_up")):
        scale = max(np.abs(ref[key][c]).max() for c in cols)
        for (e, f) in cols:
            g = r[name_][e, :, f] if key == "dwd" else r[name_][e, f, :]
            err = np.abs(bits_to_f64(to_host(g, dt), dt) - ref[key][(e, f)]).max() / scale
            assert err <= 2e-2, (key, e, f, err)
    # properties of the gate gradients at any size: sum_j dl[t, j] = 0 for every
    # token, so db and every column of dW_router sum to zero over the experts
    db = r["d_bias"].cpu().numpy().astype(np.float64)
    gwr = bits_to_f64(to_host(r["dW_router"], dt), dt)
    assert abs(db.sum()) <= 1e-3 * np.abs(db).sum() + 1e-6
    col = np.abs(gwr.sum(axis=0))
    assert np.all(col <= 2 ** -7 * np.abs(gwr).sum(axis=0) + 1e-6)
    if name == "deepseek_v3_decode":
        DeviceWeights.clear()
