"""Parity of each stage of the HIP path with the CPU oracle, through the C ABI.

Routing indices, counts, slots, drop masks, inverse maps and bucket rows are
compared bit for bit; floating-point results within bounds derived from the
arithmetic (stated at each check).
"""
import numpy as np
import pytest

import moe_inputs
import oracle
import routing_dispatch_expert_amd as moe
from tests.gpu_util import (U, Guarded, bits_to_f64, gpu_available, logits_tolerance, row_rel_err, say, to_dev,
                            to_host)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True)
def _gpu():
    assert gpu_available(), "GPU tests need an MI355X; run them with -m gpu on a GPU host"
    moe.lib()


def _i32(*shape):
    return torch.empty(shape, dtype=torch.int32, device="cuda")


def _f32(*shape):
    return torch.empty(shape, dtype=torch.float32, device="cuda")


# ------------------------------------------------------------------ routing ---

ROUTE_CASES = [
    (1000, 8, 2, "ties"), (333, 256, 8, "ties"), (64, 64, 6, "zeros"), (50, 16, 16, "equal"),
    (77, 5, 5, "normal"), (4096, 1, 1, "normal"), (1000, 300, 32, "normal"), (129, 40, 12, "ties"),
    (8192, 256, 8, "normal"), (3, 2048, 20, "ties"),
]


# rank-limited routing (T, E, k, kind, P, M): ties within and across ranks, the
# P <= 64 edge, one rank (M = 1), exactly k experts in the allowed ranks, and
# the 32-lane path (k > 16)
LIMIT_CASES = [
    (1000, 256, 8, "normal", 8, 4), (500, 32, 4, "ties", 8, 2), (333, 64, 6, "zeros", 16, 2),
    (70, 12, 3, "ties", 4, 1), (257, 256, 8, "normal", 64, 3), (100, 64, 20, "ties", 4, 2),
    (64, 16, 8, "equal", 4, 2), (129, 40, 12, "normal", 10, 3), (8192, 256, 8, "ties", 8, 4),
]


def _route_logits(T, E, k, kind):
    rng = np.random.default_rng(T * 31 + E * 7 + k)
    if kind == "ties":
        l = rng.integers(-3, 4, (T, E)).astype(np.float32)
    elif kind == "zeros":
        l = rng.choice(np.array([0.0, -0.0, 1.0, -1.0], np.float32), (T, E))
    elif kind == "equal":
        l = np.full((T, E), 0.5, np.float32)
    else:
        l = (rng.standard_normal((T, E)) * 2).astype(np.float32)
    return l


@pytest.mark.parametrize("T,E,k,kind,P,M", [c + (1, 0) for c in ROUTE_CASES] + LIMIT_CASES)
def test_route_given_logits_is_exact(T, E, k, kind, P, M):
    say(f"route T={T} E={E} k={k} {kind} P={P} max_ranks={M}")
    l = _route_logits(T, E, k, kind)
    idx_ref = oracle.rank_limited_experts(l, k, P, M)
    w_ref = oracle.gate_weights(l, idx_ref)
    idx, w = _i32(T, k), _f32(T, k)
    moe.moe_route(torch.from_numpy(l).cuda(), T, E, k, P, M, idx, w)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    # both sides evaluate the softmax in fp64 and round once: at most 1 ulp apart
    assert np.all(np.abs(w.cpu().numpy() - w_ref) <= np.spacing(np.abs(w_ref)))


ROUTER_CASES = [
    (300, 256, 8, 2, "bf16", None), (200, 1024, 64, 6, "bf16", "zipf1.2"), (130, 520, 256, 8, "bf16", None),
    (100, 128, 8, 2, "f32", None), (65, 72, 20, 3, "bf16", None), (1, 4096, 8, 2, "bf16", None),
    (64, 7168, 256, 8, "bf16", None), (40, 2048, 64, 20, "bf16", "zipf1.2"),
    # score waves of 2 and 4 token tiles of 16, each with a ragged last tile
    (4100, 4096, 8, 2, "bf16", None), (8200, 2048, 64, 6, "bf16", "zipf1.2"),
    # 128 or more experts and 256 or more tokens: scores on the grouped GEMM kernel (fp32 slices over d)
    (1000, 1024, 128, 6, "bf16", "zipf1.2"), (600, 7168, 256, 8, "bf16", None), (2304, 2048, 128, 4, "bf16", None),
]
# rank-limited: (T, d, E, k, dtype, bias, P, M, logits wanted); without logits_out
# and with several d-slices or a bias the summed scores go back over slice 0
ROUTER_LIMIT_CASES = [
    (300, 1024, 256, 8, "bf16", None, 8, 4, False), (200, 1024, 64, 6, "bf16", "zipf1.2", 8, 2, False),
    (100, 128, 8, 2, "f32", None, 4, 1, True), (64, 7168, 256, 8, "bf16", None, 8, 4, True),
    (40, 2048, 64, 20, "bf16", "zipf1.2", 4, 2, True), (1030, 512, 32, 4, "bf16", None, 8, 1, False),
]


@pytest.mark.parametrize("T,d,E,k,dtype,bias,P,M,want_logits",
                         [c + (1, 0, True) for c in ROUTER_CASES] + ROUTER_LIMIT_CASES)
def test_router_scores_choice_and_gates(T, d, E, k, dtype, bias, P, M, want_logits):
    say(f"router T={T} d={d} E={E} k={k} {dtype} bias={bias} P={P} max_ranks={M}")
    std = (1 / np.sqrt(d)) if dtype == "f32" else 1.0
    wl = moe_inputs.custom(T=T, d=d, E=E, k=k, d_ff=8, cf=1.0, dtype=dtype, seed=T + d + E,
                           x_std=std, wr_std=(1 / np.sqrt(d)) if dtype == "f32" else 0.02, bias=bias,
                           P=P, max_ranks=M)
    x64, wr64 = oracle.decode(wl.x, dtype), oracle.decode(wl.wr, dtype)
    l_ref = oracle.router_logits(x64, wr64, wl.bias_vec)
    idx_ref = oracle.rank_limited_experts(l_ref, k, P, M)
    w_ref = oracle.gate_weights(l_ref, idx_ref)
    logits, idx, w = _f32(T, E), _i32(T, k), _f32(T, k)
    b = None if wl.bias_vec is None else torch.from_numpy(wl.bias_vec).cuda()
    ws_n = moe.moe_router_workspace_size(T, d, E, dtype)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    moe.moe_router(to_dev(wl.x, dtype), to_dev(wl.wr, dtype), b, T, d, E, k, P, M, dtype, idx, w,
                   logits if want_logits else None, ws, ws_n)
    torch.cuda.synchronize()
    tol = logits_tolerance(x64, wr64, wl.bias_vec)
    if want_logits:
        err = np.abs(logits.cpu().numpy().astype(np.float64) - l_ref)
        assert np.all(err <= tol), f"max err/tol {np.max(err / tol)}"
    if M:
        ranks = idx.cpu().numpy() // (E // P)
        assert max(len(set(r)) for r in ranks.tolist()) <= M
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    # softmax sensitivity: |dw_j| <= 2 w_j max|dl|, plus one rounding
    wtol = w_ref.astype(np.float64) * (2 * tol.max(axis=1, keepdims=True) + 2 * U)
    assert np.all(np.abs(w.cpu().numpy().astype(np.float64) - w_ref) <= wtol)


# -------------------------------------------------------------- permutation ---

def _random_routes(rng, T, E, k, skew):
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        p /= p.sum()
        return np.array([rng.choice(E, k, replace=False, p=p) for _ in range(T)], np.int32).reshape(T, k)
    return np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32).reshape(T, k)


PERMUTE_CASES = [
    (1000, 8, 2, 1.25, 1, 64, "bf16", False), (777, 64, 6, 1.0, 4, 40, "bf16", True),
    (300, 256, 8, 1.25, 8, 16, "bf16", False), (65, 4, 2, 0.3, 2, 8, "f32", True),
    (64, 8, 2, 1.25, 1, 128, "f32", False), (1, 3, 2, 1.0, 1, 8, "bf16", False),
    (129, 1, 1, 2.0, 1, 8, "bf16", False), (5000, 32, 4, 0.5, 8, 24, "bf16", True),
    (40, 8, 2, 1.0, 2, 20480, "bf16", False),   # 2560 words a row: two passes of 8 words per lane
    (30, 4, 2, 1.0, 1, 8200, "f32", True),      # 2050 words a row: a second pass of 2 words
    (100, 64, 32, 0.5, 4, 64, "bf16", True),    # k = 32: every metadata lane of a wave, many drops
    (70000, 8, 2, 1.25, 2, 8, "bf16", False),    # 1094 tiles: 69 per scan lane, past the 16 held in registers
    (3000, 4096, 4, 1.0, 8, 8, "bf16", True),    # the most experts: the scan takes them 1024 at a time
    (2000, 1000, 5, 1.5, 4, 8, "bf16", False),   # 1000 experts: a 1024-wide pass with idle lanes
    (4160, 24, 4, 1.0, 2, 8, "bf16", True),      # E not a power of two: the block sums every column
    (16385, 12, 1, 0.6, 1, 8, "bf16", True),     # k = 1, 257 tiles, many drops
    (4160, 4096, 4, 1.0, 8, 8, "bf16", True),    # 65 x 4096 counts: each token sums its copies' 4 x 64
    (4161, 4096, 4, 1.0, 8, 8, "bf16", True),    # one token past both limits: scan, slots and scatter apart
    (1000, 8, 2, 1.25, 2, 2048, "bf16", True),   # one-pass rows of 256 words: a wave per token
    (300, 8, 2, 1.0, 1, 1000, "f32", False),     # 250 words: a wave per token, a ragged last word group
    (500, 16, 3, 1.0, 2, 3000, "bf16", True),    # 375 words: two waves per token
    (200, 32, 4, 1.0, 4, 7168, "bf16", True),    # 896 words: four waves per token
    # one pass, each block summing every expert's column (E not a power of two; above 1024)
    (600, 48, 4, 1.0, 4, 3000, "bf16", True),
    (800, 1536, 4, 1.0, 8, 7168, "bf16", True),
    # at the block sum's limit of 64 counts a thread, and past it (then each token sums its copies')
    (4160, 1024, 2, 1.0, 8, 8, "bf16", True),
    (4161, 1024, 2, 1.0, 8, 8, "bf16", True),
    (4160, 8, 2, 1.0, 1, 4096, "bf16", True),
    (20000, 48, 2, 1.0, 4, 8, "bf16", True),     # 313 tiles (20 a scan lane)
    # scan, slots and scatter apart: 78 tiles of 2048 experts ahead, 4 copies a token
    (5000, 2048, 4, 1.0, 8, 8, "bf16", True),
]


def _random_permute_cases(n, seed=4242):
    """Seeded shapes across the permutation's three launch plans (a block-wide
    histogram sum, a per-token one, scan and slots apart), sized so the host
    reference stays small."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        E = int(rng.choice([1, 2, 3, 5, 8, 12, 16, 24, 32, 48, 64, 100, 128, 256, 512, 1024, 1536]))
        k = int(rng.integers(1, min(E, 32) + 1))
        T = int(rng.integers(1, 12001))
        cf = float(rng.choice([0.3, 0.6, 1.0, 1.25, 2.0]))
        dtype = str(rng.choice(["bf16", "f32"]))
        d = int(rng.choice([8, 24, 64, 200, 1000, 2048, 3000]))
        P = int(rng.choice([p for p in (1, 2, 4, 8) if E % p == 0]))
        C = -(-int(cf * k * T) // E) if E else 1
        if T * k * d > 2e7 or E * max(C, 1) * d > 4e7:
            continue
        out.append((T, E, k, cf, P, d, dtype, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("T,E,k,cf,P,d,dtype,skew", PERMUTE_CASES + _random_permute_cases(24))
def test_permute_is_exact(T, E, k, cf, P, d, dtype, skew):
    say(f"permute T={T} E={E} k={k} cf={cf} P={P} d={d} {dtype} skew={skew}")
    rng = np.random.default_rng(T + E + k)
    idx = _random_routes(rng, T, E, k, skew)
    x = moe_inputs.custom(T=T, d=d, E=E, k=k, d_ff=8, cf=cf, dtype=dtype, seed=5, reject=False).x
    C = oracle.capacity(T, E, k, cf)
    assert moe.moe_capacity(T, E, k, cf) == C
    slot_r, src_r, routed_r, kept_r = oracle.assign_slots(idx, E, C)
    st = oracle.routing_stats(slot_r, routed_r, kept_r, C, P, d, 2 if dtype == "bf16" else 4)
    b_ref = oracle.dispatch_buckets(x, idx, slot_r, E, C)

    eb = 2 if dtype == "bf16" else 4
    sentinel = 0x7F7F if dtype == "bf16" else np.float32(-12345.5)
    buckets = to_dev(np.full((E, C, d), sentinel, dtype=np.uint16 if dtype == "bf16" else np.float32), dtype)
    g = Guarded()
    slot, src = g.empty((T, k), torch.int32, "slot"), g.empty((E, C), torch.int32, "src")
    routed, kept, send = g.empty((E,), torch.int32, "routed"), g.empty((E,), torch.int32, "kept"), \
        g.empty((P,), torch.int32, "send")
    totals = g.empty((4,), torch.int64, "totals")
    ws_n = moe.moe_permute_workspace_size(T, E)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    moe.moe_permute(to_dev(x, dtype), torch.from_numpy(idx).cuda(), T, d, E, k, C, P, dtype, buckets, slot,
                    src, routed, kept, send, totals, ws, ws_n)
    torch.cuda.synchronize()
    g.check()
    assert np.array_equal(slot.cpu().numpy(), slot_r)
    assert np.array_equal(src.cpu().numpy().reshape(-1), src_r)
    assert np.array_equal(routed.cpu().numpy(), routed_r)
    assert np.array_equal(kept.cpu().numpy(), kept_r)
    assert np.array_equal(send.cpu().numpy(), st["send_count"])
    assert totals.cpu().numpy().tolist() == [st["dropped"], st["fully_dropped_tokens"], st["padded_rows"],
                                             st["offrank_bytes"]]
    got = to_host(buckets, dtype)
    for e in range(E):
        n = kept_r[e]
        assert np.array_equal(got[e, :n].view(np.uint8), b_ref[e, :n].view(np.uint8)), f"expert {e}"
        assert np.all(got[e, n:].view(np.uint8) == np.full((C - n, d), sentinel, got.dtype).view(np.uint8)), \
            f"padding of expert {e} was written"
    assert eb in (2, 4)


# ------------------------------------------------------------- grouped GEMM ---

GEMM_CASES = [
    (4, 200, 256, 320, "bf16"), (8, 64, 128, 256, "f32"), (3, 300, 520, 136, "bf16"),
    (16, 5, 128, 128, "bf16"), (2, 128, 64, 64, "bf16"), (1, 1, 8, 8, "bf16"), (5, 40, 36, 20, "f32"),
    (3, 600, 256, 384, "bf16"), (2, 1100, 520, 264, "bf16"), (4, 512, 64, 1032, "bf16"),
    (3, 700, 384, 640, "bf16"), (2, 513, 128, 128, "bf16"), (5, 900, 1024, 256, "bf16"),
    (40, 12, 256, 96, "bf16"), (8, 16, 4096, 1024, "bf16"), (3, 3, 40, 24, "bf16"),
    # 256 x 256 tiles with a last round split over K on a 256-CU part: whole
    # tiles plus split ones in GEMM 1 (GEMM 2 all split), and the reverse
    (4, 768, 256, 4352, "bf16"), (8, 768, 4096, 256, "bf16"),
    # 256 < C <= 320: one 320-row tile per expert (row blocks of 32 past kept
    # skipped per wave) in GEMM 1, and in GEMM 2 where d_ff % 128 == 0; 2-, 8-
    # and 3-way splits of the last round, one stage pair (no split), N < 256
    (6, 300, 256, 320, "bf16"), (4, 320, 1024, 256, "bf16"), (3, 257, 384, 192, "bf16"),
    (5, 290, 128, 384, "bf16"),
    # more than 8 whole tiles, not a multiple of 8, no split (one stage pair):
    # every XCD slot of the tile spread must still run
    (3, 600, 128, 640, "bf16"),
    # SwiGLU over 64 or more column tiles (d_ff >= 8192) on 320-row tiles: the
    # instantiation that requests each stage at the start of the one before
    (2, 300, 256, 8192, "bf16"),
]


@pytest.mark.parametrize("E,C,d,d_ff,dtype", GEMM_CASES)
def test_grouped_gemm_rows_below_kept(E, C, d, d_ff, dtype):
    say(f"gemm E={E} C={C} d={d} d_ff={d_ff} {dtype}")
    rng = np.random.default_rng(E * C + d)
    kept = rng.integers(0, C + 1, E).astype(np.int32)
    kept[0] = C
    if E > 2:
        kept[1] = 0
    wl = moe_inputs.custom(T=E * C, d=d, E=E, k=1, d_ff=d_ff, cf=1.0, dtype=dtype, seed=E + d, reject=False,
                           x_std=1.0)
    X = wl.x.reshape(E, C, d).copy()
    nan = 0x7FC0 if dtype == "bf16" else np.float32(np.nan)
    for e in range(E):
        X[e, kept[e]:] = nan                       # padding rows must not reach any result
    wg, wu, wd = wl.all_expert_weights()
    h_ref = np.zeros((E, C, d_ff))
    y_ref = np.zeros((E, C, d))
    for e in range(E):
        n = kept[e]
        if n:
            Xe = bits_to_f64(X[e, :n], dtype)
            h_ref[e, :n] = oracle.expert_hidden(Xe, oracle.decode(wg[e], dtype), oracle.decode(wu[e], dtype))
            y_ref[e, :n] = oracle.expert_mlp(Xe, oracle.decode(wg[e], dtype), oracle.decode(wu[e], dtype),
                                             oracle.decode(wd[e], dtype))
    sent = 0x1234 if dtype == "bf16" else np.float32(777.0)
    npdt = np.uint16 if dtype == "bf16" else np.float32
    h = to_dev(np.full((E, C, d_ff), sent, npdt), dtype)
    y = to_dev(np.full((E, C, d), sent, npdt), dtype)
    ws_n = moe.moe_grouped_gemm_workspace_size(E, C)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    moe.moe_grouped_gemm(to_dev(X, dtype), torch.from_numpy(kept).cuda(), to_dev(wg, dtype), to_dev(wu, dtype),
                         to_dev(wd, dtype), E, C, d, d_ff, dtype, h, y, ws, ws_n)
    torch.cuda.synchronize()
    hg, yg = to_host(h, dtype), to_host(y, dtype)
    # bf16: h, y rounded to bf16 (2^-9 relative) and y consumes the rounded h;
    # fp32: fp32 accumulation only.
    tol_h, tol_y = (4e-3, 1e-2) if dtype == "bf16" else (1e-5, 1e-5)
    for e in range(E):
        n = kept[e]
        if n:
            assert row_rel_err(bits_to_f64(hg[e, :n], dtype), h_ref[e, :n]).max() <= tol_h, f"h expert {e}"
            assert row_rel_err(bits_to_f64(yg[e, :n], dtype), y_ref[e, :n]).max() <= tol_y, f"y expert {e}"
        assert np.all(hg[e, n:] == np.full((C - n, d_ff), sent, npdt)), f"h padding of expert {e} written"
        assert np.all(yg[e, n:] == np.full((C - n, d), sent, npdt)), f"y padding of expert {e} written"


# ------------------------------------------------------------------ combine ---

COMBINE_CASES = [(500, 64, 8, 2, 1.0, "bf16"), (300, 40, 16, 4, 0.5, "bf16"), (64, 128, 8, 2, 1.25, "f32"),
                 (200, 8, 4, 4, 0.25, "bf16"), (1, 16, 2, 1, 1.0, "f32"),
                 (1100, 6208, 8, 3, 0.5, "bf16"),   # one pass of 4 words per lane, the last ragged
                 (40, 20480, 8, 2, 1.0, "bf16"),    # 2560 words a row: two passes of 8 words per lane
                 (30, 8200, 4, 2, 1.0, "f32"),      # 2050 words a row: a second pass of 2 words
                 (100, 64, 64, 32, 0.5, "bf16"),    # k = 32: every metadata lane of a wave, many drops
                 (50, 24, 32, 32, 1.0, "f32")]      # k = E = 32


@pytest.mark.parametrize("T,d,E,k,cf,dtype", COMBINE_CASES)
def test_combine_inverse_and_passthrough(T, d, E, k, cf, dtype):
    say(f"combine T={T} d={d} E={E} k={k} cf={cf} {dtype}")
    rng = np.random.default_rng(T + d)
    idx = _random_routes(rng, T, E, k, skew=True)
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(1, keepdims=True)
    C = oracle.capacity(T, E, k, cf)
    slot, _, _, _ = oracle.assign_slots(idx, E, C)
    wl = moe_inputs.custom(T=T, d=d, E=E, k=k, d_ff=8, cf=cf, dtype=dtype, seed=T, reject=False)
    x = wl.x.copy()
    x[:, 0] = 0x8000 if dtype == "bf16" else np.float32(-0.0)     # -0.0 must pass through untouched
    ybits = moe_inputs.custom(T=E * C, d=d, E=E, k=k, d_ff=8, cf=cf, dtype=dtype, seed=T + 1,
                              reject=False).x.reshape(E, C, d)
    y64 = bits_to_f64(ybits, dtype)
    x64 = bits_to_f64(x, dtype)
    ycop = np.zeros((T, k, d))
    for t in range(T):
        for j in range(k):
            if slot[t, j] >= 0:
                ycop[t, j] = y64[idx[t, j], slot[t, j]]
    ref = oracle.combine(x64, ycop, w, slot)
    out = to_dev(np.zeros_like(x), dtype)
    moe.moe_combine(to_dev(x, dtype), to_dev(ybits, dtype), torch.from_numpy(idx).cuda(),
                    torch.from_numpy(w).cuda(), torch.from_numpy(slot).cuda(), T, d, E, k, C, dtype, out)
    torch.cuda.synchronize()
    got = to_host(out, dtype)
    dropped = np.all(slot < 0, axis=1)
    assert np.array_equal(got[dropped].view(np.uint8), x[dropped].view(np.uint8))
    mag = np.abs(x64) + np.einsum("tj,tjd->td", np.where(slot >= 0, w, 0.0), np.abs(ycop))
    # fp32 sum of k + 1 terms (k + 1 roundings), then one rounding to the output type
    out_ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -24
    tol = out_ulp * np.abs(ref) + (k + 2) * U * mag + 1e-30
    keep = ~dropped
    assert np.all(np.abs(bits_to_f64(got[keep], dtype) - ref[keep]) <= tol[keep])


def test_zero_tokens_is_a_no_op():
    moe.moe_route(torch.zeros(1, device="cuda"), 0, 8, 2, 1, 0, _i32(1), _f32(1))
    out = torch.full((4,), 3.0, device="cuda")
    moe.moe_combine(out, out, _i32(1), _f32(1), _i32(1), 0, 4, 8, 2, 1, "f32", out)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


# ------------------------------------------------- indices given by a caller ---

def test_grouped_gemm_clamps_counts_to_the_capacity():
    """kept counts above C process the C rows of the bucket, negative ones none;
    nothing is written past h or y."""
    E, C, d, F = 4, 300, 256, 384
    kept = np.array([C + 77, -5, 130, 1 << 30], np.int32)
    eff = np.clip(kept, 0, C)
    wl = moe_inputs.custom(T=E * C, d=d, E=E, k=1, d_ff=F, cf=1.0, seed=61, reject=False)
    X = wl.x.reshape(E, C, d)
    wg, wu, wd = wl.all_expert_weights()
    g = Guarded()
    h = g.empty((E, C, F), torch.bfloat16, "h")
    y = g.empty((E, C, d), torch.bfloat16, "y")
    h.view(torch.int16).fill_(0x1234)
    y.view(torch.int16).fill_(0x1234)
    ws_n = moe.moe_grouped_gemm_workspace_size(E, C)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    moe.moe_grouped_gemm(to_dev(X, "bf16"), torch.from_numpy(kept).cuda(), to_dev(wg, "bf16"), to_dev(wu, "bf16"),
                         to_dev(wd, "bf16"), E, C, d, F, "bf16", h, y, ws, ws_n)
    torch.cuda.synchronize()
    g.check()
    hg, yg = to_host(h, "bf16"), to_host(y, "bf16")
    for e in range(E):
        n = int(eff[e])
        if n:
            Xe = bits_to_f64(X[e, :n], "bf16")
            wge, wue, wde = (oracle.decode(a[e], "bf16") for a in (wg, wu, wd))
            assert row_rel_err(bits_to_f64(hg[e, :n], "bf16"), oracle.expert_hidden(Xe, wge, wue)).max() <= 4e-3
            assert row_rel_err(bits_to_f64(yg[e, :n], "bf16"), oracle.expert_mlp(Xe, wge, wue, wde)).max() <= 1e-2
        assert np.all(hg[e, n:] == 0x1234) and np.all(yg[e, n:] == 0x1234), f"rows past {n} of expert {e}"


def test_combine_treats_out_of_range_copies_as_dropped():
    T, d, E, k, C = 300, 64, 8, 3, 60
    rng = np.random.default_rng(71)
    idx = _random_routes(rng, T, E, k, skew=False)
    w = rng.random((T, k)).astype(np.float32)
    slot, _, _, _ = oracle.assign_slots(idx, E, C)
    bad_idx, bad_slot = idx.copy(), slot.copy()
    bad_idx[5, 0], bad_idx[6, 1], bad_slot[7, 2], bad_slot[8, 0] = E, -3, C, C + 1000
    bad_idx[9, :], bad_slot[10, :] = E + 1, C            # whole tokens: passed through
    eff = np.where((bad_idx >= 0) & (bad_idx < E) & (bad_slot < C), bad_slot, -1)
    wl = moe_inputs.custom(T=T, d=d, E=E, k=k, d_ff=8, cf=1.0, seed=72, reject=False)
    ybits = moe_inputs.custom(T=E * C, d=d, E=E, k=k, d_ff=8, cf=1.0, seed=73, reject=False).x.reshape(E, C, d)
    y64, x64 = bits_to_f64(ybits, "bf16"), bits_to_f64(wl.x, "bf16")
    ycop = np.zeros((T, k, d))
    for t, j in zip(*np.nonzero(eff >= 0)):
        ycop[t, j] = y64[idx[t, j], eff[t, j]]
    ref = oracle.combine(x64, ycop, w, eff)
    g = Guarded()
    out = g.empty((T, d), torch.bfloat16, "out")
    moe.moe_combine(to_dev(wl.x, "bf16"), to_dev(ybits, "bf16"), torch.from_numpy(bad_idx).cuda(),
                    torch.from_numpy(w).cuda(), torch.from_numpy(bad_slot).cuda(), T, d, E, k, C, "bf16", out)
    torch.cuda.synchronize()
    g.check()
    got = to_host(out, "bf16")
    dropped = np.all(eff < 0, axis=1)
    assert dropped[9] and dropped[10]
    assert np.array_equal(got[dropped].view(np.uint8), wl.x[dropped].view(np.uint8))
    mag = np.abs(x64) + np.einsum("tj,tjd->td", np.where(eff >= 0, w, 0.0), np.abs(ycop))
    tol = 2.0 ** -8 * np.abs(ref) + (k + 2) * U * mag + 1e-30
    assert np.all(np.abs(bits_to_f64(got, "bf16") - ref)[~dropped] <= tol[~dropped])


def test_permute_drops_out_of_range_experts():
    """An expert index outside [0, E) is dropped (slot -1) and counted in no
    expert: the result equals the permutation of the remaining copies, which
    the oracle gives when those copies go to one extra expert that keeps
    none of them."""
    T, E, k, P, d = 500, 16, 4, 4, 64
    rng = np.random.default_rng(81)
    idx = _random_routes(rng, T, E, k, skew=True)
    C = oracle.capacity(T, E, k, 1.0)
    bad = idx.copy()
    bad[3, 1], bad[100, 0], bad[101, 3] = E, -1, 1 << 20
    bad[200, :] = E + 2                                      # a whole token
    inval = (bad < 0) | (bad >= E)
    as_extra = np.where(inval, E, bad).astype(np.int32)     # the remaining copies keep their order
    slot_e, src_e, routed_e, kept_e = oracle.assign_slots(as_extra, E + 1, C)
    slot_r = np.where(inval, -1, slot_e)
    routed_r, kept_r = routed_e[:E], kept_e[:E]
    src_r = src_e[:E * C]
    st = oracle.routing_stats(slot_r, routed_r, kept_r, C, P, d, 2)
    x = moe_inputs.custom(T=T, d=d, E=E, k=k, d_ff=8, cf=1.0, seed=82, reject=False).x
    b_ref = oracle.dispatch_buckets(x, np.where(inval, 0, bad), slot_r, E, C)
    g = Guarded()
    buckets = g.empty((E, C, d), torch.bfloat16, "buckets")
    slot, src = g.empty((T, k), torch.int32, "slot"), g.empty((E, C), torch.int32, "src")
    routed, kept = g.empty((E,), torch.int32, "routed"), g.empty((E,), torch.int32, "kept")
    send, totals = g.empty((P,), torch.int32, "send"), g.empty((4,), torch.int64, "totals")
    ws_n = moe.moe_permute_workspace_size(T, E)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    moe.moe_permute(to_dev(x, "bf16"), torch.from_numpy(bad).cuda(), T, d, E, k, C, P, "bf16", buckets, slot, src,
                    routed, kept, send, totals, ws, ws_n)
    torch.cuda.synchronize()
    g.check()
    assert np.array_equal(slot.cpu().numpy(), slot_r)
    assert np.array_equal(src.cpu().numpy().reshape(-1), src_r)
    assert np.array_equal(routed.cpu().numpy(), routed_r)
    assert np.array_equal(kept.cpu().numpy(), kept_r)
    assert np.array_equal(send.cpu().numpy(), st["send_count"])
    assert totals.cpu().numpy().tolist() == [st["dropped"], st["fully_dropped_tokens"], st["padded_rows"],
                                             st["offrank_bytes"]]
    got = to_host(buckets, "bf16")
    for e in range(E):
        assert np.array_equal(got[e, :kept_r[e]], b_ref[e, :kept_r[e]]), f"expert {e}"


def test_router_scores_past_2gib_of_tokens():
    """x of more than 2^31 bytes (DeepSeek-V3 width and expert count): the
    scores are right for rows on both sides of that byte offset. x repeats a
    seeded 4096-token batch, so every row's reference is its base row's."""
    Tb, d, E, k = 4096, 7168, 256, 8
    reps = 40                                   # 163840 tokens, 2.35e9 bytes of x
    T = Tb * reps
    assert T * d * 2 >= 1 << 31
    wl = moe_inputs.custom(T=Tb, d=d, E=E, k=k, d_ff=8, cf=1.0, seed=91)
    x64, wr64 = oracle.decode(wl.x, "bf16"), oracle.decode(wl.wr, "bf16")
    l_ref = oracle.router_logits(x64, wr64, None)
    idx_ref = oracle.topk_experts(l_ref, k)
    x = to_dev(wl.x, "bf16").repeat(reps, 1)
    logits, idx, w = _f32(T, E), _i32(T, k), _f32(T, k)
    ws_n = moe.moe_router_workspace_size(T, d, E, "bf16")
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    moe.moe_router(x, to_dev(wl.wr, "bf16"), None, T, d, E, k, 1, 0, "bf16", idx, w, logits, ws, ws_n)
    torch.cuda.synchronize()
    del x
    assert np.array_equal(idx.cpu().numpy(), np.tile(idx_ref, (reps, 1)))
    tol = logits_tolerance(x64, wr64, None)
    first_past = -(-(1 << 31) // (d * 2))       # first row that starts past 2^31 bytes
    for t0 in (0, first_past - 2, T - Tb):
        rows = np.arange(t0, t0 + Tb) % T
        err = np.abs(logits[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64) - l_ref[rows % Tb])
        assert np.all(err <= tol[rows % Tb]), (t0, float(np.max(err / tol[rows % Tb])))
