"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each check uses brute force with
a different algorithm (tests/bruteforce.py), a closed form, an invariant, or a
number the pages print (tests/golden/, each file names its source).
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import moe_inputs
import oracle
from tests import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- formats ---

def test_bf16_rounding_ties_and_signs():
    one = 1.0
    ulp = 2.0 ** -7
    cases = [                           # a list: 0.0 and -0.0 are equal dict keys
        (one, 0x3F80),
        (one + ulp / 2, 0x3F80),          # tie -> even (mantissa 0)
        (one + 3 * ulp / 2, 0x3F82),      # tie -> even (mantissa 2)
        (one + ulp / 2 + 2.0 ** -30, 0x3F81),  # just above the tie: rounds up
        (-2.0, 0xC000),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (3.140625, 0x4049),
    ]
    for v, bits in cases:
        assert int(oracle.f64_to_bf16_bits(np.array([v]))[0]) == bits, v
    # a value whose fp32 rounding would land on a bf16 tie: must round from fp64 once
    v = 1.0 + ulp / 2 + 2.0 ** -40     # fp32 rounds this to exactly the tie
    assert int(oracle.f64_to_bf16_bits(np.array([v]))[0]) == 0x3F81


def test_bf16_decode_matches_generator_encoding():
    rng = np.random.default_rng(5)
    z = rng.standard_normal(10000).astype(np.float32) * np.float32(3)
    bits = moe_inputs.to_bf16_bits(z)
    back = oracle.bf16_bits_to_f64(bits)
    # each decoded value is the bf16 value nearest to z (within half a bf16 ulp)
    ulp = np.ldexp(1.0, np.frexp(np.abs(z).astype(np.float64))[1] - 8)
    assert np.all(np.abs(back - z) <= ulp / 2)
    assert np.array_equal(oracle.f64_to_bf16_bits(back), bits)


# --------------------------------------------------------------- capacity ---

@pytest.mark.parametrize("cf", [0.25, 0.5, 1.0, 1.25, 1.5, 2.0, 3.0])
def test_capacity_is_smallest_sufficient_integer(cf):
    for T, E, k in itertools.product([0, 1, 7, 64, 100, 4096], [1, 3, 8, 64, 256], [1, 2, 6, 8]):
        if k > E:
            continue
        C = oracle.capacity(T, E, k, cf)
        assert C == bf.capacity(T, E, k, float(np.float32(cf)))
        assert Fraction(C * E) >= Fraction(cf) * k * T > Fraction((C - 1) * E) or T == 0


def test_capacity_of_named_workloads_is_exact():
    # every named workload's cf*k*T/E is an integer, so ceil never rounds
    for name, cfg in moe_inputs.WORKLOADS.items():
        exact = Fraction(cfg["cf"]) * cfg["k"] * cfg["T"] / cfg["E"]
        assert exact.denominator == 1
        assert oracle.capacity(cfg["T"], cfg["E"], cfg["k"], cfg["cf"]) == exact


def test_capacity_rejects_bad_arguments():
    for args in [(-1, 8, 2, 1.0), (8, 0, 2, 1.0), (8, 8, 0, 1.0), (8, 8, 2, 0.0), (8, 8, 2, float("nan")),
                 (8, 8, 2, float("inf"))]:
        with pytest.raises(ValueError):
            oracle.capacity(*args)


# ------------------------------------------------------------------ top-k ---

def test_topk_matches_repeated_argmax_on_tied_integer_scores():
    rng = np.random.default_rng(1)
    for _ in range(300):
        E = int(rng.integers(1, 9))
        k = int(rng.integers(1, E + 1))
        T = int(rng.integers(1, 6))
        l = rng.integers(-2, 3, size=(T, E)).astype(np.float32)   # many ties
        idx = oracle.topk_experts(l, k)
        for t in range(T):
            assert list(idx[t]) == bf.topk([float(v) for v in l[t]], k)


def test_topk_special_cases():
    l = np.zeros((3, 6), np.float32)
    assert np.array_equal(oracle.topk_experts(l, 4), np.tile(np.arange(4), (3, 1)))
    l = np.array([[0.5, -1.0, 2.0, 0.25]], np.float32)
    assert list(oracle.topk_experts(l, 4)[0]) == [2, 0, 3, 1]          # k = E: full order
    l = np.array([[-0.0, 0.0, -0.0, -1.0]], np.float32)               # signed zeros tie
    assert list(oracle.topk_experts(l, 3)[0]) == [0, 1, 2]
    l = np.array([[1.0, 3.0, 3.0, 2.0]], np.float32)
    assert list(oracle.topk_experts(l, 2)[0]) == [1, 2]                 # lowest index first


def test_topk_is_max_sum_subset():
    rng = np.random.default_rng(2)
    for _ in range(100):
        E, k = 6, int(rng.integers(1, 5))
        l = rng.integers(-3, 4, size=(1, E)).astype(np.float32)
        idx = oracle.topk_experts(l, k)[0]
        best = max(sum(l[0, list(c)]) for c in itertools.combinations(range(E), k))
        assert sum(l[0, idx]) == best


# ------------------------------------------------------ rank-limited top-k ---

def _rank_cases(seed, n, maxE=8):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        P = int(rng.choice([2, 3, 4]))
        per = int(rng.integers(1, maxE // P + 1))
        E = P * per
        M = int(rng.integers(1, P))
        k = int(rng.integers(1, min(E, M * per) + 1))
        T = int(rng.integers(1, 5))
        l = rng.integers(-2, 3, size=(T, E)).astype(np.float32)   # many ties
        yield l, k, P, M


def test_rank_limited_matches_greedy_walk_and_exhaustive_search():
    for l, k, P, M in _rank_cases(11, 400):
        idx = oracle.rank_limited_experts(l, k, P, M)
        for t in range(l.shape[0]):
            row = [float(v) for v in l[t]]
            assert list(idx[t]) == bf.rank_limited_greedy(row, k, P, M)
            assert list(idx[t]) == bf.rank_limited_exhaustive(row, k, P, M)


def test_rank_limited_touches_at_most_M_ranks():
    rng = np.random.default_rng(12)
    T, E, P, k = 500, 256, 8, 8
    l = rng.standard_normal((T, E)).astype(np.float32)
    for M in (1, 2, 4):
        idx = oracle.rank_limited_experts(l, k, P, M)
        ranks = idx // (E // P)
        assert max(len(set(r)) for r in ranks.tolist()) <= M
        assert all(len(set(r)) == k for r in idx.tolist())      # k distinct experts
        # with M = 1 every pick lies in the rank of the token's best expert
        if M == 1:
            assert np.array_equal(ranks[:, 0], np.argmax(l, axis=1) // (E // P))
            assert np.all(ranks == ranks[:, :1])
    # unconstrained top-k that already spans <= M ranks is left as it is
    plain = oracle.topk_experts(l, k)
    lim = oracle.rank_limited_experts(l, k, P, 4)
    fits = np.array([len(set(r)) <= 4 for r in (plain // (E // P)).tolist()])
    assert fits.any() and np.array_equal(lim[fits], plain[fits])


def test_rank_limited_special_cases_reduce_to_plain_topk():
    rng = np.random.default_rng(13)
    l = rng.integers(-3, 4, size=(50, 12)).astype(np.float32)
    plain = oracle.topk_experts(l, 3)
    assert np.array_equal(oracle.rank_limited_experts(l, 3, 4, 0), plain)     # M = 0: no limit
    assert np.array_equal(oracle.rank_limited_experts(l, 3, 4, 4), plain)     # M = P
    assert np.array_equal(oracle.rank_limited_experts(l, 3, 1, 1), plain)     # one rank
    assert np.array_equal(oracle.rank_limited_experts(l, 3, 12, 3), plain)    # one expert per rank, M = k
    with pytest.raises(ValueError):
        oracle.rank_limited_experts(l, 5, 4, 1)                                # 1 rank holds 3 < 5


# ------------------------------------------------------------------ gates ---

def test_gates_closed_forms():
    rng = np.random.default_rng(3)
    l = (rng.standard_normal((200, 8)) * 2).astype(np.float32)
    idx1 = oracle.topk_experts(l, 1)
    assert np.all(oracle.gate_weights(l, idx1) == np.float32(1.0))     # k = 1
    idx2 = oracle.topk_experts(l, 2)
    w2 = oracle.gate_weights(l, idx2).astype(np.float64)
    l0 = np.take_along_axis(l, idx2[:, :1], 1)[:, 0].astype(np.float64)
    l1 = np.take_along_axis(l, idx2[:, 1:2], 1)[:, 0].astype(np.float64)
    sig = 1.0 / (1.0 + np.exp(l1 - l0))                                # k = 2: logistic of the gap
    assert np.allclose(w2[:, 0], sig, rtol=2 ** -23, atol=0)
    assert np.allclose(w2[:, 1], 1.0 - sig, rtol=2 ** -22, atol=0)
    for k in (3, 5, 8):
        w = oracle.gate_weights(l, oracle.topk_experts(l, k)).astype(np.float64)
        assert np.all(np.abs(w.sum(1) - 1.0) <= k * 2 ** -24)
        assert np.all(np.diff(w, axis=1) <= 0)                          # sorted scores -> sorted gates


def test_gates_shift_invariant():
    rng = np.random.default_rng(4)
    l = rng.integers(-40, 40, size=(50, 8)).astype(np.float32) / np.float32(8)
    idx = oracle.topk_experts(l, 4)
    for shift in (np.float32(16), np.float32(-3.5)):                    # exact in fp32
        assert np.array_equal(oracle.gate_weights(l + shift, idx), oracle.gate_weights(l, idx))


# ------------------------------------------------------------------ slots ---

def test_slots_match_counter_walk_and_invariants():
    rng = np.random.default_rng(6)
    for _ in range(200):
        E = int(rng.integers(1, 7))
        k = int(rng.integers(1, E + 1))
        T = int(rng.integers(0, 9))
        C = int(rng.integers(1, 5))
        idx = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
        slot, src, routed, kept = oracle.assign_slots(idx, E, C)
        fill = [0] * E
        for t in range(T):
            for j in range(k):
                e = idx[t, j]
                want = fill[e] if fill[e] < C else -1
                fill[e] += 1
                assert slot[t, j] == want
        assert list(routed) == fill and routed.sum() == T * k
        assert list(kept) == [min(f, C) for f in fill]
        for e in range(E):                      # kept slots of e are 0..kept-1, once each, in token order
            mask = idx == e
            s = slot[mask]
            s = s[s >= 0]
            assert list(s) == list(range(kept[e]))
        for e in range(E):                      # src is the inverse map
            for s in range(C):
                i = src[e * C + s]
                if s < kept[e]:
                    assert idx.reshape(-1)[i] == e and slot.reshape(-1)[i] == s
                else:
                    assert i == -1


def test_forced_overflow_keeps_first_C_tokens():
    wl = moe_inputs.custom(T=50, d=32, E=4, k=2, d_ff=16, cf=0.5, dtype="bf16", seed=9, bias="hot0")
    x64 = oracle.decode(wl.x, wl.dtype)
    l = oracle.router_logits(x64, oracle.decode(wl.wr, wl.dtype), wl.bias_vec)
    idx = oracle.topk_experts(l, wl.k)
    assert np.all(idx[:, 0] == 0)
    C = oracle.capacity(wl.T, wl.E, wl.k, wl.cf)
    assert C == 13
    slot, src, routed, kept = oracle.assign_slots(idx, wl.E, C)
    assert list(slot[:, 0]) == list(range(C)) + [-1] * (wl.T - C)
    st = oracle.routing_stats(slot, routed, kept, C, 1, wl.d, 2)
    assert st["dropped"] == wl.T * wl.k - kept.sum()
    assert st["padded_rows"] == wl.E * C - kept.sum()


# --------------------------------------------------------------- dispatch ---

def test_buckets_are_bit_copies_and_inverse():
    wl = moe_inputs.custom(T=40, d=24, E=5, k=3, d_ff=16, cf=0.7, dtype="bf16", seed=10)
    x64 = oracle.decode(wl.x, wl.dtype)
    idx = oracle.topk_experts(oracle.router_logits(x64, oracle.decode(wl.wr, "bf16")), wl.k)
    C = oracle.capacity(wl.T, wl.E, wl.k, wl.cf)
    slot, src, routed, kept = oracle.assign_slots(idx, wl.E, C)
    b = oracle.dispatch_buckets(wl.x, idx, slot, wl.E, C)
    assert (slot < 0).any()                                 # this case drops copies
    for t in range(wl.T):
        for j in range(wl.k):
            if slot[t, j] >= 0:
                assert np.array_equal(b[idx[t, j], slot[t, j]], wl.x[t])
                assert src[idx[t, j] * C + slot[t, j]] == t * wl.k + j
    for e in range(wl.E):
        for s in range(kept[e]):
            assert np.array_equal(b[e, s], wl.x[src[e * C + s] // wl.k])


def test_send_counts_partition_kept():
    kept = np.arange(16)
    for P in (1, 2, 4, 8, 16):
        sc = oracle.send_counts(kept, P)
        assert sc.sum() == kept.sum()
        assert list(sc) == [kept[p * 16 // P:(p + 1) * 16 // P].sum() for p in range(P)]
    with pytest.raises(ValueError):
        oracle.send_counts(kept, 3)


def test_dispatch_volume_reproduces_printed_bandwidth_table():
    g = golden("bandwidth_table.json")
    for row in g["rows"]:
        one = oracle.dispatch_bytes(g["T"], g["k"], g["d"], row["P"], g["bytes_per_elem"])
        assert int(one / 2 ** 20) == row["one_dispatch_MiB"]            # printed truncated to MiB
        per = one * g["all_to_alls_per_layer_step"]
        assert round(per / 2 ** 30, 1) == pytest.approx(row["per_layer_step_GiB"], abs=0.051)
        assert round(per * g["layers"] / 2 ** 30) == pytest.approx(row["whole_model_GiB"], abs=0.5)


def test_alltoall_time_of_guide_example():
    g = golden("alltoall_cost.json")
    one = oracle.dispatch_bytes(g["B"] * g["S"], 1, g["d"], g["P"], g["bytes_per_elem"])
    per_layer_ms = 2 * one / g["link_bytes_per_s"] * 1e3
    assert round(per_layer_ms, 1) == g["per_layer_ms"]
    assert round(g["layers"] * round(per_layer_ms, 1), -1) == g["per_step_ms"]


def test_token_bytes_of_fanout_example():
    g = golden("hidden_state_bytes.json")
    per_token = oracle.dispatch_bytes(1, 1, g["d"], 2, g["bytes_per_elem"]) * 2   # P=2: half leaves
    assert per_token == g["token_bytes"]
    # every one of k copies off-rank: limit P -> infinity of the per-token volume
    assert oracle.dispatch_bytes(1, g["k"], g["d"], 10 ** 9, 2) / 1024 == pytest.approx(g["max_out_KiB"], rel=1e-6)


def test_offrank_bytes_of_deepseek_shape_match_printed_dispatch():
    """deepseek_v3_prefill at P=8 is the printed table's shape: off-rank valid
    bytes must land on its 784 MiB up to routing noise (about 1%)."""
    g = golden("bandwidth_table.json")
    wl = moe_inputs.workload("deepseek_v3_prefill")
    x64 = oracle.decode(wl.x, wl.dtype)
    idx = oracle.topk_experts(oracle.router_logits(x64, oracle.decode(wl.wr, wl.dtype)), wl.k)
    C = oracle.capacity(wl.T, wl.E, wl.k, wl.cf)
    slot, src, routed, kept = oracle.assign_slots(idx, wl.E, C)
    st = oracle.routing_stats(slot, routed, kept, C, wl.P, wl.d, 2)
    printed = g["rows"][0]["one_dispatch_MiB"] * 2 ** 20
    assert (g["T"], g["k"], g["d"]) == (wl.T, wl.k, wl.d)
    assert abs(st["offrank_bytes"] - printed) / printed < 0.01


# ---------------------------------------------------------------- experts ---

def test_silu_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0, 2.5])
    s = oracle.silu(z)
    assert s[0] == 0.0
    assert s[1] == pytest.approx(1.0 / (1.0 + math.e ** -1), rel=1e-15)
    assert s[2] == pytest.approx(-1.0 / (1.0 + math.e), rel=1e-15)
    assert s[3] == pytest.approx(40.0, rel=1e-15) and abs(s[4]) < 1e-15
    assert s[1] - s[2] == pytest.approx(1.0, rel=1e-15)     # silu(z) - silu(-z) = z


def test_expert_mlp_identity_weights_and_linearity():
    rng = np.random.default_rng(7)
    X = rng.standard_normal((5, 6))
    I = np.eye(6)
    y = oracle.expert_mlp(X, I, I, I)
    assert np.allclose(y, X * X / (1.0 + np.exp(-X)), rtol=1e-15, atol=0)  # silu(x) * x per element
    wg, wu, wd = rng.standard_normal((4, 6)), rng.standard_normal((4, 6)), rng.standard_normal((6, 4))
    assert np.array_equal(oracle.expert_mlp(X, wg, wu, np.zeros((6, 4))), np.zeros((5, 6)))
    assert np.allclose(oracle.expert_mlp(X, wg, wu, 2 * wd), 2 * oracle.expert_mlp(X, wg, wu, wd), rtol=1e-14)
    assert np.allclose(oracle.expert_mlp(X, wg, 3 * wu, wd), 3 * oracle.expert_mlp(X, wg, wu, wd), rtol=1e-14)
    for r in range(5):                          # rows are independent: explicit per-row loops
        assert np.allclose(oracle.expert_mlp(X[r:r + 1], wg, wu, wd)[0],
                           bf.mlp(list(X[r]), wg.tolist(), wu.tolist(), wd.tolist()), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- combine ---

def test_combine_with_identity_experts_is_inverse_permutation():
    """With y := the bucket row itself, out_t = x_t * (1 + sum of kept gates)."""
    wl = moe_inputs.custom(T=33, d=16, E=4, k=2, d_ff=8, cf=0.75, dtype="bf16", seed=11)
    x64 = oracle.decode(wl.x, wl.dtype)
    l = oracle.router_logits(x64, oracle.decode(wl.wr, "bf16"))
    idx = oracle.topk_experts(l, wl.k)
    w = oracle.gate_weights(l, idx)
    C = oracle.capacity(wl.T, wl.E, wl.k, wl.cf)
    slot, src, routed, kept = oracle.assign_slots(idx, wl.E, C)
    b = oracle.decode(oracle.dispatch_buckets(wl.x, idx, slot, wl.E, C), "bf16")
    ycopies = np.zeros((wl.T, wl.k, wl.d))
    for t in range(wl.T):
        for j in range(wl.k):
            if slot[t, j] >= 0:
                ycopies[t, j] = b[idx[t, j], slot[t, j]]
    out = oracle.combine(x64, ycopies, w, slot)
    gsum = np.where(slot >= 0, w.astype(np.float64), 0.0).sum(1)
    assert np.allclose(out, x64 * (1.0 + gsum)[:, None], rtol=1e-15, atol=0)


def test_fully_dropped_tokens_pass_through_bitwise():
    wl = moe_inputs.custom(T=30, d=16, E=2, k=1, d_ff=8, cf=0.2, dtype="bf16", seed=12)
    wl.x[:, 0] = 0x8000                                     # -0.0 must survive untouched
    r = oracle.layer_forward(wl.x, wl.wr, wl.expert, wl.T, wl.d, wl.d_ff, wl.E, wl.k, wl.cf, "bf16")
    dropped = np.all(r["slot"] < 0, axis=1)
    assert dropped.sum() >= 20
    assert np.array_equal(r["out"][dropped], wl.x[dropped])
    assert r["stats"]["fully_dropped_tokens"] == dropped.sum()


# ------------------------------------------------------------ whole layer ---

def _as_lists(a, dtype):
    return oracle.decode(a, dtype).tolist()


@pytest.mark.parametrize("case", range(24))
def test_layer_matches_bruteforce(case):
    rng = np.random.default_rng(100 + case)
    E = int(rng.integers(1, 6))
    k = int(rng.integers(1, min(3, E) + 1))
    T = int(rng.integers(1, 7))
    d = int(rng.integers(2, 7))
    f = int(rng.integers(1, 6))
    cf = float(rng.choice([0.25, 0.5, 1.0, 1.25, 2.0]))
    dtype = "bf16" if case % 2 else "f32"
    bias = "zipf1.2" if case % 3 == 0 else None
    wl = moe_inputs.custom(T=T, d=d, E=E, k=k, d_ff=f, cf=cf, dtype=dtype, seed=200 + case,
                           wr_std=1.0, bias=bias)
    r = oracle.layer_forward(wl.x, wl.wr, wl.expert, T, d, f, E, k, cf, dtype, bias=wl.bias_vec)
    ex = [wl.expert(e) for e in range(E)]
    b = bf.layer(_as_lists(wl.x, dtype), _as_lists(wl.wr, dtype),
                 None if wl.bias_vec is None else [float(v) for v in wl.bias_vec],
                 [_as_lists(e[0], dtype) for e in ex], [_as_lists(e[1], dtype) for e in ex],
                 [_as_lists(e[2], dtype) for e in ex], k, float(np.float32(cf)))
    assert r["C"] == b["C"]
    assert np.array_equal(r["logits"], np.array(b["logits"], np.float32))
    assert r["idx"].tolist() == b["idx"]
    assert np.allclose(r["w"], np.array(b["w"], np.float32), rtol=2 ** -23, atol=0)
    assert r["slot"].tolist() == b["slot"] and r["src"].tolist() == b["src"]
    assert r["routed"].tolist() == b["routed"] and r["kept"].tolist() == b["kept"]
    assert np.allclose(r["out64"], np.array(b["out"]), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("case", range(8))
def test_rank_limited_layer_matches_bruteforce(case):
    rng = np.random.default_rng(300 + case)
    P = int(rng.choice([2, 3]))
    E = P * int(rng.integers(1, 3))
    M = int(rng.integers(1, P))
    k = int(rng.integers(1, min(3, M * (E // P)) + 1))
    T, d, f = int(rng.integers(1, 7)), int(rng.integers(2, 6)), int(rng.integers(1, 5))
    cf = float(rng.choice([0.5, 1.0, 2.0]))
    dtype = "bf16" if case % 2 else "f32"
    wl = moe_inputs.custom(T=T, d=d, E=E, k=k, d_ff=f, cf=cf, dtype=dtype, seed=400 + case, wr_std=1.0,
                           P=P, max_ranks=M)
    r = oracle.layer_forward(wl.x, wl.wr, wl.expert, T, d, f, E, k, cf, dtype, P=P, max_ranks=M)
    ex = [wl.expert(e) for e in range(E)]
    b = bf.layer(_as_lists(wl.x, dtype), _as_lists(wl.wr, dtype), None,
                 [_as_lists(e[0], dtype) for e in ex], [_as_lists(e[1], dtype) for e in ex],
                 [_as_lists(e[2], dtype) for e in ex], k, float(np.float32(cf)), P=P, M=M)
    assert r["idx"].tolist() == b["idx"]
    assert max(len(set(row)) for row in (r["idx"] // (E // P)).tolist()) <= M
    assert r["slot"].tolist() == b["slot"] and r["kept"].tolist() == b["kept"]
    assert np.allclose(r["w"], np.array(b["w"], np.float32), rtol=2 ** -23, atol=0)
    assert np.allclose(r["out64"], np.array(b["out"]), rtol=1e-12, atol=1e-13)


def test_dense_special_case_single_expert():
    """E = 1, k = 1, cf >= 1: every token kept with gate 1, out = x + MLP(x)."""
    wl = moe_inputs.custom(T=9, d=5, E=1, k=1, d_ff=4, cf=1.0, dtype="f32", seed=13)
    r = oracle.layer_forward(wl.x, wl.wr, wl.expert, 9, 5, 4, 1, 1, 1.0, "f32")
    assert np.all(r["slot"][:, 0] == np.arange(9)) and np.all(r["w"] == 1.0)
    wg, wu, wd = (a.astype(np.float64).tolist() for a in wl.expert(0))
    for t in range(9):
        xt = wl.x[t].astype(np.float64).tolist()
        want = [a + b for a, b in zip(xt, bf.mlp(xt, wg, wu, wd))]
        assert np.allclose(r["out64"][t], want, rtol=1e-12, atol=1e-14)


# -------------------------------------------------------------- generator ---

def test_generator_reproducible_and_gap_conditioned():
    a = moe_inputs.custom(T=200, d=64, E=16, k=4, d_ff=32, cf=1.0, seed=21)
    b = moe_inputs.custom(T=200, d=64, E=16, k=4, d_ff=32, cf=1.0, seed=21)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.wr, b.wr)
    for e in (0, 7, 15):
        assert all(np.array_equal(p, q) for p, q in zip(a.expert(e), b.expert(e)))
    l = oracle.router_logits(oracle.decode(a.x, "bf16"), oracle.decode(a.wr, "bf16")).astype(np.float64)
    top = -np.sort(-l, axis=1)[:, :5]
    assert (top[:, :-1] - top[:, 1:]).min() > 1e-3 - 1e-6   # fp32 rounding of the scores aside
    wg, wu, wd = a.all_expert_weights()
    assert np.array_equal(wg[7], a.expert(7)[0]) and np.array_equal(wd[15], a.expert(15)[2])


def test_generator_value_laws():
    wl = moe_inputs.custom(T=512, d=256, E=8, k=2, d_ff=128, cf=1.0, seed=22, bias="zipf1.2")
    x = oracle.decode(wl.x, "bf16")
    assert abs(x.std() - 1.0) < 0.02 and abs(x.mean()) < 0.02
    assert abs(oracle.decode(wl.wr, "bf16").std() - 0.02) < 0.002
    wg, wu, wd = (oracle.decode(a, "bf16") for a in wl.expert(3))
    assert abs(wg.std() * math.sqrt(256) - 1) < 0.02 and abs(wd.std() * math.sqrt(128) - 1) < 0.02
    assert np.allclose(wl.bias_vec, -1.2 * np.log(np.arange(1, 9)), rtol=1e-6)


def test_generator_rank_limited_gap_conditioning():
    wl = moe_inputs.custom(T=300, d=64, E=32, k=4, d_ff=16, cf=1.0, seed=23, P=8, max_ranks=2)
    l = oracle.router_logits(oracle.decode(wl.x, "bf16"), oracle.decode(wl.wr, "bf16")).astype(np.float64)
    best = -np.sort(-l.reshape(300, 8, 4).max(axis=2), axis=1)
    assert (best[:, :-1] - best[:, 1:]).min() > 1e-3 - 1e-6
    idx = oracle.rank_limited_experts(l.astype(np.float32), 4, 8, 2)
    chosen = np.take_along_axis(l, idx, axis=1)
    assert (chosen[:, :-1] - chosen[:, 1:]).min() > 1e-3 - 1e-6


# ------------------------------------------------------ hot-expert replicas ---

@pytest.mark.parametrize("case", range(8))
def test_replicated_layer_matches_per_expert_capacity_bruteforce(case):
    rng = np.random.default_rng(800 + case)
    P = int(rng.choice([1, 2]))
    E = P * int(rng.integers(1, 4))
    k = int(rng.integers(1, min(2, E) + 1))
    T, d, f = int(rng.integers(3, 10)), int(rng.integers(2, 5)), int(rng.integers(1, 4))
    cf = float(rng.choice([0.25, 0.5, 1.0]))
    dtype = "bf16" if case % 2 else "f32"
    reps = rng.integers(1, 4, size=E).astype(np.int32)
    wl = moe_inputs.custom(T=T, d=d, E=E, k=k, d_ff=f, cf=cf, dtype=dtype, seed=820 + case, wr_std=1.0,
                           bias="hot0" if case % 3 == 0 else None, P=P)
    r = oracle.layer_forward(wl.x, wl.wr, wl.expert, T, d, f, E, k, cf, dtype, P=P, bias=wl.bias_vec, replicas=reps)
    ex = [wl.expert(e) for e in range(E)]
    b = bf.layer(_as_lists(wl.x, dtype), _as_lists(wl.wr, dtype),
                 None if wl.bias_vec is None else [float(v) for v in wl.bias_vec],
                 [_as_lists(e[0], dtype) for e in ex], [_as_lists(e[1], dtype) for e in ex],
                 [_as_lists(e[2], dtype) for e in ex], k, float(np.float32(cf)), caps=[int(v) for v in reps])
    assert r["idx"].tolist() == b["idx"]
    assert ((r["slot"] >= 0) == (np.array(b["slot"]) >= 0)).all()
    assert np.allclose(r["out64"], np.array(b["out"]), rtol=1e-12, atol=1e-13)
    # per expert: kept copies = min(routed, r C) over its replicas
    inst_off, expert_of, _ = oracle.replica_layout(reps, P)
    per_expert = np.bincount(expert_of, weights=r["kept"], minlength=E)
    assert np.array_equal(per_expert, np.minimum(r["routed"], reps * r["C"]))


def test_replica_slots_invariants_and_identity():
    rng = np.random.default_rng(830)
    T, E, k, C = 400, 6, 2, 60
    idx = np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32)
    reps = np.array([3, 1, 2, 1, 4, 1], np.int32)
    inst, slot, src, routed, kept = oracle.assign_replica_slots(idx, reps, C)
    inst_off, expert_of, _ = oracle.replica_layout(reps, 1)
    assert np.sum((routed < reps * C) & (reps > 1)) >= 2 and np.sum(routed > reps * C) >= 2  # both regimes
    for e in range(E):
        ks = kept[inst_off[e]:inst_off[e + 1]]
        assert ks.sum() == min(routed[e], reps[e] * C)
        if routed[e] < reps[e] * C:                  # unsaturated: loads differ by at most one
            assert ks.max() - ks.min() <= 1
    for i in range(inst_off[-1]):
        rows = np.nonzero((inst == i) & (slot >= 0))
        s_ = slot[rows]
        assert sorted(s_.tolist()) == list(range(kept[i]))        # slots 0..kept-1
        assert np.all(np.diff(s_[np.argsort(rows[0] * k + rows[1])]) > 0)   # increasing in token order
        assert np.all(expert_of[i] == idx[rows])
    # src inverts (instance, slot)
    ids = src[src >= 0]
    assert np.array_equal(inst.reshape(-1)[ids] * C + slot.reshape(-1)[ids], np.nonzero(src >= 0)[0])
    # one replica each is the plain assignment
    s1, src1, r1, k1 = oracle.assign_slots(idx, E, C)
    i2, s2, src2, r2, k2 = oracle.assign_replica_slots(idx, np.ones(E, np.int32), C)
    assert np.array_equal(s1, s2) and np.array_equal(src1, src2) and np.array_equal(k1, k2)
    assert np.array_equal(i2, idx)


def test_replica_plan_minimises_the_worst_load_per_replica():
    from fractions import Fraction
    rng = np.random.default_rng(840)
    for _ in range(60):
        E = int(rng.integers(1, 5))
        extra = int(rng.integers(0, 6))
        routed = rng.integers(0, 50, size=E)
        plan = oracle.replica_plan(routed, extra)
        assert plan.sum() == E + extra and np.all(plan >= 1)
        worst = max(Fraction(int(a), int(b)) for a, b in zip(routed, plan))
        best = None
        for alloc in itertools.product(range(extra + 1), repeat=E):   # every way to hand out the extras
            if sum(alloc) != extra:
                continue
            w = max(Fraction(int(a), 1 + c) for a, c in zip(routed, alloc))
            best = w if best is None or w < best else best
        assert worst == best
    # ties go to the lower index
    assert oracle.replica_plan(np.array([10, 10, 3]), 1).tolist() == [2, 1, 1]


# --------------------------------------------------- where replicas live ---

def _ring_placement(replicas, P):
    """Placement walked one replica at a time: every expert's first replica on
    its home rank (the contiguous owner of E/P whole experts), each further
    replica on the rank after the previous one, wrapping after rank P - 1.
    Returns [(expert, replica j, rank)] in instance order."""
    E = len(replicas)
    out = []
    for e in range(E):
        rank = 0
        while (rank + 1) * (E // P) <= e:   # home: the rank whose slice holds e
            rank += 1
        for j in range(int(replicas[e])):
            out.append((e, j, rank))
            rank = rank + 1 if rank + 1 < P else 0
    return out


def check_replica_placement(layout):
    """Every pin of the placement reading, for a function with replica_layout's
    signature; raises AssertionError on the first violation."""
    g = golden("replica_placement.json")
    inst_off, expert_of, rank_of = layout(np.array(g["replicas"], np.int32), g["P"])
    for p in g["placement"]:    # the page's two-GPU example, replica numbers 1-based
        i = inst_off[p["expert"]] + p["replica"] - 1
        assert expert_of[i] == p["expert"] and rank_of[i] == p["gpu"], p
    rng = np.random.default_rng(850)
    for P in (2, 4, 8):
        for trial in range(12):
            E = P * int(rng.integers(1, 5))
            reps = rng.integers(1, 2 * P + 2, size=E).astype(np.int32)
            reps[rng.integers(0, E)] = 1
            inst_off, expert_of, rank_of = layout(reps, P)
            R = int(reps.sum())
            assert inst_off.tolist() == np.concatenate(([0], np.cumsum(reps))).tolist()
            assert len(rank_of) == R and np.all((rank_of >= 0) & (rank_of < P))
            walk = _ring_placement(reps, P)
            assert [w[0] for w in walk] == list(expert_of)
            assert [w[2] for w in walk] == list(rank_of), (P, reps.tolist())
            for e in range(E):
                ranks = rank_of[inst_off[e]:inst_off[e + 1]]
                assert ranks[0] == e // (E // P)                     # replica 0 on the home rank
                if reps[e] <= P:                                       # spread: one replica per rank
                    assert len(set(ranks.tolist())) == reps[e]
                else:                                                  # every rank, as evenly as possible
                    cnt = np.bincount(ranks, minlength=P)
                    assert cnt.max() - cnt.min() <= 1
            # send counts over the instances' ranks add up to every kept row
            kept = rng.integers(0, 50, size=R)
            sc = np.bincount(rank_of, weights=kept, minlength=P)
            assert sc.sum() == kept.sum()
            # with one replica each the placement is the plain contiguous ownership
            _, _, r1 = layout(np.ones(E, np.int32), P)
            assert np.array_equal(r1, np.arange(E) // (E // P))


def test_replica_placement_pins():
    check_replica_placement(oracle.replica_layout)


def _mutant(rank_fn):
    def layout(replicas, P):
        inst_off, expert_of, _ = oracle.replica_layout(replicas, P)
        E = len(replicas)
        j = np.arange(inst_off[-1]) - inst_off[expert_of]
        return inst_off, expert_of, rank_fn(expert_of, j, E, P)
    return layout


@pytest.mark.parametrize("name,rank_fn", [
    ("previous device", lambda e, j, E, P: (e // (E // P) - j) % P),
    ("no spreading", lambda e, j, E, P: e // (E // P) + 0 * j),
    ("round-robin home", lambda e, j, E, P: (e + j) % P),
    ("no wrap", lambda e, j, E, P: e // (E // P) + j),
    ("home skipped", lambda e, j, E, P: (e // (E // P) + 1 + j) % P),
    ("stride two", lambda e, j, E, P: (e // (E // P) + 2 * j) % P),
])
def test_replica_placement_pins_catch_planted_mistakes(name, rank_fn):
    with pytest.raises(AssertionError):
        check_replica_placement(_mutant(rank_fn))
