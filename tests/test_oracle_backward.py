"""Pins of the oracle's backward pass.

The gradients are checked against central finite differences of the oracle's
own forward in its unrounded fp64 mode (a different code path: the forward
composes the layer, the backward applies the chain rule by hand), along random
directions in every input and weight, with capacity drops, a router bias and a
rank limit in play. Closed forms and invariants cover the degenerate cases.
"""
import numpy as np
import pytest

import oracle

# (T, d, E, k, d_ff, cf, P, max_ranks, bias)
CASES = [
    (7, 5, 4, 2, 3, 1.0, 1, 0, False),
    (9, 4, 6, 3, 5, 0.5, 3, 2, True),     # drops, rank limit, bias
    (6, 3, 5, 1, 4, 1.0, 1, 0, True),     # k = 1: gates are constant
    (5, 6, 1, 1, 4, 1.0, 1, 0, False),    # a single expert: a dense SwiGLU MLP
    (12, 4, 4, 2, 2, 0.25, 2, 1, False),  # heavy drops, one rank of two
]


def _draw(case, seed):
    T, d, E, k, f, cf, P, M, has_b = case
    rng = np.random.default_rng(seed)
    p = {"x": rng.standard_normal((T, d)), "wr": rng.standard_normal((E, d)),
         "b": rng.standard_normal(E) if has_b else None,
         "wg": rng.standard_normal((E, f, d)) / np.sqrt(d), "wu": rng.standard_normal((E, f, d)) / np.sqrt(d),
         "wd": rng.standard_normal((E, d, f)) / np.sqrt(f)}
    dout = rng.standard_normal((T, d))
    return p, dout


def _forward(case, p):
    T, d, E, k, f, cf, P, M, _ = case
    return oracle.layer_forward(p["x"], p["wr"], lambda e: (p["wg"][e], p["wu"][e], p["wd"][e]), T, d, f, E, k, cf,
                                "f64", P=P, bias=p["b"], max_ranks=M, exact=True)


def _backward(case, p, dout):
    T, d, E, k, f, cf, P, M, _ = case
    return oracle.layer_backward(p["x"], p["wr"], lambda e: (p["wg"][e], p["wu"][e], p["wd"][e]), dout, T, d, f, E,
                                 k, cf, "f64", P=P, bias=p["b"], max_ranks=M, exact=True)


GRAD_OF = {"x": "dx", "wr": "dwr", "b": "db", "wg": "dwg", "wu": "dwu", "wd": "dwd"}


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_gradients_match_central_differences(ci):
    case = CASES[ci]
    p, dout = _draw(case, 500 + ci)
    g = _backward(case, p, dout)
    base = _forward(case, p)
    rng = np.random.default_rng(900 + ci)
    eps = 1e-5
    for name, gname in GRAD_OF.items():
        if p[name] is None:
            continue
        for _ in range(3):
            v = rng.standard_normal(p[name].shape)
            plus = dict(p, **{name: p[name] + eps * v})
            minus = dict(p, **{name: p[name] - eps * v})
            fp, fm = _forward(case, plus), _forward(case, minus)
            for r in (fp, fm):  # the choice and the drops must not move
                assert np.array_equal(r["idx"], base["idx"]) and np.array_equal(r["slot"], base["slot"])
            fd = (np.sum(dout * fp["out64"]) - np.sum(dout * fm["out64"])) / (2 * eps)
            an = np.sum(g[gname] * v)
            assert abs(fd - an) <= 1e-6 * (abs(fd) + np.linalg.norm(g[gname]) * np.linalg.norm(v)), (name, fd, an)


def test_fully_dropped_tokens_get_dout_unchanged():
    case = CASES[4]
    p, dout = _draw(case, 601)
    g = _backward(case, p, dout)
    gone = np.all(g["slot"] < 0, axis=1)
    assert gone.any()
    assert np.array_equal(g["dx"][gone], dout[gone])          # no expert, no router path
    assert np.all(g["dl"][gone] == 0) and np.all(g["dw"][gone] == 0)
    dropped = g["slot"] < 0
    assert np.all(g["dw"][dropped] == 0)


def test_single_choice_has_no_router_gradient():
    case = CASES[2]
    p, dout = _draw(case, 602)
    g = _backward(case, p, dout)
    assert np.all(g["w"] == 1.0)
    assert np.all(g["dl"] == 0) and np.all(g["dwr"] == 0) and np.all(g["db"] == 0)


def test_gradients_are_linear_in_dout_and_vanish_with_it():
    case = CASES[1]
    p, d1 = _draw(case, 603)
    _, d2 = _draw(case, 604)
    g1, g2 = _backward(case, p, d1), _backward(case, p, d2)
    g12 = _backward(case, p, 2.0 * d1 - 0.5 * d2)
    for key in ("dx", "dwr", "db", "dwg", "dwu", "dwd"):
        assert np.allclose(g12[key], 2.0 * g1[key] - 0.5 * g2[key], rtol=1e-12, atol=1e-12)
    g0 = _backward(case, p, np.zeros_like(d1))
    assert all(np.all(g0[key] == 0) for key in ("dx", "dwr", "db", "dwg", "dwu", "dwd"))


def test_gate_gradients_sum_to_zero_per_token():
    # softmax backward: sum_j dl_j = sum_j w_j dw_j - (sum_j w_j)(sum_i w_i dw_i) = 0
    case = CASES[0]
    p, dout = _draw(case, 605)
    g = _backward(case, p, dout)
    assert np.allclose(g["dl"].sum(axis=1), 0.0, atol=1e-12)
    assert np.allclose(g["db"].sum(), 0.0, atol=1e-12)


@pytest.mark.parametrize("ci", [0, 1, 4])
def test_sampled_backward_equals_the_dense_one(ci):
    case = CASES[ci]
    T, d, E, k, f, cf, P, M, _ = case
    p, dout = _draw(case, 700 + ci)
    g = _backward(case, p, dout)
    ew = lambda e: (p["wg"][e], p["wu"][e], p["wd"][e])  # noqa: E731
    cols = [(e, c) for e in range(E) for c in range(f)]
    s = oracle.layer_backward_sample(p["x"], p["wr"], ew, dout, T, d, f, E, k, cf, "f64", P=P, bias=p["b"],
                                     max_ranks=M, tokens=range(T), cols=cols)
    # the dense form rounds its scores to fp32 only in the default mode: compare that mode
    gd = oracle.layer_backward(p["x"], p["wr"], ew, dout, T, d, f, E, k, cf, "f64", P=P, bias=p["b"], max_ranks=M)
    for t in range(T):
        assert np.allclose(s["dx"][t], gd["dx"][t], rtol=1e-12, atol=1e-12)
    for (e, c) in cols:
        assert np.allclose(s["dwd"][(e, c)], gd["dwd"][e][:, c], rtol=1e-12, atol=1e-12)
        assert np.allclose(s["dwg"][(e, c)], gd["dwg"][e][c], rtol=1e-12, atol=1e-12)
        assert np.allclose(s["dwu"][(e, c)], gd["dwu"][e][c], rtol=1e-12, atol=1e-12)
    assert np.allclose(g["dx"], gd["dx"], rtol=1e-4, atol=1e-4)  # exact vs fp32-rounded scores: close
