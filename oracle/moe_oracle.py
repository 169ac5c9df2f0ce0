"""Plain CPU oracle of one mixture-of-experts (MoE) layer's hot path on one GPU.

TEST INFRASTRUCTURE. This module is the slow, obviously correct reference that
the HIP path is checked against. Only the test suite, the package smoke check
and the benchmark's CPU-baseline leg may import it; the product path never
does, and this module imports nothing from the HIP package.

What is computed, in the pages' own order (sources are cited per function):

  1. router logits, one fp32 score per (token, expert);
  2. top-k expert choice per token (optionally limited to the experts of at
     most M of the P ranks) and the k gate weights;
  3. expert capacity C and the stable token-order slot of every routed copy,
     with copies beyond C dropped;
  4. the fixed-capacity per-expert buckets (and their view as P contiguous
     per-rank send buffers);
  5. each expert's SwiGLU MLP on the copies it keeps;
  6. the combine: the inverse permutation, gate-weighted and summed onto the
     residual, with fully dropped tokens passed through unchanged;
  7. routing statistics;
  8. the backward pass: the gradients of the layer's inputs and weights.

All floating point here is fp64 (numpy), from the exact values of the inputs;
results are rounded once to the precision the path fixes (fp32 for logits and
gates, the input dtype for the layer output). Where the pages leave a step
open, the reading taken is stated in the function's docstring.

Page keys used in citations:
  [EP-glossary]   "Expert Parallelism", klaylearn.com glossary
  [EP-inferensys] "Expert Parallelism", inferensys.com glossary
  [EP-guide]      "Expert Parallelism", infra.bea.ai guide
  [EP-A2A]        "Expert Parallelism & All-to-All", neelmishra.github.io
  [EP-vs-TP]      "Expert parallelism vs tensor parallelism for MoE", fanout.sh

Parity status: every function below is pinned by the CPU test suite (brute
force on tiny inputs, closed forms, invariants and the printed bandwidth table
of [EP-A2A]); none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "f64_to_bf16_bits", "f64_to_f32", "encode", "silu",
    "decode", "capacity", "router_logits", "topk_experts", "rank_limited_experts", "gate_weights",
    "assign_slots", "dispatch_buckets", "send_counts", "expert_hidden", "expert_mlp",
    "combine", "routing_stats", "dispatch_bytes", "layer_forward", "layer_backward",
    "layer_backward_sample", "replica_plan", "replica_layout", "assign_replica_slots",
]


# ---------------------------------------------------------------------------
# number formats (bf16 is the top half of an IEEE binary32 word)
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16/int16) as float64."""
    u = np.asarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f64_to_f32(v: np.ndarray) -> np.ndarray:
    """Round float64 to float32, nearest-even (numpy's cast is IEEE RNE)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float64 to bf16 bit patterns, nearest-even, in one step.

    A value is rounded straight from fp64 (not via fp32, which could round
    twice): its significand is scaled so one bf16 ulp is 1, rounded half to
    even, and scaled back. Normal bf16 range only (no overflow or subnormals
    arise in this layer's outputs).
    """
    v = np.asarray(v, dtype=np.float64)
    # bf16 has 8 significant bits; scale each value's ulp to 1 and use RNE.
    with np.errstate(divide="ignore", invalid="ignore"):
        m, e = np.frexp(v)                         # v = m * 2**e, 0.5 <= |m| < 1
        r = np.ldexp(np.round(np.ldexp(m, 8)), e - 8)   # np.round is half-to-even
    r = np.where(v == 0.0, v, r)                   # keep the sign of zero
    f = r.astype(np.float32)                       # exact: r has <= 8 significant bits
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Inputs as float64: bf16 arrays arrive as raw 16-bit patterns. "f64" is
    the unrounded form used for finite-difference checks of the gradients."""
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def encode(v64: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 results once to the layer's dtype (bf16 as bit patterns)."""
    if dtype == "bf16":
        return f64_to_bf16_bits(v64)
    if dtype == "f64":
        return np.asarray(v64, dtype=np.float64)
    return f64_to_f32(v64)


# ---------------------------------------------------------------------------
# 1. router logits
# ---------------------------------------------------------------------------

def router_logits(x64: np.ndarray, wr64: np.ndarray, bias=None) -> np.ndarray:
    """Router scores: one linear score per (token, expert), fp32 result.

    [EP-glossary] body and [EP-inferensys] gating-network entry: the router is a
    small (typically linear) network scoring each token against every expert.
    logits[t, e] = sum_i x[t, i] * Wr[e, i] + b[e], with Wr stored [E, d] as an
    [out, in] linear layer. The sum is taken in fp64 and rounded once to fp32.
    The bias b (fp32, optional) is added before rounding; it is part of the
    score used both for the choice and for the gates.
    """
    s = x64 @ wr64.T
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return f64_to_f32(s)


# ---------------------------------------------------------------------------
# 2. top-k choice and gate weights
# ---------------------------------------------------------------------------

def topk_experts(logits32: np.ndarray, k: int) -> np.ndarray:
    """Per token, the k experts with the highest scores, best first.

    [EP-inferensys] gating-network entry (top-k gating) and [EP-guide] section 2
    (the router assigns each token its top-k experts). Ties are not settled on
    the pages; the reading taken: order by score descending, then expert index
    ascending, so the lowest index wins a tie. +0.0 and -0.0 compare equal.
    """
    l = np.asarray(logits32)
    l = l + l.dtype.type(0.0)  # -0.0 -> +0.0 (fp32 scores; fp64 ones in the unrounded mode)
    T, E = l.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # stable sort of -score: equal scores keep ascending expert order
    order = np.argsort(-l, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def rank_limited_experts(logits32: np.ndarray, k: int, P: int, M: int) -> np.ndarray:
    """Top-k choice restricted to experts held by at most M of the P ranks.

    [EP-A2A] "The bandwidth bill" (node-limited routing: a token's experts must
    sit on a small number of nodes, so that most all-to-all traffic stays on the
    fast local fabric) and [EP-vs-TP] "Expert parallelism pays in all-to-all
    dispatch" (DeepSeek-V3 allows at most 4 nodes per token). Rank p owns the
    contiguous experts [p E/P, (p+1) E/P), as in the send buffers.

    The pages name the constraint but not how the ranks are picked. Reading
    taken: a rank's score is the best score among its experts; the M ranks with
    the highest rank scores are allowed (lower rank index first on a tie); the
    k experts are then the best of the allowed ranks' experts, ordered as in
    topk_experts. M = 0 or M >= P is no limit. Needs M * (E/P) >= k.
    """
    l = np.asarray(logits32)
    l = l + l.dtype.type(0.0)
    T, E = l.shape
    if M == 0 or M >= P:
        return topk_experts(l, k)
    if P < 1 or E % P or M < 0 or M * (E // P) < k:
        raise ValueError("need E % P == 0 and M * (E / P) >= k")
    rank_score = l.reshape(T, P, E // P).max(axis=2)
    best_ranks = np.argsort(-rank_score, axis=1, kind="stable")[:, :M]
    allowed = np.zeros((T, P), dtype=bool)
    np.put_along_axis(allowed, best_ranks, True, axis=1)
    masked = np.where(np.repeat(allowed, E // P, axis=1), l, l.dtype.type(-np.inf))
    order = np.argsort(-masked, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def gate_weights(logits32: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Gate weights of the k chosen experts: a softmax over their scores.

    [EP-glossary] body and [EP-A2A] "All-to-all: the distributed transpose": the
    router also yields the weights that combine a token's k expert outputs. The
    pages give no formula; the reading taken is the softmax over the k chosen
    fp32 scores, w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), in fp64 and
    rounded once to fp32.
    """
    l = np.take_along_axis(np.asarray(logits32, np.float32), idx, axis=1).astype(np.float64)
    z = np.exp(l - l[:, :1])
    return f64_to_f32(z / z.sum(axis=1, keepdims=True))


# ---------------------------------------------------------------------------
# 3. capacity and slots
# ---------------------------------------------------------------------------

def capacity(T: int, E: int, k: int, cf: float) -> int:
    """Expert capacity C = ceil(cf * k * T / E).

    [EP-inferensys] capacity entry and [EP-A2A] "Why fixed-size buffers matter
    here": the per-expert buffer holds cf * k * T / E tokens. ([EP-guide]
    section 4 writes it without k; the k form is taken.) Rounding is not
    stated; the reading taken is ceil, evaluated in IEEE double as
    ((cf * k) * T) / E with cf the fp32 value the caller passes. No clamp.
    """
    cf64 = float(np.float32(cf))
    if T < 0 or E < 1 or k < 1 or not (cf64 > 0.0) or not math.isfinite(cf64):
        raise ValueError("bad capacity arguments")
    return int(math.ceil(cf64 * k * T / E))


def assign_slots(idx: np.ndarray, E: int, C: int):
    """Stable token-order slots, drops and the inverse map.

    [EP-inferensys] capacity entry: an expert processes at most C tokens and the
    excess is dropped. Priority among an expert's tokens is not stated; the
    reading taken is token order over the flattened copies i = t*k + j: copy i
    of expert e gets slot s = #{i' < i : expert(i') = e}; it is kept iff s < C.

    Returns slot[T, k] (-1 = dropped), src[E*C] (flattened copy id held by each
    kept slot, -1 on padding), routed[E] and kept[E] (int32/int64 counts).
    """
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    n = flat.size
    order = np.argsort(flat, kind="stable")            # groups by expert, token order inside
    routed = np.bincount(flat, minlength=E).astype(np.int64)
    start = np.concatenate(([0], np.cumsum(routed)[:-1]))
    rank = np.empty(n, dtype=np.int64)
    rank[order] = np.arange(n, dtype=np.int64) - start[flat[order]]
    keep = rank < C
    slot = np.where(keep, rank, -1).astype(np.int32).reshape(T, k)
    src = np.full(E * C, -1, dtype=np.int32)
    ids = np.nonzero(keep)[0]
    src[flat[ids] * C + rank[ids]] = ids.astype(np.int32)
    kept = np.minimum(routed, C)
    return slot, src, routed, kept


# ---------------------------------------------------------------------------
# 4. buckets and per-rank send buffers
# ---------------------------------------------------------------------------

def dispatch_buckets(x: np.ndarray, idx: np.ndarray, slot: np.ndarray, E: int, C: int) -> np.ndarray:
    """Fixed-capacity per-expert buffers [E, C, d] holding bit copies of x rows.

    [EP-inferensys] memory entry (pre-allocated contiguous buffers of maximum
    capacity) and [EP-A2A] "Why fixed-size buffers matter here" (per-expert
    buffer of C rows; underflow is padding). Kept copy (t, j) lands at
    [idx[t, j], slot[t, j]]. Padding rows are zero here and carry no meaning.
    """
    T, k = idx.shape
    out = np.zeros((E, C) + x.shape[1:], dtype=x.dtype)
    for j in range(k):
        kept = slot[:, j] >= 0
        t = np.nonzero(kept)[0]
        out[idx[t, j], slot[t, j]] = x[t]
    return out


def send_counts(kept: np.ndarray, P: int) -> np.ndarray:
    """Valid rows per destination rank when E experts sit on P ranks.

    [EP-A2A] "Why MoE forces a new axis": each of P devices owns E/P whole
    experts. Reading taken: rank p owns the contiguous experts
    [p*E/P, (p+1)*E/P), so its send buffer is a contiguous slice of the
    buckets.
    """
    E = kept.size
    if P < 1 or E % P:
        raise ValueError("E must be a multiple of P")
    return kept.reshape(P, E // P).sum(axis=1).astype(np.int64)


def dispatch_bytes(T: int, k: int, d: int, P: int, elem_bytes: int = 2) -> float:
    """Bytes one rank sends in one dispatch under balanced routing.

    [EP-A2A] "The bandwidth bill": each rank sends the (P-1)/P fraction of its
    T*k routed copies off-rank, each a d-wide row. (The formula itself is lost
    from the page's text; this is the form its table follows.)
    """
    return (P - 1) / P * T * k * d * elem_bytes


# ---------------------------------------------------------------------------
# 5. experts
# ---------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


def expert_hidden(X: np.ndarray, wg: np.ndarray, wu: np.ndarray) -> np.ndarray:
    """The gated hidden activation of one expert: h = silu(Wg x) * (Wu x), per row."""
    g = X @ wg.T
    u = X @ wu.T
    return silu(g) * u


def expert_mlp(X: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """One expert's SwiGLU MLP applied to each row of X (fp64).

    [EP-guide] section 1 (three weight matrices per expert) and [EP-A2A] "Tensor
    parallelism for experts" (gate, up and down projections). Reading taken:
    SwiGLU with no biases, Wg/Wu stored [d_ff, d] and Wd [d, d_ff] as
    [out, in] linear layers: y = Wd (silu(Wg x) * (Wu x)). Each row is
    independent; the matrix product just applies this to every row.
    """
    return expert_hidden(X, wg, wu) @ wd.T


# ---------------------------------------------------------------------------
# 6. combine
# ---------------------------------------------------------------------------

def combine(x64: np.ndarray, y_copies: np.ndarray, w: np.ndarray, slot: np.ndarray) -> np.ndarray:
    """Weighted sum of each token's kept expert outputs onto the residual (fp64).

    [EP-A2A] "All-to-all: the distributed transpose": the combine is the exact
    inverse of the dispatch; a token's k outputs are weighted by their gates
    and added to the residual stream. [EP-inferensys] capacity entry: a dropped
    copy contributes nothing (no renormalisation of the remaining gates).
    y_copies[t, j] is the output of copy (t, j) (any value where dropped).
    out[t] = x[t] + sum_j [slot[t, j] >= 0] * w[t, j] * y_copies[t, j].
    """
    keep = (slot >= 0).astype(np.float64) * w.astype(np.float64)
    return x64 + np.einsum("tj,tjd->td", keep, y_copies)


# ---------------------------------------------------------------------------
# 7. statistics
# ---------------------------------------------------------------------------

def routing_stats(slot: np.ndarray, routed: np.ndarray, kept: np.ndarray, C: int, P: int,
                  d: int, elem_bytes: int) -> dict:
    """Counts the pages use to talk about balance and traffic.

    [EP-inferensys] capacity entry (drop rate), [EP-vs-TP] "Decide from expert
    shape, batch, and fabric" (routed tokens per expert), [EP-A2A] "The
    bandwidth bill" (off-rank bytes). Rank 0 is taken as the sending rank.
    """
    T, k = slot.shape
    E = routed.size
    sc = send_counts(kept, P)
    n_kept = int(kept.sum())
    return {
        "routed": routed.astype(np.int64),
        "kept": kept.astype(np.int64),
        "send_count": sc,
        "dropped": T * k - n_kept,
        "fully_dropped_tokens": int(np.all(slot < 0, axis=1).sum()) if k else 0,
        "padded_rows": E * C - n_kept,
        "offrank_bytes": int(sc[1:].sum()) * d * elem_bytes,
    }


# ---------------------------------------------------------------------------
# hot-expert replication
# ---------------------------------------------------------------------------

def replica_plan(routed: np.ndarray, extra: int) -> np.ndarray:
    """Replica counts: one per expert, plus `extra` more for the hot ones.

    [EP-guide] section 6 "Optimizations", "Expert Replication": popular experts
    are replicated on several devices so their tokens can go to either copy,
    for better balance and fewer drops at the cost of memory; [EP-vs-TP] names a load
    balancer that re-places experts under skew. No policy is given. Reading
    taken: each extra replica goes, one at a time, to the expert with the
    highest load per replica, routed[e] / r[e] (compared exactly as integers),
    the lowest index winning a tie.
    """
    routed = np.asarray(routed, dtype=np.int64)
    r = np.ones(routed.size, dtype=np.int64)
    for _ in range(int(extra)):
        best = 0
        for e in range(1, routed.size):
            if routed[e] * r[best] > routed[best] * r[e]:
                best = e
        r[best] += 1
    return r.astype(np.int32)


def replica_layout(replicas: np.ndarray, P: int):
    """Instances of the replicated experts: offsets [E+1] (instance i of
    expert e is inst_off[e] + j for its replica j), expert_of[R] and
    rank_of[R]. Reading taken for placement ([EP-guide] section 6
    "Optimizations", "Expert Replication", puts replica 2 of expert 0 on the
    next device): replica j of expert e sits on rank (home(e) + j) mod P,
    home(e) = e // (E/P) as for unreplicated experts.
    """
    r = np.asarray(replicas, dtype=np.int64)
    E = r.size
    if P < 1 or E % P or np.any(r < 1):
        raise ValueError("need E % P == 0 and every replica count >= 1")
    inst_off = np.concatenate(([0], np.cumsum(r)))
    expert_of = np.repeat(np.arange(E), r)
    j = np.arange(inst_off[-1]) - inst_off[expert_of]
    rank_of = (expert_of // (E // P) + j) % P
    return inst_off, expert_of, rank_of


def assign_replica_slots(idx: np.ndarray, replicas: np.ndarray, C: int):
    """Slots when expert e has r_e replicas of capacity C each.

    Reading taken (the pages say only that an expert's tokens may go to either
    replica): the copies of expert e, in the token order of assign_slots, are
    dealt to its replicas in turn. Copy q (its rank among e's copies) goes to
    replica q mod r_e at slot q div r_e, and is dropped iff that slot is >= C,
    so the expert keeps min(routed, r_e C) copies and its replicas' loads
    differ by at most one. Returns instance[T, k], slot[T, k] (-1 = dropped),
    src[R*C], routed[E] and kept[R].
    """
    T, k = idx.shape
    r = np.asarray(replicas, dtype=np.int64)
    E = r.size
    inst_off = np.concatenate(([0], np.cumsum(r)))
    R = int(inst_off[-1])
    flat = idx.reshape(-1).astype(np.int64)
    n = flat.size
    order = np.argsort(flat, kind="stable")
    routed = np.bincount(flat, minlength=E).astype(np.int64)
    start = np.concatenate(([0], np.cumsum(routed)[:-1]))
    q = np.empty(n, dtype=np.int64)
    q[order] = np.arange(n, dtype=np.int64) - start[flat[order]]
    inst = inst_off[flat] + q % r[flat]
    s = q // r[flat]
    keep = s < C
    slot = np.where(keep, s, -1).astype(np.int32).reshape(T, k)
    src = np.full(R * C, -1, dtype=np.int32)
    ids = np.nonzero(keep)[0]
    src[inst[ids] * C + s[ids]] = ids.astype(np.int32)
    kept = np.bincount(inst[keep], minlength=R).astype(np.int64)
    return inst.astype(np.int32).reshape(T, k), slot, src, routed, kept


# ---------------------------------------------------------------------------
# the whole layer
# ---------------------------------------------------------------------------

def layer_forward(x, wr, expert_weights, T, d, d_ff, E, k, cf, dtype, P=1, bias=None,
                  tokens=None, max_ranks=0, exact=False, replicas=None):
    """The layer as the plain per-token definition, steps 1 to 7 above.

    x [T, d] and wr [E, d] are the inputs (bf16 as bit patterns, or fp32).
    expert_weights(e) returns (Wg [d_ff, d], Wu [d_ff, d], Wd [d, d_ff]) of
    expert e in the same format, so a caller can supply them lazily.
    Routing, slots and statistics are computed for all T tokens; the layer
    output only for `tokens` (all when None), since each output row depends
    only on its own token once the slots are known. max_ranks > 0 limits each
    token's experts to that many of the P ranks (rank_limited_experts).
    exact=True keeps the scores and gates in fp64 (no fp32 rounding): the
    smooth function that finite differences of the gradients need.
    replicas [E] (replica counts, see replica_plan) spreads each expert's
    copies over its replicas (assign_replica_slots); slot is then the row in
    the copy's instance, and kept, src and send_count are per instance.

    Returns a dict: logits, idx, w, C, slot, src, routed, kept, stats,
    tokens, out64 (fp64, unrounded), out (rounded once to dtype; a token with
    every copy dropped is a bit copy of its input row).
    """
    x = np.asarray(x)
    x64 = decode(x, dtype)
    if exact:
        logits = x64 @ decode(wr, dtype).T
        if bias is not None:
            logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
        idx = rank_limited_experts(logits, k, P, max_ranks)
        lsel = np.take_along_axis(logits, idx, axis=1)
        z = np.exp(lsel - lsel[:, :1])
        w = z / z.sum(axis=1, keepdims=True)
    else:
        logits = router_logits(x64, decode(wr, dtype), bias)
        idx = rank_limited_experts(logits, k, P, max_ranks)
        w = gate_weights(logits, idx)
    C = capacity(T, E, k, cf)
    eb = {"bf16": 2, "f32": 4, "f64": 8}[dtype]
    instance = None
    if replicas is None:
        slot, src, routed, kept = assign_slots(idx, E, C)
        stats = routing_stats(slot, routed, kept, C, P, d, eb)
    else:
        instance, slot, src, routed, kept = assign_replica_slots(idx, replicas, C)
        _, _, rank_of = replica_layout(replicas, P)
        sc = np.bincount(rank_of, weights=kept, minlength=P).astype(np.int64)
        n_kept = int(kept.sum())
        stats = {"routed": routed, "kept": kept, "send_count": sc, "dropped": T * k - n_kept,
                 "fully_dropped_tokens": int(np.all(slot < 0, axis=1).sum()),
                 "padded_rows": kept.size * C - n_kept, "offrank_bytes": int(sc[1:].sum()) * d * eb}

    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    y = np.zeros((tok.size, k, d), dtype=np.float64)
    sub_idx, sub_slot = idx[tok], slot[tok]
    for e in np.unique(sub_idx[sub_slot >= 0]):
        rows, js = np.nonzero((sub_idx == e) & (sub_slot >= 0))
        wg, wu, wd = (decode(a, dtype) for a in expert_weights(int(e)))
        y[rows, js] = expert_mlp(x64[tok[rows]], wg, wu, wd)
    out64 = combine(x64[tok], y, w[tok], sub_slot)
    out = encode(out64, dtype)
    passthru = np.all(sub_slot < 0, axis=1)
    out[passthru] = x[tok[passthru]]
    return {"logits": logits, "idx": idx, "w": w, "C": C, "slot": slot, "src": src,
            "routed": routed, "kept": kept, "stats": stats, "tokens": tok,
            "out64": out64, "out": out, "instance": instance}


# ---------------------------------------------------------------------------
# 8. the backward pass
# ---------------------------------------------------------------------------

def layer_backward(x, wr, expert_weights, dout, T, d, d_ff, E, k, cf, dtype, P=1, bias=None,
                   max_ranks=0, exact=False):
    """Gradients of the layer, given dout = dLoss/dout [T, d] in the layer dtype.

    [EP-A2A] "The bandwidth bill": the backward pass repeats the dispatch and
    combine (two more all-to-alls per layer), i.e. it runs the same routing
    in reverse. The pages give no formulas; the reading taken is the chain
    rule through the forward above, with the top-k choice and the capacity
    drops held fixed (they are piecewise constant):

      combine:   dw[t, j] = <dout[t], y[t, j]> for a kept copy, 0 if dropped;
                 dy[t, j] = w[t, j] * dout[t]; dx[t] starts at dout[t]
      gates:     dl[t, j] = w[t, j] * (dw[t, j] - sum_i w[t, i] dw[t, i])
      router:    dx += dl Wr[idx]; dWr[e] = sum_t dl[t, e] x[t]; db = sum_t dl[t]
      experts:   dh = dy Wd; dWd = dy^T h; dg = dh u silu'(g); du = dh silu(g);
                 dWg = dg^T X; dWu = du^T X; dx[t] += dg Wg + du Wu
                 with silu'(g) = s (1 + g (1 - s)), s = sigmoid(g)

    Every sum is fp64 over the copies each expert kept. Returns a dict: dx,
    dwr [E, d], db [E], dwg, dwu [E, d_ff, d], dwd [E, d, d_ff] (all fp64),
    dw and dl [T, k], and the routing (idx, w, slot).
    """
    fwd = layer_forward(x, wr, expert_weights, T, d, d_ff, E, k, cf, dtype, P=P, bias=bias,
                        tokens=np.arange(0), max_ranks=max_ranks, exact=exact)
    idx, w, slot = fwd["idx"], np.asarray(fwd["w"], dtype=np.float64), fwd["slot"]
    x64 = decode(np.asarray(x), dtype)
    g_out = decode(np.asarray(dout), dtype)
    dx = g_out.copy()
    dw = np.zeros((T, k))
    dwg = np.zeros((E, d_ff, d))
    dwu = np.zeros((E, d_ff, d))
    dwd = np.zeros((E, d, d_ff))
    for e in range(E):
        rows, js = np.nonzero((idx == e) & (slot >= 0))
        if rows.size == 0:
            continue
        wg, wu, wd = (decode(a, dtype) for a in expert_weights(e))
        X = x64[rows]
        gpre = X @ wg.T
        upre = X @ wu.T
        sg = 1.0 / (1.0 + np.exp(-gpre))
        h = gpre * sg * upre
        y = h @ wd.T
        dw[rows, js] = np.sum(g_out[rows] * y, axis=1)
        dy = w[rows, js][:, None] * g_out[rows]
        dh = dy @ wd
        dwd[e] = dy.T @ h
        dg = dh * upre * sg * (1.0 + gpre * (1.0 - sg))
        du = dh * gpre * sg
        dwg[e] = dg.T @ X
        dwu[e] = du.T @ X
        np.add.at(dx, rows, dg @ wg + du @ wu)
    dl = w * (dw - np.sum(w * dw, axis=1, keepdims=True))
    dl_full = np.zeros((T, E))
    np.put_along_axis(dl_full, idx, dl, axis=1)
    dx += dl_full @ decode(np.asarray(wr), dtype)
    return {"dx": dx, "dwr": dl_full.T @ x64, "db": dl_full.sum(axis=0), "dwg": dwg, "dwu": dwu,
            "dwd": dwd, "dw": dw, "dl": dl, "idx": idx, "w": w, "slot": slot}


def layer_backward_sample(x, wr, expert_weights, dout, T, d, d_ff, E, k, cf, dtype, P=1, bias=None,
                          max_ranks=0, tokens=(), cols=()):
    """Chosen outputs of layer_backward, each computed on its own (for layers
    too large for the dense form): dx rows of `tokens`, and for each (e, f) in
    `cols` the column dWd[e][:, f] and the rows dWg[e][f, :], dWu[e][f, :].
    Same formulas and readings as layer_backward; routing is computed for all
    T tokens. Experts are visited one at a time, so only one expert's weights
    are held in fp64. Returns {"dx": {t: row}, "dwd": {(e, f): col},
    "dwg": {...}, "dwu": {...}}.
    """
    fwd = layer_forward(x, wr, expert_weights, T, d, d_ff, E, k, cf, dtype, P=P, bias=bias,
                        tokens=np.arange(0), max_ranks=max_ranks)
    idx, w, slot = fwd["idx"], np.asarray(fwd["w"], dtype=np.float64), fwd["slot"]
    x = np.asarray(x)
    dout = np.asarray(dout)
    tok = np.asarray(list(tokens), dtype=np.int64)
    xt, gt = decode(x[tok], dtype), decode(dout[tok], dtype)
    dw = np.zeros((tok.size, k))
    dxe = np.zeros((tok.size, d))
    sub_idx, sub_slot = idx[tok], slot[tok]
    res = {"dx": {}, "dwd": {}, "dwg": {}, "dwu": {}}
    for e in sorted(set(np.unique(sub_idx[sub_slot >= 0]).tolist()) | {int(c[0]) for c in cols}):
        wg, wu, wd = (decode(a, dtype) for a in expert_weights(int(e)))
        rows, js = np.nonzero((sub_idx == e) & (sub_slot >= 0))
        if rows.size:
            gpre, upre = xt[rows] @ wg.T, xt[rows] @ wu.T
            sg = 1.0 / (1.0 + np.exp(-gpre))
            y = (gpre * sg * upre) @ wd.T
            dw[rows, js] = np.sum(gt[rows] * y, axis=1)
            dh = (w[tok[rows], js][:, None] * gt[rows]) @ wd
            dg = dh * upre * sg * (1.0 + gpre * (1.0 - sg))
            du = dh * gpre * sg
            np.add.at(dxe, rows, dg @ wg + du @ wu)
        for ce, f in cols:
            if ce != e:
                continue
            r2, j2 = np.nonzero((idx == e) & (slot >= 0))
            X = decode(x[r2], dtype)
            dy = w[r2, j2][:, None] * decode(dout[r2], dtype)
            gcol, ucol = X @ wg[f], X @ wu[f]
            s2 = 1.0 / (1.0 + np.exp(-gcol))
            res["dwd"][(int(e), int(f))] = dy.T @ (gcol * s2 * ucol)
            dh2 = dy @ wd[:, f]
            res["dwg"][(int(e), int(f))] = (dh2 * ucol * s2 * (1.0 + gcol * (1.0 - s2))) @ X
            res["dwu"][(int(e), int(f))] = (dh2 * gcol * s2) @ X
    wr64 = decode(np.asarray(wr), dtype)
    for n, t in enumerate(tok):
        dl = w[t] * (dw[n] - np.sum(w[t] * dw[n]))
        res["dx"][int(t)] = gt[n] + dxe[n] + dl @ wr64[idx[t]]
    return res
