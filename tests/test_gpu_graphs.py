"""The layer under HIP graph capture, through the C ABI: a captured
moe_layer_forward, moe_layer_forward_replicated or moe_layer_backward
replayed several times gives the eager call's outputs bit for bit on every
replay.

The library allocates nothing, never synchronises with the host and clears
its own counters with kernels, so a serving loop may capture a layer call once
and replay it. Between replays the test fills every output with a sentinel and
runs an eager call of the same entry point on other inputs over the same
workspace, so a replay that left an output unwritten, or that depended on what
an earlier call left in the workspace (split-K arrival counters, tile
histograms), shows up as a mismatch."""
import pytest

import moe_inputs
import routing_dispatch_expert_amd as moe
from tests.gpu_util import gpu_available, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

REPLAYS = 3


@pytest.fixture(autouse=True)
def _gpu():
    assert gpu_available(), "GPU tests need an MI355X; run them with -m gpu on a GPU host"
    moe.lib()
    moe.moe_set_stage_events(None)   # no profiling events inside a captured call


def _weights(wl):
    wg, wu, wd = wl.all_expert_weights()
    return to_dev(wg, wl.dtype), to_dev(wu, wl.dtype), to_dev(wd, wl.dtype)


def _bits(t):
    """A tensor's bytes, for bitwise comparison (NaN and -0.0 included)."""
    return t.detach().contiguous().view(torch.uint8).clone()


def _fill(tensors):
    for t in tensors:
        if t.dtype in (torch.int32, torch.int64):
            t.fill_(-7)
        elif t.dtype == torch.bfloat16:
            t.view(torch.int16).fill_(0x7FC1)   # a NaN
        else:
            t.fill_(float("nan"))


def _replays_match(run, outputs, disturb):
    """run(stream) launches the call on `stream`; outputs: name -> tensor."""
    _fill(outputs.values())
    run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = {n: _bits(t) for n, t in outputs.items()}
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        _fill(outputs.values())
        disturb()                 # eager work on the same workspace between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, t in outputs.items():
            assert torch.equal(_bits(t), ref[n]), f"replay {i}: {n} differs from the eager call"


FORWARD_CASES = [
    # 256-row LDS-DMA GEMMs with a split last round (arrival counters reset per call)
    dict(T=2048, d=512, E=8, k=2, d_ff=256, cf=1.25),
    # decode-sized: a wave per token in the route, the weight-streaming GEMMs
    dict(T=64, d=512, E=128, k=8, d_ff=256, cf=2.0, P=8),
    # router scores on the GEMM kernel (128 experts, 256+ tokens), a bias and a rank limit
    dict(T=512, d=256, E=128, k=4, d_ff=128, cf=1.25, P=8, max_ranks=2, bias="zipf1.2"),
]


@pytest.mark.parametrize("case", FORWARD_CASES, ids=lambda c: f"T{c['T']}-E{c['E']}-k{c['k']}")
def test_captured_forward_replays_bit_for_bit(case):
    say(f"graph forward {case}")
    wl = moe_inputs.custom(seed=17, reject=False, **case)
    other = moe_inputs.custom(seed=18, reject=False, **case)
    T, d, E, k, P, d_ff, cf = wl.T, wl.d, wl.E, wl.k, wl.P, wl.d_ff, wl.cf
    C = moe.moe_capacity(T, E, k, cf)
    x, x2 = to_dev(wl.x, wl.dtype), to_dev(other.x, wl.dtype)
    wr = to_dev(wl.wr, wl.dtype)
    wg, wu, wd = _weights(wl)
    b = None if wl.bias_vec is None else torch.from_numpy(wl.bias_vec).cuda()
    i32 = dict(dtype=torch.int32, device="cuda")
    out = {"out": torch.empty((T, d), dtype=x.dtype, device="cuda"), "topk_idx": torch.empty((T, k), **i32),
           "topk_w": torch.empty((T, k), dtype=torch.float32, device="cuda"), "slot": torch.empty((T, k), **i32),
           "src": torch.empty((E, C), **i32), "routed_count": torch.empty(E, **i32),
           "kept_count": torch.empty(E, **i32), "send_count": torch.empty(P, **i32),
           "totals": torch.empty(4, dtype=torch.int64, device="cuda"),
           "buckets": torch.empty((E, C, d), dtype=x.dtype, device="cuda")}
    other_out = {n: torch.empty_like(t) for n, t in out.items()}
    n = moe.moe_workspace_size(T, d, d_ff, E, k, cf, P, wl.dtype)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    stats = {k_: v for k_, v in out.items() if k_ != "out"}
    other_stats = {k_: v for k_, v in other_out.items() if k_ != "out"}

    def run(stream):
        moe.moe_layer_forward(x, wr, b, wg, wu, wd, T, d, d_ff, E, k, cf, P, wl.max_ranks, wl.dtype, out["out"],
                              stats, ws, n, stream)

    def disturb():
        moe.moe_layer_forward(x2, wr, b, wg, wu, wd, T, d, d_ff, E, k, cf, P, wl.max_ranks, wl.dtype,
                              other_out["out"], other_stats, ws, n)

    # every output is filled with a sentinel before the eager call and before
    # each replay, so the never-written padding rows of the buckets compare
    # equal and every written element must match
    _replays_match(run, out, disturb)


def test_captured_backward_replays_bit_for_bit():
    case = dict(T=512, d=256, E=16, k=2, d_ff=128, cf=1.25)
    say(f"graph backward {case}")
    wl = moe_inputs.custom(seed=21, reject=False, **case)
    T, d, E, k, P, d_ff, cf = wl.T, wl.d, wl.E, wl.k, wl.P, wl.d_ff, wl.cf
    x = to_dev(wl.x, wl.dtype)
    wr = to_dev(wl.wr, wl.dtype)
    wg, wu, wd = _weights(wl)
    dout = to_dev(wl.grad_out(3), wl.dtype)
    dout2 = to_dev(wl.grad_out(4), wl.dtype)
    grads = {"dx": torch.empty_like(x), "dW_router": torch.empty_like(wr), "dW_gate": torch.empty_like(wg),
             "dW_up": torch.empty_like(wu), "dW_down": torch.empty_like(wd),
             "d_bias": torch.empty(E, dtype=torch.float32, device="cuda")}
    other = {n: torch.empty_like(t) for n, t in grads.items()}
    n = moe.moe_backward_workspace_size(T, d, d_ff, E, k, cf, P, wl.dtype)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    bias = torch.zeros(E, dtype=torch.float32, device="cuda")

    def call(g_out, dy, stream):
        moe.moe_layer_backward(x, wr, bias, wg, wu, wd, dy, T, d, d_ff, E, k, cf, P, 0, wl.dtype, g_out["dx"],
                               g_out["dW_router"], g_out["d_bias"], g_out["dW_gate"], g_out["dW_up"],
                               g_out["dW_down"], ws, n, stream)

    _replays_match(lambda s: call(grads, dout, s), grads, lambda: call(other, dout2, None))


REPLICATED_CASES = [
    # 256-row tiles with a split last round over R = 9 instances (the instance
    # scan clears the split-K arrival counters and writes GEMM 1's tile map)
    (dict(T=2048, d=256, E=4, k=2, d_ff=512, cf=0.5), [3, 2, 2, 2]),
    # a skewed route with a rank limit: instances placed over 8 ranks
    (dict(T=512, d=256, E=32, k=4, d_ff=128, cf=1.0, P=8, max_ranks=2, bias="zipf1.2"), [4, 2] + [1] * 30),
]


@pytest.mark.parametrize("case,reps", REPLICATED_CASES, ids=["E4-R9-split", "E32-R36-P8-zipf"])
def test_captured_replicated_forward_replays_bit_for_bit(case, reps):
    say(f"graph replicated forward {case} replicas {reps}")
    wl = moe_inputs.custom(seed=23, reject=False, **case)
    other = moe_inputs.custom(seed=24, reject=False, **case)
    T, d, E, k, P, d_ff, cf = wl.T, wl.d, wl.E, wl.k, wl.P, wl.d_ff, wl.cf
    C = moe.moe_capacity(T, E, k, cf)
    R = sum(reps)
    replicas = torch.tensor(reps, dtype=torch.int32, device="cuda")
    x, x2 = to_dev(wl.x, wl.dtype), to_dev(other.x, wl.dtype)
    wr = to_dev(wl.wr, wl.dtype)
    wg, wu, wd = _weights(wl)
    b = None if wl.bias_vec is None else torch.from_numpy(wl.bias_vec).cuda()
    i32 = dict(dtype=torch.int32, device="cuda")
    out = {"out": torch.empty((T, d), dtype=x.dtype, device="cuda"), "topk_idx": torch.empty((T, k), **i32),
           "topk_w": torch.empty((T, k), dtype=torch.float32, device="cuda"), "slot": torch.empty((T, k), **i32),
           "instance": torch.empty((T, k), **i32), "src": torch.empty((R, C), **i32),
           "routed_count": torch.empty(E, **i32), "kept_count": torch.empty(R, **i32),
           "send_count": torch.empty(P, **i32), "totals": torch.empty(4, dtype=torch.int64, device="cuda"),
           "buckets": torch.empty((R, C, d), dtype=x.dtype, device="cuda")}
    other_out = {n: torch.empty_like(t) for n, t in out.items()}
    n = moe.moe_replicated_workspace_size(T, d, d_ff, E, k, cf, P, R, wl.dtype)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")

    def call(xx, o, stream):
        moe.moe_layer_forward_replicated(xx, wr, b, wg, wu, wd, T, d, d_ff, E, k, cf, P, wl.max_ranks, replicas, R,
                                         wl.dtype, o["out"], {k_: v for k_, v in o.items() if k_ != "out"}, ws, n,
                                         stream)

    _replays_match(lambda s: call(x, out, s), out, lambda: call(x2, other_out, None))
