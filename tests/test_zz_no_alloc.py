"""The no-allocation permutation (moe_permute_static) through the C ABI: its
results equal moe_permute's, bit for bit, on two calls in a row (the second
with a smaller input, so it runs on the contents the first left in the
library's static buffer); every output is followed by a canary region."""
import numpy as np
import pytest

import moe_inputs
import oracle
import routing_dispatch_expert_amd as moe
from tests.gpu_util import Guarded, gpu_available, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True)
def _gpu():
    assert gpu_available(), "GPU tests need an MI355X; run them with -m gpu on a GPU host"
    moe.lib()


def _routes(rng, T, E, k):
    p = 1.0 / np.arange(1, E + 1) ** 1.2
    p /= p.sum()
    return np.array([rng.choice(E, k, replace=False, p=p) for _ in range(T)], np.int32).reshape(T, k)


def _outputs(T, E, k, C, P, d):
    g = Guarded()
    o = {"buckets": g.empty((E, C, d), torch.bfloat16, "buckets"), "slot": g.empty((T, k), torch.int32, "slot"),
         "src": g.empty((E, C), torch.int32, "src"), "routed": g.empty((E,), torch.int32, "routed"),
         "kept": g.empty((E,), torch.int32, "kept"), "send": g.empty((P,), torch.int32, "send"),
         "totals": g.empty((4,), torch.int64, "totals")}
    o["buckets"].view(torch.int16).fill_(0x7F7F)
    return g, o


def _call(fn, x, idx, T, d, E, k, C, P, o, *ws):
    fn(x, idx, T, d, E, k, C, P, "bf16", o["buckets"], o["slot"], o["src"], o["routed"], o["kept"], o["send"],
       o["totals"], *ws)


@pytest.mark.parametrize("T,E,k,cf,P,d", [(5000, 64, 6, 1.0, 8, 256), (700, 16, 4, 0.5, 4, 64)])
def test_static_permute_equals_the_workspace_entry_point(T, E, k, cf, P, d):
    # the two cases run in this order in one process: the second, smaller one
    # finds the first one's contents in the static buffer
    say(f"no-alloc permute T={T} E={E} k={k} cf={cf} P={P} d={d}")
    rng = np.random.default_rng(T + E)
    idx = torch.from_numpy(_routes(rng, T, E, k)).cuda()
    x = to_dev(moe_inputs.custom(T=T, d=d, E=E, k=k, d_ff=8, cf=cf, seed=T, reject=False).x, "bf16")
    C = oracle.capacity(T, E, k, cf)
    ga, a = _outputs(T, E, k, C, P, d)
    gb, b = _outputs(T, E, k, C, P, d)
    n = moe.moe_permute_workspace_size(T, E)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    _call(moe.moe_permute, x, idx, T, d, E, k, C, P, a, ws, n)
    _call(moe.moe_permute_static, x, idx, T, d, E, k, C, P, b)
    torch.cuda.synchronize()
    ga.check()
    gb.check()
    for key in a:
        u, v = a[key], b[key]
        if u.dtype == torch.bfloat16:
            u, v = u.view(torch.int16), v.view(torch.int16)
        assert torch.equal(u, v), key
    assert int(a["totals"][0]) > 0          # drops happened: the capacity mattered
