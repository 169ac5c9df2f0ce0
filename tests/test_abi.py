"""The C-ABI library on the host: it loads, exports every entry point that
include/moe.h declares, and rejects bad arguments before touching the GPU
(none of these calls launches a kernel)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import routing_dispatch_expert_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(moe_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_entry_point():
    names = declared_functions()
    assert len(names) >= 12
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(moe.EXPORTS)


def test_status_strings():
    for s in (0, -1, -2, -3, -4):
        assert moe.status_string(s)
    assert moe.status_string(7) == "unknown status"


def test_stage_ran_host_only():
    # no layer call with events on this thread yet: nothing recorded
    assert [moe.moe_stage_ran(i) for i in range(len(moe.STAGES))] == [False] * len(moe.STAGES)
    for bad in (-1, len(moe.STAGES)):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_stage_ran(bad)
        assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    assert moe.lib().moe_stage_ran(0, None) == moe.MOE_ERR_INVALID_ARG


def test_capacity_host_only():
    assert [moe.moe_capacity(*a) for a in [(64, 8, 2, 1.25), (4096, 8, 2, 1.25), (8192, 256, 8, 1.25),
                                         (16384, 64, 6, 1.0), (64, 256, 8, 2.0)]] == [20, 1280, 320, 1536, 4]
    assert moe.moe_capacity(0, 8, 2, 1.0) == 0
    assert moe.moe_capacity(1, 1000, 1, 1.0) == 1
    for bad in [(-1, 8, 2, 1.0), (8, 0, 2, 1.0), (8, 8, 0, 1.0), (8, 8, 2, 0.0), (8, 8, 2, -1.0),
                (8, 8, 2, float("nan")), (8, 8, 2, float("inf"))]:
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_capacity(*bad)
        assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    assert moe.lib().moe_capacity(8, 8, 2, 1.0, None) == moe.MOE_ERR_INVALID_ARG


def test_capacity_matches_oracle_on_a_grid():
    import oracle
    for T in (0, 1, 5, 63, 64, 1000, 4096, 16384):
        for E in (1, 3, 8, 64, 256):
            for k in (1, 2, 6, 8):
                for cf in (0.1, 0.3, 1.0, 1.25, 1.3, 2.0):
                    assert moe.moe_capacity(T, E, k, cf) == oracle.capacity(T, E, k, cf)


def test_workspace_size_grows_with_shape():
    a = moe.moe_workspace_size(4096, 4096, 14336, 8, 2, 1.25, 1, "bf16")
    b = moe.moe_workspace_size(8192, 4096, 14336, 8, 2, 1.25, 1, "bf16")
    assert 0 < a < b
    # buckets, h and y of E*C rows dominate: E*C*(2d + d_ff)*2 bytes
    assert a >= 8 * 1280 * (2 * 4096 + 14336) * 2


FAKE = 1 << 40   # a non-NULL address that is never dereferenced: every call below fails validation first


def _layer(**kw):
    a = dict(x=FAKE, W_router=FAKE, router_bias=None, W_gate=FAKE, W_up=FAKE, W_down=FAKE, T=64, d=128, d_ff=256,
             E=8, k=2, cf=1.25, P=1, max_ranks=0, dtype="bf16", out=FAKE * 2, stats=None, workspace=FAKE * 3,
             workspace_bytes=1 << 40, stream=None)
    a.update(kw)
    return moe.moe_layer_forward(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), moe.MOE_ERR_INVALID_ARG), (dict(k=9), moe.MOE_ERR_INVALID_ARG),
    (dict(E=0), moe.MOE_ERR_INVALID_ARG), (dict(T=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(cf=0.0), moe.MOE_ERR_INVALID_ARG), (dict(cf=float("nan")), moe.MOE_ERR_INVALID_ARG),
    (dict(P=3), moe.MOE_ERR_INVALID_ARG), (dict(P=0), moe.MOE_ERR_INVALID_ARG),
    (dict(d=0), moe.MOE_ERR_INVALID_ARG), (dict(dtype=5), moe.MOE_ERR_INVALID_ARG),
    (dict(x=None), moe.MOE_ERR_INVALID_ARG), (dict(W_down=None), moe.MOE_ERR_INVALID_ARG),
    (dict(out=None), moe.MOE_ERR_INVALID_ARG), (dict(out=FAKE + 64), moe.MOE_ERR_INVALID_ARG),
    (dict(d=12), moe.MOE_ERR_UNSUPPORTED), (dict(d_ff=100), moe.MOE_ERR_UNSUPPORTED),
    (dict(E=5000, k=2), moe.MOE_ERR_UNSUPPORTED), (dict(E=64, k=33), moe.MOE_ERR_UNSUPPORTED),
    (dict(T=1 << 30, k=2), moe.MOE_ERR_UNSUPPORTED),
    (dict(workspace=None), moe.MOE_ERR_WORKSPACE), (dict(workspace_bytes=100), moe.MOE_ERR_WORKSPACE),
    (dict(workspace=FAKE * 3 + 8), moe.MOE_ERR_WORKSPACE),
    (dict(max_ranks=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(E=8, k=4, P=4, max_ranks=1), moe.MOE_ERR_INVALID_ARG),         # one rank holds 2 < k experts
    (dict(E=256, k=8, P=128, max_ranks=4), moe.MOE_ERR_UNSUPPORTED),     # limit needs P <= 64
])
def test_layer_rejects_bad_arguments_before_any_gpu_call(kw, status):
    with pytest.raises(moe.MoeError) as ei:
        _layer(**kw)
    assert ei.value.status == status
    assert moe.moe_last_error()


def _backward_saved(saved):
    moe.moe_layer_backward_saved(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 64, 128, 256, 8, 2, 1.25, 1, 0, "bf16",
                                 saved, FAKE * 2, FAKE * 3, None, FAKE * 4, FAKE * 5, FAKE * 6, FAKE * 7, 1 << 40)


def test_saved_backward_needs_the_kept_state():
    full = {name: FAKE for name in ("topk_idx", "topk_w", "buckets", "g", "u", "h")}
    for missing in [None] + sorted(full):
        saved = None if missing is None else {k: v for k, v in full.items() if k != missing}
        with pytest.raises(moe.MoeError) as ei:
            _backward_saved(saved)
        assert ei.value.status == moe.MOE_ERR_INVALID_ARG, missing
        assert moe.moe_last_error()


def test_zero_tokens_returns_ok_without_launching():
    _layer(T=0, workspace=None, workspace_bytes=0)
    moe.moe_route(FAKE, 0, 8, 2, 1, 0, FAKE, FAKE)
    moe.moe_router(FAKE, FAKE, None, 0, 128, 8, 2, 1, 0, "bf16", FAKE, FAKE, None, None, 0)
    assert moe.moe_router_workspace_size(64, 7168, 256, "bf16") >= 64 * 256 * 4
    moe.moe_permute(FAKE, FAKE, 0, 128, 8, 2, 20, 1, "bf16", FAKE, FAKE, None, FAKE, FAKE, None, None, None, 0)
    moe.moe_permute_static(FAKE, FAKE, 0, 128, 8, 2, 20, 1, "bf16", FAKE, FAKE, None, FAKE, FAKE, None, None)
    moe.moe_combine(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 128, 8, 2, 20, "bf16", FAKE * 2)


@pytest.mark.parametrize("call", [
    lambda: moe.moe_route(None, 4, 8, 2, 1, 0, FAKE, FAKE),
    lambda: moe.moe_route(FAKE, 4, 8, 9, 1, 0, FAKE, FAKE),
    lambda: moe.moe_route(FAKE, 4, 8, 2, 3, 0, FAKE, FAKE),
    lambda: moe.moe_route(FAKE, 4, 8, 4, 4, 1, FAKE, FAKE),
    lambda: moe.moe_route(FAKE, 4, 8, 2, 2, -1, FAKE, FAKE),
    lambda: moe.moe_router(FAKE, FAKE, None, 4, 128, 8, 4, 4, 1, "bf16", FAKE, FAKE, None, None, 0),
    lambda: moe.moe_router(FAKE, FAKE, None, 4, 12, 8, 2, 1, 0, "bf16", FAKE, FAKE, None, None, 0),
    lambda: moe.moe_router(FAKE, FAKE, None, 4, 128, 8, 2, 1, 0, "bf16", FAKE, FAKE, None, None, 0),
    lambda: moe.moe_permute(FAKE, FAKE, 4, 128, 8, 2, 0, 1, "bf16", FAKE, FAKE, None, FAKE, FAKE, None, None,
                            FAKE * 3, 1 << 30),
    lambda: moe.moe_permute(FAKE, FAKE, 4, 128, 8, 2, 4, 3, "bf16", FAKE, FAKE, None, FAKE, FAKE, None, None,
                            FAKE * 3, 1 << 30),
    lambda: moe.moe_permute(FAKE, FAKE, 4, 128, 8, 2, 4, 1, "bf16", FAKE, FAKE, None, FAKE, FAKE, None, None,
                            None, 0),
    lambda: moe.moe_permute_static(FAKE, FAKE, 4, 128, 8, 2, 0, 1, "bf16", FAKE, FAKE, None, FAKE, FAKE, None, None),
    lambda: moe.moe_permute_static(FAKE, FAKE, 4, 128, 8, 2, 4, 3, "bf16", FAKE, FAKE, None, FAKE, FAKE, None, None),
    lambda: moe.moe_permute_static(FAKE, None, 4, 128, 8, 2, 4, 1, "bf16", FAKE, FAKE, None, FAKE, FAKE, None, None),
    lambda: moe.moe_grouped_gemm(FAKE, FAKE, FAKE, FAKE, None, 8, 20, 128, 256, "bf16", FAKE, FAKE, FAKE * 3, 1 << 30),
    lambda: moe.moe_grouped_gemm(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 20, 128, 256, "bf16", FAKE, FAKE, None, 0),
    lambda: moe.moe_combine(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 128, 8, 2, 20, "bf16", FAKE),
    lambda: moe.moe_combine(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 100, 8, 2, 20, "bf16", FAKE * 2),
])
def test_stage_entry_points_reject_bad_arguments(call):
    with pytest.raises(moe.MoeError):
        call()


def test_library_has_no_torch_dependency():
    # the C ABI takes plain pointers: the library links no torch or python library
    import subprocess
    out = subprocess.run(["ldd", moe.LIB_PATH], capture_output=True, text=True).stdout
    assert "torch" not in out and "python" not in out
    assert isinstance(moe.lib(), ctypes.CDLL)


def test_replica_plan_matches_the_oracle():
    rng = np.random.default_rng(41)
    for _ in range(50):
        E = int(rng.integers(1, 70))
        routed = rng.integers(0, 5000, size=E).astype(np.int32)
        extra = int(rng.integers(0, 40))
        assert np.array_equal(moe.moe_replica_plan(routed, extra), oracle.replica_plan(routed, extra))


@pytest.mark.parametrize("R", [7, 4097])
def test_replicated_layer_rejects_bad_instance_counts(R):
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward_replicated(FAKE, FAKE, None, FAKE, FAKE, FAKE, 64, 128, 256, 8, 2, 1.25, 1, 0, FAKE, R,
                                         "bf16", FAKE * 2, None, FAKE * 3, 1 << 40)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError):
        moe.moe_layer_forward_replicated(FAKE, FAKE, None, FAKE, FAKE, FAKE, 64, 128, 256, 8, 2, 1.25, 1, 0, None, 8,
                                         "bf16", FAKE * 2, None, FAKE * 3, 1 << 40)


def test_static_permute_rejects_sizes_beyond_its_buffer_before_any_gpu_call():
    # 65536 tokens x 4096 experts need 2 x 1024 x 4096 x 4 bytes of scratch (32 MiB)
    assert moe.moe_permute_workspace_size(65536, 4096) > 16 << 20
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_permute_static(FAKE, FAKE, 65536, 128, 4096, 1, 16, 1, "bf16", FAKE, FAKE, None, FAKE, FAKE, None,
                               None)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    assert "static buffer" in moe.moe_last_error()
