"""The allocation-free row map (moe_make_row_id_map_noalloc) against the row
map with a caller workspace (moe_make_row_id_map), through the C ABI: bit for
bit on consecutive calls that share the library's scratch array -- a large
routing, then smaller ones, then launch shapes the others do not take -- and
the host-side limit of the scratch."""
import ctypes

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MOE_ERR_WORKSPACE = 5


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import unpermute_moe_make_amd as m
    return m._binding._lib


def P(t):
    return ctypes.c_void_p(None if t is None else t.data_ptr())


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def both(lib, idx, E):
    """(map, offsets, status) from the workspace call and the scratch call,
    outputs pre-filled with sentinels."""
    T, k = idx.shape
    out = []
    for noalloc in (False, True):
        rm = torch.full((E, T), -2, dtype=torch.int32, device=DEV)
        off = torch.full((E + 1,), -2, dtype=torch.int32, device=DEV)
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        if noalloc:
            rc = lib.moe_make_row_id_map_noalloc(P(idx), T, k, E, P(rm), P(off), P(st), stream())
        else:
            n = lib.moe_make_row_id_map_workspace_bytes(T, k, E)
            ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
            rc = lib.moe_make_row_id_map(P(idx), T, k, E, P(rm), P(off), P(st), P(ws), n,
                                         stream())
        assert rc == 0, (noalloc, rc)
        torch.cuda.synchronize()
        out.append((rm.cpu().numpy(), off.cpu().numpy(), int(st.item())))
    return out


def check(lib, idx, E, what):
    (rm0, off0, st0), (rm1, off1, st1) = both(lib, idx, E)
    assert np.array_equal(rm0, rm1), f"{what}: row_id_map differs"
    assert np.array_equal(off0, off1), f"{what}: expert_offsets differ"
    assert st0 == st1, f"{what}: status {st0} vs {st1}"
    return st1


def test_noalloc_row_map_matches_workspace_call(lib):
    # the skewed layer, then a smaller routing through the same scratch
    for name in ("skewed", "finegrain", "tiny"):
        w = workloads.ROUTED[name]()
        say(f"noalloc row map {name} T={w.T} k={w.k} E={w.num_experts}")
        assert check(lib, w.topk_idx.to(DEV), w.num_experts, name) == 0
    # past 64 token blocks (column-scan launch), then the one-launch shape
    for T, E, k, seed in ((40000, 128, 4, 31), (500, 64, 8, 32), (3, 5, 2, 33)):
        w = workloads.random_routed(T, 8, E, k, seed=seed, with_dy=False)
        say(f"noalloc row map T={T} E={E} k={k}")
        assert check(lib, w.topk_idx.to(DEV), E, f"T={T}") == 0


def test_noalloc_row_map_bad_routing(lib):
    w = workloads.random_routed(5000, 8, 16, 3, seed=34, with_dy=False)
    idx = w.topk_idx.clone()
    idx[5, 1] = idx[5, 0]          # a repeated expert
    idx[9, 2] = 16                 # an expert out of range
    say("noalloc row map with bad routing")
    st = check(lib, idx.to(DEV), 16, "bad routing")
    assert st & 0x1 and st & 0x2


def test_noalloc_row_map_limits(lib):
    # a routing whose scratch need exceeds the fixed array is refused on the
    # host (no launch); zero tokens still writes the zero offsets
    T, k, E = 200000, 2, 512
    assert lib.moe_make_row_id_map_workspace_bytes(T, k, E) > (8 << 20)
    fake = ctypes.c_void_p(1 << 20)
    assert lib.moe_make_row_id_map_noalloc(fake, T, k, E, fake, fake, None,
                                           None) == MOE_ERR_WORKSPACE
    off = torch.full((9,), -2, dtype=torch.int32, device=DEV)
    assert lib.moe_make_row_id_map_noalloc(None, 0, 2, 8, None, P(off), None, stream()) == 0
    torch.cuda.synchronize()
    assert bool((off == 0).all())
