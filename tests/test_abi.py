"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call
(so these run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_perm.h")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN = 0, 1, 2, 3
MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE = 4, 5

FAKE = 0x7F0000000000           # a 256-byte aligned address never dereferenced
MIS = FAKE + 2                  # 2-byte aligned, not 4-byte aligned


def _declared():
    src = open(HEADER).read()
    return re.findall(r"MOE_PERM_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", src)


@pytest.fixture(scope="module")
def lib():
    import unpermute_moe_make_amd as m
    return m._binding._lib


def test_header_symbols_exported(lib):
    names = _declared()
    assert len(names) == 21
    dyn = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in dyn.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n), n
    import unpermute_moe_make_amd as m
    assert set(names) == set(m.EXPORTED)


def test_status_strings(lib):
    for code in range(7):
        s = lib.moe_status_string(code)
        assert s and s != b"unknown status"
    assert lib.moe_status_string(99) == b"unknown status"


def test_workspace_query(lib):
    ws = lib.moe_make_row_id_map_workspace_bytes(4096, 6, 64)
    nb = 16
    assert ws >= nb * 4 * 64 * 8 + nb * 64 * 4
    assert lib.moe_make_row_id_map_workspace_bytes(-1, 6, 64) == 0


def test_row_map_host_errors(lib):
    f = lib.moe_make_row_id_map
    P = ctypes.c_void_p
    # shape errors
    assert f(P(FAKE), 16, 0, 32, P(FAKE), P(FAKE), None, P(FAKE), 1 << 20, None) == MOE_ERR_SHAPE
    assert f(P(FAKE), 16, 5, 4, P(FAKE), P(FAKE), None, P(FAKE), 1 << 20, None) == MOE_ERR_SHAPE
    assert f(P(FAKE), 16, 65, 100, P(FAKE), P(FAKE), None, P(FAKE), 1 << 20,
             None) == MOE_ERR_UNSUPPORTED
    assert f(P(FAKE), 16, 4, 4096, P(FAKE), P(FAKE), None, P(FAKE), 1 << 30,
             None) == MOE_ERR_UNSUPPORTED
    # null pointers
    assert f(None, 16, 4, 32, P(FAKE), P(FAKE), None, P(FAKE), 1 << 20, None) == MOE_ERR_NULL
    assert f(P(FAKE), 16, 4, 32, P(FAKE), None, None, P(FAKE), 1 << 20, None) == MOE_ERR_NULL
    # workspace too small / missing / misaligned
    need = lib.moe_make_row_id_map_workspace_bytes(16, 4, 32)
    assert f(P(FAKE), 16, 4, 32, P(FAKE), P(FAKE), None, P(FAKE), need - 1,
             None) == MOE_ERR_WORKSPACE
    assert f(P(FAKE), 16, 4, 32, P(FAKE), P(FAKE), None, None, need, None) == MOE_ERR_WORKSPACE
    assert f(P(FAKE), 16, 4, 32, P(FAKE), P(FAKE), None, P(FAKE + 16), need,
             None) == MOE_ERR_ALIGN
    assert f(P(MIS), 16, 4, 32, P(FAKE), P(FAKE), None, P(FAKE), need, None) == MOE_ERR_ALIGN


def test_permute_family_host_errors(lib):
    P = ctypes.c_void_p
    # moe_permute(x, probs, idx, map, T, H, k, E, n_out, out, out_probs, st, stream)
    f = lib.moe_permute
    assert f(P(FAKE), None, P(FAKE), P(FAKE), 16, 64, 4, 32, 63, P(FAKE), None, None,
             None) == MOE_ERR_SHAPE          # num_out_rows != T*k
    assert f(P(FAKE), None, P(FAKE), P(FAKE), 16, 0, 4, 32, 64, P(FAKE), None, None,
             None) == MOE_ERR_SHAPE
    assert f(None, None, P(FAKE), P(FAKE), 16, 64, 4, 32, 64, P(FAKE), None, None,
             None) == MOE_ERR_NULL
    assert f(P(FAKE), None, P(FAKE), P(FAKE), 16, 64, 4, 32, 64, P(FAKE), P(FAKE), None,
             None) == MOE_ERR_NULL           # out_probs without probs
    assert f(P(FAKE + 1), None, P(FAKE), P(FAKE), 16, 64, 4, 32, 64, P(FAKE), None, None,
             None) == MOE_ERR_ALIGN
    assert f(P(FAKE), None, P(MIS), P(FAKE), 16, 64, 4, 32, 64, P(FAKE), None, None,
             None) == MOE_ERR_ALIGN
    # moe_unpermute(in, probs, idx, map, T, H, k, E, n_in, out, st, stream)
    g = lib.moe_unpermute
    assert g(P(FAKE), None, P(FAKE), P(FAKE), 16, 64, 4, 32, 65, P(FAKE), None,
             None) == MOE_ERR_SHAPE
    assert g(P(FAKE), None, P(FAKE), None, 16, 64, 4, 32, 64, P(FAKE), None,
             None) == MOE_ERR_NULL
    assert g(P(FAKE), P(MIS), P(FAKE), P(FAKE), 16, 64, 4, 32, 64, P(FAKE), None,
             None) == MOE_ERR_ALIGN
    # moe_unpermute_bwd(d_out, fwd_in, probs, idx, map, T, H, k, E, n, d_in, d_probs, st, s)
    h = lib.moe_unpermute_bwd
    assert h(P(FAKE), None, P(FAKE), P(FAKE), P(FAKE), 16, 64, 4, 32, 64, P(FAKE), P(FAKE),
             None, None) == MOE_ERR_NULL     # prob grad needs fwd_in
    assert h(P(FAKE), P(FAKE), None, P(FAKE), P(FAKE), 16, 64, 4, 32, 64, P(FAKE), P(FAKE),
             None, None) == MOE_ERR_NULL     # prob grad needs probs
    # moe_permute_bwd(d_out, d_out_probs, idx, map, T, H, k, E, n, d_x, d_probs, st, s)
    q = lib.moe_permute_bwd
    assert q(P(FAKE), None, P(FAKE), P(FAKE), 16, 64, 4, 32, 64, P(FAKE), P(FAKE), None,
             None) == MOE_ERR_NULL
    assert q(P(FAKE), None, P(FAKE), P(FAKE), -1, 64, 4, 32, -4, P(FAKE), None, None,
             None) == MOE_ERR_SHAPE
    assert q(P(FAKE), None, P(FAKE), P(FAKE), 16, 64, 80, 100, 16 * 80, P(FAKE), None, None,
             None) == MOE_ERR_UNSUPPORTED
    # T == 0 is a valid no-op for the row kernels (no HIP call at all)
    assert f(None, None, None, None, 0, 64, 4, 32, 0, None, None, None, None) == MOE_OK
    assert g(None, None, None, None, 0, 64, 4, 32, 0, None, None, None) == MOE_OK


def test_chunk_host_errors(lib):
    P = ctypes.c_void_p
    f = lib.moe_sort_chunks_and_pad
    # (in, probs, eb, pb, n_cap, H, sizes, order, C, R, A, out_cap, out, out_probs,
    #  row_map, pad_off, st, stream)
    args = [P(FAKE), None, 2, 4, 100, 64, P(FAKE), P(FAKE), 128, 8, 128, 2048, P(FAKE), None,
            P(FAKE), P(FAKE), None, None]

    def call(**kw):
        a = list(args)
        names = ["in", "probs", "eb", "pb", "n_cap", "H", "sizes", "order", "C", "R", "A",
                 "out_cap", "out", "out_probs", "row_map", "pad_off", "st", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    assert call(C=130) == MOE_ERR_SHAPE                 # C % R != 0
    assert call(A=0) == MOE_ERR_SHAPE
    assert call(C=4096, R=8) == MOE_ERR_UNSUPPORTED
    assert call(eb=8) == MOE_ERR_UNSUPPORTED
    assert call(sizes=None) == MOE_ERR_NULL
    assert call(out_probs=P(FAKE)) == MOE_ERR_NULL
    assert call(out=P(FAKE + 2), eb=4) == MOE_ERR_ALIGN
    g = lib.moe_unpad_and_restore_chunks
    assert g(P(FAKE), None, 2, 4, P(FAKE), None, 128, 2048, 64, 100, P(FAKE), None, None,
             None) == MOE_ERR_NULL
    assert g(P(FAKE), None, 3, 4, P(FAKE), P(FAKE), 128, 2048, 64, 100, P(FAKE), None, None,
             None) == MOE_ERR_UNSUPPORTED
    h = lib.moe_unpad_and_restore_chunks_bwd
    assert h(P(FAKE), None, 2, 4, None, 2048, 64, 100, P(FAKE), None, None,
             None) == MOE_ERR_NULL


def test_binding_rejects_host_tensors():
    import torch
    import unpermute_moe_make_amd as m
    idx = torch.zeros(4, 2, dtype=torch.int32)
    with pytest.raises(ValueError):
        m.moe_make_row_id_map(idx, 8)
