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
    assert len(names) == 22
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


def test_row_map_noalloc_host_errors(lib):
    f = lib.moe_make_row_id_map_noalloc
    P = ctypes.c_void_p
    assert f(P(FAKE), 16, 0, 32, P(FAKE), P(FAKE), None, None) == MOE_ERR_SHAPE
    assert f(P(FAKE), 16, 65, 100, P(FAKE), P(FAKE), None, None) == MOE_ERR_UNSUPPORTED
    assert f(None, 16, 4, 32, P(FAKE), P(FAKE), None, None) == MOE_ERR_NULL
    assert f(P(FAKE), 16, 4, 32, P(FAKE), None, None, None) == MOE_ERR_NULL
    assert f(P(MIS), 16, 4, 32, P(FAKE), P(FAKE), None, None) == MOE_ERR_ALIGN
    # a routing whose scratch need exceeds the library's fixed array
    assert lib.moe_make_row_id_map_workspace_bytes(200000, 2, 512) > 8 << 20
    assert f(P(FAKE), 200000, 2, 512, P(FAKE), P(FAKE), None, None) == MOE_ERR_WORKSPACE


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
    assert call(out_probs=P(FAKE)) == MOE_ERR_NULL      # prob output with no probs (n_cap > 0)
    assert call(out=P(FAKE + 2), eb=4) == MOE_ERR_ALIGN
    g = lib.moe_unpad_and_restore_chunks
    assert g(P(FAKE), None, 2, 4, P(FAKE), None, 128, 2048, 64, 100, P(FAKE), None, None,
             None) == MOE_ERR_NULL
    assert g(P(FAKE), None, 3, 4, P(FAKE), P(FAKE), 128, 2048, 64, 100, P(FAKE), None, None,
             None) == MOE_ERR_UNSUPPORTED
    assert g(P(FAKE), None, 2, 4, P(FAKE), P(FAKE), 128, 2048, 64, 100, P(FAKE), P(FAKE), None,
             None) == MOE_ERR_NULL                   # out_probs without probs, out_cap > 0
    h = lib.moe_unpad_and_restore_chunks_bwd
    assert h(P(FAKE), None, 2, 4, None, 2048, 64, 100, P(FAKE), None, None,
             None) == MOE_ERR_NULL
    assert h(P(FAKE), None, 2, 4, P(FAKE), 2048, 64, 100, P(FAKE), P(FAKE), None,
             None) == MOE_ERR_NULL                   # d_in_probs without d_out_probs, n_cap > 0


def test_binding_rejects_host_tensors():
    import torch
    import unpermute_moe_make_amd as m
    idx = torch.zeros(4, 2, dtype=torch.int32)
    with pytest.raises(ValueError):
        m.moe_make_row_id_map(idx, 8)


def test_next_rows_host_errors(lib):
    P = ctypes.c_void_p
    # moe_unpermute_ep(in, probs, idx, map, T, H, k, E, n_in, ep, flags, out, st, stream)
    f = lib.moe_unpermute_ep
    assert f(P(FAKE), None, P(FAKE), P(FAKE), 16, 64, 4, 32, 64, 3, 1, P(FAKE), None,
             None) == MOE_ERR_SHAPE          # ep does not divide E
    assert f(P(FAKE), None, P(FAKE), P(FAKE), 16, 64, 4, 32, 64, 0, 1, P(FAKE), None,
             None) == MOE_ERR_SHAPE
    assert f(P(FAKE), None, P(FAKE), P(FAKE), 16, 64, 4, 32, 64, 4, 4, P(FAKE), None,
             None) == MOE_ERR_UNSUPPORTED    # unknown flag bit
    assert f(P(FAKE), None, P(FAKE), None, 16, 64, 4, 32, 64, 4, 1, P(FAKE), None,
             None) == MOE_ERR_NULL
    # moe_topk_softmax(logits, lb, T, E, k, idx, probs, pb, stream)
    r = lib.moe_topk_softmax
    assert r(P(FAKE), 4, 16, 8, 9, P(FAKE), P(FAKE), 4, None) == MOE_ERR_SHAPE      # k > E
    assert r(P(FAKE), 4, 16, 8, 0, P(FAKE), P(FAKE), 4, None) == MOE_ERR_SHAPE
    assert r(P(FAKE), 4, 16, 4096, 8, P(FAKE), P(FAKE), 4, None) == MOE_ERR_UNSUPPORTED
    assert r(P(FAKE), 4, 16, 128, 65, P(FAKE), P(FAKE), 4, None) == MOE_ERR_UNSUPPORTED
    assert r(P(FAKE), 3, 16, 8, 2, P(FAKE), P(FAKE), 4, None) == MOE_ERR_UNSUPPORTED
    assert r(P(FAKE), 4, 16, 8, 2, P(FAKE), P(FAKE), 8, None) == MOE_ERR_UNSUPPORTED
    assert r(None, 4, 16, 8, 2, P(FAKE), P(FAKE), 4, None) == MOE_ERR_NULL
    assert r(P(MIS), 4, 16, 8, 2, P(FAKE), P(FAKE), 4, None) == MOE_ERR_ALIGN
    assert r(None, 4, 0, 8, 2, None, None, 4, None) == MOE_OK                       # T == 0
    # moe_topk_softmax_bwd(dp, p, pb, idx, T, E, k, d_logits, lb, st, stream)
    rb = lib.moe_topk_softmax_bwd
    assert rb(P(FAKE), P(FAKE), 4, P(FAKE), 16, 8, 9, P(FAKE), 4, None, None) == MOE_ERR_SHAPE
    assert rb(P(FAKE), P(FAKE), 2, P(FAKE), 16, 8, 2, P(FAKE), 1, None,
              None) == MOE_ERR_UNSUPPORTED
    assert rb(P(FAKE), None, 4, P(FAKE), 16, 8, 2, P(FAKE), 4, None, None) == MOE_ERR_NULL
    # moe_make_mask_row_id_map(mask, mb, T, E, num_out, map, off, ws, ws_bytes, stream)
    g = lib.moe_make_mask_row_id_map
    need = lib.moe_make_mask_row_id_map_workspace_bytes(16, 8)
    assert need > 0 and lib.moe_make_mask_row_id_map_workspace_bytes(-1, 8) == 0
    assert g(P(FAKE), 2, 16, 8, -1, P(FAKE), P(FAKE), P(FAKE), need,
             None) == MOE_ERR_UNSUPPORTED    # 2-byte mask entries
    assert g(P(FAKE), 1, 16, 8, -2, P(FAKE), P(FAKE), P(FAKE), need, None) == MOE_ERR_SHAPE
    assert g(P(FAKE), 1, 16, 4096, -1, P(FAKE), P(FAKE), P(FAKE), need,
             None) == MOE_ERR_UNSUPPORTED
    assert g(None, 1, 16, 8, -1, P(FAKE), P(FAKE), P(FAKE), need, None) == MOE_ERR_NULL
    assert g(P(FAKE), 1, 16, 8, -1, P(FAKE), P(FAKE), P(FAKE), need - 1,
             None) == MOE_ERR_WORKSPACE
    assert g(P(FAKE), 4, 16, 8, -1, P(FAKE), P(FAKE), P(FAKE + 64), need,
             None) == MOE_ERR_ALIGN          # workspace not 256-byte aligned
    assert g(P(MIS), 4, 16, 8, -1, P(FAKE), P(FAKE), P(FAKE), need, None) == MOE_ERR_ALIGN
    # moe_permute_mask(x, probs, map, T, H, E, n_out, out, out_probs, st, stream)
    pm = lib.moe_permute_mask
    assert pm(P(FAKE), None, P(FAKE), 16, 0, 8, 10, P(FAKE), None, None, None) == MOE_ERR_SHAPE
    assert pm(P(FAKE), None, None, 16, 64, 8, 10, P(FAKE), None, None, None) == MOE_ERR_NULL
    assert pm(P(FAKE), None, P(FAKE), 16, 64, 8, 10, P(FAKE), P(FAKE), None,
              None) == MOE_ERR_NULL          # out_probs without probs
    # moe_unpermute_mask(in, mp, pp, map, T, H, E, n_in, out, up, st, stream)
    um = lib.moe_unpermute_mask
    assert um(P(FAKE), None, P(FAKE), P(FAKE), 16, 64, 8, 10, P(FAKE), None, None,
              None) == MOE_ERR_NULL          # permuted probs without their output
    assert um(P(FAKE), P(MIS), None, P(FAKE), 16, 64, 8, 10, P(FAKE), None, None,
              None) == MOE_ERR_ALIGN
    # moe_unpermute_mask_bwd(d_out, fwd_in, mp, map, T, H, E, n, d_in, dmp, st, stream)
    bm = lib.moe_unpermute_mask_bwd
    assert bm(P(FAKE), P(FAKE), None, P(FAKE), 16, 64, 8, 10, P(FAKE), None, None,
              None) == MOE_ERR_NULL          # merging probs are required
    assert bm(P(FAKE), None, P(FAKE), P(FAKE), 16, 64, 8, 10, P(FAKE), P(FAKE), None,
              None) == MOE_ERR_NULL          # prob grads need fwd_in
    # moe_permute_scaled(x, eb, scale, srb, probs, idx, map, T, H, k, E, n, out, out_s, out_p,
    #                    st, stream)
    ps = lib.moe_permute_scaled
    assert ps(P(FAKE), 8, None, 0, None, P(FAKE), P(FAKE), 16, 64, 4, 32, 64, P(FAKE), None,
              None, None, None) == MOE_ERR_UNSUPPORTED
    assert ps(P(FAKE), 1, P(FAKE), 16, None, P(FAKE), P(FAKE), 16, 64, 4, 32, 64, P(FAKE),
              None, None, None, None) == MOE_ERR_NULL       # scales without out_scale
    assert ps(P(FAKE), 1, P(FAKE), 0, None, P(FAKE), P(FAKE), 16, 64, 4, 32, 64, P(FAKE),
              P(FAKE), None, None, None) == MOE_ERR_SHAPE   # empty scale rows
    assert ps(P(FAKE + 1), 2, None, 0, None, P(FAKE), P(FAKE), 16, 64, 4, 32, 64, P(FAKE),
              None, None, None, None) == MOE_ERR_ALIGN
    # moe_permute_mask_scaled(x, eb, scale, srb, probs, map, T, H, E, n, out, out_s, out_p,
    #                         st, stream)
    pms = lib.moe_permute_mask_scaled
    assert pms(P(FAKE), 1, P(FAKE), 8, None, P(FAKE), 16, 64, 8, 10, P(FAKE), None, None, None,
               None) == MOE_ERR_NULL
    assert pms(None, 1, None, 0, None, None, 0, 64, 8, 0, None, None, None, None,
               None) == MOE_OK             # T == 0


def test_bench_names_the_kernels_the_library_launches():
    """bench.py names the kernels behind each op for its roofline entry; the
    sort-and-pad is one fused launch up to the library's padded-buffer limit,
    so the bench's copy of that limit must equal the library's default."""
    import bench
    src = open(os.path.join(ROOT, "unpermute_moe_make_amd", "csrc", "chunks.hip")).read()
    mt = re.search(r"#define MOE_FUSED_MAX_BYTES \((\d+)ll << (\d+)\)", src)
    assert mt, "fused sort-and-pad limit not found"
    assert bench.FUSED_PAD_MAX_BYTES == int(mt.group(1)) << int(mt.group(2))
    small = {"out_cap": 10240, "H": 2048}
    large = {"out_cap": 34816, "H": 2048}
    assert bench.op_kernels("sort_chunks_and_pad", small) == ["pad_fused_kernel"]
    assert bench.op_kernels("sort_chunks_and_pad", large) == ["chunk_map_kernel",
                                                              "pad_copy_kernel"]
    rsrc = open(os.path.join(ROOT, "unpermute_moe_make_amd", "csrc", "row_map.hip")).read()
    for name, val in (("MOE_SINGLE_MAX_ENTRIES", bench.ROWMAP_SINGLE_MAX_ENTRIES),
                      ("MOE_FUSED_MAX_BLOCKS", bench.ROWMAP_FUSED_MAX_BLOCKS)):
        mt = re.search(r"#define " + name + r" (\d+)", rsrc)
        assert mt and int(mt.group(1)) == val, name
    mt = re.search(r"constexpr int kSingleMaxExperts = (\d+);", rsrc)
    assert mt and int(mt.group(1)) == bench.ROWMAP_SINGLE_MAX_EXPERTS
    assert bench.op_kernels("row_map", {"T": 16, "k": 4, "E": 32}) == ["rowmap_single_kernel"]
    assert bench.op_kernels("row_map", {"T": 4096, "k": 6, "E": 64}) == [
        "rowmap_count_kernel", "rowmap_write_kernel"]


C_CALLER = r"""
#include <stdio.h>
#include "moe_perm.h"
int main(void) {
    /* host checks only: each call is rejected before any HIP call */
    int a = moe_permute(0, 0, 0, 0, 4, 64, 2, 8, 8, 0, 0, 0, 0);
    int b = moe_sort_chunks_and_pad(0, 0, 2, 4, 100, 64, 0, 0, 128, 8, 128, 2048, 0, 0, 0, 0,
                                    0, 0);
    size_t ws = moe_make_row_id_map_workspace_bytes(4096, 6, 64);
    printf("%d %d %zu %s\n", a, b, ws, moe_status_string(a));
    return !(a == MOE_ERR_NULL && b == MOE_ERR_NULL && ws > 0);
}
"""


def test_plain_c_caller(tmp_path):
    """The boundary is a C ABI: a C99 program built by gcc against the header
    links the library and gets its host-side answers (no GPU involved)."""
    src = tmp_path / "caller.c"
    src.write_text(C_CALLER)
    exe = tmp_path / "caller"
    libdir = os.path.join(ROOT, "unpermute_moe_make_amd")
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror",
                           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                           "-I", "/opt/rocm/include", str(src), "-L", libdir, "-lmoeperm",
                           "-Wl,-rpath," + libdir, "-o", str(exe)])
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.split()[:2] == [str(MOE_ERR_NULL), str(MOE_ERR_NULL)]
