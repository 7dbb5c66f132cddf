"""CPU oracle for the MoE permute / unpermute path (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import this package.  The product package never
imports it, and it imports nothing from the product package.

The arithmetic lives in ``moe_oracle.c`` (plain scalar C, built with gcc
``-O2 -ffp-contract=off``); this module only builds it, loads it with
``ctypes`` and marshals numpy arrays.  bf16 tensors are passed as their
16-bit patterns in ``uint16`` arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

STATUS = {
    0: "ok",
    1: "expert index out of range",
    2: "duplicate expert in a token's routing",
    3: "bad size argument",
    4: "map entry out of range",
    5: "bad chunk sizes or chunk order",
    6: "capacity overflow",
    7: "out of host memory",
    8: "pair list not in token order",
}


class OracleError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: oracle status {code} ({STATUS.get(code, '?')})")
        self.code = code


def build(force: bool = True) -> str:
    """Compile moe_oracle.c into liboracle.so next to it."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
            "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm",
        ])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L = ctypes.c_int64
        sigs = {
            "oracle_row_id_map_pairs": [P, P, L, I, I, P, P],
            "oracle_row_id_map": [P, I, I, I, P, P],
            "oracle_permute": [P, P, P, P, I, I, I, I, P, P],
            "oracle_unpermute": [P, P, P, P, I, I, I, I, L, P],
            "oracle_unpermute_bwd": [P, P, P, P, P, I, I, I, I, L, P, P],
            "oracle_permute_bwd": [P, P, P, P, I, I, I, I, L, P, P],
            "oracle_unpermute_ep": [P, P, P, P, I, I, I, I, L, I, I, I, P],
            "oracle_topk_softmax": [P, I, I, I, I, P, P, I],
            "oracle_topk_softmax_bwd": [P, P, I, P, I, I, I, P, I],
            "oracle_mask_row_id_map": [P, I, I, I, I, P, P],
            "oracle_permute_scaled": [P, L, P, L, P, P, P, I, I, I, L, P, P, P],
            "oracle_mask_permute_scaled": [P, L, P, L, P, P, I, I, I, P, P, P],
            "oracle_mask_permute": [P, P, P, I, I, I, I, P, P],
            "oracle_mask_unpermute": [P, P, P, P, I, I, I, I, P, P],
            "oracle_mask_unpermute_bwd": [P, P, P, P, I, I, I, I, P, P],
            "oracle_chunk_map": [P, P, I, I, I, I, I, P, P],
            "oracle_sort_chunks_and_pad": [P, P, I, I, I, I, P, P, I, I, I, I, P, P, P, P],
            "oracle_unpad_and_restore_chunks": [P, P, I, I, P, P, I, I, I, I, P, P],
            "oracle_sort_chunks_and_pad_bwd": [P, P, I, I, P, P, I, I, I, I, P, P],
            "oracle_unpad_and_restore_chunks_bwd": [P, P, I, I, P, I, I, I, P, P],
        }
        for name, args in sigs.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
        lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f32.restype = ctypes.c_float
        lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
        lib.oracle_fmaf.argtypes = [ctypes.c_float] * 3
        lib.oracle_fmaf.restype = ctypes.c_float
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _arr(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(code, where):
    if code != 0:
        raise OracleError(code, where)


# ---- threads -------------------------------------------------------------

def set_threads(n: int) -> int:
    """Threads of the per-token loops (n < 1 leaves the setting); returns the
    number the next such loop uses.  Results do not depend on it."""
    return int(_load().oracle_set_threads(n))


def threads() -> int:
    return set_threads(0)


# ---- scalar helpers ------------------------------------------------------

def f32_to_bf16(x: float) -> int:
    return int(_load().oracle_f32_to_bf16(x))


def f64_to_bf16(x: float) -> int:
    return int(_load().oracle_f64_to_bf16(x))


def bf16_to_f32(b: int) -> float:
    return float(_load().oracle_bf16_to_f32(b))


def fmaf(a: float, b: float, c: float) -> float:
    return float(_load().oracle_fmaf(a, b, c))


# ---- (1) row map ------------------------------------------------------------

def row_id_map(topk_idx: np.ndarray, num_experts: int):
    """Returns (row_id_map[E][T] int32, expert_offsets[E+1] int32)."""
    idx = _arr(topk_idx, np.int32)
    T, k = idx.shape
    m = np.empty((num_experts, T), np.int32)
    off = np.empty(num_experts + 1, np.int32)
    _check(_load().oracle_row_id_map(_p(idx), T, k, num_experts, _p(m), _p(off)), "row_id_map")
    return m, off


def row_id_map_pairs(pair_token, pair_expert, num_tokens: int, num_experts: int):
    """Row map from an explicit (token, expert) pair list in token order."""
    pt = _arr(pair_token, np.int32)
    pe = _arr(pair_expert, np.int32)
    m = np.empty((num_experts, num_tokens), np.int32)
    off = np.empty(num_experts + 1, np.int32)
    _check(_load().oracle_row_id_map_pairs(_p(pt), _p(pe), pt.size, num_tokens, num_experts,
                                           _p(m), _p(off)), "row_id_map_pairs")
    return m, off


# ---- (2) permute / (4) unpermute and their backwards ------------------------

def permute(x, probs, topk_idx, row_map, num_out_rows=None):
    x = _arr(x, np.uint16)
    idx = _arr(topk_idx, np.int32)
    rm = _arr(row_map, np.int32)
    probs = _arr(probs, np.float32)
    T, H = x.shape
    k = idx.shape[1]
    E = rm.shape[0]
    n = T * k if num_out_rows is None else num_out_rows
    out = np.zeros((n, H), np.uint16)
    out_probs = None if probs is None else np.zeros(n, np.float32)
    _check(_load().oracle_permute(_p(x), _p(probs), _p(idx), _p(rm), T, H, k, E, _p(out),
                                  _p(out_probs)), "permute")
    return out, out_probs


def unpermute(inp, probs, topk_idx, row_map):
    inp = _arr(inp, np.uint16)
    idx = _arr(topk_idx, np.int32)
    rm = _arr(row_map, np.int32)
    probs = _arr(probs, np.float32)
    T, k = idx.shape
    E = rm.shape[0]
    H = inp.shape[1]
    out = np.zeros((T, H), np.uint16)
    _check(_load().oracle_unpermute(_p(inp), _p(probs), _p(idx), _p(rm), T, H, k, E,
                                    inp.shape[0], _p(out)), "unpermute")
    return out


def unpermute_ep(inp, probs, topk_idx, row_map, ep_size, bf16_partials=True, fp64_cross=False):
    """EP rank-ordered combine: experts split into ep_size equal ranges."""
    inp = _arr(inp, np.uint16)
    idx = _arr(topk_idx, np.int32)
    rm = _arr(row_map, np.int32)
    probs = _arr(probs, np.float32)
    T, k = idx.shape
    E = rm.shape[0]
    H = inp.shape[1]
    out = np.zeros((T, H), np.uint16)
    _check(_load().oracle_unpermute_ep(_p(inp), _p(probs), _p(idx), _p(rm), T, H, k, E,
                                       inp.shape[0], ep_size, int(bf16_partials),
                                       int(fp64_cross), _p(out)), "unpermute_ep")
    return out


def unpermute_bwd(d_out, fwd_in, probs, topk_idx, row_map, num_rows=None):
    d_out = _arr(d_out, np.uint16)
    fwd_in = _arr(fwd_in, np.uint16)
    idx = _arr(topk_idx, np.int32)
    rm = _arr(row_map, np.int32)
    probs = _arr(probs, np.float32)
    T, H = d_out.shape
    k = idx.shape[1]
    E = rm.shape[0]
    n = T * k if num_rows is None else num_rows
    d_in = np.zeros((n, H), np.uint16)
    d_probs = None if (probs is None or fwd_in is None) else np.zeros((T, k), np.float32)
    _check(_load().oracle_unpermute_bwd(_p(d_out), _p(fwd_in), _p(probs), _p(idx), _p(rm), T, H,
                                        k, E, n, _p(d_in), _p(d_probs)), "unpermute_bwd")
    return d_in, d_probs


def permute_bwd(d_out, d_out_probs, topk_idx, row_map):
    d_out = _arr(d_out, np.uint16)
    d_out_probs = _arr(d_out_probs, np.float32)
    idx = _arr(topk_idx, np.int32)
    rm = _arr(row_map, np.int32)
    T, k = idx.shape
    E = rm.shape[0]
    H = d_out.shape[1]
    d_x = np.zeros((T, H), np.uint16)
    d_probs = None if d_out_probs is None else np.zeros((T, k), np.float32)
    _check(_load().oracle_permute_bwd(_p(d_out), _p(d_out_probs), _p(idx), _p(rm), T, H, k, E,
                                      d_out.shape[0], _p(d_x), _p(d_probs)), "permute_bwd")
    return d_x, d_probs


# ---- router ---------------------------------------------------------------

def topk_softmax(logits, k, prob_bytes=4):
    """logits: [T][E] float32, or uint16 bf16 bits.  Returns (idx int32, weights):
    weights fp32, or bf16 bit patterns (uint16) when prob_bytes is 2."""
    logits = np.ascontiguousarray(logits)
    T, E = logits.shape
    eb = logits.dtype.itemsize
    idx = np.empty((T, k), np.int32)
    probs = np.empty((T, k), np.float32 if prob_bytes == 4 else np.uint16)
    _check(_load().oracle_topk_softmax(_p(logits), eb, T, E, k, _p(idx), _p(probs), prob_bytes),
           "topk_softmax")
    return idx, probs


def topk_softmax_bwd(d_probs, probs, topk_idx, num_experts, logit_bytes=4):
    """d_probs, probs: [T][k] fp32, or both uint16 bf16 bits.  Returns d_logits
    [T][E]: fp32, or bf16 bit patterns when logit_bytes is 2."""
    probs = np.ascontiguousarray(probs)
    pb = probs.dtype.itemsize
    d_probs = _arr(d_probs, probs.dtype)
    idx = _arr(topk_idx, np.int32)
    T, k = idx.shape
    out = np.empty((T, num_experts), np.float32 if logit_bytes == 4 else np.uint16)
    _check(_load().oracle_topk_softmax_bwd(_p(d_probs), _p(probs), pb, _p(idx), T, num_experts,
                                           k, _p(out), logit_bytes), "topk_softmax_bwd")
    return out


# ---- TE mask-map interop ------------------------------------------------------

def mask_row_id_map(routing_map, num_out=-1):
    """routing_map: [T][E] uint8/bool or int32 mask.  Returns (map [T][2E+1]
    int32, expert_offsets [E+1] int32); rows at or past num_out are dropped."""
    rm = np.ascontiguousarray(routing_map)
    if rm.dtype == np.bool_:
        rm = rm.view(np.uint8)
    if rm.dtype not in (np.uint8, np.int8, np.int32):
        rm = rm.astype(np.int32)
    T, E = rm.shape
    m = np.empty((T, 2 * E + 1), np.int32)
    off = np.empty(E + 1, np.int32)
    _check(_load().oracle_mask_row_id_map(_p(rm), rm.dtype.itemsize, T, E, num_out, _p(m),
                                          _p(off)), "mask_row_id_map")
    return m, off


def mask_permute(x, probs, row_map, n_rows, out=None):
    """x: [T][H] bf16 bits; probs: [T][E] fp32 or None.  Returns (out, out_probs):
    rows no map entry names keep the values of `out` (zeros by default)."""
    x = _arr(x, np.uint16)
    rm = _arr(row_map, np.int32)
    probs = _arr(probs, np.float32)
    T, H = x.shape
    E = (rm.shape[1] - 1) // 2
    out = np.zeros((n_rows, H), np.uint16) if out is None else np.array(out, np.uint16)
    out_probs = None if probs is None else np.zeros(n_rows, np.float32)
    _check(_load().oracle_mask_permute(_p(x), _p(probs), _p(rm), T, H, E, n_rows, _p(out),
                                       _p(out_probs)), "mask_permute")
    return out, out_probs


def mask_unpermute(inp, merging_probs, row_map, permuted_probs=None):
    """Returns (out [T][H] bf16 bits, unpermuted_probs [T][E] or None)."""
    inp = _arr(inp, np.uint16)
    rm = _arr(row_map, np.int32)
    mp = _arr(merging_probs, np.float32)
    pp = _arr(permuted_probs, np.float32)
    n_rows, H = inp.shape
    T = rm.shape[0]
    E = (rm.shape[1] - 1) // 2
    out = np.empty((T, H), np.uint16)
    up = None if pp is None else np.empty((T, E), np.float32)
    _check(_load().oracle_mask_unpermute(_p(inp), _p(mp), _p(pp), _p(rm), T, H, E, n_rows,
                                         _p(out), _p(up)), "mask_unpermute")
    return out, up


def mask_unpermute_bwd(d_out, fwd_in, merging_probs, row_map, d_in=None):
    """Returns (d_in [n_rows][H] bf16 bits, d_merging_probs [T][E] fp32)."""
    d_out = _arr(d_out, np.uint16)
    fwd_in = _arr(fwd_in, np.uint16)
    mp = _arr(merging_probs, np.float32)
    rm = _arr(row_map, np.int32)
    n_rows, H = fwd_in.shape
    T = rm.shape[0]
    E = (rm.shape[1] - 1) // 2
    d_in = np.zeros((n_rows, H), np.uint16) if d_in is None else np.array(d_in, np.uint16)
    dmp = np.empty((T, E), np.float32)
    _check(_load().oracle_mask_unpermute_bwd(_p(d_out), _p(fwd_in), _p(mp), _p(rm), T, H, E,
                                             n_rows, _p(d_in), _p(dmp)), "mask_unpermute_bwd")
    return d_in, dmp


# ---- quantized rows ----------------------------------------------------------

def _byte_rows(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint8).reshape(a.shape[0], -1)


def permute_scaled(x, scale, probs, topk_idx, row_map, n_rows=None):
    """x: [T][...] rows of any dtype (copied as bytes); scale: [T][...] or None.
    Returns (out bytes [n_rows][row_bytes], out_scale bytes or None, out_probs)."""
    xb = _byte_rows(x)
    T, rb = xb.shape
    sb = None if scale is None else _byte_rows(scale)
    srb = 0 if sb is None else sb.shape[1]
    idx = _arr(topk_idx, np.int32)
    rm = _arr(row_map, np.int32)
    probs = _arr(probs, np.float32)
    k = idx.shape[1]
    E = rm.shape[0]
    n = T * k if n_rows is None else n_rows
    out = np.zeros((n, rb), np.uint8)
    out_s = None if sb is None else np.zeros((n, srb), np.uint8)
    out_p = None if probs is None else np.zeros(n, np.float32)
    _check(_load().oracle_permute_scaled(_p(xb), rb, _p(sb), srb, _p(probs), _p(idx), _p(rm),
                                         T, k, E, n, _p(out), _p(out_s), _p(out_p)),
           "permute_scaled")
    return out, out_s, out_p


def mask_permute_scaled(x, scale, probs, row_map, n_rows, out=None, out_scale=None):
    """Mask-map form of permute_scaled; rows no map entry names keep `out` /
    `out_scale` (zeros by default)."""
    xb = _byte_rows(x)
    T, rb = xb.shape
    sb = None if scale is None else _byte_rows(scale)
    srb = 0 if sb is None else sb.shape[1]
    rm = _arr(row_map, np.int32)
    probs = _arr(probs, np.float32)
    E = (rm.shape[1] - 1) // 2
    out = np.zeros((n_rows, rb), np.uint8) if out is None else np.array(out, np.uint8)
    out_s = None if sb is None else (np.zeros((n_rows, srb), np.uint8) if out_scale is None
                                     else np.array(out_scale, np.uint8))
    out_p = None if probs is None else np.zeros(n_rows, np.float32)
    _check(_load().oracle_mask_permute_scaled(_p(xb), rb, _p(sb), srb, _p(probs), _p(rm), T, E,
                                              n_rows, _p(out), _p(out_s), _p(out_p)),
           "mask_permute_scaled")
    return out, out_s, out_p


# ---- (3) chunk sort-and-pad / unpad-and-restore ------------------------------

def chunk_map(split_sizes, sorted_idx, chunks_per_group, align, n_cap, out_cap):
    s = _arr(split_sizes, np.int32)
    q = _arr(sorted_idx, np.int32)
    C = s.size
    G = C // chunks_per_group
    row_map = np.empty(out_cap, np.int32)
    pad_off = np.empty(G + 1, np.int32)
    _check(_load().oracle_chunk_map(_p(s), _p(q), C, chunks_per_group, align, n_cap, out_cap,
                                    _p(row_map), _p(pad_off)), "chunk_map")
    return row_map, pad_off


def _ebytes(a):
    return a.dtype.itemsize


def sort_chunks_and_pad(inp, probs, split_sizes, sorted_idx, chunks_per_group, align, out_cap):
    """inp: [N_cap][H] array of 2- or 4-byte elements (copied bitwise)."""
    inp = np.ascontiguousarray(inp)
    s = _arr(split_sizes, np.int32)
    q = _arr(sorted_idx, np.int32)
    N_cap, H = inp.shape
    C = s.size
    G = C // chunks_per_group
    out = np.empty((out_cap, H), inp.dtype)
    pb = 4
    out_probs = None
    if probs is not None:
        probs = np.ascontiguousarray(probs)
        pb = _ebytes(probs)
        out_probs = np.empty(out_cap, probs.dtype)
    row_map = np.empty(out_cap, np.int32)
    pad_off = np.empty(G + 1, np.int32)
    _check(_load().oracle_sort_chunks_and_pad(
        _p(inp), _p(probs), _ebytes(inp), pb, N_cap, H, _p(s), _p(q), C, chunks_per_group, align,
        out_cap, _p(out), _p(out_probs), _p(row_map), _p(pad_off)), "sort_chunks_and_pad")
    return out, out_probs, row_map, pad_off


def unpad_and_restore_chunks(inp, probs, row_map, split_sizes, n_cap, with_status=False):
    """Restore padded rows to their source rows.  with_status: return
    (out, out_probs, status) instead of raising on a non-zero status (a map
    entry at or past the token total is dropped and reported as status 4, the
    rest of the output still defined)."""
    inp = np.ascontiguousarray(inp)
    rm = _arr(row_map, np.int32)
    s = _arr(split_sizes, np.int32)
    out_cap, H = inp.shape
    out = np.empty((n_cap, H), inp.dtype)
    pb = 4
    out_probs = None
    if probs is not None:
        probs = np.ascontiguousarray(probs)
        pb = _ebytes(probs)
        out_probs = np.empty(n_cap, probs.dtype)
    st = _load().oracle_unpad_and_restore_chunks(
        _p(inp), _p(probs), _ebytes(inp), pb, _p(rm), _p(s), s.size, out_cap, H, n_cap, _p(out),
        _p(out_probs))
    if with_status:
        return out, out_probs, st
    _check(st, "unpad_and_restore_chunks")
    return out, out_probs


def sort_chunks_and_pad_bwd(d_out, d_out_probs, row_map, split_sizes, n_cap,
                            with_status=False):
    d_out = np.ascontiguousarray(d_out)
    rm = _arr(row_map, np.int32)
    s = _arr(split_sizes, np.int32)
    out_cap, H = d_out.shape
    d_in = np.empty((n_cap, H), d_out.dtype)
    pb = 4
    d_in_probs = None
    if d_out_probs is not None:
        d_out_probs = np.ascontiguousarray(d_out_probs)
        pb = _ebytes(d_out_probs)
        d_in_probs = np.empty(n_cap, d_out_probs.dtype)
    st = _load().oracle_sort_chunks_and_pad_bwd(
        _p(d_out), _p(d_out_probs), _ebytes(d_out), pb, _p(rm), _p(s), s.size, out_cap, H, n_cap,
        _p(d_in), _p(d_in_probs))
    if with_status:
        return d_in, d_in_probs, st
    _check(st, "sort_chunks_and_pad_bwd")
    return d_in, d_in_probs


def unpad_and_restore_chunks_bwd(d_out, d_out_probs, row_map, out_cap):
    d_out = np.ascontiguousarray(d_out)
    rm = _arr(row_map, np.int32)
    N_cap, H = d_out.shape
    d_in = np.empty((out_cap, H), d_out.dtype)
    pb = 4
    d_in_probs = None
    if d_out_probs is not None:
        d_out_probs = np.ascontiguousarray(d_out_probs)
        pb = _ebytes(d_out_probs)
        d_in_probs = np.empty(out_cap, d_out_probs.dtype)
    _check(_load().oracle_unpad_and_restore_chunks_bwd(
        _p(d_out), _p(d_out_probs), _ebytes(d_out), pb, _p(rm), out_cap, H, N_cap, _p(d_in),
        _p(d_in_probs)), "unpad_and_restore_chunks_bwd")
    return d_in, d_in_probs
