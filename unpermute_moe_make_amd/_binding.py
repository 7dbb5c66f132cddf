"""Thin ctypes binding of libmoeperm.so (the C ABI in include/moe_perm.h).

Argument marshalling only: the functions check dtypes and shapes of torch
tensors, allocate missing outputs with ``torch.empty`` on the input's device,
pass raw device pointers plus the current torch stream, and turn a non-zero
status into :class:`MoeError`.  Every step of the computation runs in the HIP
kernels; there is no fallback path.  The library must have been built for
gfx950 (``python unpermute_moe_make_amd/build.py``); importing this module
without it raises ImportError.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch  # loads the HIP runtime the library binds to

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoeperm.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is missing: build the HIP library first "
        "(python unpermute_moe_make_amd/build.py)")

_lib = ctypes.CDLL(_LIB_PATH)

_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t

_SIGS = {
    "moe_status_string": ([_I], ctypes.c_char_p),
    "moe_make_row_id_map_workspace_bytes": ([_I, _I, _I], _Z),
    "moe_make_row_id_map": ([_P, _I, _I, _I, _P, _P, _P, _P, _Z, _P], _I),
    "moe_make_row_id_map_noalloc": ([_P, _I, _I, _I, _P, _P, _P, _P], _I),
    "moe_permute": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P], _I),
    "moe_unpermute": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P], _I),
    "moe_unpermute_ep": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P], _I),
    "moe_unpermute_bwd": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P], _I),
    "moe_permute_bwd": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P], _I),
    "moe_permute_scaled": ([_P, _I, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P],
                           _I),
    "moe_permute_mask_scaled": ([_P, _I, _P, _I, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P],
                                _I),
    "moe_make_mask_row_id_map_workspace_bytes": ([_I, _I], _Z),
    "moe_make_mask_row_id_map": ([_P, _I, _I, _I, _I, _P, _P, _P, _Z, _P], _I),
    "moe_permute_mask": ([_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P], _I),
    "moe_unpermute_mask": ([_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P], _I),
    "moe_unpermute_mask_bwd": ([_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P], _I),
    "moe_topk_softmax": ([_P, _I, _I, _I, _I, _P, _P, _I, _P], _I),
    "moe_topk_softmax_bwd": ([_P, _P, _I, _P, _I, _I, _I, _P, _I, _P, _P], _I),
    "moe_sort_chunks_and_pad": ([_P, _P, _I, _I, _I, _I, _P, _P, _I, _I, _I, _I, _P, _P, _P,
                                 _P, _P, _P], _I),
    "moe_unpad_and_restore_chunks": ([_P, _P, _I, _I, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P],
                                     _I),
    "moe_sort_chunks_and_pad_bwd": ([_P, _P, _I, _I, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P],
                                    _I),
    "moe_unpad_and_restore_chunks_bwd": ([_P, _P, _I, _I, _P, _I, _I, _I, _P, _P, _P, _P], _I),
}
for _name, (_args, _ret) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _ret

EXPORTED = tuple(_SIGS)

# Device status bits (include/moe_perm.h).
DEV_BAD_EXPERT = 0x1
DEV_DUP_EXPERT = 0x2
DEV_BAD_ROW = 0x4
DEV_BAD_CHUNKS = 0x8
DEV_OVERFLOW = 0x10

# moe_unpermute_ep flags (include/moe_perm.h).
EP_BF16_PARTIALS = 0x1
EP_FP64_CROSS = 0x2


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib.moe_status_string(status).decode()
        super().__init__(f"{where}: status {status} ({msg})")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def _check(status: int, where: str):
    if status != 0:
        raise MoeError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _need(t: torch.Tensor, name: str, dtype=None, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _opt(t, name, dtype=None, shape=None):
    return None if t is None else _need(t, name, dtype, shape)


def _bf16_like_2d(t: torch.Tensor, name: str):
    _need(t, name)
    if t.dim() != 2 or t.element_size() != 2:
        raise TypeError(f"{name} must be a 2-D tensor of 16-bit elements (bf16)")
    return t


def _status_arg(dev_status):
    return _opt(dev_status, "dev_status", torch.int32)


# ---------------------------------------------------------------------------
# (1) row map
# ---------------------------------------------------------------------------

def moe_make_row_id_map_workspace_bytes(num_tokens: int, topk: int, num_experts: int) -> int:
    return int(_lib.moe_make_row_id_map_workspace_bytes(num_tokens, topk, num_experts))


def moe_make_row_id_map(topk_idx: torch.Tensor, num_experts: int, *, row_id_map=None,
                        expert_offsets=None, dev_status=None, workspace=None,
                        stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Stable counting-sort row map: returns (row_id_map[E][T], expert_offsets[E+1])."""
    _need(topk_idx, "topk_idx", torch.int32)
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [num_tokens, topk]")
    T, k = topk_idx.shape
    dev = topk_idx.device
    row_id_map = (torch.empty((num_experts, T), dtype=torch.int32, device=dev)
                  if row_id_map is None else _need(row_id_map, "row_id_map", torch.int32,
                                                   (num_experts, T)))
    expert_offsets = (torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
                      if expert_offsets is None else
                      _need(expert_offsets, "expert_offsets", torch.int32, (num_experts + 1,)))
    need = moe_make_row_id_map_workspace_bytes(T, k, num_experts)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace")
    _check(_lib.moe_make_row_id_map(
        _ptr(topk_idx), T, k, num_experts, _ptr(row_id_map), _ptr(expert_offsets),
        _ptr(_status_arg(dev_status)), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)), "moe_make_row_id_map")
    return row_id_map, expert_offsets


def moe_make_row_id_map_noalloc(topk_idx: torch.Tensor, num_experts: int, *, row_id_map=None,
                                expert_offsets=None, dev_status=None,
                                stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The row map with the library's fixed device scratch instead of a
    workspace (the C call allocates nothing; given outputs are used as is)."""
    _need(topk_idx, "topk_idx", torch.int32)
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [num_tokens, topk]")
    T, k = topk_idx.shape
    dev = topk_idx.device
    row_id_map = (torch.empty((num_experts, T), dtype=torch.int32, device=dev)
                  if row_id_map is None else _need(row_id_map, "row_id_map", torch.int32,
                                                   (num_experts, T)))
    expert_offsets = (torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
                      if expert_offsets is None else
                      _need(expert_offsets, "expert_offsets", torch.int32, (num_experts + 1,)))
    _check(_lib.moe_make_row_id_map_noalloc(
        _ptr(topk_idx), T, k, num_experts, _ptr(row_id_map), _ptr(expert_offsets),
        _ptr(_status_arg(dev_status)), _stream(stream)), "moe_make_row_id_map_noalloc")
    return row_id_map, expert_offsets


# ---------------------------------------------------------------------------
# (2) permute and (4) unpermute, with backwards
# ---------------------------------------------------------------------------

def _routing(topk_idx, row_id_map):
    _need(topk_idx, "topk_idx", torch.int32)
    _need(row_id_map, "row_id_map", torch.int32)
    if topk_idx.dim() != 2 or row_id_map.dim() != 2:
        raise ValueError("topk_idx is [T, k] and row_id_map is [E, T]")
    T, k = topk_idx.shape
    E = row_id_map.shape[0]
    if row_id_map.shape[1] != T:
        raise ValueError("row_id_map must be [num_experts, num_tokens]")
    return T, k, E


def moe_permute(x: torch.Tensor, topk_idx: torch.Tensor, row_id_map: torch.Tensor,
                probs: Optional[torch.Tensor] = None, *, out=None, out_probs=None,
                dev_status=None, stream=None):
    """out[r(t,j)] = x[t]; out_probs[r(t,j)] = probs[t][j].  Returns (out, out_probs)."""
    T, k, E = _routing(topk_idx, row_id_map)
    _bf16_like_2d(x, "x")
    H = x.shape[1]
    if x.shape[0] != T:
        raise ValueError("x must have num_tokens rows")
    _opt(probs, "probs", torch.float32, (T, k))
    n = T * k
    out = torch.empty((n, H), dtype=x.dtype, device=x.device) if out is None else \
        _need(out, "out", x.dtype, (n, H))
    if probs is not None and out_probs is None:
        out_probs = torch.empty(n, dtype=torch.float32, device=x.device)
    _opt(out_probs, "out_probs", torch.float32, (n,))
    _check(_lib.moe_permute(_ptr(x), _ptr(probs), _ptr(topk_idx), _ptr(row_id_map), T, H, k, E,
                            n, _ptr(out), _ptr(out_probs), _ptr(_status_arg(dev_status)),
                            _stream(stream)), "moe_permute")
    return out, out_probs


def moe_unpermute(inp: torch.Tensor, topk_idx: torch.Tensor, row_id_map: torch.Tensor,
                  probs: Optional[torch.Tensor] = None, *, out=None, dev_status=None,
                  stream=None) -> torch.Tensor:
    """out[t] = bf16(slot-order fp32 FMA chain of probs[t][j] * inp[r(t,j)])."""
    T, k, E = _routing(topk_idx, row_id_map)
    _bf16_like_2d(inp, "inp")
    H = inp.shape[1]
    if inp.shape[0] != T * k:
        raise ValueError("inp must have num_tokens*topk rows")
    _opt(probs, "probs", torch.float32, (T, k))
    out = torch.empty((T, H), dtype=inp.dtype, device=inp.device) if out is None else \
        _need(out, "out", inp.dtype, (T, H))
    _check(_lib.moe_unpermute(_ptr(inp), _ptr(probs), _ptr(topk_idx), _ptr(row_id_map), T, H, k,
                              E, T * k, _ptr(out), _ptr(_status_arg(dev_status)),
                              _stream(stream)), "moe_unpermute")
    return out


def moe_unpermute_ep(inp: torch.Tensor, topk_idx: torch.Tensor, row_id_map: torch.Tensor,
                     ep_size: int, probs: Optional[torch.Tensor] = None, *,
                     bf16_partials: bool = True, fp64_cross: bool = False, out=None,
                     dev_status=None, stream=None) -> torch.Tensor:
    """Rank-ordered combine: per-EP-rank slot-order fmaf partials (optionally
    bf16-rounded) added in rank order (fp32 or fp64), then bf16."""
    T, k, E = _routing(topk_idx, row_id_map)
    _bf16_like_2d(inp, "inp")
    H = inp.shape[1]
    if inp.shape[0] != T * k:
        raise ValueError("inp must have num_tokens*topk rows")
    _opt(probs, "probs", torch.float32, (T, k))
    out = torch.empty((T, H), dtype=inp.dtype, device=inp.device) if out is None else \
        _need(out, "out", inp.dtype, (T, H))
    flags = (EP_BF16_PARTIALS if bf16_partials else 0) | (EP_FP64_CROSS if fp64_cross else 0)
    _check(_lib.moe_unpermute_ep(_ptr(inp), _ptr(probs), _ptr(topk_idx), _ptr(row_id_map), T, H,
                                 k, E, T * k, ep_size, flags, _ptr(out),
                                 _ptr(_status_arg(dev_status)), _stream(stream)),
           "moe_unpermute_ep")
    return out


def moe_unpermute_bwd(d_out: torch.Tensor, topk_idx: torch.Tensor, row_id_map: torch.Tensor,
                      probs: Optional[torch.Tensor] = None, fwd_in: Optional[torch.Tensor] = None,
                      *, probs_grad: bool = True, d_in=None, d_probs=None, dev_status=None,
                      stream=None):
    """Returns (d_in[T*k][H], d_probs[T][k] or None)."""
    T, k, E = _routing(topk_idx, row_id_map)
    _bf16_like_2d(d_out, "d_out")
    H = d_out.shape[1]
    n = T * k
    if d_out.shape[0] != T:
        raise ValueError("d_out must have num_tokens rows")
    _opt(probs, "probs", torch.float32, (T, k))
    _opt(fwd_in, "fwd_in", d_out.dtype, (n, H))
    d_in = torch.empty((n, H), dtype=d_out.dtype, device=d_out.device) if d_in is None else \
        _need(d_in, "d_in", d_out.dtype, (n, H))
    want = probs is not None and fwd_in is not None and probs_grad
    if want and d_probs is None:
        d_probs = torch.empty((T, k), dtype=torch.float32, device=d_out.device)
    if not want:
        d_probs = None
    _opt(d_probs, "d_probs", torch.float32, (T, k))
    _check(_lib.moe_unpermute_bwd(_ptr(d_out), _ptr(fwd_in), _ptr(probs), _ptr(topk_idx),
                                  _ptr(row_id_map), T, H, k, E, n, _ptr(d_in), _ptr(d_probs),
                                  _ptr(_status_arg(dev_status)), _stream(stream)),
           "moe_unpermute_bwd")
    return d_in, d_probs


def moe_permute_bwd(d_out: torch.Tensor, topk_idx: torch.Tensor, row_id_map: torch.Tensor,
                    d_out_probs: Optional[torch.Tensor] = None, *, d_x=None, d_probs=None,
                    dev_status=None, stream=None):
    """Returns (d_x[T][H], d_probs[T][k] or None)."""
    T, k, E = _routing(topk_idx, row_id_map)
    _bf16_like_2d(d_out, "d_out")
    H = d_out.shape[1]
    n = T * k
    if d_out.shape[0] != n:
        raise ValueError("d_out must have num_tokens*topk rows")
    _opt(d_out_probs, "d_out_probs", torch.float32, (n,))
    d_x = torch.empty((T, H), dtype=d_out.dtype, device=d_out.device) if d_x is None else \
        _need(d_x, "d_x", d_out.dtype, (T, H))
    if d_out_probs is not None and d_probs is None:
        d_probs = torch.empty((T, k), dtype=torch.float32, device=d_out.device)
    _opt(d_probs, "d_probs", torch.float32, (T, k))
    _check(_lib.moe_permute_bwd(_ptr(d_out), _ptr(d_out_probs), _ptr(topk_idx),
                                _ptr(row_id_map), T, H, k, E, n, _ptr(d_x), _ptr(d_probs),
                                _ptr(_status_arg(dev_status)), _stream(stream)),
           "moe_permute_bwd")
    return d_x, d_probs


# ---------------------------------------------------------------------------
# quantized rows with scales
# ---------------------------------------------------------------------------

def _rows_any(t, name):
    _need(t, name)
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.element_size() not in (1, 2, 4):
        raise TypeError(f"{name} must have 1-, 2- or 4-byte elements")
    return t


def _scale_rows(scale, T):
    if scale is None:
        return None, 0
    _need(scale, "scale")
    if scale.dim() != 2 or scale.shape[0] != T:
        raise ValueError("scale must be [num_tokens, n]")
    return scale, scale.shape[1] * scale.element_size()


def moe_permute_scaled(x: torch.Tensor, topk_idx: torch.Tensor, row_id_map: torch.Tensor,
                       scale: Optional[torch.Tensor] = None, probs: Optional[torch.Tensor] = None,
                       *, out=None, out_scale=None, out_probs=None, dev_status=None,
                       stream=None):
    """Permute rows of any 1/2/4-byte dtype (e.g. float8_e4m3fn) with their scale
    rows moved alongside.  Returns (out, out_scale, out_probs)."""
    T, k, E = _routing(topk_idx, row_id_map)
    _rows_any(x, "x")
    if x.shape[0] != T:
        raise ValueError("x must have num_tokens rows")
    H = x.shape[1]
    n = T * k
    scale, srb = _scale_rows(scale, T)
    _opt(probs, "probs", torch.float32, (T, k))
    out = torch.empty((n, H), dtype=x.dtype, device=x.device) if out is None else \
        _need(out, "out", x.dtype, (n, H))
    if scale is not None and out_scale is None:
        out_scale = torch.empty((n, scale.shape[1]), dtype=scale.dtype, device=x.device)
    if scale is not None:
        _need(out_scale, "out_scale", scale.dtype, (n, scale.shape[1]))
    if probs is not None and out_probs is None:
        out_probs = torch.empty(n, dtype=torch.float32, device=x.device)
    _opt(out_probs, "out_probs", torch.float32, (n,))
    _check(_lib.moe_permute_scaled(_ptr(x), x.element_size(), _ptr(scale), srb, _ptr(probs),
                                   _ptr(topk_idx), _ptr(row_id_map), T, H, k, E, n, _ptr(out),
                                   _ptr(out_scale), _ptr(out_probs),
                                   _ptr(_status_arg(dev_status)), _stream(stream)),
           "moe_permute_scaled")
    return out, out_scale, out_probs


def moe_permute_mask_scaled(x: torch.Tensor, row_id_map: torch.Tensor, num_out_rows: int,
                            scale: Optional[torch.Tensor] = None,
                            probs: Optional[torch.Tensor] = None, *, out=None, out_scale=None,
                            out_probs=None, dev_status=None, stream=None):
    """Mask-map form of moe_permute_scaled (probs [T, E]; a zero prob zeroes the
    data row, the scale row still moves).  Returns (out, out_scale, out_probs)."""
    T, E = _mask_map(row_id_map)
    _rows_any(x, "x")
    if x.shape[0] != T:
        raise ValueError("x must have num_tokens rows")
    H = x.shape[1]
    n = num_out_rows
    scale, srb = _scale_rows(scale, T)
    _opt(probs, "probs", torch.float32, (T, E))
    out = torch.empty((n, H), dtype=x.dtype, device=x.device) if out is None else \
        _need(out, "out", x.dtype, (n, H))
    if scale is not None and out_scale is None:
        out_scale = torch.empty((n, scale.shape[1]), dtype=scale.dtype, device=x.device)
    if scale is not None:
        _need(out_scale, "out_scale", scale.dtype, (n, scale.shape[1]))
    if probs is not None and out_probs is None:
        out_probs = torch.empty(n, dtype=torch.float32, device=x.device)
    _opt(out_probs, "out_probs", torch.float32, (n,))
    _check(_lib.moe_permute_mask_scaled(_ptr(x), x.element_size(), _ptr(scale), srb,
                                        _ptr(probs), _ptr(row_id_map), T, H, E, n, _ptr(out),
                                        _ptr(out_scale), _ptr(out_probs),
                                        _ptr(_status_arg(dev_status)), _stream(stream)),
           "moe_permute_mask_scaled")
    return out, out_scale, out_probs


# ---------------------------------------------------------------------------
# TransformerEngine mask-map form
# ---------------------------------------------------------------------------

def moe_make_mask_row_id_map_workspace_bytes(num_tokens: int, num_experts: int) -> int:
    return int(_lib.moe_make_mask_row_id_map_workspace_bytes(num_tokens, num_experts))


def moe_make_mask_row_id_map(routing_map: torch.Tensor, *, num_out_tokens: int = -1,
                             row_id_map=None, expert_offsets=None, workspace=None, stream=None):
    """[T, E] routing mask (bool / uint8 / int8 / int32) -> (row_id_map [T, 2E+1],
    expert_offsets [E+1]); rows at or past num_out_tokens are dropped."""
    _need(routing_map, "routing_map")
    if routing_map.dim() != 2:
        raise ValueError("routing_map must be [num_tokens, num_experts]")
    if routing_map.dtype in (torch.bool, torch.uint8, torch.int8):
        mb = 1
    elif routing_map.dtype == torch.int32:
        mb = 4
    else:
        raise TypeError("routing_map must be bool, uint8, int8 or int32")
    T, E = routing_map.shape
    dev = routing_map.device
    row_id_map = (torch.empty((T, 2 * E + 1), dtype=torch.int32, device=dev)
                  if row_id_map is None else
                  _need(row_id_map, "row_id_map", torch.int32, (T, 2 * E + 1)))
    expert_offsets = (torch.empty(E + 1, dtype=torch.int32, device=dev)
                      if expert_offsets is None else
                      _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,)))
    need = moe_make_mask_row_id_map_workspace_bytes(T, E)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace")
    _check(_lib.moe_make_mask_row_id_map(
        _ptr(routing_map), mb, T, E, num_out_tokens, _ptr(row_id_map), _ptr(expert_offsets),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
        "moe_make_mask_row_id_map")
    return row_id_map, expert_offsets


def _mask_map(row_id_map):
    _need(row_id_map, "row_id_map", torch.int32)
    if row_id_map.dim() != 2 or row_id_map.shape[1] % 2 != 1:
        raise ValueError("row_id_map must be [num_tokens, 2 * num_experts + 1]")
    return row_id_map.shape[0], (row_id_map.shape[1] - 1) // 2


def moe_permute_mask(x: torch.Tensor, row_id_map: torch.Tensor, num_out_rows: int,
                     probs: Optional[torch.Tensor] = None, *, out=None, out_probs=None,
                     dev_status=None, stream=None):
    """out[row] = x[t] per map slot; with probs [T, E]: out_probs[row] = probs[t, e]
    and a zero prob writes a zero row.  Returns (out, out_probs)."""
    T, E = _mask_map(row_id_map)
    _bf16_like_2d(x, "x")
    if x.shape[0] != T:
        raise ValueError("x must have num_tokens rows")
    H = x.shape[1]
    _opt(probs, "probs", torch.float32, (T, E))
    out = torch.empty((num_out_rows, H), dtype=x.dtype, device=x.device) if out is None else \
        _need(out, "out", x.dtype, (num_out_rows, H))
    if probs is not None and out_probs is None:
        out_probs = torch.empty(num_out_rows, dtype=torch.float32, device=x.device)
    _opt(out_probs, "out_probs", torch.float32, (num_out_rows,))
    _check(_lib.moe_permute_mask(_ptr(x), _ptr(probs), _ptr(row_id_map), T, H, E, num_out_rows,
                                 _ptr(out), _ptr(out_probs), _ptr(_status_arg(dev_status)),
                                 _stream(stream)), "moe_permute_mask")
    return out, out_probs


def moe_unpermute_mask(inp: torch.Tensor, row_id_map: torch.Tensor,
                       merging_probs: Optional[torch.Tensor] = None,
                       permuted_probs: Optional[torch.Tensor] = None, *, out=None,
                       unpermuted_probs=None, dev_status=None, stream=None):
    """TE-order combine: rows in map order, times merging_probs[t, e], added in
    fp32.  Returns (out [T, H], unpermuted_probs [T, E] or None)."""
    T, E = _mask_map(row_id_map)
    _bf16_like_2d(inp, "inp")
    n, H = inp.shape
    _opt(merging_probs, "merging_probs", torch.float32, (T, E))
    _opt(permuted_probs, "permuted_probs", torch.float32, (n,))
    out = torch.empty((T, H), dtype=inp.dtype, device=inp.device) if out is None else \
        _need(out, "out", inp.dtype, (T, H))
    if permuted_probs is not None and unpermuted_probs is None:
        unpermuted_probs = torch.empty((T, E), dtype=torch.float32, device=inp.device)
    _opt(unpermuted_probs, "unpermuted_probs", torch.float32, (T, E))
    _check(_lib.moe_unpermute_mask(_ptr(inp), _ptr(merging_probs), _ptr(permuted_probs),
                                   _ptr(row_id_map), T, H, E, n, _ptr(out),
                                   _ptr(unpermuted_probs), _ptr(_status_arg(dev_status)),
                                   _stream(stream)), "moe_unpermute_mask")
    return out, unpermuted_probs


def moe_unpermute_mask_bwd(d_out: torch.Tensor, fwd_in: torch.Tensor,
                           merging_probs: torch.Tensor, row_id_map: torch.Tensor, *,
                           d_in=None, d_merging_probs=None, want_probs_grad: bool = True,
                           dev_status=None, stream=None):
    """d_in[row] = bf16(d_out[t] * p) per slot; d_merging_probs[t, e] = fp32 dot of
    fwd_in[row] and d_out[t].  Returns (d_in, d_merging_probs or None)."""
    T, E = _mask_map(row_id_map)
    _bf16_like_2d(d_out, "d_out")
    _bf16_like_2d(fwd_in, "fwd_in")
    n, H = fwd_in.shape
    if d_out.shape != (T, H):
        raise ValueError("d_out must be [num_tokens, hidden]")
    _need(merging_probs, "merging_probs", torch.float32, (T, E))
    d_in = torch.empty((n, H), dtype=d_out.dtype, device=d_out.device) if d_in is None else \
        _need(d_in, "d_in", d_out.dtype, (n, H))
    if want_probs_grad and d_merging_probs is None:
        d_merging_probs = torch.empty((T, E), dtype=torch.float32, device=d_out.device)
    _opt(d_merging_probs, "d_merging_probs", torch.float32, (T, E))
    _check(_lib.moe_unpermute_mask_bwd(_ptr(d_out), _ptr(fwd_in), _ptr(merging_probs),
                                       _ptr(row_id_map), T, H, E, n, _ptr(d_in),
                                       _ptr(d_merging_probs), _ptr(_status_arg(dev_status)),
                                       _stream(stream)), "moe_unpermute_mask_bwd")
    return d_in, d_merging_probs


# ---------------------------------------------------------------------------
# router
# ---------------------------------------------------------------------------

def moe_topk_softmax(logits: torch.Tensor, topk: int, *, fp32_routing: bool = True,
                     topk_idx=None, probs=None, stream=None):
    """Top-k of each row of logits ([T, E], bf16 or fp32; descending, ties to
    the lower index) and a softmax over the k.  Weights are fp32 with
    fp32_routing, else in the logits' dtype.  Returns (topk_idx, probs)."""
    _need(logits, "logits")
    if logits.dim() != 2 or logits.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("logits must be a 2-D bf16 or fp32 tensor")
    T, E = logits.shape
    dev = logits.device
    pdt = torch.float32 if fp32_routing else logits.dtype
    topk_idx = torch.empty((T, topk), dtype=torch.int32, device=dev) if topk_idx is None else \
        _need(topk_idx, "topk_idx", torch.int32, (T, topk))
    probs = torch.empty((T, topk), dtype=pdt, device=dev) if probs is None else \
        _need(probs, "probs", pdt, (T, topk))
    _check(_lib.moe_topk_softmax(_ptr(logits), logits.element_size(), T, E, topk,
                                 _ptr(topk_idx), _ptr(probs), probs.element_size(),
                                 _stream(stream)), "moe_topk_softmax")
    return topk_idx, probs


def moe_topk_softmax_bwd(d_probs: torch.Tensor, probs: torch.Tensor, topk_idx: torch.Tensor,
                         num_experts: int, *, logits_dtype=torch.float32, d_logits=None,
                         dev_status=None, stream=None):
    """Softmax gradient scattered to the selected experts: returns d_logits
    [T, E] in logits_dtype (fp32 or bf16).  probs and d_probs share a dtype."""
    _need(topk_idx, "topk_idx", torch.int32)
    T, k = topk_idx.shape
    if probs.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("probs must be fp32 or bf16")
    _need(probs, "probs", probs.dtype, (T, k))
    _need(d_probs, "d_probs", probs.dtype, (T, k))
    if d_logits is None:
        d_logits = torch.empty((T, num_experts), dtype=logits_dtype, device=probs.device)
    elif d_logits.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("d_logits must be fp32 or bf16")
    _need(d_logits, "d_logits", d_logits.dtype, (T, num_experts))
    _check(_lib.moe_topk_softmax_bwd(_ptr(d_probs), _ptr(probs), probs.element_size(),
                                     _ptr(topk_idx), T, num_experts, k, _ptr(d_logits),
                                     d_logits.element_size(), _ptr(_status_arg(dev_status)),
                                     _stream(stream)), "moe_topk_softmax_bwd")
    return d_logits


# ---------------------------------------------------------------------------
# (3) chunk sort-and-pad / unpad-and-restore, with backwards
# ---------------------------------------------------------------------------

def _rows2d(t, name):
    _need(t, name)
    if t.dim() != 2 or t.element_size() not in (2, 4):
        raise TypeError(f"{name} must be a 2-D tensor of 2- or 4-byte elements")
    return t


def _probs1d(t, name, n):
    if t is None:
        return None
    _need(t, name)
    if t.dim() != 1 or t.shape[0] != n or t.element_size() not in (2, 4):
        raise TypeError(f"{name} must be a 1-D tensor of {n} 2- or 4-byte elements")
    return t


def _prob_out(t, name, src, n):
    """A caller-given prob output: the dtype of the probs it receives and n
    entries (the kernels store src's element width into it)."""
    if t is None:
        return None
    return _need(t, name, src.dtype if src is not None else None, (n,))


def moe_sort_chunks_and_pad(inp: torch.Tensor, split_sizes: torch.Tensor,
                            sorted_idx: torch.Tensor, chunks_per_group: int, align: int,
                            out_cap: int, probs: Optional[torch.Tensor] = None, *, out=None,
                            out_probs=None, row_map=None, padded_offsets=None, dev_status=None,
                            stream=None):
    """Returns (out[out_cap][H], out_probs, row_map[out_cap], padded_offsets[G+1])."""
    _rows2d(inp, "inp")
    n_cap, H = inp.shape
    _need(split_sizes, "split_sizes", torch.int32)
    _need(sorted_idx, "sorted_idx", torch.int32, split_sizes.shape)
    C = split_sizes.numel()
    G = C // chunks_per_group if chunks_per_group > 0 else 0
    dev = inp.device
    _probs1d(probs, "probs", n_cap)
    out = torch.empty((out_cap, H), dtype=inp.dtype, device=dev) if out is None else \
        _need(out, "out", inp.dtype, (out_cap, H))
    if probs is not None and out_probs is None:
        out_probs = torch.empty(out_cap, dtype=probs.dtype, device=dev)
    _prob_out(out_probs, "out_probs", probs, out_cap)
    row_map = torch.empty(out_cap, dtype=torch.int32, device=dev) if row_map is None else \
        _need(row_map, "row_map", torch.int32, (out_cap,))
    padded_offsets = (torch.empty(G + 1, dtype=torch.int32, device=dev)
                      if padded_offsets is None else
                      _need(padded_offsets, "padded_offsets", torch.int32, (G + 1,)))
    pb = probs.element_size() if probs is not None else 4
    _check(_lib.moe_sort_chunks_and_pad(
        _ptr(inp), _ptr(probs), inp.element_size(), pb, n_cap, H, _ptr(split_sizes),
        _ptr(sorted_idx), C, chunks_per_group, align, out_cap, _ptr(out), _ptr(out_probs),
        _ptr(row_map), _ptr(padded_offsets), _ptr(_status_arg(dev_status)), _stream(stream)),
        "moe_sort_chunks_and_pad")
    return out, out_probs, row_map, padded_offsets


def moe_unpad_and_restore_chunks(inp: torch.Tensor, row_map: torch.Tensor,
                                 split_sizes: torch.Tensor, n_cap: int,
                                 probs: Optional[torch.Tensor] = None, *, out=None,
                                 out_probs=None, dev_status=None, stream=None):
    """Returns (out[n_cap][H], out_probs)."""
    _rows2d(inp, "inp")
    out_cap, H = inp.shape
    _need(row_map, "row_map", torch.int32, (out_cap,))
    _need(split_sizes, "split_sizes", torch.int32)
    _probs1d(probs, "probs", out_cap)
    dev = inp.device
    out = torch.empty((n_cap, H), dtype=inp.dtype, device=dev) if out is None else \
        _need(out, "out", inp.dtype, (n_cap, H))
    if probs is not None and out_probs is None:
        out_probs = torch.empty(n_cap, dtype=probs.dtype, device=dev)
    _prob_out(out_probs, "out_probs", probs, n_cap)
    pb = probs.element_size() if probs is not None else 4
    _check(_lib.moe_unpad_and_restore_chunks(
        _ptr(inp), _ptr(probs), inp.element_size(), pb, _ptr(row_map), _ptr(split_sizes),
        split_sizes.numel(), out_cap, H, n_cap, _ptr(out), _ptr(out_probs),
        _ptr(_status_arg(dev_status)), _stream(stream)), "moe_unpad_and_restore_chunks")
    return out, out_probs


def moe_sort_chunks_and_pad_bwd(d_out: torch.Tensor, row_map: torch.Tensor,
                                split_sizes: torch.Tensor, n_cap: int,
                                d_out_probs: Optional[torch.Tensor] = None, *, d_in=None,
                                d_in_probs=None, dev_status=None, stream=None):
    """Gradient of sort-and-pad w.r.t. its input.  Returns (d_in[n_cap][H], d_in_probs)."""
    _rows2d(d_out, "d_out")
    out_cap, H = d_out.shape
    _need(row_map, "row_map", torch.int32, (out_cap,))
    _need(split_sizes, "split_sizes", torch.int32)
    _probs1d(d_out_probs, "d_out_probs", out_cap)
    dev = d_out.device
    d_in = torch.empty((n_cap, H), dtype=d_out.dtype, device=dev) if d_in is None else \
        _need(d_in, "d_in", d_out.dtype, (n_cap, H))
    if d_out_probs is not None and d_in_probs is None:
        d_in_probs = torch.empty(n_cap, dtype=d_out_probs.dtype, device=dev)
    _prob_out(d_in_probs, "d_in_probs", d_out_probs, n_cap)
    pb = d_out_probs.element_size() if d_out_probs is not None else 4
    _check(_lib.moe_sort_chunks_and_pad_bwd(
        _ptr(d_out), _ptr(d_out_probs), d_out.element_size(), pb, _ptr(row_map),
        _ptr(split_sizes), split_sizes.numel(), out_cap, H, n_cap, _ptr(d_in), _ptr(d_in_probs),
        _ptr(_status_arg(dev_status)), _stream(stream)), "moe_sort_chunks_and_pad_bwd")
    return d_in, d_in_probs


def moe_unpad_and_restore_chunks_bwd(d_out: torch.Tensor, row_map: torch.Tensor, out_cap: int,
                                     d_out_probs: Optional[torch.Tensor] = None, *, d_in=None,
                                     d_in_probs=None, dev_status=None, stream=None):
    """Gradient of the restore w.r.t. the padded buffer.  Returns (d_in[out_cap][H], probs)."""
    _rows2d(d_out, "d_out")
    n_cap, H = d_out.shape
    _need(row_map, "row_map", torch.int32, (out_cap,))
    _probs1d(d_out_probs, "d_out_probs", n_cap)
    dev = d_out.device
    d_in = torch.empty((out_cap, H), dtype=d_out.dtype, device=dev) if d_in is None else \
        _need(d_in, "d_in", d_out.dtype, (out_cap, H))
    if d_out_probs is not None and d_in_probs is None:
        d_in_probs = torch.empty(out_cap, dtype=d_out_probs.dtype, device=dev)
    _prob_out(d_in_probs, "d_in_probs", d_out_probs, out_cap)
    pb = d_out_probs.element_size() if d_out_probs is not None else 4
    _check(_lib.moe_unpad_and_restore_chunks_bwd(
        _ptr(d_out), _ptr(d_out_probs), d_out.element_size(), pb, _ptr(row_map), out_cap, H,
        n_cap, _ptr(d_in), _ptr(d_in_probs), _ptr(_status_arg(dev_status)), _stream(stream)),
        "moe_unpad_and_restore_chunks_bwd")
    return d_in, d_in_probs
