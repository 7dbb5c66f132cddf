"""Seeded synthetic inputs for the MoE permute / unpermute path.

This module only draws inputs.  It holds none of the method's arithmetic and
imports neither the product package nor the oracle; both sides of every
parity check, and the benchmark, take their inputs from here.  Everything is
drawn with a torch CPU generator, so the same seed gives the same bits on any
machine; GPU code receives copies of these host tensors.

Routing is drawn upstream of the path: router logits -> top-k indices
(int32) and an fp32 softmax over the k selected logits.  The indices are
computed once on the host and fed unchanged to both sides, so a tie-break
inside top-k cannot make the two sides disagree.

Workloads (sizes of the five benchmarked configurations):
  tiny       T=16,    H=64,   E=32,  k=4   bf16 router logits (seed 1)
  finegrain  T=4096,  H=2048, E=64,  k=6   fp32 logits, near-uniform load
  chunks8k   N=8192,  H=2048, 16 experts x 8 rank chunks, align 128
  chunks32k  N=32768, H=2048, 16 experts x 8 rank chunks, align 128
  skewed     T=16384, H=7168, E=256, k=8   logits + a Zipf(1.1) expert bias
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch


@dataclass
class Routed:
    name: str
    x: torch.Tensor            # [T, H] bf16 hidden states
    topk_idx: torch.Tensor     # [T, k] int32, distinct experts per token
    probs: torch.Tensor        # [T, k] fp32 softmax over the selected logits
    num_experts: int
    dy: Optional[torch.Tensor] = None   # [T, H] bf16 upstream gradient
    seed: int = 0
    logits: Optional[torch.Tensor] = None   # [T, E] router logits the routing came from

    @property
    def T(self):
        return self.x.shape[0]

    @property
    def H(self):
        return self.x.shape[1]

    @property
    def k(self):
        return self.topk_idx.shape[1]


@dataclass
class Chunked:
    name: str
    x: torch.Tensor            # [N_cap, H] tokens, rank chunks back to back
    probs: torch.Tensor        # [N_cap] fp32 U(0,1)
    split_sizes: torch.Tensor  # [C] int32, chunk c = r * E + e (rank-major)
    sorted_idx: torch.Tensor   # [C] int32, sorted position -> input chunk
    chunks_per_group: int
    align: int
    out_cap: int
    seed: int = 0
    replays: list = field(default_factory=list)   # extra split-size draws

    @property
    def N_cap(self):
        return self.x.shape[0]

    @property
    def H(self):
        return self.x.shape[1]

    @property
    def C(self):
        return self.split_sizes.numel()


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def route(logits: torch.Tensor, k: int):
    """Top-k indices (int32) and an fp32 softmax over the k selected logits."""
    vals, idx = torch.topk(logits, k, dim=-1)
    probs = torch.softmax(vals.float(), dim=-1)
    return idx.to(torch.int32).contiguous(), probs.contiguous()


def random_routed(T: int, H: int, E: int, k: int, seed: int, with_dy: bool = True,
                  name: str = "random", zipf_s: float = 0.0) -> Routed:
    """N(0,1) hidden states and logits; optional Zipf-shaped expert bias."""
    g = _gen(seed)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    logits = torch.randn(T, E, generator=g)
    if zipf_s > 0.0:
        rank = torch.randperm(E, generator=g).to(torch.float32)
        logits = logits - zipf_s * torch.log1p(rank)[None, :]
    idx, probs = route(logits, k)
    dy = torch.randn(T, H, generator=g).to(torch.bfloat16) if with_dy else None
    return Routed(name, x, idx, probs, E, dy, seed, logits)


def tiny() -> Routed:
    """T=16, H=64, E=32, k=4; bf16 hidden and bf16 router logits, seed 1."""
    g = _gen(1)
    x = torch.randn(16, 64, generator=g).to(torch.bfloat16)
    logits = torch.randn(16, 32, generator=g).to(torch.bfloat16)
    idx, probs = route(logits, 4)
    dy = torch.randn(16, 64, generator=g).to(torch.bfloat16)
    return Routed("tiny", x, idx, probs, 32, dy, 1, logits)


def finegrain() -> Routed:
    """T=4096, H=2048, E=64, k=6; fp32 N(0,1) logits (near-uniform), seed 2."""
    return random_routed(4096, 2048, 64, 6, seed=2, name="finegrain")


def skewed() -> Routed:
    """T=16384, H=7168, E=256, k=8; logits N(0,1) plus bias -1.1*ln(1+pi(e))
    (log of a Zipf(1.1) pmf over a seeded expert permutation pi), seed 5."""
    return random_routed(16384, 7168, 256, 8, seed=5, name="skewed", zipf_s=1.1)


def chunk_sizes(N: int, num_ranks: int, num_experts: int, num_empty: int,
                g: torch.Generator) -> torch.Tensor:
    """Sizes of C = ranks*experts chunks (chunk c = r*E + e): a seeded subset
    of num_empty chunks is empty, the other chunks share N tokens by a uniform
    multinomial draw."""
    C = num_ranks * num_experts
    empty = torch.randperm(C, generator=g)[:num_empty]
    live = torch.ones(C, dtype=torch.bool)
    live[empty] = False
    live_ids = torch.nonzero(live).flatten()
    draws = torch.randint(0, live_ids.numel(), (N,), generator=g)
    sizes = torch.zeros(C, dtype=torch.int64)
    sizes.index_add_(0, live_ids[draws], torch.ones(N, dtype=torch.int64))
    return sizes.to(torch.int32)


def expert_major_order(num_ranks: int, num_experts: int) -> torch.Tensor:
    """sorted_idx[e*R + r] = r*E + e: regroup rank-major chunks by expert."""
    q = torch.empty(num_ranks * num_experts, dtype=torch.int32)
    for e in range(num_experts):
        for r in range(num_ranks):
            q[e * num_ranks + r] = r * num_experts + e
    return q


def padded_capacity(N: int, num_groups: int, align: int) -> int:
    """Worst-case padded rows: every group may add align-1 rows of padding."""
    return int(math.ceil((N + num_groups * (align - 1)) / align) * align)


def chunked(N: int, seed: int, H: int = 2048, num_ranks: int = 8, num_experts: int = 16,
            align: int = 128, num_empty: int = 16, replay_seeds=(),
            dtype=torch.bfloat16, name: str = "chunks") -> Chunked:
    g = _gen(seed)
    x = torch.randn(N, H, generator=g).to(dtype)
    probs = torch.rand(N, generator=g)
    sizes = chunk_sizes(N, num_ranks, num_experts, num_empty, g)
    order = expert_major_order(num_ranks, num_experts)
    cap = padded_capacity(N, num_experts, align)
    replays = []
    for s in replay_seeds:
        gr = _gen(s)
        # A replay draws a new total (at most N) and new sizes; buffers stay.
        n_act = int(torch.randint(N // 2, N + 1, (1,), generator=gr))
        replays.append(chunk_sizes(n_act, num_ranks, num_experts, num_empty, gr))
    return Chunked(name, x, probs, sizes, order, num_ranks, align, cap, seed, replays)


def chunks8k() -> Chunked:
    return chunked(8192, seed=3, name="chunks8k")


def chunks32k(with_replays: bool = False) -> Chunked:
    seeds = tuple(range(4000, 4008)) if with_replays else ()
    return chunked(32768, seed=4, replay_seeds=seeds, name="chunks32k")


ROUTED = {"tiny": tiny, "finegrain": finegrain, "skewed": skewed}
CHUNKED = {"chunks8k": chunks8k, "chunks32k": chunks32k}


def quantize_fp8_rows(x: torch.Tensor, block: int = 128, scale_dtype=torch.float32):
    """FP8 (OCP E4M3FN) rows with one scale per `block` elements of a row:
    scale = amax / 448 (the format's largest finite value; 1 for an all-zero
    block), q = fp8(x / scale) by torch's round-to-nearest cast.  Returns
    (q [T][H] float8_e4m3fn, scale [T][ceil(H / block)] of scale_dtype).  With
    scale_dtype torch.float8_e8m0fnu the scale is rounded up to a power of two
    first (an MX-style exponent scale).  The quantization happens upstream of
    the path: the permute moves the bytes it is given."""
    T, H = x.shape
    nb = (H + block - 1) // block
    xf = torch.nn.functional.pad(x.float(), (0, nb * block - H)).view(T, nb, block)
    amax = xf.abs().amax(dim=2)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    if scale_dtype == torch.float8_e8m0fnu:
        scale = torch.exp2(torch.ceil(torch.log2(scale)))
    q = (xf / scale[:, :, None]).view(T, nb * block)[:, :H].to(torch.float8_e4m3fn)
    return q.contiguous(), scale.to(scale_dtype).contiguous()


def bf16_bits(t: torch.Tensor):
    """numpy uint16 view of a bf16 CPU tensor's bit patterns."""
    return t.contiguous().view(torch.int16).numpy().view("uint16")


def random_rows(n: int, H: int, seed: int, device="cpu") -> torch.Tensor:
    """[n, H] bf16 N(0,1) rows drawn with a torch generator on `device`
    (used as arbitrary bf16 inputs to the combine and its gradients)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(n, H, generator=g, device=device).to(torch.bfloat16)
