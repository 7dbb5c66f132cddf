"""Pins for the CPU oracle: each test checks the oracle against something
other than itself -- values printed on the pages, brute force on tiny inputs,
exact rational arithmetic, closed forms, invariants, or an independent
library routine (torch CPU casts, numpy sorts and dots).

No test here needs a GPU.
"""
import itertools
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers ---

def _read_golden(name):
    blocks, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.replace("_", "").isalnum() and not any(c.isdigit() for c in line[:1]) \
                    and " " not in line:
                cur = line
                blocks[cur] = []
                continue
            blocks[cur].append(line.split())
    return blocks


def _bits(t):
    return workloads.bf16_bits(t)


def _to_bf16_torch(f32: np.ndarray) -> np.ndarray:
    """Reference fp32 -> bf16 RNE by torch's CPU cast (bit patterns)."""
    return _bits(torch.from_numpy(np.ascontiguousarray(f32, np.float32)).to(torch.bfloat16))


def _bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _rn_f32(q: Fraction) -> Fraction:
    """Round an exact rational to the nearest binary32 value, ties to even
    (independent of the oracle; overflow is not exercised here)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                      # subnormal range: fixed quantum
    quantum = Fraction(2) ** (e - 23)
    m = a / quantum
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * quantum


def _brute_rows(topk_idx: np.ndarray, E: int):
    """Row of every (t, j) by sorting the (expert, token) pairs: the rows
    are expert-major with ascending tokens inside an expert."""
    T, k = topk_idx.shape
    pairs = sorted((int(topk_idx[t, j]), t, j) for t in range(T) for j in range(k))
    rows = np.empty((T, k), np.int64)
    for pos, (_, t, j) in enumerate(pairs):
        rows[t, j] = pos
    ref = np.full((E, T), -1, np.int32)
    for t in range(T):
        for j in range(k):
            ref[topk_idx[t, j], t] = rows[t, j]
    counts = np.bincount(topk_idx.ravel(), minlength=E)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return ref, offs, rows


# ---------------------------------------------------- (1) the row map ------

def test_worked_example_second_pass():
    g = _read_golden("make_row_id_map_worked_example.txt")
    mask = np.array(g["routing_map"], dtype=np.int32)          # [T][E]
    pass2 = np.array(g["pass2"], dtype=np.int32)               # [T][E]
    T, E = mask.shape
    pt, pe = np.nonzero(mask)          # row-major: token order, then expert
    m, off = oracle.row_id_map_pairs(pt, pe, T, E)
    np.testing.assert_array_equal(m, pass2.T)   # our layout is [E][T]
    np.testing.assert_array_equal(off, [0, 3, 5, 7])


def test_worked_example_third_pass():
    g = _read_golden("make_row_id_map_worked_example.txt")
    mask = np.array(g["routing_map"], dtype=np.int32)
    T, E = mask.shape
    pt, pe = np.nonzero(mask)
    m, _ = oracle.row_id_map_pairs(pt, pe, T, E)
    for t, row in enumerate(g["pass3"]):
        n = int(row[2 * E])
        rows = sorted((int(m[e, t]), e) for e in range(E) if m[e, t] >= 0)[::-1]
        assert n == len(rows)
        assert [int(v) for v in row[:n]] == [r for r, _ in rows]
        assert [int(v) for v in row[E:E + n]] == [e for _, e in rows]


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (2, 3, 1), (3, 3, 2), (2, 4, 3), (3, 4, 2),
                                   (4, 3, 1), (2, 3, 3)])
def test_row_map_brute_force_all_routings(T, E, k):
    """Every routing with k distinct experts per token, in every slot order."""
    choices = list(itertools.permutations(range(E), k))
    for routing in itertools.product(choices, repeat=T):
        idx = np.array(routing, dtype=np.int32).reshape(T, k)
        m, off = oracle.row_id_map(idx, E)
        ref, ref_off, _ = _brute_rows(idx, E)
        np.testing.assert_array_equal(m, ref)
        np.testing.assert_array_equal(off, ref_off)


@pytest.mark.parametrize("seed", range(6))
def test_row_map_equals_stable_argsort(seed):
    """A stable argsort of the flattened top-k indices gives the same rows."""
    rng = np.random.default_rng(seed)
    T, E, k = int(rng.integers(1, 300)), int(rng.integers(1, 70)), 0
    k = int(rng.integers(1, min(E, 9) + 1))
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    m, off = oracle.row_id_map(idx, E)
    order = np.argsort(idx.ravel(), kind="stable")
    row_of_flat = np.empty_like(order)
    row_of_flat[order] = np.arange(order.size)
    t = np.repeat(np.arange(T), k)
    np.testing.assert_array_equal(m[idx.ravel(), t], row_of_flat)
    assert (m >= 0).sum() == T * k


def test_row_map_invariants_skewed():
    w = workloads.random_routed(2000, 8, 96, 7, seed=11, with_dy=False, zipf_s=1.1)
    idx = w.topk_idx.numpy()
    m, off = oracle.row_id_map(idx, 96)
    counts = np.bincount(idx.ravel(), minlength=96)
    assert counts.sum() == 2000 * 7 == off[-1]
    np.testing.assert_array_equal(np.diff(off), counts)
    rows = m[m >= 0]
    np.testing.assert_array_equal(np.sort(rows), np.arange(2000 * 7))   # bijection
    for e in range(96):
        r = m[e][m[e] >= 0]
        assert np.all(np.diff(r) == 1)                  # ascending tokens, dense
        if r.size:
            assert r[0] == off[e] and r[-1] == off[e + 1] - 1


def test_row_map_errors():
    with pytest.raises(oracle.OracleError) as ei:
        oracle.row_id_map(np.array([[0, 3]], np.int32), 3)
    assert ei.value.code == 1
    with pytest.raises(oracle.OracleError) as ei:
        oracle.row_id_map(np.array([[1, 1]], np.int32), 3)
    assert ei.value.code == 2
    with pytest.raises(oracle.OracleError):
        oracle.row_id_map(np.array([[-1]], np.int32), 3)


def test_row_map_empty_tokens():
    m, off = oracle.row_id_map(np.zeros((0, 2), np.int32), 5)
    assert m.shape == (5, 0)
    np.testing.assert_array_equal(off, np.zeros(6))


# ------------------------------------------------------- (2) permute -------

def _routed(T, H, E, k, seed):
    return workloads.random_routed(T, H, E, k, seed=seed)


@pytest.mark.parametrize("T,H,E,k", [(16, 64, 32, 4), (37, 24, 9, 3), (5, 7, 2, 2)])
def test_permute_is_row_copy(T, H, E, k):
    w = _routed(T, H, E, k, seed=T)
    idx = w.topk_idx.numpy()
    x = _bits(w.x)
    m, _ = oracle.row_id_map(idx, E)
    out, op = oracle.permute(x, w.probs.numpy(), idx, m)
    _, _, rows = _brute_rows(idx, E)
    exp = np.empty((T * k, H), np.uint16)
    exp_p = np.empty(T * k, np.float32)
    exp[rows.ravel()] = np.repeat(x, k, axis=0)
    exp_p[rows.ravel()] = w.probs.numpy().ravel()
    np.testing.assert_array_equal(out, exp)
    np.testing.assert_array_equal(op, exp_p)


# ----------------------------------------------------- (4) unpermute -------

def test_libm_fmaf_is_fused():
    a = 1.0 + 2.0 ** -12
    c = -(1.0 + 2.0 ** -11)
    assert oracle.fmaf(a, a, c) == 2.0 ** -24           # one rounding
    assert np.float32(np.float32(a) * np.float32(a)) + np.float32(c) == 0.0


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(3000).astype(np.float32),
        (rng.standard_normal(500) * 1e-39).astype(np.float32),          # subnormals
        np.clip(rng.standard_normal(500) * 1e38, -3.3e38, 3.3e38).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 1.0, -1.0, 3.4028235e38], np.float32),
    ])
    # exact ties: low 16 bits == 0x8000, with even and odd kept parts
    u = rng.integers(0, 2 ** 31, 1000, dtype=np.uint32)
    ties = ((u & 0xFFFF0000) | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    vals = np.concatenate([vals, ties])
    got = np.array([oracle.f32_to_bf16(float(v)) for v in vals], np.uint16)
    np.testing.assert_array_equal(got, _to_bf16_torch(vals))
    # NaN: stays NaN, quiet bit set, sign kept
    for pattern in (0x7FA00001, 0xFFC12345, 0x7F800001):
        f = np.array([pattern], np.uint32).view(np.float32)[0]
        b = oracle.f32_to_bf16(float(f))
        assert (b & 0x7F80) == 0x7F80 and (b & 0x0040) and (b >> 15) == (pattern >> 31)


def test_bf16_widening_matches_torch_for_every_pattern():
    """The oracle's bf16 -> fp32 widening, the input side of every combine and
    dot product, against torch's bf16 -> float32 conversion for all 2^16 bit
    patterns: equal bits for numbers, signed zeros, subnormals and infinities;
    NaN stays NaN with its sign (payloads pass through a Python float here)."""
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = np.array([oracle.bf16_to_f32(int(b)) for b in pats], np.float32)
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 127 and np.array_equal(np.isnan(got), nan)   # 7-bit payloads, two signs
    np.testing.assert_array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    np.testing.assert_array_equal(np.signbit(got[nan]), np.signbit(ref[nan]))


def test_unpermute_k1_is_single_rounded_product():
    """k = 1: out = bf16(RN32(p * x)); torch's fp32 multiply and bf16 cast."""
    w = _routed(64, 40, 8, 1, seed=3)
    idx = w.topk_idx.numpy()
    m, _ = oracle.row_id_map(idx, 8)
    x = _bits(w.x)
    P, _ = oracle.permute(x, None, idx, m)
    p = (w.probs * 0.0 + torch.rand(64, 1, generator=torch.Generator().manual_seed(9)))
    y = oracle.unpermute(P, p.numpy(), idx, m)
    exp = _bits((w.x.float() * p).to(torch.bfloat16))
    np.testing.assert_array_equal(y, exp)
    # unit weight (probs omitted): permute then unpermute is the identity
    y1 = oracle.unpermute(P, None, idx, m)
    np.testing.assert_array_equal(y1, x)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 6, 8])
def test_unpermute_unit_probs_k_copies(k):
    """Unit weights over k identical copies: j*x is exact in fp32 for bf16 x,
    so the result is bf16(k*x) (torch cast of the exact product)."""
    E = 12
    w = _routed(50, 33, E, k, seed=k)
    idx = w.topk_idx.numpy()
    m, _ = oracle.row_id_map(idx, E)
    P, _ = oracle.permute(_bits(w.x), None, idx, m)
    y = oracle.unpermute(P, None, idx, m)
    ones = np.ones((50, k), np.float32)
    y2 = oracle.unpermute(P, ones, idx, m)
    exp = _bits((w.x.float() * k).to(torch.bfloat16))
    np.testing.assert_array_equal(y, exp)
    np.testing.assert_array_equal(y2, exp)


@pytest.mark.parametrize("seed", [0, 1])
def test_unpermute_exact_rational_fma_chain(seed):
    """Each step acc = RN32(p_j * x_j + acc) computed with exact rationals,
    in slot order from zero, then bf16 by torch's cast.  Catches a dropped
    fusion (mul-then-add), a reversed slot order or a wrong start value."""
    T, H, E, k = 6, 12, 10, 5
    w = _routed(T, H, E, k, seed=100 + seed)
    idx = w.topk_idx.numpy()
    probs = w.probs.numpy()
    m, _ = oracle.row_id_map(idx, E)
    rng = np.random.default_rng(seed)
    P = _bits(torch.from_numpy(rng.standard_normal((T * k, H)).astype(np.float32))
              .to(torch.bfloat16))
    y = oracle.unpermute(P, probs, idx, m)
    Pf = _bf16_to_f32(P)
    acc_f = np.zeros((T, H), np.float32)
    for t in range(T):
        for h in range(H):
            acc = Fraction(0)
            for j in range(k):
                r = m[idx[t, j], t]
                acc = _rn_f32(Fraction(float(probs[t, j])) * Fraction(float(Pf[r, h])) + acc)
            acc_f[t, h] = float(acc)
    np.testing.assert_array_equal(y, _to_bf16_torch(acc_f))


# -------------------------------------------------- unpermute backward -----

def test_unpermute_bwd_act_grad_and_prob_grad():
    T, H, E, k = 40, 72, 16, 4
    w = _routed(T, H, E, k, seed=21)
    idx = w.topk_idx.numpy()
    m, _ = oracle.row_id_map(idx, E)
    _, _, rows = _brute_rows(idx, E)
    rng = np.random.default_rng(1)
    fwd_in = _bits(torch.from_numpy(rng.standard_normal((T * k, H)).astype(np.float32))
                   .to(torch.bfloat16))
    dy = _bits(w.dy)
    d_in, d_p = oracle.unpermute_bwd(dy, fwd_in, w.probs.numpy(), idx, m)
    # act grad: torch fp32 multiply, then torch bf16 cast, scattered to rows
    prod = (w.dy.float()[:, None, :] * w.probs[:, :, None]).to(torch.bfloat16)
    exp = np.empty((T * k, H), np.uint16)
    exp[rows.ravel()] = _bits(prod.reshape(T * k, H))
    np.testing.assert_array_equal(d_in, exp)
    # prob grad: numpy float64 dot of the widened rows
    fi = _bf16_to_f32(fwd_in).astype(np.float64)
    g = _bf16_to_f32(dy).astype(np.float64)
    ref = np.einsum("tjh,th->tj", fi[rows], g)
    scale = np.einsum("tjh,th->tj", np.abs(fi[rows]), np.abs(g))
    # an fp64 sum rounded once to fp32: within half an fp32 ulp of the numpy
    # value, up to the fp64 rounding of either sum (far below 1e-12 of S)
    assert np.all(np.abs(d_p.astype(np.float64) - ref) <= 2.0 ** -24 * np.abs(ref) + 1e-12 * scale)
    # crafted: the row (2^24, 1, -2^24) against (1, 1, 1) dots to exactly 1; a
    # sum kept in fp32 gives 0 (2^24 + 1 rounds back to 2^24)
    idx1 = np.array([[0]], np.int32)
    m1, _ = oracle.row_id_map(idx1, 1)
    _, p1 = oracle.unpermute_bwd(np.array([[0x3F80] * 3], np.uint16),
                                 np.array([[0x4B80, 0x3F80, 0xCB80]], np.uint16),
                                 np.ones((1, 1), np.float32), idx1, m1)
    assert float(p1[0, 0]) == 1.0
    # without probs the scatter is a bitwise copy
    d_in0, d_p0 = oracle.unpermute_bwd(dy, None, None, idx, m)
    exp0 = np.empty_like(exp)
    exp0[rows.ravel()] = np.repeat(dy, k, axis=0)
    np.testing.assert_array_equal(d_in0, exp0)
    assert d_p0 is None


# ---------------------------------------------------- permute backward -----

def test_permute_bwd_slot_order_sum():
    T, H, E, k = 30, 20, 11, 6
    w = _routed(T, H, E, k, seed=31)
    idx = w.topk_idx.numpy()
    m, _ = oracle.row_id_map(idx, E)
    _, _, rows = _brute_rows(idx, E)
    rng = np.random.default_rng(2)
    dP_t = torch.from_numpy(rng.standard_normal((T * k, H)).astype(np.float32)).to(torch.bfloat16)
    dpp = rng.standard_normal(T * k).astype(np.float32)
    dx, dprob = oracle.permute_bwd(_bits(dP_t), dpp, idx, m)
    acc = torch.zeros(T, H, dtype=torch.float32)
    rr = torch.from_numpy(rows)
    for j in range(k):                        # torch fp32 adds, slot order
        acc = acc + dP_t.float()[rr[:, j]]
    np.testing.assert_array_equal(dx, _bits(acc.to(torch.bfloat16)))
    np.testing.assert_array_equal(dprob, dpp[rows])
    # closed form: gradient rows that are k copies of dY sum to bf16(k*dY)
    dP_copy, _ = oracle.permute(_bits(w.dy), None, idx, m)
    dx2, _ = oracle.permute_bwd(dP_copy, None, idx, m)
    np.testing.assert_array_equal(dx2, _bits((w.dy.float() * k).to(torch.bfloat16)))
    # crafted: slots (in column order, not expert order) carry 2^24, 1, -2^24.
    # In slot order the fp32 sum is (2^24 + 1 -> 2^24, ties to even) - 2^24 = 0;
    # summed backwards or by expert it is 1.
    idx3 = np.array([[2, 0, 1]], np.int32)
    m3, _ = oracle.row_id_map(idx3, 3)
    d3 = np.zeros((3, 1), np.uint16)
    for j, v in enumerate((0x4B80, 0x3F80, 0xCB80)):
        d3[m3[idx3[0, j], 0], 0] = v
    dx3, _ = oracle.permute_bwd(d3, None, idx3, m3)
    assert int(dx3[0, 0]) == 0x0000


# ------------------------------------- (3) chunk sort-and-pad / restore ----

def _brute_chunk_rows(sizes, order, R, A, out_cap):
    """Padded destination rows by list concatenation, group by group."""
    src_off = np.concatenate([[0], np.cumsum(sizes)])[:-1]
    rows, offs = [], []
    for g in range(len(order) // R):
        offs.append(len(rows))
        grp = []
        for q in range(g * R, (g + 1) * R):
            c = order[q]
            grp += list(range(src_off[c], src_off[c] + sizes[c]))
        while len(grp) % A:
            grp.append(-1)
        rows += grp
    offs.append(len(rows))
    rows += [-1] * (out_cap - len(rows))
    return np.array(rows, np.int32), np.array(offs, np.int32)


def test_chunk_map_brute_force_small():
    rng = np.random.default_rng(5)
    for trial in range(400):
        R = int(rng.integers(1, 4))
        G = int(rng.integers(1, 4))
        C = R * G
        A = int(rng.choice([1, 2, 4, 3]))
        sizes = rng.integers(0, 4, C).astype(np.int32)
        order = rng.permutation(C).astype(np.int32)
        n = int(sizes.sum())
        slack = int(rng.integers(0, 5))
        out_cap = int(np.sum(-(-np.add.reduceat(sizes[order], np.arange(0, C, R)) // A) * A)) + slack
        row_map, offs = oracle.chunk_map(sizes, order, R, A, n + slack, out_cap)
        ref_rows, ref_offs = _brute_chunk_rows(sizes, order, R, A, out_cap)
        np.testing.assert_array_equal(row_map, ref_rows)
        np.testing.assert_array_equal(offs, ref_offs)


def test_chunk_copies_roundtrip_and_special_cases():
    w = workloads.chunked(600, seed=7, H=24, num_ranks=3, num_experts=4, align=8, num_empty=3)
    x = _bits(w.x)
    s = w.split_sizes.numpy()
    q = w.sorted_idx.numpy()
    p = w.probs.numpy()
    out, op, rm, offs = oracle.sort_chunks_and_pad(x, p, s, q, 3, 8, w.out_cap)
    ref_rows, ref_offs = _brute_chunk_rows(s, q, 3, 8, w.out_cap)
    np.testing.assert_array_equal(rm, ref_rows)
    np.testing.assert_array_equal(offs, ref_offs)
    mapped = ref_rows >= 0
    np.testing.assert_array_equal(out[mapped], x[ref_rows[mapped]])
    assert not out[~mapped].any() and not op[~mapped].any()
    np.testing.assert_array_equal(op[mapped], p[ref_rows[mapped]])
    pg = np.diff(offs)
    ng = np.add.reduceat(s[q], np.arange(0, len(q), 3))
    assert np.all(pg % 8 == 0) and np.all(ng <= pg) and np.all(pg < ng + 8)
    back, bp = oracle.unpad_and_restore_chunks(out, op, rm, s, w.N_cap)
    np.testing.assert_array_equal(back, x)                 # restore . pad = id
    np.testing.assert_array_equal(bp, p)
    # backward of the pad drops padding-row gradients; of the restore, zero
    # gradient on padding rows
    gpad = np.random.default_rng(0).integers(0, 2 ** 16, out.shape).astype(np.uint16)
    d_in, _ = oracle.sort_chunks_and_pad_bwd(gpad, None, rm, s, w.N_cap)
    np.testing.assert_array_equal(d_in[ref_rows[mapped]], gpad[mapped])
    d_pad, _ = oracle.unpad_and_restore_chunks_bwd(x, None, rm, w.out_cap)
    assert not d_pad[~mapped].any()
    np.testing.assert_array_equal(d_pad[mapped], x[ref_rows[mapped]])


def test_chunk_alignment_one_identity_order_is_memcpy():
    s = np.array([3, 0, 5, 2, 4, 1], np.int32)
    q = np.arange(6, dtype=np.int32)
    x = np.arange(15 * 4, dtype=np.float32).reshape(15, 4)
    out, _, rm, offs = oracle.sort_chunks_and_pad(x, None, s, q, 2, 1, 15)
    np.testing.assert_array_equal(out, x)
    np.testing.assert_array_equal(rm, np.arange(15))
    # A = 1 with a shuffled order is a pure chunk permutation
    q2 = np.array([5, 4, 3, 2, 1, 0], np.int32)
    out2, _, rm2, _ = oracle.sort_chunks_and_pad(x, None, s, q2, 3, 1, 15)
    src = np.concatenate([[0], np.cumsum(s)])
    exp = np.concatenate([x[src[c]:src[c] + s[c]] for c in q2])
    np.testing.assert_array_equal(out2, exp)


def test_chunk_restore_zero_tail_and_errors():
    s = np.array([2, 1, 0, 3], np.int32)          # 6 tokens in a buffer of 9
    q = np.array([1, 3, 0, 2], np.int32)
    x = np.arange(9 * 2, dtype=np.uint16).reshape(9, 2) + 1
    out, _, rm, offs = oracle.sort_chunks_and_pad(x, None, s, q, 2, 4, 12)
    np.testing.assert_array_equal(offs, [0, 4, 8])
    back, _ = oracle.unpad_and_restore_chunks(out, None, rm, s, 9)
    np.testing.assert_array_equal(back[:6], x[:6])
    assert not back[6:].any()
    with pytest.raises(oracle.OracleError):      # order is not a permutation
        oracle.chunk_map(s, np.array([0, 0, 1, 2], np.int32), 2, 4, 9, 12)
    with pytest.raises(oracle.OracleError):      # negative size
        oracle.chunk_map(np.array([2, -1, 0, 3], np.int32), q, 2, 4, 9, 12)
    with pytest.raises(oracle.OracleError):      # padded groups exceed capacity
        oracle.chunk_map(s, q, 2, 4, 9, 7)
    with pytest.raises(oracle.OracleError):      # tokens exceed the input buffer
        oracle.chunk_map(s, q, 2, 4, 5, 12)
    # the restore's token total past its buffer is the same capacity overflow
    # (reading Q14: capacity overflow is an error, outputs unspecified)
    with pytest.raises(oracle.OracleError) as ei:
        oracle.unpad_and_restore_chunks(out, None, rm, np.array([2, 1, 0, 7], np.int32), 9)
    assert ei.value.code == 6
    # an all-empty group takes no rows
    s0 = np.array([0, 0, 2, 1], np.int32)
    _, offs0 = oracle.chunk_map(s0, np.arange(4, dtype=np.int32), 2, 4, 3, 8)
    np.testing.assert_array_equal(offs0, [0, 0, 4])



def test_chunk_restore_stale_map():
    """A row map saved for a larger routing, restored with smaller split sizes
    (TransformerEngine PR "Fuse MoE chunk sorting and padding", Changes: the
    restore reuses the saved map).  Entries that name a source row at or past
    the new token total are dropped and reported (status 4); the restored
    buffer is still the defined one, built here by a direct walk over the map:
    zero rows from the token total on, every other mapped row copied."""
    s_big = np.array([3, 2, 0, 4, 1, 2], np.int32)     # 12 tokens
    q = np.array([1, 3, 5, 0, 2, 4], np.int32)
    n_cap, out_cap = 14, 24
    x = (np.arange(n_cap * 3, dtype=np.uint16).reshape(n_cap, 3) + 1)
    padded, pp, rm, _ = oracle.sort_chunks_and_pad(x, np.arange(n_cap, dtype=np.float32) + 1,
                                                   s_big, q, 2, 4, out_cap)
    s_small = np.array([2, 1, 0, 2, 1, 1], np.int32)   # 7 tokens: a stale map
    n_act = int(s_small.sum())
    exp = np.zeros((n_cap, 3), np.uint16)
    exp_p = np.zeros(n_cap, np.float32)
    stale = 0
    for d in range(out_cap):
        src = int(rm[d])
        if 0 <= src < n_act:
            exp[src] = padded[d]
            exp_p[src] = pp[d]
        elif src >= n_act:
            stale += 1
    assert stale > 0
    back, back_p, st = oracle.unpad_and_restore_chunks(padded, pp, rm, s_small, n_cap,
                                                      with_status=True)
    assert st == 4
    np.testing.assert_array_equal(back, exp)
    np.testing.assert_array_equal(back_p, exp_p)
    # the backward of the pad is the same restore, with the same rule
    d_in, d_in_p, st2 = oracle.sort_chunks_and_pad_bwd(padded, pp, rm, s_small, n_cap,
                                                       with_status=True)
    assert st2 == 4
    np.testing.assert_array_equal(d_in, exp)
    np.testing.assert_array_equal(d_in_p, exp_p)
    # the map that belongs to the sizes restores without a status
    back2, _, st3 = oracle.unpad_and_restore_chunks(padded, None, rm, s_big, n_cap,
                                                    with_status=True)
    assert st3 == 0
    np.testing.assert_array_equal(back2[:12], x[:12])


def test_thread_count_does_not_change_results():
    """The per-token loops give the same bits on one thread and on many."""
    w = workloads.random_routed(96, 40, 12, 3, seed=11)
    idx, pr = w.topk_idx.numpy(), w.probs.numpy()
    xb, dyb = workloads.bf16_bits(w.x), workloads.bf16_bits(w.dy)
    rm, _ = oracle.row_id_map(idx, 12)
    before = oracle.threads()
    outs = []
    try:
        for n in (1, max(2, before)):
            oracle.set_threads(n)
            P, pp = oracle.permute(xb, pr, idx, rm)
            y = oracle.unpermute(P, pr, idx, rm)
            ye = oracle.unpermute_ep(P, pr, idx, rm, 4, True, True)
            dP, dp = oracle.unpermute_bwd(dyb, P, pr, idx, rm)
            dx, dpp = oracle.permute_bwd(dP, pp, idx, rm)
            outs.append([P, pp, y, ye, dP, dp, dx, dpp])
    finally:
        oracle.set_threads(before)
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)

def _one_token_unpermute(x_vals, p_vals):
    """Unpermute of a single token whose k slots carry rows x_vals (exact
    bf16 values, one hidden element) with weights p_vals."""
    k = len(x_vals)
    idx = np.arange(k, dtype=np.int32)[None, :]
    m, _ = oracle.row_id_map(idx, k)
    P = _to_bf16_torch(np.array(x_vals, np.float32))[:, None]
    assert np.array_equal(_bf16_to_f32(P[:, 0]), np.array(x_vals, np.float32))
    probs = None if p_vals is None else np.array([p_vals], np.float32)
    return int(oracle.unpermute(P, probs, idx, m)[0, 0])


def test_unpermute_crafted_fusion_survives_bf16():
    """acc0 = -(1 - 2^-14 + 2^-20); slot 1 adds (1 - 2^-7 + 2^-20)(1 + 2^-7)
    = 1 - 2^-14 + 2^-20 + 2^-27.  One rounding leaves exactly 2^-27 (bf16
    0x3200); rounding the product first loses 2^-27 and gives +0."""
    p0 = 1.0 - 2.0 ** -14 + 2.0 ** -20
    p1 = 1.0 - 2.0 ** -7 + 2.0 ** -20
    assert np.float32(p0) == p0 and np.float32(p1) == p1
    assert _one_token_unpermute([-1.0, 1.0 + 2.0 ** -7], [p0, p1]) == 0x3200


def test_unpermute_crafted_slot_order():
    """Slots (2^30, -2^30, 1) summed in slot order give 1 (0x3F80); summed in
    the reverse order the 1 is absorbed by -2^30 and the result is 0."""
    assert _one_token_unpermute([2.0 ** 30, -(2.0 ** 30), 1.0], None) == 0x3F80
    assert _one_token_unpermute([2.0 ** 30, -(2.0 ** 30), 1.0], [1, 1, 1]) == 0x3F80


def test_unpermute_starts_from_positive_zero():
    """All contributions -0: (+0) + (-0) = +0 under round-to-nearest."""
    assert _one_token_unpermute([-0.0, -0.0], None) == 0x0000
    assert _one_token_unpermute([-0.0, -0.0], [0.5, 0.25]) == 0x0000
    assert _one_token_unpermute([-0.0], None) == 0x0000


# ------------------------------------------- EP rank-ordered combine -------

def _rn(q: Fraction, mant_bits: int, min_exp: int = -126) -> Fraction:
    """Round an exact rational to mant_bits significant bits (ties to even),
    with the subnormal quantum of a format whose smallest normal exponent is
    min_exp; independent of the oracle's conversions."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, min_exp)
    quantum = Fraction(2) ** (e - (mant_bits - 1))
    m = a / quantum
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * quantum


def _bf16_bits_of(q: Fraction, negative: bool = None) -> int:
    """bf16 pattern of RN8(q): sign kept for a zero result (RN of a tiny
    negative is -0), infinity above the largest finite bf16."""
    neg = (q < 0) if negative is None else negative
    r = _rn(abs(q), 8)
    if r > Fraction(255) * Fraction(2) ** 120:
        mag = 0x7F80
    else:
        mag = int(np.array([float(r)], np.float32).view(np.uint32)[0] >> 16)
    return mag | (0x8000 if neg else 0)


def _ep_reference(P, probs, idx, m, ep, bf16_partials, fp64_cross):
    """The rank-ordered combine with exact rationals: fp32 FMAs as RN24 of the
    exact p*x + acc, bf16 partials as RN8, fp32 / fp64 rank sums as RN24 / RN53."""
    T, k = idx.shape
    E = m.shape[0]
    per = E // ep
    H = P.shape[1]
    Pf = _bf16_to_f32(P)
    out = np.empty((T, H), np.uint16)
    for t in range(T):
        for h in range(H):
            total = Fraction(0)
            for rank in range(ep):
                acc = Fraction(0)
                for j in range(k):
                    e = int(idx[t, j])
                    if e // per != rank:
                        continue
                    p = Fraction(1) if probs is None else Fraction(float(probs[t, j]))
                    acc = _rn(p * Fraction(float(Pf[m[e, t], h])) + acc, 24)
                if bf16_partials:
                    acc = _rn(acc, 8)
                total = _rn(total + acc, 53, -1022) if fp64_cross else _rn(total + acc, 24)
            out[t, h] = _bf16_bits_of(total)
    return out


@pytest.mark.parametrize("ep,bf16_partials,fp64_cross", [(2, True, False), (4, True, True),
                                                         (4, False, False), (8, False, True),
                                                         (1, True, False)])
def test_unpermute_ep_exact_rational(ep, bf16_partials, fp64_cross):
    T, H, E, k = 5, 6, 8, 4
    w = _routed(T, H, E, k, seed=200 + ep)
    idx = w.topk_idx.numpy()
    m, _ = oracle.row_id_map(idx, E)
    rng = np.random.default_rng(ep)
    P = _to_bf16_torch(rng.standard_normal((T * k, H)).astype(np.float32))
    got = oracle.unpermute_ep(P, w.probs.numpy(), idx, m, ep, bf16_partials, fp64_cross)
    ref = _ep_reference(P, w.probs.numpy(), idx, m, ep, bf16_partials, fp64_cross)
    np.testing.assert_array_equal(got, ref)


def test_unpermute_ep_one_rank_is_the_plain_combine():
    w = _routed(60, 40, 16, 6, seed=210)
    idx = w.topk_idx.numpy()
    m, _ = oracle.row_id_map(idx, 16)
    P = _to_bf16_torch(np.random.default_rng(3).standard_normal((360, 40)).astype(np.float32))
    plain = oracle.unpermute(P, w.probs.numpy(), idx, m)
    for partials in (True, False):
        for fp64 in (True, False):
            np.testing.assert_array_equal(
                oracle.unpermute_ep(P, w.probs.numpy(), idx, m, 1, partials, fp64), plain)


def _one_token_ep(x_vals, p_vals, experts, E, ep, partials, fp64):
    k = len(x_vals)
    idx = np.array([experts], np.int32)
    m, _ = oracle.row_id_map(idx, E)
    P = np.zeros((k, 1), np.uint16)
    bits = _to_bf16_torch(np.array(x_vals, np.float32))
    for j in range(k):
        P[m[experts[j], 0], 0] = bits[j]
    probs = None if p_vals is None else np.array([p_vals], np.float32)
    return int(oracle.unpermute_ep(P, probs, idx, m, ep, partials, fp64)[0, 0])


def test_unpermute_ep_crafted_rank_order():
    """Slots (2^30 -> rank 1, 1 -> rank 0, -2^30 -> rank 1): by rank the 1 is
    added to the cancelled rank-1 partial (result 1); in plain slot order it is
    absorbed by 2^30 (result 0)."""
    x = [2.0 ** 30, 1.0, -(2.0 ** 30)]
    assert _one_token_ep(x, None, [2, 0, 3], 4, 2, True, False) == 0x3F80
    assert _one_token_unpermute(x, None) == 0x0000


def test_unpermute_ep_crafted_ranks_added_in_ascending_order():
    """Partials 2^24, 1, -2^24 on ranks 0, 1, 2 (one slot each): added from +0
    in ascending rank order ([MCORE-BI] unpermute_with_bf16_rank_partials, the
    rank-ordered cross-rank sum), fp32 rounds 2^24 + 1 back to 2^24 (a tie, to
    even) and the result is 0; in descending order it would be 1.  In fp64 the
    sum is exact in any order: 1."""
    x = [2.0 ** 24, 1.0, -(2.0 ** 24)]
    for partials in (True, False):
        assert _one_token_ep(x, None, [0, 1, 2], 3, 3, partials, False) == 0x0000
        assert _one_token_ep(x, None, [0, 1, 2], 3, 3, partials, True) == 0x3F80


def test_unpermute_ep_crafted_fp64_cross_sum():
    """Partials 1+2^-8, 2^-30, 2^-30 (fp32 partials): the fp32 rank sum drops
    the small terms and lands on the bf16 tie 1+2^-8 (-> even, 0x3F80); the
    fp64 sum keeps them, above the tie (-> 0x3F81).  With bf16 partials the
    first partial already rounds to 1 (tie to even)."""
    x = [1.0, 2.0 ** -30, 2.0 ** -30]
    p = [1.0 + 2.0 ** -8, 1.0, 1.0]
    assert _one_token_ep(x, p, [0, 1, 2], 3, 3, False, False) == 0x3F80
    assert _one_token_ep(x, p, [0, 1, 2], 3, 3, False, True) == 0x3F81
    assert _one_token_ep(x, p, [0, 1, 2], 3, 3, True, True) == 0x3F80


def test_f64_to_bf16_matches_exact_rounding():
    rng = np.random.default_rng(4)
    vals = np.concatenate([rng.standard_normal(2000),
                           rng.standard_normal(300) * 1e-39, rng.standard_normal(300) * 1e-43,
                           rng.standard_normal(300) * 3e38,
                           np.array([0.0, 1.0 + 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -40,
                                     3.3961e38, 3.3962e38, 2.0 ** -134, 2.0 ** -134 * 1.5])])
    for v in vals:
        got = oracle.f64_to_bf16(float(v))
        exp = _bf16_bits_of(Fraction(float(v)), negative=bool(np.signbit(v)))
        assert got == exp, (v, hex(got), hex(exp))


# ------------------------------------------------ top-k softmax router -----

@pytest.mark.parametrize("T,E,k,dtype", [(50, 32, 4, "f32"), (40, 64, 6, "bf16"),
                                         (20, 8, 8, "f32"), (30, 5, 1, "bf16")])
def test_topk_softmax_against_stable_sort_and_softmax(T, E, k, dtype):
    import scipy.special
    rng = np.random.default_rng(T + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 1] = logits[:, 0]                      # forced ties
    if dtype == "bf16":
        lb = _to_bf16_torch(logits)
        lv = _bf16_to_f32(lb)
        idx, probs = oracle.topk_softmax(lb, k)
    else:
        lv = logits
        idx, probs = oracle.topk_softmax(logits, k)
    ref_idx = np.argsort(-lv.astype(np.float64), axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(idx, ref_idx)      # descending, ties to lower index
    sel = np.take_along_axis(lv.astype(np.float64), ref_idx, axis=1)
    ref_p = scipy.special.softmax(sel, axis=1)
    np.testing.assert_allclose(probs, ref_p, rtol=2e-7, atol=0)


def test_topk_softmax_bwd_against_autograd():
    T, E, k = 30, 16, 4
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, probs = oracle.topk_softmax(logits, k)
    dp = rng.standard_normal((T, k)).astype(np.float32)
    got = oracle.topk_softmax_bwd(dp, probs, idx, E)
    lt = torch.from_numpy(logits.astype(np.float64)).requires_grad_(True)
    sel = torch.gather(lt, 1, torch.from_numpy(idx.astype(np.int64)))
    torch.softmax(sel, dim=1).backward(torch.from_numpy(dp.astype(np.float64)))
    np.testing.assert_allclose(got, lt.grad.numpy(), rtol=1e-6, atol=1e-7)
    selected = np.zeros((T, E), bool)
    np.put_along_axis(selected, idx.astype(np.int64), True, axis=1)
    assert np.all(got[~selected] == 0)


def _nearest_bf16(bits, ref):
    """bits (uint16) round ref (float64) to nearest: within half a bf16 ulp."""
    got = _bf16_to_f32(np.asarray(bits, np.uint16)).astype(np.float64)
    ref = np.asarray(ref, np.float64)
    ulp = np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 8)   # bf16: 8 significant bits
    return np.abs(got - ref) <= 0.5 * ulp * (1 + 1e-9) + 1e-300


def test_topk_softmax_bf16_weights_round_to_nearest():
    """Weights in bf16 (the activation dtype) are the exact softmax rounded
    once to nearest; fp32 routing keeps them in fp32."""
    import scipy.special
    rng = np.random.default_rng(11)
    T, E, k = 60, 48, 6
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, w16 = oracle.topk_softmax(logits, k, prob_bytes=2)
    idx32, w32 = oracle.topk_softmax(logits, k)
    np.testing.assert_array_equal(idx, idx32)
    sel = np.take_along_axis(logits.astype(np.float64), idx.astype(np.int64), axis=1)
    assert w16.dtype == np.uint16
    assert _nearest_bf16(w16, scipy.special.softmax(sel, axis=1)).all()


@pytest.mark.parametrize("logits,k,expect", [
    ([0.5, -1.0, 2.0], 1, [0x3F80]),                        # one expert: weight 1
    ([1.0, 1.0, -3.0], 2, [0x3F00, 0x3F00]),                 # tie: 1/2 each
    ([0.0, 0.0, 0.0, 0.0, -1.0], 4, [0x3E80] * 4),           # four equal: 1/4
    ([0.0, float(np.log(3.0)), -5.0], 2, [0x3F40, 0x3E80]),  # 3/4 and 1/4
    # exp of the logits themselves would overflow (first) or underflow (second):
    # only the differences from the largest give these weights
    ([1000.0, 1000.0, -3.0], 2, [0x3F00, 0x3F00]),
    ([-1000.0, -1000.0 + float(np.log(3.0)), -2000.0], 2, [0x3F40, 0x3E80]),
])
def test_topk_softmax_bf16_closed_forms(logits, k, expect):
    _, w = oracle.topk_softmax(np.array([logits], np.float32), k, prob_bytes=2)
    assert [int(v) for v in w[0]] == expect


def test_topk_softmax_bwd_bf16_closed_form_and_autograd():
    # w = (1/2, 1/2), dp = (1, 0): dot = 1/2, gradients +1/4 and -1/4 (exact)
    w = np.array([[0x3F00, 0x3F00]], np.uint16)
    dp = np.array([[0x3F80, 0x0000]], np.uint16)
    g = oracle.topk_softmax_bwd(dp, w, np.array([[2, 0]], np.int32), 3, logit_bytes=2)
    assert [int(v) for v in g[0]] == [0xBE80, 0x0000, 0x3E80]
    # bf16 in, bf16 out: the fp64 gradient of the widened inputs, rounded to nearest
    T, E, k = 25, 12, 3
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, w16 = oracle.topk_softmax(logits, k, prob_bytes=2)
    dp16 = _to_bf16_torch(rng.standard_normal((T, k)).astype(np.float32))
    got = oracle.topk_softmax_bwd(dp16, w16, idx, E, logit_bytes=2)
    wv = _bf16_to_f32(w16).astype(np.float64)
    dv = _bf16_to_f32(dp16).astype(np.float64)
    # softmax Jacobian diag(w) - w w^T applied to dp, token by token
    gsel = np.stack([(np.diag(wv[t]) - np.outer(wv[t], wv[t])) @ dv[t] for t in range(T)])
    ref = np.zeros((T, E))
    np.put_along_axis(ref, idx.astype(np.int64), gsel, axis=1)
    assert _nearest_bf16(got, ref).all()


# ------------------------------------------------ TE mask-map interop ------

def _brute_mask_map(mask, num_out=-1):
    """Rows by enumerating routed (expert, token) pairs expert-major; then per
    token the kept rows in descending order.  Independent of the oracle."""
    T, E = mask.shape
    dense = -np.ones((T, E), np.int64)
    es, ts = np.nonzero(mask.T)              # expert-major, tokens ascending
    dense[ts, es] = np.arange(es.size)
    if num_out >= 0:
        dense[dense >= num_out] = -1
    out = []
    for t in range(T):
        pairs = sorted(((int(dense[t, e]), e) for e in range(E) if dense[t, e] >= 0),
                       reverse=True)
        out.append(pairs)
    return out


def _check_mask_map(m, pairs, E):
    for t, pr in enumerate(pairs):
        n = len(pr)
        assert m[t, 2 * E] == n
        assert list(m[t, :n]) == [r for r, _ in pr]
        assert list(m[t, E:E + n]) == [e for _, e in pr]


@pytest.mark.parametrize("dtype", [np.int32, np.uint8])
def test_mask_map_worked_example(dtype):
    """The worked example's third pass, entry for entry (unused entries -1)."""
    g = _read_golden("make_row_id_map_worked_example.txt")
    mask = np.array(g["routing_map"], dtype=dtype)
    T, E = mask.shape
    m, off = oracle.mask_row_id_map(mask)
    for t, row in enumerate(g["pass3"]):
        for i, v in enumerate(row):
            assert m[t, i] == (-1 if v == "r" else int(v)), (t, i)
    np.testing.assert_array_equal(off, [0, 3, 5, 7])


@pytest.mark.parametrize("T,E,density,num_out", [(40, 7, 0.3, -1), (65, 16, 0.5, -1),
                                                 (33, 5, 0.9, 20), (50, 12, 0.4, 0),
                                                 (20, 3, 1.0, 59), (1, 1, 1.0, -1)])
def test_mask_map_brute_force(T, E, density, num_out):
    rng = np.random.default_rng(T * E)
    mask = (rng.random((T, E)) < density).astype(np.int32)
    m, off = oracle.mask_row_id_map(mask, num_out)
    _check_mask_map(m, _brute_mask_map(mask, num_out), E)
    counts = mask.sum(0)
    kept = np.minimum(np.concatenate([[0], np.cumsum(counts)]),
                      counts.sum() if num_out < 0 else num_out)
    np.testing.assert_array_equal(off, kept)


def test_mask_map_every_small_mask():
    """All 2^(T*E) masks of 3 tokens x 3 experts, with and without dropping."""
    for bits in range(1 << 9):
        mask = np.array([(bits >> i) & 1 for i in range(9)], np.uint8).reshape(3, 3)
        for num_out in (-1, 0, 2, 5):
            m, _ = oracle.mask_row_id_map(mask, num_out)
            _check_mask_map(m, _brute_mask_map(mask, num_out), 3)


def test_mask_permute_equals_topk_permute():
    """A mask with k experts per token moves rows exactly as the top-k permute
    with those experts (the row maps agree); probs are read from [T][E]."""
    rng = np.random.default_rng(3)
    T, E, k, H = 37, 9, 3, 16
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    mask = np.zeros((T, E), np.int32)
    np.put_along_axis(mask, idx.astype(np.int64), 1, axis=1)
    probs_te = rng.random((T, E)).astype(np.float32) + 0.1
    probs_k = np.take_along_axis(probs_te, idx.astype(np.int64), axis=1)
    x = _to_bf16_torch(rng.standard_normal((T, H)).astype(np.float32))
    mm, _ = oracle.mask_row_id_map(mask)
    out, out_p = oracle.mask_permute(x, probs_te, mm, T * k)
    rm, _ = oracle.row_id_map(idx, E)
    ref, ref_p = oracle.permute(x, probs_k, idx, rm)
    np.testing.assert_array_equal(out, ref)
    np.testing.assert_array_equal(out_p.view(np.uint32), ref_p.view(np.uint32))


def test_mask_permute_zero_prob_pads():
    """A routed slot whose prob is 0 (or -0) gets a zero row; its prob is still
    stored.  Without probs every routed slot is a copy."""
    x = np.array([[0x3F80, 0x4000], [0xC040, 0x3F00]], np.uint16)
    mask = np.array([[1, 1, 0], [0, 1, 1]], np.int32)
    probs = np.array([[0.5, 0.0, 0.0], [0.0, -0.0, 0.25]], np.float32)
    mm, _ = oracle.mask_row_id_map(mask)      # rows: e0:t0=0, e1:t0=1,t1=2, e2:t1=3
    out, out_p = oracle.mask_permute(x, probs, mm, 4)
    np.testing.assert_array_equal(out, [[0x3F80, 0x4000], [0, 0], [0, 0], [0xC040, 0x3F00]])
    np.testing.assert_array_equal(out_p.view(np.uint32),
                                  np.array([0.5, 0.0, -0.0, 0.25], np.float32).view(np.uint32))
    out2, _ = oracle.mask_permute(x, None, mm, 4)
    np.testing.assert_array_equal(out2, x[[0, 0, 1, 1]])


def test_mask_unpermute_adds_in_descending_row_order():
    """Rows 2^24, 1, -2^24 for experts 0, 1, 2 of one token: in descending row
    order (-2^24 + 1) + 2^24 = 1 exactly; ascending would round 2^24 + 1
    to 2^24 and give 0."""
    inp = np.array([[0x4B80], [0x3F80], [0xCB80]], np.uint16)   # 2^24, 1, -2^24
    mm, _ = oracle.mask_row_id_map(np.ones((1, 3), np.int32))
    out, _ = oracle.mask_unpermute(inp, None, mm)
    assert int(out[0, 0]) == 0x3F80


def test_mask_unpermute_multiplies_then_adds():
    """Product (1+2^-7)(1+2^-23) rounds in fp32 before the add: the sum with
    -(1+2^-7) is 2^-23 (bf16 0x3400); a fused multiply-add would keep
    2^-23(1+2^-7) (0x3401).  Map order: expert 1's row, then expert 0's."""
    inp = np.array([[0x3F81], [0xBF81]], np.uint16)     # rows of e0 and e1
    mp = np.array([[1.0 + 2.0 ** -23, 1.0]], np.float32)
    mm, _ = oracle.mask_row_id_map(np.ones((1, 2), np.int32))
    out, _ = oracle.mask_unpermute(inp, mp, mm)
    assert int(out[0, 0]) == 0x3400


def test_mask_unpermute_probs_scatter_and_identity():
    rng = np.random.default_rng(8)
    T, E, H = 30, 6, 12
    mask = np.zeros((T, E), np.int32)
    mask[np.arange(T), rng.integers(0, E, T)] = 1          # one expert per token
    mm, _ = oracle.mask_row_id_map(mask)
    x = _to_bf16_torch(rng.standard_normal((T, H)).astype(np.float32))
    perm, _ = oracle.mask_permute(x, None, mm, T)
    pp = rng.random(T).astype(np.float32)
    y, up = oracle.mask_unpermute(perm, None, mm, pp)
    np.testing.assert_array_equal(y, x)                     # one slot, no probs: identity
    rows = mm[:, 0]
    ref = np.zeros((T, E), np.float32)
    ref[np.arange(T), mm[:, E]] = pp[rows]
    np.testing.assert_array_equal(up, ref)


def test_mask_unpermute_bwd_against_direct_products():
    rng = np.random.default_rng(9)
    T, E, H = 20, 5, 24
    mask = (rng.random((T, E)) < 0.5).astype(np.int32)
    mm, _ = oracle.mask_row_id_map(mask)
    R = int(mask.sum())
    mp = rng.random((T, E)).astype(np.float32)
    g = _to_bf16_torch(rng.standard_normal((T, H)).astype(np.float32))
    fin = _to_bf16_torch(rng.standard_normal((R, H)).astype(np.float32))
    d_in, dmp = oracle.mask_unpermute_bwd(g, fin, mp, mm)
    gv, fv = _bf16_to_f32(g), _bf16_to_f32(fin)
    for t in range(T):
        for e in range(E):
            if not mask[t, e]:
                assert dmp[t, e] == 0.0
    for t, pairs in enumerate(_brute_mask_map(mask)):
        for r, e in pairs:
            np.testing.assert_array_equal(d_in[r], _to_bf16_torch(gv[t] * mp[t, e]))
            ref = float(np.dot(fv[r].astype(np.float64), gv[t].astype(np.float64)))
            assert abs(dmp[t, e] - ref) <= 2.0 ** -24 * abs(ref) + 1e-45


# --------------------------------------------- quantized rows with scales ---

def _route_rows(idx, rm):
    T, k = idx.shape
    return rm[idx.astype(np.int64), np.arange(T)[:, None]]      # [T][k] destination rows


@pytest.mark.parametrize("H,block,sdt", [(256, 128, "f32"), (200, 64, "f32"), (384, 128, "e8m0"),
                                         (16, 16, "f32")])
def test_permute_scaled_moves_fp8_rows_and_scales(H, block, sdt):
    """FP8 rows and their scale rows land at the destinations of the (pinned)
    row map, byte for byte; the dequantized rows are the source's."""
    rng = np.random.default_rng(H)
    T, E, k = 45, 11, 3
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32))
    q, sc = workloads.quantize_fp8_rows(x, block, torch.float32 if sdt == "f32"
                                        else torch.float8_e8m0fnu)
    qb = q.view(torch.uint8).numpy()
    sb = sc.view(torch.uint8).numpy().reshape(T, -1) if sdt == "e8m0" else sc.numpy()
    probs = rng.random((T, k)).astype(np.float32)
    rm, _ = oracle.row_id_map(idx, E)
    out, out_s, out_p = oracle.permute_scaled(qb, sb, probs, idx, rm)
    rows = _route_rows(idx, rm)
    for t in range(T):
        for j in range(k):
            r = rows[t, j]
            np.testing.assert_array_equal(out[r], qb[t])
            np.testing.assert_array_equal(out_s[r], np.ascontiguousarray(sb[t]).view(np.uint8))
            assert out_p[r] == probs[t, j]
    # dequantized: the permuted FP8 rows times their permuted scales equal the source's
    src = q.float() * sc.float().repeat_interleave(block, dim=1)[:, :H]
    outq = torch.from_numpy(out).view(torch.float8_e4m3fn).float()
    outs = (torch.from_numpy(out_s).view(torch.float8_e8m0fnu) if sdt == "e8m0"
            else torch.from_numpy(out_s.view(np.float32))).float()
    dst = outq * outs.repeat_interleave(block, dim=1)[:, :H]
    torch.testing.assert_close(dst[torch.from_numpy(rows.ravel())],
                               src.repeat_interleave(k, dim=0), rtol=0, atol=0)


def test_permute_scaled_on_bf16_rows_is_the_permute():
    rng = np.random.default_rng(2)
    T, E, k, H = 30, 8, 2, 24
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = _to_bf16_torch(rng.standard_normal((T, H)).astype(np.float32))
    probs = rng.random((T, k)).astype(np.float32)
    rm, _ = oracle.row_id_map(idx, E)
    out, out_s, out_p = oracle.permute_scaled(x, None, probs, idx, rm)
    ref, ref_p = oracle.permute(x, probs, idx, rm)
    np.testing.assert_array_equal(out.view(np.uint16), ref)
    np.testing.assert_array_equal(out_p, ref_p)
    assert out_s is None


def test_mask_permute_scaled_zero_prob_keeps_scale():
    """The padding rule zeroes the data row only; the scale row still moves."""
    x = np.array([[1, 2, 3, 4], [5, 6, 7, 8]], np.uint8)
    sc = np.array([[0.5], [2.0]], np.float32)
    mask = np.array([[1, 1], [1, 0]], np.int32)        # rows: e0: t0=0, t1=1; e1: t0=2
    probs = np.array([[0.3, 0.0], [0.7, 0.0]], np.float32)
    mm, _ = oracle.mask_row_id_map(mask)
    out, out_s, out_p = oracle.mask_permute_scaled(x, sc, probs, mm, 3)
    np.testing.assert_array_equal(out, [[1, 2, 3, 4], [5, 6, 7, 8], [0, 0, 0, 0]])
    np.testing.assert_array_equal(out_s.view(np.float32).ravel(), [0.5, 2.0, 0.5])
    np.testing.assert_array_equal(out_p, np.array([0.3, 0.7, 0.0], np.float32))
    # bf16 rows, no scales: the same as the mask-map permute
    xb = _to_bf16_torch(np.random.default_rng(1).standard_normal((2, 6)).astype(np.float32))
    o1, _, _ = oracle.mask_permute_scaled(xb, None, probs, mm, 3)
    o2, _ = oracle.mask_permute(xb, probs, mm, 3)
    np.testing.assert_array_equal(o1.view(np.uint16), o2)
