"""GPU parity: every entry point of the C ABI against the CPU oracle.

Integer, index and copy results must match bit for bit, and so must the
fixed slot-order unpermute (and the permute backward, which is the same
combine with unit weights).  The only tolerance is the prob-grad row dot
product, whose summation order the pages leave open: |g - ref| <= 1e-5 * S
with S = sum_h |fwd_in[r][h] * d_out[t][h]|.

Outputs are pre-filled with sentinels (bf16 0x7FC1, int -2, a NaN payload
for fp32) so an element the kernels fail to write shows up as a mismatch.
Every workload is compared with the oracle in full, the 16384 x 7168 one
included (the oracle runs its tokens on all host cores).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
S_BF16 = 0x7FC1
S_F32 = np.array([0x7FC00123], np.uint32).view(np.float32)[0]


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import unpermute_moe_make_amd as mod
    return mod


# ----------------------------------------------------------------- helpers --

def bits(t):
    return workloads.bf16_bits(t.cpu()) if t.dtype == torch.bfloat16 else t.cpu().numpy()


def sentinel_bf16(shape):
    t = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    t.view(torch.int16).fill_(S_BF16)
    return t


def sentinel_f32(shape):
    t = torch.empty(shape, dtype=torch.float32, device=DEV)
    t.view(torch.int32).fill_(int(np.array([S_F32]).view(np.int32)[0]))
    return t


def sentinel_i32(shape):
    return torch.full(shape, -2, dtype=torch.int32, device=DEV)


def f32_bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def assert_bits_equal(got, exp, what):
    got = np.asarray(got)
    exp = np.asarray(exp)
    assert got.shape == exp.shape, (what, got.shape, exp.shape)
    if got.dtype == np.float32:
        got, exp = f32_bits(got), f32_bits(exp)
    bad = np.nonzero(got != exp)
    n = bad[0].size
    assert n == 0, f"{what}: {n} mismatches, first at {[b[:5] for b in bad]}"


def oracle_rows(idx, row_map):
    """r(t, j) from the oracle's row map."""
    T, k = idx.shape
    return row_map[idx, np.arange(T)[:, None]]


def sub_problem(idx, sample, E=None):
    """Top-k and a row map for a token subset whose rows are i*k + j."""
    sidx = idx[sample]
    s, k = sidx.shape
    E = int(idx.max()) + 1 if E is None else E
    smap = np.full((E, s), -1, np.int32)
    for i in range(s):
        for j in range(k):
            smap[sidx[i, j], i] = i * k + j
    return sidx, smap


def dprob_ok(got, fwd_rows, dy_rows, ref, chunk=256):
    """|got - ref| <= 1e-5 * sum_h |a*b| per (token, slot); fwd_rows [T][k][H]
    and dy_rows [T][H] bf16 bits, taken a chunk of tokens at a time."""
    worst = 0.0
    for t0 in range(0, got.shape[0], chunk):
        sl = slice(t0, t0 + chunk)
        a = (fwd_rows[sl].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        b = (dy_rows[sl].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        scale = np.einsum("tjh,th->tj", np.abs(a), np.abs(b))
        err = np.abs(got[sl].astype(np.float64) - ref[sl].astype(np.float64))
        worst = max(worst, float(np.max(err / np.maximum(scale, 1e-300))))
        assert np.all(err <= 1e-5 * scale + 1e-37), f"prob grad off by {worst:.3g} of scale"
    return worst


_CACHE = {}


def routed(name):
    if name not in _CACHE:
        w = workloads.ROUTED[name]()
        m_, off = oracle.row_id_map(w.topk_idx.numpy(), w.num_experts)
        _CACHE[name] = (w, m_, off)
    return _CACHE[name]


def to_dev(w):
    return (w.x.to(DEV), w.topk_idx.to(DEV), w.probs.to(DEV),
            None if w.dy is None else w.dy.to(DEV))


# ------------------------------------------------------------ (1) row map --

@pytest.mark.parametrize("name", ["tiny", "finegrain", "skewed"])
def test_row_map_configs(m, name):
    w, ref_map, ref_off = routed(name)
    say(f"row_map {name} T={w.T} E={w.num_experts} k={w.k}")
    idx = w.topk_idx.to(DEV)
    rm = sentinel_i32((w.num_experts, w.T))
    off = sentinel_i32((w.num_experts + 1,))
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    m.moe_make_row_id_map(idx, w.num_experts, row_id_map=rm, expert_offsets=off, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert_bits_equal(rm.cpu().numpy(), ref_map, "row_id_map")
    assert_bits_equal(off.cpu().numpy(), ref_off, "expert_offsets")


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (63, 5, 2), (64, 5, 2), (255, 8, 3), (256, 8, 3),
                                   (257, 8, 3), (1000, 3, 3), (700, 2048, 8), (300, 64, 9),
                                   (130, 100, 64), (5000, 1, 1), (4097, 257, 7),
                                   (16384, 3, 2), (16385, 8, 2), (70000, 64, 4),
                                   (300000, 2, 1), (512, 64, 8), (4096, 2, 1), (683, 9, 6),
                                   (8, 512, 8), (8, 513, 8), (1024, 4, 4)])
def test_row_map_edges(m, T, E, k):
    say(f"row_map edge T={T} E={E} k={k}")
    w = workloads.random_routed(T, 8, E, k, seed=T * 31 + E, with_dy=False, zipf_s=0.7)
    ref_map, ref_off = oracle.row_id_map(w.topk_idx.numpy(), E)
    rm = sentinel_i32((E, T))
    off = sentinel_i32((E + 1,))
    m.moe_make_row_id_map(w.topk_idx.to(DEV), E, row_id_map=rm, expert_offsets=off)
    assert_bits_equal(rm.cpu().numpy(), ref_map, "row_id_map")
    assert_bits_equal(off.cpu().numpy(), ref_off, "expert_offsets")


@pytest.mark.parametrize("T,E,k", [(16, 32, 4), (300, 64, 6)])
def test_row_map_unaligned_indices(m, T, E, k):
    """topk_idx 4 bytes past a 16-byte boundary: the map takes its two-launch
    form even for short token ranges; same result."""
    say(f"row_map unaligned topk_idx T={T} E={E} k={k}")
    w = workloads.random_routed(T, 8, E, k, seed=T + 7, with_dy=False)
    ref_map, ref_off = oracle.row_id_map(w.topk_idx.numpy(), E)
    buf = torch.empty(T * k + 4, dtype=torch.int32, device=DEV)
    idx = buf[1:1 + T * k].view(T, k)
    idx.copy_(w.topk_idx)
    assert idx.data_ptr() % 16 == 4
    rm = sentinel_i32((E, T))
    off = sentinel_i32((E + 1,))
    m.moe_make_row_id_map(idx, E, row_id_map=rm, expert_offsets=off)
    assert_bits_equal(rm.cpu().numpy(), ref_map, "row_id_map")
    assert_bits_equal(off.cpu().numpy(), ref_off, "expert_offsets")


def test_row_map_empty(m):
    say("row_map T=0")
    off = sentinel_i32((9,))
    m.moe_make_row_id_map(torch.zeros((0, 2), dtype=torch.int32, device=DEV), 8,
                          expert_offsets=off)
    assert_bits_equal(off.cpu().numpy(), np.zeros(9, np.int32), "expert_offsets")


def test_routed_ops_no_tokens(m):
    """T = 0: every routed call, forward and backward, in every form, accepts
    the empty (NULL-pointer) tensors, returns OK with empty outputs and
    leaves the status clear; the maps' expert offsets are all zero."""
    say("routed ops with T=0")
    T, k, E, H = 0, 4, 8, 64
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    idx = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    rm, off = m.moe_make_row_id_map(idx, E, dev_status=st)
    assert rm.shape == (E, T) and bool((off == 0).all())
    x = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    probs = torch.empty((T, k), dtype=torch.float32, device=DEV)
    out, out_p = m.moe_permute(x, idx, rm, probs, dev_status=st)
    assert out.shape == (0, H) and out_p.shape == (0,)
    assert m.moe_unpermute(out, idx, rm, probs, dev_status=st).shape == (0, H)
    for fp64 in (False, True):
        assert m.moe_unpermute_ep(out, idx, rm, 2, probs, fp64_cross=fp64,
                                  dev_status=st).shape == (0, H)
    d_in, d_p = m.moe_unpermute_bwd(x, idx, rm, probs, out, dev_status=st)
    assert d_in.shape == (0, H) and d_p.shape == (0, k)
    d_x, d_pp = m.moe_permute_bwd(out, idx, rm, out_p, dev_status=st)
    assert d_x.shape == (0, H) and d_pp.shape == (0, k)
    x8 = torch.empty((T, H), dtype=torch.float8_e4m3fn, device=DEV)
    sc = torch.empty((T, 2), dtype=torch.float32, device=DEV)
    o8, osc, _ = m.moe_permute_scaled(x8, idx, rm, sc, dev_status=st)
    assert o8.shape == (0, H) and osc.shape == (0, 2)
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    ti, tp = m.moe_topk_softmax(logits, k)
    assert ti.shape == (0, k) and tp.shape == (0, k)
    assert m.moe_topk_softmax_bwd(tp, tp, ti, E, dev_status=st).shape == (0, E)
    mask = torch.zeros((T, E), dtype=torch.bool, device=DEV)
    mm, moff = m.moe_make_mask_row_id_map(mask)
    assert mm.shape == (0, 2 * E + 1) and bool((moff == 0).all())
    pe = torch.empty((T, E), dtype=torch.float32, device=DEV)
    mo, mop = m.moe_permute_mask(x, mm, 0, pe, dev_status=st)
    assert mo.shape == (0, H) and mop.shape == (0,)
    mu = m.moe_unpermute_mask(mo, mm, pe, dev_status=st)
    mu = mu[0] if isinstance(mu, tuple) else mu
    assert mu.shape == (0, H)
    mb = m.moe_unpermute_mask_bwd(x, mo, pe, mm, dev_status=st)
    assert mb[0].shape == (0, H)
    ms = m.moe_permute_mask_scaled(x8, mm, 0, sc, dev_status=st)
    assert ms[0].shape == (0, H)
    torch.cuda.synchronize()
    assert int(st.item()) == 0


def test_row_map_bad_routing_sets_status(m):
    say("row_map bad expert / duplicate expert")
    idx = torch.tensor([[0, 1], [2, 9], [3, 3], [1, 0]], dtype=torch.int32, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    m.moe_make_row_id_map(idx, 4, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == m.DEV_BAD_EXPERT | m.DEV_DUP_EXPERT
    # the permute sees the bad expert too and skips it without faulting
    x = torch.ones(4, 16, dtype=torch.bfloat16, device=DEV)
    rm, _ = m.moe_make_row_id_map(torch.tensor([[0, 1], [2, 3], [3, 2], [1, 0]],
                                               dtype=torch.int32, device=DEV), 4)
    st.zero_()
    m.moe_permute(x, idx, rm, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & m.DEV_BAD_EXPERT


@pytest.mark.parametrize("T,H,E,k", [(50, 136, 16, 4), (4096, 4096, 64, 8)])
def test_bad_routing_row_ops(m, T, H, E, k):
    """Routing faults only the device sees -- an expert index out of range,
    and map entries past the rows or -1 for a routed token -- in every top-k
    row op.  Each op reports both status bits, leaves the faulty slots'
    rows unwritten, and matches the oracle (run on the sound routing) on
    every other slot and on every token the faults do not touch.  The second
    size takes the streaming paths (the two-launch backward included)."""
    say(f"bad routing row ops T={T} H={H} E={E} k={k}")
    w = workloads.random_routed(T, H, E, k, seed=T + H)
    idx_np = w.topk_idx.numpy()
    ref_map, _ = oracle.row_id_map(idx_np, E)
    n = T * k
    r_all = oracle_rows(idx_np, ref_map)
    a, b, c = 3, T // 2, T - 2
    bad_idx = idx_np.copy()
    bad_idx[a, 1] = E + 3
    bad_map = ref_map.copy()
    bad_map[idx_np[b, 2], b] = n + 11
    bad_map[idx_np[c, 0], c] = -1
    skipped = [(a, 1), (b, 2), (c, 0)]
    skip_rows = np.array([r_all[t, j] for t, j in skipped])
    keep_rows = np.setdiff1d(np.arange(n), skip_rows)
    ok_tok = np.setdiff1d(np.arange(T), [a, b, c])
    x, _, probs, dy = to_dev(w)
    idx = torch.from_numpy(bad_idx).to(DEV)
    rm = torch.from_numpy(bad_map).to(DEV)
    xb, pb = workloads.bf16_bits(w.x), w.probs.numpy()

    def status(call):
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        call(st)
        torch.cuda.synchronize()
        s = int(st.item())
        assert s & m.DEV_BAD_EXPERT and s & m.DEV_BAD_ROW, s

    def rows_ok(got, ref, what):
        assert_bits_equal(got[keep_rows], ref[keep_rows], what)
        assert np.all(got[skip_rows] == S_BF16), f"{what}: a faulty slot's row was written"

    # permute (+probs)
    out, out_p = sentinel_bf16((n, H)), sentinel_f32((n,))
    status(lambda st: m.moe_permute(x, idx, rm, probs, out=out, out_probs=out_p, dev_status=st))
    o, op = oracle.permute(xb, pb, idx_np, ref_map)
    rows_ok(bits(out), o, "permute")
    assert_bits_equal(out_p.cpu().numpy()[keep_rows], op[keep_rows], "permuted probs")
    assert np.all(f32_bits(out_p.cpu().numpy()[skip_rows]) == f32_bits(np.array([S_F32])))

    # weighted unpermute, and the EP combine
    P = workloads.random_rows(n, H, seed=H + 1, device=DEV)
    Pb = bits(P)
    y = sentinel_bf16((T, H))
    status(lambda st: m.moe_unpermute(P, idx, rm, probs, out=y, dev_status=st))
    ref = oracle.unpermute(Pb, pb, idx_np, ref_map)
    assert_bits_equal(bits(y)[ok_tok], ref[ok_tok], "unpermute")
    y = sentinel_bf16((T, H))
    status(lambda st: m.moe_unpermute_ep(P, idx, rm, 4, probs, out=y, dev_status=st))
    ref = oracle.unpermute_ep(Pb, pb, idx_np, ref_map, 4)
    assert_bits_equal(bits(y)[ok_tok], ref[ok_tok], "unpermute_ep")

    # unpermute backward, with and without prob gradients
    d_in, d_p = sentinel_bf16((n, H)), sentinel_f32((T, k))
    status(lambda st: m.moe_unpermute_bwd(dy, idx, rm, probs, P, d_in=d_in, d_probs=d_p,
                                          dev_status=st))
    dyb = workloads.bf16_bits(w.dy)
    ref_in, ref_p = oracle.unpermute_bwd(dyb, Pb, pb, idx_np, ref_map)
    rows_ok(bits(d_in), ref_in, "unpermute_bwd act grad")
    got_p = d_p.cpu().numpy().copy()
    for t, j in skipped:
        got_p[t, j] = ref_p[t, j]
    dprob_ok(got_p, Pb[r_all.reshape(-1)].reshape(T, k, H), dyb, ref_p)
    d_in = sentinel_bf16((n, H))
    status(lambda st: m.moe_unpermute_bwd(dy, idx, rm, probs, P, probs_grad=False, d_in=d_in,
                                          dev_status=st))
    rows_ok(bits(d_in), ref_in, "unpermute_bwd act grad without prob grads")

    # permute backward
    dpp = torch.randn(n, generator=torch.Generator().manual_seed(H)).to(DEV)
    d_x, d_p = sentinel_bf16((T, H)), sentinel_f32((T, k))
    status(lambda st: m.moe_permute_bwd(P, idx, rm, dpp, d_x=d_x, d_probs=d_p, dev_status=st))
    ref_x, ref_pp = oracle.permute_bwd(Pb, dpp.cpu().numpy(), idx_np, ref_map)
    assert_bits_equal(bits(d_x)[ok_tok], ref_x[ok_tok], "permute_bwd")
    keep = np.ones((T, k), bool)
    for t, j in skipped:
        keep[t, j] = False
    assert_bits_equal(d_p.cpu().numpy()[keep], ref_pp[keep], "permute_bwd probs")

    # FP8 rows with their scales
    q, sc = workloads.quantize_fp8_rows(w.x, 128 if H % 128 == 0 else 8)
    qo = torch.empty((n, H), dtype=q.dtype, device=DEV)
    qo.view(torch.uint8).fill_(0x5A)
    so = torch.full((n, sc.shape[1]), -7.0, device=DEV)
    status(lambda st: m.moe_permute_scaled(q.to(DEV), idx, rm, sc.to(DEV), out=qo, out_scale=so,
                                           dev_status=st))
    src = r_all.reshape(-1).astype(np.int64)
    tok = np.repeat(np.arange(T), k)
    keep_flat = np.isin(src, keep_rows)
    qb = q.view(torch.uint8).numpy()
    got = qo.view(torch.uint8).cpu().numpy()
    np.testing.assert_array_equal(got[src[keep_flat]], qb[tok[keep_flat]])
    assert np.all(got[skip_rows] == 0x5A)
    got_s = so.cpu().numpy()
    np.testing.assert_array_equal(got_s[src[keep_flat]].view(np.uint32),
                                  sc.numpy()[tok[keep_flat]].view(np.uint32))
    assert np.all(got_s[skip_rows] == -7.0)


# --------------------------------------------- (2) permute, (4) unpermute --

@pytest.mark.parametrize("name", ["tiny", "finegrain", "skewed"])
def test_permute_configs(m, name):
    w, ref_map, _ = routed(name)
    T, H, k = w.T, w.H, w.k
    say(f"permute {name} T={T} H={H} k={k}")
    x, idx, probs, _ = to_dev(w)
    rm = torch.from_numpy(ref_map).to(DEV)
    out = sentinel_bf16((T * k, H))
    out_p = sentinel_f32((T * k,))
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    m.moe_permute(x, idx, rm, probs, out=out, out_probs=out_p, dev_status=st)
    rows = torch.from_numpy(oracle_rows(w.topk_idx.numpy(), ref_map).astype(np.int64)).to(DEV)
    exp = torch.empty_like(out)
    exp[rows.flatten()] = x.repeat_interleave(k, dim=0)         # torch scatter, full size
    assert torch.equal(out.view(torch.int16), exp.view(torch.int16))
    exp_p = torch.empty_like(out_p)
    exp_p[rows.flatten()] = probs.flatten()
    assert torch.equal(out_p.view(torch.int32), exp_p.view(torch.int32))
    assert int(st.item()) == 0
    o, op = oracle.permute(workloads.bf16_bits(w.x), w.probs.numpy(), w.topk_idx.numpy(),
                           ref_map)
    assert_bits_equal(bits(out), o, "permute")
    assert_bits_equal(out_p.cpu().numpy(), op, "permuted probs")


@pytest.mark.parametrize("name", ["tiny", "finegrain", "skewed"])
@pytest.mark.parametrize("weighted", [True, False])
def test_unpermute_configs(m, name, weighted):
    w, ref_map, _ = routed(name)
    T, H, k = w.T, w.H, w.k
    say(f"unpermute {name} weighted={weighted}")
    _, idx, probs, _ = to_dev(w)
    rm = torch.from_numpy(ref_map).to(DEV)
    P = workloads.random_rows(T * k, H, seed=77, device=DEV)
    out = sentinel_bf16((T, H))
    m.moe_unpermute(P, idx, rm, probs if weighted else None, out=out)
    p_np = w.probs.numpy() if weighted else None
    ref = oracle.unpermute(bits(P), p_np, w.topk_idx.numpy(), ref_map)
    assert_bits_equal(bits(out), ref, "unpermute")


@pytest.mark.parametrize("name,ep", [("tiny", 4), ("finegrain", 8), ("finegrain", 64),
                                     ("skewed", 8), ("skewed", 32)])
@pytest.mark.parametrize("partials,fp64", [(True, False), (True, True), (False, False)])
def test_unpermute_ep_configs(m, name, ep, partials, fp64):
    w, ref_map, _ = routed(name)
    T, H, k, E = w.T, w.H, w.k, w.num_experts
    say(f"unpermute_ep {name} ep={ep} bf16_partials={partials} fp64={fp64}")
    _, idx, probs, _ = to_dev(w)
    rm = torch.from_numpy(ref_map).to(DEV)
    P = workloads.random_rows(T * k, H, seed=81, device=DEV)
    out = sentinel_bf16((T, H))
    m.moe_unpermute_ep(P, idx, rm, ep, probs, bf16_partials=partials, fp64_cross=fp64, out=out)
    ref = oracle.unpermute_ep(bits(P), w.probs.numpy(), w.topk_idx.numpy(), ref_map, ep,
                              partials, fp64)
    assert_bits_equal(bits(out), ref, "unpermute_ep")


def test_unpermute_ep_one_rank_equals_unpermute(m):
    w, ref_map, _ = routed("finegrain")
    say("unpermute_ep ep=1 vs unpermute")
    _, idx, probs, _ = to_dev(w)
    rm = torch.from_numpy(ref_map).to(DEV)
    P = workloads.random_rows(w.T * w.k, w.H, seed=82, device=DEV)
    y = m.moe_unpermute(P, idx, rm, probs)
    for partials in (True, False):
        for fp64 in (True, False):
            y1 = m.moe_unpermute_ep(P, idx, rm, 1, probs, bf16_partials=partials,
                                    fp64_cross=fp64)
            assert torch.equal(y.view(torch.int16), y1.view(torch.int16))


@pytest.mark.parametrize("T,H,E,k,ep", [(37, 7, 12, 3, 3), (64, 64, 16, 9, 4), (40, 136, 80, 64, 8),
                                        (9, 20480, 8, 8, 8), (50, 24, 6, 6, 6), (33, 72, 40, 5, 1)])
def test_unpermute_ep_edges(m, T, H, E, k, ep):
    say(f"unpermute_ep edge T={T} H={H} E={E} k={k} ep={ep}")
    w = workloads.random_routed(T, H, E, k, seed=H + 7 * k)
    ref_map, _ = oracle.row_id_map(w.topk_idx.numpy(), E)
    _, idx, probs, _ = to_dev(w)
    rm = torch.from_numpy(ref_map).to(DEV)
    P = workloads.random_rows(T * k, H, seed=6, device=DEV)
    for partials, fp64, use_p in ((True, False, True), (False, True, True), (True, True, False)):
        y = m.moe_unpermute_ep(P, idx, rm, ep, probs if use_p else None, bf16_partials=partials,
                               fp64_cross=fp64, out=sentinel_bf16((T, H)))
        ref = oracle.unpermute_ep(bits(P), w.probs.numpy() if use_p else None,
                                  w.topk_idx.numpy(), ref_map, ep, partials, fp64)
        assert_bits_equal(bits(y), ref, f"unpermute_ep {partials} {fp64} {use_p}")


@pytest.mark.parametrize("name", ["tiny", "finegrain", "skewed"])
def test_unpermute_bwd_configs(m, name):
    w, ref_map, _ = routed(name)
    T, H, k = w.T, w.H, w.k
    say(f"unpermute_bwd {name}")
    _, idx, probs, dy = to_dev(w)
    rm = torch.from_numpy(ref_map).to(DEV)
    fwd_in = workloads.random_rows(T * k, H, seed=78, device=DEV)
    d_in = sentinel_bf16((T * k, H))
    d_p = sentinel_f32((T, k))
    m.moe_unpermute_bwd(dy, idx, rm, probs, fwd_in, d_in=d_in, d_probs=d_p)
    r_all = oracle_rows(w.topk_idx.numpy(), ref_map)
    dy_rows = workloads.bf16_bits(w.dy)
    ref_in, ref_p = oracle.unpermute_bwd(dy_rows, bits(fwd_in), w.probs.numpy(),
                                         w.topk_idx.numpy(), ref_map)
    assert_bits_equal(bits(d_in), ref_in, "unpermute_bwd act grad")
    del ref_in
    # the forward rows of each (token, slot), for the prob-grad bound
    fin_rows = bits(fwd_in[torch.from_numpy(r_all.flatten().astype(np.int64)).to(DEV)])
    worst = dprob_ok(d_p.cpu().numpy(), fin_rows.reshape(T, k, H), dy_rows, ref_p)
    say(f"  prob-grad worst error / scale = {worst:.3g}")
    # unweighted: plain scatter of d_out
    d_in0 = sentinel_bf16((T * k, H))
    m.moe_unpermute_bwd(dy, idx, rm, None, None, d_in=d_in0)
    exp = torch.empty_like(d_in0)
    exp[torch.from_numpy(r_all.flatten().astype(np.int64)).to(DEV)] = \
        dy.repeat_interleave(k, dim=0)
    assert torch.equal(d_in0.view(torch.int16), exp.view(torch.int16))


@pytest.mark.parametrize("T,H,E,k", [(4096, 4096, 64, 16), (4096, 7176, 32, 8),
                                     (2048, 20480, 16, 4)])
def test_unpermute_bwd_streaming_shapes(m, T, H, E, k):
    """Calls past the streaming threshold, in full: the two-launch backward
    with 16 slots (two batches of dot products) and with rows of 897 16-byte
    units, the fused kernel for rows longer than one workgroup pass, and the
    scatter alone when no prob gradient is asked for (row slices at 20480)."""
    say(f"unpermute_bwd streaming T={T} H={H} E={E} k={k}")
    w = workloads.random_routed(T, H, E, k, seed=H + 3 * k)
    ref_map, _ = oracle.row_id_map(w.topk_idx.numpy(), E)
    _, idx, probs, dy = to_dev(w)
    rm = torch.from_numpy(ref_map).to(DEV)
    fwd_in = workloads.random_rows(T * k, H, seed=H + 5, device=DEV)
    d_in = sentinel_bf16((T * k, H))
    d_p = sentinel_f32((T, k))
    m.moe_unpermute_bwd(dy, idx, rm, probs, fwd_in, d_in=d_in, d_probs=d_p)
    dy_rows = workloads.bf16_bits(w.dy)
    ref_in, ref_p = oracle.unpermute_bwd(dy_rows, bits(fwd_in), w.probs.numpy(),
                                         w.topk_idx.numpy(), ref_map)
    assert_bits_equal(bits(d_in), ref_in, "unpermute_bwd act grad")
    r_all = oracle_rows(w.topk_idx.numpy(), ref_map)
    fin_rows = bits(fwd_in[torch.from_numpy(r_all.flatten().astype(np.int64)).to(DEV)])
    worst = dprob_ok(d_p.cpu().numpy(), fin_rows.reshape(T, k, H), dy_rows, ref_p)
    say(f"  prob-grad worst error / scale = {worst:.3g}")
    del fin_rows
    d_in1 = sentinel_bf16((T * k, H))
    _, none = m.moe_unpermute_bwd(dy, idx, rm, probs, fwd_in, probs_grad=False, d_in=d_in1)
    assert none is None
    assert_bits_equal(bits(d_in1), ref_in, "unpermute_bwd act grad without prob grads")


@pytest.mark.parametrize("name", ["tiny", "finegrain", "skewed"])
def test_permute_bwd_configs(m, name):
    w, ref_map, _ = routed(name)
    T, H, k = w.T, w.H, w.k
    say(f"permute_bwd {name}")
    _, idx, _, _ = to_dev(w)
    rm = torch.from_numpy(ref_map).to(DEV)
    dP = workloads.random_rows(T * k, H, seed=79, device=DEV)
    dpp = torch.randn(T * k, generator=torch.Generator().manual_seed(80)).to(DEV)
    d_x = sentinel_bf16((T, H))
    d_p = sentinel_f32((T, k))
    m.moe_permute_bwd(dP, idx, rm, dpp, d_x=d_x, d_probs=d_p)
    ref_x, ref_p = oracle.permute_bwd(bits(dP), dpp.cpu().numpy(), w.topk_idx.numpy(), ref_map)
    assert_bits_equal(bits(d_x), ref_x, "permute_bwd")
    assert_bits_equal(d_p.cpu().numpy(), ref_p, "permute_bwd probs")


@pytest.mark.parametrize("T,H,E,k", [(1, 8, 2, 1), (37, 7, 9, 3), (100, 24, 16, 2),
                                     (64, 64, 12, 9), (40, 136, 80, 64), (33, 2056, 12, 5),
                                     (29, 4104, 12, 5), (19, 8200, 10, 3),
                                     (20, 7168, 16, 4), (9, 20480, 8, 8), (17, 20481, 4, 2),
                                     (300, 512, 32, 1), (50, 96, 6, 6), (3, 8, 64, 64),
                                     (17, 1, 4, 2)])
def test_row_kernels_edges(m, T, H, E, k):
    say(f"row kernels edge T={T} H={H} E={E} k={k}")
    w = workloads.random_routed(T, H, E, k, seed=H + k)
    ref_map, _ = oracle.row_id_map(w.topk_idx.numpy(), E)
    x, idx, probs, dy = to_dev(w)
    rm, _ = m.moe_make_row_id_map(idx, E)
    torch.cuda.synchronize()
    assert_bits_equal(rm.cpu().numpy(), ref_map, "row_id_map")
    xb, pb, ib = workloads.bf16_bits(w.x), w.probs.numpy(), w.topk_idx.numpy()
    out, out_p = m.moe_permute(x, idx, rm, probs, out=sentinel_bf16((T * k, H)),
                               out_probs=sentinel_f32((T * k,)))
    o, op = oracle.permute(xb, pb, ib, ref_map)
    assert_bits_equal(bits(out), o, "permute")
    assert_bits_equal(out_p.cpu().numpy(), op, "permuted probs")
    P = workloads.random_rows(T * k, H, seed=5, device=DEV)
    y = m.moe_unpermute(P, idx, rm, probs, out=sentinel_bf16((T, H)))
    assert_bits_equal(bits(y), oracle.unpermute(bits(P), pb, ib, ref_map), "unpermute")
    d_in, d_p = m.moe_unpermute_bwd(dy, idx, rm, probs, P, d_in=sentinel_bf16((T * k, H)),
                                    d_probs=sentinel_f32((T, k)))
    ref_in, ref_p = oracle.unpermute_bwd(workloads.bf16_bits(w.dy), bits(P), pb, ib, ref_map)
    assert_bits_equal(bits(d_in), ref_in, "unpermute_bwd")
    rows = oracle_rows(ib, ref_map)
    dprob_ok(d_p.cpu().numpy(), bits(P)[rows], workloads.bf16_bits(w.dy), ref_p)
    # without prob grads a long row may be split over several workgroups
    d_in2, none = m.moe_unpermute_bwd(dy, idx, rm, probs, P, probs_grad=False,
                                      d_in=sentinel_bf16((T * k, H)))
    assert none is None
    assert_bits_equal(bits(d_in2), ref_in, "unpermute_bwd without prob grads")
    dpp = torch.randn(T * k, generator=torch.Generator().manual_seed(3)).to(DEV)
    d_x, d_pp = m.moe_permute_bwd(P, idx, rm, dpp, d_x=sentinel_bf16((T, H)),
                                  d_probs=sentinel_f32((T, k)))
    rx, rp = oracle.permute_bwd(bits(P), dpp.cpu().numpy(), ib, ref_map)
    assert_bits_equal(bits(d_x), rx, "permute_bwd")
    assert_bits_equal(d_pp.cpu().numpy(), rp, "permute_bwd probs")


def test_permute_streaming_unaligned_rows(m):
    """A call large enough to stream (and prefetch the source row of the token
    two dispatch rounds ahead), with rows that are not whole 128-byte lines
    (7176 bf16 = 14352 bytes), in full against the oracle."""
    T, H, E, k = 6000, 7176, 40, 4
    say(f"permute streaming unaligned rows T={T} H={H} E={E} k={k}")
    w = workloads.random_routed(T, H, E, k, seed=71, with_dy=False)
    ref_map, _ = oracle.row_id_map(w.topk_idx.numpy(), E)
    x, idx, probs, _ = to_dev(w)
    rm = torch.from_numpy(ref_map).to(DEV)
    assert 2 * H * (T * k + T) > 256 << 20                  # the streaming path
    out, out_p = m.moe_permute(x, idx, rm, probs, out=sentinel_bf16((T * k, H)),
                               out_probs=sentinel_f32((T * k,)))
    o, op = oracle.permute(workloads.bf16_bits(w.x), w.probs.numpy(), w.topk_idx.numpy(),
                           ref_map)
    assert_bits_equal(bits(out), o, "permute")
    assert_bits_equal(out_p.cpu().numpy(), op, "permuted probs")
    y = m.moe_unpermute(out, idx, rm, probs, out=sentinel_bf16((T, H)))
    assert_bits_equal(bits(y), oracle.unpermute(o, w.probs.numpy(), w.topk_idx.numpy(),
                                                ref_map), "unpermute")


def test_row_kernels_misaligned_views(m):
    """Row pointers that are 2- but not 16-byte aligned take the element path."""
    T, H, E, k = 50, 64, 8, 3
    say("row kernels misaligned views")
    w = workloads.random_routed(T, H, E, k, seed=9)
    ref_map, _ = oracle.row_id_map(w.topk_idx.numpy(), E)
    idx = w.topk_idx.to(DEV)
    rm = torch.from_numpy(ref_map).to(DEV)
    xbuf = torch.empty(T * H + 1, dtype=torch.bfloat16, device=DEV)
    x = xbuf[1:].view(T, H)
    x.copy_(w.x.to(DEV))
    obuf = sentinel_bf16((T * k * H + 1,))
    out = obuf[1:].view(T * k, H)
    m.moe_permute(x, idx, rm, out=out)
    o, _ = oracle.permute(workloads.bf16_bits(w.x), None, w.topk_idx.numpy(), ref_map)
    assert_bits_equal(bits(out), o, "permute misaligned")
    ybuf = sentinel_bf16((T * H + 1,))
    y = ybuf[1:].view(T, H)
    m.moe_unpermute(out, idx, rm, w.probs.to(DEV), out=y)
    assert_bits_equal(bits(y), oracle.unpermute(o, w.probs.numpy(), w.topk_idx.numpy(), ref_map),
                      "unpermute misaligned")


def test_roundtrip_k1_identity(m):
    say("permute -> unpermute, k=1, unit weights")
    w = workloads.random_routed(1000, 2048, 16, 1, seed=4)
    x, idx, _, _ = to_dev(w)
    rm, _ = m.moe_make_row_id_map(idx, 16)
    P, _ = m.moe_permute(x, idx, rm)
    y = m.moe_unpermute(P, idx, rm)
    assert torch.equal(y.view(torch.int16), x.view(torch.int16))


def test_bitwise_repeatable(m):
    say("repeatability of the prob-grad reduction and the combine")
    w, ref_map, _ = routed("finegrain")
    _, idx, probs, dy = to_dev(w)
    rm = torch.from_numpy(ref_map).to(DEV)
    P = workloads.random_rows(w.T * w.k, w.H, seed=11, device=DEV)
    first = None
    for _ in range(5):
        y = m.moe_unpermute(P, idx, rm, probs)
        d_in, d_p = m.moe_unpermute_bwd(dy, idx, rm, probs, P)
        cur = (y.view(torch.int16).clone(), d_in.view(torch.int16).clone(),
               d_p.view(torch.int32).clone())
        if first is None:
            first = cur
        else:
            for a, b in zip(first, cur):
                assert torch.equal(a, b)


def test_two_streams_at_once(m):
    """The library keeps no state between calls: two routed chains with
    different shapes and routings, each with its own workspace, enqueued
    alternately on two streams so that they overlap, give the oracle's
    results on both."""
    say("two routed chains on two streams at once")
    cases = [(700, 2048, 64, 6, 31), (900, 1536, 32, 4, 32)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    work, outs = [], []
    for (T, H, E, k, seed) in cases:
        w = workloads.random_routed(T, H, E, k, seed=seed)
        x, idx, probs, dy = to_dev(w)
        ws = torch.empty(m.moe_make_row_id_map_workspace_bytes(T, k, E), dtype=torch.uint8,
                         device=DEV)
        work.append((w, x, idx, probs, ws))
    torch.cuda.synchronize()
    for rep in range(3):
        for i, (w, x, idx, probs, ws) in enumerate(work):
            with torch.cuda.stream(streams[i]):
                rm, off = m.moe_make_row_id_map(idx, w.num_experts, workspace=ws)
                out, out_p = m.moe_permute(x, idx, rm, probs)
                y = m.moe_unpermute(out, idx, rm, probs)
                if rep == 2:
                    outs.append((rm, out, out_p, y))
    torch.cuda.synchronize()
    for (w, _, _, _, _), (rm, out, out_p, y) in zip(work, outs):
        ib, pb = w.topk_idx.numpy(), w.probs.numpy()
        ref_map, _ = oracle.row_id_map(ib, w.num_experts)
        assert_bits_equal(rm.cpu().numpy(), ref_map, "row_id_map")
        o, op = oracle.permute(workloads.bf16_bits(w.x), pb, ib, ref_map)
        assert_bits_equal(bits(out), o, "permute")
        assert_bits_equal(out_p.cpu().numpy(), op, "permuted probs")
        assert_bits_equal(bits(y), oracle.unpermute(o, pb, ib, ref_map), "unpermute")


def test_graph_replay_routing(m):
    """Map + permute + unpermute captured once, replayed with new routings."""
    T, H, E, k = 1024, 1024, 32, 4
    say("graph replay, routing")
    idx_s = torch.empty((T, k), dtype=torch.int32, device=DEV)
    probs_s = torch.empty((T, k), dtype=torch.float32, device=DEV)
    x_s = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    rm = torch.empty((E, T), dtype=torch.int32, device=DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    ws = torch.empty(m.moe_make_row_id_map_workspace_bytes(T, k, E), dtype=torch.uint8,
                     device=DEV)
    P = torch.empty((T * k, H), dtype=torch.bfloat16, device=DEV)
    pp = torch.empty(T * k, dtype=torch.float32, device=DEV)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)

    def step():
        m.moe_make_row_id_map(idx_s, E, row_id_map=rm, expert_offsets=off, workspace=ws)
        m.moe_permute(x_s, idx_s, rm, probs_s, out=P, out_probs=pp)
        m.moe_unpermute(P, idx_s, rm, probs_s, out=y)

    w0 = workloads.random_routed(T, H, E, k, seed=1000, with_dy=False)
    idx_s.copy_(w0.topk_idx)
    probs_s.copy_(w0.probs)
    x_s.copy_(w0.x)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(8):
        w = workloads.random_routed(T, H, E, k, seed=1001 + rep, with_dy=False,
                                    zipf_s=0.3 * rep)
        idx_s.copy_(w.topk_idx)
        probs_s.copy_(w.probs)
        x_s.copy_(w.x)
        P.view(torch.int16).fill_(S_BF16)
        g.replay()
        torch.cuda.synchronize()
        ref_map, ref_off = oracle.row_id_map(w.topk_idx.numpy(), E)
        assert_bits_equal(rm.cpu().numpy(), ref_map, f"replay {rep} row map")
        assert_bits_equal(off.cpu().numpy(), ref_off, f"replay {rep} offsets")
        o, _ = oracle.permute(workloads.bf16_bits(w.x), None, w.topk_idx.numpy(), ref_map)
        assert_bits_equal(bits(P), o, f"replay {rep} permute")
        ref_y = oracle.unpermute(o, w.probs.numpy(), w.topk_idx.numpy(), ref_map)
        assert_bits_equal(bits(y), ref_y, f"replay {rep} unpermute")


def test_graph_replay_streaming_path(m):
    """The whole routed path at a size where every op streams (the two-launch
    backward included), captured once and replayed with three routings.
    Each replay equals an eager run of the same path bit for bit, prob
    gradients included, and the oracle (prob gradients within their bound)."""
    T, H, E, k = 4096, 4096, 64, 8
    n = T * k
    say(f"graph replay, streaming path T={T} H={H} E={E} k={k}")

    def buf(shape, dt):
        return torch.empty(shape, dtype=dt, device=DEV)

    idx_s, probs_s = buf((T, k), torch.int32), buf((T, k), torch.float32)
    x_s, dy_s = buf((T, H), torch.bfloat16), buf((T, H), torch.bfloat16)
    rm, off = buf((E, T), torch.int32), buf((E + 1,), torch.int32)
    ws = buf((m.moe_make_row_id_map_workspace_bytes(T, k, E),), torch.uint8)

    def outs():
        return dict(P=buf((n, H), torch.bfloat16), pp=buf((n,), torch.float32),
                    y=buf((T, H), torch.bfloat16), d_in=buf((n, H), torch.bfloat16),
                    d_p=buf((T, k), torch.float32), d_x=buf((T, H), torch.bfloat16),
                    d_pp=buf((T, k), torch.float32))

    def step(o):
        m.moe_make_row_id_map(idx_s, E, row_id_map=rm, expert_offsets=off, workspace=ws)
        m.moe_permute(x_s, idx_s, rm, probs_s, out=o["P"], out_probs=o["pp"])
        m.moe_unpermute(o["P"], idx_s, rm, probs_s, out=o["y"])
        m.moe_unpermute_bwd(dy_s, idx_s, rm, probs_s, o["P"], d_in=o["d_in"], d_probs=o["d_p"])
        m.moe_permute_bwd(o["d_in"], idx_s, rm, o["pp"], d_x=o["d_x"], d_probs=o["d_pp"])

    def load(w):
        idx_s.copy_(w.topk_idx)
        probs_s.copy_(w.probs)
        x_s.copy_(w.x)
        dy_s.copy_(w.dy)

    def host(o):
        return {key: (bits(t) if t.dtype == torch.bfloat16 else f32_bits(t.cpu().numpy()))
                for key, t in o.items()}

    g_out, e_out = outs(), outs()
    load(workloads.random_routed(T, H, E, k, seed=2000))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(g_out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(g_out)
    for rep in range(3):
        w = workloads.random_routed(T, H, E, k, seed=2001 + rep, zipf_s=0.6 * rep)
        load(w)
        for t in g_out.values():
            t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).fill_(-3)
        g.replay()
        torch.cuda.synchronize()
        got, rm_g, off_g = host(g_out), rm.cpu().numpy(), off.cpu().numpy()
        step(e_out)
        torch.cuda.synchronize()
        eager = host(e_out)
        for key in got:
            assert_bits_equal(got[key], eager[key], f"replay {rep} {key} against eager")
        idx_np, p_np = w.topk_idx.numpy(), w.probs.numpy()
        ref_map, ref_off = oracle.row_id_map(idx_np, E)
        assert_bits_equal(rm_g, ref_map, f"replay {rep} row map")
        assert_bits_equal(off_g, ref_off, f"replay {rep} offsets")
        o, op = oracle.permute(workloads.bf16_bits(w.x), p_np, idx_np, ref_map)
        assert_bits_equal(got["P"], o, f"replay {rep} permute")
        assert_bits_equal(got["pp"], f32_bits(op), f"replay {rep} permuted probs")
        assert_bits_equal(got["y"], oracle.unpermute(o, p_np, idx_np, ref_map),
                          f"replay {rep} unpermute")
        dyb = workloads.bf16_bits(w.dy)
        ref_in, ref_p = oracle.unpermute_bwd(dyb, o, p_np, idx_np, ref_map)
        assert_bits_equal(got["d_in"], ref_in, f"replay {rep} unpermute_bwd act grad")
        r_all = oracle_rows(idx_np, ref_map).reshape(-1)
        dprob_ok(got["d_p"].view(np.float32), o[r_all].reshape(T, k, H), dyb, ref_p)
        ref_x, ref_pp = oracle.permute_bwd(ref_in, op, idx_np, ref_map)
        assert_bits_equal(got["d_x"], ref_x, f"replay {rep} permute_bwd")
        assert_bits_equal(got["d_pp"], f32_bits(ref_pp), f"replay {rep} permute_bwd probs")


# ------------------------------------------------ (3) chunk sort / restore --

def _chunk_ref(cw, sizes=None):
    s = (cw.split_sizes if sizes is None else sizes).numpy()
    xb = workloads.bf16_bits(cw.x) if cw.x.dtype == torch.bfloat16 else cw.x.numpy()
    return oracle.sort_chunks_and_pad(xb, cw.probs.numpy(), s, cw.sorted_idx.numpy(),
                                      cw.chunks_per_group, cw.align, cw.out_cap)


def _run_chunks(m, cw, x, probs, sizes, order, st=None):
    out = sentinel_bf16((cw.out_cap, cw.H)) if x.dtype == torch.bfloat16 else \
        torch.full((cw.out_cap, cw.H), float("nan"), dtype=x.dtype, device=DEV)
    out_p = sentinel_f32((cw.out_cap,)) if probs.dtype == torch.float32 else \
        torch.full((cw.out_cap,), float("nan"), dtype=probs.dtype, device=DEV)
    rm = sentinel_i32((cw.out_cap,))
    off = sentinel_i32((cw.C // cw.chunks_per_group + 1,))
    m.moe_sort_chunks_and_pad(x, sizes, order, cw.chunks_per_group, cw.align, cw.out_cap, probs,
                              out=out, out_probs=out_p, row_map=rm, padded_offsets=off,
                              dev_status=st)
    return out, out_p, rm, off


def _raw(t):
    t = t.cpu()
    if t.dtype == torch.bfloat16 or t.dtype == torch.float16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy().view(np.uint32)


@pytest.mark.parametrize("name", ["chunks8k", "chunks32k"])
def test_chunks_configs(m, name):
    cw = workloads.CHUNKED[name]()
    say(f"sort_chunks_and_pad + restore {name} N={cw.N_cap} cap={cw.out_cap}")
    x, probs = cw.x.to(DEV), cw.probs.to(DEV)
    sizes, order = cw.split_sizes.to(DEV), cw.sorted_idx.to(DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, out_p, rm, off = _run_chunks(m, cw, x, probs, sizes, order, st)
    r_out, r_p, r_rm, r_off = _chunk_ref(cw)
    assert int(st.item()) == 0
    assert_bits_equal(rm.cpu().numpy(), r_rm, "row_map")
    assert_bits_equal(off.cpu().numpy(), r_off, "padded_offsets")
    assert_bits_equal(_raw(out), r_out, "padded tokens")
    assert_bits_equal(out_p.cpu().numpy(), r_p, "padded probs")
    back = sentinel_bf16((cw.N_cap, cw.H))
    back_p = sentinel_f32((cw.N_cap,))
    m.moe_unpad_and_restore_chunks(out, rm, sizes, cw.N_cap, out_p, out=back, out_probs=back_p,
                                   dev_status=st)
    ref_b, ref_bp = oracle.unpad_and_restore_chunks(r_out, r_p, r_rm, cw.split_sizes.numpy(),
                                                    cw.N_cap)
    assert_bits_equal(_raw(back), ref_b, "restored tokens")
    assert_bits_equal(back_p.cpu().numpy(), ref_bp, "restored probs")
    assert torch.equal(back.view(torch.int16), x.view(torch.int16))   # restore . pad = id
    # backwards: gradients of random bits
    gpad = workloads.random_rows(cw.out_cap, cw.H, seed=3, device=DEV)
    gpp = torch.rand(cw.out_cap, generator=torch.Generator().manual_seed(4)).to(DEV)
    d_in, d_inp = m.moe_sort_chunks_and_pad_bwd(gpad, rm, sizes, cw.N_cap, gpp,
                                                d_in=sentinel_bf16((cw.N_cap, cw.H)),
                                                d_in_probs=sentinel_f32((cw.N_cap,)))
    rd, rdp = oracle.sort_chunks_and_pad_bwd(bits(gpad), gpp.cpu().numpy(), r_rm,
                                             cw.split_sizes.numpy(), cw.N_cap)
    assert_bits_equal(bits(d_in), rd, "sort_and_pad bwd")
    assert_bits_equal(d_inp.cpu().numpy(), rdp, "sort_and_pad bwd probs")
    grest = workloads.random_rows(cw.N_cap, cw.H, seed=5, device=DEV)
    d_pad, d_padp = m.moe_unpad_and_restore_chunks_bwd(grest, rm, cw.out_cap, probs,
                                                       d_in=sentinel_bf16((cw.out_cap, cw.H)),
                                                       d_in_probs=sentinel_f32((cw.out_cap,)))
    rp_, rpp = oracle.unpad_and_restore_chunks_bwd(bits(grest), cw.probs.numpy(), r_rm,
                                                   cw.out_cap)
    assert_bits_equal(bits(d_pad), rp_, "restore bwd")
    assert_bits_equal(d_padp.cpu().numpy(), rpp, "restore bwd probs")
    assert int(st.item()) == 0


@pytest.mark.parametrize("case", ["fp32_tokens", "fp16_probs", "odd_hidden", "align1_identity",
                                  "empty_group", "short_total", "big_cap", "all_empty",
                                  "h1536", "h7168", "h7000_fp32", "wide_two_launch",
                                  "tall_one_launch", "chunks512", "chunks2048",
                                  "chunks512_two_launch"])
def test_chunk_edges(m, case):
    say(f"chunk edge {case}")
    kw = dict(N=3000, seed=50, H=256, num_ranks=4, num_experts=6, align=16, num_empty=5)
    if case == "chunks512":            # past 256 chunks: 8 per lane in the table build
        kw.update(num_ranks=8, num_experts=64, num_empty=100)
    if case == "chunks2048":           # the most chunks a call takes
        kw.update(N=20000, num_ranks=16, num_experts=128, num_empty=300, align=8)
    if case == "chunks512_two_launch":
        kw.update(N=2100, H=32768, num_ranks=8, num_experts=64, num_empty=100)
    if case == "wide_two_launch":      # a 143 MB padded buffer: map and copy launched apart
        kw.update(N=2100, H=32768)
    if case == "tall_one_launch":      # 140000 short rows: 64 rows per fused workgroup
        kw.update(N=140000, H=64)
    if case == "fp32_tokens":
        kw["dtype"] = torch.float32
    if case == "odd_hidden":
        kw["H"] = 37
    if case in ("h1536", "h7168"):     # rows of 192 and 896 16-byte units
        kw["H"] = int(case[1:])
    if case == "h7000_fp32":           # 1750 units per row
        kw["H"] = 7000
        kw["dtype"] = torch.float32
    cw = workloads.chunked(**kw)
    sizes = cw.split_sizes.clone()
    if case == "align1_identity":
        cw.align = 1
        cw.sorted_idx = torch.arange(cw.C, dtype=torch.int32)
        cw.out_cap = cw.N_cap
    if case == "empty_group":
        order = cw.sorted_idx
        for q in range(4, 8):            # every chunk of group 1 empty
            sizes[order[q]] = 0
        sizes[order[0]] += cw.N_cap - int(sizes.sum())
    if case == "short_total":
        sizes = workloads.chunk_sizes(2000, 4, 6, 5, torch.Generator().manual_seed(1))
    if case == "big_cap":
        cw.out_cap += 777
    if case == "all_empty":
        sizes = torch.zeros_like(sizes)
    cw.split_sizes = sizes
    probs = cw.probs.to(torch.float16) if case == "fp16_probs" else cw.probs
    cw.probs = probs
    x = cw.x.to(DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, out_p, rm, off = _run_chunks(m, cw, x, probs.to(DEV), sizes.to(DEV),
                                      cw.sorted_idx.to(DEV), st)
    xr = _raw(cw.x)
    pr = _raw(probs)
    r_out, r_p, r_rm, r_off = oracle.sort_chunks_and_pad(
        xr, pr, sizes.numpy(), cw.sorted_idx.numpy(), cw.chunks_per_group, cw.align,
        cw.out_cap)
    assert int(st.item()) == 0
    assert_bits_equal(rm.cpu().numpy(), r_rm, "row_map")
    assert_bits_equal(off.cpu().numpy(), r_off, "padded_offsets")
    assert_bits_equal(_raw(out), r_out, "padded tokens")
    assert_bits_equal(_raw(out_p), r_p, "padded probs")
    back, back_p = m.moe_unpad_and_restore_chunks(out, rm, sizes.to(DEV), cw.N_cap, out_p)
    ref_b, ref_bp = oracle.unpad_and_restore_chunks(r_out, r_p, r_rm, sizes.numpy(), cw.N_cap)
    assert_bits_equal(_raw(back), ref_b, "restored tokens")
    assert_bits_equal(_raw(back_p), ref_bp, "restored probs")


def test_chunk_bad_metadata_sets_status(m):
    say("chunk bad metadata")
    cw = workloads.chunked(1000, seed=51, H=64, num_ranks=2, num_experts=4, align=8,
                           num_empty=1)
    x, probs = cw.x.to(DEV), cw.probs.to(DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    bad_order = cw.sorted_idx.clone()
    bad_order[1] = bad_order[0]                        # not a permutation
    out, out_p, rm, off = _run_chunks(m, cw, x, probs, cw.split_sizes.to(DEV),
                                      bad_order.to(DEV), st)
    torch.cuda.synchronize()
    assert int(st.item()) & m.DEV_BAD_CHUNKS
    assert bool((rm == -1).all()) and bool((out.view(torch.int16) == 0).all())
    st.zero_()
    big = cw.split_sizes.clone()
    big[0] += 5                                         # tokens exceed the buffer
    _run_chunks(m, cw, x, probs, big.to(DEV), cw.sorted_idx.to(DEV), st)
    torch.cuda.synchronize()
    assert int(st.item()) & m.DEV_OVERFLOW
    st.zero_()
    small_cap = workloads.Chunked(cw.name, cw.x, cw.probs, cw.split_sizes, cw.sorted_idx,
                                  cw.chunks_per_group, cw.align, 512)
    _run_chunks(m, small_cap, x, probs, cw.split_sizes.to(DEV), cw.sorted_idx.to(DEV), st)
    torch.cuda.synchronize()
    assert int(st.item()) & m.DEV_OVERFLOW


@pytest.mark.parametrize("out_cap", [0, 1, 100, 5000])
def test_chunk_no_source_rows(m, out_cap):
    """N_cap = 0 (an empty, null input): every chunk is empty, so every padded
    row is zero and unmapped, every padded offset 0; the restore of nothing
    writes nothing."""
    say(f"chunk sort-and-pad with no source rows, out_cap={out_cap}")
    C, R, H = 8, 4, 256
    x = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    probs = torch.empty(0, dtype=torch.float32, device=DEV)
    sizes = torch.zeros(C, dtype=torch.int32)
    order = torch.arange(C, dtype=torch.int32)
    cw = workloads.Chunked("empty", x.cpu(), probs.cpu(), sizes, order, R, 16, out_cap)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, out_p, rm, off = _run_chunks(m, cw, x, probs, sizes.to(DEV), order.to(DEV), st)
    r_out, r_p, r_rm, r_off = oracle.sort_chunks_and_pad(
        np.zeros((0, H), np.uint16), np.zeros(0, np.float32), sizes.numpy(), order.numpy(), R,
        16, out_cap)
    assert int(st.item()) == 0
    assert_bits_equal(rm.cpu().numpy(), r_rm, "row_map")
    assert_bits_equal(off.cpu().numpy(), r_off, "padded_offsets")
    assert_bits_equal(_raw(out), r_out, "padded tokens")
    assert_bits_equal(_raw(out_p), r_p, "padded probs")
    back, back_p = m.moe_unpad_and_restore_chunks(out, rm, sizes.to(DEV), 0, out_p, dev_status=st)
    torch.cuda.synchronize()
    assert back.shape == (0, H) and back_p.shape == (0,) and int(st.item()) == 0


@pytest.mark.parametrize("H,dtype,pkind,n_cap,n_act,extra", [
    (1, torch.bfloat16, "f16", 3000, 500, 7),     # 2-byte units, one per row
    (3, torch.bfloat16, "f32", 2500, 700, 0),     # odd row width
    (8, torch.bfloat16, None, 4096, 4000, 300),   # one 16-byte unit per row
    (5, torch.float32, "f32", 1500, 1499, 1),     # 4-byte units
    (2048, torch.bfloat16, "f16", 300, 120, 64),  # 256 units per row
    (8, torch.bfloat16, "f32", 5000, 0, 0),       # no tokens: all zero tail
])
def test_restore_slice_edges(m, H, dtype, pkind, n_cap, n_act, extra):
    """The restore reads each workgroup's map entries, padded rows and probs
    as slices of one contiguous range of units: slices that straddle the end
    of the padded buffer, restored buffers longer than the padded one (the
    zero tail past the token total), rows of one unit (a workgroup spans
    hundreds of rows), and every prob width, each against the oracle."""
    say(f"restore slice edges H={H} dtype={dtype} probs={pkind} n_cap={n_cap} n_act={n_act}")
    g = torch.Generator().manual_seed(n_cap + H)
    R, E, A = 4, 8, 8
    x = torch.randn(n_cap, H, generator=g).to(dtype)
    probs = None
    if pkind is not None:
        probs = torch.rand(n_cap, generator=g)
        if pkind == "f16":
            probs = probs.to(torch.float16)
    sizes = workloads.chunk_sizes(n_act, R, E, 3, g)
    order = workloads.expert_major_order(R, E)
    out_cap = workloads.padded_capacity(n_act, E, A) + extra
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    sd = sizes.to(DEV)
    out, out_p, rm, _ = m.moe_sort_chunks_and_pad(
        x.to(DEV), sd, order.to(DEV), R, A, out_cap, None if probs is None else probs.to(DEV),
        dev_status=st)
    pr = None if probs is None else _raw(probs)
    r_out, r_p, r_rm, _ = oracle.sort_chunks_and_pad(_raw(x), pr, sizes.numpy(), order.numpy(),
                                                     R, A, out_cap)
    assert_bits_equal(rm.cpu().numpy(), r_rm, "row_map")
    assert_bits_equal(_raw(out), r_out, "padded rows")
    nan_fill = torch.full((n_cap, H), float("nan"), dtype=dtype, device=DEV)
    nan_probs = None if probs is None else torch.full((n_cap,), float("nan"), dtype=probs.dtype,
                                                      device=DEV)
    back, back_p = m.moe_unpad_and_restore_chunks(out, rm, sd, n_cap, out_p, out=nan_fill,
                                                  out_probs=nan_probs, dev_status=st)
    ref_b, ref_bp = oracle.unpad_and_restore_chunks(r_out, r_p, r_rm, sizes.numpy(), n_cap)
    assert_bits_equal(_raw(back), ref_b, "restored rows")
    if probs is not None:
        assert_bits_equal(_raw(back_p), ref_bp, "restored probs")
    else:
        assert back_p is None
    torch.cuda.synchronize()
    assert int(st.item()) == 0


def test_chunk_negative_size_sets_status(m):
    """A negative chunk size is bad metadata: the status says so and the whole
    padded buffer is zero and unmapped, through the one-launch path (small
    buffer) and the two-launch path (a buffer past its size limit)."""
    say("chunk negative size")
    for H in (64, 32768):
        cw = workloads.chunked(2100, seed=52, H=H, num_ranks=4, num_experts=6, align=16,
                               num_empty=5)
        sizes = cw.split_sizes.clone()
        sizes[3] = -1
        x, probs = cw.x.to(DEV), cw.probs.to(DEV)
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        out, out_p, rm, off = _run_chunks(m, cw, x, probs, sizes.to(DEV),
                                          cw.sorted_idx.to(DEV), st)
        torch.cuda.synchronize()
        assert int(st.item()) & m.DEV_BAD_CHUNKS, H
        assert bool((rm == -1).all()) and bool((out.view(torch.int16) == 0).all()), H
        assert bool((off == 0).all()) and bool((out_p == 0).all()), H


@pytest.mark.parametrize("H,N,bwd", [(64, 2100, False), (64, 2100, True),
                                     (2048, 9000, False), (7168, 700, True)])
def test_restore_stale_map(m, H, N, bwd):
    """A row map saved for larger split sizes, restored with smaller ones: the
    entries at or past the new token total are dropped and reported (a status
    bit, no race with the zero tail), and every row matches the oracle's
    defined output.  Also through the backward of the pad (the same copy)."""
    say(f"restore stale map H={H} N={N} bwd={bwd}")
    cw = workloads.chunked(N, seed=61, H=H, num_ranks=4, num_experts=6, align=16, num_empty=3)
    x, probs = cw.x.to(DEV), cw.probs.to(DEV)
    order = cw.sorted_idx.to(DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, out_p, rm, _ = _run_chunks(m, cw, x, probs, cw.split_sizes.to(DEV), order, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    small = workloads.chunk_sizes(N // 2, 4, 6, 3, torch.Generator().manual_seed(62))
    nan_fill = sentinel_bf16((cw.N_cap, H))
    nan_probs = sentinel_f32((cw.N_cap,))
    st2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    call = m.moe_sort_chunks_and_pad_bwd if bwd else m.moe_unpad_and_restore_chunks
    kw = {"d_in": nan_fill, "d_in_probs": nan_probs} if bwd else \
        {"out": nan_fill, "out_probs": nan_probs}
    back, back_p = call(out, rm, small.to(DEV), cw.N_cap, out_p, dev_status=st2, **kw)
    torch.cuda.synchronize()
    ref_b, ref_bp, ost = oracle.unpad_and_restore_chunks(
        bits(out), out_p.cpu().numpy(), rm.cpu().numpy(), small.numpy(), cw.N_cap,
        with_status=True)
    assert ost == 4
    assert int(st2.item()) & m.DEV_BAD_ROW
    assert_bits_equal(bits(back), ref_b, "restored rows (stale map)")
    assert_bits_equal(back_p.cpu().numpy(), ref_bp, "restored probs (stale map)")


def test_binding_rejects_bad_shapes(m):
    """Caller-given buffers of the wrong size or dtype are refused before any
    launch (a short buffer would be read or written past its end)."""
    say("binding shape checks")
    w = workloads.random_routed(32, 64, 8, 2, seed=3)
    x, idx, probs, dy = to_dev(w)
    rm, _ = m.moe_make_row_id_map(idx, 8)
    P, pp = m.moe_permute(x, idx, rm, probs)
    with pytest.raises(ValueError):                          # d_out one token short
        m.moe_unpermute_bwd(dy[:-1], idx, rm, probs, P)
    cw = workloads.chunked(300, seed=4, H=64, num_ranks=2, num_experts=4, align=8,
                           num_empty=1)
    cx, cp = cw.x.to(DEV), cw.probs.to(DEV)
    sz, order = cw.split_sizes.to(DEV), cw.sorted_idx.to(DEV)
    with pytest.raises(TypeError):                           # bf16 slot for fp32 probs
        m.moe_sort_chunks_and_pad(cx, sz, order, cw.chunks_per_group, cw.align, cw.out_cap, cp,
                                  out_probs=torch.empty(cw.out_cap, dtype=torch.bfloat16,
                                                        device=DEV))
    out, out_p, rmap, _ = m.moe_sort_chunks_and_pad(cx, sz, order, cw.chunks_per_group,
                                                    cw.align, cw.out_cap, cp)
    with pytest.raises(TypeError):
        m.moe_unpad_and_restore_chunks(out, rmap, sz, cw.N_cap, out_p,
                                       out_probs=torch.empty(cw.N_cap, dtype=torch.bfloat16,
                                                             device=DEV))
    with pytest.raises(ValueError):                          # prob output too short
        m.moe_unpad_and_restore_chunks(out, rmap, sz, cw.N_cap, out_p,
                                       out_probs=torch.empty(cw.N_cap - 1, dtype=torch.float32,
                                                             device=DEV))
    with pytest.raises(ValueError):
        m.moe_sort_chunks_and_pad_bwd(out, rmap, sz, cw.N_cap, out_p,
                                      d_in_probs=torch.empty(3, dtype=torch.float32,
                                                             device=DEV))
    with pytest.raises(TypeError):
        m.moe_unpad_and_restore_chunks_bwd(cx, rmap, cw.out_cap, cp,
                                           d_in_probs=torch.empty(cw.out_cap,
                                                                  dtype=torch.bfloat16,
                                                                  device=DEV))
    torch.cuda.synchronize()


@pytest.mark.parametrize("N", [8192, 32768])
def test_chunk_graph_replay(m, N):
    """Sort-and-pad + restore captured once, replayed with eight different
    split-size draws at fixed buffer sizes: at 8192 tokens the one-launch
    sort-and-pad, at 32768 the map + copy pair."""
    if N == 32768:
        cw = workloads.chunks32k(with_replays=True)
    else:
        cw = workloads.chunked(N, seed=3, replay_seeds=tuple(range(3000, 3008)), name="c8k")
    say(f"chunk graph replay {N} tokens, 8 routings")
    x, probs = cw.x.to(DEV), cw.probs.to(DEV)
    sizes_s = cw.split_sizes.to(DEV)
    order = cw.sorted_idx.to(DEV)
    G = cw.C // cw.chunks_per_group
    out = torch.empty((cw.out_cap, cw.H), dtype=torch.bfloat16, device=DEV)
    out_p = torch.empty(cw.out_cap, dtype=torch.float32, device=DEV)
    rm = torch.empty(cw.out_cap, dtype=torch.int32, device=DEV)
    off = torch.empty(G + 1, dtype=torch.int32, device=DEV)
    back = torch.empty((cw.N_cap, cw.H), dtype=torch.bfloat16, device=DEV)
    back_p = torch.empty(cw.N_cap, dtype=torch.float32, device=DEV)

    def step():
        m.moe_sort_chunks_and_pad(x, sizes_s, order, cw.chunks_per_group, cw.align, cw.out_cap,
                                  probs, out=out, out_probs=out_p, row_map=rm,
                                  padded_offsets=off)
        m.moe_unpad_and_restore_chunks(out, rm, sizes_s, cw.N_cap, out_p, out=back,
                                       out_probs=back_p)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    xb = workloads.bf16_bits(cw.x)
    for rep, sizes in enumerate(cw.replays):
        sizes_s.copy_(sizes)
        out.view(torch.int16).fill_(S_BF16)
        back.view(torch.int16).fill_(S_BF16)
        g.replay()
        torch.cuda.synchronize()
        r_out, r_p, r_rm, r_off = oracle.sort_chunks_and_pad(
            xb, cw.probs.numpy(), sizes.numpy(), cw.sorted_idx.numpy(), cw.chunks_per_group,
            cw.align, cw.out_cap)
        assert_bits_equal(rm.cpu().numpy(), r_rm, f"replay {rep} row_map")
        assert_bits_equal(off.cpu().numpy(), r_off, f"replay {rep} offsets")
        assert_bits_equal(bits(out), r_out, f"replay {rep} padded")
        assert_bits_equal(out_p.cpu().numpy(), r_p, f"replay {rep} padded probs")
        ref_b, ref_bp = oracle.unpad_and_restore_chunks(r_out, r_p, r_rm, sizes.numpy(),
                                                        cw.N_cap)
        assert_bits_equal(bits(back), ref_b, f"replay {rep} restored")
        assert_bits_equal(back_p.cpu().numpy(), ref_bp, f"replay {rep} restored probs")


def _assert_bits_nan_aware(got, exp, what):
    """Bit-exact, except that IEEE 754 leaves the payload of a NaN produced by
    arithmetic open: where the oracle gives a NaN the kernel must give a NaN."""
    got = np.asarray(got).astype(np.uint16)
    exp = np.asarray(exp).astype(np.uint16)
    nan_e = (exp & 0x7F80) == 0x7F80
    nan_e &= (exp & 0x007F) != 0
    nan_g = ((got & 0x7F80) == 0x7F80) & ((got & 0x007F) != 0)
    assert np.array_equal(nan_g, nan_e), f"{what}: NaN positions differ"
    assert_bits_equal(got[~nan_e], exp[~nan_e], what)


def test_special_values(m):
    """Infinities, NaNs, subnormals, signed zeros, values near the bf16 maximum
    and rounding ties through the combine, its backward and the permute bwd."""
    T, H, E, k = 64, 64, 8, 4
    say("special values")
    w = workloads.random_routed(T, H, E, k, seed=77)
    ref_map, _ = oracle.row_id_map(w.topk_idx.numpy(), E)
    rng = np.random.default_rng(9)
    P = workloads.bf16_bits(workloads.random_rows(T * k, H, seed=8)).copy()
    specials = np.array([0x7F80, 0xFF80, 0x7FC1, 0xFFA3, 0x0001, 0x8003, 0x007F, 0x7F7F, 0xFF7F,
                         0x8000, 0x0000, 0x3F81, 0x0080], np.uint16)
    pos = rng.choice(P.size, 600, replace=False)
    P.ravel()[pos] = rng.choice(specials, 600)
    probs = w.probs.numpy().copy()
    probs.ravel()[rng.choice(probs.size, 40, replace=False)] = 1.0 + 2.0 ** -8
    probs.ravel()[rng.choice(probs.size, 20, replace=False)] = 1e-30
    probs.ravel()[rng.choice(probs.size, 10, replace=False)] = 3e38
    idx = w.topk_idx.to(DEV)
    rm = torch.from_numpy(ref_map).to(DEV)
    Pd = torch.from_numpy(P.view(np.int16)).to(DEV).view(torch.bfloat16)
    pd = torch.from_numpy(probs).to(DEV)
    ib = w.topk_idx.numpy()
    y = m.moe_unpermute(Pd, idx, rm, pd)
    _assert_bits_nan_aware(bits(y), oracle.unpermute(P, probs, ib, ref_map), "unpermute")
    for partials, fp64 in ((True, False), (False, True), (True, True)):
        y = m.moe_unpermute_ep(Pd, idx, rm, 4, pd, bf16_partials=partials, fp64_cross=fp64)
        _assert_bits_nan_aware(bits(y), oracle.unpermute_ep(P, probs, ib, ref_map, 4, partials,
                                                             fp64), "unpermute_ep")
    dy = P[:T].copy()
    dyd = torch.from_numpy(dy.view(np.int16)).to(DEV).view(torch.bfloat16)
    d_in, _ = m.moe_unpermute_bwd(dyd, idx, rm, pd, Pd, probs_grad=False)
    ref_in, _ = oracle.unpermute_bwd(dy, None, probs, ib, ref_map)
    _assert_bits_nan_aware(bits(d_in), ref_in, "unpermute_bwd act grad")
    d_x, _ = m.moe_permute_bwd(Pd, idx, rm)
    ref_x, _ = oracle.permute_bwd(P, None, ib, ref_map)
    _assert_bits_nan_aware(bits(d_x), ref_x, "permute_bwd")
