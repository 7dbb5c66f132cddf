"""GPU parity for the TransformerEngine mask-map form: map builder, permute,
unpermute and the unpermute backward, against the CPU oracle.

Maps, copies, the TE-order combine and the act-grad products must match
bit for bit.  Map entries the page leaves unused, output rows no map entry
names and rows past the kept count must keep the sentinel the test wrote
(the kernels do not touch them).  The prob-grad dot products are compared
on the scale S = sum_h |fwd_in[row][h] * d_out[t][h]|: |g - ref| <= 1e-5 S.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
S_I32 = -7
S_BF16 = 0x7FC1


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import unpermute_moe_make_amd as mod
    return mod


def bits(t):
    return workloads.bf16_bits(t.cpu())


def sentinel_bf16(shape):
    t = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    t.view(torch.int16).fill_(S_BF16)
    return t


def mask_from_topk(idx, E):
    T = idx.shape[0]
    mask = torch.zeros((T, E), dtype=torch.bool)
    mask.scatter_(1, idx.long(), True)
    return mask


def random_mask(T, E, density, seed, min_one=False):
    g = torch.Generator().manual_seed(seed)
    mask = torch.rand(T, E, generator=g) < density
    if min_one:
        mask[torch.arange(T), torch.randint(0, E, (T,), generator=g)] = True
    return mask


def build_map(m, mask_dev, num_out=-1):
    T, E = mask_dev.shape
    rm = torch.full((T, 2 * E + 1), S_I32, dtype=torch.int32, device=DEV)
    off = torch.full((E + 1,), S_I32, dtype=torch.int32, device=DEV)
    m.moe_make_mask_row_id_map(mask_dev, num_out_tokens=num_out, row_id_map=rm,
                               expert_offsets=off)
    return rm.cpu().numpy(), off.cpu().numpy()


def assert_map_equal(got, ref, E):
    """Defined entries equal the oracle's; the others still hold the sentinel."""
    n = ref[:, 2 * E]
    np.testing.assert_array_equal(got[:, 2 * E], n)
    col = np.arange(E)[None, :]
    used = col < n[:, None]
    for lo in (0, E):
        g, r = got[:, lo:lo + E], ref[:, lo:lo + E]
        assert np.array_equal(g[used], r[used]), f"map entries differ at offset {lo}"
        assert np.all(g[~used] == S_I32), "an unused map entry was written"


def oracle_mask(mask):
    return mask.numpy().astype(np.uint8)


# ------------------------------------------------------------------ map ----

@pytest.mark.parametrize("name", ["tiny", "finegrain", "skewed"])
@pytest.mark.parametrize("dtype", [torch.bool, torch.int32])
def test_mask_map_configs(m, name, dtype):
    w = workloads.ROUTED[name]()
    say(f"mask map {name} {dtype}")
    mask = mask_from_topk(w.topk_idx, w.num_experts)
    got, off = build_map(m, mask.to(dtype).to(DEV))
    ref, ref_off = oracle.mask_row_id_map(oracle_mask(mask))
    assert_map_equal(got, ref, w.num_experts)
    np.testing.assert_array_equal(off, ref_off)


@pytest.mark.parametrize("T,E,density,num_out", [
    (1, 1, 1.0, -1), (63, 5, 0.5, -1), (257, 7, 0.3, -1), (300, 160, 0.6, -1),
    (100, 2048, 0.05, -1), (20000, 16, 0.25, -1), (1000, 64, 0.2, 5000), (1000, 64, 0.2, 0),
    (500, 33, 0.9, 100000), (17000, 8, 0.5, 30000), (1024, 64, 0.3, -1),
    (1025, 64, 0.3, 20000), (700, 48, 0.5, 1000), (16, 64, 1.0, -1), (1024, 16, 0.0, -1)])
@pytest.mark.parametrize("dtype", [torch.uint8, torch.int32])
def test_mask_map_shapes_and_dropping(m, T, E, density, num_out, dtype):
    """Tokens routed to more than 64 experts, E not a multiple of 4, over 64
    token blocks (the column-scan path), empty masks, and dropping."""
    say(f"mask map T={T} E={E} d={density} num_out={num_out} {dtype}")
    mask = random_mask(T, E, density, seed=T + E)
    got, off = build_map(m, mask.to(dtype).to(DEV), num_out)
    ref, ref_off = oracle.mask_row_id_map(oracle_mask(mask), num_out)
    assert_map_equal(got, ref, E)
    np.testing.assert_array_equal(off, ref_off)


def test_mask_map_misaligned_mask(m):
    """A mask view that starts one element in takes the scalar-load path."""
    say("mask map misaligned view")
    T, E = 200, 12
    base = random_mask(T * E + 1, 1, 0.4, seed=3).reshape(-1).to(torch.int32)
    mask_dev = base.to(DEV)[1:].view(T, E)
    got, off = build_map(m, mask_dev)
    ref, ref_off = oracle.mask_row_id_map(base[1:].view(T, E).numpy())
    assert_map_equal(got, ref, E)
    np.testing.assert_array_equal(off, ref_off)


def test_mask_map_empty(m):
    say("mask map T=0")
    off = torch.full((5,), S_I32, dtype=torch.int32, device=DEV)
    m.moe_make_mask_row_id_map(torch.zeros((0, 4), dtype=torch.bool, device=DEV),
                               expert_offsets=off)
    assert off.cpu().tolist() == [0, 0, 0, 0, 0]


# ------------------------------------------------------- row kernels -------

def _case(name_or_shape, seed=0):
    """(x, mask, probs[T,E]) for a routed workload or a random mask."""
    if isinstance(name_or_shape, str):
        w = workloads.ROUTED[name_or_shape]()
        mask = mask_from_topk(w.topk_idx, w.num_experts)
        probs = torch.zeros((w.T, w.num_experts))
        probs.scatter_(1, w.topk_idx.long(), w.probs)
        return w.x, mask, probs, w.dy
    T, H, E, density = name_or_shape
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    mask = random_mask(T, E, density, seed=seed + 1)
    probs = torch.rand(T, E, generator=g) * mask
    dy = torch.randn(T, H, generator=g).to(torch.bfloat16)
    return x, mask, probs, dy


SMALL = [(37, 7, 9, 0.4), (64, 64, 16, 0.5), (40, 136, 160, 0.6), (9, 20480, 8, 0.9),
         (50, 24, 6, 0.0), (33, 72, 2048, 0.02)]


@pytest.mark.parametrize("case", ["finegrain", "skewed"] + SMALL)
@pytest.mark.parametrize("with_probs", [True, False])
def test_mask_permute(m, case, with_probs):
    x, mask, probs, _ = _case(case, seed=11)
    T, H = x.shape
    E = mask.shape[1]
    say(f"mask permute {case if isinstance(case, str) else (T, H, E)} probs={with_probs}")
    if with_probs:
        probs[::5] = 0.0          # padded slots: zero rows
    ref_map, _ = oracle.mask_row_id_map(oracle_mask(mask))
    R = int(mask.sum())
    n_out = R + 3                 # three rows no map entry names
    rm = torch.from_numpy(ref_map).to(DEV)
    out = sentinel_bf16((n_out, H))
    out_p = torch.full((n_out,), -5.0, device=DEV) if with_probs else None
    m.moe_permute_mask(x.to(DEV), rm, n_out, probs.to(DEV) if with_probs else None,
                       out=out, out_probs=out_p)
    ob = bits(out)
    assert np.all(ob[R:] == S_BF16)
    if T * H <= (1 << 24):
        ref, ref_p = oracle.mask_permute(bits(x), probs.numpy() if with_probs else None,
                                         ref_map, n_out, out=ob.copy() * 0 + S_BF16)
        np.testing.assert_array_equal(ob, ref)
        if with_probs:
            np.testing.assert_array_equal(out_p.cpu().numpy()[:R].view(np.uint32),
                                          ref_p[:R].view(np.uint32))
    else:
        # full check by a gather on the GPU: row map entries -> source token
        # and expert; a zero prob gives a zero row
        src = np.full(R, -1, np.int64)
        exp_e = np.full(R, -1, np.int64)
        for lo in range(E):
            used = ref_map[:, 2 * E] > lo
            src[ref_map[used, lo]] = np.nonzero(used)[0]
            exp_e[ref_map[used, lo]] = ref_map[used, E + lo]
        assert np.all(src >= 0)
        exp = x.to(DEV)[torch.from_numpy(src).to(DEV)]
        if with_probs:
            p_row = probs.numpy()[src, exp_e]
            exp[torch.from_numpy(p_row == 0.0).to(DEV)] = 0
            np.testing.assert_array_equal(out_p.cpu().numpy()[:R].view(np.uint32),
                                          p_row.view(np.uint32))
        assert torch.equal(out[:R].view(torch.int16), exp.view(torch.int16))


@pytest.mark.parametrize("case", ["finegrain", "skewed"] + SMALL)
@pytest.mark.parametrize("merge,scatter", [(True, True), (False, False), (True, False)])
def test_mask_unpermute(m, case, merge, scatter):
    x, mask, probs, _ = _case(case, seed=12)
    T, H = x.shape
    E = mask.shape[1]
    say(f"mask unpermute {case if isinstance(case, str) else (T, H, E)} merge={merge} "
        f"scatter={scatter}")
    ref_map, _ = oracle.mask_row_id_map(oracle_mask(mask))
    R = int(mask.sum())
    rm = torch.from_numpy(ref_map).to(DEV)
    P = workloads.random_rows(R, H, seed=31, device=DEV)
    pp = torch.rand(R, generator=torch.Generator().manual_seed(5)) if scatter else None
    out = sentinel_bf16((T, H))
    y, up = m.moe_unpermute_mask(P, rm, probs.to(DEV) if merge else None,
                                 pp.to(DEV) if scatter else None, out=out)
    ref, ref_up = oracle.mask_unpermute(bits(P), probs.numpy() if merge else None, ref_map,
                                        pp.numpy() if scatter else None)
    np.testing.assert_array_equal(bits(y), ref)
    if scatter:
        np.testing.assert_array_equal(up.cpu().numpy().view(np.uint32), ref_up.view(np.uint32))


def _f64(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _dot_ok(got, fwd_bits, dy_bits, ref_map, E, ref, chunk=1024):
    """|got - ref| <= 1e-5 * sum_h |a*b| at every routed (token, expert);
    fwd_bits [rows][H] and dy_bits [T][H] bf16 bits, a chunk of tokens at a
    time."""
    T = ref_map.shape[0]
    n = ref_map[:, 2 * E]
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        b = np.abs(_f64(dy_bits[t0:t1]))
        for j in range(int(n[t0:t1].max(initial=0))):
            toks = np.nonzero(n[t0:t1] > j)[0]
            r = ref_map[t0 + toks, j]
            e = ref_map[t0 + toks, E + j]
            scale = np.einsum("uh,uh->u", np.abs(_f64(fwd_bits[r])), b[toks])
            err = np.abs(got[t0 + toks, e].astype(np.float64) -
                         ref[t0 + toks, e].astype(np.float64))
            assert np.all(err <= 1e-5 * scale + 1e-37), (t0, j)


@pytest.mark.parametrize("case", ["finegrain", "skewed"] + SMALL)
@pytest.mark.parametrize("want_dot", [True, False])
def test_mask_unpermute_bwd(m, case, want_dot):
    x, mask, probs, dy = _case(case, seed=13)
    T, H = x.shape
    E = mask.shape[1]
    say(f"mask unpermute bwd {case if isinstance(case, str) else (T, H, E)} dot={want_dot}")
    ref_map, _ = oracle.mask_row_id_map(oracle_mask(mask))
    R = int(mask.sum())
    rm = torch.from_numpy(ref_map).to(DEV)
    fin = workloads.random_rows(R + 2, H, seed=41, device=DEV)
    d_in = sentinel_bf16((R + 2, H))
    d_in, dmp = m.moe_unpermute_mask_bwd(dy.to(DEV), fin, probs.to(DEV), rm, d_in=d_in,
                                         want_probs_grad=want_dot)
    db = bits(d_in)
    assert np.all(db[R:] == S_BF16)
    fv = workloads.bf16_bits(fin.cpu())
    dyb = bits(dy)
    ref_din, ref_dmp = oracle.mask_unpermute_bwd(dyb, fv, probs.numpy(), ref_map,
                                                 d_in=db.copy())
    np.testing.assert_array_equal(db, ref_din)
    del ref_din
    if want_dot:
        got = dmp.cpu().numpy()
        sel = np.zeros((T, E), bool)
        for lo in range(E):
            used = ref_map[:, 2 * E] > lo
            sel[np.nonzero(used)[0], ref_map[used, E + lo]] = True
        assert np.all(got[~sel].view(np.uint32) == 0)
        _dot_ok(got, fv, dyb, ref_map, E, ref_dmp)


@pytest.mark.parametrize("T,H,E,density", [(4096, 4096, 64, 0.25), (2048, 4104, 256, 0.3)])
def test_mask_unpermute_bwd_streaming_shapes(m, T, H, E, density):
    """Calls past the streaming threshold, in full: the two-launch backward
    with many slots per token (several batches of dot products; more than 64
    slots, two chunks, at 256 experts; rows of 513 16-byte units), and the
    scatter alone without merging-prob gradients."""
    x, mask, probs, dy = _case((T, H, E, density), seed=E)
    say(f"mask unpermute bwd streaming {(T, H, E, density)}")
    ref_map, _ = oracle.mask_row_id_map(oracle_mask(mask))
    R = int(mask.sum())
    rm = torch.from_numpy(ref_map).to(DEV)
    fin = workloads.random_rows(R, H, seed=43, device=DEV)
    d_in = sentinel_bf16((R, H))
    d_in, dmp = m.moe_unpermute_mask_bwd(dy.to(DEV), fin, probs.to(DEV), rm, d_in=d_in)
    fv = workloads.bf16_bits(fin.cpu())
    dyb = bits(dy)
    ref_din, ref_dmp = oracle.mask_unpermute_bwd(dyb, fv, probs.numpy(), ref_map)
    np.testing.assert_array_equal(bits(d_in), ref_din)
    got = dmp.cpu().numpy()
    sel = np.zeros((T, E), bool)
    for lo in range(E):
        used = ref_map[:, 2 * E] > lo
        sel[np.nonzero(used)[0], ref_map[used, E + lo]] = True
    assert np.all(got[~sel].view(np.uint32) == 0)
    _dot_ok(got, fv, dyb, ref_map, E, ref_dmp)
    d_in1 = sentinel_bf16((R, H))
    d_in1, none = m.moe_unpermute_mask_bwd(dy.to(DEV), fin, probs.to(DEV), rm, d_in=d_in1,
                                           want_probs_grad=False)
    assert none is None
    np.testing.assert_array_equal(bits(d_in1), ref_din)


def test_mask_roundtrip_identity_one_expert(m):
    """One expert per token, no merging probs: unpermute(permute(x)) == x."""
    say("mask roundtrip one expert")
    T, H, E = 1000, 520, 24
    g = torch.Generator().manual_seed(4)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16).to(DEV)
    mask = torch.zeros(T, E, dtype=torch.bool)
    mask[torch.arange(T), torch.randint(0, E, (T,), generator=g)] = True
    rm, _ = m.moe_make_mask_row_id_map(mask.to(DEV))
    P, _ = m.moe_permute_mask(x, rm, T)
    y, _ = m.moe_unpermute_mask(P, rm)
    assert torch.equal(y.view(torch.int16), x.view(torch.int16))


def test_mask_chain_on_gpu_with_dropping(m):
    """Map (with dropping) -> permute -> unpermute, all on the GPU, against the
    same chain in the oracle."""
    say("mask chain with dropping")
    x, mask, probs, _ = _case((700, 264, 40, 0.2), seed=21)
    T, H = x.shape
    R = int(mask.sum())
    num_out = R * 3 // 4
    rm, off = m.moe_make_mask_row_id_map(mask.to(DEV), num_out_tokens=num_out)
    out = sentinel_bf16((num_out, H))
    P, pp = m.moe_permute_mask(x.to(DEV), rm, num_out, probs.to(DEV), out=out)
    y, up = m.moe_unpermute_mask(P, rm, probs.to(DEV), pp)
    ref_map, ref_off = oracle.mask_row_id_map(oracle_mask(mask), num_out)
    np.testing.assert_array_equal(off.cpu().numpy(), ref_off)
    ref_P, ref_pp = oracle.mask_permute(bits(x), probs.numpy(), ref_map, num_out)
    np.testing.assert_array_equal(bits(P), ref_P)
    ref_y, ref_up = oracle.mask_unpermute(ref_P, probs.numpy(), ref_map, ref_pp)
    np.testing.assert_array_equal(bits(y), ref_y)
    np.testing.assert_array_equal(up.cpu().numpy().view(np.uint32), ref_up.view(np.uint32))


@pytest.mark.parametrize("T,H,E,density", [(64, 64, 16, 0.5), (4096, 4096, 64, 0.25)])
def test_mask_bad_map_row_ops(m, T, H, E, density):
    """Map faults only the device sees, at a small and a streaming size (the
    two-launch backward): an expert out of range in one token's slot, a row
    past the rows in another's, a slot count past E in a third (the whole
    token is skipped).  Each op reports both status bits, leaves the faulty
    slots' rows unwritten and matches the oracle (on the sound map) on every
    other row and token."""
    say(f"mask bad map row ops {(T, H, E, density)}")
    x, mask, probs, dy = _case((T, H, E, density), seed=E + 5)
    ref_map, _ = oracle.mask_row_id_map(oracle_mask(mask))
    R = int(mask.sum())
    n = ref_map[:, 2 * E]
    cand = np.nonzero(n >= 2)[0]
    a, b, c = int(cand[0]), int(cand[len(cand) // 2]), int(cand[-1])
    bad = ref_map.copy()
    bad[a, E] = E + 1
    bad[b, 1] = R + 5
    bad[c, 2 * E] = E + 1
    skip_rows = np.array([ref_map[a, 0], ref_map[b, 1]] + list(ref_map[c, :n[c]]))
    keep_rows = np.setdiff1d(np.arange(R), skip_rows)
    ok_tok = np.setdiff1d(np.arange(T), [a, b, c])
    rm = torch.from_numpy(bad).to(DEV)
    xd, pd, dyd = x.to(DEV), probs.to(DEV), dy.to(DEV)
    pn = probs.numpy()

    def status(call):
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        out = call(st)
        torch.cuda.synchronize()
        s = int(st.item())
        assert s & m.DEV_BAD_EXPERT and s & m.DEV_BAD_ROW, s
        return out

    def rows_ok(got, ref, what):
        np.testing.assert_array_equal(got[keep_rows], ref[keep_rows], what)
        assert np.all(got[skip_rows] == S_BF16), f"{what}: a faulty slot's row was written"

    P = sentinel_bf16((R, H))
    P, pp = status(lambda st: m.moe_permute_mask(xd, rm, R, pd, out=P, dev_status=st))
    ref_P, ref_pp = oracle.mask_permute(bits(x), pn, ref_map, R)
    rows_ok(bits(P), ref_P, "mask permute")
    np.testing.assert_array_equal(pp.cpu().numpy()[keep_rows].view(np.uint32),
                                  ref_pp[keep_rows].view(np.uint32))

    fin = workloads.random_rows(R, H, seed=H + 2, device=DEV)
    fv = workloads.bf16_bits(fin.cpu())
    y = sentinel_bf16((T, H))
    y, _ = status(lambda st: m.moe_unpermute_mask(fin, rm, pd, out=y, dev_status=st))
    ref_y, _ = oracle.mask_unpermute(fv, pn, ref_map)
    np.testing.assert_array_equal(bits(y)[ok_tok], ref_y[ok_tok])

    dyb = bits(dy)
    ref_din, ref_dmp = oracle.mask_unpermute_bwd(dyb, fv, pn, ref_map)
    for want in (True, False):
        d_in = sentinel_bf16((R, H))
        d_in, dmp = status(lambda st: m.moe_unpermute_mask_bwd(
            dyd, fin, pd, rm, d_in=d_in, want_probs_grad=want, dev_status=st))
        rows_ok(bits(d_in), ref_din, f"mask bwd act grad (prob grads {want})")
        if want:
            got = dmp.cpu().numpy()[ok_tok]
            sub = ref_map[ok_tok]
            sel = np.zeros(got.shape, bool)
            for lo in range(E):
                used = sub[:, 2 * E] > lo
                sel[np.nonzero(used)[0], sub[used, E + lo]] = True
            assert np.all(got[~sel].view(np.uint32) == 0)
            _dot_ok(got, fv, dyb[ok_tok], sub, E, ref_dmp[ok_tok])

    q, sc = workloads.quantize_fp8_rows(x, 128 if H % 128 == 0 else 8)
    qo = torch.empty((R, H), dtype=q.dtype, device=DEV)
    qo.view(torch.uint8).fill_(0x5A)
    so = torch.full((R, sc.shape[1]), -7.0, device=DEV)
    status(lambda st: m.moe_permute_mask_scaled(q.to(DEV), rm, R, sc.to(DEV), out=qo,
                                                out_scale=so, dev_status=st))
    ref_q, ref_s, _ = oracle.mask_permute_scaled(q.view(torch.uint8).numpy(),
                                                 sc.view(torch.uint8).numpy(), None, ref_map, R)
    got_q = qo.view(torch.uint8).cpu().numpy()
    np.testing.assert_array_equal(got_q[keep_rows], ref_q[keep_rows])
    assert np.all(got_q[skip_rows] == 0x5A)
    got_s = so.view(torch.uint8).cpu().numpy()
    np.testing.assert_array_equal(got_s[keep_rows], ref_s[keep_rows])
    assert np.all(so.cpu().numpy()[skip_rows] == -7.0)


def test_mask_bad_map_sets_status(m):
    say("mask bad map entries")
    T, H, E = 8, 16, 4
    mm = np.full((T, 2 * E + 1), -1, np.int32)
    mm[:, 2 * E] = 1
    mm[:, 0] = np.arange(T)
    mm[:, E] = 0
    mm[2, 0] = T + 5        # row out of range
    mm[3, E] = E            # expert out of range
    mm[4, 2 * E] = E + 1    # count out of range
    rm = torch.from_numpy(mm).to(DEV)
    x = torch.randn(T, H).to(torch.bfloat16).to(DEV)
    for fn in ("permute", "unpermute", "bwd"):
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        if fn == "permute":
            m.moe_permute_mask(x, rm, T, dev_status=st)
        elif fn == "unpermute":
            m.moe_unpermute_mask(x, rm, dev_status=st)
        else:
            m.moe_unpermute_mask_bwd(x, x, torch.ones(T, E, device=DEV), rm, dev_status=st)
        s = int(st.item())
        assert s & m.DEV_BAD_ROW and s & m.DEV_BAD_EXPERT, (fn, s)
