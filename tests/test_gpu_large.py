"""GPU parity past 32-bit offsets.

Routed rows: 40960 tokens x 8 slots of 7168-wide bf16 rows make a permuted
buffer of 2.35e9 elements (4.7 GB), past both 2^31 elements and 2^32 bytes,
through the row map, permute, unpermute backward, unpermute and permute
backward.  Chunks: 327680 rows of 7168 bf16 (4.7 GB) through sort-and-pad and
restore (32-bit flat unit indices with large quotients), and, where the GPU
has the memory, 2^20 rows of 32768 bf16 (two 69 GB buffers) whose flat
(row, 16-byte unit) index passes 2^32, the copy kernels' 64-bit index path.

The oracle cannot take these inputs whole, so each check runs it on a seeded
sample of tokens or rows -- always including the owners of the last rows of
every buffer, whose offsets are the largest -- as a sub-problem with the same
per-token arithmetic; whole-buffer properties (the row map, restore . pad =
identity) are checked in full.  Every test is skipped when the GPU lacks the
memory it needs.

Launches of more than 2^20 workgroups spill into gridDim.z (a dispatch
counts its grid in work-items, 32 bits per dimension); the token-per-
workgroup kernels and the router are run past that point with short rows
and compared with the oracle in full.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from test_gpu_parity import assert_bits_equal, bits, dprob_ok, oracle_rows, sub_problem
from test_gpu_router import check_probs, grad_bound

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import unpermute_moe_make_amd as mod
    return mod


def need_gib(n):
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    if free < (n << 30):
        pytest.skip(f"needs {n} GiB of free device memory, {free >> 30} GiB free")


def test_row_kernels_past_2g_elements(m):
    T, H, E, k = 40960, 7168, 256, 8
    R = T * k
    assert R * H > 2**31 and 2 * R * H > 2**32
    need_gib(20)
    say(f"row kernels past 2^31 elements T={T} H={H} E={E} k={k}")
    w = workloads.random_routed(T, 8, E, k, seed=901, with_dy=False, zipf_s=1.1)
    idx_np, probs_np = w.topk_idx.numpy(), w.probs.numpy()
    ref_map, ref_off = oracle.row_id_map(idx_np, E)
    idx, probs = w.topk_idx.to(DEV), w.probs.to(DEV)
    rm, off = m.moe_make_row_id_map(idx, E)
    assert_bits_equal(rm.cpu().numpy(), ref_map, "row_id_map")
    assert_bits_equal(off.cpu().numpy(), ref_off, "expert_offsets")

    rows = oracle_rows(idx_np, ref_map)                 # [T][k]
    owner = np.empty(R, np.int64)
    owner[rows.ravel()] = np.repeat(np.arange(T), k)
    rng = np.random.default_rng(904)
    sample = np.unique(np.concatenate([rng.choice(T, 160, replace=False), owner[-48:],
                                       np.arange(T - 4, T)]))
    r = rows[sample].ravel()
    rt = torch.from_numpy(r.astype(np.int64)).to(DEV)
    st_ = torch.from_numpy(sample).to(DEV)
    sidx, smap = sub_problem(idx_np, sample, E)
    ps = probs_np[sample]

    x = workloads.random_rows(T, H, seed=902, device=DEV)
    P, Pp = m.moe_permute(x, idx, rm, probs)
    ref_P, ref_Pp = oracle.permute(bits(x[st_]), ps, sidx, smap)
    assert_bits_equal(bits(P[rt]), ref_P, "permute sample")
    assert_bits_equal(Pp.cpu().numpy()[r], ref_Pp, "permuted probs sample")
    del x

    dy = workloads.random_rows(T, H, seed=903, device=DEV)
    dP, dpr = m.moe_unpermute_bwd(dy, idx, rm, probs, P)
    fin_rows = bits(P[rt])
    dy_rows = bits(dy[st_])
    ref_dP, ref_dpr = oracle.unpermute_bwd(dy_rows, fin_rows, ps, sidx, smap)
    assert_bits_equal(bits(dP[rt]), ref_dP, "unpermute_bwd act grad sample")
    worst = dprob_ok(dpr.cpu().numpy()[sample], fin_rows.reshape(len(sample), k, H), dy_rows,
                     ref_dpr)
    say(f"  prob-grad worst error / scale = {worst:.3g}")
    del P, dy

    # the slot rows of dP differ per slot, so the combines see k distinct rows
    dP_rows = bits(dP[rt])
    y = m.moe_unpermute(dP, idx, rm, probs)
    assert_bits_equal(bits(y[st_]), oracle.unpermute(dP_rows, ps, sidx, smap),
                      "unpermute sample")
    dx, dxp = m.moe_permute_bwd(dP, idx, rm, Pp)
    ref_dx, ref_dxp = oracle.permute_bwd(dP_rows, Pp.cpu().numpy()[r], sidx, smap)
    assert_bits_equal(bits(dx[st_]), ref_dx, "permute_bwd sample")
    assert_bits_equal(dxp.cpu().numpy()[sample], ref_dxp, "permute_bwd probs sample")


def _chunk_case(N, H, seed):
    g = torch.Generator().manual_seed(seed)
    sizes = workloads.chunk_sizes(N, 8, 16, 16, g)
    order = workloads.expert_major_order(8, 16)
    cap = workloads.padded_capacity(N, 16, 128)
    return sizes, order, cap


def _row_sample(n, seed, extra=()):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([rng.choice(n, 256, replace=False), np.arange(n - 64, n),
                                     np.asarray(extra, np.int64)]))


def test_chunks_past_4gib(m):
    N, H = 327680, 7168
    sizes, order, cap = _chunk_case(N, H, 905)
    assert 2 * N * H > 2**32
    need_gib(20)
    say(f"chunk pad/restore past 4 GiB N={N} H={H} cap={cap}")
    ref_rm, ref_off = oracle.chunk_map(sizes.numpy(), order.numpy(), 8, 128, N, cap)
    x = workloads.random_rows(N, H, seed=906, device=DEV)
    probs = torch.rand(N, generator=torch.Generator().manual_seed(907)).to(DEV)
    out, out_p, rm, off = m.moe_sort_chunks_and_pad(x, sizes.to(DEV), order.to(DEV), 8, 128, cap,
                                                    probs)
    assert_bits_equal(rm.cpu().numpy(), ref_rm, "row_map")
    assert_bits_equal(off.cpu().numpy(), ref_off, "padded_offsets")
    # padded rows: the oracle's copy of the sampled rows' sources (or zeros)
    d = _row_sample(cap, 908)
    src = ref_rm[d]
    dt = torch.from_numpy(d).to(DEV)
    exp = np.zeros((len(d), H), np.uint16)
    have = src >= 0
    exp[have] = bits(x[torch.from_numpy(src[have].astype(np.int64)).to(DEV)])
    assert_bits_equal(bits(out[dt]), exp, "padded rows sample")
    exp_p = np.zeros(len(d), np.float32)
    exp_p[have] = probs.cpu().numpy()[src[have]]
    assert_bits_equal(out_p.cpu().numpy()[d], exp_p, "padded probs sample")
    back, back_p = m.moe_unpad_and_restore_chunks(out, rm, sizes.to(DEV), N, out_p)
    assert torch.equal(back.view(torch.int16), x.view(torch.int16))   # restore . pad = id
    assert torch.equal(back_p.view(torch.int32), probs.view(torch.int32))


def _pattern_rows(n, H, dev):
    """[n, H] bf16 rows whose bits are (a(row) + b(col)) mod 2^16: built in place
    by a broadcast add, so no full-size temporary is needed; a row and column
    mixup changes the bits."""
    t = torch.empty((n, H), dtype=torch.bfloat16, device=dev)
    a = ((torch.arange(n, device=dev, dtype=torch.int64) * 7919) % 65521).to(torch.int32)
    b = ((torch.arange(H, device=dev, dtype=torch.int64) * 40503) % 65519).to(torch.int32)
    for i0 in range(0, n, 1 << 14):      # 2^14-row slabs keep the int32 sum small
        i1 = min(n, i0 + (1 << 14))
        s = ((a[i0:i1, None] + b[None, :] + 32768) & 0xFFFF) - 32768   # int16 range
        t[i0:i1].view(torch.int16).copy_(s.to(torch.int16))
    return t, a.cpu().numpy(), b.cpu().numpy()


def _pattern_bits(a, b, rows):
    return ((a[rows][:, None] + b[None, :]) & 0xFFFF).astype(np.uint16)


def test_chunks_64bit_flat_index(m):
    """2^20 rows of 32768 bf16: out_cap * 4096 units > 2^32, so both copies
    take their 64-bit flat-index path."""
    N, H = 1 << 20, 32768
    sizes, order, cap = _chunk_case(N, H, 909)
    assert cap * (H // 8) > 2**32
    need_gib(2 * (cap * H * 2 >> 30) + 6)
    say(f"chunk pad/restore with 64-bit flat index N={N} H={H} cap={cap}")
    ref_rm, _ = oracle.chunk_map(sizes.numpy(), order.numpy(), 8, 128, N, cap)
    x, a, b = _pattern_rows(N, H, DEV)
    out = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    _, _, rm, _ = m.moe_sort_chunks_and_pad(x, sizes.to(DEV), order.to(DEV), 8, 128, cap,
                                            out=out, dev_status=st)
    assert_bits_equal(rm.cpu().numpy(), ref_rm, "row_map")
    d = _row_sample(cap, 910)
    src = ref_rm[d]
    exp = np.zeros((len(d), H), np.uint16)
    have = src >= 0
    exp[have] = _pattern_bits(a, b, src[have])
    assert_bits_equal(bits(out[torch.from_numpy(d).to(DEV)]), exp, "padded rows sample")
    # restore into the source buffer: every row is rewritten from the padded copy
    x.view(torch.int16).fill_(0x7FC1)
    m.moe_unpad_and_restore_chunks(out, rm, sizes.to(DEV), N, out=x, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    starts = np.cumsum(sizes.numpy().astype(np.int64))[:-1]      # first rows of chunks
    rows = _row_sample(N, 911, extra=starts[starts < N])
    assert_bits_equal(bits(x[torch.from_numpy(rows).to(DEV)]), _pattern_bits(a, b, rows),
                      "restored rows sample")


def test_row_kernels_spill_grid(m):
    """More than 2^20 tokens: one workgroup per token spills into gridDim.z."""
    T, H, E, k, ep = (1 << 20) + 4099, 8, 6, 3, 3
    need_gib(2)
    say(f"row kernels past 2^20 workgroups T={T} H={H} E={E} k={k}")
    w = workloads.random_routed(T, H, E, k, seed=912, zipf_s=0.5)
    idx_np, p_np = w.topk_idx.numpy(), w.probs.numpy()
    x_np, dy_np = workloads.bf16_bits(w.x), workloads.bf16_bits(w.dy)
    ref_map, _ = oracle.row_id_map(idx_np, E)
    idx, probs, x, dy = w.topk_idx.to(DEV), w.probs.to(DEV), w.x.to(DEV), w.dy.to(DEV)
    rm = torch.from_numpy(ref_map).to(DEV)
    P, Pp = m.moe_permute(x, idx, rm, probs)
    ref_P, ref_Pp = oracle.permute(x_np, p_np, idx_np, ref_map)
    assert_bits_equal(bits(P), ref_P, "permute")
    assert_bits_equal(Pp.cpu().numpy(), ref_Pp, "permuted probs")
    y = m.moe_unpermute(P, idx, rm, probs)
    assert_bits_equal(bits(y), oracle.unpermute(ref_P, p_np, idx_np, ref_map), "unpermute")
    y_ep = m.moe_unpermute_ep(P, idx, rm, ep, probs, bf16_partials=True, fp64_cross=True)
    assert_bits_equal(bits(y_ep), oracle.unpermute_ep(ref_P, p_np, idx_np, ref_map, ep, True,
                                                      True), "unpermute_ep")
    dP, dpr = m.moe_unpermute_bwd(dy, idx, rm, probs, P)
    ref_dP, ref_dpr = oracle.unpermute_bwd(dy_np, ref_P, p_np, idx_np, ref_map)
    assert_bits_equal(bits(dP), ref_dP, "unpermute_bwd act grad")
    rows = oracle_rows(idx_np, ref_map)
    dprob_ok(dpr.cpu().numpy(), ref_P[rows.ravel()].reshape(T, k, H), dy_np, ref_dpr)
    dx, dxp = m.moe_permute_bwd(dP, idx, rm, Pp)
    ref_dx, ref_dxp = oracle.permute_bwd(ref_dP, ref_Pp, idx_np, ref_map)
    assert_bits_equal(bits(dx), ref_dx, "permute_bwd")
    assert_bits_equal(dxp.cpu().numpy(), ref_dxp, "permute_bwd probs")


def test_mask_kernels_spill_grid(m):
    """The mask-map row kernels past 2^20 tokens."""
    T, H, E = (1 << 20) + 777, 8, 5
    need_gib(2)
    say(f"mask-map row kernels past 2^20 workgroups T={T} H={H} E={E}")
    g = torch.Generator().manual_seed(913)
    mask = torch.rand(T, E, generator=g) < 0.4
    pr = torch.rand(T, E, generator=g) * mask
    xx = torch.randn(T, H, generator=g).to(torch.bfloat16)
    gg = torch.randn(T, H, generator=g).to(torch.bfloat16)
    R = int(mask.sum())
    ref_map, _ = oracle.mask_row_id_map(mask.numpy().astype(np.uint8), -1)
    rm, _ = m.moe_make_mask_row_id_map(mask.to(DEV))
    got = rm.cpu().numpy()
    n = ref_map[:, 2 * E]
    assert np.array_equal(got[:, 2 * E], n)
    used = np.arange(E)[None, :] < n[:, None]
    assert np.array_equal(got[:, :E][used], ref_map[:, :E][used]), "mask row map"
    P, pp = m.moe_permute_mask(xx.to(DEV), rm, R, pr.to(DEV))
    ref_P, ref_pp = oracle.mask_permute(workloads.bf16_bits(xx), pr.numpy(), ref_map, R)
    assert_bits_equal(bits(P), ref_P, "mask permute")
    assert_bits_equal(pp.cpu().numpy(), ref_pp, "mask permuted probs")
    y, up = m.moe_unpermute_mask(P, rm, pr.to(DEV), pp)
    ref_y, ref_up = oracle.mask_unpermute(ref_P, pr.numpy(), ref_map, ref_pp)
    assert_bits_equal(bits(y), ref_y, "mask unpermute")
    assert_bits_equal(up.cpu().numpy(), ref_up, "mask unpermuted probs")
    dP, _ = m.moe_unpermute_mask_bwd(gg.to(DEV), P, pr.to(DEV), rm)
    ref_dP, _ = oracle.mask_unpermute_bwd(workloads.bf16_bits(gg), ref_P, pr.numpy(), ref_map)
    assert_bits_equal(bits(dP), ref_dP, "mask unpermute bwd act grad")


def test_router_spill_grid(m):
    """16 tokens per router workgroup and 4 per backward workgroup: past
    2^24 tokens both launches spill into gridDim.z."""
    T, E, k = (1 << 24) + 1000, 8, 2
    need_gib(4)
    say(f"router past 2^20 workgroups T={T} E={E} k={k}")
    g = torch.Generator().manual_seed(914)
    logits = torch.randn(T, E, generator=g)
    idx = torch.full((T, k), -2, dtype=torch.int32, device=DEV)
    probs = torch.full((T, k), float("nan"), device=DEV)
    m.moe_topk_softmax(logits.to(DEV), k, topk_idx=idx, probs=probs)
    ref_idx, ref_p = oracle.topk_softmax(logits.numpy(), k)
    got_idx = idx.cpu().numpy()
    assert np.array_equal(got_idx, ref_idx), f"{int((got_idx != ref_idx).sum())} indices differ"
    check_probs(probs.cpu().numpy(), ref_p, ref_idx, logits.numpy().astype(np.float64),
                "router")
    d_probs = torch.randn(T, k, generator=g)
    got = m.moe_topk_softmax_bwd(d_probs.to(DEV), torch.from_numpy(ref_p).to(DEV),
                                 torch.from_numpy(ref_idx).to(DEV), E).cpu().numpy()
    ref = oracle.topk_softmax_bwd(d_probs.numpy(), ref_p, ref_idx, E)
    sel = np.zeros((T, E), bool)
    np.put_along_axis(sel, ref_idx.astype(np.int64), True, axis=1)
    assert np.all(got[~sel].view(np.uint32) == 0), "unselected experts must hold +0"
    err = np.abs(np.take_along_axis(got, ref_idx.astype(np.int64), axis=1).astype(np.float64)
                 - np.take_along_axis(ref, ref_idx.astype(np.int64), axis=1))
    assert np.all(err <= grad_bound(d_probs.numpy(), ref_p, k) + 1e-44)
