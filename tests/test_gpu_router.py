"""GPU parity for the fused top-k softmax router and its gradient.

Expert indices must match the oracle bit for bit, ties included (the lower
expert index wins).  The weights are an fp32 softmax whose exponentials and
sum the kernel takes in fp32 while the oracle takes them in fp64 and rounds
once, so they are compared to a relative bound: each of the k terms carries
an fp32 subtraction, an expf (a few ulp) and a share of the sum, which
stays under (k + 16) * 2^-24 * (1 + |l_j - l_0|) of the value.  The
gradient w_j (dp_j - sum_i w_i dp_i) is compared to
(k + 4) * 2^-23 * w_j (|dp_j| + sum_i |w_i dp_i|): the fp32 dot product's
error bound.  Experts not selected must hold an exact +0.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

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


def oracle_in(logits):
    """The oracle takes fp32 arrays or bf16 bit patterns."""
    if logits.dtype == torch.bfloat16:
        return workloads.bf16_bits(logits.cpu())
    return logits.cpu().numpy()


def logit_values(logits):
    return logits.float().cpu().numpy().astype(np.float64)


def check_probs(got, ref, idx, logits64, what, rows=None):
    T, k = idx.shape
    lv = np.take_along_axis(logits64, idx.astype(np.int64), axis=1)
    spread = np.abs(lv - lv[:, :1])
    bound = (k + 16) * 2.0 ** -24 * (1.0 + spread) * np.abs(ref.astype(np.float64))
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    ok = err <= bound + 1e-44
    if rows is not None:
        ok = ok | ~rows[:, None]
    assert ok.all(), f"{what}: {int((~ok).sum())} weights out of bound, worst rel " \
                     f"{float(np.max(err / np.maximum(np.abs(ref), 1e-38))):.3g}"


def run_router(m, logits, k):
    T = logits.shape[0]
    idx = torch.full((T, k), -2, dtype=torch.int32, device=DEV)
    probs = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
    m.moe_topk_softmax(logits, k, topk_idx=idx, probs=probs)
    return idx.cpu().numpy(), probs.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "finegrain", "skewed"])
def test_router_configs(m, name):
    w = workloads.ROUTED[name]()
    say(f"router {name} T={w.T} E={w.num_experts} k={w.k} {w.logits.dtype}")
    idx, probs = run_router(m, w.logits.to(DEV), w.k)
    ref_idx, ref_probs = oracle.topk_softmax(oracle_in(w.logits), w.k)
    assert np.array_equal(idx, ref_idx), f"{int((idx != ref_idx).sum())} indices differ"
    check_probs(probs, ref_probs, ref_idx, logit_values(w.logits), name)


@pytest.mark.parametrize("T,E,k", [(70, 1, 1), (33, 3, 3), (65, 65, 7), (100, 100, 64),
                                   (20, 2048, 64), (130, 256, 8), (5, 2047, 33), (3, 64, 64),
                                   (257, 128, 2)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_router_ties_and_shapes(m, T, E, k, dtype):
    """Integer logits in [-2, 2] make most comparisons ties."""
    say(f"router ties T={T} E={E} k={k} {dtype}")
    g = torch.Generator().manual_seed(T * 7919 + E * 31 + k)
    logits = torch.randint(-2, 3, (T, E), generator=g).to(dtype)
    idx, probs = run_router(m, logits.to(DEV), k)
    ref_idx, ref_probs = oracle.topk_softmax(oracle_in(logits), k)
    assert np.array_equal(idx, ref_idx), f"{int((idx != ref_idx).sum())} indices differ"
    check_probs(probs, ref_probs, ref_idx, logit_values(logits), "ties")


def test_router_special_values(m):
    """-inf and huge logits: exp underflows to 0 on both sides."""
    say("router special values")
    g = torch.Generator().manual_seed(99)
    T, E, k = 96, 160, 6
    logits = torch.randn(T, E, generator=g) * 4
    logits[::3, 5:50] = float("-inf")
    logits[1::4, 7] = 3e38
    logits[2::5, 100] = -3e38
    idx, probs = run_router(m, logits.to(DEV), k)
    ref_idx, ref_probs = oracle.topk_softmax(logits.numpy(), k)
    assert np.array_equal(idx, ref_idx)
    check_probs(probs, ref_probs, ref_idx, logit_values(logits), "special")


def test_router_nan_ranks_last(m):
    """A NaN logit ranks below every number, ties among NaNs to the lower
    index -- the oracle's order on the same logits with NaN made -inf (no
    genuine -inf present).  Weights are checked on rows that selected none."""
    say("router NaN logits")
    g = torch.Generator().manual_seed(98)
    T, E, k = 64, 72, 8
    logits = torch.randn(T, E, generator=g)
    nan_mask = torch.rand(T, E, generator=g) < 0.2
    nan_mask[:4] = torch.rand(4, E, generator=g) < 0.95   # rows with fewer than k numbers
    logits[nan_mask] = float("nan")
    idx, probs = run_router(m, logits.to(DEV), k)
    ref_idx, ref_probs = oracle.topk_softmax(
        torch.where(nan_mask, torch.tensor(float("-inf")), logits).numpy(), k)
    assert np.array_equal(idx, ref_idx)
    picked_nan = np.take_along_axis(nan_mask.numpy(), ref_idx.astype(np.int64), axis=1)
    clean = ~picked_nan.any(axis=1)
    assert clean.sum() > T // 2
    check_probs(probs, ref_probs, ref_idx, np.nan_to_num(logit_values(logits)), "nan", clean)


def test_router_rejects_bad_shapes(m):
    say("router argument checks")
    x = torch.zeros(4, 8, dtype=torch.float32, device=DEV)
    for k in (0, 9):
        with pytest.raises(m.MoeError):
            m.moe_topk_softmax(x, k)
    with pytest.raises(m.MoeError):
        m.moe_topk_softmax(torch.zeros(2, 4096, device=DEV), 4)
    with pytest.raises(m.MoeError):
        m.moe_topk_softmax(torch.zeros(2, 128, device=DEV), 65)
    idx, probs = m.moe_topk_softmax(torch.zeros(0, 16, device=DEV), 2)
    assert idx.shape == (0, 2) and probs.shape == (0, 2)


def grad_bound(d_probs, probs, k):
    wdp = np.abs(probs.astype(np.float64) * d_probs.astype(np.float64))
    return (k + 4) * 2.0 ** -23 * np.abs(probs) * (np.abs(d_probs) + wdp.sum(1, keepdims=True))


@pytest.mark.parametrize("name", ["tiny", "finegrain", "skewed"])
def test_router_bwd_configs(m, name):
    w = workloads.ROUTED[name]()
    T, E, k = w.T, w.num_experts, w.k
    say(f"router bwd {name}")
    g = torch.Generator().manual_seed(17)
    d_probs = torch.randn(T, k, generator=g)
    d_logits = torch.full((T, E), float("nan"), device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    m.moe_topk_softmax_bwd(d_probs.to(DEV), w.probs.to(DEV), w.topk_idx.to(DEV), E,
                           d_logits=d_logits, dev_status=st)
    assert int(st.item()) == 0
    got = d_logits.cpu().numpy()
    ref = oracle.topk_softmax_bwd(d_probs.numpy(), w.probs.numpy(), w.topk_idx.numpy(), E)
    sel = np.zeros((T, E), bool)
    np.put_along_axis(sel, w.topk_idx.numpy().astype(np.int64), True, axis=1)
    assert np.all(got[~sel].view(np.uint32) == 0), "unselected experts must hold +0"
    gsel = np.take_along_axis(got, w.topk_idx.numpy().astype(np.int64), axis=1)
    rsel = np.take_along_axis(ref, w.topk_idx.numpy().astype(np.int64), axis=1)
    bound = grad_bound(d_probs.numpy(), w.probs.numpy(), k)
    err = np.abs(gsel.astype(np.float64) - rsel)
    assert np.all(err <= bound + 1e-44), f"worst {float(np.max(err - bound)):.3g} over bound"


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (65, 3, 2), (40, 2048, 64), (129, 100, 64),
                                   (7, 64, 64)])
def test_router_bwd_edges(m, T, E, k):
    say(f"router bwd edge T={T} E={E} k={k}")
    g = torch.Generator().manual_seed(T + E + k)
    logits = torch.randn(T, E, generator=g)
    idx, probs = oracle.topk_softmax(logits.numpy(), k)
    d_probs = torch.randn(T, k, generator=g).numpy()
    got = m.moe_topk_softmax_bwd(torch.from_numpy(d_probs).to(DEV),
                                 torch.from_numpy(probs).to(DEV),
                                 torch.from_numpy(idx).to(DEV), E).cpu().numpy()
    ref = oracle.topk_softmax_bwd(d_probs, probs, idx, E)
    sel = np.zeros((T, E), bool)
    np.put_along_axis(sel, idx.astype(np.int64), True, axis=1)
    assert np.all(got[~sel].view(np.uint32) == 0)
    err = np.abs(np.take_along_axis(got, idx.astype(np.int64), axis=1).astype(np.float64)
                 - np.take_along_axis(ref, idx.astype(np.int64), axis=1))
    assert np.all(err <= grad_bound(d_probs, probs, k) + 1e-44)


def test_router_bwd_bad_expert_sets_status(m):
    say("router bwd bad expert")
    T, E, k = 8, 16, 2
    idx = torch.tensor([[0, 1]] * T, dtype=torch.int32)
    idx[3, 1] = E
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    m.moe_topk_softmax_bwd(torch.ones(T, k, device=DEV), torch.full((T, k), 0.5, device=DEV),
                           idx.to(DEV), E, dev_status=st)
    assert int(st.item()) & m.DEV_BAD_EXPERT


def test_router_feeds_row_map_and_permute(m):
    """Router -> row map -> permute on the GPU equals the same chain in the oracle."""
    w = workloads.ROUTED["finegrain"]()
    T, H, E, k = w.T, w.H, w.num_experts, w.k
    say("router -> row map -> permute chain")
    idx, probs = m.moe_topk_softmax(w.logits.to(DEV), k)
    rm, off = m.moe_make_row_id_map(idx, E)
    x = w.x.to(DEV)
    out, out_p = m.moe_permute(x, idx, rm, probs)
    ref_idx, ref_probs = oracle.topk_softmax(oracle_in(w.logits), k)
    ref_map, ref_off = oracle.row_id_map(ref_idx, E)
    assert np.array_equal(rm.cpu().numpy(), ref_map)
    assert np.array_equal(off.cpu().numpy(), ref_off)
    ref_out, ref_out_p = oracle.permute(workloads.bf16_bits(w.x), probs.cpu().numpy(), ref_idx,
                                        ref_map)
    assert np.array_equal(workloads.bf16_bits(out.cpu()), ref_out)
    # permuted probs are the router's own weights, moved bit for bit
    assert np.array_equal(out_p.cpu().numpy().view(np.uint32), ref_out_p.view(np.uint32))


def bf16_value(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_bf16_rounding(got_bits, ref_bits, ref_f32, bound, what):
    """got and ref are bf16 roundings of two fp32/fp64 values within `bound`
    of each other: equal, except where the rounding boundary between the two
    candidates lies within `bound` (plus half an fp32 ulp) of the fp32 value."""
    got_bits = np.asarray(got_bits, np.uint16)
    ref_bits = np.asarray(ref_bits, np.uint16)
    diff = got_bits != ref_bits
    if not diff.any():
        return
    a, b = bf16_value(got_bits[diff]), bf16_value(ref_bits[diff])
    r = np.asarray(ref_f32, np.float64)[diff]
    slack = np.asarray(bound, np.float64)[diff] + np.abs(r) * 2.0 ** -24 + 1e-44
    near = np.abs((a + b) / 2 - r) <= slack
    one_ulp = np.abs(a - b) <= np.ldexp(1.0, np.frexp(np.maximum(np.abs(a), np.abs(b)))[1] - 8)
    assert (near & one_ulp).all(), f"{what}: {int((~(near & one_ulp)).sum())} bf16 values off"


@pytest.mark.parametrize("name", ["tiny", "finegrain", "skewed"])
def test_router_bf16_weights(m, name):
    """Weights in the activation dtype (fp32_routing off): the kernel's fp32
    weight rounded to nearest-even bf16."""
    w = workloads.ROUTED[name]()
    lg = w.logits.to(torch.bfloat16)
    k, E = w.k, w.num_experts
    say(f"router bf16 weights {name}")
    idx16, p16 = m.moe_topk_softmax(lg.to(DEV), k, fp32_routing=False)
    idx32, p32 = m.moe_topk_softmax(lg.to(DEV), k)
    assert p16.dtype == torch.bfloat16
    assert torch.equal(idx16, idx32)
    assert np.array_equal(workloads.bf16_bits(p16.cpu()), workloads.bf16_bits(p32.cpu().to(torch.bfloat16)))
    lb = workloads.bf16_bits(lg)
    ref_idx, ref16 = oracle.topk_softmax(lb, k, prob_bytes=2)
    _, ref32 = oracle.topk_softmax(lb, k)
    assert np.array_equal(idx16.cpu().numpy(), ref_idx)
    lv = np.take_along_axis(logit_values(lg), ref_idx.astype(np.int64), axis=1)
    bound = (k + 16) * 2.0 ** -24 * (1.0 + np.abs(lv - lv[:, :1])) * np.abs(ref32)
    assert_bf16_rounding(workloads.bf16_bits(p16.cpu()), ref16, ref32, bound, name)


@pytest.mark.parametrize("pdt,ldt", [(torch.bfloat16, torch.bfloat16), (torch.bfloat16, torch.float32),
                                     (torch.float32, torch.bfloat16)])
@pytest.mark.parametrize("T,E,k", [(300, 64, 6), (77, 256, 8), (20, 2048, 64)])
def test_router_bwd_dtypes(m, pdt, ldt, T, E, k):
    say(f"router bwd {pdt} -> {ldt} T={T} E={E} k={k}")
    g = torch.Generator().manual_seed(T * 3 + k)
    logits = torch.randn(T, E, generator=g)
    idx, probs = oracle.topk_softmax(logits.numpy(), k)
    w = torch.from_numpy(probs).to(pdt)
    dp = torch.randn(T, k, generator=g).to(pdt)
    got = m.moe_topk_softmax_bwd(dp.to(DEV), w.to(DEV), torch.from_numpy(idx).to(DEV), E,
                                 logits_dtype=ldt).cpu()
    assert got.dtype == ldt
    w_in = workloads.bf16_bits(w) if pdt == torch.bfloat16 else w.numpy()
    dp_in = workloads.bf16_bits(dp) if pdt == torch.bfloat16 else dp.numpy()
    ref32 = oracle.topk_softmax_bwd(dp_in, w_in, idx, E)
    il = idx.astype(np.int64)
    bound_sel = grad_bound(dp.float().numpy(), w.float().numpy(), k)
    bound = np.zeros((T, E))
    np.put_along_axis(bound, il, bound_sel, axis=1)
    sel = np.zeros((T, E), bool)
    np.put_along_axis(sel, il, True, axis=1)
    if ldt == torch.float32:
        gv = got.numpy()
        assert np.all(gv[~sel].view(np.uint32) == 0)
        assert np.all(np.abs(gv.astype(np.float64) - ref32) <= bound + 1e-44)
    else:
        gb = workloads.bf16_bits(got)
        assert np.all(gb[~sel] == 0)
        ref16 = oracle.topk_softmax_bwd(dp_in, w_in, idx, E, logit_bytes=2)
        assert_bf16_rounding(gb, ref16, ref32, bound, "bwd bf16")
