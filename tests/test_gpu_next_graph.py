"""Graph capture and repeatability of the next rows' entry points.

Each chain is captured once in a hipGraph and replayed with new device-resident
inputs (routing, masks, logits) between eager work and synchronisations; every
replay must match the oracle chain on the same inputs, bit for bit where the
single calls are bit-exact.  Repeated eager calls must give identical bits.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from test_gpu_router import check_probs

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


def capture(step):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    return g


def bf16_of(t):
    return workloads.bf16_bits(t.cpu())


def test_graph_router_to_ep_combine(m):
    """Router -> row map -> FP8 permute with scales -> EP combine, replayed with
    new logits and rows."""
    T, H, E, k, ep = 512, 512, 64, 6, 8
    say("graph replay: router -> row map -> fp8 permute -> EP combine")
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    x8 = torch.empty((T, H), dtype=torch.float8_e4m3fn, device=DEV)
    sc = torch.empty((T, H // 128), dtype=torch.float32, device=DEV)
    P = torch.empty((T * k, H), dtype=torch.bfloat16, device=DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    probs = torch.empty((T, k), dtype=torch.float32, device=DEV)
    rm = torch.empty((E, T), dtype=torch.int32, device=DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    ws = torch.empty(m.moe_make_row_id_map_workspace_bytes(T, k, E), dtype=torch.uint8,
                     device=DEV)
    q8 = torch.empty((T * k, H), dtype=torch.float8_e4m3fn, device=DEV)
    qs = torch.empty((T * k, H // 128), dtype=torch.float32, device=DEV)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)

    def step():
        m.moe_topk_softmax(logits, k, topk_idx=idx, probs=probs)
        m.moe_make_row_id_map(idx, E, row_id_map=rm, expert_offsets=off, workspace=ws)
        m.moe_permute_scaled(x8, idx, rm, sc, out=q8, out_scale=qs)
        m.moe_unpermute_ep(P, idx, rm, ep, probs, bf16_partials=True, fp64_cross=True, out=y)

    g = capture(step)
    for rep in range(6):
        gen = torch.Generator().manual_seed(7000 + rep)
        lg = torch.randn(T, E, generator=gen) - 0.4 * rep * torch.log1p(
            torch.randperm(E, generator=gen).float())[None, :]
        xq, xs = workloads.quantize_fp8_rows(torch.randn(T, H, generator=gen), 128)
        rows = workloads.random_rows(T * k, H, seed=7100 + rep)
        logits.copy_(lg)
        x8.copy_(xq)
        sc.copy_(xs)
        P.copy_(rows)
        q8.view(torch.uint8).fill_(0xA5)
        g.replay()
        torch.cuda.synchronize()
        ref_idx, ref_p = oracle.topk_softmax(lg.numpy(), k)
        assert np.array_equal(idx.cpu().numpy(), ref_idx), f"replay {rep} router indices"
        got_p = probs.cpu().numpy()
        check_probs(got_p, ref_p, ref_idx, lg.numpy().astype(np.float64),
                    f"replay {rep} router weights")
        ref_rm, ref_off = oracle.row_id_map(ref_idx, E)
        assert np.array_equal(rm.cpu().numpy(), ref_rm), f"replay {rep} row map"
        assert np.array_equal(off.cpu().numpy(), ref_off)
        ref_q, ref_s, _ = oracle.permute_scaled(xq.view(torch.uint8).numpy(), xs.numpy(), None,
                                                ref_idx, ref_rm)
        assert np.array_equal(q8.cpu().view(torch.uint8).numpy(), ref_q), f"replay {rep} fp8"
        assert np.array_equal(qs.cpu().numpy().view(np.uint8).reshape(T * k, -1), ref_s)
        # the combine weights are the router's own (GPU) weights on both sides
        ref_y = oracle.unpermute_ep(bf16_of(rows), got_p, ref_idx, ref_rm, ep, True, True)
        assert np.array_equal(bf16_of(y), ref_y), f"replay {rep} EP combine"


def test_graph_mask_chain(m):
    """Mask map (fixed capacity) -> permute -> unpermute -> backward, replayed
    with masks whose routed totals change."""
    T, H, E = 600, 264, 20
    cap = T * 6
    say("graph replay: mask-map chain")
    mask = torch.empty((T, E), dtype=torch.bool, device=DEV)
    probs = torch.empty((T, E), dtype=torch.float32, device=DEV)
    x = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    dy = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    rm = torch.empty((T, 2 * E + 1), dtype=torch.int32, device=DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    ws = torch.empty(m.moe_make_mask_row_id_map_workspace_bytes(T, E), dtype=torch.uint8,
                     device=DEV)
    P = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    pp = torch.empty(cap, dtype=torch.float32, device=DEV)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    up = torch.empty((T, E), dtype=torch.float32, device=DEV)
    dP = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    dmp = torch.empty((T, E), dtype=torch.float32, device=DEV)

    def step():
        m.moe_make_mask_row_id_map(mask, num_out_tokens=cap, row_id_map=rm, expert_offsets=off,
                                   workspace=ws)
        m.moe_permute_mask(x, rm, cap, probs, out=P, out_probs=pp)
        m.moe_unpermute_mask(P, rm, probs, pp, out=y, unpermuted_probs=up)
        m.moe_unpermute_mask_bwd(dy, P, probs, rm, d_in=dP, d_merging_probs=dmp)

    g = capture(step)
    for rep in range(5):
        gen = torch.Generator().manual_seed(8000 + rep)
        mk = torch.rand(T, E, generator=gen) < 0.05 * (rep + 1)
        pr = torch.rand(T, E, generator=gen) * mk
        xx = torch.randn(T, H, generator=gen).to(torch.bfloat16)
        gg = torch.randn(T, H, generator=gen).to(torch.bfloat16)
        mask.copy_(mk)
        probs.copy_(pr)
        x.copy_(xx)
        dy.copy_(gg)
        P.view(torch.int16).fill_(0x7FC1)
        dP.view(torch.int16).fill_(0x7FC1)
        g.replay()
        torch.cuda.synchronize()
        R = int(mk.sum())
        ref_map, ref_off = oracle.mask_row_id_map(mk.numpy().astype(np.uint8), cap)
        got_map = rm.cpu().numpy()
        n = ref_map[:, 2 * E]
        assert np.array_equal(got_map[:, 2 * E], n)
        used = np.arange(E)[None, :] < n[:, None]
        assert np.array_equal(got_map[:, :E][used], ref_map[:, :E][used]), f"replay {rep} map"
        assert np.array_equal(off.cpu().numpy(), ref_off)
        ref_P, ref_pp = oracle.mask_permute(bf16_of(xx), pr.numpy(), ref_map, cap,
                                            out=np.full((cap, H), 0x7FC1, np.uint16))
        assert np.array_equal(bf16_of(P), ref_P), f"replay {rep} permute"
        kept = int(n.sum())
        assert np.array_equal(pp.cpu().numpy()[:kept].view(np.uint32),
                              ref_pp[:kept].view(np.uint32)), f"replay {rep} permuted probs"
        ref_y, ref_up = oracle.mask_unpermute(ref_P, pr.numpy(), ref_map, pp.cpu().numpy())
        assert np.array_equal(bf16_of(y), ref_y), f"replay {rep} unpermute"
        assert np.array_equal(up.cpu().numpy().view(np.uint32), ref_up.view(np.uint32))
        ref_dP, _ = oracle.mask_unpermute_bwd(bf16_of(gg), ref_P, pr.numpy(), ref_map,
                                              d_in=np.full((cap, H), 0x7FC1, np.uint16))
        assert np.array_equal(bf16_of(dP), ref_dP), f"replay {rep} act grad"
        assert R <= cap


def test_next_rows_repeatable(m):
    """The same call twice gives the same bits (no atomics decide any value)."""
    say("repeatability of the next rows")
    w = workloads.ROUTED["skewed"]()
    T, H, E, k = w.T, w.H, w.num_experts, w.k
    lg = w.logits.to(DEV)
    a = m.moe_topk_softmax(lg, k)
    b = m.moe_topk_softmax(lg, k)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))
    d1 = m.moe_topk_softmax_bwd(torch.ones_like(a[1]), a[1], a[0], E)
    d2 = m.moe_topk_softmax_bwd(torch.ones_like(a[1]), a[1], a[0], E)
    assert torch.equal(d1.view(torch.int32), d2.view(torch.int32))
    idx = w.topk_idx.to(DEV)
    rm, _ = m.moe_make_row_id_map(idx, E)
    Tn = 2048                                   # a token prefix keeps this test short
    P = workloads.random_rows(Tn * k, H, seed=5, device=DEV)
    sub = idx[:Tn].contiguous()
    rms, _ = m.moe_make_row_id_map(sub, E)
    probs = w.probs[:Tn].to(DEV)
    y1 = m.moe_unpermute_ep(P, sub, rms, 16, probs, fp64_cross=True)
    y2 = m.moe_unpermute_ep(P, sub, rms, 16, probs, fp64_cross=True)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    mask = torch.zeros((Tn, E), dtype=torch.bool, device=DEV)
    mask.scatter_(1, sub.long(), True)
    pte = torch.zeros((Tn, E), device=DEV)
    pte.scatter_(1, sub.long(), probs)
    mm, _ = m.moe_make_mask_row_id_map(mask)
    dy = workloads.random_rows(Tn, H, seed=6, device=DEV)
    r1 = m.moe_unpermute_mask_bwd(dy, P, pte, mm)
    r2 = m.moe_unpermute_mask_bwd(dy, P, pte, mm)
    assert torch.equal(r1[0].view(torch.int16), r2[0].view(torch.int16))
    assert torch.equal(r1[1].view(torch.int32), r2[1].view(torch.int32))
