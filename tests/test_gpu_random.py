"""GPU parity on seeded random shapes: the whole routed chain and the whole
chunk chain on shapes drawn from a fixed generator -- odd and even hidden
sizes, any k up to 16, skewed and uniform routing, every chunk alignment --
each compared with the CPU oracle to the same bar as the named workloads
(bit for bit; the prob-grad dots within 1e-5 of their absolute-product sum).

The draws are fixed at import, so every run tests the same shapes and each
case id names its shape.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from test_gpu_parity import (DEV, _raw, assert_bits_equal, bits, dprob_ok, oracle_rows, say,
                             sentinel_bf16, sentinel_f32, sentinel_i32)

pytestmark = pytest.mark.gpu


def _routed_cases(n=24, seed=20261):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        E = int(rng.choice([1, 2, 3, 7, 16, 33, 64, 100, 256, 300]))
        k = int(rng.integers(1, min(E, 16) + 1))
        T = int(rng.integers(1, 600))
        H = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(8, 1000)) * 8,
                            int(rng.integers(64, 9000))]))
        zipf = float(rng.choice([0.0, 1.1]))
        divisors = [d for d in range(1, E + 1) if E % d == 0]
        ep = int(rng.choice(divisors))
        cases.append((T, H, E, k, zipf, ep, 1000 + i))
    return cases


def _chunk_cases(n=16, seed=20262):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        ranks = int(rng.integers(1, 9))
        experts = int(rng.integers(1, 33))
        align = int(rng.choice([1, 2, 8, 16, 64, 128]))
        N = int(rng.integers(0, 5000))
        H = int(rng.choice([int(rng.integers(1, 40)), int(rng.integers(8, 600)) * 8]))
        empty = int(rng.integers(0, ranks * experts))
        extra = int(rng.integers(0, 300))
        fp32 = bool(rng.random() < 0.3)
        half_probs = bool(rng.random() < 0.3)
        cases.append((N, H, ranks, experts, align, empty, extra, fp32, half_probs, 2000 + i))
    return cases


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import unpermute_moe_make_amd as mod
    return mod


@pytest.mark.parametrize("T,H,E,k,zipf,ep,seed", _routed_cases())
def test_random_routed_chain(m, T, H, E, k, zipf, ep, seed):
    say(f"random routed T={T} H={H} E={E} k={k} zipf={zipf} ep={ep} seed={seed}")
    w = workloads.random_routed(T, H, E, k, seed=seed, zipf_s=zipf)
    ib, pb, xb = w.topk_idx.numpy(), w.probs.numpy(), workloads.bf16_bits(w.x)
    ref_map, ref_off = oracle.row_id_map(ib, E)
    x, idx, probs, dy = (w.x.to(DEV), w.topk_idx.to(DEV), w.probs.to(DEV), w.dy.to(DEV))
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    rm, off = m.moe_make_row_id_map(idx, E, row_id_map=sentinel_i32((E, T)),
                                    expert_offsets=sentinel_i32((E + 1,)), dev_status=st)
    torch.cuda.synchronize()
    assert_bits_equal(rm.cpu().numpy(), ref_map, "row_id_map")
    assert_bits_equal(off.cpu().numpy(), ref_off, "expert_offsets")
    out, out_p = m.moe_permute(x, idx, rm, probs, out=sentinel_bf16((T * k, H)),
                               out_probs=sentinel_f32((T * k,)), dev_status=st)
    o, op = oracle.permute(xb, pb, ib, ref_map)
    assert_bits_equal(bits(out), o, "permute")
    assert_bits_equal(out_p.cpu().numpy(), op, "permuted probs")
    P = workloads.random_rows(T * k, H, seed=seed + 7, device=DEV)
    y = m.moe_unpermute(P, idx, rm, probs, out=sentinel_bf16((T, H)), dev_status=st)
    assert_bits_equal(bits(y), oracle.unpermute(bits(P), pb, ib, ref_map), "unpermute")
    for partials, fp64 in ((True, False), (False, True)):
        ye = m.moe_unpermute_ep(P, idx, rm, ep, probs, bf16_partials=partials, fp64_cross=fp64,
                                out=sentinel_bf16((T, H)), dev_status=st)
        ref = oracle.unpermute_ep(bits(P), pb, ib, ref_map, ep, partials, fp64)
        assert_bits_equal(bits(ye), ref, f"unpermute_ep partials={partials} fp64={fp64}")
    d_in, d_p = m.moe_unpermute_bwd(dy, idx, rm, probs, P, d_in=sentinel_bf16((T * k, H)),
                                    d_probs=sentinel_f32((T, k)), dev_status=st)
    ref_in, ref_p = oracle.unpermute_bwd(workloads.bf16_bits(w.dy), bits(P), pb, ib, ref_map)
    assert_bits_equal(bits(d_in), ref_in, "unpermute_bwd")
    dprob_ok(d_p.cpu().numpy(), bits(P)[oracle_rows(ib, ref_map)], workloads.bf16_bits(w.dy),
             ref_p)
    dpp = torch.randn(T * k, generator=torch.Generator().manual_seed(seed)).to(DEV)
    d_x, d_pp = m.moe_permute_bwd(P, idx, rm, dpp, d_x=sentinel_bf16((T, H)),
                                  d_probs=sentinel_f32((T, k)), dev_status=st)
    rx, rp = oracle.permute_bwd(bits(P), dpp.cpu().numpy(), ib, ref_map)
    assert_bits_equal(bits(d_x), rx, "permute_bwd")
    assert_bits_equal(d_pp.cpu().numpy(), rp, "permute_bwd probs")
    torch.cuda.synchronize()
    assert int(st.item()) == 0


# Calls past the 256 MiB streaming threshold (non-temporal rows, the permute's
# prefetch, the two-launch backward), with hidden sizes that are not powers of
# two and rows longer than one workgroup pass.
STREAMING = [(2048, 8200, 64, 8, 0.0, 4, 6000), (1024, 7168, 256, 16, 1.1, 8, 6001),
             (4096, 4096, 32, 8, 0.0, 32, 6002), (3000, 5120, 100, 6, 1.1, 4, 6003),
             (1500, 12288, 16, 8, 0.0, 2, 6004), (2048, 7168, 512, 12, 1.1, 16, 6005),
             (640, 20488, 24, 8, 0.0, 3, 6006)]


@pytest.mark.parametrize("T,H,E,k,zipf,ep,seed", STREAMING)
def test_random_routed_chain_streaming(m, T, H, E, k, zipf, ep, seed):
    assert 2 * H * (2 * T * k + T) > 256 << 20
    test_random_routed_chain(m, T, H, E, k, zipf, ep, seed)


@pytest.mark.parametrize("N,H,ranks,experts,align,empty,extra,fp32,half_probs,seed",
                         _chunk_cases())
def test_random_chunk_chain(m, N, H, ranks, experts, align, empty, extra, fp32, half_probs,
                            seed):
    say(f"random chunks N={N} H={H} ranks={ranks} experts={experts} align={align} "
        f"empty={empty} extra={extra} fp32={fp32} half_probs={half_probs} seed={seed}")
    g = torch.Generator().manual_seed(seed)
    dtype = torch.float32 if fp32 else torch.bfloat16
    x = torch.randn(N, H, generator=g).to(dtype)
    probs = torch.rand(N, generator=g)
    if half_probs:
        probs = probs.to(torch.float16)
    sizes = workloads.chunk_sizes(N, ranks, experts, empty, g)
    order = workloads.expert_major_order(ranks, experts)
    out_cap = workloads.padded_capacity(N, experts, align) + extra
    C, R = ranks * experts, ranks
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    xd, pd, sd, od = x.to(DEV), probs.to(DEV), sizes.to(DEV), order.to(DEV)
    fill = (lambda shape: sentinel_bf16(shape)) if not fp32 else \
        (lambda shape: torch.full(shape, float("nan"), device=DEV))
    pfill = (lambda n: sentinel_f32((n,))) if not half_probs else \
        (lambda n: torch.full((n,), float("nan"), dtype=torch.float16, device=DEV))
    out, out_p, rm, off = m.moe_sort_chunks_and_pad(
        xd, sd, od, R, align, out_cap, pd, out=fill((out_cap, H)), out_probs=pfill(out_cap),
        row_map=sentinel_i32((out_cap,)), padded_offsets=sentinel_i32((experts + 1,)),
        dev_status=st)
    xr, pr = _raw(x), _raw(probs)
    r_out, r_p, r_rm, r_off = oracle.sort_chunks_and_pad(xr, pr, sizes.numpy(), order.numpy(), R,
                                                         align, out_cap)
    assert_bits_equal(rm.cpu().numpy(), r_rm, "row_map")
    assert_bits_equal(off.cpu().numpy(), r_off, "padded_offsets")
    assert_bits_equal(_raw(out), r_out, "padded rows")
    assert_bits_equal(_raw(out_p), r_p, "padded probs")
    back, back_p = m.moe_unpad_and_restore_chunks(out, rm, sd, N, out_p, out=fill((N, H)),
                                                  out_probs=pfill(N), dev_status=st)
    ref_b, ref_bp = oracle.unpad_and_restore_chunks(r_out, r_p, r_rm, sizes.numpy(), N)
    assert_bits_equal(_raw(back), ref_b, "restored rows")
    assert_bits_equal(_raw(back_p), ref_bp, "restored probs")
    gpad = torch.randn(out_cap, H, generator=g).to(dtype)
    gpp = torch.rand(out_cap, generator=g).to(probs.dtype)
    d_in, d_inp = m.moe_sort_chunks_and_pad_bwd(gpad.to(DEV), rm, sd, N, gpp.to(DEV),
                                                d_in=fill((N, H)), d_in_probs=pfill(N),
                                                dev_status=st)
    rd, rdp = oracle.sort_chunks_and_pad_bwd(_raw(gpad), _raw(gpp), r_rm, sizes.numpy(), N)
    assert_bits_equal(_raw(d_in), rd, "sort-and-pad bwd rows")
    assert_bits_equal(_raw(d_inp), rdp, "sort-and-pad bwd probs")
    grest = torch.randn(N, H, generator=g).to(dtype)
    d_pad, d_padp = m.moe_unpad_and_restore_chunks_bwd(grest.to(DEV), rm, out_cap, pd,
                                                       d_in=fill((out_cap, H)),
                                                       d_in_probs=pfill(out_cap),
                                                       dev_status=st)
    rpd, rpp = oracle.unpad_and_restore_chunks_bwd(_raw(grest), pr, r_rm, out_cap)
    assert_bits_equal(_raw(d_pad), rpd, "restore bwd rows")
    assert_bits_equal(_raw(d_padp), rpp, "restore bwd probs")
    torch.cuda.synchronize()
    assert int(st.item()) == 0
