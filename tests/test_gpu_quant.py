"""GPU parity for quantized rows: FP8 (OCP E4M3FN) data rows with their block
scales (fp32 or E8M0) permuted alongside, in the top-k and the mask-map form.

Everything here is a byte copy, so the bar is bit-exact against the oracle;
rows and scale rows that no route names must keep the caller's sentinel.
The dequantized permuted rows are also checked to equal the dequantized
source rows, which is what a consumer of the permuted FP8 tensor relies on.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SENT = 0xA5


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import unpermute_moe_make_amd as mod
    return mod


def byte_view(t):
    t = t.contiguous().cpu()
    return t.view(torch.uint8).numpy().reshape(t.shape[0], -1)


def sentinel_like(shape, dtype):
    t = torch.empty(shape, dtype=dtype, device=DEV)
    t.view(torch.uint8).fill_(SENT)
    return t


def dequant(q, s, block, H):
    return q.float() * s.float().repeat_interleave(block, dim=1)[:, :H]


def fp8_case(x, block, sdt):
    return workloads.quantize_fp8_rows(x, block, sdt)


def mask_from_topk(idx, E):
    mask = torch.zeros((idx.shape[0], E), dtype=torch.bool)
    mask.scatter_(1, idx.long(), True)
    return mask


@pytest.mark.parametrize("name", ["tiny", "finegrain", "skewed"])
@pytest.mark.parametrize("sdt", [torch.float32, torch.float8_e8m0fnu])
def test_permute_scaled_configs(m, name, sdt):
    w = workloads.ROUTED[name]()
    T, H, E, k = w.T, w.H, w.num_experts, w.k
    block = 128 if H % 128 == 0 else 32
    say(f"permute fp8 {name} block={block} scale={sdt}")
    q, sc = fp8_case(w.x, block, sdt)
    rm_ref, _ = oracle.row_id_map(w.topk_idx.numpy(), E)
    idx, rm = w.topk_idx.to(DEV), torch.from_numpy(rm_ref).to(DEV)
    out = sentinel_like((T * k, H), q.dtype)
    out_s = sentinel_like((T * k, sc.shape[1]), sc.dtype)
    out_p = torch.full((T * k,), -3.0, device=DEV)
    m.moe_permute_scaled(q.to(DEV), idx, rm, sc.to(DEV), w.probs.to(DEV), out=out,
                         out_scale=out_s, out_probs=out_p)
    if T * H <= (1 << 24):
        ref, ref_s, ref_p = oracle.permute_scaled(byte_view(q), byte_view(sc), w.probs.numpy(),
                                                  w.topk_idx.numpy(), rm_ref)
        np.testing.assert_array_equal(byte_view(out), ref)
        np.testing.assert_array_equal(byte_view(out_s), ref_s)
        np.testing.assert_array_equal(out_p.cpu().numpy().view(np.uint32), ref_p.view(np.uint32))
    else:
        rows = torch.from_numpy(
            rm_ref[w.topk_idx.numpy().astype(np.int64), np.arange(T)[:, None]].ravel()).to(DEV)
        src = torch.arange(T, device=DEV).repeat_interleave(k)
        qd = q.to(DEV)
        exp = torch.empty_like(out)
        exp.view(torch.uint8)[rows] = qd.view(torch.uint8)[src]
        assert torch.equal(out.view(torch.uint8), exp.view(torch.uint8))
        exp_s = torch.empty_like(out_s)
        exp_s.view(torch.uint8)[rows] = sc.to(DEV).view(torch.uint8)[src]
        assert torch.equal(out_s.view(torch.uint8), exp_s.view(torch.uint8))
        exp_p = torch.empty_like(out_p)
        exp_p[rows] = w.probs.to(DEV).reshape(-1)
        assert torch.equal(out_p.view(torch.int32), exp_p.view(torch.int32))
    # what a consumer sees: dequantized permuted rows are the source rows
    rows = rm_ref[w.topk_idx.numpy().astype(np.int64), np.arange(T)[:, None]].ravel()
    sample = np.random.default_rng(1).choice(T * k, min(T * k, 512), replace=False)
    tok = np.repeat(np.arange(T), k)[np.argsort(rows)][sample]
    got = dequant(out.cpu()[sample], out_s.cpu()[sample], block, H)
    assert torch.equal(got, dequant(q[tok], sc[tok], block, H))


@pytest.mark.parametrize("T,H,E,k,elem,block,srb", [
    (37, 201, 9, 3, 1, 67, None),     # odd-length FP8 rows: byte units
    (37, 200, 9, 3, 1, 64, None),     # FP8 rows of 200 bytes: 4-byte units
    (64, 130, 16, 2, 1, 13, "e8m0"),  # 10 one-byte scales per row: byte side rows
    (50, 24, 6, 6, 4, 8, None),       # fp32 rows, 4-byte units
    (33, 72, 40, 5, 2, 24, None),     # bf16 rows with scales
    (9, 65536, 8, 8, 1, 128, None),   # long FP8 rows: two slices per token
    (40, 256, 80, 64, 1, 128, "none"),  # no scales, k = 64
])
def test_permute_scaled_edges(m, T, H, E, k, elem, block, srb):
    say(f"permute scaled edge T={T} H={H} E={E} k={k} elem={elem} block={block} scales={srb}")
    w = workloads.random_routed(T, H, E, k, seed=H + k, with_dy=False)
    if elem == 1:
        q, sc = fp8_case(w.x, block, torch.float8_e8m0fnu if srb == "e8m0" else torch.float32)
    elif elem == 4:
        q = w.x.float()
        sc = torch.rand(T, (H + block - 1) // block)
    else:
        q = w.x
        sc = torch.rand(T, (H + block - 1) // block)
    if srb == "none":
        sc = None
    rm_ref, _ = oracle.row_id_map(w.topk_idx.numpy(), E)
    out = sentinel_like((T * k, H), q.dtype)
    out_s = None if sc is None else sentinel_like((T * k, sc.shape[1]), sc.dtype)
    o, os_, _ = m.moe_permute_scaled(q.to(DEV), w.topk_idx.to(DEV),
                                     torch.from_numpy(rm_ref).to(DEV),
                                     None if sc is None else sc.to(DEV), out=out,
                                     out_scale=out_s)
    ref, ref_s, _ = oracle.permute_scaled(byte_view(q), None if sc is None else byte_view(sc),
                                          None, w.topk_idx.numpy(), rm_ref)
    np.testing.assert_array_equal(byte_view(o), ref)
    if sc is not None:
        np.testing.assert_array_equal(byte_view(os_), ref_s)


@pytest.mark.parametrize("num_out_frac", [None, 0.8])
def test_mask_permute_scaled(m, num_out_frac):
    say(f"mask permute fp8 dropping={num_out_frac}")
    g = torch.Generator().manual_seed(12)
    T, H, E = 500, 1024, 24
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    q, sc = fp8_case(x, 128, torch.float32)
    mask = torch.rand(T, E, generator=g) < 0.25
    probs = torch.rand(T, E, generator=g) * mask
    probs[::7] = 0.0                   # padded slots: zero data rows, scales still move
    R = int(mask.sum())
    num_out = -1 if num_out_frac is None else int(R * num_out_frac)
    n_rows = R + 2 if num_out < 0 else num_out
    ref_map, _ = oracle.mask_row_id_map(mask.numpy().astype(np.uint8), num_out)
    rm = torch.from_numpy(ref_map).to(DEV)
    out = sentinel_like((n_rows, H), q.dtype)
    out_s = sentinel_like((n_rows, sc.shape[1]), sc.dtype)
    o, os_, op = m.moe_permute_mask_scaled(q.to(DEV), rm, n_rows, sc.to(DEV), probs.to(DEV),
                                           out=out, out_scale=out_s)
    ref, ref_s, ref_p = oracle.mask_permute_scaled(
        byte_view(q), byte_view(sc), probs.numpy(), ref_map, n_rows,
        out=np.full((n_rows, H), SENT, np.uint8),
        out_scale=np.full((n_rows, sc.shape[1] * 4), SENT, np.uint8))
    np.testing.assert_array_equal(byte_view(o), ref)
    np.testing.assert_array_equal(byte_view(os_), ref_s)
    kept = int(ref_map[:, 2 * E].sum())
    np.testing.assert_array_equal(op.cpu().numpy()[:kept].view(np.uint32),
                                  ref_p[:kept].view(np.uint32))


def test_permute_scaled_rejects_bad_args(m):
    say("permute scaled argument checks")
    w = workloads.ROUTED["tiny"]()
    rm, _ = m.moe_make_row_id_map(w.topk_idx.to(DEV), w.num_experts)
    q, sc = fp8_case(w.x, 32, torch.float32)
    with pytest.raises(m.MoeError):      # scale rows without an output for them
        m._binding._check(m._binding._lib.moe_permute_scaled(
            q.to(DEV).data_ptr(), 1, sc.to(DEV).data_ptr(), 8, None, w.topk_idx.to(DEV).data_ptr(),
            rm.data_ptr(), w.T, w.H, w.k, w.num_experts, w.T * w.k,
            torch.empty(w.T * w.k, w.H, dtype=torch.uint8, device=DEV).data_ptr(), None, None,
            None, None), "moe_permute_scaled")
    with pytest.raises(m.MoeError):      # 8-byte elements
        m._binding._check(m._binding._lib.moe_permute_scaled(
            q.to(DEV).data_ptr(), 8, None, 0, None, w.topk_idx.to(DEV).data_ptr(), rm.data_ptr(),
            w.T, w.H, w.k, w.num_experts, w.T * w.k,
            torch.empty(w.T * w.k, w.H, dtype=torch.uint8, device=DEV).data_ptr(), None, None,
            None, None), "moe_permute_scaled")
