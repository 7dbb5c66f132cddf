"""Benchmark of the MoE permute / unpermute hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole routed path over one batch of synthetic
input already resident in HBM:
  routed workloads (finegrain, skewed, tiny):
      row map -> permute (+probs) -> weighted unpermute
      -> unpermute backward (act grad + prob grads) -> permute backward
  chunk workloads (chunks8k, chunks32k):
      sort-and-pad (+probs) -> unpad-and-restore (+probs)
The default workload is the fine-grained MoE layer (T=4096, H=2048, E=64,
k=6).  Every call goes straight through the C ABI (ctypes, precomputed
device pointers) on torch's current stream.

Printed: one JSON line with the throughput in algorithmic GB/s (bytes the
method must move, divided by the measured step time); the per-op times from
a breakdown pass with HIP events around every op (before the timed region)
and from a cold pass (the Infinity Cache flushed by a 512 MiB read before
each op); the rate of the step replayed from a captured hipGraph; the
roofline of the dominant kernel (its events inside the timed region, its
HBM bytes from stored rocprofv3 counters while the kernel sources match);
and the CPU oracle's rate on a bounded sample as a reported baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
METRIC = "permute+unpermute roundtrip GB/s & % of HBM peak (µs/call) per T,H,E,k"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="finegrain",
                    choices=["tiny", "finegrain", "skewed", "chunks8k", "chunks32k"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample (0 disables it)")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="skip timing the step replayed from a captured hipGraph")
    ap.add_argument("--no-cold", dest="cold", action="store_false",
                    help="skip the cold-cache per-op pass (keeps a kernel trace to the "
                         "warm calls)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="after timing, run a plain device copy of MIB MiB three times "
                         "(a known-size reference for hardware byte counters)")
    return ap.parse_args()


# --------------------------------------------------------------- bytes ----

def routed_bytes(T, H, E, k):
    """Algorithmic bytes per op of a routed step (bf16 rows, fp32 probs,
    int32 indices; each (t, j) lookup reads topk_idx and row_id_map)."""
    row = 2 * H
    look = 8 * T * k
    return {
        "row_map": 4 * T * k + 4 * E * T + 4 * (E + 1),
        "permute": T * row + T * k * row + look + 4 * T * k + 4 * T * k,
        "unpermute": T * k * row + T * row + look + 4 * T * k,
        "unpermute_bwd": T * row + 2 * T * k * row + look + 4 * T * k + 4 * T * k,
        "permute_bwd": T * k * row + T * row + look + 4 * T * k + 4 * T * k,
    }


def mask_bytes(T, H, E, k):
    """Algorithmic bytes of the mask-map ops on a routing with k experts per
    token (bool mask; each slot reads two map entries and its [T, E] prob)."""
    row = 2 * H
    look = 8 * T * k + 4 * T
    return {
        "mask_row_map": T * E + 4 * T * (2 * k + 1) + 4 * (E + 1),
        "mask_permute": T * row + T * k * row + look + 4 * T * k + 4 * T * k,
        "mask_unpermute": T * k * row + T * row + look + 4 * T * k,
        "mask_unpermute_bwd": T * row + 2 * T * k * row + look + 4 * T * k + 4 * T * E,
    }


def chunk_bytes(N, H, cap, eb=2):
    row = eb * H
    return {
        "sort_chunks_and_pad": N * row + cap * row + 4 * N + 4 * cap + 4 * cap + 4 * cap,
        "unpad_and_restore": N * row + N * row + 4 * cap + 4 * N + 4 * N,
    }


# Kernels each op launches (the op's events bracket all of them).
OP_KERNELS = {
    "row_map": ["rowmap_count_kernel", "rowmap_write_kernel"],
    "permute": ["permute_kernel"],
    "unpermute": ["combine_kernel"],
    "unpermute_bwd": ["combine_bwd_kernel"],
    "permute_bwd": ["combine_kernel"],
    "sort_chunks_and_pad": ["chunk_map_kernel", "pad_copy_kernel"],
    "unpad_and_restore": ["restore_copy_kernel"],
}
# The library's launch rules that change which kernels an op runs: padded
# buffers up to FUSED_PAD_MAX_BYTES are written by one launch that also
# builds the map; a row map of at most ROWMAP_SINGLE_MAX_ENTRIES (token,
# slot) entries and ROWMAP_SINGLE_MAX_EXPERTS experts (16-byte aligned
# indices, as here) is one launch; past ROWMAP_FUSED_MAX_BLOCKS blocks of
# 256 tokens a column scan runs between its two kernels.
FUSED_PAD_MAX_BYTES = 128 << 20
ROWMAP_SINGLE_MAX_ENTRIES = 4096
ROWMAP_SINGLE_MAX_EXPERTS = 512
ROWMAP_FUSED_MAX_BLOCKS = 64


def op_kernels(op, cfg):
    """Kernels that op launches for the workload configuration cfg."""
    if op == "sort_chunks_and_pad" and cfg.get("out_cap", 0) * cfg.get("H", 0) * 2 <= \
            FUSED_PAD_MAX_BYTES:
        return ["pad_fused_kernel"]
    if op == "row_map":
        T, k, E = cfg.get("T", 0), cfg.get("k", 0), cfg.get("E", 0)
        if T * k <= ROWMAP_SINGLE_MAX_ENTRIES and E <= ROWMAP_SINGLE_MAX_EXPERTS:
            return ["rowmap_single_kernel"]
        if (T + 255) // 256 > ROWMAP_FUSED_MAX_BLOCKS:
            return ["rowmap_count_kernel", "rowmap_colscan_kernel", "rowmap_write_kernel"]
    return OP_KERNELS[op]


def kernel_source_hash() -> str:
    """sha256 over the HIP sources, to tell whether stored counters still apply."""
    import hashlib
    d = os.path.join(ROOT, "unpermute_moe_make_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def pmc_traffic(workload: str, op: str):
    """HBM bytes per launch of the op's kernels from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary (profiles/pmc_traffic.json), scaled by the
    copy-kernel calibration factors; None when the kernels changed since."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_sha256") != kernel_source_hash():
        return None
    e = d.get("workloads", {}).get(workload, {}).get(op)
    if e is None:
        return None
    return round(e["fetch_kib"] * 1024 * d["fetch_factor"] +
                 e["write_kib"] * 1024 * d["write_factor"])


# --------------------------------------------------------------- setup ----

# hipEventDisableSystemFence: recording such an event takes no system-scope
# fence, i.e. no L2 write-back and invalidate at every marker.  The events
# here only time work (their results are read after a device synchronize), and
# without the flag every marker flushes the caches: on the 4096-token step the
# markers around one op per step cost 6.7 us per step, and an op's event time
# exceeded its kernel time by 1.6 us.
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000

# Steps captured in one hipGraph for the graph-replay timing.
GRAPH_STEPS = 10


class HipEvents:
    """Raw HIP events recorded through ctypes: far less host overhead per
    record than torch.cuda.Event, so timing every op does not starve the GPU."""

    def __init__(self, flags: int = HIP_EVENT_DISABLE_SYSTEM_FENCE):
        import torch  # noqa: F401  (the HIP runtime is already loaded by torch)
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.flags = flags
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                     ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        if self.hip.hipEventCreateWithFlags(ctypes.byref(ev), self.flags) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return ev

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_us(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value * 1e3


class Step:
    """A list of (name, fn, args) calls straight into the C ABI; the stream
    argument (always last) is supplied at run time."""

    def __init__(self):
        self.ops = []
        self.keep = []
        self.extra = []   # (name, bytes, fn, args) timed outside the step

    def add(self, name, fn, *args):
        self.ops.append((name, fn, args))

    def run(self, events=None, stream=None, hev=None):
        import torch
        s = ctypes.c_void_p(stream if stream is not None
                            else torch.cuda.current_stream().cuda_stream)
        for name, fn, args in self.ops:
            if events is not None:
                hev.record(events[name][0], s)
            st = fn(*args, s)
            if events is not None:
                hev.record(events[name][1], s)
            if st != 0:
                raise RuntimeError(f"{name}: status {st}")


def build_routed(m, w):
    import torch
    import workloads
    dev = "cuda:0"
    T, H, E, k = w.T, w.H, w.num_experts, w.k
    lib = m._binding._lib
    x, idx, probs, dy = (w.x.to(dev), w.topk_idx.to(dev), w.probs.to(dev), w.dy.to(dev))
    rm = torch.empty((E, T), dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    ws_n = m.moe_make_row_id_map_workspace_bytes(T, k, E)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    P = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    pp = torch.empty(T * k, dtype=torch.float32, device=dev)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    dP = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    dprob = torch.empty((T, k), dtype=torch.float32, device=dev)
    d_pp = workloads.random_rows(1, T * k, seed=7, device=dev).float().reshape(-1)
    dx = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    dprob2 = torch.empty((T, k), dtype=torch.float32, device=dev)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    step = Step()
    step.keep = [x, idx, probs, dy, rm, off, ws, P, pp, y, dP, dprob, d_pp, dx, dprob2]
    n = T * k
    step.add("row_map", lib.moe_make_row_id_map, p(idx), T, k, E, p(rm), p(off), None, p(ws),
             ws_n,)
    step.add("permute", lib.moe_permute, p(x), p(probs), p(idx), p(rm), T, H, k, E, n, p(P),
             p(pp), None,)
    step.add("unpermute", lib.moe_unpermute, p(P), p(probs), p(idx), p(rm), T, H, k, E, n, p(y),
             None,)
    step.add("unpermute_bwd", lib.moe_unpermute_bwd, p(dy), p(P), p(probs), p(idx), p(rm), T, H,
             k, E, n, p(dP), p(dprob), None,)
    step.add("permute_bwd", lib.moe_permute_bwd, p(dP), p(d_pp), p(idx), p(rm), T, H, k, E, n,
             p(dx), p(dprob2), None,)
    # The library's further operations (EP combine, router, mask-map form, FP8
    # rows), timed on their own after the step.
    y_ep = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    logits = w.logits.to(dev).contiguous()
    r_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    r_probs = torch.empty((T, k), dtype=torch.float32, device=dev)
    d_logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    step.keep += [y_ep, logits, r_idx, r_probs, d_logits]
    ub = routed_bytes(T, H, E, k)["unpermute"]
    eb = logits.element_size()
    step.extra = [
        ("unpermute_ep8_bf16partials", ub, lib.moe_unpermute_ep,
         (p(P), p(probs), p(idx), p(rm), T, H, k, E, n, 8, 1, p(y_ep), None)),
        ("unpermute_ep8_bf16partials_fp64", ub, lib.moe_unpermute_ep,
         (p(P), p(probs), p(idx), p(rm), T, H, k, E, n, 8, 3, p(y_ep), None)),
        # router: logits in, k indices + k weights out; bwd: 3 k-vectors in, [T, E] out
        ("topk_softmax", T * E * eb + T * k * 8, lib.moe_topk_softmax,
         (p(logits), eb, T, E, k, p(r_idx), p(r_probs), 4)),
        ("topk_softmax_bwd", T * k * 12 + T * E * 4, lib.moe_topk_softmax_bwd,
         (p(dprob), p(probs), 4, p(idx), T, E, k, p(d_logits), 4, None)),
    ]
    # TransformerEngine mask-map form on the same routing.
    mask = torch.zeros((T, E), dtype=torch.bool, device=dev)
    mask.scatter_(1, idx.long(), True)
    probs_te = torch.zeros((T, E), dtype=torch.float32, device=dev)
    probs_te.scatter_(1, idx.long(), probs)
    mmap = torch.empty((T, 2 * E + 1), dtype=torch.int32, device=dev)
    moff = torch.empty(E + 1, dtype=torch.int32, device=dev)
    mws_n = m.moe_make_mask_row_id_map_workspace_bytes(T, E)
    mws = torch.empty(mws_n, dtype=torch.uint8, device=dev)
    m.moe_make_mask_row_id_map(mask, row_id_map=mmap, expert_offsets=moff, workspace=mws)
    mP = torch.empty((n, H), dtype=torch.bfloat16, device=dev)
    mpp = torch.empty(n, dtype=torch.float32, device=dev)
    my = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    mdP = torch.empty((n, H), dtype=torch.bfloat16, device=dev)
    mdp = torch.empty((T, E), dtype=torch.float32, device=dev)
    step.keep += [mask, probs_te, mmap, moff, mws, mP, mpp, my, mdP, mdp]
    # Quantized rows: FP8 (E4M3FN) tokens with fp32 scales per 128 elements.
    q8, sc8 = workloads.quantize_fp8_rows(w.x, 128)
    q8, sc8 = q8.to(dev), sc8.to(dev)
    S = sc8.shape[1]
    qP = torch.empty((n, H), dtype=q8.dtype, device=dev)
    qS = torch.empty((n, S), dtype=torch.float32, device=dev)
    step.keep += [q8, sc8, qP, qS]
    fp8_bytes = T * H + n * H + 4 * S * (T + n) + 8 * n + 4 * n + 4 * n
    mb = mask_bytes(T, H, E, k)
    step.extra += [
        ("permute_fp8_scaled", fp8_bytes, lib.moe_permute_scaled,
         (p(q8), 1, p(sc8), 4 * S, p(probs), p(idx), p(rm), T, H, k, E, n, p(qP), p(qS), p(pp),
          None)),
    ]
    step.extra += [
        ("mask_row_map", mb["mask_row_map"], lib.moe_make_mask_row_id_map,
         (p(mask), 1, T, E, -1, p(mmap), p(moff), p(mws), mws_n)),
        ("mask_permute", mb["mask_permute"], lib.moe_permute_mask,
         (p(x), p(probs_te), p(mmap), T, H, E, n, p(mP), p(mpp), None)),
        ("mask_unpermute", mb["mask_unpermute"], lib.moe_unpermute_mask,
         (p(mP), p(probs_te), None, p(mmap), T, H, E, n, p(my), None, None)),
        ("mask_unpermute_bwd", mb["mask_unpermute_bwd"], lib.moe_unpermute_mask_bwd,
         (p(dy), p(mP), p(probs_te), p(mmap), T, H, E, n, p(mdP), p(mdp), None)),
    ]
    return step, routed_bytes(T, H, E, k)


def build_chunks(m, cw):
    import torch
    dev = "cuda:0"
    lib = m._binding._lib
    x, probs = cw.x.to(dev), cw.probs.to(dev)
    sizes, order = cw.split_sizes.to(dev), cw.sorted_idx.to(dev)
    G = cw.C // cw.chunks_per_group
    out = torch.empty((cw.out_cap, cw.H), dtype=x.dtype, device=dev)
    out_p = torch.empty(cw.out_cap, dtype=torch.float32, device=dev)
    rm = torch.empty(cw.out_cap, dtype=torch.int32, device=dev)
    off = torch.empty(G + 1, dtype=torch.int32, device=dev)
    back = torch.empty_like(x)
    back_p = torch.empty_like(probs)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    step = Step()
    step.keep = [x, probs, sizes, order, out, out_p, rm, off, back, back_p]
    eb = x.element_size()
    step.add("sort_chunks_and_pad", lib.moe_sort_chunks_and_pad, p(x), p(probs), eb, 4,
             cw.N_cap, cw.H, p(sizes), p(order), cw.C, cw.chunks_per_group, cw.align, cw.out_cap,
             p(out), p(out_p), p(rm), p(off), None,)
    step.add("unpad_and_restore", lib.moe_unpad_and_restore_chunks, p(out), p(out_p), eb, 4,
             p(rm), p(sizes), cw.C, cw.out_cap, cw.H, cw.N_cap, p(back), p(back_p), None,)
    return step, chunk_bytes(int(cw.split_sizes.sum()), cw.H, cw.out_cap, eb)


# --------------------------------------------------------- CPU baseline ----

def op_stats(times, nbytes):
    """Mean, median, p10 / p90 of sorted event times (µs) and the rate at the
    median."""
    n = len(times)
    mean = sum(times) / n
    med = times[n // 2]
    return {"us_mean": round(mean, 2), "us_median": round(med, 2),
            "us_p10": round(times[n // 10], 2), "us_p90": round(times[(9 * n) // 10], 2),
            "bytes": nbytes, "GBps": round(nbytes / (med * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100 * nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)}


def cpu_baseline(name, w, target_s, step_bytes):
    """The oracle, untuned and single-threaded, on a bounded sample of the
    same workload: whole steps on a prefix of the tokens, repeated until
    about target_s seconds of CPU work."""
    import numpy as np
    import oracle
    import workloads
    if name.startswith("chunks"):
        xb = workloads.bf16_bits(w.x)
        p = w.probs.numpy()
        s = w.split_sizes.numpy()
        q = w.sorted_idx.numpy()

        def one():
            out, op, rm, _ = oracle.sort_chunks_and_pad(xb, p, s, q, w.chunks_per_group,
                                                        w.align, w.out_cap)
            oracle.unpad_and_restore_chunks(out, op, rm, s, w.N_cap)
        frac = 1.0
        sample = f"whole {name} roundtrip"
    else:
        T = w.T
        Ts = min(T, max(64, int(T * 0.25)))          # a token prefix
        idx = w.topk_idx.numpy()[:Ts]
        pr = w.probs.numpy()[:Ts]
        xb = workloads.bf16_bits(w.x[:Ts])
        dyb = workloads.bf16_bits(w.dy[:Ts])
        d_pp = np.linspace(-1, 1, Ts * w.k, dtype=np.float32)

        def one():
            rm, _ = oracle.row_id_map(idx, w.num_experts)
            P, _ = oracle.permute(xb, pr, idx, rm)
            oracle.unpermute(P, pr, idx, rm)
            dP, _ = oracle.unpermute_bwd(dyb, P, pr, idx, rm)
            oracle.permute_bwd(dP, d_pp, idx, rm)
        frac = Ts / T
        sample = f"whole steps on the first {Ts} of {T} tokens"
    one()                                           # warm-up
    reps, t0 = 0, time.perf_counter()
    while True:
        one()
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    per_step = el / reps
    gbs = step_bytes * frac / per_step / 1e9
    result = {"value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
              "sample": f"{sample}, {reps} repetitions, {el:.1f} s, single thread",
              "seconds_per_full_step": round(per_step / frac, 4)}
    return result


# ----------------------------------------------------------------- main ----

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested); this path is "
              "built and measured per GPU and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    import torch
    import unpermute_moe_make_amd as m
    import workloads

    torch.cuda.init()
    name = args.workload
    if name in workloads.ROUTED:
        w = workloads.ROUTED[name]()
        step, op_bytes = build_routed(m, w)
        cfg = {"workload": name, "T": w.T, "H": w.H, "E": w.num_experts, "k": w.k,
               "step": "row_map+permute+unpermute+unpermute_bwd+permute_bwd",
               "probs": "fp32", "launch": "eager, C ABI via ctypes"}
    else:
        w = workloads.CHUNKED[name]()
        step, op_bytes = build_chunks(m, w)
        cfg = {"workload": name, "N": w.N_cap, "H": w.H, "chunks": w.C,
               "chunks_per_group": w.chunks_per_group, "align": w.align, "out_cap": w.out_cap,
               "step": "sort_chunks_and_pad+unpad_and_restore", "probs": "fp32",
               "launch": "eager, C ABI via ctypes"}
    step_bytes = sum(op_bytes.values())

    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    names = [n for n, _, _ in step.ops]
    hev = HipEvents()
    sv = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    # Breakdown pass: HIP events around every op (one marker pair per call).
    K2 = max(10, args.steps // 2)
    evs = [{n: (hev.create(), hev.create()) for n in names} for _ in range(K2)]
    for i in range(K2):
        step.run(evs[i], hev=hev)
    torch.cuda.synchronize()
    per_op = {}
    for n in names:
        times = sorted(hev.elapsed_us(evs[i][n][0], evs[i][n][1]) for i in range(K2))
        per_op[n] = op_stats(times, op_bytes[n])
    dom = max(names, key=lambda n: per_op[n]["us_mean"])

    # Cold pass: a 512 MiB read of an unrelated buffer before every op
    # (outside its events) evicts the op's inputs from the Infinity Cache and
    # writes back whatever was dirty, so the op starts from clean, unrelated
    # cache contents.  (A write pass would leave 256 MB of dirty lines whose
    # write-back the op would then pay.)
    K3 = K2 if args.cold else 0
    flush = torch.ones(512 << 18 if K3 else 1, dtype=torch.float32, device="cuda:0")
    evc = [{n: (hev.create(), hev.create()) for n in names} for _ in range(K3)]
    for i in range(K3):
        for n, fn, a in step.ops:
            flush.sum()
            hev.record(evc[i][n][0], sv)
            st = fn(*a, sv)
            hev.record(evc[i][n][1], sv)
            if st != 0:
                raise RuntimeError(f"{n}: status {st}")
    torch.cuda.synchronize()
    del flush
    per_op_cold = {n: op_stats(sorted(hev.elapsed_us(evc[i][n][0], evc[i][n][1])
                                      for i in range(K3)), op_bytes[n]) for n in names} \
        if K3 else None

    # Timed region: exactly K steps; events only around the dominant op.
    K = args.steps
    dev_ev = [(hev.create(), hev.create()) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        for n, fn, a in step.ops:
            if n == dom:
                hev.record(dev_ev[i][0], sv)
            st = fn(*a, sv)
            if n == dom:
                hev.record(dev_ev[i][1], sv)
            if st != 0:
                raise RuntimeError(f"{n}: status {st}")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / K * 1e3
    dom_us = sum(hev.elapsed_us(a, b) for a, b in dev_ev) / K

    achieved = op_bytes[dom] / (dom_us * 1e-6) / 1e9
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": cfg,
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
        "step_bytes": step_bytes,
        "per_op": per_op,
        "per_op_cold": per_op_cold,
        "roofline": {"bound": "hbm", "kernel": dom, "kernels": op_kernels(dom, cfg),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "us_per_launch": round(dom_us, 2),
                     "bytes_per_launch": op_bytes[dom],
                     "traffic": pmc_traffic(name, dom)},
    }
    if args.graph:
        # The same step (same buffers) captured GRAPH_STEPS times in one
        # hipGraph, so one host launch covers several steps, and replayed
        # until K steps have run.
        R = max(1, min(GRAPH_STEPS, K))
        reps = max(1, K // R)
        g = torch.cuda.CUDAGraph()
        s2 = torch.cuda.Stream()
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s2):
            step.run(stream=s2.cuda_stream)
        torch.cuda.current_stream().wait_stream(s2)
        with torch.cuda.graph(g, stream=s2):
            for _ in range(R):
                step.run(stream=s2.cuda_stream)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        gms = (time.perf_counter() - t0) / (reps * R) * 1e3
        result["graph_replay"] = {"steps_per_graph": R, "ms_per_step": round(gms, 4),
                                  "GBps": round(step_bytes / (gms * 1e-3) / 1e9, 1)}
    if step.extra:
        extra = {}
        for n, nbytes, fn, a in step.extra:
            for _ in range(3):
                fn(*a, sv)
            evx = [(hev.create(), hev.create()) for _ in range(K2)]
            for e0, e1 in evx:
                hev.record(e0, sv)
                st = fn(*a, sv)
                hev.record(e1, sv)
                if st != 0:
                    raise RuntimeError(f"{n}: status {st}")
            torch.cuda.synchronize()
            us = sum(hev.elapsed_us(e0, e1) for e0, e1 in evx) / K2
            extra[n] = {"us_mean": round(us, 2), "bytes": nbytes,
                        "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                        "pct_hbm_peak": round(100 * nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)}
        result["extra_ops"] = extra
    if args.copy_probe > 0:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = {"read": 4 * n, "write": 4 * n}
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(name, w, args.cpu_seconds, step_bytes)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
