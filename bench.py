"""Benchmark of the MoE permute / unpermute hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

The metric is the permute + unpermute roundtrip (GB/s of algorithmic bytes,
% of the 8 TB/s HBM peak, us per call).  For a routed workload (default: the
skewed MoE layer, T=16384, H=7168, E=256, k=8) a timed step is one roundtrip
over one batch of synthetic input already resident in HBM:

    permute (+probs) -> fixed slot-order weighted unpermute

and `value` is the roundtrip's bytes divided by the wall time per roundtrip
over exactly K steps.  For a chunk workload (chunks8k, chunks32k) the step is
sort-and-pad (+probs) -> unpad-and-restore (+probs).  Every call goes
straight through the C ABI (ctypes, precomputed device pointers) on torch's
current stream.

Also printed in the same JSON line, all timed with HIP events on that stream:
  per_op          every op of the whole routed path (row map, permute,
                  unpermute, unpermute backward, permute backward), warm:
                  each op called back to back, so its inputs are as its
                  own previous call left them;
  per_op_cold     the same ops, each after a 512 MiB read of an unrelated
                  buffer (nothing of the op's inputs left in the Infinity
                  Cache);
  roundtrip_cold  the roundtrip after such a read, timed as one unit;
  full_step       the whole routed path (all five ops) timed like the step;
  graph_replay    the roundtrip captured in a hipGraph and replayed;
  chunks32k       the 32768-token chunk sort-and-pad / restore roundtrip,
                  warm and cold (with a routed workload);
  extra_ops       the library's further operations (EP combine, router,
                  mask-map form, FP8 rows) on the same input, warm and cold;
  roofline        the dominant kernel of the step: its algorithmic bytes per
                  launch over its event time in the timed region (warm) and
                  in the cold pass, and its HBM bytes from stored rocprofv3
                  counters while the kernel sources are unchanged;
  cpu_baseline    the CPU oracle on the same roundtrip on the host's cores,
                  one thread and all threads (a reported baseline only).
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
    ap.add_argument("--workload", default="skewed",
                    choices=["tiny", "finegrain", "skewed", "chunks8k", "chunks32k"])
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="CPU time per row of the oracle baseline (0 disables it)")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="skip timing the step replayed from a captured hipGraph")
    ap.add_argument("--no-cold", dest="cold", action="store_false",
                    help="skip the cold-cache passes (keeps a kernel trace to the warm calls)")
    ap.add_argument("--cold-only", action="store_true",
                    help="run only the cold-cache passes after the warm-up (so a kernel trace "
                         "holds the cold launches alone)")
    ap.add_argument("--no-chunks", dest="chunks", action="store_false",
                    help="with a routed workload, skip the 32768-token chunk roundtrip block")
    ap.add_argument("--no-extra", dest="extra", action="store_false",
                    help="skip the library's further operations")
    ap.add_argument("--no-full-step", dest="full_step", action="store_false",
                    help="skip timing the whole routed path (so a kernel trace of the warm "
                         "calls holds the roundtrip's calls and the per-op calls only)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="after timing, run a plain device copy of MIB MiB three times "
                         "(a known-size reference for hardware byte counters)")
    return ap.parse_args()


# --------------------------------------------------------------- bytes ----

def routed_bytes(T, H, E, k):
    """Algorithmic bytes per op of the routed path (bf16 rows, fp32 probs,
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


ROUNDTRIP_OPS = {"routed": ("permute", "unpermute"),
                 "chunks": ("sort_chunks_and_pad", "unpad_and_restore")}

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
# An unpermute backward with prob gradients that moves more than
# STREAM_BYTES, on rows of whole 16-byte units that fit one workgroup pass
# (at most BWD_SPLIT_MAX_UNITS units), runs as a scaled scatter and then a
# dot-product gather.
STREAM_BYTES = 256 << 20
BWD_SPLIT_MAX_UNITS = 2048


def op_kernels(op, cfg):
    """Kernels that op launches for the workload configuration cfg."""
    if op == "sort_chunks_and_pad" and cfg.get("out_cap", 0) * cfg.get("H", 0) * 2 <= \
            FUSED_PAD_MAX_BYTES:
        return ["pad_fused_kernel"]
    if op == "unpermute_bwd":
        T, H, k = cfg.get("T", 0), cfg.get("H", 0), cfg.get("k", 0)
        if H % 8 == 0 and H // 8 <= BWD_SPLIT_MAX_UNITS and \
                2 * H * (2 * T * k + T) > STREAM_BYTES:
            return ["scale_scatter_kernel", "dot_gather_kernel"]
    if op == "row_map":
        T, k, E = cfg.get("T", 0), cfg.get("k", 0), cfg.get("E", 0)
        if T * k <= ROWMAP_SINGLE_MAX_ENTRIES and E <= ROWMAP_SINGLE_MAX_EXPERTS:
            return ["rowmap_single_kernel"]
        if (T + 255) // 256 > ROWMAP_FUSED_MAX_BLOCKS:
            return ["rowmap_count_kernel", "rowmap_colscan_kernel", "rowmap_write_kernel"]
    return OP_KERNELS[op]


def _code_only(text: str) -> str:
    """C/C++ source without its comments and with whitespace runs folded, so
    that a comment edit does not count as a kernel change.  String and
    character literals are kept as they are."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """sha256 over the HIP sources' code (comments and layout left out), to
    tell whether stored counters still apply."""
    import hashlib
    d = os.path.join(ROOT, "unpermute_moe_make_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), encoding="utf-8") as fh:
            h.update(f.encode() + b"\0" + _code_only(fh.read()).encode())
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
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                     ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]

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


class Ops:
    """Named calls straight into the C ABI; the stream argument (always last)
    is supplied at run time."""

    def __init__(self):
        self.calls = {}      # name -> (fn, args)
        self.keep = []

    def add(self, name, fn, *args):
        self.calls[name] = (fn, args)

    def run(self, names, stream, events=None, hev=None):
        for name in names:
            fn, args = self.calls[name]
            if events is not None:
                hev.record(events[name][0], stream)
            st = fn(*args, stream)
            if events is not None:
                hev.record(events[name][1], stream)
            if st != 0:
                raise RuntimeError(f"{name}: status {st}")


def build_routed(m, w, extra=True):
    """The whole routed path on workload w, plus (extra) the library's
    further operations on the same routing.  Returns (ops, bytes per op,
    extra op names)."""
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
    ops = Ops()
    ops.keep = [x, idx, probs, dy, rm, off, ws, P, pp, y, dP, dprob, d_pp, dx, dprob2]
    n = T * k
    ops.add("row_map", lib.moe_make_row_id_map, p(idx), T, k, E, p(rm), p(off), None, p(ws),
            ws_n)
    ops.add("permute", lib.moe_permute, p(x), p(probs), p(idx), p(rm), T, H, k, E, n, p(P),
            p(pp), None)
    ops.add("unpermute", lib.moe_unpermute, p(P), p(probs), p(idx), p(rm), T, H, k, E, n, p(y),
            None)
    ops.add("unpermute_bwd", lib.moe_unpermute_bwd, p(dy), p(P), p(probs), p(idx), p(rm), T, H,
            k, E, n, p(dP), p(dprob), None)
    ops.add("permute_bwd", lib.moe_permute_bwd, p(dP), p(d_pp), p(idx), p(rm), T, H, k, E, n,
            p(dx), p(dprob2), None)
    nbytes = routed_bytes(T, H, E, k)
    if not extra:
        return ops, nbytes, []
    # The library's further operations, timed on their own after the step.
    y_ep = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    logits = w.logits.to(dev).contiguous()
    r_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    r_probs = torch.empty((T, k), dtype=torch.float32, device=dev)
    d_logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    ops.keep += [y_ep, logits, r_idx, r_probs, d_logits]
    ub = nbytes["unpermute"]
    eb = logits.element_size()
    ops.add("unpermute_ep8_bf16partials", lib.moe_unpermute_ep, p(P), p(probs), p(idx), p(rm),
            T, H, k, E, n, 8, 1, p(y_ep), None)
    ops.add("unpermute_ep8_bf16partials_fp64", lib.moe_unpermute_ep, p(P), p(probs), p(idx),
            p(rm), T, H, k, E, n, 8, 3, p(y_ep), None)
    # router: logits in, k indices + k weights out; bwd: 3 k-vectors in, [T, E] out
    ops.add("topk_softmax", lib.moe_topk_softmax, p(logits), eb, T, E, k, p(r_idx), p(r_probs),
            4)
    ops.add("topk_softmax_bwd", lib.moe_topk_softmax_bwd, p(dprob), p(probs), 4, p(idx), T, E,
            k, p(d_logits), 4, None)
    nbytes.update({"unpermute_ep8_bf16partials": ub, "unpermute_ep8_bf16partials_fp64": ub,
                   "topk_softmax": T * E * eb + T * k * 8,
                   "topk_softmax_bwd": T * k * 12 + T * E * 4})
    # Quantized rows: FP8 (E4M3FN) tokens with fp32 scales per 128 elements.
    q8, sc8 = workloads.quantize_fp8_rows(w.x, 128)
    q8, sc8 = q8.to(dev), sc8.to(dev)
    S = sc8.shape[1]
    qP = torch.empty((n, H), dtype=q8.dtype, device=dev)
    qS = torch.empty((n, S), dtype=torch.float32, device=dev)
    ops.keep += [q8, sc8, qP, qS]
    ops.add("permute_fp8_scaled", lib.moe_permute_scaled, p(q8), 1, p(sc8), 4 * S, p(probs),
            p(idx), p(rm), T, H, k, E, n, p(qP), p(qS), p(pp), None)
    nbytes["permute_fp8_scaled"] = T * H + n * H + 4 * S * (T + n) + 8 * n + 4 * n + 4 * n
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
    ops.keep += [mask, probs_te, mmap, moff, mws, mP, mpp, my, mdP, mdp]
    ops.add("mask_row_map", lib.moe_make_mask_row_id_map, p(mask), 1, T, E, -1, p(mmap),
            p(moff), p(mws), mws_n)
    ops.add("mask_permute", lib.moe_permute_mask, p(x), p(probs_te), p(mmap), T, H, E, n, p(mP),
            p(mpp), None)
    ops.add("mask_unpermute", lib.moe_unpermute_mask, p(mP), p(probs_te), None, p(mmap), T, H,
            E, n, p(my), None, None)
    ops.add("mask_unpermute_bwd", lib.moe_unpermute_mask_bwd, p(dy), p(mP), p(probs_te),
            p(mmap), T, H, E, n, p(mdP), p(mdp), None)
    nbytes.update(mask_bytes(T, H, E, k))
    extra_names = ["unpermute_ep8_bf16partials", "unpermute_ep8_bf16partials_fp64",
                   "topk_softmax", "topk_softmax_bwd", "permute_fp8_scaled", "mask_row_map",
                   "mask_permute", "mask_unpermute", "mask_unpermute_bwd"]
    return ops, nbytes, extra_names


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
    ops = Ops()
    ops.keep = [x, probs, sizes, order, out, out_p, rm, off, back, back_p]
    eb = x.element_size()
    ops.add("sort_chunks_and_pad", lib.moe_sort_chunks_and_pad, p(x), p(probs), eb, 4,
            cw.N_cap, cw.H, p(sizes), p(order), cw.C, cw.chunks_per_group, cw.align, cw.out_cap,
            p(out), p(out_p), p(rm), p(off), None)
    ops.add("unpad_and_restore", lib.moe_unpad_and_restore_chunks, p(out), p(out_p), eb, 4,
            p(rm), p(sizes), cw.C, cw.out_cap, cw.H, cw.N_cap, p(back), p(back_p), None)
    return ops, chunk_bytes(int(cw.split_sizes.sum()), cw.H, cw.out_cap, eb)


# -------------------------------------------------------------- timing ----

def op_stats(times, nbytes):
    """Mean, median, p10 / p90 of event times (µs) and the rate at the median."""
    times = sorted(times)
    n = len(times)
    mean = sum(times) / n
    med = times[n // 2]
    return {"us_mean": round(mean, 2), "us_median": round(med, 2),
            "us_p10": round(times[n // 10], 2), "us_p90": round(times[(9 * n) // 10], 2),
            "bytes": nbytes, "GBps": round(nbytes / (med * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100 * nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)}


class Timer:
    """Event-timed passes over named ops on one stream."""

    def __init__(self, ops, nbytes, stream):
        import torch
        self.torch = torch
        self.ops, self.nbytes, self.s = ops, nbytes, stream
        self.hev = HipEvents()
        self._flush = None

    def flush(self):
        # A 512 MiB read of an unrelated buffer evicts the op's inputs from
        # the Infinity Cache and writes back whatever was dirty, so the op
        # starts from clean, unrelated cache contents.  (A write pass would
        # leave 256 MB of dirty lines whose write-back the op would pay.)
        if self._flush is None:
            self._flush = self.torch.ones(512 << 18, dtype=self.torch.float32, device="cuda:0")
        self._flush.sum()

    def per_op(self, names, reps, cold=False):
        """Each op of `names` reps times back to back, events around each
        call (cold: a flush before each call, outside its events)."""
        evs = [{n: (self.hev.create(), self.hev.create()) for n in names} for _ in range(reps)]
        for n in names:
            for i in range(reps):
                if cold:
                    self.flush()
                self.ops.run([n], self.s, evs[i], self.hev)
        self.torch.cuda.synchronize()
        return {n: op_stats([self.hev.elapsed_us(*evs[i][n]) for i in range(reps)],
                            self.nbytes[n]) for n in names}

    def unit(self, names, reps, cold=False):
        """The ops of `names` back to back, timed as one unit (cold: one
        flush before the unit)."""
        evs = [(self.hev.create(), self.hev.create()) for _ in range(reps)]
        for i in range(reps):
            if cold:
                self.flush()
            self.hev.record(evs[i][0], self.s)
            self.ops.run(names, self.s)
            self.hev.record(evs[i][1], self.s)
        self.torch.cuda.synchronize()
        return op_stats([self.hev.elapsed_us(a, b) for a, b in evs],
                        sum(self.nbytes[n] for n in names))

    def wall(self, names, steps, mark=None):
        """Exactly `steps` passes over `names` bracketed by device
        synchronizes; events around op `mark` only.  Returns (ms per pass,
        mean event µs of `mark`)."""
        evs = [(self.hev.create(), self.hev.create()) for _ in range(steps)]
        calls = [(n, *self.ops.calls[n]) for n in names]
        s = self.s
        self.torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            for n, fn, a in calls:
                if n == mark:
                    self.hev.record(evs[i][0], s)
                st = fn(*a, s)
                if n == mark:
                    self.hev.record(evs[i][1], s)
                if st != 0:
                    raise RuntimeError(f"{n}: status {st}")
        self.torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / steps * 1e3
        us = sum(self.hev.elapsed_us(a, b) for a, b in evs) / steps if mark else None
        return ms, us

    def graph(self, names, steps):
        """`names` captured GRAPH_STEPS times in one hipGraph, replayed until
        `steps` passes have run; ms per pass."""
        torch = self.torch
        R = max(1, min(GRAPH_STEPS, steps))
        reps = max(1, steps // R)
        g = torch.cuda.CUDAGraph()
        s2 = torch.cuda.Stream()
        s2.wait_stream(torch.cuda.current_stream())
        sv2 = ctypes.c_void_p(s2.cuda_stream)
        with torch.cuda.stream(s2):
            self.ops.run(names, sv2)
        torch.cuda.current_stream().wait_stream(s2)
        with torch.cuda.graph(g, stream=s2):
            for _ in range(R):
                self.ops.run(names, sv2)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / (reps * R) * 1e3, R


def rate(nbytes, us):
    gbs = nbytes / (us * 1e-6) / 1e9
    return round(gbs, 1), round(100 * gbs / HBM_PEAK_GBS, 1)


# --------------------------------------------------------- CPU baseline ----

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(name, w, target_s, rt_bytes):
    """The oracle, as it stands, on the same roundtrip: one thread (pinned to
    one core) and all the threads this process may use.  Each row repeats
    whole roundtrips until about target_s seconds have run (at least one)."""
    import numpy as np  # noqa: F401
    import oracle
    import workloads
    if name.startswith("chunks"):
        xb = workloads.bf16_bits(w.x)
        p, s, q = w.probs.numpy(), w.split_sizes.numpy(), w.sorted_idx.numpy()

        def one():
            out, op, rm, _ = oracle.sort_chunks_and_pad(xb, p, s, q, w.chunks_per_group,
                                                        w.align, w.out_cap)
            oracle.unpad_and_restore_chunks(out, op, rm, s, w.N_cap)
        what = f"whole {name} sort-and-pad + restore roundtrips"
    else:
        idx, pr = w.topk_idx.numpy(), w.probs.numpy()
        xb = workloads.bf16_bits(w.x)
        rm, _ = oracle.row_id_map(idx, w.num_experts)   # the map is not part of the roundtrip

        def one():
            P, _ = oracle.permute(xb, pr, idx, rm)
            oracle.unpermute(P, pr, idx, rm)
        what = f"whole {name} permute + unpermute roundtrips (T={w.T})"

    def timed(n_threads, pin):
        before_aff = os.sched_getaffinity(0)
        before_thr = oracle.threads()
        try:
            if pin is not None:
                os.sched_setaffinity(0, {pin})
            used = oracle.set_threads(n_threads)
            reps, t0 = 0, time.perf_counter()
            while True:
                one()
                reps += 1
                el = time.perf_counter() - t0
                if el >= target_s:
                    break
        finally:
            oracle.set_threads(before_thr)
            if pin is not None:
                os.sched_setaffinity(0, before_aff)
        per = el / reps
        gbs = rt_bytes / per / 1e9
        return {"value": round(gbs, 3), "unit": "GB/s", "cores": used,
                "seconds_per_roundtrip": round(per, 4), "repetitions": reps,
                "seconds": round(el, 1)}

    aff = sorted(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    n_all = min(len(aff), int(omp)) if omp.isdigit() and int(omp) > 0 else len(aff)
    oracle.set_threads(n_all)
    one()                                               # warm-up: first touch of the buffers
    one_thr = timed(1, aff[0])
    all_thr = timed(n_all, None)
    return {"value": all_thr["value"], "unit": "GB/s", "cores": all_thr["cores"],
            "kind": "oracle", "sample": what,
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(), "cpus_allowed": len(aff),
            "rows": [dict(one_thr, threads="1, pinned to one core"),
                     dict(all_thr, threads="all allowed (OpenMP over tokens)")]}


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
    K, W = args.steps, args.warmup
    K2 = max(10, K // 2)            # samples of the per-op and cold passes
    sv = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    routed = name in workloads.ROUTED
    if routed:
        w = workloads.ROUTED[name]()
        ops, nbytes, extra_names = build_routed(m, w, extra=args.extra and not args.cold_only)
        path_ops = ["row_map", "permute", "unpermute", "unpermute_bwd", "permute_bwd"]
        rt = list(ROUNDTRIP_OPS["routed"])
        cfg = {"workload": name, "T": w.T, "H": w.H, "E": w.num_experts, "k": w.k,
               "step": "permute+unpermute", "probs": "fp32", "launch": "eager, C ABI via ctypes"}
    else:
        w = workloads.CHUNKED[name]()
        ops, nbytes = build_chunks(m, w)
        extra_names = []
        path_ops = list(ROUNDTRIP_OPS["chunks"])
        rt = path_ops
        cfg = {"workload": name, "N": w.N_cap, "H": w.H, "chunks": w.C,
               "chunks_per_group": w.chunks_per_group, "align": w.align, "out_cap": w.out_cap,
               "step": "sort_chunks_and_pad+unpad_and_restore", "probs": "fp32",
               "launch": "eager, C ABI via ctypes"}
    rt_bytes = sum(nbytes[n] for n in rt)
    tm = Timer(ops, nbytes, sv)
    for _ in range(W):
        ops.run(path_ops, sv)
    torch.cuda.synchronize()

    if args.cold_only:
        # Only cold launches after the warm-up (for a kernel trace of them).
        cold = tm.per_op(path_ops, K2, cold=True)
        rtc = tm.unit(rt, K2, cold=True)
        print(json.dumps({"workload": name, "per_op_cold": cold, "roundtrip_cold": rtc}),
              flush=True)
        return

    # Breakdown pass: HIP events around every op of the path.
    per_op = tm.per_op(path_ops, K2)
    dom = max(rt, key=lambda n: per_op[n]["us_mean"])
    per_op_cold = tm.per_op(path_ops, K2, cold=True) if args.cold else None
    rt_cold = tm.unit(rt, K2, cold=True) if args.cold else None

    # Timed region: exactly K roundtrips; events only around the dominant op.
    ms, dom_us = tm.wall(rt, K, mark=dom)
    value = rt_bytes / (ms * 1e-3) / 1e9
    achieved = nbytes[dom] / (dom_us * 1e-6) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": cfg,
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
        "us_per_roundtrip": round(ms * 1e3, 1),
        "step_bytes": rt_bytes,
        "roundtrip_cold": rt_cold,
        "per_op": per_op,
        "per_op_cold": per_op_cold,
    }
    roof = {"bound": "hbm", "kernel": dom, "kernels": op_kernels(dom, cfg),
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "us_per_launch": round(dom_us, 2),
            "bytes_per_launch": nbytes[dom], "traffic": pmc_traffic(name, dom)}
    if per_op_cold is not None:
        cu = per_op_cold[dom]["us_median"]
        roof.update({"us_per_launch_cold": cu,
                     "achieved_cold": round(nbytes[dom] / (cu * 1e-6) / 1e9, 1),
                     "frac_cold": round(nbytes[dom] / (cu * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
    result["roofline"] = roof
    if routed and args.full_step:
        fms, _ = tm.wall(path_ops, K)
        fb = sum(nbytes[n] for n in path_ops)
        result["full_step"] = {"ops": "+".join(path_ops), "bytes": fb, "ms": round(fms, 4),
                               "GBps": rate(fb, fms * 1e3)[0],
                               "pct_hbm_peak": rate(fb, fms * 1e3)[1]}
    if args.graph:
        gms, R = tm.graph(rt, K)
        result["graph_replay"] = {"steps_per_graph": R, "ms_per_step": round(gms, 4),
                                  "GBps": rate(rt_bytes, gms * 1e3)[0]}
    if extra_names:
        extra = {}
        for n in extra_names:
            for _ in range(3):
                ops.run([n], sv)
            warm = tm.per_op([n], K2)[n]
            e = {"us_median": warm["us_median"], "bytes": nbytes[n], "GBps": warm["GBps"],
                 "pct_hbm_peak": warm["pct_hbm_peak"]}
            if args.cold:
                c = tm.per_op([n], K2, cold=True)[n]
                e.update({"us_median_cold": c["us_median"], "GBps_cold": c["GBps"],
                          "pct_hbm_peak_cold": c["pct_hbm_peak"]})
            extra[n] = e
        result["extra_ops"] = extra
    if routed and args.chunks:
        cw = workloads.chunks32k()
        cops, cbytes = build_chunks(m, cw)
        ct = Timer(cops, cbytes, sv)
        cn = list(ROUNDTRIP_OPS["chunks"])
        cb = sum(cbytes.values())
        for _ in range(W):
            cops.run(cn, sv)
        cms, _ = ct.wall(cn, K)
        cblk = {"N": cw.N_cap, "H": cw.H, "chunks": cw.C, "align": cw.align,
                "out_cap": cw.out_cap, "bytes": cb, "us_per_roundtrip": round(cms * 1e3, 1),
                "GBps": rate(cb, cms * 1e3)[0], "pct_hbm_peak": rate(cb, cms * 1e3)[1],
                "per_op": ct.per_op(cn, K2)}
        if args.cold:
            cblk["per_op_cold"] = ct.per_op(cn, K2, cold=True)
            cblk["roundtrip_cold"] = ct.unit(cn, K2, cold=True)
        result["chunks32k"] = cblk
        del cops, ct
    if args.copy_probe > 0:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = {"read": 4 * n, "write": 4 * n}
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(name, w, args.cpu_seconds, rt_bytes)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
