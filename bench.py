"""Throughput of the attention hot path on one MI355X.

One step = one pass of the whole hot path over resident synthetic inputs:
  * prefill: causal GQA bf16 attention forward with LSE,
    B=2, H=32, Hkv=8, Sq=Sk=4096, D=128                      (attn_fwd)
  * decode:  split-KV bf16 decode, B=64, H=32, Hkv=8, D=128, lengths uniform
    in [512, 32768] (cache 32768), n_splits=8               (attn_decode_ws)
both launched on the same stream.  ``value`` is the prefill rate in TFLOP/s of
algorithmic work (4*D flops per allowed (query, key) pair) divided by the
prefill kernel's mean duration from HIP events over the timed steps (recorded
with a device-scope release, so that an interval holds the kernel and not the
L2 writeback a system-scope event forces after it); the
decode rate in GB/s (K/V bytes of the valid keys, once per KV head, plus Q and
O) is reported beside it.  The window/offset and clustered-image workloads are
timed too, as extra lines of context, and so is the same decode batch stored
in a paged serving cache (block size 16, shuffled physical blocks;
attn_decode_paged), and the causal GQA prefill with soft-capping and ALiBi
(attn_fwd_flex), its backward (attn_bwd), and block-sparse attention on the
image workload (top-10% key blocks by centroid score).  ``cpu_baseline`` times the fp64 oracle
on the host on a bounded sample (whole heads) of the prefill workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]

The GPU needs about a hundred prefill launches to reach its steady clock, so
the default warm-up is 100 steps.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
# The CPU baseline's BLAS threads: the CPUs this process may run on, unless the
# environment already fixes them (set before NumPy is first imported).
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_var, str(len(os.sched_getaffinity(0))))

METRIC = ("attn fwd bf16 TFLOP/s (prefill) + decode KV GB/s, % of roofline, 1 MI355X")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "prefill": ["scaled_dot_product_attn_amd/csrc/attn_fwd_bf16.hip",
                "scaled_dot_product_attn_amd/csrc/attn_common.h"],
    "decode": ["scaled_dot_product_attn_amd/csrc/attn_decode.hip"],
    "decode_paged": ["scaled_dot_product_attn_amd/csrc/attn_decode.hip"],
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def allowed_pairs(Sq, Sk, causal, window, input_pos, k_len):
    """Allowed (query, key) pairs of one (batch, head), counted row by row."""
    import numpy as np
    p = input_pos + np.arange(Sq, dtype=np.int64)
    kl = min(max(k_len, 0), Sk)
    hi = np.clip(p + 1, 0, kl) if causal else np.full(Sq, kl)
    lo = np.clip(p - window + 1, 0, kl) if window > 0 else np.zeros(Sq, dtype=np.int64)
    return int(np.maximum(hi - lo, 0).sum())


def prefill_flops(w) -> int:
    B, H, Sq, D = w.q.shape
    Sk = w.k.shape[2]
    total = 0
    for b in range(B):
        kl = Sk if w.k_lengths is None else int(w.k_lengths[b])
        total += H * allowed_pairs(Sq, Sk, w.causal, w.window, w.input_pos, kl)
    return 4 * D * total


def decode_bytes(w) -> int:
    B, H, D = w.q.shape
    if hasattr(w, "k_cache"):
        Hkv = w.k_cache.shape[2]
        cap = w.block_tables.shape[1] * w.k_cache.shape[1]
    else:
        Hkv, cap = w.k.shape[1], w.k.shape[2]
    lens = w.lengths.cpu().clamp(0, cap).long().sum().item()
    return int(lens) * Hkv * D * 2 * 2 + B * H * D * 2 * 2


def traffic_for(kind: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if current."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)[kind]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_hash") != source_hash(kind):
        return None
    return t.get("bytes_per_launch")


# hipDeviceAttribute_t values (hip/hip_runtime_api.h of this ROCm)
_HIP_ATTR = {"clock_khz": 5, "memory_bus_bits": 59, "memory_clock_khz": 60, "cus": 63}
FLOP_PER_CLK_PER_CU_BF16 = 4096  # dense bf16 MFMA on gfx950 (4 SIMDs x 1024)


def device_info(torch) -> dict:
    """The GPU's own figures (hipDeviceGetAttribute) and the dense bf16 MFMA
    peak they imply (CUs x 4096 flop/clk x the peak engine clock).  The memory
    clock and bus width are reported as the runtime gives them; the HBM peak
    stays the published 8 TB/s."""
    import ctypes
    dev = torch.cuda.current_device()
    props = torch.cuda.get_device_properties(dev)
    info = {"name": props.name, "arch": getattr(props, "gcnArchName", None)}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return info
    for key, attr in _HIP_ATTR.items():
        v = ctypes.c_int(0)
        rc = hip.hipDeviceGetAttribute(ctypes.byref(v), ctypes.c_int(attr), ctypes.c_int(dev))
        info[key] = v.value if rc == 0 else None
    if info.get("cus") and info.get("clock_khz"):
        info["peak_bf16_tflops_at_clock"] = round(
            info["cus"] * FLOP_PER_CLK_PER_CU_BF16 * info["clock_khz"] * 1e3 / 1e12, 1)
    return info


class DeviceEvent:
    """A timing event recorded with a device-scope release (hipEventCreateWithFlags
    with hipEventReleaseToDevice).  A default event's record is a system-scope
    release: it writes the L2's dirty lines back to HBM, so the interval it closes
    also holds the writeback of what the kernel before it wrote (the prefill's
    67 MB of O).  Work between two of these events is timed as the kernels take
    it, as the profiler's kernel trace times it; the host sees results only after
    a full synchronization, as before."""
    _hip = None
    RELEASE_TO_DEVICE = 0x40000000  # hipEventReleaseToDevice (hip_runtime_api.h)

    def __init__(self):
        import ctypes
        if DeviceEvent._hip is None:
            h = ctypes.CDLL("libamdhip64.so")
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            DeviceEvent._hip = h
        self._ct = ctypes
        self.h = ctypes.c_void_p()
        rc = DeviceEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.h),
                                                      DeviceEvent.RELEASE_TO_DEVICE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags returned {rc}")

    def record(self, stream):
        rc = DeviceEvent._hip.hipEventRecord(self.h, self._ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord returned {rc}")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (both recorded and completed)."""
        ms = self._ct.c_float(0.0)
        rc = DeviceEvent._hip.hipEventElapsedTime(self._ct.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime returned {rc}")
        return ms.value

    def __del__(self):
        if self.h and DeviceEvent._hip is not None:
            DeviceEvent._hip.hipEventDestroy(self.h)


def cpu_baseline(w, seconds: float):
    """The fp64 oracle on whole (batch, head) pairs of the prefill workload."""
    import numpy as np
    from oracle import attn_oracle as ora
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    q = w.q.float().cpu().numpy().astype(np.float64)
    k = w.k.float().cpu().numpy().astype(np.float64)
    v = w.v.float().cpu().numpy().astype(np.float64)
    B, H, Sq, D = q.shape
    per_head = 4 * D * allowed_pairs(Sq, w.k.shape[2], w.causal, w.window, w.input_pos,
                                     w.k.shape[2])
    done, t0 = 0, time.perf_counter()
    for b in range(B):
        for h in range(H):
            ora.attn_ref(q, k, v, w.causal, w.window, w.input_pos, None, heads=[(b, h)])
            done += 1
            if time.perf_counter() - t0 >= seconds:
                break
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": per_head * done / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{done} of {B * H} (batch, head) pairs of the causal GQA prefill "
                      f"(Sq=Sk={Sq}, D={D}), fp64 NumPy, {dt:.1f} s"}


def _cores():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def cpu_rows(pre, dec, dO, slopes, img, keep, seconds: float, paged=None, doc=None):
    """The fp64 oracle beside each row after the hot path, each on a bounded
    sample of the same inputs the GPU ran (whole (batch, head) pairs, whole
    sequences), as a rate in the row's own unit."""
    import numpy as np
    from oracle import attn_oracle as ora
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    cores = _cores()
    out = {}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    # decode: whole sequences, longest first until `seconds`
    lens = dec.lengths.cpu().long()
    order = sorted(range(len(lens)), key=lambda b: -int(lens[b]))
    done_b, nbytes, dt = [], 0, 0.0
    Hkv, D = dec.k.shape[1], dec.k.shape[3]
    for b in order:
        L = int(lens[b])
        q = f64(dec.q[b:b + 1])
        k, v = f64(dec.k[b:b + 1, :, :L]), f64(dec.v[b:b + 1, :, :L])
        dt += timed(lambda: ora.decode_ref(q, k, v, np.array([L])))
        nbytes += L * Hkv * D * 2 * 2 + dec.q.shape[1] * D * 2 * 2
        done_b.append(b)
        if dt >= seconds:
            break
    out["decode"] = {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": cores,
                     "kind": "oracle",
                     "sample": f"{len(done_b)} of {len(lens)} sequences (the longest), "
                               f"decode_ref, {dt:.1f} s"}
    # paged decode: whole sequences, longest first, each gathered through its
    # block table by the oracle (the caches handed over hold only its blocks)
    if paged is not None:
        lens = paged.lengths.cpu().long()
        tables = paged.block_tables.cpu().long()
        bs, Hkv_p = paged.k_cache.shape[1], paged.k_cache.shape[2]
        order = sorted(range(len(lens)), key=lambda b: -int(lens[b]))
        done, nbytes, dt = 0, 0, 0.0
        for b in order:
            L = int(lens[b])
            nb = (L + bs - 1) // bs
            blocks = tables[b, :nb].to(paged.k_cache.device)
            kc, vc = f64(paged.k_cache[blocks]), f64(paged.v_cache[blocks])
            q = f64(paged.q[b:b + 1])
            table = np.arange(nb)[None, :]
            dt += timed(lambda: ora.decode_paged_ref(q, kc, vc, table, np.array([L])))
            nbytes += L * Hkv_p * D * 2 * 2 + paged.q.shape[1] * D * 2 * 2
            done += 1
            if dt >= seconds:
                break
        out["decode_paged"] = {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s",
                               "cores": cores, "kind": "oracle",
                               "sample": f"{done} of {len(lens)} sequences (the longest), "
                                         f"decode_paged_ref, {dt:.1f} s"}
    # prefill-shaped rows: one (batch, head) pair each
    B, H, Sq, D = pre.q.shape
    pairs = allowed_pairs(Sq, pre.k.shape[2], pre.causal, pre.window, pre.input_pos,
                          pre.k.shape[2])
    q, k, v = f64(pre.q[:1]), f64(pre.k[:1]), f64(pre.v[:1])
    dt = timed(lambda: ora.flex_ref(q, k, v, True, softcap=30.0,
                                    alibi_slopes=f64(slopes), heads=[(0, 0)]))
    out["flex_softcap_alibi"] = {
        "value": round(4 * D * pairs / dt / 1e12, 5), "unit": "TFLOP/s", "cores": cores,
        "kind": "oracle", "sample": f"1 of {B * H} (batch, head) pairs, flex_ref, {dt:.1f} s"}
    if doc is not None:
        d0 = doc[:1].cpu().numpy()
        dt = timed(lambda: ora.flex_ref(q, k, v, True, doc_q=d0, doc_kv=d0, heads=[(0, 0)]))
        out["flex_documents"] = {
            "value": round(document_flops(doc[:1], 1, D) / dt / 1e12, 5), "unit": "TFLOP/s",
            "cores": cores, "kind": "oracle",
            "sample": f"1 of {B * H} (batch, head) pairs, flex_ref with documents, {dt:.1f} s"}
    g = f64(dO[:1])
    dt = timed(lambda: ora.attn_bwd_ref(q, k, v, g, True, heads=[(0, 0)]))
    out["backward"] = {
        "value": round(10 * D * pairs / dt / 1e12, 5), "unit": "TFLOP/s", "cores": cores,
        "kind": "oracle", "sample": f"1 of {B * H} (batch, head) pairs, attn_bwd_ref, {dt:.1f} s"}
    # block-sparse: one head of the image workload
    qi, ki, vi = f64(img.q[:1, :1]), f64(img.k[:1, :1]), f64(img.v[:1, :1])
    kp = keep[:1, :1].cpu().numpy().astype(bool)
    kept = int(kp.sum())
    dt = timed(lambda: ora.block_sparse_attn_ref(qi, ki, vi, kp))
    out["block_sparse"] = {
        "value": round(4 * qi.shape[3] * kept * 64 * 64 / dt / 1e12, 5), "unit": "TFLOP/s",
        "cores": cores, "kind": "oracle",
        "sample": f"1 of {img.q.shape[1]} heads, block_sparse_attn_ref, {dt:.1f} s"}
    dt = timed(lambda: ora.rbs_block_scores_ref(qi, ki))
    out["block_estimate"] = {
        "value": round(dt * img.q.shape[1] * 1e3, 1), "unit": "ms (whole workload, "
        "extrapolated)", "cores": cores, "kind": "oracle",
        "sample": f"1 of {img.q.shape[1]} heads, rbs_block_scores_ref, {dt:.1f} s"}
    return out


def document_flops(doc, H: int, D: int) -> int:
    """4 D flops per allowed pair of causal attention inside each document of
    the (B, S) id rows (ids constant on contiguous runs), over H heads."""
    total = 0
    for row in doc.cpu().tolist():
        run = 0
        for i, d in enumerate(row):
            run = run + 1 if i > 0 and d == row[i - 1] else 1
            total += run  # row i sees the `run` keys of its document up to itself
    return 4 * D * H * total


def timing_stats(times_ms):
    """Mean, median and min of per-launch times (ms)."""
    t = sorted(times_ms)
    n = len(t)
    med = t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2])
    return {"mean": round(sum(t) / n, 4), "median": round(med, 4), "min": round(t[0], 4)}


def profile_prefill(torch, attn, w, args):
    """One prefill workload alone: warm-up, then timed launches on one stream."""
    B, H, Sq, D = w.q.shape
    O = torch.empty_like(w.q)
    LSE = torch.empty(B, H, Sq, dtype=torch.float32, device=w.q.device)
    stream = torch.cuda.current_stream()
    run = lambda: attn.attn_fwd(O, w.q, w.k, w.v, LSE, w.causal, w.window, w.input_pos,
                                w.k_lengths)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ev = []
    for _ in range(args.steps):
        s, e = DeviceEvent(), DeviceEvent()
        s.record(stream)
        run()
        e.record(stream)
        ev.append((s, e))
    torch.cuda.synchronize()
    t = timing_stats([s.elapsed_time(e) for s, e in ev])
    f = prefill_flops(w)
    print(json.dumps({"profile_prefill": args.profile_prefill, "flops": f, "ms": t,
                      "TFLOP/s_median": round(f / (t["median"] * 1e-3) / 1e12, 2)}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--profile-prefill", choices=["gqa_causal", "window_offset", "image_clustered"],
                    help="time only this prefill workload (for per-workload profiler passes) and "
                         "print its timing line instead of the bench line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the kernels run on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import torch
    import scaled_dot_product_attn_amd as attn
    from scaled_dot_product_attn_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.profile_prefill:
        profile_prefill(torch, attn, wl.make(args.profile_prefill, device=dev), args)
        return
    log("generating inputs")
    pre = wl.make("gqa_causal", device=dev)
    dec = wl.make("decode_split", device=dev)
    extra = {} if args.no_extra else {n: wl.make(n, device=dev)
                                     for n in ("window_offset", "image_clustered")}
    paged = None if args.no_extra else wl.make("decode_paged", device=dev)
    # flex: the causal GQA prefill with soft-capping (cap 30) and ALiBi slopes
    gflex = torch.Generator().manual_seed(7)
    flex_slopes = (-torch.rand(pre.q.shape[1], generator=gflex) * 0.01).to(dev)
    B, H, Sq, D = pre.q.shape
    O = torch.empty_like(pre.q)
    LSE = torch.empty(B, H, Sq, dtype=torch.float32, device=dev)
    Od = torch.empty_like(dec.q)
    Bd, Hd, Dd = dec.q.shape
    ws = torch.empty(attn.attn_decode_workspace_bytes(Bd, Hd, dec.n_splits, Dd),
                     dtype=torch.uint8, device=dev)
    ext_out = {n: (torch.empty_like(w.q),
                   torch.empty(w.q.shape[:3], dtype=torch.float32, device=dev))
               for n, w in extra.items()}
    stream = torch.cuda.current_stream()

    def run_prefill(w, o, l):
        attn.attn_fwd(o, w.q, w.k, w.v, l, w.causal, w.window, w.input_pos, w.k_lengths)

    def run_decode():
        attn.attn_decode_ws(Od, dec.q, dec.k, dec.v, dec.lengths, dec.n_splits, ws)

    Op = torch.empty_like(dec.q)

    def run_paged():
        attn.attn_decode_paged(Op, paged.q, paged.k_cache, paged.v_cache, paged.block_tables,
                               paged.lengths, paged.n_splits, workspace=ws)

    Of, Lf = torch.empty_like(pre.q), torch.empty_like(LSE)
    # backward of the causal GQA prefill (dO seeded, O / LSE from attn_fwd)
    if not args.no_extra:
        gb = torch.Generator().manual_seed(8)
        dO = torch.randn(pre.q.shape, generator=gb).bfloat16().to(dev)
        Ob, Lb = torch.empty_like(pre.q), torch.empty_like(LSE)
        attn.attn_fwd(Ob, pre.q, pre.k, pre.v, Lb, True)
        dQ, dK, dV = torch.empty_like(pre.q), torch.empty_like(pre.k), torch.empty_like(pre.v)
        bws = torch.empty(attn.attn_bwd_workspace_bytes(B, H, Sq, D), dtype=torch.uint8,
                          device=dev)

    def run_bwd():
        attn.attn_bwd(dQ, dK, dV, dO, pre.q, pre.k, pre.v, Ob, Lb, True, workspace=bws)

    # block-sparse: the image workload, centroid (RBS base) block scores, the
    # top 10 % of key blocks per row block, attention on the kept blocks
    if not args.no_extra:
        img = extra["image_clustered"]
        nbq = -(-img.q.shape[2] // attn.BLOCK)
        nbk = -(-img.k.shape[2] // attn.BLOCK)
        bs_scores = torch.empty(img.q.shape[0], img.q.shape[1], nbq, nbk, device=dev)
        bs_keep = torch.empty(bs_scores.shape, dtype=torch.uint8, device=dev)
        bs_ws = torch.empty(attn.attn_block_scores_workspace_bytes(
            img.k.shape[0], img.k.shape[1], img.k.shape[2], img.k.shape[3]),
            dtype=torch.uint8, device=dev)
        bs_topk = max(1, -(-nbk // 10))
        Obs, Lbs = torch.empty_like(img.q), torch.empty(img.q.shape[:3], device=dev)

    def run_block_estimate():
        attn.attn_block_scores(bs_scores, None, img.q, img.k, attn.BLOCK_SCORES_RBS,
                               workspace=bs_ws)
        attn.attn_block_mask(bs_keep, bs_scores, attn.BLOCK_MASK_TOPK, k=bs_topk)

    def run_block_sparse():
        attn.attn_fwd_block_sparse(Obs, img.q, img.k, img.v, bs_keep, Lbs, False)

    def run_flex():
        attn.attn_fwd_flex(Of, pre.q, pre.k, pre.v, Lf, True, softcap=30.0,
                           alibi_slopes=flex_slopes)

    # documents: the gqa_causal tensors packed as 16 documents per sequence,
    # causal inside each document (DocumentMask); the BlockMask is built once,
    # as a caller would per batch layout, and timed on its own
    if not args.no_extra:
        doc = wl.documents_of(pre)
        doc_bm = attn.build_block_mask(Sq, pre.k.shape[2], B, causal=True, doc_q=doc,
                                       doc_kv=doc, device=dev)

    def run_doc_build():
        attn.attn_build_block_mask(doc_bm, Sq, pre.k.shape[2], True, doc_q=doc, doc_kv=doc)

    def run_doc(block_mask):
        attn.attn_fwd_flex(Of, pre.q, pre.k, pre.v, Lf, True, doc_q=doc, doc_kv=doc,
                           block_mask=block_mask)

    names = ["prefill", "decode"] + list(extra) + (["decode_paged"] if paged is not None else [])
    if not args.no_extra:
        names += ["flex_softcap_alibi", "backward", "block_estimate", "block_sparse",
                  "flex_documents", "flex_documents_dense", "block_mask_build"]
    ev = {n: [] for n in names}

    def step(record):
        marks = {}
        for n in names:
            if record:
                s, e = DeviceEvent(), DeviceEvent()
                s.record(stream)
            if n == "prefill":
                run_prefill(pre, O, LSE)
            elif n == "decode":
                run_decode()
            elif n == "decode_paged":
                run_paged()
            elif n == "flex_softcap_alibi":
                run_flex()
            elif n == "backward":
                run_bwd()
            elif n == "block_estimate":
                run_block_estimate()
            elif n == "block_sparse":
                run_block_sparse()
            elif n == "flex_documents":
                run_doc(doc_bm)
            elif n == "flex_documents_dense":
                run_doc(None)
            elif n == "block_mask_build":
                run_doc_build()
            else:
                run_prefill(extra[n], *ext_out[n])
            if record:
                e.record(stream)
                marks[n] = (s, e)
        if record:
            for n in names:
                ev[n].append(marks[n])

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {n: sum(s.elapsed_time(e) for s, e in ev[n]) / args.steps for n in names}
    timing = {n: timing_stats([s.elapsed_time(e) for s, e in ev[n]]) for n in names}
    log("kernel ms: " + ", ".join(f"{n}={ms[n]:.4f}" for n in names))

    fl = prefill_flops(pre)
    pre_tf = fl / (ms["prefill"] * 1e-3) / 1e12
    db = decode_bytes(dec)
    dec_gbs = db / (ms["decode"] * 1e-3) / 1e9

    def roof(bound, achieved, peak, unit, traffic):
        return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic}

    out = {
        "metric": METRIC,
        "value": round(pre_tf, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "gqa_causal prefill + decode_split decode",
            "prefill": "B=2 H=32 Hkv=8 Sq=Sk=4096 D=128 causal, LSE saved",
            "decode": "B=64 H=32 Hkv=8 D=128 len~U[512,32768] cache 32768 n_splits=8",
            "prefill_flops": fl,
            "decode_bytes": db,
        },
        "roofline": roof("mfma", pre_tf, PEAK_BF16_TFLOPS, "TFLOP/s", traffic_for("prefill")),
        "device": device_info(torch),
        "timing_ms": timing,
        "prefill_ms": round(ms["prefill"], 4),
        "decode": {
            "value": round(dec_gbs, 1), "unit": "GB/s", "ms": round(ms["decode"], 4),
            "roofline": roof("hbm", dec_gbs, PEAK_HBM_GBS, "GB/s", traffic_for("decode")),
        },
    }
    if extra:
        out["extra"] = {}
        for n, w in extra.items():
            f = prefill_flops(w)
            tf = f / (ms[n] * 1e-3) / 1e12
            out["extra"][n] = {"ms": round(ms[n], 4), "TFLOP/s": round(tf, 2),
                               "frac": round(tf / PEAK_BF16_TFLOPS, 4), "flops": f}
    if "flex_softcap_alibi" in ms:
        tf = fl / (ms["flex_softcap_alibi"] * 1e-3) / 1e12
        out["flex_softcap_alibi"] = {
            "ms": round(ms["flex_softcap_alibi"], 4), "TFLOP/s": round(tf, 2),
            "frac": round(tf / PEAK_BF16_TFLOPS, 4), "flops": fl,
            "config": "gqa_causal prefill with soft-cap 30 and ALiBi slopes (attn_fwd_flex)"}
    if "backward" in ms:
        bf = fl * 5 // 2  # five contractions against the forward's two
        tf = bf / (ms["backward"] * 1e-3) / 1e12
        out["backward"] = {
            "ms": round(ms["backward"], 4), "TFLOP/s": round(tf, 2),
            "frac": round(tf / PEAK_BF16_TFLOPS, 4), "flops": bf,
            "config": "attn_bwd of the gqa_causal prefill (delta + dK/dV + dQ kernels); "
                      "flops = 2.5 x forward (S, dP, dV, dK, dQ)"}
    if "block_sparse" in ms:
        kept = int(bs_keep.sum().item())
        bfl = 4 * img.q.shape[3] * kept * attn.BLOCK * attn.BLOCK
        tf = bfl / (ms["block_sparse"] * 1e-3) / 1e12
        out["block_sparse"] = {
            "ms": round(ms["block_sparse"], 4), "TFLOP/s": round(tf, 2),
            "frac": round(tf / PEAK_BF16_TFLOPS, 4), "flops": bfl,
            "kept_fraction": round(kept / bs_keep.numel(), 4),
            "estimate_ms": round(ms["block_estimate"], 4),
            "config": "image_clustered, RBS-base block scores, top-10% key blocks per row "
                      "block (attn_block_scores + attn_block_mask, then attn_fwd_block_sparse); "
                      "flops = 4 D per pair of the kept blocks"}
    if "flex_documents" in ms:
        dfl = document_flops(doc, H, D)
        tf = dfl / (ms["flex_documents"] * 1e-3) / 1e12
        tfd = dfl / (ms["flex_documents_dense"] * 1e-3) / 1e12
        bmc = doc_bm.cpu()
        out["flex_documents"] = {
            "ms": round(ms["flex_documents"], 4), "TFLOP/s": round(tf, 2),
            "frac": round(tf / PEAK_BF16_TFLOPS, 4), "flops": dfl,
            "dense_ms": round(ms["flex_documents_dense"], 4),
            "dense_TFLOP/s": round(tfd, 2),
            "speedup_vs_dense": round(ms["flex_documents_dense"] / ms["flex_documents"], 3),
            "block_mask_build_ms": round(ms["block_mask_build"], 4),
            "blocks_empty_partial_full": [int((bmc == c).sum()) for c in (0, 1, 2)],
            "config": "gqa_documents: the gqa_causal tensors, 16 documents per 4096-token "
                      "sequence, causal within each (attn_fwd_flex with doc_q/doc_kv and the "
                      "BlockMask of attn_build_block_mask; dense = the same call without it, "
                      "masking every tile of the causal union element by element); "
                      "flops = 4 D per allowed pair"}
    if paged is not None:
        pb = decode_bytes(paged)
        gbs = pb / (ms["decode_paged"] * 1e-3) / 1e9
        out["decode_paged"] = {
            "value": round(gbs, 1), "unit": "GB/s", "ms": round(ms["decode_paged"], 4),
            "config": "same sequences as decode, cache (num_blocks, 16, 8, 128) with "
                      "shuffled physical blocks",
            "roofline": roof("hbm", gbs, PEAK_HBM_GBS, "GB/s", traffic_for("decode_paged")),
        }
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle)")
        out["cpu_baseline"] = cpu_baseline(pre, args.cpu_seconds)
        if extra:
            log("fp64 oracle beside the other rows")
            rows = cpu_rows(pre, dec, dO, flex_slopes, img, bs_keep, args.cpu_seconds / 5,
                            paged, doc)
            for n, r in rows.items():
                if n in out:
                    out[n]["cpu_oracle"] = r
                elif n == "block_estimate" and "block_sparse" in out:
                    out["block_sparse"]["estimate_cpu_oracle"] = r
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
