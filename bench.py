"""Benchmark of IBP batched gather + decompress on one MI355X.

A step is one gather + decompress launch (participation scan, payload fetch,
decode, dense store) over one fresh batch of ids drawn from the workload's id
law.  The default workload is the sparse GNN feature table (2^20 rows of 1,433
fp32, 1 KB chunks, Mask from a 1 % sample, 8,192 uniform ids per batch) held
compressed in pinned host memory: every step reads the compressed payloads
over PCIe with GPU-initiated loads.

Prints ONE JSON line.  `value` is decompressed GB/s (ids x tensor bytes per
second of wall time over the timed steps, inputs already resident).  Extra
objects:
  roofline           the gather kernel against the host-link peak (63 GB/s
                     published; the measured DMA and zero-copy peaks beside it),
                     with the link bytes rocprofv3 counted per launch as traffic;
  cpu_baseline       the CPU oracle on a bounded sample of the same batches;
  hybrid_path        cache hits from HBM and misses over PCIe in one launch, at a
                     fixed HBM budget, compressed against uncompressed tensors;
  configs            the tiny table as an HBM cache (config 1) and the sparse
                     table at T = 0.95 (config 2);
  pinned_path        dense GNN and DLRM tables from pinned host memory (link
                     fractions on the bytes of each batch's distinct tensors);
  hbm_path           the same tables as compressed caches in HBM: the workload's
                     batch, 1M Zipf ids and 1M distinct ids, three cache layouts,
                     against the uncompressed gather of the same ids;
  kv_step            the OPT-13B K/V decode step, all 80 (layer, K|V) pairs;
  sampled_metadata   Masks from 1 %, 5 %, 10 % samples against all tensors;
  weight_stream      one OPT-13B decoder layer's BF16 weights streamed in;
  saving_sweep       throughput against space saving (0-90 %) and chunk size;
  transfer_ablation  small random tensors by transfer method;
and the transfer speedup over an uncompressed GPU gather of the same rows
([JH] Table 1 discussion: transfer speedup against plain transfers).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload sparse_gnn]
       [--pinned-workloads dense_gnn,dlrm_1k,dlrm_2k|none] [--kv-pairs-default 80]
       [--hbm-workloads dense_gnn,dlrm_1k|none] [--hbm-large-batch N] [--no-extras]
       [--mode default|ablation|sweep|kv-step|configs]
       [--host-flags default|coherent|noncoherent] [--no-cpu-baseline] [--threshold T]
"""
import argparse
import json
import os
import platform
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PCIE5_X16_GBPS = 63.0      # PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes x 128/130 / 8
HBM_PEAK_GBPS = 8000.0     # MI355X HBM3E

# Traffic of the headline launch (8,192 sparse_gnn ids) from rocprofv3 counter
# runs of this benchmark, bytes per dispatch, each counter calibrated by a
# transfer of known size in the same run: host-link reads
# (TCC_EA0_RDREQ_IO_32B x 32 B, a 1 GiB zero-copy read reads as 1.000), HBM reads
# and writes (TCC_EA0_RDREQ_DRAM_32B and TCC_EA0_WRREQ_WRITE_DRAM_32B x 32 B, a 4
# GiB read and a 2 GiB HBM copy read as 1.000), and FETCH_SIZE / WRITE_SIZE in KiB
# (factors 2.000 / 1.000).  Valid only for the gather code they were measured
# on: bench.py reports them while the sources (comments and spacing aside)
# still hash to GATHER_SOURCES_SHA256, else traffic is null.
GATHER_SOURCES = ("host_transfer_amd/csrc/gather.hip", "host_transfer_amd/csrc/ibp_plan.h",
                  "host_transfer_amd/csrc/ibp_device.h")
GATHER_SOURCES_SHA256 = "470bd05ffa9d23b09395737559715907ac362081fa8a67c568a0b60209e244d9"
HEADLINE_COUNTERS = {"link_read": 10632453, "hbm_read": 1694317, "hbm_write": 49649810,
                     "fetch_size_kib": 6191.5, "write_size_kib": 48511.6}
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
# HBM bytes (read, written) per 1M-id cache launch, from the same runs (the
# summary in profiles/k_gather_cache__dense_gnn_dlrm_1k_hbm.md), for the code
# of gather_cache.hip they were measured on (CACHE_SOURCES_SHA256).
CACHE_SOURCES = ("host_transfer_amd/csrc/gather_cache.hip", "host_transfer_amd/csrc/ibp_plan.h",
                 "host_transfer_amd/csrc/ibp_device.h")
CACHE_SOURCES_SHA256 = "b685aa934fc992145b138a565a900cad876ad4772c99020426b89da4a5ac9a92"
HBM_COUNTERS = {
    ("dense_gnn", "zipf"): {"index_128B": (184.20e6, 536.87e6), "index_16B": (222.95e6, 536.87e6),
                            "table_16B": (262.47e6, 536.87e6), "raw": (179.09e6, 536.87e6)},
    ("dense_gnn", "distinct"): {"index_128B": (577.12e6, 536.87e6),
                                "index_16B": (684.97e6, 536.87e6),
                                "table_16B": (794.26e6, 536.87e6), "raw": (553.66e6, 536.88e6)},
    ("dlrm_1k", "zipf"): {"index_128B": (512.94e6, 1073.74e6), "index_16B": (512.96e6, 1073.74e6),
                          "table_16B": (575.51e6, 1073.74e6), "raw": (542.20e6, 1073.74e6)},
    ("dlrm_1k", "distinct"): {"index_128B": (1075.99e6, 1073.75e6),
                              "index_16B": (1075.99e6, 1073.75e6),
                              "table_16B": (1192.33e6, 1073.74e6), "raw": (1107.31e6, 1073.75e6)},
}


def code_text(src):
    """C++ source without comments and with runs of whitespace collapsed, so
    that only changes to the code itself change its hash."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def gather_sources_sha256(read=None, sources=GATHER_SOURCES):
    import hashlib
    h = hashlib.sha256()
    for rel in sources:
        if read is None:
            with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
                text = f.read()
        else:
            text = read(rel)
        h.update(code_text(text).encode())
    return h.hexdigest()


def profiled_traffic():
    """Counter bytes of the headline launch (see HEADLINE_COUNTERS), or None
    when the gather code has changed since they were taken."""
    if GATHER_SOURCES_SHA256 is None or gather_sources_sha256() != GATHER_SOURCES_SHA256:
        return None
    c = HEADLINE_COUNTERS
    return {"link_read": c["link_read"], "hbm_read": c["hbm_read"], "hbm_write": c["hbm_write"],
            "fetch_size": round(c["fetch_size_kib"] * 1024 * FETCH_SCALE),
            "write_size": round(c["write_size_kib"] * 1024 * WRITE_SCALE)}


def profiled_hbm_bytes(key, kind):
    """Counter HBM bytes {launch: [read, written]} of a 1M-id cache launch, or
    None when gather_cache.hip has changed since they were taken."""
    if (CACHE_SOURCES_SHA256 is None or
            gather_sources_sha256(sources=CACHE_SOURCES) != CACHE_SOURCES_SHA256):
        return None
    c = HBM_COUNTERS.get((key, kind))
    return None if c is None else {k: [round(v[0]), round(v[1])] for k, v in c.items()}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="sparse_gnn")
    p.add_argument("--hbm-workloads", default="dense_gnn,dlrm_1k",
                   help="comma-separated workloads measured as compressed HBM caches, or 'none'")
    p.add_argument("--hbm-large-batch", type=int, default=1 << 20)
    p.add_argument("--host-flags", default="default", choices=["default", "coherent", "noncoherent"])
    p.add_argument("--threshold", type=float, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--mode", default="default",
                   choices=["default", "ablation", "sweep", "kv-step", "configs"],
                   help="default: the headline and the cache paths; ablation: transfer methods "
                        "for small random tensors; sweep: throughput against space saving and "
                        "chunk size; kv-step: the online OPT-13B K/V path; configs: one row per "
                        "workload (oracle on 1 and all threads, GPU from pinned memory and HBM)")
    p.add_argument("--kv-pairs", type=int, default=80, help="(layer, K|V) pairs in --mode kv-step")
    p.add_argument("--pinned-workloads", default="dense_gnn,dlrm_1k,dlrm_2k",
                   help="other workloads measured from pinned host memory, or 'none'")
    p.add_argument("--kv-pairs-default", type=int, default=80,
                   help="(layer, K|V) pairs of the K/V decode step in the default run (0: skip)")
    p.add_argument("--no-extras", dest="extras", action="store_false",
                   help="skip the other configurations and rows of the default run (tiny and "
                        "T=0.95 configs, sampled metadata, weight stream, saving sweep, "
                        "transfer ablation)")
    return p.parse_args()


def host_info():
    info = {"cpu": platform.processor() or "", "cores": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0))}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            k, _, v = line.partition(":")
            if k.strip() in ("Model name", "Socket(s)", "NUMA node(s)", "Thread(s) per core"):
                info[k.strip()] = v.strip()
    except Exception:
        pass
    return info


class Timer:
    """HIP events on torch's current stream (the stream the kernels use)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, s):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append((s, e))

    def ms(self):
        self.torch.cuda.synchronize()
        return [s.elapsed_time(e) for s, e in self.pairs]


class Table:
    """One workload compressed on the GPU into a store (pinned host or HBM)."""

    def __init__(self, torch, ibp, W, w, T, where, host_flags, keep_raw=True):
        import numpy as np
        self.w, self.T, self.where = w, T, where
        B, C, S, N = w.tensor_bytes, w.chunk_bytes, w.slot_bytes, w.n_tensors
        self.n_c = ibp.num_chunks(B, C)
        t0 = time.time()
        # raw rows in pinned host memory, slot-strided (also the raw-gather source)
        self.raw = ibp.HostBuffer(N * S, host_flags)
        view = self.raw.array.reshape(N, S)
        W.rows(w, 0, N, out=view[:, :B])
        log(f"{w.key}: generated {N} x {B} B in {time.time() - t0:.1f} s")
        # metadata from the sample (rows read by the GPU from pinned memory)
        sid = W.sample_ids(w)
        n_s = N if sid is None else len(sid)
        d_sid = None if sid is None else torch.from_numpy(sid).cuda()
        self.mask = torch.zeros(B // 4, dtype=torch.int32, device="cuda")
        self.bitval = torch.zeros_like(self.mask)
        counts = torch.zeros(8 * B, dtype=torch.int32, device="cuda")
        ev = Timer(torch)
        s = ev.start()
        ibp.build_metadata(self.raw, S, d_sid, n_s, B, T, self.mask, self.bitval, counts)
        ev.stop(s)
        # compress into the store
        if where == "pinned":
            self.store = ibp.HostBuffer(N * S, host_flags)
        else:
            self.store = torch.empty(N * S, dtype=torch.uint8, device="cuda")
        self.part = torch.zeros((N * self.n_c + 31) // 32, dtype=torch.int32, device="cuda")
        self.lengths = torch.zeros(N, dtype=torch.int32, device="cuda")
        s = ev.start()
        ibp.compress(self.raw, S, N, 0, N, B, C, self.mask, self.bitval, self.store, S, self.part,
                     self.lengths)
        ev.stop(s)
        self.offsets = None
        self.cache = None
        self.store_bytes = N * S
        if where == "hbm":
            # compacted cache in HBM
            self.offsets = torch.zeros(N + 1, dtype=torch.int64, device="cuda")
            s = ev.start()
            ibp.compact_offsets(self.lengths, N, self.offsets)
            ev.stop(s)
            total = int(self.offsets[-1].item())
            self.cache = torch.empty(max(total, 16), dtype=torch.uint8, device="cuda")
            s = ev.start()
            ibp.compact(self.store, S, N, self.offsets, self.cache, total)
            ev.stop(s)
            self.store_bytes = total
            del self.store
            self.store = self.cache
        ms = ev.ms()
        self.meta_ms, self.compress_ms = ms[0], ms[1]
        self.compact_ms = sum(ms[2:]) if where == "hbm" else None
        # the metadata build again, warm (the first call also pays for the first
        # touch of the sampled rows' pages)
        self.meta_bytes = n_s * B
        m2, v2 = torch.zeros_like(self.mask), torch.zeros_like(self.bitval)
        warm = Timer(torch)
        for _ in range(3):
            s = warm.start()
            ibp.build_metadata(self.raw, S, d_sid, n_s, B, T, m2, v2, counts)
            warm.stop(s)
        self.meta_warm_ms = min(warm.ms())
        if not (bool((m2 == self.mask).all().item()) and bool((v2 == self.bitval).all().item())):
            raise SystemExit("bench: a repeated metadata build gave another Mask/Bitval")
        self.len_host = self.lengths.cpu().numpy().view(np.uint32)
        self.mask_host = self.mask.cpu().numpy().view(np.uint32)
        self.bitval_host = self.bitval.cpu().numpy().view(np.uint32)
        if not keep_raw:
            self.raw.free()
            self.raw = None
        log(f"{w.key}: metadata {self.meta_ms:.2f} ms, compress {self.compress_ms:.2f} ms, "
            f"mean payload {self.len_host.mean() / B:.4f} of {B} B")

    def to_hbm(self, torch, ibp):
        """Compacts the pinned store into a cache in HBM; gathers then read the cache."""
        w = self.w
        N, S = w.n_tensors, w.slot_bytes
        ev = Timer(torch)
        self.offsets = torch.zeros(N + 1, dtype=torch.int64, device="cuda")
        s = ev.start()
        ibp.compact_offsets(self.lengths, N, self.offsets)
        ev.stop(s)
        total = int(self.offsets[-1].item())
        self.cache = torch.empty(max(total, 16), dtype=torch.uint8, device="cuda")
        s = ev.start()
        ibp.compact(self.store, S, N, self.offsets, self.cache, total)
        ev.stop(s)
        self.compact_ms = sum(ev.ms())
        if isinstance(self.store, ibp.HostBuffer):
            self.store.free()
        self.store = self.cache
        self.store_bytes = total
        self.where = "hbm"

    def gather(self, ibp, d_ids, n_ids, out, flags=0):
        w = self.w
        ibp.gather_decompress_ex(self.store, self.store_bytes, w.slot_bytes, self.offsets,
                                 self.part, w.n_tensors, d_ids, n_ids, w.tensor_bytes,
                                 w.chunk_bytes, self.mask, self.bitval, out, flags)


def percentiles_us(ms):
    """mean, min, p10, median, p90, max of launch times given in ms, in us."""
    q = sorted(ms)

    def at(f):
        return q[min(len(q) - 1, int(round(f * (len(q) - 1))))]
    return {"mean": round(statistics.mean(q) * 1e3, 2), "min": round(q[0] * 1e3, 2),
            "p10": round(at(0.1) * 1e3, 2), "median": round(statistics.median(q) * 1e3, 2),
            "p90": round(at(0.9) * 1e3, 2), "max": round(q[-1] * 1e3, 2), "launches": len(q)}


def region_launches(torch, fn, warmup, steps):
    """`steps` launches back to back after `warmup`, bracketed by one pair of
    HIP events on the launch stream and by synchronisations.  Returns (mean ms
    per launch from the events, wall seconds of the region)."""
    for k in range(warmup):
        fn(k)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for k in range(warmup, warmup + steps):
        fn(k)
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return a.elapsed_time(b) / steps, wall


def two_stream_launches(torch, fn, warmup, steps):
    """Launches fn(k) on two streams in turn (default priority), so launch k+1
    can start while launch k drains, as a caller that pipelines its batches
    would run them; the region is bracketed by HIP events on the current
    stream, which the two streams wait on and join.  Returns mean ms per
    launch."""
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    cur = torch.cuda.current_stream()
    for k in range(warmup):
        with torch.cuda.stream(streams[k % 2]):
            fn(k)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(cur)
    for st in streams:
        st.wait_event(a)
    for k in range(warmup, warmup + steps):
        with torch.cuda.stream(streams[k % 2]):
            fn(k)
    for st in streams:
        cur.wait_stream(st)
    b.record(cur)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def graph_launches(torch, fn, k, reps):
    """Launches fn(0..k-1) captured in one HIP graph and replayed `reps` times,
    against the same k launches issued eagerly `reps` times (the same id
    buffers both ways, so caches see the same reuse): mean us per launch."""
    for i in range(k):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(k):
            fn(i)
    g.replay()
    torch.cuda.synchronize()

    def region(body):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            body()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * k)

    def eager():
        for i in range(k):
            fn(i)
    graph_us = region(g.replay)
    eager_us = region(eager)
    del g
    return {"launches": k, "replays": reps, "graph_us_per_launch": round(graph_us, 2),
            "eager_us_per_launch": round(eager_us, 2)}


def time_gather(torch, ibp, table, batches, warmup, steps, out, raw_baseline=False, raw_flags=0,
                flags=0):
    """The timed region (`steps` launches back to back), then the same
    launches again one at a time between their own events.  Returns (wall
    seconds of the region, mean ms per launch in the region, per-launch ms of
    the isolated launches)."""
    w = table.w
    n = w.batch

    def run(k):
        d = batches[k]
        if raw_baseline:
            ibp.raw_gather(table.raw, w.slot_bytes, w.n_tensors, d, n, w.tensor_bytes, out,
                           raw_flags)
        else:
            table.gather(ibp, d, n, out, flags)
    region_ms, wall = region_launches(torch, run, warmup, steps)
    isolated = timed_launches(torch, run, warmup, steps)  # ends on the last batch again
    return wall, region_ms, isolated


def check_rows(table, ids_host, out):
    """The gathered rows are the original rows (lossless), on a sample."""
    import numpy as np
    w = table.w
    got = out.cpu().numpy().view(np.uint8).reshape(-1, w.tensor_bytes)
    view = table.raw.array.reshape(w.n_tensors, w.slot_bytes)[:, :w.tensor_bytes]
    pick = np.linspace(0, len(ids_host) - 1, 64).astype(np.int64)
    if not (got[pick] == view[ids_host[pick]]).all():
        raise SystemExit("bench: gathered rows differ from the original rows")


def probes(torch, ibp, host_flags):
    """Host-link read peak: DMA copy and zero-copy streaming read of 1 GiB."""
    GiB = 1 << 30
    src = torch.empty(GiB, dtype=torch.uint8).pin_memory()
    dst = torch.empty(GiB, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        dst.copy_(src, non_blocking=True)
    tm = Timer(torch)
    for _ in range(10):
        s = tm.start()
        dst.copy_(src, non_blocking=True)
        tm.stop(s)
    dma = GiB / (statistics.median(tm.ms()) * 1e-3) / 1e9
    del src
    hb = ibp.HostBuffer(GiB, host_flags)
    hb.array[:] = 1
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        ibp.stream_read(hb, GiB, 0x9E3779B9, sink)
    tm = Timer(torch)
    for _ in range(10):
        s = tm.start()
        ibp.stream_read(hb, GiB, 0x9E3779B9, sink)
        tm.stop(s)
    zc = GiB / (statistics.median(tm.ms()) * 1e-3) / 1e9
    hb.free()
    # HBM streaming read, 4 GiB (far beyond the 256 MB last-level cache)
    big = torch.ones(4 * GiB, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        ibp.stream_read(big, 4 * GiB, 0x9E3779B9, sink)
    tm = Timer(torch)
    for _ in range(10):
        s = tm.start()
        ibp.stream_read(big, 4 * GiB, 0x9E3779B9, sink)
        tm.stop(s)
    hbm = 4 * GiB / (statistics.median(tm.ms()) * 1e-3) / 1e9
    del big, dst
    torch.cuda.empty_cache()
    # HBM copy, 2 GiB to 2 GiB (reads and writes together, like a gather):
    # bytes read + bytes written per second
    a = torch.ones(2 * GiB, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(2):
        ibp.stream_copy(a, b, 2 * GiB)
    tm = Timer(torch)
    for _ in range(10):
        s = tm.start()
        ibp.stream_copy(a, b, 2 * GiB)
        tm.stop(s)
    copy = 4 * GiB / (statistics.median(tm.ms()) * 1e-3) / 1e9
    if not bool(torch.equal(a[:: 1 << 20], b[:: 1 << 20])):
        raise SystemExit("bench: the copy probe did not copy")
    del a, b
    torch.cuda.empty_cache()
    return {"h2d_dma_GBps": round(dma, 2), "h2d_zero_copy_read_GBps": round(zc, 2),
            "hbm_stream_read_GBps": round(hbm, 1), "hbm_copy_read_plus_write_GBps": round(copy, 1)}


def cpu_baseline(table, batches_host, seconds):
    """The oracle's gather + decompress of the same batches from the same
    (host-resident) store, timed on the host cores; bounded to ~`seconds`."""
    import numpy as np
    from oracle import oracle as O
    w = table.w
    part = table.part.cpu().numpy().view(np.uint32)
    if table.where == "pinned":
        store = table.store.array
        offs = None
    else:
        store = table.cache.cpu().numpy()
        offs = table.offsets.cpu().numpy().view(np.uint64)
    out = np.empty((w.batch, w.tensor_bytes), np.uint8)

    def run(limit):
        rows, k = 0, 0
        t0 = time.perf_counter()
        while True:
            ids = batches_host[k % len(batches_host)]
            O.gather_decompress(store, part, w.n_tensors, ids, w.tensor_bytes, w.chunk_bytes,
                                table.mask_host, table.bitval_host, slot_bytes=w.slot_bytes,
                                offsets=offs, out=out)
            rows += len(ids)
            k += 1
            el = time.perf_counter() - t0
            if el >= limit or k >= 4 * len(batches_host):
                return rows, k, el

    # the oracle's OpenMP runtime: all host threads, then one
    import ctypes
    gomp = ctypes.CDLL("libgomp.so.1")
    threads = gomp.omp_get_max_threads()
    rows, k, el = run(seconds)
    gomp.omp_set_num_threads(1)
    rows1, k1, el1 = run(seconds / 3)
    gomp.omp_set_num_threads(threads)
    return {"value": round(rows * w.tensor_bytes / el / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{k} batches of {w.batch} ids ({rows} rows) of the timed id sequence, "
                      f"{el:.1f} s",
            "value_1_thread": round(rows1 * w.tensor_bytes / el1 / 1e9, 4),
            "sample_1_thread": f"{k1} batches ({rows1} rows), {el1:.1f} s"}


def measure_workload(torch, ibp, W, key, T, where, host_flags, steps, warmup, with_raw):
    import numpy as np
    w = W.WORKLOADS[key]
    T = w.threshold if T is None else T
    table = Table(torch, ibp, W, w, T, where, host_flags, keep_raw=True)
    nb = warmup + steps
    ids_host = [W.batch_ids(w, k) for k in range(nb)]
    batches = [torch.from_numpy(i).cuda() for i in ids_host]
    out = torch.empty(w.batch * w.tensor_bytes, dtype=torch.uint8, device="cuda")
    # batches that repeat ids (Zipf) read from slots: rows routed to XCDs
    route = ibp.GATHER_ROUTE_XCD if (w.id_law == "zipf" and where == "pinned") else 0
    wall, region_ms, ms = time_gather(torch, ibp, table, batches, warmup, steps, out, flags=route)
    check_rows(table, ids_host[-1], out)
    comp = [int(table.len_host[i].sum()) for i in ids_host[warmup:]]
    res = {"table": table, "ids_host": ids_host, "wall": wall, "kernel_ms": region_ms,
           "isolated_ms": ms, "comp_bytes": comp, "T": T, "routed": bool(route)}
    if route:
        _, res["unrouted_kernel_ms"], _ = time_gather(torch, ibp, table, batches, warmup, steps,
                                                      out)
    if with_raw:
        _, rregion, rms = time_gather(torch, ibp, table, batches, warmup, steps, out,
                                      raw_baseline=True)
        res["raw_kernel_ms"] = rregion
        res["raw_isolated_ms"] = rms
        _, rregion, _ = time_gather(torch, ibp, table, batches, warmup, steps, out,
                                    raw_baseline=True, raw_flags=ibp.RAW_ROUTE_XCD)
        res["raw_routed_kernel_ms"] = rregion
    return res


def lines_bytes(lengths):
    """Bytes of the 128 B lines that payloads of these lengths occupy when
    each starts on a line (the cache compacted with 128 B entries)."""
    import numpy as np
    return float(((np.asarray(lengths, np.int64) + 127) // 128 * 128).sum())


def measure_hbm(torch, ibp, W, table, args, pr):
    """The workload's table as compressed caches in HBM, gathered with the
    workload's batch, a 1M-id batch of the same Zipf law and a 1M-id batch of
    distinct ids (uniform, no repeats), against the uncompressed gather of the
    same ids from the rows in HBM.  Two layouts of the same payloads: entries
    on 128 B lines found through the rank index (ibp_gather_decompress_indexed)
    and entries at 16 B found through the offset table (ibp_gather_decompress).
    Bytes per launch, counted without the GPU's caches: the payloads of the
    distinct tensors (in whole 128 B lines), the dense rows written and the
    ids read."""
    import numpy as np
    w = table.w
    key = w.key
    B, C, S, N = w.tensor_bytes, w.chunk_bytes, w.slot_bytes, w.n_tensors
    raw_dev = torch.from_numpy(table.raw.array).cuda()   # uncompressed rows in HBM
    # 128 B entries + rank index, and 16 B entries + offset table
    off128 = torch.zeros(N + 1, dtype=torch.int64, device="cuda")
    ibp.compact_offsets_aligned(table.lengths, N, 128, off128)
    tot128 = int(off128[-1].item())
    cache128 = torch.empty(max(tot128, 16), dtype=torch.uint8, device="cuda")
    tm = Timer(torch)
    s0 = tm.start()
    ibp.cache_fill(table.store, S, table.lengths, N, off128, cache128, tot128)
    index = torch.zeros((N + 31) // 32, dtype=torch.int64, device="cuda")
    ibp.cache_index(table.part, N, index)
    tm.stop(s0)
    del off128
    off16 = torch.zeros(N + 1, dtype=torch.int64, device="cuda")
    ibp.compact_offsets(table.lengths, N, off16)
    tot16 = int(off16[-1].item())
    cache16 = torch.empty(max(tot16, 16), dtype=torch.uint8, device="cuda")
    ibp.compact(table.store, S, N, off16, cache16, tot16)
    torch.cuda.synchronize()
    build_ms = tm.ms()[0]
    res = {"workload": f"{key}: {N} x {B} B, {C} B chunks, T={w.threshold}, Mask from "
                       f"{w.sample_fraction:.0%} of the tensors",
           "cache_128B_entries": {"GB": round(tot128 / 1e9, 3),
                                  "tensors_per_GB_over_raw": round(N * B / tot128, 4),
                                  "fill_and_index_ms": round(build_ms, 2)},
           "cache_16B_entries": {"GB": round(tot16 / 1e9, 3),
                                 "tensors_per_GB_over_raw": round(N * B / tot16, 4)},
           "batches": []}
    rng = np.random.default_rng(20261203)
    perm = rng.permutation(N)
    big = args.hbm_large_batch
    for kind, nb in (("workload batch", w.batch), ("zipf", big), ("distinct", big)):
        steps = max(3, min(args.steps, (64 << 20) // max(1, nb)))
        seqs = []
        for k in range(args.warmup + steps):
            if kind == "distinct":
                o = (k * 40503) % (N - nb + 1)
                seqs.append(perm[o:o + nb].astype(np.int64))
            else:
                nbatches = (nb + w.batch - 1) // w.batch
                seqs.append(np.concatenate([W.batch_ids(w, k * nbatches + i)
                                            for i in range(nbatches)])[:nb])
        d = [torch.from_numpy(i).cuda() for i in seqs]
        out = torch.empty(nb * B, dtype=torch.uint8, device="cuda")

        def run_idx(k):
            ibp.gather_decompress_indexed(cache128, tot128, 128, index, N, d[k], nb, B, C,
                                          table.mask, table.bitval, out)

        def run_idx16(k):
            ibp.gather_decompress_indexed(cache16, tot16, 16, index, N, d[k], nb, B, C,
                                          table.mask, table.bitval, out)

        def run_tab(k):
            ibp.gather_decompress(cache16, tot16, S, off16, table.part, N, d[k], nb, B, C,
                                  table.mask, table.bitval, out)

        def run_raw(k):
            ibp.raw_gather(raw_dev, S, N, d[k], nb, B, out)
        # each launch kind timed twice, alternating, the faster region kept
        # (short launches vary from one region to the next)
        fns = {"idx": run_idx, "idx16": run_idx16, "tab": run_tab, "raw": run_raw}
        best = {k: float("inf") for k in fns}
        for _ in range(2):
            for name, f in fns.items():
                best[name] = min(best[name], region_launches(torch, f, args.warmup, steps)[0])
        km, km16, tm16, rm = best["idx"], best["idx16"], best["tab"], best["raw"]
        last = seqs[-1]
        pick = np.linspace(0, nb - 1, 256).astype(np.int64)
        want = raw_dev.view(N, S)[torch.from_numpy(last[pick]).cuda(), :B].cpu().numpy()
        for f in (run_idx, run_idx16, run_tab):
            out.zero_()
            f(len(seqs) - 1)
            torch.cuda.synchronize()
            got = out.view(nb, B)[torch.from_numpy(pick).cuda()].cpu().numpy()
            if not (got == want).all():
                raise SystemExit(f"bench: {key} HBM gather differs from the original rows")
        uniq = [np.unique(i) for i in seqs[args.warmup:]]
        upay = statistics.mean(lines_bytes(table.len_host[u]) for u in uniq)
        traffic = upay + nb * (B + 8)
        achieved = traffic / (km * 1e-3) / 1e9
        r = {"ids": nb, "id_law": "uniform, no repeats" if kind == "distinct" else
             f"{w.id_law} alpha={w.zipf_alpha}",
             "unique_ids": round(statistics.mean(len(u) for u in uniq), 1),
             "kernel": "k_gather_cache (rank index, 128 B entries)",
             "kernel_us": round(km * 1e3, 2),
             "decompressed_GBps": round(nb * B / (km * 1e-3) / 1e9, 1),
             "raw_hbm_gather_us": round(rm * 1e3, 2),
             "speedup_vs_raw_hbm_gather": round(rm / km, 3),
             "index_16B_entries_us": round(km16 * 1e3, 2),
             "index_16B_speedup_vs_raw": round(rm / km16, 3),
             "table_16B_entries_us": round(tm16 * 1e3, 2),
             "table_16B_speedup_vs_raw": round(rm / tm16, 3),
             "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                          "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                          "bytes_per_launch": round(traffic, 1),
                          "bytes": "distinct tensors' payload lines + rows written + ids",
                          # a ratio to the copy probe's rate (ibp_stream_copy), not a
                          # fraction of a bound
                          "over_measured_device_copy": round(
                              achieved / pr["hbm_copy_read_plus_write_GBps"], 4)}}
        if kind == "workload batch":
            r["hip_graph"] = graph_launches(torch, run_idx, min(16, len(d)), max(3, steps // 4))
        else:
            r["counter_hbm_bytes_read_written"] = profiled_hbm_bytes(key, kind)
        res["batches"].append(r)
        log(f"{key} HBM {kind}: {r}")
        del out, d
    del raw_dev, cache128, cache16, off16, index
    torch.cuda.empty_cache()
    return res


def measure_pinned(torch, ibp, W, key, flags, args, pr):
    """A workload's batches from its pinned-host store, with the raw
    GPU gather of the same rows from pinned memory beside it.  Returns the
    result and the table (still pinned)."""
    w = W.WORKLOADS[key]
    m = measure_workload(torch, ibp, W, key, None, "pinned", flags, args.steps, args.warmup,
                         with_raw=True)
    import numpy as np
    table = m["table"]
    comp = statistics.mean(m["comp_bytes"])
    # bytes of the distinct tensors of a batch: repeated ids are read from
    # the GPU's caches, not over the link, so this is the link-side count
    uniq = statistics.mean(float(table.len_host[np.unique(i)].sum())
                           for i in m["ids_host"][args.warmup:])
    # the same tensors in the whole 128 B lines that cross the link (slots
    # start on a line; a payload of len bytes is read as ceil(len / 128) lines)
    uniq_lines = statistics.mean(lines_bytes(table.len_host[np.unique(i)])
                                 for i in m["ids_host"][args.warmup:])
    link = max(pr["h2d_dma_GBps"], pr["h2d_zero_copy_read_GBps"])
    km, rm = m["kernel_ms"], m["raw_kernel_ms"]
    achieved = comp / (km * 1e-3) / 1e9
    achieved_u = uniq / (km * 1e-3) / 1e9
    res = {"workload": f"{key}: {w.n_tensors} x {w.tensor_bytes} B, {w.chunk_bytes} B chunks, "
                       f"T={w.threshold}, {w.batch} {w.id_law} ids per launch",
           "kernel_us": round(km * 1e3, 2),
           "decompressed_GBps": round(w.batch * w.tensor_bytes / (km * 1e-3) / 1e9, 2),
           "payload_all_ids_GBps": round(achieved, 2),
           "unique_ids": round(statistics.mean(len(np.unique(i)) for i in m["ids_host"][args.warmup:]), 1),
           "unique_payload_GBps_over_link": round(achieved_u, 2),
           "unique_frac_of_measured": round(achieved_u / link, 4),
           "unique_frac_of_zero_copy_read": round(achieved_u / pr["h2d_zero_copy_read_GBps"], 4),
           "unique_line_frac_of_measured": round(uniq_lines / (km * 1e-3) / 1e9 / link, 4),
           "batch_payload_over_dense": round(comp / (w.batch * w.tensor_bytes), 5),
           "raw_gather_us": round(rm * 1e3, 2),
           "transfer_speedup_vs_raw_gpu_gather": round(rm / km, 3),
           "raw_gather_xcd_routed_us": round(m["raw_routed_kernel_ms"] * 1e3, 2),
           "transfer_speedup_vs_raw_xcd_routed": round(m["raw_routed_kernel_ms"] / km, 3),
           "xcd_routed": m["routed"]}
    if m["routed"]:
        res["kernel_us_unrouted"] = round(m["unrouted_kernel_ms"] * 1e3, 2)
    # 16 batches in one launch: the launch's fixed cost (ramp and drain) spread
    # over 16 times the bytes; link bytes = the distinct tensors of all 16
    ids16 = [np.concatenate(m["ids_host"][16 * k:16 * k + 16])
             for k in range(max(1, len(m["ids_host"]) // 16))]
    nb16 = min(len(i) for i in ids16)
    d16 = [torch.from_numpy(i[:nb16]).cuda() for i in ids16]
    out16 = torch.empty(nb16 * w.tensor_bytes, dtype=torch.uint8, device="cuda")
    flags16 = ibp.GATHER_ROUTE_XCD if m["routed"] else 0
    ms16, _ = region_launches(torch, lambda k: table.gather(ibp, d16[k % len(d16)], nb16, out16,
                                                            flags16), 2, 6)
    u16 = statistics.mean(float(table.len_host[np.unique(i[:nb16])].sum()) for i in ids16)
    l16 = statistics.mean(lines_bytes(table.len_host[np.unique(i[:nb16])]) for i in ids16)
    res["one_launch_16_batches"] = {
        "ids": nb16, "kernel_us": round(ms16 * 1e3, 2),
        "unique_payload_GBps_over_link": round(u16 / (ms16 * 1e-3) / 1e9, 2),
        "unique_frac_of_measured": round(u16 / (ms16 * 1e-3) / 1e9 / link, 4),
        "unique_line_frac_of_measured": round(l16 / (ms16 * 1e-3) / 1e9 / link, 4)}
    del out16, d16
    log(f"{key} pinned: {res}")
    return res, table


def measure_multi_table(torch, ibp, W, table, args, pr, n_tables=8):
    """Embedding lookups in several tables at once ([JH] DLRM paragraph): the
    workload's tensors split into n_tables tables of equal size, one Zipf batch
    per table (the workload's batch size and law over that table), gathered in
    one ibp_gather_decompress_segments launch (one segment per table, each
    with its Mask) against one ibp_gather_decompress launch per table, each
    way with and without XCD routing.  The
    tables here share the workload's Mask, which changes no timing."""
    import numpy as np
    w = table.w
    B, S, N = w.tensor_bytes, w.slot_bytes, w.n_tensors
    per = N // n_tables
    wt = w.scaled(per)
    steps = max(3, min(args.steps, 20))
    sets = []
    for k in range(args.warmup + steps):
        ids = [W.batch_ids(wt, k * n_tables + t) + t * per for t in range(n_tables)]
        sets.append(ids)
    d_all = [torch.from_numpy(np.concatenate(ids)).cuda() for ids in sets]
    d_each = [[torch.from_numpy(i).cuda() for i in ids] for ids in sets]
    nb = [len(i) for i in sets[0]]
    seg = np.concatenate([[0], np.cumsum(nb)]).astype(np.uint64)
    n_all = int(seg[-1])
    masks = table.mask.repeat(n_tables)
    bitvals = table.bitval.repeat(n_tables)
    out = torch.empty(n_all * B, dtype=torch.uint8, device="cuda")

    def one(k, flags=0):
        ibp.gather_decompress_segments(table.store, table.store_bytes, S, table.offsets, table.part,
                                       N, d_all[k], seg, B, w.chunk_bytes, masks, bitvals, out,
                                       flags)

    def one_routed(k):
        one(k, ibp.GATHER_ROUTE_XCD)

    def separate(k):
        for t in range(n_tables):
            ibp.gather_decompress(table.store, table.store_bytes, S, table.offsets, table.part, N,
                                  d_each[k][t], nb[t], B, w.chunk_bytes, table.mask, table.bitval,
                                  out[int(seg[t]) * B:])
    def separate_routed(k):
        for t in range(n_tables):
            ibp.gather_decompress_ex(table.store, table.store_bytes, S, table.offsets, table.part,
                                     N, d_each[k][t], nb[t], B, w.chunk_bytes, table.mask,
                                     table.bitval, out[int(seg[t]) * B:], ibp.GATHER_ROUTE_XCD)
    one_ms, _ = region_launches(torch, one, args.warmup, steps)
    oner_ms, _ = region_launches(torch, one_routed, args.warmup, steps)
    sep_ms, _ = region_launches(torch, separate, args.warmup, steps)
    sepr_ms, _ = region_launches(torch, separate_routed, args.warmup, steps)
    ids_last = np.concatenate(sets[-1])
    pick = np.linspace(0, n_all - 1, 128).astype(np.int64)
    want = table.raw.array.reshape(N, S)[ids_last[pick], :B]
    for f in (one, one_routed):
        out.zero_()
        f(len(sets) - 1)
        torch.cuda.synchronize()
        got = out.view(n_all, B)[torch.from_numpy(pick).cuda()].cpu().numpy()
        if not (got == want).all():
            raise SystemExit("bench: the multi-table gather differs from the original rows")
    del out, d_all, d_each
    # link-side bytes: each distinct tensor of a table's batch once (repeats
    # are served from the GPU's caches), as for the single-table launches
    uniq = statistics.mean(sum(float(table.len_host[np.unique(i)].sum()) for i in ids)
                           for ids in sets[args.warmup:])
    link = max(pr["h2d_dma_GBps"], pr["h2d_zero_copy_read_GBps"])
    return {"tables": n_tables, "rows_per_table": per, "ids_per_table": nb[0],
            "unique_bytes_per_launch": round(uniq, 1),
            "one_launch_routed_unique_frac_of_measured": round(uniq / (oner_ms * 1e-3) / 1e9 /
                                                               link, 4),
            "one_launch_us": round(one_ms * 1e3, 2),
            "one_launch_routed_us": round(oner_ms * 1e3, 2),
            "separate_launches_us": round(sep_ms * 1e3, 2),
            "speedup_one_launch": round(sep_ms / one_ms, 3),
            "separate_routed_launches_us": round(sepr_ms * 1e3, 2),
            "speedup_one_launch_routed": round(sepr_ms / oner_ms, 3)}


def measure_hybrid(torch, ibp, table, batches, ids_host, args, budget_fraction):
    """Cache + store in one launch at a fixed HBM budget: compressed tensors
    against uncompressed ones (the same kernel with Mask = 0 over the raw
    rows, whose payloads are the rows themselves)."""
    import numpy as np
    w = table.w
    N, B, C, S = w.n_tensors, w.tensor_bytes, w.chunk_bytes, w.slot_bytes
    budget = int(budget_fraction * N * B)
    order = np.random.default_rng(7).permutation(N)
    zero_words = torch.zeros(B // 4, dtype=torch.int32, device="cuda")
    n_c = ibp.num_chunks(B, C)
    zero_bits = torch.zeros((N * n_c + 31) // 32, dtype=torch.int32, device="cuda")
    raw_len = torch.full((N,), B, dtype=torch.int32, device="cuda")
    out = torch.empty(w.batch * B, dtype=torch.uint8, device="cuda")
    res = {"hbm_budget_GB": round(budget / 1e9, 3), "ids": w.batch}
    for name, store, lengths, len_host, mask, bitval, bits in (
            ("compressed", table.store, table.lengths, table.len_host, table.mask, table.bitval,
             table.part),
            ("uncompressed", table.raw, raw_len, np.full(N, B, np.uint32), zero_words,
             zero_words, zero_bits)):
        pad = (len_host[order].astype(np.int64) + 15) // 16 * 16
        k = int(np.searchsorted(np.cumsum(pad), budget, side="right"))
        select = np.zeros(N, np.uint32)
        select[order[:k]] = 1
        offsets = torch.zeros(N + 1, dtype=torch.int64, device="cuda")
        ibp.cache_offsets(lengths, torch.from_numpy(select).cuda(), N, offsets)
        total = int(offsets[-1].item())
        cache = torch.empty(max(total, 16), dtype=torch.uint8, device="cuda")
        ibp.cache_fill(store, S, lengths, N, offsets, cache, total)

        def run(i):
            ibp.gather_decompress_hybrid(store, N * S, S, cache, total, offsets, bits, N,
                                         batches[i], w.batch, B, C, mask, bitval, out)
        ms, _ = region_launches(torch, run, args.warmup, args.steps)
        run(len(batches) - 1)
        torch.cuda.synchronize()
        got = out.view(w.batch, B)[:64].cpu().numpy()
        want = table.raw.array.reshape(N, S)[ids_host[-1][:64], :B]
        if not (got == want).all():
            raise SystemExit(f"bench: hybrid gather ({name}) differs from the original rows")
        hits = float(np.mean([select[i].mean() for i in ids_host[args.warmup:]]))
        res[name] = {"cached_tensors": k, "hit_rate": round(hits, 4),
                     "kernel_us": round(ms * 1e3, 2),
                     "decompressed_GBps": round(w.batch * B / (ms * 1e-3) / 1e9, 1)}
        del cache, offsets
    res["speedup"] = round(res["uncompressed"]["kernel_us"] / res["compressed"]["kernel_us"], 3)
    del zero_words, zero_bits, raw_len, out
    torch.cuda.empty_cache()
    return res


def timed_launches(torch, fn, warmup, steps):
    """HIP-event duration (ms) of each of `steps` launches after `warmup`."""
    for k in range(warmup):
        fn(k)
    torch.cuda.synchronize()
    tm = Timer(torch)
    for k in range(warmup, warmup + steps):
        s = tm.start()
        fn(k)
        tm.stop(s)
    return tm.ms()


# ---------------------------------------------------------------- other modes

def hip_runtime():
    """torch's HIP runtime (already loaded), for plain hipMemcpyAsync calls."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipMemcpyAsync.restype = ctypes.c_int
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                   ctypes.c_void_p]
    return hip


def run_ablation(torch, ibp, args, pr, pool_bytes=4 << 30):
    """Copy throughput of small random tensors from pinned host memory to the
    GPU by transfer method ([JH] Figure 5 and aligned-copy paragraphs):
    per-tensor DMA issued by the CPU, a CPU gather into a staging buffer
    followed by one DMA, GPU zero-copy reads of packed rows (4 B loads, rows
    at any 4 B offset) and GPU zero-copy reads of 128 B-aligned rows (16 B
    loads)."""
    import concurrent.futures as cf
    import numpy as np
    hip = hip_runtime()
    H2D = 1
    hb = ibp.HostBuffer(pool_bytes + 4096)
    rng = np.random.default_rng(5)
    view64 = hb.array[:(pool_bytes // 8) * 8].view(np.uint64)
    for i in range(0, view64.size, 1 << 24):
        view64[i:i + (1 << 24)] = rng.integers(0, 1 << 63, min(1 << 24, view64.size - i),
                                               dtype=np.uint64)
    n = 8192
    stream = torch.cuda.current_stream().cuda_stream
    threads = min(16, os.cpu_count() or 1)
    rows = []
    for size in (64, 256, 1024, 4096, 16384):
        S = (size + 127) // 128 * 128
        n_al = pool_bytes // S
        n_pk = (pool_bytes - 4) // size
        ids = rng.integers(0, min(n_al, n_pk), n)
        d_ids = torch.from_numpy(ids).cuda()
        out = torch.empty(n * size, dtype=torch.uint8, device="cuda")
        r = {"tensor_bytes": size}
        # GPU zero-copy, 128 B-aligned rows, 16 B loads
        ms, _ = region_launches(torch, lambda k: ibp.raw_gather(hb, S, n_al, d_ids, n, size, out),
                                3, 20)
        r["gpu_aligned_GBps"] = round(n * size / (ms * 1e-3) / 1e9, 2)
        # GPU zero-copy, packed rows at a 4 B offset, 4 B loads
        ms, _ = region_launches(torch, lambda k: ibp.raw_gather(hb.ptr + 4, size, n_pk, d_ids, n,
                                                                size, out), 3, 20)
        r["gpu_unaligned_GBps"] = round(n * size / (ms * 1e-3) / 1e9, 2)
        # CPU gather into pinned staging (all host threads) + one DMA
        staging = ibp.HostBuffer(n * size)
        stage = staging.array.reshape(n, size)
        src = hb.array[:n_al * S].reshape(n_al, S)

        def cpu_gather(chunk):
            lo, hi = chunk
            stage[lo:hi] = src[ids[lo:hi], :size]
        chunks = [(i, min(n, i + n // threads + 1)) for i in range(0, n, n // threads + 1)]
        best = float("inf")
        with cf.ThreadPoolExecutor(threads) as ex:
            for _ in range(5):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                list(ex.map(cpu_gather, chunks))
                hip.hipMemcpyAsync(out.data_ptr(), staging.ptr, n * size, H2D, stream)
                torch.cuda.synchronize()
                best = min(best, time.perf_counter() - t0)
        r["cpu_bulk_GBps"] = round(n * size / best / 1e9, 2)
        staging.free()
        # one DMA per tensor, issued by the CPU (a bounded number of rows)
        m = 1024
        best = float("inf")
        for _ in range(3):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(m):
                hip.hipMemcpyAsync(out.data_ptr() + i * size, hb.ptr + int(ids[i]) * S, size, H2D,
                                   stream)
            torch.cuda.synchronize()
            best = min(best, time.perf_counter() - t0)
        r["cpu_fine_GBps"] = round(m * size / best / 1e9, 3)
        r["aligned_over_unaligned"] = round(r["gpu_aligned_GBps"] / r["gpu_unaligned_GBps"], 3)
        rows.append(r)
        log(f"ablation {r}")
        del out, d_ids
    hb.free()
    return {"metric": "CPU-to-GPU copy throughput of 8,192 random tensors by transfer method",
            "unit": "GB/s", "higher_is_better": True, "pool_GiB": pool_bytes / (1 << 30),
            "limit": {"pcie5_x16_GBps": PCIE5_X16_GBPS, **pr}, "results": rows,
            "host_threads": threads}


def run_sweep(torch, ibp, args, pr):
    """Decompression throughput against space saving and chunk size ([G-EN]
    Results and [JH] Figure 7 paragraph: above 95 % of the ideal rate below
    50 % saving, for 256 B, 1 KB and 4 KB chunks), on synthetic 4 KB tensors
    whose words keep k random low bits under 32-k fixed high bits, so the
    saving is (32-k)/32; plus a stream of BF16 weight tensors."""
    import numpy as np
    rng = np.random.default_rng(11)
    N, B, n = 65536, 4096, 8192
    S = B
    link = max(pr["h2d_dma_GBps"], pr["h2d_zero_copy_read_GBps"])
    raw = ibp.HostBuffer(N * S)
    store = ibp.HostBuffer(N * S)
    out = torch.empty(n * B, dtype=torch.uint8, device="cuda")
    ids = rng.integers(0, N, n)
    d_ids = torch.from_numpy(ids).cuda()
    counts = torch.zeros(8 * B, dtype=torch.int32, device="cuda")
    mask = torch.zeros(B // 4, dtype=torch.int32, device="cuda")
    bitval = torch.zeros_like(mask)
    results = []

    def measure(label, C, extra):
        n_c = ibp.num_chunks(B, C)
        part = torch.zeros((N * n_c + 31) // 32, dtype=torch.int32, device="cuda")
        lengths = torch.zeros(N, dtype=torch.int32, device="cuda")
        ibp.build_metadata(raw, S, None, N, B, 0.99, mask, bitval, counts)
        ibp.compress(raw, S, N, 0, N, B, C, mask, bitval, store, S, part, lengths)
        ms, _ = region_launches(
            torch, lambda k: ibp.gather_decompress(store, N * S, S, None, part, N, d_ids, n, B, C,
                                                   mask, bitval, out), 3, 20)
        got = out.view(n, B)[:16].cpu().numpy()
        if not (got == raw.array.reshape(N, S)[ids[:16]]).all():
            raise SystemExit("bench: sweep gather is not lossless")
        L = lengths.cpu().numpy().astype(np.float64)
        ratio = float(L[ids].mean()) / B
        dec = n * B / (ms * 1e-3) / 1e9
        ideal = link / ratio
        r = {"case": label, "chunk_bytes": C, "saving": round(1 - ratio, 4),
             "kernel_us": round(ms * 1e3, 2), "decompressed_GBps": round(dec, 1),
             "ideal_GBps": round(ideal, 1), "frac_of_ideal": round(dec / ideal, 4), **extra}
        results.append(r)
        log(f"sweep {r}")

    words = raw.array.reshape(N, S).view(np.uint32)
    for k in (32, 28, 24, 20, 16, 12, 8, 4, 3):
        hi = rng.integers(0, 1 << 32, B // 4, dtype=np.uint64).astype(np.uint32)
        low = (1 << k) - 1
        for i in range(0, N, 8192):
            r = rng.integers(0, 1 << 32, (min(8192, N - i), B // 4), dtype=np.uint64)
            words[i:i + 8192] = (r.astype(np.uint32) & np.uint32(low)) | (hi & np.uint32(~low & 0xFFFFFFFF))
        for C in (256, 1024, 4096):
            measure(f"kept {k} of 32 bits", C, {"kept_bits": k})
    raw.free()
    store.free()
    return {"metric": "decompressed GB/s against space saving (pinned host store)",
            "unit": "GB/s", "higher_is_better": True, "link_peak_GBps": link,
            "ids": n, "tensors": N, "tensor_bytes": B, "results": results}


def bf16_rne(x):
    """bfloat16 encodings (uint16) of float32 values, rounded to nearest even."""
    import numpy as np
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def run_weight_stream(torch, ibp, args, pr):
    """BF16 weight offloading ([G-EN] Results: BF16 weights offloaded to CPU
    memory compress by up to 27 % and cut latency by 22 %): the weight matrices
    of one OPT-13B decoder layer (hidden 5,120, MLP 20,480: four 5,120 x 5,120
    attention matrices and two 5,120 x 20,480 MLP matrices, 314.6 M bf16
    values, 629 MB) held in pinned host memory as 10,240 B rows (5,120 bf16;
    an MLP row of 20,480 values is four such rows), values N(0, s^2) with
    s = 0.02 (attention) and 0.014 (MLP), Mask from a 1 % sample of the rows,
    256 B chunks.  A step fetches the whole layer in row order (a contiguous
    stream) in one gather + decompress launch, against one DMA of the raw
    weights and the raw GPU gather of the same rows."""
    import numpy as np
    B, C = 10240, 256
    H, F = 5120, 20480
    n_attn = 4 * H * H // (B // 2)           # 20,480 rows
    n_mlp = 2 * H * F // (B // 2)            # 40,960 rows
    N = n_attn + n_mlp
    S = B
    rng = np.random.default_rng(13)
    raw = ibp.HostBuffer(N * S)
    rows = raw.array.reshape(N, S).view(np.uint16)
    blk = 2048
    for i in range(0, N, blk):
        k = min(blk, N - i)
        sd = 0.02 if i < n_attn else 0.014
        rows[i:i + k] = bf16_rne(rng.standard_normal((k, B // 2), dtype=np.float32) * sd)
    sample = np.sort(rng.choice(N, N // 100, replace=False)).astype(np.int64)
    mask = torch.zeros(B // 4, dtype=torch.int32, device="cuda")
    bitval = torch.zeros_like(mask)
    counts = torch.zeros(8 * B, dtype=torch.int32, device="cuda")
    ibp.build_metadata(raw, S, torch.from_numpy(sample).cuda(), len(sample), B, 0.99, mask,
                       bitval, counts)
    store = ibp.HostBuffer(N * S)
    n_c = ibp.num_chunks(B, C)
    part = torch.zeros((N * n_c + 31) // 32, dtype=torch.int32, device="cuda")
    lengths = torch.zeros(N, dtype=torch.int32, device="cuda")
    ibp.compress(raw, S, N, 0, N, B, C, mask, bitval, store, S, part, lengths)
    ids = torch.arange(N, dtype=torch.int64, device="cuda")
    out = torch.empty(N * B, dtype=torch.uint8, device="cuda")
    steps = max(3, min(args.steps, 10))
    km, _ = region_launches(torch, lambda k: ibp.gather_decompress(
        store, N * S, S, None, part, N, ids, N, B, C, mask, bitval, out), 2, steps)
    pick = np.linspace(0, N - 1, 97).astype(np.int64)
    got = out.view(N, B)[torch.from_numpy(pick).cuda()].cpu().numpy()
    if not (got == raw.array.reshape(N, S)[pick]).all():
        raise SystemExit("bench: the weight stream is not lossless")
    rm, _ = region_launches(torch, lambda k: ibp.raw_gather(raw, S, N, ids, N, B, out), 2, steps)
    hip = hip_runtime()
    stream = torch.cuda.current_stream().cuda_stream
    dm, _ = region_launches(torch, lambda k: hip.hipMemcpyAsync(out.data_ptr(), raw.ptr, N * B, 1,
                                                                stream), 2, steps)
    L = lengths.cpu().numpy().view(np.uint32).astype(np.float64)
    comp = float(L.sum())
    link = max(pr["h2d_dma_GBps"], pr["h2d_zero_copy_read_GBps"])
    res = {"workload": f"OPT-13B decoder layer weights, bf16, {N} rows x {B} B ({N * B / 1e6:.0f} MB), "
                       f"{C} B chunks, T=0.99, Mask from 1 % of the rows, pinned host",
           "saving": round(1 - comp / (N * B), 4),
           "kernel_ms": round(km, 3), "dma_ms": round(dm, 3), "raw_gather_ms": round(rm, 3),
           "latency_cut_vs_dma": round(1 - km / dm, 4),
           "speedup_vs_dma": round(dm / km, 3), "speedup_vs_raw_gather": round(rm / km, 3),
           "decompressed_GBps": round(N * B / (km * 1e-3) / 1e9, 1),
           "payload_GBps_over_link": round(comp / (km * 1e-3) / 1e9, 2),
           "frac_of_measured_link": round(comp / (km * 1e-3) / 1e9 / link, 4)}
    raw.free()
    store.free()
    del out, ids
    torch.cuda.empty_cache()
    log(f"weight stream: {res}")
    return res


def measure_sampling(torch, ibp, table, fractions=(0.01, 0.05, 0.10, 1.0)):
    """Mask/Bitval from samples of 1 %, 5 % and 10 % of the tensors against all
    of them ([JH] sampling paragraph: compression ratios from such samples
    stay close to those of the full data): for each, the Mask words that
    differ from the full-data Mask and the mean payload of the whole table
    compressed with it."""
    import numpy as np
    w = table.w
    B, C, S, N = w.tensor_bytes, w.chunk_bytes, w.slot_bytes, w.n_tensors
    rng = np.random.default_rng(31)
    n_c = ibp.num_chunks(B, C)
    part = torch.zeros((N * n_c + 31) // 32, dtype=torch.int32, device="cuda")
    lengths = torch.zeros(N, dtype=torch.int32, device="cuda")
    store = torch.empty(N * S, dtype=torch.uint8, device="cuda")
    counts = torch.zeros(8 * B, dtype=torch.int32, device="cuda")
    out = []
    masks = {}
    for f in sorted(fractions, reverse=True):
        n = max(1, int(round(f * N)))
        sid = None if n == N else torch.from_numpy(
            np.sort(rng.choice(N, n, replace=False)).astype(np.int64)).cuda()
        m = torch.zeros(B // 4, dtype=torch.int32, device="cuda")
        v = torch.zeros_like(m)
        ibp.build_metadata(table.raw, S, sid, n, B, w.threshold, m, v, counts)
        ibp.compress(table.raw, S, N, 0, N, B, C, m, v, store, S, part, lengths)
        L = lengths.cpu().numpy().view(np.uint32).astype(np.float64)
        masks[f] = m.cpu().numpy().view(np.uint32)
        out.append({"sample": f, "rows": n,
                    "mask_words_differing_from_full": int((masks[f] != masks[1.0]).sum()),
                    "mean_payload_over_tensor": round(float(L.mean()) / B, 5)})
    del store, part, lengths
    torch.cuda.empty_cache()
    full = out[0]["mean_payload_over_tensor"]
    for r in out:
        r["payload_over_full_data_payload"] = round(r["mean_payload_over_tensor"] / full, 5)
    return {"workload": w.key, "T": w.threshold, "results": sorted(out, key=lambda r: r["sample"])}


def run_kv_step(torch, ibp, W, args, pr, pairs=None):
    """The online K/V path on OPT-13B shapes ([JH] LLM paragraph): Mask and
    Bitval of each (layer, K|V) pair from its own prefill K/V (38,400 rows),
    compress-on-write of each decode token's 20 rows into the pinned store, and
    the decode step's fetch: one gather + decompress launch of 2,560 rows per
    pair, 80 launches, against an uncompressed GPU gather of the same rows."""
    import numpy as np
    w = W.WORKLOADS["kv_opt13b"]
    P = max(1, min(W.KV_PAIRS, args.kv_pairs if pairs is None else pairs))
    R = W.KV_ROWS_PER_PAIR
    N, B, C, S = P * R, w.tensor_bytes, w.chunk_bytes, w.slot_bytes
    n_c = ibp.num_chunks(B, C)
    raw = ibp.HostBuffer(N * S)
    W.rows(w, 0, N, out=raw.array.reshape(N, S)[:, :B])
    store = ibp.HostBuffer(N * S)
    part = torch.zeros((N * n_c + 31) // 32, dtype=torch.int32, device="cuda")
    lengths = torch.zeros(N, dtype=torch.int32, device="cuda")
    counts = torch.zeros(8 * B, dtype=torch.int32, device="cuda")
    masks, meta_ms = [], []
    for p in range(P):
        pre = torch.from_numpy(W.kv_prefill_rows(w, p)).cuda()
        m = torch.zeros(B // 4, dtype=torch.int32, device="cuda")
        v = torch.zeros_like(m)
        ms = timed_launches(torch, lambda k: ibp.build_metadata(pre, B, None, pre.shape[0], B,
                                                                w.threshold, m, v, counts), 1, 3)
        meta_ms.append(statistics.median(ms))
        masks.append((m, v))
        del pre
        if p % 10 == 9:
            log(f"kv-step: Mask/Bitval of {p + 1} pairs")
    # compress-on-write: token j of every sequence, per pair (rows of a pair
    # are stored token-major so one token's 20 rows are contiguous)
    tok = W.KV_SEQS
    tm = Timer(torch)
    for j in range(W.KV_DECODE):
        s0 = tm.start()
        for p in range(P):
            first = p * R + j * tok
            ibp.compress(raw.ptr + first * S, S, tok, first, N, B, C, masks[p][0], masks[p][1],
                         store, S, part, lengths)
        tm.stop(s0)
    write_ms = tm.ms()
    # the same compress-on-write with one launch per token: one segment per pair
    masks_all = torch.cat([mv[0] for mv in masks])
    bitvals_all = torch.cat([mv[1] for mv in masks])
    tm = Timer(torch)
    for j in range(W.KV_DECODE):
        firsts = [p * R + j * tok for p in range(P)]
        s0 = tm.start()
        ibp.compress_segments(raw.ptr, S, firsts, firsts, [tok] * P, N, B, C, masks_all,
                              bitvals_all, store, S, part, lengths)
        tm.stop(s0)
    write_seg_ms = tm.ms()
    L = lengths.cpu().numpy()
    out = torch.empty(R * B, dtype=torch.uint8, device="cuda")
    d_ids = [torch.arange(p * R, (p + 1) * R, dtype=torch.int64, device="cuda") for p in range(P)]

    def step_ibp(k):
        for p in range(P):
            ibp.gather_decompress(store, N * S, S, None, part, N, d_ids[p], R, B, C, masks[p][0],
                                  masks[p][1], out)

    def step_raw(k):
        for p in range(P):
            ibp.raw_gather(raw, S, N, d_ids[p], R, B, out)
    steps = max(3, min(args.steps, 20))
    ibp_ms, _ = region_launches(torch, step_ibp, 2, steps)
    raw_ms, _ = region_launches(torch, step_raw, 2, steps)
    # the whole step in one launch: one segment per pair, each with its Mask
    d_all = torch.arange(N, dtype=torch.int64, device="cuda")
    seg = [p * R for p in range(P + 1)]
    out_all = torch.empty(N * B, dtype=torch.uint8, device="cuda")

    def step_seg(k):
        ibp.gather_decompress_segments(store, N * S, S, None, part, N, d_all, seg, B, C, masks_all,
                                       bitvals_all, out_all)
    seg_ms, _ = region_launches(torch, step_seg, 2, steps)
    torch.cuda.synchronize()
    pick = np.linspace(0, N - 1, 257).astype(np.int64)
    if not (out_all.view(N, B)[torch.from_numpy(pick).cuda()].cpu().numpy() ==
            raw.array.reshape(N, S)[pick, :B]).all():
        raise SystemExit("bench: the segmented K/V step is not lossless")
    del out_all, d_all
    step_ibp(0)
    torch.cuda.synchronize()
    if not (out.view(R, B)[:32].cpu().numpy() == raw.array.reshape(N, S)[(P - 1) * R:
                                                                         (P - 1) * R + 32, :B]).all():
        raise SystemExit("bench: kv-step gather is not lossless")
    dense = P * R * B
    comp = float(L.astype(np.float64).sum())
    link = max(pr["h2d_dma_GBps"], pr["h2d_zero_copy_read_GBps"])
    res = {"metric": f"OPT-13B K/V decode-step fetch (gather + decompress, {P} launches)",
           "workload": f"kv_opt13b: {P} (layer, K|V) pairs x {R} rows x {B} B, {C} B chunks, "
                       f"T={w.threshold}, Mask per pair from its {W.KV_PREFILL_ROWS} prefill rows",
           "unit": "GB/s", "higher_is_better": True, "pairs": P,
           "rows_per_launch": R, "tensor_bytes": B, "chunk_bytes": C,
           "mean_payload_over_tensor": round(comp / (N * B), 5),
           "step_ms": round(ibp_ms, 3), "decompressed_GBps": round(dense / (ibp_ms * 1e-3) / 1e9, 2),
           "compressed_GBps_over_link": round(comp / (ibp_ms * 1e-3) / 1e9, 2),
           "frac_of_link_peak": round(comp / (ibp_ms * 1e-3) / 1e9 / link, 4),
           "raw_step_ms": round(raw_ms, 3), "speedup_vs_raw": round(raw_ms / ibp_ms, 3),
           "one_launch_step_ms": round(seg_ms, 3),
           "one_launch_frac_of_link_peak": round(comp / (seg_ms * 1e-3) / 1e9 / link, 4),
           "one_launch_speedup_vs_raw": round(raw_ms / seg_ms, 3),
           "prefill_mask_ms_per_pair": round(statistics.mean(meta_ms), 3),
           "prefill_mask_ms_all_pairs": round(sum(meta_ms), 2),
           "prefill_mask_over_decode_fetch": round(sum(meta_ms) / (W.KV_DECODE * ibp_ms), 4),
           "prefill_rows_per_pair": W.KV_PREFILL_ROWS,
           "compress_on_write_us_per_token": round(statistics.median(write_ms) * 1e3, 1),
           "compress_on_write_one_launch_us_per_token": round(statistics.median(write_seg_ms) * 1e3,
                                                              1),
           "device": torch.cuda.get_device_name(0)}
    raw.free()
    store.free()
    return res


def run_configs(torch, ibp, W, args, pr):
    """One row per workload: space saving, the oracle on one thread and on all
    host threads, the GPU gather from pinned memory (against the link) and,
    for the cache workloads, from a compacted HBM cache (against 8 TB/s)."""
    import numpy as np
    from oracle import oracle as O
    link = max(pr["h2d_dma_GBps"], pr["h2d_zero_copy_read_GBps"])
    steps, warmup = max(5, min(args.steps, 30)), max(2, min(args.warmup, 5))
    rows_out = []
    for key in ("tiny", "sparse_gnn", "dense_gnn", "dlrm_1k", "dlrm_2k"):
        w = W.WORKLOADS[key]
        m = measure_workload(torch, ibp, W, key, None, "pinned", args.host_flags_value, steps,
                             warmup, with_raw=False)
        t = m["table"]
        B = w.tensor_bytes
        km = m["kernel_ms"]
        comp = statistics.mean(m["comp_bytes"])
        uniq = statistics.mean(float(t.len_host[np.unique(i)].sum()) for i in m["ids_host"][warmup:])
        cpu = cpu_baseline(t, m["ids_host"][warmup:], 3.0)
        r = {"config": key, "tensor_bytes": B, "batch": w.batch,
             "space_saving": round(1.0 - float(t.len_host.mean()) / B, 4),
             "oracle_1_thread_GBps": cpu["value_1_thread"], "oracle_all_GBps": cpu["value"],
             "oracle_threads": cpu["cores"],
             "gpu_pinned_GBps": round(w.batch * B / (km * 1e-3) / 1e9, 2),
             "pcie_frac_all_ids": round(comp / (km * 1e-3) / 1e9 / link, 4),
             "pcie_frac_unique": round(uniq / (km * 1e-3) / 1e9 / link, 4),
             "xcd_routed": m["routed"]}
        if key in ("tiny", "dense_gnn", "dlrm_1k"):
            t.to_hbm(torch, ibp)
            for nb, tag in ((w.batch, ""), (args.hbm_large_batch, "_1M_ids")):
                if tag and key == "tiny":
                    continue
                nbatches = (nb + w.batch - 1) // w.batch
                n_seq = warmup + steps
                seqs = [np.concatenate([W.batch_ids(w, k * nbatches + i)
                                        for i in range(nbatches)])[:nb] for k in range(n_seq)]
                d = [torch.from_numpy(i).cuda() for i in seqs]
                out = torch.empty(nb * B, dtype=torch.uint8, device="cuda")
                hm, _ = region_launches(torch, lambda k: t.gather(ibp, d[k], nb, out), warmup,
                                        steps)
                hc = statistics.mean(float(t.len_host[i].sum()) for i in seqs[warmup:])
                traffic = hc + nb * (B + 16)
                r["gpu_hbm" + tag + "_GBps"] = round(nb * B / (hm * 1e-3) / 1e9, 1)
                r["hbm" + tag + "_frac"] = round(traffic / (hm * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
                del out, d
            if key == "tiny":
                r["note"] = "the 1.8 MB cache fits the 256 MB last-level cache: a latency point"
        if t.raw is not None:
            t.raw.free()
        if isinstance(t.store, ibp.HostBuffer):
            t.store.free()
        del t, m
        torch.cuda.empty_cache()
        rows_out.append(r)
        log(f"configs: {r}")
    # K/V: one (layer, K|V) pair, Mask from its prefill rows, its 2,560 decode rows
    w = W.WORKLOADS["kv_opt13b"]
    B, C, S, R = w.tensor_bytes, w.chunk_bytes, w.slot_bytes, W.KV_ROWS_PER_PAIR
    pre = torch.from_numpy(W.kv_prefill_rows(w, 0)).cuda()
    mask = torch.zeros(B // 4, dtype=torch.int32, device="cuda")
    bitval = torch.zeros_like(mask)
    counts = torch.zeros(8 * B, dtype=torch.int32, device="cuda")
    ibp.build_metadata(pre, B, None, pre.shape[0], B, w.threshold, mask, bitval, counts)
    del pre
    raw = ibp.HostBuffer(R * S)
    W.rows(w, 0, R, out=raw.array.reshape(R, S)[:, :B])
    store = ibp.HostBuffer(R * S)
    part = torch.zeros((R * ibp.num_chunks(B, C) + 31) // 32, dtype=torch.int32, device="cuda")
    lengths = torch.zeros(R, dtype=torch.int32, device="cuda")
    ibp.compress(raw, S, R, 0, R, B, C, mask, bitval, store, S, part, lengths)
    ids = np.arange(R, dtype=np.int64)
    d = torch.from_numpy(ids).cuda()
    out = torch.empty(R * B, dtype=torch.uint8, device="cuda")
    km, _ = region_launches(torch, lambda k: ibp.gather_decompress(
        store, R * S, S, None, part, R, d, R, B, C, mask, bitval, out), warmup, steps)
    if not (out.view(R, B)[::97].cpu().numpy() == raw.array.reshape(R, S)[::97, :B]).all():
        raise SystemExit("bench: kv_opt13b gather is not lossless")
    len_h = lengths.cpu().numpy().view(np.uint32)
    comp = float(len_h.astype(np.float64).sum())
    part_h, mask_h, bitval_h = (x.cpu().numpy().view(np.uint32) for x in (part, mask, bitval))
    import ctypes
    gomp = ctypes.CDLL("libgomp.so.1")
    threads = gomp.omp_get_max_threads()
    rates = {}
    for nt in (threads, 1):
        gomp.omp_set_num_threads(nt)
        t0 = time.perf_counter()
        k = 0
        while True:
            O.gather_decompress(store.array, part_h, R, ids, B, C, mask_h, bitval_h, slot_bytes=S)
            k += 1
            el = time.perf_counter() - t0
            if el >= 2.0 or k >= 20:
                break
        rates[nt] = round(k * R * B / el / 1e9, 4)
    gomp.omp_set_num_threads(threads)
    rows_out.append({"config": "kv_opt13b", "tensor_bytes": B, "batch": R,
                     "space_saving": round(1.0 - float(len_h.mean()) / B, 4),
                     "oracle_1_thread_GBps": rates[1], "oracle_all_GBps": rates[threads],
                     "oracle_threads": threads,
                     "gpu_pinned_GBps": round(R * B / (km * 1e-3) / 1e9, 2),
                     "pcie_frac_all_ids": round(comp / (km * 1e-3) / 1e9 / link, 4),
                     "pcie_frac_unique": round(comp / (km * 1e-3) / 1e9 / link, 4),
                     "xcd_routed": False})
    raw.free()
    store.free()
    return {"metric": "per-workload gather + decompress: oracle and GPU", "unit": "GB/s",
            "higher_is_better": True, "link_peak_GBps": link, "hbm_peak_GBps": HBM_PEAK_GBPS,
            "configs": rows_out, "device": torch.cuda.get_device_name(0), "host": host_info()}


def measure_tiny(torch, ibp, W, args):
    """Config 1: 4,096 tensors of 512 B held as a compacted cache in HBM
    (about 1.8 MB, so it sits in the 256 MB last-level cache: a latency point,
    not an HBM-bandwidth one), gathered in a seeded permutation of all ids,
    against the uncompressed gather of the same rows from HBM."""
    import numpy as np
    w = W.WORKLOADS["tiny"]
    table = Table(torch, ibp, W, w, w.threshold, "hbm", ibp.HOST_DEFAULT, keep_raw=True)
    B, S, N = w.tensor_bytes, w.slot_bytes, w.n_tensors
    raw_dev = torch.from_numpy(table.raw.array).cuda()
    steps = max(5, args.steps)
    seqs = [W.batch_ids(w, k) for k in range(args.warmup + steps)]
    d = [torch.from_numpy(i).cuda() for i in seqs]
    out = torch.empty(w.batch * B, dtype=torch.uint8, device="cuda")
    km, _ = region_launches(torch, lambda k: table.gather(ibp, d[k], w.batch, out), args.warmup,
                            steps)
    check_rows(table, seqs[-1], out)
    rm, _ = region_launches(torch, lambda k: ibp.raw_gather(raw_dev, S, N, d[k], w.batch, B, out),
                            args.warmup, steps)
    res = {"workload": f"tiny: {N} x {B} B, {w.chunk_bytes} B chunks, T={w.threshold}, Mask from "
                       f"all tensors, compacted cache of {table.store_bytes / 1e6:.2f} MB in HBM",
           "ids": w.batch, "id_law": "a permutation of all ids",
           "mean_payload_over_tensor": round(float(table.len_host.mean()) / B, 5),
           "kernel_us": round(km * 1e3, 2),
           "decompressed_GBps": round(w.batch * B / (km * 1e-3) / 1e9, 1),
           "raw_hbm_gather_us": round(rm * 1e3, 2), "speedup_vs_raw_hbm_gather": round(rm / km, 3),
           "offline": {"metadata_ms": round(table.meta_ms, 3),
                       "compress_ms": round(table.compress_ms, 3),
                       "compact_ms": round(table.compact_ms, 3)},
           "note": "cache and rows fit the 256 MB last-level cache: launch latency, not bandwidth"}
    table.raw.free()
    del table, raw_dev, out, d
    torch.cuda.empty_cache()
    log(f"tiny: {res}")
    return res


def measure_sparse_t95(torch, ibp, W, args, flags, pr):
    """Config 2 at T = 0.95 (the same sparse features and batches as the
    headline, a lower threshold)."""
    import numpy as np
    m = measure_workload(torch, ibp, W, "sparse_gnn", 0.95, "pinned", flags, args.steps,
                         args.warmup, with_raw=True)
    t, w = m["table"], W.WORKLOADS["sparse_gnn"]
    km = m["kernel_ms"]
    comp = statistics.mean(m["comp_bytes"])
    link = max(pr["h2d_dma_GBps"], pr["h2d_zero_copy_read_GBps"])
    res = {"workload": f"sparse_gnn: {w.n_tensors} x {w.tensor_bytes} B, {w.chunk_bytes} B chunks, "
                       f"T=0.95, Mask from 1 % of the tensors, pinned host, {w.batch} uniform ids",
           "mean_payload_over_tensor": round(float(t.len_host.mean()) / w.tensor_bytes, 5),
           "kernel_us": round(km * 1e3, 2),
           "decompressed_GBps": round(w.batch * w.tensor_bytes / (km * 1e-3) / 1e9, 2),
           "payload_GBps_over_link": round(comp / (km * 1e-3) / 1e9, 2),
           "frac_of_measured_link": round(comp / (km * 1e-3) / 1e9 / link, 4),
           "raw_gather_us": round(m["raw_kernel_ms"] * 1e3, 2),
           "transfer_speedup_vs_raw_gpu_gather": round(m["raw_kernel_ms"] / km, 3)}
    t.raw.free()
    t.store.free()
    del t, m
    torch.cuda.empty_cache()
    log(f"sparse_gnn T=0.95: {res}")
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(gathered tensors are independent, so a batch would split across GPUs "
              "with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from host_transfer_amd import ibp
    from host_transfer_amd import workloads as W

    torch.cuda.set_device(0)
    flags = {"default": ibp.HOST_DEFAULT, "coherent": ibp.HOST_COHERENT,
             "noncoherent": ibp.HOST_NONCOHERENT}[args.host_flags]
    log(f"device {torch.cuda.get_device_name(0)}; host {host_info()}")
    pr = probes(torch, ibp, flags)
    log(f"probes {pr}")
    if args.mode == "ablation":
        print(json.dumps(run_ablation(torch, ibp, args, pr)), flush=True)
        return
    if args.mode == "sweep":
        print(json.dumps({"sweep": run_sweep(torch, ibp, args, pr),
                          "weight_stream": run_weight_stream(torch, ibp, args, pr)}), flush=True)
        return
    if args.mode == "kv-step":
        print(json.dumps(run_kv_step(torch, ibp, W, args, pr)), flush=True)
        return
    if args.mode == "configs":
        args.host_flags_value = flags
        print(json.dumps(run_configs(torch, ibp, W, args, pr)), flush=True)
        return

    # --- headline: the workload from pinned host memory
    key = args.workload
    m = measure_workload(torch, ibp, W, key, args.threshold, "pinned", flags, args.steps,
                         args.warmup, with_raw=True)
    w, table = W.WORKLOADS[key], m["table"]
    K = args.steps
    dense_bytes = w.batch * w.tensor_bytes
    value = dense_bytes * K / m["wall"] / 1e9
    kern_ms = m["kernel_ms"]
    comp = statistics.mean(m["comp_bytes"])
    uniq = statistics.mean(float(table.len_host[np.unique(i)].sum())
                           for i in m["ids_host"][args.warmup:])
    achieved = comp / (kern_ms * 1e-3) / 1e9
    raw_ms = m["raw_kernel_ms"]
    link_peak = max(pr["h2d_dma_GBps"], pr["h2d_zero_copy_read_GBps"])
    traffic = profiled_traffic()
    log(f"{key}: {value:.1f} GB/s decompressed, kernel {kern_ms * 1e3:.1f} us, "
        f"{achieved:.1f} GB/s compressed over the link, raw gather {raw_ms * 1e3:.1f} us")

    result = {
        "metric": "decompressed GB/s for batched gather+decompress; % of PCIe/HBM roofline",
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(m["wall"] * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic (seeded generators shaped like the pages' workloads)",
        "config": {
            "workload": f"{key}: {w.n_tensors} tensors x {w.tensor_bytes} B, {w.chunk_bytes} B "
                        f"chunks, T={m['T']}, Mask from "
                        f"{'all' if w.sample_fraction >= 1 else f'{w.sample_fraction:.0%}'} of "
                        f"the tensors, store in pinned host memory ({args.host_flags}), "
                        f"{w.batch} ids per batch ({w.id_law})",
            "batch": w.batch, "tensor_bytes": w.tensor_bytes, "chunk_bytes": w.chunk_bytes,
            "store": "pinned-host", "host_flags": args.host_flags,
        },
        "roofline": {
            "bound": "pcie",
            "achieved": round(achieved, 3),
            "peak": PCIE5_X16_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PCIE5_X16_GBPS, 4),
            "traffic": None if traffic is None else traffic["link_read"],
            "traffic_unit": "bytes per launch read over the host link (rocprofv3 counters)",
            "traffic_counters": traffic,
            "link_bytes_frac_of_measured": None if traffic is None else
            round(traffic["link_read"] / (kern_ms * 1e-3) / 1e9 / link_peak, 4),
            "peak_measured": round(link_peak, 2),
            "frac_of_measured": round(achieved / link_peak, 4),
            "peak_zero_copy_read": pr["h2d_zero_copy_read_GBps"],
            "frac_of_zero_copy_read": round(achieved / pr["h2d_zero_copy_read_GBps"], 4),
            "kernel": "k_gather_decompress",
            "kernel_us": round(kern_ms * 1e3, 2),
            "isolated_launch_us": percentiles_us(m["isolated_ms"]),
            "bytes_per_launch": round(comp, 1),
            "unique_bytes_per_launch": round(uniq, 1),
            "unique_frac_of_measured": round(uniq / (kern_ms * 1e-3) / 1e9 / link_peak, 4),
        },
        "compression": {
            "mean_payload_over_tensor": round(float(table.len_host.mean()) / w.tensor_bytes, 5),
            "batch_payload_over_dense": round(comp / dense_bytes, 5),
        },
        "transfer_speedup_vs_raw_gpu_gather": round(raw_ms / kern_ms, 3),
        "raw_gather_GBps": round(dense_bytes / (raw_ms * 1e-3) / 1e9, 2),
        "offline": {"metadata_ms": round(table.meta_ms, 3),
                    "metadata_warm_ms": round(table.meta_warm_ms, 3),
                    "metadata_sample_bytes": table.meta_bytes,
                    "metadata_warm_frac_of_measured": round(
                        table.meta_bytes / (table.meta_warm_ms * 1e-3) / 1e9 / link_peak, 4),
                    "compress_ms": round(table.compress_ms, 3),
                    "compress_frac_of_measured": round(
                        w.n_tensors * w.tensor_bytes / (table.compress_ms * 1e-3) / 1e9
                        / link_peak, 4)},
        "probes": pr,
        "host": host_info(),
        "device": torch.cuda.get_device_name(0),
    }
    # one launch over 16 batches: the per-launch fixed cost spread over 16x the bytes
    n16 = max(1, min(2, len(m["ids_host"]) // 16))
    big_ids = [np.concatenate(m["ids_host"][16 * k:16 * k + 16]) for k in range(n16)]
    nb16 = min(len(i) for i in big_ids)
    d16 = [torch.from_numpy(i).cuda() for i in big_ids]
    out16 = torch.empty(nb16 * w.tensor_bytes, dtype=torch.uint8, device="cuda")
    ms16, _ = region_launches(torch, lambda k: table.gather(ibp, d16[k % len(d16)], nb16, out16),
                              2, 6)
    comp16 = statistics.mean(float(table.len_host[i].sum()) for i in big_ids)
    result["roofline"]["one_launch_16_batches"] = {
        "ids": nb16, "kernel_us": round(ms16 * 1e3, 2),
        "achieved": round(comp16 / (ms16 * 1e-3) / 1e9, 3),
        "frac_of_measured": round(comp16 / (ms16 * 1e-3) / 1e9 / link_peak, 4),
        "frac_of_zero_copy_read": round(comp16 / (ms16 * 1e-3) / 1e9 /
                                        pr["h2d_zero_copy_read_GBps"], 4)}
    del out16, d16
    # the same batches on two streams in turn: a launch's ramp overlaps the
    # previous launch's drain (each stream has its own output buffer)
    d2 = [torch.from_numpy(i).cuda() for i in m["ids_host"]]
    outs = [torch.empty(dense_bytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    ms2 = two_stream_launches(
        torch, lambda k: table.gather(ibp, d2[k % len(d2)], w.batch, outs[k % 2]),
        args.warmup, K)
    last = args.warmup + K - 1
    check_rows(table, m["ids_host"][last % len(d2)], outs[last % 2])
    comp2 = statistics.mean(m["comp_bytes"])
    result["roofline"]["two_streams"] = {
        "kernel_us_per_batch": round(ms2 * 1e3, 2),
        "achieved": round(comp2 / (ms2 * 1e-3) / 1e9, 3),
        "frac_of_measured": round(comp2 / (ms2 * 1e-3) / 1e9 / link_peak, 4),
        "note": "the timed batches launched alternately on two streams (default priority)"}
    log(f"two streams: {result['roofline']['two_streams']}")
    del outs, d2
    log("cache + store at a 10 % HBM budget ...")
    batches_dev = [torch.from_numpy(i).cuda() for i in m["ids_host"]]
    result["hybrid_path"] = measure_hybrid(torch, ibp, table, batches_dev, m["ids_host"], args,
                                           0.10)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(table, m["ids_host"][args.warmup:], args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    sampling = [measure_sampling(torch, ibp, table)] if args.extras else []
    table.raw.free()
    table.store.free()
    del table, m
    torch.cuda.empty_cache()

    # --- the other pinned-host workloads (their own batch sizes), then
    #     the same tables compacted into HBM caches: the workload's batch and a
    #     large batch (1M ids) that fills the GPU
    if args.extras:
        result["configs"] = {"tiny_hbm": measure_tiny(torch, ibp, W, args),
                             "sparse_gnn_T095": measure_sparse_t95(torch, ibp, W, args, flags, pr)}
    result["pinned_path"] = []
    result["hbm_path"] = []
    hbm = [] if args.hbm_workloads == "none" else args.hbm_workloads.split(",")
    pinned = [] if args.pinned_workloads == "none" else args.pinned_workloads.split(",")
    for key in pinned + [k for k in hbm if k not in pinned]:
        res, tb = measure_pinned(torch, ibp, W, key, flags, args, pr)
        if key == "dlrm_1k" and key in pinned:
            res["multi_table"] = measure_multi_table(torch, ibp, W, tb, args, pr)
            log(f"{key} multi-table: {res['multi_table']}")
        if key in pinned:
            result["pinned_path"].append(res)
        if args.extras:
            sampling.append(measure_sampling(torch, ibp, tb))
            log(f"{key} sampling: {sampling[-1]}")
        if key in hbm:
            result["hbm_path"].append(measure_hbm(torch, ibp, W, tb, args, pr))
        if tb.raw is not None:
            tb.raw.free()
        if isinstance(tb.store, ibp.HostBuffer):
            tb.store.free()
        del tb
        torch.cuda.empty_cache()
    if args.kv_pairs_default > 0:
        result["kv_step"] = run_kv_step(torch, ibp, W, args, pr, pairs=args.kv_pairs_default)
    if args.extras:
        result["sampled_metadata"] = sampling
        result["weight_stream"] = run_weight_stream(torch, ibp, args, pr)
        result["saving_sweep"] = run_sweep(torch, ibp, args, pr)
        result["transfer_ablation"] = run_ablation(torch, ibp, args, pr, pool_bytes=1 << 30)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
