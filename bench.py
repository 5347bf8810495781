"""Benchmark of the TurboQuant decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only headline]

A step is one decode step of one attention layer: tq_store of the step's new
K/V token for every sequence (B tokens x Hk heads), then tq_decode_attention
(stage 1 + stage 2) of one query per sequence over the whole compressed
cache.  The headline workload is the Llama-3-8B-shaped layer (k8v4, 32
sequences x 4096 tokens, 32/8 heads, block 16).  ``value`` is the effective
decode-attention bandwidth: compressed-cache bytes the step reads
(sum_b L_b * Hk * slot_size) over the step's wall time, inputs resident in HBM.
The same bytes over one tq_decode_attention call alone (no store) are
reported as ``config.decode_call_gbs``.

Timing: twelve steps are captured in one HIP graph, rotating over three
copies of the cache (3 x 411 MB for the headline, so the 256 MB Infinity Cache
cannot serve a step's reads from the previous one), the way a multi-layer
decode graph strings layers together; the graph is replayed on torch's
current stream and K steps are bracketed by events after a synchronize.  The roofline figure times stage-1
launches alone with events on the same stream.  The CPU baseline is the
oracle (NumPy) decoding a bounded sample of the same workload.

Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
N_COPIES = 3
# Steps (or decode calls) captured in one graph: four passes over the three
# cache copies, as a stretch of a multi-layer decode graph strings layers
# together.  Replaying a graph costs a gap of ~8 us on the GPU before its first
# kernel (measured in a kernel trace: kernels inside a graph start back to
# back); over 12 calls that is ~0.7 us per call.
GRAPH_STEPS = 12


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def dev16(torch, bits, dtype):
    x = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return x.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def warm_gpu(torch, fn, ms=150.0):
    """Launch fn() until `ms` of GPU time has passed: after seconds of host
    work the GPU has idled and its clock is back down, and the first few ms of
    VALU-bound kernels run 20-30% slow."""
    spent = 0.0
    while spent < ms:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(10):
            fn()
        b.record()
        torch.cuda.synchronize()
        spent += a.elapsed_time(b)


DIST_REPLAYS = 60  # timed repetitions behind every median / p10 / p90


def spread(torch, fn, reps, per_rep):
    """Run fn() `reps` times back to back on torch's current stream, each
    bracketed by events; returns {median, p10, p90, mean} in ms per unit of
    work (one call of fn is `per_rep` units)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    fn()
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = np.array(sorted(a.elapsed_time(b) for a, b in ev)) / per_rep
    return {"median": float(np.median(t)), "p10": float(np.percentile(t, 10)), "p90": float(np.percentile(t, 90)),
            "mean": float(t.mean()), "reps": reps}


MORE_PRESETS = ("turboquant_k8v3", "turboquant_k4v3_nc", "turboquant_2bit_nc", "turboquant_k8v3lm", "turboquant_3bit_lm",
                "turboquant_k8v4lm", "turboquant_4bit_lm", "turboquant_2bit_lm")
SPARSE_V_GATE = 1e-3
# head_dim 256 leg: the headline preset, FP8 keys with Lloyd-Max values (the pages' fp8k_turbo3v), 3-bit MSE
HEAD256_PRESETS = ("turboquant_k8v4", "turboquant_k8v3lm", "turboquant_3bit_nc")


class DecodeBench:
    """Device state of one decode workload: N_COPIES caches, the step's new
    tokens, queries, tables, workspace."""

    def __init__(self, torch, tq, w: W.Workload, num_kv_splits: int, block_layout: str = "aos",
                 sliding_window: int = 0, sinks=None, value_gate: float = 0.0, scale_mult: float = 1.0,
                 warm: bool = True):
        self.torch, self.tq, self.w = torch, tq, w
        self.S = num_kv_splits
        self.window = sliding_window
        self.gate = value_gate
        D = w.head_dim
        self.lay = tq.layout_init(w.preset, D, block_layout)
        self.lens = W.seq_lens(w)
        table = W.block_table(w)
        self.table_np = table
        self.nb = W.num_blocks(w)
        self.tab = tq.Tables(self.lay, W.signs(w))
        shape = tq.kv_cache_shape(self.lay, self.nb, w.block_size, w.num_kv_heads)
        log(f"[{w.name}] generating inputs")
        t0 = time.time()
        K, V = W.kv_all(w, threads=16)
        log(f"[{w.name}] inputs in {time.time() - t0:.1f}s; storing the context")
        cache = torch.zeros(shape, dtype=torch.uint8, device="cuda")
        newk, newv, newslots = [], [], []
        for b in range(w.batch):
            L = int(self.lens[b])
            slots = W.slot_mapping_for_sequence(w, b, table, self.lens)
            kd, vd = dev16(torch, K[b], w.dtype), dev16(torch, V[b], w.dtype)
            tq.store(self.lay, kd, vd, torch.from_numpy(slots).cuda(), cache, self.tab.signs, self.tab.centroids,
                     self.tab.boundaries)
            newk.append(K[b][L - 1 : L])
            newv.append(V[b][L - 1 : L])
            newslots.append(slots[L - 1 : L])
        del K, V
        torch.cuda.synchronize()
        self.caches = [cache] + [cache.clone() for _ in range(N_COPIES - 1)]
        # the step re-stores each sequence's last token (its new token)
        self.knew = dev16(torch, np.concatenate(newk), w.dtype)
        self.vnew = dev16(torch, np.concatenate(newv), w.dtype)
        self.snew = torch.from_numpy(np.concatenate(newslots)).cuda()
        self.q = dev16(torch, W.queries(w), w.dtype)
        self.bt = torch.from_numpy(table).cuda()
        self.sl = torch.from_numpy(self.lens).cuda()
        self.ws = torch.empty(tq.decode_workspace_bytes(w.batch, w.num_q_heads, D, self.S), dtype=torch.uint8,
                              device="cuda")
        self.out = torch.empty((w.batch, w.num_q_heads, D), dtype=self.q.dtype, device="cuda")
        self.lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device="cuda")
        self.scale = scale_mult / math.sqrt(D)
        seen = np.minimum(self.lens, sliding_window) if sliding_window > 0 else self.lens
        self.bytes_read = int(seen.astype(np.int64).sum()) * w.num_kv_heads * self.lay.slot_size_aligned
        self.row_bytes = w.num_kv_heads * self.lay.slot_size_aligned  # one token row, all KV heads
        self.sinks = None if sinks is None else torch.from_numpy(np.asarray(sinks, np.float32)).cuda()
        torch.cuda.synchronize()
        if warm:
            it = iter(range(1 << 30))
            warm_gpu(torch, lambda: self.step(next(it) % N_COPIES))

    def store(self, i):
        self.tq.store(self.lay, self.knew, self.vnew, self.snew, self.caches[i], self.tab.signs, self.tab.centroids,
                      self.tab.boundaries)

    def stage1(self, i):
        self.tq.decode_stage1(self.lay, self.q, self.caches[i], self.bt, self.sl, self.tab.signs, self.tab.centroids,
                              self.scale, self.S, self.ws, sliding_window=self.window, value_gate=self.gate)

    def stage2(self):
        self.tq.decode_stage2(self.w.batch, self.w.num_q_heads, self.w.head_dim, self.S, self.ws, self.out, self.lse,
                              sinks=self.sinks)

    def step(self, i):
        self.store(i)
        self.stage1(i)
        self.stage2()

    def graphs(self):
        """One graph holding GRAPH_STEPS consecutive steps (cache copy i % 3
        for step i), like a stretch of a multi-layer decode graph, plus
        one-step graphs for a remainder."""
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(N_COPIES):  # warm the launch path once outside capture
                self.step(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all):
            for i in range(GRAPH_STEPS):
                self.step(i % N_COPIES)
        singles = []
        for i in range(N_COPIES):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step(i)
            singles.append(g)
        torch.cuda.synchronize()
        return g_all, singles

    def time_steps(self, steps, warmup):
        """ms per step over exactly `steps` steps (graph replays), then the
        per-step spread over DIST_REPLAYS further replays of the step graph."""
        torch = self.torch
        g_all, singles = self.graphs()
        for _ in range(max(1, warmup // GRAPH_STEPS)):
            g_all.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps // GRAPH_STEPS):
            g_all.replay()
        for i in range(steps % GRAPH_STEPS):
            singles[i % N_COPIES].replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        return ms, spread(torch, g_all.replay, DIST_REPLAYS, GRAPH_STEPS)

    def decode_graph(self):
        """One graph of GRAPH_STEPS tq_decode_attention calls (stage 1 +
        stage 2, no store), rotating over the cache copies."""
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(GRAPH_STEPS):
                self.stage1(i % N_COPIES)
                self.stage2()
        g.replay()
        torch.cuda.synchronize()
        return g

    def time_decode(self, reps=None):
        """Per tq_decode_attention call: median / p10 / p90 (ms) over `reps`
        replays of the decode graph (GRAPH_STEPS calls each)."""
        g = self.decode_graph()
        return spread(self.torch, g.replay, reps or DIST_REPLAYS, GRAPH_STEPS)

    def time_gather(self, launches=None):
        """The decode's tile reads alone (the probe library's gather kernel:
        every 16-token tile of every sequence through the block table, split
        evenly over 1024 workgroups, no arithmetic), median / p10 / p90 (ms)
        of `launches` launches rotating
        over the cache copies: the ceiling of this read pattern.  Token rows
        must be whole 16-byte chunks (the probe's load width)."""
        torch, w = self.torch, self.w
        L = _probe_lib()
        groups = 1024
        out = torch.empty(4 * groups, dtype=torch.int32, device="cuda")
        prefix = torch.from_numpy(np.concatenate([[0], np.cumsum(-(-self.lens // 16))]).astype(np.int32)).cuda()
        row = self.row_bytes
        it = iter(range(1 << 30))

        def launch():
            c = self.caches[next(it) % N_COPIES]
            rc = L.tq_probe_gather_read(c.data_ptr(), self.bt.data_ptr(), self.bt.shape[1], prefix.data_ptr(),
                                        w.batch, w.block_size, row, groups, out.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream)
            assert rc == 0, rc

        warm_gpu(torch, launch, 30.0)
        return spread(torch, launch, launches or DIST_REPLAYS, 1)

    def time_stage1(self, launches=None):
        """Stage-1 kernel duration: median / p10 / p90 (ms) of `launches`
        back-to-back launches (rotating caches), each bracketed by events on
        the launch stream."""
        it = iter(range(1 << 30))
        return spread(self.torch, lambda: self.stage1(next(it) % N_COPIES), launches or DIST_REPLAYS, 1)


def store_sweep(torch, tq, steps, block_layout="aos", presets=None, head_dim=128):
    """Store sweep: 65536 tokens x 8 KV heads, bs 32, per preset (Mtok/s)."""
    s = W.STORE_WORKLOAD
    K, V, slots, nb = W.store_inputs(head_dim=head_dim)
    kd, vd = dev16(torch, K, s["dtype"]), dev16(torch, V, s["dtype"])
    sd = torch.from_numpy(slots).cuda()
    res = {}
    for preset in presets or s["presets"]:
        lay = tq.layout_init(preset, head_dim, block_layout)
        tab = tq.Tables(lay, W.signs(s["seed"], head_dim))
        caches = [torch.zeros(tq.kv_cache_shape(lay, nb, s["block_size"], s["num_kv_heads"]), dtype=torch.uint8,
                              device="cuda") for _ in range(N_COPIES)]
        for c in caches:
            tq.store(lay, kd, vd, sd, c, tab.signs, tab.centroids, tab.boundaries)
        warm_gpu(torch, lambda: tq.store(lay, kd, vd, sd, caches[0], tab.signs, tab.centroids, tab.boundaries), 50.0)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i, (a, b) in enumerate(evs):
            a.record()
            tq.store(lay, kd, vd, sd, caches[i % N_COPIES], tab.signs, tab.centroids, tab.boundaries)
            b.record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
        n = s["num_tokens"]
        bytes_moved = n * s["num_kv_heads"] * (2 * head_dim * 2 + lay.slot_size_aligned) + n * 8
        res[preset] = {"mtok_s": n / (ms * 1e-3) / 1e6, "ms": ms, "gbs": bytes_moved / (ms * 1e-3) / 1e9,
                       "frac_hbm": bytes_moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del caches
    torch.cuda.empty_cache()
    # the ceiling of moving that many bytes: a plain device copy of half of
    # them (read + write = the store's reads + writes at the first preset)
    first = res[next(iter(res))]
    copy = copy_ceiling(torch, int(first["gbs"] * first["ms"] * 1e6) // 2)
    for k in list(res):
        res[k]["frac_of_copy"] = res[k]["gbs"] / copy["gbs"]
    res["copy"] = copy
    return res


def copy_ceiling(torch, nbytes, reps=30):
    """Median rate (read + write bytes per second) of a plain device copy of
    `nbytes` (the probe library's copy kernel; three buffer pairs rotated so
    that the 256 MB Infinity Cache cannot serve a copy from the previous)."""
    L = _probe_lib()
    nbytes = nbytes // 16 * 16
    src = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(i + 1) for i in range(N_COPIES)]
    dst = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(N_COPIES)]
    it = iter(range(1 << 30))

    def launch():
        i = next(it) % N_COPIES
        rc = L.tq_probe_copy(src[i].data_ptr(), dst[i].data_ptr(), nbytes, 4096, torch.cuda.current_stream().cuda_stream)
        assert rc == 0, rc

    warm_gpu(torch, launch, 30.0)
    t = spread(torch, launch, reps, 1)
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_each_way": nbytes, "us_median": t["median"] * 1e3, "gbs": 2 * nbytes / (t["median"] * 1e-3) / 1e9}


def cpu_baseline(w: W.Workload, budget_s: float = 12.0, store_budget_s: float = 6.0):
    """The oracle, as it stands, on the host cores: (1) decoding whole
    (sequence, KV head) groups of the workload (stored by the oracle) with
    all their query heads until `budget_s` of CPU time is spent, in GB/s of
    compressed cache; (2) storing rows of the store-sweep inputs (encode +
    slot write) for the headline preset and 3bit_nc until `store_budget_s`
    each, in Mtok/s (one token = all of its KV heads)."""
    import oracle as O

    lay = O.layout(w.preset, 128)
    lens = W.seq_lens(w)
    signs = W.signs(w).astype(np.float64)
    c32, b32 = (None, None) if lay.key_fp8 else O.codebook_tables(128, lay.key_bits)
    R = O.rotation(signs) if O.needs_rotation(lay) else None
    q = O.widen(W.queries(w), w.dtype)
    g = w.num_q_heads // w.num_kv_heads
    scale = 1.0 / math.sqrt(128)
    spent, nbytes, groups = 0.0, 0, 0
    for b in range(w.batch):
        K, V = W.kv_sequence(w, b, lens)
        for hk in range(w.num_kv_heads):
            slots = O.encode_slots(lay, O.widen(K[:, hk], w.dtype), O.widen(V[:, hk], w.dtype), R, c32, b32)
            t0 = time.perf_counter()
            Kd, Vd = O.decode_slots(lay, slots, c32, R)
            for j in range(g):
                qq = q[b, hk * g + j] if lay.key_fp8 else R @ q[b, hk * g + j]
                O.attend(qq, Kd, Vd, scale)
            spent += time.perf_counter() - t0
            nbytes += int(lens[b]) * lay.slot_size_aligned
            groups += 1
            if spent >= budget_s:
                break
        if spent >= budget_s:
            break
    cores = len(os.sched_getaffinity(0))
    # store: chunks of the store sweep's tokens, all 8 KV heads each
    s = W.STORE_WORKLOAD
    Ks, Vs, slots_all, nb = W.store_inputs(num_tokens=16384)
    store = {}
    for preset in (w.preset, "turboquant_3bit_nc"):
        sl = O.layout(preset, 128)
        sc32, sb32 = (None, None) if sl.key_fp8 else O.codebook_tables(128, sl.key_bits)
        cache = np.zeros((nb, s["block_size"], s["num_kv_heads"], sl.slot_size_aligned), np.uint8)
        t_spent, toks, chunk = 0.0, 0, 2048
        while t_spent < store_budget_s and toks < Ks.shape[0]:
            a = toks
            t0 = time.perf_counter()
            O.store_rows(sl, O.widen(Ks[a : a + chunk], s["dtype"]), O.widen(Vs[a : a + chunk], s["dtype"]),
                         slots_all[a : a + chunk], cache, signs, sc32, sb32)
            t_spent += time.perf_counter() - t0
            toks += chunk
        store[preset] = {"mtok_s": toks / t_spent / 1e6, "tokens": toks, "seconds": t_spent}
    return {"value": nbytes / spent / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{groups} (sequence, KV head) groups of the {w.name} workload ({nbytes} compressed bytes), "
                      f"oracle-stored, decoded with all {g} query heads each; {spent:.1f}s of CPU time; NumPy/BLAS "
                      f"threads up to the {cores} cores in the affinity mask",
            "store": {"unit": "Mtok/s", "sample": "store-sweep tokens (8 KV heads each, bf16) in chunks of 2048, "
                                                   "encoded and written by the oracle", **store}}


KERNEL_SOURCES = ("quantized_decode_attention_tq_amd/csrc/tq_decode.hip", "quantized_decode_attention_tq_amd/csrc/tq_bits.h",
                  "quantized_decode_attention_tq_amd/csrc/tq_internal.h", "include/tq.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "tq_decode_stage1_k8v4_llama8b_traffic.txt")


def kernel_source_hash():
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per stage-1 launch from the committed rocprofv3 counter
    summary, or None when it is missing or was taken on other kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _probe_lib():
    """libtq_probe.so: the streaming-read, tile-gather and copy kernels used
    for the bandwidth ceilings and the counter calibration (built with libtq)."""
    import ctypes

    import torch  # noqa: F401  (torch's HIP runtime first, as for libtq)

    path = os.path.join(ROOT, "quantized_decode_attention_tq_amd", "libtq_probe.so")
    L = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    L.tq_probe_stream_read.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, vp, vp]
    L.tq_probe_copy.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int, vp]
    L.tq_probe_gather_read.argtypes = [vp, vp, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                       ctypes.c_int, vp, vp]
    return L


STREAM_CHUNK = 64 << 10


def stream_ceiling(torch, nbytes):
    """Median / p10 / p90 of a plain streaming read of `nbytes` (three
    buffers rotated, so the 256 MB Infinity Cache cannot serve a launch from
    the previous one), in GB/s: the practical ceiling of the decode's read."""
    L = _probe_lib()
    nbytes = nbytes // 16 * 16
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(i + 1) for i in range(N_COPIES)]
    out = torch.zeros(-(-nbytes // STREAM_CHUNK), dtype=torch.int32, device="cuda")
    it = iter(range(1 << 30))

    def launch():
        st = torch.cuda.current_stream().cuda_stream
        rc = L.tq_probe_stream_read(bufs[next(it) % N_COPIES].data_ptr(), nbytes, STREAM_CHUNK, out.data_ptr(), st)
        assert rc == 0, rc

    warm_gpu(torch, launch, 30.0)
    t = spread(torch, launch, DIST_REPLAYS, 1)
    del bufs
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "chunk": STREAM_CHUNK, "us_median": t["median"] * 1e3,
            "gbs_median": nbytes / (t["median"] * 1e-3) / 1e9, "gbs_p10_time": nbytes / (t["p90"] * 1e-3) / 1e9,
            "gbs_p90_time": nbytes / (t["p10"] * 1e-3) / 1e9}


def calibrate_copy(torch, mib: int = 512, reps: int = 5):
    """A plain device-to-device copy of known size (the probe library's copy
    kernel), for scaling the FETCH_SIZE / WRITE_SIZE counters (run under
    rocprofv3 --pmc)."""
    L = _probe_lib()
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        assert L.tq_probe_copy(src.data_ptr(), dst.data_ptr(), n, 4096, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    print(json.dumps({"calibrate_copy_bytes": n, "reps": reps}))


def profile_stage1(torch, tq, name, launches, splits):
    """Only stage-1 launches of one decode workload (after the inputs are
    stored; no warm-up launches), for rocprofv3 counter runs."""
    S = {"longctx": 32}.get(name, splits)
    b = DecodeBench(torch, tq, W.WORKLOADS[name], S, warm=False)
    torch.cuda.synchronize()
    for i in range(launches):
        b.stage1(i % N_COPIES)
    torch.cuda.synchronize()
    print(json.dumps({"profiled": name, "stage1_launches": launches, "num_kv_splits": S}))


DEQUANT_TOKENS, DEQUANT_HK, DEQUANT_BS = 131072, 8, 128


def dequant_sweep(torch, tq, reps, block_layout="aos", presets=None, head_dim=128):
    """Cached prefix back to dense fp16 K/V (tq_dequant_kv): one sequence of
    131072 tokens x 8 KV heads in 128-token blocks (the long-context shape),
    per preset.  Bytes = slots read + 2 x head_dim fp16 written per (token, head);
    3 cache copies rotate so no launch finds its input in the 256 MB MALL."""
    n, Hk, bs = DEQUANT_TOKENS, DEQUANT_HK, DEQUANT_BS
    nb = n // bs
    g = torch.Generator(device="cuda").manual_seed(21)
    D = head_dim
    K = torch.randn((n, Hk, D), device="cuda", generator=g).to(torch.bfloat16)
    V = torch.randn((n, Hk, D), device="cuda", generator=g).to(torch.bfloat16)
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(22)).to(torch.int32)
    table = perm.cuda()
    slots = (perm.to(torch.int64).repeat_interleave(bs) * bs + torch.arange(bs).repeat(nb)).cuda()
    ko = torch.empty((n, Hk, D), dtype=torch.float16, device="cuda")
    vo = torch.empty_like(ko)
    res = {}
    for preset in presets or ("turboquant_k8v4", "turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc"):
        lay = tq.layout_init(preset, D, block_layout)
        tab = tq.Tables(lay, W.signs(21, D))
        caches = [torch.zeros(tq.kv_cache_shape(lay, nb, bs, Hk), dtype=torch.uint8, device="cuda")
                  for _ in range(N_COPIES)]
        for c in caches:
            tq.store(lay, K, V, slots, c, tab.signs, tab.centroids, tab.boundaries)
        for i in range(N_COPIES):
            tq.dequant_kv(lay, caches[i], table, n, tab.signs, tab.centroids, key_out=ko, value_out=vo)
        warm_gpu(torch, lambda: tq.dequant_kv(lay, caches[0], table, n, tab.signs, tab.centroids, key_out=ko,
                                              value_out=vo), 50.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            tq.dequant_kv(lay, caches[i % N_COPIES], table, n, tab.signs, tab.centroids, key_out=ko, value_out=vo)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nbytes = n * Hk * (lay.slot_size_aligned + 2 * D * 2)
        res[preset] = {"us": ms * 1e3, "gbs": nbytes / (ms * 1e-3) / 1e9,
                       "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "bytes": nbytes,
                       "mtok_s": n / (ms * 1e-3) / 1e6}
        del caches
        torch.cuda.empty_cache()
    return res


def _us(t):
    return {k: (v * 1e3 if k != "reps" else v) for k, v in t.items()}


def decode_leg(torch, tq, w, S, steps=None, warmup=None, **kw):
    """Stage 1 alone, the decode call (stage 1 + stage 2) and, when `steps`
    is given, the whole step (store + decode) of one workload: medians and
    p10 / p90 in us, and GB/s of compressed cache read at the medians."""
    b = DecodeBench(torch, tq, w, S, **kw)
    res = {"preset": w.preset, "num_kv_splits": S, "bytes_read": b.bytes_read}
    if steps is not None:
        ms, st = b.time_steps(steps, warmup)
        res["step_ms_exact_k"] = ms
        res["step_us"] = _us(st)
        res["step_gbs"] = b.bytes_read / (st["median"] * 1e-3) / 1e9
    d = b.time_decode()
    s1 = b.time_stage1()
    res["decode_call_us"] = _us(d)
    res["decode_gbs"] = b.bytes_read / (d["median"] * 1e-3) / 1e9
    res["decode_frac_hbm"] = res["decode_gbs"] / HBM_PEAK_GBS
    res["stage1_us"] = _us(s1)
    res["stage1_gbs"] = b.bytes_read / (s1["median"] * 1e-3) / 1e9
    if kw.get("block_layout", "aos") == "aos" and not kw.get("sliding_window") and b.row_bytes % 16 == 0:
        gr = b.time_gather()
        res["gather_read_us"] = _us(gr)
        res["gather_read_gbs"] = b.bytes_read / (gr["median"] * 1e-3) / 1e9
    del b
    torch.cuda.empty_cache()
    gather = f"; tile reads alone {res['gather_read_gbs']:.0f} GB/s" if "gather_read_gbs" in res else ""
    log(f"[{w.name}{' ' + str(kw) if kw else ''}] decode call {res['decode_call_us']['median']:.1f} us "
        f"(p10 {res['decode_call_us']['p10']:.1f}, p90 {res['decode_call_us']['p90']:.1f}) -> {res['decode_gbs']:.0f} "
        f"GB/s; stage 1 {res['stage1_us']['median']:.1f} us -> {res['stage1_gbs']:.0f} GB/s{gather}")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--splits", type=int, default=8)
    ap.add_argument("--only", choices=["all", "headline"], default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain copy of 512 MiB (counter calibration) and exit")
    ap.add_argument("--profile", choices=["llama8b", "longctx", "qwen32b"],
                    help="only launch stage 1 of this workload --steps times (for rocprofv3) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    import quantized_decode_attention_tq_amd as tq

    if args.profile:
        profile_stage1(torch, tq, args.profile, args.steps, args.splits)
        return

    w = W.WORKLOADS["llama8b"]
    head = decode_leg(torch, tq, w, args.splits, steps=args.steps, warmup=args.warmup)
    ms = head["step_ms_exact_k"]
    gbs = head["bytes_read"] / (ms * 1e-3) / 1e9
    stream = stream_ceiling(torch, head["bytes_read"])
    log(f"[llama8b] step {ms * 1e3:.1f} us -> {gbs:.0f} GB/s; streaming read of the same bytes "
        f"{stream['us_median']:.1f} us -> {stream['gbs_median']:.0f} GB/s")

    extra = {}
    if args.only == "all":
        for name, S in (("longctx", 32), ("qwen32b", args.splits)):
            extra[name] = decode_leg(torch, tq, W.WORKLOADS[name], S, steps=max(21, args.steps // 4),
                                     warmup=max(6, args.warmup // 4))
            extra[name]["stream_read"] = stream_ceiling(torch, extra[name]["bytes_read"])
        extra["store_sweep"] = store_sweep(torch, tq, 50)
        log(f"[store] {json.dumps({k: round(v['mtok_s'], 1) for k, v in extra['store_sweep'].items() if k != 'copy'})}")
        extra["dequant"] = dequant_sweep(torch, tq, 20)
        log(f"[dequant] {json.dumps({k: round(v['gbs']) for k, v in extra['dequant'].items()})} GB/s")
        # the same workloads with the cache in the SoA block convention
        soa = {}
        for name, S in (("llama8b", args.splits), ("longctx", 32), ("qwen32b", args.splits)):
            soa[name] = decode_leg(torch, tq, W.WORKLOADS[name], S, block_layout="soa")
        soa["store_sweep"] = store_sweep(torch, tq, 50, "soa")
        soa["dequant"] = dequant_sweep(torch, tq, 20, "soa")
        log(f"[soa store] {json.dumps({k: round(v['mtok_s'], 1) for k, v in soa['store_sweep'].items() if k != 'copy'})}; "
            f"[soa dequant] {json.dumps({k: round(v['gbs']) for k, v in soa['dequant'].items()})} GB/s")
        extra["soa"] = soa
        # the further presets (asymmetric pairs, 2-bit, Lloyd-Max values) on the llama8b shape
        more = {}
        for preset in MORE_PRESETS:
            wk = W.scaled(W.WORKLOADS["llama8b"], name=f"llama8b/{preset}", preset=preset)
            more[preset] = decode_leg(torch, tq, wk, args.splits)
        more["store_sweep"] = store_sweep(torch, tq, 50, presets=MORE_PRESETS)
        more["dequant"] = dequant_sweep(torch, tq, 20, presets=MORE_PRESETS)
        log(f"[more store] {json.dumps({k: round(v['mtok_s'], 1) for k, v in more['store_sweep'].items() if k != 'copy'})}; "
            f"[more dequant] {json.dumps({k: round(v['gbs']) for k, v in more['dequant'].items()})} GB/s")
        extra["more_presets"] = more
        # head_dim 256: decode on the hd256 shape, store and dequant sweeps
        h256 = {}
        for preset in HEAD256_PRESETS:
            wk = W.scaled(W.WORKLOADS["hd256"], name=f"hd256/{preset}", preset=preset)
            h256[preset] = decode_leg(torch, tq, wk, args.splits)
        h256["store_sweep"] = store_sweep(torch, tq, 50, presets=HEAD256_PRESETS, head_dim=256)
        h256["dequant"] = dequant_sweep(torch, tq, 20, presets=HEAD256_PRESETS, head_dim=256)
        log(f"[hd256 store] {json.dumps({k: round(v['mtok_s'], 1) for k, v in h256['store_sweep'].items() if k != 'copy'})}; "
            f"[hd256 dequant] {json.dumps({k: round(v['gbs']) for k, v in h256['dequant'].items()})} GB/s")
        extra["head256"] = h256
        # the opt-in sparse-V gate at 1e-3 (the pages' threshold), and with the
        # softmax scale x4 (attention concentrated on few tokens), gated vs not
        sv = {"value_gate": SPARSE_V_GATE}
        for name, S in (("llama8b", args.splits), ("longctx", 32), ("qwen32b", args.splits)):
            sv[name] = decode_leg(torch, tq, W.WORKLOADS[name], S, value_gate=SPARSE_V_GATE)
        for name, S in (("llama8b", args.splits), ("qwen32b", args.splits)):
            sv[f"{name}_scale_x4"] = {
                "ungated": decode_leg(torch, tq, W.WORKLOADS[name], S, scale_mult=4.0),
                "gated": decode_leg(torch, tq, W.WORKLOADS[name], S, value_gate=SPARSE_V_GATE, scale_mult=4.0)}
        extra["sparse_v"] = sv
        # sliding window + attention sinks: long context with an 8192-token window
        wk = W.WORKLOADS["longctx"]
        extra["window_sinks"] = decode_leg(torch, tq, wk, 32, sliding_window=8192,
                                           sinks=np.random.default_rng(0).uniform(-2, 6, wk.num_q_heads))
        extra["window_sinks"]["workload"] = "longctx, sliding_window 8192, per-head sinks"

    cpu = None if args.no_cpu_baseline else cpu_baseline(w)
    s1 = head["stage1_us"]["median"]
    st1_gbs = head["bytes_read"] / (s1 * 1e-6) / 1e9
    dec = head["decode_call_us"]["median"]
    line = {
        "metric": "TQ decode-attn effective HBM GB/s (% of peak) + store Mtok/s, k8v4/3bit_nc",
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama8b: k8v4 decode step, 32 seqs x 4096 tokens, 32/8 heads, head_dim 128, block 16",
                   "global_batch": w.batch, "seq_len": int(w.seq_len), "num_kv_splits": args.splits,
                   "frac_hbm_peak": gbs / HBM_PEAK_GBS, "bytes_read_per_step": head["bytes_read"],
                   "step_us": head["step_us"], "decode_call_us": head["decode_call_us"],
                   "decode_call_gbs": head["decode_gbs"], "decode_call_frac_hbm_peak": head["decode_frac_hbm"],
                   "decode_call_frac_stream_read": head["decode_gbs"] / stream["gbs_median"],
                   "decode_call_frac_gather_read": head["decode_gbs"] / head["gather_read_gbs"]},
        "roofline": {"bound": "hbm", "achieved": st1_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": st1_gbs / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": "tq_decode_stage1_kernel<k8v4>", "stage1_us": head["stage1_us"],
                     "stream_read_gbs": stream["gbs_median"], "frac_of_stream_read": st1_gbs / stream["gbs_median"],
                     "stream_read": stream, "gather_read_gbs": head["gather_read_gbs"],
                     "frac_of_gather_read": st1_gbs / head["gather_read_gbs"]},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
