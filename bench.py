#!/usr/bin/env python3
"""Benchmark: exact split-KV attention decode on one MI355X.

Default workload (the headline): long-context GQA decode, B=1, 32 query heads
/ 8 KV heads, d=128, L = 1,048,576 cached tokens, bf16 K/V/Q ~ N(0,1) with one
planted needle key per KV head (scaled logit ~30), fp32 accumulation, fp32 O
and lse.  One step = one full decode call (split-KV kernel + merge kernel).
Other workload shapes are selectable with --workload.

Prints one JSON line: KV tokens/s (value), whole-path HBM GB/s against the
8 TB/s peak, the roofline record of the dominant kernel (its per-launch time
from HIP events recorded on the stream it runs on), and the fp64 CPU oracle
timed on a bounded sample of the same workload.  Whole-call times are also
given as median / 10th / 90th percentile, for the back-to-back timed calls
(call_ms) and for calls that each follow a 1 GiB read evicting L2 and the
Infinity Cache (call_ms_cold_cache; the bifurcated batch, ~203 MB, would
otherwise stay cache-resident between calls), and for the call captured once
into a HIP graph and replayed (call_ms_graph, with the wall time per replay).
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KV tokens/s and achieved HBM GB/s (% of peak), 1M-token GQA decode"
PEAK_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
WORKLOADS = {
    "long_context_1m": "long-context GQA decode (1M tokens)",
    "long_context_5m": "long-context GQA decode (5.12M tokens)",
    "llama3_8b_gqa": "Llama-3-8B-shaped GQA decode (B=8, L=32768)",
    "llama31_70b_ragged": "Llama-3.1-70B-shaped ragged decode (B=16, 4 causal query tokens)",
    "single_query_fp32": "single-query fp32 decode (L=4096, 8 chunks)",
    "bifurcated_prefix": "bifurcated shared-prefix sampling (64 samples, 16384 + 512 tokens)",
    "long_context_1m_energy": "long-context GQA energy only, lse from K (1M tokens)",
    "long_context_1m_zeta": "long-context GQA energy F(zeta) from K and V (1M tokens)",
    "paged_long_context_1m": "long-context GQA decode (1M tokens) in 16-token head-major pages",
    "paged_llama31_70b_ragged": "Llama-3.1-70B-shaped ragged decode in 16-token token-major pages",
    "anchor_prefill": "anchor-block context encoding: 2 blocks of 8192 tokens behind an 8192-token "
                      "anchor (Hq=32, Hkv=8, d=128)",
}
# Workloads that reuse another one's inputs: name -> (inputs of, call mode, paging)
VARIANTS = {
    "long_context_1m_energy": ("long_context_1m", "energy", None),
    "long_context_1m_zeta": ("long_context_1m", "zeta", None),
    "paged_long_context_1m": ("long_context_1m", "full", (16, "head_major")),
    "paged_llama31_70b_ragged": ("llama31_70b_ragged", "full", (16, "token_major")),
}
# rocprofv3 counter summaries (HBM bytes per launch of the dominant kernel),
# one per workload.  A summary's figures are used only while the kernel
# sources it lists still hash to its source_sha256.
COUNTERS = {
    "long_context_1m": "profiles/split_kv_valu_long_context_1m.counters.txt",
    "long_context_1m_energy": "profiles/split_kv_valu_energy_long_context_1m.counters.txt",
    "paged_long_context_1m": "profiles/split_kv_valu_paged_long_context_1m.counters.txt",
    "llama31_70b_ragged": "profiles/split_kv_mfma_llama31_70b_ragged.counters.txt",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--min-warmup-s", type=float, default=0.5,
                    help="keep warming up until this much wall time has passed (clock ramp)")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="long_context_1m")
    ap.add_argument("--cpu-rows", type=int, default=32,
                    help="query rows of the workload the CPU oracle baseline computes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the HBM read-stream reference measurement")
    ap.add_argument("--page-size", type=int, default=0,
                    help="paged workloads: tokens per page (0: the workload's own, 16)")
    ap.add_argument("--graph-calls", type=int, default=100,
                    help="extra calls replayed from a captured HIP graph (0: skip)")
    ap.add_argument("--cold-calls", type=int, default=20,
                    help="extra calls after the timed steps, each behind a 1 GiB read that "
                         "evicts L2 and the Infinity Cache (0: skip)")
    return ap.parse_args()


# ----------------------------------------------------------------------------
# Reference figures
# ----------------------------------------------------------------------------
def source_hash(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_traffic(workload):
    """HBM bytes per dominant-kernel launch from the workload's committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, each scaled by its
    copy-kernel calibration factor), or None when there is none or the kernel
    sources changed since it was taken."""
    path = os.path.join(ROOT, COUNTERS.get(workload, "-"))
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.lstrip().startswith("#"):
                key, val = line.split("=", 1)
                kv[key.strip()] = val.strip()
    files = [f.strip() for f in kv.get("sources", "").split(",") if f.strip()]
    if not files or kv.get("source_sha256") != source_hash(files):
        return None
    return float(kv["traffic_bytes_per_launch"])


def read_ceiling(torch):
    """Best HBM read bandwidth of the reference stream kernel (non-temporal
    16-byte loads, one 256-thread block per CU) over a 4 GiB buffer."""
    import ctypes
    from long_context_exact_split_amd import hbm_probe
    lib = hbm_probe.load()
    n = 4 << 30
    src = torch.empty(n // 4, dtype=torch.int32, device="cuda").random_()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(cus, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    best = 0.0
    for rep in range(13):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        lib.hbm_read_probe(ctypes.c_void_p(src.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()),
                           cus, 1, ctypes.c_void_p(s.cuda_stream))
        b.record(s)
        torch.cuda.synchronize()
        if rep >= 3:
            best = max(best, n / (a.elapsed_time(b) * 1e-3) / 1e9)
    del src
    return best


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return 1


# ----------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------
def make_workload(name):
    from long_context_exact_split_amd import inputs
    if name in VARIANTS:
        return make_workload(VARIANTS[name][0])
    if name == "long_context_1m":
        return inputs.long_context_gqa(L=1 << 20, seed=31)
    if name == "long_context_5m":
        return inputs.long_context_gqa(L=5_120_000, seed=3)
    if name == "llama3_8b_gqa":
        return inputs.llama3_8b_gqa(seed=2)
    if name == "llama31_70b_ragged":
        return inputs.llama31_70b_ragged(seed=5)
    if name == "single_query_fp32":
        return inputs.single_query_fp32(seed=1)
    if name == "bifurcated_prefix":
        return inputs.bifurcated_prefix(seed=4)
    if name == "anchor_prefill":
        return inputs.anchor_blocks(seed=6)
    raise ValueError(name)


def dev(torch, a):
    import numpy as np
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class DecodeRunner:
    """One decode call split into its two launches (split kernel, merge).

    mode "full": O and lse; "energy": lse from K alone; "zeta": the energy
    F(zeta) from K and V, one call (split + merge, timed together).  paging
    (P, layout): the cache is scattered into P-token pages in a seeded random
    physical order first (outside the timed region)."""

    def __init__(self, torch, w, mode="full", paging=None):
        import numpy as np
        from long_context_exact_split_amd import binding, inputs
        self.w, self.mode, self.binding = w, mode, binding
        self.pc = None
        q = dev(torch, w.q)
        lens = None
        if not (w.kv_lens == w.L_max).all() or paging is not None:
            lens = torch.from_numpy(w.kv_lens.astype(np.int32)).cuda()
        paged = None
        if paging is not None:
            P, layout = paging
            self.pc = inputs.page_cache(w, P, layout=layout, seed=11)
            shape = ((self.pc.num_pages, w.Hkv, P, w.D) if layout == "head_major"
                     else (self.pc.num_pages, P, w.Hkv, w.D))
            k = dev(torch, self.pc.k_pool.reshape(shape))
            v = dev(torch, self.pc.v_pool.reshape(shape))
            table = torch.from_numpy(self.pc.block_table).cuda()
            paged = binding.PagedCache(k, v, table, layout=layout, max_kv_len=w.L_max)
        else:
            k, v = dev(torch, w.k), dev(torch, w.v)
        self.q, self.k, self.v, self.lens = q, k, v, lens
        if mode == "zeta":
            rng = np.random.default_rng(17)
            z = rng.standard_normal(w.q.shape).astype(np.float32) * np.float32(0.25)
            if w.dtype == "bf16":
                z = inputs.bf16_to_f32(inputs.f32_to_bf16(z))  # the values the GPU sees
            self.zeta_host = z
            self.zeta = dev(torch, inputs.f32_to_bf16(z) if w.dtype == "bf16" else z)
            self.lse = torch.empty(w.q.shape[:3], dtype=torch.float32, device="cuda")
            desc = binding.make_desc(batch=w.B, q_len=w.q_len, num_q_heads=w.Hq,
                                     num_kv_heads=w.Hkv, head_dim=w.D, max_kv_len=w.L_max)
            self.ws = torch.empty(max(1, binding.workspace_bytes(desc)), dtype=torch.uint8,
                                  device="cuda")
            self.plan = binding.plan(desc)
            self.plan["kernel"] = 0  # F(zeta) always runs on the vector-ALU kernel
        else:
            self.ph_args = ((q, k, None if mode == "energy" else v, lens),
                            dict(scale=w.scale, causal=w.causal, chunk_len=w.chunk_len, paged=paged))
            self.ph = binding.Phases(*self.ph_args[0], **self.ph_args[1])
            self.plan = self.ph.plan
        esz = 2 if w.dtype == "bf16" else 4
        self.kv_tokens = int(w.kv_lens.sum())
        tensors = 1 if mode == "energy" else 2
        self.kv_bytes = tensors * self.kv_tokens * w.Hkv * w.D * esz
        self.q_bytes = w.B * w.q_len * w.Hq * w.D * esz * (2 if mode == "zeta" else 1)
        self.out_bytes = w.B * w.q_len * w.Hq * ((w.D + 1) if mode == "full" else 1) * 4
        rows = w.G * w.q_len
        self.flops = 2 * tensors * rows * w.D * self.kv_tokens * w.Hkv
        name = {0: "split_kv_valu", 1: "split_kv_mfma", 2: "split_kv_mfma_rows"}[self.plan["kernel"]]
        self.kernel = f"{name}<{w.dtype},{w.D},rows={self.plan['rows_per_block']}" + \
            ("" if mode == "full" else f",{mode}") + \
            ("" if paging is None else f",pages={paging[0]} {paging[1]}") + ">" + \
            (" + merge (one call)" if mode == "zeta" else "")

    def first(self):
        if self.mode == "zeta":
            w = self.w
            self.binding.decode_energy_zeta(self.q, self.k, self.v, self.zeta, self.lens,
                                            scale=w.scale, causal=w.causal, lse=self.lse,
                                            workspace=self.ws)
        else:
            self.ph.partials()

    def second(self):
        if self.mode != "zeta":
            self.ph.merge()

    def make_graph_call(self):
        """The call on buffers of its own, bound to the current stream (for
        capture into a HIP graph); None when not capturable as is."""
        if self.mode == "zeta":
            return None
        ph = self.binding.Phases(*self.ph_args[0], **self.ph_args[1])

        def call():
            ph.partials()
            ph.merge()
        return call

    def outputs(self):
        if self.mode == "zeta":
            return None, self.lse.cpu().numpy()
        return (None if self.ph.out is None else self.ph.out.cpu().numpy()), self.ph.lse.cpu().numpy()

    def oracle_rows(self, n_rows):
        w = self.w
        rows = [(b, i, h) for b in range(w.B) for i in range(w.q_len) for h in range(w.Hq)]
        step = max(1, len(rows) // n_rows)
        return rows[::step][:n_rows]

    def oracle(self, rows):
        import oracle
        w = self.w
        if self.mode == "zeta":
            return None, oracle.energy_rows(w.q, w.k, w.v, w.kv_lens, w.scale, self.zeta_host,
                                            w.causal, rows=rows)
        v = None if self.mode == "energy" else w.v
        if self.pc is not None:
            pc = self.pc
            return oracle.attend_paged(w.q, pc.k_pool, pc.v_pool, pc.block_table, w.kv_lens,
                                       w.scale, page_size=pc.page_size,
                                       page_stride=pc.page_stride, head_stride=pc.head_stride,
                                       token_stride=pc.token_stride, num_kv_heads=w.Hkv,
                                       L_max=w.L_max, causal=w.causal, rows=rows)
        return oracle.attend(w.q, w.k, v, w.kv_lens, w.scale, w.causal, rows=rows)


class BifurcatedRunner:
    """The shared-prefix call, timed as one unit (three launches)."""

    def __init__(self, torch, w):
        from long_context_exact_split_amd import binding
        self.w, self.binding = w, binding
        self.t = [dev(torch, x) for x in (w.q, w.kp, w.vp, w.ks, w.vs)]
        self.call = binding.BifurcatedCall(*self.t, scale=w.scale)
        self.out, self.lse = self.call.out, self.call.lse
        self.plan = {"prefix_rows": w.S * w.G, "workspace_bytes": self.call.nbytes}
        self.kv_tokens = w.S * (w.Lp + w.Ls)             # logical tokens attended
        self.kv_bytes = 2 * (w.Lp + w.S * w.Ls) * w.Hkv * w.D * 2   # physical bytes read
        self.q_bytes = w.S * w.Hq * w.D * 2
        self.out_bytes = w.S * w.Hq * (w.D + 1) * 4
        self.flops = 4 * w.S * w.Hq * w.D * (w.Lp + w.Ls)
        self.kernel = "bifurcated (prefix split kernel + suffix split kernel + merge)"

    def first(self):
        self.call.run()

    def make_graph_call(self):
        call = self.binding.BifurcatedCall(*self.t, scale=self.w.scale)
        return call.run

    def second(self):
        pass

    def outputs(self):
        return self.out.cpu().numpy()[:, None], self.lse.cpu().numpy()[:, None]

    def oracle_rows(self, n_rows):
        w = self.w
        rows = [(s, 0, h) for s in range(w.S) for h in range(w.Hq)]
        step = max(1, len(rows) // n_rows)
        return rows[::step][:n_rows]

    def oracle(self, rows):
        import oracle
        w = self.w
        samples = sorted({s for (s, _, _) in rows})
        O, lse = oracle.attend_bifurcated(w.q, w.kp, w.vp, w.ks, w.vs, w.scale, samples=samples)
        return O[:, None], lse[:, None]


class AnchorRunner:
    """One anchor-block context encoding call (anchor split, local split,
    merge), timed as one unit; bound by the matrix cores."""

    def __init__(self, torch, w):
        from long_context_exact_split_amd import binding
        self.w, self.binding = w, binding
        self.t = [dev(torch, x) for x in (w.q, w.ka, w.va, w.kb, w.vb)]
        N, Lb, Hq, D = w.q.shape
        Hkv, A = w.Hkv, w.A
        self.out = torch.empty((N, Lb, Hq, D), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((N, Lb, Hq), dtype=torch.float32, device="cuda")
        desc = binding.anchor_desc(self.t[0], self.t[1], self.t[3], w.scale)
        import ctypes
        n = ctypes.c_size_t(0)
        assert binding.load_library().attn_anchor_workspace_bytes(ctypes.byref(desc),
                                                                  ctypes.byref(n)) == 0
        self.ws = torch.empty(max(1, n.value), dtype=torch.uint8, device="cuda")
        self.plan = {"blocks": N, "block_len": Lb, "anchor_len": A, "workspace_bytes": n.value}
        self.kv_tokens = N * (A + Lb)
        self.kv_bytes = 2 * (A + N * Lb) * Hkv * D * 2
        self.q_bytes = N * Lb * Hq * D * 2
        self.out_bytes = N * Lb * Hq * (D + 1) * 4
        G = Hq // Hkv
        # visible (query row, key) pairs: every anchor key, and the causal triangle
        pairs = N * Hkv * G * (Lb * A + Lb * (Lb + 1) // 2)
        self.flops = 4 * D * pairs
        self.kernel = "anchor prefill (anchor split + local causal split + merge)"

    def first(self):
        self.binding.prefill_anchor(*self.t, scale=self.w.scale, out=self.out, lse=self.lse,
                                    workspace=self.ws)

    def second(self):
        pass

    def outputs(self):
        return self.out.cpu().numpy(), self.lse.cpu().numpy()

    def oracle_rows(self, n_rows):
        w = self.w
        N, Lb, Hq, _ = w.q.shape
        rows = [(b, i, h) for b in range(N) for i in (0, Lb // 3, Lb - 1) for h in range(Hq)]
        return rows[:: max(1, len(rows) // n_rows)][:n_rows]

    def oracle(self, rows):
        import oracle
        w = self.w
        return oracle.attend_anchor_blocks(w.q, w.ka, w.va, w.kb, w.vb, w.scale, rows=rows)


def cpu_baseline(run, n_rows, O_gpu, lse_gpu):
    """Time the fp64 oracle on a sample of the workload's query rows (each row
    over its full visible cache) and check the GPU's values on those rows."""
    import numpy as np
    rows = run.oracle_rows(n_rows)
    t0 = time.perf_counter()
    Or, lr = run.oracle(rows)
    dt = time.perf_counter() - t0
    idx = tuple(np.array(rows).T)
    dO = float(np.abs(O_gpu[idx] - Or[idx]).max()) if O_gpu is not None and Or is not None else None
    fin = np.isfinite(lr[idx])
    dl = float((np.abs(lse_gpu[idx][fin] - lr[idx][fin]) /
                np.maximum(1.0, np.abs(lr[idx][fin]))).max()) if fin.any() else 0.0
    total_rows = lse_gpu.shape[0] * lse_gpu.shape[1] * lse_gpu.shape[2]
    frac = len(rows) / total_rows
    return {"value": run.kv_tokens * frac / dt, "unit": "KV tokens/s", "cores": int(cpu_threads()),
            "kind": "oracle",
            "sample": f"{len(rows)} of {total_rows} query rows, each over its whole visible cache "
                      f"({dt:.2f} s); rate = KV tokens of the call x {len(rows)}/{total_rows} / time",
            "seconds": dt, "parity_max_abs_dO": dO, "parity_max_rel_dlse": dl}


FLUSH_BYTES = 1 << 30  # > 8 x 4 MB L2 + 256 MB Infinity Cache


def spread(ms):
    """Median, 10th and 90th percentile of a list of call times (ms)."""
    xs = sorted(ms)

    def pct(p):
        return xs[min(len(xs) - 1, max(0, int(round(p / 100 * (len(xs) - 1)))))]
    return {"median": statistics.median(xs), "p10": pct(10), "p90": pct(90), "calls": len(xs)}


def cold_calls(torch, run, n):
    """Whole-call times (HIP events around every launch of the call) with the
    caches cleared before each call by a 1 GiB read, outside the events.  A
    read rather than a write: evicted dirty lines would otherwise be written
    back to HBM while the timed call runs."""
    stream = torch.cuda.current_stream()
    junk = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for i in range(n):
        torch.amax(junk)
        ev[i][0].record(stream)
        run.first()
        run.second()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    del junk
    out = spread([a.elapsed_time(b) for a, b in ev])
    out["flush_bytes"] = FLUSH_BYTES
    return out


def graph_calls(torch, run, n):
    """Whole-call times when the call is captured once into a HIP graph and
    replayed (no per-call host work: what a serving loop would do).  The call
    gets buffers of its own, bound to a side stream that is captured."""
    make = getattr(run, "make_graph_call", None)
    if make is None:
        return None
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        call = make()
        if call is None:
            return None
        for _ in range(3):
            call()
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < 0.3:  # clocks up again
        g.replay()
    for i in range(n):
        ev[i][0].record(stream)
        g.replay()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        g.replay()
    torch.cuda.synchronize()
    out = spread([a.elapsed_time(b) for a, b in ev])
    out["wall_ms_per_call"] = (time.perf_counter() - t0) * 1e3 / n
    del g
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the path runs on one GPU; --gpus must be 1 "
                                   "(sharding the KV cache across GPUs is not implemented)"}))
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    t_gen = time.perf_counter()
    w = make_workload(args.workload)
    print(f"# generated {args.workload} in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr,
          flush=True)
    if args.workload == "bifurcated_prefix":
        run = BifurcatedRunner(torch, w)
    elif args.workload == "anchor_prefill":
        run = AnchorRunner(torch, w)
    else:
        _, mode, paging = VARIANTS.get(args.workload, (None, "full", None))
        if paging is not None and args.page_size:
            paging = (args.page_size, paging[1])
        run = DecodeRunner(torch, w, mode, paging)
    print(f"# plan {run.plan}", file=sys.stderr, flush=True)

    K = args.steps
    # Events are created before the warm-up: creating them afterwards would
    # leave the GPU idle long enough for its clocks to drop again.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    stream = torch.cuda.current_stream()

    # Untimed warm-up: at least --warmup steps and --min-warmup-s seconds.  From
    # idle the GPU needs ~30-40 back-to-back steps (~25 ms) to reach its
    # steady clocks; the timed region measures the steady state.
    warm, t_w = 0, time.perf_counter()
    while warm < args.warmup or time.perf_counter() - t_w < args.min_warmup_s:
        run.first()
        run.second()
        warm += 1
        if warm % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()  # barrier (one rank)
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        run.first()
        ev[i][1].record(stream)
        run.second()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    first_ms = [e[0].elapsed_time(e[1]) for e in ev]
    second_ms = [e[1].elapsed_time(e[2]) for e in ev]
    call_ms = [e[0].elapsed_time(e[2]) for e in ev]

    step_ms = wall * 1e3 / K
    first_avg = statistics.mean(first_ms)
    alg = run.kv_bytes + run.q_bytes
    dom_gbps = alg / (first_avg * 1e-3) / 1e9
    path_gbps = (alg + run.out_bytes) / (step_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": run.kv_tokens / (step_ms * 1e-3),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "warmup_steps_run": warm,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": getattr(w, "dtype", "bf16"),
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload], **run.plan},
        "hbm_gbps": path_gbps,
        "hbm_frac_of_peak": path_gbps / PEAK_GBPS,
        "dominant_kernel_ms": first_avg,
        "dominant_kernel_ms_median": statistics.median(first_ms),
        "second_launch_ms": statistics.mean(second_ms),
        "call_ms": spread(call_ms),
        "tflops": run.flops / (first_avg * 1e-3) / 1e12,
        "roofline": {"bound": "hbm", "achieved": dom_gbps, "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": dom_gbps / PEAK_GBPS, "traffic": counter_traffic(args.workload),
                     "kernel": run.kernel, "algorithmic_bytes_per_launch": alg},
    }
    if args.workload == "bifurcated_prefix":
        result["kv_tokens_physical"] = w.Lp + w.S * w.Ls
    if args.workload == "anchor_prefill":
        # A dense contraction (256 and more query rows per KV tile): bound by
        # the bf16 matrix cores, priced against their dense peak.
        tf = result["tflops"]
        result["roofline"] = {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
                              "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS, "traffic": None,
                              "kernel": run.kernel, "algorithmic_flops_per_launch": run.flops}
    if args.cold_calls > 0:
        result["call_ms_cold_cache"] = cold_calls(torch, run, args.cold_calls)
    if args.graph_calls > 0:
        result["call_ms_graph"] = graph_calls(torch, run, args.graph_calls)
    if not args.no_ceiling:
        ceil = read_ceiling(torch)
        result["hbm_read_ceiling_gbps"] = ceil
        result["roofline"]["frac_of_read_ceiling"] = dom_gbps / ceil
    if not args.no_cpu_baseline:
        O, lse = run.outputs()
        result["cpu_baseline"] = cpu_baseline(run, args.cpu_rows, O, lse)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
