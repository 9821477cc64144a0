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
timed on a bounded sample of the same workload.  Events bracket one timed
step in four (event_every; every step when there are fewer than 40), so that
the markers they put in the stream leave the other steps' time untouched.
Whole-call times are also given as median / 10th / 90th percentile, for the
event-timed calls (call_ms) and for calls that each follow a 1 GiB read evicting L2 and the
Infinity Cache (call_ms_cold_cache; the bifurcated batch, ~203 MB, would
otherwise stay cache-resident between calls), and for the call captured once
into a HIP graph and replayed (call_ms_graph, with the wall time per replay).

With the default workload the same line also carries ``configs``: every other
measured configuration (single-query fp32, Llama-3-8B-shaped GQA, the
5.12M-token cache with its energy-only and F(zeta) calls, the shared-prefix
batch and the Llama-3.1-70B-shaped ragged batch), each timed the same way and
checked against the oracle on sampled rows.  The run exits non-zero when any
sampled row misses the parity bar.
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
O_TOL, LSE_RTOL = 2e-3, 1e-4   # parity bar: max|dO|, |dlse| / max(1, |lse|)
WORKLOADS = {
    "long_context_1m": "long-context GQA decode (1M tokens)",
    "long_context_5m": "long-context GQA decode (5.12M tokens)",
    "long_context_5m_energy": "long-context GQA energy only, lse from K (5.12M tokens)",
    "long_context_5m_zeta": "long-context GQA energy F(zeta) from K and V (5.12M tokens)",
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
    "long_context_5m_share8": "one device's share of the 5.12M-token GQA decode cut into 8 token "
                              "shares (640,000 tokens) + the merge of the 8 shares' (O, lse)",
}
# Workloads that reuse another one's inputs: name -> (inputs of, call mode, paging)
VARIANTS = {
    "long_context_1m_energy": ("long_context_1m", "energy", None),
    "long_context_1m_zeta": ("long_context_1m", "zeta", None),
    "long_context_5m_energy": ("long_context_5m", "energy", None),
    "long_context_5m_zeta": ("long_context_5m", "zeta", None),
    "paged_long_context_1m": ("long_context_1m", "full", (16, "head_major")),
    "paged_llama31_70b_ragged": ("llama31_70b_ragged", "full", (16, "token_major")),
    "long_context_5m_share8": ("long_context_5m", "share8", None),
}
# The configurations reported beside the headline: (workload, timed steps,
# oracle rows sampled for parity).  Steps follow the per-config iteration
# counts of the measurement plan; rows are chosen so that the oracle (which
# reads every key of a row's KV head) stays within seconds.
CONFIGS = [
    ("single_query_fp32", 200, None),
    ("llama3_8b_gqa", 50, 16),
    ("long_context_5m", 10, 8),
    ("long_context_5m_energy", 10, 8),
    ("long_context_5m_zeta", 10, 2),
    ("long_context_5m_share8", 50, 8),
    ("bifurcated_prefix", 200, 16),
    ("llama31_70b_ragged", 30, 16),
]
# Configs whose oracle is also timed on one core (small enough to do whole).
ONE_CORE = ("single_query_fp32", "llama3_8b_gqa")
# rocprofv3 counter summaries (HBM bytes per launch of the dominant kernel),
# one per workload.  A summary's figures are used only while the kernel
# sources it lists still hash to its source_sha256.
COUNTERS = {
    "long_context_1m": "profiles/split_kv_valu_long_context_1m.counters.txt",
    "long_context_1m_energy": "profiles/split_kv_valu_energy_long_context_1m.counters.txt",
    "paged_long_context_1m": "profiles/split_kv_valu_paged_long_context_1m.counters.txt",
    "llama31_70b_ragged": "profiles/split_kv_mfma_llama31_70b_ragged.counters.txt",
    "llama3_8b_gqa": "profiles/split_kv_valu_llama3_8b_gqa.counters.txt",
    "long_context_5m": "profiles/split_kv_valu_long_context_5m.counters.txt",
    "bifurcated_prefix": "profiles/bifurcated_call_bifurcated_prefix.counters.txt",
    "long_context_5m_share8": "profiles/split_kv_valu_long_context_5m_share8.counters.txt",
    "long_context_5m_energy": "profiles/split_kv_valu_energy_long_context_5m.counters.txt",
    "long_context_5m_zeta": "profiles/split_kv_valu_zeta_long_context_5m.counters.txt",
}


def parse(argv=None):
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
    ap.add_argument("--no-configs", action="store_true",
                    help="do not measure the other configurations beside the headline")
    ap.add_argument("--page-size", type=int, default=0,
                    help="paged workloads: tokens per page (0: the workload's own, 16)")
    ap.add_argument("--graph-calls", type=int, default=100,
                    help="extra calls replayed from a captured HIP graph (0: skip)")
    ap.add_argument("--cold-calls", type=int, default=20,
                    help="extra calls after the timed steps, each behind a 1 GiB read that "
                         "evicts L2 and the Infinity Cache (0: skip)")
    ap.add_argument("--wg-stamps", type=int, default=0, metavar="REPS",
                    help="instead of the bench line: time every workgroup of the vector-ALU "
                         "split kernel (start, end, XCD) over REPS launches with the "
                         "stamping build of the library, and print a per-XCD summary")
    return ap.parse_args(argv)


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


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


# ----------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------
_WORKLOAD_CACHE = {}


def make_workload(name):
    from long_context_exact_split_amd import inputs
    if name in VARIANTS:
        return make_workload(VARIANTS[name][0])
    if name in _WORKLOAD_CACHE:
        return _WORKLOAD_CACHE[name]
    if name == "long_context_1m":
        w = inputs.long_context_gqa(L=1 << 20, seed=31)
    elif name == "long_context_5m":
        w = inputs.long_context_gqa(L=5_120_000, seed=3)
    elif name == "llama3_8b_gqa":
        w = inputs.llama3_8b_gqa(seed=2)
    elif name == "llama31_70b_ragged":
        w = inputs.llama31_70b_ragged(seed=5)
    elif name == "single_query_fp32":
        w = inputs.single_query_fp32(seed=1)
    elif name == "bifurcated_prefix":
        w = inputs.bifurcated_prefix(seed=4)
    elif name == "anchor_prefill":
        w = inputs.anchor_blocks(seed=6)
    else:
        raise ValueError(name)
    _WORKLOAD_CACHE[name] = w
    return w


def dev(torch, a):
    import numpy as np
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


_DEVICE_CACHE = {}


def device_kv(torch, w):
    """q, k, v of a workload on the GPU, uploaded once per workload (the
    5.12M-token cache serves three configs)."""
    key = id(w)
    if key not in _DEVICE_CACHE:
        _DEVICE_CACHE[key] = (dev(torch, w.q), dev(torch, w.k), dev(torch, w.v))
    return _DEVICE_CACHE[key]


def forget(torch, w):
    _DEVICE_CACHE.pop(id(w), None)
    for k, v in list(_WORKLOAD_CACHE.items()):
        if v is w:
            del _WORKLOAD_CACHE[k]
    torch.cuda.empty_cache()


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
        lens = None
        if not (w.kv_lens == w.L_max).all() or paging is not None:
            lens = torch.from_numpy(w.kv_lens.astype(np.int32)).cuda()
        paged = None
        if paging is not None:
            P, layout = paging
            self.pc = inputs.page_cache(w, P, layout=layout, seed=11)
            shape = ((self.pc.num_pages, w.Hkv, P, w.D) if layout == "head_major"
                     else (self.pc.num_pages, P, w.Hkv, w.D))
            q = dev(torch, w.q)
            k = dev(torch, self.pc.k_pool.reshape(shape))
            v = dev(torch, self.pc.v_pool.reshape(shape))
            table = torch.from_numpy(self.pc.block_table).cuda()
            paged = binding.PagedCache(k, v, table, layout=layout, max_kv_len=w.L_max)
        else:
            q, k, v = device_kv(torch, w)
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
        self.bound = "hbm"

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
        """n_rows rows spread over the call; with planted needles, the needle
        rows (the group's first query head, whose logit the needle dominates)
        come first."""
        w = self.w
        rows = [(b, i, h) for b in range(w.B) for i in range(w.q_len) for h in range(w.Hq)]
        first = [(b, 0, w.G * kvh) for (b, kvh, _) in w.notes.get("needles", [])]
        rest = [r for r in rows if r not in set(first)]
        step = max(1, len(rest) // max(1, n_rows - len(first)))
        return (first + rest[::step])[:n_rows]

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

    def row_groups(self, rows):
        """Rows split into independent oracle calls: one per (sequence, KV head)."""
        G = self.w.G
        groups = {}
        for r in rows:
            groups.setdefault((r[0], r[2] // G), []).append(r)
        return list(groups.values())


class ShardRunner(DecodeRunner):
    """Sequence sharding as one device of N sees it: the cache's token axis
    is cut into N equal shares (one per device); a step decodes this device's
    share (share 0, at its real shape: split kernel, then its merge into
    slot 0 of the parts buffer) and merges the N shares' (O, lse) with
    attn_merge_results (the exchange step after an all-gather of the parts;
    the other N - 1 parts are computed once beforehand, from the same cache).
    The merged rows are the whole cache's: parity is against the oracle over
    all of it."""

    def __init__(self, torch, w, n=8):
        from long_context_exact_split_amd import binding
        self.w, self.mode, self.binding, self.pc = w, "full", binding, None
        q, k, v = device_kv(torch, w)
        S = w.L_max // n
        assert S * n == w.L_max and (w.kv_lens == w.L_max).all()
        B, q_len, Hq, D = w.q.shape
        self.parts_o = torch.empty((n, B, q_len, Hq, D), dtype=torch.float32, device="cuda")
        self.parts_lse = torch.empty((n, B, q_len, Hq), dtype=torch.float32, device="cuda")
        for p in range(n - 1, -1, -1):
            ks = k[:, :, p * S:(p + 1) * S].contiguous()
            vs = v[:, :, p * S:(p + 1) * S].contiguous()
            if p:
                binding.decode(q, ks, vs, scale=w.scale, out=self.parts_o[p],
                               lse=self.parts_lse[p])
                del ks, vs
        self.q, self.k, self.v, self.lens = q, ks, vs, None
        self.ph_args = ((q, ks, vs, None), dict(scale=w.scale))
        self.ph = binding.Phases(*self.ph_args[0], **self.ph_args[1])
        self.ph.out, self.ph.lse = self.parts_o[0], self.parts_lse[0]
        self.plan = self.ph.plan
        self.out = torch.empty((B, q_len, Hq, D), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((B, q_len, Hq), dtype=torch.float32, device="cuda")
        self.kv_tokens = S * B
        self.oracle_kv_tokens = w.L_max * B  # the oracle reads the whole cache of a row
        self.kv_bytes = 2 * S * B * w.Hkv * w.D * 2
        self.q_bytes = B * q_len * Hq * D * 2
        self.out_bytes = B * q_len * Hq * (D + 1) * 4
        self.flops = 4 * w.G * q_len * w.D * S * B * w.Hkv
        self.kernel = (f"split_kv_valu<bf16,{w.D},rows={self.plan['rows_per_block']}> on a "
                       f"{S}-token share")
        self.bound = "hbm"
        torch.cuda.synchronize()

    def second(self):
        self.ph.merge()
        self.binding.merge_results(self.parts_o, self.parts_lse, out=self.out, lse=self.lse)

    def make_graph_call(self):
        return None

    def outputs(self):
        return self.out.cpu().numpy(), self.lse.cpu().numpy()


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
        self.prefix_flops = 4 * w.S * w.Hq * w.D * w.Lp
        self.kernel = "bifurcated (prefix split kernel + suffix split kernel + merge)"
        self.bound = "hbm"

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

    def row_groups(self, rows):
        groups = {}
        for r in rows:
            groups.setdefault(r[0], []).append(r)
        return list(groups.values())


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
        self.bound = "mfma"

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

    def row_groups(self, rows):
        groups = {}
        for r in rows:
            groups.setdefault(r[0], []).append(r)
        return list(groups.values())


def make_runner(torch, name, page_size=0):
    w = make_workload(name)
    if name == "bifurcated_prefix":
        return BifurcatedRunner(torch, w)
    if name == "anchor_prefill":
        return AnchorRunner(torch, w)
    _, mode, paging = VARIANTS.get(name, (None, "full", None))
    if mode == "share8":
        return ShardRunner(torch, w, 8)
    if paging is not None and page_size:
        paging = (page_size, paging[1])
    return DecodeRunner(torch, w, mode, paging)


# ----------------------------------------------------------------------------
# The oracle on sampled rows, and parity
# ----------------------------------------------------------------------------
def run_oracle(run, rows, threads):
    """The oracle over `rows`, its independent (sequence, KV head) calls spread
    over `threads` host threads (numpy's BLAS pinned to one thread each, so the
    thread count is the core count used).  Returns (O, lse, seconds, threads
    actually used)."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    groups = run.row_groups(rows)
    used = max(1, min(threads, len(groups)))
    t0 = time.perf_counter()
    with threadpool_limits(limits=1, user_api="blas"):
        if used == 1:
            parts = [run.oracle(g) for g in groups]
        else:
            with ThreadPoolExecutor(used) as ex:
                parts = list(ex.map(run.oracle, groups))
    dt = time.perf_counter() - t0
    O, lse = parts[0]
    for g, (Og, lg) in zip(groups[1:], parts[1:]):
        for r in g:
            lse[r] = lg[r]
            if O is not None:
                O[r] = Og[r]
    return O, lse, dt, used


def parity(rows, O_gpu, lse_gpu, Or, lr):
    """Worst deviations on the sampled rows and whether they meet the bar
    (an empty row must give lse = -inf and O = 0 exactly; NaN never)."""
    import numpy as np
    idx = tuple(np.array(rows).T)
    lg, lo = lse_gpu[idx].astype(np.float64), lr[idx]
    empty = np.isneginf(lo)
    ok = bool(not np.isnan(lg).any() and (lg[empty] == -np.inf).all())
    dl = float((np.abs(lg[~empty] - lo[~empty]) / np.maximum(1.0, np.abs(lo[~empty]))).max()) \
        if (~empty).any() else 0.0
    ok = ok and dl <= LSE_RTOL
    dO = None
    if O_gpu is not None and Or is not None:
        og, oo = O_gpu[idx].astype(np.float64), Or[idx]
        ok = ok and not np.isnan(og).any() and bool((og[empty] == 0).all())
        dO = float(np.abs(og[~empty] - oo[~empty]).max()) if (~empty).any() else 0.0
        ok = ok and dO <= O_TOL
    return {"rows": len(rows), "max_abs_dO": dO, "max_rel_dlse": dl, "ok": bool(ok)}


def cpu_baseline(run, n_rows, O_gpu, lse_gpu):
    """Time the fp64 oracle on a sample of the workload's query rows (each row
    over its full visible cache) and check the GPU's values on those rows."""
    rows = run.oracle_rows(n_rows)
    cores = host_cores()
    Or, lr, dt, used = run_oracle(run, rows, cores)
    total_rows = lse_gpu.shape[0] * lse_gpu.shape[1] * lse_gpu.shape[2]
    frac = len(rows) / total_rows
    par = parity(rows, O_gpu, lse_gpu, Or, lr)
    otok = getattr(run, "oracle_kv_tokens", run.kv_tokens)
    return {"value": otok * frac / dt, "unit": "KV tokens/s", "cores": used,
            "kind": "oracle",
            "sample": f"{len(rows)} of {total_rows} query rows, each over its whole visible cache "
                      f"({dt:.2f} s on {used} threads, one (sequence, KV head) group each); "
                      f"rate = KV tokens of the call x {len(rows)}/{total_rows} / time",
            "seconds": dt, "host_cores": cores, "cpu_model": cpu_model(), "blas_threads": 1,
            "parity_max_abs_dO": par["max_abs_dO"], "parity_max_rel_dlse": par["max_rel_dlse"],
            "parity_ok": par["ok"]}


# ----------------------------------------------------------------------------
# Timing
# ----------------------------------------------------------------------------
FLUSH_BYTES = 1 << 30  # > 8 x 4 MB L2 + 256 MB Infinity Cache


def spread(ms):
    """Median, 10th and 90th percentile of a list of call times (ms)."""
    xs = sorted(ms)

    def pct(p):
        return xs[min(len(xs) - 1, max(0, int(round(p / 100 * (len(xs) - 1)))))]
    return {"median": statistics.median(xs), "p10": pct(10), "p90": pct(90), "calls": len(xs)}


# Steps per event-timed step in the timed region: every event record is a
# marker in the stream that the GPU processes between the launches, measured
# at ~4 us on the shared-prefix call (~67 us per step with three per step,
# ~55 us with none) and ~1 us on the 1M decode.
EVENT_EVERY = 4


def event_stride(K, every=EVENT_EVERY):
    """Event-timed steps are one in `every`, but at least ~10 of the K."""
    return max(1, min(every, K // 10))


def timed_steps(torch, run, K, warmup, min_warmup_s, every=EVENT_EVERY):
    """Untimed warm-up (at least `warmup` steps and `min_warmup_s` seconds:
    from idle the GPU needs ~30-40 back-to-back steps to reach its steady
    clocks), then K steps.  Steps 0, n, 2n, ... (n = event_stride) are
    bracketed by HIP events on the launch stream (before the first launch,
    between the two launches, after the second); the others run without
    markers.  Returns the per-launch event times of those steps and the wall
    time of all K steps."""
    n = event_stride(K, every)
    # Events are created before the warm-up: creating them afterwards would
    # leave the GPU idle long enough for its clocks to drop again.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(0, K, n)]
    stream = torch.cuda.current_stream()
    warm, t_w = 0, time.perf_counter()
    while warm < warmup or time.perf_counter() - t_w < min_warmup_s:
        run.first()
        run.second()
        warm += 1
        if warm % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()  # barrier (one rank)
    t0 = time.perf_counter()
    for i in range(K):
        if i % n:
            run.first()
            run.second()
            continue
        e = ev[i // n]
        e[0].record(stream)
        run.first()
        e[1].record(stream)
        run.second()
        e[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return {"first_ms": [e[0].elapsed_time(e[1]) for e in ev],
            "second_ms": [e[1].elapsed_time(e[2]) for e in ev],
            "call_ms": [e[0].elapsed_time(e[2]) for e in ev], "wall_s": wall, "warmup": warm,
            "event_every": n}


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


def roofline(run, first_avg_ms, workload):
    """Roofline record of the dominant launch (or of the whole call for the
    bifurcated and anchor workloads, which time their launches together)."""
    if run.bound == "mfma":
        tf = run.flops / (first_avg_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": tf / PEAK_BF16_TFLOPS, "traffic": None, "kernel": run.kernel,
                "algorithmic_flops_per_launch": run.flops}
    alg = run.kv_bytes + run.q_bytes
    gbps = alg / (first_avg_ms * 1e-3) / 1e9
    traffic = counter_traffic(workload)
    return {"bound": "hbm", "achieved": gbps, "peak": PEAK_GBPS, "unit": "GB/s",
            "frac": gbps / PEAK_GBPS, "traffic": traffic,
            "traffic_ratio": None if traffic is None else traffic / alg,
            "kernel": run.kernel, "algorithmic_bytes_per_launch": alg}


def measure_config(torch, name, K, n_rows, warmup, min_warmup_s):
    """One configuration beside the headline: timed steps, roofline of its
    dominant launch, whole-call times with cold caches where the inputs fit in
    the Infinity Cache, and oracle parity on sampled rows (with the oracle's
    time on them; one-core times too for the small configs)."""
    w = make_workload(name)
    run = make_runner(torch, name)
    t = timed_steps(torch, run, K, warmup, min_warmup_s)
    first_avg = statistics.mean(t["first_ms"])
    call_avg = statistics.mean(t["call_ms"])
    rec = {"workload": WORKLOADS[name], "seed": getattr(w, "seed", None),
           "dtype": getattr(w, "dtype", "bf16"), "steps": K,
           "ms_per_step": t["wall_s"] * 1e3 / K, "event_every": t["event_every"],
           "call_ms_mean": call_avg,
           "call_ms": spread(t["call_ms"]), "dominant_kernel_ms": first_avg,
           "kv_tokens_per_call": run.kv_tokens,
           "kv_tokens_per_s": run.kv_tokens / (call_avg * 1e-3),
           "roofline": roofline(run, first_avg, name)}
    if isinstance(run, BifurcatedRunner):
        rec["call_ms_cold_cache"] = cold_calls(torch, run, 20)
        rec["kv_tokens_physical"] = w.Lp + w.S * w.Ls
        rec["tflops_counted"] = run.flops / (first_avg * 1e-3) / 1e12
    O, lse = run.outputs()
    rows = run.oracle_rows(n_rows if n_rows else lse.size)
    Or, lr, dt, used = run_oracle(run, rows, host_cores())
    rec["parity"] = parity(rows, O, lse, Or, lr)
    total_rows = lse.size
    otok = getattr(run, "oracle_kv_tokens", run.kv_tokens)  # tokens the oracle's rows read
    rec["oracle"] = {"seconds": dt, "threads": used,
                     "kv_tokens_per_s": otok * len(rows) / total_rows / dt}
    if name in ONE_CORE:
        _, _, dt1, _ = run_oracle(run, rows, 1)
        rec["oracle"]["one_core_seconds"] = dt1
        rec["oracle"]["one_core_kv_tokens_per_s"] = run.kv_tokens * len(rows) / total_rows / dt1
    return rec


def stamp_summary(st, ev_ms):
    """Per-workgroup stamps of one launch ([n, 4]: start, end, XCC id, HW id;
    clocks in 10 ns ticks) -> summary dict (microseconds)."""
    import numpy as np
    t0, t1 = st[:, 0].astype(np.int64), st[:, 1].astype(np.int64)
    base = t0.min()
    start, end, dur = (t0 - base) * 0.01, (t1 - base) * 0.01, (t1 - t0) * 0.01
    xcc = (st[:, 2] & 0xF).astype(np.int64)
    per = {}
    for x in sorted(set(xcc.tolist())):
        sel = xcc == x
        per[str(x)] = {"workgroups": int(sel.sum()),
                       "end_median_us": float(np.median(end[sel])),
                       "end_max_us": float(end[sel].max()),
                       "duration_median_us": float(np.median(dur[sel])),
                       "duration_spread_us": float(dur[sel].max() - dur[sel].min())}
    ends = np.array([v["end_max_us"] for v in per.values()])
    span = float(end.max())
    return {"event_us": ev_ms * 1e3, "span_us": span,
            "start_spread_us": float(start.max()),
            "duration_min_med_max_us": [float(dur.min()), float(np.median(dur)), float(dur.max())],
            "xcd_end_min_max_us": [float(ends.min()), float(ends.max())],
            # if the work had been shared out in proportion to each XCD's own rate
            "balanced_span_us": float(len(ends) / np.sum(1.0 / ends)),
            "xcd": per,
            "wg_duration_us": [round(float(x), 1) for x in dur],
            "wg_hw_id": [int(x) for x in st[:, 3]]}


def wg_stamps(torch, args):
    """Per-workgroup timing of the headline split kernel: after the warm-up,
    REPS launches each following an idle gap (isolated) and, after a run of
    back-to-back steps, the last of them (sustained); then the same for the
    reference share-read kernel over the same bytes and workgroups."""
    import ctypes
    import numpy as np
    from long_context_exact_split_amd import binding
    lib = binding.load_library()
    run = make_runner(torch, args.workload, args.page_size)
    if isinstance(run, BifurcatedRunner):
        return wg_stamps_bifurcated(torch, args, run, lib)
    if run.plan.get("kernel") not in (0, 1) or getattr(run, "mode", "full") == "zeta":
        raise RuntimeError("--wg-stamps covers the decode split kernels (vector-ALU, 32-row MFMA)")
    readback = getattr(lib, ("attn_probe_wg_stamps", "attn_probe_wg_stamps_mfma")[run.plan["kernel"]],
                       None)
    if readback is None:
        raise RuntimeError(f"{binding.library_path()} is not the stamping build")
    readback.argtypes = [ctypes.c_void_p, ctypes.c_int]
    n = int(run.plan["work_items"])
    stream = torch.cuda.current_stream()

    def launch_and_read(back_to_back):
        for _ in range(back_to_back):
            run.first()
            run.second()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        run.first()
        b.record(stream)
        torch.cuda.synchronize()
        st = np.zeros((n, 4), dtype=np.uint64)
        if readback(st.ctypes.data, n) != 0:
            raise RuntimeError("stamp read-back failed")
        run.second()
        torch.cuda.synchronize()
        return stamp_summary(st, a.elapsed_time(b))

    timed_steps(torch, run, 20, args.warmup, args.min_warmup_s)
    out = {"workload": WORKLOADS[args.workload], "kernel": run.kernel, "workgroups": n,
           "library": os.path.basename(binding.library_path()), "isolated": [], "sustained": []}
    for rep in range(args.wg_stamps):
        time.sleep(0.005)
        out["isolated"].append(launch_and_read(0))
        out["sustained"].append(launch_and_read(100))
        print(f"# rep {rep}: isolated {out['isolated'][-1]['event_us']:.1f} us, sustained "
              f"{out['sustained'][-1]['event_us']:.1f} us", file=sys.stderr, flush=True)

    # The same bytes read by the reference share-read kernel (the decode's
    # access pattern without its arithmetic) over as many workgroups.
    from long_context_exact_split_amd import hbm_probe
    probe = hbm_probe.load()
    nbytes = run.kv_bytes // 16 * 16
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").random_()
    sink = torch.zeros(n, dtype=torch.int32, device="cuda")

    def read_and_stamp(back_to_back):
        for _ in range(back_to_back + 1):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            if probe.hbm_read_share_probe(src.data_ptr(), nbytes, sink.data_ptr(), n,
                                          stream.cuda_stream) != 0:
                raise RuntimeError("hbm_read_share_probe failed")
            b.record(stream)
        torch.cuda.synchronize()
        st = np.zeros((n, 4), dtype=np.uint64)
        if probe.attn_probe_wg_stamps(st.ctypes.data, n) != 0:
            raise RuntimeError("attn_probe_wg_stamps (probe) failed")
        return stamp_summary(st, a.elapsed_time(b))

    out["read_share"] = {"bytes": nbytes, "isolated": [], "sustained": []}
    read_and_stamp(30)
    for rep in range(args.wg_stamps):
        time.sleep(0.005)
        out["read_share"]["isolated"].append(read_and_stamp(0))
        out["read_share"]["sustained"].append(read_and_stamp(100))
        print(f"# read_share rep {rep}: isolated "
              f"{out['read_share']['isolated'][-1]['event_us']:.1f} us, sustained "
              f"{out['read_share']['sustained'][-1]['event_us']:.1f} us", file=sys.stderr,
              flush=True)
    print(json.dumps(out))


def wg_stamps_bifurcated(torch, args, run, lib):
    """Per-workgroup timing of the one-launch shared-prefix kernel: REPS
    launches after a run of back-to-back calls, each workgroup's start and end
    summarised separately for the prefix workgroups and the suffix ones (the
    split the planner chose, read from the test build's hook)."""
    import ctypes
    import numpy as np
    from long_context_exact_split_amd import binding
    readback = getattr(lib, "attn_probe_wg_stamps_bif", None)
    if readback is None:
        raise RuntimeError(f"{binding.library_path()} is not the stamping build")
    readback.argtypes = [ctypes.c_void_p, ctypes.c_int]
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    tl = binding.load_testing_library()
    fused, npre, nsuf = ctypes.c_int32(0), ctypes.c_int64(0), ctypes.c_int64(0)
    desc = binding.bifurcated_desc(run.t[0], run.t[1], run.t[3], run.w.scale)
    if tl.attn_testing_bifurcated_form(ctypes.byref(desc), cu, ctypes.byref(fused),
                                       ctypes.byref(npre), ctypes.byref(nsuf)) != 0:
        raise RuntimeError("attn_testing_bifurcated_form failed")
    split = bool(fused.value) and npre.value + nsuf.value == cu
    n = cu if fused.value else 0
    if n == 0:
        raise RuntimeError("this batch does not run the one-launch kernel")
    timed_steps(torch, run, 20, args.warmup, args.min_warmup_s)
    out = {"workload": WORKLOADS[args.workload], "kernel": "split_kv_bifurcated<128> (stamped)",
           "workgroups": n, "form": "split" if split else "shared",
           "prefix_workgroups": int(npre.value) if split else n,
           "library": os.path.basename(binding.library_path()), "launches": []}
    stream = torch.cuda.current_stream()
    for rep in range(args.wg_stamps):
        for _ in range(100):
            run.first()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        run.first()
        b.record(stream)
        torch.cuda.synchronize()
        st = np.zeros((n, 4), dtype=np.uint64)
        if readback(st.ctypes.data, n) != 0:
            raise RuntimeError("stamp read-back failed")
        t0, t1 = st[:, 0].astype(np.int64), st[:, 1].astype(np.int64)
        base = t0.min()
        start, end = (t0 - base) * 0.01, (t1 - base) * 0.01
        rec = {"call_us": a.elapsed_time(b) * 1e3, "span_us": float(end.max())}
        parts = ({"prefix": slice(0, int(npre.value)), "suffix": slice(int(npre.value), n)}
                 if split else {"all": slice(0, n)})
        for name, sl in parts.items():
            rec[name] = {"start_max_us": float(start[sl].max()),
                         "end_min_med_max_us": [float(end[sl].min()), float(np.median(end[sl])),
                                                float(end[sl].max())]}
        out["launches"].append(rec)
        print(f"# rep {rep}: " + ", ".join(
            f"{k} ends {v['end_min_med_max_us'][1]:.1f}/{v['end_min_med_max_us'][2]:.1f} us"
            for k, v in rec.items() if isinstance(v, dict)), file=sys.stderr, flush=True)
    print(json.dumps(out))


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(json.dumps({"error": "the path runs on one GPU; --gpus must be 1 "
                                   "(sharding the KV cache across GPUs is not implemented)"}))
        sys.exit(2)
    if args.wg_stamps > 0:
        from long_context_exact_split_amd import build
        os.environ.setdefault("ATTN_LIB", os.path.join(build.PKG, build.STAMPS_LIB_NAME))
    import torch

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.wg_stamps > 0:
        wg_stamps(torch, args)
        return
    t_gen = time.perf_counter()
    w = make_workload(args.workload)
    print(f"# generated {args.workload} in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr,
          flush=True)
    run = make_runner(torch, args.workload, args.page_size)
    print(f"# plan {run.plan}", file=sys.stderr, flush=True)

    K = args.steps
    t = timed_steps(torch, run, K, args.warmup, args.min_warmup_s)
    step_ms = t["wall_s"] * 1e3 / K
    first_avg = statistics.mean(t["first_ms"])
    alg = run.kv_bytes + run.q_bytes
    path_gbps = (alg + run.out_bytes) / (step_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": run.kv_tokens / (step_ms * 1e-3),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "warmup_steps_run": t["warmup"],
        "ms_per_step": step_ms,
        "event_every": t["event_every"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": getattr(w, "dtype", "bf16"),
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload], **run.plan},
        "hbm_gbps": path_gbps,
        "hbm_frac_of_peak": path_gbps / PEAK_GBPS,
        "dominant_kernel_ms": first_avg,
        "dominant_kernel_ms_median": statistics.median(t["first_ms"]),
        "second_launch_ms": statistics.mean(t["second_ms"]),
        "call_ms": spread(t["call_ms"]),
        "tflops": run.flops / (first_avg * 1e-3) / 1e12,
        "roofline": roofline(run, first_avg, args.workload),
    }
    if args.workload == "bifurcated_prefix":
        result["kv_tokens_physical"] = w.Lp + w.S * w.Ls
    if args.cold_calls > 0:
        result["call_ms_cold_cache"] = cold_calls(torch, run, args.cold_calls)
    if args.graph_calls > 0:
        result["call_ms_graph"] = graph_calls(torch, run, args.graph_calls)
    if not args.no_ceiling:
        ceil = read_ceiling(torch)
        result["hbm_read_ceiling_gbps"] = ceil
        result["roofline"]["frac_of_read_ceiling"] = result["roofline"]["achieved"] / ceil \
            if result["roofline"]["unit"] == "GB/s" else None
    parity_ok = True
    if not args.no_cpu_baseline:
        O, lse = run.outputs()
        result["cpu_baseline"] = cpu_baseline(run, args.cpu_rows, O, lse)
        parity_ok = result["cpu_baseline"]["parity_ok"]
    if args.workload == "long_context_1m" and not args.no_configs:
        del run
        forget(torch, w)
        configs = {}
        for name, steps, n_rows in CONFIGS:
            t_c = time.perf_counter()
            configs[name] = measure_config(torch, name, steps, n_rows, args.warmup,
                                           min(args.min_warmup_s, 0.3))
            parity_ok = parity_ok and configs[name]["parity"]["ok"]
            print(f"# config {name}: {configs[name]['call_ms_mean']:.4f} ms per call, parity "
                  f"{configs[name]['parity']} ({time.perf_counter() - t_c:.1f} s)",
                  file=sys.stderr, flush=True)
            if name in ("long_context_5m_share8", "llama31_70b_ragged", "bifurcated_prefix"):
                forget(torch, make_workload(name))
        result["configs"] = configs
    result["parity_ok"] = parity_ok
    print(json.dumps(result), flush=True)
    if not parity_ok:
        print("# parity bar missed on sampled rows", file=sys.stderr, flush=True)
        sys.exit(3)


if __name__ == "__main__":
    main()
