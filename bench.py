"""Benchmark of the quantised MoE FFN layer on one MI355X.

A step is one call of moe_w4a16_forward (route, union, experts, combine) on
one batch.  Steps cycle over L independent layer instances (each with all
E + 1 experts resident and its own router and input) captured in one HIP
graph by the library (moe_step_graph_create), so the touched weights per
graph replay far exceed the 256 MB Infinity Cache and every step streams its
experts from HBM.

Prints one JSON line: the headline workload (decode, batch 1, 6144 x 2048,
256 experts top-8 + shared, int4 per-row scales) with a roofline object for
its dominant kernel and the CPU oracle timed on a bounded sample.  Other
workloads are reported under "secondary".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import quantized_moe_expert_02_amd as moe  # noqa: E402
from quantized_moe_expert_02_amd import synth  # noqa: E402

METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode) / MFMA util (prefill), 1 GPU"
HBM_PEAK_GBPS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")

# Stage names per path (HIP events the library records between launches) and
# the dominant kernel: (stage index, name in rocprofv3 output).  On the decode
# path the shared expert's gate/up runs in the routing launch, so the gate/up
# launch streams the routed experts only.
# decode stage 0 also runs the shared expert's gate/up when T > 1 (for one
# token that moves into stage 1)
STAGES = {"decode": ("route", "gate_up", "down"), "prefill": ("route", "gate_up", "down")}
DOMINANT = {"decode": (1, "k_gu_phase"), "prefill": (1, "k_expert_gemm<gate_up>")}
WEIGHT_NAMES = {synth.INT4_ROW: "int4_row", synth.E2M1_B16: "e2m1_b16", synth.INT8_ROW: "int8_row",
                synth.INT2_ROW: "int2_row"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---- algorithmic work -------------------------------------------------------
def scale_bytes(d, rows, cols):
    return rows * 2 if d.wfmt in synth.ROW_SCALED else rows * (cols // 16)


def expert_gu_bytes(d):
    return 2 * d.inter * d.hidden * synth.code_bits(d.wfmt) // 8 + 2 * scale_bytes(d, d.inter, d.hidden)


def expert_dn_bytes(d):
    return d.hidden * d.inter * synth.code_bits(d.wfmt) // 8 + scale_bytes(d, d.hidden, d.inter)


def layer_bytes(d, T, n_touched):
    """Bytes the layer must move: each touched expert once (plus the shared
    expert), the router, x in and y out."""
    n = n_touched + d.has_shared
    return n * (expert_gu_bytes(d) + expert_dn_bytes(d)) + d.n_experts * d.hidden * 4 + 2 * T * d.hidden * 2


def gu_kernel_bytes(d, T, n_touched):
    """Algorithmic bytes of the gate/up kernel: touched gate/up weights and
    scales, x read, h written."""
    n = n_touched + d.has_shared
    return n * expert_gu_bytes(d) + T * d.hidden * 2 + (T * d.top_k + T * d.has_shared) * d.inter * 2


def layer_flops(d, T):
    return 2 * 3 * d.hidden * d.inter * T * (d.top_k + d.has_shared)


# ---- layer chain -------------------------------------------------------------
class Chain:
    def __init__(self, workload: str, L: int, seed: int = 0):
        w = synth.WORKLOADS[workload]
        self.name = workload
        self.dims = w["dims"]
        self.T = w["tokens"]
        t0 = time.time()
        base = synth.make_layer(self.dims, (workload if "e2m1" not in workload else "e2m1", seed, 0),
                                device="cuda", zipf=w.get("zipf", 0.0))
        self.canon0 = base
        pl0 = moe.PackedLayer.from_layer(base)
        self.layers = [pl0]
        for l in range(1, L):
            rw, rb = synth.make_router(self.dims, (workload, seed, l, "r"), device="cuda", zipf=w.get("zipf", 0.0))
            p = moe.PackedLayer(self.dims, pl0.packed.clone(), rw, rb)
            self.layers.append(p)
        self.x = [synth.make_tokens(self.dims, self.T, (workload, seed, l, "x"), device="cuda") for l in range(L)]
        self.y = [torch.empty((self.T, self.dims.hidden), dtype=torch.float16, device="cuda") for _ in range(L)]
        self.ws = moe.workspace(self.dims, self.T)
        torch.cuda.synchronize()
        log(f"[bench] {workload}: {L} layers x {self.packed_gb():.2f} GB built in {time.time() - t0:.1f}s")

    def packed_gb(self):
        return self.layers[0].packed.numel() / 1e9

    def call(self, l, stream=None):
        moe.moe_w4a16_forward(self.layers[l], self.x[l], y=self.y[l], ws=self.ws, stream=stream)

    def touched(self):
        """Realised union size per layer (read back once, outside timing)."""
        out = []
        for l, pl in enumerate(self.layers):
            r = moe.moe_route(pl, self.x[l])
            out.append(int(r["n_unique"][0]))
        torch.cuda.synchronize()
        return out


def time_chain(ch: Chain, steps: int, warmup: int):
    """Replays of the L layer calls as one graph captured by the library
    (moe_step_graph_create; every layer with its own input), timed with
    events on the stream the graphs are launched on."""
    L = len(ch.layers)
    full, rem = divmod(steps, L)
    for l in range(L):  # eager warm-up of every layer before capture
        ch.call(l)
    torch.cuda.synchronize()
    g_full = moe.StepGraph(ch.layers, ch.x, ch.y, ch.ws)
    g_rem = moe.StepGraph(ch.layers[:rem], ch.x[:rem], ch.y[:rem], ch.ws) if rem else None
    for _ in range(max(1, -(-warmup // L))):
        g_full.launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record()
    for _ in range(full):
        g_full.launch()
    if g_rem is not None:
        g_rem.launch()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1)
    g_full.close()
    if g_rem is not None:
        g_rem.close()
    return ms, wall


class _Hip:
    """A few HIP runtime calls through ctypes (raw events the library can
    record; torch creates its own event handles lazily)."""

    def __init__(self):
        import ctypes
        self.c = ctypes
        L = ctypes.CDLL("libamdhip64.so")
        L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        L.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.L = L

    def event(self):
        h = self.c.c_void_p()
        if self.L.hipEventCreate(self.c.byref(h)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return h.value

    def elapsed_ms(self, a, b) -> float:
        ms = self.c.c_float(0)
        rc = self.L.hipEventElapsedTime(self.c.byref(ms), self.c.c_void_p(a), self.c.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def destroy(self, h):
        self.L.hipEventDestroy(self.c.c_void_p(h))


def time_stages(ch: Chain, reps: int):
    """Mean duration (ms) of each stage of a forward call, from HIP events
    that the stage's first and last kernel dispatches record (start / end
    timestamps of the dispatch packets, so launch overhead is excluded)."""
    hip = _Hip()
    L = len(ch.layers)
    evs = [[hip.event() for _ in range(6)] for _ in range(reps * L)]
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)  # let the host queue every call before the GPU starts them
    i = 0
    for r in range(reps):
        for l in range(L):
            moe.moe_w4a16_forward_profiled(ch.layers[l], ch.x[l], ch.y[l], ch.ws, evs[i])
            i += 1
    torch.cuda.synchronize()
    n = len(evs)
    out = [sum(hip.elapsed_ms(e[2 * j], e[2 * j + 1]) for e in evs) / n for j in range(3)]
    for e in evs:
        for h in e:
            hip.destroy(h)
    return out


def traffic_record(kernel: str, workload: str):
    """Counter-measured HBM bytes per launch of `kernel` (FETCH_SIZE +
    WRITE_SIZE, calibrated against a plain copy) if the committed record
    matches the current kernel source; else None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    src = kv.get("source")
    if not src or hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest() != kv.get("source_sha256"):
        return None
    return float(kv["bytes_per_launch"])


# ---- CPU baseline (the oracle, test infrastructure) ------------------------
class _Indexable:
    """Host copies of some experts' tensors, indexed by expert id."""

    def __init__(self, d, n):
        self.d, self.shape = d, (n,)

    def __getitem__(self, e):
        return self.d[int(e)]


class _HostExperts:
    """Host copies of the experts a sample needs, indexable like a Layer."""

    def __init__(self, layer, experts):
        self.dims = layer.dims
        n = layer.q_gate.shape[0]
        for name in ("q_gate", "s_gate", "q_up", "s_up", "q_down", "s_down"):
            src = getattr(layer, name)
            setattr(self, name, _Indexable({int(e): src[int(e)].cpu() for e in experts}, n))
        self.g3 = layer.g3.cpu()
        self.router_w = layer.router_w.cpu()
        self.router_b = None if layer.router_b is None else layer.router_b.cpu()


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _time_oracle(host, xs, r, threads, budget_s, max_tokens):
    """Single-token oracle calls on `threads` threads until the budget or the
    sample runs out; returns (tokens done, seconds)."""
    import oracle
    done, t0 = 0, time.perf_counter()
    while done < max_tokens and (time.perf_counter() - t0) < budget_s:
        oracle.forward(host, xs, tokens=[done], experts_needed=[int(e) for e in r.topk_idx[done] if e >= 0],
                       threads=threads)
        done += 1
    return done, time.perf_counter() - t0


def cpu_baseline(ch: Chain, budget_s: float = 10.0, max_tokens: int = 64, single_budget_s: float = 8.0):
    """The CPU oracle (fp64 C++, OpenMP over independent output rows) on a
    bounded sample of tokens of the same layer, on all host threads and on
    one thread.  Tokens are processed one call each (the oracle's cost per
    token does not depend on the batch), so the same figure serves decode
    and prefill workloads; the sample's tokens are drawn like the workload's."""
    import numpy as np
    import oracle

    layer = ch.canon0
    d = layer.dims
    n_all = oracle.max_threads()  # before any call sets the thread count
    xs = synth.make_tokens(d, max_tokens, (ch.name, "cpu-sample"), device="cpu")
    r = oracle.route(d, xs, layer.router_w.cpu(), None if layer.router_b is None else layer.router_b.cpu())
    need = set(np.unique(r.topk_idx[r.topk_idx >= 0]).tolist()) | ({d.n_experts} if d.has_shared else set())
    host = _HostExperts(layer, need)
    done, el = _time_oracle(host, xs, r, n_all, budget_s, max_tokens)
    done1, el1 = _time_oracle(host, xs, r, 1, single_budget_s, max_tokens)
    oracle.forward(host, xs, tokens=[0], experts_needed=[int(e) for e in r.topk_idx[0] if e >= 0], threads=n_all)
    # parity of the GPU path (one call per token, as timed) on the same sample
    pl = moe.PackedLayer(d, ch.layers[0].packed, layer.router_w, layer.router_b)
    xg = xs[:done].to("cuda")
    y = torch.cat([moe.moe_w4a16_forward(pl, xg[t:t + 1].contiguous()) for t in range(done)])
    torch.cuda.synchronize()
    y_ref = oracle.forward(host, xs, tokens=list(range(done)), experts_needed=sorted(need - {d.n_experts}),
                           threads=n_all)
    err = y.double().cpu().numpy() - y_ref
    rel = float(np.linalg.norm(err) / np.linalg.norm(y_ref))
    model = cpu_model()
    return {"value": done / el, "unit": "tokens/s", "cores": n_all, "kind": "oracle",
            "sample": f"{done} tokens of the {ch.name} layer (seeded, drawn like its inputs), one oracle call "
                      f"each, {el:.1f}s on {n_all} threads of {model}; fp64 C++ oracle, OpenMP over output rows",
            "cpu_model": model,
            "single_thread": {"value": done1 / el1, "unit": "tokens/s", "cores": 1,
                              "sample": f"{done1} tokens of the same sample, {el1:.1f}s, OMP on one thread"},
            "parity_rel_l2_on_sample": rel}


# ---- main ----------------------------------------------------------------------
def tiered_decode(n_layers: int = 2, slots: int = 32, tokens: int = 48, warmup: int = 16, rho: float = 0.9):
    """Batch-1 decode of n_layers layers of the headline shape whose routed
    experts live in pinned host memory (moe_tier.h), through a host-driven
    loop.  Tokens follow a seeded random walk (consecutive tokens correlated
    by rho) and pass through the layers on a residual stream,
    x_{l+1} = x_l + y_l.  Modes:
      hbm        every expert in HBM (the same loop, for reference);
      host       no slots: every routed expert is read over PCIe (the
                 unions are still reported, to count the misses);
      lru_after  LRU slots; the layer runs first (misses read over PCIe),
                 then its union is reported and the misses are promoted;
      lru_load   LRU slots; the layer is routed first, its union reported,
                 and the compute stream waits for the promotions before the
                 layer runs (every expert read from HBM, misses copied once);
      lru_load_next  lru_load plus the next-layer prefetch: before layer l
                 runs, layer l+1's router is applied to the current residual
                 and its union prefetched, overlapping layer l;
      hot        HOT slots (most used experts); misses read over PCIe."""
    import ctypes
    d = synth.WORKLOADS["decode_b1"]["dims"]
    E = d.n_experts
    t0 = time.time()
    base = synth.make_layer(d, ("tiered", 0), device="cuda")
    pl0 = moe.PackedLayer.from_layer(base)
    del base
    pb = pl0.packed.shape[1]
    routers = [synth.make_router(d, ("tiered", l), device="cuda") for l in range(n_layers)]
    layers = [moe.PackedLayer(d, pl0.packed, rw, rb) for rw, rb in routers]  # same experts, own routers
    buf = torch.empty(n_layers * E * pb + 256, dtype=torch.uint8, pin_memory=True)
    off = (-buf.data_ptr()) % 256
    host = buf[off:off + n_layers * E * pb].view(n_layers, E, pb)
    for l in range(n_layers):
        host[l].copy_(pl0.packed[:E].cpu())
    ptrs = [host.data_ptr() + (l * E + e) * pb for l in range(n_layers) for e in range(E)]
    slot_mem = torch.empty(max(1, n_layers * slots) * pb, dtype=torch.uint8, device="cuda")
    table = torch.zeros(n_layers * E, dtype=torch.int64, device="cuda")
    copy_stream = torch.cuda.Stream()
    ws = moe.workspace(d, 1)
    log(f"[bench] tiered: {n_layers} layers x {E * pb / 1e9:.2f} GB pinned, built in {time.time() - t0:.1f}s")
    g = torch.Generator(device="cpu").manual_seed(1234)
    walk = [torch.randn((1, d.hidden), generator=g)]
    for _ in range(tokens + warmup - 1):
        walk.append(rho * walk[-1] + (1 - rho * rho) ** 0.5 * torch.randn((1, d.hidden), generator=g))
    xs = [w.to(torch.float16).to("cuda") for w in walk]
    ti = torch.empty((1, d.top_k), dtype=torch.int32, device="cuda")
    y = torch.empty((1, d.hidden), dtype=torch.float16, device="cuda")
    dd = moe._dims(d)

    def union_of(layer, x):
        r = moe.moe_route(layer, x, ws=ws)
        return r["uniq_ids"][:int(r["n_unique"][0])].cpu().tolist()

    out = {"workload": "tiered_decode_b1", "layers": n_layers, "slots_per_layer": slots, "tokens": tokens,
           "warmup": warmup, "rho": rho, "expert_bytes": pb, "modes": {}}
    for mode in ("hbm", "host", "lru_after", "lru_load", "lru_load_next", "hot"):
        C = 0 if mode in ("hbm", "host") else slots
        policy = moe.MOE_TIER_HOT if mode == "hot" else moe.MOE_TIER_LRU
        tier = moe.Tier(d, n_layers, ptrs, C, slots=slot_mem if C else None, table=table, copy_stream=copy_stream,
                        policy=policy)
        st0, t_start = None, None
        for t in range(tokens + warmup):
            if t == warmup:
                torch.cuda.synchronize()
                st0, t_start = tier.stats(), time.perf_counter()
            x = xs[t]
            for l in range(n_layers):
                if mode in ("lru_load", "lru_load_next"):
                    tier.use(l, union_of(layers[l], x))
                    tier.sync()
                if mode == "lru_load_next" and l + 1 < n_layers:
                    tier.prefetch(l + 1, union_of(layers[l + 1], x))
                if mode == "hbm":
                    w = layers[l].weights()
                else:
                    w = tier.weights(l, layers[l].router_w, layers[l].router_b, layers[l].shared_ptr)
                rc = moe.lib().moe_w4a16_forward(ctypes.byref(dd), ctypes.byref(w), moe._p(x), 1, moe._p(y),
                                                 moe._p(ti), None, moe._p(ws), ws.numel(), moe._stream(None))
                if rc != moe.MOE_OK:
                    raise moe.MoeError(rc, "moe_w4a16_forward")
                if mode in ("host", "lru_after", "hot"):
                    tier.use(l, sorted(set(ti.cpu().numpy().ravel().tolist())))
                x = x + y
        torch.cuda.synchronize()
        dt = time.perf_counter() - t_start
        st = tier.stats()
        tier.close()
        torch.cuda.current_stream().wait_stream(copy_stream)
        torch.cuda.synchronize()
        hits, misses = st["hits"] - st0["hits"], st["misses"] - st0["misses"]
        promos = st["promotions"] - st0["promotions"]
        res = {"ms_per_token": dt / tokens * 1e3, "tokens_per_s": tokens / dt}
        if mode != "hbm":
            # bytes over PCIe: promotions, plus the misses that the layer itself read from host memory
            read = 0 if mode.startswith("lru_load") else misses
            res.update({"hit_rate": hits / max(1, hits + misses), "misses_per_token": misses / tokens,
                        "promotions_per_token": promos / tokens,
                        "pcie_gb_per_token": (read + promos) * pb / tokens / 1e9,
                        "pcie_gbps": (read + promos) * pb / dt / 1e9})
        out["modes"][mode] = res
        log(f"[bench] tiered {mode}: " + json.dumps({k: round(v, 4) for k, v in res.items()}))
    del host, buf, slot_mem, layers, pl0
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch._C._host_emptyCache()  # return the pinned host buffers now, not at interpreter exit
    torch.cuda.empty_cache()
    return out


def path_of(T):
    return "decode" if T <= moe.moe_decode_max_tokens() else "prefill"


def dominant_bytes(d, T, n_touched):
    """Algorithmic bytes of the dominant (gate/up) kernel: on the decode path
    the routed experts' gate/up weights and scales, x read and the routed h
    rows written -- for one token the launch also runs the shared expert's
    gate/up (its weights and h row); on the prefill path the shared expert as
    well."""
    if path_of(T) == "decode":
        shared = d.has_shared if T == 1 else 0
        return ((n_touched + shared) * expert_gu_bytes(d) + T * d.hidden * 2
                + T * (d.top_k + shared) * d.inter * 2)
    return gu_kernel_bytes(d, T, n_touched)


def run_workload(name, L, steps, warmup, stage_reps=4):
    ch = Chain(name, L)
    touched = ch.touched()
    ms, wall = time_chain(ch, steps, warmup)
    stages = time_stages(ch, stage_reps)
    d, T = ch.dims, ch.T
    ms_step = ms / steps
    U = sum(touched) / len(touched)
    lb = sum(layer_bytes(d, T, u) for u in touched) / len(touched)
    res = {
        "workload": name, "tokens": T, "layers_chained": L, "steps": steps,
        "ms_per_step": ms_step, "tokens_per_s": T * steps / (ms / 1e3),
        "mean_unique_experts": U, "layer_bytes": lb,
        "layer_hbm_gbps": lb / (ms_step / 1e3) / 1e9,
        "stage_ms": dict(zip(STAGES[path_of(T)], stages)),
        "wall_s": wall,
    }
    if T > moe.moe_decode_max_tokens():
        res["mfma_util"] = layer_flops(d, T) / (ms_step / 1e3) / (FP16_MFMA_PEAK_TFLOPS * 1e12)
        res["roofline"] = prefill_roofline(d, T, res["stage_ms"], name)
    return ch, res, touched


def prefill_roofline(d, T, stage_ms, workload):
    """Matrix-core roofline of the grouped-GEMM path: the gate/up launch
    (k_expert_gemm<., 2, .>, the dominant kernel) and the down launch,
    algorithmic fp16 flops per launch (2 flops per multiply-add; every
    (token, expert) pair including the shared expert, without the padding of
    partly filled tiles) over the launch's mean duration."""
    pairs = T * (d.top_k + d.has_shared)
    gu_flops = 2 * 2 * d.hidden * d.inter * pairs
    dn_flops = 2 * d.hidden * d.inter * pairs
    gu_ms, dn_ms = stage_ms["gate_up"], stage_ms["down"]
    achieved = gu_flops / (gu_ms / 1e3) / 1e12
    return {"bound": "mfma", "kernel": "k_expert_gemm<gate_up>", "achieved": achieved,
            "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved / FP16_MFMA_PEAK_TFLOPS,
            "traffic": traffic_record("k_expert_gemm_gu", workload),
            "algorithmic_flops_per_launch": gu_flops, "avg_launch_ms": gu_ms,
            "down": {"kernel": "k_expert_gemm<down>+k_combine", "algorithmic_flops_per_launch": dn_flops,
                     "avg_ms": dn_ms, "achieved": dn_flops / (dn_ms / 1e3) / 1e12,
                     "frac": dn_flops / (dn_ms / 1e3) / 1e12 / FP16_MFMA_PEAK_TFLOPS}}


def reference_rates():
    """Rates the box reaches with library code that is not this project's:
    HBM read (torch.sum over 4 GiB of binary16), HBM copy (torch.neg, read
    + write) and a dense binary16 GEMM (torch.matmul, 8192^3, hipBLASLt) --
    measured context beside the published peaks (8 TB/s, 2.5 PFLOP/s)."""
    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / 1e3
    n = 2 << 30  # binary16 elements: 4 GiB
    a = torch.ones(n, dtype=torch.float16, device="cuda")
    t_sum = timed(lambda: torch.sum(a, dtype=torch.float32), 10)
    b = torch.empty_like(a)
    t_neg = timed(lambda: torch.neg(a, out=b), 10)
    del a, b
    m = torch.randn((8192, 8192), dtype=torch.float16, device="cuda")
    w = torch.randn((8192, 8192), dtype=torch.float16, device="cuda")
    t_mm = timed(lambda: torch.matmul(m, w), 20)
    del m, w
    torch.cuda.empty_cache()
    # the library's own probes: a plain 128-bit streaming read over 8 GiB and
    # a pure matrix-core loop
    nb = 8 << 30
    buf = torch.ones(nb // 4, dtype=torch.int32, device="cuda")
    rb = 256 * 8
    sink = torch.empty(max(rb * 256, 1024 * 512), dtype=torch.int32, device="cuda")
    t_rd = timed(lambda: moe.probe_stream_read(buf, rb, sink), 5)
    del buf
    torch.cuda.empty_cache()
    mb, iters = 1024, 1000
    flops = mb * 8 * iters * 16 * 2 * 16 * 16 * 32
    t_mf = timed(lambda: moe.probe_mfma(sink, mb, iters), 5)
    return {"hbm_read_gbps": 2 * n / t_sum / 1e9, "hbm_copy_gbps": 4 * n / t_neg / 1e9,
            "fp16_gemm_tflops": 2 * 8192 ** 3 / t_mm / 1e12,
            "stream_read_gbps": nb / t_rd / 1e9, "mfma_f16_tflops": flops / t_mf / 1e12,
            "how": "torch.sum over 4 GiB binary16; torch.neg over 4 GiB (read + write); torch.matmul 8192^3 "
                   "binary16; moe_probe_stream_read: one 128-bit non-temporal read of 8 GiB (2,048 x 256 "
                   "threads); moe_probe_mfma: 1,024 x 8 wavefronts x 1,000 rounds of 16 independent "
                   "v_mfma_f32_16x16x32_f16"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--workload", default="decode_b1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--tiered-only", action="store_true", help="run only the tiered-residency decode line")
    ap.add_argument("--reference-rates", action="store_true",
                    help="print only the rates torch reaches on this box (HBM read/copy, fp16 GEMM) and exit")
    ap.add_argument("--no-measured-peaks", action="store_true",
                    help="skip the library-code reference rates (copy, GEMM) measured after the workloads")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="first run a plain elementwise copy (torch.neg) over this many MB, so that hardware "
                         "traffic counters taken over the run can be scaled against a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (expert- and tensor-parallel "
              "sharding of the layer is a design, not code). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    torch.cuda.init()
    moe.lib()
    if args.calibrate_copy_mb:
        n = args.calibrate_copy_mb * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.float16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    if args.tiered_only:
        print(json.dumps(tiered_decode()))
        return
    if args.reference_rates:
        print(json.dumps(reference_rates()))
        return
    ch, res, touched = run_workload(args.workload, args.layers, args.steps, args.warmup)
    d, T = ch.dims, ch.T
    path = path_of(T)
    U = res["mean_unique_experts"]
    if path == "decode":
        st_idx, kname = DOMINANT[path]
        k_ms = res["stage_ms"][STAGES[path][st_idx]]
        alg = sum(dominant_bytes(d, T, u) for u in touched) / len(touched)
        achieved = alg / (k_ms / 1e3) / 1e9
        roofline = {"bound": "hbm", "kernel": kname, "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic_record(kname, args.workload),
                    "algorithmic_bytes_per_launch": alg, "avg_launch_ms": k_ms}
    else:
        roofline = res["roofline"]

    def baseline(chain, **kw):
        try:
            return cpu_baseline(chain, **kw)
        except Exception as e:  # the baseline is context, never the headline
            return {"value": None, "unit": "tokens/s", "cores": None, "kind": "oracle", "sample": f"failed: {e}"}

    cpu = None if args.no_cpu_baseline else baseline(ch)
    secondary = []
    del ch
    torch.cuda.empty_cache()
    roofline_prefill = cpu_prefill = None
    if not args.no_secondary:
        for name, L, steps in (("decode_b8", 8, 128), ("decode_b1_topp", 8, 512), ("e2m1_b1", 32, 512),
                               ("e2m1_b4", 32, 256), ("int8_b1", 8, 512), ("int2_b1", 8, 512),
                               ("int2_b8", 8, 128), ("prefill_2048", 2, 8),
                               ("prefill_2048_uniform", 2, 8)):
            try:
                c2, r2, _ = run_workload(name, L, steps, 32, stage_reps=2)
                if name == "prefill_2048":
                    roofline_prefill = r2["roofline"]
                    if not args.no_cpu_baseline:
                        cpu_prefill = r2["cpu_baseline"] = baseline(c2, budget_s=6.0, max_tokens=32,
                                                                    single_budget_s=4.0)
                secondary.append(r2)
                del c2
                torch.cuda.empty_cache()
            except Exception as e:
                secondary.append({"workload": name, "error": str(e)})
        try:
            secondary.append(tiered_decode())
        except Exception as e:
            secondary.append({"workload": "tiered_decode_b1", "error": str(e)})
    # achievable rates measured on the same box (library code, not this
    # project's), beside the published peaks the rooflines use
    try:
        if args.no_measured_peaks:
            raise RuntimeError("not measured (--no-measured-peaks)")
        ref = reference_rates()
        for rl in (roofline, roofline_prefill):
            if rl:
                # against the library's streaming-read and matrix-core probes
                rl["frac_of_measured"] = rl["achieved"] / (ref["stream_read_gbps"] if rl["unit"] == "GB/s"
                                                           else ref["mfma_f16_tflops"])
    except Exception as e:
        ref = {"error": str(e)}
    out = {
        "metric": METRIC,
        "value": res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": args.workload, "hidden": d.hidden, "inter": d.inter, "experts": d.n_experts,
                   "shared_experts": d.has_shared, "top_k": d.top_k, "tokens": T,
                   "weights": WEIGHT_NAMES[d.wfmt], "layers_chained": args.layers},
        "layer_hbm_gbps": res["layer_hbm_gbps"],
        "layer_hbm_frac": res["layer_hbm_gbps"] / HBM_PEAK_GBPS,
        "mean_unique_experts": U,
        "stage_ms": res["stage_ms"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "roofline_prefill": roofline_prefill,
        "measured_peaks": ref,
        "layer_hbm_frac_of_measured": (res["layer_hbm_gbps"] / ref["stream_read_gbps"]
                                       if "stream_read_gbps" in ref else None),
        "cpu_baseline_prefill": cpu_prefill,
        "secondary": secondary,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
