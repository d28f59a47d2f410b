#!/usr/bin/env python3
"""Benchmark of the Kimi-K2 routed MoE FFN layer on one MI355X.

One step = one moe_layer_forward (router, grouping, expert FFNs, combine) over
one batch of synthetic tokens whose inputs are already resident in HBM; steps
rotate among 4 such batches.
Default workload: Kimi-K2 decode, T = 128 tokens, bf16, all 384 experts + 1
shared resident.  A step is captured once in a HIP graph and replayed (the
library only launches kernels: no memset, no host synchronisation); --eager
launches every step from the host instead.  For an expert-parallel rank workload (ep_size > 1) a step
is that rank's expert FFN share (moe_expert_ffn over the rows dispatched to
its local experts plus the shared expert over its own tokens), and value is
the rank's own tokens per second.  For a sub-block workload (block) a step is
one moe_block_forward (pre-MoE RMSNorm, the layer, the residual add).  Prints ONE JSON line (value = tokens/s) with:
  roofline      -- the dominant kernel (grouped gate_up GEMM): algorithmic
                   bytes or flops per launch / its mean duration, timed with
                   HIP events the library records around that launch, as a
                   fraction of the spec peak (frac) and of the measured
                   ceiling (frac_measured);
  prefill       -- (default decode run) the other half of the metric: the
                   Zipf-skewed prefill, T = 8192, on the same resident
                   weights, with its gate_up and down rooflines (MFMA);
  ceilings      -- what this GPU sustains: HBM read rate of whole-line
                   nontemporal loads, the MFMA issue rate (bf16, fp8) of a
                   register-only loop, and hipBLASLt (torch.matmul) on the
                   dense 8192 x 4096 x 7168 bf16 shape;
  cpu_baseline  -- the fp64 oracle timed on a bounded sample of the same
                   workload on the host cores.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sparse_moe_transformer_sigmoid_amd import binding as B  # noqa: E402
from sparse_moe_transformer_sigmoid_amd import inputs as gen  # noqa: E402

METRIC = "MoE-layer tokens/s; % HBM peak (decode T=128), % MFMA peak (prefill T=8192)"
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {gen.BF16: 2500.0, gen.FP8: 5000.0, gen.F32: 157.3}
KERNEL_SOURCES = ["ffn_stream.hip", "ffn_tile.hip", "ffn_fp8.hip", "common.h"]


class Hip:
    """Raw hipEvent handles (the library records them on its own stream)."""

    def __init__(self):
        # the HIP runtime already mapped into this process (torch's copy, which
        # libmoe binds to as well); a second copy would not know its handles
        paths = {ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64.so" in ln}
        if len(paths) != 1:
            raise RuntimeError(f"expected exactly one HIP runtime mapped, found {sorted(paths)}")
        self.lib = ctypes.CDLL(paths.pop())

    def event(self) -> int:
        ev = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(ev)) == 0
        return ev.value

    def elapsed_ms(self, a: int, b: int):
        """Milliseconds between two recorded events, None if either was never
        recorded (the failed query's sticky error is cleared)."""
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            self.lib.hipGetLastError()
            return None
        return ms.value


class ProbeLib:
    """The measured-ceiling kernels (libmoe_probe.so, built beside libmoe.so)."""

    def __init__(self):
        path = os.path.join(ROOT, "sparse_moe_transformer_sigmoid_amd", "libmoe_probe.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built: run `python -m sparse_moe_transformer_sigmoid_amd.build`")
        self.lib = ctypes.CDLL(path)
        self.lib.moe_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                            ctypes.c_void_p]
        self.lib.moe_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                            ctypes.c_void_p]


def timed(fn, reps: int, warm: int = 2) -> float:
    """Mean milliseconds of fn() over `reps` launches on the current stream."""
    for _ in range(warm):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    b.synchronize()
    return a.elapsed_time(b) / reps


def measure_ceilings():
    """Measured peaks of this GPU (see ProbeLib): HBM read GB/s, MFMA TFLOP/s
    of a register-only loop (bf16 32x32x16, fp8 32x32x64 block-scaled), and
    hipBLASLt's bf16 GEMM (torch.matmul) on 8192 x 4096 x 7168."""
    p = ProbeLib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes, blocks = 4 << 30, 2048
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(blocks * 16, dtype=torch.uint8, device="cuda")

    def read():
        assert p.lib.moe_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes, blocks,
                                    ctypes.c_void_p(sink.data_ptr()), st) == 0
    read_ms = timed(read, 5)
    del buf
    fsink = torch.empty(4096, dtype=torch.float32, device="cuda")
    out = {"hbm_read_gbs": round(nbytes / (read_ms * 1e-3) / 1e9, 1)}
    for fp8, iters, name in ((0, 64, "mfma_bf16_loop_tflops"), (1, 32, "mfma_fp8_loop_tflops")):
        def mfma(fp8=fp8, iters=iters):
            assert p.lib.moe_probe_mfma(fp8, 2048, iters, ctypes.c_void_p(fsink.data_ptr()), st) == 0
        ms = timed(mfma, 5)
        flops = 2048 * 4 * iters * 4 * 2 * 32 * 32 * (64 if fp8 else 16)
        out[name] = round(flops / (ms * 1e-3) / 1e12, 1)
    a = torch.randn(8192, 7168, device="cuda").to(torch.bfloat16)
    b = torch.randn(7168, 4096, device="cuda").to(torch.bfloat16)
    ms = timed(lambda: torch.mm(a, b), 20, warm=3)
    out["hipblaslt_bf16_tflops_8192x4096x7168"] = round(2 * 8192 * 4096 * 7168 / (ms * 1e-3) / 1e12, 1)
    out["how"] = ("4 GiB read by 2048 blocks, 16-byte nontemporal loads (1 KB per wave instruction), 8 in flight; "
                  "2048 x 4 waves of 4 independent MFMA chains; torch.mm on resident bf16 operands; hipEvent means")
    return out


def with_measured(rl: dict, ceilings) -> dict:
    """Adds the fraction of the measured ceiling of the roofline's bound."""
    if not ceilings:
        return rl
    if rl["bound"] == "hbm":
        peak = ceilings["hbm_read_gbs"]
    else:
        peak = ceilings["mfma_fp8_loop_tflops" if rl["peak"] == PEAK_TFLOPS[gen.FP8] else "mfma_bf16_loop_tflops"]
    return {**rl, "peak_measured": peak, "frac_measured": round(rl["achieved"] / peak, 4)}


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        p = os.path.join(ROOT, "sparse_moe_transformer_sigmoid_amd", "csrc", f)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


X_BATCHES = 4


def setup(wl: gen.Workload, T: int):
    """Resident inputs: X_BATCHES independent token batches (steps rotate
    among them, so no step finds its x, and the routing it causes, cached
    from the step before), the router and the expert weights."""
    xs = [gen.gen_x(wl, T, b).cuda() for b in range(X_BATCHES)]
    d = {"x": xs[0], "xs": xs, "router_w": gen.gen_router(wl).cuda(), "router_bias": gen.gen_bias(wl).cuda(),
         "norm_weight": gen.gen_norm_weight(wl).cuda()}
    d.update(gen.gen_expert_weights(wl, device="cuda"))
    torch.cuda.synchronize()
    return d


def weight_bytes_per_expert_gate_up(wl: gen.Workload, F: int) -> int:
    H = wl.hidden_size
    if wl.weight_dtype == gen.FP8:
        return 2 * F * H + 2 * (F // 128) * (H // 128) * 4
    return 2 * F * H * (4 if wl.weight_dtype == gen.F32 else 2)


def roofline(wl: gen.Workload, T: int, n_active: int, gate_up_ms: float, traffic, routed_rows=None,
             kernel: str = "gate_up"):
    """Algorithmic work of one gate_up (or down) launch against the bound it
    sits on: the weights of the active and the shared experts once (bytes),
    and 2 * 2 * rows * H * F for the gate and up products (down: 2 * rows *
    H * F) (flops)."""
    F, Fs, H, k = wl.moe_intermediate_size, wl.shared_intermediate_size, wl.hidden_size, wl.num_experts_per_tok
    rows = T * k if routed_rows is None else routed_rows
    part = 1.0 if kernel == "gate_up" else 0.5
    bytes_ = round(n_active * weight_bytes_per_expert_gate_up(wl, F) * part)
    if Fs:
        bytes_ += round(weight_bytes_per_expert_gate_up(wl, Fs) * part)
    flops = 4.0 * part * (rows * F + T * Fs) * H
    peak_tf = PEAK_TFLOPS[wl.weight_dtype]
    ridge = peak_tf * 1e12 / (PEAK_HBM_GBS * 1e9)
    sec = gate_up_ms * 1e-3
    if flops / bytes_ > ridge:
        ach = flops / sec / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(ach / peak_tf, 4), "traffic": traffic,
                "kernel": kernel, "kernel_ms": round(gate_up_ms, 4), "algorithmic_flops": flops}
    ach = bytes_ / sec / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic,
            "kernel": kernel, "kernel_ms": round(gate_up_ms, 4), "algorithmic_bytes": bytes_}


def source_hash(name: str) -> str:
    p = os.path.join(ROOT, "sparse_moe_transformer_sigmoid_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16] if os.path.exists(p) else ""


def stored_traffic(workload: str, num_tokens: int):
    """HBM bytes per gate_up launch measured by rocprofv3 counters (FETCH_SIZE +
    WRITE_SIZE scaled by a 1 GiB copy), if they were taken for this token
    count on the current sources of that kernel (else None)."""
    p = os.path.join(ROOT, "profiles", f"traffic_gate_up_{workload}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("num_tokens") != num_tokens:
        return None
    if any(source_hash(f) != h for f, h in d.get("sources", {}).items()):
        return None
    return d.get("traffic_bytes")


# the gate_up kernel of each bench workload, and the sources its code comes from
GATE_UP_KERNEL = {"k2_decode_bf16": ("gate_up_stream_bf16<", ["ffn_stream.hip", "common.h"]),
                  "k2_prefill_bf16_zipf": ("ffn_tile_bf16<0,", ["ffn_tile.hip", "common.h"]),
                  "k2_fp8": ("ffn_tile_fp8<0,", ["ffn_tile_fp8.hip", "common.h"])}


def counter_means(run_dir: str, counter: str) -> dict:
    """Mean value per dispatch of one rocprofv3 counter, per kernel name, from
    the counter_collection.csv files of a `rocprofv3 --pmc <counter>
    --output-format csv -d <run_dir>` run."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), max(v)) for k, v in vals.items()}


def write_traffic(workload: str, num_tokens: int, fetch_dir: str, write_dir: str) -> dict:
    """profiles/traffic_gate_up_<workload>.json from a FETCH_SIZE and a
    WRITE_SIZE pass of `bench.py --workload <workload> --calib-copy` (KiB per
    dispatch): each counter is scaled by what it reads for the 1 GiB device
    copy of the same run (gfx950's FETCH_SIZE reads half of the bytes moved),
    and the gate_up kernel's scaled mean is its HBM traffic per launch."""
    prefix, sources = GATE_UP_KERNEL[workload]
    fetch, write = counter_means(fetch_dir, "FETCH_SIZE"), counter_means(write_dir, "WRITE_SIZE")
    copy = [k for k in fetch if "copyBuffer" in k]
    if not copy:
        sys.exit("no 1 GiB copy in the FETCH_SIZE run (pass --calib-copy)")
    gib_kib = float(1 << 20)
    fscale = gib_kib / fetch[copy[0]][1]
    wcopy = [k for k in write if "copyBuffer" in k]
    wscale = gib_kib / write[wcopy[0]][1]
    names = [k for k in fetch if prefix in k]
    if len(names) != 1:
        sys.exit(f"expected one {prefix} kernel in the counter run, found {names}")
    name = names[0]
    traffic = fetch[name][0] * 1024 * fscale + write[name][0] * 1024 * wscale
    d = {"workload": workload, "num_tokens": num_tokens, "kernel": name, "traffic_bytes": int(round(traffic)),
         "fetch_kib": round(fetch[name][0], 1), "write_kib": round(write[name][0], 1),
         "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4),
         "sources": {f: source_hash(f) for f in sources}}
    with open(os.path.join(ROOT, "profiles", f"traffic_gate_up_{workload}.json"), "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")
    return d


def cpu_baseline(wl, case, T, budget_s):
    """The fp64 oracle (as it stands) on a bounded sample of the same tokens."""
    import threadpoolctl
    import oracle
    x64 = case["x"].double().cpu().numpy()
    rw = case["router_w"].double().cpu().numpy()
    b = case["router_bias"].double().cpu().numpy()
    kw = dict(num_experts_per_tok=wl.num_experts_per_tok, n_group=wl.n_group, topk_group=wl.topk_group,
              norm_topk_prob=wl.norm_topk_prob, routed_scaling_factor=wl.routed_scaling_factor)
    fp8 = wl.weight_dtype == gen.FP8
    g64, eps = case["norm_weight"].double().cpu().numpy(), float(np.float32(wl.rms_norm_eps))
    # what the router sees: x, or for the sub-block the rounded RMSNorm of x
    xin = oracle.round_act(oracle.rms_norm(x64, g64, eps), wl.act_dtype) if wl.block else x64
    # one token first to size the sample to the time budget
    n = 1
    while True:
        toks = np.linspace(0, T - 1, n).astype(np.int64) if n > 1 else np.array([0])
        need = np.unique(oracle.route(xin[toks], rw, b, **kw).ids)
        host = {}
        for e in need:  # host copies of the stored weights (outside the timed region)
            host[int(e)] = {m: case["w_" + m][e].cpu() for m in ("gate", "up", "down")}
            if fp8:
                host[int(e)].update({"s_" + m: case["s_" + m][e].cpu() for m in ("gate", "up", "down")})
        sh = {m: case["sh_" + m].cpu() for m in ("gate", "up", "down")}
        if fp8:
            sh.update({"s_" + m: case["sh_s_" + m].cpu() for m in ("gate", "up", "down")})

        def mat(d, m):
            if fp8:
                return oracle.dequant_weight(d[m].numpy(), d["s_" + m].numpy())
            return d[m].to(torch.float64).numpy()

        ex = lambda e: tuple(mat(host[e], m) for m in ("gate", "up", "down"))  # noqa: E731
        shw = tuple(mat(sh, m) for m in ("gate", "up", "down")) if wl.n_shared_experts else None
        t0 = time.perf_counter()
        if wl.block:
            oracle.block_forward(x64, g64, eps, rw, b, ex, shw, act_dtype=wl.act_dtype, fp8_act=fp8, tokens=toks, **kw)
        else:
            oracle.layer_forward(x64, rw, b, ex, shw, fp8_act=fp8, tokens=toks, **kw)
        dt = time.perf_counter() - t0
        # the reported sample is the last one: at least half the budget
        # (10 s by default), or every token, or 64 tokens
        if dt >= budget_s / 2 or n >= T or n >= 64:
            break
        n = min(T, max(n + 1, int(n * budget_s / max(dt, 1e-3) * 0.6)), 64)
    threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) \
        if threadpoolctl.threadpool_info() else 1
    return {"value": round(n / dt, 4), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} of the {T} tokens (evenly spaced), {len(need)} routed experts + shared, "
                      f"fp64 numpy, {dt:.1f} s", "host_cpus": len(os.sched_getaffinity(0))}


def setup_rank(wl: gen.Workload):
    """One expert-parallel rank: its own tokens (shared expert) and the rows
    dispatched to its local experts, grouped by expert, in a buffer of T * cap
    rows (cap = rows per local token, rounded up)."""
    counts = gen.gen_dispatch_counts(wl)
    R, T = int(counts.sum()), wl.num_tokens
    cap = max(1, -(-R // T))
    rows = torch.zeros((T * cap, wl.hidden_size), dtype=gen.torch_dtype(wl.act_dtype), device="cuda")
    rows[:R] = gen.gen_dispatched_rows(wl, R).cuda()
    offsets = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).cuda()
    d = {"x": gen.gen_x(wl).cuda(), "x_rows": rows, "offsets": offsets}
    d.update(gen.gen_expert_weights(wl, device="cuda"))
    torch.cuda.synchronize()
    return d, cap, R, int((counts > 0).sum())


def make_rank_step(cfg, weights, wl, case, T):
    """The rank's share between the dispatch and combine exchanges: one
    moe_expert_ffn over the dispatched rows plus the shared expert."""
    y = torch.empty_like(case["x_rows"])
    y_sh = torch.empty((T, wl.hidden_size), dtype=gen.torch_dtype(wl.act_dtype), device="cuda")
    ws = B.alloc_workspace(cfg, T)

    def step():
        B.moe_expert_ffn(cfg, weights, case["x"], case["x_rows"], None, case["offsets"], y, y_sh, ws)
    return [step], None


def make_step(cfg, weights, wl, case, T):
    """One layer step per resident token batch, on pre-allocated buffers
    (inputs resident in HBM); returns the steps and each batch's ids."""
    ws = B.alloc_workspace(cfg, T)
    eps = float(np.float32(wl.rms_norm_eps))
    steps, ids_all = [], []
    for x in case["xs"]:
        out = torch.empty((T, wl.hidden_size), dtype=gen.torch_dtype(wl.act_dtype), device="cuda")
        ids = torch.zeros((T, wl.num_experts_per_tok), dtype=torch.int32, device="cuda")
        wts = torch.empty((T, wl.num_experts_per_tok), dtype=torch.float32, device="cuda")

        def step(x=x, out=out, ids=ids, wts=wts):
            if wl.block:
                B.moe_block_forward(cfg, weights, x, case["norm_weight"], eps, case["router_w"],
                                    case["router_bias"], out, ws, ids, wts)
            else:
                B.moe_layer_forward(cfg, weights, x, case["router_w"], case["router_bias"], out, ws, ids, wts)
        steps.append(step)
        ids_all.append(ids)
    return steps, ids_all


def rotate(fns):
    """A callable that runs fns[0], fns[1], ... in turn, one per call."""
    state = {"i": 0}

    def run():
        fns[state["i"] % len(fns)]()
        state["i"] += 1
    return run


def graphed(step):
    """One step captured in a HIP graph (the library launches kernels only);
    returns a callable that replays it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step()
    torch.cuda.synchronize()
    # the first replay of a graph also uploads it: part of the set-up, so
    # that no timed step (with fewer warm-up steps than token batches) pays it
    g.replay()
    torch.cuda.synchronize()
    return g.replay


GRAPH = False
LAST_DOWN_MS = None   # mean down-GEMM launch of the last measure()


def measure(cfg, weights, wl, case, T, steps, warmup, hip, factory=make_step):
    """Time `steps` layer steps after `warmup` untimed ones (synchronised on
    both sides), the steps rotating among the resident token batches; the
    gate_up launch of every timed step is bracketed by HIP events the library
    records on its own stream (not with graph replay, which records no
    events: gate_up is then timed on as many eager steps after the timed
    region).  Before the timed region a 512 MB buffer is written, so the
    256 MB MALL holds none of the inputs.  n_active is the mean over the
    batches of the experts their tokens select."""
    fns, ids = factory(cfg, weights, wl, case, T)
    eager = rotate(fns)
    step = rotate([graphed(f) for f in fns]) if GRAPH else eager
    for _ in range(warmup):
        step()
    evs = [(hip.event(), hip.event()) for _ in range(steps)]
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    flush.fill_(1)
    torch.cuda.synchronize()
    del flush
    evd = [(hip.event(), hip.event()) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        if not GRAPH:
            B.moe_profile_arm(B.MOE_KID_GATE_UP, *evs[i])
            B.moe_profile_arm(B.MOE_KID_DOWN, *evd[i])
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if GRAPH:
        for i in range(steps):
            B.moe_profile_arm(B.MOE_KID_GATE_UP, *evs[i])
            B.moe_profile_arm(B.MOE_KID_DOWN, *evd[i])
            eager()
        torch.cuda.synchronize()
    gate_up_ms = float(np.mean([hip.elapsed_ms(a, b) for a, b in evs]))  # every eager step launches it
    global LAST_DOWN_MS
    LAST_DOWN_MS = float(np.mean([hip.elapsed_ms(a, b) for a, b in evd]))
    n_active = None
    if ids is not None:
        for f in fns:   # every batch once more, so that each one's ids are there
            f()
        torch.cuda.synchronize()
        n_active = float(np.mean([torch.unique(i).numel() for i in ids]))
    return eager, step, wall, gate_up_ms, n_active


def layer_bytes(wl, T, n_active, router=True):
    """Algorithmic HBM bytes of one layer step: every active expert's and the
    shared expert's weights once, the router (unless `router` is false), x in
    and out."""
    F, Fs, H, E = wl.moe_intermediate_size, wl.shared_intermediate_size, wl.hidden_size, wl.n_routed_experts
    per = weight_bytes_per_expert_gate_up(wl, F) * 3 // 2
    sh = weight_bytes_per_expert_gate_up(wl, Fs) * 3 // 2 if Fs else 0
    act = 2 if wl.act_dtype == gen.BF16 else 4
    return round(n_active * per) + sh + (E * H * act + 4 * E if router else 0) + 2 * T * H * act


def layer_flops(wl, T, routed_rows=None):
    """Algorithmic flops of one layer step: 2 * 3 * H * F per routed row and
    2 * 3 * H * Fs per token for the shared expert, plus the router's 2*T*H*E
    (padded tile rows and skipped experts not counted)."""
    F, Fs, H, E, k = (wl.moe_intermediate_size, wl.shared_intermediate_size, wl.hidden_size,
                      wl.n_routed_experts, wl.num_experts_per_tok)
    rows = T * k if routed_rows is None else routed_rows
    router = 0 if routed_rows is not None else 2.0 * T * H * E
    return 6.0 * H * (rows * F + T * Fs) + router


def layer_roofline(wl, T, n_active, ms, routed_rows=None):
    """Whole-layer fractions of the HBM and MFMA peaks, and which one binds:
    max(t_bytes, t_flops) / t."""
    by = layer_bytes(wl, T, n_active, router=routed_rows is None)   # a rank's FFN share has no router
    if routed_rows is not None:   # ... but reads and writes its dispatched rows as well
        by += 2 * routed_rows * wl.hidden_size * (2 if wl.act_dtype == gen.BF16 else 4)
    fl = layer_flops(wl, T, routed_rows)
    sec = ms * 1e-3
    t_b, t_f = by / (PEAK_HBM_GBS * 1e9), fl / (PEAK_TFLOPS[wl.weight_dtype] * 1e12)
    return {"bytes": by, "flops": fl, "hbm_frac": round(t_b / sec, 4), "mfma_frac": round(t_f / sec, 4),
            "binding": "hbm" if t_b >= t_f else "mfma", "binding_frac": round(max(t_b, t_f) / sec, 4)}


def sweep(args, wl, case, cfg, weights, hip, ceilings=None):
    """Sweep over token counts on the same resident weights; one JSON record
    per point (tokens/s, time per step, active experts, the whole layer's
    fractions of 8 TB/s and of the dtype's MFMA peak, and the two grouped
    GEMMs' rooflines, each also against the measured ceilings when given)."""
    recs = []
    for T in [int(t) for t in args.sweep_tokens.split(",")]:
        c = dict(case)
        c["xs"] = [gen.gen_x(wl, T, b).cuda() for b in range(X_BATCHES)]
        _, _, wall, gu_ms, n_act = measure(cfg, weights, wl, c, T, args.steps, args.warmup, hip)
        ms = wall * 1e3 / args.steps
        by = layer_bytes(wl, T, n_act)
        lr = layer_roofline(wl, T, n_act, ms)
        rec = {"workload": wl.name, "num_tokens": T, "ms_per_step": round(ms, 4),
               "tokens_per_s": round(T / ms * 1e3, 1), "active_experts": n_act,
               "layer_bytes": by, "layer_hbm_frac": round(by / (ms * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
               "layer_mfma_frac": lr["mfma_frac"], "binding": lr["binding"],
               "gate_up_ms": round(gu_ms, 4), "down_ms": round(LAST_DOWN_MS, 4),
               "gate_up_roofline": with_measured(roofline(wl, T, n_act, gu_ms, None), ceilings),
               "down_roofline": with_measured(roofline(wl, T, n_act, LAST_DOWN_MS, None, kernel="down"), ceilings)}
        if ceilings:
            peak = ceilings["mfma_fp8_loop_tflops" if wl.weight_dtype == gen.FP8 else "mfma_bf16_loop_tflops"]
            rec["layer_mfma_frac_measured"] = round(layer_flops(wl, T) / (ms * 1e-3) / 1e12 / peak, 4)
            rec["layer_hbm_frac_measured"] = round(by / (ms * 1e-3) / 1e9 / ceilings["hbm_read_gbs"], 4)
        print(f"[sweep] {json.dumps(rec)}", file=sys.stderr)
        recs.append(rec)
    return recs


PREFILL = "k2_prefill_bf16_zipf"


def prefill_leg(case, steps, warmup, hip, ceilings):
    """The prefill half of the metric on the decode run's resident weights:
    the Zipf-skewed K2 layer at T = 8192 (same expert and router weights;
    its own bias and 4 token batches), graph-replayed as the decode line."""
    wl = gen.WORKLOADS[PREFILL]
    dec = gen.WORKLOADS["k2_decode_bf16"]
    same = ("hidden_size", "moe_intermediate_size", "n_routed_experts", "n_shared_experts", "weight_dtype",
            "act_dtype", "weight_std", "seed")
    assert all(getattr(wl, f) == getattr(dec, f) for f in same), "prefill needs the decode run's weights"
    T = wl.num_tokens
    c = {k: v for k, v in case.items() if k not in ("x", "xs", "router_bias")}
    c["xs"] = [gen.gen_x(wl, T, b).cuda() for b in range(X_BATCHES)]
    c["x"] = c["xs"][0]
    c["router_bias"] = gen.gen_bias(wl).cuda()
    cfg = B.MoeConfig.from_fields(wl.fields())
    weights = B.MoeWeights.from_tensors(c)
    _, timed_step, wall, gu_ms, n_act = measure(cfg, weights, wl, c, T, steps, warmup, hip)
    dn_ms = LAST_DOWN_MS
    ms = wall * 1e3 / steps
    singles = [timed(timed_step, 1, warm=0) for _ in range(10)]
    rec = {"workload": wl.name, "num_tokens": T, "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4),
           "tokens_per_s": round(T * steps / wall, 1), "active_experts": n_act,
           "roofline": with_measured(roofline(wl, T, n_act, gu_ms, stored_traffic(PREFILL, T)), ceilings),
           "down_roofline": with_measured(roofline(wl, T, n_act, dn_ms, None, kernel="down"), ceilings),
           "layer_roofline": layer_roofline(wl, T, n_act, ms),
           "step_ms_p10_p50_p90": [round(float(np.percentile(singles, q)), 4) for q in (10, 50, 90)]}
    if ceilings:
        rec["layer_roofline"]["mfma_frac_measured"] = round(
            layer_flops(wl, T) / (ms * 1e-3) / 1e12 / ceilings["mfma_bf16_loop_tflops"], 4)
    del c
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="k2_decode_bf16", choices=sorted(gen.WORKLOADS))
    ap.add_argument("--tokens", type=int, default=None, help="override the workload's token count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work")
    ap.add_argument("--breakdown", action="store_true", help="per-kernel times to stderr")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--extra-out", default=None, help="append a detail JSON line to this file")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from the host instead of replaying one captured HIP graph")
    ap.add_argument("--sweep-tokens", default=None,
                    help="comma-separated token counts measured after the main line (stderr / --extra-out)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill (T=8192, Zipf) object of the default decode run")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured-ceiling probes")
    ap.add_argument("--ceilings-only", action="store_true", help="print the measured ceilings and exit")
    ap.add_argument("--traffic-json", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="write profiles/traffic_gate_up_<workload>.json from the csv output of a FETCH_SIZE "
                         "and a WRITE_SIZE rocprofv3 pass of this workload (with --calib-copy), then exit")
    args = ap.parse_args()
    if args.traffic_json:
        wl = gen.WORKLOADS[args.workload]
        print(json.dumps(write_traffic(args.workload, args.tokens or wl.num_tokens, *args.traffic_json)))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer runs unsharded on a single MI355X)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.ceilings_only:
        print(json.dumps({"ceilings": measure_ceilings()}))
        return
    wl = gen.WORKLOADS[args.workload]
    T = args.tokens or wl.num_tokens
    global GRAPH
    GRAPH = not args.eager
    B.load()
    hip = Hip()
    ceilings = None if args.no_ceilings else measure_ceilings()
    torch.cuda.empty_cache()
    rank = wl.ep_size > 1
    routed_rows = None
    if rank:
        if args.tokens or args.sweep_tokens or not args.no_cpu_baseline:
            print("an expert-parallel rank workload runs at its own token count, without the oracle "
                  "baseline (pass --no-cpu-baseline)", file=sys.stderr)
            sys.exit(2)
        case, cap, routed_rows, n_local = setup_rank(wl)
        cfg = B.MoeConfig.from_fields(dict(wl.fields(), num_experts_per_tok=cap))
    else:
        case = setup(wl, T)
        cfg = B.MoeConfig.from_fields(wl.fields())
    weights = B.MoeWeights.from_tensors(case)
    step, timed_step, wall, gate_up_ms, n_active = measure(cfg, weights, wl, case, T, args.steps, args.warmup, hip,
                                               make_rank_step if rank else make_step)
    if rank:
        n_active = n_local
    ms_per_step = wall * 1e3 / args.steps

    detail = {}
    if args.breakdown:
        names = ["router_logits", "router_topk", "permute", "tiles", "gather", "act_quant", "gate_up", "down",
                 "combine", "norm"]
        per = {n: [] for n in names}
        for _ in range(5):
            pairs = [(hip.event(), hip.event()) for _ in names]
            for kid, (a, b) in enumerate(pairs):
                B.moe_profile_arm(kid, a, b)
            step()
            torch.cuda.synchronize()
            for kid, (a, b) in enumerate(pairs):
                ms = hip.elapsed_ms(a, b)
                if ms is not None:
                    per[names[kid]].append(ms)
            for kid in range(len(names)):
                B.moe_profile_arm(kid, None, None)
        detail = {n: round(float(np.median(v)), 4) for n, v in per.items() if v}
        print(f"[breakdown ms] {detail}", file=sys.stderr)
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    down_ms = LAST_DOWN_MS
    rl = with_measured(roofline(wl, T, n_active, gate_up_ms, stored_traffic(args.workload, T), routed_rows),
                       ceilings)
    # spread of 20 single steps after the timed region, launched as the timed
    # ones were (the timed figure is the mean over exactly `steps` back-to-back steps)
    singles = []
    for _ in range(20):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        timed_step()
        e1.record()
        e1.synchronize()
        singles.append(e0.elapsed_time(e1))
    res = {
        "metric": METRIC, "value": round(T * args.steps / wall, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3" if wl.weight_dtype == gen.FP8 else wl.act_dtype, "data": "synthetic",
        "config": {"workload": wl.name, "num_tokens": T, "hidden_size": wl.hidden_size,
                   "moe_intermediate_size": wl.moe_intermediate_size, "n_routed_experts": wl.n_routed_experts,
                   "num_experts_per_tok": wl.num_experts_per_tok, "n_shared_experts": wl.n_shared_experts,
                   "n_group": wl.n_group, "topk_group": wl.topk_group, "active_experts": n_active,
                   "parallelism": "none (one GPU, all experts resident)",
                   "launch": "eager" if args.eager else "hip graph replay (one captured layer step per token batch)"},
        "roofline": rl,
        "down_roofline": with_measured(roofline(wl, T, n_active, down_ms, None, routed_rows, kernel="down"),
                                       ceilings),
        "layer_roofline": layer_roofline(wl, T, n_active, ms_per_step, routed_rows),
        "step_ms_p10_p50_p90": [round(float(np.percentile(singles, q)), 4) for q in (10, 50, 90)],
    }
    if ceilings:
        lr = res["layer_roofline"]
        lr["hbm_frac_measured"] = round(lr["bytes"] / (ms_per_step * 1e-3) / 1e9 / ceilings["hbm_read_gbs"], 4)
        res["ceilings"] = ceilings
    if args.workload == "k2_decode_bf16" and not args.tokens and not args.no_prefill:
        res["prefill"] = prefill_leg(case, args.prefill_steps, min(args.warmup, 3), hip, ceilings)
    if rank:
        res["config"].update(parallelism=f"one rank of ep{wl.ep_size} (its expert FFN share only)",
                             global_experts=wl.n_routed_experts * wl.ep_size, dispatched_rows=routed_rows,
                             row_capacity_per_token=cap)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, case, T, args.cpu_budget)
    recs = sweep(args, wl, case, cfg, weights, hip, ceilings) if args.sweep_tokens else []
    if args.extra_out:
        with open(args.extra_out, "a") as f:
            f.write(json.dumps({**res, "breakdown_ms": detail, "kernel_hash": kernel_hash()}) + "\n")
            for r in recs:
                f.write(json.dumps({"sweep": r}) + "\n")
    print(json.dumps(res))


if __name__ == "__main__":
    main()
