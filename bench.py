"""Benchmark of the W4A4G4 quantized linear (FourTune) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2] [--no-cpu-baseline]
    python bench.py --calibrate-copy     (a plain 512 MiB device copy, for counter scaling)
    python bench.py --ablation           (fusion ablation; one JSON line of its own)
    python bench.py --dit                (every linear of a FLUX-shaped DiT; one JSON line)
    python bench.py --granularity        (32x32 blocks vs 1x32 groups: error study; one JSON line)
    python bench.py --precision          (the four precision configurations at c2; one JSON line)
    python bench.py --gemm-sweep         (both 4-bit GEMMs of every linear of c2..c5; one JSON line)
    python bench.py --hbm-sweep          (quantizer, fused quantize + down-projection, MLP pass, c2..c5)

One step = the whole hot path once over one batch: the layer's forward (fused
quantize + down-projection, 4-bit GEMM + up-projection) and backward (fused quantize +
down-projection of dY, transposed 4-bit GEMM + up-projection, LoRA gradients), every
kernel of `fourtune_linear_fwd` and `fourtune_linear_bwd`. Inputs are seeded synthetic
tensors of the named workload, resident in HBM before timing; several independent
input/weight sets are rotated so that the 256 MB Infinity Cache cannot carry a step's
operands over from the step before.

Prints one JSON line. `value` is 4*M*N*K (the 4-bit GEMM flops of forward and
backward) divided by the whole step's time. `roofline` is the dominant kernel (the
forward 4-bit GEMM) against the dense MXFP4 peak, its duration taken with HIP events
on the stream it is launched on; `traffic` comes from the rocprofv3 counter summary
in profiles/ when that summary was taken on the current kernel source, else null.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MXFP4_TFLOPS = 10100.0   # MI355X dense MXFP4 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_fwd_c2_traffic.json")
GEMM_SRC = os.path.join(ROOT, "bit_quantized_lora_fp4_amd", "csrc", "gemm.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--sets", type=int, default=20,
                    help="rotated input/weight sets (20 at c2: the per-kernel timings stream more "
                         "than twice the 256 MB Infinity Cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--ablation", action="store_true",
                    help="fusion ablation: bf16 LoRA, unfused and fused W4A4G4 at c2 (linear), c3 (MLP)")
    ap.add_argument("--dit", action="store_true",
                    help="all linears of a FLUX-shaped DiT (synthetic weights), W4A4G4 vs bf16 LoRA")
    ap.add_argument("--granularity", action="store_true",
                    help="32x32 blocks vs 1x32 groups for X and dY: quantization error study")
    ap.add_argument("--precision", action="store_true",
                    help="W4A4G4 vs W4A16G4 / W4A4G16 / W4A16G16 at c2")
    ap.add_argument("--hbm-sweep", action="store_true",
                    help="HBM-bound kernels (quantizer, fused quantize + down-projection, MLP pass) of c2..c5")
    ap.add_argument("--gemm-sweep", action="store_true",
                    help="4-bit GEMM TFLOPS and MXFP4-peak fraction for every linear of c2..c5")
    ap.add_argument("--double-blocks", type=int, default=19)
    ap.add_argument("--single-blocks", type=int, default=38)
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


# --------------------------------------------------------------------------- GPU side
def build_sets(case, nsets, torch, abi):
    """Device copies of one linear's operands; set i gets its own buffers."""
    dt = {"fp32": torch.float32, "bf16": torch.bfloat16}
    m, k = case["X"].shape
    n = case["R"].shape[0]
    sets = []
    for i in range(nsets):
        def d(a, dtype):
            return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dt[dtype])
        L = abi.make_linear(d(case["R"], "fp32"), d(case["A"], "bf16"), d(case["B"], "bf16"),
                            d(case["L1"], "bf16"), d(case["L2"], "bf16"))
        rt = L.rank + L.stab_rank
        s = dict(L=L, x=d(case["X"], case["x_dtype"]), dy=d(case["dY"], case["dy_dtype"]),
                 y=torch.empty((m, n), dtype=torch.bfloat16, device="cuda"),
                 dx=torch.empty((m, k), dtype=torch.bfloat16, device="cuda"),
                 xl=torch.empty((m, rt), dtype=torch.bfloat16, device="cuda"),
                 da=torch.empty((L.rank, k), dtype=torch.float32, device="cuda"),
                 db=torch.empty((n, L.rank), dtype=torch.float32, device="cuda"),
                 ws=abi.workspace(abi.fourtune_linear_workspace_bytes(m, L)),
                 xq=abi.Mx4.empty(m, k), gq=abi.Mx4.empty(m, n),
                 gb=(torch.randn((m, rt), device="cuda") * 1e-3).to(torch.bfloat16))
        sets.append(s)
    return sets


def step(abi, s):
    abi.fourtune_linear_fwd(s["L"], s["x"], s["y"], s["xl"], s["ws"])
    abi.fourtune_linear_bwd(s["L"], s["dy"], s["x"], s["xl"], s["dx"], s["da"], s["db"], s["ws"])


def time_region(torch, fn, iters):
    """Seconds for `iters` calls, bracketed by a synchronize on both sides. Python's
    cyclic garbage collector is paused inside the region, as timeit does: a collection
    pass that lands there holds the calling thread for tens of milliseconds (observed:
    one 40 ms gap in 20 calls of a 0.11 ms step), and the GPU idles meanwhile."""
    import gc

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    was_enabled = gc.isenabled()
    gc.collect()
    gc.disable()
    try:
        torch.cuda.synchronize()
        start.record()
        for i in range(iters):
            fn(i)
        end.record()
        torch.cuda.synchronize()
    finally:
        if was_enabled:
            gc.enable()
    return start.elapsed_time(end) / 1000.0


def time_graph(torch, fn, iters):
    """Mean duration of fn(i) launched back to back from a captured HIP graph, timed by
    events on the stream the graph replays on: no host call overhead between launches,
    so the figure is the kernels' own time (the library allocates nothing and never
    synchronizes, so its calls capture as they are)."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(iters):
            fn(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1000.0 / iters


def traffic_for(m, n, k):
    """Counter-measured HBM bytes per forward-GEMM launch, if taken on this source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("gemm_src_sha256_16") != source_hash(GEMM_SRC) or t.get("shape") != [m, n, k]:
        return None
    return t.get("bytes_per_launch")


def calibrate_copy():
    import torch
    nbytes = 512 << 20
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": nbytes, "bytes_written": nbytes, "launches": 5}))
    return 0


# --------------------------------------------------------------------------- fusion ablation
def _torch_lora_linear(torch, case, dev="cuda"):
    """Standard bf16 LoRA linear (frozen W, adapter A, B; no stabilizer, nothing
    quantized): the baseline the pages compare against. Right-hand operands are kept
    contiguous; only left operands are transposed views."""
    bf = torch.bfloat16

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(bf)

    W = d(case["R"].astype(np.float32) + case["L2"].astype(np.float32) @ case["L1"].astype(np.float32))
    A, B = d(case["A"]), d(case["B"])
    return dict(W=W, Wt=W.t().contiguous(), A=A, At=A.t().contiguous(), B=B, Bt=B.t().contiguous())


def _lora_fwd(torch, p, x):
    xa = torch.mm(x, p["At"])
    return torch.mm(x, p["Wt"]) + torch.mm(xa, p["Bt"]), xa


def _lora_bwd(torch, p, dy, x, xa):
    gb = torch.mm(dy, p["B"])
    dx = torch.mm(dy, p["W"]) + torch.mm(gb, p["A"])
    da = torch.mm(gb.t(), x)
    db = torch.mm(dy.t(), xa)
    return dx, da, db


def ablation(args):
    """Layer-level reproduction of the structure of the pages' fusion breakdown (FourTune
    §4, Figure 9): the same W4A4G4 layer unfused (every step a launch, intermediates in
    HBM), with LoRA fusion only, fully fused; and a standard bf16 LoRA layer. Times are
    per fwd+bwd, from HIP graph replays (kernel time) and from plain back-to-back calls
    bracketed by events (what a caller sees, launch overheads included)."""
    import torch
    import torch.nn.functional as F
    from bit_quantized_lora_fp4_amd import abi
    from synth import workloads as wl

    abi.lib()
    it = max(args.steps, 10)
    res = {}

    def both(fn, n_sets):
        for i in range(args.warmup):
            fn(i % n_sets)
        torch.cuda.synchronize()
        eager = time_region(torch, lambda i: fn(i % n_sets), it) / it
        return dict(graph_ms=round(1e3 * time_graph(torch, lambda i: fn(i % n_sets), it), 4),
                    eager_ms=round(1e3 * eager, 4))

    # ---- one linear, c2
    log("[ablation] c2 linear")
    case = wl.linear_case("c2")
    m, k = case["X"].shape
    n = case["R"].shape[0]
    sets = build_sets(case, 2, torch, abi)
    for s in sets:
        s["ws_ab"] = abi.workspace(abi.fourtune_ablation_workspace_bytes(m, s["L"]))
        s["lora"] = _torch_lora_linear(torch, case)
        s["xa"] = torch.empty((m, s["L"].rank), dtype=torch.bfloat16, device="cuda")

    def lin_fused(i):
        step(abi, sets[i])

    def lin_unfused(i):
        s = sets[i]
        abi.fourtune_linear_fwd_unfused(s["L"], s["x"], s["y"], s["xl"], s["ws_ab"])
        abi.fourtune_linear_bwd_unfused(s["L"], s["dy"], s["x"], s["xl"], s["dx"], s["da"], s["db"], s["ws_ab"])

    def lin_bf16(i):
        s = sets[i]
        y, xa = _lora_fwd(torch, s["lora"], s["x"])
        _lora_bwd(torch, s["lora"], s["dy"], s["x"], xa)

    lin = dict(bf16_lora=both(lin_bf16, 2), w4_unfused=both(lin_unfused, 2), w4_fused=both(lin_fused, 2))
    for key in ("graph_ms", "eager_ms"):
        lin[f"lora_fusion_speedup_{key[:-3]}"] = round(lin["w4_unfused"][key] / lin["w4_fused"][key], 3)
        lin[f"fused_vs_bf16_lora_{key[:-3]}"] = round(lin["bf16_lora"][key] / lin["w4_fused"][key], 3)
    lin["shape"] = dict(m=m, n=n, k=k, lora_rank=case["A"].shape[0], stab_rank=case["L1"].shape[0])
    res["linear_c2"] = lin
    del sets
    torch.cuda.empty_cache()

    # ---- the MLP pair, c3
    log("[ablation] c3 MLP")
    mc = wl.mlp_case("c3")
    m, dm = mc["X"].shape
    f = mc["fc1"]["R"].shape[0]
    bf = dict(dtype=torch.bfloat16, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")

    def dv(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(
            torch.bfloat16 if dt == "bf16" else torch.float32)

    msets = []
    for i in range(2):
        p1, p2 = mc["fc1"], mc["fc2"]
        fc1 = abi.make_linear(dv(p1["R"], "fp32"), dv(p1["A"], "bf16"), dv(p1["B"], "bf16"), dv(p1["L1"], "bf16"),
                              dv(p1["L2"], "bf16"))
        fc2 = abi.make_linear(dv(p2["R"], "fp32"), dv(p2["A"], "bf16"), dv(p2["B"], "bf16"), dv(p2["L1"], "bf16"),
                              dv(p2["L2"], "bf16"))
        rt1, rt2 = fc1.rank + fc1.stab_rank, fc2.rank + fc2.stab_rank
        s = dict(fc1=fc1, fc2=fc2, x=dv(mc["X"], mc["x_dtype"]), dy=dv(mc["dY"], mc["dy_dtype"]),
                 y=torch.empty((m, dm), **bf), dx=torch.empty((m, dm), **bf),
                 xl1=torch.empty((m, rt1), **bf), pre=torch.empty((m, f), **bf), h=torch.empty((m, f), **bf),
                 hl2=torch.empty((m, rt2), **bf),
                 g=[torch.empty((fc1.rank, dm), **f32), torch.empty((f, fc1.rank), **f32),
                    torch.empty((fc2.rank, f), **f32), torch.empty((dm, fc2.rank), **f32)],
                 ws=abi.workspace(abi.fourtune_mlp_workspace_bytes(m, fc1, fc2)),
                 ws_ab=abi.workspace(abi.fourtune_ablation_workspace_bytes(m, fc1, fc2)),
                 l1=_torch_lora_linear(torch, p1), l2=_torch_lora_linear(torch, p2))
        msets.append(s)
    torch.cuda.synchronize()

    def mlp_level(lf):
        def fn(i):
            s = msets[i]
            abi.fourtune_mlp_fwd_unfused(s["fc1"], s["fc2"], lf, s["x"], s["y"], s["xl1"], s["pre"], s["h"],
                                         s["hl2"], s["ws_ab"])
            abi.fourtune_mlp_bwd_unfused(s["fc1"], s["fc2"], lf, s["dy"], s["x"], s["xl1"], s["pre"], s["h"],
                                         s["hl2"], s["dx"], *s["g"], s["ws_ab"])
        return fn

    def mlp_fused(i):
        s = msets[i]
        abi.fourtune_mlp_fwd(s["fc1"], s["fc2"], s["x"], s["y"], s["xl1"], s["pre"], s["hl2"], s["ws"])
        abi.fourtune_mlp_bwd(s["fc1"], s["fc2"], s["dy"], s["x"], s["xl1"], s["pre"], s["hl2"], s["dx"], *s["g"],
                             s["ws"])

    def mlp_bf16(i):
        s = msets[i]
        p, xa1 = _lora_fwd(torch, s["l1"], s["x"])
        h = F.gelu(p, approximate="tanh")
        y, xa2 = _lora_fwd(torch, s["l2"], h)
        dh, _, _ = _lora_bwd(torch, s["l2"], s["dy"], h, xa2)
        dp = torch.ops.aten.gelu_backward(dh, p, approximate="tanh")
        _lora_bwd(torch, s["l1"], dp, s["x"], xa1)

    mlp = dict(bf16_lora=both(mlp_bf16, 2), w4_unfused=both(mlp_level(False), 2),
               w4_lora_fused=both(mlp_level(True), 2), w4_all_fused=both(mlp_fused, 2))
    for key in ("graph_ms", "eager_ms"):
        tag = key[:-3]
        mlp[f"lora_fusion_speedup_{tag}"] = round(mlp["w4_unfused"][key] / mlp["w4_lora_fused"][key], 3)
        mlp[f"mlp_fusion_speedup_{tag}"] = round(mlp["w4_lora_fused"][key] / mlp["w4_all_fused"][key], 3)
        mlp[f"all_fused_vs_bf16_lora_{tag}"] = round(mlp["bf16_lora"][key] / mlp["w4_all_fused"][key], 3)
    mlp["shape"] = dict(m=m, d=dm, f=f, lora_rank=mc["fc1"]["A"].shape[0], stab_rank=mc["fc1"]["L1"].shape[0])
    res["mlp_c3"] = mlp
    out = {"metric": "fusion ablation: fwd+bwd time per variant (FourTune Fig. 9 structure)", "unit": "ms",
           "higher_is_better": False, "n_gpus": 1, "iters": it, "data": "synthetic",
           "pages_for_context": {"lora_fusion_speedup": 1.82, "mlp_fusion_speedup": 1.10,
                                 "all_fused_vs_bf16_lora": 2.52},
           **res}
    print(json.dumps(out), flush=True)
    return 0


# --------------------------------------------------------------------------- granularity
def _deq_gpu(torch, q, groups):
    """Values of GPU-produced MXFP4 codes, as fp32 on the device (measurement only: the
    layer itself never dequantizes)."""
    grid = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], device="cuda")
    c = q.codes
    codes = torch.stack([c & 0xF, c >> 4], dim=2).reshape(c.shape[0], c.shape[1] * 2)
    mag = grid[(codes & 7).long()]
    val = torch.where((codes & 8) != 0, -mag, mag)
    s = q.scales.to(torch.int32)
    if groups:
        s = s.repeat_interleave(32, dim=1)
    else:
        s = s.repeat_interleave(32, dim=0)[: codes.shape[0]].repeat_interleave(32, dim=1)
    out = val * torch.exp2((s - 127).to(torch.float32))
    return torch.where(s == 0xFF, torch.full_like(out, float("nan")), out)


def granularity(args):
    """Synthetic stand-in for the pages' granularity comparison (FourTune §4 "Impact of
    Quantization Granularity", Table 5: block-wise against group-wise scales, measured
    there as image fidelity on a dataset that is not here): the relative Frobenius error
    of the 4-bit backbone products against the unquantized ones, with X and dY quantized
    in 32x32 blocks (what the layer uses: readable transposed) or in 1x32 groups, R in
    32x32 blocks either way, on c4's heavy-tailed activations and c2's outlier channels.
    Codes come from the library's quantizers; products are fp32 torch matmuls."""
    import torch
    from bit_quantized_lora_fp4_amd import abi
    from synth import workloads as wl

    abi.lib()
    res = {}
    for key, name in (("c4", "qkv"), ("c4", "o"), ("c2", None)):
        log(f"[granularity] {key} {name or ''}")
        case = wl.linear_case(key, name)
        dt = {"fp32": torch.float32, "bf16": torch.bfloat16}
        x = torch.from_numpy(np.ascontiguousarray(case["X"])).to("cuda").to(dt[case["x_dtype"]])
        g = torch.from_numpy(np.ascontiguousarray(case["dY"])).to("cuda").to(dt[case["dy_dtype"]])
        R = torch.from_numpy(np.ascontiguousarray(case["R"])).to("cuda").float()
        m, k = x.shape
        n = R.shape[0]
        rq = abi.quantize(R)
        Rd = _deq_gpu(torch, rq, False)
        out = {"m": m, "n": n, "k": k}
        for tname, T in (("x", x), ("dy", g)):
            qb = abi.quantize(T)
            qg = abi.Mx4.empty_groups(*T.shape)
            abi.fourtune_quantize_groups(T, qg)
            Tf = T.float()
            e = {}
            for lbl, q, grp in (("block_32x32", qb, False), ("group_1x32", qg, True)):
                Td = _deq_gpu(torch, q, grp)
                e[lbl] = {"tensor": float((Td - Tf).norm() / Tf.norm())}
                if tname == "x":
                    ref = Tf @ R.t()
                    e[lbl]["Y"] = float((Td @ Rd.t() - ref).norm() / ref.norm())
                else:
                    ref = Tf @ R
                    e[lbl]["dX"] = float((Td @ Rd - ref).norm() / ref.norm())
                del Td, ref
            t_b = time_graph(torch, lambda i: abi.fourtune_quantize(T, qb), 20)
            t_g = time_graph(torch, lambda i: abi.fourtune_quantize_groups(T, qg), 20)
            eb = T.element_size()
            byt_b = T.numel() * (eb + 0.5) + qb.scales.numel()
            byt_g = T.numel() * (eb + 0.5) + qg.scales.numel()
            e["quantize_us"] = {"block_32x32": round(t_b * 1e6, 2), "group_1x32": round(t_g * 1e6, 2)}
            e["quantize_gbps"] = {"block_32x32": round(byt_b / t_b / 1e9, 1), "group_1x32": round(byt_g / t_g / 1e9, 1)}
            out[tname] = e
        res[f"{key}_{name}" if name else key] = out
        del x, g, R, Rd
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "relative Frobenius error of the 4-bit backbone products vs unquantized, "
                                "32x32 blocks vs 1x32 groups for X and dY (FourTune Table 5 stand-in)",
                      "unit": "relative error", "data": "synthetic", "n_gpus": 1, **res}), flush=True)
    return 0


# --------------------------------------------------------------------------- GEMM sweep
def time_graph_stats(torch, fn, per_graph=10, replays=20):
    """Per-launch time of fn(i) from `replays` replays of a graph of `per_graph`
    back-to-back launches: (median, p10, p90) over the replays, in seconds."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            fn(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(replays):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) / 1000.0 / per_graph)
    ts = np.array(ts)
    return float(np.median(ts)), float(np.percentile(ts, 10)), float(np.percentile(ts, 90))


def gemm_sweep(args):
    """Both 4-bit GEMM kernels (forward Q(X)Q(R)^T + XL U^T; backward Q(dY)Q(R) + GB D)
    of every linear of c2..c5 at full size: TFLOP/s of the 2*M*N*K backbone flops and
    the fraction of the dense MXFP4 peak, median / p10 / p90 over graph replays. Codes
    and block scales are random bytes (every nibble is an E2M1 code; scale bytes kept
    in 110..140), the low-rank operands random bf16: the kernels' time does not depend
    on the values. Input sets rotate so that operands are not cache-resident."""
    import torch
    from bit_quantized_lora_fp4_amd import abi
    from synth import workloads as wl

    abi.lib()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)

    def codes(rows, cols):
        q = abi.Mx4.empty(rows, cols)
        q.codes.copy_(torch.randint(0, 256, q.codes.shape, generator=gen, device="cuda", dtype=torch.int32).to(torch.uint8))
        q.scales.copy_(torch.randint(110, 141, q.scales.shape, generator=gen, device="cuda", dtype=torch.int32).to(torch.uint8))
        return q

    def bf(shape):
        return (torch.randn(shape, generator=gen, device="cuda") * 0.01).to(torch.bfloat16)

    res = {}
    for key in ("c2", "c3", "c4", "c5"):
        spec = wl.WORKLOADS[key]
        m = spec.m
        lins = []
        for ls in spec.layers:
            if isinstance(ls, wl.LinearSpec):
                lins.append((ls.name, ls.n, ls.k, ls.r, ls.s))
            else:
                lins += [(ls.name + ".fc1", ls.f, ls.d, ls.r, ls.s), (ls.name + ".fc2", ls.d, ls.f, ls.r, ls.s)]
        for name, n, k, r, s in lins:
            nsets = 2 if m * max(n, k) > 1 << 27 else 4
            sets = []
            for _ in range(nsets):
                L = abi.Linear(codes(n, k), bf((r, k)), bf((n, r)), bf((s, k)), bf((n, s)))
                sets.append(dict(L=L, xq=codes(m, k), gq=codes(m, n), xl=bf((m, r + s)), gb=bf((m, r + s)),
                                 y=torch.empty((m, n), dtype=torch.bfloat16, device="cuda"),
                                 dx=torch.empty((m, k), dtype=torch.bfloat16, device="cuda")))
            torch.cuda.synchronize()
            S = lambda i: sets[i % nsets]
            f = time_graph_stats(torch, lambda i: abi.fourtune_gemm_fwd(S(i)["L"], S(i)["xq"], S(i)["xl"], S(i)["y"]))
            b = time_graph_stats(torch, lambda i: abi.fourtune_gemm_bwd(S(i)["L"], S(i)["gq"], S(i)["gb"], S(i)["dx"]))
            flops = 2.0 * m * n * k
            row = {"m": m, "n": n, "k": k, "rt": r + s}
            for tag, (med, p10, p90) in (("fwd", f), ("bwd", b)):
                row[tag] = {"us_median": round(med * 1e6, 2), "us_p10": round(p10 * 1e6, 2), "us_p90": round(p90 * 1e6, 2),
                            "tflops": round(flops / med / 1e12, 1), "frac": round(flops / med / 1e12 / PEAK_MXFP4_TFLOPS, 4)}
            row["fwd_bwd_frac"] = round(2 * flops / (f[0] + b[0]) / 1e12 / PEAK_MXFP4_TFLOPS, 4)
            res[f"{key}.{name}"] = row
            log(f"[gemm-sweep] {key}.{name} m={m} n={n} k={k}: fwd {f[0]*1e6:.1f} us, bwd {b[0]*1e6:.1f} us, "
                f"{row['fwd_bwd_frac']*100:.1f}% of peak")
            del sets
            torch.cuda.empty_cache()
    print(json.dumps({"metric": "4-bit GEMM kernels: 2*M*N*K / time, fraction of dense MXFP4 peak",
                      "unit": "TFLOP/s", "peak": PEAK_MXFP4_TFLOPS, "n_gpus": 1, "data": "synthetic codes",
                      **res}), flush=True)
    return 0


# --------------------------------------------------------------------------- HBM-bound kernels
def hbm_sweep(args):
    """The HBM-bound kernels of every workload at full size, against the 8 TB/s peak:
    the quantizer on each activation (bf16 read 2 B + codes 0.5 B + scales 1/1024 B per
    element), the fused quantize + down-projection of each linear's forward with its
    partial sum (plus 2 rt / K B per element for the saved XL; taken as the linear's
    forward minus its GEMM), and the MLP's pass over the saved P^ (GELU, Q(H), HL2: P^
    read 2 B + 0.5 B codes per element; taken as the MLP forward minus FC1's linear
    forward and FC2's GEMM). Graph replays over rotated input sets, at least 640 MB of X
    in rotation so that it streams from HBM rather than the 256 MB Infinity Cache;
    median per launch; random bf16 operands (the kernels' time does not depend on the
    values). Per-kernel durations of the same run come from rocprofv3's kernel trace."""
    import torch
    from bit_quantized_lora_fp4_amd import abi
    from synth import workloads as wl

    abi.lib()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)

    def bf(shape, std=1.0):
        return (torch.randn(shape, generator=gen, device="cuda") * std).to(torch.bfloat16)

    def lin(n, k, r, s):
        return abi.Linear(abi.quantize(bf((n, k), 0.02)), bf((r, k), 0.01), bf((n, r), 0.01), bf((s, k), 0.1),
                          bf((n, s), 0.1))

    def gbps(nbytes, t):
        return round(nbytes / t / 1e9, 1)

    res = {}
    for key in ("c2", "c3", "c4", "c5"):
        spec = wl.WORKLOADS[key]
        m = spec.m
        for ls in spec.layers:
            is_mlp = not isinstance(ls, wl.LinearSpec)
            k = ls.d if is_mlp else ls.k
            n = ls.f if is_mlp else ls.n
            r, s_ = ls.r, ls.s
            rt = r + s_
            # enough input sets that X streams from HBM in rotation, not from the 256 MB cache
            nsets = max(2, -(-(640 << 20) // (m * k * 2)))
            sets = []
            for _ in range(nsets):
                st = dict(x=bf((m, k)), L=lin(n, k, r, s_), y=torch.empty((m, n), dtype=torch.bfloat16, device="cuda"),
                          xl=torch.empty((m, rt), dtype=torch.bfloat16, device="cuda"), xq=abi.Mx4.empty(m, k))
                if is_mlp:
                    st["fc2"] = lin(ls.d, ls.f, r, s_)
                    st["hq"] = abi.quantize(bf((m, ls.f)))
                    st["hl2"] = bf((m, rt), 0.1)
                    st["out"] = torch.empty((m, ls.d), dtype=torch.bfloat16, device="cuda")
                    st["ws"] = abi.workspace(max(abi.fourtune_mlp_workspace_bytes(m, st["L"], st["fc2"]),
                                                 abi.fourtune_linear_workspace_bytes(m, st["L"])))
                else:
                    st["ws"] = abi.workspace(abi.fourtune_linear_workspace_bytes(m, st["L"]))
                sets.append(st)
            torch.cuda.synchronize()
            S = lambda i: sets[i % nsets]
            tq = time_graph_stats(torch, lambda i: abi.fourtune_quantize(S(i)["x"], S(i)["xq"]))[0]
            tf = time_graph_stats(torch, lambda i: abi.fourtune_linear_fwd(S(i)["L"], S(i)["x"], S(i)["y"], S(i)["xl"],
                                                                           S(i)["ws"]))[0]
            tg = time_graph_stats(torch, lambda i: abi.fourtune_gemm_fwd(S(i)["L"], S(i)["xq"], S(i)["xl"], S(i)["y"]))[0]
            q_bytes = m * k * 2.5 + ((m + 31) // 32) * (k // 32)
            qd_bytes = q_bytes + m * rt * 2
            name = f"{key}.{ls.name}" + (".fc1" if is_mlp else "")
            row = {"m": m, "k": k, "n": n, "rt": rt,
                   "quantize_us": round(tq * 1e6, 2), "quantize_gbps": gbps(q_bytes, tq),
                   "quantize_frac": round(q_bytes / tq / 1e9 / PEAK_HBM_GBPS, 4),
                   "quant_down_us": round((tf - tg) * 1e6, 2), "quant_down_gbps": gbps(qd_bytes, tf - tg),
                   "quant_down_frac": round(qd_bytes / (tf - tg) / 1e9 / PEAK_HBM_GBPS, 4)}
            if is_mlp:
                f = ls.f
                tm = time_graph_stats(torch, lambda i: abi.fourtune_mlp_fwd(S(i)["L"], S(i)["fc2"], S(i)["x"], S(i)["out"],
                                                                            S(i)["xl"], S(i)["y"], S(i)["hl2"],
                                                                            S(i)["ws"]))[0]
                tg2 = time_graph_stats(torch, lambda i: abi.fourtune_gemm_fwd(S(i)["fc2"], S(i)["hq"], S(i)["hl2"],
                                                                              S(i)["out"]))[0]
                tp = tm - tf - tg2
                p_bytes = m * f * 2.5 + ((m + 31) // 32) * (f // 32) + m * rt * 2
                row.update({"gelu_pass_us": round(tp * 1e6, 2), "gelu_pass_gbps": gbps(p_bytes, tp),
                            "gelu_pass_frac": round(p_bytes / tp / 1e9 / PEAK_HBM_GBPS, 4)})
            res[name] = row
            log(f"[hbm-sweep] {name}: " + ", ".join(f"{k_}={v}" for k_, v in row.items()))
            del sets
            torch.cuda.empty_cache()
    print(json.dumps({"metric": "HBM-bound kernels: algorithmic bytes / time, fraction of 8 TB/s",
                      "unit": "GB/s", "peak": PEAK_HBM_GBPS, "n_gpus": 1, "data": "synthetic", **res}), flush=True)
    return 0


# --------------------------------------------------------------------------- precision configurations
def precision(args):
    """The c2 linear's fwd+bwd in the four precision configurations of the pages'
    ablation (FourTune §4 "Impact of Precision Configurations"; the pages measure
    training quality there and note that only W4A4G4 uses 4-bit arithmetic throughout):
    forward and backward times from graph replays, and the backbone product's rate."""
    import torch
    from bit_quantized_lora_fp4_amd import abi
    from synth import workloads as wl

    abi.lib()
    case = wl.linear_case("c2")
    m, k = case["X"].shape
    n = case["R"].shape[0]
    sets = build_sets(case, args.sets, torch, abi)
    it = max(args.steps, 10)

    def S(i):
        return sets[i % len(sets)]

    res = {}
    for prec in ("W4A4G4", "W4A16G4", "W4A4G16", "W4A16G16"):
        fwd = lambda i, p=prec: abi.fourtune_linear_fwd_prec(S(i)["L"], p, S(i)["x"], S(i)["y"], S(i)["xl"], S(i)["ws"])
        bwd = lambda i, p=prec: abi.fourtune_linear_bwd_prec(S(i)["L"], p, S(i)["dy"], S(i)["x"], S(i)["xl"], S(i)["dx"],
                                                             S(i)["da"], S(i)["db"], S(i)["ws"])
        for i in range(args.warmup):
            fwd(i)
            bwd(i)
        torch.cuda.synchronize()
        tf, tb = time_graph(torch, fwd, it), time_graph(torch, bwd, it)
        res[prec] = {"fwd_us": round(tf * 1e6, 2), "bwd_us": round(tb * 1e6, 2),
                     "fwd_bwd_us": round((tf + tb) * 1e6, 2),
                     "backbone_tflops": round(4.0 * m * n * k / (tf + tb) / 1e12, 1)}
        log(f"[precision] {prec}: fwd {tf*1e6:.1f} us, bwd {tb*1e6:.1f} us")
    base = res["W4A4G4"]["fwd_bwd_us"]
    for p in res:
        res[p]["slowdown_vs_w4a4g4"] = round(res[p]["fwd_bwd_us"] / base, 3)
    print(json.dumps({"metric": "c2 linear fwd+bwd per precision configuration", "unit": "us",
                      "higher_is_better": False, "n_gpus": 1, "data": "synthetic",
                      "config": {"workload": "c2", "m": m, "n": n, "k": k}, **res}), flush=True)
    return 0


# --------------------------------------------------------------------------- whole DiT
HIDDEN, MLP_DIM, QKV_DIM = 3072, 12288, 9216
DIT_RANK, DIT_STAB = 64, 32
IMG_TOKENS, TXT_TOKENS = 4096, 512


def dit_linears(n_double, n_single):
    """The token-wise linears of a FLUX.1-dev-shaped DiT at batch 1, as (tokens, kind):
    a double-stream block holds an image stream (4096 tokens) and a text stream (512
    tokens) with weights of their own, a single-stream block one stream of 4608 tokens.
    Each stream has QKV [9216 x 3072], the attention output projection [3072 x 3072]
    and the MLP 3072 -> 12288 -> 3072 (the single-stream block's fused linears hold
    the same products: its first linear is QKV and FC1 side by side, its second the
    output projection and FC2 summed)."""
    streams = []
    for _ in range(n_double):
        streams += [IMG_TOKENS, TXT_TOKENS]
    streams += [IMG_TOKENS + TXT_TOKENS] * n_single
    return streams


def dit_weight_bytes(n_double, n_single, r=DIT_RANK, s=DIT_STAB):
    """Weight bytes of the blocks' linears, token-wise and modulation (adaLN: 6 x hidden
    outputs per stream of a double block, 3 x hidden for a single block), for W4A4G4
    (MXFP4 codes + one scale byte per 32x32 block, bf16 LoRA and stabilizer factors)
    and for bf16 LoRA (bf16 weight + bf16 LoRA factors). Embedders, norms and the final
    layer (under 1% of the parameters) are left out of both."""
    per_stream = [(QKV_DIM, HIDDEN), (HIDDEN, HIDDEN), (MLP_DIM, HIDDEN), (HIDDEN, MLP_DIM)]
    lins = []
    for _ in range(n_double):
        lins += per_stream * 2 + [(6 * HIDDEN, HIDDEN)] * 2
    for _ in range(n_single):
        lins += per_stream + [(3 * HIDDEN, HIDDEN)]
    w4 = sum(n * k // 2 + (n // 32) * (k // 32) + 2 * (r + s) * (n + k) for n, k in lins)
    bf = sum(2 * n * k + 2 * r * (n + k) for n, k in lins)
    params = sum(n * k for n, k in lins)
    return dict(params=params, w4a4g4_bytes=w4, bf16_lora_bytes=bf, ratio=round(bf / w4, 3),
                bits_per_weight_w4=round(8 * sum(n * k // 2 + (n // 32) * (k // 32) for n, k in lins) / params, 4))


def dit(args):
    """One training step's linears over a whole FLUX-shaped DiT (FourTune §4 reports a
    DiT step and its weight memory against bf16 LoRA): every token-wise linear of every
    block, forward then backward in reverse block order, with weights of its own
    (synthetic, drawn on the device) and LoRA gradients; attention, norms and
    modulation are not run. Inputs are synthetic tensors of each stream's shape."""
    import torch
    import torch.nn.functional as F
    from bit_quantized_lora_fp4_amd import abi

    abi.lib()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    streams = dit_linears(args.double_blocks, args.single_blocks)
    bf = dict(dtype=torch.bfloat16, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    r, s = DIT_RANK, DIT_STAB
    rt = r + s

    def randn(shape, std, dtype=torch.bfloat16):
        return (torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32) * std).to(dtype)

    def w4_linear(n, k):
        R = randn((n, k), 0.02, torch.float32)
        L = abi.make_linear(R, randn((r, k), 0.01), randn((n, r), 0.01), randn((s, k), 0.01), randn((n, s), 0.01))
        del R
        return L

    log(f"[dit] {len(streams)} streams ({args.double_blocks} double, {args.single_blocks} single blocks): "
        "drawing W4A4G4 weights")
    # inputs per token count (synthetic; Student-t activations as in the DiT block workload)
    torch.manual_seed(1234)
    t3 = torch.distributions.StudentT(torch.tensor(3.0, device="cuda"))
    xin = {m: (t3.sample((m, HIDDEN)) * 0.5).to(torch.bfloat16) for m in sorted(set(streams))}
    dyin = {m: randn((m, HIDDEN), 1e-3) for m in xin}
    dqkv = {m: randn((m, QKV_DIM), 1e-3) for m in xin}
    big_ws = 0
    w4 = []
    for m in streams:
        blk = dict(m=m, qkv=w4_linear(QKV_DIM, HIDDEN), o=w4_linear(HIDDEN, HIDDEN),
                   fc1=w4_linear(MLP_DIM, HIDDEN), fc2=w4_linear(HIDDEN, MLP_DIM))
        blk["xl_qkv"] = torch.empty((m, rt), **bf)
        blk["xl_o"] = torch.empty((m, rt), **bf)
        blk["xl1"], blk["hl2"] = torch.empty((m, rt), **bf), torch.empty((m, rt), **bf)
        blk["pre"] = torch.empty((m, MLP_DIM), **bf)
        big_ws = max(big_ws, abi.fourtune_linear_workspace_bytes(m, blk["qkv"]),
                     abi.fourtune_mlp_workspace_bytes(m, blk["fc1"], blk["fc2"]))
        w4.append(blk)
    ws = abi.workspace(big_ws)
    out = {m: dict(qkv=torch.empty((m, QKV_DIM), **bf), o=torch.empty((m, HIDDEN), **bf),
                   y=torch.empty((m, HIDDEN), **bf), dx=torch.empty((m, HIDDEN), **bf))
           for m in xin}
    grads = dict(a_h=torch.empty((r, HIDDEN), **f32), b_qkv=torch.empty((QKV_DIM, r), **f32),
                 b_h=torch.empty((HIDDEN, r), **f32), b_f=torch.empty((MLP_DIM, r), **f32),
                 a_f=torch.empty((r, MLP_DIM), **f32))
    torch.cuda.synchronize()

    def w4_step():
        for b in w4:
            m, o = b["m"], out[b["m"]]
            abi.fourtune_linear_fwd(b["qkv"], xin[m], o["qkv"], b["xl_qkv"], ws)
            abi.fourtune_linear_fwd(b["o"], xin[m], o["o"], b["xl_o"], ws)
            abi.fourtune_mlp_fwd(b["fc1"], b["fc2"], xin[m], o["y"], b["xl1"], b["pre"], b["hl2"], ws)
        g = grads
        for b in reversed(w4):
            m, o = b["m"], out[b["m"]]
            abi.fourtune_mlp_bwd(b["fc1"], b["fc2"], dyin[m], xin[m], b["xl1"], b["pre"], b["hl2"], o["dx"],
                                 g["a_h"], g["b_f"], g["a_f"], g["b_h"], ws)
            abi.fourtune_linear_bwd(b["o"], dyin[m], xin[m], b["xl_o"], o["dx"], g["a_h"], g["b_h"], ws)
            abi.fourtune_linear_bwd(b["qkv"], dqkv[m], xin[m], b["xl_qkv"], o["dx"], g["a_h"], g["b_qkv"], ws)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        return 1e3 * time_region(torch, lambda i: fn(), args.steps) / args.steps

    log("[dit] timing W4A4G4")
    t_w4 = timed(w4_step)
    mem_w4 = torch.cuda.memory_allocated()
    del w4, ws
    torch.cuda.empty_cache()

    log("[dit] drawing bf16 LoRA weights")

    def bf_linear(n, k):
        W = randn((n, k), 0.02)
        A, B = randn((r, k), 0.01), randn((n, r), 0.01)
        return dict(W=W, Wt=W.t().contiguous(), A=A, At=A.t().contiguous(), B=B, Bt=B.t().contiguous())

    bl = [dict(m=m, qkv=bf_linear(QKV_DIM, HIDDEN), o=bf_linear(HIDDEN, HIDDEN), fc1=bf_linear(MLP_DIM, HIDDEN),
               fc2=bf_linear(HIDDEN, MLP_DIM)) for m in streams]
    torch.cuda.synchronize()

    def bf_step():
        saved = []
        for b in bl:
            x = xin[b["m"]]
            _, xa_q = _lora_fwd(torch, b["qkv"], x)
            _, xa_o = _lora_fwd(torch, b["o"], x)
            p, xa1 = _lora_fwd(torch, b["fc1"], x)
            h = F.gelu(p, approximate="tanh")
            _, xa2 = _lora_fwd(torch, b["fc2"], h)
            saved.append((xa_q, xa_o, p, xa1, h, xa2))
        for b, (xa_q, xa_o, p, xa1, h, xa2) in zip(reversed(bl), reversed(saved)):
            m = b["m"]
            x = xin[m]
            dh, _, _ = _lora_bwd(torch, b["fc2"], dyin[m], h, xa2)
            dp = torch.ops.aten.gelu_backward(dh, p, approximate="tanh")
            _lora_bwd(torch, b["fc1"], dp, x, xa1)
            _lora_bwd(torch, b["o"], dyin[m], x, xa_o)
            _lora_bwd(torch, b["qkv"], dqkv[m], x, xa_q)

    log("[dit] timing bf16 LoRA")
    t_bf = timed(bf_step)
    flops_w4 = sum(4.0 * m * HIDDEN * (QKV_DIM + HIDDEN + 2 * MLP_DIM) for m in streams)
    res = {"metric": "DiT linears fwd+bwd step time, W4A4G4 vs bf16 LoRA (FourTune §4 DiT step)",
           "unit": "ms", "higher_is_better": False, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "data": "synthetic weights and inputs",
           "config": {"model": "FLUX.1-dev-shaped DiT linears", "double_blocks": args.double_blocks,
                      "single_blocks": args.single_blocks, "hidden": HIDDEN, "mlp": MLP_DIM,
                      "image_tokens": IMG_TOKENS, "text_tokens": TXT_TOKENS, "lora_rank": r, "stab_rank": s,
                      "excluded": "attention, norms, modulation (M = 1), embedders"},
           "w4a4g4_ms": round(t_w4, 3), "bf16_lora_ms": round(t_bf, 3), "speedup": round(t_bf / t_w4, 3),
           "w4a4g4_tflops_4bit": round(flops_w4 / (t_w4 * 1e-3) / 1e12, 1),
           "weights": dit_weight_bytes(args.double_blocks, args.single_blocks),
           "device_bytes_allocated_w4_run": mem_w4,
           "pages_for_context": {"dit_step_ms": {"fourtune": 612.4, "bf16_lora": 1541.0},
                                 "weight_gb": {"fourtune": 7.71, "bf16_lora": 22.59}}}
    print(json.dumps(res), flush=True)
    return 0


# --------------------------------------------------------------------------- CPU side
def cpu_baseline(case, seconds):
    """The oracle as it stands, fwd+bwd on a row sample of the same layer."""
    from oracle import layer, mx4

    lin = layer.Linear(R=case["R"].astype(np.float64), A=case["A"].astype(np.float64),
                       B=case["B"].astype(np.float64), L1=case["L1"].astype(np.float64),
                       L2=case["L2"].astype(np.float64))
    Rq = mx4.fake_quant(lin.R)  # frozen weight: quantized once, outside the timing
    rows = 512
    X = case["X"][:rows].astype(np.float64)
    G = case["dY"][:rows].astype(np.float64)
    n, k = lin.R.shape
    reps, t0 = 0, time.perf_counter()
    while True:
        Y, XL = layer.linear_forward(X, lin, Rq=Rq)
        layer.linear_backward(G, X, XL, lin, Rq=Rq)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    threads = None
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or None
    except Exception:  # noqa: BLE001 - report what is known
        pass
    flops = 4.0 * rows * n * k * reps
    blas = None
    try:
        cfg = np.show_config(mode="dicts")
        blas = cfg.get("Build Dependencies", {}).get("blas", {}).get("name")
    except Exception:  # noqa: BLE001 - report what is known
        pass
    return dict(value=round(flops / el / 1e12, 5), unit="TFLOP/s", blas=blas,
                cores=threads or len(os.sched_getaffinity(0)), kind="oracle",
                sample=f"fwd+bwd of the same linear on the first {rows} of {case['X'].shape[0]} "
                       f"token rows, {reps} repetitions in {el:.1f} s (numpy fp64)")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the hot path runs on a single MI355X; how it would shard is a design note).",
              file=sys.stderr)
        return 2
    if args.calibrate_copy:
        return calibrate_copy()
    if args.ablation:
        return ablation(args)
    if args.dit:
        return dit(args)
    if args.granularity:
        return granularity(args)
    if args.precision:
        return precision(args)
    if args.gemm_sweep:
        return gemm_sweep(args)
    if args.hbm_sweep:
        return hbm_sweep(args)
    import torch
    from bit_quantized_lora_fp4_amd import abi
    from synth import workloads as wl

    abi.lib()  # fails loudly when the library is not built
    spec = wl.WORKLOADS[args.workload]
    lin_spec = spec.layers[0]
    if not isinstance(lin_spec, wl.LinearSpec):
        raise SystemExit(f"workload {args.workload} has no single linear; use c1 or c2")
    log(f"[bench] generating {args.workload} inputs")
    case = wl.linear_case(args.workload)
    m, k = case["X"].shape
    n = case["R"].shape[0]
    r, s = lin_spec.r, lin_spec.s
    sets = build_sets(case, args.sets, torch, abi)
    torch.cuda.synchronize()
    log(f"[bench] {args.sets} sets resident; warmup {args.warmup}")

    for st in sets:  # fill each set's Q(X) and Q(dY) for the GEMM-only timings
        abi.fourtune_linear_fwd(st["L"], st["x"], st["y"], st["xl"], st["ws"], xq_out=st["xq"])
        abi.fourtune_linear_bwd(st["L"], st["dy"], st["x"], st["xl"], st["dx"], st["da"], st["db"],
                                st["ws"], gq_out=st["gq"])
    for i in range(args.warmup):
        step(abi, sets[i % len(sets)])
    torch.cuda.synchronize()

    # ---- timed region: K whole steps
    t = time_region(torch, lambda i: step(abi, sets[i % len(sets)]), args.steps)
    ms_per_step = 1000.0 * t / args.steps
    value = 4.0 * m * n * k / (t / args.steps) / 1e12
    log(f"[bench] step {ms_per_step:.4f} ms -> {value:.1f} TFLOP/s")

    # ---- per-kernel: the two 4-bit GEMMs alone, the layer halves, the quantizer
    def S(i):
        return sets[i % len(sets)]

    it = max(args.steps, 10)
    t_gf = time_graph(torch, lambda i: abi.fourtune_gemm_fwd(S(i)["L"], S(i)["xq"], S(i)["xl"], S(i)["y"]), it)
    t_gb = time_graph(torch, lambda i: abi.fourtune_gemm_bwd(S(i)["L"], S(i)["gq"], S(i)["gb"], S(i)["dx"]), it)
    t_fwd = time_graph(torch, lambda i: abi.fourtune_linear_fwd(S(i)["L"], S(i)["x"], S(i)["y"], S(i)["xl"],
                                                               S(i)["ws"]), it)
    t_bwd = time_graph(torch, lambda i: abi.fourtune_linear_bwd(S(i)["L"], S(i)["dy"], S(i)["x"], S(i)["xl"],
                                                               S(i)["dx"], S(i)["da"], S(i)["db"], S(i)["ws"]), it)
    t_q = time_graph(torch, lambda i: abi.fourtune_quantize(S(i)["x"], S(i)["xq"]), it)
    # the forward's fused quantize + down-projection (and its partial sum) is the rest
    # of the forward: Q(X) codes and scales, XL, one read of X
    t_qd = max(t_fwd - t_gf, 1e-9)
    qd_bytes = m * k * (4 if case["x_dtype"] == "fp32" else 2) + m * k / 2 + ((m + 31) // 32) * (k // 32) \
        + m * (r + s) * 2
    qd_gbps = qd_bytes / t_qd / 1e9
    gemm_flops = 2.0 * m * n * k
    tf_gf, tf_gb = gemm_flops / t_gf / 1e12, gemm_flops / t_gb / 1e12
    xbytes = 4 if case["x_dtype"] == "fp32" else 2
    q_bytes = m * k * xbytes + m * k / 2 + ((m + 31) // 32) * (k // 32)
    q_gbps = q_bytes / t_q / 1e9
    log(f"[bench] gemm_fwd {t_gf*1e6:.1f} us ({tf_gf:.0f} TF/s), gemm_bwd {t_gb*1e6:.1f} us "
        f"({tf_gb:.0f} TF/s), linear_fwd {t_fwd*1e6:.1f} us, linear_bwd {t_bwd*1e6:.1f} us, "
        f"quantize X {t_q*1e6:.1f} us ({q_gbps:.0f} GB/s)")

    out = {
        "metric": "W4A4G4 linear fwd+bwd TFLOPS (4-bit backbone flops / whole step time)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {spec.title}, W4A4G4 linear fwd+bwd",
                   "m": m, "k": k, "n": n, "lora_rank": r, "stab_rank": s,
                   "x_dtype": case["x_dtype"], "out_dtype": "bf16", "input_sets": args.sets},
        "roofline": {"kernel": "k_gemm_mx4 forward (4-bit GEMM + up-projection)", "bound": "mfma",
                     "achieved": round(tf_gf, 1), "peak": PEAK_MXFP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf_gf / PEAK_MXFP4_TFLOPS, 4),
                     "traffic": traffic_for(m, n, k)},
        "kernels_us": {"gemm_fwd": round(t_gf * 1e6, 2), "gemm_bwd": round(t_gb * 1e6, 2),
                       "linear_fwd": round(t_fwd * 1e6, 2), "linear_bwd": round(t_bwd * 1e6, 2),
                       "quantize_x": round(t_q * 1e6, 2), "fused_quant_down_fwd": round(t_qd * 1e6, 2)},
        "gemm_tflops": {"fwd": round(tf_gf, 1), "bwd": round(tf_gb, 1),
                        "fwd_bwd": round(2 * gemm_flops / (t_gf + t_gb) / 1e12, 1),
                        "frac_of_mxfp4_peak": round(2 * gemm_flops / (t_gf + t_gb) / 1e12 / PEAK_MXFP4_TFLOPS, 4)},
        "quantize_gbps": round(q_gbps, 1),
        "quantize_frac_of_hbm": round(q_gbps / PEAK_HBM_GBPS, 4),
        "fused_quant_down_gbps": round(qd_gbps, 1),
        "fused_quant_down_frac_of_hbm": round(qd_gbps / PEAK_HBM_GBPS, 4),
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
