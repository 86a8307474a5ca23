#!/usr/bin/env python3
"""Benchmark of single-token GQA decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one call of the library (split-KV kernel + merge kernel) over one
batch of seeded synthetic inputs already resident in HBM. The timed region
replays a HIP graph that holds exactly K calls, cycling over R distinct copies
of the inputs (R * KV bytes >= 1 GiB, so the 256 MB last-level cache and the
L2s cannot serve the KV cache from one call to the next). Prints ONE JSON line.

Metric: effective KV GB/s = K and V bytes the call attends (each read once)
divided by the time per call, and its fraction of the 8 TB/s HBM peak.
`roofline.achieved` uses the split kernel's own duration: HIP events recorded
on the launch stream around a replay of a graph of K split-only launches
(gqa_decode_partial), divided by K.
`cpu_baseline` times the fp64 oracle on the host's cores in a subprocess
(and on one thread, as an extra key). `extra_workloads` holds the same
measurement on the other Llama-70B workloads (the ragged batch of 8, one
sequence of 32k and of 1M tokens) and on the plan made without a length
hint (8k, 1M), with inputs drawn on the GPU from a seeded generator.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import re
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E datasheet peak
DEFAULT_WORKLOAD = "llama70b_gqa_b1_s8192"
ROTATE_BYTES = 1 << 30
KERNEL_SOURCES = ["gqa_common.h", "split_kv_mfma.h", "split_kv_valu.h", "merge.h", "fused_tail.h",
                  "kv_append.h", "packed_offsets.h", "split_kv_tiles.h", "gqa_decode.hip"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_only(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed: what the
    compiler sees, so an edit of a comment keeps recorded counters valid."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "decode_attention_gqa_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_only(fh.read()).encode())
    return h.hexdigest()[:16]


class Hip:
    """The few HIP runtime calls bench.py needs for events, via ctypes."""

    def __init__(self):
        path = None
        for cand in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
            try:
                self.lib = ctypes.CDLL(cand)
                path = cand
                break
            except OSError:
                continue
        if path is None:
            raise RuntimeError("libamdhip64.so not found")
        L = self.lib
        L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def elapsed_ms(self, a, b) -> float:
        assert self.lib.hipEventSynchronize(b) == 0
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value


def host_cores() -> int:
    """Host cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _time_oracle(name: str, budget_s: float, threads: int) -> dict:
    """Time oracle.attend on the host in a child process with `threads` BLAS
    and OpenMP threads."""
    code = f"""
import json, os, sys, time
sys.path.insert(0, {ROOT!r})
import numpy as np
import oracle, workloads
w = workloads.WORKLOADS[{name!r}]
inp = workloads.make_inputs(w)
heads = None
groups = w.h_kv
if inp.kv_bytes() > (1 << 30):          # very long context: time one kv group of sequence 0
    heads = [(0, h) for h in range(w.n_rep)]
    groups = 1
t0 = time.perf_counter(); n = 0
while True:
    oracle.attend(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, w.h_kv, dtype=w.dtype, heads=heads)
    n += 1
    if time.perf_counter() - t0 >= {budget_s}:
        break
dt = (time.perf_counter() - t0) / n
if heads is None:
    sample_bytes = inp.kv_bytes()
    sample = f"whole workload per call, {{n}} call(s)"
else:
    sample_bytes = 2 * int(inp.seq_lens[0]) * w.d * 2
    sample = f"kv group 0 of sequence 0 ({{w.n_rep}} query heads, {{int(inp.seq_lens[0])}} tokens) per call, {{n}} call(s)"
print(json.dumps(dict(seconds_per_call=dt, sample_bytes=sample_bytes, calls=n, sample=sample)))
"""
    t = str(threads)
    env = dict(os.environ, OMP_NUM_THREADS=t, OPENBLAS_NUM_THREADS=t, MKL_NUM_THREADS=t,
               HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=600)
    if r.returncode != 0:
        raise RuntimeError("cpu baseline failed: " + r.stderr[-2000:])
    return json.loads(r.stdout.strip().splitlines()[-1])


def cpu_baseline(name: str, budget_s: float) -> dict:
    """The fp64 oracle on the host's cores (BLAS and OpenMP threads = the
    cores this process may use), and on one thread for comparison."""
    cores = host_cores()
    d = _time_oracle(name, budget_s, cores)
    d1 = _time_oracle(name, budget_s / 2, 1)
    gbs = d["sample_bytes"] / d["seconds_per_call"] / 1e9
    return {"value": gbs, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 numpy oracle on {name}: {d['sample']}; "
                      f"{d['seconds_per_call'] * 1e3:.1f} ms per sample (BLAS and OpenMP threads = {cores})",
            "value_one_thread": d1["sample_bytes"] / d1["seconds_per_call"] / 1e9,
            "ms_per_sample_one_thread": d1["seconds_per_call"] * 1e3}


def traffic_from_profile(name: str, src_hash: str):
    """HBM bytes per split-kernel launch from committed rocprofv3 counters,
    or None when absent or taken on different kernel sources."""
    p = os.path.join(ROOT, "profiles", f"counters_split_kv_{name}.json")
    if not os.path.exists(p):
        return None, None
    d = json.load(open(p))
    if d.get("kernel_source_hash") != src_hash:
        return None, d
    return d.get("hbm_bytes_per_launch"), d


EXTRA_WORKLOADS = [
    # (key, workload whose shapes and lengths are used, hint given to the library, steps)
    ("llama70b_gqa_b8_ragged", "llama70b_gqa_b8_ragged", True, 60),
    ("llama70b_gqa_b1_s32768", None, True, 100),
    ("llama70b_gqa_b1_s1m", "llama70b_gqa_b1_s1m", True, 12),
    ("llama70b_gqa_b1_s8192_no_hint", "llama70b_gqa_b1_s8192", False, 100),
    ("llama70b_gqa_b1_s1m_no_hint", "llama70b_gqa_b1_s1m", False, 12),
]


def measure_extra(gqa, hip, key: str, base: str | None, with_hint: bool, steps: int) -> dict:
    """One call (split + merge) of another Llama-70B workload, timed like the
    headline (a HIP graph of `steps` calls over rotating inputs, split-only
    graph for the split kernel), with inputs drawn on the GPU from a seeded
    generator (same shapes, lengths and distributions as the named workload;
    not the oracle's bits: these are timing runs). Without a hint the call
    plans as the base entry point does (gqa_decode_attn: no length known)."""
    import numpy as np
    import torch

    import workloads
    if base is None:
        w = workloads.WORKLOADS["llama70b_gqa_b1_s8192"]
        lens_np = np.array([32768], dtype=np.int32)
    else:
        w = workloads.WORKLOADS[base]
        lens_np = workloads.seq_lens_for(w)
    dev = torch.device("cuda:0")
    B, T = len(lens_np), int(lens_np.sum())
    kv_bytes = 2 * T * w.h_kv * w.d * 2
    free, _ = torch.cuda.mem_get_info()
    R = max(1, min(math.ceil(ROTATE_BYTES / kv_bytes), int(0.4 * free // kv_bytes)))
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 + w.seed)
    sets = []
    for _ in range(R):
        q = torch.randn((B, w.h_q, w.d), generator=gen, device=dev).to(torch.bfloat16)
        k = torch.empty((T, w.h_kv, w.d), dtype=torch.bfloat16, device=dev)
        v = torch.empty_like(k)
        for t0 in range(0, T, 1 << 18):             # in slices: bounded fp32 temporaries
            t1 = min(T, t0 + (1 << 18))
            k[t0:t1] = (w.k_sigma * torch.randn((t1 - t0, w.h_kv, w.d), generator=gen, device=dev)).to(torch.bfloat16)
            v[t0:t1] = torch.randn((t1 - t0, w.h_kv, w.d), generator=gen, device=dev).to(torch.bfloat16)
        sets.append((q, k, v))
    lens = torch.from_numpy(lens_np).to(dev)
    hint = int(lens_np.max()) if with_hint else 0
    ns = gqa.gqa_decode_pick_splits_d(B, w.h_kv, w.d, hint)
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(B, w.h_q, w.d, ns), dtype=torch.uint8, device=dev)
    out = torch.empty((B, w.h_q, w.d), dtype=torch.float32, device=dev)
    scale = float(np.float32(1.0 / math.sqrt(w.d)))
    stream = torch.cuda.Stream()

    def call(i):
        q, k, v = sets[i % R]
        gqa.gqa_decode_attn_ex(q, k, v, lens, out, scale=scale, s_kv_hint=hint, workspace=ws)

    def partial(i):
        q, k, v = sets[i % R]
        gqa.gqa_decode_partial(q, k, v, lens, ws, scale=scale, s_kv_hint=hint)

    def graph_us(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(steps):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = hip.event(), hip.event()
        hip.lib.hipEventRecord(e0, ctypes.c_void_p(stream.cuda_stream))
        g.replay()
        hip.lib.hipEventRecord(e1, ctypes.c_void_p(stream.cuda_stream))
        us = hip.elapsed_ms(e0, e1) * 1e3 / steps
        hip.lib.hipEventDestroy(e0)
        hip.lib.hipEventDestroy(e1)
        return us

    with torch.cuda.stream(stream):
        for i in range(3):
            call(i)
        torch.cuda.synchronize()
        us = graph_us(call)
        split_us = graph_us(partial)
    if not torch.isfinite(out).all():
        raise RuntimeError(f"{key}: non-finite output")
    res = {"us_per_call": round(us, 3), "effective_gbs": round(kv_bytes / us / 1e3, 1),
           "pct_hbm_peak": round(100.0 * kv_bytes / us / 1e3 / HBM_PEAK_GBS, 2),
           "split_kernel_us": round(split_us, 3), "kv_bytes_per_call": kv_bytes,
           "frac": round(kv_bytes / split_us / 1e3 / HBM_PEAK_GBS, 4),
           "n_splits": ns, "s_kv_hint": hint, "B": B, "rotating_input_sets": R, "steps": steps,
           "seq_lens": lens_np.tolist() if B <= 16 else f"{B} sequences"}
    del sets, ws
    torch.cuda.empty_cache()
    log(f"[bench] {key}: {us:.2f} us per call, split kernel {split_us:.2f} us (frac {res['frac']:.3f})")
    return res


def bench_append_or_step(args) -> int:
    """KV-cache append (gqa_kv_append) alone, or a decode step: append one
    token per sequence, then attend with the new lengths - as two calls
    (`step`) or as one gqa_decode_step with the append folded into the split
    kernel (`step1`). Padded caches with capacity S_max + n_new rows per
    sequence, R copies rotated as above."""
    import numpy as np
    import torch

    import decode_attention_gqa_amd as gqa
    import workloads

    w = workloads.WORKLOADS[args.workload]
    if w.dtype != "bf16":
        raise SystemExit("--op append/step use the bf16 workloads")
    lens0 = workloads.seq_lens_for(w)
    n_new = args.n_new if args.op == "append" else 1
    is_step = args.op in ("step", "step1")
    cap = int(lens0.max()) + n_new
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] {args.op}: {w.name}, capacity {cap} rows per sequence")
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    cache_bytes = 2 * w.B * cap * w.h_kv * w.d * 2
    free, _ = torch.cuda.mem_get_info()
    R = max(1, min(math.ceil(ROTATE_BYTES / cache_bytes), int(0.4 * free // cache_bytes)))
    caches = [(torch.randn((w.B * cap, w.h_kv, w.d), generator=gen, device=dev, dtype=torch.bfloat16),
               torch.randn((w.B * cap, w.h_kv, w.d), generator=gen, device=dev, dtype=torch.bfloat16))
              for _ in range(R)]
    kn = torch.randn((w.B, n_new, w.h_kv, w.d), generator=gen, device=dev, dtype=torch.bfloat16)
    vn = torch.randn_like(kn)
    q = torch.randn((w.B, w.h_q, w.d), generator=gen, device=dev, dtype=torch.bfloat16)
    lens_in = torch.from_numpy(lens0).to(dev)
    lens_out = torch.empty_like(lens_in)
    offs = torch.arange(w.B, dtype=torch.int64, device=dev) * cap
    ns = gqa.gqa_decode_pick_splits_d(w.B, w.h_kv, w.d, cap)
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(w.B, w.h_q, w.d, ns), dtype=torch.uint8, device=dev)
    out = torch.empty((w.B, w.h_q, w.d), dtype=torch.float32, device=dev)

    def step(i):
        k, v = caches[i % R]
        # every step appends at the same positions (lens_in is not advanced), so
        # the timed work is the same in every step
        if args.op == "step1":
            gqa.gqa_decode_step(q, kn, vn, k, v, lens_in, lens_out, out, capacity=cap, kv_token_offsets=offs,
                                workspace=ws)
            return
        gqa.gqa_kv_append(kn, vn, k, v, lens_in, capacity=cap, seq_lens_out=lens_out, kv_token_offsets=offs)
        if args.op == "step":
            gqa.gqa_decode_attn_ex(q, k, v, lens_out, out, kv_token_offsets=offs, s_kv_hint=cap, workspace=ws)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(args.steps):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    sec = (t1 - t0) / args.steps
    appended = 2 * w.B * n_new * w.h_kv * w.d * 2          # bytes written (and read from k_new/v_new)
    attended = 2 * int((lens0.astype(np.int64) + 1).sum()) * w.h_kv * w.d * 2
    res = {
        "metric": "decode step (KV append + attention) us" if is_step else "KV-cache append bytes/s",
        "value": round(sec * 1e6, 3) if is_step else round(2 * appended / sec / 1e9, 3),
        "unit": "us" if is_step else "GB/s (read + write)",
        "higher_is_better": not is_step,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": sec * 1e3,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "op": args.op, "B": w.B, "h_kv": w.h_kv, "d_head": w.d,
                   "new_tokens_per_sequence": n_new, "capacity": cap, "rotating_caches": R,
                   "timing": "one HIP graph holding the K steps"},
        "us_per_call": sec * 1e6,
        "append_bytes_written": appended,
    }
    if is_step:
        res["launches_per_step"] = 2 if args.op == "step1" else 3
        res["attended_kv_bytes"] = attended
        res["effective_kv_gbs"] = attended / sec / 1e9
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seq-lens", default="",
                    help="comma-separated lengths overriding the workload's (B = their count)")
    ap.add_argument("--n-splits", type=int, default=0)
    ap.add_argument("--valu", action="store_true", help="vector-ALU split kernel (comparison)")
    ap.add_argument("--eager", action="store_true", help="time eager calls instead of a HIP graph")
    ap.add_argument("--s-q", type=int, default=1,
                    help="query tokens per sequence (> 1: multi-token decode, causal among them)")
    ap.add_argument("--op", choices=["attend", "append", "step", "step1"], default="attend",
                    help="attend (default): the attention call; append: KV-cache append of "
                         "--n-new tokens per sequence; step: append one token, then attend (two "
                         "calls); step1: the same as one gqa_decode_step")
    ap.add_argument("--n-new", type=int, default=1, help="tokens per sequence for --op append")
    ap.add_argument("--fused", action="store_true",
                    help="single-launch form (GQA_FLAG_FUSED) instead of split + merge kernels")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the extra workloads (ragged batch, 32k, 1M, no-hint plans)")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work on all cores (half as long on one thread)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one elementwise copy-like kernel over this many MiB first "
                         "(calibrates HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import decode_attention_gqa_amd as gqa
    import workloads

    if args.op != "attend":
        return bench_append_or_step(args)
    src_hash = kernel_source_hash()
    w = workloads.WORKLOADS[args.workload]
    if args.seq_lens:
        lens_o = [int(x) for x in args.seq_lens.split(",")]
        inp = workloads.custom(f"{w.name}_lens", B=len(lens_o), h_q=w.h_q, h_kv=w.h_kv, d=w.d,
                               seq_lens=lens_o, dtype=w.dtype, seed=w.seed, k_sigma=w.k_sigma)
        w = inp.w
        log(f"[bench] custom lengths {lens_o} with the shapes of {args.workload}")
    else:
        log(f"[bench] workload {w.name}: generating inputs")
        inp = workloads.make_inputs(w)
    kv_bytes = inp.kv_bytes()
    s_max = int(inp.seq_lens.max())
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(a):
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    q0, k0, v0 = up(inp.q), up(inp.k), up(inp.v)
    lens = torch.from_numpy(inp.seq_lens).to(dev)
    free, _ = torch.cuda.mem_get_info()
    R = max(1, min(math.ceil(ROTATE_BYTES / kv_bytes), int(0.5 * free // max(1, kv_bytes))))
    sets = [(q0, k0, v0)] + [(q0.clone(), k0.clone(), v0.clone()) for _ in range(R - 1)]
    log(f"[bench] {R} rotating input set(s) of {kv_bytes / 2**20:.1f} MiB KV")

    if args.copy_calibration_mib:
        # A plain elementwise kernel of known traffic (reads n bytes, writes n
        # bytes; its name in a trace contains "neg"), to scale HBM counters.
        n = args.copy_calibration_mib << 20
        a = torch.ones(n // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        log(f"[bench] counter calibration: neg over {n} bytes")

    ns = args.n_splits if args.n_splits > 0 else gqa.gqa_decode_pick_splits_d(w.B, w.h_kv, w.d, s_max)
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(w.B, w.h_q, w.d, ns), dtype=torch.uint8, device=dev)
    out = torch.empty((w.B, w.h_q, w.d), dtype=torch.float32, device=dev)
    scale = float(inp.scale)

    if args.s_q > 1:
        # several query tokens per sequence: q [B, S_q, h_q, d], seeded like the rest
        qm = workloads.normals(w.seed, 9, w.B * args.s_q * w.h_q * w.d, 1.0, w.dtype).reshape(
            w.B, args.s_q, w.h_q, w.d)
        qms = [up(qm)] + [up(qm) for _ in range(R - 1)]
        ns = gqa.multi_splits(w.B, args.s_q, w.h_q, w.h_kv, s_max, args.n_splits, w.d)
        ws = torch.empty(gqa.gqa_decode_workspace_bytes(w.B * args.s_q, w.h_q, w.d, ns),
                         dtype=torch.uint8, device=dev)
        out = torch.empty((w.B, args.s_q, w.h_q, w.d), dtype=torch.float32, device=dev)

    def call(i):
        q, k, v = sets[i % R]
        if args.s_q > 1:
            gqa.gqa_decode_attn_multi(qms[i % R], k, v, lens, out, scale=scale, n_splits=args.n_splits,
                                      s_kv_hint=s_max, workspace=ws)
            return
        gqa.gqa_decode_attn_ex(q, k, v, lens, out, scale=scale, n_splits=args.n_splits,
                               s_kv_hint=s_max, workspace=ws, valu=args.valu, fused=args.fused)

    stream = torch.cuda.Stream()
    hip = Hip()
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            call(i)
        torch.cuda.synchronize()
        log(f"[bench] {args.warmup} warmup calls done")

        # ---- the timed region: exactly K calls
        if args.eager:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(args.steps):
                call(i)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
        else:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(args.steps):
                    call(i)
            g.replay()                       # first replay uploads the graph (untimed)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            g.replay()
            torch.cuda.synchronize()
            t1 = time.perf_counter()
        log(f"[bench] timed {args.steps} calls")
        sec_per_call = (t1 - t0) / args.steps

        # ---- spread (outside the timed region): a graph of G calls replayed
        # N times, each replay between HIP events on the launch stream.
        spread = None
        if not args.eager:
            G, N = 20, 21
            gs = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gs, stream=stream):
                for i in range(G):
                    call(i)
            gs.replay()
            torch.cuda.synchronize()
            per = []
            for _ in range(N):
                a, b = hip.event(), hip.event()
                hip.lib.hipEventRecord(a, ctypes.c_void_p(stream.cuda_stream))
                gs.replay()
                hip.lib.hipEventRecord(b, ctypes.c_void_p(stream.cuda_stream))
                per.append(hip.elapsed_ms(a, b) * 1e3 / G)
                hip.lib.hipEventDestroy(a)
                hip.lib.hipEventDestroy(b)
            per.sort()
            spread = {"p10": per[N // 10], "p50": per[N // 2], "p90": per[(9 * N) // 10],
                      "what": f"us per call over {N} replays of a graph of {G} calls (HIP events)"}

        # ---- the split kernel alone: a HIP graph of K split-only launches
        # (gqa_decode_partial) over the same rotating inputs, with HIP events
        # recorded on the launch stream around one replay.
        def partial(i):
            q, k, v = sets[i % R]
            gqa.gqa_decode_partial(q, k, v, lens, ws, scale=scale, n_splits=args.n_splits,
                                   s_kv_hint=s_max, valu=args.valu)

        if args.s_q > 1:
            graph_p = None                           # no split-only entry point for S_q > 1
        elif args.eager:
            graph_p = None
        else:
            graph_p = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph_p, stream=stream):
                for i in range(args.steps):
                    partial(i)
            graph_p.replay()
        torch.cuda.synchronize()
        e0, e1 = hip.event(), hip.event()
        hip.lib.hipEventRecord(e0, ctypes.c_void_p(stream.cuda_stream))
        if graph_p is not None:
            graph_p.replay()
        elif args.s_q > 1:
            for i in range(args.steps):
                call(i)
        else:
            for i in range(args.steps):
                partial(i)
        hip.lib.hipEventRecord(e1, ctypes.c_void_p(stream.cuda_stream))
        split_us = hip.elapsed_ms(e0, e1) * 1e3 / args.steps
        hip.lib.hipEventDestroy(e0)
        hip.lib.hipEventDestroy(e1)
        call(0)
        torch.cuda.synchronize()
    log(f"[bench] split kernel alone: {split_us:.2f} us per launch")

    # sanity: finite output
    if not torch.isfinite(out).all():
        raise RuntimeError("non-finite output")

    gbs = kv_bytes / sec_per_call / 1e9
    achieved = kv_bytes / (split_us * 1e-6) / 1e9
    traffic, tinfo = traffic_from_profile(w.name, src_hash)
    res = {
        "metric": "decode attention effective KV GB/s (and % of HBM peak, us/call) at Llama-70B GQA shapes",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec_per_call * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normals; shapes of the Llama-2-70B decode workload)",
        "config": {
            "workload": w.name, "B": w.B, "h_q": w.h_q, "h_kv": w.h_kv, "d_head": w.d,
            "seq_lens": inp.seq_lens.tolist() if w.B <= 16 else f"{w.B} sequences",
            "kv_bytes_per_call": kv_bytes, "n_splits": ns,
            "split_kernel": "valu" if args.valu else ("mfma" if w.dtype == "bf16" else "valu"),
            "timing": "eager calls" if args.eager else "one HIP graph holding the K calls",
            "launches_per_call": 1 if args.fused else 2,
            "query_tokens_per_sequence": args.s_q,
            "rotating_input_sets": R,
        },
        "us_per_call": sec_per_call * 1e6,
        "pct_hbm_peak": 100.0 * gbs / HBM_PEAK_GBS,
        "roofline": {
            "bound": "hbm",
            "kernel": ("split_kv_mfma" if (w.dtype == "bf16" and not args.valu) else "split_kv_valu")
                      + (" (whole call, eager: no split-only path for S_q > 1)" if args.s_q > 1 else ""),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kv_bytes,
            "kernel_us": split_us,
        },
        "kernel_source_hash": src_hash,
        "us_per_call_spread": spread,
        "device": {"name": torch.cuda.get_device_name(dev),
                   "arch": getattr(torch.cuda.get_device_properties(dev), "gcnArchName", None),
                   "cus": torch.cuda.get_device_properties(dev).multi_processor_count,
                   "hip": torch.version.hip},
    }
    if args.s_q > 1:
        # Several query tokens: the call is a batch of small matrix products
        # (intensity grows with S_q), so its roofline is the bf16 matrix-core
        # peak. Algorithmic FLOPs: QK^T and PV, 2*d each per (query token,
        # head, attended position), token i of sequence b attending its
        # S_b - S_q + i + 1 positions (causal among the new tokens). Timed as
        # whole calls (split + merge) in the graph: there is no split-only
        # entry point for S_q > 1.
        import numpy as np
        lens_np = inp.seq_lens.astype(np.int64)
        att = np.clip(lens_np[:, None] - args.s_q + np.arange(args.s_q)[None, :] + 1, 0, None)
        flops = float(att.sum()) * w.h_q * 4 * w.d
        tflops = flops / sec_per_call / 1e12
        res["roofline"] = {
            "bound": "mfma",
            "kernel": "multi-token split + merge (whole call)",
            "achieved": round(tflops, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
            "traffic": None,
            "algorithmic_flops_per_call": flops,
            "kernel_us": sec_per_call * 1e6,
            "kv_gbs_by_eager_calls": round(achieved, 2),
        }
    if not args.no_extra and args.workload == DEFAULT_WORKLOAD and not args.seq_lens and args.s_q == 1 \
            and not (args.valu or args.fused or args.eager or args.n_splits):
        del sets
        torch.cuda.empty_cache()
        res["extra_workloads"] = {key: measure_extra(gqa, hip, key, base, hint, st)
                                  for key, base, hint, st in EXTRA_WORKLOADS}
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host")
        res["cpu_baseline"] = cpu_baseline(w.name, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
