#!/usr/bin/env python3
"""Throughput of the clustered sparse-KV hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
prefill clustering of every KV head (10 cosine k-means iterations and the
cluster index), then the workload's decode steps, each of which selects
clusters for every KV head and runs sparse attention over the recalled tokens
(for append workloads, a new token is first appended per head).

Inputs are generated on the host with the seeded generator and copied to HBM
before timing starts. The timed region holds exactly --steps passes between
two synchronisations. Kernel durations come from HIP events recorded on the
stream the kernels run on. The CPU oracle is timed over the same workload as
a reported baseline. After the headline workload 4, a cold-stack record runs
the decode of workload 5's 32 layers, whose K/V no cache holds.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode steps/s at L=32k, B=1k (select+gather+attn); k-means TFLOP/s; % roofline"
PEAK_HBM = 8.0e12    # B/s, MI355X HBM3E
PEAK_BF16 = 2.5e15   # flop/s, dense bf16 matrix cores
PEAK_F64 = 78.6e12   # flop/s, fp64 vector
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch has loaded."""

    def __init__(self, n: int):
        import torch  # noqa: F401  (loads the runtime)
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        self.rt = ctypes.CDLL(path or "libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            assert self.rt.hipEventCreate(ctypes.byref(h)) == 0
            self.ev[i] = h
        self.n = n

    def record(self, i: int, stream_handle: int):
        assert self.rt.hipEventRecord(self.ev[i], ctypes.c_void_p(stream_handle)) == 0

    def ms(self, a: int, b: int) -> float:
        out = ctypes.c_float()
        assert self.rt.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b]) == 0
        return float(out.value)

    def sub(self, start: int, count: int):
        return (ctypes.c_void_p * count)(*[self.ev[start + i] for i in range(count)])


def source_digest() -> str:
    """Digest of the kernel sources' code: comments and blank or indentation-only differences do not
    change it, any change to a statement does."""
    h = hashlib.sha256()
    for name in ("kvc_build.hip", "kvc_decode.hip", "kvc_device.h", "kvc_internal.h", "kvc_host.cpp"):
        with open(os.path.join(ROOT, "clustered_sparse_attention_kv_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [" ".join(l.split()) for l in text.splitlines()]
        h.update("\n".join(l for l in lines if l).encode())
    return h.hexdigest()[:16]


def algorithmic(w):
    """Algorithmic work of one pass, per kernel launch: the bytes each launch must move (selection and
    attention: centroids, index metadata, selected K/V rows, queries and outputs) and the flops the
    assignment must compute (2 L C d per head)."""
    e = 2 if w.dtype == 1 else 4
    S = min(w.B, w.capacity)
    H, G, C, d = w.heads, w.G, w.C, w.d
    return {
        # assignment contraction of one k-means iteration: 2 L C d flops per head
        "assign_flops": 2.0 * H * w.L * C * d,
        # select: centroids, sizes, offsets, the emitted members' ids (read) and sel_ids (written), queries
        "select_bytes": H * (C * d * 4 + C * 4 + (C + 1) * 4 + S * 4 + S * 4 + G * d * e),
        # decode: selected ids, K and V rows, queries, fp32 output
        "decode_bytes": H * (S * 4 + 2 * S * d * e + G * d * e + G * d * 4),
        # whole decode step (select + gather + attention), each byte once
        "step_bytes": H * (C * d * 4 + C * 4 + (C + 1) * 4 + S * 4 + 2 * S * d * e + G * d * e + G * d * 4),
        "kmeans_flops": 2.0 * w.iters * H * w.L * C * d,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=4, help="synthetic configuration 1-5 (default 4)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--decode-path", choices=["fused", "split"], default="fused",
                    help="fused: kv_cluster_select_decode (one kernel per step); "
                         "split: kv_cluster_select then kv_sparse_decode")
    ap.add_argument("--token-split", choices=["auto", "on", "off"], default="auto",
                    help="fused path: give kv_cluster_select_decode a workspace, so that the blocks of a KV head "
                         "split the selected tokens and the last of them merges the partial results (auto: "
                         "wherever the path has it, bf16 with at most 4 query heads per KV head)")
    ap.add_argument("--sinks", type=int, default=0,
                    help="attention sinks per head: kept out of the clustering, always selected (default 0)")
    ap.add_argument("--metric", choices=["cosine", "l2", "inner_product"], default="cosine",
                    help="assignment distance of the k-means (default cosine, the method's; L2 and inner product "
                         "are the alternatives the pages compare it with)")
    ap.add_argument("--recall-heads", type=int, default=16, help="KV heads in the recall sample")
    ap.add_argument("--recall-steps", type=int, default=4, help="decode steps in the recall sample")
    ap.add_argument("--offload", type=int, default=-1,
                    help="KV in pinned host memory, read by the kernels over the host link: 0 loads every selected "
                         "row from the host at each step; R >= 1 keeps the rows selected in the last R steps in a "
                         "GPU cluster cache and loads only absent clusters (default -1: KV in HBM)")
    ap.add_argument("--drift", type=float, default=-1.0,
                    help="mixture workloads: queries whose three components persist across steps, each replaced "
                         "with this probability per step (default: independent queries per step)")
    ap.add_argument("--window", type=int, default=0,
                    help="append workloads: generated tokens join a window that is always recalled, and every "
                         "WINDOW steps the window is clustered on its own into --window-clusters new clusters "
                         "(default 0: each new token joins its nearest centroid)")
    ap.add_argument("--window-clusters", type=int, default=4, help="clusters made from each window (default 4)")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every decode step from the host (default: the decode steps of a pass are "
                         "captured once in a HIP graph and replayed; the same kernels and work)")
    ap.add_argument("--no-pack", action="store_true",
                    help="decode from the caches through the token ids (no cluster-ordered copy)")
    ap.add_argument("--no-cold-stack", action="store_true",
                    help="workload 4: skip the cold-stack record (workload 5's 32 layers, whose 34 GB of K/V "
                         "no cache holds, decoded after the headline measurement)")
    ap.add_argument("--cold-steps", type=int, default=2, help="timed passes of the cold-stack record")
    ap.add_argument("--no-unpacked", action="store_true",
                    help="workload 4: skip the unpacked record (the same decode reading the rows from the caches "
                         "through the token ids, without the cluster-ordered copy)")
    ap.add_argument("--no-full-kv", action="store_true", help="skip the full-KV comparator")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the path runs on a single MI355X (across GPUs it would shard "
              "by KV head, with no exchange between them). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import clustered_sparse_attention_kv_amd as kvc
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    kvc.lib()  # fails loudly without the built library
    result = measure(synth.workload(args.workload), args)
    if args.workload == 4 and not args.no_pack and not args.no_unpacked:
        # the headline decodes from the cluster-ordered copy; the same workload
        # without it reads every selected row from the caches through the ids
        torch.cuda.empty_cache()
        log("[bench] unpacked: workload 4 without the cluster-ordered copy")
        up = argparse.Namespace(**vars(args))
        up.no_pack, up.no_cpu, up.no_full_kv = True, True, True
        up.steps, up.warmup = max(1, min(args.steps, 3)), 1
        ru = measure(synth.workload(4), up)
        sd = ru["rooflines"].get("select_decode", {})
        result["unpacked"] = {
            "decode_steps_per_s": ru["value"], "step_us": ru["decode_step_us"],
            "hbm_frac": ru["decode_step_hbm_frac"], "kernel": sd.get("kernel"),
            "steps": up.steps, "warmup": up.warmup, "decode_launch": ru["decode_launch"]}
    if args.workload == 4 and not args.no_cold_stack:
        # the same path over the 32-layer stack of workload 5: every decode step
        # streams 1.5 GB of centroids and K/V rows, far past the 256 MB
        # Infinity Cache, so its rate is the DRAM-bound one
        torch.cuda.empty_cache()
        log("[bench] cold stack: workload 5 (32 layers)")
        cold = argparse.Namespace(**vars(args))
        cold.workload, cold.steps, cold.warmup = 5, args.cold_steps, 1
        cold.no_cpu, cold.no_full_kv = True, True
        w5 = synth.workload(5)
        r5 = measure(w5, cold)
        sd = r5["rooflines"].get("select_decode", {})
        result["cold_stack"] = {
            "workload": w5.name, "layers": w5.layers, "kv_heads_per_layer": w5.heads, "B": w5.B,
            "decode_steps_per_s": r5["value"], "step_us": r5["decode_step_us"],
            "us_per_layer": r5["decode_step_us"] / w5.layers,
            "hbm_frac": r5["decode_step_hbm_frac"], "kernel": sd.get("kernel"),
            "bytes_per_step": algorithmic(w5)["step_bytes"] * w5.layers,
            "kmeans_tflops": r5["kmeans_tflops"], "kmeans_ms_per_layer": r5["kmeans_ms"] / w5.layers,
            "steps": cold.steps, "warmup": cold.warmup, "decode_launch": r5["decode_launch"]}
    print(json.dumps(result), flush=True)


def measure(w, args):
    """One workload through the whole path: returns the bench record (without printing it)."""
    import numpy as np
    import torch

    import clustered_sparse_attention_kv_amd as kvc
    import synth

    dev = torch.device("cuda:0")
    NL = w.layers
    H, G, L, d, C, B, cap = w.heads, w.G, w.L, w.d, w.C, w.B, w.capacity
    tdt = torch.bfloat16 if w.dtype == synth.BF16 else torch.float32
    packed = not args.no_pack and args.decode_path == "fused"
    fused = args.decode_path == "fused"
    M, NC = args.window, args.window_clusters
    metric = {"cosine": kvc.COSINE, "l2": kvc.L2, "inner_product": kvc.INNER_PRODUCT}[args.metric]
    offload = args.offload
    if offload >= 0 and not fused:
        print("--offload runs the fused path", file=sys.stderr)
        sys.exit(2)
    if args.drift >= 0 and w.query != "mixture":
        print("--drift needs a workload with mixture queries (4 or 5)", file=sys.stderr)
        sys.exit(2)
    if M and not w.append:
        print("--window needs a workload that generates tokens (an append workload)", file=sys.stderr)
        sys.exit(2)
    n_windows = w.steps // M if M else 0
    slots = C + n_windows * NC

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ---------------- inputs (host generation, then copy to HBM) -------------
    # one independent seeded mixture per layer; each layer has its own caches
    # and index, all resident in HBM before timing starts
    t0 = time.time()
    lay = []
    for li in range(NL):
        base = synth.config_seed(w.config, li)
        K, _, means = synth.mixture_keys(base, H, cap, d, w.M, w.sigma, w.n_out, w.out_scale, w.dtype,
                                         want_means=(w.query == "mixture"))
        V = synth.values(base, H, cap, d, w.dtype)
        qs = []
        for s in range(w.steps):
            n_cur = L + (s + 1 if w.append else 0)
            if w.query == "mixture" and args.drift >= 0:
                qs.append(synth.queries_drift(base, s, H * G, G, means, w.q_sigma, args.drift, w.dtype))
            elif w.query == "mixture":
                qs.append(synth.queries_mixture(base, s, H * G, G, means, w.q_sigma, w.dtype))
            else:
                qs.append(synth.queries_noisy_key(base, s, H * G, G, K, n_cur, w.q_sigma))
        Q = np.stack(qs)
        # the build draws its initial centroids from this seed (seeded shuffle on the device)
        e = {"Qd": to_dev(Q), "seed": base}
        if w.append:  # appended rows come in through the append call
            e["Knew"] = to_dev(np.ascontiguousarray(K[:, L:].transpose(1, 0, 2)))  # [steps, H, d]
            e["Vnew"] = to_dev(np.ascontiguousarray(V[:, L:].transpose(1, 0, 2)))
            K[:, L:] = 0
            V[:, L:] = 0
        e["Kd"], e["Vd"] = to_dev(K), to_dev(V)
        e["idx"] = kvc.ClusterIndex(H, C, cap, tdt, device=dev, packed=packed, n_sink=args.sinks, c_slots=slots,
                                    metric=metric, packed_on_host=offload >= 0)
        if offload >= 0:
            # the decode reads the KV from pinned host memory; the prefill
            # clustering still runs on the copy in HBM
            e["Kh"], e["Vh"] = e["Kd"].cpu().pin_memory(), e["Vd"].cpu().pin_memory()
            if offload >= 1:
                e["cache"] = kvc.ClusterCache(e["idx"], offload, B, device=dev)
        else:
            e["Kh"], e["Vh"] = e["Kd"], e["Vd"]
        # initial centroids of each window's clustering: seeded positions in the window
        e["winit"] = [to_dev(synth.init_idx(synth.stream_seed(base, 7, k), H, M, NC) + np.int32(L + k * M))
                      for k in range(n_windows)]
        if li == 0:
            base0, Q0 = base, Q
        lay.append(e)
        del K, V
    log(f"[bench] generated {w.name} inputs ({NL} layer(s)) in {time.time() - t0:.1f}s")
    ws_build = torch.empty(kvc.build_workspace_bytes(H, L, C, w.iters), dtype=torch.uint8, device=dev)
    ws_dec = torch.empty(kvc.decode_workspace_bytes(H, H * G, B), dtype=torch.uint8, device=dev)
    # the library uses the workspace for bf16 and at most 4 query heads per KV head
    tsplit = fused and w.dtype == synth.BF16 and G <= 4 and args.token_split in ("on", "auto")
    # (its arrival counters must start at zero; every call leaves them zero)
    ws_sd = (torch.zeros(kvc.select_decode_workspace_bytes(H, H * G), dtype=torch.uint8, device=dev)
             if tsplit else None)
    ws_win = (torch.empty(kvc.window_workspace_bytes(H, M, NC, w.iters), dtype=torch.uint8, device=dev)
              if M else None)
    ws_cache = (torch.empty(kvc.cache_workspace_bytes(H, H * G, B), dtype=torch.uint8, device=dev)
                if offload >= 1 else None)
    sel = torch.empty(H, B, dtype=torch.int32, device=dev)
    cnt = torch.empty(H, dtype=torch.int32, device=dev)
    out = torch.empty(H * G, d, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    # plain copy of a known size, for scaling the profiler's byte counters
    cal_src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    del cal_src, cal_dst

    # events per pass: 2*iters per layer around the assignment kernels inside
    # the builds, 4 bracketing the builds, the packed copies and the decode
    # phase, and, on every SAMPLE-th decode step only (events between kernels
    # add dispatch gaps), 6 around that step's first-layer kernels (append,
    # select, decode), and 2 around each window clustering of the first layer
    SAMPLE = 8
    sampled = [s for s in range(w.steps) if s % SAMPLE == 0]
    A = 2 * w.iters * NL
    WB = A + 4 + 6 * len(sampled)
    per_pass = WB + 2 * n_windows
    total_passes = args.warmup + args.steps
    ev = HipEvents(per_pass * total_passes + 2)

    def prepare(o: int):
        """Builds (and packed copies, cache resets) of every layer: each resets the index's state."""
        ev.record(o + A, sh)
        for li, e in enumerate(lay):
            kvc.build(e["idx"], e["Kd"], L, w.iters, seed=e["seed"], workspace=ws_build,
                      assign_events=ev.sub(o + 2 * w.iters * li, 2 * w.iters))
        ev.record(o + A + 3, sh)
        if packed:
            for e in lay:
                kvc.pack(e["idx"], e["Kd"], e["Vd"])
                if offload >= 1:
                    kvc.cache_reset(e["idx"], e["cache"])
        ev.record(o + A + 1, sh)

    def decode_steps(o):
        """The workload's decode steps; with o set, events around the kernels of
        every SAMPLE-th step (first layer) and around each window clustering."""
        b = o + A + 4 if o is not None else None
        for s in range(w.steps):
            for li, e in enumerate(lay):
                e6 = b + 6 * (s // SAMPLE) if (b is not None and s % SAMPLE == 0 and li == 0) else None
                rec = (lambda i: ev.record(e6 + i, sh)) if e6 is not None else (lambda i: None)
                if w.append:
                    rec(0)
                    if M:
                        kvc.append_window(e["idx"], e["Kd"], e["Vd"], e["Knew"][s].unsqueeze(1),
                                          e["Vnew"][s].unsqueeze(1))
                    else:
                        kvc.append(e["idx"], e["Kd"], e["Vd"], e["Knew"][s].unsqueeze(1), e["Vnew"][s].unsqueeze(1))
                    rec(1)
                    if M and (s + 1) % M == 0:
                        k = (s + 1) // M - 1
                        if li == 0 and o is not None:
                            ev.record(o + WB + 2 * k, sh)
                        kvc.cluster_window(e["idx"], e["Kd"], e["Vd"], NC, w.iters, e["winit"][k], workspace=ws_win)
                        if li == 0 and o is not None:
                            ev.record(o + WB + 2 * k + 1, sh)
                rec(2)
                if fused and offload >= 1:
                    rec(3)
                    kvc.cached_select_decode(e["idx"], e["cache"], e["Qd"][s], e["Kh"], e["Vh"], scale, out=out,
                                             workspace=ws_cache)
                elif fused:
                    rec(3)
                    kvc.select_decode(e["idx"], e["Qd"][s], e["Kh"], e["Vh"], B, scale, out=out, workspace=ws_sd)
                else:
                    kvc.select(e["idx"], e["Qd"][s], B, sel, cnt)
                    rec(3)
                    kvc.sparse_decode(e["Qd"][s], e["Kd"], e["Vd"], sel, cnt, scale, out=out, workspace=ws_dec)
                rec(4)

    def one_pass(p: int, graph=None):
        o = p * per_pass
        prepare(o)
        if graph is None:
            decode_steps(o)
        else:
            graph.replay()
        ev.record(o + A + 2, sh)

    use_graph = not args.no_graph
    # passes whose per-kernel events are read: launched step by step from the
    # host (the warm-up passes with graphs, else the timed ones)
    eager = list(range(max(args.warmup, 1))) if use_graph else list(range(args.warmup, total_passes))
    graph = None
    for p in range(args.warmup):
        one_pass(p)
    if use_graph:
        if args.warmup == 0:
            one_pass(0)  # a pass for the per-kernel events
        torch.cuda.synchronize()
        # capture one pass's decode steps after a build (the build resets the
        # index state, so the captured arguments fit every pass)
        prepare(0)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, capture_error_mode="relaxed"):
            decode_steps(None)
        torch.cuda.synchronize()
        graph.replay()  # a warm replay before timing
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev.record(per_pass * total_passes, sh)
    for p in range(args.warmup, total_passes):
        one_pass(p, graph)
    ev.record(per_pass * total_passes + 1, sh)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    total_ms = ev.ms(per_pass * total_passes, per_pass * total_passes + 1)

    assign_ms, build_ms, select_ms, decode_ms, append_ms, phase_ms, pack_ms = [], [], [], [], [], [], []
    window_ms = []
    for p in range(args.warmup, total_passes):
        o = p * per_pass
        assign_ms += [ev.ms(o + 2 * t, o + 2 * t + 1) for t in range(w.iters * NL)]
        build_ms.append(ev.ms(o + A, o + A + 3))
        pack_ms.append(ev.ms(o + A + 3, o + A + 1))
        phase_ms.append(ev.ms(o + A + 1, o + A + 2))
    for p in eager:
        o = p * per_pass
        b = o + A + 4
        for i in range(len(sampled)):
            e6 = b + 6 * i
            if w.append:
                append_ms.append(ev.ms(e6, e6 + 1))
            select_ms.append(ev.ms(e6 + 2, e6 + 3))
            decode_ms.append(ev.ms(e6 + 3, e6 + 4))
        window_ms += [ev.ms(o + WB + 2 * k, o + WB + 2 * k + 1) for k in range(n_windows)]

    alg = algorithmic(w)
    mean = lambda x: sum(x) / len(x) if x else 0.0
    a_ms, s_ms, dd_ms = mean(assign_ms), mean(select_ms), mean(decode_ms)
    decode_phase_s = sum(phase_ms) / 1e3
    n_dec = args.steps * w.steps
    # when the decode phase is nothing but back-to-back launches of the fused
    # kernel (one per step and layer, replayed from a graph), its per-launch
    # time is the phase time over the launches: no events between the kernels
    phase_only = use_graph and fused and not w.append and offload < 1
    if phase_only:
        dd_ms = sum(phase_ms) / (n_dec * NL)
    value = n_dec / decode_phase_s
    step_ms = sum(phase_ms) / n_dec
    kmeans_tflops = alg["kmeans_flops"] * NL * args.steps / (sum(build_ms) / 1e3) / 1e12

    assign_peak = PEAK_BF16 if w.dtype == synth.BF16 else PEAK_F64
    rl = {
        "assign": {"bound": "mfma" if w.dtype == synth.BF16 else "alu", "achieved": alg["assign_flops"] / (a_ms / 1e3) / 1e12,
                   "peak": assign_peak / 1e12, "unit": "TFLOP/s", "avg_us": a_ms * 1e3,
                   "share": sum(assign_ms) / total_ms},
    }
    kernel_names = {"assign": "assign_bf16_mfma_kernel" if w.dtype == synth.BF16 else "assign_exact_kernel"}
    if fused:
        rl["select_decode"] = {"bound": "hbm", "achieved": alg["step_bytes"] / (dd_ms / 1e3) / 1e9,
                               "peak": PEAK_HBM / 1e9, "unit": "GB/s", "avg_us": dd_ms * 1e3,
                               "share": dd_ms * n_dec * NL / total_ms}
        kernel_names["select_decode"] = ("select_decode_bf16_kernel" if w.dtype == synth.BF16
                                         else "select_decode_kernel")
        if ws_sd is not None:
            kernel_names["select_decode"] = "select_decode_bf16_kernel (token split, merged by the last block)"
        if offload >= 1:
            kernel_names["select_decode"] = "cache_assemble_kernel + decode_split_kernel + decode_combine_kernel"
    else:
        rl["sparse_decode"] = {"bound": "hbm", "achieved": alg["decode_bytes"] / (dd_ms / 1e3) / 1e9,
                               "peak": PEAK_HBM / 1e9, "unit": "GB/s", "avg_us": dd_ms * 1e3,
                               "share": dd_ms * n_dec * NL / total_ms}
        rl["select"] = {"bound": "hbm", "achieved": alg["select_bytes"] / (s_ms / 1e3) / 1e9, "peak": PEAK_HBM / 1e9,
                        "unit": "GB/s", "avg_us": s_ms * 1e3, "share": s_ms * n_dec * NL / total_ms}
        kernel_names["sparse_decode"] = "decode_split_kernel + decode_combine_kernel"
        kernel_names["select"] = "select_kernel"
    traffic = {}
    if os.path.exists(PROFILE_TRAFFIC):
        with open(PROFILE_TRAFFIC) as f:
            prof = json.load(f)
        rec = prof.get(w.name, {})
        if rec.get("source_digest") == source_digest():
            traffic = rec.get("bytes_per_launch", {})
    for k, r in rl.items():
        r["frac"] = r["achieved"] / r["peak"]
        # the record is keyed by the kernel's symbol name (the first word of the display name); a
        # phase of several kernels has none
        name = kernel_names[k]
        r["traffic"] = None if "+" in name else traffic.get(name.split()[0])
        r["kernel"] = kernel_names[k]
    dominant = max(rl, key=lambda k: rl[k]["share"])
    roofline = {k2: rl[dominant][k2] for k2 in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    roofline["kernel"] = kernel_names[dominant]
    roofline["avg_us"] = rl[dominant]["avg_us"]

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == synth.BF16 else "f32",
        "data": "synthetic (seeded Gaussian-mixture keys with outlier channels, N(0,1) values)",
        "config": {"workload": w.name, "layers": NL, "kv_heads_total": H * NL, "q_heads_total": H * G * NL, "G": G,
                   "L": L, "d": d, "C": C,
                   "kmeans_iters": w.iters, "B": B, "decode_steps_per_step": w.steps, "append": w.append,
                   "decode_path": args.decode_path, "token_split": ws_sd is not None, "packed_kv": packed,
                   "sinks": args.sinks, "window": M, "window_clusters": NC if M else 0, "metric": args.metric,
                   "offload": offload, "query_drift": args.drift},
        "kmeans_tflops": kmeans_tflops,
        "kmeans_ms": mean(build_ms),
        "pack_ms": mean(pack_ms),
        "decode_step_us": step_ms * 1e3,
        "decode_step_hbm_frac": alg["step_bytes"] * NL / (step_ms / 1e3) / PEAK_HBM,
        "kernel_timing": (("HIP events around every assignment kernel; the fused kernel's launch time is the "
                           "event-bracketed decode phase over its launches (the phase replays only that kernel)")
                          if phase_only and ws_sd is None else
                          ("HIP events around every assignment kernel; the fused kernel's launch time (token "
                           "split, merged in the kernel) is the event-bracketed decode phase over its launches "
                           "(the phase replays only that kernel)")
                          if phase_only else
                          f"HIP events around every kernel of 1 in {SAMPLE} decode steps (passes launched step "
                          "by step) and around every assignment kernel; value from events bracketing each pass's "
                          "decode phase"),
        "decode_launch": "HIP graph of the pass's decode steps, replayed" if use_graph else "step by step",
        "wall_s_timed": wall,
        "roofline": roofline,
        "rooflines": rl,
    }
    if w.append:
        result["append_us"] = mean(append_ms) * 1e3
    if offload >= 0:
        # bytes read from host memory per decode step: the selected K/V rows
        # that did not come from the cache (all of them without one)
        e_b = 2 if w.dtype == synth.BF16 else 4
        sel_bytes = H * NL * min(B, L) * 2 * d * e_b
        hit = lay[0]["cache"].hit_rates()["token_hit_rate"] if offload >= 1 else 0.0
        host_bytes = sel_bytes * (1.0 - hit)
        result["offload"] = {"R": offload, "kv": "pinned host memory, read by the kernels over the host link",
                             "drift": args.drift, "host_bytes_per_step": host_bytes,
                             "host_GBps": host_bytes / (step_ms / 1e3) / 1e9}
        if offload >= 1:
            result["offload"]["hit_rates"] = lay[0]["cache"].hit_rates()
    if M:
        result["cluster_window_us"] = mean(window_ms) * 1e3
        result["clusters_after_pass"] = C + n_windows * NC

    # ---------------- full-KV comparator (dense decode over all L rows) -----
    if w.dtype == synth.BF16 and not args.no_full_kv:
        e0 = lay[0]
        ws_dense = torch.empty(kvc.dense_decode_workspace_bytes(H, H * G, L), dtype=torch.uint8, device=dev)
        for i in range(3):
            kvc.dense_decode(e0["Qd"][i % w.steps], e0["Kd"], e0["Vd"], L, scale, out=out, workspace=ws_dense)
        R = 20
        dev_ev = HipEvents(2)
        dev_ev.record(0, sh)
        for i in range(R):
            kvc.dense_decode(e0["Qd"][i % w.steps], e0["Kd"], e0["Vd"], L, scale, out=out, workspace=ws_dense)
        dev_ev.record(1, sh)
        torch.cuda.synchronize()
        dense_ms = dev_ev.ms(0, 1) / R
        e = 2
        full_bytes = H * (2 * L * d * e + G * d * e + G * d * 4)
        full_step_us = dense_ms * 1e3 * NL
        result["full_kv"] = {
            "what": "kv_dense_decode: attention over all L rows of every KV head, per decode step (all layers)",
            "decode_steps_per_s": 1e6 / full_step_us, "step_us": full_step_us,
            "hbm_frac": full_bytes / (dense_ms / 1e3) / PEAK_HBM,
            "sparse_speedup": value / (1e6 / full_step_us)}

    # ---------------- CPU oracle baseline (bounded sample) -----------------
    if not args.no_cpu:
        log("[bench] CPU oracle over the workload")
        result["cpu_baseline"] = cpu_baseline(w, args, base0, Q0)
        # still the CPU leg, after the timed region: the oracle's exact top-B
        # attention tokens against the GPU's selections of the first decode
        # steps (layer 0, sampled heads, a fresh build of the prompt, no
        # generated tokens), reported as the selection_recall diagnostic
        e0 = lay[0]
        kvc.build(e0["idx"], e0["Kd"], L, w.iters, seed=e0["seed"], workspace=ws_build)
        sels = []
        for s_ in range(min(args.recall_steps, w.steps)):
            kvc.select(e0["idx"], e0["Qd"][s_], B, sel, cnt)
            torch.cuda.synchronize()
            sels.append((s_, sel.cpu().numpy(), cnt.cpu().numpy()))
        result["selection_recall"] = recall_sample(w, args, base0, Q0, sels)
    return result


def cpu_baseline(w, args, base, Q):
    """The oracle as it stands, on the host cores, over the whole workload: the
    k-means of every KV head (all iterations), then every decode step (append
    for the append workloads, selection and attention of every head). A stack
    of layers runs its first layer and is scaled to all of them."""
    import numpy as np

    import oracle
    import synth

    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    rows = w.capacity
    K, _, _ = synth.mixture_keys(base, w.heads, rows, w.d, w.M, w.sigma, w.n_out, w.out_scale, w.dtype)
    V = synth.values(base, w.heads, rows, w.d, w.dtype)
    metric = {"cosine": oracle.COSINE, "l2": oracle.L2, "inner_product": oracle.IP}[args.metric]
    t0 = time.perf_counter()
    built = oracle.build(np.ascontiguousarray(K[:, :w.L]), w.C, w.iters, seed=base, early_exit=False,
                         n_sink=args.sinks, metric=metric)
    t_km = time.perf_counter() - t0
    scale = 1.0 / math.sqrt(w.d)
    index = oracle.Index(built, rows, metric=metric) if w.append else None
    t0 = time.perf_counter()
    for s in range(w.steps):
        q = np.ascontiguousarray(Q[s])
        if index is not None:
            index.append(np.ascontiguousarray(K[:, w.L + s]))
            c, sz, off, ids = index.c, index.sizes, index.offsets, index.token_ids
        else:
            c, sz, off, ids = built["c"], built["sizes"], built["offsets"], built["token_ids"]
        sel, cnt, _, _ = oracle.select(q, w.G, c, sz, off, ids, w.B, n_sink=args.sinks)
        oracle.decode(q, w.G, K, V, sel, cnt, scale)
    t_dec = time.perf_counter() - t0
    per_step = t_dec / w.steps * w.layers
    flops = 2.0 * w.iters * w.heads * w.L * w.C * w.d
    sample = (f"the whole workload: k-means of all {w.heads} KV heads ({w.iters} iterations, no early exit) and all "
              f"{w.steps} decode steps ({'append, ' if w.append else ''}selection and attention of every head)")
    if w.layers > 1:
        sample = f"layer 0 of {w.layers} ({sample[len('the whole workload: '):]}), decode time scaled x{w.layers}"
    return {"value": 1.0 / per_step, "unit": "decode steps/s", "cores": threads, "kind": "oracle", "sample": sample,
            "kmeans_s": t_km, "kmeans_gflops": flops / t_km / 1e9, "decode_s": t_dec}


def recall_sample(w, args, base, Q, sels):
    """Recall of the exact top-B attention tokens (oracle, fp64) by the GPU's
    selections (a list of (decode step, sel_ids, sel_count)), for the first
    KV heads of layer 0."""
    import numpy as np

    import oracle
    import synth

    nh = min(args.recall_heads, w.heads)
    K, _, _ = synth.mixture_keys(base, nh, w.L, w.d, w.M, w.sigma, w.n_out, w.out_scale, w.dtype)
    rs = []
    for s, sel, cnt in sels:
        rs.append(oracle.recall(np.ascontiguousarray(Q[s, :nh * w.G]), w.G, K, w.L, np.ascontiguousarray(sel[:nh]),
                                np.ascontiguousarray(cnt[:nh])))
    r = np.concatenate(rs)
    return {"mean": float(r.mean()), "min": float(r.min()), "budget": w.B, "metric": args.metric,
            "sample": f"{nh} KV heads ({nh * w.G} query heads) x decode steps 0..{len(sels) - 1}, layer 0"}


if __name__ == "__main__":
    main()
