"""Benchmark of the fused o-projection + AttnRes decode step on one MI355X.

Headline workload: M = 8 tokens, K = 4096, N = H = 7168, nb = 4 saved blocks,
non-write layer (delta path), one aux copy, non-final boundary. One "step" is
one attnres_oproj_run call (one launch of the fused kernel) over one batch.
The same run also times the other two workloads the metric names (M = 1,
K = 1024, nb = 1; M = 64, K = 8192, nb = 8 with a block write) under the
same protocol and reports each in `workloads`.

Protocol, per workload:
  * L distinct layer copies (W, x, prefix, blocks, out, aux, workspace) with a
    footprint of at least 640 MB, so the 256 MB Infinity Cache cannot serve W;
    the first call on copy 0 is checked against the FP64 oracle before timing
    (new prefix within one projection ulp, output within two bf16 ulps of the
    oracle's AttnRes on the GPU's own new prefix).
  * `--warmup` eager steps, then one HIP graph holding exactly `--steps` calls
    that cycle through the copies; the graph is replayed once untimed (upload)
    and once timed, bracketed by synchronisations and HIP events on the stream
    the kernels run on. Afterwards every copy's workspace is checked (a wait
    that gave up would invalidate the results and fails the run).
  * value = algorithmic bytes per step / measured time per step (GB/s);
    roofline.achieved is the same figure for the fused kernel, the only kernel
    of a step, against the 8 TB/s HBM peak.
  * cpu_baseline: the FP64 oracle (oracle/, plain C) on the headline step,
    timed on one host thread and on every core the process may use, in the
    same process.

Prints one JSON line. `--config` picks another headline among the fused
workloads (0, 1, 2; `--only` times just that one); `--config 3` (attnres_run,
T=256, nb = 0..8, final boundary), `--config 4` (wsgemm_run, K=7168, N=4096,
M = 1, 8, 16, 48, 64; beyond 32 tokens also wsgemm_run_ws, which alone takes
M = 128; at M = 8 and 64 also the MoE-front epilogue) and `--config 5`
(look-ahead statistics: attnres_oproj_ahead_run beside attnres_oproj_run on
workloads 0-2, attnres_post_run beside attnres_run at T=256, nb=8) print one
JSON line per case, timed the same way.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FOOTPRINT = 640e6

# HBM bytes per launch of the fused kernel from two rocprofv3 --pmc runs
# (FETCH_SIZE, WRITE_SIZE; each scaled by what the counter reads for a plain
# device copy of known size, run with --calibrate-copy-mb). A figure holds only
# for the kernel sources it was measured on: `digest` is the SHA-256 of their
# code (comments and whitespace aside), and roofline.traffic is null when the
# sources differ.
KERNEL_SOURCES = ("common.hpp", "token.hpp", "gemm.hpp", "launch.hpp", "fused.hip")
MEASURED_TRAFFIC = {  # (workload, "prepared" | "row-major") -> {"digest", "fetch", "write"}
    (1, "prepared"): {"digest": "d133d4a31d163a6ffafa53f73847f825f5380153708ef44b95f7aa4cb620129a", "fetch": 60886117, "write": 917504},
    (1, "row-major"): {"digest": "d133d4a31d163a6ffafa53f73847f825f5380153708ef44b95f7aa4cb620129a", "fetch": 61041276, "write": 1468928},
    (0, "prepared"): {"digest": "d133d4a31d163a6ffafa53f73847f825f5380153708ef44b95f7aa4cb620129a", "fetch": 14986008, "write": 114688},
    (0, "row-major"): {"digest": "d133d4a31d163a6ffafa53f73847f825f5380153708ef44b95f7aa4cb620129a", "fetch": 14982403, "write": 183616},
    (2, "prepared"): {"digest": "d133d4a31d163a6ffafa53f73847f825f5380153708ef44b95f7aa4cb620129a", "fetch": 139301207, "write": 9175040},
    (2, "row-major"): {"digest": "d133d4a31d163a6ffafa53f73847f825f5380153708ef44b95f7aa4cb620129a", "fetch": 139203367, "write": 9175040},
}

WORKLOADS = {
    0: dict(M=1, K=1024, nb=1, cap=1, write=-1, has_delta=1),
    1: dict(M=8, K=4096, nb=4, cap=4, write=-1, has_delta=1),
    2: dict(M=64, K=8192, nb=8, cap=9, write=8, has_delta=1),
}
H = 7168


def algorithmic_bytes(M, K, nb, write, has_delta, aux=1, H=H):
    """What the step must move, each byte once: W, x, three gain rows, and per
    token the old prefix (if read), the nb scored blocks, the new prefix, the
    aux copy, the written block slot and the output row."""
    row = 2 * H
    return 2 * H * K + 2 * M * K + 3 * row + M * row * (
        has_delta + nb + 1 + aux + (1 if write >= 0 else 0) + 1)


def code_text(src: str) -> str:
    """Source text without comments and with whitespace collapsed: what the
    compiler sees (a comment edit does not change the kernel)."""
    import re

    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_digest() -> str:
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "skinny_gemm_attention_amd", "csrc", f)) as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()


def graph_time_us(torch, step, steps, warmup):
    """Average µs per call of `steps` calls captured in one HIP graph (replayed
    once untimed, once timed between HIP events on the launch stream)."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            for i in range(steps):
                step(i)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


def stream_read_gbs(torch, sga, dev, gb, reps=10):
    """Streaming-read bandwidth: attnres_stream_read over a `gb` GB buffer,
    `reps` launches between HIP events on one stream (one warm-up launch)."""
    n = int(gb * 1e9) // 16 * 16
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    sink = torch.empty(sga.STREAM_READ_SINK_WORDS, dtype=torch.int32, device=dev)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        sga.attnres_stream_read(src, sink, stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            sga.attnres_stream_read(src, sink, stream)
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del src, sink
    torch.cuda.empty_cache()
    return {"gbs": round(n / (us * 1e-6) / 1e9, 1), "bytes": n, "us_per_pass": round(us, 2),
            "kernel": "stream_read_kernel (attnres_stream_read): 16-byte non-temporal loads, "
                      "65536 workgroups x 512 threads, grid-stride",
            "frac_of_peak": round(n / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def side_configs(args, np, torch, sga, synth):
    """Standalone AttnRes (T=256, nb = 0..8, final boundary), standalone GEMM
    (K=7168, N=4096, M = 1, 8, 16, 64) or the look-ahead statistics: one JSON
    line per case."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    steps = min(args.steps, 400)
    if args.config == 5:
        lookahead_configs(args, np, torch, sga, synth, up, steps)
        return
    if args.config == 3:
        T = 256
        for nb in range(9):
            s = synth.config_inputs(3, nb=nb)
            row = 2 * H
            nbytes = 3 * row + T * row * (1 + 1 + nb + 1 + 1 + 1)  # delta, prefix, blocks, writes
            L = max(2, math.ceil(FOOTPRINT / (T * row * (nb + 5))))
            base = dict(delta=up(s.delta), prefix=up(s.prefix), blocks=up(s.blocks))
            nq = [up(s.norm), up(s.query), up(s.out_norm)]
            cp = []
            for i in range(L):
                t = {k: v.clone() for k, v in base.items()}
                t["out"] = torch.zeros((T, H), dtype=torch.int16, device=dev)
                t["aux"] = torch.zeros((T, H), dtype=torch.int16, device=dev)
                cp.append(t)
            torch.cuda.synchronize()

            def step(i):
                t = cp[i % L]
                sga.attnres_run(t["delta"], t["prefix"], t["blocks"], *nq, t["out"], t["aux"],
                                nb=nb, write=-1, has_delta=1, final_boundary=1)

            us = graph_time_us(torch, step, steps, args.warmup)
            print(json.dumps({"metric": "attnres_run µs/call + achieved HBM GB/s",
                              "value": round(nbytes / us / 1e3, 1), "unit": "GB/s",
                              "us_per_call": round(us, 3), "pct_of_hbm_peak":
                              round(100 * nbytes / us / 1e3 / HBM_PEAK_GBS, 1),
                              "algorithmic_bytes": nbytes, "dtype": "bf16",
                              "data": "synthetic", "config": {
                                  "workload": f"attnres_run T={T} H={H} nb={nb} final=1 aux=1",
                                  "layer_copies": L}}), flush=True)
            del cp
    else:
        N, K = 4096, 7168
        for M in (1, 8, 16, 48, 64, 128):
            x, W = synth.gemm_inputs(M, N, K)
            nbytes = 2 * N * K + 2 * M * K + 2 * M * N
            L = max(2, math.ceil(FOOTPRINT / (2 * N * K)))
            xg = up(x)
            Ws = [up(W)]
            for i in range(1, L):
                Ws.append(Ws[0].clone())
            ys = [torch.zeros((M, N), dtype=torch.int16, device=dev) for _ in range(L)]
            torch.cuda.synchronize()

            def step(i):
                sga.wsgemm_run(xg, Ws[i % L], ys[i % L])

            if M <= 64:  # beyond 64 tokens only the workspace call takes them
                us = graph_time_us(torch, step, steps, args.warmup)
                _line("wsgemm_run µs/call + achieved HBM GB/s", nbytes, us,
                      f"wsgemm_run M={M} N={N} K={K}", layer_copies=L)
            if M in (8, 64):  # the same GEMM with the MoE-front epilogue
                valid, split, width = 384, 512, 7168
                mbytes = 2 * N * K + 2 * M * K + M * (4 * valid + 2 * (N - split))
                outs = [torch.zeros((M, width), dtype=torch.int16, device=dev) for _ in range(L)]
                torch.cuda.synchronize()

                def step_moe(i):
                    sga.wsgemm_moe_front_run(xg, Ws[i % L], outs[i % L], router_base=3584,
                                             slot=0, base=0, valid=valid, split=split)

                us = graph_time_us(torch, step_moe, steps, args.warmup)
                _line("wsgemm_moe_front_run µs/call + achieved HBM GB/s", mbytes, us,
                      f"wsgemm_moe_front_run M={M} N={N} K={K} valid={valid} split={split} "
                      f"router_base=3584 base=0", layer_copies=L)
                del outs
            if M > 32:  # the same GEMM with a workspace: K split across workgroups
                wss = [sga.make_gemm_workspace(M, N, dev) for _ in range(L)]
                torch.cuda.synchronize()

                def step_ws(i):
                    sga.wsgemm_run_ws(xg, Ws[i % L], ys[i % L], wss[i % L])

                us = graph_time_us(torch, step_ws, steps, args.warmup)
                _line("wsgemm_run_ws µs/call + achieved HBM GB/s", nbytes, us,
                      f"wsgemm_run_ws M={M} N={N} K={K}", layer_copies=L)
                del wss
            del Ws, ys


def _line(metric, nbytes, us, workload, **extra):
    d = {"metric": metric, "value": round(nbytes / us / 1e3, 1), "unit": "GB/s",
         "us_per_call": round(us, 3), "pct_of_hbm_peak":
         round(100 * nbytes / us / 1e3 / HBM_PEAK_GBS, 1), "algorithmic_bytes": nbytes,
         "dtype": "bf16", "data": "synthetic", "config": {"workload": workload, **extra}}
    print(json.dumps(d), flush=True)


def lookahead_configs(args, np, torch, sga, synth, up, steps):
    """The fused step with and without the next layer's saved-block statistics
    (mixture [M, H] FP32 + [M, 2] written on top), on row-major and on
    prepared W, and AttnRes on carried
    statistics (reads the FP32 mixture instead of nb saved blocks) beside
    attnres_run."""
    dev = torch.device("cuda:0")
    for c, cfg in WORKLOADS.items():
        M, K, nb, cap, write = (cfg[k] for k in ("M", "K", "nb", "cap", "write"))
        s = synth.decode_step(M, K, nb, cap=cap, write=write, seed=0)
        nx = synth.decode_step(1, None, 0, seed=0, layer=1)
        copy_bytes = 2 * (2 * H * K) + 2 * M * K + M * 2 * H * (4 + cap) + M * H * 4  # W twice
        L = max(2, math.ceil(FOOTPRINT / copy_bytes))
        base = dict(x=up(s.x), W=up(s.W), prefix=up(s.prefix), blocks=up(s.blocks))
        base["Wp"] = sga.attnres_pack_weights(base["W"])
        nq = [up(s.norm), up(s.query), up(s.out_norm)]
        nn, nqq = up(nx.norm), up(nx.query)
        layers = []
        for i in range(L):
            t = {k: v.clone() for k, v in base.items()}
            t["out"] = torch.zeros((M, H), dtype=torch.int16, device=dev)
            t["aux"] = torch.zeros((M, H), dtype=torch.int16, device=dev)
            t["ws"] = sga.make_workspace(M, H, nb, dev)
            t["mix"] = torch.zeros((M, H), dtype=torch.float32, device=dev)
            t["scal"] = torch.zeros((M, 2), dtype=torch.float32, device=dev)
            layers.append(t)
        torch.cuda.synchronize()

        def plain(i):
            t = layers[i % L]
            sga.attnres_oproj_run(t["x"], t["W"], t["prefix"], t["blocks"], *nq, t["out"],
                                  t["aux"], t["ws"], nb=nb, write=write)

        def ahead(i):
            t = layers[i % L]
            sga.attnres_oproj_ahead_run(t["x"], t["W"], t["prefix"], t["blocks"], *nq, t["out"],
                                        t["aux"], t["ws"], nn, nqq, t["mix"], t["scal"], nb=nb,
                                        write=write)

        def packed_plain(i):
            t = layers[i % L]
            sga.attnres_oproj_packed_run(t["x"], t["Wp"], H, t["prefix"], t["blocks"], *nq,
                                         t["out"], t["aux"], t["ws"], nb=nb, write=write)

        def packed_ahead(i):
            t = layers[i % L]
            sga.attnres_oproj_packed_ahead_run(t["x"], t["Wp"], H, t["prefix"], t["blocks"], *nq,
                                               t["out"], t["aux"], t["ws"], nn, nqq, t["mix"],
                                               t["scal"], nb=nb, write=write)

        base_bytes = algorithmic_bytes(M, K, nb, write, 1)
        extra = 2 * 2 * H + M * H * 4 + M * 8  # next norm + query, mixture, scal
        for name, fn, nbytes in (("attnres_oproj_run", plain, base_bytes),
                                 ("attnres_oproj_ahead_run", ahead, base_bytes + extra),
                                 ("attnres_oproj_packed_run", packed_plain, base_bytes),
                                 ("attnres_oproj_packed_ahead_run", packed_ahead,
                                  base_bytes + extra)):
            us = graph_time_us(torch, fn, steps, args.warmup)
            _line(f"{name} µs/call + achieved HBM GB/s", nbytes, us,
                  f"{name} M={M} K={K} N=H={H} nb={nb} write={write}", layer_copies=L)
        del layers
    T, nb = 256, 8
    s = synth.config_inputs(3, nb=nb)
    mix_ref = torch.zeros((T, H), dtype=torch.float32, device=dev)
    row = 2 * H
    L = max(2, math.ceil(FOOTPRINT / (T * row * (nb + 5))))
    cp = []
    for i in range(L):
        cp.append(dict(delta=up(s.delta), prefix=up(s.prefix), blocks=up(s.blocks),
                       out=torch.zeros((T, H), dtype=torch.int16, device=dev),
                       aux=torch.zeros((T, H), dtype=torch.int16, device=dev),
                       mix=mix_ref.clone().uniform_(-1, 1),
                       scal=torch.tensor([[0.0, 3.0]] * T, dtype=torch.float32, device=dev)))
    nq = [up(s.norm), up(s.query), up(s.out_norm)]
    torch.cuda.synchronize()

    def run(i):
        t = cp[i % L]
        sga.attnres_run(t["delta"], t["prefix"], t["blocks"], *nq, t["out"], t["aux"], nb=nb,
                        final_boundary=1)

    def post(i):
        t = cp[i % L]
        sga.attnres_post_run(t["delta"], t["prefix"], None, *nq, t["out"], t["aux"], t["mix"],
                             t["scal"], nb=nb, final_boundary=1)

    run_bytes = 3 * row + T * row * (1 + 1 + nb + 1 + 1 + 1)
    post_bytes = 3 * row + T * row * (1 + 1 + 1 + 1 + 1) + T * (H * 4 + 8)
    for name, fn, nbytes in (("attnres_run", run, run_bytes), ("attnres_post_run", post, post_bytes)):
        us = graph_time_us(torch, fn, steps, args.warmup)
        _line(f"{name} µs/call + achieved HBM GB/s", nbytes, us,
              f"{name} T={T} H={H} nb={nb} final=1 aux=1", layer_copies=L)


def fused_measure(cfg_id, args, np, torch, sga, synth, dev, final=0, packed=False):
    """One fused workload: parity of the first call on copy 0 against the
    oracle, then `steps` calls in one HIP graph, timed. Every layer copy's
    workspace is checked after the timed replay (a wait that gave up would
    make the results invalid). With `packed` each copy's W is prepared once
    (attnres_pack_weights, outside the timed region, as a layer binds its
    weight when it is prepared) and the step is attnres_oproj_packed_run.
    Returns the workload's figures and inputs."""
    cfg = WORKLOADS[cfg_id]
    M, K, nb, cap, write, has_delta = (cfg[k] for k in ("M", "K", "nb", "cap", "write",
                                                      "has_delta"))
    s = synth.decode_step(M, K, nb, cap=cap, write=write, has_delta=has_delta, final=final,
                          seed=0)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    step_bytes = algorithmic_bytes(M, K, nb, write, has_delta)
    copy_bytes = 2 * H * K + 2 * M * K + M * 2 * H * (4 + cap)
    L = max(2, math.ceil(FOOTPRINT / copy_bytes))
    base = dict(x=up(s.x), W=up(s.W), prefix=up(s.prefix), blocks=up(s.blocks))
    norm, query, out_norm = up(s.norm), up(s.query), up(s.out_norm)
    layers = []
    for i in range(L):
        t = {k: v.clone() for k, v in base.items()}
        if packed:
            t["W"] = sga.attnres_pack_weights(t["W"])
        t["out"] = torch.zeros((M, H), dtype=torch.int16, device=dev)
        t["aux"] = torch.zeros((M, H), dtype=torch.int16, device=dev)
        t["ws"] = sga.make_workspace(M, H, nb, dev)
        layers.append(t)
    del base
    torch.cuda.synchronize()

    def step(i):
        t = layers[i % L]
        if packed:
            sga.attnres_oproj_packed_run(t["x"], t["W"], H, t["prefix"], t["blocks"], norm, query,
                                         out_norm, t["out"], t["aux"], t["ws"], nb=nb,
                                         write=write, has_delta=has_delta, final_boundary=final)
        else:
            sga.attnres_oproj_run(t["x"], t["W"], t["prefix"], t["blocks"], norm, query,
                                  out_norm, t["out"], t["aux"], t["ws"], nb=nb, write=write,
                                  has_delta=has_delta, final_boundary=final)

    if not args.no_check:
        # the first call on copy 0 (fresh inputs) against the oracle: the new
        # prefix within one projection ulp, the output within two bf16 ulps
        # of the oracle's AttnRes on the GPU's own new prefix
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from parity_tools import check_fused_step

        step(0)
        torch.cuda.synchronize()
        sga.check_workspace(layers[0]["ws"])

        def down(t):
            return t.cpu().numpy().view(np.uint16)

        check_fused_step(x=s.x, W=s.W, old_prefix=s.prefix, blocks=s.blocks, norm=s.norm,
                         query=s.query, out_norm=s.out_norm, nb=nb, write=write,
                         has_delta=has_delta, final=final, eps=s.eps, out_eps=s.out_eps,
                         gpu_out=down(layers[0]["out"]), gpu_new=down(layers[0]["prefix"]),
                         what=f"bench config {cfg_id}", nthreads=len(os.sched_getaffinity(0)))

    us_step = graph_time_us(torch, step, args.steps, args.warmup)
    for t in layers:  # every copy: no wait gave up during the timed replays
        sga.check_workspace(t["ws"])
    del layers
    torch.cuda.empty_cache()
    gbs = step_bytes / (us_step * 1e-6) / 1e9
    rec = MEASURED_TRAFFIC.get((cfg_id, "prepared" if packed else "row-major"))
    traffic = None
    if rec is not None and final == 0 and rec["digest"] == kernel_digest():
        traffic = rec["fetch"] + rec["write"]
    fig = {
        "workload": f"fused o-proj + AttnRes, M={M}, K={K}, N=H={H}, nb={nb}, "
                    f"write={write}, has_delta={has_delta}, aux=1, final={final}, "
                    f"W {'prepared (tile-major)' if packed else 'row-major'}",
        "M": M, "K": K, "nb": nb, "write": write, "w_layout": "prepared" if packed else "row-major",
        "us_per_layer_step": round(us_step, 3),
        "achieved_GBs": round(gbs, 1),
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 1),
        "frac": round(gbs / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_launch": step_bytes,
        "traffic": traffic,
        "layer_copies": L, "footprint_MB": round(L * copy_bytes / 1e6, 1),
    }
    return fig, s


def cpu_baseline(args, np, s, cfg_id, final):
    """The FP64 oracle on the same step (copy 0 of the inputs), timed twice on
    the host: one thread, then every core this process may run on (the oracle
    splits the GEMM over output elements and AttnRes over tokens, with the
    same bits either way). Each leg runs for about `--cpu-seconds`."""
    import oracle

    cfg = WORKLOADS[cfg_id]
    M, K, nb, write, has_delta = (cfg[k] for k in ("M", "K", "nb", "write", "has_delta"))
    step_bytes = algorithmic_bytes(M, K, nb, write, has_delta)
    cores = len(os.sched_getaffinity(0))

    def leg(threads):
        times = []
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            oracle.attnres_oproj(s.x, s.W, s.prefix, s.blocks, s.norm, s.query, s.out_norm,
                                 nb=nb, write=write, has_delta=has_delta, final=final,
                                 nthreads=threads)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start >= args.cpu_seconds or len(times) >= 200:
                break
        return float(np.median(times)), len(times)

    t_all, n_all = leg(cores)
    t_one, n_one = leg(1)
    return {
        "value": round(step_bytes / t_all / 1e9, 3),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{n_all} full steps of the headline workload (config {cfg_id}, copy 0) on "
                  f"{cores} threads, median {t_all * 1e3:.2f} ms/step; {n_one} steps on one "
                  f"thread, median {t_one * 1e3:.2f} ms/step; FP64 C oracle (GEMM split over "
                  f"output elements, AttnRes over tokens)",
        "ms_per_step": round(t_all * 1e3, 3),
        "single_thread": {"value": round(step_bytes / t_one / 1e9, 3), "unit": "GB/s",
                          "cores": 1, "ms_per_step": round(t_one * 1e3, 3)},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1, choices=sorted(WORKLOADS) + [3, 4, 5])
    ap.add_argument("--only", action="store_true",
                    help="time only --config (the default run times configs 0, 1 and 2)")
    ap.add_argument("--final", type=int, default=0)
    ap.add_argument("--w-layout", choices=["prepared", "row-major", "both"], default="both",
                    help="W layout of the timed steps (the headline takes the first measured)")
    ap.add_argument("--cpu-seconds", type=float, default=6.0,
                    help="bounded host time per leg of the oracle baseline (0 skips it)")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--stream-read-gb", type=float, default=2.0,
                    help="size of the streaming-read reference measurement (0: skip)")
    ap.add_argument("--calibrate-copy-mb", type=float, default=0.0,
                    help="also run 3 plain device copies of this many MB (for scaling "
                         "HBM byte counters read under a profiler); 0 skips them")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    import skinny_gemm_attention_amd as sga
    import synth

    if args.config in (3, 4, 5):
        side_configs(args, np, torch, sga, synth)
        return

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy_mb > 0:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings give
        # the factor from those counters to bytes
        n = int(args.calibrate_copy_mb * 1e6) // 16 * 16
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    head = args.config
    order = [head] if args.only else [head] + [c for c in sorted(WORKLOADS) if c != head]
    layouts = {"prepared": [True], "row-major": [False], "both": [True, False]}[args.w_layout]
    figs, inputs = {}, {}
    for c in order:
        for pk in layouts:
            figs[(c, pk)], inputs[c] = fused_measure(c, args, np, torch, sga, synth, dev,
                                                     final=args.final, packed=pk)
    f = figs[(head, layouts[0])]
    us_step = f["us_per_layer_step"]
    gbs = f["achieved_GBs"]

    result = {
        "metric": "µs/layer-step + achieved HBM GB/s (% of peak), o-proj+AttnRes, M=1/8/64",
        "value": gbs,
        "unit": "GB/s",
        "us_per_layer_step": us_step,
        "pct_of_hbm_peak": f["pct_of_hbm_peak"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_step / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64 normals, bf16)",
        "config": {
            "workload": f["workload"],
            "M": f["M"], "K": f["K"], "N": H, "nb": f["nb"], "write": f["write"],
            "final": args.final, "layer_copies": f["layer_copies"],
            "footprint_MB": f["footprint_MB"],
            "timing": "one HIP graph of `steps` calls per workload, HIP events on the launch "
                      "stream; every workspace checked after the timed replay",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": f["frac"],
            "traffic": f["traffic"],
            "kernel": ("fused_packed_kernel (attnres_oproj_packed_run on W prepared by attnres_pack_weights)"
                       if f["w_layout"] == "prepared" else "fused_kernel (attnres_oproj_run)")
                      + ", one launch per step",
            "algorithmic_bytes_per_launch": f["algorithmic_bytes_per_launch"],
            "traffic_note": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated); "
                            "null unless measured on these kernel sources",
        },
        "workloads": [figs[k] for k in sorted(figs, key=lambda k: (k[0], not k[1]))],
    }

    if args.stream_read_gb > 0:
        # what a plain 16-byte non-temporal read of HBM reaches on this device
        # (attnres_stream_read), beside the 8 TB/s spec figure
        rd = stream_read_gbs(torch, sga, dev, args.stream_read_gb)
        result["stream_read"] = rd
        result["pct_of_measured_read_bw"] = round(100.0 * gbs / rd["gbs"], 1)
        for w in result["workloads"]:
            w["pct_of_measured_read_bw"] = round(100.0 * w["achieved_GBs"] / rd["gbs"], 1)

    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(args, np, inputs[head], head, args.final)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
