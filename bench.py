"""Benchmark of the bidirectional Mamba state hot path on one MI355X.

One step = one pass of the whole hot path over one decoding block of the 700M-shape
layer (48 heads x 64, d_state 128, ngroups 1, batch 1, bf16 inputs, fp32 state):
  1. bdssm_prefix_scan over the 8192-token prefix (y in bf16, final state),
  2. bdssm_state_ops: that cached state in the block step's operand form,
  3. 64 denoising steps of bdssm_block_step_ops (T = 32, distinct fwd/rev inputs per step)
     against it,
  4. bdssm_commit of the block's clean inputs.
value = active (denoised) tokens per second = steps * 64 * 32 / wall time.

Per-kernel times come from HIP events recorded on the launch stream around every call in
the timed region. The roofline object describes the kernel with the largest share of the
step. Two more workloads are timed the same way and reported under "secondary": the
64-stream running-set block step (T = 128, HBM-bound) and the 65,536-token prefix scan
with per-chunk states (matrix-core-bound). The CPU baseline times the float64 oracle on
the host on one whole step of the same workload.
"""
import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15    # flop/s, dense bf16 matrix cores
METRIC = "block-step active tokens/s + HBM GB/s; prefix-scan tokens/s + MFMA util"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--secondary-only", action="store_true",
                    help="only the 64-stream block step and the 65,536-token prefix scan")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


def src_hash():
    """Hash of the kernel sources with comments and blank lines removed (a comment edit
    leaves the counters valid; any code change invalidates them)."""
    h = hashlib.sha256()
    cdir = os.path.join(ROOT, "bidirectional_mamba_state_amd", "csrc")
    for f in sorted(os.listdir(cdir)):
        text = open(os.path.join(cdir, f), encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
        h.update(f.encode() + b"\0" + "\n".join(lines).encode())
    return h.hexdigest()[:16]


class Timer:
    """HIP events around launches on the current stream; durations read after sync."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def run(self, name, fn):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.pairs.setdefault(name, []).append((a, b))

    def avg_us(self, name):
        ps = self.pairs.get(name, [])
        return 1e3 * sum(a.elapsed_time(b) for a, b in ps) / len(ps) if ps else 0.0

    def total_us(self, name):
        return self.avg_us(name) * len(self.pairs.get(name, []))


def capture(torch, fn):
    """Capture fn() into a HIP graph (after one warm run on a side stream)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def block_step_bytes(b, H, P, N, G, T, in_bytes, y_bytes):
    state = b * H * N * P * 4
    inputs = 2 * b * T * (H * P + H + 2 * G * N) * in_bytes + 2 * H * 4
    return state + inputs + b * T * H * P * y_bytes


def commit_bytes(b, H, P, N, G, T, in_bytes):
    return 2 * b * H * N * P * 4 + b * T * (H * P + H + G * N) * in_bytes + 2 * H * 4


def prefix_bytes(b, H, P, N, G, L, Q, in_bytes, y_bytes, chunk_states):
    nch = -(-L // Q)
    io = b * L * (H * P + H + 2 * G * N) * in_bytes + b * L * H * P * y_bytes
    return io + b * H * N * P * 4 + (b * nch * H * N * P * 4 if chunk_states else 0)


def prefix_state_bytes(b, H, P, N, G, L, in_bytes):
    """State-only prefix scan: x, dt and B read once, the final state written once, A and D."""
    return b * L * (H * P + G * N + H) * in_bytes + b * H * N * P * 4 + 2 * H * 4


def prefix_flops(b, H, P, N, G, L, Q):
    """Dense matrix-form flops of the chunked scan: per chunk and head, C.B^T (shared by
    the H/G heads of a group), the masked (Q x Q)(Q x P) product, the chunk state
    B^T (Q x P) and the state-to-output product C (N x P)."""
    nch = -(-L // Q)
    hpg = H // G
    per = 2 * Q * Q * N / hpg + 2 * Q * Q * P + 2 * Q * N * P + 2 * Q * N * P
    return b * nch * H * per


def make_roofline(kind, work, avg_us, traffic=None):
    if kind == "hbm":
        ach = work / (avg_us * 1e-6) / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": round(ach / (HBM_PEAK / 1e9), 4), "traffic": traffic}
    ach = work / (avg_us * 1e-6) / 1e12
    return {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK / 1e12,
            "unit": "TFLOP/s", "frac": round(ach / (MFMA_BF16_PEAK / 1e12), 4), "traffic": traffic}


def traffic_for(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken on
    the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    e = d.get(kernel)
    if not e or e.get("src_hash") != src_hash():
        return None
    return e.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this hot path has no multi-GPU mode "
              "(streams or heads would shard with no exchange); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from bidirectional_mamba_state_amd import bdssm, configs, inputs

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = 1 << 28
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n * 4, "bytes_written": n * 4}))
        return

    bdssm.load()
    if args.secondary_only:
        print(json.dumps({"secondary": secondary(torch, np, bdssm, configs, inputs)}), flush=True)
        return
    cfg = configs.get(1)
    b, H, P, N, G, L, Q, T = (cfg.batch, cfg.nheads, cfg.headdim, cfg.d_state, cfg.ngroups,
                              cfg.prefix_len, cfg.chunk, cfg.block_len)
    S = cfg.steps_per_block
    A, D = inputs.params(cfg)
    d = bdssm.dims(b, H, P, N, G, cfg.in_dtype, bdssm.BF16)
    Ad, Dd = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    pre_np = inputs.prefix(cfg)
    pre = bdssm.seq_to_device(pre_np)
    steps_np = [(inputs.block(cfg, 0, s, inputs.FWD), inputs.block(cfg, 0, s, inputs.REV)) for s in range(S)]
    steps = [(bdssm.seq_to_device(f), bdssm.seq_to_device(r)) for f, r in steps_np]
    clean_np = inputs.block(cfg, 0, 0, inputs.CLEAN)
    clean = bdssm.seq_to_device(clean_np)
    h = torch.empty((b, H, N, P), device="cuda")
    h_ops = torch.empty(bdssm.state_ops_bytes(d), dtype=torch.uint8, device="cuda")
    y_pre = torch.empty((b, L, H, P), dtype=torch.bfloat16, device="cuda")
    y_blk = [torch.empty((b, T, H, P), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    wsb = bdssm.prefix_scan_workspace(d, L, Q, True, False)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")

    def run_prefix():
        bdssm.prefix_scan(d, L, Q, pre, Ad, Dd, None, y_pre, None, h, ws, wsb)

    def run_state_ops():
        bdssm.state_ops(d, h, h_ops)

    def run_blocks():
        for s in range(S):
            f, r = steps[s]
            bdssm.block_step_ops(d, T, h_ops, f, r, Ad, Dd, y_blk[s])

    def run_blocks_fp32_state():
        for s in range(S):
            f, r = steps[s]
            bdssm.block_step(d, T, h, f, r, Ad, Dd, y_blk[s])

    def run_commit():
        bdssm.commit(d, T, clean, Ad, Dd, h)

    parts = (("prefix_scan", run_prefix), ("state_ops", run_state_ops), ("block_step", run_blocks),
             ("commit", run_commit))
    for _ in range(args.warmup):
        for _, fn in parts:
            fn()
    torch.cuda.synchronize()

    # A step is one HIP graph replay of the whole path (prefix scan, operand form of the
    # state, the 64 block steps, the commit), so launch overhead is off the clock, as in the
    # pages' own graph-captured decoding measurements; `value` and `ms_per_step` time exactly
    # K replays. The parts are then timed on their own: the same work as one graph per part,
    # with HIP events between the replays on the launch stream; the block-step average
    # includes the gaps between the 64 back-to-back launches of its graph.
    def run_all():
        for _, fn in parts:
            fn()

    whole = capture(torch, run_all)
    for _ in range(2):
        whole.replay()
    torch.cuda.synchronize()
    e_all = [torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
    t0 = time.perf_counter()
    e_all[0].record()
    for i in range(args.steps):
        whole.replay()
        print(f"[bench] step {i + 1}/{args.steps}", file=sys.stderr, flush=True)
    e_all[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms_per_step = e_all[0].elapsed_time(e_all[1]) / args.steps
    del whole

    graphs = [capture(torch, fn) for _, fn in parts]
    names = [k for k, _ in parts]
    ev = []
    torch.cuda.synchronize()
    for i in range(args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)]
        e[0].record()
        for g, en in zip(graphs, e[1:]):
            g.replay()
            en.record()
        ev.append(e)
    torch.cuda.synchronize()
    per_step = {"prefix_scan": 1, "state_ops": 1, "block_step": S, "commit": 1}
    part_ms = {k: sum(e[j].elapsed_time(e[j + 1]) for e in ev) / args.steps for j, k in enumerate(names)}
    parts_ms = sum(e[0].elapsed_time(e[len(parts)]) for e in ev) / args.steps
    avg_us = {k: 1e3 * part_ms[k] / per_step[k] for k in part_ms}
    del graphs
    fp32_state_us = graph_us(torch, run_blocks_fp32_state) / S
    timing = ("one HIP graph replay per step (prefix scan, state operand form, 64 block steps, commit); "
              "per-part times from the same work as one graph per part with HIP events between them on "
              "the launch stream")
    ms_per_step = 1e3 * wall / args.steps
    active = args.steps * S * b * T
    value = active / wall

    ib, yb = 2, 2
    k_bytes = {"block_step": block_step_bytes(b, H, P, N, G, T, ib, yb),
               "state_ops": 2 * b * H * N * P * 4,
               "commit": commit_bytes(b, H, P, N, G, T, ib),
               "prefix_scan": prefix_bytes(b, H, P, N, G, L, Q, ib, yb, False)}
    pf = prefix_flops(b, H, P, N, G, L, Q)
    breakdown = {}
    for k in names:
        us = avg_us[k]
        breakdown[k] = {"launches_per_step": per_step[k], "avg_us": round(us, 3),
                        "share_of_step": round(part_ms[k] / parts_ms, 4),
                        "alg_bytes": k_bytes[k],
                        "hbm_frac": round(k_bytes[k] / (us * 1e-6) / HBM_PEAK, 4)}
    breakdown["prefix_scan"]["tokens_per_s"] = round(b * L / (avg_us["prefix_scan"] * 1e-6), 1)
    breakdown["prefix_scan"]["mfma_frac"] = round(pf / (avg_us["prefix_scan"] * 1e-6) / MFMA_BF16_PEAK, 5)
    breakdown["block_step"]["active_tokens_per_s"] = round(b * T / (avg_us["block_step"] * 1e-6), 1)
    breakdown["block_step"]["from_fp32_state_us"] = round(fp32_state_us, 3)
    dom = max(part_ms, key=part_ms.get)
    if dom == "prefix_scan":
        roof = make_roofline("mfma", pf, avg_us[dom], traffic_for(dom))
    else:
        roof = make_roofline("hbm", k_bytes[dom], avg_us[dom], traffic_for(dom))
    roof["kernel"] = dom
    roof["work_per_launch"] = pf if dom == "prefix_scan" else k_bytes[dom]

    out = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "gpu_ms_per_step": round(gpu_ms_per_step, 4),
           "timing": timing,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded; random-init layer parameters)",
           "config": {"workload": "700M-shape Mamba-2 layer, 48 heads x 64, d_state 128, ngroups 1, "
                                  "batch 1, bf16 inputs, fp32 state: 8192-token prefix scan + "
                                  "state operand form + 64 block steps (T=32) + commit per step",
                      "global_batch": b, "seq_len": L, "block_len": T, "steps_per_block": S,
                      "parallelism": "none (1 GPU)"},
           "roofline": roof, "breakdown": breakdown}

    # the same 64 block steps + commit (+ the operand form of the advanced state) through the
    # library's decode-loop graph (one HIP graph recorded by bdssm_decode_graph_create),
    # timed per replay
    dg = bdssm.DecodeGraph(d, T, h, [f for f, _ in steps], [r for _, r in steps], Ad, Dd, y_blk, clean,
                           h_ops=h_ops)
    for _ in range(2):
        dg.launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        dg.launch()
    e1.record()
    torch.cuda.synchronize()
    blk_us = 1e3 * e0.elapsed_time(e1) / reps
    dg.close()
    out["decode_graph"] = {"workload": "bdssm_decode_graph: 64 block steps (T=32) + commit of one block "
                                       "+ operand form of the advanced state, 700M shape, replayed back "
                                       "to back",
                           "us_per_block": round(blk_us, 2), "us_per_launch": round(blk_us / (S + 2), 3),
                           "active_tokens_per_s": round(S * b * T / (blk_us * 1e-6), 1)}

    if not args.no_secondary:
        out["conv_state"] = conv_workloads(torch, bdssm, cfg, inputs, d, h, steps, Ad, Dd, y_blk, pre, L,
                                           fp32_state_us)
        out["secondary"] = secondary(torch, np, bdssm, configs, inputs)
        out["extra"] = extra(torch, np, bdssm, configs, inputs)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(np, cfg, A, D, pre_np, steps_np, clean_np)
    print(json.dumps(out), flush=True)


def conv_bytes(b, H, P, N, G, L, W, in_bytes, state):
    ch = H * P + 2 * G * N
    return 2 * b * L * ch * in_bytes + ch * (W + 1) * 4 + (2 * b * (W - 1) * ch * in_bytes if state else 0)


def conv_workloads(torch, bdssm, cfg, inputs, d, h, steps, Ad, Dd, y_blk, pre, L, plain_step_us, reps=20):
    """The convolution state at the 700M shape (width 4, SiLU): the 64 block steps through
    bdssm_block_step_conv (both directions' convolutions in one launch, then the block step),
    captured in one graph like the main step, and the forward convolution of the 8192-token
    prefix that writes the conv state (HBM-bound)."""
    b, H, P, N, G, T = cfg.batch, cfg.nheads, cfg.headdim, cfg.d_state, cfg.ngroups, cfg.block_len
    W = 4
    ch = H * P + 2 * G * N
    wf, bf = (torch.from_numpy(a).cuda() for a in inputs.conv_params(cfg, W, inputs.FWD))
    wr, br = (torch.from_numpy(a).cuda() for a in inputs.conv_params(cfg, W, inputs.REV))
    cpf, cpr = bdssm.conv_params(wf, bf, 1), bdssm.conv_params(wr, br, 1)
    cs = torch.zeros((b, W - 1, ch), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(2 * bdssm.conv_workspace(d, T), dtype=torch.uint8, device="cuda")
    S = len(steps)

    def run_steps():
        for s in range(S):
            f, r = steps[s]
            bdssm.block_step_conv(d, T, cpf, cpr, h, cs, f, r, Ad, Dd, y_blk[s], ws)

    g = capture(torch, run_steps)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    tm = Timer(torch)
    for _ in range(reps):
        tm.run("k", g.replay)
    torch.cuda.synchronize()
    step_us = tm.avg_us("k") / S
    post = tuple(torch.empty_like(t) for t in pre)
    cso = torch.empty_like(cs)
    tm = Timer(torch)
    for i in range(reps + 3):
        (tm if i >= 3 else Timer(torch)).run("c", lambda: bdssm.conv(d, L, cpf, False, None, pre, post, cso))
    torch.cuda.synchronize()
    conv_us = tm.avg_us("c")
    nb = conv_bytes(b, H, P, N, G, L, W, 2, True)
    return {"block_step_conv": {"workload": "64 block steps (T=32) on unconvolved inputs, width-4 SiLU "
                                            "convolution of x, B, C per direction, 700M shape, one graph",
                                "us_per_step": round(step_us, 3), "plain_block_step_us": round(plain_step_us, 3),
                                "active_tokens_per_s": round(b * T / (step_us * 1e-6), 1)},
            "prefix_conv": {"workload": "forward convolution of an 8192-token prefix (x, B, C; width 4, "
                                        "SiLU) writing the conv state, 700M shape, bf16",
                            "avg_us": round(conv_us, 3), "alg_bytes": nb,
                            "roofline": make_roofline("hbm", nb, conv_us, None)}}


def prefix_flops_causal(b, H, P, N, G, L, Q):
    """As prefix_flops, counting only the causal half (s <= t) of the quadratic products."""
    nch = -(-L // Q)
    hpg = H // G
    tri = Q * (Q + 1) / 2
    per = 2 * tri * N / hpg + 2 * tri * P + 2 * Q * N * P + 2 * Q * N * P
    return b * nch * H * per


def graph_us(torch, fn, reps=10, warm=2):
    """Average time of fn() captured as one HIP graph, replayed `reps` times (HIP events)."""
    g = capture(torch, fn)
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / reps


def extra(torch, np, bdssm, configs, inputs):
    """The remaining figures of the measurement plan: the block step as a single launch
    (median of 20 after 5 warm-ups), with every buffer cold (rotation over more than the
    256 MiB last-level cache) and cache-resident, at configs 0 and 3; the state-only prefix
    builds of configs 3 and 4; the commit chain."""
    res = {}
    c1 = configs.get(1)
    b, H, P, N, G, T = c1.batch, c1.nheads, c1.headdim, c1.d_state, c1.ngroups, c1.block_len
    A, D = inputs.params(c1)
    Ad, Dd = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    d = bdssm.dims(b, H, P, N, G, c1.in_dtype, bdssm.BF16)
    f = bdssm.seq_to_device(inputs.block(c1, 0, 0, inputs.FWD))
    r = bdssm.seq_to_device(inputs.block(c1, 0, 0, inputs.REV))
    def ops_of(dd, hh):
        o = torch.empty(bdssm.state_ops_bytes(dd), dtype=torch.uint8, device="cuda")
        bdssm.state_ops(dd, hh, o)
        return o

    h = ops_of(d, torch.randn((b, H, N, P), device="cuda") * 0.05)
    y = torch.empty((b, T, H, P), dtype=torch.bfloat16, device="cuda")
    ts = []
    for i in range(25):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        bdssm.block_step_ops(d, T, h, f, r, Ad, Dd, y)
        e1.record()
        torch.cuda.synchronize()
        if i >= 5:
            ts.append(1e3 * e0.elapsed_time(e1))
    res["block_step_single_launch"] = {"workload": "700M shape, T=32, state in operand form, one launch "
                                                   "between synchronizations",
                                       "median_us": round(float(np.median(ts)), 3)}
    # cold: 256 sets of (state, inputs, y), about 540 MB, one launch each; warm: one set
    nset = 256
    sets = []
    for k in range(nset):
        sets.append((ops_of(d, torch.randn((b, H, N, P), device="cuda") * 0.05),
                     tuple(t.clone() for t in f), tuple(t.clone() for t in r),
                     torch.empty_like(y)))
    cold = graph_us(torch, lambda: [bdssm.block_step_ops(d, T, hh, ff, rr, Ad, Dd, yy) for hh, ff, rr, yy in sets]) / nset
    warm = graph_us(torch, lambda: [bdssm.block_step_ops(d, T, h, f, r, Ad, Dd, y) for _ in range(nset)]) / nset
    nb = block_step_bytes(b, H, P, N, G, T, 2, 2)
    res["block_step_cold_warm"] = {"workload": "700M shape, T=32, state in operand form, 256 launches in one graph",
                                   "cold_us": round(cold, 3), "warm_us": round(warm, 3),
                                   "rotation_bytes": nset * nb}
    del sets
    # configs 3 and 0: 64 (resp. 4) steps with distinct inputs in one graph
    for ci in (3, 0):
        c = configs.get(ci)
        b, H, P, N, G, T = c.batch, c.nheads, c.headdim, c.d_state, c.ngroups, c.block_len
        A, D = inputs.params(c)
        Ad3, Dd3 = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
        yd = bdssm.BF16 if c.in_dtype == 1 else bdssm.F32
        d3 = bdssm.dims(b, H, P, N, G, c.in_dtype, yd)
        S = c.steps_per_block
        st = [(bdssm.seq_to_device(inputs.block(c, 0, k, inputs.FWD)), bdssm.seq_to_device(inputs.block(c, 0, k, inputs.REV)))
              for k in range(S)]
        hh = torch.randn((b, H, N, P), device="cuda") * 0.05
        ys = [torch.empty((b, T, H, P), dtype=torch.bfloat16 if yd == bdssm.BF16 else torch.float32, device="cuda")
              for _ in range(S)]
        if bdssm.state_ops_bytes(d3) != ctypes.c_size_t(-1).value and c.in_dtype == 1:
            ho = ops_of(d3, hh)   # the operand form where the shape has one
            us = graph_us(torch, lambda: [bdssm.block_step_ops(d3, T, ho, ff, rr, Ad3, Dd3, yy)
                                          for (ff, rr), yy in zip(st, ys)]) / S
        else:
            us = graph_us(torch, lambda: [bdssm.block_step(d3, T, hh, ff, rr, Ad3, Dd3, yy)
                                          for (ff, rr), yy in zip(st, ys)]) / S
        ib = 2 if c.in_dtype == 1 else 4
        nb = block_step_bytes(b, H, P, N, G, T, ib, ib)
        res[f"block_step_config{ci}"] = {"workload": c.name, "us_per_step": round(us, 3),
                                         "active_tokens_per_s": round(b * T / (us * 1e-6), 1),
                                         "hbm_frac": round(nb / (us * 1e-6) / HBM_PEAK, 4), "alg_bytes": nb}
    # state-only prefix builds of configs 3 and 4 (the long-context cache: 262,144 tokens x
    # 80 heads; the running set's caches: 64 streams x 32,768 tokens x 48 heads). Inputs of
    # the configs' shapes and distributions drawn on the device (values do not change the
    # time; the seeded host generator would take minutes at 3-14 GB)
    for ci in (3, 4):
        c = configs.get(ci)
        b, H, P, N, G, L, Q = c.batch, c.nheads, c.headdim, c.d_state, c.ngroups, c.prefix_len, c.chunk
        A, D = inputs.params(c)
        Adv, Ddv = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
        gen = torch.Generator(device="cuda")
        gen.manual_seed(ci)
        x = torch.empty((b, L, H, P), dtype=torch.bfloat16, device="cuda")
        for k in range(b):  # one stream at a time keeps the float32 temporary small
            x[k] = torch.randn((L, H, P), device="cuda", generator=gen).to(torch.bfloat16)
        Bv = (0.25 * torch.randn((b, L, G, N), device="cuda", generator=gen)).to(torch.bfloat16)
        dt = torch.nn.functional.softplus(torch.randn((b, L, H), device="cuda", generator=gen) - 4.0)
        dt = dt.clamp(1e-3, 0.1).to(torch.bfloat16)
        dv = bdssm.dims(b, H, P, N, G, 1, bdssm.BF16)
        hv = torch.empty((b, H, N, P), device="cuda")
        wsb = bdssm.prefix_scan_workspace(dv, L, Q, False, False)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
        seq = (x, dt, Bv, None)
        tm = Timer(torch)
        for i in range(7):
            (tm if i >= 2 else Timer(torch)).run("p", lambda: bdssm.prefix_scan(dv, L, Q, seq, Adv, Ddv, None, None,
                                                                                 None, hv, ws, wsb))
        torch.cuda.synchronize()
        us = tm.avg_us("p")
        nb = prefix_state_bytes(b, H, P, N, G, L, 2)
        res[f"prefix_build_config{ci}"] = {"workload": f"state-only prefix scan, {c.name}, {b} x {L} tokens",
                                           "avg_us": round(us, 1), "prefix_tokens_per_s": round(b * L / (us * 1e-6), 1),
                                           "hbm_frac": round(nb / (us * 1e-6) / HBM_PEAK, 4), "alg_bytes": nb,
                                           "data": "device-generated, same shapes and distributions"}
        del x, Bv, dt, hv, ws, seq
        torch.cuda.empty_cache()
    # commit chain, config 2: 2048 commits of 32 tokens over the 65,536-token prefix
    c2 = configs.get(2)
    b, H, P, N, G, L, T = c2.batch, c2.nheads, c2.headdim, c2.d_state, c2.ngroups, c2.prefix_len, c2.commit_len
    A, D = inputs.params(c2)
    Ad2, Dd2 = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    d2 = bdssm.dims(b, H, P, N, G, c2.in_dtype, bdssm.BF16)
    pre = bdssm.seq_to_device(inputs.prefix(c2))
    blocks = [tuple(t[:, k * T:(k + 1) * T].contiguous() for t in pre) for k in range(L // T)]
    hc = torch.zeros((b, H, N, P), device="cuda")
    us = graph_us(torch, lambda: [bdssm.commit(d2, T, blk, Ad2, Dd2, hc) for blk in blocks], reps=3, warm=1)
    res["commit_chain_config2"] = {"workload": "2,048 commits of 32 tokens (350M shape), one graph",
                                   "us_per_commit": round(us / len(blocks), 3),
                                   "tokens_per_s": round(L / (us * 1e-6), 1)}
    return res


def secondary(torch, np, bdssm, configs, inputs, reps=20):
    res = []
    # 64-stream running set: T = 128, the cached fp32 state per stream in operand form (made
    # once per commit, i.e. once per 16 steps of this workload; its time is reported beside);
    # values do not affect timing: the state is drawn at random, inputs from the seeded
    # generator
    c4 = configs.get(4)
    b, H, P, N, G, T = c4.batch, c4.nheads, c4.headdim, c4.d_state, c4.ngroups, c4.block_len
    A, D = inputs.params(c4)
    Ad, Dd = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    d = bdssm.dims(b, H, P, N, G, c4.in_dtype, bdssm.BF16)
    h = torch.randn((b, H, N, P), device="cuda") * 0.05
    ops = torch.empty(bdssm.state_ops_bytes(d), dtype=torch.uint8, device="cuda")
    bdssm.state_ops(d, h, ops)
    f = bdssm.seq_to_device(inputs.block(c4, 0, 0, inputs.FWD))
    r = bdssm.seq_to_device(inputs.block(c4, 0, 0, inputs.REV))
    y = torch.empty((b, T, H, P), dtype=torch.bfloat16, device="cuda")
    tm = Timer(torch)
    for name, fn in (("k", lambda: bdssm.block_step_ops(d, T, ops, f, r, Ad, Dd, y)),
                     ("f32", lambda: bdssm.block_step(d, T, h, f, r, Ad, Dd, y)),
                     ("ops", lambda: bdssm.state_ops(d, h, ops))):
        for i in range(reps + 3):  # each kernel back to back with itself
            (tm if i >= 3 else Timer(torch)).run(name, fn)
    torch.cuda.synchronize()
    us = tm.avg_us("k")
    nb = block_step_bytes(b, H, P, N, G, T, 2, 2)
    res.append({"workload": "block step, 700M shape x 64 streams, running set T=128, bf16 in/out, "
                            "cached state in operand form",
                "avg_us": round(us, 3), "active_tokens_per_s": round(b * T / (us * 1e-6), 1),
                "roofline": make_roofline("hbm", nb, us, traffic_for("block_step_c4")),
                "alg_bytes": nb, "from_fp32_state_us": round(tm.avg_us("f32"), 3),
                "state_ops_us": round(tm.avg_us("ops"), 3)})
    del h, ops, f, r, y
    # 350M prefix: 65,536 tokens, chunk 256, bf16 y + fp32 chunk states
    c2 = configs.get(2)
    b, H, P, N, G, L, Q = c2.batch, c2.nheads, c2.headdim, c2.d_state, c2.ngroups, c2.prefix_len, c2.chunk
    A, D = inputs.params(c2)
    Ad, Dd = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    d = bdssm.dims(b, H, P, N, G, c2.in_dtype, bdssm.BF16)
    pre = bdssm.seq_to_device(inputs.prefix(c2))
    y = torch.empty((b, L, H, P), dtype=torch.bfloat16, device="cuda")
    cs = torch.empty((b, -(-L // Q), H, N, P), device="cuda")
    ho = torch.empty((b, H, N, P), device="cuda")
    wsb = bdssm.prefix_scan_workspace(d, L, Q, True, True)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    tm = Timer(torch)
    for i in range(8):
        (tm if i >= 2 else Timer(torch)).run(
            "k", lambda: bdssm.prefix_scan(d, L, Q, pre, Ad, Dd, None, y, cs, ho, ws, wsb))
    torch.cuda.synchronize()
    us = tm.avg_us("k")
    fl = prefix_flops(b, H, P, N, G, L, Q)
    nb = prefix_bytes(b, H, P, N, G, L, Q, 2, 2, True)
    res.append({"workload": "prefix scan, 350M shape, 65,536 tokens, chunk 256, bf16 y + fp32 chunk states",
                "avg_us": round(us, 3), "prefix_tokens_per_s": round(b * L / (us * 1e-6), 1),
                "roofline": make_roofline("mfma", fl, us, traffic_for("prefix_scan_c2")),
                "mfma_frac_causal_count": round(prefix_flops_causal(b, H, P, N, G, L, Q) / (us * 1e-6) / MFMA_BF16_PEAK, 4),
                "hbm_frac": round(nb / (us * 1e-6) / HBM_PEAK, 4), "alg_bytes": nb, "flops": fl})
    return res


def cpu_baseline(np, cfg, A, D, pre_np, steps_np, clean_np):
    """The float64 oracle on the host cores, one whole step of the same workload."""
    import oracle
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    _, _, h = oracle.scan(pre_np, A, D, cfg.chunk, want_y=True, want_chunk_states=False)
    hf = h.astype(np.float32).astype(np.float64)
    for f, r in steps_np:
        oracle.block_step(hf, f, r, A, D)
    oracle.commit(hf, clean_np, A, D)
    wall = time.perf_counter() - t0
    active = cfg.steps_per_block * cfg.batch * cfg.block_len
    return {"value": round(active / wall, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "one whole step (8192-token prefix scan with y, 64 block steps, commit) of the "
                      f"same workload; {wall:.2f} s of host time"}


if __name__ == "__main__":
    main()
