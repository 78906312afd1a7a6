"""Benchmark of the bidirectional Mamba state hot path on one MI355X.

Headline workload: the 64-stream running set of the 700M-shape layer (48 heads x 64,
d_state 128, ngroups 1, bf16 inputs, fp32 state). Each stream has its own cached state,
built by a state-only prefix scan over its own 32,768 tokens. One step is one block cycle
of the running set:
  1. 16 denoising steps of bdssm_block_step_ops over the running set of four 32-token blocks
     (T = 128, distinct fwd/rev inputs per step), from the cached states in operand form,
  2. bdssm_commit_refresh of the oldest 32-token block of every stream (its clean inputs):
     the states advance and their operand form for the next cycle's steps is written in the
     same pass.
The step is captured as one HIP graph and replayed; value = active (denoised) tokens per
second = 16 * 64 * 128 per step / wall time. The 64 x 32,768-token prefix build (and the
first operand form of its states) is timed as its own part: once per context, not per
block.

The parts are also timed on their own (each as its own graph, warmed before timing, median
over replays), and the dominant kernel's launches one by one with HIP events on the launch
stream: the roofline object describes that kernel. Secondary lines: the 700M batch-1 block
cycle (prefix + 64 steps + commit), the 65,536-token prefix scan with chunk states (the
matrix-core target), the long-context builds, the decode graph, the convolution state. The
CPU baseline times the float64 oracle on the host on a bounded sample of the headline step.

Inputs are seeded synthetic draws with the workload's distributions (x ~ N(0,1);
B, C ~ N(0,1/16); dt = softplus(N(-4,1)) clipped to [1e-3, 0.1]; rounded to bf16), drawn on
the device for the multi-GB tensors and by the seeded host generator elsewhere; values do
not change the time.
"""
import argparse
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
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed replays of the step's graph before the timed ones (the clock "
                         "ramps up over the first ~20 ms of work after the host-side set-up)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--only", choices=("headline", "c0", "c1", "c2prefix", "builds", "fullwindow", "step4",
                                       "build4", "build3"),
                    help="run one workload only (for profiler runs); step4: the running set's step "
                         "(16 block steps + commit) on a seeded cached state, no prefix build; build4, "
                         "build3: the running set's / the long-context cache's prefix build alone")
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


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


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


def warmed(torch, g, warm=2, min_ms=20.0):
    """Replays g at least `warm` times and for at least min_ms of wall time (the clock ramps
    up over the first tens of milliseconds of work after an idle spell)."""
    t0 = time.perf_counter()
    n = 0
    while n < warm or 1e3 * (time.perf_counter() - t0) < min_ms:
        g.replay()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return g


def replay_times_us(torch, g, reps):
    """Per-replay durations (HIP events on the current stream), after the caller warmed g."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return [1e3 * ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]


def launch_times_us(torch, fns, reps=1):
    """Durations of individual launches enqueued back to back on the current stream, one HIP
    event between each: per fn, the list over reps."""
    out = [[] for _ in fns]
    for _ in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
        ev[0].record()
        for i, fn in enumerate(fns):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        for i in range(len(fns)):
            out[i].append(1e3 * ev[i].elapsed_time(ev[i + 1]))
    return out


def graph_us(torch, fn, reps=10, warm=2):
    """Median time of fn() captured as one HIP graph, warmed, replayed `reps` times."""
    g = warmed(torch, capture(torch, fn), warm)
    return median(replay_times_us(torch, g, reps))


# ---------------------------------------------------------------- algorithmic work
def block_step_bytes(b, H, P, N, G, T, in_bytes, y_bytes):
    state = b * H * N * P * 4
    inputs = 2 * b * T * (H * P + H + 2 * G * N) * in_bytes + 2 * H * 4
    return state + inputs + b * T * H * P * y_bytes


def commit_bytes(b, H, P, N, G, T, in_bytes):
    """State read and written, the clean block's x, dt and B, and A (a commit writes no y, so
    neither C nor D is read)."""
    return 2 * b * H * N * P * 4 + b * T * (H * P + H + G * N) * in_bytes + H * 4


def state_ops_bytes(b, H, P, N):
    return 2 * b * H * N * P * 4


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


def prefix_flops_causal(b, H, P, N, G, L, Q):
    """As prefix_flops, counting only the causal half (s <= t) of the quadratic products."""
    nch = -(-L // Q)
    hpg = H // G
    tri = Q * (Q + 1) / 2
    per = 2 * tri * N / hpg + 2 * tri * P + 2 * Q * N * P + 2 * Q * N * P
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


# ---------------------------------------------------------------- inputs on the device
def dev_seq(torch, gen, b, L, H, P, G, N, with_c=True, chunk_streams=4):
    """Seeded draws of one segment on the device with the workload's distributions, rounded
    to bf16 (torch's conversion rounds to nearest even); drawn a few streams at a time so
    that the float32 temporaries stay small."""
    bf = torch.bfloat16
    x = torch.empty((b, L, H, P), dtype=bf, device="cuda")
    dt = torch.empty((b, L, H), dtype=bf, device="cuda")
    B = torch.empty((b, L, G, N), dtype=bf, device="cuda")
    C = torch.empty((b, L, G, N), dtype=bf, device="cuda") if with_c else None
    for s0 in range(0, b, chunk_streams):
        s1 = min(b, s0 + chunk_streams)
        n = s1 - s0
        x[s0:s1] = torch.randn((n, L, H, P), device="cuda", generator=gen).to(bf)
        z = torch.randn((n, L, H), device="cuda", generator=gen) - 4.0
        dt[s0:s1] = torch.nn.functional.softplus(z).clamp(1e-3, 0.1).to(bf)
        B[s0:s1] = (0.25 * torch.randn((n, L, G, N), device="cuda", generator=gen)).to(bf)
        if with_c:
            C[s0:s1] = (0.25 * torch.randn((n, L, G, N), device="cuda", generator=gen)).to(bf)
    return (x, dt, B, C)


# ---------------------------------------------------------------- headline: config 4
def step4(torch, bdssm, configs, inputs, reps=3):
    """The running set's step alone, for counter runs (each dispatch is then serialized and
    counted, so the prefix build's input draws are left out): the cached state is seeded
    random, put in operand form; 16 block steps (T = 128) and the commit of the oldest 32
    tokens, reps times, each call on its own."""
    cfg = configs.get(4)
    b, H, P, N, G = cfg.batch, cfg.nheads, cfg.headdim, cfg.d_state, cfg.ngroups
    T, S, TC = cfg.block_len, cfg.steps_per_block, cfg.commit_len
    A, D = inputs.params(cfg)
    Ad, Dd = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    d = bdssm.dims(b, H, P, N, G, cfg.in_dtype, bdssm.BF16)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(44)
    h = torch.randn((b, H, N, P), device="cuda", generator=gen) * 0.05
    ops = torch.empty(bdssm.state_ops_bytes(d), dtype=torch.uint8, device="cuda")
    bdssm.state_ops(d, h, ops)
    steps = [(dev_seq(torch, gen, b, T, H, P, G, N, chunk_streams=b), dev_seq(torch, gen, b, T, H, P, G, N, chunk_streams=b))
             for _ in range(S)]
    clean = dev_seq(torch, gen, b, TC, H, P, G, N, with_c=False, chunk_streams=b)
    y = torch.empty((b, T, H, P), dtype=torch.bfloat16, device="cuda")
    fns = [(lambda f=f, r=r: bdssm.block_step_ops(d, T, ops, f, r, Ad, Dd, y)) for f, r in steps]
    fns.append(lambda: bdssm.commit_refresh(d, TC, clean, Ad, Dd, h, ops, bdssm.STATE_OPS))
    t = launch_times_us(torch, fns, reps=reps)
    return {"workload": "running set step: 64 streams x 48 heads, 16 block steps (T=128) + commit of 32 tokens",
            "block_step_us": round(median([x for v in t[:-1] for x in v]), 3),
            "commit_refresh_us": round(median(t[-1]), 3)}


def build_only(torch, bdssm, configs, inputs, index, reps=3):
    """A state-only prefix build alone, reps times, for counter runs: the running set's
    (config 4: 64 streams x 32,768 tokens) or the long-context cache's (config 3: 262,144
    tokens x 80 heads)."""
    cfg = configs.get(index)
    b, H, P, N, G, L, Q = cfg.batch, cfg.nheads, cfg.headdim, cfg.d_state, cfg.ngroups, cfg.prefix_len, cfg.chunk
    A, D = inputs.params(cfg)
    Ad, Dd = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    d = bdssm.dims(b, H, P, N, G, cfg.in_dtype, bdssm.BF16)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(40 + index)
    pre = dev_seq(torch, gen, b, L, H, P, G, N, with_c=False, chunk_streams=4 if b > 1 else 1)
    h = torch.empty((b, H, N, P), device="cuda")
    wsb = bdssm.prefix_scan_workspace(d, L, Q, False, False)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    fn = lambda: bdssm.prefix_scan(d, L, Q, pre, Ad, Dd, None, None, None, h, ws, wsb)
    t = launch_times_us(torch, [fn], reps=reps)[0]
    return {"workload": f"state-only prefix build, {b} stream(s) x {L:,} tokens, {H} heads x {P}, "
                        f"{G} group(s), d_state {N}",
            "avg_us": round(median(t), 1), "alg_bytes": prefix_state_bytes(b, H, P, N, G, L, 2)}


def headline(args, torch, np, bdssm, configs, inputs):
    cfg = configs.get(4)
    b, H, P, N, G, L, Q = cfg.batch, cfg.nheads, cfg.headdim, cfg.d_state, cfg.ngroups, cfg.prefix_len, cfg.chunk
    T, S, TC = cfg.block_len, cfg.steps_per_block, cfg.commit_len
    A, D = inputs.params(cfg)
    Ad, Dd = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    d = bdssm.dims(b, H, P, N, G, cfg.in_dtype, bdssm.BF16)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)

    # the cached states: a state-only prefix scan over each stream's 32,768 tokens
    print("[bench] headline: drawing the 64 x 32,768-token prefixes on the device", file=sys.stderr, flush=True)
    pre = dev_seq(torch, gen, b, L, H, P, G, N, with_c=False)
    h = torch.empty((b, H, N, P), device="cuda")
    wsb = bdssm.prefix_scan_workspace(d, L, Q, False, False)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")

    def run_prefix():
        bdssm.prefix_scan(d, L, Q, pre, Ad, Dd, None, None, None, h, ws, wsb)

    run_prefix()
    torch.cuda.synchronize()
    pre_us = median(launch_times_us(torch, [run_prefix], reps=5)[0])
    pre_nb = prefix_state_bytes(b, H, P, N, G, L, 2)
    h0 = h.clone()
    del pre
    torch.cuda.empty_cache()

    print("[bench] headline: drawing the running set's inputs", file=sys.stderr, flush=True)
    steps = [(dev_seq(torch, gen, b, T, H, P, G, N), dev_seq(torch, gen, b, T, H, P, G, N)) for _ in range(S)]
    clean = dev_seq(torch, gen, b, TC, H, P, G, N, with_c=False)
    ops = torch.empty(bdssm.state_ops_bytes(d), dtype=torch.uint8, device="cuda")
    ys = [torch.empty((b, T, H, P), dtype=torch.bfloat16, device="cuda") for _ in range(S)]

    def run_ops():
        bdssm.state_ops(d, h, ops)

    run_ops()  # the first cycle's operand form (with the prefix build, once per context)
    step_fns = [(lambda f=f, r=r, y=y: bdssm.block_step_ops(d, T, ops, f, r, Ad, Dd, y))
                for (f, r), y in zip(steps, ys)]

    def run_steps():
        for fn in step_fns:
            fn()

    def run_commit():
        bdssm.commit_refresh(d, TC, clean, Ad, Dd, h, ops, bdssm.STATE_OPS)

    parts = (("block_step", run_steps, S), ("commit_refresh", run_commit, 1))

    def run_all():
        for _, fn, _ in parts:
            fn()

    # the step: one graph replay; `warmup` untimed replays, then exactly K replays on the clock
    whole = capture(torch, run_all)
    for _ in range(args.warmup):
        whole.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        whole.replay()
        print(f"[bench] step {i + 1}/{args.steps}", file=sys.stderr, flush=True)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms_per_step = e0.elapsed_time(e1) / args.steps
    step_med_us = median(replay_times_us(torch, whole, args.steps))
    del whole

    # the parts, each as its own warmed graph (median over replays)
    part_us = {}
    for name, fn, _ in parts:
        g = warmed(torch, capture(torch, fn))
        part_us[name] = median(replay_times_us(torch, g, max(args.steps, 5)))
        del g
    parts_sum = sum(part_us.values())
    if any(v > 1.02 * step_med_us for v in part_us.values()):
        print(f"[bench] inconsistent timing: a part exceeds the whole step ({part_us} vs {step_med_us:.1f} us)",
              file=sys.stderr, flush=True)
        sys.exit(3)

    # cold: the same 16 steps with the cached states rotated over R copies of the operand form
    # (R x 100.7 MB > 512 MiB), so that no state a step reads can still sit in the 256 MB
    # last-level cache from an earlier read; the inputs are distinct per step anyway
    nb_ops_one = bdssm.state_ops_bytes(d)
    R = (512 << 20) // nb_ops_one + 1
    ops_rot = [ops.clone() for _ in range(R)]
    cold_fns = [(lambda f=f, r=r, y=y, o=ops_rot[i % R]: bdssm.block_step_ops(d, T, o, f, r, Ad, Dd, y))
                for i, ((f, r), y) in enumerate(zip(steps, ys))]
    cold_us = graph_us(torch, lambda: [fn() for fn in cold_fns], reps=max(args.steps, 5)) / S
    del ops_rot, cold_fns
    torch.cuda.empty_cache()

    # the dominant kernel's launches one by one (HIP events on the launch stream)
    per_launch = launch_times_us(torch, step_fns, reps=3)
    blk_us = median([t for v in per_launch for t in v])
    ops_us = median(launch_times_us(torch, [run_ops], reps=9)[0])
    h.copy_(h0)
    commit_us = median(launch_times_us(torch, [run_commit], reps=9)[0])
    h.copy_(h0)
    plain_commit_us = median(launch_times_us(torch, [lambda: bdssm.commit(d, TC, clean, Ad, Dd, h)], reps=9)[0])
    h.copy_(h0)

    nb_step = block_step_bytes(b, H, P, N, G, T, 2, 2)
    nb_ops = state_ops_bytes(b, H, P, N)
    nb_commit = commit_bytes(b, H, P, N, G, TC, 2) + nb_ops // 2   # + the operand form written
    nb_all = S * nb_step + nb_commit
    ms_per_step = 1e3 * wall / args.steps
    active = S * b * T
    breakdown = {
        "block_step": {"launches_per_step": S, "graph_us": round(part_us["block_step"], 3),
                       "launch_us": round(blk_us, 3), "alg_bytes": nb_step,
                       "hbm_frac": round(nb_step / (blk_us * 1e-6) / HBM_PEAK, 4),
                       "cold_us": round(cold_us, 3), "cold_hbm_frac": round(nb_step / (cold_us * 1e-6) / HBM_PEAK, 4),
                       "cold_states": R,
                       "active_tokens_per_s": round(b * T / (blk_us * 1e-6), 1)},
        "commit_refresh": {"launches_per_step": 1, "graph_us": round(part_us["commit_refresh"], 3),
                           "launch_us": round(commit_us, 3), "alg_bytes": nb_commit,
                           "hbm_frac": round(nb_commit / (commit_us * 1e-6) / HBM_PEAK, 4),
                           "commit_alone_us": round(plain_commit_us, 3),
                           "operand_form_alone_us": round(ops_us, 3)},
        "parts_sum_us": round(parts_sum, 3), "step_median_us": round(step_med_us, 3),
    }
    shares = {"block_step": S * blk_us, "commit_refresh": commit_us}
    dom = max(shares, key=shares.get)
    work = {"block_step": nb_step, "commit_refresh": nb_commit}[dom]
    avg = {"block_step": blk_us, "commit_refresh": commit_us}[dom]
    kname = {"block_step": "k_block_bw", "commit_refresh": "k_fold1 (state-only walk writing the operand form)"}[dom]
    roof = make_roofline("hbm", work, avg, traffic_for({"block_step": "block_step_c4",
                                                        "commit_refresh": "commit_refresh_c4"}[dom]))
    roof.update({"kernel": kname, "part": dom, "work_per_launch": work, "avg_launch_us": round(avg, 3),
                 "launches_per_step": S if dom == "block_step" else 1})
    if dom == "block_step":
        # the window's 16 steps read the same cached states (100.7 MB), part of which the 256 MB
        # last-level cache still holds from the step before; with the states rotated over
        # more than 512 MiB every byte comes from HBM
        roof.update({"cold_avg_launch_us": round(cold_us, 3),
                     "cold_frac": round(work / (cold_us * 1e-6) / HBM_PEAK, 4),
                     "note": "frac: the workload as it runs (each cached state re-read by the window's 16 "
                             "steps, partly served by the last-level cache); cold_frac: states rotated over "
                             "> 512 MiB, every byte from HBM"})
    out = {"metric": METRIC, "value": round(active / (wall / args.steps), 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "gpu_ms_per_step": round(gpu_ms_per_step, 4),
           "timing": "one HIP graph replay per step (16 block steps, commit of the oldest block with the operand "
                     "form refreshed in the same pass); exactly `steps` replays on the clock; parts timed as their "
                     "own warmed graphs and the kernels launch by launch with HIP events on the launch stream",
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded device draws with the workload's distributions; random-init layer parameters)",
           "config": {"workload": "running set of 64 independent streams, 700M-shape Mamba-2 layer (48 heads x 64, "
                                  "d_state 128, ngroups 1), bf16 inputs, fp32 cached state per stream built from "
                                  "32,768 prefix tokens; one step = 16 block steps of the 4 x 32 = 128-token window "
                                  "+ commit of the oldest 32 tokens (refreshing the states' operand form)",
                      "global_batch": b, "seq_len": L, "block_len": T, "steps_per_block": S, "commit_len": TC,
                      "parallelism": "none (1 GPU)"},
           "roofline": roof, "breakdown": breakdown,
           "step_hbm_frac": round(nb_all / (step_med_us * 1e-6) / HBM_PEAK, 4), "step_alg_bytes": nb_all,
           "prefix_build": {"workload": "state-only prefix scan building the 64 cached states, 64 x 32,768 tokens",
                            "avg_us": round(pre_us, 1), "prefix_tokens_per_s": round(b * L / (pre_us * 1e-6), 1),
                            "alg_bytes": pre_nb,
                            "roofline": make_roofline("hbm", pre_nb, pre_us, traffic_for("prefix_build_c4"))}}
    del steps, clean, ys, ops, h, h0, ws
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- config 0: tiny fp32 block step
def config0(torch, bdssm, configs, inputs, steps=64):
    """The tiny fp32 shape (4 heads x 16, d_state 16, T = 16): 64 block steps from the fp32
    cached state, seeded host draws with distinct inputs per step, in one graph; and one
    launch between synchronizations."""
    cfg = configs.get(0)
    b, H, P, N, G, T = cfg.batch, cfg.nheads, cfg.headdim, cfg.d_state, cfg.ngroups, cfg.block_len
    A, D = inputs.params(cfg)
    Ad, Dd = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    d = bdssm.dims(b, H, P, N, G, cfg.in_dtype, bdssm.F32)
    st = [(bdssm.seq_to_device(inputs.block(cfg, 0, s, inputs.FWD)), bdssm.seq_to_device(inputs.block(cfg, 0, s, inputs.REV)))
          for s in range(steps)]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(10)
    h = torch.randn((b, H, N, P), device="cuda", generator=gen) * 0.1
    ys = [torch.empty((b, T, H, P), device="cuda") for _ in range(steps)]
    us = graph_us(torch, lambda: [bdssm.block_step(d, T, h, f, r, Ad, Dd, y) for (f, r), y in zip(st, ys)], reps=20) / steps
    one = median(launch_times_us(torch, [lambda: bdssm.block_step(d, T, h, st[0][0], st[0][1], Ad, Dd, ys[0])],
                                 reps=20)[0])
    nb = block_step_bytes(b, H, P, N, G, T, 4, 4)
    return {"workload": "tiny fp32 shape (4 heads x 16, d_state 16), T=16: 64 block steps with distinct inputs "
                        "in one graph", "us_per_step": round(us, 3), "single_launch_us": round(one, 3),
            "active_tokens_per_s": round(b * T / (us * 1e-6), 1), "alg_bytes": nb,
            "hbm_frac": round(nb / (us * 1e-6) / HBM_PEAK, 5)}


# ---------------------------------------------------------------- config 1: batch-1 block cycle
def config1(args, torch, np, bdssm, configs, inputs):
    """The 700M batch-1 decode: a block cycle as one graph -- 64 block steps (T = 32) from the
    cached state in operand form, then the commit that refreshes it -- with the parts as
    warmed graphs; the 8192-token prefix scan (bf16 y) that builds the first cached state,
    once per context, timed on its own."""
    cfg = configs.get(1)
    b, H, P, N, G, L, Q, T = (cfg.batch, cfg.nheads, cfg.headdim, cfg.d_state, cfg.ngroups,
                              cfg.prefix_len, cfg.chunk, cfg.block_len)
    S = cfg.steps_per_block
    A, D = inputs.params(cfg)
    d = bdssm.dims(b, H, P, N, G, cfg.in_dtype, bdssm.BF16)
    Ad, Dd = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    pre = bdssm.seq_to_device(inputs.prefix(cfg))
    steps = [(bdssm.seq_to_device(inputs.block(cfg, 0, s, inputs.FWD)),
              bdssm.seq_to_device(inputs.block(cfg, 0, s, inputs.REV))) for s in range(S)]
    clean = bdssm.seq_to_device(inputs.block(cfg, 0, 0, inputs.CLEAN))
    h = torch.empty((b, H, N, P), device="cuda")
    h_ops = torch.empty(bdssm.state_ops_bytes(d), dtype=torch.uint8, device="cuda")
    y_pre = torch.empty((b, L, H, P), dtype=torch.bfloat16, device="cuda")
    y_blk = [torch.empty((b, T, H, P), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    wsb = bdssm.prefix_scan_workspace(d, L, Q, True, False)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")

    def run_prefix():
        bdssm.prefix_scan(d, L, Q, pre, Ad, Dd, None, y_pre, None, h, ws, wsb)

    def run_blocks():
        for s in range(S):
            f, r = steps[s]
            bdssm.block_step_ops(d, T, h_ops, f, r, Ad, Dd, y_blk[s])

    def run_blocks_fp32():
        for s in range(S):
            f, r = steps[s]
            bdssm.block_step(d, T, h, f, r, Ad, Dd, y_blk[s])

    def run_commit():
        bdssm.commit_refresh(d, T, clean, Ad, Dd, h, h_ops, bdssm.STATE_OPS)

    run_prefix()
    bdssm.state_ops(d, h, h_ops)
    parts = (("block_step", run_blocks, S), ("commit_refresh", run_commit, 1))

    def run_all():
        for _, fn, _ in parts:
            fn()

    for _ in range(2):
        run_all()
    whole = warmed(torch, capture(torch, run_all))
    step_us = median(replay_times_us(torch, whole, 20))
    del whole
    res = {"workload": "700M shape, batch 1: block cycle of 64 block steps (T=32) + commit refreshing the operand "
                       "form, one graph; the 8192-token prefix scan (bf16 y) timed on its own",
           "cycle_us": round(step_us, 2), "active_tokens_per_s": round(S * b * T / (step_us * 1e-6), 1)}
    # each part as its own warmed graph; the commit (one launch per cycle) 16 times in a row in
    # one graph, so that a graph replay's own launch cost does not count as the commit's
    CR = 16

    def run_commits():
        for _ in range(CR):
            run_commit()

    for name, fn, n in (("block_step", run_blocks, S), ("commit_refresh", run_commits, CR)):
        us = graph_us(torch, fn, reps=20)
        if us / n * (S if name == "block_step" else 1) > 1.02 * step_us:
            print(f"[bench] inconsistent timing: config 1 {name} {us / n:.1f} us per launch > cycle {step_us:.1f} us",
                  file=sys.stderr, flush=True)
            sys.exit(3)
        res[name + "_us"] = round(us / n, 3)
    res["prefix_scan_us"] = round(graph_us(torch, run_prefix, reps=20), 3)
    nb = block_step_bytes(b, H, P, N, G, T, 2, 2)
    res["block_step_hbm_frac"] = round(nb / (res["block_step_us"] * 1e-6) / HBM_PEAK, 4)
    # cold: RC steps in one graph, each with its own copy of the cached state's operand form,
    # its own inputs and output (RC x ~2.2 MB > 512 MiB: nothing a step reads was read before)
    per_set = bdssm.state_ops_bytes(d) + 2 * b * T * (H * P + H + 2 * G * N) * 2 + b * T * H * P * 2
    RC = (512 << 20) // per_set + 1
    gen = torch.Generator(device="cuda")
    gen.manual_seed(21)
    cold = [(h_ops.clone(), dev_seq(torch, gen, b, T, H, P, G, N), dev_seq(torch, gen, b, T, H, P, G, N),
             torch.empty((b, T, H, P), dtype=torch.bfloat16, device="cuda")) for _ in range(RC)]
    us = graph_us(torch, lambda: [bdssm.block_step_ops(d, T, o, f, r, Ad, Dd, y) for o, f, r, y in cold], reps=5)
    res["block_step_cold_us"] = round(us / RC, 3)
    res["block_step_cold_sets"] = RC
    del cold
    torch.cuda.empty_cache()
    res["block_step_from_fp32_state_us"] = round(graph_us(torch, run_blocks_fp32, reps=20) / S, 3)
    pf = prefix_flops(b, H, P, N, G, L, Q)
    res["prefix_mfma_frac"] = round(pf / (res["prefix_scan_us"] * 1e-6) / MFMA_BF16_PEAK, 4)
    res["prefix_mfma_frac_causal"] = round(prefix_flops_causal(b, H, P, N, G, L, Q) /
                                           (res["prefix_scan_us"] * 1e-6) / MFMA_BF16_PEAK, 4)
    # the same block through the library's decode graph (64 steps + commit + operand form)
    dg = bdssm.DecodeGraph(d, T, h, [f for f, _ in steps], [r for _, r in steps], Ad, Dd, y_blk, clean,
                           h_ops=h_ops)
    for _ in range(2):
        dg.launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        dg.launch()
    e1.record()
    torch.cuda.synchronize()
    dg.close()
    res["decode_graph_us_per_block"] = round(1e3 * e0.elapsed_time(e1) / 20, 2)
    # a single launch between synchronizations
    ts = []
    for i in range(25):
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        bdssm.block_step_ops(d, T, h_ops, steps[0][0], steps[0][1], Ad, Dd, y_blk[0])
        a1.record()
        torch.cuda.synchronize()
        if i >= 5:
            ts.append(1e3 * a0.elapsed_time(a1))
    res["block_step_single_launch_us"] = round(median(ts), 3)
    return res


# ---------------------------------------------------------------- full-window comparison
def full_window_c1(torch, np, bdssm, configs, inputs, block_step_us=None, reps=10):
    """The system the method replaces, timed beside the block step: one denoising step of a
    full-window bidirectional Mamba layer (bdssm_full_window) over the 700M shape's window of
    8192 prefix tokens plus the 32-token block (both directions from zero, every token's
    output), against one block step from the cached state."""
    cfg = configs.get(1)
    b, H, P, N, G, Q = cfg.batch, cfg.nheads, cfg.headdim, cfg.d_state, cfg.ngroups, cfg.chunk
    L = cfg.prefix_len + cfg.block_len
    A, D = inputs.params(cfg)
    Ad, Dd = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    d = bdssm.dims(b, H, P, N, G, cfg.in_dtype, bdssm.BF16)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(13)
    fwd = dev_seq(torch, gen, b, L, H, P, G, N)
    rev = dev_seq(torch, gen, b, L, H, P, G, N)
    y = torch.empty((b, L, H, P), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(bdssm.full_window_workspace(d, L, Q), 1), dtype=torch.uint8, device="cuda")
    fn = lambda: bdssm.full_window(d, L, Q, fwd, rev, Ad, Dd, None, None, y, ws)
    fn()
    torch.cuda.synchronize()
    # device time of one call (a warmed graph of the call, median over replays), as the block
    # step it is compared with is timed; the call's latency from the host beside it
    us = graph_us(torch, fn, reps=reps)
    single_us = median(launch_times_us(torch, [fn], reps=reps)[0])
    nb = 2 * prefix_bytes(b, H, P, N, G, L, Q, 2, 2, False) + b * L * H * P * 2
    out = {"workload": "full-window bidirectional scan (both directions from zero over 8192 prefix + 32 block "
                       "tokens, all outputs, bf16 y), 700M shape, batch 1: one denoising step of the "
                       "comparison system", "avg_us": round(us, 2), "single_call_us": round(single_us, 2),
           "window_tokens": L,
           "hbm_frac": round(nb / (us * 1e-6) / HBM_PEAK, 4), "alg_bytes": nb,
           "mfma_frac": round(2 * prefix_flops(b, H, P, N, G, L, Q) / (us * 1e-6) / MFMA_BF16_PEAK, 4)}
    if block_step_us:
        out["block_step_us"] = block_step_us
        out["full_window_over_block_step"] = round(us / block_step_us, 1)
    return out


# ---------------------------------------------------------------- config 2: prefix scan
def config2_prefix(torch, np, bdssm, configs, inputs, reps=10):
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
    fn = lambda: bdssm.prefix_scan(d, L, Q, pre, Ad, Dd, None, y, cs, ho, ws, wsb)
    fn()
    torch.cuda.synchronize()
    # device time of one call: its three kernels captured as one graph, warmed, median over
    # replays (the launches' host gaps are not the kernels' work); the latency of a single
    # call from the host, launch by launch on an idle GPU, is reported beside it
    us = graph_us(torch, fn, reps=reps)
    single_us = median(launch_times_us(torch, [fn], reps=reps)[0])
    fl = prefix_flops(b, H, P, N, G, L, Q)
    nb = prefix_bytes(b, H, P, N, G, L, Q, 2, 2, True)
    return {"workload": "prefix scan, 350M shape (32 heads x 64, d_state 128), 65,536 tokens, chunk 256, bf16 y + "
                        "fp32 chunk states", "avg_us": round(us, 3), "single_call_us": round(single_us, 3),
            "prefix_tokens_per_s": round(b * L / (us * 1e-6), 1),
            "roofline": make_roofline("mfma", fl, us, traffic_for("prefix_scan_c2")),
            "mfma_frac_causal_count": round(prefix_flops_causal(b, H, P, N, G, L, Q) / (us * 1e-6) / MFMA_BF16_PEAK, 4),
            "hbm_frac": round(nb / (us * 1e-6) / HBM_PEAK, 4), "alg_bytes": nb, "flops_dense": fl,
            "flops_causal": prefix_flops_causal(b, H, P, N, G, L, Q)}


def builds(torch, np, bdssm, configs, inputs):
    """The state-only prefix build of the long-context cache (262,144 tokens x 80 heads, 8
    groups) and the config-2 commit chain."""
    res = {}
    c = configs.get(3)
    b, H, P, N, G, L, Q = c.batch, c.nheads, c.headdim, c.d_state, c.ngroups, c.prefix_len, c.chunk
    A, D = inputs.params(c)
    Adv, Ddv = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    seq = dev_seq(torch, gen, b, L, H, P, G, N, with_c=False, chunk_streams=1)
    dv = bdssm.dims(b, H, P, N, G, 1, bdssm.BF16)
    hv = torch.empty((b, H, N, P), device="cuda")
    wsb = bdssm.prefix_scan_workspace(dv, L, Q, False, False)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    fn = lambda: bdssm.prefix_scan(dv, L, Q, seq, Adv, Ddv, None, None, None, hv, ws, wsb)
    fn()
    torch.cuda.synchronize()
    us = median(launch_times_us(torch, [fn], reps=7)[0])
    nb = prefix_state_bytes(b, H, P, N, G, L, 2)
    res["prefix_build_config3"] = {"workload": "state-only prefix scan, 3B shape (80 heads x 64, 8 groups), "
                                               "262,144 tokens", "avg_us": round(us, 1),
                                   "prefix_tokens_per_s": round(b * L / (us * 1e-6), 1),
                                   "roofline": make_roofline("hbm", nb, us, traffic_for("prefix_build_c3")),
                                   "alg_bytes": nb}
    del seq, hv, ws
    # the block step of the 3B shape (64 steps with distinct inputs in one graph)
    T, S = c.block_len, c.steps_per_block
    d3 = bdssm.dims(b, H, P, N, G, 1, bdssm.BF16)
    st = [(dev_seq(torch, gen, b, T, H, P, G, N), dev_seq(torch, gen, b, T, H, P, G, N)) for _ in range(S)]
    hh = torch.randn((b, H, N, P), device="cuda", generator=gen) * 0.05
    ho = torch.empty(bdssm.state_ops_bytes(d3), dtype=torch.uint8, device="cuda")
    bdssm.state_ops(d3, hh, ho)
    ys = [torch.empty((b, T, H, P), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    us = graph_us(torch, lambda: [bdssm.block_step_ops(d3, T, ho, f, r, Adv, Ddv, y) for (f, r), y in zip(st, ys)]) / S
    nb = block_step_bytes(b, H, P, N, G, T, 2, 2)
    res["block_step_config3"] = {"workload": "block step, 3B shape, T=32, 64 distinct inputs in one graph",
                                 "us_per_step": round(us, 3), "active_tokens_per_s": round(b * T / (us * 1e-6), 1),
                                 "hbm_frac": round(nb / (us * 1e-6) / HBM_PEAK, 4), "alg_bytes": nb}
    # commit chain, config 2: 2048 commits of 32 tokens over the 65,536-token prefix
    c2 = configs.get(2)
    b, H, P, N, G, L, T = c2.batch, c2.nheads, c2.headdim, c2.d_state, c2.ngroups, c2.prefix_len, c2.commit_len
    A, D = inputs.params(c2)
    Ad2, Dd2 = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    d2 = bdssm.dims(b, H, P, N, G, c2.in_dtype, bdssm.BF16)
    pre = dev_seq(torch, gen, b, L, H, P, G, N, with_c=False)
    blocks = [tuple(None if t is None else t[:, k * T:(k + 1) * T].contiguous() for t in pre) for k in range(L // T)]
    hc = torch.zeros((b, H, N, P), device="cuda")
    us = graph_us(torch, lambda: [bdssm.commit(d2, T, blk, Ad2, Dd2, hc) for blk in blocks], reps=3, warm=1)
    res["commit_chain_config2"] = {"workload": "2,048 commits of 32 tokens (350M shape), one graph",
                                   "us_per_commit": round(us / len(blocks), 3),
                                   "tokens_per_s": round(L / (us * 1e-6), 1)}
    return res


def conv_workloads(torch, bdssm, configs, inputs, reps=20):
    """The convolution state at the 700M shape (width 4, SiLU): 64 block steps through
    bdssm_block_step_conv in one graph, and the forward convolution of the 8192-token prefix
    that writes the conv state (HBM-bound)."""
    cfg = configs.get(1)
    b, H, P, N, G, T, L = cfg.batch, cfg.nheads, cfg.headdim, cfg.d_state, cfg.ngroups, cfg.block_len, cfg.prefix_len
    W = 4
    ch = H * P + 2 * G * N
    A, D = inputs.params(cfg)
    Ad, Dd = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    d = bdssm.dims(b, H, P, N, G, cfg.in_dtype, bdssm.BF16)
    wf, bf = (torch.from_numpy(a).cuda() for a in inputs.conv_params(cfg, W, inputs.FWD))
    wr, br = (torch.from_numpy(a).cuda() for a in inputs.conv_params(cfg, W, inputs.REV))
    cpf, cpr = bdssm.conv_params(wf, bf, 1), bdssm.conv_params(wr, br, 1)
    cs = torch.zeros((b, W - 1, ch), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(2 * bdssm.conv_workspace(d, T), dtype=torch.uint8, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    S = cfg.steps_per_block
    steps = [(dev_seq(torch, gen, b, T, H, P, G, N), dev_seq(torch, gen, b, T, H, P, G, N)) for _ in range(S)]
    h = torch.randn((b, H, N, P), device="cuda", generator=gen) * 0.05
    ys = [torch.empty((b, T, H, P), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    step_us = graph_us(torch, lambda: [bdssm.block_step_conv(d, T, cpf, cpr, h, cs, f, r, Ad, Dd, y, ws)
                                       for (f, r), y in zip(steps, ys)], reps=reps) / S
    pre = dev_seq(torch, gen, b, L, H, P, G, N)
    post = tuple(torch.empty_like(t) for t in pre)
    cso = torch.empty_like(cs)
    fn = lambda: bdssm.conv(d, L, cpf, False, None, pre, post, cso)
    fn()
    torch.cuda.synchronize()
    conv_us = median(launch_times_us(torch, [fn], reps=reps)[0])
    nb = 2 * b * L * ch * 2 + ch * (W + 1) * 4 + 2 * b * (W - 1) * ch * 2
    return {"block_step_conv": {"workload": "64 block steps (T=32) on unconvolved inputs, width-4 SiLU "
                                            "convolution of x, B, C per direction, 700M shape, one graph",
                                "us_per_step": round(step_us, 3),
                                "active_tokens_per_s": round(b * T / (step_us * 1e-6), 1)},
            "prefix_conv": {"workload": "forward convolution of an 8192-token prefix (x, B, C; width 4, SiLU) "
                                        "writing the conv state, 700M shape, bf16",
                            "avg_us": round(conv_us, 3), "alg_bytes": nb,
                            "roofline": make_roofline("hbm", nb, conv_us, None)}}


# ---------------------------------------------------------------- CPU baseline
def cpu_baseline(np, configs, inputs):
    """The float64 oracle on the host cores, on a bounded sample of the headline step: the
    16 block steps of the running set (T = 128) and the oldest-block commit, for 4 streams on
    one thread and for all 64 streams on all threads (threads over (stream, head) pairs).
    Each figure is active tokens of the sample per second of host time."""
    import oracle
    cfg = configs.get(4)
    A, D = inputs.params(cfg)
    H, P, N = cfg.nheads, cfg.headdim, cfg.d_state
    S = cfg.steps_per_block
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count() or 1
    all_threads = max(1, min(oracle.max_threads(), affinity))

    def run(nstreams, nthreads):
        streams = list(range(nstreams))
        rng = np.random.default_rng(5)
        h = rng.standard_normal((nstreams, H, N, P)) * 0.05
        steps = [(inputs.block(cfg, 0, s, inputs.FWD, streams=streams),
                  inputs.block(cfg, 0, s, inputs.REV, streams=streams)) for s in range(S)]
        clean = inputs.block(cfg, 0, 0, inputs.CLEAN, streams=streams)
        t0 = time.perf_counter()
        for f, r in steps:
            oracle.block_step(h, f, r, A, D, nthreads=nthreads)
        oracle.commit(h, clean, A, D, nthreads=nthreads)
        wall = time.perf_counter() - t0
        return nstreams * S * cfg.block_len / wall, wall

    few = 4
    one, w1 = run(few, 1)
    many_streams = cfg.batch
    allv, wall_all = run(many_streams, all_threads)
    return {"value": round(allv, 2), "unit": "tokens/s", "cores": all_threads, "kind": "oracle",
            "sample": f"the headline step's 16 block steps (T=128) + oldest-block commit for {many_streams} of the "
                      f"64 streams on {all_threads} threads ({wall_all:.1f} s of host time); rate = active tokens "
                      "of the sample per second",
            "single_thread": {"value": round(one, 2), "unit": "tokens/s", "cores": 1,
                              "sample": f"the same for {few} streams on 1 thread ({w1:.1f} s)"},
            "host_cpus_in_affinity_mask": affinity, "host_cpu_count": os.cpu_count(),
            "openmp_max_threads": oracle.max_threads()}


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
    if args.only:
        fn = {"headline": lambda: headline(args, torch, np, bdssm, configs, inputs),
              "c0": lambda: config0(torch, bdssm, configs, inputs),
              "c1": lambda: config1(args, torch, np, bdssm, configs, inputs),
              "c2prefix": lambda: config2_prefix(torch, np, bdssm, configs, inputs),
              "builds": lambda: builds(torch, np, bdssm, configs, inputs),
              "fullwindow": lambda: full_window_c1(torch, np, bdssm, configs, inputs),
              "step4": lambda: step4(torch, bdssm, configs, inputs),
              "build4": lambda: build_only(torch, bdssm, configs, inputs, 4),
              "build3": lambda: build_only(torch, bdssm, configs, inputs, 3)}.get(args.only)
        print(json.dumps({args.only: fn()}), flush=True)
        return
    out = headline(args, torch, np, bdssm, configs, inputs)
    if not args.no_secondary:
        print("[bench] secondary workloads", file=sys.stderr, flush=True)
        c1 = config1(args, torch, np, bdssm, configs, inputs)
        out["secondary"] = {"config0_block_step": config0(torch, bdssm, configs, inputs),
                            "config1_block_cycle": c1,
                            "config2_prefix_scan": config2_prefix(torch, np, bdssm, configs, inputs),
                            "full_window_config1": full_window_c1(torch, np, bdssm, configs, inputs,
                                                                  c1["block_step_us"])}
        out["secondary"].update(builds(torch, np, bdssm, configs, inputs))
        out["secondary"]["conv_state"] = conv_workloads(torch, bdssm, configs, inputs)
    if not args.no_cpu_baseline:
        print("[bench] CPU baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(np, configs, inputs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
