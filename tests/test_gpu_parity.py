"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Bounds (relative L2 over the whole tensor, float64): 1e-5 for float32 inputs, 5e-3 for
bfloat16 inputs with float32 state. y is checked twice: as returned (with D x) and with
D = 0, because D x dominates y's norm and would hide a wrong scan term.
"""
import numpy as np
import pytest

import oracle
from bidirectional_mamba_state_amd import bdssm, configs, inputs
from bidirectional_mamba_state_amd.inputs import Seq

from harness import (within, TOL_BF16, TOL_F32, gpu_block_step, gpu_commit, gpu_prefix, max_head_rel,
                     rel, slice_seq, streams_of, tol_for, f32_round)

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _check_prefix(seq, A, D, chunk, h_init=None, want_y=True, want_cs=True, heads=None,
                  y_dtype=bdssm.F32, in_place=False, label="", also_bf16_y=False):
    """also_bf16_y: the same scan again with a bf16 y (and chunk states), against the same
    oracle results."""
    _case(f"prefix {label} len={seq.length} chunk={chunk} y={want_y} cs={want_cs} "
          f"y_dtype={y_dtype} in_place={in_place}")
    tol = tol_for(seq.dtype) if y_dtype == bdssm.F32 else max(tol_for(seq.dtype), 5e-3)
    y, cs, h = gpu_prefix(seq, A, D, chunk, h_init, want_y, want_cs, y_dtype, in_place)
    yo, cso, ho = oracle.scan(seq, A, D, chunk, h_init=h_init, want_y=want_y,
                              want_chunk_states=want_cs, heads=heads)
    hs = slice(None) if heads is None else list(heads)
    assert within(rel(h[:, hs], ho[:, hs]), tol_for(seq.dtype), "final state")
    if want_cs:
        assert within(rel(cs[:, :, hs], cso[:, :, hs]), tol_for(seq.dtype), "chunk states")
        assert np.array_equal(cs[:, -1], h), "last chunk state == h_out"
    if want_y:
        assert within(rel(y[:, :, hs], yo[:, :, hs]), tol, "y")
        assert within(max_head_rel(y[:, :, hs], yo[:, :, hs], 2), 4 * tol, "y, worst head")
        # the scan part alone (D = 0)
        Dz = np.zeros_like(D)
        yz, _, _ = gpu_prefix(seq, A, Dz, chunk, h_init, True, False, y_dtype)
        yzo, _, _ = oracle.scan(seq, A, Dz, chunk, h_init=h_init, want_chunk_states=False, heads=heads)
        assert within(rel(yz[:, :, hs], yzo[:, :, hs]), tol, "y - D x")
        if also_bf16_y:
            tb = max(tol_for(seq.dtype), 5e-3)
            yb, csb, hb = gpu_prefix(seq, A, D, chunk, h_init, True, want_cs, bdssm.BF16)
            assert within(rel(yb[:, :, hs], yo[:, :, hs]), tb, "bf16 y")
            assert within(max_head_rel(yb[:, :, hs], yo[:, :, hs], 2), 4 * tb, "bf16 y, worst head")
            assert within(rel(hb[:, hs], ho[:, hs]), tol_for(seq.dtype), "final state, bf16 y")
            if want_cs:
                assert within(rel(csb[:, :, hs], cso[:, :, hs]), tol_for(seq.dtype), "chunk states, bf16 y")
            yzb, _, _ = gpu_prefix(seq, A, Dz, chunk, h_init, True, False, bdssm.BF16)
            assert within(rel(yzb[:, :, hs], yzo[:, :, hs]), tb, "bf16 y - D x")
    return h


def _check_block(h_prefix, fwd, rev, A, D, y_dtype=bdssm.F32, heads=None, label=""):
    _case(f"block_step {label} T={fwd.length} y_dtype={y_dtype}")
    tol = tol_for(fwd.dtype) if y_dtype == bdssm.F32 else max(tol_for(fwd.dtype), 5e-3)
    y = gpu_block_step(h_prefix, fwd, rev, A, D, y_dtype)
    yo, _, _ = oracle.block_step(h_prefix, fwd, rev, A, D, heads=heads)
    hs = slice(None) if heads is None else list(heads)
    assert within(rel(y[:, :, hs], yo[:, :, hs]), tol, "block y")
    Dz = np.zeros_like(D)
    yz = gpu_block_step(h_prefix, fwd, rev, A, Dz, y_dtype)
    yzo, _, _ = oracle.block_step(h_prefix, fwd, rev, A, Dz, heads=heads)
    assert within(rel(yz[:, :, hs], yzo[:, :, hs]), tol, "block y - D x")
    assert within(max_head_rel(yz[:, :, hs], yzo[:, :, hs], 2), 4 * tol, "block y - D x, worst head")


def _check_commit(h, clean, A, D, label=""):
    _case(f"commit {label} T={clean.length}")
    hn, y = gpu_commit(h, clean, A, D, want_y=True)
    hno, yo = oracle.commit(h, clean, A, D, want_y=True)
    assert within(rel(hn, hno), tol_for(clean.dtype), "commit state")
    assert within(rel(y, yo), tol_for(clean.dtype), "commit y")
    # without y the commit runs the state-only walk (another summation order): the same
    # state within the bound
    hn2, _ = gpu_commit(h, clean, A, D, want_y=False)
    assert within(rel(hn2, hno), tol_for(clean.dtype), "commit state, no y")
    assert within(rel(hn2, hn), tol_for(clean.dtype), "commit state with and without y")
    return hn


# ------------------------------------------------------------------ per config
def test_config0_tiny_fp32_full_path():
    cfg = configs.get(0)
    A, D = inputs.params(cfg)
    pre = inputs.prefix(cfg)
    h = _check_prefix(pre, A, D, cfg.chunk, label="c0")
    _check_prefix(pre, A, D, cfg.chunk, y_dtype=bdssm.BF16, want_cs=False, label="c0 bf16 y")
    h = f32_round(h)
    for k in range(cfg.n_blocks):
        for step in range(cfg.steps_per_block):
            fwd = inputs.block(cfg, k, step, inputs.FWD)
            rev = inputs.block(cfg, k, step, inputs.REV)
            _check_block(h, fwd, rev, A, D, label=f"c0 block {k} step {step}")
        h = f32_round(_check_commit(h, inputs.block(cfg, k, 0, inputs.CLEAN), A, D, label=f"c0 block {k}"))


def test_config1_700m_four_blocks():
    """The 700M batch-1 plan: the 8192-token prefix scan (y and state), then four blocks of
    64 denoising steps each followed by a commit. Every step of block 0 and the last step of
    blocks 1-3 are checked (y, and y - D x on the first and last step of each block), and
    every post-commit state; the oracle continues from the GPU's float32 state, as the next
    block's steps do."""
    cfg = configs.get(1)
    A, D = inputs.params(cfg)
    pre = inputs.prefix(cfg)
    h = f32_round(_check_prefix(pre, A, D, cfg.chunk, want_cs=False, label="c1"))
    S = cfg.steps_per_block
    for k in range(cfg.n_blocks):
        for step in (range(S) if k == 0 else (S - 1,)):
            fwd = inputs.block(cfg, k, step, inputs.FWD)
            rev = inputs.block(cfg, k, step, inputs.REV)
            if step in (0, S - 1):
                _check_block(h, fwd, rev, A, D, label=f"c1 block {k} step {step}")
            else:
                _case(f"block_step c1 block {k} step {step}")
                y = gpu_block_step(h, fwd, rev, A, D)
                yo, _, _ = oracle.block_step(h, fwd, rev, A, D)
                assert within(rel(y, yo), TOL_BF16, "block y")
        if k == 0:
            _check_block(h, inputs.block(cfg, 0, 0, inputs.FWD), inputs.block(cfg, 0, 0, inputs.REV), A, D,
                         y_dtype=bdssm.BF16, label="c1 bf16 y")
        h = f32_round(_check_commit(h, inputs.block(cfg, k, 0, inputs.CLEAN), A, D, label=f"c1 block {k}"))


def test_config2_prefix_chunk_states_all_heads():
    cfg = configs.get(2)
    A, D = inputs.params(cfg)
    pre = inputs.prefix(cfg)
    h = _check_prefix(pre, A, D, cfg.chunk, label="c2 (all 32 heads)", also_bf16_y=True)
    _check_commit(f32_round(h), inputs.block(cfg, 0, 0, inputs.CLEAN), A, D, label="c2")


def test_config3_long_context_grouped():
    """The 3B long-context plan: the 262,144-token state-only prefix (all 80 heads, 8
    groups of 10), then 64 denoising steps (each checked; y - D x on the first and last) and
    the commit."""
    cfg = configs.get(3)
    A, D = inputs.params(cfg)
    pre = inputs.prefix(cfg)
    h = _check_prefix(pre, A, D, cfg.chunk, want_y=False, want_cs=False, label="c3 (all 80 heads)")
    del pre
    hf = f32_round(h)
    S = cfg.steps_per_block
    for step in range(S):
        fwd = inputs.block(cfg, 0, step, inputs.FWD)
        rev = inputs.block(cfg, 0, step, inputs.REV)
        if step in (0, S - 1):
            _check_block(hf, fwd, rev, A, D, label=f"c3 step {step}")
        else:
            _case(f"block_step c3 step {step}")
            y = gpu_block_step(hf, fwd, rev, A, D)
            yo, _, _ = oracle.block_step(hf, fwd, rev, A, D)
            assert within(rel(y, yo), TOL_BF16, "block y")
    _check_commit(hf, inputs.block(cfg, 0, 0, inputs.CLEAN), A, D, label="c3")


# ------------------------------------------------------------------ edge cases
def _small(b=2, L=100, H=4, P=16, N=16, G=2, dtype=1, seed=0):
    rng = np.random.default_rng(seed)
    from test_oracle_pins import rand_seq
    return rand_seq(rng, b, L, H, P, N, G, dtype), rng


@pytest.mark.parametrize("chunk", [16, 32, 64, 128, 256])
def test_chunk_invariance(chunk):
    seq, rng = _small(L=300, dtype=0)
    A = (-np.exp(rng.uniform(0, np.log(16), 4))).astype(np.float32)
    D = rng.standard_normal(4).astype(np.float32)
    h0 = rng.standard_normal((2, 4, 16, 16)) * 0.1
    _check_prefix(seq, A, D, chunk, h_init=h0, label=f"chunk sweep {chunk}")


@pytest.mark.parametrize("L", [1, 15, 16, 17, 257])
def test_ragged_lengths(L):
    seq, rng = _small(L=L, dtype=0)
    A = (-np.exp(rng.uniform(0, np.log(16), 4))).astype(np.float32)
    D = rng.standard_normal(4).astype(np.float32)
    _check_prefix(seq, A, D, 16, label=f"ragged {L}")
    _check_prefix(seq, A, D, 16, want_y=False, want_cs=False, label=f"ragged {L} state-only")


def test_in_place_state_update():
    seq, rng = _small(L=200, dtype=1, P=64, N=128, H=4, G=1)
    A = (-np.exp(rng.uniform(0, np.log(16), 4))).astype(np.float32)
    D = rng.standard_normal(4).astype(np.float32)
    h0 = rng.standard_normal((2, 4, 128, 64)) * 0.1
    for want_y, want_cs in ((True, True), (True, False), (False, True), (False, False)):
        _check_prefix(seq, A, D, 64, h_init=h0, want_y=want_y, want_cs=want_cs, in_place=True,
                      label="in place")


@pytest.mark.parametrize("T", [1, 7, 16, 33, 128, 256])
def test_block_lengths(T):
    rng = np.random.default_rng(T)
    from test_oracle_pins import rand_seq
    fwd = rand_seq(rng, 2, T, 4, 64, 128, 2, 1)
    rev = rand_seq(rng, 2, T, 4, 64, 128, 2, 1)
    A = (-np.exp(rng.uniform(0, np.log(16), 4))).astype(np.float32)
    D = rng.standard_normal(4).astype(np.float32)
    h = f32_round(rng.standard_normal((2, 4, 128, 64)) * 0.1)
    _check_block(h, fwd, rev, A, D, label=f"T={T}")
    _check_commit(h, fwd, A, D, label=f"T={T}")


def test_empty_inputs():
    t = pytest.importorskip("torch")
    d = bdssm.dims(1, 4, 16, 16, 1, bdssm.F32)
    e = t.empty(0, device="cuda")
    A = t.full((4,), -1.0, device="cuda")
    D = t.ones(4, device="cuda")
    h0 = t.randn(1, 4, 16, 16, device="cuda")
    ho = t.full((1, 4, 16, 16), 7.0, device="cuda")
    seq = (t.empty(16, device="cuda"),) * 4
    bdssm.prefix_scan(d, 0, 64, seq, A, D, h0, None, None, ho)   # zero tokens: h_out = h_init
    t.cuda.synchronize()
    assert t.equal(ho, h0)
    bdssm.prefix_scan(d, 0, 64, seq, A, D, None, None, None, ho)  # ... or zero
    t.cuda.synchronize()
    assert not ho.any()
    y = t.full((4,), 3.0, device="cuda")
    bdssm.block_step(d, 0, h0, seq, seq, A, D, y)                 # nothing to do
    hb = h0.clone()
    bdssm.commit(d, 0, seq, A, D, hb)
    d0 = bdssm.dims(0, 4, 16, 16, 1, bdssm.F32)
    bdssm.block_step(d0, 16, h0, seq, seq, A, D, y)
    t.cuda.synchronize()
    assert t.equal(hb, h0) and bool((y == 3.0).all())
    del e


# ------------------------------------------------------------------ invariants
def test_cached_state_untouched_and_deterministic():
    t = pytest.importorskip("torch")
    cfg = configs.get(1)
    A, D = inputs.params(cfg)
    rng = np.random.default_rng(1)
    h = t.from_numpy((rng.standard_normal((1, 48, 128, 64)) * 0.05).astype(np.float32)).cuda()
    h_copy = h.clone()
    fwd = inputs.block(cfg, 0, 0, inputs.FWD)
    rev = inputs.block(cfg, 0, 0, inputs.REV)
    d = bdssm.dims(1, 48, 64, 128, 1, bdssm.BF16)
    Ad, Dd = t.from_numpy(A).cuda(), t.from_numpy(D).cuda()
    fd, rd = bdssm.seq_to_device(fwd), bdssm.seq_to_device(rev)
    ys = []
    for _ in range(8):
        y = t.empty((1, 32, 48, 64), device="cuda")
        bdssm.block_step(d, 32, h, fd, rd, Ad, Dd, y)
        ys.append(y)
    t.cuda.synchronize()
    assert t.equal(h, h_copy), "block step wrote the cached state"
    for y in ys[1:]:
        assert t.equal(y, ys[0]), "block step is not deterministic"


def test_reverse_locality_and_stream_independence():
    t = pytest.importorskip("torch")
    rng = np.random.default_rng(2)
    from test_oracle_pins import rand_seq
    b, T, H, P, N = 3, 32, 4, 64, 128
    fwd = rand_seq(rng, b, T, H, P, N, 1, 1)
    rev = rand_seq(rng, b, T, H, P, N, 1, 1)
    A = (-np.exp(rng.uniform(0, np.log(16), H))).astype(np.float32)
    D = np.zeros(H, np.float32)
    h1 = f32_round(rng.standard_normal((b, H, N, P)) * 0.1)
    h2 = h1.copy()
    h2[1] += f32_round(rng.standard_normal((H, N, P)) * 0.1)
    y1 = gpu_block_step(h1, fwd, rev, A, D)
    y2 = gpu_block_step(h2, fwd, rev, A, D)
    assert np.array_equal(y1[[0, 2]], y2[[0, 2]]), "perturbing stream 1 changed other streams"
    # the change is exactly the forward state term, independent of the reverse inputs
    zero_x = Seq(np.zeros_like(fwd.x), fwd.dt, fwd.B, fwd.C, fwd.dtype)
    zero_r = Seq(np.zeros_like(rev.x), rev.dt, rev.B, rev.C, rev.dtype)
    dh = h2 - h1
    yd = gpu_block_step(dh, zero_x, zero_r, A, D)
    ydo, _, _ = oracle.block_step(dh, zero_x, zero_r, A, D)
    assert within(rel(yd, ydo), TOL_BF16, "state term alone")
    assert within(rel(y2 - y1, ydo), TOL_BF16, "difference of two steps = state term")


def test_commit_chain_equals_prefix_scan():
    cfg = configs.get(1)
    A, D = inputs.params(cfg)
    pre = inputs.prefix(cfg, length=1024)
    _case("commit chain: 32 commits of 32 tokens vs one 1024-token scan")
    _, cs, h_scan = gpu_prefix(pre, A, D, 256, want_y=False, want_cs=True)
    h = np.zeros((1, 48, 128, 64))
    for k in range(32):
        h, _ = gpu_commit(h, slice_seq(pre, 32 * k, 32 * (k + 1)), A, D)
        if (k + 1) % 8 == 0:
            assert within(rel(h, cs[:, (k + 1) // 8 - 1]), 1e-5, "commit chain vs chunk state")
    assert within(rel(h, h_scan), 1e-5, "commit chain vs scan final state")
    _, _, ho = oracle.scan(pre, A, D, 256, want_y=False, want_chunk_states=False)
    assert within(rel(h, ho), TOL_BF16, "commit chain vs oracle")


@pytest.mark.parametrize("T", [17, 32, 64, 128])
def test_block_step_launch_shapes(launch_override, T):
    """Both block-step kernels give the oracle's result: the bandwidth kernel at every
    (heads per workgroup, column split) launch shape, and the latency kernel (one workgroup
    per head, row block and column part, of 2 or 4 wavefronts; T <= 32) with float32 and
    bfloat16 y."""
    rng = np.random.default_rng(100 + T)
    from test_oracle_pins import rand_seq
    b, H, G = 3, 12, 2        # 6 heads per group
    fwd = rand_seq(rng, b, T, H, 64, 128, G, 1)
    rev = rand_seq(rng, b, T, H, 64, 128, G, 1)
    A = (-np.exp(rng.uniform(0, np.log(16), H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    h = f32_round(rng.standard_normal((b, H, 128, 64)) * 0.1)
    yo, _, _ = oracle.block_step(h, fwd, rev, A, D)
    Dz = np.zeros_like(D)
    yzo, _, _ = oracle.block_step(h, fwd, rev, A, Dz)
    shapes = [(hpw, ps) for hpw in (1, 2, 3, 6) for ps in (1, 2, 4)] if T in (32, 128) else [(1, 4), (6, 1)]
    for hpw, ps in shapes:
        launch_override(block_kernel=bdssm.KERNEL_BANDWIDTH, bw_heads=hpw, bw_splits=ps)
        _case(f"launch shape T={T} hpw={hpw} ps={ps}")
        y = gpu_block_step(h, fwd, rev, A, D)
        yz = gpu_block_step(h, fwd, rev, A, Dz)
        assert within(rel(y, yo), TOL_BF16, f"y hpw={hpw} ps={ps}")
        assert within(rel(yz, yzo), TOL_BF16, f"y - D x hpw={hpw} ps={ps}")
    if T <= 32:
        for wpg, y_dtype in ((2, bdssm.F32), (2, bdssm.BF16), (4, bdssm.F32), (4, bdssm.BF16)):
            launch_override(block_kernel=bdssm.KERNEL_SMALL_BATCH, lat_waves=wpg)
            _case(f"latency kernel T={T} wavefronts per workgroup {wpg} y_dtype={y_dtype}")
            y = gpu_block_step(h, fwd, rev, A, D, y_dtype)
            yz = gpu_block_step(h, fwd, rev, A, Dz, y_dtype)
            assert within(rel(y, yo), TOL_BF16, "y, latency kernel")
            assert within(rel(yz, yzo), TOL_BF16, "y - D x, latency kernel")
            assert within(max_head_rel(yz, yzo, 2), 4 * TOL_BF16, "y - D x, latency kernel, worst head")


def test_config4_running_set_shape():
    """64 streams x 48 heads, T = 128 (the running set of four 32-token blocks), in the
    launch configuration the benchmark times; cached states from a 1024-token prefix per
    stream; oracle on streams {0, 31, 63}."""
    cfg = configs.get(4)
    A, D = inputs.params(cfg)
    pre = inputs.prefix(cfg, length=1024)
    _, _, h = gpu_prefix(pre, A, D, cfg.chunk, want_y=False, want_cs=False)
    sample = [0, 31, 63]
    _, _, ho = oracle.scan(streams_of(pre, sample), A, D, cfg.chunk, want_y=False, want_chunk_states=False)
    assert within(rel(h[sample], ho), TOL_BF16, "c4 prefix state (sampled streams)")
    fwd = inputs.block(cfg, 0, 0, inputs.FWD)
    rev = inputs.block(cfg, 0, 0, inputs.REV)
    for y_dtype in (bdssm.F32, bdssm.BF16):
        _case(f"c4 block step y_dtype={y_dtype}")
        y = gpu_block_step(h, fwd, rev, A, D, y_dtype)
        yo, _, _ = oracle.block_step(h[sample], streams_of(fwd, sample), streams_of(rev, sample), A, D)
        assert within(rel(y[sample], yo), TOL_BF16, "c4 block y (sampled streams)")
    Dz = np.zeros_like(D)
    yz = gpu_block_step(h, fwd, rev, A, Dz)
    yzo, _, _ = oracle.block_step(h[sample], streams_of(fwd, sample), streams_of(rev, sample), A, Dz)
    assert within(rel(yz[sample], yzo), TOL_BF16, "c4 block y - D x (sampled streams)")
    assert within(max_head_rel(yz[sample], yzo, 2), 4 * TOL_BF16, "y - D x, worst head")


@pytest.mark.parametrize("b,H,G,L,chunk,want_y,want_cs,init", [
    (1, 4, 1, 640, 64, True, True, True),       # several segments, full pass
    (2, 6, 2, 1000, 128, True, False, False),   # ragged tail, groups, y only
    (1, 4, 2, 777, 256, False, True, True),     # chunk states only, ragged
    (1, 4, 1, 4096, 256, False, False, True),   # state only, several segments + scan
    (64, 8, 1, 192, 64, True, True, True),      # one segment per (stream, head): single pass
    (64, 8, 4, 300, 64, False, False, True),    # single pass, state only, ragged
    # one stream, 32 segments of 10 sub-chunks, the last a single ragged one
    (1, 16, 1, 20037, 256, True, True, True),
])
def test_prefix_matrix_core_paths(b, H, G, L, chunk, want_y, want_cs, init):
    rng = np.random.default_rng(L + H)
    from test_oracle_pins import rand_seq
    seq = rand_seq(rng, b, L, H, 64, 128, G, 1)
    A = (-np.exp(rng.uniform(0, np.log(16), H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    h0 = f32_round(rng.standard_normal((b, H, 128, 64)) * 0.1) if init else None
    _check_prefix(seq, A, D, chunk, h_init=h0, want_y=want_y, want_cs=want_cs,
                  label=f"mfma paths b={b} H={H} G={G}")
    if want_y:
        _check_prefix(seq, A, D, chunk, h_init=h0, want_y=True, want_cs=False,
                      y_dtype=bdssm.BF16, label="mfma paths bf16 y")


@pytest.mark.parametrize("cfg_index", [0, 1])
def test_block_step_separate_reverse_params(cfg_index):
    """bdssm_block_step_ex: the reverse scan with its own decay A_rev and skip weight
    D_rev, against the oracle; with A_rev = A and no D_rev it is bdssm_block_step."""
    import torch
    cfg = configs.get(cfg_index)
    A, D = inputs.params(cfg)
    rng = np.random.default_rng(40 + cfg_index)
    H = cfg.nheads
    A_rev = (-np.exp(rng.uniform(0, np.log(16), H))).astype(np.float32)
    D_rev = rng.standard_normal(H).astype(np.float32)
    pre = inputs.prefix(cfg, length=min(cfg.prefix_len, 512))
    _, _, h = oracle.scan(pre, A, D, cfg.chunk, want_y=False, want_chunk_states=False)
    h = f32_round(h)
    fwd = inputs.block(cfg, 0, 0, inputs.FWD)
    rev = inputs.block(cfg, 0, 0, inputs.REV)
    b, T, _, P = fwd.x.shape
    d = bdssm.dims(b, H, P, cfg.d_state, cfg.ngroups, cfg.in_dtype, bdssm.F32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    hd, fd, rd = dev(h), bdssm.seq_to_device(fwd), bdssm.seq_to_device(rev)
    tol = TOL_BF16 if cfg.in_dtype == 1 else TOL_F32
    _case(f"block step, separate reverse parameters, config {cfg_index}")
    for Dv, Drv, what in ((D, D_rev, "y"), (np.zeros_like(D), None, "y - skip terms")):
        y = torch.empty((b, T, H, P), device="cuda")
        bdssm.block_step_ex(d, T, hd, fd, rd, dev(A), dev(Dv), dev(A_rev),
                            None if Drv is None else dev(Drv), y)
        torch.cuda.synchronize()
        yo, _, _ = oracle.block_step(h, fwd, rev, A, Dv, A_rev=A_rev, D_rev=Drv)
        assert within(rel(y.cpu().numpy(), yo), tol, f"block step ex {what}")
    y1 = torch.empty((b, T, H, P), device="cuda")
    y2 = torch.empty((b, T, H, P), device="cuda")
    bdssm.block_step(d, T, hd, fd, rd, dev(A), dev(D), y1)
    bdssm.block_step_ex(d, T, hd, fd, rd, dev(A), dev(D), dev(A), None, y2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
