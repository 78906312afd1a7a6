"""The cached state in operand form (bdssm_state_ops) and the block step that reads it
(bdssm_block_step_ops): the encoding is exactly the bf16 hi/lo pair its definition states,
and the block step from it gives bitwise the y of bdssm_block_step_ex from the float32 state
(the small-batch kernel forms the same pair on every call), hence the oracle's y."""
import numpy as np
import pytest

import oracle
from bidirectional_mamba_state_amd import bdssm, configs, inputs
from harness import TOL_BF16, f32_round, max_head_rel, rel, within

pytestmark = pytest.mark.gpu


def _expected_ops(h):
    """[b][H][N][P] float32 -> [b][H][2][N/8][P][8] uint16: hi = bf16(h), lo = bf16(h - hi),
    both rounded to nearest even (h - hi is exact in float32)."""
    h = np.asarray(h, np.float32)
    hi = inputs.round_bf16_bits(h.astype(np.float64))
    lo = inputs.round_bf16_bits(h.astype(np.float64) - inputs.bf16_bits_to_f32(hi).astype(np.float64))
    b, H, N, P = h.shape
    both = np.stack([hi, lo], axis=2)                         # [b][H][2][N][P]
    return both.reshape(b, H, 2, N // 8, 8, P).transpose(0, 1, 2, 3, 5, 4).copy()


def test_state_ops_encoding():
    import torch
    rng = np.random.default_rng(11)
    b, H, N, P = 2, 4, 128, 64
    h = (rng.standard_normal((b, H, N, P)) * np.exp(rng.uniform(-20, 20, (b, H, N, P)))).astype(np.float32)
    # special values: zeros, exact bf16 values (lo = 0), halfway cases that round to even
    h[0, 0, 0, :8] = 0.0
    h[0, 0, 1, :8] = -0.0
    h[0, 0, 2, :8] = np.float32(1.5)
    h[0, 0, 3, :8] = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x3F80FFFF] * 2, np.uint32).view(np.float32)
    print(f"[case] state ops encoding b={b} H={H}", flush=True)
    d = bdssm.dims(b, H, P, N, 1, bdssm.BF16, bdssm.F32)
    hd = torch.from_numpy(h).cuda()
    ops = torch.full((bdssm.state_ops_bytes(d) // 2,), -1, dtype=torch.int16, device="cuda")
    bdssm.state_ops(d, hd, ops)
    torch.cuda.synchronize()
    got = ops.cpu().numpy().view(np.uint16).reshape(b, H, 2, N // 8, P, 8)
    want = _expected_ops(h)
    assert np.array_equal(got, want), int((got != want).sum())
    assert torch.equal(hd.cpu(), torch.from_numpy(h))          # the state is read only


def _case_inputs(b, H, G, T, seed):
    from test_oracle_pins import rand_seq
    rng = np.random.default_rng(seed)
    fwd = rand_seq(rng, b, T, H, 64, 128, G, 1)
    rev = rand_seq(rng, b, T, H, 64, 128, G, 1)
    A = (-np.exp(rng.uniform(0, np.log(16), H))).astype(np.float32)
    Ar = (-np.exp(rng.uniform(0, np.log(16), H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    Dr = rng.standard_normal(H).astype(np.float32)
    h = f32_round(rng.standard_normal((b, H, 128, 64)) * 0.1)
    return fwd, rev, A, D, Ar, Dr, h


@pytest.mark.parametrize("b,H,G,T", [(1, 48, 1, 32), (3, 12, 2, 17), (3, 12, 2, 32), (2, 40, 8, 1)])
def test_block_step_ops_bitwise(launch_override, b, H, G, T):
    import torch
    fwd, rev, A, D, Ar, Dr, h = _case_inputs(b, H, G, T, 1000 + 7 * H + T)
    tf, tr = bdssm.seq_to_device(fwd), bdssm.seq_to_device(rev)
    Ad, Dd, Ard, Drd = (torch.from_numpy(v).cuda() for v in (A, D, Ar, Dr))
    hd = torch.from_numpy(h.astype(np.float32)).cuda()
    d32 = bdssm.dims(b, H, 64, 128, G, bdssm.BF16, bdssm.F32)
    ops = torch.empty(bdssm.state_ops_bytes(d32), dtype=torch.uint8, device="cuda")
    bdssm.state_ops(d32, hd, ops)
    for wpg in (2, 4):
        launch_override(block_kernel=bdssm.KERNEL_SMALL_BATCH, lat_waves=wpg)
        for y_dt, tdt in ((bdssm.F32, torch.float32), (bdssm.BF16, torch.bfloat16)):
            for sep in (False, True):
                print(f"[case] block step ops b={b} H={H} G={G} T={T} wpg={wpg} y={y_dt} separate={sep}", flush=True)
                d = bdssm.dims(b, H, 64, 128, G, bdssm.BF16, y_dt)
                y_ref = torch.full((b, T, H, 64), 7.0, dtype=tdt, device="cuda")
                y_ops = torch.full((b, T, H, 64), -7.0, dtype=tdt, device="cuda")
                A_rev, D_rev = (Ard, Drd) if sep else (Ad, None)
                bdssm.block_step_ex(d, T, hd, tf, tr, Ad, Dd, A_rev, D_rev, y_ref)
                bdssm.block_step_ops(d, T, ops, tf, tr, Ad, Dd, y_ops, A_rev=A_rev, D_rev=D_rev)
                torch.cuda.synchronize()
                assert torch.equal(y_ops, y_ref)
    yo, _, _ = oracle.block_step(h, fwd, rev, A, D)
    assert within(rel(y_ops.float().cpu().numpy(), oracle.block_step(h, fwd, rev, A, D, A_rev=Ar, D_rev=Dr)[0]),
                  TOL_BF16, "block step ops, separate reverse parameters, bf16 y")
    y32 = torch.empty((b, T, H, 64), device="cuda")
    bdssm.block_step_ops(d32, T, ops, tf, tr, Ad, Dd, y32)
    torch.cuda.synchronize()
    assert within(rel(y32.cpu().numpy(), yo), TOL_BF16, "block step ops vs oracle")


@pytest.mark.parametrize("cfg_index,steps", [(1, 3), (4, 2)])
def test_decode_graph_with_state_ops(cfg_index, steps):
    """The decode graph on the operand form: its steps equal eager bdssm_block_step_ops
    calls, its commit advances h, and it leaves h_ops = state_ops(advanced h), replay after
    replay (700M shape: one stream, T = 32, the small-batch kernel; 64 streams, T = 128,
    the bandwidth kernel)."""
    import torch
    cfg = configs.get(cfg_index)
    A, D = inputs.params(cfg)
    b, H, P, N, T = cfg.batch, cfg.nheads, cfg.headdim, cfg.d_state, cfg.block_len
    print(f"[case] decode graph with state ops: config {cfg_index}, {b} streams, {steps} steps + commit, "
          f"{H} heads, T={T}", flush=True)
    rng = np.random.default_rng(8)
    h0 = f32_round(rng.standard_normal((b, H, N, P)) * 0.05)
    fwd = [bdssm.seq_to_device(inputs.block(cfg, 0, k, inputs.FWD)) for k in range(steps)]
    rev = [bdssm.seq_to_device(inputs.block(cfg, 0, k, inputs.REV)) for k in range(steps)]
    # the graph commits block_len tokens (config 4's own commits take the oldest 32)
    clean = bdssm.seq_to_device(inputs.block(cfg, 0, 0, inputs.CLEAN, length=T))
    d = bdssm.dims(b, H, P, N, cfg.ngroups, cfg.in_dtype, bdssm.F32)
    Ad, Dd = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    h_init = torch.from_numpy(h0.astype(np.float32)).cuda()
    nb = bdssm.state_ops_bytes(d)

    h_e = h_init.clone()
    ops_e = torch.empty(nb, dtype=torch.uint8, device="cuda")
    bdssm.state_ops(d, h_e, ops_e)
    y_e = [torch.empty((b, T, H, P), device="cuda") for _ in range(steps)]
    for k in range(steps):
        bdssm.block_step_ops(d, T, ops_e, fwd[k], rev[k], Ad, Dd, y_e[k])
    bdssm.commit(d, T, clean, Ad, Dd, h_e)
    bdssm.state_ops(d, h_e, ops_e)
    torch.cuda.synchronize()

    h_g = h_init.clone()
    ops_g = torch.empty(nb, dtype=torch.uint8, device="cuda")
    y_g = [torch.empty((b, T, H, P), device="cuda") for _ in range(steps)]
    g = bdssm.DecodeGraph(d, T, h_g, fwd, rev, Ad, Dd, y_g, clean, None, h_ops=ops_g)
    try:
        for replay in range(3):
            h_g.copy_(h_init)
            bdssm.state_ops(d, h_g, ops_g)
            for t in y_g:
                t.zero_()
            g.launch()
            torch.cuda.synchronize()
            for k in range(steps):
                assert torch.equal(y_g[k], y_e[k]), (replay, k)
            assert torch.equal(h_g, h_e), replay
            assert torch.equal(ops_g, ops_e), replay
    finally:
        g.close()


@pytest.mark.parametrize("b,H,G,T,lat_off,hpws", [
    (12, 48, 1, 128, False, (1, 2, 3, 6)),   # 576 (stream, head) pairs: the bandwidth kernel
    (2, 12, 2, 77, False, (1, 2, 3, 6)),     # T > 32: 8 row blocks, ragged
    (3, 8, 2, 40, False, (1, 2, 4)),         # 4 row blocks, ragged
    (16, 32, 1, 32, False, (1, 2, 4)),       # 512 pairs, T = 32: 2 row blocks
    (2, 16, 4, 5, True, (1, 2)),             # 2 row blocks, mostly past T
])
def test_block_step_ops_bandwidth_kernel(launch_override, b, H, G, T, lat_off, hpws):
    """bdssm_block_step_ops where it runs the kernel that copies the operand-form state and x
    into LDS: y matches the oracle for float32 and bf16 y, with and without separate reverse
    parameters, also with D = 0 (the scan terms alone), and does not depend on how many
    heads a workgroup walks (bitwise)."""
    import torch
    fwd, rev, A, D, Ar, Dr, h = _case_inputs(b, H, G, T, 2000 + 7 * H + T)
    tf, tr = bdssm.seq_to_device(fwd), bdssm.seq_to_device(rev)
    Ad, Dd, Ard, Drd = (torch.from_numpy(v).cuda() for v in (A, D, Ar, Dr))
    Dz = torch.zeros_like(Dd)
    hd = torch.from_numpy(h.astype(np.float32)).cuda()
    d32 = bdssm.dims(b, H, 64, 128, G, bdssm.BF16, bdssm.F32)
    ops = torch.empty(bdssm.state_ops_bytes(d32), dtype=torch.uint8, device="cuda")
    bdssm.state_ops(d32, hd, ops)
    kernel = bdssm.KERNEL_BANDWIDTH if lat_off else bdssm.KERNEL_AUTO
    want = {
        (False, False): oracle.block_step(h, fwd, rev, A, D)[0],
        (False, True): oracle.block_step(h, fwd, rev, A, np.zeros_like(D))[0],
        (True, False): oracle.block_step(h, fwd, rev, A, D, A_rev=Ar, D_rev=Dr)[0],
    }
    for y_dt, tdt in ((bdssm.F32, torch.float32), (bdssm.BF16, torch.bfloat16)):
        d = bdssm.dims(b, H, 64, 128, G, bdssm.BF16, y_dt)
        for sep, dz in ((False, False), (False, True), (True, False)):
            first = None
            for hpw in hpws:
                launch_override(block_kernel=kernel, bw_heads=hpw)
                print(f"[case] block step ops (bandwidth) b={b} H={H} G={G} T={T} hpw={hpw} y={y_dt} "
                      f"separate={sep} D=0:{dz}", flush=True)
                y = torch.full((b, T, H, 64), float("nan"), dtype=tdt, device="cuda")
                A_rev, D_rev = (Ard, Drd) if sep else (Ad, None)
                bdssm.block_step_ops(d, T, ops, tf, tr, Ad, Dz if dz else Dd, y, A_rev=A_rev, D_rev=D_rev)
                torch.cuda.synchronize()
                if first is None:
                    first = y.clone()
                    assert within(rel(y.float().cpu().numpy(), want[(sep, dz)]), TOL_BF16,
                                  f"block step ops (bandwidth), y={y_dt}, separate={sep}, D=0:{dz}")
                else:
                    assert torch.equal(y, first), f"heads per workgroup {hpw} changed y"
    assert torch.equal(hd.cpu(), torch.from_numpy(h.astype(np.float32)))  # the state is read only


def test_config4_ops_running_set():
    """64 streams x 48 heads, T = 128, in the launch configuration the benchmark times: the
    operand form of cached states from a 1024-token prefix per stream, one block step from
    it; oracle on streams {0, 31, 63} (y with and without D x)."""
    import torch
    from harness import gpu_prefix, streams_of
    cfg = configs.get(4)
    A, D = inputs.params(cfg)
    b, H, P, N, G, T = cfg.batch, cfg.nheads, cfg.headdim, cfg.d_state, cfg.ngroups, cfg.block_len
    pre = inputs.prefix(cfg, length=1024)
    print("[case] c4 prefix for the cached states", flush=True)
    _, _, h = gpu_prefix(pre, A, D, cfg.chunk, want_y=False, want_cs=False)
    fwd = inputs.block(cfg, 0, 0, inputs.FWD)
    rev = inputs.block(cfg, 0, 0, inputs.REV)
    tf, tr = bdssm.seq_to_device(fwd), bdssm.seq_to_device(rev)
    hd = torch.from_numpy(np.asarray(h, np.float32)).cuda()
    d = bdssm.dims(b, H, P, N, G, cfg.in_dtype, bdssm.BF16)
    ops = torch.empty(bdssm.state_ops_bytes(d), dtype=torch.uint8, device="cuda")
    bdssm.state_ops(d, hd, ops)
    Ad = torch.from_numpy(A).cuda()
    sample = [0, 31, 63]
    hs = np.asarray(h, np.float64)[sample]
    fs, rs = streams_of(fwd, sample), streams_of(rev, sample)
    for Dv, label in ((D, "y"), (np.zeros_like(D), "y - D x")):
        print(f"[case] c4 block step ops, {label}", flush=True)
        y = torch.empty((b, T, H, P), dtype=torch.bfloat16, device="cuda")
        bdssm.block_step_ops(d, T, ops, tf, tr, Ad, torch.from_numpy(Dv).cuda(), y)
        torch.cuda.synchronize()
        yo, _, _ = oracle.block_step(hs, fs, rs, A, Dv)
        yg = y.float().cpu().numpy()[sample]
        assert within(rel(yg, yo), TOL_BF16, f"c4 block step ops, {label} (sampled streams)")
        assert within(max_head_rel(yg, yo, 2), 4 * TOL_BF16, f"c4 block step ops, {label}, worst head")


@pytest.mark.parametrize("b,H,G,T,form,with_y", [
    (1, 48, 1, 32, bdssm.STATE_OPS, False),     # 700M shape: one head per workgroup
    (64, 48, 1, 32, bdssm.STATE_OPS, False),    # running set: two heads per workgroup
    (64, 48, 1, 32, bdssm.STATE_BF16, False),
    (2, 12, 2, 77, bdssm.STATE_BF16, False),    # ragged block
    (1, 48, 1, 32, bdssm.STATE_OPS, True),      # with y: a commit and an encoding launch
    (2, 12, 2, 0, bdssm.STATE_OPS, False),      # no tokens: the copy only
])
def test_commit_refresh_bitwise(b, H, G, T, form, with_y):
    """bdssm_commit_refresh gives bitwise the state of bdssm_commit and the copy of
    bdssm_state_ops / bdssm_state_bf16 of that state."""
    import torch
    from test_oracle_pins import rand_seq
    rng = np.random.default_rng(300 + b + T)
    clean = rand_seq(rng, b, max(T, 1), H, 64, 128, G, 1)
    if T == 0:
        clean = inputs.Seq(*(np.ascontiguousarray(a[:, :0]) for a in (clean.x, clean.dt, clean.B, clean.C)), 1)
    A = (-np.exp(rng.uniform(0, np.log(16), H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    h0 = (rng.standard_normal((b, H, 128, 64)) * 0.1).astype(np.float32)
    d = bdssm.dims(b, H, 64, 128, G, bdssm.BF16, bdssm.F32)
    print(f"[case] commit refresh b={b} H={H} G={G} T={T} form={form} y={with_y}", flush=True)
    cd = bdssm.seq_to_device(clean) if T > 0 else tuple(torch.empty(16, device="cuda") for _ in range(4))
    Ad, Dd = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    nbytes = bdssm.state_ops_bytes(d) if form == bdssm.STATE_OPS else bdssm.state_bf16_bytes(d)
    h1 = torch.from_numpy(h0).cuda()
    c1 = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda")
    y1 = torch.empty((b, T, H, 64), device="cuda") if with_y else None
    bdssm.commit_refresh(d, T, cd, Ad, Dd, h1, c1, form, y1)
    h2 = torch.from_numpy(h0).cuda()
    c2 = torch.zeros((nbytes,), dtype=torch.uint8, device="cuda")
    y2 = torch.empty((b, T, H, 64), device="cuda") if with_y else None
    bdssm.commit(d, T, cd, Ad, Dd, h2, y2)
    (bdssm.state_ops if form == bdssm.STATE_OPS else bdssm.state_bf16)(d, h2, c2)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2)
    assert torch.equal(c1, c2)
    if with_y:
        assert torch.equal(y1, y2)


def test_commit_refresh_vector_alu_shape():
    """The tiny fp32 shape: the commit, then the bf16 copy (two launches), bitwise."""
    import torch
    from test_oracle_pins import rand_seq
    rng = np.random.default_rng(310)
    b, H, G, T = 2, 4, 1, 16
    clean = rand_seq(rng, b, T, H, 16, 16, G, 0)
    A = (-np.exp(rng.uniform(0, np.log(16), H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    h0 = (rng.standard_normal((b, H, 16, 16)) * 0.1).astype(np.float32)
    d = bdssm.dims(b, H, 16, 16, G, bdssm.F32, bdssm.F32)
    print("[case] commit refresh, fp32 inputs, d_state 16", flush=True)
    cd = bdssm.seq_to_device(clean)
    Ad, Dd = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    h1, h2 = torch.from_numpy(h0).cuda(), torch.from_numpy(h0).cuda()
    c1 = torch.empty(bdssm.state_bf16_bytes(d), dtype=torch.uint8, device="cuda")
    c2 = torch.empty_like(c1)
    bdssm.commit_refresh(d, T, cd, Ad, Dd, h1, c1, bdssm.STATE_BF16)
    bdssm.commit(d, T, cd, Ad, Dd, h2)
    bdssm.state_bf16(d, h2, c2)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2) and torch.equal(c1, c2)
    with pytest.raises(bdssm.BdssmError):
        bdssm.commit_refresh(d, T, cd, Ad, Dd, h1, c1, bdssm.STATE_OPS)   # no operand form at this shape
