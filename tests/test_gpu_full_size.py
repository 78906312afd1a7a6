"""Parity at the running-set workload's stated size, in the launch configuration the
benchmark times, and bitwise repeatability of the prefix scan and the commit.

Running set (64 streams x 48 heads, d_state 128, headdim 64, bf16 inputs): every stream's
cached state is built by one batch-64 state-only prefix scan over its own 32,768 tokens (the
x tensor alone holds 6.4 G elements, so element offsets pass 2^32), then put in operand form;
16 denoising steps of the 128-token window follow, with distinct inputs, then the commit of
the oldest 32-token block. Streams {0, 31, 63} come from the seeded host generator and are
checked against the oracle; the other 61 are drawn on the device (streams are independent).
"""
import numpy as np
import pytest

import oracle
from bidirectional_mamba_state_amd import bdssm, configs, inputs
from harness import TOL_BF16, max_head_rel, mixed_seq, rel, within

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def test_config4_full_size_running_set():
    import torch
    cfg = configs.get(4)
    b, H, P, N, G, L, Q = cfg.batch, cfg.nheads, cfg.headdim, cfg.d_state, cfg.ngroups, cfg.prefix_len, cfg.chunk
    T, S, TC = cfg.block_len, cfg.steps_per_block, cfg.commit_len
    sample = [0, 31, 63]
    A, D = inputs.params(cfg)
    Ad, Dd = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    Dz = torch.zeros_like(Dd)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(404)
    d = bdssm.dims(b, H, P, N, G, cfg.in_dtype, bdssm.F32)

    _case(f"c4 prefix: {b} streams x {L} tokens, state only, one call")
    pre_dev, pre_host = mixed_seq(cfg, gen, inputs.PREFIX, 0, inputs.FWD, L, sample)
    assert pre_dev[0].numel() > 2 ** 32
    h = torch.empty((b, H, N, P), device="cuda")
    wsb = bdssm.prefix_scan_workspace(d, L, Q, False, False)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    bdssm.prefix_scan(d, L, Q, pre_dev, Ad, Dd, None, None, None, h, ws, wsb)
    torch.cuda.synchronize()
    del pre_dev
    torch.cuda.empty_cache()
    _, _, ho = oracle.scan(pre_host, A, D, Q, want_y=False, want_chunk_states=False)
    del pre_host
    hg = h.cpu().numpy().astype(np.float64)
    assert within(rel(hg[sample], ho), TOL_BF16, "c4 prefix states (streams 0, 31, 63)")
    assert within(max_head_rel(hg[sample], ho, 1), 4 * TOL_BF16, "c4 prefix states, worst head")
    assert np.isfinite(hg).all()
    hs = hg[sample]      # the oracle continues from the GPU's float32 states

    ops = torch.empty(bdssm.state_ops_bytes(d), dtype=torch.uint8, device="cuda")
    bdssm.state_ops(d, h, ops)
    h_before = h.clone()
    for s in range(S):
        fwd_dev, fwd = mixed_seq(cfg, gen, inputs.BLOCK(0), s, inputs.FWD, T, sample)
        rev_dev, rev = mixed_seq(cfg, gen, inputs.BLOCK(0), s, inputs.REV, T, sample)
        checks = ((D, Dd, "y"), (np.zeros_like(D), Dz, "y - D x")) if s in (0, S - 1) else ((D, Dd, "y"),)
        for Dv, Dt, what in checks:
            _case(f"c4 step {s}: {what}")
            y = torch.empty((b, T, H, P), device="cuda")
            bdssm.block_step_ops(d, T, ops, fwd_dev, rev_dev, Ad, Dt, y)
            torch.cuda.synchronize()
            yo, _, _ = oracle.block_step(hs, fwd, rev, A, Dv)
            yg = y.cpu().numpy()[sample]
            assert within(rel(yg, yo), TOL_BF16, f"c4 step {s} {what} (streams 0, 31, 63)")
            if s in (0, S - 1):
                assert within(max_head_rel(yg, yo, 2), 4 * TOL_BF16, f"c4 step {s} {what}, worst head")
    assert torch.equal(h, h_before), "the block steps wrote the cached states"

    _case(f"c4 commit of the oldest {TC}-token block")
    clean_dev, clean = mixed_seq(cfg, gen, inputs.BLOCK(0), 0, inputs.CLEAN, TC, sample)
    bdssm.commit(d, TC, clean_dev, Ad, Dd, h)
    torch.cuda.synchronize()
    hn, _ = oracle.commit(hs, clean, A, D)
    assert within(rel(h.cpu().numpy()[sample], hn), TOL_BF16, "c4 post-commit states (streams 0, 31, 63)")


def _prefix_outputs(torch, d, L, Q, seq, Ad, Dd, with_y, with_cs):
    b, H, P, N = d.batch, d.nheads, d.headdim, d.d_state
    y = torch.full((b, L, H, P), float("nan"), device="cuda") if with_y else None
    cs = torch.full((b, -(-L // Q), H, N, P), float("nan"), device="cuda") if with_cs else None
    ho = torch.full((b, H, N, P), float("nan"), device="cuda")
    wsb = bdssm.prefix_scan_workspace(d, L, Q, with_y, with_cs)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    bdssm.prefix_scan(d, L, Q, seq, Ad, Dd, None, y, cs, ho, ws, wsb)
    torch.cuda.synchronize()
    return [t for t in (y, cs, ho) if t is not None]


@pytest.mark.parametrize("cfg_index,with_y,with_cs", [(2, True, True), (1, True, False), (2, False, True)])
def test_prefix_scan_bitwise_repeatable(cfg_index, with_y, with_cs):
    """Three runs of the same prefix scan give identical bits (y, chunk states, final state):
    every reduction has a fixed order and the barriers' partial waits let no read see a copy
    still in flight. The 65,536-token scan with chunk states is the multi-segment plan whose
    full pass waits on exactly the y stores at its top barrier."""
    import torch
    cfg = configs.get(cfg_index)
    A, D = inputs.params(cfg)
    Ad, Dd = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    L, Q = cfg.prefix_len, cfg.chunk
    seq = bdssm.seq_to_device(inputs.prefix(cfg))
    d = bdssm.dims(cfg.batch, cfg.nheads, cfg.headdim, cfg.d_state, cfg.ngroups, cfg.in_dtype, bdssm.F32)
    _case(f"prefix scan x3, config {cfg_index}, y={with_y} chunk states={with_cs}")
    first = _prefix_outputs(torch, d, L, Q, seq, Ad, Dd, with_y, with_cs)
    assert all(bool(torch.isfinite(t).all()) for t in first)
    for rep in range(2):
        again = _prefix_outputs(torch, d, L, Q, seq, Ad, Dd, with_y, with_cs)
        for a, b in zip(first, again):
            assert torch.equal(a, b), f"run {rep + 2} differs"


@pytest.mark.parametrize("cfg_index", [1, 4])
def test_commit_bitwise_repeatable(cfg_index):
    """Three commits of the same block from the same state give identical bits."""
    import torch
    cfg = configs.get(cfg_index)
    A, D = inputs.params(cfg)
    Ad, Dd = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    b, H, P, N = cfg.batch, cfg.nheads, cfg.headdim, cfg.d_state
    d = bdssm.dims(b, H, P, N, cfg.ngroups, cfg.in_dtype, bdssm.F32)
    clean = bdssm.seq_to_device(inputs.block(cfg, 0, 0, inputs.CLEAN))
    rng = np.random.default_rng(77)
    h0 = torch.from_numpy((rng.standard_normal((b, H, N, P)) * 0.1).astype(np.float32)).cuda()
    _case(f"commit x3, config {cfg_index}")
    outs = []
    for _ in range(3):
        h = h0.clone()
        y = torch.empty((b, cfg.commit_len, H, P), device="cuda")
        bdssm.commit(d, cfg.commit_len, clean, Ad, Dd, h, y)
        torch.cuda.synchronize()
        outs.append((h, y))
    for h, y in outs[1:]:
        assert torch.equal(h, outs[0][0]) and torch.equal(y, outs[0][1])
