"""The decode-loop graph (bdssm_decode_graph_*): the steps of one active block and its
commit, recorded once and replayed, give exactly the results of the eager calls, replay
after replay, with unrelated eager work in between; and the oracle's results."""
import numpy as np
import pytest

import oracle
from bidirectional_mamba_state_amd import bdssm, configs, inputs
from harness import TOL_BF16, f32_round, rel, within

pytestmark = pytest.mark.gpu


def test_decode_graph_replays_match_eager_calls():
    import torch
    cfg = configs.get(1)   # 700M shape: 48 heads x 64, d_state 128, T = 32
    A, D = inputs.params(cfg)
    H, P, N, T, steps = cfg.nheads, cfg.headdim, cfg.d_state, cfg.block_len, 4
    print(f"[case] decode graph: {steps} block steps + commit, 48 heads, T={T}", flush=True)
    rng = np.random.default_rng(7)
    h0 = f32_round(rng.standard_normal((1, H, N, P)) * 0.05)
    fwd_np = [inputs.block(cfg, 0, k, inputs.FWD) for k in range(steps)]
    rev_np = [inputs.block(cfg, 0, k, inputs.REV) for k in range(steps)]
    clean_np = inputs.block(cfg, 0, 0, inputs.CLEAN)
    d = bdssm.dims(1, H, P, N, 1, cfg.in_dtype, bdssm.F32)
    Ad, Dd = torch.from_numpy(A).cuda(), torch.from_numpy(D).cuda()
    fwd = [bdssm.seq_to_device(s) for s in fwd_np]
    rev = [bdssm.seq_to_device(s) for s in rev_np]
    clean = bdssm.seq_to_device(clean_np)
    h_init = torch.from_numpy(h0.astype(np.float32)).cuda()

    # eager calls
    h_e = h_init.clone()
    y_e = [torch.empty((1, T, H, P), device="cuda") for _ in range(steps)]
    yc_e = torch.empty((1, T, H, P), device="cuda")
    for k in range(steps):
        bdssm.block_step(d, T, h_e, fwd[k], rev[k], Ad, Dd, y_e[k])
    bdssm.commit(d, T, clean, Ad, Dd, h_e, yc_e)
    torch.cuda.synchronize()

    # the same calls as one graph
    h_g = h_init.clone()
    y_g = [torch.empty((1, T, H, P), device="cuda") for _ in range(steps)]
    yc_g = torch.empty((1, T, H, P), device="cuda")
    g = bdssm.DecodeGraph(d, T, h_g, fwd, rev, Ad, Dd, y_g, clean, yc_g)
    other_y = torch.empty((1, T, H, P), device="cuda")
    try:
        for replay in range(3):
            h_g.copy_(h_init)
            for t in y_g:
                t.zero_()
            yc_g.zero_()
            g.launch()
            torch.cuda.synchronize()
            for k in range(steps):
                assert torch.equal(y_g[k], y_e[k]), (replay, k)
            assert torch.equal(yc_g, yc_e), replay
            assert torch.equal(h_g, h_e), replay
            # unrelated eager work between replays
            bdssm.block_step(d, T, h_init, fwd[0], rev[0], Ad, Dd, other_y)
            torch.cuda.synchronize()
    finally:
        g.close()

    # and the oracle's results
    yo, _, _ = oracle.block_step(h0, fwd_np[steps - 1], rev_np[steps - 1], A, D)
    assert within(rel(y_e[steps - 1].cpu().numpy(), yo), TOL_BF16, "graph step y")
    ho, yco = oracle.commit(h0, clean_np, A, D, want_y=True)
    assert within(rel(h_e.cpu().numpy(), ho), TOL_BF16, "graph commit state")
    assert within(rel(yc_e.cpu().numpy(), yco), TOL_BF16, "graph commit y")
