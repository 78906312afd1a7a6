"""The full-window bidirectional scan (bdssm_full_window) against the oracle: forward and
reverse scans over the whole window of prefix and active block, from zero states, every
token's output. At the 700M shape the window is the 8192-token prefix plus the 32-token
block; on the block's tokens the result also equals the block step from the prefix scan's
state (two different kernel paths)."""
import numpy as np
import pytest

import oracle
from bidirectional_mamba_state_amd import bdssm, configs, inputs
from bidirectional_mamba_state_amd.inputs import Seq
from harness import TOL_BF16, TOL_F32, gpu_block_step, gpu_prefix, max_head_rel, rel, within

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _cat(u, v):
    return Seq(*(np.concatenate([p, q], axis=1) for p, q in zip((u.x, u.dt, u.B, u.C), (v.x, v.dt, v.B, v.C))),
               u.dtype)


def gpu_full_window(fwd, rev, A, D, chunk, A_rev=None, D_rev=None, y_dtype=bdssm.F32):
    import torch
    b, L, H, P = fwd.x.shape
    G, N = fwd.B.shape[2], fwd.B.shape[3]
    d = bdssm.dims(b, H, P, N, G, fwd.dtype, y_dtype)
    dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    tdt = torch.bfloat16 if y_dtype == bdssm.BF16 else torch.float32
    y = torch.full((b, L, H, P), float("nan"), dtype=tdt, device="cuda")
    wsb = bdssm.full_window_workspace(d, L, chunk)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    bdssm.full_window(d, L, chunk, bdssm.seq_to_device(fwd), bdssm.seq_to_device(rev), dev(A), dev(D),
                      dev(A_rev), dev(D_rev), y, ws)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def _check(fwd, rev, A, D, chunk, A_rev=None, D_rev=None, label="", y_dtype=bdssm.F32):
    tol = TOL_BF16 if fwd.dtype == bdssm.BF16 else TOL_F32
    if y_dtype == bdssm.BF16:
        tol = max(tol, 5e-3)
    _case(f"full window {label}: len={fwd.length} chunk={chunk} separate={A_rev is not None} y_dtype={y_dtype}")
    y = gpu_full_window(fwd, rev, A, D, chunk, A_rev, D_rev, y_dtype)
    yo = oracle.full_window(fwd, rev, A, D, A_rev=A_rev, D_rev=D_rev)
    assert within(rel(y, yo), tol, f"full window y {label}")
    assert within(max_head_rel(y, yo, 2), 4 * tol, f"full window y {label}, worst head")
    Dz = np.zeros_like(D)
    yz = gpu_full_window(fwd, rev, A, Dz, chunk, A_rev, None, y_dtype)
    yzo = oracle.full_window(fwd, rev, A, Dz, A_rev=A_rev)
    assert within(rel(yz, yzo), tol, f"full window y - skip terms {label}")
    return y


def test_full_window_700m_shape():
    """The 700M shape's window: the 8192-token prefix and the 32-token block, both
    directions' own inputs; the block tokens' outputs equal the block step's from the
    prefix scan's state."""
    cfg = configs.get(1)
    A, D = inputs.params(cfg)
    L, T = cfg.prefix_len, cfg.block_len
    pre_f = inputs.prefix(cfg)
    pre_r = inputs.segment(cfg, inputs.PREFIX, 0, inputs.REV, L)
    blk_f = inputs.block(cfg, 0, 0, inputs.FWD)
    blk_r = inputs.block(cfg, 0, 0, inputs.REV)
    fwd, rev = _cat(pre_f, blk_f), _cat(pre_r, blk_r)
    y = _check(fwd, rev, A, D, cfg.chunk, label="c1")
    # the block's tokens: the block step from the prefix's cached state
    _, _, h = gpu_prefix(pre_f, A, D, cfg.chunk, want_y=False, want_cs=False)
    yb = gpu_block_step(np.asarray(h, np.float32).astype(np.float64), blk_f, blk_r, A, D)
    assert within(rel(y[:, L:], yb), TOL_BF16, "full window on the block == block step")
    # separate reverse parameters and bf16 y
    rng = np.random.default_rng(9)
    Ar = (-np.exp(rng.uniform(0, np.log(16), cfg.nheads))).astype(np.float32)
    Dr = rng.standard_normal(cfg.nheads).astype(np.float32)
    _check(fwd, rev, A, D, cfg.chunk, A_rev=Ar, D_rev=Dr, label="c1 separate reverse parameters")
    _check(fwd, rev, A, D, cfg.chunk, label="c1 bf16 y", y_dtype=bdssm.BF16)


def test_full_window_tiny_fp32():
    """The tiny fp32 shape (vector-ALU path): the 256-token prefix plus the 16-token block."""
    cfg = configs.get(0)
    A, D = inputs.params(cfg)
    L = cfg.prefix_len
    fwd = _cat(inputs.prefix(cfg), inputs.block(cfg, 0, 0, inputs.FWD))
    rev = _cat(inputs.segment(cfg, inputs.PREFIX, 0, inputs.REV, L), inputs.block(cfg, 0, 0, inputs.REV))
    _check(fwd, rev, A, D, cfg.chunk, label="c0")
    rng = np.random.default_rng(10)
    Ar = (-np.exp(rng.uniform(0, np.log(16), cfg.nheads))).astype(np.float32)
    _check(fwd, rev, A, D, 16, A_rev=Ar, D_rev=D[::-1].copy(), label="c0 chunk 16 separate")


@pytest.mark.parametrize("b,H,G,L,chunk,dtype", [
    (1, 4, 1, 1, 64, bdssm.BF16),        # one token
    (2, 6, 2, 63, 64, bdssm.BF16),       # shorter than a sub-chunk
    (1, 4, 2, 1000, 128, bdssm.BF16),    # ragged tail, several segments
    (3, 8, 4, 4160, 256, bdssm.BF16),    # several segments per (stream, head), groups
    (64, 8, 1, 200, 64, bdssm.BF16),     # one segment per (stream, head)
    (2, 4, 2, 333, 32, bdssm.F32),       # vector-ALU path, ragged
])
def test_full_window_shapes(b, H, G, L, chunk, dtype):
    from test_oracle_pins import rand_seq
    rng = np.random.default_rng(L + 7 * H + b)
    P, N = (64, 128) if dtype == bdssm.BF16 else (16, 16)
    fwd = rand_seq(rng, b, L, H, P, N, G, dtype)
    rev = rand_seq(rng, b, L, H, P, N, G, dtype)
    A = (-np.exp(rng.uniform(0, np.log(16), H))).astype(np.float32)
    Ar = (-np.exp(rng.uniform(0, np.log(16), H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    _check(fwd, rev, A, D, chunk, A_rev=Ar, label=f"b={b} H={H} G={G}")


def test_full_window_bitwise_repeatable():
    """Three runs give identical bits (the reverse half reads the forward half's y)."""
    cfg = configs.get(1)
    A, D = inputs.params(cfg)
    fwd = inputs.prefix(cfg, length=2048)
    rev = inputs.segment(cfg, inputs.PREFIX, 0, inputs.REV, 2048)
    _case("full window x3, 2048 tokens, 700M shape")
    ys = [gpu_full_window(fwd, rev, A, D, cfg.chunk) for _ in range(3)]
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])
