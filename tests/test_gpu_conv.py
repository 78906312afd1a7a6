"""Parity of the convolution-state calls (bdssm_conv, bdssm_block_step_conv,
bdssm_commit_conv) with the float64 oracle, through the C ABI.

The convolution output is rounded to the input dtype on both sides; the GPU convolves in
float32 with the hardware exp, so a rounding may land one unit in the last place apart
(rarely). The new conv state is a copy of raw rows and must be bit-exact.
"""
import numpy as np
import pytest

import oracle
from bidirectional_mamba_state_amd import bdssm, configs, inputs
from bidirectional_mamba_state_amd.inputs import Seq, bf16_bits_to_f32

from harness import within, TOL_BF16, TOL_F32, rel, f32_round, to_np

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _dev(a):
    import torch
    return bdssm.to_device(a)


def _dev32(a):
    return bdssm.to_device(np.ascontiguousarray(a, np.float32))


def _dims(seq, y_dtype=bdssm.F32):
    b, _, H, P = seq.x.shape
    G, N = seq.B.shape[2], seq.B.shape[3]
    return bdssm.dims(b, H, P, N, G, seq.dtype, y_dtype)


def _decode(a, dtype):
    return bf16_bits_to_f32(a).astype(np.float64) if dtype == 1 else np.asarray(a, np.float64)


def _raw_np(t, dtype):
    """device tensor -> numpy in the handout format (uint16 bf16 bits or float32)"""
    import torch
    if dtype == 1:
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def _conv_params(cfg, W, direction, act=1):
    w, bias = inputs.conv_params(cfg, W, direction)
    wd, bd = _dev32(w), _dev32(bias)
    return (w, bias, act), bdssm.conv_params(wd, bd, act), (wd, bd)


def _history(cfg, W, b, seed):
    """A conv state: W-1 raw rows per stream, drawn like the inputs (x ~ N(0,1),
    B, C ~ N(0, 1/16)), in the input dtype."""
    rng = np.random.default_rng(seed)
    HP, GN = cfg.nheads * cfg.headdim, cfg.ngroups * cfg.d_state
    v = np.concatenate([rng.standard_normal((b, W - 1, HP)), 0.25 * rng.standard_normal((b, W - 1, 2 * GN))],
                       axis=2)
    return inputs.round_bf16_bits(v) if cfg.in_dtype == 1 else v.astype(np.float32)


def _check_conv_out(got, want, dtype, what):
    g = np.concatenate([_decode(a, dtype).reshape(a.shape[0], a.shape[1], -1) for a in got], axis=2)
    w = np.concatenate([_decode(a, dtype).reshape(a.shape[0], a.shape[1], -1) for a in want], axis=2)
    # one unit in the last place of the output dtype, plus float32 rounding of a sum whose
    # terms may cancel (absolute, scaled to the tensor's RMS)
    ulp = 2.0 ** -7 if dtype == 1 else 2.0 ** -22
    atol = 4e-6 * np.sqrt(np.mean(w * w))
    excess = np.max(np.abs(g - w) - ulp * np.abs(w))
    frac = np.mean(g != w)
    print(f"[parity] {what}: rel {rel(g, w):.2e}, max excess over the bound {excess:.2e} "
          f"(atol {atol:.1e}), unequal fraction {frac:.2e}", flush=True)
    assert np.all(np.abs(g - w) <= ulp * np.abs(w) + atol), what
    assert rel(g, w) < (1e-3 if dtype == 1 else 1e-6), what
    if dtype == 1:
        assert frac < 1e-3, what


@pytest.mark.parametrize("cfg_index,W,act,length", [
    (0, 4, 1, 37), (0, 1, 0, 16), (0, 3, 1, 2), (1, 4, 1, 32), (1, 2, 0, 129), (1, 4, 1, 1000)])
def test_conv_forward_reverse_and_state(cfg_index, W, act, length):
    """bdssm_conv both ways against oracle_conv: outputs (to one unit in the last place),
    the new conv state (bit-exact), in place and out of place; long runs (> 512 tokens use
    16-token runs per thread) and segments shorter than the history."""
    import torch
    cfg = configs.get(cfg_index)
    _case(f"conv config {cfg_index} W={W} act={act} len={length}")
    seq = inputs.block(cfg, 0, 0, inputs.FWD, length=length)
    d = _dims(seq)
    (w, bias, _), cp, keep = _conv_params(cfg, W, inputs.FWD, act)
    hist = _history(cfg, W, seq.x.shape[0], 5)
    raw = bdssm.seq_to_device(seq)
    for reverse in (False, True):
        out = tuple(torch.empty_like(t) for t in raw)
        state_in = None if reverse else _dev(hist)
        state_out = None if reverse else torch.empty_like(state_in)
        bdssm.conv(d, length, cp, reverse, state_in, raw, out, state_out)
        torch.cuda.synchronize()
        o, so = oracle.conv(seq, w, bias, act, reverse=reverse, state_in=None if reverse else hist)
        got = [_raw_np(out[i], seq.dtype) for i in (0, 2, 3)]
        _check_conv_out(got, [o.x, o.B, o.C], seq.dtype, f"conv {'reverse' if reverse else 'forward'}")
        if not reverse:
            assert np.array_equal(_raw_np(state_out, seq.dtype), so), "new conv state"
            # in place: the same result
            st = _dev(hist)
            out2 = tuple(torch.empty_like(t) for t in raw)
            bdssm.conv(d, length, cp, False, st, raw, out2, st)
            torch.cuda.synchronize()
            assert np.array_equal(_raw_np(st, seq.dtype), so), "new conv state, in place"
            for i in (0, 2, 3):
                assert torch.equal(out[i], out2[i])
    # from a zero history (the start of a sequence)
    out = tuple(torch.empty_like(t) for t in raw)
    so_d = torch.empty((seq.x.shape[0], W - 1, hist.shape[2]), dtype=raw[0].dtype, device="cuda")
    bdssm.conv(d, length, cp, False, None, raw, out, so_d)
    torch.cuda.synchronize()
    o, so = oracle.conv(seq, w, bias, act, state_in=None)
    _check_conv_out([_raw_np(out[i], seq.dtype) for i in (0, 2, 3)], [o.x, o.B, o.C], seq.dtype,
                    "conv forward from zero history")
    assert np.array_equal(_raw_np(so_d, seq.dtype), so)


def _block_case(cfg, W_f, W_r, act, sep_rev, y_dtype):
    import torch
    A, D = inputs.params(cfg)
    rng = np.random.default_rng(77)
    H = cfg.nheads
    A_rev = (-np.exp(rng.uniform(0, np.log(16), H))).astype(np.float32) if sep_rev else None
    D_rev = rng.standard_normal(H).astype(np.float32) if sep_rev else None
    pre = inputs.prefix(cfg, length=min(cfg.prefix_len, 256))
    _, _, h = oracle.scan(pre, A, D, cfg.chunk, want_y=False, want_chunk_states=False)
    h = f32_round(h)
    fwd = inputs.block(cfg, 0, 0, inputs.FWD)
    rev = inputs.block(cfg, 0, 0, inputs.REV)
    b, T, _, P = fwd.x.shape
    cf, cpf, kf = _conv_params(cfg, W_f, inputs.FWD, act)
    cr, cpr, kr = _conv_params(cfg, W_r, inputs.REV, act)
    hist = _history(cfg, W_f, b, 6)
    d = _dims(fwd, y_dtype)
    ws = torch.empty(2 * bdssm.conv_workspace(d, T), dtype=torch.uint8, device="cuda")
    hd, histd = _dev32(h), (_dev(hist) if W_f > 1 else None)
    fd, rd = bdssm.seq_to_device(fwd), bdssm.seq_to_device(rev)
    ytd = torch.bfloat16 if y_dtype == bdssm.BF16 else torch.float32
    tol = TOL_BF16 if cfg.in_dtype == 1 or y_dtype == bdssm.BF16 else TOL_F32
    for Dv, Drv, what in ((D, D_rev, "y"), (np.zeros_like(D), None, "y - skip terms")):
        y = torch.empty((b, T, H, P), dtype=ytd, device="cuda")
        bdssm.block_step_conv(d, T, cpf, cpr, hd, histd, fd, rd, _dev32(A), _dev32(Dv), y, ws,
                              A_rev=None if A_rev is None else _dev32(A_rev),
                              D_rev=None if Drv is None else _dev32(Drv))
        torch.cuda.synchronize()
        yo, _, _ = oracle.block_step_conv(h, hist if W_f > 1 else np.zeros((b, 0, hist.shape[2]), hist.dtype),
                                          fwd, rev, cf, cr, A, Dv, A_rev=A_rev, D_rev=Drv)
        assert within(rel(to_np(y), yo), tol, f"block step with conv, {what}")
    # the cached SSM state and conv state are read only
    assert np.array_equal(hd.cpu().numpy(), h.astype(np.float32))
    if W_f > 1:
        assert np.array_equal(_raw_np(histd, fwd.dtype), hist)


@pytest.mark.parametrize("cfg_index,W_f,W_r,act,sep_rev,y_dtype", [
    (0, 4, 4, 1, False, bdssm.F32), (1, 4, 4, 1, False, bdssm.F32), (1, 4, 4, 1, True, bdssm.BF16),
    (1, 4, 2, 1, False, bdssm.F32), (1, 1, 1, 0, False, bdssm.F32), (3, 4, 4, 1, False, bdssm.BF16)])
def test_block_step_conv(cfg_index, W_f, W_r, act, sep_rev, y_dtype):
    """bdssm_block_step_conv against the oracle (convolution, then eqs. (11)-(13)): one
    launch for both directions' convolutions when their widths match, two otherwise; with
    and without separate reverse parameters; y with and without the skip terms."""
    cfg = configs.get(cfg_index)
    _case(f"block step conv config {cfg_index} W=({W_f},{W_r}) act={act} sep_rev={sep_rev} y={y_dtype}")
    _block_case(cfg, W_f, W_r, act, sep_rev, y_dtype)


@pytest.mark.parametrize("cfg_index", [0, 1])
def test_prefix_then_steps_then_commits_with_conv(cfg_index):
    """The whole path with conv state: a prefix convolved from a zero history (its conv
    state written) and scanned, a block step from both states, then three commits that
    advance both states in place; against the oracle's composition of the same steps."""
    import torch
    cfg = configs.get(cfg_index)
    _case(f"conv path config {cfg_index}")
    A, D = inputs.params(cfg)
    W = 4
    cf, cpf, kf = _conv_params(cfg, W, inputs.FWD)
    cr, cpr, kr = _conv_params(cfg, W, inputs.REV)
    L = min(cfg.prefix_len, 512)
    pre = inputs.prefix(cfg, length=L)
    b = pre.x.shape[0]
    d = _dims(pre)
    # prefix: convolve, then scan
    raw = bdssm.seq_to_device(pre)
    post = tuple(torch.empty_like(t) for t in raw)
    CH = cfg.nheads * cfg.headdim + 2 * cfg.ngroups * cfg.d_state
    cs = torch.empty((b, W - 1, CH), dtype=raw[0].dtype, device="cuda")
    bdssm.conv(d, L, cpf, False, None, raw, post, cs)
    post = (post[0], raw[1], post[2], post[3])
    h = torch.empty((b, cfg.nheads, cfg.d_state, cfg.headdim), device="cuda")
    wsb = bdssm.prefix_scan_workspace(d, L, cfg.chunk, False, False)
    wsp = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    bdssm.prefix_scan(d, L, cfg.chunk, post, _dev32(A), _dev32(D), None, None, None, h, wsp, wsb)
    torch.cuda.synchronize()
    po, so = oracle.conv(pre, *cf, state_in=None)
    _, _, ho = oracle.scan(po, A, D, cfg.chunk, want_y=False, want_chunk_states=False)
    tol = TOL_BF16 if cfg.in_dtype == 1 else TOL_F32
    assert np.array_equal(_raw_np(cs, pre.dtype), so), "prefix conv state"
    assert within(rel(to_np(h), ho), tol, "prefix state over convolved inputs")
    # a block step from the GPU's states
    fwd = inputs.block(cfg, 0, 0, inputs.FWD)
    rev = inputs.block(cfg, 0, 0, inputs.REV)
    T = fwd.x.shape[1]
    ws = torch.empty(2 * bdssm.conv_workspace(d, T), dtype=torch.uint8, device="cuda")
    y = torch.empty((b, T, cfg.nheads, cfg.headdim), device="cuda")
    bdssm.block_step_conv(d, T, cpf, cpr, h, cs, bdssm.seq_to_device(fwd), bdssm.seq_to_device(rev),
                          _dev32(A), _dev32(D), y, ws)
    torch.cuda.synchronize()
    hg, sg = to_np(h), _raw_np(cs, pre.dtype)
    yo, _, _ = oracle.block_step_conv(hg, sg, fwd, rev, cf, cr, A, D)
    assert within(rel(to_np(y), yo), tol, "block step from the prefix's states")
    # three commits, both states advanced in place
    hh, ss = ho, so
    for k in range(3):
        clean = inputs.block(cfg, k, 0, inputs.CLEAN)
        bdssm.commit_conv(d, T, cpf, bdssm.seq_to_device(clean), _dev32(A), _dev32(D), h, cs, ws)
        hh, ss, _ = oracle.commit_conv(hh, ss, clean, cf, A, D)
    torch.cuda.synchronize()
    assert np.array_equal(_raw_np(cs, pre.dtype), ss), "conv state after the commits"
    assert within(rel(to_np(h), hh), tol, "SSM state after the commits")
