"""The block step's variants (bdssm_block_step_variant): the bf16 cached state
(bdssm_state_bf16) and skip weights per head and channel, against the oracle, on every
kernel path (vector-ALU at the tiny fp32 shape; the small-batch kernel at the 700M shape;
the bandwidth kernels at many (stream, head) pairs), plus the identities with the plain
calls."""
import numpy as np
import pytest

import oracle
from bidirectional_mamba_state_amd import bdssm, configs, inputs
from harness import TOL_BF16, TOL_F32, f32_round, max_head_rel, rel, within

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _bf16_layout(h):
    """[b][H][N][P] float -> [b][H][N/8][P][8] uint16 bf16 bits (round to nearest even)."""
    b, H, N, P = h.shape
    bits = inputs.round_bf16_bits(np.asarray(h, np.float64))
    return bits.reshape(b, H, N // 8, 8, P).transpose(0, 1, 2, 4, 3).copy()


def _bf16_values(h):
    """The bf16 state's values, float64 [b][H][N][P] (what the kernels read)."""
    return inputs.bf16_bits_to_f32(inputs.round_bf16_bits(np.asarray(h, np.float64))).astype(np.float64)


def _dev(a):
    import torch
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


@pytest.mark.parametrize("N,P", [(128, 64), (16, 16)])
def test_state_bf16_encoding(N, P):
    import torch
    rng = np.random.default_rng(21 + N)
    b, H = 2, 3
    h = (rng.standard_normal((b, H, N, P)) * np.exp(rng.uniform(-20, 20, (b, H, N, P)))).astype(np.float32)
    h[0, 0, 0, :8] = 0.0
    h[0, 0, 1, :8] = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x3F80FFFF] * 2, np.uint32).view(np.float32)
    _case(f"bf16 state encoding N={N} P={P}")
    d = bdssm.dims(b, H, P, N, 1, bdssm.BF16, bdssm.F32)
    out = torch.full((bdssm.state_bf16_bytes(d) // 2,), -1, dtype=torch.int16, device="cuda")
    hd = torch.from_numpy(h).cuda()
    bdssm.state_bf16(d, hd, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16).reshape(b, H, N // 8, P, 8)
    assert np.array_equal(got, _bf16_layout(h))
    assert torch.equal(hd.cpu(), torch.from_numpy(h))


def _run(d, T, state, form, fwd, rev, A, D, A_rev=None, D_rev=None, dch=False, y_dtype=bdssm.F32):
    import torch
    b, _, H, P = fwd.x.shape
    y = torch.full((b, T, H, P), float("nan"), dtype=torch.bfloat16 if y_dtype == bdssm.BF16 else torch.float32,
                   device="cuda")
    bdssm.block_step_variant(d, T, state, form, bdssm.seq_to_device(fwd), bdssm.seq_to_device(rev), _dev(A),
                             _dev(D), y, A_rev=_dev(A_rev), D_rev=_dev(D_rev), skip_per_channel=dch)
    torch.cuda.synchronize()
    return y


def _states(torch, d, h):
    """float32, operand form and bf16 forms of the cached state h (numpy float64)."""
    hd = torch.from_numpy(np.asarray(h, np.float32)).cuda()
    forms = {bdssm.STATE_F32: hd}
    if d.in_dtype == bdssm.BF16 and d.d_state == 128 and d.headdim == 64:
        ops = torch.empty(bdssm.state_ops_bytes(d), dtype=torch.uint8, device="cuda")
        bdssm.state_ops(d, hd, ops)
        forms[bdssm.STATE_OPS] = ops
    hb = torch.empty(bdssm.state_bf16_bytes(d), dtype=torch.uint8, device="cuda")
    bdssm.state_bf16(d, hd, hb)
    forms[bdssm.STATE_BF16] = hb
    return forms


def _check_variants(fwd, rev, h, A, D, Ar, Dr, Dc, Drc, label):
    """Every state form x per-head / per-channel skip weights against the oracle."""
    import torch
    b, T, H, P = fwd.x.shape
    G, N = fwd.B.shape[2], fwd.B.shape[3]
    tol = TOL_BF16 if fwd.dtype == bdssm.BF16 else TOL_F32
    d = bdssm.dims(b, H, P, N, G, fwd.dtype, bdssm.F32)
    forms = _states(torch, d, h)
    hb = _bf16_values(h)
    for form, state in forms.items():
        hs = hb if form == bdssm.STATE_BF16 else h
        name = {bdssm.STATE_F32: "f32", bdssm.STATE_OPS: "ops", bdssm.STATE_BF16: "bf16"}[form]
        _case(f"variants {label}: state {name}, per-channel skip weights")
        y = _run(d, T, state, form, fwd, rev, A, Dc, Ar, Drc, dch=True)
        yo = oracle.block_step_per_channel(hs, fwd, rev, A, Dc, A_rev=Ar, D_rev=Drc)
        assert within(rel(y.cpu().numpy(), yo), tol, f"{label} {name} per-channel D, D_rev")
        # the scan terms alone, each state form against the oracle on the same state values
        yz = _run(d, T, state, form, fwd, rev, A, np.zeros_like(D), Ar, None)
        yzo, _, _ = oracle.block_step(hs, fwd, rev, A, np.zeros_like(D), A_rev=Ar)
        assert within(rel(yz.cpu().numpy(), yzo), tol, f"{label} {name} y - skip terms")
        assert within(max_head_rel(yz.cpu().numpy(), yzo, 2), 4 * tol, f"{label} {name} y - skip terms, worst head")
        # per-channel weights that repeat the per-head ones give the per-head step, bitwise
        y1 = _run(d, T, state, form, fwd, rev, A, np.repeat(D[:, None], P, 1), Ar, np.repeat(Dr[:, None], P, 1),
                  dch=True)
        y2 = _run(d, T, state, form, fwd, rev, A, D, Ar, Dr)
        assert torch.equal(y1, y2), f"{label} {name}: per-channel repeat of per-head weights"
        yo2, _, _ = oracle.block_step(hs, fwd, rev, A, D, A_rev=Ar, D_rev=Dr)
        assert within(rel(y2.cpu().numpy(), yo2), tol, f"{label} {name} per-head D, D_rev")
    # identities with the plain calls
    hd = forms[bdssm.STATE_F32]
    ye = torch.empty((b, T, H, P), device="cuda")
    bdssm.block_step_ex(d, T, hd, bdssm.seq_to_device(fwd), bdssm.seq_to_device(rev), _dev(A), _dev(D), _dev(Ar),
                        _dev(Dr), ye)
    torch.cuda.synchronize()
    assert torch.equal(_run(d, T, hd, bdssm.STATE_F32, fwd, rev, A, D, Ar, Dr), ye)
    if bdssm.STATE_OPS in forms:
        yp = torch.empty((b, T, H, P), device="cuda")
        bdssm.block_step_ops(d, T, forms[bdssm.STATE_OPS], bdssm.seq_to_device(fwd), bdssm.seq_to_device(rev),
                             _dev(A), _dev(D), yp, A_rev=_dev(Ar), D_rev=_dev(Dr))
        torch.cuda.synchronize()
        assert torch.equal(_run(d, T, forms[bdssm.STATE_OPS], bdssm.STATE_OPS, fwd, rev, A, D, Ar, Dr), yp)


def _params(rng, H, P):
    A = (-np.exp(rng.uniform(0, np.log(16), H))).astype(np.float32)
    Ar = (-np.exp(rng.uniform(0, np.log(16), H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    Dr = rng.standard_normal(H).astype(np.float32)
    Dc = rng.standard_normal((H, P)).astype(np.float32)
    Drc = rng.standard_normal((H, P)).astype(np.float32)
    return A, D, Ar, Dr, Dc, Drc


@pytest.mark.parametrize("cfg_index", [0, 1])
def test_variants_at_config_shapes(cfg_index):
    """The tiny fp32 shape (vector-ALU kernel, bound 1e-5) and the 700M shape (small-batch
    kernel), with the cached state of a prefix scan."""
    cfg = configs.get(cfg_index)
    A, D = inputs.params(cfg)
    rng = np.random.default_rng(50 + cfg_index)
    _, Dd, Ar, Dr, Dc, Drc = _params(rng, cfg.nheads, cfg.headdim)
    pre = inputs.prefix(cfg, length=min(cfg.prefix_len, 1024))
    _, _, h = oracle.scan(pre, A, D, cfg.chunk, want_y=False, want_chunk_states=False)
    h = f32_round(h)
    fwd = inputs.block(cfg, 0, 0, inputs.FWD)
    rev = inputs.block(cfg, 0, 0, inputs.REV)
    _check_variants(fwd, rev, h, A, D, Ar, Dr, Dc, Drc, f"config {cfg_index}")


@pytest.mark.parametrize("b,H,G,T,kernel", [
    (12, 48, 1, 128, bdssm.KERNEL_AUTO),       # many pairs: bandwidth kernels (8 row blocks)
    (3, 12, 2, 77, bdssm.KERNEL_AUTO),         # T > 32: bandwidth kernels, ragged
    (3, 12, 2, 32, bdssm.KERNEL_BANDWIDTH),    # forced bandwidth kernels at T = 32
    (2, 8, 4, 17, bdssm.KERNEL_SMALL_BATCH),   # small-batch kernel, ragged
])
def test_variants_on_every_kernel(launch_override, b, H, G, T, kernel):
    from test_oracle_pins import rand_seq
    rng = np.random.default_rng(60 + T + H)
    fwd = rand_seq(rng, b, T, H, 64, 128, G, 1)
    rev = rand_seq(rng, b, T, H, 64, 128, G, 1)
    A, D, Ar, Dr, Dc, Drc = _params(rng, H, 64)
    h = f32_round(rng.standard_normal((b, H, 128, 64)) * 0.1)
    launch_override(block_kernel=kernel)
    _check_variants(fwd, rev, h, A, D, Ar, Dr, Dc, Drc, f"b={b} H={H} G={G} T={T} kernel={kernel}")


def test_bf16_state_config4_shape():
    """The running set's shape (64 streams x 48 heads, T = 128) from the bf16 cached state:
    the bandwidth kernel reads half the state bytes; oracle on streams {0, 31, 63}."""
    import torch
    from harness import streams_of
    cfg = configs.get(4)
    A, D = inputs.params(cfg)
    b, H, P, N, G, T = cfg.batch, cfg.nheads, cfg.headdim, cfg.d_state, cfg.ngroups, cfg.block_len
    rng = np.random.default_rng(64)
    h = f32_round(rng.standard_normal((b, H, N, P)) * 0.05)
    fwd = inputs.block(cfg, 0, 0, inputs.FWD)
    rev = inputs.block(cfg, 0, 0, inputs.REV)
    d = bdssm.dims(b, H, P, N, G, cfg.in_dtype, bdssm.BF16)
    hb = torch.empty(bdssm.state_bf16_bytes(d), dtype=torch.uint8, device="cuda")
    bdssm.state_bf16(d, torch.from_numpy(h.astype(np.float32)).cuda(), hb)
    sample = [0, 31, 63]
    hs = _bf16_values(h)[sample]
    for Dv, what in ((D, "y"), (np.zeros_like(D), "y - D x")):
        _case(f"c4 bf16 state, {what}")
        y = _run(d, T, hb, bdssm.STATE_BF16, fwd, rev, A, Dv, y_dtype=bdssm.BF16)
        yo, _, _ = oracle.block_step(hs, streams_of(fwd, sample), streams_of(rev, sample), A, Dv)
        assert within(rel(y.float().cpu().numpy()[sample], yo), TOL_BF16, f"c4 bf16 state {what}")
