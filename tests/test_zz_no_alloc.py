"""bdssm_prefix_scan_static, the prefix scan that takes no workspace and allocates nothing
(its workspace is the library's static scratch buffer): through the C ABI it gives bitwise
the outputs of bdssm_prefix_scan with a caller-provided workspace, on two calls in a row,
the second with a smaller input (the buffer then holds the first call's leftovers), on the
matrix-core path (several segments, with and without y and chunk states) and on the
vector-ALU path (chunk-local states in the workspace)."""
import numpy as np
import pytest

import oracle
from bidirectional_mamba_state_amd import bdssm
from harness import TOL_BF16, TOL_F32, f32_round, rel, within

pytestmark = pytest.mark.gpu


def _inputs(rng, b, L, H, P, N, G, dtype, init):
    from test_oracle_pins import rand_seq
    seq = rand_seq(rng, b, L, H, P, N, G, dtype)
    A = (-np.exp(rng.uniform(0, np.log(16), H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    h0 = f32_round(rng.standard_normal((b, H, N, P)) * 0.1) if init else None
    return seq, A, D, h0


def _run(seq, A, D, h0, chunk, want_y, want_cs, static):
    import torch
    b, L, H, P = seq.x.shape
    G, N = seq.B.shape[2], seq.B.shape[3]
    d = bdssm.dims(b, H, P, N, G, seq.dtype, bdssm.F32)
    xs = bdssm.seq_to_device(seq)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    y = torch.full((b, L, H, P), float("nan"), device="cuda") if want_y else None
    cs = torch.full((b, -(-L // chunk), H, N, P), float("nan"), device="cuda") if want_cs else None
    ho = torch.full((b, H, N, P), float("nan"), device="cuda")
    hi = dev(h0) if h0 is not None else None
    if static:
        bdssm.prefix_scan_static(d, L, chunk, xs, dev(A), dev(D), hi, y, cs, ho)
    else:
        wsb = bdssm.prefix_scan_workspace(d, L, chunk, want_y, want_cs)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
        bdssm.prefix_scan(d, L, chunk, xs, dev(A), dev(D), hi, y, cs, ho, ws, wsb)
    torch.cuda.synchronize()
    return y, cs, ho


# (b, H, G, P, N, dtype, chunk, y, chunk states, h_init, first length, second length)
CASES = [
    (1, 4, 1, 64, 128, bdssm.BF16, 256, True, True, True, 4096, 1000),    # matrix cores, full pass
    (1, 6, 2, 64, 128, bdssm.BF16, 64, False, False, True, 8192, 777),    # matrix cores, state only
    (2, 4, 2, 16, 16, bdssm.F32, 16, True, False, True, 700, 333),        # vector ALU, local states
]


@pytest.mark.parametrize("b,H,G,P,N,dtype,chunk,want_y,want_cs,init,L1,L2", CASES)
def test_static_scratch_matches_workspace_call(b, H, G, P, N, dtype, chunk, want_y, want_cs, init, L1, L2):
    import torch
    rng = np.random.default_rng(L1 + L2 + H)
    d = bdssm.dims(b, H, P, N, G, dtype, bdssm.F32)
    assert bdssm.prefix_scan_workspace(d, L1, chunk, want_y, want_cs) > 0, "the case must use a workspace"
    for k, L in enumerate((L1, L2)):
        print(f"[case] prefix_scan_static call {k + 1}: b={b} H={H} G={G} P={P} N={N} dtype={dtype} "
              f"chunk={chunk} L={L} y={want_y} cs={want_cs} h_init={init} "
              f"workspace={bdssm.prefix_scan_workspace(d, L, chunk, want_y, want_cs)}", flush=True)
        seq, A, D, h0 = _inputs(rng, b, L, H, P, N, G, dtype, init)
        got = _run(seq, A, D, h0, chunk, want_y, want_cs, static=True)
        ref = _run(seq, A, D, h0, chunk, want_y, want_cs, static=False)
        for g, r, what in zip(got, ref, ("y", "chunk states", "h_out")):
            if r is not None:
                assert torch.equal(g, r), f"call {k + 1}: {what} differs from bdssm_prefix_scan"
        _, _, ho = oracle.scan(seq, A, D, chunk, h_init=h0, want_y=False, want_chunk_states=False)
        tol = TOL_BF16 if dtype == bdssm.BF16 else TOL_F32
        assert within(rel(got[2].cpu().numpy(), ho), tol, f"call {k + 1}: final state vs oracle")
