"""The algorithmic work bench.py divides by, rebuilt on the CPU from the size of each tensor
a call reads or writes: the roofline fractions it reports are these figures over measured
times. Per call, every input is read once, the cached state read once (and written once by a
commit), y written once; A (and D where y is written) are H floats each."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from bidirectional_mamba_state_amd import configs  # noqa: E402


def _shape(i):
    c = configs.get(i)
    return c, c.batch, c.nheads, c.headdim, c.d_state, c.ngroups


def test_block_step_bytes_from_tensor_sizes():
    # (config, expected bytes with y in the input dtype, with an fp32 y)
    for i, want_in, want_f32 in ((0, 21_024, 21_024), (1, 2_201_984, 2_398_592), (2, 1_478_912, 1_609_984),
                                 (3, 3_877_504, 4_205_184), (4, 261_620_096, 311_951_744)):
        c, b, H, P, N, G = _shape(i)
        eb = 4 if c.in_dtype == 0 else 2
        T = 128 if i == 4 else (16 if i == 0 else 32)
        state = b * H * N * P * 4
        per_dir = b * T * H * P * eb + b * T * H * eb + 2 * b * T * G * N * eb  # x, dt, B and C
        params = 2 * H * 4  # A, D
        y = b * T * H * P
        assert state + 2 * per_dir + params + y * eb == want_in, i
        assert state + 2 * per_dir + params + y * 4 == want_f32, i
        assert bench.block_step_bytes(b, H, P, N, G, T, eb, eb) == want_in, i
        assert bench.block_step_bytes(b, H, P, N, G, T, eb, 4) == want_f32, i


def test_commit_bytes_from_tensor_sizes():
    # state read + written, the clean block's x, dt and B, A; no C, D or y
    for i, T, want in ((0, 16, 13_584), (1, 32, 3_353_792), (2, 32, 2_238_592), (3, 32, 5_641_536),
                       (4, 32, 214_630_592)):
        c, b, H, P, N, G = _shape(i)
        eb = 4 if c.in_dtype == 0 else 2
        state = b * H * N * P * 4
        clean = b * T * (H * P + H + G * N) * eb
        assert 2 * state + clean + H * 4 == want, i
        assert bench.commit_bytes(b, H, P, N, G, T, eb) == want, i


def test_prefix_work_of_the_350m_scan():
    c, b, H, P, N, G = _shape(2)
    L, Q = c.prefix_len, c.chunk
    nch = L // Q
    io = b * L * (H * P + H + 2 * G * N) * 2  # x, dt, B, C in bf16
    y = b * L * H * P * 2                     # bf16 y
    states = b * nch * H * N * P * 4 + b * H * N * P * 4  # chunk states and the final state
    assert io + y + states == 844_103_680
    assert bench.prefix_bytes(b, H, P, N, G, L, Q, 2, 2, True) == 844_103_680
    # per chunk and head: C.B^T once per group (shared by the group's heads), (L o S) X, the
    # chunk state and the state's output; dense and with the causal half of the square
    dense = nch * H * (2 * Q * Q * N / (H // G) + 2 * Q * Q * P + 4 * Q * N * P)
    causal = nch * H * (2 * (Q * (Q + 1) / 2) * N / (H // G) + 2 * (Q * (Q + 1) / 2) * P + 4 * Q * N * P)
    assert abs(bench.prefix_flops(b, H, P, N, G, L, Q) - dense) < 1e-6 * dense
    assert abs(bench.prefix_flops(b, H, P, N, G, L, Q) - 141.73e9) < 0.01e9
    assert abs(bench.prefix_flops_causal(b, H, P, N, G, L, Q) - causal) < 1e-6 * causal
    assert abs(bench.prefix_flops_causal(b, H, P, N, G, L, Q) - 105.37e9) < 0.01e9


def test_state_only_build_bytes():
    c, b, H, P, N, G = _shape(4)
    L = c.prefix_len
    want = b * L * H * P * 2 + b * L * G * N * 2 + b * L * H * 2 + b * H * N * P * 4 + 2 * H * 4
    assert want == 13_723_763_072
    assert bench.prefix_state_bytes(b, H, P, N, G, L, 2) == want
