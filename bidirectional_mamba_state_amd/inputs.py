"""Seeded synthetic inputs for the bidirectional Mamba state hot path.

This module only draws and rounds numbers; it contains none of the scan's arithmetic.
Both the HIP path and the CPU oracle receive the arrays it returns, so both see the
same already-rounded values.

Distributions (every config), following the workload recipe:
  x ~ N(0, 1);  B, C ~ N(0, 1/16);
  dt = softplus(z), z ~ N(-4, 1), computed in float64 and clipped to [1e-3, 0.1]
       (dt is handed over post-softplus: the scan itself applies no softplus or clamp);
  A_h = -exp(U(0, ln 16)) per head (float32);  D_h ~ N(0, 1) per head (float32);
  convolution weights and bias (when used) ~ U(-1/sqrt(W), 1/sqrt(W)), float32.
bf16 configs round x, dt, B and C from float64 to bfloat16 with round-to-nearest-even
and hand over the 16-bit patterns (numpy uint16); fp32 configs round to float32.

Seeding: each tensor of each (config, stream, segment, step, direction) is cut into
pieces of PIECE tokens; every piece has its own PCG64 generator seeded by
SeedSequence(0, spawn_key=(config, stream, segment, step, direction, tensor, piece)) and
is drawn in token-major order. Any token range can therefore be drawn on its own and in
parallel, and drawing a segment in token chunks reproduces a single draw.
"""
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from .configs import BF16, F32, Config

ROOT_SEED = 0

# segment ids
PREFIX = 0


def BLOCK(k):
    return 1 + k


# direction ids
FWD, REV, CLEAN = 0, 1, 2
# tensor ids
T_X, T_DT, T_B, T_C = 0, 1, 2, 3
_PARAM_KEY = 0x7FFF
PIECE = 4096


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(ROOT_SEED, spawn_key=key)))


def round_bf16_bits(v):
    """float64 -> bfloat16 bit patterns, round-to-nearest-even, without passing through
    float32 (which would round twice)."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    qexp = np.maximum(e - 8, -133)          # 8 significant bits; bf16 subnormal quantum 2^-133
    r = np.ldexp(np.rint(np.ldexp(v, -qexp)), qexp)   # np.rint: ties to even
    f = r.astype(np.float32)                # exact: r has at most 8 significant bits
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _round(v, dtype):
    if dtype == BF16:
        return round_bf16_bits(v)
    if dtype == F32:
        return np.asarray(v, dtype=np.float64).astype(np.float32)
    raise ValueError(dtype)


def as_f32(a, dtype):
    """Decode an input array handed out by this module to float32 (exact)."""
    return bf16_bits_to_f32(a) if dtype == BF16 else np.asarray(a, dtype=np.float32)


def params(cfg: Config):
    """Per-head A (negative) and D, float32."""
    u = _rng(cfg.index, _PARAM_KEY, 0).uniform(0.0, np.log(16.0), size=cfg.nheads)
    A = (-np.exp(u)).astype(np.float32)
    D = _rng(cfg.index, _PARAM_KEY, 1).standard_normal(cfg.nheads).astype(np.float32)
    return A, D


def conv_params(cfg: Config, width: int = 4, direction: int = FWD):
    """Depthwise convolution weights [H*P + 2*G*N, width] and bias [H*P + 2*G*N] of one
    direction, float32, both U(-1/sqrt(width), 1/sqrt(width)) (a conv layer's usual
    initialization with fan-in = width)."""
    ch = cfg.nheads * cfg.headdim + 2 * cfg.ngroups * cfg.d_state
    bound = 1.0 / np.sqrt(width)
    g = _rng(cfg.index, _PARAM_KEY, 2 + direction, width)
    w = g.uniform(-bound, bound, (ch, width)).astype(np.float32)
    bias = g.uniform(-bound, bound, ch).astype(np.float32)
    return w, bias


@dataclass
class Seq:
    """One token segment: x [b, len, H, P], dt [b, len, H], B and C [b, len, G, N].
    Arrays are uint16 bf16 patterns or float32, per ``dtype``."""
    x: np.ndarray
    dt: np.ndarray
    B: np.ndarray
    C: np.ndarray
    dtype: int

    @property
    def length(self):
        return self.x.shape[1]


def _tail(cfg, tensor):
    if tensor == T_X:
        return (cfg.nheads, cfg.headdim)
    if tensor == T_DT:
        return (cfg.nheads,)
    return (cfg.ngroups, cfg.d_state)


def _draw_piece(cfg, key, tensor, piece, ntok):
    """The first ``ntok`` tokens of one PIECE-token piece of one tensor, rounded."""
    g = _rng(*key, tensor, piece)
    v = g.standard_normal((ntok,) + _tail(cfg, tensor))
    if tensor == T_X:
        pass
    elif tensor == T_DT:
        v = np.clip(np.log1p(np.exp(v - 4.0)), 1e-3, 0.1)
    else:
        v *= 0.25
    return _round(v, cfg.in_dtype)


def _out_dtype(cfg):
    return np.uint16 if cfg.in_dtype == BF16 else np.float32


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1)))
    return _POOL


_POOL = None


def draw(cfg: Config, stream: int, segment_id: int, step: int, direction: int, t0: int, t1: int,
         out=None):
    """Tokens [t0, t1) of one stream's segment: returns (x, dt, B, C), or fills ``out``
    (a tuple of four arrays shaped [t1 - t0, ...]). Any token range can be drawn on its
    own: each PIECE-token piece of each tensor has its own generator."""
    key = (cfg.index, stream, segment_id, step, direction)
    n = t1 - t0
    if out is None:
        out = tuple(np.empty((n,) + _tail(cfg, t), _out_dtype(cfg)) for t in (T_X, T_DT, T_B, T_C))
    jobs = []
    for piece in range(t0 // PIECE, (t1 + PIECE - 1) // PIECE if n > 0 else 0):
        p0 = piece * PIECE
        lo, hi = max(t0, p0), min(t1, p0 + PIECE)
        for ti, t in enumerate((T_X, T_DT, T_B, T_C)):
            jobs.append((ti, t, piece, p0, lo, hi))

    def run(job):
        ti, t, piece, p0, lo, hi = job
        out[ti][lo - t0:hi - t0] = _draw_piece(cfg, key, t, piece, hi - p0)[lo - p0:]

    if len(jobs) > 4:
        list(_pool().map(run, jobs))
    else:
        for j in jobs:
            run(j)
    return out


def segment(cfg: Config, segment_id: int, step: int, direction: int, length: int,
            streams=None) -> Seq:
    """Draw a whole segment of ``length`` tokens for the given streams (default: all)."""
    streams = list(range(cfg.batch) if streams is None else streams)
    dt_ = _out_dtype(cfg)
    arrs = tuple(np.empty((len(streams), length) + _tail(cfg, t), dt_) for t in (T_X, T_DT, T_B, T_C))
    for i, s in enumerate(streams):
        draw(cfg, s, segment_id, step, direction, 0, length, out=tuple(a[i] for a in arrs))
    return Seq(*arrs, cfg.in_dtype)


def prefix(cfg: Config, streams=None, length=None) -> Seq:
    return segment(cfg, PREFIX, 0, FWD, cfg.prefix_len if length is None else length, streams)


def block(cfg: Config, k: int, step: int, direction: int, streams=None, length=None) -> Seq:
    """Inputs of block ``k`` at denoising ``step`` (direction FWD or REV), or the block's
    clean inputs for the commit (direction CLEAN, step 0)."""
    n = length if length is not None else (cfg.commit_len if direction == CLEAN else cfg.block_len)
    return segment(cfg, BLOCK(k), step, direction, n, streams)
