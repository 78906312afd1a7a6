"""The five workload shapes of the bidirectional block-diffusion Mamba hot path.

Shapes follow the block-diffusion Mamba-H paper ("Training Hybrid Block Diffusion
Language Models with Partial Bidirectionality": 700M random-init inference at batch 1,
context up to 262K) and DiffuApriel's Table 1 (d_state 128) and its block size 32; the
running set of four consecutive 32-token blocks follows "Multi-Block Diffusion Language
Models" (MultiBD running set). Sizes the pages leave open (chunk length, number of
blocks and steps) are fixed here and listed as readings in the design notes.

Nothing here computes anything of the method; it only names sizes.
"""
from dataclasses import dataclass

F32 = 0
BF16 = 1


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    batch: int          # independent streams
    nheads: int         # H
    headdim: int        # P
    d_state: int        # N
    ngroups: int        # G (B and C are shared by H/G consecutive heads)
    in_dtype: int       # F32 or BF16 for x, dt, B, C
    prefix_len: int     # L: tokens folded into the cached state
    chunk: int          # Q: chunk length of the prefix scan
    block_len: int      # T: tokens in one block-step window
    steps_per_block: int
    n_blocks: int
    commit_len: int     # tokens folded by one commit
    prefix_y: bool      # whether the prefix scan writes y (else state-only)
    prefix_chunk_states: bool

    @property
    def hpg(self):
        return self.nheads // self.ngroups


CONFIGS = [
    Config(0, "tiny fp32 sanity: 4 heads x 16, d_state 16, prefix 256, block 16",
           batch=1, nheads=4, headdim=16, d_state=16, ngroups=1, in_dtype=F32,
           prefix_len=256, chunk=64, block_len=16, steps_per_block=4, n_blocks=2,
           commit_len=16, prefix_y=True, prefix_chunk_states=True),
    Config(1, "700M shape: 48 heads x 64, d_state 128, batch 1, prefix 8192, block 32, 64 steps",
           batch=1, nheads=48, headdim=64, d_state=128, ngroups=1, in_dtype=BF16,
           prefix_len=8192, chunk=256, block_len=32, steps_per_block=64, n_blocks=4,
           commit_len=32, prefix_y=True, prefix_chunk_states=False),
    Config(2, "350M prefix/commit: 32 heads x 64, d_state 128, prefix 65536, chunk 256",
           batch=1, nheads=32, headdim=64, d_state=128, ngroups=1, in_dtype=BF16,
           prefix_len=65536, chunk=256, block_len=32, steps_per_block=1, n_blocks=1,
           commit_len=32, prefix_y=True, prefix_chunk_states=True),
    Config(3, "3B long context: 80 heads x 64, d_state 128, 8 groups, prefix 262144, block 32",
           batch=1, nheads=80, headdim=64, d_state=128, ngroups=8, in_dtype=BF16,
           prefix_len=262144, chunk=256, block_len=32, steps_per_block=64, n_blocks=1,
           commit_len=32, prefix_y=False, prefix_chunk_states=False),
    Config(4, "700M shape x 64 streams: prefix 32768 each, running set 4 x 32 = 128 tokens",
           batch=64, nheads=48, headdim=64, d_state=128, ngroups=1, in_dtype=BF16,
           prefix_len=32768, chunk=256, block_len=128, steps_per_block=16, n_blocks=1,
           commit_len=32, prefix_y=False, prefix_chunk_states=False),
]


def get(index):
    return CONFIGS[index]
