"""bidirectional_mamba_state_amd: the block-diffusion bidirectional Mamba state hot path
(prefix scan -> cached fp32 boundary state -> block-local bidirectional block step ->
commit) as hand-written HIP kernels for gfx950 behind a C ABI (``include/bdssm.h``).

Importing the package loads nothing; ``bidirectional_mamba_state_amd.bdssm`` is the
ctypes binding of the shared library.
"""
