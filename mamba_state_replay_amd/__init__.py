"""ReplaySSM decode hot path for a Mamba-2 layer on MI355X (gfx950).

The compute path is the C-ABI library `libreplayssm.so` (hand-written HIP
kernels); `binding` marshals arguments to it.  `synth` draws seeded inputs.
Importing the package loads nothing; `binding` loads the library on first use
and raises if it is missing.
"""
