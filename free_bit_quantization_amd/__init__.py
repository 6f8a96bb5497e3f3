"""OrbitQuant quantized linear layer on AMD MI355X (gfx950).

``oq`` binds the C ABI of liboq (include/oq.h); ``synth`` holds the seeded
synthetic workloads; ``build`` compiles liboq.so for gfx950.
"""

from . import synth  # noqa: F401
