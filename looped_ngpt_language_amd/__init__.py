"""Looped normalised-GPT forward pass on MI355X (gfx950).

The compute path is the C-ABI library ``libdory.so`` (hand-written HIP kernels
plus a host scheduler and paged-KV manager); :mod:`.dory` is its ctypes binding
and :mod:`.synth` the seeded input generator. Importing this package loads
nothing native; the binding loads the library on first use.
"""
