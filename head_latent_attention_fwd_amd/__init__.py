"""MI355X (gfx950) multi-head latent attention forward: HIP kernels behind a C ABI.

The compute path lives in the shared library built from csrc/ (libmla.so);
this package only marshals arguments to it (see api.py). Loading is lazy so
that the seeded input generator (synth.py) can be used without a GPU; any
call into the library raises if the built library is missing.
"""
__all__ = ["api", "synth"]
