"""MI355X (gfx950) Block Sparse Attention over 3D video latent cubes.

The compute path is libbsa.so (hand-written HIP kernels behind the C ABI in include/bsa.h);
`bsa` is its thin ctypes binding and `synth` draws the seeded synthetic workloads.
"""
from . import synth  # noqa: F401

__all__ = ["synth", "bsa"]


def __getattr__(name):
    if name == "bsa":
        import importlib
        return importlib.import_module(".bsa", __name__)
    raise AttributeError(name)
