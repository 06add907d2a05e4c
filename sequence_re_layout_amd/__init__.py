"""sequence_re_layout_amd -- the BASP / Ulysses attention-boundary re-layout
on MI355X (gfx950): hand-written HIP kernels behind the C ABI of
``include/basp.h`` (``libbasp.so``), with a thin ctypes binding.

The binding is loaded on first use of any of its names, so that
``sequence_re_layout_amd.inputs`` and ``sequence_re_layout_amd.build`` work
before the library is built.  Using a binding name without a built
``libbasp.so`` raises ImportError: there is no other code path.
"""


_SUBMODULES = ("autograd", "binding", "build", "inputs", "launch_shapes", "workloads")


def __getattr__(name):
    import importlib
    if name.startswith("__"):
        raise AttributeError(name)
    if name in _SUBMODULES:   # `from sequence_re_layout_amd import build` before a build
        return importlib.import_module(__name__ + "." + name)
    binding = importlib.import_module(__name__ + ".binding")
    try:
        return getattr(binding, name)
    except AttributeError:
        raise AttributeError("module %r has no attribute %r" % (__name__, name)) from None
