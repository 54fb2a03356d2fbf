"""DHSA sparse prefill on MI355X (gfx950): HIP kernels behind a C ABI.

``dhsa`` is the thin ctypes binding over ``libdhsa.so``; ``synth`` draws the
seeded synthetic inputs.  Importing the binding raises if the library has not
been built: there is no CPU fallback.
"""
