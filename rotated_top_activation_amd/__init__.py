"""Rotated Top-K sparse activation (LaRoSA) decode path for MI355X (gfx950).

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``liblarosa.so``, declared in ``include/larosa.h``); ``_lib`` is a thin
ctypes binding with the same entry-point names.
"""
