"""HiSparse swap-in hot path for MI355X (gfx950).

The compute path lives in the C-ABI library ``libhisparse.so`` built from
``csrc/``; :mod:`.binding` is the thin ctypes layer over it and
:mod:`.workloads` holds the seeded synthetic input generators.  Importing the
package does not load the library; :func:`binding.lib` does, and raises if it
has not been built.
"""
