"""PISA pyramid Top-K block selection and block-sparse attention for MI355X (gfx950).

The compute lives in the HIP library ``libpisa.so`` (built from ``csrc/``); the
Python module :mod:`long_context_block_amd.pisa` is a thin ctypes binding with the
same entry-point names. Importing this package loads nothing: the binding loads
the library on first use and raises if it is missing.
"""
