"""MI355X (gfx950) row-wise reduction-reuse operators: softmax, LayerNorm, RMSNorm.

The compute path is the HIP library ``libcredit.so`` built from ``csrc/``; the
Python binding in ``credit.py`` only marshals arguments to its C ABI.  Importing
this package loads nothing; the library is loaded on first use and its absence
is an error.
"""
