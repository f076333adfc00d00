"""MI355X-native DSA stage: Lightning Indexer scoring, Top-K and Sparse Flash Attention.

The compute runs in hand-written HIP kernels for gfx950 behind a C ABI
(include/dsa.h, built as libdsa.so in this package).  `binding` marshals
torch device tensors into those calls; `inputs` draws seeded synthetic
workloads.  Importing the package loads nothing; the library is loaded on
first use and its absence is an error.
"""
