"""MI355X-native tree-structured KV search (ZHA hot path).

``tree_structured_kv_amd.zha`` is the thin ctypes binding over the HIP C-ABI
library ``libzha.so``; ``tree_structured_kv_amd.synth`` draws the seeded
synthetic workloads.  Importing the package loads neither.
"""
