"""MI355X-native sparse embedding layer: multi-table EmbeddingBag forward,
id sort/unique, segmented gradient reduction with fused Adagrad, and a
dynamic raw-key hash table, as hand-written HIP kernels for gfx950 behind a
C ABI (``include/embtab.h``).

Submodules:
  embtab  -- ctypes binding of libembtab.so (loads the HIP library; raises if
             it is missing)
  synth   -- seeded synthetic inputs (numpy only)
"""
__all__ = ["embtab", "synth"]
