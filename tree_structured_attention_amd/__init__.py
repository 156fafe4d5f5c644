"""Layout-grounded tree attention for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libtree_attn.so`` built from ``csrc/``;
``tree_structured_attention_amd.binding`` is a thin ctypes layer over its
C ABI (argument marshalling only).  Importing this package does not load the
library; the first call into ``binding`` does, and fails loudly if it is not
built.
"""
__all__ = ["binding", "synth"]
