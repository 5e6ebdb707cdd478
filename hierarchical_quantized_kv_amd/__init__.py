"""Hierarchical INT8 KV cache (QuantSpec) decode attention for AMD MI355X (gfx950).

The compute path is the HIP library ``libquantspec.so`` (built from ``csrc/``) behind the C ABI
declared in ``include/quantspec.h``; ``binding`` marshals torch tensors to it.  Importing this
package does not load the library: ``binding.lib()`` does, and raises if it is not built.
"""
__all__ = ["binding", "synth"]
