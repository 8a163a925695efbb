"""Query-aware block-sparse decode attention over a paged KV cache, for
AMD MI355X (gfx950).

Modules
  kvs    ctypes binding of libkvs.so (the C ABI in include/kvs.h); importing
         it fails when the library is not built
  step   decode-step drivers that chain the C entry points and own workspaces
  synth  seeded synthetic workloads (inputs only)
  build  compiles libkvs.so with hipcc

The binding is imported lazily so that ``synth`` and ``build`` work on a
machine where the library has not been built yet.
"""

__all__ = ["kvs", "step", "synth", "build"]
