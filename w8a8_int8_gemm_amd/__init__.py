"""MI355X (gfx950) W8A8 INT8 projection GEMM.

Submodules:
  binding  -- ctypes binding of libw8a8.so (include/w8a8.h); importing it
              does not load the library, the first call does (and fails
              loudly if it was not built).
  datagen  -- seeded synthetic inputs of the DiT projection workloads.
  build    -- hipcc build of libw8a8.so for gfx950.
"""
