"""MI355X-native neural-memory test-time update (Titans / ATLAS) behind a C ABI.

The compute path is the HIP library `libatlasmem.so` built from `csrc/`;
`atlasmem` is its thin ctypes binding.  Importing this package does not load
the library; `atlasmem.load()` does, and raises if it is missing.
"""
