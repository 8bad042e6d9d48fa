"""MI355X-native Simple GLA: chunked forward, chunked backward and decode.

The compute lives in ``libsgla.so`` (HIP kernels for gfx950 behind a C ABI,
declared in include/sgla.h); ``binding`` marshals torch tensors into it.
Importing this package loads nothing; the library is opened on first use.
"""
