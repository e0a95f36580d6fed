"""MI355X-native TurboQuant/TurboESM-style KV-cache codec: packed-KV decode attention and
inner-product search behind the C-ABI library `libtq.so` (HIP kernels for gfx950).

`vector_quantization_rope_amd.tq` is the thin ctypes binding (it loads the built library and
raises if it is missing); `workloads` holds the seeded synthetic inputs.  Importing the
package itself loads nothing.
"""
