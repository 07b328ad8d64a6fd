"""KIVI-style quantized KV cache for AMD MI355X (gfx950).

The compute path is the HIP library ``libkvq.so`` built from ``csrc/``;
``kivi_quantized_kv_amd.kvq`` is its thin ctypes binding.  Importing this
package loads nothing; ``kvq`` loads the library on first use and raises if
it is missing.
"""
