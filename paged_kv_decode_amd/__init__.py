"""MI355X (gfx950) paged-KV decode attention: a C-ABI HIP library plus this thin binding.

Importing the package loads nothing; the HIP library is opened on first use by
``paged_kv_decode_amd.binding`` and its absence is an error (there is no CPU
path).  ``paged_kv_decode_amd.workloads`` draws seeded synthetic inputs.
"""
