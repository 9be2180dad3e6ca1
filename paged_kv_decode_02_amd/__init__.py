"""MI355X-native paged decode attention over a shared pool of BF16 KV pages.

``paged_kv_decode_02_amd.binding`` wraps the C-ABI library ``libpakv.so``
(HIP kernels for gfx950). ``paged_kv_decode_02_amd.workloads`` draws seeded
synthetic inputs. Importing the package loads neither.
"""

__all__ = ["binding", "workloads"]
