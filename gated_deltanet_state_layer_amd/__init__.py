"""MI355X-native Gated DeltaNet state layer: a slot pool with multi-slot
decode, speculative verify (one call, or over a ring of committed tokens)
and chunked prefill, run by the HIP kernels of
libgdn.so (see include/gdn.h) through a thin ctypes binding."""
from .binding import (  # noqa: F401
    GDN_BF16, GDN_F32, GDN_GROUP_KERNEL, GDN_VALIDATE, GdnError, Pool, PoolDesc, load_library, make_desc,
    pool_bytes, ring_layout, status_string,
)
