"""MI355X (gfx950) low-latency decode megakernel behind a C ABI (include/mk.h).

The HIP library ``libmk.so`` is built in-tree by ``persistent_megakernel_cu_amd.build``;
``persistent_megakernel_cu_amd.binding`` is the thin ctypes layer over it.
"""

from .binding import Engine, MkError, lib, plan_describe, to_device  # noqa: F401
