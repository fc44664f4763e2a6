"""Layer-aware KV decode attention (DELTA's full / delta / sparse layer tiers) for
MI355X (gfx950): HIP kernels behind the C ABI of include/lak.h, with a thin ctypes
binding.  There is no CPU fallback: the first use raises if liblak.so is missing."""
from ._lib import LakError, lib  # noqa: F401
from .cache import PagedKVCache  # noqa: F401
from .stack import DeltaStack, layer_tiers  # noqa: F401
