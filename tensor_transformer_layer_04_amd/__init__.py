"""MI355X-native tensor-parallel transformer-layer shard (libmtp).

``mtp`` is the ctypes binding of the C ABI in include/mtp.h; ``layer``
sequences the shard calls of a whole pre-LN layer (and the vocab-parallel
cross-entropy head) on one device.  Importing the package does not load the
library; the first call does, and fails loudly if it is not built.
"""
from . import mtp  # noqa: F401

__all__ = ["mtp"]
