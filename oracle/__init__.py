"""fp64 CPU oracle (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  The product path
(``tensor_transformer_layer_04_amd``) never imports, links or runs it.
"""
from .layer import *  # noqa: F401,F403
from .layer import __all__  # noqa: F401
