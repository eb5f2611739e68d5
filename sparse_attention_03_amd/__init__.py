"""MI355X (gfx950) DeepSeek Sparse Attention hot path.

* ``libdsa``  -- ctypes binding of the C interface (include/libdsa.h); loads libdsa.so.
* ``dsa``     -- tensor-level helpers that allocate outputs / workspaces with torch
                 and call libdsa.
* ``inputs``  -- seeded synthetic workloads.

``libdsa`` and ``dsa`` are imported lazily so that ``inputs`` works without the
built library.
"""
__all__ = ["libdsa", "dsa", "inputs"]
