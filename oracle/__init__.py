"""CPU oracle for the HSTU layer forward — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything in this package.  The product path (the HIP
library and its Python binding) never imports, calls or falls back to it.

Modules:
  hstu_oracle  vectorised NumPy float64 implementation of the layer.
  brute        scalar pure-Python loops of the same definition, for tiny inputs.

Function pins (what ties each function to the pages rather than to itself)
are listed in each module's header.  ``ln_eps``'s exact value is not given by
the pages: parity unpinned for that constant (any eps much smaller than the
row variance gives the same result within tolerance).
"""
