"""CPU oracle for TBQ4 attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the HIP
library and its Python binding) never imports, links or runs it, and the
oracle never imports the product path.

``tbq4_oracle``   vectorised numpy fp64 oracle (quantiser, dequantiser,
                  decode and prefill attention, split-K merge).
``scalar_oracle`` scalar pure-Python transcription for tiny inputs, used to
                  check the vectorised one.

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (see ``tests/test_oracle_*.py``).
"""
