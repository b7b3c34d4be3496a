"""CPU oracle of the decode step (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  See ``oracle/decode.py``.
"""
