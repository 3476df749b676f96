"""CPU oracle for the Q4_0 x Q8_0 GEMV.  Test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path.
"""
