"""CPU oracle for FAVOR+ attention — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the GPU library never does.
``reference`` is the numpy fp64 oracle, ``native`` the plain-C fp64 one.
"""
