"""Oracle for pair-biased (gated) triangle self-attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 CPU implementations that the HIP library is checked
against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import anything from here; the library itself never
does, and this package imports nothing from the library.

* ``oracle.ref``   -- vectorised NumPy float64, materialises the full softmax.
* ``oracle.brute`` -- pure-Python scalar loops for tiny inputs.
* ``oracle.aaq``   -- the token-wise quantization codec (records, decode).
* ``oracle.knn``   -- the k-nearest-neighbour sparse atom-pair encoder.

Parity status: every function here is pinned by ``tests/test_oracle.py``,
``tests/test_oracle_aaq.py`` and ``tests/test_oracle_knn.py``
(brute force, torch CPU library routines, closed forms, invariants, and
hand-derived cases written into those tests: the two-key closed form at
c_z = 2 in test_oracle.py and the worked INT8 / INT4 records in
test_oracle_aaq.py).  No function is "parity unpinned".
"""
