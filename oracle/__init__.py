"""CPU oracle for the Mamba-2 SSD layer core -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (``mamba_ssd_scan_amd``)
never imports it, and it never imports the product: the two share no code.

* ``oracle.ref``       -- fp64 sequential recurrence in plain C (the definition).
* ``oracle.quadratic`` -- fp64 brute-force quadratic ("attention") form, numpy.
* ``oracle.chunked``   -- fp64 chunked evaluation in the order of the method's
                          steps (intra-chunk, chunk states, inter-chunk
                          recurrence, off-diagonal output), numpy.
* ``oracle.gated``     -- the model-adjacent options around the recurrence
                          (dt = softplus(dt + bias), the z gate), fp64.

Every function is pinned by tests in ``tests/test_oracle_*.py`` against
closed forms, textbook special cases and invariants; see each module.
"""
