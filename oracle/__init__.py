"""fp64 CPU oracle for windowed, grouped-query, packed-batch attention, and for
the linear cross-entropy loss (the second workload).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package.
The product path (the HIP library and its Python binding) never does, and it
shares no code with it: no kernels, helpers, tables or constants. Both sides
take their inputs from ``sliding_window_flash_amd.workloads``, which holds
random draws and shapes only.

Modules:
  dense  - the plain definition: builds the full masked score matrix per
           (sequence, head) in fp64, row panel by row panel.
  loop   - brute force, one query (or token) at a time, in plain Python floats.
  fd     - central finite differences of the loss sum(O * dO).
  ce     - the linear cross-entropy: logits H W^T row panel by row panel,
           per-token NLL, LSE and target logit, and dH.

Every function here is pinned by tests against closed forms, invariants and
finite differences (see tests/test_oracle_pins.py and tests/test_ce_oracle.py).
No function is left "parity unpinned".
"""
