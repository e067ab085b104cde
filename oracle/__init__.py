"""The oracle: a plain, slow, obviously correct CPU statement of what the DVM
hot path computes.

THIS PACKAGE IS TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The HIP path
(``device_bytecode_vm_amd``) never imports it, and it never imports the HIP
path: the two share no code, no tables and no constants.  Where both follow
the same rule (the tiling and fusion rules), each side states it in its own
code.

Sources: the DVM paper review page ("DVM: A Bytecode Virtual Machine Approach
for Dynamic Tensor Computation", sections 4.1-4.4 and 5.1-5.2) and the
MindSpore DVM summary page (sections 3.2-3.3).  Where those pages leave a step
open, the reading taken is stated in the function that implements it.

Modules
-------
numerics  bf16 / fp32 rounding and the tolerance comparators.
ops       fp64 definitions of every operation and of the workload graphs.
graph     fp64 evaluator of a primitive op list (the fused-graph semantics).
tiling    the shape-tiling rules (dominant shape, shrink path, cost, header,
          tile ranges, element -> tile map).
fusion    the streaming-fusion partition rules.

Parity pins live in ``tests/test_oracle_*.py`` (run with ``-m "not gpu"``).
Every function there is pinned; none is "parity unpinned".
"""
