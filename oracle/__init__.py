"""CPU oracle of the Mamba-3 selective scan and decode step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import anything here.  It shares no
code with the HIP library under ``selective_state_space_mimo_amd``; the two
meet only through the seeded inputs of ``m3inputs``.

- ``ref``      numpy fp64: sequential, quadratic, chunked and unrotated-state
               forms, one decode step, and an op-counting decode step.
- ``ref_cpu``  plain C fp64 sequential recurrence (OpenMP over streams).
- ``model``    the pages' byte / operation accounting of a decode step.
- ``block``    the layer steps around the scan (activations, BCNorm, x lift,
               readout recombination, D skip, gate), whole sequence and one
               decode step, on top of ``ref``.
- ``pcs``      numpy fp64: the per-coordinate selective scan (Mamba 1 preset):
               recurrence, sum over token pairs, associative prefix form.
- ``pcs_cpu``  plain C fp64 recurrence of the same (OpenMP over channels).

Parity status of every function is pinned by ``tests/test_oracle*.py``; no
function here is "parity unpinned".
"""
