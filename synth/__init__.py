"""Seeded synthetic inputs for the SR-SWA hot path (tests, smoke and bench).

Holds the counter-based generator (``rng``), the workload recipes
(``workloads``) and, in ``fill.hip``, the device-side fill of the same bits.
It contains none of the attention method's arithmetic.
"""
