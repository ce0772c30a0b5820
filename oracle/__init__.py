"""fp64 CPU oracle of the Kamera reuse operator (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg import
this package. It shares no code with the HIP library and imports nothing from
it.
"""
