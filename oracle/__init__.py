"""CPU oracle for MaxSim scoring -- test infrastructure only.

Imported by the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU
baseline; never by the HIP path.
"""
