"""CPU oracle for the KVarN quantizer -- test infrastructure only.

Imported by the test suite, the smoke check and the benchmark's CPU-baseline leg;
never by the library path.
"""
