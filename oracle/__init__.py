"""CPU oracle for the Muon-style optimizer step -- test infrastructure only.

Imported by the tests, by the smoke check and by the benchmark's CPU-baseline
leg; never by the product library or its binding.  It shares no code with the
HIP path.
"""
