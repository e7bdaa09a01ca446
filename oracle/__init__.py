"""fp64 CPU oracle of the KDA recurrence -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package; the HIP library never imports, links or calls it.
"""
