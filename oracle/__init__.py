"""The oracle: a plain float64 CPU implementation of the attention forward.

TEST INFRASTRUCTURE ONLY.  Imported by tests/, the smoke check and the
benchmark's CPU-baseline leg; never by the product package.
"""
