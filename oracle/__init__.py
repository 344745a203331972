"""CPU oracle for the rank-ordered gather and the rank-ordered sum.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  See ``oracle/oracle.py``.
"""
