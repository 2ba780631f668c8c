"""CPU oracle for the FP4 W4A4 hot path -- test infrastructure only.

Imported by the tests, the smoke check and the CPU baseline leg of the
benchmark; never by the product library.
"""
