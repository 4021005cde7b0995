"""CPU oracle for quantized paged KV append and decode attention.

TEST INFRASTRUCTURE ONLY. The test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only code allowed to import it; the GPU
library and its Python binding never do, and share no code with it.
"""
