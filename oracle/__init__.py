"""CPU oracle for ggml block-quantized GEMV.

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's
CPU-baseline leg may import this; the product path never does.
"""
