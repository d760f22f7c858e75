"""fp64 CPU oracle for shifted-window attention.

Test infrastructure: only tests/, the smoke check and the bench's CPU-baseline
leg may import it. The product path never does.
"""
