"""Plain CPU oracle for paged decode attention and its block manager.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT: only tests/, the smoke entry
point and the CPU-baseline leg of the benchmark may import this package.  It
shares no code with paged_kv_cache_328_amd/ and imports nothing from it.
"""
