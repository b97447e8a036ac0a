"""MI355X (gfx950) DTensor-to-DTensor reshard.

The library (``libreshard.so``, C ABI in ``include/reshard.h``) plans a reshard
on the host -- exact source/destination shard intersections, one source replica
per overlap, merged contiguous dims -- and executes it as one fused gfx950 copy
kernel that reads every overlap once and writes it to each destination replica.
``reshard`` is its Python binding; ``workloads`` holds the seeded synthetic
inputs used by the tests and the benchmark.
"""
from .reshard import *  # noqa: F401,F403
from .reshard import ReshardError, REPLICATE, dtype_code  # noqa: F401
