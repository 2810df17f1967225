"""Seeded synthetic inputs for the paged-attention hot path.

This package is shared by the HIP path's tests and benchmark and by the
oracle's tests.  It only *makes inputs*: shapes, block placements, schedules,
random values and their storage encodings.  It contains none of the method's
arithmetic (no slot computation, no cache write, no attention); the block
allocator here decides *which* physical blocks a sequence owns, which is an
input to every kernel.

Modules:
  * ``rng``       -- seeded value generators (bf16 / fp32 / fp8 storage)
  * ``allocator`` -- a host block pool with reference counts, prefix sharing
                     and the copy-on-write decision
  * ``configs``   -- the five workloads, as plain dataclasses
"""

from . import allocator, configs, rng  # noqa: F401
