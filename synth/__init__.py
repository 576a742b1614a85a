"""Seeded synthetic inputs shared by the oracle tests and the HIP path.

This package only draws random numbers and lays out block tables and slot
mappings. It holds none of the method's arithmetic (no quantisation, no
calibration, no attention), so neither side of a parity test can borrow the
other's maths through it.
"""

from .workloads import (  # noqa: F401
    PagedBatch,
    SEED_BASE,
    make_batch,
    make_config,
    CONFIG_NAMES,
)
