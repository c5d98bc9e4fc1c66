"""Seeded synthetic inputs for the round-robin CP sparse-attention path.

This module only draws random tensors and encodes them into their storage
formats (float32, bfloat16 bit patterns, OCP e4m3fn codes with a per-block
scale).  It holds none of the method's arithmetic: no token ownership, no
metadata, no scores, no selection, no attention.  Both the CPU oracle side
and the HIP side of the tests (and ``bench.py``) take their inputs from
here.
"""

from .workloads import WORKLOADS, Workload, get  # noqa: F401
from .draw import draw_prefill, draw_decode, draw_page_table  # noqa: F401
