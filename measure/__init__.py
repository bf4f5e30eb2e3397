"""Measurement tools beside the benchmark (not part of the library): the
algorithmic-work accounting of the grouped FFN (accounting.py), and the
hardware-counter traffic runs (traffic.py) with their native driver of the C
ABI (moe_probe.cpp)."""
