"""Persistent MoE decode layer for MI355X (gfx950).

The layer runs as one persistent HIP kernel behind the C ABI declared in
``include/moe_decode.h``; ``binding`` is a thin ctypes wrapper over it and
``synth`` draws the seeded synthetic inputs.
"""
