"""MI355X (gfx950) learned-relative grouped-query attention forward with per-query sinks.

``binding`` holds the ctypes binding of the HIP library (libinkattn.so, built
by ``python -m transformer_attention_03_amd.build``); ``workloads`` holds the
seeded synthetic input generators.  Importing the package loads nothing.
"""
