"""QLoRA NF4 hot path on MI355X (gfx950): thin Python binding over the C ABI.

The library is loaded lazily so that ``bit_nf4_quantized_22_amd.synth`` (the
seeded input generators) can be imported without it.
"""
