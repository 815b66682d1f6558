"""MI355X-native per-rank attention for Hybrid Data Parallelism (packed varlen + ring chunks).

The compute lives in libhdpattn.so (HIP for gfx950) behind the C ABI in include/hdp_attn.h;
`ops` is its thin Python binding.  Importing this package loads nothing; importing `ops`
requires the built library.
"""
__all__ = ["ops", "synth", "build"]
