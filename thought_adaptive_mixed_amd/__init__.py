"""MI355X-native ThinKV decode hot path.

The HIP library (``libthinkv.so``, built from ``csrc/``) is loaded lazily by
``thought_adaptive_mixed_amd.binding``; importing this package does not touch
the GPU, so the workload generator can be used on a CPU-only host.
"""
__all__ = ["binding", "synth"]
