"""MI355X-native confidence-scheduled, flattened speculative verification.

The compute path is the C-ABI library built from csrc/ (HIP for gfx950); the
Python side is a ctypes binding (``binding``) that only marshals arguments,
and a seeded synthetic input generator (``workloads``).
"""
