"""Lossless BF16 weight restore on AMD MI355X (gfx950).

``afx``   -- ctypes binding of libafx (C ABI in include/afx.h): afx_query,
            afx_decode_tensor, afx_decode_layer_async, and the host encoder.
``synth`` -- seeded synthetic Qwen3-14B-shaped BF16 weights.
``ready`` -- the time-to-ready arithmetic of Eq. (1) and Eq. (2).
``stream``-- layer-by-layer streaming of a compressed model from pinned host
            memory (copy of unit i+1 overlapped with the restore of unit i).
"""
