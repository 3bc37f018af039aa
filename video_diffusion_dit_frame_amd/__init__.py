"""MI355X-native DraftAttention2 hot path: draft-guided tier planning and
phased 16-bit / 8-bit (INT8 Q K^T, FP8 P V) / MXFP4 block-sparse attention,
behind the C-ABI library libda2.

Importing the package loads nothing; ``video_diffusion_dit_frame_amd.da2``
binds the HIP library and raises if it is missing.
"""
__all__ = ["configs", "synth"]
