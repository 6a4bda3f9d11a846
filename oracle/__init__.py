"""CPU oracle for the TileQ fused MoE expert forward.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library under bit_rank_post_amd/.
"""
from . import pack_ref, tileq_ref, tiny_ref  # noqa: F401
