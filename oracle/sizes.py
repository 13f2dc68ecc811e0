"""Guidance-record size arithmetic (TRACE §3.2 "Motivation" and §4.2
"Rollout Efficiency").

TEST INFRASTRUCTURE ONLY (see the package docstring).

A record keeps b code bits per element plus the block scale amortized over the
block (8 bits per 16 elements for NVFP4's E4M3, per 32 for MXFP4's E8M0). The
per-tensor FP32 global scale is ignored here, as in the paper's own counts.
The paper's "KB" and "TB" are binary units (KiB, TiB): 2048 x 20 x 1.5 bits is
7,680 bytes, which it calls 7.5 KB.
"""

from __future__ import annotations

BLOCK = {"nvfp4": 16, "mxfp4": 32}
SCALE_BITS = 8


def bits_per_element(fmt: str, code_bits: int) -> float:
    """Code bits kept per element plus the amortized block scale."""
    return code_bits + SCALE_BITS / BLOCK[fmt]


def activation_bits_per_token(hidden: int, layers: int, bits_per_elem: float) -> float:
    """One token's activation guidance: one record element per hidden channel
    per guided layer."""
    return hidden * layers * bits_per_elem


def kv_bits_per_token(head_dim: int, kv_heads: int, attn_layers: int,
                      bits_per_elem: float) -> float:
    """One token's KV guidance: K and V, each kv_heads x head_dim, per
    full-attention layer."""
    return head_dim * kv_heads * 2 * attn_layers * bits_per_elem


def step_bytes(bytes_per_token: float, trajectories: int, tokens: int) -> float:
    """Records of one RL step: every token of every trajectory."""
    return bytes_per_token * trajectories * tokens


def transfer_seconds(nbytes: float, bytes_per_second: float) -> float:
    return nbytes / bytes_per_second


def record_plane_bytes(n_elements: int, fmt: str, code_bits: int) -> dict:
    """Bytes of each plane a guidance call writes for n elements: the packed
    code-bit plane, the scale plane and (NVFP4) the 4-byte global scale."""
    return dict(guide=n_elements * code_bits // 8,
                scales=n_elements // BLOCK[fmt],
                gscale=4 if fmt == "nvfp4" else 0)
