"""Seeded synthetic inputs shaped like the workloads of the TRACE paper.

This module only draws random tensors. It holds none of the quantization
arithmetic: no scales, no rounding, no codes. Both the CPU oracle and the
HIP path take their inputs from here, so that they see identical bytes.

Paper: "TRACE: Rollout-Guided Quantization-Aware Training for FP4
Reinforcement Learning of MoE Language Models" (arXiv 2610.07767).
The shapes follow its model description in §3.2 (hidden size 2048, KV head
dimension 256, two KV heads, 40 MoE layers) and its guidance policy in
§3.2 / §4.2 (the deepest 20 layers carry guidance).

Every generator takes a ``device``: on a GPU the draw is fast enough for the
full streamed workload; on the CPU it gives the small cases the oracle runs.
The same seed on two devices gives two different (but each reproducible)
tensors, because torch's CPU and GPU generators differ. A test therefore
generates once and hands the same tensor to both sides.

All tensors are returned as ``torch.bfloat16``.
"""

from __future__ import annotations

import torch

HIDDEN = 2048          # activation hidden size (§3.2)
KV_HEADS = 2           # KV heads (§3.2)
HEAD_DIM = 256         # KV head dimension (§3.2)
MOE_LAYERS = 40        # MoE layers (§3.2)
GUIDED_LAYERS = tuple(range(20, 40))   # deepest 20 of 40 (§3.2, §4.2)
NUM_EXPERTS = 256
TOP_K = 8
STREAM_TOKENS = 8192 + 131072          # 8K prompt + 128K response
STREAM_CHUNK = 8192
STREAM_CHUNKS = STREAM_TOKENS // STREAM_CHUNK   # 17

# Config ids used to separate seed streams.
CFG_TINY, CFG_MOE, CFG_KV, CFG_MX, CFG_STREAM = 1, 2, 3, 4, 5


def _gen(device, *key: int) -> torch.Generator:
    """A generator seeded from a tuple of small non-negative ints."""
    seed = 0
    for k in key:
        seed = seed * 1_000_003 + int(k) + 1
    g = torch.Generator(device=device)
    g.manual_seed(seed % (2 ** 62))
    return g


def _student_t4(shape, g, device) -> torch.Tensor:
    """Student-t with 4 degrees of freedom, as Z / sqrt(V / 4).

    V is chi-square with 4 degrees of freedom, drawn as -2 ln(U1 U2)
    (the sum of two exponentials of mean 2). U is taken in (0, 1].
    """
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    u1 = 1.0 - torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    u2 = 1.0 - torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    v = -2.0 * (torch.log(u1) + torch.log(u2))
    return z * torch.rsqrt(v * 0.25)


def channel_scales(cols: int, g, device) -> torch.Tensor:
    """Per-channel log-normal(0, 1) scale, exp(N(0, 1))."""
    return torch.exp(torch.randn(cols, generator=g, device=device, dtype=torch.float32))


def rollout_from_train(x_t: torch.Tensor, std: float, g, device) -> torch.Tensor:
    """Rollout copy: bf16(x_t * (1 + eps)), eps ~ N(0, std) (std, not variance)."""
    eps = torch.randn(x_t.shape, generator=g, device=device, dtype=torch.float32)
    return (x_t.float() * (1.0 + std * eps)).to(torch.bfloat16)


def activation_pair(rows: int, cols: int, key, device="cpu", noise_std=0.01,
                    sigma: torch.Tensor | None = None):
    """Train/rollout activation pair: Student-t(4) times a per-channel
    log-normal scale, rounded to bf16; rollout = train * (1 + N(0, 0.01)).

    ``key`` is a tuple of ints naming the seed stream. ``sigma`` (float32 [cols])
    overrides the channel scales, so chunks of one layer can share them.
    """
    g = _gen(device, *key)
    if sigma is None:
        sigma = channel_scales(cols, g, device)
    x_t = (_student_t4((rows, cols), g, device) * sigma).to(torch.bfloat16)
    x_r = rollout_from_train(x_t, noise_std, g, device)
    return x_t, x_r


def tiny_pair(device="cpu"):
    """256 tokens x 2048 hidden, seed 0."""
    return activation_pair(256, HIDDEN, (CFG_TINY, 0), device)


def moe_routing(tokens: int, layer: int, device="cpu"):
    """Top-8 of 256 experts over a seeded N(0, 1) logit matrix.

    Returns (token index per permuted row, expert offsets [E + 1]). Rows are
    sorted by (expert, token). Ties in the logits go to the lower expert id.
    """
    g = _gen(device, CFG_MOE, layer, 7)
    logits = torch.randn((tokens, NUM_EXPERTS), generator=g, device=device,
                         dtype=torch.float32)
    # torch.topk is not guaranteed stable; break ties by expert id explicitly
    # with a stable sort on (-logit).
    order = torch.sort(-logits, dim=1, stable=True).indices[:, :TOP_K]
    tok = torch.arange(tokens, device=device).repeat_interleave(TOP_K)
    exp = order.reshape(-1)
    key = exp.to(torch.int64) * tokens + tok
    perm = torch.sort(key, stable=True).indices
    rows_token = tok[perm]
    counts = torch.bincount(exp, minlength=NUM_EXPERTS)
    offsets = torch.zeros(NUM_EXPERTS + 1, dtype=torch.int64, device=device)
    offsets[1:] = torch.cumsum(counts, 0)
    return rows_token, offsets


def moe_pair(layer: int, tokens: int = 8192, device="cpu"):
    """Routed-expert inputs of one MoE layer: token activations permuted into
    (expert, token) order, 8 rows per token. Train and rollout share the
    routing (routing replay), so a row of X_t and X_r is the same token."""
    x_t_tok, x_r_tok = activation_pair(tokens, HIDDEN, (CFG_MOE, layer), device)
    rows_token, offsets = moe_routing(tokens, layer, device)
    return x_t_tok[rows_token].contiguous(), x_r_tok[rows_token].contiguous(), rows_token, offsets


def kv_pair(layer: int, which: int, tokens: int = 32768, device="cpu"):
    """K (which=0) or V (which=1) of one layer as [tokens * 2 heads, 256]:
    N(0, 1) with 5 of the 512 head-channels (1%) scaled by 20, chosen per
    tensor; rollout = train * (1 + N(0, 0.005))."""
    g = _gen(device, CFG_KV, layer, which)
    x = torch.randn((tokens, KV_HEADS * HEAD_DIM), generator=g, device=device,
                    dtype=torch.float32)
    n_out = round(0.01 * KV_HEADS * HEAD_DIM)
    chans = torch.randperm(KV_HEADS * HEAD_DIM, generator=g, device=device)[:n_out]
    x[:, chans] *= 20.0
    x_t = x.to(torch.bfloat16)
    x_r = rollout_from_train(x_t, 0.005, g, device)
    return (x_t.reshape(tokens * KV_HEADS, HEAD_DIM).contiguous(),
            x_r.reshape(tokens * KV_HEADS, HEAD_DIM).contiguous())


# Magnitudes, in units of the block's power-of-two step 2^(floor(log2 amax) - 2),
# that sit exactly halfway between two neighbouring E2M1 magnitudes.
MIDPOINT_MULTIPLES = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _inject_midpoints(x: torch.Tensor, frac: float, block: int, g, device) -> torch.Tensor:
    """Overwrite a fraction ``frac`` of the elements with values lying on the
    E2M1 midpoints of their 32-element block's power-of-two grid.

    The grid step of a block is 2^(floor(log2 amax) - 2): the binade of the
    block's largest magnitude, shifted down by two. Every injected magnitude is
    below 2^(floor(log2 amax) + 1), so the block's binade does not change. The
    block's largest element is never overwritten. Signs are random.
    """
    flat = x.reshape(-1, block).float()
    nblk = flat.shape[0]
    amax, arg = flat.abs().max(dim=1)
    _, e = torch.frexp(amax)                 # amax = m * 2^e, m in [0.5, 1)
    step = torch.ldexp(torch.ones_like(amax), (e - 3).to(torch.int32))  # 2^(floor(log2 amax) - 2)
    n = flat.numel()
    k = int(round(frac * n))
    pos = torch.randperm(n, generator=g, device=device)[: 2 * k]
    pos = pos[(pos % block) != arg[pos // block]][:k]
    m = torch.tensor(MIDPOINT_MULTIPLES, device=device, dtype=torch.float32)
    pick = torch.randint(0, len(MIDPOINT_MULTIPLES), (pos.numel(),), generator=g, device=device)
    sign = torch.where(torch.rand(pos.numel(), generator=g, device=device) < 0.5, -1.0, 1.0)
    bi = pos // block
    vals = sign * m[pick] * step[bi]
    ok = amax[bi] > 0
    out = flat.reshape(-1).clone()
    out[pos[ok]] = vals[ok]
    return out.reshape(x.shape).to(torch.bfloat16)


def mxfp4_pair(rows: int = 65536, cols: int = HIDDEN, device="cpu", frac: float = 0.001,
               layer: int | None = None):
    """MXFP4 workload: the Student-t / log-normal pair plus 0.1% of the
    elements placed exactly on E2M1 rounding midpoints of their block, in the
    train tensor and, independently, in the rollout tensor. ``layer`` draws an
    independent pair per deep layer (None: the single-tensor workload)."""
    g = _gen(device, CFG_MX, rows) if layer is None else _gen(device, CFG_MX, rows, layer)
    sigma = channel_scales(cols, g, device)
    x_t = (_student_t4((rows, cols), g, device) * sigma).to(torch.bfloat16)
    x_t = _inject_midpoints(x_t, frac, 32, g, device)
    x_r = rollout_from_train(x_t, 0.01, g, device)
    x_r = _inject_midpoints(x_r, frac, 32, g, device)
    return x_t, x_r


def stream_sigma(layer: int, device="cpu") -> torch.Tensor:
    """Per-layer channel scales of the streamed workload."""
    g = _gen(device, CFG_STREAM, layer, 10 ** 6)
    return channel_scales(HIDDEN, g, device)


def stream_pair(layer: int, chunk: int, device="cpu", sigma: torch.Tensor | None = None,
                rows: int = STREAM_CHUNK):
    """One 8192-token chunk of one deep layer of the 136K-token stream."""
    if sigma is None:
        sigma = stream_sigma(layer, device)
    return activation_pair(rows, HIDDEN, (CFG_STREAM, layer, chunk), device, sigma=sigma)


def bits_u16(x: torch.Tensor):
    """bf16 tensor -> numpy uint16 array of its bit patterns (host copy)."""
    return x.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")
