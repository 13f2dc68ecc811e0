"""Pins for oracle.sizes against the numbers the paper prints (§3.2, §4.2),
and of the record planes against the 1.5 bits/element claim."""

import pytest

from oracle import sizes


def test_compact_guidance_size(golden):
    g = golden("guidance_sizes.json")
    m, p = g["model"], g["printed"]
    bpe = sizes.bits_per_element("nvfp4", 1)
    assert bpe == p["compact_bits_per_element"]
    bits = sizes.activation_bits_per_token(m["hidden"], m["guided_layers"], bpe)
    assert bits == p["compact_bits_per_token"]
    assert bits / 8 / 1024 == p["compact_KB_per_token"]


def test_full_guidance_size(golden):
    g = golden("guidance_sizes.json")
    m, p = g["model"], g["printed"]
    bpe = sizes.bits_per_element("nvfp4", 4)
    assert bpe == p["full_bits_per_value"]
    act = sizes.activation_bits_per_token(m["hidden"], m["moe_layers"], bpe) / 8
    kv = sizes.kv_bits_per_token(m["kv_head_dim"], m["kv_heads"], m["full_attention_layers"], bpe) / 8
    assert act / 1024 == p["full_activation_KB_per_token"]
    assert round(kv / 1024, 1) == p["full_kv_KB_per_token"]
    # "about 50 KB" in total: 45 KB + 5.625 KB
    assert int((act + kv) / 1024) == p["full_total_KB_per_token"]
    step = sizes.step_bytes(act + kv, m["trajectories"], m["max_response_tokens"])
    assert round(step / 2 ** 40) == p["step_TB"]
    t_gpu = sizes.transfer_seconds(step, p["gpu_to_cpu_GBps"] * 1e9)
    t_sto = sizes.transfer_seconds(step, p["storage_GBps"] * 1e9)
    assert round(t_gpu / 60) == p["gpu_to_cpu_minutes"]
    assert round(t_sto / 3600) == p["storage_hours"]
    # compact (20 layers, 1.5 bits) vs full activation (40 layers, 4.5 bits)
    compact = sizes.activation_bits_per_token(m["hidden"], m["guided_layers"],
                                              sizes.bits_per_element("nvfp4", 1)) / 8
    assert act / compact == p["reduction_factor"]


@pytest.mark.parametrize("fmt,bits,expect", [("nvfp4", 1, 1.5), ("nvfp4", 2, 2.5), ("nvfp4", 3, 3.5),
                                             ("nvfp4", 4, 4.5), ("mxfp4", 1, 1.25), ("mxfp4", 2, 2.25),
                                             ("mxfp4", 3, 3.25), ("mxfp4", 4, 4.25)])
def test_record_planes(fmt, bits, expect):
    n = 8192 * 2048
    p = sizes.record_plane_bytes(n, fmt, bits)
    assert (p["guide"] + p["scales"]) * 8 / n == expect


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_encode_writes_the_counted_planes(bits):
    """The oracle's encode writes exactly the plane sizes counted above."""
    import numpy as np
    from oracle import fp4
    x = np.random.default_rng(bits).integers(0, 0x7F00, 4096).astype(np.uint16)
    o = fp4.encode_guidance(fp4.NVFP4, bits, x)
    p = sizes.record_plane_bytes(x.size, "nvfp4", bits)
    assert o["guide"].size == p["guide"] and o["scales"].size == p["scales"]
