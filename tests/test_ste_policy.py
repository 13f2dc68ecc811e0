"""The guided-layer policy (§3.2 "Key Design"; §4.3 "Modular Sensitivity
Study": records for the latter 20 of 40 layers, or 40, 10, 5). Host logic
only, no GPU."""

import pytest

from precision_rl_nvfp4_amd import ste


@pytest.mark.parametrize("keep,first", [(40, 0), (20, 20), (10, 30), (5, 35), (0, 40)])
def test_deepest_layers_are_guided(keep, first):
    r = ste.guided_layers(40, keep)
    assert list(r) == list(range(first, 40))
    assert len(r) == keep


def test_default_is_the_latter_half():
    assert list(ste.guided_layers(40)) == list(range(20, 40))
    assert list(ste.guided_layers(7)) == [4, 5, 6]


@pytest.mark.parametrize("n,keep", [(40, 41), (40, -1), (-1, None)])
def test_rejects_bad_policy(n, keep):
    with pytest.raises(ValueError):
        ste.guided_layers(n, keep)


def test_qat_dispatch_keeps_records_of_guided_layers_only():
    qat = ste.GuidedQAT(40, 20)
    assert not qat.is_guided(19) and qat.is_guided(20) and qat.is_guided(39)
    qat.put("act", 3, object())          # not a guided layer: dropped
    qat.put("act", 25, "record")
    assert list(qat.records) == [(25, "act")]
    qat.clear()
    assert not qat.records
