"""Record path on the GPU: ring copies are byte-exact and ordered after the
producer's work, the slot cycle (busy, wait, release, wrap-around) behaves
as declared, and the page gather matches the oracle's (ragged and word-sized
pages, bad ids, empty lists)."""

import numpy as np
import pytest
import torch

import precision_rl_nvfp4_amd as tq
import synthetic as syn
from oracle import fp4 as ofp4
from oracle import record as orec
from precision_rl_nvfp4_amd import _abi
from precision_rl_nvfp4_amd.record import RecordRing, gather_pages
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def test_ring_copies_encode_outputs_without_a_host_sync():
    """encode_guidance, then push its planes on the same stream at once: the
    slot holds exactly the planes (the copy waited for the kernel)."""
    G.say("record ring: encode outputs")
    xt, xr = syn.activation_pair(512, 2048, (93, 0))
    r = xr.to(G.DEV)
    with RecordRing(1 << 20, 3) as ring:
        g = tq.encode_guidance(r, "nvfp4", 1)
        slot = ring.push([g.guide, g.scales, g.gscale])
        ring.wait(slot)
        host = ring.view(slot)
        want = np.concatenate([G.u8(g.guide), G.u8(g.scales),
                               g.gscale.cpu().numpy().view(np.uint8).reshape(-1)])
        assert host.size == want.size == 512 * 2048 // 8 + 512 * 2048 // 16 + 8
        G.assert_same(host, want, "slot bytes")
        ring.release(slot)


def test_ring_keeps_pushed_tensors_until_copied():
    """Push a record's planes and drop them at once, then let the producer
    stream allocate and overwrite memory of the same sizes before the ring's
    copies are waited on: the slot still holds the record's bytes (the ring
    keeps the sources alive until the copies are done)."""
    G.say("record ring: sources dropped right after push")
    _, xr = syn.activation_pair(1024, 2048, (94, 0))
    r = xr.to(G.DEV)
    xr_b = G.bits_of(r)
    o = ofp4.encode_guidance(ofp4.NVFP4, 1, xr_b)
    want = np.concatenate([o["guide"], o["scales"], np.array([o["gscale"], o["amax"]], np.float32).view(np.uint8)])
    with RecordRing(1 << 20, 2) as ring:
        # keep the producer stream busy so the copies cannot start before
        # the overwrites below are enqueued
        busy = torch.empty(1 << 28, dtype=torch.uint8, device=G.DEV)
        g = tq.encode_guidance(r, "nvfp4", 1)
        for _ in range(8):
            busy.fill_(3)
        slot = ring.push([g.guide, g.scales, g.gscale])
        sizes = [(t.numel(), t.dtype) for t in (g.guide, g.scales, g.gscale)]
        del g
        junk = [torch.full((n,), 0x5A, dtype=torch.uint8, device=G.DEV) if dt == torch.uint8 else
                torch.full((n,), -1.0, dtype=dt, device=G.DEV) for n, dt in sizes]
        ring.wait(slot)
        G.assert_same(ring.view(slot), want, "slot bytes after the sources were dropped")
        ring.release(slot)
        del junk, busy


def test_ring_slot_cycle():
    G.say("record ring: slot cycle")
    a = torch.arange(4096, dtype=torch.int32, device=G.DEV)
    with RecordRing(a.numel() * 4, 2) as ring:
        s0 = ring.push([a])
        s1 = ring.push([a[:10]])
        assert (s0, s1) == (0, 1)
        with pytest.raises(_abi.TraceError) as e:
            ring.push([a])                            # slot 0 not released
        assert e.value.status == _abi.EBUSY
        with pytest.raises(_abi.TraceError):
            ring.release(s0)                          # not waited on yet
        ring.wait(s0)
        assert ring.ready(s0)
        np.testing.assert_array_equal(ring.view(s0).view(np.int32), np.arange(4096, dtype=np.int32))
        ring.release(s0)
        with pytest.raises(_abi.TraceError):
            ring.push([a, a[:1]])                     # more than a slot
        s2 = ring.push([a[100:200]])                  # wraps to slot 0
        assert s2 == 0
        ring.wait(s1)
        ring.wait(s2)
        np.testing.assert_array_equal(ring.view(s1).view(np.int32), np.arange(10, dtype=np.int32))
        np.testing.assert_array_equal(ring.view(s2).view(np.int32), np.arange(100, 200, dtype=np.int32))
        with pytest.raises(RuntimeError):
            ring.release(s1)
            ring.view(s1)                             # released: no longer readable


@pytest.mark.parametrize("page_bytes,npool,n", [(4096, 64, 200), (48, 37, 101), (40, 33, 77), (1, 5, 9),
                                                (16, 8, 0)])
def test_gather_pages_vs_oracle(page_bytes, npool, n):
    G.say(f"gather pages page_bytes={page_bytes} pool={npool} n={n}")
    rng = np.random.default_rng(page_bytes + n)
    pool = rng.integers(0, 256, npool * page_bytes).astype(np.uint8)
    ids = rng.integers(-3, npool + 3, n).astype(np.int32)
    dpool = torch.from_numpy(pool).to(G.DEV)
    dids = torch.from_numpy(ids).to(G.DEV)
    bad = torch.zeros(1, dtype=torch.int32, device=G.DEV)
    out = gather_pages(dpool, page_bytes, dids, bad=bad.view(torch.uint32))
    want, nbad = orec.gather_pages(pool, page_bytes, ids)
    G.assert_same(out.cpu().numpy(), want, "gathered pages")
    assert int(bad.cpu()[0]) == nbad


def test_gather_kv_planes_of_a_request():
    """A paged FP4 KV cache: pages of 16 tokens x (2 heads x 256) codes, a
    request owning a scattered list of pages; the gathered code plane equals
    the request's codes in token order."""
    G.say("gather: KV request pages")
    tokens_per_page, row_bytes = 16, 2 * 256 // 2
    page_bytes = tokens_per_page * row_bytes
    npool = 512
    rng = np.random.default_rng(7)
    pool = rng.integers(0, 256, npool * page_bytes).astype(np.uint8)
    pages = rng.permutation(npool)[:45].astype(np.int32)
    out = gather_pages(torch.from_numpy(pool).to(G.DEV), page_bytes, torch.from_numpy(pages).to(G.DEV))
    want = pool.reshape(npool, page_bytes)[pages].reshape(-1)
    G.assert_same(out.cpu().numpy(), want, "request codes")
