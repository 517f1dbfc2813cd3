"""Pins of the oracle's paged layout and multi-token appends.

A paged cache keeps its tile records in a pool of pages found through a page map
(one page = the K and V records of every kv head for one group of one sequence); the
same tokens must give the same records, dequantized values and attention as the
per-sequence layout, whatever pages the map names. append_tokens must equal that many
single-token appends, and a chunk appended to a prefilled cache must equal one prefill of
the whole sequence (appends are bit-identical to prefill).
"""
import numpy as np

from oracle import kvarn_ref as R
from kv_cache_bit_amd import synth

B, H, G, CAP = 3, 2, 32, 128
TILES = CAP // G


def cache(paged=False, n_it=3, pages=None):
    g = R.Geom(B, H, 128, CAP, G, n_it, 2, 0, (B * TILES + 2) if paged else 0)
    c = R.Cache(g, synth.sign_vector(8))
    if paged:
        c.set_pages(pages if pages is not None else np.arange(B * TILES).reshape(B, TILES))
    return c


def same_tokens(a: R.Cache, b: R.Cache):
    """Equal lengths, tail bytes and record bytes of every stored tile."""
    assert np.array_equal(a.lens, b.lens)
    for bb in range(B):
        for h in range(H):
            for s in range(2):
                n = int(a.lens[bb, h, s])
                for tile in range(n // G):
                    ra, rb = a.record(bb, h, tile, s), b.record(bb, h, tile, s)
                    assert ra is not None and rb is not None and np.array_equal(ra, rb), (bb, h, tile, s)
                assert np.array_equal(a.tail(bb, h, s)[:n % G], b.tail(bb, h, s)[:n % G])


def test_header_and_layout():
    c = cache(paged=True, pages=np.full((B, TILES), -1))
    g = c.g
    assert g.map_offset == 512 + 8 * B * H
    assert g.header == R.align256(512 + 8 * B * H + 4 * B * TILES)
    assert g.tail_offset == g.header + R.align256((B * TILES + 2) * H * 2 * g.tr)
    assert np.all(c.page_map == -1)
    assert c.record(0, 0, 0, 0) is None
    # the per-sequence layout's header has no map
    assert cache().g.header == R.align256(512 + 8 * B * H)


def test_append_tokens_equals_prefill_and_chunks():
    T1, T2 = 45, 50
    k, v = synth.kv_host(40, B, T1 + T2, H)
    whole = cache()
    R.quantize_prefill(whole, k, v, T1 + T2)
    chunked = cache()
    R.quantize_prefill(chunked, k[:, :T1], v[:, :T1], T1)
    R.append_tokens(chunked, k[:, T1:], v[:, T1:])
    same_tokens(whole, chunked)
    fresh = cache()
    R.append_tokens(fresh, k, v)
    same_tokens(whole, fresh)


def test_ragged_counts_and_masks():
    """Sequence b takes counts[b] tokens; each sequence equals a cache holding only it."""
    T = 70
    k, v = synth.kv_host(41, B, T, H)
    counts = np.array([70, 0, 33])
    c = cache()
    R.append_tokens(c, k, v, counts)
    assert np.array_equal(c.lens[:, 0, 0], counts)
    for bb in range(B):
        one = cache()
        kb, vb = np.repeat(k[bb:bb + 1], B, 0), np.repeat(v[bb:bb + 1], B, 0)
        R.append_tokens(one, kb, vb, np.full(B, counts[bb]))
        n = counts[bb]
        for h in range(H):
            for s in range(2):
                for tile in range(n // G):
                    assert np.array_equal(one.record(0, h, tile, s), c.record(bb, h, tile, s))
                assert np.array_equal(one.tail(0, h, s)[:n % G], c.tail(bb, h, s)[:n % G])
    # a mask (counts 0/1) leaves the other sequences' bytes alone
    before = c.buf.copy()
    R.append_tokens(c, k[:, :1], v[:, :1], np.array([0, 1, 0]))
    assert np.array_equal(c.lens[:, 0, 0], counts + np.array([0, 1, 0]))
    changed = np.nonzero(before != c.buf)[0]
    rows = [c.g.tail_slot_offset(1, h, s, 0) for h in range(H) for s in range(2)]
    for o in changed:  # the new tail rows of sequence 1 and its len entries only
        in_tail = any(r <= o < r + 256 for r in rows)
        in_len = 512 + 4 * 2 * H * 1 <= o < 512 + 4 * 2 * H * 2
        assert in_tail or in_len, o


def test_paged_equals_per_sequence_layout():
    """A shuffled page map (and two spare pages) stores the same records, dequantizes to the
    same values and gives the same attention as the per-sequence layout."""
    rng = np.random.default_rng(0)
    pages = rng.permutation(B * TILES + 2)[:B * TILES].reshape(B, TILES)
    T = 100
    k, v = synth.kv_host(42, B, T + 3, H)
    a, p = cache(), cache(paged=True, pages=pages)
    for c in (a, p):
        R.quantize_prefill(c, k[:, :T], v[:, :T], T)
        R.append_tokens(c, k[:, T:], v[:, T:])
    same_tokens(a, p)
    assert p.flags & R.FLAG_UNMAPPED == 0
    ka, va = R.dequantize(a, CAP)
    kp, vp = R.dequantize(p, CAP)
    assert np.array_equal(ka, kp) and np.array_equal(va, vp)
    q = synth.q_host(43, B, 4)
    assert np.array_equal(R.attn_decode(a, q, 4), R.attn_decode(p, q, 4))
    # records sit where the map says: page pages[b][tile], head h, stream s
    g = p.g
    o = g.page_offset(int(pages[1, 2]), 1, 1)
    assert np.array_equal(p.buf[o:o + g.tr], a.record(1, 1, 2, 1))


def test_unmapped_tiles_are_skipped_and_flagged():
    """Without pages the writers drop the tiles (FLAG_UNMAPPED); dequantization gives zeros
    for their tokens and attention skips them, so a cache of 2G + 5 tokens without pages
    attends like a cache holding only its 5 tail tokens."""
    T = 2 * G + 5
    k, v = synth.kv_host(44, B, T, H)
    p = cache(paged=True, pages=np.full((B, TILES), -1))
    R.quantize_prefill(p, k, v, T)
    assert p.flags & R.FLAG_UNMAPPED
    kd, _ = R.dequantize(p, T)
    assert np.all(kd[:, :2 * G] == 0)
    only_tail = cache()
    R.quantize_prefill(only_tail, k[:, 2 * G:], v[:, 2 * G:], 5)
    q = synth.q_host(45, B, 4)
    assert np.allclose(R.attn_decode(p, q, 4), R.attn_decode(only_tail, q, 4), rtol=1e-13, atol=0)
