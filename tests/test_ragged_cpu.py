"""Host logic of the paged ragged layer: page tables and per-page cache pieces.

A paged cache holds sequence b's row j in row j mod P of page
page_table[b, j // P] of one pool (the layout the ragged calls document);
these checks build the layer on the host and verify the table and the pieces
that seed() copies through, with no GPU involved.
"""
import torch

from long_context_compressed_06_amd.ragged import RaggedLayer


def _layer(**kw):
    args = dict(mode="csa", B=3, H=4, d=32, m=4, W=8, capacity=1000, k=8, HI=4, dI=32, device="cpu")
    args.update(kw)
    return RaggedLayer(**args)


def test_default_page_table_is_a_permutation_of_the_pool():
    L = _layer(page_rows=16)
    assert (L.cap_e, L.max_pages, L.n_pages) == (250, 16, 48)
    t = L.page_table
    assert t.shape == (3, 16) and t.dtype == torch.int32
    ids = t.flatten().tolist()
    assert sorted(ids) == list(range(48))                  # every page once, none shared
    assert L.entries.shape == (48, 16, 32) and L.k_idx.shape == (48, 16, 32)
    # another seed deals the pool differently
    assert not torch.equal(_layer(page_rows=16, seed=1).page_table, t)


def test_cache_pieces_follow_the_page_table():
    L = _layer(page_rows=16)
    L.page_table[1] = torch.arange(47, 31, -1, dtype=torch.int32)  # pages 47, 46, ... for sequence 1
    n = 37
    pieces = L._cache_rows(L.entries, 1, n)
    assert [(lo, hi) for _, lo, hi in pieces] == [(0, 16), (16, 32), (32, 37)]
    for (view, lo, hi), page in zip(pieces, (47, 46, 45)):
        assert view.shape == (hi - lo, 32)
        assert view.data_ptr() == L.entries[page].data_ptr()  # the page's first row
    # writing through the pieces lands row j of the sequence in row j % 16 of its page
    src = torch.arange(n * 32, dtype=torch.float32).reshape(n, 32).to(L.entries.dtype)
    for view, lo, hi in pieces:
        view.copy_(src[lo:hi])
    for j in (0, 15, 16, 31, 32, 36):
        assert torch.equal(L.entries[47 - j // 16, j % 16], src[j])


def test_contiguous_pieces_and_assign_pages():
    L = _layer()
    assert L.pages is None and L.entries.shape == (3, 250, 32)
    [(view, lo, hi)] = L._cache_rows(L.entries, 2, 40)
    assert (lo, hi) == (0, 40) and view.data_ptr() == L.entries[2].data_ptr()
    P = _layer(page_rows=32, n_pages=100)
    P.assign_pages(0, [7, 3])
    assert P.page_table[0, :2].tolist() == [7, 3]
