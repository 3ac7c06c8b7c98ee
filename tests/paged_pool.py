"""Scatter of a contiguous KV cache into a shuffled page pool, shared by the paged decode tests.

Pure data movement on seeded inputs: none of the method's arithmetic.
"""

import torch


def paginate(cache, page_size, n_extra, gen):
    """Scatter [B, L, Hkv, D] into a shuffled pool of pages; returns (pool, block_table).

    Pages that no sequence references hold noise, so a read of one shows in a parity check.
    Called twice with a generator in the same state (K, then V), it gives the same table.
    """
    B, L, Hkv, D = cache.shape
    max_pages = (L + page_size - 1) // page_size
    n_pages = B * max_pages + n_extra
    perm = torch.randperm(n_pages, generator=gen, device="cpu")[:B * max_pages].to(cache.device)
    fill = torch.Generator(device=cache.device)
    fill.manual_seed(int(torch.randint(0, 1 << 30, (1,), generator=gen)))
    pool = torch.randn((n_pages, page_size, Hkv, D), generator=fill, device=cache.device).to(cache.dtype)
    padded = torch.zeros((B, max_pages * page_size, Hkv, D), dtype=cache.dtype, device=cache.device)
    padded[:, :L] = cache
    pool[perm] = padded.view(B * max_pages, page_size, Hkv, D)
    return pool, perm.view(B, max_pages).to(torch.int32)


def logical_rows(pool, block_table_row, n):
    """Rows 0..n-1 of one sequence, gathered from a pool [num_pages, page_size, ...] through its
    block-table row (a CPU tensor or array): row j is row j % page_size of page table[j // page_size]."""
    page_size = pool.shape[1]
    j = torch.arange(n)
    pages = torch.as_tensor(block_table_row, dtype=torch.long)[j // page_size]
    return pool[pages, j % page_size]
