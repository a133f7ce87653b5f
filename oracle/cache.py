"""Reference context-cache append after a block is committed (NumPy, exact copies).

Test infrastructure only: imported by tests/, never by the library.

Definition followed (Nemotron-TwoTower explainer, gist.science, "Generierungsprozess"): once every
position of a block is committed, the frozen context tower encodes the block and its keys and
values join the cache that the next block attends to. The cache side of that step, with the
readings this build takes where the pages are silent (they describe no cache layout or page
allocator):

* the block's S rows of every layer go to context positions L .. L+S-1 of the sequence, L being
  its length before the append, which then becomes L+S;
* a row t lives in page block_table[b, t // page_size] at offset t % page_size (the same paging
  as the attention's context reads), stored in the tiled page layouts the attention oracle
  decodes: K [pool, Hkv, page // T, D // CK, T, CK] with element (o, d) at
  [page, g, o // T, d // CK, o % T, d % CK], V [pool, Hkv, page // T, T // CV, D, CV] with
  element (o, d) at [page, g, o // T, (o % T) // CV, d, o % CV] (widths read from the shapes);
* new pages come from the top of a free-page stack (the last valid entry first), sequences
  served in order b = 0, 1, ...; a sequence that does not fit (its table is too short, the stack
  runs out, or a page id it would write is outside the pool) is left untouched and flagged.
"""
from __future__ import annotations

import numpy as np

OUT_OF_PAGES = 1
NO_ROOM_IN_TABLE = 2
BAD_PAGE = 4


def append_block(k_pages, v_pages, block_table, ctx_lens, free_pages, free_count, k_new, v_new):
    """Append the block rows of every layer.

    k_pages / v_pages: lists (one per layer) of arrays as above; k_new[l] [B, Hkv, S, D];
    v_new[l] [B, Hkv, D, S]. Returns new copies (k_pages, v_pages, block_table, ctx_lens,
    free_count, status); the inputs are not modified.
    """
    k_pages = [np.array(k, copy=True) for k in k_pages]
    v_pages = [np.array(v, copy=True) for v in v_pages]
    table = np.array(block_table, dtype=np.int32, copy=True)
    lens = np.array(ctx_lens, dtype=np.int32, copy=True)
    free = np.asarray(free_pages, dtype=np.int32)
    top = int(free_count)
    status = 0
    pool, _, n_tiles, _, T, CK = k_pages[0].shape
    CV = v_pages[0].shape[-1]
    page = n_tiles * T
    B, max_pages = table.shape
    S = k_new[0].shape[2]
    for b in range(B):
        L = int(lens[b])
        if L < 0 or L + S > max_pages * page:
            status |= NO_ROOM_IN_TABLE
            continue
        in_use = -(-L // page)                        # pages holding rows 0 .. L-1
        need = -(-(L + S) // page) - in_use
        if need > top:
            status |= OUT_OF_PAGES
            continue
        new_pages = [int(free[top - 1 - j]) for j in range(need)]
        touched = new_pages + ([int(table[b, L // page])] if L % page else [])
        if any(not 0 <= pg < pool for pg in touched):
            status |= BAD_PAGE
            continue
        for j, pg in enumerate(new_pages):
            table[b, in_use + j] = pg
        top -= need
        for i in range(S):
            t = L + i
            pg, off = int(table[b, t // page]), t % page
            tile, o = off // T, off % T
            for layer in range(len(k_pages)):
                for d in range(k_new[layer].shape[3]):
                    k_pages[layer][pg, :, tile, d // CK, o, d % CK] = k_new[layer][b, :, i, d]
                v_pages[layer][pg, :, tile, o // CV, :, o % CV] = v_new[layer][b, :, :, i]
        lens[b] = L + S
    return k_pages, v_pages, table, lens, top, status
