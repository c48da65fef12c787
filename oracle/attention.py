"""Oracle for stage 3: varlen GQA verify attention over a paged KV cache.

TEST INFRASTRUCTURE (see the package docstring): never imported by the product path.

Paged cache layout (the pages only say the cache is paged with a page table kept on the
device, [SGL] "Zero-overhead scheduling 与 kernel"; the layout below is this library's
documented choice):

* ``k_cache[page, kv_head, slot, d]``  -- shape [num_pages, Hkv, page_size, D]
* ``v_cache[page, kv_head, slot // VB, d, slot % VB]`` -- shape
  [num_pages, Hkv, page_size // VB, D, VB]: V transposed in column blocks of VB slots,
  VB = 32 when page_size is a multiple of 32, else VB = page_size
* sequence position p of request b lives in physical page
  ``block_table[b, p // page_size]`` at slot ``p % page_size``.
"""

from __future__ import annotations

import math

import numpy as np


def _softmax_weights(scores):
    m = np.max(scores)
    e = np.exp(scores - m)
    return e / np.sum(e)


def verify_attention(q, k_new, v_new, k_cache, v_cache, block_table, context_lens,
                     cu_seqlens, tier, softmax_scale):
    """Per-token attention of the packed verify rows, each against its own request only.

    [SGL] "Ragged verify under full CUDA graphs" and [CSDN] section 3: each packed token
    attends only to its own request's KV, delimited by cu_seqlens; the window's own
    tokens are causal among themselves.  For window row i of request b (packed row
    ``r = cu[b] + i``) and query head h in kv group ``g = h // (Hq // Hkv)``:

    * visible keys/values: cache positions ``0 .. L_b - 1`` read through the page table,
      then the window's own rows ``0 .. i`` taken from ``k_new``/``v_new``;
    * ``o = softmax(q . K^T * scale) V``, everything in float64 on the given inputs.

    Rows ``M .. tier-1`` (padding) are zero.  The window's K/V are also written into the
    cache at positions ``L_b + i`` (returned as updated copies of both caches).

    Shapes: q [R, Hq, D], k_new/v_new [R, Hkv, D] with R >= tier, k_cache
    [P, Hkv, page, D], v_cache [P, Hkv, page // VB, D, VB], block_table [B, max_pages].
    Returns (out [R, Hq, D] float64, k_cache', v_cache').
    """
    q = np.asarray(q, dtype=np.float64)
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    k_cache = np.array(k_cache, dtype=np.float64, copy=True)
    v_cache = np.array(v_cache, dtype=np.float64, copy=True)
    R, Hq, D = q.shape
    Hkv = k_new.shape[1]
    page = k_cache.shape[2]
    VB = v_cache.shape[4]
    assert VB == v_block(page) and v_cache.shape[2] * VB == page
    assert Hq % Hkv == 0
    group = Hq // Hkv
    scale = float(np.float32(softmax_scale))
    B = len(context_lens)
    out = np.zeros((R, Hq, D), dtype=np.float64)

    for b in range(B):
        L = int(context_lens[b])
        r0, r1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        w = r1 - r0
        # keys/values of the cached context, gathered through the page table
        Kc = np.empty((Hkv, L, D))
        Vc = np.empty((Hkv, L, D))
        for p in range(L):
            pg = int(block_table[b, p // page])
            s = p % page
            Kc[:, p, :] = k_cache[pg, :, s, :]
            Vc[:, p, :] = v_cache[pg, :, s // VB, :, s % VB]
        for i in range(w):
            r = r0 + i
            for h in range(Hq):
                g = h // group
                K = np.concatenate([Kc[g], k_new[r0:r + 1, g, :]], axis=0)
                V = np.concatenate([Vc[g], v_new[r0:r + 1, g, :]], axis=0)
                s = (K @ q[r, h]) * scale
                out[r, h] = _softmax_weights(s) @ V
        # append the window's K/V at positions L .. L + w - 1
        for i in range(w):
            p = L + i
            pg = int(block_table[b, p // page])
            s = p % page
            k_cache[pg, :, s, :] = k_new[r0 + i]
            v_cache[pg, :, s // VB, :, s % VB] = v_new[r0 + i]
    # rows M .. tier-1 stay zero (already zero)
    return out, k_cache, v_cache


def v_block(page_size):
    """Column-block width of the V cache layout (see the module docstring)."""
    return 32 if page_size % 32 == 0 else page_size


def default_scale(D):
    """Softmax scale 1/sqrt(D) (float32), the usual dot-product attention scale."""
    return np.float32(1.0 / math.sqrt(D))
