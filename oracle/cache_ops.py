"""KV append, pre-copy of completed pages to the host pool, and demotion of
resident pages (oracle side): the steps on either side of a decode step.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Page "Un contexte d'un million sur huit H200", section "Les trois états de
résidence": with full residency the whole cache is on the GPU and completed
prefix pages are copied to the host ahead of time, so that they can give up
their GPU block later without a new copy; with mixed residency the request's
tail stays on the GPU and is never evicted while older pages live only on the
host.  Section "Ce qui se passe": the indexer's cache stays resident.  Page
"Un contexte..." section "Les trois états", last paragraph: a freed block can
become capacity for another request (one shared pool).

Readings taken (the pages give the states, not the bookkeeping):

* Append.  Each request gains n_new[b] tokens (0 <= n_new[b] <= P, the tokens
  a step accepted), written after its last token: the latent row of every
  layer with its fp32 row scale, and the indexer key.  A token that starts a
  page (t % 64 == 0) opens a new latent block and a new indexer block, popped
  from two free lists; the indexer block takes the fp32 scale supplied with
  that token (keys arrive quantized against their block's scale).  The free
  lists are stacks: blocks[0 .. count-1], the top is blocks[count-1]; pops go
  in request order, then token order.  The call is all-or-nothing: if any
  request would pass T_stride or take more than P tokens, if the page that
  receives a request's first new token is not resident (when that token does
  not open it), or if the pages to open exceed a free list, no token is
  appended and an error bit is set.
* Pre-copy.  A completed page (every one of its 64 tokens below T_b) that is
  resident (bt >= 0) and has no host copy (host_bt < 0) is copied, rows and
  row scales of every layer, to its host slot: host row b * T_stride + 64 * p
  (the host pool reserves a slot per page).  host_bt then records that row.
  At most max_pages pages per request per call, lowest page first.
* Demote.  Under pressure the caller asks each request to give up n_demote[b]
  blocks: the lowest pages that are resident, have a host copy and are not
  among the request's last tail_pages pages (the tail, counted from the page
  holding its last token) lose their block: bt = -1 and the block is pushed on
  the latent free list, in request order then page order.  Fewer pages than
  asked is not an error.  All-or-nothing if the free list would overflow.
  The indexer cache is never demoted.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BLOCK = 64

ERR_APPEND_RANGE = 4      # a request would pass T_stride or P, or its partial last page is not resident
ERR_APPEND_NO_BLOCK = 8   # a free list has fewer blocks than the pages to open
ERR_DEMOTE_FULL = 16      # the latent free list cannot take the demoted blocks


@dataclass
class CacheState:
    """Everything the three operations read or write (numpy arrays, modified in place)."""
    ctx_len: np.ndarray       # [B] int32
    bt: np.ndarray            # [B, T_stride/64] int32, latent block or -1
    idx_bt: np.ndarray        # [B, T_stride/64] int32, indexer block or -1
    host_bt: np.ndarray       # [B, T_stride/64] int64, host row of the page's first token or -1
    pool: np.ndarray          # [L, N_rows, D] latent rows (uint8 codes or float32)
    row_scale: np.ndarray | None    # [L, N_rows] float32
    idx_pool: np.ndarray      # [N_idx_blocks, 64, Dk] keys
    idx_scale: np.ndarray | None    # [N_idx_blocks] float32
    host_rows: np.ndarray     # [L, B*T_stride, D]
    host_scale: np.ndarray | None   # [L, B*T_stride] float32
    free: list = field(default_factory=list)       # latent free list, bottom .. top
    idx_free: list = field(default_factory=list)   # indexer free list
    free_capacity: int = 0

    @property
    def T_stride(self) -> int:
        return self.bt.shape[1] * BLOCK


def _pages_opened(T: int, n: int) -> int:
    """Number of t in [T, T + n) with t % 64 == 0."""
    return sum(1 for t in range(T, T + n) if t % BLOCK == 0)


def append_tokens(st: CacheState, n_new, new_rows, new_row_scale, new_keys, new_key_scale) -> int:
    """Append n_new[b] tokens to every request; returns the error bits.

    new_rows [B, P, L, D], new_row_scale [B, P, L] or None, new_keys [B, P, Dk],
    new_key_scale [B, P] or None (only read for tokens that open a page).
    """
    B = len(st.ctx_len)
    P = np.asarray(new_keys).shape[1]
    n_new = np.asarray(n_new)
    err = 0
    need = 0
    for b in range(B):
        T, n = int(st.ctx_len[b]), int(n_new[b])
        partial = n > 0 and T % BLOCK != 0
        if (n < 0 or n > P or T + n > st.T_stride or
                (partial and (st.bt[b, T // BLOCK] < 0 or st.idx_bt[b, T // BLOCK] < 0))):
            err |= ERR_APPEND_RANGE
            continue
        need += _pages_opened(T, n)
    if need > len(st.free) or need > len(st.idx_free):
        err |= ERR_APPEND_NO_BLOCK
    if err:
        return err
    L = st.pool.shape[0]
    for b in range(B):
        T = int(st.ctx_len[b])
        for i in range(int(n_new[b])):
            t = T + i
            p, r = divmod(t, BLOCK)
            if r == 0:
                st.bt[b, p] = st.free.pop()
                st.idx_bt[b, p] = st.idx_free.pop()
                if st.idx_scale is not None:
                    st.idx_scale[st.idx_bt[b, p]] = np.float32(new_key_scale[b, i])
            row = int(st.bt[b, p]) * BLOCK + r
            for l in range(L):
                st.pool[l, row] = new_rows[b, i, l]
                if st.row_scale is not None:
                    st.row_scale[l, row] = np.float32(new_row_scale[b, i, l])
            st.idx_pool[st.idx_bt[b, p], r] = new_keys[b, i]
        st.ctx_len[b] = T + int(n_new[b])
    return 0


def precopy_pages(st: CacheState, max_pages: int) -> list:
    """Copy up to max_pages completed, resident, not-yet-copied pages per request
    to the host pool.  Returns the (request, page) pairs copied, in order."""
    B = len(st.ctx_len)
    L = st.pool.shape[0]
    done = []
    for b in range(B):
        full = int(st.ctx_len[b]) // BLOCK
        k = 0
        for p in range(full):
            if k == max_pages:
                break
            if st.bt[b, p] < 0 or st.host_bt[b, p] >= 0:
                continue
            src = int(st.bt[b, p]) * BLOCK
            dst = b * st.T_stride + p * BLOCK
            for l in range(L):
                st.host_rows[l, dst:dst + BLOCK] = st.pool[l, src:src + BLOCK]
                if st.host_scale is not None:
                    st.host_scale[l, dst:dst + BLOCK] = st.row_scale[l, src:src + BLOCK]
            st.host_bt[b, p] = dst
            done.append((b, p))
            k += 1
    return done


def demote_pages(st: CacheState, n_demote, tail_pages: int):
    """Give up to n_demote[b] blocks per request (lowest eligible pages first).
    Returns (error bits, list of (request, page, block) demoted in order)."""
    B = len(st.ctx_len)
    plan = []
    for b in range(B):
        T = int(st.ctx_len[b])
        if T == 0:
            continue
        last = (T - 1) // BLOCK
        k = 0
        for p in range(0, last - tail_pages + 1):
            if k == int(n_demote[b]):
                break
            if st.bt[b, p] >= 0 and st.host_bt[b, p] >= 0:
                plan.append((b, p, int(st.bt[b, p])))
                k += 1
    if len(st.free) + len(plan) > st.free_capacity:
        return ERR_DEMOTE_FULL, []
    for b, p, blk in plan:
        st.free.append(blk)
        st.bt[b, p] = -1
    return 0, plan


def logical_rows(st: CacheState, b: int, tokens, layer: int):
    """Rows and scales of tokens as the decode step would read them: from the
    pool when the page is resident, else from the host pool (test helper)."""
    out, sc = [], []
    for t in np.asarray(tokens):
        p, r = divmod(int(t), BLOCK)
        if st.bt[b, p] >= 0:
            row = int(st.bt[b, p]) * BLOCK + r
            out.append(st.pool[layer, row])
            sc.append(None if st.row_scale is None else st.row_scale[layer, row])
        else:
            row = int(st.host_bt[b, p]) + r
            out.append(st.host_rows[layer, row])
            sc.append(None if st.host_scale is None else st.host_scale[layer, row])
    return np.array(out), sc
