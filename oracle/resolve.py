"""The fused resolve step: residency state machine (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The page "Un contexte d'un million sur huit H200", section "Les trois états de
résidence", describes the mechanism: in mixed residency the request's tail
stays on the GPU and is never evicted, older pages live only in host memory,
and rows the indexer asks for are placed in hot buffers.  One fused kernel
resolves the top-K: resident tokens are read in place, hot tokens refresh
their LRU entry, and a fault copies a single row from pinned host memory.
Nothing on the decode path waits for a CPU decision.  Hot buffers are ordinary
blocks of the same pool (same section, last paragraph; restated on
"A vLLM új módszere ..." under "Csak a fontos tokenek maradnak a
gyorsítón").  Default capacity is 2 x top-K rows per request, and
(num_speculative_tokens + 2) x top-K with MTP ("Ce qu'il faut en retenir").

The pages name an LRU but give no policy.  Reading taken (bit-exact contract
between this oracle and the GPU):

1. One step number s = step + 1 for the whole call; step <- s afterwards.
2. Per request b, U = the sorted distinct tokens selected by any position.
3. Each t in U, in ascending order, with page j = t // 64:
   * bt[b, j] >= 0           -> RESIDENT, row = bt[b, j] * 64 + t % 64
   * tok2slot[b, t] = v >= 0 -> HIT, stamp[b, v] <- s,
                                row = hot_blocks[b, v // 64] * 64 + v % 64
   * host_bt[b, j] < 0       -> unresolvable (no copy anywhere): error bit 2,
                                row -1, no slot
   * otherwise               -> FAULT, appended to F (ascending tokens)
4. Victims: every slot v with stamp[b, v] < s (hits were refreshed first, so
   no slot used in this step is a victim), ordered by (stamp, v) ascending;
   empty slots carry stamp 0 and come first.  The i-th fault takes the i-th
   victim.  Faults beyond the number of victims set error bit 1 and get row -1.
5. Fault t -> victim v: if slot2tok[b, v] = old >= 0 then tok2slot[b, old] <- -1
   (an eviction); slot2tok[b, v] <- t; tok2slot[b, t] <- v; stamp[b, v] <- s;
   for every layer l the 576-element row host_l[host_bt[b, j] + t % 64] and
   its scale are copied to pool row hot_blocks[b, v // 64] * 64 + v % 64.
6. row_ids[b, p, k] = row of topk[b, p, k] (-1 stays -1);
   counts[b] = (#resident, #hit, #fault served, #evicted), over U.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BLOCK = 64


@dataclass
class ResidencyState:
    """Mutable residency tables of a batch (all int32 except host_bt)."""
    bt: np.ndarray            # [B, max_blocks]  physical latent block, -1 = host-only page
    hot_blocks: np.ndarray    # [B, C // 64]     pool blocks forming the hot buffer
    tok2slot: np.ndarray      # [B, T_stride]    hot slot of a token, -1 = not hot
    slot2tok: np.ndarray      # [B, C]           token held by a slot, -1 = empty
    stamp: np.ndarray         # [B, C]           last step that used the slot, 0 = never
    host_bt: np.ndarray       # [B, max_blocks]  int64 host row of token 64*j, -1 = none
    step: int = 0

    def copy(self) -> "ResidencyState":
        return ResidencyState(self.bt.copy(), self.hot_blocks.copy(), self.tok2slot.copy(),
                              self.slot2tok.copy(), self.stamp.copy(), self.host_bt.copy(),
                              int(self.step))


@dataclass
class ResolveResult:
    row_ids: np.ndarray                   # [B, P, K] int32
    counts: np.ndarray                    # [B, 4] int32: resident, hit, fault, evicted
    faults: list = field(default_factory=list)   # per request: int32 [n, 2] (token, slot)
    copies: list = field(default_factory=list)   # per request: int64 [n, 2] (host row, pool row)
    err: int = 0
    classes: list = field(default_factory=list)  # per request: (U, class) 0=res 1=hit 2=fault 3=unresolvable


def slot_row(hot_blocks_row: np.ndarray, v):
    """Pool row of hot slot v."""
    v = np.asarray(v, dtype=np.int64)
    return hot_blocks_row[v // BLOCK].astype(np.int64) * BLOCK + v % BLOCK


def resolve(topk: np.ndarray, state: ResidencyState) -> tuple[ResidencyState, ResolveResult]:
    """One resolve call.  Returns the new state (inputs are not modified)."""
    st = state.copy()
    B, P, K = topk.shape
    C = st.slot2tok.shape[1]
    s = st.step + 1
    st.step = s
    row_ids = np.full((B, P, K), -1, dtype=np.int32)
    counts = np.zeros((B, 4), dtype=np.int32)
    res = ResolveResult(row_ids=row_ids, counts=counts)
    err = 0
    for b in range(B):
        sel = topk[b].reshape(-1)
        U = np.unique(sel[sel >= 0]).astype(np.int64)        # sorted distinct
        row_of = {}
        cls = np.zeros(len(U), dtype=np.int8)
        F = []
        for i, t in enumerate(U):
            j = t // BLOCK
            if st.bt[b, j] >= 0:
                cls[i] = 0
                row_of[t] = int(st.bt[b, j]) * BLOCK + t % BLOCK
            elif st.tok2slot[b, t] >= 0:
                v = int(st.tok2slot[b, t])
                cls[i] = 1
                st.stamp[b, v] = s
                row_of[t] = int(slot_row(st.hot_blocks[b], v))
            elif st.host_bt[b, j] < 0:
                cls[i] = 3
                err |= 2
                row_of[t] = -1
            else:
                cls[i] = 2
                F.append(int(t))
        # victims: (stamp, slot) ascending over slots not used in this step
        cand = np.nonzero(st.stamp[b] < s)[0]
        order = np.lexsort((cand, st.stamp[b][cand]))
        victims = cand[order]
        n_served = min(len(F), len(victims))
        if n_served < len(F):
            err |= 1
        evicted = 0
        flist = np.zeros((n_served, 2), dtype=np.int32)
        clist = np.zeros((n_served, 2), dtype=np.int64)
        for i in range(n_served):
            t, v = F[i], int(victims[i])
            old = int(st.slot2tok[b, v])
            if old >= 0:
                st.tok2slot[b, old] = -1
                evicted += 1
            st.slot2tok[b, v] = t
            st.tok2slot[b, t] = v
            st.stamp[b, v] = s
            prow = int(slot_row(st.hot_blocks[b], v))
            row_of[t] = prow
            flist[i] = (t, v)
            clist[i] = (int(st.host_bt[b, t // BLOCK]) + t % BLOCK, prow)
        for t in F[n_served:]:
            row_of[t] = -1
        for p in range(P):
            for k in range(K):
                t = int(topk[b, p, k])
                row_ids[b, p, k] = -1 if t < 0 else row_of[t]
        counts[b] = (int(np.sum(cls == 0)), int(np.sum(cls == 1)), n_served, evicted)
        res.faults.append(flist)
        res.copies.append(clist)
        res.classes.append((U, cls))
    res.err = err
    return st, res

