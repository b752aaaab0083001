"""One decode step, composed from the oracle's stages.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Order of a step ("Un contexte d'un million sur huit H200", sections "Ce qui se
passe" and "Les trois états de résidence"): the indexer scores every cached
token, the top-K is taken, the fused resolve maps every selected token to a
row (faulting host-only rows in), then sparse MLA attention runs.  With
IndexShare one indexer layer serves four sparse-MLA layers (same page,
"Ce qui se passe"), so one score/top-K/resolve feeds L attention layers that
share the residency state, each with its own query and its own latent.

``wl`` is any object with the attributes the generator's workloads carry
(plain numpy arrays); this module does not import the generator.
"""

from __future__ import annotations

import numpy as np

from . import indexer, topk as topk_mod, resolve as resolve_mod, attention


def decode_step(wl, state: resolve_mod.ResidencyState, q_idx, q_layers, pairs=None,
                scores=None, selection=None):
    """Run one step.  ``scores`` / ``selection`` let a caller feed a stage the
    inputs another implementation's previous stage produced (stage isolation).

    Returns a dict with scores, topk, the new state, the resolve result and
    per-layer (out, lse).
    """
    if selection is None:
        if scores is None:
            scores = indexer.indexer_scores(q_idx, wl.q_dtype, wl.w, wl.idx_pool, wl.k_dtype,
                                            wl.idx_scale, wl.idx_bt, wl.ctx_len, wl.bias,
                                            T_stride=wl.T_stride)
        selection = topk_mod.topk(scores, wl.ctx_len, wl.K)
    new_state, rr = resolve_mod.resolve(selection, state)
    outs = []
    for l in range(wl.L):
        outs.append(attention.sparse_mla(q_layers[l], wl.q_dtype, wl.lat[l],
                                         None if wl.lat_scale is None else wl.lat_scale[l],
                                         wl.kv_dtype, selection, wl.sm_scale, pairs=pairs))
    return {"scores": scores, "topk": selection, "state": new_state, "resolve": rr,
            "attn": outs}
