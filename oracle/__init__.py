"""Plain float64 CPU oracle for one decode step of indexer-driven sparse MLA
attention with hybrid GPU/host KV residency ("Hybrid HiSparse").

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library or its Python binding, and imports neither.

The method is described on four web pages (cited by title and section):

* "Un contexte d'un million sur huit H200" (veilletech.fr, 2026-09-08) -- the
  primary description: indexer, top-K, the three residency states and the
  fused resolve step ("Ce qui se passe", "Les trois états de résidence",
  "Ce qu'il faut en retenir").
* "vLLM sert GLM-5.3 en contexte 1M sur 16 H200" (veilletech.fr, 2026-10-24)
  -- the follow-up with the ``sparse_mla_force_mqa`` option ("Comment s'y
  prendre") and the indexer-versus-attention cost remark ("Le mécanisme").
* "A vLLM új módszere 1 millió tokenes GLM 5.3 futtatást tesz lehetővé"
  (aihirek.info) -- a restatement that adds that the indexer cache is handled
  on its own and that hot buffers share the one block pool.

The pages fix the mechanism but not the formulas.  Where they are silent the
oracle takes one stated reading, written in the docstring of the function
that applies it; the tests under ``tests/test_oracle_*.py`` pin each function
to something other than itself:

* ``numerics``  -- OCP FP8 E4M3FN decode table, bf16 decode.
* ``indexer``   -- S[b,p,t] = sum_h w[b,p,h] * ReLU(q[b,p,h,:] . k[b,t,:]) + bias.
* ``quant``     -- optional E4M3 queries for the indexer: per-head absmax scale
  to 448, binary32 rounding to the nearest code, scale folded into w.
* ``topk``      -- K largest scores, ties to the lower token, ascending output.
* ``cache_ops`` -- KV append, pre-copy of completed pages to the host pool,
  demotion of resident pages (the steps on either side of a decode step).
* ``resolve``   -- the residency state machine (resident / hot hit with LRU
  refresh / single-row fault from host).
* ``attention`` -- absorbed-MQA softmax attention over the selected latent rows,
  plus the dense reference over every visible token.
* ``step``      -- the four stages composed.
"""

from . import numerics, indexer, topk, resolve, attention, step  # noqa: F401
