"""Device-side plumbing for one decode step: torch tensors for every input,
state and output buffer of the C ABI, the pinned host pool, and the four calls
of a step on one stream.  No arithmetic of the method happens here.

Layouts (HBM unless noted; B requests, P positions, L layers, T = T_stride):
  indexer   q_idx [B,P,H,D] bf16 | w [B,P,H] f32 | idx_pool [N,64,D] e4m3
            idx_scale [N] f32 | idx_bt [B,T/64] i32 | bias [B,T] f32
  latent    pool [L, N_rows, 576] e4m3 | row_scale [L, N_rows] f32
  residency bt [B,T/64] | hot_blocks [B,C/64] | tok2slot [B,T] | slot2tok [B,C]
            stamp [B,C] | step [1] | err [1]            (all i32)
  host      host_rows [L, B*T, 576] e4m3 (pinned host memory, read by the GPU
            in place) | host_scale [L, B*T] f32 (HBM) | host_bt [B,T/64] i64
  step      scores [B,P,T] f32 | topk [B,P,K] | row_ids [B,P,K] | faults [B,P*K,2]
            counts [B,4] (i32) | q [L,B,P,16,576] bf16 | out [L,B,P,16,512] f32
            lse [L,B,P,16] f32
"""

from __future__ import annotations

import numpy as np

from . import _lib


def _torch():
    import torch
    return torch


def _dev(a, device, dtype_tag=None):
    torch = _torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class DeviceStep:
    """All device buffers of a workload, ready to run decode steps.

    ``wl`` is any object with the workload attributes used below (sizes, dtype
    tags, the indexer cache, residency tables, host pool and per-step queries as
    numpy arrays) and a ``physical_pool()`` method giving the initial pool
    contents; this module imports no workload generator."""

    def __init__(self, wl, device: str = "cuda:0", host_pool: bool = True,
                 indexer_q: str | None = None, host_layout: str = "interleaved"):
        """indexer_q: the indexer's query type, "bf16" (the workload's own
        queries) or "e4m3" (quantized per head every step by
        hs_quantize_queries before the indexer).
        host_layout: "interleaved" keeps the L rows of a host token together
        ([tokens, L, 576], host_row_pitch = L: one contiguous read per fault),
        "layer_major" keeps one plane per layer ([L, tokens, 576]); the same
        for one layer."""
        torch = _torch()
        _lib.load()
        self.wl = wl
        self.device = torch.device(device)
        d = self.device
        B, P, K, L, Ts = wl.B, wl.P, wl.K, wl.L, wl.T_stride
        self.ctx_len = _dev(wl.ctx_len.astype(np.int32), d)
        self.batch = _lib.make_batch(B, P, Ts, self.ctx_len)
        # indexer cache
        self.w = _dev(wl.w, d)
        self.idx_pool = _dev(wl.idx_pool, d)
        self.idx_scale = None if wl.idx_scale is None else _dev(wl.idx_scale, d)
        self.idx_bt = _dev(wl.idx_bt.astype(np.int32), d)
        self.bias = None if wl.bias is None else _dev(wl.bias, d)
        qdt = torch.float32 if wl.q_dtype == "f32" else torch.int16
        self.q_idx = torch.empty((B, P, wl.H_idx, wl.D_idx), dtype=qdt, device=d)
        self.q = torch.empty((L, B, P, wl.Hq, 576), dtype=qdt, device=d)
        self.indexer_q = indexer_q or wl.q_dtype
        self.q8 = self.w_scaled = None
        if self.indexer_q == "e4m3":
            if wl.q_dtype != "bf16" or wl.k_dtype != "e4m3":
                raise ValueError("E4M3 indexer queries need bf16 queries and E4M3 keys")
            self.q8 = torch.empty((B, P, wl.H_idx, wl.D_idx), dtype=torch.uint8, device=d)
            self.w_scaled = torch.empty((B, P, wl.H_idx), dtype=torch.float32, device=d)
        elif self.indexer_q != wl.q_dtype:
            raise ValueError(f"indexer_q={indexer_q!r} not available for this workload")
        # step buffers
        self.scores = torch.empty((B, P, Ts), dtype=torch.float32, device=d)
        self.topk = torch.empty((B, P, K), dtype=torch.int32, device=d)
        self.row_ids = torch.empty((B, P, K), dtype=torch.int32, device=d)
        self.faults = torch.zeros((B, P * K, 2), dtype=torch.int32, device=d)
        self.counts = torch.zeros((B, 4), dtype=torch.int32, device=d)
        self.out = torch.empty((L, B, P, wl.Hq, 512), dtype=torch.float32, device=d)
        self.lse = torch.empty((L, B, P, wl.Hq), dtype=torch.float32, device=d)
        # zero-filled once: the fused indexer adds its histograms into it, and
        # every selection returns what it wrote to zero
        self.ws_topk = torch.zeros(max(_lib.workspace_bytes(_lib.HS_OP_TOPK, B, P, Ts, K), 16),
                                   dtype=torch.uint8, device=d)
        mla_ws = _lib.workspace_bytes(_lib.HS_OP_MLA, B, P, Ts, K, wl.Hq)
        if L > 1:
            mla_ws = max(mla_ws, _lib.mla_layers_workspace_bytes(B, P, K, wl.Hq, L))
        self.ws_mla = torch.empty(max(mla_ws, 16), dtype=torch.uint8, device=d) if mla_ws else None
        # latent pool and residency tables: the workload supplies the pool's
        # initial contents (resident pages and occupied hot slots)
        pool, rsc = wl.physical_pool()
        self.pool = _dev(pool, d)
        self.row_scale = None if rsc is None else _dev(rsc, d)
        del pool
        self.n_rows = self.pool.shape[1]
        self.bt = _dev(wl.bt.astype(np.int32), d)
        C = wl.C
        self.hot_blocks = _dev(wl.hot_blocks.astype(np.int32), d) if C else None
        self.tok2slot = _dev(wl.tok2slot, d) if C else None
        self.slot2tok = _dev(wl.slot2tok, d) if C else None
        self.stamp = _dev(wl.stamp, d) if C else None
        # one step counter per request chunk of the pipelined step (all equal);
        # the single-stream step uses the first one
        self.max_chunks = 16
        self.steps_dev = torch.full((self.max_chunks,), wl.step, dtype=torch.int32, device=d)
        self.step_t = self.steps_dev[:1]
        self.err = torch.zeros(1, dtype=torch.int32, device=d)
        self.host_rows = self.host_scale = self.host_bt = None
        host_rows_dev = host_scale_dev = None
        if host_layout not in ("interleaved", "layer_major"):
            raise ValueError(f"host_layout={host_layout!r}")
        self.host_layout = host_layout
        inter = host_layout == "interleaved"
        # host row of (layer l, host token h) = l * host_layer_rows + h * host_row_pitch
        self.host_layer_rows, self.host_row_pitch = (1, L) if inter else (B * Ts, 1)
        if wl.has_host and host_pool:
            hr = wl.host_rows                                     # [L, B*Ts, 576]
            shape = (hr.shape[1], L, hr.shape[2]) if inter else hr.shape
            self.host_rows = torch.empty(shape, dtype=torch.uint8 if hr.dtype == np.uint8
                                         else torch.float32, pin_memory=True)
            self.host_rows.numpy()[...] = hr.transpose(1, 0, 2) if inter else hr
            host_rows_dev = _lib.host_device_ptr(self.host_rows)
            if wl.host_scale is not None:
                # the per-row scales of the host pool are a small table: kept in
                # HBM so a fault reads only its row over the host link
                hs_ = wl.host_scale                               # [L, B*Ts]
                self.host_scale = _dev(np.ascontiguousarray(hs_.T) if inter else hs_, d)
                host_scale_dev = self.host_scale.data_ptr()
            self.host_bt = _dev(wl.host_bt, d)
        kv_t = _lib.DTYPES[wl.kv_dtype]
        self.res = _lib.Residency(
            C, L, kv_t, self.host_row_pitch, self.n_rows, self.host_layer_rows,
            self.bt.data_ptr(), _p(self.hot_blocks), _p(self.tok2slot), _p(self.slot2tok),
            _p(self.stamp), self.step_t.data_ptr(), self.err.data_ptr(), self.pool.data_ptr(),
            _p(self.row_scale), host_rows_dev, host_scale_dev, _p(self.host_bt))
        self._host_rows_dev, self._host_scale_dev = host_rows_dev, host_scale_dev
        # decode loop with KV append: the two free lists (stacks) and the caches'
        # descriptors the append call writes through
        self.free = self.idx_free = None
        if getattr(wl, "appends", False):
            def stack(ids):
                t = torch.zeros(len(ids), dtype=torch.int32, device=d)
                t.copy_(torch.from_numpy(np.asarray(ids, np.int32)))
                n = torch.tensor([len(ids)], dtype=torch.int32, device=d)
                return t, n
            self.free, self.free_n = stack(wl.free_blocks)
            self.idx_free, self.idx_free_n = stack(wl.idx_free_blocks)
            self.idx_cache = _lib.IndexCache(_lib.DTYPES[wl.k_dtype], wl.D_idx,
                                             self.idx_pool.data_ptr(), _p(self.idx_scale),
                                             self.idx_bt.data_ptr())
            self.ws_cache = torch.empty(_lib.workspace_bytes(_lib.HS_OP_CACHE, B, P, Ts, 1),
                                        dtype=torch.uint8, device=d)
        self._chunks = {}
        self._streams = None
        self.set_queries(1)

    # ---------------------------------------------------------------- inputs
    def set_queries(self, s: int = 1):
        q_idx, q = self.wl.step_inputs(s)
        self.q_idx.copy_(_dev(q_idx, self.device))
        self.q.copy_(_dev(q, self.device))

    # ---------------------------------------------------------------- stages
    def run_quantize(self, stream=None):
        wl = self.wl
        _lib.quantize_queries(self.batch, wl.H_idx, wl.D_idx, self.q_idx, self.w, self.q8,
                              self.w_scaled, stream)

    def _indexer_inputs(self, stream, quantize=True):
        """(query type, queries, head weights) the indexer reads; quantizes first
        when the indexer runs on E4M3 queries (unless `quantize` is False: the
        codes of the last quantization are reused)."""
        if self.indexer_q == "e4m3":
            if quantize:
                self.run_quantize(stream)
            return "e4m3", self.q8, self.w_scaled
        return self.wl.q_dtype, self.q_idx, self.w

    def run_indexer(self, stream=None, quantize=True):
        wl = self.wl
        qt, qi, w = self._indexer_inputs(stream, quantize)
        _lib.indexer_scores(self.batch, wl.H_idx, wl.D_idx, qt, qi, w,
                            wl.k_dtype, self.idx_pool, self.idx_scale, self.idx_bt, self.bias,
                            self.scores, stream)

    def run_topk(self, stream=None):
        _lib.topk(self.batch, self.wl.K, self.scores, self.topk, self.ws_topk, stream)

    def run_indexer_topk(self, stream=None):
        """Indexer and top-K in one call (histogram pass fused into the indexer)."""
        wl = self.wl
        qt, qi, w = self._indexer_inputs(stream)
        _lib.indexer_topk(self.batch, wl.H_idx, wl.D_idx, qt, qi, w,
                          wl.k_dtype, self.idx_pool, self.idx_scale, self.idx_bt, self.bias,
                          self.scores, wl.K, self.topk, self.ws_topk, stream)

    def run_indexer_topk_scores(self, stream=None, quantize=True):
        """First half of run_indexer_topk: the indexer with the top-K histogram
        in its epilogue (run_indexer_topk_select must follow)."""
        wl = self.wl
        qt, qi, w = self._indexer_inputs(stream, quantize)
        _lib.indexer_topk_scores(self.batch, wl.H_idx, wl.D_idx, qt, qi, w, wl.k_dtype,
                                 self.idx_pool, self.idx_scale, self.idx_bt, self.bias,
                                 self.scores, wl.K, self.ws_topk, stream)

    def run_indexer_topk_select(self, stream=None):
        """Second half of run_indexer_topk: the selection."""
        _lib.indexer_topk_select(self.batch, self.indexer_q, self.wl.K, self.scores, self.topk,
                                 self.ws_topk, stream)

    def run_indexer_topk_select_resolve(self, stream=None):
        """The selection half of run_indexer_topk followed by the resolve tables, in
        one call (one kernel for the finalize and the tables with one position)."""
        _lib.indexer_topk_select_resolve(self.batch, self.indexer_q, self.wl.K, self.scores,
                                         self.topk, self.ws_topk, self.res, self.row_ids,
                                         self.faults, self.counts, stream)

    def run_resolve(self, stream=None):
        _lib.resolve_rows(self.batch, self.wl.K, self.topk, self.res, self.row_ids, self.faults,
                          self.counts, stream)

    def run_resolve_tables(self, stream=None):
        _lib.resolve_tables(self.batch, self.wl.K, self.topk, self.res, self.row_ids, self.faults,
                            self.counts, stream)

    def run_copy_faults(self, workgroups: int = 0, stream=None):
        _lib.copy_faults(self.batch, self.wl.K, self.res, self.faults, self.counts, workgroups,
                         stream=stream)

    def run_attention(self, layer: int, stream=None):
        wl = self.wl
        _lib.sparse_mla_decode(self.batch, wl.K, wl.Hq, wl.q_dtype, self.q[layer], wl.kv_dtype,
                               self.pool[layer],
                               None if self.row_scale is None else self.row_scale[layer],
                               self.row_ids, wl.sm_scale, self.out[layer], self.lse[layer],
                               self.ws_mla, stream)

    def run_attention_layers(self, stream=None):
        """Attention of all L layers over the shared row ids in one call."""
        wl = self.wl
        _lib.sparse_mla_decode_layers(self.batch, wl.K, wl.Hq, wl.L, wl.q_dtype, self.q,
                                      wl.kv_dtype, self.pool, self.n_rows, self.row_scale,
                                      self.row_ids, wl.sm_scale, self.out, self.lse, self.ws_mla,
                                      stream)

    def run(self, stream=None, fused_resolve: bool = True):
        """One whole decode step: indexer + top-K, resolve (+ fault copies), attention of
        the L layers (one call for several layers).  fused_resolve: the top-K's
        selection half and the resolve tables in one call (hs_indexer_topk_select_resolve),
        else hs_indexer_topk then hs_resolve_rows; the results are the same."""
        if fused_resolve:
            self.run_indexer_topk_scores(stream)
            self.run_indexer_topk_select_resolve(stream)
            self.run_copy_faults(stream=stream)
        else:
            self.run_indexer_topk(stream)
            self.run_resolve(stream)
        if self.wl.L > 1:
            self.run_attention_layers(stream)
        else:
            self.run_attention(0, stream)

    def run_layer_pipelined(self, copy_workgroups: int = 0, groups: int = 0):
        """One decode step with the layers of one shared selection overlapped:
        indexer + top-K and resolve tables on the current stream, then the
        fault copies one group of layers at a time on a copy stream, and each
        group's attention on the current stream as soon as that group's rows
        are in, so that group g's attention runs while group g + 1's rows cross
        the host link.  groups: layer groups (a divisor of L; 0 = one per
        layer).  Same tables, pool rows and step as run()."""
        torch = _torch()
        wl = self.wl
        G = groups or wl.L
        if wl.L % G:
            raise ValueError(f"groups={G} does not divide L={wl.L}")
        lg = wl.L // G
        if self._streams is None:
            self._streams = (torch.cuda.Stream(device=self.device),
                             torch.cuda.Stream(device=self.device))
        need = _lib.mla_layers_workspace_bytes(wl.B, wl.P, wl.K, wl.Hq, lg)
        if self.ws_mla is None or self.ws_mla.numel() < need:
            self.ws_mla = torch.empty(need, dtype=torch.uint8, device=self.device)
        xs = self._streams[1]
        main = torch.cuda.current_stream(self.device)
        self.run_indexer_topk()
        self.run_resolve_tables()
        xs.wait_stream(main)
        done = []
        with torch.cuda.stream(xs):
            for g in range(G):
                _lib.copy_faults_layers(self.batch, wl.K, self.res, self.faults, self.counts,
                                        g * lg, lg, copy_workgroups)
                ev = torch.cuda.Event()
                ev.record(xs)
                done.append(ev)
        for g in range(G):
            main.wait_event(done[g])
            ls = slice(g * lg, (g + 1) * lg)
            _lib.sparse_mla_decode_layers(self.batch, wl.K, wl.Hq, lg, wl.q_dtype, self.q[ls],
                                          wl.kv_dtype, self.pool[ls], self.n_rows,
                                          None if self.row_scale is None else self.row_scale[ls],
                                          self.row_ids, wl.sm_scale, self.out[ls], self.lse[ls],
                                          self.ws_mla)
        main.wait_stream(xs)

    def append(self, s: int, stream=None):
        """KV append after step s of a decode-loop workload: one token per request
        (its latent rows in every layer and its indexer key) through
        hs_append_tokens; the context grows by one on the device."""
        torch = _torch()
        n_new, rows, rsc, keys, ksc = self.wl.append_inputs(s)
        dev = lambda a: None if a is None else torch.from_numpy(a).to(self.device)
        self._app_in = [dev(a) for a in (n_new, rows, rsc, keys, ksc)]   # kept until run
        n_d, rows_d, rsc_d, keys_d, ksc_d = self._app_in
        _lib.append_tokens(self.batch, self.ctx_len, n_d, self.res, rows_d, rsc_d, self.idx_cache,
                           keys_d, ksc_d,
                           _lib.FreeList(self.free.data_ptr(), self.free_n.data_ptr(),
                                         self.free.numel(), 0),
                           _lib.FreeList(self.idx_free.data_ptr(), self.idx_free_n.data_ptr(),
                                         self.idx_free.numel(), 0),
                           self.ws_cache, stream)

    # ---------------------------------------------------------------- pipelined step
    def _chunk(self, c: int, nchunks: int):
        """Views, batch and residency structs of request chunk c of nchunks."""
        key = (c, nchunks)
        if key in self._chunks:
            return self._chunks[key]
        wl = self.wl
        bounds = np.linspace(0, wl.B, nchunks + 1).round().astype(int)
        b0, b1 = int(bounds[c]), int(bounds[c + 1])
        e = self.ctx_len.element_size()
        batch = _lib.Batch(b1 - b0, wl.P, wl.T_stride, wl.T_stride // 64,
                           self.ctx_len.data_ptr() + e * b0)
        sl = slice(b0, b1)
        ch = {"b0": b0, "b1": b1, "batch": batch, "sl": sl}
        C = wl.C

        def off(t, rows):
            return None if t is None else t[rows].data_ptr()
        ch["res"] = _lib.Residency(
            C, wl.L, _lib.DTYPES[wl.kv_dtype], self.host_row_pitch, self.n_rows,
            self.host_layer_rows,
            off(self.bt, sl), off(self.hot_blocks, sl), off(self.tok2slot, sl),
            off(self.slot2tok, sl), off(self.stamp, sl), self.steps_dev[c:c + 1].data_ptr(),
            self.err.data_ptr(), self.pool.data_ptr(), _p(self.row_scale), self._host_rows_dev,
            self._host_scale_dev, off(self.host_bt, sl))
        self._chunks[key] = ch
        return ch

    def _ensure_pipeline(self, nchunks: int):
        torch = _torch()
        if self._streams is None:
            self._streams = (torch.cuda.Stream(device=self.device), torch.cuda.Stream(device=self.device))
        wl = self.wl
        need = 16
        for c in range(nchunks):
            ch = self._chunk(c, nchunks)
            need = max(need, _lib.workspace_bytes(_lib.HS_OP_MLA, ch["b1"] - ch["b0"], wl.P,
                                                  wl.T_stride, wl.K, wl.Hq))
        if self.ws_mla is None or self.ws_mla.numel() < need:
            self.ws_mla = torch.empty(need, dtype=torch.uint8, device=self.device)

    def run_pipelined(self, nchunks: int = 4, copy_workgroups: int = 32):
        """One decode step with the batch split into request chunks on two streams:
        a compute stream runs indexer -> top-K -> resolve tables chunk after chunk,
        and a copy stream runs each chunk's host-link fault copies and attention
        as soon as its tables are resolved, so the copies overlap the following
        chunks' HBM-bound work.  The copies use `copy_workgroups` workgroups so
        that most compute units stay with the HBM-bound kernels.  Same results
        as run() (per-chunk step counters all advance together)."""
        torch = _torch()
        if nchunks > self.max_chunks or nchunks > self.wl.B:
            raise ValueError(f"nchunks={nchunks} out of range")
        self._ensure_pipeline(nchunks)
        wl = self.wl
        cs, xs = self._streams
        main = torch.cuda.current_stream(self.device)
        cs.wait_stream(main)
        xs.wait_stream(main)
        if nchunks > 1:
            with torch.cuda.stream(cs):   # every chunk starts from the same step number
                self.steps_dev[1:nchunks].copy_(self.steps_dev[0].expand(nchunks - 1))
        with torch.cuda.stream(cs):
            qt, qi, qw = self._indexer_inputs(None)
        for c in range(nchunks):
            ch = self._chunk(c, nchunks)
            sl, batch, res = ch["sl"], ch["batch"], ch["res"]
            with torch.cuda.stream(cs):
                _lib.indexer_topk(batch, wl.H_idx, wl.D_idx, qt, qi[sl],
                                  qw[sl], wl.k_dtype, self.idx_pool, self.idx_scale,
                                  self.idx_bt[sl], None if self.bias is None else self.bias[sl],
                                  self.scores[sl], wl.K, self.topk[sl], self.ws_topk)
                _lib.resolve_tables(batch, wl.K, self.topk[sl], res, self.row_ids[sl],
                                    self.faults[sl], self.counts[sl])
                ev = torch.cuda.Event()
                ev.record(cs)
            xs.wait_event(ev)
            with torch.cuda.stream(xs):
                _lib.copy_faults(batch, wl.K, res, self.faults[sl], self.counts[sl],
                                 copy_workgroups)
                for l in range(wl.L):
                    _lib.sparse_mla_decode(batch, wl.K, wl.Hq, wl.q_dtype, self.q[l][sl],
                                           wl.kv_dtype, self.pool[l],
                                           None if self.row_scale is None else self.row_scale[l],
                                           self.row_ids[sl], wl.sm_scale, self.out[l][sl],
                                           self.lse[l][sl], self.ws_mla)
        main.wait_stream(cs)
        main.wait_stream(xs)

    # ---------------------------------------------------------------- state
    def snapshot(self) -> dict:
        """Copies of the mutable state (tables, step, pool rows and scales)."""
        snap = {"step": self.steps_dev.clone(), "err": self.err.clone(), "pool": self.pool.clone()}
        if self.row_scale is not None:
            snap["row_scale"] = self.row_scale.clone()
        if self.wl.C:
            snap.update(tok2slot=self.tok2slot.clone(), slot2tok=self.slot2tok.clone(),
                        stamp=self.stamp.clone())
        if self.free is not None:
            # what the appends change (the rows they write are rewritten identically)
            snap.update(ctx_len=self.ctx_len.clone(), bt=self.bt.clone(),
                        idx_bt=self.idx_bt.clone(), idx_scale=self.idx_scale.clone(),
                        free_n=self.free_n.clone(), idx_free_n=self.idx_free_n.clone())
        return snap

    def restore(self, snap: dict):
        self.steps_dev.copy_(snap["step"])
        self.err.copy_(snap["err"])
        self.pool.copy_(snap["pool"])
        if "row_scale" in snap:
            self.row_scale.copy_(snap["row_scale"])
        if self.wl.C:
            self.tok2slot.copy_(snap["tok2slot"])
            self.slot2tok.copy_(snap["slot2tok"])
            self.stamp.copy_(snap["stamp"])
        if "ctx_len" in snap:
            for k in ("ctx_len", "bt", "idx_bt", "idx_scale", "free_n", "idx_free_n"):
                getattr(self, k).copy_(snap[k])

    def state_numpy(self) -> dict:
        """Host copies of the residency tables (for checks)."""
        r = {"step": int(self.step_t.item()), "err": int(self.err.item())}
        if self.wl.C:
            r.update(tok2slot=self.tok2slot.cpu().numpy(), slot2tok=self.slot2tok.cpu().numpy(),
                     stamp=self.stamp.cpu().numpy())
        return r


def _p(t):
    return None if t is None else t.data_ptr()
