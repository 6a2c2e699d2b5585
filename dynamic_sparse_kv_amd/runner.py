"""Host driver of the decode loop: buffers, schedule, per-step launches.

This is the orchestration layer above the C ABI (the schedule of the
Slow-Fast Inference pages, technical summary section 3.A: fast steps by
default, a slow step at a semantic boundary or once the reuse budget is
spent).  It owns device buffers (torch tensors used as plain memory), stages
every per-step argument on the device up front, and issues libsfi calls on a
stream, so a whole run can also be captured into one HIP graph.  It computes
nothing itself.
"""
from __future__ import annotations

import numpy as np
import torch

from . import sfi


class LenHints(tuple):
    """Host row-count hints of one step's lists (int32 arrays in list
    order): [0] the slow list, [1] the fast list, and .fast_old / .fast_new
    the two halves of the fast list that the pipelined schedule issues."""

    def __new__(cls, slow, fast, fast_old, fast_new):
        t = super().__new__(cls, (slow, fast))
        t.fast_old, t.fast_new = fast_old, fast_new
        return t


def _dev_i32(x, device):
    return torch.as_tensor(np.ascontiguousarray(x, dtype=np.int32), device=device)


class DecodePlan:
    """Per-step device arguments of one run.

    slow[s, b] (host bool) says whether sequence b takes a slow step at step
    s.  seq_len[s, b] = ctx_b + s + 1 keys are visible at step s.  With
    k_div > 0 a slow step of sequence b keeps min(k_cap, seq_len // k_div)
    keys (k_seq[s, b]); otherwise every list holds up to the decoder's k.
    """

    def __init__(self, slow: np.ndarray, ctx: np.ndarray, device, k_cap: int = 0, k_div: int = 0):
        steps, B = slow.shape
        self.steps, self.B = steps, B
        self.slow = slow.astype(bool)
        lens = ctx[None, :].astype(np.int64) + np.arange(steps)[:, None] + 1
        self.seq_len_host = lens.astype(np.int32)
        self.seq_len = _dev_i32(lens, device)               # [steps][B]
        self.k_seq = None
        self.k_div = k_div
        self.k_seq_host = None
        if k_div > 0:
            self.k_seq_host = np.minimum(k_cap, lens // k_div).astype(np.int32)
            self.k_seq = _dev_i32(self.k_seq_host, device)
        self._hints = {}
        slow_ids = np.zeros((steps, B), dtype=np.int32)
        fast_ids = np.zeros((steps, B), dtype=np.int32)
        self.n_slow = np.zeros(steps, dtype=np.int64)
        self.n_fast = np.zeros(steps, dtype=np.int64)
        for s in range(steps):
            si = np.nonzero(self.slow[s])[0]
            fi = np.nonzero(~self.slow[s])[0]
            slow_ids[s, : len(si)] = si
            fast_ids[s, : len(fi)] = fi
            self.n_slow[s] = len(si)
            self.n_fast[s] = len(fi)
        self.slow_ids = _dev_i32(slow_ids, device)
        self.fast_ids = _dev_i32(fast_ids, device)
        # fast sequences split by whether they were refreshed on the step before
        old_ids = np.zeros((steps, B), dtype=np.int32)
        new_ids = np.zeros((steps, B), dtype=np.int32)
        self.n_fast_old = np.zeros(steps, dtype=np.int64)
        self.n_fast_new = np.zeros(steps, dtype=np.int64)
        for s in range(steps):
            fresh = self.slow[s - 1] if s > 0 else np.zeros(B, dtype=bool)
            oi = np.nonzero(~self.slow[s] & ~fresh)[0]
            ni = np.nonzero(~self.slow[s] & fresh)[0]
            old_ids[s, : len(oi)] = oi
            new_ids[s, : len(ni)] = ni
            self.n_fast_old[s] = len(oi)
            self.n_fast_new[s] = len(ni)
        self.fast_old_ids = _dev_i32(old_ids, device)
        self.fast_new_ids = _dev_i32(new_ids, device)
        self.fast_old_ids_host, self.fast_new_ids_host = old_ids, new_ids

    def slow_list(self, s: int):
        """Step s's slow-sequence list, or None when it is every sequence in
        order (a NULL list: the kernels then need no id load before their
        first dependent loads)."""
        return None if self.n_slow[s] == self.B else self.slow_ids[s]

    def fast_list(self, s: int):
        """Step s's fast-sequence list, or None when it is every sequence."""
        return None if self.n_fast[s] == self.B else self.fast_ids[s]

    def len_hints(self, s: int, n_sink: int, window: int, k: int):
        """Host row-count hints of step s's lists (sfi.with_len_hints): the
        slow sequences' lengths, and for each fast sequence its sinks and
        window within its length plus its selection's size bound (k, or
        min(k, seq_len // k_div) when the plan caps lists by length: a list
        chosen at an earlier, shorter step is no longer).  Cached, so the
        arrays outlive the calls that read them."""
        key = (s, n_sink, window, k)
        h = self._hints.get(key)
        if h is None:
            lens = self.seq_len_host[s].astype(np.int64)
            kk = np.full(self.B, k, dtype=np.int64)
            if self.k_seq_host is not None:
                kk = np.minimum(kk, self.k_seq_host[s])
            fb = np.minimum(lens, n_sink + window) + np.minimum(kk, np.maximum(lens - n_sink - window, 0))
            slow = self.slow[s]
            old = self.fast_old_ids_host[s, : self.n_fast_old[s]]
            new = self.fast_new_ids_host[s, : self.n_fast_new[s]]
            i32 = lambda a: np.ascontiguousarray(a, dtype=np.int32)
            h = LenHints(i32(lens[slow]), i32(fb[~slow]), i32(fb[old]), i32(fb[new]))
            self._hints[key] = h
        return h


def stats_prior_steps(plan: DecodePlan) -> np.ndarray:
    """Steps of a run whose every row comes through the library's appends
    (from a cache that holds the prefill only) at which the key-norm
    statistics are current for every slow sequence, so the combined
    step-and-select call may form its prior from them: those after each of
    their slow sequences' first slow step.  The order of SFIDecoder.step's
    own bookkeeping, for callers that issue the calls themselves."""
    covered = np.full(plan.B, -1, dtype=np.int64)
    use = np.zeros(plan.steps, dtype=bool)
    for s in range(plan.steps):
        lens = plan.seq_len_host[s].astype(np.int64)
        b = plan.slow[s]
        use[s] = plan.n_slow[s] > 0 and bool(np.all(covered[b] == lens[b] - 1))
        covered = np.where((covered == lens - 1) | b, lens, -1)
    return use


class SFIDecoder:
    """Slow/fast decode of one attention layer over a resident KV cache."""

    def __init__(self, K, V, Hq: int, max_len: int, *, n_sink: int, window: int, k: int,
                 lam: float, norm_coef: float = 0.5, pos_tau: float = 1024.0,
                 page_table=None, page_size: int = 0, keep_fused: bool = False,
                 nms_radius: int = 0, nms_alpha: float = 0.0, excl_beta: float = 0.0,
                 norm_stats: bool = True):
        dev = K.device
        self.dev = dev
        self.K, self.V = K, V
        self.Hq = Hq
        self.page_table = page_table
        if page_table is None:
            B, Hkv, cap, d = K.shape
        else:
            Hkv, d = K.shape[1], K.shape[3]
            B = page_table.shape[0]
        self.B, self.Hkv, self.d = B, Hkv, d
        self.max_len = int(max_len)
        self.n_sink, self.window, self.k = n_sink, window, k
        self._dummy_len = torch.full((B,), self.max_len, dtype=torch.int32, device=dev)
        self.kv = sfi.make_kv(K, V, self._dummy_len, Hq, self.max_len, page_table, page_size)
        # Key-norm statistics of the cache rows, kept current by every call
        # that appends rows; _stats_len[b] is the row count they cover for
        # sequence b as far as the host can tell (-1: unknown), so a planned
        # step knows when a combined step-and-select call may form the prior
        # from them.
        self.nstat = None
        self._stats_len = np.full(B, -1, dtype=np.int64)
        if norm_stats:
            self.nstat = torch.zeros((B, Hkv, 2), dtype=torch.float64, device=dev)
            self.kv.norm_stats = self.nstat.data_ptr()
        self.params = sfi.select_params(sfi.SFI_SCORE_FUSED, lam, k, n_sink, window, norm_coef, pos_tau,
                                        nms_radius=nms_radius, nms_alpha=nms_alpha,
                                        excl_beta=excl_beta)
        self.ld = self.max_len
        f32 = dict(dtype=torch.float32, device=dev)
        self.out = torch.zeros((B, Hq, d), **f32)
        self.evidence = torch.zeros((B, Hkv, self.ld), **f32)
        self.key_norm = torch.zeros((B, Hkv, self.ld), **f32)
        self.fused = torch.zeros((B, Hkv, self.ld), **f32) if keep_fused else None
        self.sel_idx = torch.full((B, Hkv, k), -1, dtype=torch.int32, device=dev)
        self.sel_count = torch.zeros((B, Hkv), dtype=torch.int32, device=dev)
        self.ck = self.cv = None  # compact copies of the selected rows (allocated by compact())
        # second evidence / key-norm copy for the pipelined schedule (allocated
        # here, never inside a graph capture)
        self.evidence_alt = torch.zeros((B, Hkv, self.ld), **f32)
        self.key_norm_alt = torch.zeros((B, Hkv, self.ld), **f32)
        # Events of the multi-stream schedules.  They stay referenced for the
        # decoder's lifetime: an event destroyed while a graph capture that
        # recorded or waited on it is still open leaves the capture holding a
        # dangling handle.
        self._events = []
        u8 = dict(dtype=torch.uint8, device=dev)
        self.ws_slow_bytes = sfi.sfi_slow_workspace_bytes(self.kv)
        self.ws_sel_bytes = sfi.sfi_select_workspace_bytes(B, Hkv, self.max_len)
        self.ws_fast_bytes = sfi.sfi_fast_workspace_bytes(self.kv, k, n_sink, window)
        self.ws_step_bytes = sfi.sfi_decode_step_workspace_bytes(self.kv, k, n_sink, window)
        self.ws_slow = torch.zeros(self.ws_slow_bytes, **u8)
        self.ws_sel = torch.zeros(self.ws_sel_bytes, **u8)
        self.ws_fast = torch.zeros(self.ws_fast_bytes, **u8)
        self.ws_step = torch.zeros(self.ws_step_bytes, **u8)
        self.ws_stepsel_bytes = sfi.sfi_decode_step_select_workspace_bytes(self.kv, k, n_sink, window)
        self.ws_stepsel = torch.zeros(self.ws_stepsel_bytes, **u8)

    # -- single calls -------------------------------------------------------
    # new_rows = (k_new, v_new), each [B][Hkv][d] bf16 (or [B][1][Hkv][d]):
    # the call also appends each listed sequence's row at cache row
    # seq_len - 1 (the fused append of the sfi_kv description).
    def _kvx(self, new_rows, stats_valid: bool = False, len_hints=None):
        kv = self.kv if new_rows is None else sfi.with_new_rows(self.kv, new_rows[0], new_rows[1])
        if stats_valid:
            if self.nstat is None:
                raise ValueError("this decoder keeps no key-norm statistics")
            kv = sfi.with_norm_stats(kv, self.nstat, True)
        if len_hints is not None:
            kv = sfi.with_len_hints(kv, len_hints[0], len_hints[1])
        return kv

    def hints(self, plan: "DecodePlan", s: int):
        """Row-count hints of step s's lists for this decoder's fast state."""
        return plan.len_hints(s, self.n_sink, self.window, self.k)

    def slow(self, q, seq_len, batch_ids, batch_n: int, stream=None, select: bool = True, out=None,
             k_seq=None, new_rows=None, len_hints=None):
        """Dense step + evidence for the listed sequences, then the selector.
        len_hints = (slow lengths, unused) as DecodePlan.len_hints gives."""
        self.kv.seq_len = seq_len.data_ptr() if torch.is_tensor(seq_len) else seq_len
        sl = None if len_hints is None else (len_hints[0], None)
        sfi.sfi_slow_step(self._kvx(new_rows, len_hints=sl), batch_ids, batch_n, q, self.out if out is None else out,
                          self.evidence, self.key_norm, self.ld, self.ws_slow, self.ws_slow_bytes,
                          stream)
        if select:
            self.slow_select_only(self.kv.seq_len, batch_ids, batch_n, stream, k_seq=k_seq)

    def slow_select_only(self, seq_len, batch_ids, batch_n: int, stream=None, k_seq=None):
        """The selector over the evidence and norms of the last slow step;
        k_seq (device int32 [B]) optionally caps each sequence's list."""
        ptr = seq_len.data_ptr() if torch.is_tensor(seq_len) else seq_len
        self.params.k_per_seq = None if k_seq is None else k_seq.data_ptr()
        try:
            sfi.sfi_select(self.params, batch_ids, batch_n, ptr, self.B, self.Hkv, self.max_len,
                           self.evidence, self.key_norm, self.ld, self.sel_idx, self.sel_count,
                           self.fused, self.ws_sel, self.ws_sel_bytes, stream)
        finally:
            self.params.k_per_seq = None

    def append(self, k_new, v_new, seq_len, batch_ids, batch_n: int, stream=None):
        """Write the step's new K/V rows (k_new, v_new [B][T][Hkv][d]) at cache
        rows seq_len - T .. seq_len - 1 of the listed sequences."""
        self.kv.seq_len = seq_len.data_ptr() if torch.is_tensor(seq_len) else seq_len
        sfi.sfi_append_kv(self.kv, batch_ids, batch_n, k_new, v_new, int(k_new.shape[1]), stream)

    def dense(self, q, seq_len, batch_ids, batch_n: int, stream=None, new_rows=None, len_hints=None):
        """Plain dense attention (no evidence): the full-KV comparator;
        len_hints = the listed sequences' lengths (host int32), or None."""
        self.kv.seq_len = seq_len.data_ptr() if torch.is_tensor(seq_len) else seq_len
        sl = None if len_hints is None else (len_hints, None)
        sfi.sfi_slow_step(self._kvx(new_rows, len_hints=sl), batch_ids, batch_n, q, self.out, None, None, self.ld,
                          self.ws_slow, self.ws_slow_bytes, stream)

    def fast(self, q, seq_len, batch_ids, batch_n: int, stream=None, out=None, new_rows=None,
             len_hints=None):
        self.kv.seq_len = seq_len.data_ptr() if torch.is_tensor(seq_len) else seq_len
        fl = None if len_hints is None else (None, len_hints[1])
        sfi.sfi_fast_step(self._kvx(new_rows, len_hints=fl), batch_ids, batch_n, q, self.sel_idx, self.sel_count, self.Hkv,
                          self.k, self.n_sink, self.window, self.out if out is None else out,
                          self.ws_fast, self.ws_fast_bytes, stream)

    def compact(self, seq_len, batch_ids, batch_n: int, stream=None):
        """Copy the selected K/V rows of the listed sequences into the
        compact buffers (allocated on first use, outside any capture)."""
        if self.ck is None:
            self.ck = torch.zeros((self.B, self.Hkv, self.k, self.d), dtype=torch.bfloat16, device=self.dev)
            self.cv = torch.zeros_like(self.ck)
        self.kv.seq_len = seq_len.data_ptr() if torch.is_tensor(seq_len) else seq_len
        sfi.sfi_compact_selected(self.kv, batch_ids, batch_n, self.sel_idx, self.sel_count, self.Hkv,
                                 self.k, self.ck, self.cv, stream)

    def fast_compact(self, q, seq_len, batch_ids, batch_n: int, stream=None, out=None, new_rows=None):
        """Fast step reading the selected rows from the compact buffers."""
        self.kv.seq_len = seq_len.data_ptr() if torch.is_tensor(seq_len) else seq_len
        sfi.sfi_fast_step_compact(self._kvx(new_rows), batch_ids, batch_n, q, self.sel_idx, self.sel_count, self.Hkv,
                                  self.k, self.n_sink, self.window, self.ck, self.cv,
                                  self.out if out is None else out, self.ws_fast, self.ws_fast_bytes, stream)

    def co_step(self, q, seq_len, slow_ids, n_slow: int, fast_ids, n_fast: int, stream=None,
                out=None, select: bool = True, k_seq=None, new_rows=None, len_hints=None):
        """Slow steps of slow_ids and fast steps of fast_ids in one co-launched
        pass, then the selector of the slow sequences."""
        self.kv.seq_len = seq_len.data_ptr() if torch.is_tensor(seq_len) else seq_len
        sfi.sfi_decode_step(self._kvx(new_rows, len_hints=len_hints), slow_ids, n_slow, fast_ids, n_fast, q,
                            self.out if out is None else out, self.evidence, self.key_norm, self.ld,
                            self.sel_idx, self.sel_count, self.Hkv, self.k, self.n_sink, self.window,
                            self.ws_step, self.ws_step_bytes, stream)
        if select and n_slow:
            self.slow_select_only(self.kv.seq_len, slow_ids, n_slow, stream, k_seq=k_seq)

    def step_select(self, q, seq_len, slow_ids, n_slow: int, fast_ids, n_fast: int, stream=None,
                    out=None, k_seq=None, new_rows=None, use_stats: bool = False, len_hints=None):
        """One call for the step and the slow sequences' new selections
        (sfi_decode_step_select): the slow step forms the selector's prior
        statistics, so the selection runs only its key and pick passes.
        use_stats vouches that the key-norm statistics are current for the
        slow sequences (rows before this call's own): the prior then comes
        from them and the key pass runs inside the step's finalize."""
        self.kv.seq_len = seq_len.data_ptr() if torch.is_tensor(seq_len) else seq_len
        self.params.k_per_seq = None if k_seq is None else k_seq.data_ptr()
        try:
            sfi.sfi_decode_step_select(self._kvx(new_rows, use_stats, len_hints), self.params, slow_ids, n_slow, fast_ids, n_fast, q,
                                       self.out if out is None else out, self.evidence, self.key_norm,
                                       self.ld, self.sel_idx, self.sel_count, self.fused, self.ws_stepsel,
                                       self.ws_stepsel_bytes, stream)
        finally:
            self.params.k_per_seq = None

    def layer_step(self, plan: "DecodePlan", s: int, q_steps, pending=None, stream=None, out=None,
                   new_kv=None, hints: bool = True):
        """Decode step s of this layer in a stack (sfi_decode_layer_step): the
        previous layer's deferred selection (pending, an sfi_deferred or None)
        runs inside this call's grids and this layer's own selection is
        deferred.  Returns it (active when step s has slow sequences); pass it
        to the next layer's call, or to sfi_run_deferred after the last.
        new_kv as in step(): the call appends the rows itself."""
        self._note_stats(plan, s, new_kv is not None, ns_refresh=int(plan.n_slow[s]) > 0)
        ks = None if plan.k_seq is None else plan.k_seq[s]
        ns, nf = int(plan.n_slow[s]), int(plan.n_fast[s])
        self.kv.seq_len = plan.seq_len[s].data_ptr()
        kvx = self._kvx(None if new_kv is None else (new_kv[0][s], new_kv[1][s]),
                        len_hints=self.hints(plan, s) if hints else None)
        self.params.k_per_seq = None if ks is None else ks.data_ptr()
        own = sfi.sfi_deferred()
        try:
            sfi.sfi_decode_layer_step(kvx, self.params, plan.slow_list(s), ns, plan.fast_list(s), nf,
                                      q_steps[s], self.out if out is None else out, self.evidence,
                                      self.key_norm, self.ld, self.sel_idx, self.sel_count, self.fused,
                                      self.ws_stepsel, self.ws_stepsel_bytes, pending, own, stream)
        finally:
            self.params.k_per_seq = None
        return own

    def _stats_current(self, plan: DecodePlan, s: int) -> bool:
        """Whether the statistics cover exactly the rows before step s for
        every slow sequence of step s."""
        if self.nstat is None or plan.n_slow[s] == 0:
            return False
        b = plan.slow[s]
        return bool(np.all(self._stats_len[b] == plan.seq_len_host[s][b].astype(np.int64) - 1))

    def _note_stats(self, plan: DecodePlan, s: int, appended: bool, ns_refresh: bool):
        """Host record of the statistics after step s: sequences whose rows
        the step appended through the library keep (or, for the slow
        sequences of a prior-forming call, get) exact statistics; rows that
        appear any other way leave them unknown."""
        lens = plan.seq_len_host[s].astype(np.int64)
        if not appended:
            self._stats_len[:] = -1
            return
        ok = self._stats_len == lens - 1
        if ns_refresh:
            ok |= plan.slow[s]
        self._stats_len = np.where(ok, lens, -1)

    def _new_event(self):
        # events of earlier runs that have completed are released here
        self._events = [e for e in self._events if not e.query()]
        e = torch.cuda.Event()
        self._events.append(e)
        return e

    @staticmethod
    def _no_capture(what: str):
        """The multi-stream schedules run eagerly only: capturing their
        fork/join structure into a HIP graph ended the host process inside
        the capture's end, and that is not fixed, so a capture is refused."""
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError(f"{what}: multi-stream schedules cannot be captured into a HIP graph; "
                               "run them eagerly, or capture the one-stream step()")

    # -- one decode step of a planned run ------------------------------------
    def step(self, plan: DecodePlan, s: int, q_steps, stream=None, out=None, co: bool = True,
             fused_select: bool = True, new_kv=None, fused_append: bool = True, hints: bool = True):
        """Decode step s: q_steps is the device tensor [steps][B][Hq][d].

        new_kv = (K_new, V_new), each [steps][B][1][Hkv][d]: the step appends
        every sequence's new row at row seq_len - 1, inside its own calls
        (fused_append) or by a separate sfi_append_kv call first.

        With co=True a step that has slow sequences runs as one call that
        co-launches its slow and fast shares and refreshes the slow
        sequences' selections (sfi_decode_step_select; with
        fused_select=False: sfi_decode_step, then sfi_select); with co=False
        the slow step, the selector and the fast step are separate calls.
        hints: pass the step's host row-count hints (DecodePlan.len_hints),
        so the launches plan each sequence's workgroups from its own length."""
        q = q_steps[s]
        lh = self.hints(plan, s) if hints else None
        sl = plan.seq_len[s]
        ks = None if plan.k_seq is None else plan.k_seq[s]
        ns, nf = int(plan.n_slow[s]), int(plan.n_fast[s])
        sids, fids = plan.slow_list(s), plan.fast_list(s)
        nr = None
        if new_kv is not None:
            if fused_append:
                nr = (new_kv[0][s], new_kv[1][s])
            else:
                self.append(new_kv[0][s], new_kv[1][s], sl, None, self.B, stream)
        combined = bool(co and ns and fused_select)
        use_stats = combined and new_kv is not None and self._stats_current(plan, s)
        self._note_stats(plan, s, new_kv is not None, ns_refresh=combined)
        if combined:
            self.step_select(q, sl, sids, ns, fids, nf, stream, out=out, k_seq=ks, new_rows=nr,
                             use_stats=use_stats, len_hints=lh)
            return
        if co and ns and nf:
            self.co_step(q, sl, sids, ns, fids, nf, stream, out=out, k_seq=ks, new_rows=nr, len_hints=lh)
            return
        if ns:
            self.slow(q, sl, sids, ns, stream, out=out, k_seq=ks, new_rows=nr, len_hints=lh)
        if nf:
            self.fast(q, sl, fids, nf, stream, out=out, new_rows=nr, len_hints=lh)

    def run_pipelined(self, plan: DecodePlan, q_steps, s_begin: int, s_end: int, stream_a,
                      stream_b, stream_c, out_steps, hints: bool = True):
        """Steps [s_begin, s_end) as three overlapping chains.

        A: slow steps (dense attention + evidence), C: the selector, B: fast
        steps -- the asynchronous pipeline of the Slow-Fast Inference pages
        (technical summary section 3.C), which hides the selector behind other
        attention work.  The evidence and key-norm buffers alternate between
        two copies by step parity, so the slow step of s+1 may run while the
        selector of s still reads the copy of s.  Dependencies, per step s:
          A(s) after the last selector that read copy s % 2;
          C(s) after A(s) and after B(s-1) (fast steps still reading the
               index lists C(s) rewrites);
          B(s) fast steps of sequences refreshed at s-1 after C(s-1); the
               other fast steps need nothing new (B is one ordered chain).
        out_steps ([steps][B][Hq][d]) receives each step's output: the chains
        may run different steps at the same time.  All chains join back into
        stream_a.
        """
        self._no_capture("run_pipelined")
        for st in (stream_a, stream_b, stream_c):
            with torch.cuda.stream(st):
                self._no_capture("run_pipelined")
        copies = [(self.evidence, self.key_norm), (self.evidence_alt, self.key_norm_alt)]
        ev = self._new_event
        start = ev()
        start.record(stream_a)
        stream_b.wait_event(start)
        stream_c.wait_event(start)
        last_c_parity = [None, None]
        prev_b = None
        prev_c = None
        for s in range(s_begin, s_end):
            q = q_steps[s]
            sl = plan.seq_len[s]
            out = out_steps[s]
            ns = int(plan.n_slow[s])
            lh = self.hints(plan, s) if hints else None
            c_ev = None
            if ns:
                ev_buf, kn_buf = copies[s % 2]
                if last_c_parity[s % 2] is not None:
                    stream_a.wait_event(last_c_parity[s % 2])
                self.kv.seq_len = sl.data_ptr()
                kvs = self.kv if lh is None else self._kvx(None, len_hints=(lh[0], None))
                sfi.sfi_slow_step(kvs, plan.slow_ids[s], ns, q, out, ev_buf, kn_buf, self.ld,
                                  self.ws_slow, self.ws_slow_bytes, stream_a)
                a_ev = ev()
                a_ev.record(stream_a)
                stream_c.wait_event(a_ev)
                if prev_b is not None:
                    stream_c.wait_event(prev_b)
                sfi.sfi_select(self.params, plan.slow_ids[s], ns, sl.data_ptr(), self.B, self.Hkv,
                               self.max_len, ev_buf, kn_buf, self.ld, self.sel_idx, self.sel_count,
                               None, self.ws_sel, self.ws_sel_bytes, stream_c)
                c_ev = ev()
                c_ev.record(stream_c)
                last_c_parity[s % 2] = c_ev
            no, nn = int(plan.n_fast_old[s]), int(plan.n_fast_new[s])
            if no:
                self.fast(q, sl, plan.fast_old_ids[s], no, stream_b, out=out,
                          len_hints=None if lh is None else (None, lh.fast_old))
            if nn:
                if prev_c is not None:
                    stream_b.wait_event(prev_c)
                self.fast(q, sl, plan.fast_new_ids[s], nn, stream_b, out=out,
                          len_hints=None if lh is None else (None, lh.fast_new))
            b_ev = ev()
            b_ev.record(stream_b)
            prev_b = b_ev
            prev_c = c_ev
        end_b = ev()
        end_b.record(stream_b)
        end_c = ev()
        end_c.record(stream_c)
        stream_a.wait_event(end_b)
        stream_a.wait_event(end_c)

    def run_two_streams(self, plan: DecodePlan, q_steps, s_begin: int, s_end: int, stream_a,
                        stream_b, out_steps=None, new_kv=None, hints: bool = True):
        """Steps [s_begin, s_end) as two overlapping chains.

        Stream A carries each step's slow steps and selector, stream B its fast
        steps, so slow and fast kernels co-run and the selector of step s runs
        while fast steps stream their rows (the asynchronous pipeline of the
        Slow-Fast Inference pages, technical summary section 3.C).  Ordering:
        B(s) waits for A(s-1) (a sequence refreshed at s-1 reads its new index
        list at s); A(s)'s selector waits for B(s-1) (it may only overwrite a
        list once the fast steps that read it are done), and with a shared
        output buffer (out_steps None) so does A(s)'s slow step (a sequence
        fast at s-1 and slow at s writes the same output slot).  With new_kv
        each chain's step call appends its own sequences' rows (fused
        append).  Both chains join back into stream_a.  Eager only (see
        _no_capture).
        """
        self._no_capture("run_two_streams")
        for st in (stream_a, stream_b):
            with torch.cuda.stream(st):
                self._no_capture("run_two_streams")
        ev = self._new_event
        start = ev()
        start.record(stream_a)
        stream_b.wait_event(start)
        prev_a = prev_b = None
        for s in range(s_begin, s_end):
            q = q_steps[s]
            sl = plan.seq_len[s]
            out = None if out_steps is None else out_steps[s]
            ns, nf = int(plan.n_slow[s]), int(plan.n_fast[s])
            lh = self.hints(plan, s) if hints else None
            if ns:
                sids = plan.slow_list(s)
                nr = None if new_kv is None else (new_kv[0][s], new_kv[1][s])
                if out_steps is None and prev_b is not None:
                    stream_a.wait_event(prev_b)
                self.slow(q, sl, sids, ns, stream_a, out=out, select=False, new_rows=nr, len_hints=lh)
                if prev_b is not None:
                    stream_a.wait_event(prev_b)
                self.slow_select_only(sl, sids, ns, stream_a,
                                      k_seq=None if plan.k_seq is None else plan.k_seq[s])
            ev_a = ev()
            ev_a.record(stream_a)
            if prev_a is not None:
                stream_b.wait_event(prev_a)
            if nf:
                fids = plan.fast_list(s)
                nr = None if new_kv is None else (new_kv[0][s], new_kv[1][s])
                self.fast(q, sl, fids, nf, stream_b, out=out, new_rows=nr, len_hints=lh)
            ev_b = ev()
            ev_b.record(stream_b)
            prev_a, prev_b = ev_a, ev_b
        if prev_b is not None:
            stream_a.wait_event(prev_b)


class VegasDecoder:
    """Verify -> select -> draft iterations over a resident KV cache."""

    def __init__(self, K, V, Hq: int, max_len: int, T: int, *, n_sink: int, window: int, k: int,
                 page_table=None, page_size: int = 0, keep_raw: bool = False):
        dev = K.device
        self.dev = dev
        self.Hq, self.T = Hq, T
        if page_table is None:
            B, Hkv, cap, d = K.shape
        else:
            Hkv, d = K.shape[1], K.shape[3]
            B = page_table.shape[0]
        self.B, self.Hkv, self.d = B, Hkv, d
        self.max_len = int(max_len)
        self.n_sink, self.window, self.k = n_sink, window, k
        self._dummy_len = torch.full((B,), self.max_len, dtype=torch.int32, device=dev)
        self.kv = sfi.make_kv(K, V, self._dummy_len, Hq, self.max_len, page_table, page_size)
        self.params = sfi.select_params(sfi.SFI_SCORE_RAW, 0.0, k, n_sink, window)
        self.ld = self.max_len
        f32 = dict(dtype=torch.float32, device=dev)
        self.vout = torch.zeros((B, T, Hq, d), **f32)
        self.out = torch.zeros((B, Hq, d), **f32)
        self.agg = torch.zeros((B, self.ld), **f32)
        # raw-logit emission: room for every row's logits; a call with R
        # collected rows fills it as [B][R][Hq][ld] (raw_view(R))
        self.raw_logits = torch.zeros((B, T, Hq, self.ld), **f32) if keep_raw else None
        self.sel_idx = torch.full((B, 1, k), -1, dtype=torch.int32, device=dev)
        self.sel_count = torch.zeros((B, 1), dtype=torch.int32, device=dev)
        u8 = dict(dtype=torch.uint8, device=dev)
        self.ws_ver_bytes = sfi.sfi_verify_workspace_bytes(self.kv, T)
        self.ws_sel_bytes = sfi.sfi_select_workspace_bytes(B, 1, self.max_len)
        self.ws_fast_bytes = sfi.sfi_fast_workspace_bytes(self.kv, k, n_sink, window)
        self.ws_ver = torch.zeros(self.ws_ver_bytes, **u8)
        self.ws_sel = torch.zeros(self.ws_sel_bytes, **u8)
        self.ws_fast = torch.zeros(self.ws_fast_bytes, **u8)

    def verify(self, q_rows, seq_len, row_mask: int, batch_ids=None, batch_n=None, stream=None,
               raw: bool = False):
        """q_rows [B][T][Hq][d] bf16; seq_len counts the T verified rows.
        raw: emit the collected rows' logits to self.raw_logits and sum them
        in a second pass (sfi_verify_raw_logits) instead of aggregating in
        the kernel."""
        self.kv.seq_len = seq_len.data_ptr() if torch.is_tensor(seq_len) else seq_len
        bn = self.B if batch_n is None else batch_n
        if raw:
            sfi.sfi_verify_raw_logits(self.kv, batch_ids, bn, q_rows, self.T, row_mask, self.vout, self.agg,
                                      self.ld, self.raw_logits, self.ld, self.ws_ver, self.ws_ver_bytes, stream)
            return
        sfi.sfi_verify_aggregate(self.kv, batch_ids, bn, q_rows, self.T, row_mask, self.vout,
                                 self.agg, self.ld, self.ws_ver, self.ws_ver_bytes, stream)

    def raw_view(self, R: int):
        """The emitted logits of a call that collected R rows, [B][R][Hq][ld]."""
        n = self.B * R * self.Hq * self.ld
        return self.raw_logits.view(-1)[:n].view(self.B, R, self.Hq, self.ld)

    def append(self, k_new, v_new, seq_len, batch_ids=None, batch_n=None, stream=None):
        """Write new K/V rows (k_new, v_new [B][T'][Hkv][d]) at cache rows
        seq_len - T' .. seq_len - 1 (sfi_append_kv)."""
        self.kv.seq_len = seq_len.data_ptr() if torch.is_tensor(seq_len) else seq_len
        bn = self.B if batch_n is None else batch_n
        sfi.sfi_append_kv(self.kv, batch_ids, bn, k_new, v_new, int(k_new.shape[1]), stream)

    def select(self, seq_len, batch_ids=None, batch_n=None, stream=None):
        ptr = seq_len.data_ptr() if torch.is_tensor(seq_len) else seq_len
        bn = self.B if batch_n is None else batch_n
        sfi.sfi_select(self.params, batch_ids, bn, ptr, self.B, 1, self.max_len, self.agg, None,
                       self.ld, self.sel_idx, self.sel_count, None, self.ws_sel, self.ws_sel_bytes,
                       stream)

    def draft(self, q, seq_len, batch_ids=None, batch_n=None, stream=None, new_rows=None):
        """Draft step (sparse attention on the selection); new_rows =
        (k_new, v_new) [B][Hkv][d] appends the step's row in the same call."""
        self.kv.seq_len = seq_len.data_ptr() if torch.is_tensor(seq_len) else seq_len
        bn = self.B if batch_n is None else batch_n
        kv = self.kv if new_rows is None else sfi.with_new_rows(self.kv, new_rows[0], new_rows[1])
        sfi.sfi_fast_step(kv, batch_ids, bn, q, self.sel_idx, self.sel_count, 1, self.k,
                          self.n_sink, self.window, self.out, self.ws_fast, self.ws_fast_bytes,
                          stream)
