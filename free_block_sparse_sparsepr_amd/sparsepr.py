"""Python front end of the SparsePR call (thin wrapper over include/sparsepr.h).

torch allocates the device buffers and supplies the current HIP stream; the five entry
points (partition, route, attend, probe_fit, apply) and the dense baseline all run in
libsparsepr.so.  There is no fallback: without the library every call raises.
"""
import ctypes
import dataclasses
from dataclasses import dataclass

import torch

from . import _binding as B


@dataclass
class Config:
    heads_q: int
    heads_kv: int
    n: int
    d: int
    dtype: str = "bf16"          # "bf16" or "fp32"
    groups_q: int = 64
    groups_k: int = 64
    rho_exec: float = 0.22
    r_k: int = 48
    r_q: int = 64
    n_probe: int = 64
    rank: int = 16
    lam: float = 0.1
    kmeans_iters: int = 10
    softmax_scale: float = 0.0
    ablation: int = 0           # _binding.ABLATE_*: 0 = the method
    probe_mode: int = 0         # _binding.PROBES_*: 0 = stratified radial probes
    partition_mode: int = 0     # _binding.PARTITION_*: 0 = response-coupled
    budget_mode: int = 0        # _binding.BUDGET_*: 0 = per KV head, 1 = shared by all KV heads
    cost_mode: int = 0          # _binding.COST_*: 0 = pairs, 1 = tile-padded pairs

    @property
    def key_feat(self):
        """Width of the key features (r_k, or d for the semantic partition)."""
        return self.d if self.partition_mode == B.PARTITION_SEMANTIC else self.r_k

    @property
    def query_feat(self):
        """Width of the query features (G_K, or d for the semantic partition)."""
        return self.d if self.partition_mode == B.PARTITION_SEMANTIC else self.groups_k

    @property
    def corr_rank(self):
        """Columns of A / rows of B: rank, or n_probe for the unprojected ridge."""
        return self.n_probe if self.ablation == B.ABLATE_RIDGE_ONLY else self.rank

    @property
    def g(self):
        return self.heads_q // self.heads_kv

    @property
    def n_pad(self):
        return (self.n + 15) // 16 * 16

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def params(self) -> B.Params:
        return B.Params(self.heads_q, self.heads_kv, self.n, self.d,
                        B.BF16 if self.dtype == "bf16" else B.FP32, self.groups_q, self.groups_k,
                        self.r_k, self.r_q, self.n_probe, self.rank, self.lam, self.rho_exec, 64,
                        self.kmeans_iters, self.softmax_scale, self.ablation, self.probe_mode,
                        self.partition_mode, self.budget_mode, self.cost_mode)


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def workspace_bytes(cfg: Config) -> int:
    lib = B.load()
    out = ctypes.c_size_t(0)
    prm = cfg.params()
    B.check(lib.sparsepr_workspace_size(ctypes.byref(prm), ctypes.byref(out)))
    return out.value


class SparsePR:
    """Owns the device buffers of one call shape; `__call__` runs the unfused order
    partition -> route -> attend -> probe_fit -> apply on the current stream."""

    def __init__(self, cfg: Config, device="cuda"):
        self.cfg = cfg
        self.lib = B.load()
        self.prm = cfg.params()
        self.prm_defer = cfg.params()      # the same call with the K/V gathers left to gather_kv
        self.prm_defer.defer_kv_gather = 1
        dev = torch.device(device)
        c = cfg
        i32, f32 = torch.int32, torch.float32
        e = lambda *shape, dt=i32: torch.empty(shape, dtype=dt, device=dev)  # noqa: E731
        self.ws = e(max(workspace_bytes(cfg), 256), dt=torch.uint8)
        self.part = dict(
            responses_s=e(c.heads_kv, c.r_k, c.n, dt=f32), responses_u=e(c.heads_q, c.n, c.groups_k, dt=f32),
            exponents=e(c.heads_kv, 2), key_labels=e(c.heads_kv, c.n),
            key_centroids_int=e(c.heads_kv, c.groups_k, c.key_feat), key_perm=e(c.heads_kv, c.n),
            key_offsets=e(c.heads_kv, c.groups_k + 1), key_centroids=e(c.heads_kv, c.groups_k, c.d, dt=f32),
            query_features=e(c.heads_kv, c.n, c.query_feat, dt=torch.int8), query_labels=e(c.heads_kv, c.n),
            query_centroids=e(c.heads_kv, c.groups_q, c.query_feat), query_perm=e(c.heads_kv, c.n),
            query_offsets=e(c.heads_kv, c.groups_q + 1),
            q_gm=e(c.heads_kv, c.n, c.g, c.d, dt=c.torch_dtype), k_gm=e(c.heads_kv, c.n, c.d, dt=c.torch_dtype),
            v_gm=e(c.heads_kv, c.d, c.n_pad, dt=c.torch_dtype))
        if c.g > 1:   # the head-summed query coordinate the features quantise (read back by tests)
            self.part["query_coord_sum"] = e(c.heads_kv, c.n, c.query_feat, dt=f32)
        self.route_buf = dict(
            row_ptr=e(c.heads_kv, c.groups_q + 1), cols=e(c.heads_kv, c.groups_q * c.groups_k),
            kept_mask=e(c.heads_kv, c.groups_q, dt=torch.int64), pairs=e(c.heads_kv, dt=torch.int64),
            cell_mass=e(c.heads_kv, c.groups_q, c.groups_k, dt=torch.int64))
        self.fit = dict(
            probe_tokens=e(c.heads_kv, c.n_probe), probe_groups=e(c.heads_kv, c.n_probe),
            probe_weights=e(c.heads_kv, c.n_probe, dt=torch.float64),
            o_dense=e(c.heads_q, c.n_probe, c.d, dt=f32), o_sparse=e(c.heads_q, c.n_probe, c.d, dt=f32),
            A=e(c.heads_q, c.d, c.corr_rank, dt=f32), B=e(c.heads_q, c.corr_rank, c.d, dt=f32),
            c0=e(c.heads_q, c.d, dt=f32),
            r_eff=e(c.heads_q), eig=e(c.heads_q, c.rank + 1, dt=f32))
        self.o_gm = e(c.heads_kv, c.n, c.g, c.d, dt=f32)
        self.lse = e(c.heads_kv, c.n, c.g, dt=f32)
        self._part_t = B.PartitionT(*[self.part[k].data_ptr() if k in self.part else None
                                      for k in B.PARTITION_FIELDS])
        self._route_t = B.RouteT(*[self.route_buf[k].data_ptr() for k in B.ROUTE_FIELDS])
        self._fit_t = B.FitT(*[self.fit[k].data_ptr() for k in B.FIT_FIELDS])

    # -- input checks (shape/dtype/device only; the library validates everything else)
    def _check_qkv(self, q, k, v):
        c = self.cfg
        for t, h in ((q, c.heads_q), (k, c.heads_kv), (v, c.heads_kv)):
            if t is None:
                continue
            if t.shape != (h, c.n, c.d) or t.dtype != c.torch_dtype or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"expected contiguous {c.torch_dtype} cuda tensor of shape {(h, c.n, c.d)}, "
                                 f"got {tuple(t.shape)} {t.dtype} {t.device}")

    def partition(self, q, k, v, defer_kv=False):
        """defer_kv: leave k_gm and v_gm to gather_kv (which may then run on another stream)."""
        self._check_qkv(q, k, v)
        prm = self.prm_defer if defer_kv else self.prm
        B.check(self.lib.sparsepr_partition(ctypes.byref(prm), _p(q), _p(k), _p(v),
                                            ctypes.byref(self._part_t), _p(self.ws), self.ws.numel(), _stream()))

    def gather_kv(self, k, v):
        self._check_qkv(None, k, v)
        B.check(self.lib.sparsepr_gather_kv(ctypes.byref(self.prm), _p(k), _p(v), ctypes.byref(self._part_t),
                                            _stream()))

    def route(self):
        B.check(self.lib.sparsepr_route(ctypes.byref(self.prm), ctypes.byref(self._part_t),
                                        ctypes.byref(self._route_t), _p(self.ws), self.ws.numel(), _stream()))

    def attend(self):
        B.check(self.lib.sparsepr_attend(ctypes.byref(self.prm), ctypes.byref(self._part_t),
                                         ctypes.byref(self._route_t), _p(self.o_gm), _p(self.lse), _p(self.ws),
                                         self.ws.numel(), _stream()))

    def attend_noalloc(self):
        """attend() through sparsepr_attend_noalloc: no workspace, the schedule in the
        library's fixed device array."""
        B.check(self.lib.sparsepr_attend_noalloc(ctypes.byref(self.prm), ctypes.byref(self._part_t),
                                                 ctypes.byref(self._route_t), _p(self.o_gm), _p(self.lse),
                                                 _stream()))

    def probe_fit(self, q):
        self._check_qkv(q, None, None)
        B.check(self.lib.sparsepr_probe_fit(ctypes.byref(self.prm), _p(q), ctypes.byref(self._part_t),
                                            ctypes.byref(self._route_t), ctypes.byref(self._fit_t), _p(self.ws),
                                            self.ws.numel(), _stream()))

    def apply(self, out=None):
        c = self.cfg
        if out is None:
            out = torch.empty((c.heads_q, c.n, c.d), dtype=c.torch_dtype, device=self.o_gm.device)
        B.check(self.lib.sparsepr_apply(ctypes.byref(self.prm), _p(self.o_gm), ctypes.byref(self._part_t),
                                        ctypes.byref(self._fit_t), _p(out), _stream()))
        return out

    def attend_apply(self, out=None):
        c = self.cfg
        if out is None:
            out = torch.empty((c.heads_q, c.n, c.d), dtype=c.torch_dtype, device=self.o_gm.device)
        B.check(self.lib.sparsepr_attend_apply(ctypes.byref(self.prm), ctypes.byref(self._part_t),
                                               ctypes.byref(self._route_t), ctypes.byref(self._fit_t), _p(out),
                                               _p(self.ws), self.ws.numel(), _stream()))
        return out

    def __call__(self, q, k, v, out=None):
        """Unfused order: partition -> route -> attend -> probe_fit -> apply."""
        self.partition(q, k, v)
        self.route()
        self.attend()
        self.probe_fit(q)
        return self.apply(out)

    def fused(self, q, k, v, out=None):
        """Fused order: partition -> route -> probe_fit -> attend_apply."""
        self.partition(q, k, v)
        self.route()
        self.probe_fit(q)
        return self.attend_apply(out)

    def side_stream(self):
        """The second stream of the overlapped order (default priority), created on first use."""
        if getattr(self, "_side", None) is None:
            self._side = torch.cuda.Stream(device=self.o_gm.device)
        return self._side

    def overlapped(self, q, k, v, out=None):
        """Unfused order on two streams: the partition leaves the K/V gathers to the second
        stream, where they run beside the route; then probe_fit (second stream) runs beside
        attend (current stream, after the gathers), and apply once both are done.  The
        branches share only read-only partition and route buffers: the gathers write k_gm
        and v_gm, attend o_gm and lse, probe_fit the fit buffers and its workspace region."""
        main = torch.cuda.current_stream()
        side = self.side_stream()
        self.partition(q, k, v, defer_kv=True)
        side.wait_stream(main)
        with torch.cuda.stream(side):
            self.gather_kv(k, v)
            kv_ready = torch.cuda.Event()
            kv_ready.record(side)
        self.route()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            self.probe_fit(q)
        main.wait_event(kv_ready)
        self.attend()
        main.wait_stream(side)
        return self.apply(out)

    def _head_views(self, kv0, kv1):
        """The call's buffers restricted to KV heads [kv0, kv1) (every buffer is head-major):
        params and partition / route / fit structs of that sub-call, its O_gm and LSE rows,
        and a workspace of the sub-call's size of its own (the attention keeps its tile
        schedule there, so two head ranges can run at once)."""
        views = self.__dict__.setdefault("_views", {})
        if (kv0, kv1) in views:
            return views[(kv0, kv1)]
        c = self.cfg
        h0, h1 = kv0 * c.g, kv1 * c.g
        sub = dataclasses.replace(c, heads_kv=kv1 - kv0, heads_q=h1 - h0)
        per_query_head = {"responses_u", "o_dense", "o_sparse", "A", "B", "c0", "r_eff", "eig"}
        cut = lambda name, t: t[h0:h1] if name in per_query_head else t[kv0:kv1]  # noqa: E731
        part = {k: cut(k, t) for k, t in self.part.items()}
        route = {k: cut(k, t) for k, t in self.route_buf.items()}
        fit = {k: cut(k, t) for k, t in self.fit.items()}
        v = dict(prm=sub.params(), h0=h0, h1=h1, o_gm=self.o_gm[kv0:kv1], lse=self.lse[kv0:kv1],
                 ws=torch.empty(max(workspace_bytes(sub), 256), dtype=torch.uint8, device=self.ws.device),
                 part=B.PartitionT(*[part[k].data_ptr() if k in part else None for k in B.PARTITION_FIELDS]),
                 route=B.RouteT(*[route[k].data_ptr() for k in B.ROUTE_FIELDS]),
                 fit=B.FitT(*[fit[k].data_ptr() for k in B.FIT_FIELDS]))
        views[(kv0, kv1)] = v
        return v

    def third_stream(self):
        """The third stream of the split order (default priority), created on first use."""
        if getattr(self, "_third", None) is None:
            self._third = torch.cuda.Stream(device=self.o_gm.device)
        return self._third

    def split_point(self):
        """KV heads whose attention runs beside the probe stage in the split order: a sixth of
        them (the fastest of 4, 6 and 8 of 24 at the 720p shape), at least one, and at least
        one left for the fused part."""
        return max(1, min(self.cfg.heads_kv - 1, self.cfg.heads_kv // 6))

    SPLIT_STAGES = ["partition", "gather_kv (second stream)", "route", "probe_fit (second stream)",
                    "attend (first KV heads)", "attend_apply (other KV heads, third stream)",
                    "apply (first KV heads)"]

    def split(self, q, k, v, out=None, first_kv=None, events=None):
        """The overlapped order with the write-back fused where the fit is already there: the
        attention of the first ``first_kv`` KV heads (fp32 group-major rows) runs beside
        probe_fit, as in ``overlapped``; as soon as the fit is done, attend_apply runs the
        other heads' attention with the correction in its epilogue on a third stream (it
        shares no buffer with the first heads' attention, so its blocks fill the CUs as the
        first launch drains), and apply writes back the first heads' rows.  Every head's
        arithmetic is that of the unfused call (the fused heads as in ``fused``).  ``events``:
        optional dict stage (``SPLIT_STAGES``) -> (start, end) torch events, recorded on the
        stream that runs the stage (for timing)."""
        c = self.cfg
        if out is None:
            out = torch.empty((c.heads_q, c.n, c.d), dtype=c.torch_dtype, device=self.o_gm.device)
        first = self.split_point() if first_kv is None else int(first_kv)
        if not 0 < first < c.heads_kv:
            raise ValueError(f"first_kv must leave heads on both sides: 0 < {first} < {c.heads_kv}")
        a, b = self._head_views(0, first), self._head_views(first, c.heads_kv)
        main, side, third = torch.cuda.current_stream(), self.side_stream(), self.third_stream()

        def stage(i, stream, fn):
            with torch.cuda.stream(stream):
                if events is not None:
                    events[self.SPLIT_STAGES[i]][0].record(stream)
                fn()
                if events is not None:
                    events[self.SPLIT_STAGES[i]][1].record(stream)

        stage(0, main, lambda: self.partition(q, k, v, defer_kv=True))
        side.wait_stream(main)
        stage(1, side, lambda: self.gather_kv(k, v))
        kv_ready = torch.cuda.Event()
        kv_ready.record(side)
        stage(2, main, self.route)
        side.wait_stream(main)
        stage(3, side, lambda: self.probe_fit(q))
        fit_done = torch.cuda.Event()
        fit_done.record(side)
        main.wait_event(kv_ready)
        stage(4, main, lambda: B.check(self.lib.sparsepr_attend(
            ctypes.byref(a["prm"]), ctypes.byref(a["part"]), ctypes.byref(a["route"]), _p(a["o_gm"]),
            _p(a["lse"]), _p(a["ws"]), a["ws"].numel(), _stream())))
        third.wait_event(fit_done)
        stage(5, third, lambda: B.check(self.lib.sparsepr_attend_apply(
            ctypes.byref(b["prm"]), ctypes.byref(b["part"]), ctypes.byref(b["route"]), ctypes.byref(b["fit"]),
            _p(out[b["h0"]:b["h1"]]), _p(b["ws"]), b["ws"].numel(), _stream())))
        main.wait_event(fit_done)
        stage(6, main, lambda: B.check(self.lib.sparsepr_apply(
            ctypes.byref(a["prm"]), _p(a["o_gm"]), ctypes.byref(a["part"]), ctypes.byref(a["fit"]),
            _p(out[a["h0"]:a["h1"]]), _stream())))
        main.wait_stream(third)
        return out

    def capture(self, q, k, v, out, order="fused"):
        """Records one whole call of the given order ("fused", "unfused", "overlapped" or "split") into
        a HIP graph and returns it (``graph.replay()`` reruns the call on the same buffers).
        One eager call runs first, on a side stream (the usual warm-up before a capture: torch's
        own lazy set-up, such as the side stream of the overlapped order, happens outside it)."""
        fn = {"fused": self.fused, "unfused": self.__call__, "overlapped": self.overlapped, "split": self.split}[order]
        warm = torch.cuda.Stream(device=out.device)
        warm.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(warm):
            fn(q, k, v, out)
        torch.cuda.current_stream().wait_stream(warm)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn(q, k, v, out)
        return graph

    def residual_diagnostics(self, q, k, v):
        """[Hq, 4] float64: ||R||^2, ||R - mean R||^2, affine-orthogonal energy, explainable
        fraction of R = O_dense - O_sparse over every row (needs partition and route first;
        allocates its own large workspace for the call)."""
        c = self.cfg
        self._check_qkv(q, k, v)
        nbytes = ctypes.c_size_t(0)
        B.check(self.lib.sparsepr_diagnostics_workspace_size(ctypes.byref(self.prm), ctypes.byref(nbytes)))
        ws = torch.empty(max(nbytes.value, 256), dtype=torch.uint8, device=q.device)
        out = torch.empty((c.heads_q, 4), dtype=torch.float64, device=q.device)
        B.check(self.lib.sparsepr_residual_diagnostics(ctypes.byref(self.prm), _p(q), _p(k), _p(v),
                                                       ctypes.byref(self._part_t), ctypes.byref(self._route_t),
                                                       _p(out), _p(ws), ws.numel(), _stream()))
        return out

    def support_diagnostics(self, q, k, sets, mass=0.9, with_scores=False):
        """90 %-mass supports: ``sets`` [Hq, n_sets, s] int32 query tokens (device).  Returns
        (row_support [Hq, n_sets, s], shared_support [Hq, n_sets]) int32 key counts; needs
        only Q and K (allocates its own workspace for the call).  With ``with_scores`` (at
        most 512 items) also the fp32 scores the decisions were taken on, [Hq, n_sets, s, n],
        read back from the workspace."""
        c = self.cfg
        if sets.dtype != torch.int32 or sets.dim() != 3 or sets.shape[0] != c.heads_q or not sets.is_contiguous():
            raise ValueError("sets must be a contiguous int32 tensor [heads_q, n_sets, set_size]")
        if sets.device != q.device or k.device != q.device:
            raise ValueError("q, k and sets must be on one device")
        n_sets, s = int(sets.shape[1]), int(sets.shape[2])
        nbytes = ctypes.c_size_t(0)
        B.check(self.lib.sparsepr_support_workspace_size(ctypes.byref(self.prm), n_sets, s, ctypes.byref(nbytes)))
        ws = torch.empty(max(nbytes.value, 256), dtype=torch.uint8, device=q.device)
        rows = torch.empty((c.heads_q, n_sets, s), dtype=torch.int32, device=q.device)
        union = torch.empty((c.heads_q, n_sets), dtype=torch.int32, device=q.device)
        B.check(self.lib.sparsepr_support_diagnostics(ctypes.byref(self.prm), _p(q), _p(k), _p(sets), n_sets, s,
                                                      float(mass), _p(rows), _p(union), _p(ws), ws.numel(),
                                                      _stream()))
        if with_scores:
            if c.heads_q * n_sets > 512:
                raise ValueError("scores are kept for at most 512 (head, set) items")
            nsc = c.heads_q * n_sets * s * c.n
            scores = ws[:nsc * 4].view(torch.float32).view(c.heads_q, n_sets, s, c.n)
            return rows, union, scores
        return rows, union

    def dense(self, q, k, v, out=None):
        self._check_qkv(q, k, v)
        c = self.cfg
        if out is None:
            out = torch.empty((c.heads_q, c.n, c.d), dtype=c.torch_dtype, device=q.device)
        B.check(self.lib.sparsepr_dense_attention(ctypes.byref(self.prm), _p(q), _p(k), _p(v), _p(out),
                                                  _p(self.ws), self.ws.numel(), _stream()))
        return out


def config_from_workload(w, **overrides) -> Config:
    """Config of a sparsepr_workloads.Workload (keyword overrides, e.g. ablation=...)."""
    kw = dict(heads_q=w.heads_q, heads_kv=w.heads_kv, n=w.n, d=w.d, dtype=w.dtype, groups_q=w.groups_q,
              groups_k=w.groups_k, rho_exec=w.rho_exec, r_k=w.r_k, r_q=w.r_q, n_probe=w.n_probe,
              rank=w.rank, lam=w.lam, kmeans_iters=w.kmeans_iters)
    kw.update(overrides)
    return Config(**kw)


class PipelinedSparsePR:
    """The SparsePR call over chunks of KV heads, pipelined on three streams (default
    priority): chunk i's partition and route run beside chunk i-1's attention, so only the
    first chunk's partition, route and probe stage are exposed.  Every head's arithmetic is
    that of one SparsePR call (each chunk is a SparsePR instance on its slice of the
    heads), so the output is identical.  The budget must be per KV head (a shared budget
    couples the heads).

    fused=True:  partition, route (stream P) -> probe_fit (stream F) -> attend_apply (stream A).
    fused=False: partition, route (P) -> attend (A) beside probe_fit (F) -> apply (A)."""

    def __init__(self, cfg: Config, chunks=4, device="cuda", fused=True):
        if cfg.budget_mode != B.BUDGET_PER_HEAD:
            raise ValueError("a budget shared across heads cannot be split into head chunks")
        chunks = max(1, min(chunks, cfg.heads_kv))
        base, extra = divmod(cfg.heads_kv, chunks)
        self.cfg, self.fused = cfg, fused
        self.parts = []      # (kv0, kv1, SparsePR)
        kv0 = 0
        for i in range(chunks):
            nkv = base + (1 if i < extra else 0)
            sub = dataclasses.replace(cfg, heads_kv=nkv, heads_q=nkv * cfg.g)
            self.parts.append((kv0, kv0 + nkv, SparsePR(sub, device=device)))
            kv0 += nkv
        dev = torch.device(device)
        self.streams = [torch.cuda.Stream(device=dev) for _ in range(3)]   # P, F, A

    def __call__(self, q, k, v, out=None, events=None):
        """``events``: optional dict stage -> list of (start, end) torch events per chunk,
        recorded on the stream that runs the stage (for timing)."""
        c = self.cfg
        if out is None:
            out = torch.empty((c.heads_q, c.n, c.d), dtype=c.torch_dtype, device=q.device)
        main = torch.cuda.current_stream()
        sp_, sf, sa = self.streams
        for s in self.streams:
            s.wait_stream(main)

        def run(stage, i, stream, fn):
            with torch.cuda.stream(stream):
                if events is not None:
                    events[stage][i][0].record(stream)
                fn()
                if events is not None:
                    events[stage][i][1].record(stream)

        for i, (kv0, kv1, sp) in enumerate(self.parts):
            h0, h1 = kv0 * c.g, kv1 * c.g
            qc, kc, vc, oc = q[h0:h1], k[kv0:kv1], v[kv0:kv1], out[h0:h1]
            run("partition", i, sp_, lambda: sp.partition(qc, kc, vc))
            run("route", i, sp_, sp.route)
            sf.wait_stream(sp_)
            run("probe_fit", i, sf, lambda: sp.probe_fit(qc))
            if self.fused:
                sa.wait_stream(sf)
                run("attend_apply", i, sa, lambda: sp.attend_apply(oc))
            else:
                sa.wait_stream(sp_)
                run("attend", i, sa, sp.attend)
                sa.wait_stream(sf)
                run("apply", i, sa, lambda: sp.apply(oc))
        for s in self.streams:
            main.wait_stream(s)
        return out

    def capture(self, q, k, v, out, order=None):
        """Records one pipelined call into a HIP graph (the three streams join the capture);
        one eager call runs first so one-time set-up stays outside it."""
        self(q, k, v, out)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self(q, k, v, out)
        return graph
