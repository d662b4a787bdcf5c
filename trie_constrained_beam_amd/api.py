"""Python face of libtcb: the same calls as include/tcb.h, with torch for device memory
and streams. Every step of the beam path and of single-pass scoring runs in the HIP
library; this module only marshals arguments.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import _lib as L
from ._lib import check, lib


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else C.c_void_p(0)


class Trie:
    """Prefix trie of a SID catalog (host build, optional device upload)."""

    def __init__(self, sids, V: int = 256, mask_depths=None, device=None):
        sids = np.ascontiguousarray(sids, dtype=np.uint8)
        if sids.ndim != 2:
            raise ValueError("sids must be [n_items, L]")
        n, depth = sids.shape
        mask_depths = L.TCB_MASK_AUTO if mask_depths is None else int(mask_depths)
        h = C.c_void_p()
        check(lib().tcb_build_trie(sids.ctypes.data, n, depth, V, mask_depths, C.byref(h)))
        self._h = h
        self._destroy = lib().tcb_trie_destroy        # held so teardown at exit needs no globals
        self.info = L.TrieInfo()
        check(lib().tcb_trie_info(h, C.byref(self.info)))
        self.L, self.V = int(self.info.L), int(self.info.V)
        self.mask_depths = int(self.info.mask_depths)
        self.d_image = None
        self.d_codes = None
        if device is not None:
            self.upload(device)

    def __del__(self):
        if getattr(self, "_h", None):
            self._destroy(self._h)
            self._h = None

    @property
    def handle(self):
        return self._h

    @property
    def n_distinct(self):
        return int(self.info.n_distinct)

    @property
    def nodes_per_depth(self):
        return [int(self.info.nodes_per_depth[d]) for d in range(self.L + 1)]

    @property
    def node_offset(self):
        return [int(self.info.node_offset[d]) for d in range(self.L + 2)]

    def host_arrays(self):
        """Copies of (child_begin, child_code, leaf_item) as numpy arrays."""
        cb, cc, li = C.c_void_p(), C.c_void_p(), C.c_void_p()
        check(lib().tcb_trie_host_arrays(self._h, C.byref(cb), C.byref(cc), C.byref(li)))
        off = self.node_offset
        n_int, n_all = off[self.L], off[self.L + 1]
        a = np.ctypeslib.as_array(C.cast(cb, C.POINTER(C.c_uint32)), shape=(n_int + 1,)).copy()
        b = np.ctypeslib.as_array(C.cast(cc, C.POINTER(C.c_uint8)), shape=(n_all,)).copy()
        c = np.ctypeslib.as_array(C.cast(li, C.POINTER(C.c_int32)), shape=(self.n_distinct,)).copy()
        return a, b, c

    def upload(self, device="cuda"):
        nbytes = int(self.info.device_bytes)
        self.d_image = torch.empty(nbytes, dtype=torch.uint8, device=device)
        check(lib().tcb_trie_upload(self._h, _ptr(self.d_image), nbytes, _stream()))
        return self

    def upload_codes(self, device="cuda"):
        """Copy every leaf's codes to the device (needed by ``score_catalog``)."""
        if self.d_image is None:
            self.upload(device)
        nb = C.c_size_t()
        check(lib().tcb_trie_codes_bytes(self._h, C.byref(nb)))
        self.d_codes = torch.empty(max(int(nb.value), 1), dtype=torch.uint8, device=device)
        check(lib().tcb_trie_upload_codes(self._h, _ptr(self.d_codes), self.d_codes.numel(), _stream()))
        return self


class Beams:
    """A decode wave: slot budget, requests, and the per-slot beam state on the GPU."""

    def __init__(self, trie: Trie, max_slots: int, max_requests: int, max_width: int,
                 norm: str = "children", device="cuda"):
        if trie.d_image is None:
            trie.upload(device)
        self.trie = trie
        self.max_slots, self.max_requests, self.max_width = max_slots, max_requests, max_width
        nb = C.c_size_t()
        check(lib().tcb_beams_workspace_bytes(trie.handle, max_slots, max_requests, max_width,
                                              C.byref(nb)))
        self.ws = torch.empty(int(nb.value), dtype=torch.uint8, device=device)
        n = {"children": L.TCB_NORM_CHILDREN, "level": L.TCB_NORM_LEVEL, "open": L.TCB_NORM_OPEN}[norm]
        h = C.c_void_p()
        check(lib().tcb_beams_create(trie.handle, max_slots, max_requests, max_width, n,
                                     _ptr(self.ws), int(nb.value), _stream(), C.byref(h)))
        self._h = h
        self._destroy = lib().tcb_beams_destroy
        self.device = device
        self._trace = None

    def __del__(self):
        if getattr(self, "_h", None):
            self._destroy(self._h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def init(self, widths):
        w = np.ascontiguousarray(widths, dtype=np.int32)
        ids = np.zeros(w.size, dtype=np.int32)
        bases = np.zeros(w.size, dtype=np.int32)
        check(lib().tcb_beam_init(self._h, w.size, w.ctypes.data, ids.ctypes.data,
                                  bases.ctypes.data, _stream()))
        return ids, bases

    def step(self, logits: torch.Tensor, temperature: float = 0.0, seed: int = 0):
        """One step. temperature 0: deterministic top-k; above 0: the Gumbel top-k
        without replacement of tcb_beam_step_sampled with this step's noise seed."""
        if logits.dtype == torch.float32:
            dt = L.TCB_F32
        elif logits.dtype == torch.bfloat16:
            dt = L.TCB_BF16
        else:
            raise TypeError("logits must be float32 or bfloat16")
        if logits.dim() != 2 or logits.stride(1) != 1 or not logits.is_cuda:
            raise ValueError("logits must be a row-major [max_slots, ld] CUDA tensor")
        if logits.shape[0] < self.max_slots:
            raise ValueError("logits must have max_slots rows")
        if temperature == 0.0:
            check(lib().tcb_beam_step(self._h, _ptr(logits), logits.stride(0), dt, _stream()))
        else:
            check(lib().tcb_beam_step_sampled(self._h, _ptr(logits), logits.stride(0), dt,
                                              float(temperature), int(seed) & (2 ** 64 - 1), _stream()))

    def step_lmhead(self, hidden: torch.Tensor, weight: torch.Tensor):
        if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
            raise TypeError("hidden and weight must be bfloat16")
        if hidden.dim() != 2 or hidden.stride(1) != 1 or hidden.shape[0] < self.max_slots:
            raise ValueError("hidden must be a row-major [max_slots, ld] CUDA tensor")
        if not weight.is_contiguous() or weight.shape[0] != self.trie.L or weight.shape[1] != 256:
            raise ValueError("weight must be a contiguous [L, 256, H] tensor")
        H = int(weight.shape[2])
        check(lib().tcb_beam_step_lmhead(self._h, _ptr(hidden), hidden.stride(0), H,
                                         _ptr(weight), _stream()))

    def export(self):
        S, R, Lv = self.max_slots, self.max_requests, self.trie.L
        dev = self.device
        out = {"node": torch.empty(S, dtype=torch.int32, device=dev),
               "score": torch.empty(S, dtype=torch.float32, device=dev),
               "phi": torch.empty(S, dtype=torch.float32, device=dev),
               "parent_slot": torch.empty(S, dtype=torch.int32, device=dev),
               "hist": torch.empty((Lv, S), dtype=torch.int32, device=dev),
               "rows": torch.empty(R, dtype=torch.int32, device=dev),
               "level": torch.empty(R, dtype=torch.int32, device=dev)}
        check(lib().tcb_beam_export(self._h, _ptr(out["node"]), _ptr(out["score"]), _ptr(out["phi"]),
                                    _ptr(out["parent_slot"]), _ptr(out["hist"]),
                                    _ptr(out["rows"]), _ptr(out["level"]), _stream()))
        return out

    def flush(self):
        """Bring the wave state up to date without copying it: launches a merge the last step
        left to the next step's tile kernel (tcb_beam_export with every buffer NULL)."""
        check(lib().tcb_beam_export(self._h, None, None, None, None, None, None, None, _stream()))

    def set_read_mode(self, mode: str = "auto"):
        """'auto', 'dense' or 'gather': how rows' logits are read (results identical)."""
        m = {"auto": L.TCB_READ_AUTO, "dense": L.TCB_READ_DENSE, "gather": L.TCB_READ_GATHER}[mode]
        check(lib().tcb_beams_set_read_mode(self._h, m))

    def set_validate(self, on: bool = True):
        check(lib().tcb_beams_set_validate(self._h, 1 if on else 0))

    def check(self):
        check(lib().tcb_beam_check(self._h, _stream()))

    def status(self):
        st = L.BeamsStatus()
        check(lib().tcb_beams_status(self._h, C.byref(st)))
        return {k: int(getattr(st, k)) for k, _ in L.BeamsStatus._fields_}

    def level(self, req_id: int) -> int:
        v = C.c_int32()
        check(lib().tcb_request_level(self._h, int(req_id), C.byref(v)))
        return int(v.value)

    def enable_timing(self, capacity: int, repeat: int = 1):
        """Record HIP events around the kernels of the next ``capacity`` steps, each kernel
        launched ``repeat`` times back to back (durations are reported per launch)."""
        check(lib().tcb_beams_enable_timing(self._h, int(capacity), int(repeat)))

    def timing(self):
        """(head_ms, tile_ms, merge_ms, steps) summed over the recorded steps; synchronises."""
        h, a, b, n = C.c_double(), C.c_double(), C.c_double(), C.c_int32()
        check(lib().tcb_beams_timing(self._h, C.byref(h), C.byref(a), C.byref(b), C.byref(n)))
        return float(h.value), float(a.value), float(b.value), int(n.value)

    def set_trace(self, capacity_words: int = 0):
        """Arm a phase trace of the kernels launched from now on into a device buffer of
        ``capacity_words`` 64-bit words (0: off). Diagnostics only."""
        self._trace = (torch.zeros(int(capacity_words), dtype=torch.int64, device=self.device)
                       if capacity_words > 0 else None)
        check(lib().tcb_beams_set_trace(self._h, _ptr(self._trace), int(capacity_words)))

    def pause_trace(self, paused: bool):
        """Stop recording into the armed trace buffer (True), or start again at its beginning
        (False), without allocating. Diagnostics only."""
        if self._trace is None:
            return
        if paused:
            check(lib().tcb_beams_set_trace(self._h, None, 0))
        else:
            check(lib().tcb_beams_set_trace(self._h, _ptr(self._trace), int(self._trace.numel())))

    def trace(self):
        """The traced launches: a list of (kind, level, records) with records an int64
        array [workgroups, TCB_TRACE_SLOTS] (word 0 = 1 + XCD, then clock marks). Synchronises."""
        n = C.c_int32()
        check(lib().tcb_beams_trace_log(self._h, None, 0, C.byref(n)))
        log = np.zeros((max(1, n.value), 4), dtype=np.int32)
        check(lib().tcb_beams_trace_log(self._h, log.ctypes.data, n.value, C.byref(n)))
        buf = self._trace.cpu().numpy() if self._trace is not None else np.zeros(0, dtype=np.int64)
        out = []
        for kind, level, grid, off in log[:n.value]:
            out.append((int(kind), int(level), buf[off:off + grid * L.TCB_TRACE_SLOTS].reshape(grid, -1)))
        return out

    def finalize(self, req_ids):
        """Ranked beams of finished requests (host arrays); releases their slots."""
        ids = np.ascontiguousarray(req_ids, dtype=np.int32)
        n, B, Lv = ids.size, self.max_width, self.trie.L
        sids = np.zeros((n, B, Lv), dtype=np.uint8)
        scores = np.zeros((n, B), dtype=np.float32)
        items = np.zeros((n, B), dtype=np.int64)
        counts = np.zeros(n, dtype=np.int32)
        check(lib().tcb_beam_finalize(self._h, n, ids.ctypes.data, sids.ctypes.data,
                                      scores.ctypes.data, items.ctypes.data, counts.ctypes.data,
                                      _stream()))
        return {"sids": sids, "scores": scores, "items": items, "counts": counts}

    def finalize_device(self, req_ids, out=None):
        """As finalize, into device tensors, without synchronising."""
        ids = np.ascontiguousarray(req_ids, dtype=np.int32)
        n, B, Lv = ids.size, self.max_width, self.trie.L
        if out is None:
            dev = self.device
            out = {"sids": torch.empty((n, B, Lv), dtype=torch.uint8, device=dev),
                   "scores": torch.empty((n, B), dtype=torch.float32, device=dev),
                   "items": torch.empty((n, B), dtype=torch.int64, device=dev),
                   "counts": torch.empty(n, dtype=torch.int32, device=dev)}
        check(lib().tcb_beam_finalize_device(self._h, n, ids.ctypes.data, _ptr(out["sids"]),
                                             _ptr(out["scores"]), _ptr(out["items"]),
                                             _ptr(out["counts"]), _stream()))
        return out

    def set_finish_outputs(self, out=True):
        """Finish requests inside the step that completes them: from now on a step that
        brings a request to depth L writes its beams (as ``finalize_device`` would) into row
        ``req_id`` of the device tensors of ``out`` and releases its id and slots at once.
        ``out``: a dict with ``sids`` [max_requests, max_width, L] uint8, ``scores`` and
        ``items`` [max_requests, max_width] float32 / int64 and ``counts`` [max_requests]
        int32 on the wave's device; ``True`` allocates one; ``None`` turns the mode off.
        Returns the dict (kept referenced while set)."""
        if out is None:
            check(lib().tcb_beams_set_finish_outputs(self._h, None, None, None, None))
            self._finish_out = None
            return None
        R, B, Lv = self.max_requests, self.max_width, self.trie.L
        if out is True:
            dev = self.device
            out = {"sids": torch.zeros((R, B, Lv), dtype=torch.uint8, device=dev),
                   "scores": torch.zeros((R, B), dtype=torch.float32, device=dev),
                   "items": torch.zeros((R, B), dtype=torch.int64, device=dev),
                   "counts": torch.zeros(R, dtype=torch.int32, device=dev)}
        want = {"sids": ((R, B, Lv), torch.uint8), "scores": ((R, B), torch.float32),
                "items": ((R, B), torch.int64), "counts": ((R,), torch.int32)}
        for k, (shape, dt) in want.items():
            t = out[k]
            if tuple(t.shape) != shape or t.dtype != dt or not t.is_contiguous() or t.device.type != "cuda":
                raise ValueError(f"set_finish_outputs: {k} must be a contiguous {dt} {shape} device tensor")
        check(lib().tcb_beams_set_finish_outputs(self._h, _ptr(out["sids"]), _ptr(out["scores"]),
                                                 _ptr(out["items"]), _ptr(out["counts"])))
        self._finish_out = out
        return out


def invalid_rate(out) -> float:
    """Share of returned beams that are not catalog SIDs (item < 0) in a finalize result:
    0 under the SID constraint; the open-vocabulary comparison of flashrec 0.1.0,
    Evaluation reports how many beams an unconstrained decode leaves illegal."""
    items, counts = out["items"], out["counts"]
    if isinstance(items, torch.Tensor):
        items, counts = items.cpu().numpy(), counts.cpu().numpy()
    total = int(np.sum(counts))
    if total == 0:
        return 0.0
    bad = sum(int(np.sum(items[i, :int(c)] < 0)) for i, c in enumerate(counts))
    return bad / total


def score_workspace_bytes(trie: Trie, max_users: int) -> int:
    nb = C.c_size_t()
    check(lib().tcb_score_workspace_bytes(trie.handle, int(max_users), C.byref(nb)))
    return int(nb.value)


def score_catalog(trie: Trie, table, k: int, table_kind: str = "logprob", user_vec=None,
                  sid_emb=None, sid_weight: float = 1.0, want_lse: bool = True, workspace=None, out=None):
    """Single-pass scoring of every valid SID for a batch of users (tcb_score_catalog;
    ``workspace="static"``: tcb_score_catalog_static, the library's static scratch, with
    ``out`` the caller's output tensors so that nothing is allocated).

    ``table``: float32 [U, L, V] on the device, per-position log-probabilities
    ("logprob") or raw logits ("logits"); ``user_vec`` bfloat16 [U, D] and ``sid_emb``
    bfloat16 [n_distinct, D] (leaf order) for the SID-level term, or both None.
    Returns device tensors: leaf, item (int32 [U, k]), score (float32 [U, k]) and lse
    (float32 [U], or None)."""
    if trie.d_codes is None:
        trie.upload_codes(table.device)
    U = int(table.shape[0])
    if table.dtype != torch.float32 or not table.is_contiguous() or tuple(table.shape[1:]) != (trie.L, trie.V):
        raise ValueError("table must be a contiguous float32 [U, L, V] tensor")
    D = 0
    if user_vec is not None or sid_emb is not None:
        if user_vec is None or sid_emb is None:
            raise ValueError("user_vec and sid_emb go together")
        for t in (user_vec, sid_emb):
            if t.dtype != torch.bfloat16 or not t.is_contiguous():
                raise ValueError("user_vec and sid_emb must be contiguous bfloat16")
        D = int(user_vec.shape[1])
        if tuple(user_vec.shape) != (U, D) or tuple(sid_emb.shape) != (trie.n_distinct, D):
            raise ValueError("user_vec must be [U, D] and sid_emb [n_distinct, D]")
    kind = {"logprob": L.TCB_TABLE_LOGPROB, "logits": L.TCB_TABLE_LOGITS}[table_kind]
    dev = table.device
    if out is None:
        out = {"leaf": torch.empty((U, k), dtype=torch.int32, device=dev),
               "item": torch.empty((U, k), dtype=torch.int32, device=dev),
               "score": torch.empty((U, k), dtype=torch.float32, device=dev),
               "lse": torch.empty(U, dtype=torch.float32, device=dev) if want_lse else None}
    args = (trie.handle, U, _ptr(table), kind, _ptr(user_vec), _ptr(sid_emb), D, float(sid_weight), int(k),
            _ptr(out["leaf"]), _ptr(out["item"]), _ptr(out["score"]), _ptr(out["lse"]))
    if workspace == "static":
        check(lib().tcb_score_catalog_static(*args, _stream()))
    else:
        nb = score_workspace_bytes(trie, U)
        if workspace is None or workspace.numel() < nb:
            workspace = torch.empty(nb, dtype=torch.uint8, device=dev)
        check(lib().tcb_score_catalog(*args, _ptr(workspace), workspace.numel(), _stream()))
    return out
