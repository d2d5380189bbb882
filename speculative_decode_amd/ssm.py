"""Python face of the C ABI: a cache object and prefill / verify / commit calls.

Torch supplies device memory and the current stream; every computation happens in
the HIP library behind `mil_ssm_*`.  Names follow the layer of "The Mamba in the
Llama" (x from V, B from K, C from Q, step size dt, decay rate A, skip D) and the
speculative protocol of the QbitAI article's walkthrough (K drafts, accepted length j).
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib as L

_DTYPES = {torch.float32: L.MIL_F32, torch.bfloat16: L.MIL_BF16}
_TORCH = {L.MIL_F32: torch.float32, L.MIL_BF16: torch.bfloat16}


def _dtype_code(dtype) -> int:
    if isinstance(dtype, str):
        return {"f32": L.MIL_F32, "bf16": L.MIL_BF16}[dtype]
    if isinstance(dtype, torch.dtype):
        return _DTYPES[dtype]
    return int(dtype)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t) -> ctypes.c_void_p | None:
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def cache_layout(batch, H, P, N, G, k_max, dtype) -> L.Layout:
    d = L.Dims(batch, H, P, N, G)
    lay = L.Layout()
    L.check(L.lib().mil_ssm_cache_layout(ctypes.byref(d), k_max, _dtype_code(dtype), ctypes.byref(lay)),
            "mil_ssm_cache_layout")
    return lay


def supported(batch, H, P, N, G, dtype) -> bool:
    d = L.Dims(batch, H, P, N, G)
    return L.lib().mil_ssm_supported(ctypes.byref(d), _dtype_code(dtype)) == L.MIL_OK


class SSMCache:
    """Per-layer state cache for `batch` sequence slots (fp32 state [batch][H][N][P],
    head blocks 256-B aligned) plus the pending accepted-token rows and counters."""

    def __init__(self, batch, H, P, N, G, k_max, dtype, device="cuda", attach_to=None):
        """attach_to: a uint8 device tensor that already holds a cache of this shape (for
        instance a byte copy of another SSMCache's `buffer`), described with
        mil_ssm_cache_attach instead of being set up from zeros; it must be 256-byte
        aligned and at least `layout.bytes` long."""
        self.batch, self.H, self.P, self.N, self.G, self.k_max = batch, H, P, N, G, k_max
        self.dtype_code = _dtype_code(dtype)
        self.torch_dtype = _TORCH[self.dtype_code]
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.dims = L.Dims(batch, H, P, N, G)
        self.layout = cache_layout(batch, H, P, N, G, k_max, self.dtype_code)
        nbytes = self.layout.bytes
        self.desc = L.CacheDesc()
        if attach_to is not None:
            if attach_to.dtype != torch.uint8 or attach_to.device != self.device or attach_to.numel() < nbytes:
                raise ValueError(f"attach_to must be a uint8 tensor of at least {nbytes} bytes on {self.device}")
            self._raw = attach_to
            self.buffer = attach_to[:nbytes]
            L.check(L.lib().mil_ssm_cache_attach(ctypes.byref(self.desc), ctypes.byref(self.dims), k_max,
                                                self.dtype_code, _ptr(self.buffer), nbytes),
                    "mil_ssm_cache_attach")
            return
        # over-allocate so that the carved base is 256-B aligned whatever the allocator does
        self._raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        off = (-self._raw.data_ptr()) % 256
        self.buffer = self._raw[off:off + nbytes]
        L.check(L.lib().mil_ssm_cache_init(ctypes.byref(self.desc), ctypes.byref(self.dims), k_max,
                                          self.dtype_code, _ptr(self.buffer), nbytes, _stream(self.device)),
                "mil_ssm_cache_init")

    # ---- views into the cache buffer (for inspection and tests) ----
    def state(self) -> torch.Tensor:
        """fp32 view [batch][H][N][P] of the stored state (before pending rows are folded)."""
        lay = self.layout
        stride = lay.state_head_stride // 4
        flat = self.buffer[lay.state_off:lay.state_off + self.batch * self.H * lay.state_head_stride]
        f = flat.view(torch.float32)
        return f.as_strided((self.batch, self.H, self.N, self.P),
                            (self.H * stride, stride, self.P, 1))

    def _i32(self, off) -> torch.Tensor:
        return self.buffer[off:off + 4 * self.batch].view(torch.int32)

    def pos(self) -> torch.Tensor:
        return self._i32(self.layout.pos_off)

    def pending(self) -> torch.Tensor:
        return self._i32(self.layout.pending_off)

    def append(self) -> torch.Tensor:
        """Per slot, the pending row at which the next commit puts its first accepted row
        (0 when the verify before it wrote the folded state back)."""
        return self._i32(self.layout.append_off)

    def err(self) -> torch.Tensor:
        return self._i32(self.layout.err_off)

    SCAN_ROW, SCAN_EPOCH = 68, 64

    def scan_words(self) -> torch.Tensor:
        """int32 view [batch][H][8][68] of the single-launch prefill's handoff rows: 64 chunk
        flags ((epoch << 2) | kind), the row's epoch, padding."""
        off = self.layout.scan_off
        n = self.batch * self.H * 8 * self.SCAN_ROW
        return self.buffer[off:off + 4 * n].view(torch.int32).view(self.batch, self.H, 8, self.SCAN_ROW)

    def prefill_kernels(self, nseq, L_tokens, chunk=256) -> int:
        """Bit mask of the traceable kernels a prefill of these sizes launches (mil_ssm_prefill_kernels)."""
        return int(L.lib().mil_ssm_prefill_kernels(ctypes.byref(self.desc), nseq, L_tokens, chunk))

    def phase(self) -> int:
        return L.lib().mil_ssm_cache_phase(ctypes.byref(self.desc))

    def status(self, clear: bool = False) -> int:
        """Synchronise and return the first slot with a device-side error, or -1."""
        bad = ctypes.c_int32(-1)
        st = L.lib().mil_ssm_cache_status(ctypes.byref(self.desc), ctypes.byref(bad), int(clear),
                                          _stream(self.device))
        if st not in (L.MIL_OK, L.MIL_E_INVALID):
            L.check(st, "mil_ssm_cache_status")
        return bad.value

    def _check_tokens(self, what, *ts):
        for t in ts:
            if t is None:
                continue
            if t.dtype != self.torch_dtype:
                raise TypeError(f"{what}: expected {self.torch_dtype}, got {t.dtype}")
            if not t.is_contiguous() or t.device != self.device:
                raise ValueError(f"{what}: tensors must be contiguous and on {self.device}")

    def _check_shapes(self, what, nseq, T, x, B, C, dt, A, D, y):
        """The ABI takes bare pointers, so sizes are checked here before any call."""
        want = {"x": (nseq, T, self.H, self.P), "B": (nseq, T, self.G, self.N), "C": (nseq, T, self.G, self.N),
                "dt": (nseq, T, self.H), "A": (self.H,), "D": (self.H,), "y": (nseq, T, self.H, self.P)}
        for name, t in (("x", x), ("B", B), ("C", C), ("dt", dt), ("A", A), ("D", D), ("y", y)):
            if t is None:
                continue
            if tuple(t.shape) != want[name]:
                raise ValueError(f"{what}: {name} has shape {tuple(t.shape)}, expected {want[name]}")
            if name in ("A", "D", "y") and (t.dtype != torch.float32 or not t.is_contiguous()
                                            or t.device != self.device):
                raise TypeError(f"{what}: {name} must be a contiguous float32 tensor on {self.device}")

    # ---- the three calls ----
    def workspace_bytes(self, nseq, L_tokens, chunk=256) -> int:
        return L.lib().mil_ssm_prefill_workspace_bytes(ctypes.byref(self.dims), nseq, L_tokens, chunk)

    def prefill(self, x, B, C, dt, A, D, slot0=0, y=None, chunk=256, cont=False, ws=None, want_y=True):
        """Scan x [nseq][L][H][P], B/C [nseq][L][G][N], dt [nseq][L][H] into slots
        [slot0, slot0+nseq).  Returns y [nseq][L][H][P] fp32 (or None when want_y is False)."""
        nseq, Lt = x.shape[0], x.shape[1]
        self._check_tokens("prefill", x, B, C, dt)
        if want_y and y is None:
            y = torch.empty((nseq, Lt, self.H, self.P), dtype=torch.float32, device=self.device)
        self._check_shapes("prefill", nseq, Lt, x, B, C, dt, A, D, y if want_y else None)
        if not 0 <= slot0 <= self.batch - nseq:
            raise ValueError("prefill: slots out of range")
        need = self.workspace_bytes(nseq, Lt, chunk)
        if need == 0:
            raise L.MilError(L.MIL_E_INVALID, "mil_ssm_prefill_workspace_bytes")
        if ws is None or ws.numel() < need:
            ws = torch.empty(need + 256, dtype=torch.uint8, device=self.device)
        off = (-ws.data_ptr()) % 256
        wsv = ws[off:]
        st = L.lib().mil_ssm_prefill(ctypes.byref(self.desc), slot0, nseq, Lt, chunk, _ptr(x), _ptr(B), _ptr(C),
                                     _ptr(dt), _ptr(A), _ptr(D), _ptr(y if want_y else None), _ptr(wsv),
                                     wsv.numel(), L.MIL_PREFILL_CONTINUE if cont else 0, _stream(self.device))
        L.check(st, "mil_ssm_prefill")
        return y

    def verify(self, x, B, C, dt, A, D, y=None):
        """Outputs y [batch][K][H][P] for K drafts from each slot's logical state."""
        K = x.shape[1]
        self._check_tokens("verify", x, B, C, dt)
        if y is None:
            y = torch.empty((self.batch, K, self.H, self.P), dtype=torch.float32, device=self.device)
        self._check_shapes("verify", self.batch, K, x, B, C, dt, A, D, y)
        st = L.lib().mil_ssm_verify(ctypes.byref(self.desc), K, _ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(A),
                                    _ptr(D), _ptr(y), _stream(self.device))
        L.check(st, "mil_ssm_verify")
        return y

    def commit(self, accepted, x, B, dt, A=None, D=None, materialize=False):
        """Keep the first accepted[b] drafts of each slot (device int32 [batch])."""
        K = x.shape[1]
        self._check_tokens("commit", x, B, dt)
        if accepted.dtype != torch.int32 or accepted.device != self.device:
            raise TypeError("accepted must be an int32 tensor on the cache's device")
        if tuple(accepted.shape) != (self.batch,) or not accepted.is_contiguous():
            raise ValueError(f"commit: accepted must have shape ({self.batch},)")
        self._check_shapes("commit", self.batch, K, x, B, None, dt, A, D, None)
        st = L.lib().mil_ssm_commit(ctypes.byref(self.desc), K, _ptr(accepted), _ptr(x), _ptr(B), _ptr(dt),
                                    _ptr(A), _ptr(D), L.MIL_COMMIT_MATERIALIZE if materialize else 0,
                                    _stream(self.device))
        L.check(st, "mil_ssm_commit")

    def _check_int_rows(self, what, t, shape):
        if t.dtype != torch.int32 or t.device != self.device:
            raise TypeError(f"{what} must be an int32 tensor on the cache's device")
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{what} must be a contiguous tensor of shape {shape}")

    def verify_tree(self, parent, x, B, C, dt, A, D, y=None):
        """Outputs y [batch][K][H][P] for a tree of K drafts per slot: parent [batch][K]
        int32 (-1..k-1, -1 = the committed state); draft k's output runs over its root path."""
        K = x.shape[1]
        self._check_tokens("verify_tree", x, B, C, dt)
        self._check_int_rows("verify_tree: parent", parent, (self.batch, K))
        if y is None:
            y = torch.empty((self.batch, K, self.H, self.P), dtype=torch.float32, device=self.device)
        self._check_shapes("verify_tree", self.batch, K, x, B, C, dt, A, D, y)
        st = L.lib().mil_ssm_verify_tree(ctypes.byref(self.desc), K, _ptr(parent), _ptr(x), _ptr(B), _ptr(C),
                                         _ptr(dt), _ptr(A), _ptr(D), _ptr(y), _stream(self.device))
        L.check(st, "mil_ssm_verify_tree")
        return y

    def commit_tree(self, parent, accepted_node, x, B, dt, A=None, D=None, materialize=False):
        """Keep the root path of accepted_node[b] (device int32 [batch], -1..K-1; -1 keeps
        nothing) of each slot's draft tree."""
        K = x.shape[1]
        self._check_tokens("commit_tree", x, B, dt)
        self._check_int_rows("commit_tree: parent", parent, (self.batch, K))
        self._check_int_rows("commit_tree: accepted_node", accepted_node, (self.batch,))
        self._check_shapes("commit_tree", self.batch, K, x, B, None, dt, A, D, None)
        st = L.lib().mil_ssm_commit_tree(ctypes.byref(self.desc), K, _ptr(parent), _ptr(accepted_node), _ptr(x),
                                         _ptr(B), _ptr(dt), _ptr(A), _ptr(D),
                                         L.MIL_COMMIT_MATERIALIZE if materialize else 0, _stream(self.device))
        L.check(st, "mil_ssm_commit_tree")

    def greedy_workspace_bytes(self, K: int, vocab: int) -> int:
        return int(L.lib().mil_ssm_greedy_workspace_bytes(ctypes.byref(self.dims), K, vocab))

    def commit_greedy(self, draft_tokens, logits, x, B, dt, A=None, D=None, materialize=False,
                      want_tokens=False, accepted=None, ws=None, noalloc=False):
        """Greedy acceptance on the device, then the commit: draft_tokens [batch][K] int32,
        logits [batch][K][vocab] (float32 or bfloat16).  Returns (accepted [batch] int32,
        verifier_tokens [batch][K] int32 or None).  noalloc=True calls
        mil_ssm_commit_greedy_noalloc (the library's own scratch, no workspace; `ws` unused)."""
        K = x.shape[1]
        self._check_tokens("commit_greedy", x, B, dt)
        self._check_shapes("commit_greedy", self.batch, K, x, B, None, dt, A, D, None)
        if draft_tokens.dtype != torch.int32 or draft_tokens.device != self.device:
            raise TypeError("draft_tokens must be an int32 tensor on the cache's device")
        if tuple(draft_tokens.shape) != (self.batch, K) or not draft_tokens.is_contiguous():
            raise ValueError(f"commit_greedy: draft_tokens must have shape ({self.batch}, {K})")
        if logits.device != self.device or logits.dim() != 3 or not logits.is_contiguous():
            raise ValueError("commit_greedy: logits must be a contiguous [batch][K][vocab] tensor on the device")
        if tuple(logits.shape[:2]) != (self.batch, K):
            raise ValueError(f"commit_greedy: logits must start with ({self.batch}, {K})")
        ldt = {torch.float32: L.MIL_F32, torch.bfloat16: L.MIL_BF16}.get(logits.dtype)
        if ldt is None:
            raise TypeError("logits must be float32 or bfloat16")
        vocab = int(logits.shape[2])
        if accepted is None:
            accepted = torch.empty(self.batch, dtype=torch.int32, device=self.device)
        tokens = torch.empty((self.batch, K), dtype=torch.int32, device=self.device) if want_tokens else None
        if noalloc:
            st = L.lib().mil_ssm_commit_greedy_noalloc(ctypes.byref(self.desc), K, _ptr(draft_tokens), _ptr(logits),
                                                       vocab, ldt, _ptr(accepted), _ptr(tokens), _ptr(x), _ptr(B),
                                                       _ptr(dt), _ptr(A), _ptr(D),
                                                       L.MIL_COMMIT_MATERIALIZE if materialize else 0,
                                                       _stream(self.device))
            L.check(st, "mil_ssm_commit_greedy_noalloc")
            return accepted, tokens
        need = self.greedy_workspace_bytes(K, vocab)
        if ws is None:
            ws = torch.empty(need + 256, dtype=torch.uint8, device=self.device)
        wp = (ws.data_ptr() + 255) // 256 * 256
        st = L.lib().mil_ssm_commit_greedy(ctypes.byref(self.desc), K, _ptr(draft_tokens), _ptr(logits), vocab, ldt,
                                           _ptr(accepted), _ptr(tokens), _ptr(x), _ptr(B), _ptr(dt), _ptr(A),
                                           _ptr(D), ctypes.c_void_p(wp), ws.numel() - (wp - ws.data_ptr()),
                                           L.MIL_COMMIT_MATERIALIZE if materialize else 0, _stream(self.device))
        L.check(st, "mil_ssm_commit_greedy")
        return accepted, tokens


def commit_layers(caches, accepted, xs, Bs, dts):
    """One round's commit for several layers' caches at once: caches[l] keeps the first
    accepted[b] drafts of slot b from xs[l], Bs[l], dts[l] (the draft buffers given to its
    verify).  The same as caches[l].commit(accepted, xs[l], Bs[l], dts[l]) for every l, in
    one launch per MIL_COMMIT_LAYERS_MAX layers."""
    n = len(caches)
    if n < 1 or not (len(xs) == len(Bs) == len(dts) == n):
        raise ValueError("commit_layers: one x, B and dt per cache")
    c0 = caches[0]
    K = xs[0].shape[1]
    for c, x, B, dt in zip(caches, xs, Bs, dts):
        c._check_tokens("commit_layers", x, B, dt)
        c._check_shapes("commit_layers", c.batch, K, x, B, None, dt, None, None, None)
    if accepted.dtype != torch.int32 or accepted.device != c0.device:
        raise TypeError("accepted must be an int32 tensor on the caches' device")
    if tuple(accepted.shape) != (c0.batch,) or not accepted.is_contiguous():
        raise ValueError(f"commit_layers: accepted must have shape ({c0.batch},)")
    descs = (ctypes.POINTER(L.CacheDesc) * n)(*[ctypes.pointer(c.desc) for c in caches])
    arr = lambda ts: (ctypes.c_void_p * n)(*[_ptr(t) for t in ts])  # noqa: E731
    st = L.lib().mil_ssm_commit_layers(descs, n, K, _ptr(accepted), arr(xs), arr(Bs), arr(dts), _stream(c0.device))
    L.check(st, "mil_ssm_commit_layers")


def project_workspace_bytes(H, P, N, G, T, d_model) -> int:
    d = L.Dims(1, H, P, N, G)
    return int(L.lib().mil_ssm_project_workspace_bytes(ctypes.byref(d), T, d_model))


def project(u, w_x, w_B, w_C, w_dt, H, P, N, G, dt_bias=None, out_dtype=torch.bfloat16, out=None, ws=None):
    """Input projections of the layer (mil_ssm_project): u [..., d_model] bf16 and the four
    bf16 weight blocks w_x [H*P][d], w_B and w_C [G*N][d], w_dt [H][d].  Returns
    (x [..., H, P], B [..., G, N], C [..., G, N], dt [..., H]) in out_dtype, the layouts
    verify and prefill take; `out` may supply those four tensors."""
    lead = tuple(u.shape[:-1])
    d_model = int(u.shape[-1])
    T = 1
    for s in lead:
        T *= int(s)
    dev = u.device
    want = {"w_x": (w_x, (H * P, d_model)), "w_B": (w_B, (G * N, d_model)), "w_C": (w_C, (G * N, d_model)),
            "w_dt": (w_dt, (H, d_model))}
    for name, t in [("u", u)] + [(k, v[0]) for k, v in want.items()]:
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.device != dev:
            raise TypeError(f"project: {name} must be a contiguous bfloat16 tensor on {dev}")
    for name, (t, shape) in want.items():
        if tuple(t.shape) != shape:
            raise ValueError(f"project: {name} has shape {tuple(t.shape)}, expected {shape}")
    if dt_bias is not None and (dt_bias.dtype != torch.float32 or tuple(dt_bias.shape) != (H,)
                                or not dt_bias.is_contiguous() or dt_bias.device != dev):
        raise ValueError(f"project: dt_bias must be a contiguous float32 tensor of shape ({H},) on {dev}")
    code = _dtype_code(out_dtype)
    tdt = _TORCH[code]
    shapes = [lead + (H, P), lead + (G, N), lead + (G, N), lead + (H,)]
    if out is None:
        out = [torch.empty(s, dtype=tdt, device=dev) for s in shapes]
    for t, s in zip(out, shapes):
        if tuple(t.shape) != s or t.dtype != tdt or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"project: an output tensor does not have shape {s} and dtype {tdt}")
    dims = L.Dims(1, H, P, N, G)
    need = int(L.lib().mil_ssm_project_workspace_bytes(ctypes.byref(dims), T, d_model))
    wp, wbytes = None, 0
    if need > 0:
        if ws is None:
            ws = torch.empty(need + 256, dtype=torch.uint8, device=dev)
        wp = ctypes.c_void_p((ws.data_ptr() + 255) // 256 * 256)
        wbytes = ws.numel() - (wp.value - ws.data_ptr())
    st = L.lib().mil_ssm_project(ctypes.byref(dims), T, d_model, _ptr(u), _ptr(w_x), _ptr(w_B), _ptr(w_C),
                                 _ptr(w_dt), _ptr(dt_bias), code, _ptr(out[0]), _ptr(out[1]), _ptr(out[2]),
                                 _ptr(out[3]), wp, wbytes, _stream(dev))
    L.check(st, "mil_ssm_project")
    return tuple(out)
