"""ctypes binding of the C ABI in ``include/dg.h``.

Argument marshalling only: torch tensors supply device memory and the
stream; every step of the pass runs in the HIP library.  The library must
have been built (``python -m canvas_denoising_moe_amd.build``); loading fails
loudly otherwise -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_uint64, c_void_p
from typing import Optional, Sequence

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libdg.so")

DG_OK, DG_EINVAL, DG_ENOMEM, DG_EHIP, DG_ESTATE, DG_EUNSUPPORTED = 0, -1, -2, -3, -4, -5
DG_F32, DG_BF16 = 0, 1
STATUS_NAMES = {0: "DG_OK", -1: "DG_EINVAL", -2: "DG_ENOMEM", -3: "DG_EHIP", -4: "DG_ESTATE",
                -5: "DG_EUNSUPPORTED"}


class DGConfig(ctypes.Structure):
    _fields_ = [
        ("n_layers", c_int32), ("hidden", c_int32), ("n_heads", c_int32), ("n_kv_heads", c_int32),
        ("head_dim", c_int32), ("n_experts", c_int32), ("top_k", c_int32), ("n_shared", c_int32),
        ("expert_ffn", c_int32), ("vocab", c_int32), ("canvas_len", c_int32), ("window", c_int32),
        ("max_batch", c_int32), ("max_prompt_len", c_int32), ("global_layer_mask", c_uint64),
        ("rope_theta", c_float), ("prope_frac", c_float), ("rms_eps", c_float), ("dtype", c_int32),
        ("has_lm_head", c_int32), ("post_ffn_norm", c_int32), ("expert_format", c_int32),
    ]


LAYER_FIELDS = ("wq", "wk", "wv", "wo", "router", "w_gate", "w_up", "w_down", "sh_gate", "sh_up",
                "sh_down", "norm_in", "norm_pa", "norm_pf", "norm_pf2")


class DGLayerWeights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in LAYER_FIELDS]


class DGError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None

_SIGS = {
    "dg_create": (c_int32, [POINTER(DGConfig), c_int32, c_void_p, POINTER(c_void_p)]),
    "dg_destroy": (c_int32, [c_void_p]),
    "dg_last_error": (c_char_p, [c_void_p]),
    "dg_set_layer_weights": (c_int32, [c_void_p, c_int32, POINTER(DGLayerWeights)]),
    "dg_set_embedding": (c_int32, [c_void_p, c_void_p, c_void_p]),
    "dg_init_weights": (c_int32, [c_void_p, c_void_p, c_void_p, POINTER(DGLayerWeights)]),
    "dg_load_prompt_kv": (c_int32, [c_void_p, c_int32, c_int32, POINTER(c_void_p), POINTER(c_void_p)]),
    "dg_denoise_step": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, POINTER(c_int32), c_void_p, c_void_p]),
    "dg_generate_block": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
    "dg_commit_block": (c_int32, [c_void_p, c_int32, c_void_p]),
    "dg_commit_tokens": (c_int32, [c_void_p, c_int32, c_void_p, c_int32]),
    "dg_eb_step": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_int32, POINTER(ctypes.c_uint32),
                             ctypes.c_uint32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dg_generate_block_eb": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, POINTER(ctypes.c_uint32),
                                       ctypes.c_uint32, c_int32, POINTER(c_int32)]),
    "dg_get_prompt_kv": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
    "dg_get_expert_weight": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
    "dg_forward_hidden": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p]),
    "dg_forward_layers": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p]),
    "dg_set_trace": (c_int32, [c_void_p, c_void_p]),
    "dg_k_argmax_conf": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
    "dg_k_lock_select": (c_int32, [c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                   POINTER(c_int32), c_void_p]),
    "dg_k_eb_rows": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, POINTER(ctypes.c_uint32),
                               ctypes.c_uint32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dg_k_eb_noise": (c_int32, [c_int32, c_int32, c_int32, c_int32, POINTER(ctypes.c_uint32), ctypes.c_uint32,
                                c_void_p, c_void_p]),
    "dg_k_eb_select": (c_int32, [c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_int32, c_int32, c_void_p]),
    "dg_k_moe_route": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_void_p]),
    "dg_k_qkv": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dg_k_canvas_attn": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_int32]),
    "dg_k_moe_ffn": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dg_k_lm_head": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p]),
    "dg_k_lm_argmax": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p]),
    "dg_k_lm_argmax_noalloc": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p]),
    "dg_k_lm_sample": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_int32, POINTER(ctypes.c_uint32),
                                 ctypes.c_uint32, c_void_p, c_void_p, c_void_p]),
    "dg_profile": (c_int32, [c_void_p, c_int32]),
    "dg_profile_read": (c_int32, [c_void_p, c_int32, POINTER(c_int32), POINTER(ctypes.c_double)]),
}

PROF_GATE_UP, PROF_DOWN, PROF_ATTN, PROF_LM_HEAD, PROF_PASS, PROF_COUNT = range(6)
EXPERT_FORMATS = {"native": 0, "mxfp4": 1}
PROF_KEEP = 1 << 30


def lib():
    """Load ``libdg.so`` (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library {LIB_PATH} is missing; build it with "
                               "`python -m canvas_denoising_moe_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def exported_symbols() -> Sequence[str]:
    return tuple(_SIGS)


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(t, dtype=None, name="tensor"):
    """Device address of a contiguous CUDA(HIP) tensor (None -> NULL)."""
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    return c_void_p(t.data_ptr())


def _need(t, n: int, name: str):
    """Element count check ahead of a C call: a tensor shorter than the call
    reads or writes would send a kernel or a copy out of bounds.  None
    passes (optional outputs)."""
    if t is None:
        return
    if not hasattr(t, "numel"):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if int(t.numel()) != int(n):
        raise ValueError(f"{name}: {int(t.numel())} elements, expected {int(n)}")


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream)


def _check(status: int, ctx_handle=None):
    if status != DG_OK:
        msg = lib().dg_last_error(ctx_handle)
        raise DGError(status, msg.decode() if msg else "")


def make_config(model, max_batch: int, max_prompt_len: int) -> DGConfig:
    """dg_config from any object with the architecture fields (e.g. a
    ``ModelConfig``)."""
    c = DGConfig()
    for f in ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "n_experts", "top_k",
              "n_shared", "expert_ffn", "vocab", "canvas_len", "window"):
        setattr(c, f, int(getattr(model, f)))
    c.max_batch = int(max_batch)
    c.max_prompt_len = int(max_prompt_len)
    c.global_layer_mask = int(model.global_layer_mask)
    c.rope_theta = float(model.rope_theta)
    c.prope_frac = float(model.prope_frac)
    c.rms_eps = float(model.rms_eps)
    c.dtype = DG_BF16 if model.dtype == "bf16" else DG_F32
    c.has_lm_head = int(bool(model.has_lm_head))
    c.post_ffn_norm = int(bool(model.post_ffn_norm))
    fmt = getattr(model, "expert_format", "native")
    if fmt not in EXPERT_FORMATS:
        raise ValueError(f"expert_format {fmt!r} is not one of {sorted(EXPERT_FORMATS)}")
    c.expert_format = EXPERT_FORMATS[fmt]
    return c


def _wdtype(model):
    import torch
    return torch.bfloat16 if model.dtype == "bf16" else torch.float32


class Context:
    """One library context (``dg_ctx``) on one device and stream."""

    def __init__(self, model, max_batch: int = 1, max_prompt_len: int = 0, device: int = 0,
                 stream=None):
        import torch
        self.model = model
        self.max_batch = max_batch
        self.device = torch.device("cuda", device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        self.wdtype = _wdtype(model)
        cfg = make_config(model, max_batch, max_prompt_len)
        h = c_void_p()
        _check(lib().dg_create(ctypes.byref(cfg), device, _stream(self.stream), ctypes.byref(h)), None)
        self._h = h
        self._keep = []

    # -- lifetime ------------------------------------------------------------
    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().dg_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    @property
    def handle(self):
        return self._h

    def _c(self, status):
        _check(status, self._h)

    # -- argument sizes (checked before any C call) ------------------------------
    def _batch(self, B: int) -> int:
        B = int(B)
        if not 1 <= B <= self.max_batch:
            raise ValueError(f"batch {B} outside [1, {self.max_batch}]")
        return B

    def _canvas(self, tokens, **named):
        """Batch of ``tokens [B, N]``; every other tensor holds B*N entries."""
        if tokens is None or not hasattr(tokens, "shape") or tokens.dim() != 2:
            raise ValueError("tokens: expected a [batch, canvas_len] tensor")
        N = self.model.canvas_len
        if int(tokens.shape[1]) != N:
            raise ValueError(f"tokens: {int(tokens.shape[1])} positions per canvas, expected {N}")
        B = self._batch(tokens.shape[0])
        for name, buf in named.items():
            _need(buf, B * N, name)
        return B

    def _rows(self, x, width: int, name: str) -> int:
        """Batch of a row-major ``[B*N, width]`` tensor."""
        N = self.model.canvas_len
        n = int(x.numel()) if hasattr(x, "numel") else -1
        if n <= 0 or n % (N * width):
            raise ValueError(f"{name}: {n} elements is not a whole number of canvases of {N} x {width}")
        return self._batch(n // (N * width))

    def _trace_ok(self, B: int):
        t = self._keep[0] if self._keep else None
        if t is not None:
            need = self.model.n_layers * B * self.model.canvas_len * self.model.top_k
            if int(t.numel()) < need:
                raise ValueError(f"route trace holds {int(t.numel())} entries, a batch of {B} records {need}")

    # -- weights and prompt ----------------------------------------------------
    def _layer_sizes(self):
        m = self.model
        H, F, E = m.hidden, m.expert_ffn, m.n_experts
        q, kv = m.n_heads * m.head_dim, m.n_kv_heads * m.head_dim
        return {"wq": H * q, "wk": H * kv, "wv": H * kv, "wo": q * H, "router": H * E,
                "w_gate": E * H * F, "w_up": E * H * F, "w_down": E * F * H,
                "sh_gate": H * F, "sh_up": H * F, "sh_down": F * H,
                "norm_in": H, "norm_pa": H, "norm_pf": H, "norm_pf2": H}

    def _check_layer(self, w: dict):
        for n, size in self._layer_sizes().items():
            _need(w[n], size, n)

    def set_layer_weights(self, layer: int, w: dict):
        self._check_layer(w)
        lw = DGLayerWeights()
        for n in LAYER_FIELDS:
            setattr(lw, n, _ptr(w[n], self.wdtype, n))
        self._c(lib().dg_set_layer_weights(self._h, layer, ctypes.byref(lw)))

    def set_embedding(self, embed, norm_final):
        _need(embed, self.model.vocab * self.model.hidden, "embed")
        _need(norm_final, self.model.hidden, "norm_final")
        self._c(lib().dg_set_embedding(self._h, _ptr(embed, self.wdtype, "embed"),
                                       _ptr(norm_final, self.wdtype, "norm_final")))

    def init_weights(self, embed, norm_final, layers: Sequence[dict]):
        if len(layers) != self.model.n_layers:
            raise ValueError(f"{len(layers)} layers given, the model has {self.model.n_layers}")
        if self.model.has_lm_head:
            _need(embed, self.model.vocab * self.model.hidden, "embed")
            _need(norm_final, self.model.hidden, "norm_final")
        for w in layers:
            self._check_layer(w)
        arr = (DGLayerWeights * len(layers))()
        for i, w in enumerate(layers):
            for n in LAYER_FIELDS:
                setattr(arr[i], n, _ptr(w[n], self.wdtype, n))
        self._c(lib().dg_init_weights(self._h, _ptr(embed, self.wdtype, "embed"),
                                      _ptr(norm_final, self.wdtype, "norm_final"), arr))

    def load_prompt_kv(self, slot: int, prompt_len: int, ks: Sequence, vs: Sequence):
        m = self.model
        if len(ks) != m.n_layers or len(vs) != m.n_layers:
            raise ValueError(f"k and v need one tensor per layer ({m.n_layers})")
        for l in range(m.n_layers):
            n_l = m.kv_len(l, prompt_len) * m.n_kv_heads * m.head_dim
            for name, buf in (("k", ks[l]), ("v", vs[l])):
                if n_l == 0 and (buf is None or buf.numel() == 0):
                    continue
                _need(buf, n_l, f"{name}[{l}]")
        n = len(ks)
        karr = (c_void_p * n)(*[_ptr(k, self.wdtype, "k") if k is not None and k.numel() else None for k in ks])
        varr = (c_void_p * n)(*[_ptr(v, self.wdtype, "v") if v is not None and v.numel() else None for v in vs])
        self._c(lib().dg_load_prompt_kv(self._h, slot, prompt_len, karr, varr))

    # -- the pass --------------------------------------------------------------
    def denoise_step(self, tokens, locked, steps_left: Sequence[int], conf=None, pred=None):
        import torch
        B = self._canvas(tokens, locked=locked, conf=conf, pred=pred)
        if len(steps_left) != B:
            raise ValueError(f"{len(steps_left)} steps_left values for a batch of {B}")
        self._trace_ok(B)
        sl = (c_int32 * B)(*[int(s) for s in steps_left])
        self._c(lib().dg_denoise_step(self._h, B, _ptr(tokens, torch.int32, "tokens"),
                                      _ptr(locked, torch.uint8, "locked"), sl,
                                      _ptr(conf, torch.float32, "conf"), _ptr(pred, torch.int32, "pred")))

    def generate_block(self, tokens, locked, n_steps: int):
        import torch
        self._trace_ok(self._canvas(tokens, locked=locked))
        self._c(lib().dg_generate_block(self._h, tokens.shape[0], n_steps, _ptr(tokens, torch.int32, "tokens"),
                                        _ptr(locked, torch.uint8, "locked")))

    # -- entropy-bounded denoising ------------------------------------------------
    def eb_step(self, tokens, locked, t: int, t_max: int, seeds: Sequence[int], block: int, prev_pred, status,
                entropy=None, sample=None, pred=None):
        """One EB pass (dg_eb_step); ``prev_pred [B, N]`` and ``status [B]``
        (int32, device) carry the per-canvas state between passes."""
        import torch
        B = self._canvas(tokens, locked=locked, prev_pred=prev_pred, entropy=entropy, sample=sample, pred=pred)
        _need(status, B, "status")
        self._trace_ok(B)
        sd = _seeds(seeds, B)
        self._c(lib().dg_eb_step(self._h, B, _ptr(tokens, torch.int32, "tokens"), _ptr(locked, torch.uint8, "locked"),
                                 t, t_max, sd, block, _ptr(prev_pred, torch.int32, "prev_pred"),
                                 _ptr(status, torch.int32, "status"), _ptr(entropy, torch.float32, "entropy"),
                                 _ptr(sample, torch.int32, "sample"), _ptr(pred, torch.int32, "pred")))

    def generate_block_eb(self, tokens, locked, seeds: Sequence[int], block: int = 0, t_max: int = 48):
        """EB passes until every canvas is done (dg_generate_block_eb); returns
        the number of passes after which each canvas was done."""
        import torch
        B = self._canvas(tokens, locked=locked)
        self._trace_ok(B)
        sd = _seeds(seeds, B)
        passes = (c_int32 * B)()
        self._c(lib().dg_generate_block_eb(self._h, B, _ptr(tokens, torch.int32, "tokens"),
                                           _ptr(locked, torch.uint8, "locked"), sd, block, t_max, passes))
        return [int(p) for p in passes]

    def commit_block(self, tokens):
        """Commit the canvases ``tokens [batch, N]`` (int32, device) to the
        prompt KV caches (dg_commit_block): every slot's prompt_len grows by N."""
        import torch
        self._trace_ok(self._canvas(tokens))
        self._c(lib().dg_commit_block(self._h, tokens.shape[0], _ptr(tokens, torch.int32, "tokens")))

    def commit_tokens(self, tokens, n: int):
        """Commit the first ``n`` tokens of each row of ``tokens [batch, N]``
        (dg_commit_tokens): every slot's prompt_len grows by n."""
        import torch
        self._trace_ok(self._canvas(tokens))
        self._c(lib().dg_commit_tokens(self._h, tokens.shape[0], _ptr(tokens, torch.int32, "tokens"), int(n)))

    def prefill(self, tokens):
        """Build the prompt KV from prompt ids ``tokens [batch, L]`` (int32,
        device) by successive commits of N tokens and a shorter last one."""
        import torch
        B, L = tokens.shape
        N = self.model.canvas_len
        with torch.cuda.stream(self.stream):  # the copies are ordered with the commits that read them
            buf = torch.zeros((B, N), dtype=torch.int32, device=tokens.device)
            for p0 in range(0, L, N):
                n = min(N, L - p0)
                buf[:, :n].copy_(tokens[:, p0:p0 + n])
                self.commit_tokens(buf, n)

    def prompt_kv_len(self, slot: int, layer: int) -> int:
        n = c_int32()
        self._c(lib().dg_get_prompt_kv(self._h, slot, layer, None, None, ctypes.byref(n)))
        return n.value

    def get_prompt_kv(self, slot: int, layer: int, k, v):
        """Copy the slot's cache of one layer into ``k, v [len, Hkv, D]``."""
        n = self.prompt_kv_len(slot, layer) * self.model.n_kv_heads * self.model.head_dim
        _need(k, n, "k")
        _need(v, n, "v")
        self._c(lib().dg_get_prompt_kv(self._h, slot, layer, _ptr(k, self.wdtype, "k"),
                                       _ptr(v, self.wdtype, "v"), None))

    def get_expert_weight(self, layer: int, expert: int, which: int, values=None, codes=None, scales=None):
        """One expert matrix as the GEMMs use it (dg_get_expert_weight): which
        0 gate [H, F], 1 up [H, F], 2 down [F, H]; MXFP4 codes / scales too."""
        import torch
        m = self.model
        K, N = (m.expert_ffn, m.hidden) if which == 2 else (m.hidden, m.expert_ffn)
        _need(values, K * N, "values")
        _need(codes, K * N, "codes")
        _need(scales, (K // 32) * N, "scales")
        self._c(lib().dg_get_expert_weight(self._h, layer, expert, which, _ptr(values, self.wdtype, "values"),
                                           _ptr(codes, torch.uint8, "codes"), _ptr(scales, torch.uint8, "scales")))

    def forward_hidden(self, x_in, x_out):
        import torch
        B = self._rows(x_in, self.model.hidden, "x_in")
        _need(x_out, x_in.numel(), "x_out")
        self._trace_ok(B)
        self._c(lib().dg_forward_hidden(self._h, B, _ptr(x_in, torch.float32, "x_in"),
                                        _ptr(x_out, torch.float32, "x_out")))

    def forward_layers(self, first: int, count: int, x_in, x_out):
        import torch
        B = self._rows(x_in, self.model.hidden, "x_in")
        _need(x_out, x_in.numel(), "x_out")
        self._trace_ok(B)
        self._c(lib().dg_forward_layers(self._h, B, first, count, _ptr(x_in, torch.float32, "x_in"),
                                        _ptr(x_out, torch.float32, "x_out")))

    def set_trace(self, route_idx=None):
        import torch
        self._keep = [route_idx]
        self._c(lib().dg_set_trace(self._h, _ptr(route_idx, torch.int32, "route_idx")))

    # -- kernel timing -------------------------------------------------------------
    def profile(self, kernels=(), keep: bool = False):
        """Time the given kernel classes (PROF_* ids; True = all, () = off).
        keep: change the classes without synchronising or clearing the record."""
        if kernels is True:
            mask = (1 << PROF_COUNT) - 1
        else:
            mask = 0
            for k in (kernels or ()):
                mask |= 1 << int(k)
        self._c(lib().dg_profile(self._h, mask | (PROF_KEEP if keep else 0)))

    def profile_read(self, kernel: int):
        """(launches, total milliseconds) recorded for a kernel class."""
        n = c_int32()
        ms = ctypes.c_double()
        self._c(lib().dg_profile_read(self._h, kernel, ctypes.byref(n), ctypes.byref(ms)))
        return n.value, ms.value

    # -- single kernels ----------------------------------------------------------
    def k_qkv(self, layer: int, batch: int, a, q, k, v):
        m = self.model
        M = self._batch(batch) * m.canvas_len
        _need(a, M * m.hidden, "a")
        _need(q, M * m.n_heads * m.head_dim, "q")
        _need(k, M * m.n_kv_heads * m.head_dim, "k")
        _need(v, M * m.n_kv_heads * m.head_dim, "v")
        self._c(lib().dg_k_qkv(self._h, layer, batch, _ptr(a, self.wdtype, "a"), _ptr(q, self.wdtype, "q"),
                               _ptr(k, self.wdtype, "k"), _ptr(v, self.wdtype, "v")))

    def k_canvas_attn(self, layer: int, batch: int, q, k, v, o, canvas_keys: bool = True):
        m = self.model
        M = self._batch(batch) * m.canvas_len
        _need(q, M * m.n_heads * m.head_dim, "q")
        _need(k, M * m.n_kv_heads * m.head_dim, "k")
        _need(v, M * m.n_kv_heads * m.head_dim, "v")
        _need(o, M * m.n_heads * m.head_dim, "o")
        self._c(lib().dg_k_canvas_attn(self._h, layer, batch, _ptr(q, self.wdtype, "q"),
                                       _ptr(k, self.wdtype, "k"), _ptr(v, self.wdtype, "v"),
                                       _ptr(o, self.wdtype, "o"), int(bool(canvas_keys))))

    def k_moe_ffn(self, layer: int, batch: int, f, idx, gates, m):
        import torch
        M = self._batch(batch) * self.model.canvas_len
        _need(f, M * self.model.hidden, "f")
        _need(idx, M * self.model.top_k, "idx")
        _need(gates, M * self.model.top_k, "gates")
        _need(m, M * self.model.hidden, "m")
        self._c(lib().dg_k_moe_ffn(self._h, layer, batch, _ptr(f, self.wdtype, "f"),
                                   _ptr(idx, torch.int32, "idx"), _ptr(gates, torch.float32, "gates"),
                                   _ptr(m, torch.float32, "m")))

    def k_lm_head(self, batch: int, h, logits):
        import torch
        M = self._batch(batch) * self.model.canvas_len
        _need(h, M * self.model.hidden, "h")
        _need(logits, M * self.model.vocab, "logits")
        self._c(lib().dg_k_lm_head(self._h, batch, _ptr(h, self.wdtype, "h"),
                                   _ptr(logits, torch.float32, "logits")))

    def k_lm_argmax(self, batch: int, h, pred, conf):
        import torch
        M = self._batch(batch) * self.model.canvas_len
        _need(h, M * self.model.hidden, "h")
        _need(pred, M, "pred")
        _need(conf, M, "conf")
        self._c(lib().dg_k_lm_argmax(self._h, batch, _ptr(h, self.wdtype, "h"),
                                     _ptr(pred, torch.int32, "pred"), _ptr(conf, torch.float32, "conf")))

    def k_lm_argmax_noalloc(self, batch: int, h, pred, conf):
        """dg_k_lm_argmax with its partials in the library's static scratch
        (allocates nothing; see include/dg.h for the size limit)."""
        import torch
        M = self._batch(batch) * self.model.canvas_len
        _need(h, M * self.model.hidden, "h")
        _need(pred, M, "pred")
        _need(conf, M, "conf")
        self._c(lib().dg_k_lm_argmax_noalloc(self._h, batch, _ptr(h, self.wdtype, "h"),
                                             _ptr(pred, torch.int32, "pred"), _ptr(conf, torch.float32, "conf")))

    def k_lm_sample(self, batch: int, h, t: int, t_max: int, seeds: Sequence[int], block: int, pred, entropy, sample):
        import torch
        M = self._batch(batch) * self.model.canvas_len
        _need(h, M * self.model.hidden, "h")
        for name, buf in (("pred", pred), ("entropy", entropy), ("sample", sample)):
            _need(buf, M, name)
        sd = _seeds(seeds, batch)
        self._c(lib().dg_k_lm_sample(self._h, batch, _ptr(h, self.wdtype, "h"), t, t_max, sd, block,
                                     _ptr(pred, torch.int32, "pred"), _ptr(entropy, torch.float32, "entropy"),
                                     _ptr(sample, torch.int32, "sample")))


def _seeds(seeds: Sequence[int], n: int):
    if len(seeds) != n:
        raise ValueError(f"{n} seeds expected, got {len(seeds)}")
    return (ctypes.c_uint32 * max(1, n))(*[int(x) & 0xFFFFFFFF for x in seeds])


def k_eb_rows(logits, canvas_len: int, t: int, t_max: int, seeds: Sequence[int], block: int, pred, entropy, sample,
              stream=None):
    import torch
    rows, V = logits.shape
    for name, buf in (("pred", pred), ("entropy", entropy), ("sample", sample)):
        _need(buf, rows, name)
    sd = _seeds(seeds, rows // canvas_len)
    _check(lib().dg_k_eb_rows(_ptr(logits, torch.float32, "logits"), rows, V, canvas_len, t, t_max, sd, block,
                              _ptr(pred, torch.int32, "pred"), _ptr(entropy, torch.float32, "entropy"),
                              _ptr(sample, torch.int32, "sample"), _stream(stream)))


def k_eb_noise(rows: int, vocab: int, canvas_len: int, t: int, seeds: Sequence[int], block: int, noise, stream=None):
    import torch
    _need(noise, rows * vocab, "noise")
    sd = _seeds(seeds, rows // canvas_len)
    _check(lib().dg_k_eb_noise(rows, vocab, canvas_len, t, sd, block, _ptr(noise, torch.float32, "noise"),
                               _stream(stream)))


def k_eb_select(entropy, sample, pred, tokens, locked, prev_pred, status, t: int, t_max: int, stream=None):
    import torch
    B, N = tokens.shape
    for name, buf in (("entropy", entropy), ("sample", sample), ("pred", pred), ("locked", locked),
                    ("prev_pred", prev_pred)):
        _need(buf, B * N, name)
    _need(status, B, "status")
    _check(lib().dg_k_eb_select(B, N, _ptr(entropy, torch.float32, "entropy"), _ptr(sample, torch.int32, "sample"),
                                _ptr(pred, torch.int32, "pred"), _ptr(tokens, torch.int32, "tokens"),
                                _ptr(locked, torch.uint8, "locked"), _ptr(prev_pred, torch.int32, "prev_pred"),
                                _ptr(status, torch.int32, "status"), t, t_max, _stream(stream)))


def k_argmax_conf(logits, pred, conf, stream=None):
    import torch
    rows, V = logits.shape
    _need(pred, rows, "pred")
    _need(conf, rows, "conf")
    _check(lib().dg_k_argmax_conf(_ptr(logits, torch.float32, "logits"), rows, V,
                                  _ptr(pred, torch.int32, "pred"), _ptr(conf, torch.float32, "conf"),
                                  _stream(stream)))


def k_lock_select(conf, pred, tokens, locked, steps_left: Sequence[int], stream=None):
    import torch
    B, N = tokens.shape
    for name, buf in (("conf", conf), ("pred", pred), ("locked", locked)):
        _need(buf, B * N, name)
    if len(steps_left) != B:
        raise ValueError(f"{len(steps_left)} steps_left values for a batch of {B}")
    sl = (c_int32 * max(1, B))(*[int(s) for s in steps_left])
    _check(lib().dg_k_lock_select(B, N, _ptr(conf, torch.float32, "conf"), _ptr(pred, torch.int32, "pred"),
                                  _ptr(tokens, torch.int32, "tokens"), _ptr(locked, torch.uint8, "locked"),
                                  sl, _stream(stream)))


def k_moe_route(logits, top_k: int, idx, gates, counts=None, offsets=None, perm=None, stream=None):
    import torch
    rows, E = logits.shape
    _need(idx, rows * top_k, "idx")
    _need(gates, rows * top_k, "gates")
    _need(counts, E, "counts")
    _need(offsets, E + 2, "offsets")
    _need(perm, rows * top_k, "perm")
    _check(lib().dg_k_moe_route(_ptr(logits, torch.float32, "logits"), rows, E, top_k,
                                _ptr(idx, torch.int32, "idx"), _ptr(gates, torch.float32, "gates"),
                                _ptr(counts, torch.int32, "counts"), _ptr(offsets, torch.int32, "offsets"),
                                _ptr(perm, torch.int32, "perm"), _stream(stream)))
