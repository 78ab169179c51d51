"""ctypes binding of libqkv.so (argument marshalling only).

Every step of the decode path runs in the HIP library; this module only turns
torch tensors into device pointers and the current torch stream into the
stream argument.  Importing it on a host without the built library raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqkv.so")

OK, EINVAL, ECAPACITY, ERANGE, EHIP, ESTATE = 0, -1, -2, -3, -4, -5
POLICY = {"qevict": 0, "h2o": 1, "hqekv": 2}
KIND_K_PER_CHANNEL, KIND_PER_TOKEN, KIND_INT1_NORMAL = 0, 1, 2
DTYPE_BF16, DTYPE_F32 = 0, 1
TIER_EMPTY, TIER_SINK, TIER_RECENT, TIER_FULL, TIER_QUANT, TIER_EVICTED = range(6)
EXPORT = {"tiers": 0, "scores": 1, "ledger": 2, "kcodes": 3, "vcodes": 4, "kparams": 5, "vparams": 6,
          "keys": 7, "values": 8, "routed": 9, "state": 10, "keys_raw": 11, "event": 12, "victims": 13}
# fields of an exported routing-event record (int32 words, then float32 margins)
EVENT_FIELDS = ("tokens", "candidates", "full", "quant", "evicted", "promoted", "demoted", "first_packs",
                "reused", "freed")
EVENT_MARGINS = ("margin_full", "margin_quant", "margin_min")
INFO = {"tokens": 0, "units": 1, "steps": 2, "routes": 3, "splits": 4, "workspace": 5, "list_capacity": 6,
        "layers": 7}
# what each policy's session snapshot holds (qkv_import restores them all)
SNAPSHOT = {0: ("state", "tiers", "scores", "ledger", "routed", "kcodes", "vcodes", "kparams", "vparams",
                "keys", "values"),
            1: ("state", "tiers", "scores", "routed", "keys", "values"),
            2: ("state", "tiers", "scores", "routed", "keys", "values", "kcodes", "vcodes", "kparams", "vparams")}


class QkvError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        detail = f" [{_lib().qkv_hip_error_detail().decode()}]" if code == EHIP else ""
        super().__init__(f"{what}: {_lib().qkv_strerror(code).decode()} ({code}){detail}")


class QkvConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("policy", ctypes.c_int32), ("window", ctypes.c_int32),
        ("omega", ctypes.c_int32), ("n_sink", ctypes.c_int32), ("n_recent", ctypes.c_int32),
        ("k_full", ctypes.c_int32), ("k_quant", ctypes.c_int32), ("ratios", ctypes.c_float * 5),
        ("quant_bits", ctypes.c_int32), ("group", ctypes.c_int32), ("max_ctx", ctypes.c_int32),
        ("n_splits", ctypes.c_int32), ("score_window", ctypes.c_int32), ("chunk", ctypes.c_int32),
        ("n_layers", ctypes.c_int32), ("rope", ctypes.c_int32),
    ]


_LIB = None
_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t


def _lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libqkv.so is not built ({LIB_PATH}); run __graft_entry__.build()")
        # torch carries its own HIP runtime under the same soname; loading it
        # first makes the library bind to that one (a second runtime loaded
        # beside it would find no device)
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        L.qkv_strerror.restype = ctypes.c_char_p
        L.qkv_strerror.argtypes = [ctypes.c_int]
        L.qkv_hip_error_detail.restype = ctypes.c_char_p
        L.qkv_hip_error_detail.argtypes = []
        L.qkv_workspace_bytes.restype = _sz
        L.qkv_workspace_bytes.argtypes = [ctypes.POINTER(QkvConfig)]
        L.qkv_check_config.argtypes = [ctypes.POINTER(QkvConfig)]
        L.qkv_plan_capacities.argtypes = [ctypes.POINTER(QkvConfig), ctypes.c_double, ctypes.c_double, _i32,
                                          ctypes.POINTER(_i32), ctypes.POINTER(_i32)]
        L.qkv_create.argtypes = [ctypes.POINTER(QkvConfig), _vp, _sz, _vp, ctypes.POINTER(_vp)]
        L.qkv_create_static.argtypes = [ctypes.POINTER(QkvConfig), _vp, ctypes.POINTER(_vp)]
        L.qkv_destroy.argtypes = [_vp]
        L.qkv_append.argtypes = [_vp, _vp, _vp, _i32, _vp]
        L.qkv_decode_attend.argtypes = [_vp, _vp, _vp, _vp, _vp]
        L.qkv_append_layer.argtypes = [_vp, _i32, _vp, _vp, _i32, _vp]
        L.qkv_set_rope.argtypes = [_vp, _vp, _i32]
        L.qkv_decode_step_layer.argtypes = [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp]
        L.qkv_decode_attend_layer.argtypes = [_vp, _i32, _vp, _vp, _vp, _vp]
        L.qkv_route.argtypes = [_vp, _vp]
        L.qkv_prefill_score.argtypes = [_vp, _vp, _i32, _vp]
        L.qkv_quantize_window.argtypes = [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp]
        L.qkv_quantize_status.argtypes = [_vp]
        L.qkv_rank_tiers.argtypes = [_vp, _vp, _vp, _i32, _vp, _i32, _vp, _vp]
        L.qkv_export.argtypes = [_vp, _i32, _vp, _sz, _vp]
        L.qkv_import.argtypes = [_vp, _i32, _vp, _sz, _vp]
        L.qkv_export_bytes.restype = _sz
        L.qkv_export_bytes.argtypes = [_vp, _i32]
        L.qkv_info.argtypes = [_vp, _i32, ctypes.POINTER(ctypes.c_int64)]
        L.qkv_status.argtypes = [_vp, _vp]
        L.qkv_profile_start.argtypes = [_vp, _i32, _i32]
        L.qkv_profile_read.argtypes = [_vp, ctypes.POINTER(ctypes.c_float), _i32]
        _LIB = L
    return _LIB


def lib() -> ctypes.CDLL:
    return _lib()


def _check(rc: int, what: str) -> None:
    if rc != OK:
        raise QkvError(rc, what)


def _stream(stream=None) -> int:
    """The raw HIP stream of `stream`, or of the current device's current
    stream (read without building a Stream object: that costs a few
    microseconds per call, which a decode step of a small batch notices)."""
    import torch
    if stream is not None:
        return stream.cuda_stream
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is None:
        return torch.cuda.current_stream().cuda_stream
    return raw(torch.cuda.current_device())


def _ptr(t) -> int:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor required")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor required")
    return t.data_ptr()


def _check_tensor(t, what: str, shape, kind: str) -> None:
    """The C calls take raw pointers: a tensor of the wrong element size or
    shape would be read or written past its end, so both are checked here.
    kind '16': 2-byte elements (bfloat16 bits as bfloat16, int16 or uint16);
    'f32': float32."""
    import torch
    ok16 = (torch.bfloat16, torch.int16, torch.float16) + ((torch.uint16,) if hasattr(torch, "uint16") else ())
    if kind == "16" and t.dtype not in ok16:
        raise ValueError(f"{what}: 2-byte (bfloat16 bits) tensor required, got {t.dtype}")
    if kind == "f32" and t.dtype != torch.float32:
        raise ValueError(f"{what}: float32 tensor required, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(shape)} required, got {tuple(t.shape)}")


def make_config(cfg=None, *, n_splits: int = 0, max_ctx: int | None = None, **kw) -> QkvConfig:
    """Build the C configuration from an object with the workload attributes
    (batch, n_q_heads, ..., prefill, steps) or from keyword arguments."""
    src = dict(kw)
    if cfg is not None:
        for f, _ in QkvConfig._fields_:
            if hasattr(cfg, f) and f not in src:
                src[f] = getattr(cfg, f)
        if max_ctx is None and hasattr(cfg, "prefill"):
            max_ctx = cfg.prefill + cfg.steps
        if "policy" in src and isinstance(src["policy"], str):
            src["policy"] = POLICY[src["policy"]]
    c = QkvConfig()
    for f, _ in QkvConfig._fields_:
        if f == "ratios":
            r = src.get("ratios", (0, 0, 0, 0, 0))
            for i in range(5):
                c.ratios[i] = float(r[i])
        elif f == "max_ctx":
            c.max_ctx = int(max_ctx if max_ctx is not None else src.get("max_ctx", 0))
        elif f == "n_splits":
            c.n_splits = int(n_splits)
        elif f == "policy":
            p = src.get("policy", 0)
            c.policy = POLICY[p] if isinstance(p, str) else int(p)
        elif f == "rope":
            # a workload with a rotary table base has keys before the rotation
            c.rope = int(src.get("rope", 1 if getattr(cfg, "rope_base", 0) else 0))
        else:
            setattr(c, f, int(src.get(f, 32 if f == "group" else (2 if f == "quant_bits" else 0))))
    return c


def plan_capacities(c: QkvConfig, budget_bytes: float, q: float, layers: int = 1) -> tuple[int, int]:
    """(K_f, K_q) that a byte budget buys over `layers` layers of this
    configuration (QEvict Eq.(3)); raises ValueError where the C call
    reports QKV_EINVAL."""
    kf, kq = ctypes.c_int32(), ctypes.c_int32()
    rc = _lib().qkv_plan_capacities(ctypes.byref(c), float(budget_bytes), float(q), int(layers),
                                    ctypes.byref(kf), ctypes.byref(kq))
    if rc != 0:
        raise ValueError(_lib().qkv_strerror(rc).decode())
    return kf.value, kq.value


def workspace_bytes(c: QkvConfig) -> int:
    return int(_lib().qkv_workspace_bytes(ctypes.byref(c)))


STATIC_WORKSPACE_BYTES = 64 << 20


class Cache:
    """One layer's tiered KV cache for a batch of sequences (device state).

    static=True: the cache lives in the library's own per-device array
    (qkv_create_static, no allocation; one such cache per device)."""

    def __init__(self, c: QkvConfig, device="cuda", stream=None, static: bool = False):
        import torch
        self.c = c
        n = workspace_bytes(c)
        if n == 0:
            raise QkvError(_lib().qkv_check_config(ctypes.byref(c)), "qkv config")
        h = _vp()
        if static:
            self.workspace = None
            self._device = torch.device(device if not isinstance(device, str) or ":" in device
                                        else f"{device}:{torch.cuda.current_device()}")
            _check(_lib().qkv_create_static(ctypes.byref(c), _stream(stream), ctypes.byref(h)), "qkv_create_static")
        else:
            self.workspace = torch.empty(n + 256, dtype=torch.uint8, device=device)
            self._device = self.workspace.device
            base = self.workspace.data_ptr()
            self._base = (base + 255) // 256 * 256
            _check(_lib().qkv_create(ctypes.byref(c), self._base, n, _stream(stream), ctypes.byref(h)), "qkv_create")
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            _lib().qkv_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def append(self, k, v, stream=None, layer: int = 0):
        """k, v: bf16 [B, Hkv, n, d] device tensors (of `layer`)."""
        c = self.c
        if k.dim() != 4:
            raise ValueError("k: [B, Hkv, n, d] required")
        n = int(k.shape[2])
        _check_tensor(k, "k", (c.batch, c.n_kv_heads, n, c.head_dim), "16")
        _check_tensor(v, "v", (c.batch, c.n_kv_heads, n, c.head_dim), "16")
        _check(_lib().qkv_append_layer(self.h, int(layer), _ptr(k), _ptr(v), n, _stream(stream)), "qkv_append")

    def decode_attend(self, q, out, mass_out=None, stream=None, layer: int = 0):
        """q: bf16 [B, Hq, d]; out: float32 [B, Hq, d]; mass_out: optional
        float32 [B, Hkv, units] (of `layer`)."""
        c = self.c
        _check_tensor(q, "q", (c.batch, c.n_q_heads, c.head_dim), "16")
        _check_tensor(out, "out", (c.batch, c.n_q_heads, c.head_dim), "f32")
        if mass_out is not None:
            _check_tensor(mass_out, "mass_out", (c.batch, c.n_kv_heads, self.info("units")), "f32")
        _check(_lib().qkv_decode_attend_layer(self.h, int(layer), _ptr(q), _ptr(out), _ptr(mass_out),
                                              _stream(stream)), "qkv_decode_attend")

    def decode_step(self, k, v, q, out, mass_out=None, stream=None, layer: int = 0):
        """append(k, v) of one token, then decode_attend(q, out, mass_out), in
        one call (for the window policy one launch): k, v bf16 [B, Hkv, 1, d]."""
        c = self.c
        _check_tensor(k, "k", (c.batch, c.n_kv_heads, 1, c.head_dim), "16")
        _check_tensor(v, "v", (c.batch, c.n_kv_heads, 1, c.head_dim), "16")
        _check_tensor(q, "q", (c.batch, c.n_q_heads, c.head_dim), "16")
        _check_tensor(out, "out", (c.batch, c.n_q_heads, c.head_dim), "f32")
        if mass_out is not None:
            _check_tensor(mass_out, "mass_out", (c.batch, c.n_kv_heads, self.info("units")), "f32")
        _check(_lib().qkv_decode_step_layer(self.h, int(layer), _ptr(k), _ptr(v), _ptr(q), _ptr(out), _ptr(mass_out),
                                            _stream(stream)), "qkv_decode_step")

    def set_rope(self, table):
        """table: float32 [n_positions, d/2, 2] device tensor (kept by the caller)."""
        import torch
        if table.dtype != torch.float32 or table.dim() != 3 or int(table.shape[1]) * 2 != self.c.head_dim \
                or int(table.shape[2]) != 2:
            raise ValueError("rope table: float32 [n_positions, d/2, 2] required")
        self._rope = table
        _check(_lib().qkv_set_rope(self.h, _ptr(table), int(table.shape[0])), "qkv_set_rope")

    def route(self, stream=None):
        _check(_lib().qkv_route(self.h, _stream(stream)), "qkv_route")

    def prefill_score(self, q, stream=None):
        """q: bf16 [B, n_queries, Hq, d] queries of the last appended positions."""
        c = self.c
        if q.dim() != 4:
            raise ValueError("q: [B, n_queries, Hq, d] required")
        _check_tensor(q, "q", (c.batch, int(q.shape[1]), c.n_q_heads, c.head_dim), "16")
        _check(_lib().qkv_prefill_score(self.h, _ptr(q), int(q.shape[1]), _stream(stream)), "qkv_prefill_score")

    def export(self, what: str, stream=None):
        import torch
        code = EXPORT[what]
        nbytes = int(_lib().qkv_export_bytes(self.h, code))
        if nbytes == 0:
            raise QkvError(EINVAL, f"qkv_export({what})")
        dst = torch.empty(nbytes, dtype=torch.uint8, device=self._device)
        _check(_lib().qkv_export(self.h, code, _ptr(dst), nbytes, _stream(stream)), "qkv_export")
        return dst

    def import_(self, what: str, src, stream=None):
        """Restore one kind of state from a uint8 device tensor that export()
        returned for a cache of the same configuration."""
        import torch
        if src.dtype != torch.uint8 or src.dim() != 1:
            raise ValueError("src: 1-D uint8 tensor (as export returns) required")
        _check(_lib().qkv_import(self.h, EXPORT[what], _ptr(src), int(src.numel()), _stream(stream)),
               f"qkv_import({what})")

    def last_event(self, layer: int = 0) -> list[dict]:
        """The last routing event of each sequence of `layer` (QEvict), or the
        last eviction call / assignment event of each (sequence, KV head)
        (H2O, HqeKV, in b * Hkv + h order): its counters, cut margins and
        victims (window ids or positions; best-ranked first, HqeKV in
        position order).  HqeKV records also name the INT4 and INT1 counts,
        the re-quantized tokens and the margins at all four cuts."""
        import numpy as np
        import torch
        tok = self.c.policy != POLICY["qevict"]
        n_unit = self.c.max_ctx if tok else self.info("units")
        ev = self.export("event").cpu().numpy().view(np.int32).reshape(-1, 16)
        vic = self.export("victims").cpu().numpy().view(np.int32).reshape(-1, n_unit)
        torch.cuda.synchronize()
        if not tok:
            B = self.c.batch
            ev, vic = ev[layer * B:(layer + 1) * B], vic[layer * B:(layer + 1) * B]
        f32 = lambda w: float(w.view(np.float32)[0])
        out = []
        for r_ev, r_vic in zip(ev, vic):
            r = {k: int(r_ev[i]) for i, k in enumerate(EVENT_FIELDS)}
            r.update({k: f32(r_ev[10 + i:11 + i]) for i, k in enumerate(EVENT_MARGINS)})
            if self.c.policy == POLICY["hqekv"]:
                r.update({"requantized": r["first_packs"], "int4": r["reused"], "int1": r["freed"],
                          "int2": r["quant"], "moved": r["demoted"],
                          "margins": [r["margin_full"], r["margin_quant"], f32(r_ev[13:14]), f32(r_ev[14:15])]})
            r["victims"] = [int(u) for u in r_vic[:r["evicted"]]]
            out.append(r)
        return out

    def snapshot(self, stream=None) -> dict:
        """Every kind of state this policy holds, as export() tensors."""
        kinds = SNAPSHOT[self.c.policy] + (("keys_raw",) if self.c.rope else ())
        return {w: self.export(w, stream) for w in kinds}

    def restore(self, snap: dict, stream=None) -> None:
        for w, t in snap.items():
            self.import_(w, t, stream)

    def info(self, what: str) -> int:
        v = ctypes.c_int64()
        _check(_lib().qkv_info(self.h, INFO[what], ctypes.byref(v)), "qkv_info")
        return int(v.value)

    def profile_start(self, n: int, stride: int = 1) -> None:
        """Time every stride-th of the next attention launches, n in all."""
        _check(_lib().qkv_profile_start(self.h, int(n), int(stride)), "qkv_profile_start")

    def profile_read(self, n: int):
        buf = (ctypes.c_float * n)()
        _check(_lib().qkv_profile_read(self.h, buf, int(n)), "qkv_profile_read")
        return list(buf)

    def status(self, stream=None) -> int:
        return int(_lib().qkv_status(self.h, _stream(stream)))


def quantize_window(x, kind: int, bits: int, group: int = 32, stream=None):
    """x: [n_blocks, tokens, d] bf16 (as int16/uint16/bfloat16) or float32 device tensor.
    Returns (codes uint8 [n_blocks, code_bytes], params uint16 [n_blocks, ...])."""
    import torch
    if x.dim() != 3:
        raise ValueError("x: [n_blocks, tokens, d] required")
    n_blocks, tokens, d = (int(s) for s in x.shape)
    if x.dtype != torch.float32:
        _check_tensor(x, "x", (n_blocks, tokens, d), "16")
    dtype = DTYPE_F32 if x.dtype == torch.float32 else DTYPE_BF16
    code_bytes = (tokens * d * bits + 7) // 8
    if kind == KIND_K_PER_CHANNEL:
        n_params = d * ((tokens + group - 1) // group) * 2
    elif kind == KIND_PER_TOKEN:
        n_params = tokens * (d // group) * 2
    else:
        n_params = tokens * 2
    codes = torch.zeros((n_blocks, code_bytes), dtype=torch.uint8, device=x.device)
    params = torch.zeros((n_blocks, n_params), dtype=torch.int16, device=x.device)
    _check(_lib().qkv_quantize_window(_ptr(x), dtype, n_blocks, tokens, d, bits, group, kind, _ptr(codes),
                                      _ptr(params), _stream(stream)), "qkv_quantize_window")
    return codes, params


def quantize_status(stream=None) -> int:
    return int(_lib().qkv_quantize_status(_stream(stream)))


def rank_tiers(score, pos, eligible, counts, stream=None):
    import torch
    n = int(score.numel())
    if score.dtype != torch.float32 or pos.dtype != torch.int32 or eligible.dtype != torch.uint8 \
            or counts.dtype != torch.int32:
        raise ValueError("rank_tiers: score float32, pos int32, eligible uint8, counts int32 required")
    if int(pos.numel()) != n or int(eligible.numel()) != n:
        raise ValueError("rank_tiers: score, pos and eligible must have the same length")
    out = torch.empty(n, dtype=torch.uint8, device=score.device)
    _check(_lib().qkv_rank_tiers(_ptr(score), _ptr(pos), _ptr(eligible), n, _ptr(counts), int(counts.numel()),
                                 _ptr(out), _stream(stream)), "qkv_rank_tiers")
    return out
