"""Thin Python binding of ``libstca.so`` (C ABI in ``include/stca.h``).

Argument marshalling only: every step of the forward runs in the HIP
library.  PyTorch supplies device memory and the current HIP stream.  There
is no fallback: if the library is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libstca.so")

# enums (mirror include/stca.h)
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
SCORE = {"softmax": 0, "relu": 1}
QMODE = {"fusion": 0, "linear": 1, "hyformer": 2}
PATH = {"staged": 0, "fused": 1}
ENCODER = {"swiglu": 0, "longer": 1}
FLAG_KV_LN, FLAG_Z_LN, FLAG_DEDUP = 1, 2, 4
DEV_BAD_HIST_OFFSETS, DEV_BAD_TGT_OFFSETS, DEV_BAD_ID = 1, 2, 4

EXPORTS = ("stca_workspace_size", "stca_forward", "stca_attention_workspace_size",
           "stca_attention", "stca_backward_workspace_size", "stca_backward",
           "stca_peak_mfma_bf16", "stca_peak_hbm_read", "stca_status_string", "stca_last_error",
           "stca_version", "stca_forward_noalloc", "stca_forward_for_backward")

NOALLOC_SCRATCH_BYTES = 128 << 20   # STCA_NOALLOC_SCRATCH_BYTES

_vp = C.c_void_p


class Config(C.Structure):
    _fields_ = [("B", C.c_int32), ("d", C.c_int32), ("H", C.c_int32), ("hidden", C.c_int32),
                ("M", C.c_int32), ("table_rows", C.c_int64), ("dtype", C.c_int32),
                ("score", C.c_int32), ("qmode", C.c_int32), ("path", C.c_int32),
                ("flags", C.c_int32), ("chunk_keys", C.c_int32), ("n_ns", C.c_int32),
                ("q_hidden", C.c_int32), ("head_map", C.POINTER(C.c_int32)), ("encoder", C.c_int32),
                ("l_short", C.c_int32)]


class Batch(C.Structure):
    _fields_ = [("hist_offsets", _vp), ("hist_ids", _vp), ("tgt_offsets", _vp), ("tgt_ids", _vp),
                ("q0", _vp), ("table", _vp), ("n_hist", C.c_int64), ("n_tgt", C.c_int64),
                ("max_tgt_per_user", C.c_int32), ("ns_feats", _vp), ("key_mask", _vp),
                ("score_bias", _vp)]


class Ffn(C.Structure):
    _fields_ = [("w1", _vp), ("w3", _vp), ("w2", _vp), ("ln_g", _vp), ("ln_b", _vp)]


class Layer(C.Structure):
    _fields_ = [("kv", Ffn), ("q", Ffn), ("wk", _vp), ("wv", _vp), ("wq", _vp), ("wo", _vp),
                ("wc", _vp), ("r", _vp), ("boost_w1", _vp), ("boost_w3", _vp), ("boost_w2", _vp),
                ("enc_wq", _vp), ("enc_wk", _vp), ("enc_wv", _vp), ("enc_wo", _vp)]


class Weights(C.Structure):
    _fields_ = [("layers", C.POINTER(Layer)), ("z", Ffn), ("wz", _vp), ("qgen_w1", _vp), ("qgen_w3", _vp),
                ("qgen_w2", _vp)]


class Outputs(C.Structure):
    _fields_ = [("z", _vp), ("o_layers", _vp), ("attn", _vp), ("active", _vp), ("q_dump", _vp),
                ("kv_dump", _vp), ("x_dump", _vp), ("dev_status", _vp),
                ("stage_events", C.POINTER(_vp)), ("n_stage_events", C.c_int32), ("lse", _vp),
                ("clock_probe", _vp)]


class FfnGrad(C.Structure):
    _fields_ = [("w1", _vp), ("w3", _vp), ("w2", _vp), ("ln_g", _vp), ("ln_b", _vp)]


class LayerGrad(C.Structure):
    _fields_ = [("kv", FfnGrad), ("q", FfnGrad), ("wk", _vp), ("wv", _vp), ("wq", _vp), ("wo", _vp),
                ("wc", _vp)]


class Grads(C.Structure):
    _fields_ = [("layers", C.POINTER(LayerGrad)), ("z", FfnGrad), ("wz", _vp), ("table", _vp),
                ("d_hist", _vp), ("d_tgt", _vp), ("z_out", _vp), ("dq_dump", _vp), ("da_dump", _vp),
                ("dkv_dump", _vp), ("dev_status", _vp), ("stage_events", C.POINTER(_vp)),
                ("n_stage_events", C.c_int32), ("saved_forward", C.c_int32)]


class AttnArgs(C.Structure):
    _fields_ = [("B", C.c_int32), ("d", C.c_int32), ("H", C.c_int32), ("dtype", C.c_int32),
                ("score", C.c_int32), ("chunk_keys", C.c_int32), ("hist_offsets", _vp),
                ("tgt_offsets", _vp), ("n_hist", C.c_int64), ("n_tgt", C.c_int64),
                ("max_tgt_per_user", C.c_int32), ("q", _vp), ("k", _vp), ("v", _vp),
                ("attn", _vp), ("active", _vp), ("dev_status", _vp), ("key_mask", _vp),
                ("head_map", C.POINTER(C.c_int32)), ("score_bias", _vp)]


_LIB = None


class StcaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{status_string(code)}: {msg}")
        self.code = code


def load() -> C.CDLL:
    """Load libstca.so from the package directory (or the path in the
    STCA_LIBRARY environment variable); raises if it is not built."""
    global _LIB
    if _LIB is None:
        path = os.environ.get("STCA_LIBRARY", LIB_PATH)
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m recsys_ultra_long_amd.build`")
        lib = C.CDLL(path)
        lib.stca_workspace_size.argtypes = [C.POINTER(Config), C.POINTER(Batch), C.POINTER(C.c_size_t)]
        lib.stca_forward.argtypes = [C.POINTER(Config), C.POINTER(Batch), C.POINTER(Weights),
                                     C.POINTER(Outputs), _vp, C.c_size_t, _vp]
        lib.stca_forward_noalloc.argtypes = [C.POINTER(Config), C.POINTER(Batch), C.POINTER(Weights),
                                             C.POINTER(Outputs), _vp]
        lib.stca_attention_workspace_size.argtypes = [C.POINTER(AttnArgs), C.POINTER(C.c_size_t)]
        lib.stca_attention.argtypes = [C.POINTER(AttnArgs), _vp, C.c_size_t, _vp]
        lib.stca_backward_workspace_size.argtypes = [C.POINTER(Config), C.POINTER(Batch),
                                                     C.POINTER(C.c_size_t)]
        lib.stca_backward.argtypes = [C.POINTER(Config), C.POINTER(Batch), C.POINTER(Weights), _vp,
                                      C.POINTER(Grads), _vp, C.c_size_t, _vp]
        lib.stca_forward_for_backward.argtypes = [C.POINTER(Config), C.POINTER(Batch), C.POINTER(Weights), _vp,
                                                  _vp, _vp, C.c_size_t, _vp]
        lib.stca_peak_mfma_bf16.argtypes = [C.c_int32, C.c_int32, _vp, _vp, _vp]
        lib.stca_peak_hbm_read.argtypes = [_vp, C.c_int64, C.c_int32, _vp, _vp]
        lib.stca_status_string.restype = C.c_char_p
        lib.stca_status_string.argtypes = [C.c_int]
        lib.stca_last_error.restype = C.c_char_p
        lib.stca_version.restype = C.c_int
        for f in ("stca_workspace_size", "stca_forward", "stca_attention_workspace_size",
                  "stca_attention", "stca_backward_workspace_size", "stca_backward", "stca_peak_mfma_bf16",
                  "stca_peak_hbm_read", "stca_forward_noalloc", "stca_forward_for_backward"):
            getattr(lib, f).restype = C.c_int
        _LIB = lib
    return _LIB


def status_string(code: int) -> str:
    return load().stca_status_string(code).decode()


def last_error() -> str:
    return load().stca_last_error().decode()


def _check(code: int):
    if code != OK:
        raise StcaError(code, last_error())


# ---------------------------------------------------------------- device data
def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


@dataclass
class DeviceProblem:
    """A problem's arrays on the GPU (torch tensors; bf16 kept as raw int16 bits)."""
    cfg: Config
    hist_offsets: object
    hist_ids: object
    tgt_offsets: object
    tgt_ids: object
    q0: object
    table: object
    layers: list          # per layer dict of device tensors (same keys as inputs.Problem)
    z: Optional[dict]
    wz: object
    n_hist: int
    n_tgt: int
    max_tgt: int
    ns: object = None     # HyFormer: non-sequence tokens [B, n_ns, d]
    qgen: Optional[dict] = None
    key_mask: object = None   # Cross-Mask: [n_hist] visibility bits (int32 view of uint32)
    head_map: object = None   # Cross-Mask: ctypes int32 array [H] (kept alive here)
    score_bias: object = None  # context-similarity score bias [n_hist, H] fp32


def _dev(a, device):
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def upload(p, device="cuda", table=None, path="staged", chunk_keys=0, dedup=False) -> DeviceProblem:
    """Copy an ``inputs.Problem`` to the device.  ``table`` may be a device
    tensor already holding the embedding table (avoids a second copy)."""
    import torch
    sp = p.spec
    flags = (FLAG_KV_LN if sp.kv_ln else 0) | (FLAG_Z_LN if sp.z_ln else 0) | (FLAG_DEDUP if dedup else 0)
    cfg = Config(B=sp.B, d=sp.d, H=sp.H, hidden=sp.hidden, M=sp.M, table_rows=sp.table_rows,
                 dtype=BF16 if sp.dtype == "bf16" else F32, score=SCORE[sp.score],
                 qmode=QMODE[sp.qmode], path=PATH[path], flags=flags, chunk_keys=chunk_keys,
                 n_ns=sp.n_ns, q_hidden=(sp.hy_hidden or sp.d) if sp.qmode == "hyformer" else 0,
                 encoder=ENCODER[getattr(sp, "encoder", "swiglu")], l_short=getattr(sp, "l_short", 0))

    def conv(w):
        if w is None:
            return None
        if isinstance(w, dict):
            return {k: conv(v) for k, v in w.items()}
        return _dev(w, device)
    if table is None:
        table = _dev(p.table, device)
    m = np.diff(p.tgt_offsets)
    km = p.extra.get("key_mask")
    hm = p.extra.get("head_map")
    hmap = None
    if hm is not None:
        hmap = (C.c_int32 * len(hm))(*[int(x) for x in hm])
        cfg.head_map = C.cast(hmap, C.POINTER(C.c_int32))
    return DeviceProblem(cfg, _dev(p.hist_offsets, device), _dev(p.hist_ids, device),
                         _dev(p.tgt_offsets, device), _dev(p.tgt_ids, device), _dev(p.q0, device),
                         table, [conv(l) for l in p.layers], conv(p.z), _dev(p.wz, device),
                         p.n_hist, p.n_tgt, max(1, int(m.max()) if len(m) else 1),
                         _dev(p.extra.get("ns"), device), conv(p.extra.get("qgen")),
                         _dev(None if km is None else np.asarray(km, np.uint32).view(np.int32), device), hmap,
                         _dev(None if p.extra.get("score_bias") is None
                              else np.asarray(p.extra["score_bias"], np.float32), device))


def _ffn(f) -> Ffn:
    if f is None:
        return Ffn()
    return Ffn(_ptr(f["w1"]), _ptr(f["w3"]), _ptr(f["w2"]), _ptr(f.get("ln_g")), _ptr(f.get("ln_b")))


def _structs(dp: DeviceProblem):
    layers = (Layer * len(dp.layers))()
    for i, l in enumerate(dp.layers):
        bo = l.get("boost") or {}
        en = l.get("enc") or {}
        layers[i] = Layer(_ffn(l["kv"]), _ffn(l.get("q")), _ptr(l["wk"]), _ptr(l["wv"]),
                          _ptr(l["wq"]), _ptr(l["wo"]), _ptr(l.get("wc")), _ptr(l.get("r")),
                          _ptr(bo.get("w1")), _ptr(bo.get("w3")), _ptr(bo.get("w2")),
                          _ptr(en.get("wq")), _ptr(en.get("wk")), _ptr(en.get("wv")), _ptr(en.get("wo")))
    qg = dp.qgen or {}
    w = Weights(layers, _ffn(dp.z), _ptr(dp.wz), _ptr(qg.get("w1")), _ptr(qg.get("w3")), _ptr(qg.get("w2")))
    b = Batch(_ptr(dp.hist_offsets), _ptr(dp.hist_ids), _ptr(dp.tgt_offsets), _ptr(dp.tgt_ids),
              _ptr(dp.q0), _ptr(dp.table), dp.n_hist, dp.n_tgt, dp.max_tgt, _ptr(dp.ns),
              _ptr(dp.key_mask), _ptr(dp.score_bias))
    return b, w, layers


def workspace_bytes(dp: DeviceProblem) -> int:
    lib = load()
    b, _, _ = _structs(dp)
    n = C.c_size_t(0)
    _check(lib.stca_workspace_size(C.byref(dp.cfg), C.byref(b), C.byref(n)))
    return n.value


class StageEvents:
    """hipEvent_t handles for the stage-boundary timing of ``stca_forward``
    (created with the HIP runtime directly so they live on the same stream as
    the library's kernels; read with ``elapsed`` after the stream completes)."""

    def __init__(self, n: int):
        self.hip = C.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [C.POINTER(_vp)]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), _vp, _vp]
        self.hip.hipEventDestroy.argtypes = [_vp]
        self.n = n
        self.arr = (_vp * n)()
        for i in range(n):
            ev = _vp()
            if self.hip.hipEventCreate(C.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.arr[i] = ev
        self.ptr = C.cast(self.arr, C.POINTER(_vp))

    def elapsed(self, i: int, j: int) -> float:
        """Milliseconds between boundary i and boundary j (after synchronisation)."""
        ms = C.c_float(0)
        r = self.hip.hipEventElapsedTime(C.byref(ms), self.arr[i], self.arr[j])
        if r != 0:
            raise RuntimeError(f"hipEventElapsedTime({i},{j}) failed: {r}")
        return ms.value

    def close(self):
        for i in range(self.n):
            if self.arr[i]:
                self.hip.hipEventDestroy(self.arr[i])
                self.arr[i] = None


def n_stage_events(M: int, longer: bool = False) -> int:
    """Stage events of stca_forward (with the LONGER pre-pass's after them)."""
    return 9 * M + 4 if longer else 5 * M + 3


def n_backward_stage_events(M: int) -> int:
    return 5 * M + 4


class Forward:
    """Reusable forward call: outputs and workspace are allocated once.
    ``noalloc``: call ``stca_forward_noalloc`` (no workspace; the library's
    static scratch) instead of ``stca_forward``."""

    def __init__(self, dp: DeviceProblem, want=("o", "attn", "active"), dumps=(), stream=None,
                 events: Optional[StageEvents] = None, noalloc: bool = False):
        import torch
        self.dp = dp
        self.lib = load()
        cfg = dp.cfg
        dev = dp.table.device
        T, d, M, H = dp.n_tgt, cfg.d, cfg.M, cfg.H
        lo = torch.int16 if cfg.dtype == BF16 else torch.float32
        self.z = torch.empty((T, d), dtype=torch.float32, device=dev)
        self.o = torch.empty((M, T, d), dtype=torch.float32, device=dev) if "o" in want else None
        self.attn = torch.empty((M, T, d), dtype=torch.float32, device=dev) if "attn" in want else None
        self.active = (torch.empty((M, T, H), dtype=torch.int32, device=dev)
                       if ("active" in want and cfg.score == 1) else None)
        self.q_dump = torch.empty((M, T, d), dtype=lo, device=dev) if "q" in dumps else None
        self.kv_dump = (torch.empty((M, 2, dp.n_hist, d), dtype=lo, device=dev)
                        if "kv" in dumps else None)
        self.x_dump = torch.empty((dp.n_hist, d), dtype=lo, device=dev) if "x" in dumps else None
        self.lse = torch.empty((M, T, H), dtype=torch.float32, device=dev) if "lse" in want else None
        self.status = torch.zeros(4, dtype=torch.int32, device=dev)
        self.b, self.w, self._layers = _structs(dp)
        self.out = Outputs(_ptr(self.z), _ptr(self.o), _ptr(self.attn), _ptr(self.active),
                           _ptr(self.q_dump), _ptr(self.kv_dump), _ptr(self.x_dump),
                           _ptr(self.status))
        self.out.lse = _ptr(self.lse)
        if events is not None:
            self.out.stage_events = events.ptr
            self.out.n_stage_events = events.n
        self.noalloc = noalloc
        self.stream = stream
        if noalloc:
            self.ws, self.ws_bytes = None, 0
            return
        n = C.c_size_t(0)
        _check(self.lib.stca_workspace_size(C.byref(cfg), C.byref(self.b), C.byref(n)))
        self.ws_bytes = n.value
        self.ws = torch.empty(max(1, self.ws_bytes), dtype=torch.uint8, device=dev)

    def __call__(self):
        import torch
        s = self.stream if self.stream is not None else torch.cuda.current_stream()
        if self.noalloc:
            _check(self.lib.stca_forward_noalloc(C.byref(self.dp.cfg), C.byref(self.b), C.byref(self.w),
                                                 C.byref(self.out), s.cuda_stream))
            return self
        _check(self.lib.stca_forward(C.byref(self.dp.cfg), C.byref(self.b), C.byref(self.w),
                                     C.byref(self.out), self.ws.data_ptr(), self.ws_bytes,
                                     s.cuda_stream))
        return self

    def results(self) -> dict:
        r = {"z": self.z, "o": self.o, "attn": self.attn, "active": self.active,
             "q": self.q_dump, "kv": self.kv_dump, "x": self.x_dump, "lse": self.lse,
             "status": self.status}
        return {k: v for k, v in r.items() if v is not None}


class Backward:
    """Reusable backward call (``stca_backward``): gradient buffers, upstream
    gradient and workspace are allocated once.  ``grads`` mirrors the weight
    nesting (layers[i]["kv"|"q"][w1|w3|w2|ln_g|ln_b], wk, wv, wq, wo, wc;
    z[...]; wz) with fp32 tensors; the library accumulates into them, so
    ``zero()`` them before a fresh step."""

    def __init__(self, dp: DeviceProblem, dz, outputs=("table", "d_hist", "d_tgt", "z"), dumps=(),
                 stream=None, events: Optional[StageEvents] = None):
        import torch
        self.dp = dp
        self.lib = load()
        cfg = dp.cfg
        dev = dp.table.device
        T, d, M = dp.n_tgt, cfg.d, cfg.M
        f32 = dict(dtype=torch.float32, device=dev)

        def like(w):
            if w is None:
                return None
            if isinstance(w, dict):
                return {k: like(v) for k, v in w.items()}
            return torch.zeros(tuple(w.shape), **f32)
        self.grads = {"layers": [like({k: v for k, v in l.items() if k != "r"}) for l in dp.layers],
                      "z": like(dp.z), "wz": like(dp.wz)}
        self.dz = dz
        self.table = torch.zeros((cfg.table_rows, d), **f32) if "table" in outputs else None
        self.d_hist = torch.empty((dp.n_hist, d), **f32) if "d_hist" in outputs else None
        self.d_tgt = torch.empty((T, d), **f32) if "d_tgt" in outputs else None
        self.z_out = torch.empty((T, d), **f32) if "z" in outputs else None
        self.dq_dump = torch.empty((M, T, d), **f32) if "dq" in dumps else None
        self.da_dump = torch.empty((M, T, d), **f32) if "da" in dumps else None
        self.dkv_dump = (torch.empty((M, dp.n_hist, 2 * d), dtype=torch.int16, device=dev)
                         if "dkv" in dumps else None)
        self.status = torch.zeros(4, dtype=torch.int32, device=dev)
        self.b, self.w, self._layers = _structs(dp)

        def fg(g):
            if g is None:
                return FfnGrad()
            return FfnGrad(_ptr(g["w1"]), _ptr(g["w3"]), _ptr(g["w2"]), _ptr(g.get("ln_g")),
                           _ptr(g.get("ln_b")))
        lg = (LayerGrad * M)()
        for i, g in enumerate(self.grads["layers"]):
            lg[i] = LayerGrad(fg(g["kv"]), fg(g["q"]), _ptr(g["wk"]), _ptr(g["wv"]), _ptr(g["wq"]),
                              _ptr(g["wo"]), _ptr(g.get("wc")))
        self._lg = lg
        self.g = Grads(lg, fg(self.grads["z"]), _ptr(self.grads["wz"]), _ptr(self.table),
                       _ptr(self.d_hist), _ptr(self.d_tgt), _ptr(self.z_out), _ptr(self.dq_dump),
                       _ptr(self.da_dump), _ptr(self.dkv_dump), _ptr(self.status))
        if events is not None:
            self.g.stage_events = events.ptr
            self.g.n_stage_events = events.n
        n = C.c_size_t(0)
        _check(self.lib.stca_backward_workspace_size(C.byref(cfg), C.byref(self.b), C.byref(n)))
        self.ws_bytes = n.value
        self.ws = torch.empty(max(1, self.ws_bytes), dtype=torch.uint8, device=dev)
        self.stream = stream

    def zero(self):
        def z(g):
            if g is None:
                return
            if isinstance(g, dict):
                for v in g.values():
                    z(v)
            elif isinstance(g, list):
                for v in g:
                    z(v)
            else:
                g.zero_()
        z(self.grads)
        if self.table is not None:
            self.table.zero_()
        return self

    def __call__(self, saved_forward: bool = False):
        """stca_backward; saved_forward: skip its recompute, using the
        activations forward_for_backward() left in the workspace."""
        import torch
        s = self.stream if self.stream is not None else torch.cuda.current_stream()
        self.g.saved_forward = 1 if saved_forward else 0
        _check(self.lib.stca_backward(C.byref(self.dp.cfg), C.byref(self.b), C.byref(self.w),
                                      _ptr(self.dz), C.byref(self.g), self.ws.data_ptr(), self.ws_bytes,
                                      s.cuda_stream))
        return self

    def forward_for_backward(self, z):
        """stca_forward_for_backward into this call's workspace: z (fp32
        [n_tgt, d] device tensor) is written, the activations stay for a
        following ``self(saved_forward=True)``."""
        import torch
        s = self.stream if self.stream is not None else torch.cuda.current_stream()
        _check(self.lib.stca_forward_for_backward(C.byref(self.dp.cfg), C.byref(self.b), C.byref(self.w),
                                                  _ptr(z), _ptr(self.status), self.ws.data_ptr(), self.ws_bytes,
                                                  s.cuda_stream))
        return z


def forward(dp: DeviceProblem, want=("o", "attn", "active"), dumps=()) -> dict:
    return Forward(dp, want, dumps)().results()


def attention(q, k, v, hist_offsets, tgt_offsets, H: int, score: str = "softmax",
              max_tgt: Optional[int] = None, chunk_keys: int = 0, key_mask=None, head_map=None,
              score_bias=None):
    """The attention core alone (``stca_attention``) on device tensors.
    q: [T, d] (already scaled by 1/sqrt(d_h)), k/v: [n_hist, d]; fp32, or
    bf16 bits as int16.  Returns (attn fp32 [T, d], active int32 [T, H] or None,
    dev_status)."""
    import torch
    lib = load()
    T, d = q.shape
    dtype = BF16 if q.dtype in (torch.int16, torch.bfloat16) else F32
    B = hist_offsets.numel() - 1
    if max_tgt is None:
        max_tgt = max(1, int((tgt_offsets[1:] - tgt_offsets[:-1]).max().item())) if B > 0 else 1
    attn = torch.empty((T, d), dtype=torch.float32, device=q.device)
    active = torch.empty((T, H), dtype=torch.int32, device=q.device) if score == "relu" else None
    status = torch.zeros(4, dtype=torch.int32, device=q.device)
    a = AttnArgs(B=B, d=d, H=H, dtype=dtype, score=SCORE[score], chunk_keys=chunk_keys,
                 hist_offsets=_ptr(hist_offsets), tgt_offsets=_ptr(tgt_offsets),
                 n_hist=k.shape[0], n_tgt=T, max_tgt_per_user=max_tgt, q=_ptr(q), k=_ptr(k),
                 v=_ptr(v), attn=_ptr(attn), active=_ptr(active), dev_status=_ptr(status),
                 key_mask=_ptr(key_mask), score_bias=_ptr(score_bias))
    hmap = None
    if head_map is not None:
        hmap = (C.c_int32 * len(head_map))(*[int(x) for x in head_map])
        a.head_map = C.cast(hmap, C.POINTER(C.c_int32))
    n = C.c_size_t(0)
    _check(lib.stca_attention_workspace_size(C.byref(a), C.byref(n)))
    ws = torch.empty(max(1, n.value), dtype=torch.uint8, device=q.device)
    _check(lib.stca_attention(C.byref(a), ws.data_ptr(), n.value,
                              torch.cuda.current_stream().cuda_stream))
    return attn, active, status


def to_numpy_stored(t) -> np.ndarray:
    """Device tensor -> numpy in the stored convention (bf16 bits as uint16)."""
    a = t.detach().cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a


def clock_ghz(c) -> float:
    """Shader clock (GHz) from {s_memtime, s_memrealtime} pairs at start and
    end (rows of 4 counters, as the library writes them; rows with no elapsed
    100 MHz ticks are ignored)."""
    c = np.asarray(c, dtype=np.int64).reshape(-1, 4)
    ticks = c[:, 3] - c[:, 1]
    ok = ticks > 0
    if not ok.any():
        return float("nan")
    return float(np.mean((c[ok, 2] - c[ok, 0]) / ticks[ok]) * 0.1)


def peak_hbm_read(nbytes: int = 2 << 30, blocks: int = 1024, repeats: int = 4) -> float:
    """Attainable HBM read rate (GB/s): the best of `repeats` timed launches
    of the library's streaming-read kernel over a fresh buffer of `nbytes`
    (larger than the 256 MB memory-side cache by default)."""
    import torch
    lib = load()
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    args = (C.c_void_p(buf.data_ptr()), nbytes, blocks, C.c_void_p(out.data_ptr()), C.c_void_p(s.cuda_stream))
    _check(lib.stca_peak_hbm_read(*args))
    best = 0.0
    for _ in range(repeats):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        _check(lib.stca_peak_hbm_read(*args))
        b.record(s)
        b.synchronize()
        best = max(best, nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
    del buf
    return best


def peak_mfma_bf16(blocks: int = 1024, iters: int = 20000, repeats: int = 3, mixed: bool = False):
    """Attainable dense bf16 MFMA rate (TFLOP/s), the best of `repeats` timed
    launches of the library's MFMA-only measurement kernel, and the shader
    clock (GHz) during that launch.  ``mixed``: operands that vary like real
    data (the kernel's iters < 0 mode)."""
    import torch
    lib = load()
    out = torch.empty(blocks * 4, dtype=torch.float32, device="cuda")
    clk = torch.zeros(4, dtype=torch.int64, device="cuda")
    s = torch.cuda.current_stream()
    flops = blocks * 4 * iters * 8 * 32768
    best, best_clk = 0.0, float("nan")
    args = (blocks, -iters if mixed else iters, C.c_void_p(out.data_ptr()), C.c_void_p(clk.data_ptr()),
            C.c_void_p(s.cuda_stream))
    _check(lib.stca_peak_mfma_bf16(*args))
    for _ in range(repeats):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        _check(lib.stca_peak_mfma_bf16(*args))
        b.record(s)
        b.synchronize()
        rate = flops / (a.elapsed_time(b) * 1e-3) / 1e12
        if rate > best:
            best, best_clk = rate, clock_ghz(clk.cpu().numpy())
    return best, best_clk
