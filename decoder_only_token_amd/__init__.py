"""Python binding of libqd, the MI355X (gfx950) single-sequence decoder-step library.

This module only marshals arguments (ctypes mirrors of the structs in
include/qd.h, device pointers taken from torch tensors, the current HIP
stream).  Every step of the forward pass runs in the HIP kernels of
libqd.so; there is no Python or CPU fallback, and importing the binding
without the built library raises.
"""
from __future__ import annotations

import atexit
import ctypes
import os
import sys
import weakref
from typing import Dict, List, Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqd.so")

QD_ABI_VERSION = 2
QD_W_BF16, QD_W_INT4_G128, QD_W_Q8_0 = 0, 1, 2
QD_DECODE_PERSISTENT, QD_DECODE_GRAPH = 0, 1
QD_KV_F32, QD_KV_BF16 = 0, 1
QD_CAP_EMBED, QD_CAP_LAYER_OUT, QD_CAP_FINAL_NORM, QD_CAP_LOGITS = 0, 1, 2, 3
QD_XCH = {"x0": 0, "x1": 1, "qkv": 2, "attn": 3, "act": 4}
QD_PROJ = {"wq": 0, "wk": 1, "wv": 2, "wo": 3, "w_gate": 4, "w_up": 5, "w_down": 6}
STATUS = {0: "QD_OK", -1: "QD_E_ARG", -2: "QD_E_ABI", -3: "QD_E_STATE", -4: "QD_E_RANGE", -5: "QD_E_OOM",
          -6: "QD_E_HIP"}

_P = ctypes.c_void_p
_PP = ctypes.POINTER(ctypes.c_void_p)


class QdConfig(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("abi_version", ctypes.c_uint32),
                ("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("qk_norm", ctypes.c_uint8), ("qkv_bias", ctypes.c_uint8), ("tie_embeddings", ctypes.c_uint8),
                ("weight_format", ctypes.c_uint8), ("max_pos", ctypes.c_int32), ("max_prefill", ctypes.c_int32),
                ("lora_rank_max", ctypes.c_int32), ("decode_path", ctypes.c_int32), ("kv_format", ctypes.c_int32)]


class QdWeights(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("embed", _P), ("final_norm", _P), ("lm_head", _P)] + \
               [(n, _PP) for n in ("attn_norm", "mlp_norm", "q_norm", "k_norm", "wq", "wk", "wv", "wo", "bq", "bk",
                                   "bv", "w_gate", "w_up", "w_down")]


class QdSampling(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("temperature", ctypes.c_float), ("top_k", ctypes.c_int32),
                ("top_p", ctypes.c_float), ("seed", ctypes.c_uint64)]


class QdLora(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("rank", ctypes.c_int32), ("alpha", ctypes.c_float),
                ("a_q", _PP), ("b_q", _PP), ("a_v", _PP), ("b_v", _PP)]


EXPORTS = ["qd_create", "qd_load_weights", "qd_reset_kv", "qd_prefill", "qd_decode_step", "qd_decode_steps", "qd_set_lora",
           "qd_clear_lora", "qd_enable_capture", "qd_get_capture", "qd_enable_phase_trace", "qd_get_phase_trace",
           "qd_get_quantized", "qd_get_exchange", "qd_sync_token", "qd_get_abandoned", "qd_get_position",
           "qd_last_error", "qd_destroy", "qd_sizeof_config", "qd_sizeof_weights", "qd_sizeof_sampling",
           "qd_sizeof_lora", "qd_sample_workspace_bytes", "qd_sample_logits", "qd_sample_logits_static",
           "qd_verify", "qd_rewind"]

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libqd.so (built by decoder_only_token_amd.build) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libqd.so not built: {path} is missing (run decoder_only_token_amd/build.py)")
    L = ctypes.CDLL(path)
    i32, u64, sz = ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
    H = _P
    sig = {
        "qd_create": (i32, [ctypes.POINTER(QdConfig), _P, ctypes.POINTER(H)]),
        "qd_load_weights": (i32, [H, ctypes.POINTER(QdWeights)]),
        "qd_reset_kv": (i32, [H]),
        "qd_prefill": (i32, [H, ctypes.POINTER(ctypes.c_int32), i32, ctypes.POINTER(QdSampling), _P, _P]),
        "qd_decode_step": (i32, [H, ctypes.POINTER(QdSampling), _P, _P]),
        "qd_decode_steps": (i32, [H, i32, ctypes.POINTER(QdSampling), _P, _P]),
        "qd_verify": (i32, [H, ctypes.POINTER(ctypes.c_int32), i32, _P, _P]),
        "qd_rewind": (i32, [H, i32, i32]),
        "qd_set_lora": (i32, [H, ctypes.POINTER(QdLora)]),
        "qd_clear_lora": (i32, [H]),
        "qd_enable_capture": (i32, [H, i32]),
        "qd_get_capture": (i32, [H, i32, i32, ctypes.POINTER(ctypes.c_float), sz, ctypes.POINTER(sz)]),
        "qd_enable_phase_trace": (i32, [H, i32]),
        "qd_get_phase_trace": (i32, [H, ctypes.POINTER(ctypes.c_uint64), sz, ctypes.POINTER(sz),
                                     ctypes.POINTER(ctypes.c_int32)]),
        "qd_get_quantized": (i32, [H, i32, i32, ctypes.POINTER(ctypes.c_int8), sz, ctypes.POINTER(ctypes.c_uint16),
                                   sz]),
        "qd_get_exchange": (i32, [H, i32, ctypes.POINTER(ctypes.c_float), sz, ctypes.POINTER(sz)]),
        "qd_sync_token": (i32, [H, ctypes.POINTER(ctypes.c_int32)]),
        "qd_get_abandoned": (i32, [H, ctypes.POINTER(ctypes.c_int64)]),
        "qd_get_position": (i32, [H, ctypes.POINTER(ctypes.c_int32)]),
        "qd_last_error": (ctypes.c_char_p, [H]),
        "qd_destroy": (None, [H]),
        "qd_sizeof_config": (sz, []),
        "qd_sizeof_weights": (sz, []),
        "qd_sizeof_sampling": (sz, []),
        "qd_sizeof_lora": (sz, []),
        "qd_sample_workspace_bytes": (sz, [i32, ctypes.POINTER(QdSampling)]),
        "qd_sample_logits": (i32, [_P, i32, ctypes.POINTER(QdSampling), u64, _P, _P, sz, _P]),
        "qd_sample_logits_static": (i32, [_P, i32, ctypes.POINTER(QdSampling), u64, _P, _P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    for name, cls in (("qd_sizeof_config", QdConfig), ("qd_sizeof_weights", QdWeights),
                      ("qd_sizeof_sampling", QdSampling), ("qd_sizeof_lora", QdLora)):
        if getattr(L, name)() != ctypes.sizeof(cls):
            raise ImportError(f"ctypes mirror of {cls.__name__} does not match the C struct size")
    _lib = L
    return L


class QdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


def make_config(shape, max_prefill: int, lora_rank_max: int = 0, max_pos: Optional[int] = None,
                decode_path: Optional[int] = None, kv_format: int = QD_KV_F32) -> QdConfig:
    """Fill a QdConfig from any object with the model-shape attribute names.
    decode_path None: the persistent step for bf16 weights; the graph for int4
    weights (faster on the graph, where their single-row projections run on
    the int8 matrix cores over every CU) and for Q8_0 weights (the only path
    they run on)."""
    if decode_path is None:
        decode_path = QD_DECODE_PERSISTENT if int(shape.weight_format) == QD_W_BF16 else QD_DECODE_GRAPH
    c = QdConfig()
    c.struct_size = ctypes.sizeof(QdConfig)
    c.abi_version = QD_ABI_VERSION
    for f in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "intermediate", "vocab"):
        setattr(c, f, int(getattr(shape, f)))
    c.rope_theta = float(shape.rope_theta)
    c.rms_eps = float(shape.rms_eps)
    c.qk_norm = int(bool(shape.qk_norm))
    c.qkv_bias = int(bool(shape.qkv_bias))
    c.tie_embeddings = 1
    c.weight_format = int(shape.weight_format)
    c.max_pos = int(max_pos if max_pos is not None else shape.max_pos)
    c.max_prefill = int(max_prefill)
    c.lora_rank_max = int(lora_rank_max)
    c.decode_path = int(decode_path)
    c.kv_format = int(kv_format)
    return c


QD_VERIFY_MAX = 16


def accepted_drafts(drafts: Sequence[int], choices: Sequence[int]) -> int:
    """Greedy acceptance: the number of leading drafts d[i] that equal the
    choice made before them (choices[i] follows the i-th verified row)."""
    a = 0
    while a < len(drafts) and int(drafts[a]) == int(choices[a]):
        a += 1
    return a


def make_sampling(temperature: float, top_k: int, top_p: float, seed: int) -> QdSampling:
    s = QdSampling()
    s.struct_size = ctypes.sizeof(QdSampling)
    s.temperature, s.top_k, s.top_p, s.seed = float(temperature), int(top_k), float(top_p), int(seed)
    return s


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _ptr_array(ts: Sequence) -> ctypes.Array:
    return (ctypes.c_void_p * len(ts))(*[_ptr(t) for t in ts])


_live = weakref.WeakSet()  # open decoders, closed before the interpreter exits


@atexit.register
def _close_all():
    """Release every open handle (and torch's cached device memory) while the
    HIP runtime and any attached profiler are still up: process-exit handlers
    of those run after the interpreter's own exit handlers."""
    for d in list(_live):
        try:
            d.close()
        except Exception:
            pass
    torch = sys.modules.get("torch")
    try:
        if torch is not None and torch.cuda.is_initialized():
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
    except Exception:
        pass


class Decoder:
    """One model on the current GPU behind the C ABI.

    Device tensors (torch, on the current CUDA/HIP device) supply the memory the
    library reads and writes; the current torch stream is the stream every call
    enqueues on.  Weights are dicts of bf16 tensors (any 16-bit dtype holding
    bf16 bit patterns).
    """

    def __init__(self, cfg: QdConfig, stream_ptr: int):
        self.lib = load_library()
        self.cfg = cfg
        h = ctypes.c_void_p()
        rc = self.lib.qd_create(ctypes.byref(cfg), ctypes.c_void_p(stream_ptr), ctypes.byref(h))
        if rc != 0:
            raise QdError(rc, "qd_create failed (reason printed on stderr)")
        self.h = h
        _live.add(self)

    def _check(self, rc: int):
        if rc != 0:
            raise QdError(rc, self.lib.qd_last_error(self.h).decode())

    def close(self):
        if getattr(self, "h", None):
            self.lib.qd_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            if sys.is_finalizing():  # the HIP runtime may already be gone; _close_all ran earlier
                return
            self.close()
        except Exception:
            pass

    def load_weights(self, w: Dict):
        """w = {"embed", "final_norm", "layers": [ {name: tensor} ]} of device tensors."""
        layers = w["layers"]
        qw = QdWeights()
        qw.struct_size = ctypes.sizeof(QdWeights)
        qw.embed = _ptr(w["embed"])
        qw.final_norm = _ptr(w["final_norm"])
        qw.lm_head = None
        keep = []
        for name in ("attn_norm", "mlp_norm", "q_norm", "k_norm", "wq", "wk", "wv", "wo", "bq", "bk", "bv",
                     "w_gate", "w_up", "w_down"):
            if name in layers[0]:
                arr = _ptr_array([lw[name] for lw in layers])
                keep.append(arr)
                setattr(qw, name, ctypes.cast(arr, _PP))
        self._check(self.lib.qd_load_weights(self.h, ctypes.byref(qw)))

    def reset_kv(self):
        self._check(self.lib.qd_reset_kv(self.h))

    def prefill(self, tokens: Sequence[int], sampling: Optional[QdSampling] = None, logits_out=None, token_out=None):
        arr = (ctypes.c_int32 * len(tokens))(*[int(t) for t in tokens])
        self._check(self.lib.qd_prefill(self.h, arr, len(tokens), ctypes.byref(sampling) if sampling else None,
                                        ctypes.c_void_p(_ptr(logits_out)), ctypes.c_void_p(_ptr(token_out))))

    def decode_step(self, sampling: Optional[QdSampling] = None, logits_out=None, token_out=None):
        self._check(self.lib.qd_decode_step(self.h, ctypes.byref(sampling) if sampling else None,
                                            ctypes.c_void_p(_ptr(logits_out)), ctypes.c_void_p(_ptr(token_out))))

    def decode_steps(self, n: int, sampling: Optional[QdSampling] = None, logits_out=None, tokens_out=None):
        """n decode steps with device-resident token feedback (tokens_out: int32 device tensor of n)."""
        self._check(self.lib.qd_decode_steps(self.h, int(n), None if sampling is None else ctypes.byref(sampling),
                                             _ptr(logits_out), _ptr(tokens_out)))

    def verify(self, tokens: Sequence[int], logits_out=None, choices_out=None):
        """Speculative verification of len(tokens) <= QD_VERIFY_MAX tokens: the
        greedy choice after every row into choices_out (int32 device tensor),
        the rows' logits into logits_out (float32 device tensor [m, V])."""
        arr = (ctypes.c_int32 * len(tokens))(*[int(t) for t in tokens])
        self._check(self.lib.qd_verify(self.h, arr, len(tokens), ctypes.c_void_p(_ptr(logits_out)),
                                       ctypes.c_void_p(_ptr(choices_out))))

    def rewind(self, n: int, next_token: int):
        """Drop the last n positions and make next_token the next input token."""
        self._check(self.lib.qd_rewind(self.h, int(n), int(next_token)))

    def speculative_step(self, next_token: int, drafts: Sequence[int], choices_out):
        """One greedy speculative step: verify [next_token, *drafts], accept the
        leading drafts that equal the choice before them, rewind the rest.
        Returns the new tokens (the accepted drafts and one more choice), which
        are those of as many greedy decode steps.  choices_out: an int32 device
        tensor of at least len(drafts) + 1 entries (read back here)."""
        m = len(drafts) + 1
        self.verify([next_token, *drafts], choices_out=choices_out)
        self.sync_token()  # the library's stream, which need not be torch's current one
        c = [int(v) for v in choices_out[:m].cpu().tolist()]
        a = accepted_drafts(drafts, c)
        self.rewind(m - 1 - a, c[a])
        return list(drafts[:a]) + [c[a]]

    def set_lora(self, lora_layers: List[Dict], rank: int, alpha: float):
        q = QdLora()
        q.struct_size = ctypes.sizeof(QdLora)
        q.rank, q.alpha = int(rank), float(alpha)
        keep = []
        for name in ("a_q", "b_q", "a_v", "b_v"):
            arr = _ptr_array([lw[name] for lw in lora_layers])
            keep.append(arr)
            setattr(q, name, ctypes.cast(arr, _PP))
        self._check(self.lib.qd_set_lora(self.h, ctypes.byref(q)))

    def clear_lora(self):
        self._check(self.lib.qd_clear_lora(self.h))

    def enable_capture(self, on: bool = True):
        self._check(self.lib.qd_enable_capture(self.h, int(on)))

    def get_capture(self, what: int, layer: int, capacity: int):
        import numpy as np
        out = np.empty(capacity, dtype=np.float32)
        written = ctypes.c_size_t()
        self._check(self.lib.qd_get_capture(self.h, what, layer,
                                            out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), capacity,
                                            ctypes.byref(written)))
        return out[:written.value]

    def enable_phase_trace(self, on: bool = True):
        self._check(self.lib.qd_enable_phase_trace(self.h, int(on)))

    def get_phase_trace(self):
        """Stamps of the last decode step as a uint64 array [n_cu, 1 + 2 (5 L + 2)] (100 MHz ticks)."""
        import numpy as np
        n = 4096 * (1 + 2 * (5 * self.cfg.n_layers + 2))
        out = np.empty(n, dtype=np.uint64)
        written, ncu = ctypes.c_size_t(), ctypes.c_int32()
        self._check(self.lib.qd_get_phase_trace(self.h, out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), n,
                                                ctypes.byref(written), ctypes.byref(ncu)))
        return out[:written.value].reshape(ncu.value, -1)

    def get_quantized(self, layer: int, name: str, shape):
        """int4 / Q8_0 encoding of projection `name` ("wq", ..., "w_down") of
        `layer`: (codes int8 [N, K], scales float16 [N, K / B]), B = 128 (int4)
        or 32 (Q8_0)."""
        import numpy as np
        n, k = shape
        b = 32 if self.cfg.weight_format == QD_W_Q8_0 else 128
        codes = np.empty((n, k), dtype=np.int8)
        scales = np.empty((n, k // b), dtype=np.uint16)
        self._check(self.lib.qd_get_quantized(self.h, layer, QD_PROJ[name],
                                              codes.ctypes.data_as(ctypes.POINTER(ctypes.c_int8)), codes.size,
                                              scales.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), scales.size))
        return codes, scales.view(np.float16)

    def get_exchange(self, name: str, n: int):
        """A persistent-step exchange buffer ("x0", "x1", "qkv", "attn", "act") after the last step."""
        import numpy as np
        out = np.empty(n, dtype=np.float32)
        written = ctypes.c_size_t()
        self._check(self.lib.qd_get_exchange(self.h, QD_XCH[name], out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                             n, ctypes.byref(written)))
        return out[:written.value]

    def sync_token(self) -> int:
        t = ctypes.c_int32()
        self._check(self.lib.qd_sync_token(self.h, ctypes.byref(t)))
        return t.value

    def abandoned(self) -> int:
        """Cache episodes since creation in which a persistent decode step was abandoned (synchronises)."""
        n = ctypes.c_int64()
        self._check(self.lib.qd_get_abandoned(self.h, ctypes.byref(n)))
        return n.value

    @property
    def position(self) -> int:
        p = ctypes.c_int32()
        self._check(self.lib.qd_get_position(self.h, ctypes.byref(p)))
        return p.value


def _sp_ref(sampling: Optional[QdSampling]):
    return None if sampling is None else ctypes.byref(sampling)


def sample_workspace_bytes(vocab: int, sampling: Optional[QdSampling] = None) -> int:
    """Device scratch bytes qd_sample_logits needs for `vocab` logits (0: invalid arguments)."""
    return int(load_library().qd_sample_workspace_bytes(int(vocab), _sp_ref(sampling)))


def sample_logits(logits, sampling: Optional[QdSampling], step: int, token_out, workspace, stream_ptr: int = 0):
    """Choose a token from `logits` (f32 device tensor, 1-D) into `token_out`
    (int32 device tensor, 1 element) with the caller's `workspace` (device
    tensor of at least sample_workspace_bytes(...) bytes), enqueued on the
    stream `stream_ptr`."""
    L = load_library()
    rc = L.qd_sample_logits(_ptr(logits), int(logits.numel()), _sp_ref(sampling), int(step), _ptr(token_out),
                            _ptr(workspace), int(workspace.numel() * workspace.element_size()), stream_ptr)
    if rc != 0:
        raise QdError(rc, L.qd_last_error(None).decode())


def sample_logits_static(logits, sampling: Optional[QdSampling], step: int, token_out, stream_ptr: int = 0):
    """sample_logits with the library's static per-device scratch (no workspace)."""
    L = load_library()
    rc = L.qd_sample_logits_static(_ptr(logits), int(logits.numel()), _sp_ref(sampling), int(step), _ptr(token_out),
                                   stream_ptr)
    if rc != 0:
        raise QdError(rc, L.qd_last_error(None).decode())
