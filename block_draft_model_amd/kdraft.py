"""ctypes binding of libkdraft (include/kdraft.h, include/kdraft_debug.h).

Argument marshalling only: every step of a round runs in the library's HIP
kernels. torch supplies device memory and the HIP stream handle. If the
library is missing this module raises on first use; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkdraft.so")

KD_OK, KD_ERR_ARG, KD_ERR_STATE, KD_ERR_OOM, KD_ERR_HIP, KD_ERR_UNSUPPORTED, KD_ERR_RANGE = 0, -1, -2, -3, -4, -5, -6
KD_QUANT_FP8_BLOCK64, KD_QUANT_NVFP4, KD_QUANT_BF16 = 1, 2, 3
KD_MAX_INGEST = 8

c_int, c_float, c_void_p, c_int64 = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int64


class KdConfig(ctypes.Structure):
    _fields_ = [(n, c_int) for n in ("hidden", "heads", "head_dim", "ffn", "layers", "block",
                                      "rank", "taps", "window", "draft_vocab", "full_vocab",
                                      "max_streams")] + [
        ("rope_theta", c_float), ("rms_eps", c_float), ("body_quant", c_int), ("head_quant", c_int)]


class KdMatrix(ctypes.Structure):
    _fields_ = [("q", c_void_p), ("s", c_void_p), ("s4", c_void_p), ("g", c_float)]


class KdLayerWeights(ctypes.Structure):
    _fields_ = [(n, KdMatrix) for n in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")] + [
        ("attn_norm", c_void_p), ("ffn_norm", c_void_p), ("spine_norm", c_void_p),
        ("spine_a", KdMatrix), ("spine_u", KdMatrix)]


class KdWeights(ctypes.Structure):
    _fields_ = [(n, KdMatrix) for n in ("fuse", "fc", "pred_a", "pred_b", "pred_u")] + [
        ("mask_row", c_void_p), ("layer", KdLayerWeights * 4), ("final_norm", c_void_p),
        ("head_q4", c_void_p), ("head_s4", c_void_p), ("head_g", c_float),
        ("draft_vocab", c_void_p), ("embed_table", c_void_p), ("kv_rot_signs", c_void_p),
        ("head_bf16", c_void_p), ("head_fp8", KdMatrix)]


KD_KV_BF16, KD_KV_INT4_ROT = 0, 1


class KdKV(ctypes.Structure):
    _fields_ = [("k", c_void_p * 4), ("v", c_void_p * 4), ("stride_stream", c_int64),
                ("stride_head", c_int64), ("stride_slot", c_int64), ("capacity", c_int),
                ("format", c_int), ("k_so", c_void_p * 4), ("v_so", c_void_p * 4)]


EXPORTS = ["kd_default_config", "kd_create", "kd_load_weights", "kd_round", "kd_round_depth",
           "kd_ingest", "kd_copy_draft", "kd_copy_guard_init", "kd_copy_guard_armed",
           "kd_copy_guard_record", "kd_copy_guard_advance",
           "kd_set_stream", "kd_destroy", "kd_status_string", "kd_last_error",
           "kd_probe_decode_e4m3", "kd_probe_decode_e4m3_f16", "kd_probe_decode_nvfp4", "kd_debug_set_layers",
           "kd_debug_buffers", "kd_debug_set_path", "kd_debug_last_path",
           "kd_debug_set_trace", "kd_copy_draft_noalloc", "kd_debug_set_fused"]

KD_MAX_COPY = 48
KD_GUARD_MAX_WINDOW = 64


class KdCopyGuard(ctypes.Structure):
    _fields_ = [("window", c_int), ("pause", c_int), ("paused_left", c_int), ("count", c_int),
                ("next", c_int), ("min_accept", c_float),
                ("proposed", c_int * KD_GUARD_MAX_WINDOW), ("accepted", c_int * KD_GUARD_MAX_WINDOW)]


_lib = None


class KDraftError(RuntimeError):
    def __init__(self, status, msg=""):
        self.status = status
        super().__init__(f"libkdraft: {status_string(status)} ({status})" + (f": {msg}" if msg else ""))


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libkdraft.so (built by block_draft_model_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libkdraft.so not found at {path}; run python -m block_draft_model_amd.build")
    # torch carries its own HIP runtime; loading it first makes the library bind
    # to that same runtime, so that torch's device memory and streams are valid
    # in the library's calls (loaded the other way round, a process holds two
    # HIP runtimes and the library's launches do not reach torch's device state)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.kd_default_config.argtypes = [P(KdConfig)]
    lib.kd_default_config.restype = None
    lib.kd_create.argtypes = [P(KdConfig), c_void_p, P(c_void_p)]
    lib.kd_create.restype = c_int
    lib.kd_load_weights.argtypes = [c_void_p, P(KdWeights)]
    lib.kd_load_weights.restype = c_int
    lib.kd_round.argtypes = [c_void_p, c_int, c_void_p, c_void_p, c_void_p, P(KdKV), c_void_p,
                             c_void_p, c_void_p]
    lib.kd_round.restype = c_int
    lib.kd_round_depth.argtypes = [c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, P(KdKV),
                                   c_void_p, c_void_p, c_void_p]
    lib.kd_round_depth.restype = c_int
    lib.kd_copy_draft.argtypes = [c_void_p, c_int, c_void_p, ctypes.c_longlong, c_void_p, c_void_p,
                                  ctypes.c_longlong, c_int, c_void_p, c_void_p]
    lib.kd_copy_draft.restype = c_int
    lib.kd_copy_draft_noalloc.argtypes = [c_void_p, c_int, c_void_p, ctypes.c_longlong, c_void_p, c_void_p,
                                          ctypes.c_longlong, c_int, c_void_p, c_void_p]
    lib.kd_copy_draft_noalloc.restype = c_int
    lib.kd_copy_guard_init.argtypes = [P(KdCopyGuard), c_int, c_float, c_int]
    lib.kd_copy_guard_init.restype = None
    lib.kd_copy_guard_armed.argtypes = [P(KdCopyGuard)]
    lib.kd_copy_guard_armed.restype = c_int
    lib.kd_copy_guard_record.argtypes = [P(KdCopyGuard), c_int, c_int]
    lib.kd_copy_guard_record.restype = None
    lib.kd_copy_guard_advance.argtypes = [P(KdCopyGuard), c_int]
    lib.kd_copy_guard_advance.restype = None
    lib.kd_ingest.argtypes = [c_void_p, c_int, c_int, c_void_p, c_void_p, P(KdKV), c_void_p]
    lib.kd_ingest.restype = c_int
    lib.kd_set_stream.argtypes = [c_void_p, c_void_p]
    lib.kd_set_stream.restype = c_int
    lib.kd_destroy.argtypes = [c_void_p]
    lib.kd_destroy.restype = None
    lib.kd_status_string.argtypes = [c_int]
    lib.kd_status_string.restype = ctypes.c_char_p
    lib.kd_last_error.argtypes = [c_void_p]
    lib.kd_last_error.restype = ctypes.c_char_p
    lib.kd_probe_decode_e4m3.argtypes = [c_void_p]
    lib.kd_probe_decode_e4m3.restype = c_int
    lib.kd_probe_decode_e4m3_f16.argtypes = [c_void_p]
    lib.kd_probe_decode_e4m3_f16.restype = c_int
    lib.kd_probe_decode_nvfp4.argtypes = [c_void_p]
    lib.kd_probe_decode_nvfp4.restype = c_int
    lib.kd_debug_set_layers.argtypes = [c_void_p, c_int]
    lib.kd_debug_set_layers.restype = c_int
    lib.kd_debug_buffers.argtypes = [c_void_p, P(c_void_p), P(c_void_p)]
    lib.kd_debug_buffers.restype = c_int
    lib.kd_debug_set_path.argtypes = [c_void_p, c_int]
    lib.kd_debug_set_path.restype = c_int
    lib.kd_debug_set_fused.argtypes = [c_void_p, c_int]
    lib.kd_debug_set_fused.restype = c_int
    lib.kd_debug_last_path.argtypes = [c_void_p]
    lib.kd_debug_last_path.restype = c_int
    lib.kd_debug_set_trace.argtypes = [c_void_p, c_void_p, c_int, P(c_int)]
    lib.kd_debug_set_trace.restype = c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().kd_status_string(int(status)).decode()


def default_config(**over) -> KdConfig:
    cfg = KdConfig()
    load_library().kd_default_config(ctypes.byref(cfg))
    for k, v in over.items():
        setattr(cfg, k, v)
    return cfg


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


KD_COPY_NOALLOC_MAX_STREAMS = 1024


def copy_draft_noalloc(streams, tokens, stride, lens, corpus, corpus_len, K, out_ids, out_info,
                       stream=None) -> int:
    """kd_copy_draft_noalloc on `stream` (default: torch's current stream);
    returns the kd_status code (no context, so no message)."""
    lib = load_library()
    return int(lib.kd_copy_draft_noalloc(_stream_handle(stream), int(streams), _ptr(tokens), int(stride),
                                         _ptr(lens), _ptr(corpus), int(corpus_len), int(K), _ptr(out_ids),
                                         _ptr(out_info)))


def kv_struct(k_layers, v_layers) -> KdKV:
    """K/V cache description from per-layer torch tensors [B][heads][capacity][head_dim] (bf16)."""
    kv = KdKV()
    ref = k_layers[0]
    for l in range(4):
        for t in (k_layers[l], v_layers[l]):
            if t.stride() != ref.stride() or t.shape != ref.shape or t.stride(-1) != 1:
                raise ValueError("K/V layers must share one contiguous-head_dim layout")
        kv.k[l] = k_layers[l].data_ptr()
        kv.v[l] = v_layers[l].data_ptr()
    kv.stride_stream, kv.stride_head, kv.stride_slot = ref.stride(0), ref.stride(1), ref.stride(2)
    kv.capacity = ref.shape[2]
    kv.format = KD_KV_BF16
    return kv


def kv_struct_int4(k_layers, v_layers, kso_layers, vso_layers) -> KdKV:
    """Rotated 4-bit cache description from per-layer torch tensors: codes
    uint8 [B][heads][capacity][head_dim/2] and (scale, offset) fp16 bits
    [B][heads][capacity][2] (any 16-bit dtype). The library takes strides in
    rows, so both tensors must index rows the same way."""
    kv = KdKV()
    ref, sref = k_layers[0], kso_layers[0]
    for l in range(4):
        for t in (k_layers[l], v_layers[l]):
            if (t.shape != ref.shape or t.stride() != ref.stride() or t.element_size() != 1
                    or t.shape[-1] != 64 or t.stride(-1) != 1):
                raise ValueError("4-bit code tensors must share one [B][heads][capacity][64] byte layout")
        for t in (kso_layers[l], vso_layers[l]):
            if (t.shape != sref.shape or t.stride() != sref.stride() or t.element_size() != 2
                    or t.shape[-1] != 2 or t.stride(-1) != 1):
                raise ValueError("scale tensors must share one [B][heads][capacity][2] 16-bit layout")
        kv.k[l], kv.v[l] = k_layers[l].data_ptr(), v_layers[l].data_ptr()
        kv.k_so[l], kv.v_so[l] = kso_layers[l].data_ptr(), vso_layers[l].data_ptr()
    if tuple(sref.shape[:3]) != tuple(ref.shape[:3]):
        raise ValueError("codes and scales must cover the same rows")
    rows = []
    for i in range(3):
        if ref.stride(i) % 64 or sref.stride(i) % 2 or ref.stride(i) // 64 != sref.stride(i) // 2:
            raise ValueError("codes and scales must use the same row strides")
        rows.append(ref.stride(i) // 64)
    kv.stride_stream, kv.stride_head, kv.stride_slot = rows
    kv.capacity = ref.shape[2]
    kv.format = KD_KV_INT4_ROT
    return kv


def _host(t):
    """Contiguous host numpy array of a torch tensor or array (kept alive by the caller)."""
    if isinstance(t, np.ndarray):
        return np.ascontiguousarray(t)
    t = t.detach()
    if t.dtype.is_floating_point and t.dtype != __import__("torch").float32:
        raise ValueError("weights vectors must be fp32")
    return np.ascontiguousarray(t.cpu().numpy())


class Drafter:
    """Owns one kd_ctx. Methods mirror kd_load_weights / kd_round / kd_round_depth / kd_ingest."""

    def __init__(self, max_streams: int = 256, stream=None, **cfg_over):
        self.lib = load_library()
        self.cfg = default_config(max_streams=max_streams, **cfg_over)
        h = c_void_p()
        st = self.lib.kd_create(ctypes.byref(self.cfg), c_void_p(_stream_handle(stream)), ctypes.byref(h))
        if st != KD_OK:
            raise KDraftError(st, "kd_create")
        self.ctx = h

    def _check(self, st, what):
        if st != KD_OK:
            raise KDraftError(st, f"{what}: {self.lib.kd_last_error(self.ctx).decode()}")

    def set_stream(self, stream):
        self._check(self.lib.kd_set_stream(self.ctx, c_void_p(_stream_handle(stream))), "kd_set_stream")

    def load_weights(self, model: dict):
        """model: the synthetic model dict (torch tensors); the table must be on the GPU."""
        keep = []

        def h(x):
            a = _host(x)
            keep.append(a)
            return a.ctypes.data

        def fp8(name):
            return KdMatrix(h(model[name + ".q"]), h(model[name + ".s"]), None, 0.0)

        body = model.get("body_format", "fp8")

        def mat(name):
            """A body matrix in the model's body format (the context's body_quant)."""
            if body == "nvfp4":
                return KdMatrix(h(model[name + ".q4"]), None, h(model[name + ".s4"]), float(model[name + ".g"]))
            if body == "bf16":
                import torch
                v = model[name + ".bf16"]
                return KdMatrix(h(v.view(torch.int16) if isinstance(v, torch.Tensor) else v), None, None, 0.0)
            return fp8(name)

        w = KdWeights()
        w.fuse, w.fc = mat("fuse"), mat("fc")
        w.pred_a, w.pred_b, w.pred_u = mat("pred_a"), mat("pred_b"), mat("pred_u")
        w.mask_row = h(model["mask"])
        for l in range(4):
            p = f"layers.{l}."
            L = w.layer[l]
            for nm in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
                setattr(L, nm, mat(p + nm))
            L.attn_norm, L.ffn_norm = h(model[p + "attn_norm"]), h(model[p + "ffn_norm"])
            if l >= 1:
                sp = f"spine.{l}."
                L.spine_norm = h(model[sp + "norm"])
                L.spine_a, L.spine_u = mat(sp + "a"), mat(sp + "u")
        w.final_norm = h(model["final_norm"])
        w.head_q4, w.head_s4 = h(model["head.q4"]), h(model["head.s4"])
        w.head_g = float(model["head.g"])
        w.draft_vocab = h(model["vocab"])
        if model.get("kv_rot_signs") is not None:
            w.kv_rot_signs = h(model["kv_rot_signs"])
        if model.get("head_bf16") is not None:
            import torch
            hb = model["head_bf16"]
            w.head_bf16 = h(hb.view(torch.int16) if isinstance(hb, torch.Tensor) else hb)
        if model.get("head_fp8.q") is not None:
            w.head_fp8 = fp8("head_fp8")
        table = model["table"]
        if not getattr(table, "is_cuda", False):
            raise ValueError("the embedding table must be a device tensor (it is borrowed)")
        self.table = table
        w.embed_table = table.data_ptr()
        self._check(self.lib.kd_load_weights(self.ctx, ctypes.byref(w)), "kd_load_weights")

    def round(self, streams, taps, anchor, pred, kv: KdKV, lens, out_ids, out_logits=None):
        self._check(self.lib.kd_round(self.ctx, int(streams), _ptr(taps), _ptr(anchor), _ptr(pred),
                                      ctypes.byref(kv), _ptr(lens), _ptr(out_ids), _ptr(out_logits)),
                    "kd_round")

    def round_depth(self, depth, streams, taps, anchor, pred, kv: KdKV, lens, out_ids,
                    out_logits=None):
        self._check(self.lib.kd_round_depth(self.ctx, int(depth), int(streams), _ptr(taps),
                                            _ptr(anchor), _ptr(pred), ctypes.byref(kv), _ptr(lens),
                                            _ptr(out_ids), _ptr(out_logits)),
                    "kd_round_depth")

    def copy_draft(self, streams, tokens, stride, lens, corpus, corpus_len, K, out_ids, out_info):
        self._check(self.lib.kd_copy_draft(self.ctx, int(streams), _ptr(tokens), int(stride),
                                           _ptr(lens), _ptr(corpus), int(corpus_len), int(K),
                                           _ptr(out_ids), _ptr(out_info)), "kd_copy_draft")

    def ingest(self, streams, n_new, taps, next_ids, kv: KdKV, lens):
        self._check(self.lib.kd_ingest(self.ctx, int(streams), int(n_new), _ptr(taps), _ptr(next_ids),
                                       ctypes.byref(kv), _ptr(lens)), "kd_ingest")

    def debug_set_layers(self, n: int):
        self._check(self.lib.kd_debug_set_layers(self.ctx, int(n)), "kd_debug_set_layers")

    def debug_set_path(self, path: int):
        """0 automatic, 1 general multi-kernel, 2 small-batch phases as launches,
        3 small-batch persistent kernel (paths 2-3 only for <= 4 streams)."""
        self._check(self.lib.kd_debug_set_path(self.ctx, int(path)), "kd_debug_set_path")

    def debug_set_fused(self, on: bool):
        """General path above 32 block rows: fused projection epilogues (True,
        the default) or the separate epilogue kernels (False)."""
        self._check(self.lib.kd_debug_set_fused(self.ctx, int(bool(on))), "kd_debug_set_fused")

    def debug_set_trace(self, buf, phases: int) -> int:
        """Stage timestamps of later rounds into buf (device uint64 [phases][G][8]);
        None turns tracing off. Returns G, the workgroup count."""
        g = c_int(0)
        self._check(self.lib.kd_debug_set_trace(self.ctx, _ptr(buf), int(phases), ctypes.byref(g)),
                    "kd_debug_set_trace")
        return g.value

    def last_path(self) -> int:
        return int(self.lib.kd_debug_last_path(self.ctx))

    def debug_buffers(self):
        hid, fus = c_void_p(), c_void_p()
        self._check(self.lib.kd_debug_buffers(self.ctx, ctypes.byref(hid), ctypes.byref(fus)),
                    "kd_debug_buffers")
        return hid.value, fus.value

    def close(self):
        if getattr(self, "ctx", None):
            self.lib.kd_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def probe_decode_e4m3(out) -> None:
    st = load_library().kd_probe_decode_e4m3(_ptr(out))
    if st != KD_OK:
        raise KDraftError(st, "kd_probe_decode_e4m3")


def probe_decode_e4m3_f16(out) -> None:
    st = load_library().kd_probe_decode_e4m3_f16(_ptr(out))
    if st != KD_OK:
        raise KDraftError(st, "kd_probe_decode_e4m3_f16")


def probe_decode_nvfp4(out) -> None:
    st = load_library().kd_probe_decode_nvfp4(_ptr(out))
    if st != KD_OK:
        raise KDraftError(st, "kd_probe_decode_nvfp4")


class CopyGuard:
    """kd_copy_guard: the copy source's acceptance pause guard (host only)."""

    def __init__(self, window=24, min_accept=0.5, pause=256):
        self.lib = load_library()
        self.g = KdCopyGuard()
        self.lib.kd_copy_guard_init(ctypes.byref(self.g), int(window), float(min_accept), int(pause))

    def armed(self) -> bool:
        return bool(self.lib.kd_copy_guard_armed(ctypes.byref(self.g)))

    def record(self, proposed, accepted):
        self.lib.kd_copy_guard_record(ctypes.byref(self.g), int(proposed), int(accepted))

    def advance(self, tokens):
        self.lib.kd_copy_guard_advance(ctypes.byref(self.g), int(tokens))
