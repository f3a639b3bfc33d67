"""ctypes binding of the C ABI in include/dec.h -- argument marshalling only.

Every function has the name of its C counterpart. Host arrays are numpy int32
arrays; device buffers are passed as integer addresses (e.g. a torch tensor's
``data_ptr()``) and streams as integer hipStream_t handles (torch's
``cuda_stream``). Non-zero return codes raise ``DecError`` with the library's
message. Nothing here computes any part of the forward pass.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch already loaded (same soname), and device pointers and
streams from torch are valid in it.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

import torch  # noqa: F401  (loads the process's HIP runtime first)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdec.so")

DEC_OK = 0
DEC_E_ARG = -1
DEC_E_UNSUPPORTED = -2
DEC_E_CAPACITY = -3
DEC_E_BLOCK = -4
DEC_E_POSITION = -5
DEC_E_TOKEN = -6
DEC_E_HIP = -7

DEC_F32, DEC_BF16, DEC_F16, DEC_UINT4_G32, DEC_INT4_SYM_G32 = 0, 1, 2, 3, 4
DEC_LOGITS_ALL, DEC_LOGITS_LAST, DEC_LOGITS_NONE = 0, 1, 2

ERROR_NAMES = {DEC_E_ARG: "DEC_E_ARG", DEC_E_UNSUPPORTED: "DEC_E_UNSUPPORTED", DEC_E_CAPACITY: "DEC_E_CAPACITY",
               DEC_E_BLOCK: "DEC_E_BLOCK", DEC_E_POSITION: "DEC_E_POSITION", DEC_E_TOKEN: "DEC_E_TOKEN",
               DEC_E_HIP: "DEC_E_HIP"}


class DecError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


class dec_config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ff_hidden", ctypes.c_int32),
        ("vocab", ctypes.c_int32), ("max_context", ctypes.c_int32), ("rms_eps", ctypes.c_float),
        ("rope_base", ctypes.c_double), ("rope_split", ctypes.c_int32), ("qk_norm", ctypes.c_int32),
        ("tie_embeddings", ctypes.c_int32), ("weight_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("block_tokens", ctypes.c_int32), ("n_blocks", ctypes.c_int32), ("max_rows", ctypes.c_int32),
        ("max_seqs", ctypes.c_int32),
    ]


class dec_weight_info(ctypes.Structure):
    _fields_ = [
        ("name", ctypes.c_char * 32), ("layer", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("offset", ctypes.c_size_t),
        ("bytes", ctypes.c_size_t), ("scale_offset", ctypes.c_size_t), ("zp_offset", ctypes.c_size_t),
        ("group_bytes", ctypes.c_size_t),
    ]


class dec_sampling(ctypes.Structure):
    _fields_ = [
        ("temperature", ctypes.c_double), ("top_p", ctypes.c_double), ("min_p", ctypes.c_double),
        ("repetition_penalty", ctypes.c_double), ("presence_penalty", ctypes.c_double),
        ("frequency_penalty", ctypes.c_double), ("top_k", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class dec_history(ctypes.Structure):
    _fields_ = [("prompt_offset", ctypes.c_int32), ("prompt_len", ctypes.c_int32),
                ("output_offset", ctypes.c_int32), ("output_len", ctypes.c_int32)]


DEC_PURPOSE_SAMPLE = 4
DEC_SAMPLE_MAX_NUCLEUS = 1024

EXPORTS = ["dec_check_config", "dec_weight_bytes", "dec_weight_count", "dec_weight_entry", "dec_kv_pool_bytes",
           "dec_workspace_bytes", "dec_init", "dec_free", "dec_last_error", "dec_prefill", "dec_decode_step",
           "dec_decode_step_static", "dec_check_step", "dec_debug_dequant", "dec_quantize_int4_sym", "dec_rng_stream", "dec_sample", "dec_pool_create",
           "dec_pool_destroy", "dec_pool_last_error", "dec_pool_alloc", "dec_pool_retain", "dec_pool_release",
           "dec_pool_set_fill", "dec_pool_register", "dec_pool_lookup", "dec_pool_block_info", "dec_pool_counts",
           "dec_prefix_key", "dec_kv_export_bytes", "dec_kv_export", "dec_kv_import", "dec_config_from_json",
           "dec_load_safetensors", "dec_timing_enable", "dec_timing_read"]

DEC_BLOCK_FREE, DEC_BLOCK_USED, DEC_BLOCK_CACHED = 0, 1, 2

KERNEL_CLASSES = ["embed", "rmsnorm", "gemm_qkv", "qk_rope_kv", "attn_prefill", "attn_rows", "attn_combine",
                  "gemm_o", "gemm_gateup", "gemm_down", "gemm_lmhead", "argmax"]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m decoder_forward_pass_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    cfgp = P(dec_config)
    i32p = P(ctypes.c_int32)
    sig = {
        "dec_check_config": (ctypes.c_int, [cfgp]),
        "dec_weight_bytes": (SZ, [cfgp]),
        "dec_weight_count": (ctypes.c_int, [cfgp]),
        "dec_weight_entry": (ctypes.c_int, [cfgp, ctypes.c_int, P(dec_weight_info)]),
        "dec_kv_pool_bytes": (SZ, [cfgp]),
        "dec_workspace_bytes": (SZ, [cfgp]),
        "dec_init": (ctypes.c_int, [cfgp, VP, SZ, VP, SZ, VP, SZ, VP, P(VP)]),
        "dec_free": (None, [VP]),
        "dec_last_error": (ctypes.c_char_p, [VP]),
        "dec_prefill": (ctypes.c_int, [VP, VP, I32, i32p, i32p, i32p, i32p, I32, I32, VP, VP]),
        "dec_decode_step": (ctypes.c_int, [VP, VP, I32, i32p, VP, i32p, i32p, I32, VP, VP]),
        "dec_decode_step_static": (ctypes.c_int, [VP, VP, I32, i32p, VP, i32p, i32p, I32, VP, VP]),
        "dec_check_step": (ctypes.c_int, [cfgp, I32, i32p, i32p, i32p, i32p, I32, I32, ctypes.c_char_p, SZ]),
        "dec_debug_dequant": (ctypes.c_int, [VP, VP, ctypes.c_int, VP]),
        "dec_quantize_int4_sym": (ctypes.c_int, [VP, VP, ctypes.c_int64, ctypes.c_int64, VP, VP]),
        "dec_rng_stream": (None, [ctypes.c_uint64, ctypes.c_uint64, P(ctypes.c_uint64)]),
        "dec_sample": (ctypes.c_int, [VP, VP, I32, VP, ctypes.c_int64, P(dec_sampling), P(dec_history), VP,
                                      ctypes.c_int64, VP, VP, VP]),
        "dec_pool_create": (ctypes.c_int, [I32, I32, I32, P(VP)]),
        "dec_pool_destroy": (None, [VP]),
        "dec_pool_last_error": (ctypes.c_char_p, [VP]),
        "dec_pool_alloc": (ctypes.c_int, [VP, I32, i32p]),
        "dec_pool_retain": (ctypes.c_int, [VP, I32]),
        "dec_pool_release": (ctypes.c_int, [VP, I32]),
        "dec_pool_set_fill": (ctypes.c_int, [VP, I32, I32]),
        "dec_pool_register": (ctypes.c_int, [VP, I32, ctypes.c_uint64, i32p]),
        "dec_pool_lookup": (ctypes.c_int, [VP, ctypes.c_uint64, i32p]),
        "dec_pool_block_info": (ctypes.c_int, [VP, I32, i32p, i32p, i32p]),
        "dec_pool_counts": (None, [VP, i32p, i32p, i32p]),
        "dec_prefix_key": (ctypes.c_uint64, [ctypes.c_uint64, i32p, I32]),
        "dec_kv_export_bytes": (SZ, [VP, I32]),
        "dec_kv_export": (ctypes.c_int, [VP, VP, i32p, i32p, I32, VP, SZ]),
        "dec_kv_import": (ctypes.c_int, [VP, VP, VP, SZ, i32p, I32, i32p]),
        "dec_config_from_json": (ctypes.c_int, [ctypes.c_char_p, SZ, cfgp, ctypes.c_char_p, SZ]),
        "dec_load_safetensors": (ctypes.c_int, [ctypes.c_char_p, cfgp, VP, SZ, ctypes.c_char_p, SZ]),
        "dec_timing_enable": (ctypes.c_int, [VP, ctypes.c_uint32]),
        "dec_timing_read": (ctypes.c_int, [VP, ctypes.c_int, P(ctypes.c_double), P(ctypes.c_int64)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()
lib = _lib


def _i32(a):
    """A C-contiguous int32 numpy array and its pointer (None stays NULL)."""
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _check(rc: int, ctx=None) -> None:
    if rc != DEC_OK:
        msg = _lib.dec_last_error(ctx)
        raise DecError(rc, msg.decode() if msg else "")


def dec_check_config(cfg: dec_config) -> None:
    _check(_lib.dec_check_config(ctypes.byref(cfg)))


def dec_weight_bytes(cfg: dec_config) -> int:
    n = _lib.dec_weight_bytes(ctypes.byref(cfg))
    if n == 0:
        _check(_lib.dec_check_config(ctypes.byref(cfg)))
    return n


def dec_weight_count(cfg: dec_config) -> int:
    return _lib.dec_weight_count(ctypes.byref(cfg))


def dec_weight_entry(cfg: dec_config, index: int) -> dec_weight_info:
    info = dec_weight_info()
    _check(_lib.dec_weight_entry(ctypes.byref(cfg), index, ctypes.byref(info)))
    return info


def dec_kv_pool_bytes(cfg: dec_config) -> int:
    return _lib.dec_kv_pool_bytes(ctypes.byref(cfg))


def dec_workspace_bytes(cfg: dec_config) -> int:
    return _lib.dec_workspace_bytes(ctypes.byref(cfg))


def dec_init(cfg: dec_config, weights: int, weight_bytes: int, kv_pool: int, kv_bytes: int, workspace: int,
             workspace_bytes: int, stream: int = 0) -> int:
    out = ctypes.c_void_p()
    _check(_lib.dec_init(ctypes.byref(cfg), weights, weight_bytes, kv_pool, kv_bytes, workspace, workspace_bytes,
                         stream or None, ctypes.byref(out)))
    return out.value


def dec_free(ctx: int) -> None:
    _lib.dec_free(ctx)


def dec_last_error(ctx) -> str:
    m = _lib.dec_last_error(ctx)
    return m.decode() if m else ""


def dec_prefill(ctx: int, stream: int, start, n_new, tokens, block_tables, logits_mode: int, logits: int,
                next_tokens: int = 0) -> None:
    _, sp = _i32(start)
    nn, np_ = _i32(n_new)
    _, tp = _i32(tokens)
    bt = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    if bt.ndim != 2:
        raise ValueError("block_tables must be [n_seqs, max_blocks]")
    bp = bt.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    _check(_lib.dec_prefill(ctx, stream or None, len(nn), sp, np_, tp, bp, bt.shape[1], logits_mode,
                            logits or None, next_tokens or None), ctx)


def dec_decode_step(ctx: int, stream: int, positions, block_tables, logits: int, next_tokens: int = 0,
                    tokens_host=None, tokens_device: int = 0, static: bool = False) -> None:
    """dec_decode_step, or dec_decode_step_static (scratch in the library's static device array)."""
    pos, pp = _i32(positions)
    _, tp = _i32(tokens_host)
    bt = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    bp = bt.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    fn = _lib.dec_decode_step_static if static else _lib.dec_decode_step
    _check(fn(ctx, stream or None, len(pos), tp, tokens_device or None, pp, bp, bt.shape[1], logits or None,
              next_tokens or None), ctx)


def dec_check_step(cfg: dec_config, start, n_new, tokens, block_tables, logits_mode: int):
    """Returns (code, message) without raising."""
    st, sp = _i32(start)
    _, np_ = _i32(n_new)
    _, tp = _i32(tokens)
    bt = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    if bt.ndim != 2:
        bt = bt.reshape(len(st), -1)
    bp = bt.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    buf = ctypes.create_string_buffer(512)
    rc = _lib.dec_check_step(ctypes.byref(cfg), len(st), sp, np_, tp, bp, bt.shape[1], logits_mode, buf, 512)
    return rc, buf.value.decode()


def dec_debug_dequant(ctx: int, stream: int, index: int, out: int) -> None:
    _check(_lib.dec_debug_dequant(ctx, stream or None, index, out), ctx)


def dec_quantize_int4_sym(stream: int, w: int, rows: int, cols: int, q: int, scale: int) -> None:
    """Device addresses: w float32 [rows][cols] -> q uint8 [rows][cols/2], scale f16 bits [rows][cols/32]."""
    _check(_lib.dec_quantize_int4_sym(stream or None, w, rows, cols, q, scale))


def dec_rng_stream(seed: int, purpose: int = DEC_PURPOSE_SAMPLE):
    """(state, increment) of the PCG32 stream(seed, purpose)."""
    out = (ctypes.c_uint64 * 2)()
    _lib.dec_rng_stream(seed & (2 ** 64 - 1), purpose, out)
    return int(out[0]), int(out[1])


def dec_sample(ctx: int, stream: int, logits: int, ld: int, params, history, ids: int, n_ids: int, rng: int,
               next_ids: int, logprob: int = 0) -> None:
    """params: sequence of dec_sampling; history: sequence of dec_history (host); the rest device addresses."""
    n = len(params)
    if len(history) != n:
        raise ValueError("params and history must have one entry per sequence")
    pa = (dec_sampling * n)(*params)
    ha = (dec_history * n)(*history)
    _check(_lib.dec_sample(ctx, stream or None, n, logits, ld, pa, ha, ids or None, n_ids, rng, next_ids,
                           logprob or None), ctx)


class BlockPool:
    """The library's KV block manager (dec_pool_*): one method per C call, errors as DecError."""

    def __init__(self, n_blocks: int, block_tokens: int, prefix_cache: bool = True):
        h = ctypes.c_void_p()
        rc = _lib.dec_pool_create(n_blocks, block_tokens, int(prefix_cache), ctypes.byref(h))
        if rc != DEC_OK:
            raise DecError(rc, "dec_pool_create refused the configuration")
        self.h = h.value

    def _check(self, rc):
        if rc != DEC_OK:
            msg = _lib.dec_pool_last_error(self.h)
            raise DecError(rc, msg.decode() if msg else "")

    def close(self):
        if self.h:
            _lib.dec_pool_destroy(self.h)
            self.h = None

    def alloc(self, n: int) -> list:
        ids = (ctypes.c_int32 * max(n, 1))()
        self._check(_lib.dec_pool_alloc(self.h, n, ids))
        return list(ids[:n])

    def retain(self, i: int):
        self._check(_lib.dec_pool_retain(self.h, i))

    def release(self, i: int):
        self._check(_lib.dec_pool_release(self.h, i))

    def set_fill(self, i: int, n: int):
        self._check(_lib.dec_pool_set_fill(self.h, i, n))

    def register(self, i: int, key: int) -> int:
        c = ctypes.c_int32(-1)
        self._check(_lib.dec_pool_register(self.h, i, key, ctypes.byref(c)))
        return c.value

    def lookup(self, key: int) -> int:
        c = ctypes.c_int32(-1)
        self._check(_lib.dec_pool_lookup(self.h, key, ctypes.byref(c)))
        return c.value

    def info(self, i: int):
        st, ref, fill = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        self._check(_lib.dec_pool_block_info(self.h, i, ctypes.byref(st), ctypes.byref(ref), ctypes.byref(fill)))
        return st.value, ref.value, fill.value

    def counts(self):
        f, u, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _lib.dec_pool_counts(self.h, ctypes.byref(f), ctypes.byref(u), ctypes.byref(c))
        return f.value, u.value, c.value


def dec_prefix_key(parent: int, tokens) -> int:
    arr, p = _i32(tokens)
    return int(_lib.dec_prefix_key(parent & (2 ** 64 - 1), p, len(arr)))


def dec_kv_export(ctx: int, stream: int, ids, fills) -> bytes:
    ia, ip = _i32(ids)
    fa, fp = _i32(fills)
    n = len(ia)
    size = _lib.dec_kv_export_bytes(ctx, n)
    buf = ctypes.create_string_buffer(size)
    _check(_lib.dec_kv_export(ctx, stream or None, ip, fp, n, buf, size), ctx)
    return buf.raw


def dec_kv_import(ctx: int, stream: int, data: bytes, ids):
    ia, ip = _i32(ids)
    n = len(ia)
    fills = (ctypes.c_int32 * n)()
    _check(_lib.dec_kv_import(ctx, stream or None, data, len(data), ip, n, fills), ctx)
    return list(fills)


def dec_config_from_json(text: bytes, cfg: dec_config) -> None:
    """Fill cfg's shape fields from a config.json's bytes; DecError on a refusal."""
    buf = ctypes.create_string_buffer(512)
    rc = _lib.dec_config_from_json(text, len(text), ctypes.byref(cfg), buf, 512)
    if rc != DEC_OK:
        raise DecError(rc, buf.value.decode())


def dec_load_safetensors(path: str, cfg: dec_config) -> np.ndarray:
    """The weights blob (host uint8 array) read from a model.safetensors file; DecError on a refusal."""
    n = dec_weight_bytes(cfg)
    blob = np.zeros(n, dtype=np.uint8)
    buf = ctypes.create_string_buffer(512)
    rc = _lib.dec_load_safetensors(os.fsencode(path), ctypes.byref(cfg), blob.ctypes.data, n, buf, 512)
    if rc != DEC_OK:
        raise DecError(rc, buf.value.decode())
    return blob


def dec_timing_enable(ctx: int, class_mask: int) -> None:
    _check(_lib.dec_timing_enable(ctx, class_mask), ctx)


def dec_timing_read(ctx: int, kernel_class: int):
    """(total milliseconds, launches) of the recorded launches of one kernel class."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(_lib.dec_timing_read(ctx, kernel_class, ctypes.byref(ms), ctypes.byref(n)), ctx)
    return ms.value, n.value
