"""ctypes binding of libdory.so (argument marshalling only).

Every step of the forward pass runs in the library's HIP kernels; PyTorch only
allocates device memory (weights, KV pool, workspace, inputs, outputs) and
provides the stream. The library must be built (``python -m
looped_ngpt_language_amd.build``); there is no fallback: a missing or
unloadable library raises at first use.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import synth

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdory.so")
CHECKED_LIB_PATH = os.path.join(_HERE, "libdory_checked.so")
# bytes past the KV pool that a checked-build context keeps unused, so that a page id one past the
# pool (the guard tests' injected fault) stays inside the allocation even before the guard clamps it
CHECKED_POOL_GUARD = 1 << 20

DORY_OK, DORY_E_INVALID, DORY_E_STATE, DORY_E_NOMEM, DORY_E_HIP = 0, -1, -2, -3, -4
KV_MODES = {"per_loop": 0, "last_loop": 1}
FLAG_DRY_RUN = 1
FLAG_MXFP8_GEMV = 4
FLAG_SWA_RECYCLE = 8
FLAG_MXFP4_GEMV = 16


class DoryError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class Config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("d_model", "n_heads", "n_kv_heads", "head_dim", "d_ff", "vocab", "n_in",
                                         "n_rec", "n_out", "full_every", "window", "dtype", "page_size", "max_seqs",
                                         "max_model_len", "max_loops", "max_tokens")] + \
              [("flags", C.c_uint32), ("rope_theta", C.c_float), ("attn_scale", C.c_float)]


class WeightsC(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("lm_head", C.c_void_p), ("w_qkv", C.POINTER(C.c_void_p)),
                ("w_o", C.POINTER(C.c_void_p)), ("w_gu", C.POINTER(C.c_void_p)), ("w_down", C.POINTER(C.c_void_p)),
                ("alpha_attn", C.POINTER(C.c_void_p)), ("alpha_mlp", C.POINTER(C.c_void_p))]


class Stats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("calls", "block_apps", "sublayer_apps", "full_apps", "swa_apps",
                                         "kernel_launches")] + \
              [(n, C.c_int32) for n in ("n_slots", "pages_total", "pages_in_use", "live_seqs", "swa_pages_total",
                                        "swa_pages_in_use", "max_attn_splits")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class KernelTime(C.Structure):
    _fields_ = [("name", C.c_char * 32), ("launches", C.c_int64), ("bytes", C.c_double), ("flops", C.c_double),
                ("timed_launches", C.c_int64), ("total_ms", C.c_double)]


class SpecStats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("rounds", "drafted", "accepted", "produced")] + \
              [(n, C.c_double) for n in ("draft_ms", "verify_ms")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


EXPORTS = {
    "dory_query_sizes": (C.c_int, [C.POINTER(Config), C.c_int32, C.c_int64, C.POINTER(C.c_size_t),
                                   C.POINTER(C.c_size_t)]),
    "dory_create": (C.c_int, [C.POINTER(Config), C.POINTER(WeightsC), C.c_int32, C.c_void_p, C.c_size_t, C.c_void_p,
                              C.c_size_t, C.c_void_p, C.POINTER(C.c_void_p)]),
    "dory_destroy": (None, [C.c_void_p]),
    "dory_set_loops": (C.c_int, [C.c_void_p, C.c_int32]),
    "dory_get_loops": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32)]),
    "dory_kv_mode": (C.c_int, [C.c_void_p, C.c_int32]),
    "dory_prefill": (C.c_int, [C.c_void_p, C.c_int32, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]),
    "dory_decode": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_int32), C.c_void_p, C.c_void_p, C.c_void_p]),
    "dory_seq_truncate": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32]),
    "dory_seq_release": (C.c_int, [C.c_void_p, C.c_int32]),
    "dory_seq_len": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_int32)]),
    "dory_kv_bytes_in_use": (C.c_int, [C.c_void_p, C.POINTER(C.c_size_t)]),
    "dory_get_stats": (C.c_int, [C.c_void_p, C.POINTER(Stats)]),
    "dory_last_hidden": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32]),
    "dory_device_flags": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.c_int32]),
    "dory_checked_build": (C.c_int32, []),
    "dory_debug_set_page": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_int32)]),
    "dory_quantize_mxfp8": (C.c_int, [C.c_void_p, C.c_int64, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]),
    "dory_quantize_mxfp4": (C.c_int, [C.c_void_p, C.c_int64, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]),
    "dory_sample": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_float, C.c_float, C.c_void_p, C.c_void_p,
                              C.c_void_p]),
    "dory_sample_static": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_float, C.c_float, C.c_void_p,
                                     C.c_void_p, C.c_void_p]),
    "dory_sample_scratch_bytes": (C.c_size_t, [C.c_int32, C.c_int32]),
    "dory_spec_decode": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                   C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
    "dory_get_spec_stats": (C.c_int, [C.c_void_p, C.POINTER(SpecStats), C.c_int32]),
    "dory_set_timing": (C.c_int, [C.c_void_p, C.c_int32]),
    "dory_get_timing": (C.c_int, [C.c_void_p, C.POINTER(KernelTime), C.c_int32, C.POINTER(C.c_int32), C.c_int32]),
    "dory_last_error": (C.c_char_p, [C.c_void_p]),
    "dory_status_string": (C.c_char_p, [C.c_int32]),
}

_libs = {}


def lib(checked: bool = False):
    """Load libdory.so (or, checked=True, its bounds-checked debug build libdory_checked.so) once;
    raise if it is missing (no fallback path exists)."""
    checked = bool(checked)
    if checked not in _libs:
        path = CHECKED_LIB_PATH if checked else LIB_PATH
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; run python -m looped_ngpt_language_amd.build")
        L = C.CDLL(path)
        for name, (res, args) in EXPORTS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _libs[checked] = L
    return _libs[checked]


def make_config(shape: synth.ModelShape, *, max_seqs=1, max_model_len=4096, max_loops=4, max_tokens=4096,
                dry_run=False, gemv_weights="bf16", swa_recycle=False) -> Config:
    if gemv_weights not in ("bf16", "mxfp8", "mxfp4"):
        raise ValueError(gemv_weights)
    return Config(d_model=shape.d_model, n_heads=shape.n_heads, n_kv_heads=shape.n_kv_heads,
                  head_dim=shape.head_dim, d_ff=shape.d_ff, vocab=shape.vocab, n_in=shape.n_in, n_rec=shape.n_rec,
                  n_out=shape.n_out, full_every=shape.full_every, window=shape.window,
                  dtype=0 if shape.dtype == synth.F32 else 1, page_size=shape.page_size, max_seqs=max_seqs,
                  max_model_len=max_model_len, max_loops=max_loops, max_tokens=max_tokens,
                  flags=(FLAG_DRY_RUN if dry_run else 0) | (FLAG_MXFP8_GEMV if gemv_weights == "mxfp8" else 0)
                  | (FLAG_MXFP4_GEMV if gemv_weights == "mxfp4" else 0)
                  | (FLAG_SWA_RECYCLE if swa_recycle else 0),
                  rope_theta=shape.rope_theta, attn_scale=shape.scale)


def query_sizes(cfg: Config, kv_mode: str, kv_tokens: int, checked: bool = False):
    kv = C.c_size_t()
    ws = C.c_size_t()
    st = lib(checked).dory_query_sizes(C.byref(cfg), KV_MODES[kv_mode], int(kv_tokens), C.byref(kv), C.byref(ws))
    if st != DORY_OK:
        raise DoryError(st, "dory_query_sizes rejected the configuration")
    return kv.value, ws.value


def quantize_mxfp8(w, stream=None):
    """bf16 device tensor [rows, cols] -> (codes uint8 [rows, cols], scales uint8 [rows, cols/32]) on its device."""
    import torch
    rows, cols = w.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=w.device)
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=w.device)
    st = stream if stream is not None else torch.cuda.current_stream(w.device)
    r = lib().dory_quantize_mxfp8(_ptr(w), int(rows), int(cols), _ptr(codes), _ptr(scales), C.c_void_p(st.cuda_stream))
    if r != DORY_OK:
        raise DoryError(r, "dory_quantize_mxfp8 rejected its arguments")
    return codes, scales


def quantize_mxfp4(w, stream=None):
    """bf16 device tensor [rows, cols] -> (codes uint8 [rows, cols/2], two per byte with element 2i in the
    low nibble, scales uint8 [rows, cols/32]) on its device."""
    import torch
    rows, cols = w.shape
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=w.device)
    st = stream if stream is not None else torch.cuda.current_stream(w.device)
    r = lib().dory_quantize_mxfp4(_ptr(w), int(rows), int(cols), _ptr(codes), _ptr(scales), C.c_void_p(st.cuda_stream))
    if r != DORY_OK:
        raise DoryError(r, "dory_quantize_mxfp4 rejected its arguments")
    return codes, scales


def sample(logits, uniforms, temperature=1.0, top_p=0.95, stream=None, static_scratch=False, ids=None):
    """fp32 device logits [rows, V] and uniforms [rows] -> int32 ids [rows] (temperature / top-p draw).
    static_scratch=True calls dory_sample_static (no allocation inside the library); `ids` may be
    a preallocated int32 device tensor [rows]."""
    import torch
    rows, vocab = logits.shape
    if logits.dtype != torch.float32 or uniforms.dtype != torch.float32 or not logits.is_contiguous():
        raise DoryError(DORY_E_INVALID, "sample needs contiguous fp32 logits and fp32 uniforms")
    if uniforms.numel() != rows or uniforms.device != logits.device:
        raise DoryError(DORY_E_INVALID, "one uniform per row, on the logits' device")
    if ids is None:
        ids = torch.empty(rows, dtype=torch.int32, device=logits.device)
    st = stream if stream is not None else torch.cuda.current_stream(logits.device)
    u = uniforms.contiguous()
    fn = lib().dory_sample_static if static_scratch else lib().dory_sample
    r = fn(_ptr(logits), int(rows), int(vocab), float(temperature), float(top_p), _ptr(u),
           _ptr(ids), C.c_void_p(st.cuda_stream))
    if r != DORY_OK:
        raise DoryError(r, "dory_sample rejected its arguments")
    if st != torch.cuda.current_stream(logits.device):
        for t in (logits, u, ids):  # allocated on the current stream, used on the sampler's
            t.record_stream(st)
    return ids


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _device_matrix(a: np.ndarray, dtype: str, device):
    import torch
    if dtype == synth.BF16:
        bits = synth.to_bf16_bits(a).view(np.int16)
        return torch.from_numpy(bits).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


class Model:
    """One looped nGPT context on one GPU (or a host-only dry-run context)."""

    def __init__(self, shape: synth.ModelShape, weights=None, *, kv_mode="per_loop", max_loops=4, max_seqs=1,
                 max_model_len=4096, max_tokens=None, kv_tokens=None, device="cuda:0", dry_run=False, stream=None,
                 share_weights_from=None, gemv_weights="bf16", swa_recycle=False, checked=False):
        """gemv_weights="mxfp8" / "mxfp4": calls of at most 2 rows stream MXFP8 / MXFP4 copies of the weights.
        swa_recycle: sliding-window layers keep only the pages their window (plus a 64-token
        rollback reserve) can reach; kv_tokens then sizes the full-attention pages.
        checked: run on the bounds-checked debug build (libdory_checked.so)."""
        self._L = lib(checked)
        self.checked = bool(checked)
        self.shape = shape
        self.dry = dry_run
        max_tokens = max_tokens or max_model_len
        self.cfg = make_config(shape, max_seqs=max_seqs, max_model_len=max_model_len, max_loops=max_loops,
                               max_tokens=max_tokens, dry_run=dry_run, gemv_weights=gemv_weights,
                               swa_recycle=swa_recycle)
        kv_tokens = kv_tokens if kv_tokens is not None else max_seqs * (max_model_len + 16)
        kv_bytes, ws_bytes = query_sizes(self.cfg, kv_mode, kv_tokens, checked)
        self.kv_bytes, self.ws_bytes = kv_bytes, ws_bytes
        self._keep = []
        ctx = C.c_void_p()
        if dry_run:
            st = self._L.dory_create(C.byref(self.cfg), None, KV_MODES[kv_mode], None, kv_bytes, None, ws_bytes, None,
                                   C.byref(ctx))
        else:
            import torch
            self.device = torch.device(device)
            self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
            wc = self._share_weights(share_weights_from) if share_weights_from else self._upload_weights(weights)
            pad = CHECKED_POOL_GUARD if checked else 0
            self.pool = torch.empty(max(kv_bytes, 256) + pad, dtype=torch.uint8, device=self.device)
            self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=self.device)
            st = self._L.dory_create(C.byref(self.cfg), C.byref(wc), KV_MODES[kv_mode], _ptr(self.pool), kv_bytes,
                                   _ptr(self.ws), ws_bytes, C.c_void_p(self.stream.cuda_stream), C.byref(ctx))
        if st != DORY_OK:
            raise DoryError(st, "dory_create failed")
        self.ctx = ctx

    # -- weights ------------------------------------------------------------
    def _share_weights(self, other):
        """Use the device weights another context already holds (same shape)."""
        assert other.shape == self.shape
        self.w_embed, self.w_lm, self.w_blocks = other.w_embed, other.w_lm, other.w_blocks
        arrs = other._keep[0]
        self._keep.append(arrs)
        return WeightsC(embed=_ptr(self.w_embed), lm_head=_ptr(self.w_lm), w_qkv=arrs["qkv"], w_o=arrs["o"],
                        w_gu=arrs["gu"], w_down=arrs["d"], alpha_attn=arrs["aa"], alpha_mlp=arrs["am"])

    def _upload_weights(self, w):
        import torch
        s = self.shape
        dev = self.device
        if w is None:
            raise ValueError("weights are required")
        blocks = []
        for blk in w.blocks:
            qkv = np.concatenate([blk["wq"], blk["wk"], blk["wv"]], axis=0)
            gu = np.concatenate([blk["wg"], blk["wu"]], axis=0)
            blocks.append({"qkv": _device_matrix(qkv, s.dtype, dev), "o": _device_matrix(blk["wo"], s.dtype, dev),
                           "gu": _device_matrix(gu, s.dtype, dev), "d": _device_matrix(blk["wd"], s.dtype, dev),
                           "aa": torch.from_numpy(np.asarray(blk["alpha_attn"], np.float32)).to(dev),
                           "am": torch.from_numpy(np.asarray(blk["alpha_mlp"], np.float32)).to(dev)})
        self.w_embed = _device_matrix(w.embed, s.dtype, dev)
        self.w_lm = _device_matrix(w.lm_head, s.dtype, dev)
        self.w_blocks = blocks
        n = len(blocks)
        arrs = {}
        for key in ("qkv", "o", "gu", "d", "aa", "am"):
            arrs[key] = (C.c_void_p * n)(*[_ptr(b[key]) for b in blocks])
        self._keep.append(arrs)
        return WeightsC(embed=_ptr(self.w_embed), lm_head=_ptr(self.w_lm), w_qkv=arrs["qkv"], w_o=arrs["o"],
                        w_gu=arrs["gu"], w_down=arrs["d"], alpha_attn=arrs["aa"], alpha_mlp=arrs["am"])

    # -- helpers ------------------------------------------------------------
    def _check(self, st, what):
        if st != DORY_OK:
            msg = self._L.dory_last_error(self.ctx)
            raise DoryError(st, f"{what}: {msg.decode() if msg else ''}")

    def _tokens(self, tokens):
        import torch
        if isinstance(tokens, torch.Tensor):
            t = tokens.to(self.device, torch.int32).contiguous()
        else:
            t = torch.from_numpy(np.ascontiguousarray(tokens, dtype=np.int32)).to(self.device)
        return t

    def _hold(self, *tensors):
        """Device tensors a call reads or writes were allocated on torch's current stream; when the
        library runs on another stream, tell the caching allocator so their memory is not handed
        out again before that stream's kernels are done with it."""
        import torch
        if self.stream != torch.cuda.current_stream(self.device):
            for t in tensors:
                if t is not None:
                    t.record_stream(self.stream)

    def close(self):
        if getattr(self, "ctx", None):
            self._L.dory_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- calls --------------------------------------------------------------
    def set_loops(self, k: int):
        self._check(self._L.dory_set_loops(self.ctx, int(k)), "dory_set_loops")

    def loops(self) -> int:
        k = C.c_int32()
        self._check(self._L.dory_get_loops(self.ctx, C.byref(k)), "dory_get_loops")
        return k.value

    def set_kv_mode(self, mode: str):
        self._check(self._L.dory_kv_mode(self.ctx, KV_MODES[mode]), "dory_kv_mode")

    def prefill(self, seq_id: int, tokens, logits_rows: int = 1, logits=None, ids=True):
        """Returns (logits [rows, V] fp32 device tensor, ids [rows] int32 device tensor or None)."""
        n = len(tokens)
        if self.dry:
            st = self._L.dory_prefill(self.ctx, seq_id, None, n, logits_rows, None, None)
            self._check(st, "dory_prefill")
            return None, None
        import torch
        tok = self._tokens(tokens)
        if logits is None:
            logits = torch.empty((logits_rows, self.shape.vocab), dtype=torch.float32, device=self.device)
        out_ids = torch.empty(logits_rows, dtype=torch.int32, device=self.device) if ids else None
        st = self._L.dory_prefill(self.ctx, int(seq_id), _ptr(tok), n, int(logits_rows), _ptr(logits), _ptr(out_ids))
        self._check(st, "dory_prefill")
        self._hold(tok, logits, out_ids)
        self._keep_call = tok
        return logits, out_ids

    def decode(self, seq_ids, tokens, logits=True, out_ids=None):
        """One token per listed sequence. tokens: device int32 tensor (or array) [n]."""
        sids = (C.c_int32 * len(seq_ids))(*[int(s) for s in seq_ids])
        n = len(seq_ids)
        if self.dry:
            self._check(self._L.dory_decode(self.ctx, n, sids, None, None, None), "dory_decode")
            return None, None
        import torch
        tok = self._tokens(tokens)
        lg = torch.empty((n, self.shape.vocab), dtype=torch.float32, device=self.device) if logits is True else logits
        if out_ids is None:
            out_ids = torch.empty(n, dtype=torch.int32, device=self.device)
        st = self._L.dory_decode(self.ctx, n, sids, _ptr(tok), _ptr(lg) if lg is not None else None, _ptr(out_ids))
        self._check(st, "dory_decode")
        self._hold(tok, lg, out_ids)
        self._keep_call = tok
        return lg, out_ids

    def truncate(self, seq_id: int, new_len: int):
        self._check(self._L.dory_seq_truncate(self.ctx, int(seq_id), int(new_len)), "dory_seq_truncate")

    def release(self, seq_id: int):
        self._check(self._L.dory_seq_release(self.ctx, int(seq_id)), "dory_seq_release")

    def seq_len(self, seq_id: int) -> int:
        n = C.c_int32()
        self._check(self._L.dory_seq_len(self.ctx, int(seq_id), C.byref(n)), "dory_seq_len")
        return n.value

    def kv_bytes_in_use(self) -> int:
        b = C.c_size_t()
        self._check(self._L.dory_kv_bytes_in_use(self.ctx, C.byref(b)), "dory_kv_bytes_in_use")
        return b.value

    def stats(self) -> dict:
        s = Stats()
        self._check(self._L.dory_get_stats(self.ctx, C.byref(s)), "dory_get_stats")
        return s.as_dict()

    def last_hidden(self, rows: int):
        import torch
        out = torch.empty((rows, self.shape.d_model), dtype=torch.float32, device=self.device)
        self._check(self._L.dory_last_hidden(self.ctx, _ptr(out), int(rows)), "dory_last_hidden")
        self._hold(out)
        return out

    def device_flags(self, reset=True) -> int:
        """Device error flags (bit 0: an out-of-range token id was clamped; checked build also bit 1: a
        page-table index, bit 2: a page id, bit 3: a RoPE position out of range)."""
        v = C.c_int32()
        self._check(self._L.dory_device_flags(self.ctx, C.byref(v), int(reset)), "dory_device_flags")
        return v.value

    def debug_set_page(self, seq_id: int, page_index: int, page_id: int) -> int:
        """Checked build only: overwrite one device page-table entry; returns the previous entry."""
        old = C.c_int32()
        self._check(self._L.dory_debug_set_page(self.ctx, int(seq_id), int(page_index), int(page_id), C.byref(old)),
                    "dory_debug_set_page")
        return old.value

    def set_timing(self, enable: bool):
        self._check(self._L.dory_set_timing(self.ctx, 1 if enable else 0), "dory_set_timing")

    def timing(self, reset: bool = False) -> dict:
        """Per kernel role: launches, algorithmic bytes/flops, timed launches and milliseconds."""
        buf = (KernelTime * 32)()
        n = C.c_int32()
        self._check(self._L.dory_get_timing(self.ctx, buf, 32, C.byref(n), 1 if reset else 0), "dory_get_timing")
        out = {}
        for i in range(min(n.value, 32)):
            e = buf[i]
            out[e.name.decode()] = {"launches": e.launches, "bytes": e.bytes, "flops": e.flops,
                                    "timed_launches": e.timed_launches, "ms": e.total_ms}
        return out

    def spec_stats(self, reset: bool = False) -> dict:
        """Counters of spec_decode since the last reset: rounds, drafted, accepted, produced,
        draft_ms and verify_ms (GPU time of the two phases)."""
        s = SpecStats()
        self._check(self._L.dory_get_spec_stats(self.ctx, C.byref(s), 1 if reset else 0), "dory_get_spec_stats")
        return s.as_dict()

    def spec_decode(self, seq_id: int, last: int, n_new: int, gamma=4, k_draft=1, k_verify=4, reuse=False):
        """reuse=True (k_draft 1): the verify pass reuses the draft's input-stack output, loop-1
        state and cache instead of recomputing them."""
        buf = (C.c_int32 * (n_new + gamma + 1))()
        n = C.c_int32()
        st = self._L.dory_spec_decode(self.ctx, int(seq_id), int(last), int(n_new), int(gamma), int(k_draft),
                                    int(k_verify), int(bool(reuse)), buf, C.byref(n))
        self._check(st, "dory_spec_decode")
        return np.array(buf[:n.value], dtype=np.int32)
