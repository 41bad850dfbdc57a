"""Python binding of libsf, the Summaryformer per-block memory on MI355X.

Thin ctypes marshalling over the C-ABI declared in include/sf.h: the functions
here carry the C names and do no arithmetic of the method; every step runs in
the library's gfx950 kernels.  Device memory and streams come from PyTorch
(tensors' data pointers, torch.cuda streams).  Importing fails loudly when the
library has not been built (python compressed_memory_kv_amd/build.py); there is
no fallback path.

Model card "GTA world model: weights and inference code", section "One buffer,
no mask": one preallocated K/V buffer per block, Z0 | RAW | SUM, fed by
eviction and read by one dense, unmasked attention.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# SF_LIB_PATH points the binding at another build of the same C-ABI (e.g. a tuning build).
LIB_PATH = os.environ.get("SF_LIB_PATH") or os.path.join(_HERE, "libsf.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python compressed_memory_kv_amd/build.py` "
                      "(the HIP library is the only implementation; there is no fallback)")
_lib = ctypes.CDLL(LIB_PATH)

SF_OK, SF_E_ARG, SF_E_ORDER, SF_E_RANGE, SF_E_STATE, SF_E_HIP, SF_E_UNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
SF_F32, SF_BF16 = 0, 1
SF_MAX_SEGMENTS = 4
SF_MAX_BATCH = 64
DTYPES = {"f32": SF_F32, "bf16": SF_BF16}

EXPORTED = (
    "sf_config_check", "sf_buffer_bytes", "sf_kv_bytes", "sf_kv_offset", "sf_buffer_create",
    "sf_buffer_destroy", "sf_write_record", "sf_evict", "sf_attend", "sf_step", "sf_query", "sf_plan",
    "sf_status_str", "sf_last_error", "sf_debug_fail_next_launch", "sf_profile_enable", "sf_kernel_times_read",
    "sf_record_slot", "sf_commit_record", "sf_state_bytes", "sf_state_export", "sf_state_import", "sf_rope_rows",
    "sf_set_recency_bias", "sf_attend_static_scratch", "sf_debug_lds_copy", "sf_debug_range_form",
)
(SF_K_FILL, SF_K_WRITE, SF_K_EVICT, SF_K_ATTEND, SF_K_COMBINE, SF_K_TAIL, SF_K_SINK, SF_K_ROPE, SF_K_BIAS,
 SF_K_KINDS) = range(10)
KERNEL_KINDS = ("fill", "write", "evict", "attend", "combine", "tail", "sink", "rope", "bias")
SF_ROPE_CALLER, SF_ROPE_LEVEL_REPLACE, SF_ROPE_LEVEL_ADD = 0, 1, 2
ROPE_MODES = {"caller": SF_ROPE_CALLER, "replace": SF_ROPE_LEVEL_REPLACE, "add": SF_ROPE_LEVEL_ADD}


class sf_config(ctypes.Structure):
    _fields_ = [("hw", ctypes.c_int32), ("x", ctypes.c_int32), ("y", ctypes.c_int32), ("w", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("n_blocks", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("max_frames", ctypes.c_int64), ("sink_gap", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("rope_mode", ctypes.c_int32), ("recency_bias", ctypes.c_int32)]


class sf_view(ctypes.Structure):
    _fields_ = [("t_cur", ctypes.c_int64), ("n_keys", ctypes.c_int64), ("evicted_for", ctypes.c_int64),
                ("n_seg", ctypes.c_int32), ("raw_slot", ctypes.c_int32), ("blocks_written", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("seg_begin", ctypes.c_int64 * SF_MAX_SEGMENTS),
                ("seg_len", ctypes.c_int64 * SF_MAX_SEGMENTS), ("raw_frame", ctypes.POINTER(ctypes.c_int64)),
                ("sum_frame", ctypes.POINTER(ctypes.c_int64)), ("z0_frame", ctypes.c_int64)]


class sf_kernel_times(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * SF_K_KINDS), ("launches", ctypes.c_int64 * SF_K_KINDS)]


_P = ctypes.c_void_p
_CFG = ctypes.POINTER(sf_config)
_sig = {
    "sf_config_check": (ctypes.c_int, [_CFG]),
    "sf_buffer_bytes": (ctypes.c_size_t, [_CFG]),
    "sf_kv_bytes": (ctypes.c_size_t, [_CFG]),
    "sf_kv_offset": (ctypes.c_int64, [_CFG, ctypes.c_int32, ctypes.c_int32]),
    "sf_buffer_create": (ctypes.c_int, [_CFG, _P, ctypes.c_size_t, _P, ctypes.POINTER(_P)]),
    "sf_buffer_destroy": (ctypes.c_int, [_P]),
    "sf_write_record": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int64, _P, _P, _P]),
    "sf_evict": (ctypes.c_int, [_P, ctypes.c_int64, _P]),
    "sf_attend": (ctypes.c_int, [ctypes.POINTER(_P), ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_P),
                                 ctypes.POINTER(_P), ctypes.c_float, _P]),
    "sf_step": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int64, _P, _P, _P, _P, ctypes.c_float, _P]),
    "sf_query": (ctypes.c_int, [_P, ctypes.POINTER(sf_view)]),
    "sf_plan": (ctypes.c_int, [_CFG, ctypes.c_int64, ctypes.POINTER(sf_view)]),
    "sf_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "sf_last_error": (ctypes.c_char_p, [_P]),
    "sf_debug_fail_next_launch": (ctypes.c_int, [_P]),
    "sf_debug_lds_copy": (ctypes.c_int, [_P, _P, ctypes.c_size_t, _P]),
    "sf_debug_range_form": (ctypes.c_int, [ctypes.c_int32]),
    "sf_profile_enable": (ctypes.c_int, [_P, ctypes.c_int32]),
    "sf_kernel_times_read": (ctypes.c_int, [_P, ctypes.POINTER(sf_kernel_times)]),
    "sf_record_slot": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(_P), ctypes.POINTER(_P)]),
    "sf_commit_record": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int64]),
    "sf_state_bytes": (ctypes.c_size_t, [_CFG]),
    "sf_state_export": (ctypes.c_int, [_P, _P, ctypes.c_size_t]),
    "sf_state_import": (ctypes.c_int, [_P, _P, ctypes.c_size_t]),
    "sf_rope_rows": (ctypes.c_int, [_CFG, ctypes.c_int64, _P, _P, _P]),
    "sf_set_recency_bias": (ctypes.c_int, [_P, _P, _P]),
    "sf_attend_static_scratch": (ctypes.c_int, [ctypes.POINTER(_P), ctypes.c_int32, ctypes.c_int32,
                                                ctypes.POINTER(_P), ctypes.POINTER(_P), ctypes.c_float, _P]),
}
for _name, (_res, _args) in _sig.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class SfError(RuntimeError):
    """A libsf call returned a negative sf_status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_lib.sf_status_str(status).decode()}: {message}")
        self.status = status


def _check(status: int, handle=None):
    if status != SF_OK:
        raise SfError(status, (_lib.sf_last_error(handle) or b"").decode())


def _ptr(x) -> int | None:
    """Device address of a torch tensor, or an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s) -> int | None:
    if s is None:
        try:
            import torch
            if torch.cuda.is_available():
                return torch.cuda.current_stream().cuda_stream
        except Exception:  # torch missing: the default stream
            pass
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def make_config(hw, x, y, w, n_heads, head_dim, n_blocks=1, dtype="bf16", max_frames=0, sink_gap=0,
                rope_theta=10000.0, rope_mode="caller", recency_bias=False, **_ignored) -> sf_config:
    """sf_config from keyword fields (extra keys, e.g. of a workload dict, are ignored).
    rope_mode: "caller", "replace" or "add" (or the SF_ROPE_* value); recency_bias: a bias
    table (sf_set_recency_bias) on summary keys."""
    return sf_config(hw, x, y, w, n_heads, head_dim, n_blocks, DTYPES[dtype] if isinstance(dtype, str) else dtype,
                     max_frames, sink_gap, rope_theta,
                     ROPE_MODES[rope_mode] if isinstance(rope_mode, str) else rope_mode, int(bool(recency_bias)))


# --------------------------------------------------------------- the C calls
def sf_config_check(cfg: sf_config) -> None:
    _check(_lib.sf_config_check(ctypes.byref(cfg)))


def sf_buffer_bytes(cfg: sf_config) -> int:
    return _lib.sf_buffer_bytes(ctypes.byref(cfg))


def sf_kv_bytes(cfg: sf_config) -> int:
    return _lib.sf_kv_bytes(ctypes.byref(cfg))


def sf_kv_offset(cfg: sf_config, block: int, which: int) -> int:
    return _lib.sf_kv_offset(ctypes.byref(cfg), block, which)


def sf_buffer_create(cfg: sf_config, dev_mem=None, nbytes: int = 0, stream=None) -> int:
    """Returns the handle (an address).  dev_mem None with nbytes 0 makes a dry-run handle."""
    h = _P()
    _check(_lib.sf_buffer_create(ctypes.byref(cfg), _ptr(dev_mem), nbytes,
                                 _stream(stream) if dev_mem is not None else None, ctypes.byref(h)))
    return h.value


def sf_buffer_destroy(handle: int) -> None:
    _check(_lib.sf_buffer_destroy(handle))


def sf_write_record(handle: int, block: int, t: int, k, v, stream=None) -> None:
    _check(_lib.sf_write_record(handle, block, t, _ptr(k), _ptr(v), _stream(stream)), handle)


def sf_evict(handle: int, t: int, stream=None) -> None:
    _check(_lib.sf_evict(handle, t, _stream(stream)), handle)


def sf_attend(handles, block: int, q, out, scale: float = 0.0, stream=None) -> None:
    """Batched dense read: handles, q and out are equal-length sequences (one per session)."""
    n = len(handles)
    hs = (_P * n)(*handles)
    qs = (_P * n)(*[_ptr(x) for x in q]) if q is not None else None
    os_ = (_P * n)(*[_ptr(x) for x in out]) if out is not None else None
    _check(_lib.sf_attend(hs, n, block, qs, os_, scale, _stream(stream)), None)


def sf_attend_static_scratch(handles, block: int, q, out, scale: float = 0.0, stream=None) -> None:
    n = len(handles)
    hs = (_P * n)(*handles)
    qs = (_P * n)(*[_ptr(x) for x in q]) if q is not None else None
    os_ = (_P * n)(*[_ptr(x) for x in out]) if out is not None else None
    _check(_lib.sf_attend_static_scratch(hs, n, block, qs, os_, scale, _stream(stream)), None)


def sf_step(handle: int, block: int, t: int, q, k, v, out, scale: float = 0.0, stream=None) -> None:
    _check(_lib.sf_step(handle, block, t, _ptr(q), _ptr(k), _ptr(v), _ptr(out), scale, _stream(stream)), handle)


def sf_rope_rows(cfg: sf_config, t: int, src, dst, stream=None) -> None:
    _check(_lib.sf_rope_rows(ctypes.byref(cfg), t, _ptr(src), _ptr(dst), _stream(stream)), None)


def sf_set_recency_bias(handle: int, table, stream=None) -> None:
    _check(_lib.sf_set_recency_bias(handle, _ptr(table), _stream(stream)), handle)


def _view_dict(v: sf_view, raw, summ) -> dict:
    return {
        "t_cur": v.t_cur, "n_keys": v.n_keys, "evicted_for": v.evicted_for, "raw_slot": v.raw_slot,
        "blocks_written": v.blocks_written,
        "segments": [(v.seg_begin[i], v.seg_len[i]) for i in range(v.n_seg)],
        "raw_frame": list(raw), "sum_frame": list(summ), "z0_frame": v.z0_frame,
    }


def sf_query(handle: int, cfg: sf_config) -> dict:
    raw = (ctypes.c_int64 * (cfg.y + 1))()
    summ = (ctypes.c_int64 * (cfg.w - cfg.y))()
    v = sf_view()
    v.raw_frame = ctypes.cast(raw, ctypes.POINTER(ctypes.c_int64))
    v.sum_frame = ctypes.cast(summ, ctypes.POINTER(ctypes.c_int64))
    _check(_lib.sf_query(handle, ctypes.byref(v)), handle)
    return _view_dict(v, raw, summ)


def sf_plan(cfg: sf_config, t: int) -> dict:
    raw = (ctypes.c_int64 * (cfg.y + 1))()
    summ = (ctypes.c_int64 * (cfg.w - cfg.y))()
    v = sf_view()
    v.raw_frame = ctypes.cast(raw, ctypes.POINTER(ctypes.c_int64))
    v.sum_frame = ctypes.cast(summ, ctypes.POINTER(ctypes.c_int64))
    _check(_lib.sf_plan(ctypes.byref(cfg), t, ctypes.byref(v)))
    return _view_dict(v, raw, summ)


def sf_status_str(status: int) -> str:
    return _lib.sf_status_str(status).decode()


def sf_last_error(handle: int | None = None) -> str:
    return (_lib.sf_last_error(handle) or b"").decode()


def sf_debug_fail_next_launch(handle: int) -> None:
    _check(_lib.sf_debug_fail_next_launch(handle), handle)


def sf_debug_range_form(form: int) -> None:
    _check(_lib.sf_debug_range_form(int(form)))


def sf_debug_lds_copy(dst, src, nbytes: int, stream=None) -> None:
    """Measurement aid: copies nbytes (a multiple of 16384) from src to dst through LDS with the
    attention kernels' buffer-to-LDS transfer (for calibrating traffic counters)."""
    _check(_lib.sf_debug_lds_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream)))


def sf_profile_enable(handle: int, on: bool = True) -> None:
    _check(_lib.sf_profile_enable(handle, 1 if on else 0), handle)


def sf_kernel_times_read(handle: int) -> dict:
    """{kind: (total ms, launches)} of the kernels launched since the last read (waits for them)."""
    t = sf_kernel_times()
    _check(_lib.sf_kernel_times_read(handle, ctypes.byref(t)), handle)
    return {KERNEL_KINDS[k]: (t.ms[k], t.launches[k]) for k in range(SF_K_KINDS)}


def sf_record_slot(handle: int, block: int, t: int):
    """(k_rows, v_rows) device addresses where record t of a block goes (0 on a dry handle)."""
    k, v = _P(), _P()
    _check(_lib.sf_record_slot(handle, block, t, ctypes.byref(k), ctypes.byref(v)), handle)
    return k.value or 0, v.value or 0


def sf_commit_record(handle: int, block: int, t: int) -> None:
    _check(_lib.sf_commit_record(handle, block, t), handle)


def sf_state_bytes(cfg: sf_config) -> int:
    return _lib.sf_state_bytes(ctypes.byref(cfg))


def sf_state_export(handle: int, cfg: sf_config) -> bytes:
    n = sf_state_bytes(cfg)
    buf = ctypes.create_string_buffer(n)
    _check(_lib.sf_state_export(handle, buf, n), handle)
    return buf.raw


def sf_state_import(handle: int, data: bytes) -> None:
    buf = ctypes.create_string_buffer(bytes(data), len(data))
    _check(_lib.sf_state_import(handle, buf, len(data)), handle)


# ------------------------------------------------------- a session on torch
class Session:
    """One session's memory: a torch uint8 device tensor of sf_buffer_bytes plus its handle.

    dry=True makes a dry-run handle (no device memory; for host-side checks).
    """

    def __init__(self, cfg: sf_config, device="cuda", stream=None, dry=False):
        self.cfg = cfg
        self.dry = dry
        self.nbytes = sf_buffer_bytes(cfg)
        if self.nbytes == 0:
            sf_config_check(cfg)
            raise SfError(SF_E_ARG, "invalid config")
        if dry:
            self.mem = None
            self.handle = sf_buffer_create(cfg)
        else:
            import torch
            self.mem = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
            self.handle = sf_buffer_create(cfg, self.mem, self.nbytes, stream)

    def close(self):
        if self.handle:
            sf_buffer_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def rows(self) -> int:
        return self.cfg.hw + self.cfg.x

    @property
    def capacity(self) -> int:
        c = self.cfg
        return self.rows * (c.y + 2) + (c.w - c.y) * c.x

    def kv(self, block: int):
        """(K, V) of one block as [capacity][H][d] tensor views of the session memory."""
        import torch
        dt = torch.bfloat16 if self.cfg.dtype == SF_BF16 else torch.float32
        n = self.capacity * self.cfg.n_heads * self.cfg.head_dim
        eb = 2 if self.cfg.dtype == SF_BF16 else 4
        ko = sf_kv_offset(self.cfg, block, 0)
        vo = sf_kv_offset(self.cfg, block, 1)
        shape = (self.capacity, self.cfg.n_heads, self.cfg.head_dim)
        k = self.mem[ko:ko + n * eb].view(dt).view(shape)
        v = self.mem[vo:vo + n * eb].view(dt).view(shape)
        return k, v

    def kv_bytes_view(self):
        return self.mem[: sf_kv_bytes(self.cfg)]

    def _check(self, x, is_out=False):
        """A [R][H][d] contiguous device tensor of the session dtype (fp32 for outputs)."""
        import torch
        want = torch.float32 if (is_out or self.cfg.dtype == SF_F32) else torch.bfloat16
        shape = (self.rows, self.cfg.n_heads, self.cfg.head_dim)
        if not isinstance(x, torch.Tensor) or x.dtype != want or not x.is_contiguous() or not x.is_cuda \
                or x.numel() != shape[0] * shape[1] * shape[2]:
            raise SfError(SF_E_ARG, f"expected a contiguous {want} device tensor of {shape} elements")
        if x.data_ptr() % 16:
            raise SfError(SF_E_ARG, "device tensors must start on a 16-byte boundary")
        return x

    def write_record(self, block, t, k, v, stream=None):
        sf_write_record(self.handle, block, t, self._check(k), self._check(v), stream)

    def evict(self, t, stream=None):
        sf_evict(self.handle, t, stream)

    def attend(self, block, q, out, scale=0.0, stream=None):
        sf_attend([self.handle], block, [self._check(q)], [self._check(out, True)], scale, stream)

    def step(self, block, t, q, k, v, out, scale=0.0, stream=None):
        sf_step(self.handle, block, t, self._check(q), self._check(k), self._check(v), self._check(out, True),
                scale, stream)

    def set_recency_bias(self, table, stream=None):
        """The session's recency bias: a contiguous fp32 device tensor [n_heads][w + 1]."""
        import torch
        shape = (self.cfg.n_heads, self.cfg.w + 1)
        if self.dry:
            sf_set_recency_bias(self.handle, None, stream)
            return
        if not isinstance(table, torch.Tensor) or table.dtype != torch.float32 or not table.is_cuda \
                or not table.is_contiguous() or tuple(table.shape) != shape:
            raise SfError(SF_E_ARG, f"expected a contiguous float32 device tensor of shape {shape}")
        sf_set_recency_bias(self.handle, table, stream)

    def rope_rows(self, t, src, dst=None, stream=None):
        """The rotation the session's rope mode applies at frame t (in place when dst is None)."""
        dst = src if dst is None else dst
        sf_rope_rows(self.cfg, t, self._check(src), self._check(dst), stream)
        return dst

    def view(self) -> dict:
        return sf_query(self.handle, self.cfg)

    def record_slot(self, block, t):
        """(K, V) rows where record t of a block goes, as [R][H][d] views of the session memory."""
        import torch
        ka, va = sf_record_slot(self.handle, block, t)
        dt = torch.bfloat16 if self.cfg.dtype == SF_BF16 else torch.float32
        eb = 2 if self.cfg.dtype == SF_BF16 else 4
        n = self.rows * self.cfg.n_heads * self.cfg.head_dim * eb
        base = self.mem.data_ptr()
        shape = (self.rows, self.cfg.n_heads, self.cfg.head_dim)
        return (self.mem[ka - base:ka - base + n].view(dt).view(shape),
                self.mem[va - base:va - base + n].view(dt).view(shape))

    def commit_record(self, block, t):
        sf_commit_record(self.handle, block, t)

    def export_state(self) -> bytes:
        return sf_state_export(self.handle, self.cfg)

    def import_state(self, data: bytes):
        sf_state_import(self.handle, data)


def attend_batch(sessions, block, qs, outs, scale=0.0, stream=None):
    """One batched sf_attend over several Session objects, with each tensor checked."""
    sf_attend([s.handle for s in sessions], block, [s._check(q) for s, q in zip(sessions, qs)],
              [s._check(o, True) for s, o in zip(sessions, outs)], scale, stream)
