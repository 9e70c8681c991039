"""ctypes binding of libmt.so (``include/mt.h`` and ``include/mt_kernels.h``).

Argument marshalling only: every step of the training path runs in the
library.  PyTorch is used by callers for device memory and streams; this
module passes raw pointers (``tensor.data_ptr()``, ``stream.cuda_stream``).
Importing it loads ``libmt.so`` from this package directory (or the build
that ``MT_LIBRARY`` names) and raises if the library is missing, so a missing build fails loudly instead of falling
back to anything else.
"""
import ctypes as C
import os

import numpy as np

# MT_LIBRARY names another build of the same sources (the host-sanitizer copy);
# by default the library built in this directory is loaded.
_LIB_PATH = os.environ.get("MT_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmt.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is not built; run `python -m layer_streaming_amd.build`")
lib = C.CDLL(_LIB_PATH)

MT_OK, MT_E_INVAL, MT_E_NOMEM, MT_E_HIP, MT_E_STATE, MT_E_INTERNAL, MT_E_IO = 0, -1, -2, -3, -4, -5, -6
MT_W, MT_G, MT_MASTER, MT_M, MT_V = 0, 1, 2, 3, 4
MT_MAX_SITES = 48
MT_MAX_MICRO = 4096


class mt_shape(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn_dim", C.c_int32),
                ("vocab", C.c_int32), ("rms_eps", C.c_float), ("rope_base", C.c_float)]


class mt_options(C.Structure):
    _fields_ = [("max_batch", C.c_int32), ("max_seq", C.c_int32), ("n_weight_slots", C.c_int32),
                ("n_grad_slabs", C.c_int32), ("slot_mode", C.c_int32), ("ckpt_on_host", C.c_int32),
                ("resident", C.c_int32), ("host_threads", C.c_int32), ("head_chunk", C.c_int32),
                ("profile_kernels", C.c_int32), ("pin_store", C.c_int32), ("cross_step", C.c_int32),
                ("ckpt_interval", C.c_int32),
                ("pin_weights", C.c_int32), ("head_vocab_chunk", C.c_int32), ("poison_released", C.c_int32),
                ("keep_grads", C.c_int32), ("ckpt_attn", C.c_int32),
                ("slot_bytes_override", C.c_uint64), ("workspace_bytes_override", C.c_uint64),
                ("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float), ("adam_eps", C.c_float),
                ("init_std", C.c_float), ("seed", C.c_uint64)]


class mt_stats(C.Structure):
    _fields_ = [("step_ms", C.c_double), ("fwd_ms", C.c_double), ("head_ms", C.c_double),
                ("bwd_ms", C.c_double), ("adam_tail_ms", C.c_double), ("compute_busy_ms", C.c_double),
                ("h2d_busy_ms", C.c_double), ("d2h_busy_ms", C.c_double), ("pack_ms", C.c_double),
                ("adam_ms", C.c_double), ("adam_wait_ms", C.c_double), ("overlap_ratio", C.c_double),
                ("pcie_busy_frac", C.c_double), ("overlap_phase", C.c_double * 3),
                ("exposed_transfer_ms", C.c_double * 3),
                ("h2d_bytes", C.c_uint64), ("d2h_bytes", C.c_uint64), ("gpu_arena_bytes", C.c_uint64),
                ("pinned_bytes", C.c_uint64), ("host_store_bytes", C.c_uint64), ("n_sites", C.c_int32),
                ("site_ms", C.c_double * MT_MAX_SITES), ("site_launches", C.c_uint64 * MT_MAX_SITES),
                ("fp16_saturated", C.c_uint64), ("compute_union_ms", C.c_double),
                ("copy_union_ms", C.c_double), ("overlap_ms", C.c_double), ("switch_gap_ms", C.c_double * 3),
                ("device_idle_ms", C.c_double * 3), ("h2d_idle_ms", C.c_double * 9),
                ("ready_switch_ms", C.c_double * 2), ("ready_switches", C.c_int32), ("switches", C.c_int32)]


class mt_tensor_info(C.Structure):
    _fields_ = [("name", C.c_char * 16), ("offset_elems", C.c_uint64), ("rows", C.c_int64),
                ("cols", C.c_int64), ("dtype", C.c_int32)]


_P = C.c_void_p
_SIGS = {
    "mt_default_options": (C.c_int, [C.POINTER(mt_options)]),
    "mt_workspace_bytes": (C.c_int, [C.POINTER(mt_shape), C.POINTER(mt_options), C.POINTER(C.c_uint64),
                                     C.POINTER(C.c_uint64), C.POINTER(C.c_uint64)]),
    "mt_init": (C.c_int, [C.POINTER(mt_shape), C.POINTER(mt_options), _P, C.c_uint64, C.POINTER(_P),
                          C.POINTER(_P)]),
    "mt_train_step": (C.c_int, [_P, C.POINTER(C.c_int32), C.POINTER(C.c_int32), C.c_int32, C.c_int32,
                                C.POINTER(C.c_float), C.POINTER(mt_stats)]),
    "mt_train_step_accum": (C.c_int, [_P, C.POINTER(C.c_int32), C.POINTER(C.c_int32), C.c_int32, C.c_int32,
                                      C.c_int32, C.POINTER(C.c_float), C.POINTER(mt_stats)]),
    "mt_layer_fwd": (C.c_int, [_P, C.c_int32, _P, _P, C.c_int32, C.c_int32]),
    "mt_layer_bwd": (C.c_int, [_P, C.c_int32, _P, _P, _P, _P, C.c_int32, C.c_int32]),
    "mt_tensor_desc": (C.c_int, [C.POINTER(mt_shape), C.c_int32, C.c_int32, C.POINTER(mt_tensor_info)]),
    "mt_unit_tensors": (C.c_int, [C.POINTER(mt_shape), C.c_int32]),
    "mt_unit_elems": (C.c_uint64, [C.POINTER(mt_shape), C.c_int32]),
    "mt_get_tensor": (C.c_int, [_P, C.c_int32, C.c_int32, C.c_int32, _P, C.c_uint64]),
    "mt_set_tensor": (C.c_int, [_P, C.c_int32, C.c_int32, C.c_int32, _P, C.c_uint64]),
    "mt_step_count": (C.c_int, [_P, C.POINTER(C.c_int64)]),
    "mt_sync": (C.c_int, [_P]),
    "mt_checkpoint_save": (C.c_int, [_P, C.c_char_p]),
    "mt_checkpoint_restore": (C.c_int, [_P, C.c_char_p, C.c_int32]),
    "mt_abi_sizeof": (C.c_int64, [C.c_int32]),
    "mt_site_name": (C.c_char_p, [C.c_int32]),
    "mt_destroy": (None, [_P]),
    "mt_strerror": (C.c_char_p, [C.c_int]),
    "mt_last_error": (C.c_char_p, []),
    # test entries
    "mt_k_gemm": (C.c_int, [C.c_int32, C.c_int32, _P, C.c_int64, _P, C.c_int64, _P, C.c_int64, _P, C.c_int64,
                            _P, C.c_int64, C.c_int32, C.c_int32, C.c_int32, _P]),
    "mt_k_gemm_split": (C.c_int, [C.c_int32, C.c_int32, _P, C.c_int64, _P, C.c_int64, _P, C.c_int64, _P, C.c_int64,
                                  _P, C.c_int64, C.c_int32, C.c_int32, C.c_int32, _P, C.c_int64, C.c_int32, _P]),
    "mt_k_gemm_split_plan": (C.c_int, [C.c_int64, C.c_int64, C.c_int64, C.c_int64, _P, _P, _P]),
    "mt_k_gemm_amax": (C.c_int, [C.c_int32, _P, C.c_int64, _P, C.c_int64, _P, C.c_int64, C.c_int32, C.c_int32,
                                 C.c_int32, _P, _P]),
    "mt_k_qkv_rope_cvt_vmax": (C.c_int, [_P, C.c_int64, _P, C.c_int64, _P, C.c_int32, C.c_int32, C.c_int32,
                                         C.c_int32, C.c_int32, C.c_float, _P, _P, _P]),
    "mt_k_rmsnorm_fwd": (C.c_int, [_P, C.c_int32, _P, _P, _P, _P, C.c_int32, C.c_int32, C.c_float, _P, _P]),
    "mt_k_rmsnorm_bwd_scratch_elems": (C.c_int64, [C.c_int32, C.c_int32]),
    "mt_k_rmsnorm_bwd": (C.c_int, [_P, _P, C.c_int32, _P, _P, _P, _P, _P, _P, C.c_int32, C.c_int32, _P]),
    "mt_k_rmsnorm_bwd_noalloc": (C.c_int, [_P, _P, C.c_int32, _P, _P, _P, _P, _P, C.c_int32, C.c_int32, _P]),
    "mt_k_rope": (C.c_int, [_P, C.c_int64, _P, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_float, C.c_int32,
                            _P]),
    "mt_k_swiglu_fwd": (C.c_int, [_P, _P, C.c_int32, C.c_int32, _P]),
    "mt_k_swiglu_bwd": (C.c_int, [_P, _P, _P, C.c_int32, C.c_int32, _P]),
    "mt_k_attn_fwd": (C.c_int, [_P, C.c_int64, _P, C.c_int64, _P, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                C.c_int32, _P, _P]),
    "mt_k_attn_bwd_work_bytes": (C.c_int64, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32]),
    "mt_k_attn_dkdv_splits": (C.c_int32, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32]),
    "mt_k_attn_bwd": (C.c_int, [_P, C.c_int64, _P, _P, C.c_int64, _P, _P, _P, C.c_int64, C.c_int32, C.c_int32,
                                C.c_int32, C.c_int32, C.c_int32, _P, C.c_int64, C.c_int32, C.c_int32, _P, _P]),
    "mt_k_attn_bwd_rope": (C.c_int, [_P, C.c_int64, _P, _P, C.c_int64, _P, _P, _P, C.c_int64, C.c_int32, C.c_int32,
                                     C.c_int32, C.c_int32, C.c_int32, _P, C.c_int64, C.c_int32, C.c_int32, _P, _P,
                                     C.c_float, C.c_int32, _P]),
    "mt_k_rope_f32_bf16": (C.c_int, [_P, C.c_int64, _P, C.c_int64, _P, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                     C.c_float, C.c_int32, _P]),
    "mt_k_ce": (C.c_int, [_P, _P, _P, _P, C.c_int32, C.c_int32, C.c_float, _P]),
    "mt_k_mean": (C.c_int, [_P, _P, C.c_int32, _P]),
    "mt_k_f32_to_bf16": (C.c_int, [_P, _P, C.c_int64, _P]),
    "mt_k_transpose16": (C.c_int, [_P, C.c_int64, _P, C.c_int64, C.c_int32, C.c_int32, C.c_int32, _P]),
    "mt_k_qkv_rope_cvt": (C.c_int, [_P, C.c_int64, _P, C.c_int64, _P, C.c_int64, _P, C.c_int32, C.c_int32,
                                    C.c_int32, C.c_int32, C.c_int32, C.c_float, _P, _P]),
    "mt_k_bf16_to_f16": (C.c_int, [_P, _P, C.c_int64, _P, _P]),
    "mt_host_adam": (C.c_int, [_P, _P, _P, _P, _P, _P, C.c_int64, C.c_int64, C.c_float, C.c_float, C.c_float,
                               C.c_float, C.c_int32]),
    "mt_host_accum": (C.c_int, [_P, _P, C.c_int64, C.c_int32]),
    "mt_host_init_unit": (C.c_int, [C.POINTER(mt_shape), C.c_int32, C.c_uint64, C.c_float, C.c_int32, _P,
                                    C.c_uint64]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


class MTError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = lib.mt_strerror(status).decode()
        detail = lib.mt_last_error().decode()
        super().__init__(f"{where}: {msg} ({status}): {detail}")


def check(status, where=""):
    if status != MT_OK:
        raise MTError(status, where)
    return status


def make_shape(n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab, rms_eps=1e-6,
               rope_base=10000.0):
    return mt_shape(n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab, rms_eps, rope_base)


def default_options(**kw):
    o = mt_options()
    check(lib.mt_default_options(C.byref(o)), "mt_default_options")
    for k, v in kw.items():
        if not hasattr(o, k):
            raise AttributeError(k)
        setattr(o, k, v)
    return o


def workspace_bytes(shape, opt):
    a, p, h = C.c_uint64(), C.c_uint64(), C.c_uint64()
    check(lib.mt_workspace_bytes(C.byref(shape), C.byref(opt), C.byref(a), C.byref(p), C.byref(h)),
          "mt_workspace_bytes")
    return a.value, p.value, h.value


def tensor_desc(shape, unit, idx):
    info = mt_tensor_info()
    check(lib.mt_tensor_desc(C.byref(shape), unit, idx, C.byref(info)), "mt_tensor_desc")
    return {"name": info.name.decode(), "offset": info.offset_elems, "rows": info.rows, "cols": info.cols}


def unit_tensors(shape, unit):
    r = lib.mt_unit_tensors(C.byref(shape), unit)
    check(r if r < 0 else 0, "mt_unit_tensors")
    return r


def unit_elems(shape, unit):
    return int(lib.mt_unit_elems(C.byref(shape), unit))


def site_names():
    out = []
    i = 0
    while True:
        n = lib.mt_site_name(i)
        if n is None:
            return out
        out.append(n.decode())
        i += 1


class Context:
    """Owns an ``mt_ctx``.  ``arena_ptr`` and ``streams`` stay owned by the
    caller and must outlive the context."""

    def __init__(self, shape, opt, arena_ptr, arena_bytes, streams=(None, None, None)):
        self.shape, self.opt = shape, opt
        sarr = (C.c_void_p * 3)(*[s if s else None for s in streams])
        ptr = C.c_void_p()
        check(lib.mt_init(C.byref(shape), C.byref(opt), C.c_void_p(arena_ptr), arena_bytes, sarr, C.byref(ptr)),
              "mt_init")
        self._ptr = ptr

    @property
    def handle(self):
        return self._ptr

    def close(self):
        if self._ptr:
            lib.mt_destroy(self._ptr)
            self._ptr = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def train_step(self, tokens, labels, stats=True):
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        labels = np.ascontiguousarray(labels, dtype=np.int32)
        b, s = tokens.shape
        loss = C.c_float()
        st = mt_stats() if stats else None
        check(lib.mt_train_step(self._ptr, tokens.ctypes.data_as(C.POINTER(C.c_int32)),
                                labels.ctypes.data_as(C.POINTER(C.c_int32)), b, s, C.byref(loss),
                                C.byref(st) if st is not None else None), "mt_train_step")
        return loss.value, st

    def train_step_accum(self, tokens, labels, stats=True):
        """tokens, labels: [n_micro, batch, seq]."""
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        labels = np.ascontiguousarray(labels, dtype=np.int32)
        n, b, s = tokens.shape
        loss = C.c_float()
        st = mt_stats() if stats else None
        check(lib.mt_train_step_accum(self._ptr, tokens.ctypes.data_as(C.POINTER(C.c_int32)),
                                      labels.ctypes.data_as(C.POINTER(C.c_int32)), n, b, s, C.byref(loss),
                                      C.byref(st) if st is not None else None), "mt_train_step_accum")
        return loss.value, st

    def layer_fwd(self, layer, x_ptr, y_ptr, batch, seq):
        check(lib.mt_layer_fwd(self._ptr, layer, C.c_void_p(x_ptr), C.c_void_p(y_ptr), batch, seq), "mt_layer_fwd")

    def layer_bwd(self, layer, x_ptr, dy_ptr, dx_ptr, gtile_ptr, batch, seq):
        check(lib.mt_layer_bwd(self._ptr, layer, C.c_void_p(x_ptr), C.c_void_p(dy_ptr), C.c_void_p(dx_ptr),
                               C.c_void_p(gtile_ptr), batch, seq), "mt_layer_bwd")

    def get_tensor(self, unit, idx, which):
        d = tensor_desc(self.shape, unit, idx)
        dt = np.uint16 if which in (MT_W, MT_G) else np.float32
        out = np.empty((d["rows"], d["cols"]), dtype=dt)
        check(lib.mt_get_tensor(self._ptr, unit, idx, which, out.ctypes.data, out.nbytes), "mt_get_tensor")
        return out if d["rows"] > 1 else out.reshape(-1)

    def set_tensor(self, unit, idx, which, arr):
        dt = np.uint16 if which in (MT_W, MT_G) else np.float32
        a = np.ascontiguousarray(arr, dtype=dt)
        check(lib.mt_set_tensor(self._ptr, unit, idx, which, a.ctypes.data, a.nbytes), "mt_set_tensor")

    def sync(self):
        check(lib.mt_sync(self._ptr), "mt_sync")

    def checkpoint_save(self, path):
        check(lib.mt_checkpoint_save(self._ptr, os.fsencode(path)), "mt_checkpoint_save")

    def checkpoint_restore(self, path, lazy=False):
        check(lib.mt_checkpoint_restore(self._ptr, os.fsencode(path), 1 if lazy else 0), "mt_checkpoint_restore")

    def step_count(self):
        v = C.c_int64()
        check(lib.mt_step_count(self._ptr, C.byref(v)), "mt_step_count")
        return v.value


def stats_dict(st):
    names = site_names()
    arrays = ("overlap_phase", "exposed_transfer_ms", "switch_gap_ms", "device_idle_ms", "h2d_idle_ms",
              "ready_switch_ms")
    d = {k: getattr(st, k) for k, _ in mt_stats._fields_ if k not in ("site_ms", "site_launches") + arrays}
    for k in arrays:
        d[k] = list(getattr(st, k))
    d["sites"] = {names[i]: {"ms": st.site_ms[i], "launches": st.site_launches[i]}
                  for i in range(min(st.n_sites, len(names)))}
    return d
