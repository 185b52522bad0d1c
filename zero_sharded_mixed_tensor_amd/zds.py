"""ctypes binding of libzds (include/zds.h), one Python function per C entry
point and with the same name. Argument marshalling only: tensors are passed
as device pointers, torch's current HIP stream as the stream, and every step
of the optimizer path runs in the library's kernels.

The library must have been built (python -m zero_sharded_mixed_tensor_amd.build);
loading fails loudly otherwise. torch is imported first so that the library
binds to the HIP runtime torch already loaded.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# ZDS_LIBRARY selects another build of the library (the host-sanitizer
# build, for the CPU tests run under AddressSanitizer).
LIB_PATH = os.environ.get("ZDS_LIBRARY") or os.path.join(_HERE, "libzds.so")

ZDS_OK, ZDS_EINVAL, ZDS_EALIGN, ZDS_ENOMEM, ZDS_EHIP, ZDS_EIO = 0, 1, 2, 3, 4, 5
ZDS_FP16, ZDS_BF16, ZDS_FP32 = 0, 1, 2
ZDS_COPY, ZDS_OVERWRITE, ZDS_ACCUMULATE = 0, 1, 2
ZDS_ON_DEVICE, ZDS_ON_HOST = 0, 1

STATE_BYTES = 64
SCALARS_BYTES = 64


class ZdsError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("zds status %d: %s" % (status, msg))
        self.status = status


class AdamWHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float)]


class ScalerConfig(ctypes.Structure):
    _fields_ = [("dynamic", ctypes.c_int32), ("initial_scale_power", ctypes.c_int32),
                ("window", ctypes.c_int32), ("hysteresis", ctypes.c_int32),
                ("min_scale", ctypes.c_float), ("static_scale", ctypes.c_float)]


class StepState(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_float), ("good_steps", ctypes.c_int32),
                ("hyst_left", ctypes.c_int32), ("window", ctypes.c_int32),
                ("hysteresis", ctypes.c_int32), ("min_scale", ctypes.c_float),
                ("dynamic", ctypes.c_int32), ("last_skip", ctypes.c_uint32),
                ("t", ctypes.c_int64), ("beta1_pow", ctypes.c_double),
                ("beta2_pow", ctypes.c_double), ("steps_seen", ctypes.c_uint32),
                ("steps_skipped", ctypes.c_uint32)]


class StepScalars(ctypes.Structure):
    _fields_ = [("overflow", ctypes.c_uint32), ("accum_steps", ctypes.c_int32),
                ("sumsq", ctypes.c_double), ("norm", ctypes.c_float),
                ("clip_coef", ctypes.c_float), ("grad_scale", ctypes.c_float),
                ("scale_used", ctypes.c_float), ("inv_bc2_sqrt", ctypes.c_double),
                ("step_size", ctypes.c_float), ("bc2_sqrt", ctypes.c_float), ("decay", ctypes.c_float),
                ("beta1", ctypes.c_float), ("beta2", ctypes.c_float), ("eps", ctypes.c_float)]


class CheckpointMeta(ctypes.Structure):
    _fields_ = [("world", ctypes.c_int32), ("rank", ctypes.c_int32), ("flat_align", ctypes.c_int32),
                ("stage", ctypes.c_int32), ("offload", ctypes.c_int32), ("num_tensors", ctypes.c_int32),
                ("flat_total", ctypes.c_int64), ("lo", ctypes.c_int64), ("hi", ctypes.c_int64)]

    def as_tuple(self):
        return tuple(getattr(self, f) for f, _ in self._fields_)


assert ctypes.sizeof(StepState) == STATE_BYTES and ctypes.sizeof(StepScalars) == SCALARS_BYTES
assert ctypes.sizeof(CheckpointMeta) == 48

_P = ctypes.c_void_p
_I32, _I64, _U32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
_PI64 = ctypes.POINTER(ctypes.c_int64)
_SIGS = {
    "zds_flat_layout": (_I32, [_PI64, _I32, _I32, _PI64, _PI64]),
    "zds_shard_range": (_I32, [_I64, _I32, _I32, _I32, _PI64, _PI64]),
    "zds_shard_entries": (_I32, [_PI64, _I32, _I32, _I64, _I64, _PI64, _I32,
                                 ctypes.POINTER(ctypes.c_int32)]),
    "zds_plan_create": (_I32, [ctypes.POINTER(_P), _PI64, _I32, _I32, _I64, _I64]),
    "zds_plan_destroy": (None, [_P]),
    "zds_plan_num_entries": (_I32, [_P]),
    "zds_plan_entry": (_I32, [_P, _I32, _PI64]),
    "zds_grad_accumulate": (_I32, [_P, ctypes.POINTER(_P), _I32, _P, _I32, _I32, _P]),
    "zds_workspace_bytes": (ctypes.c_size_t, [_I64]),
    "zds_reduce_peer_slices": (_I32, [ctypes.POINTER(_P), _I32, _I32, _I64, _P, _I32, _I32, _P]),
    "zds_plan_norm_workspace_bytes": (ctypes.c_size_t, [_P]),
    "zds_reduce_norm_workspace_bytes": (ctypes.c_size_t, [_I64]),
    "zds_reduce_peer_slices_norm": (_I32, [ctypes.POINTER(_P), _I32, _I32, _I64, _P, _I32, _I32, _I32,
                                           ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P]),
    "zds_grad_accumulate_norm": (_I32, [_P, ctypes.POINTER(_P), _I32, _P, _I32, _I32, _I32, ctypes.c_float,
                                        _P, _P, _P, ctypes.c_size_t, _P]),
    "zds_overflow_and_norm": (_I32, [_P, _I32, _I64, _I32, ctypes.c_float, _P, _P, _P,
                                     ctypes.c_size_t, _P]),
    "zds_overflow_and_norm_noalloc": (_I32, [_P, _I32, _I64, _I32, ctypes.c_float, _P, _P, _P]),
    "zds_adam_step": (_I32, [ctypes.POINTER(AdamWHparams), _P, _I32, _P, _P, _P, _P, _I32, _I64,
                             _P, _P, _P]),
    "zds_cpu_adam_step": (_I32, [ctypes.POINTER(AdamWHparams), _P, _I32, _P, _P, _P, _P, _I32, _I64,
                                 ctypes.POINTER(StepScalars), ctypes.POINTER(StepState), _I32]),
    "zds_onebit_compress": (_I32, [_P, _P, _I64, _I32, _P, _P, _P]),
    "zds_onebit_decompress": (_I32, [ctypes.POINTER(_P), ctypes.POINTER(_P), _I32, _I64, _I32, _P, _I32, _P]),
    "zds_checkpoint_save": (_I32, [ctypes.c_char_p, ctypes.POINTER(CheckpointMeta), _PI64, _P, _P, _P, _P,
                                   _I32, _P]),
    "zds_checkpoint_read_meta": (_I32, [ctypes.c_char_p, ctypes.POINTER(CheckpointMeta),
                                        ctypes.POINTER(StepState), _PI64, _I32]),
    "zds_checkpoint_load": (_I32, [ctypes.c_char_p, ctypes.POINTER(CheckpointMeta), _PI64, _P, _P, _P, _P,
                                   _I32, _P]),
    "zds_consolidate_fp32": (_I32, [ctypes.POINTER(ctypes.c_char_p), _I32, _I32, _P, _I64]),
    "zds_step_state_init": (_I32, [_P, ctypes.POINTER(ScalerConfig), _I64, ctypes.c_double,
                                   ctypes.c_double, _P]),
    "zds_loss_scaler_update": (_I32, [_P, _P, ctypes.POINTER(AdamWHparams), _P]),
    "zds_step_state_init_host": (_I32, [ctypes.POINTER(StepState), ctypes.POINTER(ScalerConfig),
                                        _I64, ctypes.c_double, ctypes.c_double]),
    "zds_loss_scaler_update_host": (_I32, [ctypes.POINTER(StepState), _U32,
                                           ctypes.POINTER(AdamWHparams)]),
    "zds_adam_constants_host": (_I32, [ctypes.POINTER(AdamWHparams), ctypes.POINTER(StepState),
                                       ctypes.POINTER(ctypes.c_float)]),
    "zds_clip_scalars_host": (_I32, [ctypes.c_double, ctypes.c_float, _I32, ctypes.c_float,
                                     ctypes.POINTER(StepScalars)]),
    "zds_last_error": (ctypes.c_char_p, []),
    "zds_status_string": (ctypes.c_char_p, [_I32]),
    "zds_abi_version": (_I32, []),
}


def _load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError("libzds.so is not built at %s; run "
                          "`python -m zero_sharded_mixed_tensor_amd.build`" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def _check(status):
    if status != ZDS_OK:
        raise ZdsError(status, lib.zds_last_error().decode())


def _i64arr(xs):
    return (ctypes.c_int64 * max(1, len(xs)))(*[int(x) for x in xs])


_DT = {torch.float16: ZDS_FP16, torch.bfloat16: ZDS_BF16, torch.float32: ZDS_FP32}


def dtype_code(t):
    try:
        return _DT[t.dtype]
    except KeyError:
        raise ZdsError(ZDS_EINVAL, "unsupported dtype %s" % t.dtype)


def _numel(x):
    return x.numel() if isinstance(x, torch.Tensor) else int(x.size)


def _need(x, n, what):
    """The library takes plain pointers and sizes: a buffer shorter than the
    call's n would be read or written past its end, so the binding refuses it."""
    if x is not None and _numel(x) < n:
        raise ZdsError(ZDS_EINVAL, "%s holds %d elements, the call needs %d" % (what, _numel(x), n))


def _need_bytes(x, nbytes, what):
    if x is None:
        return
    have = _numel(x) * (x.element_size() if isinstance(x, torch.Tensor) else x.itemsize)
    if have < nbytes:
        raise ZdsError(ZDS_EINVAL, "%s holds %d bytes, the call needs %d" % (what, have, nbytes))


def _dev_ptr(t, what):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ZdsError(ZDS_EINVAL, "%s must be a device tensor" % what)
    if not t.is_contiguous():
        raise ZdsError(ZDS_EINVAL, "%s must be contiguous" % what)
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def hparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01):
    return AdamWHparams(lr, beta1, beta2, eps, weight_decay)


def scaler_config(dynamic=True, initial_scale_power=16, window=1000, hysteresis=1,
                  min_scale=1.0, static_scale=1.0):
    return ScalerConfig(int(bool(dynamic)), initial_scale_power, window, hysteresis, min_scale,
                        static_scale)


# ------------------------------------------------------------------ geometry

def zds_flat_layout(numels, flat_align):
    offs = (ctypes.c_int64 * max(1, len(numels)))()
    total = ctypes.c_int64()
    _check(lib.zds_flat_layout(_i64arr(numels), len(numels), flat_align, offs, ctypes.byref(total)))
    return list(offs)[:len(numels)], total.value


def zds_shard_range(flat_total, world, rank, flat_align):
    lo, hi = ctypes.c_int64(), ctypes.c_int64()
    _check(lib.zds_shard_range(flat_total, world, rank, flat_align, ctypes.byref(lo), ctypes.byref(hi)))
    return lo.value, hi.value


def zds_shard_entries(numels, flat_align, lo, hi):
    cnt = ctypes.c_int32()
    st = lib.zds_shard_entries(_i64arr(numels), len(numels), flat_align, lo, hi, None, 0,
                               ctypes.byref(cnt))
    if st != ZDS_OK and cnt.value == 0:
        _check(st)
    out = (ctypes.c_int64 * (4 * max(1, cnt.value)))()
    _check(lib.zds_shard_entries(_i64arr(numels), len(numels), flat_align, lo, hi, out, cnt.value,
                                 ctypes.byref(cnt)))
    v = list(out)
    return [tuple(v[4 * i:4 * i + 4]) for i in range(cnt.value)]


# ------------------------------------------------------------------ plans

class Plan:
    """Owning handle of a zds_plan (tensor table of one flat range)."""

    def __init__(self, handle, num_tensors):
        self.handle = handle
        self.num_tensors = num_tensors
        ents = self.entries()
        # elements each source tensor must hold, and the destination's length
        self.src_need = {}
        for t, start, length, _ in ents:
            self.src_need[t] = max(self.src_need.get(t, 0), start + length)
        self.span = max((off + length for _, _, length, off in ents), default=0)

    @property
    def num_entries(self):
        return lib.zds_plan_num_entries(self.handle)

    def entries(self):
        out = []
        buf = (ctypes.c_int64 * 4)()
        for e in range(self.num_entries):
            _check(lib.zds_plan_entry(self.handle, e, buf))
            out.append(tuple(buf))
        return out

    def close(self):
        if self.handle:
            lib.zds_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def zds_plan_create(numels, flat_align, lo, hi):
    h = ctypes.c_void_p()
    _check(lib.zds_plan_create(ctypes.byref(h), _i64arr(numels), len(numels), flat_align, lo, hi))
    return Plan(h, len(numels))


# ------------------------------------------------------------------ hot calls

class SourceSet:
    """A plan's source tensors, marshalled once: a training loop whose grads
    live in fixed buffers binds them once and passes the set on every call
    instead of the list (building the pointer array costs about 0.5 us per
    tensor per call). Keeps the tensors' storages alive; rebind after
    replacing a tensor or its storage."""

    def __init__(self, plan, srcs):
        self.ptrs, self.dtype = _src_array(plan, srcs)
        self._storages = [None if t is None else t.untyped_storage() for t in srcs]
        self.num_tensors = len(srcs)


def _sources(plan, srcs):
    if isinstance(srcs, SourceSet):
        if srcs.num_tensors != plan.num_tensors:
            raise ZdsError(ZDS_EINVAL, "source set of %d tensors for a plan of %d" % (srcs.num_tensors,
                                                                                      plan.num_tensors))
        return srcs.ptrs, srcs.dtype
    return _src_array(plan, srcs)


def zds_grad_accumulate(plan, srcs, dst, mode, stream=None):
    """srcs: one device tensor per tensor of the plan's layout (None where the
    plan has no entry), or a SourceSet of them; dst: the flat device buffer
    of the plan's range."""
    _need(dst, plan.span, "dst")
    ptrs, sdt = _sources(plan, srcs)
    _check(lib.zds_grad_accumulate(plan.handle, ptrs, sdt, _dev_ptr(dst, "dst"), dtype_code(dst),
                                   mode, _stream(stream)))


def _src_array(plan, srcs):
    if len(srcs) != plan.num_tensors:
        raise ZdsError(ZDS_EINVAL, "need %d source tensors" % plan.num_tensors)
    sdt = None
    ptrs = (ctypes.c_void_p * max(1, len(srcs)))()
    for i, need in plan.src_need.items():
        if srcs[i] is None:
            raise ZdsError(ZDS_EINVAL, "source %d is None but the plan reads %d of its elements" % (i, need))
        _need(srcs[i], need, "source %d" % i)
    for i, t in enumerate(srcs):
        if t is None:
            continue
        c = dtype_code(t)
        if sdt is None:
            sdt = c
        elif c != sdt:
            raise ZdsError(ZDS_EINVAL, "source tensors must share one dtype")
        ptrs[i] = _dev_ptr(t, "source %d" % i)
    return ptrs, (ZDS_FP16 if sdt is None else sdt)


def zds_plan_norm_workspace_bytes(plan):
    return lib.zds_plan_norm_workspace_bytes(plan.handle)


def zds_grad_accumulate_norm(plan, srcs, dst, mode, accum_steps, max_norm, state, scalars, ws, stream=None):
    """zds_grad_accumulate plus the step's overflow flag, norm and clip
    scalars formed from the stored values (see include/zds.h)."""
    _need(dst, plan.span, "dst")
    ptrs, sdt = _sources(plan, srcs)
    _check(lib.zds_grad_accumulate_norm(plan.handle, ptrs, sdt, _dev_ptr(dst, "dst"), dtype_code(dst), mode,
                                        accum_steps, max_norm, _dev_ptr(state, "state"),
                                        _dev_ptr(scalars, "scalars"), _dev_ptr(ws, "workspace"),
                                        ws.numel() * ws.element_size(), _stream(stream)))


def zds_reduce_peer_slices(peers, dst, mode, stream=None, n=None):
    """dst (+)= sum over the peer slices (device tensors of one 16-bit dtype),
    in peer order, in fp32 (see include/zds.h)."""
    n = dst.numel() if n is None else n
    _need(dst, n, "dst")
    arr, sdt = _peer_array(peers, n)
    _check(lib.zds_reduce_peer_slices(arr, len(peers), sdt, n, _dev_ptr(dst, "dst"), dtype_code(dst), mode,
                                      _stream(stream)))


def _peer_array(peers, n):
    if not peers:
        raise ZdsError(ZDS_EINVAL, "need at least one peer slice")
    sdt = dtype_code(peers[0])
    for k, t in enumerate(peers):
        if dtype_code(t) != sdt or t.numel() < n:
            raise ZdsError(ZDS_EINVAL, "peer %d: wrong dtype or too short" % k)
    return (ctypes.c_void_p * len(peers))(*[_dev_ptr(t, "peer %d" % k) for k, t in enumerate(peers)]), sdt


def zds_reduce_norm_workspace_bytes(n):
    return lib.zds_reduce_norm_workspace_bytes(n)


def new_reduce_workspace(n, device="cuda"):
    return torch.empty((zds_reduce_norm_workspace_bytes(n) + 7) // 8, dtype=torch.float64, device=device)


def zds_reduce_peer_slices_norm(peers, dst, mode, accum_steps, max_norm, state, scalars, ws, stream=None, n=None):
    """zds_reduce_peer_slices plus the step's overflow flag, norm and clip
    scalars formed from the stored values (see include/zds.h)."""
    n = dst.numel() if n is None else n
    _need(dst, n, "dst")
    _need_bytes(state, STATE_BYTES, "state")
    _need_bytes(scalars, SCALARS_BYTES, "scalars")
    arr, sdt = _peer_array(peers, n)
    _check(lib.zds_reduce_peer_slices_norm(arr, len(peers), sdt, n, _dev_ptr(dst, "dst"), dtype_code(dst), mode,
                                           accum_steps, max_norm, _dev_ptr(state, "state"),
                                           _dev_ptr(scalars, "scalars"), _dev_ptr(ws, "workspace"),
                                           ws.numel() * ws.element_size(), _stream(stream)))


def zds_workspace_bytes(n):
    return lib.zds_workspace_bytes(n)


def zds_overflow_and_norm(grads, accum_steps, max_norm, state, scalars, ws, stream=None, n=None):
    n = grads.numel() if n is None else n
    _need(grads, n, "grads")
    _check(lib.zds_overflow_and_norm(_dev_ptr(grads, "grads"), dtype_code(grads), n, accum_steps,
                                     max_norm, _dev_ptr(state, "state"), _dev_ptr(scalars, "scalars"),
                                     _dev_ptr(ws, "workspace"), ws.numel() * ws.element_size(),
                                     _stream(stream)))


def zds_overflow_and_norm_noalloc(grads, accum_steps, max_norm, state, scalars, stream=None, n=None):
    n = grads.numel() if n is None else n
    _need(grads, n, "grads")
    _check(lib.zds_overflow_and_norm_noalloc(_dev_ptr(grads, "grads"), dtype_code(grads), n, accum_steps,
                                             max_norm, _dev_ptr(state, "state"), _dev_ptr(scalars, "scalars"),
                                             _stream(stream)))


def zds_adam_step(hp, grads, master, exp_avg, exp_avg_sq, params_out, scalars, state, stream=None,
                  n=None):
    n = master.numel() if n is None else n
    for name, t in (("master", master), ("grads", grads), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq),
                    ("params_out", params_out)):
        _need(t, n, name)
    pdt = dtype_code(params_out) if params_out is not None else ZDS_FP16
    _check(lib.zds_adam_step(ctypes.byref(hp), _dev_ptr(grads, "grads"), dtype_code(grads),
                             _dev_ptr(master, "master"), _dev_ptr(exp_avg, "exp_avg"),
                             _dev_ptr(exp_avg_sq, "exp_avg_sq"), _dev_ptr(params_out, "params_out"),
                             pdt, n, _dev_ptr(scalars, "scalars"), _dev_ptr(state, "state"),
                             _stream(stream)))


def _host_ptr(x, what):
    """Host buffer address: a CPU torch tensor or a C-contiguous numpy array."""
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        if x.device.type != "cpu" or not x.is_contiguous():
            raise ZdsError(ZDS_EINVAL, "%s must be a contiguous host tensor" % what)
        return x.data_ptr()
    import numpy as np
    if not isinstance(x, np.ndarray) or not x.flags["C_CONTIGUOUS"]:
        raise ZdsError(ZDS_EINVAL, "%s must be a contiguous host array" % what)
    return x.ctypes.data


_NP_DT = {"float16": ZDS_FP16, "float32": ZDS_FP32}


def _host_dtype(x, declared=None):
    if declared is not None:
        return declared
    if isinstance(x, torch.Tensor):
        return dtype_code(x)
    return _NP_DT[str(x.dtype)]


def zds_cpu_adam_step(hp, grads, master, exp_avg, exp_avg_sq, params_out, scalars, state, num_threads=0,
                      grad_dtype=None, param_dtype=None, n=None):
    """AdamW on host buffers (see include/zds.h). Buffers are CPU torch
    tensors or numpy arrays; 16-bit numpy data given as uint16 needs
    grad_dtype / param_dtype (ZDS_FP16 or ZDS_BF16). scalars and state are
    StepScalars / StepState host structs."""
    n = _numel(master) if n is None else n
    for name, t in (("master", master), ("grads", grads), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq),
                    ("params_out", params_out)):
        _need(t, n, name)
    gdt = _host_dtype(grads, grad_dtype)
    pdt = ZDS_FP16 if params_out is None else _host_dtype(params_out, param_dtype)
    _check(lib.zds_cpu_adam_step(ctypes.byref(hp), _host_ptr(grads, "grads"), gdt, _host_ptr(master, "master"),
                                 _host_ptr(exp_avg, "exp_avg"), _host_ptr(exp_avg_sq, "exp_avg_sq"),
                                 _host_ptr(params_out, "params_out"), pdt, n, ctypes.byref(scalars),
                                 ctypes.byref(state), num_threads))


# ------------------------------------------------------------------ 1-bit codec

def onebit_payload(n, chunk, device="cuda"):
    """Device buffers of one encoded message: (words, scales); words are
    32-bit, 64 per 2048 elements."""
    return (torch.zeros(64 * ((n + 2047) // 2048), dtype=torch.int32, device=device),
            torch.zeros((n + chunk - 1) // chunk, dtype=torch.float32, device=device))


def _need_payload(words, scales, n, chunk):
    if chunk < 1:
        raise ZdsError(ZDS_EINVAL, "chunk must be positive")
    _need_bytes(words, 256 * ((n + 2047) // 2048), "words")
    _need_bytes(scales, 4 * ((n + chunk - 1) // chunk), "scales")


def zds_onebit_compress(x, error, chunk, words, scales, stream=None, n=None):
    n = x.numel() if n is None else n
    if x.dtype != torch.float32 or (error is not None and error.dtype != torch.float32):
        raise ZdsError(ZDS_EINVAL, "x and error must be fp32")
    _need(x, n, "x")
    _need(error, n, "error")
    _need_payload(words, scales, n, chunk)
    _check(lib.zds_onebit_compress(_dev_ptr(x, "x"), _dev_ptr(error, "error"), n, chunk, _dev_ptr(words, "words"),
                                   _dev_ptr(scales, "scales"), _stream(stream)))


def zds_onebit_decompress(payloads, chunk, dst, mode=ZDS_OVERWRITE, stream=None, n=None):
    """payloads: [(words, scales)] of the peers, in sum order."""
    n = dst.numel() if n is None else n
    if dst.dtype != torch.float32:
        raise ZdsError(ZDS_EINVAL, "dst must be fp32")
    _need(dst, n, "dst")
    for w, sc in payloads:
        _need_payload(w, sc, n, chunk)
    W = (_P * len(payloads))(*[_dev_ptr(w, "words") for w, _ in payloads])
    S = (_P * len(payloads))(*[_dev_ptr(s, "scales") for _, s in payloads])
    _check(lib.zds_onebit_decompress(W, S, len(payloads), n, chunk, _dev_ptr(dst, "dst"), mode, _stream(stream)))


# ------------------------------------------------------------------ checkpoints

def checkpoint_meta(numels, world, rank, flat_align, stage=1, offload=0):
    """The CheckpointMeta of rank's shard of the layout of numels."""
    _, total = zds_flat_layout(numels, flat_align)
    lo, hi = zds_shard_range(total, world, rank, flat_align)
    return CheckpointMeta(world, rank, flat_align, stage, int(offload), len(numels), total, lo, hi)


def _is_device(x):
    return isinstance(x, torch.Tensor) and x.device.type == "cuda"


def _ckpt_buffers(meta, master, exp_avg, exp_avg_sq, state):
    """Location and addresses of a shard: all device tensors (state: the
    64-byte device state), or all host buffers (state: a StepState)."""
    for name, t in (("master", master), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        _need(t, meta.hi - meta.lo, name)
    if _is_device(master):
        _need_bytes(state, STATE_BYTES, "state")
        ptrs = [_dev_ptr(master, "master"), _dev_ptr(exp_avg, "exp_avg"), _dev_ptr(exp_avg_sq, "exp_avg_sq"),
                _dev_ptr(state, "state")]
        return ZDS_ON_DEVICE, ptrs
    if not isinstance(state, StepState):
        raise ZdsError(ZDS_EINVAL, "a host shard takes its state as a StepState")
    ptrs = [_host_ptr(master, "master"), _host_ptr(exp_avg, "exp_avg"), _host_ptr(exp_avg_sq, "exp_avg_sq"),
            ctypes.addressof(state)]
    return ZDS_ON_HOST, ptrs


def zds_checkpoint_save(path, meta, numels, master, exp_avg, exp_avg_sq, state, stream=None):
    loc, p = _ckpt_buffers(meta, master, exp_avg, exp_avg_sq, state)
    _check(lib.zds_checkpoint_save(os.fsencode(path), ctypes.byref(meta), _i64arr(numels), p[0], p[1], p[2],
                                   p[3], loc, _stream(stream) if loc == ZDS_ON_DEVICE else None))


def zds_checkpoint_read_meta(path, max_tensors=1 << 20):
    """(CheckpointMeta, StepState, tensor table) of a checkpoint file."""
    meta, st = CheckpointMeta(), StepState()
    _check(lib.zds_checkpoint_read_meta(os.fsencode(path), ctypes.byref(meta), ctypes.byref(st), None, 0))
    table = (ctypes.c_int64 * max(1, meta.num_tensors))()
    _check(lib.zds_checkpoint_read_meta(os.fsencode(path), ctypes.byref(meta), None, table,
                                        min(meta.num_tensors, max_tensors)))
    return meta, st, [int(x) for x in table[:meta.num_tensors]]


def zds_checkpoint_load(path, meta, numels, master, exp_avg, exp_avg_sq, state, stream=None):
    loc, p = _ckpt_buffers(meta, master, exp_avg, exp_avg_sq, state)
    _check(lib.zds_checkpoint_load(os.fsencode(path), ctypes.byref(meta), _i64arr(numels), p[0], p[1], p[2],
                                   p[3], loc, _stream(stream) if loc == ZDS_ON_DEVICE else None))


def zds_consolidate_fp32(paths, section=0, out=None):
    """Merged fp32 tensors of a world's shard files: a flat float32 numpy
    array, tensors one after another in table order (see
    split_consolidated)."""
    import numpy as np
    _, _, numels = zds_checkpoint_read_meta(paths[0])
    total = int(sum(numels))
    if out is None:
        out = np.empty(total, dtype=np.float32)
    arr = (ctypes.c_char_p * len(paths))(*[os.fsencode(x) for x in paths])
    n = out.numel() if isinstance(out, torch.Tensor) else out.size
    _check(lib.zds_consolidate_fp32(arr, len(paths), section, _host_ptr(out, "out") if total else None, n))
    return out


def split_consolidated(flat, numels):
    outs, a = [], 0
    for n in numels:
        outs.append(flat[a:a + n])
        a += n
    return outs


def zds_step_state_init(state, cfg, t0=0, beta1_pow0=1.0, beta2_pow0=1.0, stream=None):
    _need_bytes(state, STATE_BYTES, "state")
    _check(lib.zds_step_state_init(_dev_ptr(state, "state"), ctypes.byref(cfg), t0, beta1_pow0,
                                   beta2_pow0, _stream(stream)))


def zds_loss_scaler_update(state, scalars, hp, stream=None):
    _need_bytes(state, STATE_BYTES, "state")
    _need_bytes(scalars, SCALARS_BYTES, "scalars")
    _check(lib.zds_loss_scaler_update(_dev_ptr(state, "state"), _dev_ptr(scalars, "scalars"),
                                      ctypes.byref(hp), _stream(stream)))


# ------------------------------------------------------------------ host twins

def zds_step_state_init_host(cfg, t0=0, beta1_pow0=1.0, beta2_pow0=1.0):
    s = StepState()
    _check(lib.zds_step_state_init_host(ctypes.byref(s), ctypes.byref(cfg), t0, beta1_pow0, beta2_pow0))
    return s


def zds_loss_scaler_update_host(state, overflow, hp):
    _check(lib.zds_loss_scaler_update_host(ctypes.byref(state), int(overflow), ctypes.byref(hp)))
    return state


def zds_adam_constants_host(hp, state):
    out = (ctypes.c_float * 5)()
    _check(lib.zds_adam_constants_host(ctypes.byref(hp), ctypes.byref(state), out))
    return dict(zip(("step_size", "bc2_sqrt", "decay", "omb1", "omb2"), list(out)))


def zds_clip_scalars_host(sumsq, scale, accum_steps, max_norm):
    s = StepScalars()
    _check(lib.zds_clip_scalars_host(sumsq, scale, accum_steps, max_norm, ctypes.byref(s)))
    return s


def zds_last_error():
    return lib.zds_last_error().decode()


def zds_abi_version():
    return lib.zds_abi_version()


# ------------------------------------------------------------------ device structs

def new_state(device="cuda"):
    return torch.zeros(STATE_BYTES, dtype=torch.uint8, device=device)


def new_scalars(device="cuda"):
    return torch.zeros(SCALARS_BYTES, dtype=torch.uint8, device=device)


def new_workspace(n, device="cuda"):
    return torch.empty((zds_workspace_bytes(n) + 7) // 8, dtype=torch.float64, device=device)


def new_plan_workspace(plan, device="cuda"):
    return torch.empty(max(1, (zds_plan_norm_workspace_bytes(plan) + 7) // 8), dtype=torch.float64,
                       device=device)


def read_state(t):
    return StepState.from_buffer_copy(bytes(t.cpu().numpy().tobytes()))


def read_scalars(t):
    return StepScalars.from_buffer_copy(bytes(t.cpu().numpy().tobytes()))


def write_scalars(t, scalars):
    """Host -> device copy of a StepScalars (tests force flags this way)."""
    import numpy as np
    buf = np.frombuffer(bytes(scalars), dtype=np.uint8).copy()
    t.copy_(torch.from_numpy(buf).to(t.device))
