"""ctypes binding of librank_step.so (C ABI in include/fsdp_step.h).

Argument marshalling only: every function here converts its Python arguments
(torch tensors, ints, dicts) to the C types of the entry point of the same
name, calls it, and raises ``FsdpError`` on a nonzero status.  No arithmetic of
the step happens here.  The library is loaded on first use and a missing
library is an error -- there is no fallback.

Pointer arguments accept a torch tensor (its ``data_ptr()``), a raw address
(int) or None (NULL).  Stream arguments accept a ``torch.cuda.Stream``, a raw
``hipStream_t`` (int) or None, which means torch's current stream on the
current device so that the work is ordered with torch's own.
"""

import ctypes
import os
import threading

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librank_step.so")
_lib = None
_lock = threading.Lock()

FSDP_OK = 0
ERRORS = {-1: "FSDP_E_ARG", -2: "FSDP_E_DTYPE", -3: "FSDP_E_ALIGN", -4: "FSDP_E_ALIAS",
          -5: "FSDP_E_HIP", -6: "FSDP_E_CAPACITY", -7: "FSDP_E_STATE"}
DTYPES = {"f32": 0, "bf16": 1}
LAYOUTS = {"flat": 0, "shard0": 1, "owner": 2}

# Every function the header declares; the CPU tests check each is exported.
EXPORTS = ("fsdp_last_error", "fsdp_shard_layout", "fsdp_rank_buffer_layout", "fsdp_reduce_grad_shard",
           "fsdp_adamw_shard_step", "fsdp_cast_unshard_bf16", "fsdp_mt_plan_create",
           "fsdp_mt_step", "fsdp_mt_step_capturable", "fsdp_mt_step_clipped_capturable",
           "fsdp_mt_step_amax_capturable", "fsdp_mt_step_fp8_capturable",
           "fsdp_mt_plan_get_info", "fsdp_mt_plan_destroy",
           "fsdp_mt_reduce_sqnorm", "fsdp_clip_coef", "fsdp_mt_step_clipped",
           "fsdp_mt_step_amax", "fsdp_mt_cast_fp8", "fsdp_mt_step_fp8",
           "fsdp_mt_reduce_accumulate", "fsdp_grad_accumulate", "fsdp_reduce_sqnorm_noalloc")

# fsdp_reduce_sqnorm_noalloc's limit (FSDP_NOALLOC_MAX_NUMEL in the header)
NOALLOC_MAX_NUMEL = 33_292_288


class FsdpError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code
        self.name = ERRORS.get(code, str(code))


class TensorShape(ctypes.Structure):
    _fields_ = [("numel", ctypes.c_int64), ("dim0", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class ShardView(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("shard_numel", "valid", "global_offset",
                                              "view_offset", "view_numel", "tensor_offset",
                                              "owner")]


class LayoutSummary(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("logical_numel", "physical_numel", "shard_numel",
                                              "pad_numel", "bytes_param", "bytes_grad",
                                              "bytes_optim", "bytes_master",
                                              "bytes_grad_unsharded")]


class RankBuffers(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("total_bytes", "region_align", "slice_stride",
                                              "param_offset", "exp_avg_offset", "exp_avg_sq_offset",
                                              "slices_offset", "bf16_offset", "grad_out_offset",
                                              "fp8_offset")]


class AdamWHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
                ("step", ctypes.c_int64)]


class MtTensor(ctypes.Structure):
    _fields_ = [("param_fp32", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p),
                ("exp_avg_sq", ctypes.c_void_p), ("grad_slices", ctypes.c_void_p),
                ("slice_stride", ctypes.c_int64), ("unshard_bf16_out", ctypes.c_void_p),
                ("grad_shard_out", ctypes.c_void_p), ("shard_numel", ctypes.c_int64),
                ("valid", ctypes.c_int64), ("unshard_fp8_out", ctypes.c_void_p),
                ("grad_slice_ptrs", ctypes.c_void_p)]


class MtPlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("n_tensors", "n_chunks", "n_blocks", "total_numel",
                                              "total_valid", "chunk_numel")] + [
        ("n_slices", ctypes.c_int32), ("slice_dtype", ctypes.c_int32),
        ("step_one_range", ctypes.c_int32), ("store_policy", ctypes.c_int32)]


def lib_path():
    return _LIB_PATH


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it first "
                               "(python -m rank_step_amd.build or __graft_entry__.build())")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.fsdp_last_error.restype = ctypes.c_char_p
        L.fsdp_last_error.argtypes = []
        sig = {
            "fsdp_shard_layout": [i32, i32, i32, ctypes.POINTER(TensorShape), i32, i32,
                                  ctypes.POINTER(ShardView), ctypes.POINTER(LayoutSummary)],
            "fsdp_rank_buffer_layout": [ctypes.c_int64, i32, i32, i32, i32, i32, ctypes.POINTER(RankBuffers)],
            "fsdp_reduce_grad_shard": [vp, vp, i32, i64, i32, i64, i64, vp],
            "fsdp_adamw_shard_step": [vp, vp, vp, vp, i64, i64, ctypes.POINTER(AdamWHparams), vp],
            "fsdp_cast_unshard_bf16": [vp, vp, i64, i64, vp],
            "fsdp_mt_plan_create": [ctypes.POINTER(vp), ctypes.POINTER(MtTensor), i32, i32, i32, vp],
            "fsdp_mt_step": [vp, ctypes.POINTER(AdamWHparams), vp],
            "fsdp_mt_step_capturable": [vp, ctypes.POINTER(AdamWHparams), vp, vp, vp],
            "fsdp_mt_step_clipped_capturable": [vp, ctypes.POINTER(AdamWHparams), vp, vp, vp, vp],
            "fsdp_mt_step_amax_capturable": [vp, ctypes.POINTER(AdamWHparams), vp, vp, vp, vp],
            "fsdp_mt_step_fp8_capturable": [vp, ctypes.POINTER(AdamWHparams), vp, vp, vp, vp, vp],
            "fsdp_mt_plan_get_info": [vp, ctypes.POINTER(MtPlanInfo)],
            "fsdp_mt_plan_destroy": [vp],
            "fsdp_mt_reduce_sqnorm": [vp, vp, vp],
            "fsdp_clip_coef": [vp, vp, vp, i32, ctypes.c_double, vp],
            "fsdp_mt_step_clipped": [vp, ctypes.POINTER(AdamWHparams), vp, vp],
            "fsdp_mt_step_amax": [vp, ctypes.POINTER(AdamWHparams), vp, vp],
            "fsdp_mt_cast_fp8": [vp, vp, i32, vp, vp],
            "fsdp_mt_step_fp8": [vp, ctypes.POINTER(AdamWHparams), vp, vp, vp],
            "fsdp_mt_reduce_accumulate": [vp, i32, vp, vp],
            "fsdp_grad_accumulate": [vp, vp, i32, i64, i32, vp],
            "fsdp_reduce_sqnorm_noalloc": [vp, vp, vp, i32, i64, i32, i64, i64, vp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = i32
        _lib = L
        return L


def _check(code):
    if code != FSDP_OK:
        msg = lib().fsdp_last_error().decode(errors="replace")
        raise FsdpError(code, msg)


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _dtype(d):
    return DTYPES[d] if isinstance(d, str) else int(d)


def _hparams(hp, step):
    return AdamWHparams(float(hp["lr"]), float(hp["beta1"]), float(hp["beta2"]),
                        float(hp["eps"]), float(hp["weight_decay"]), int(step))


# ---------------------------------------------------------------- entry points

def fsdp_rank_buffer_layout(shard_numel, n_slices, slice_dtype, bf16_slots=1, grad_out=False,
                            fp8_out=False):
    """Placement of one rank's step buffers in one allocation, as a dict of
    ints named as in the header (offsets in bytes, -1 for absent buffers)."""
    r = RankBuffers()
    _check(lib().fsdp_rank_buffer_layout(int(shard_numel), int(n_slices), _dtype(slice_dtype),
                                         int(bf16_slots), int(bool(grad_out)), int(bool(fp8_out)),
                                         ctypes.byref(r)))
    return {f: getattr(r, f) for f, _ in RankBuffers._fields_}


def fsdp_shard_layout(mode, world_size, rank, shapes, has_master):
    """``shapes``: (numel, dim0, dtype) triples.  Returns (views, summary) as
    lists/dicts of ints, fields named as in the header."""
    n = len(shapes)
    arr = (TensorShape * max(n, 1))()
    for i, (numel, dim0, dt) in enumerate(shapes):
        arr[i] = TensorShape(int(numel), int(dim0), _dtype(dt), 0)
    views = (ShardView * max(n, 1))()
    summ = LayoutSummary()
    m = LAYOUTS[mode] if isinstance(mode, str) else int(mode)
    _check(lib().fsdp_shard_layout(m, int(world_size), int(rank), arr, n, int(bool(has_master)),
                                   views, ctypes.byref(summ)))
    vs = [{f: getattr(views[i], f) for f, _ in ShardView._fields_} for i in range(n)]
    return vs, {f: getattr(summ, f) for f, _ in LayoutSummary._fields_}


def fsdp_reduce_grad_shard(grad_shard_out, grad_slices, slice_dtype, slice_stride, n_slices,
                           shard_numel, valid, stream=None):
    _check(lib().fsdp_reduce_grad_shard(_ptr(grad_shard_out), _ptr(grad_slices),
                                        _dtype(slice_dtype), int(slice_stride), int(n_slices),
                                        int(shard_numel), int(valid), _stream(stream)))


def fsdp_adamw_shard_step(param_fp32, exp_avg, exp_avg_sq, grad_shard, shard_numel, valid, hp,
                          step, stream=None):
    h = _hparams(hp, step)
    _check(lib().fsdp_adamw_shard_step(_ptr(param_fp32), _ptr(exp_avg), _ptr(exp_avg_sq),
                                       _ptr(grad_shard), int(shard_numel), int(valid),
                                       ctypes.byref(h), _stream(stream)))


def fsdp_cast_unshard_bf16(unshard_bf16_out, param_fp32, shard_numel, valid, stream=None):
    _check(lib().fsdp_cast_unshard_bf16(_ptr(unshard_bf16_out), _ptr(param_fp32),
                                        int(shard_numel), int(valid), _stream(stream)))


def fsdp_mt_plan_create(tensors, n_slices, slice_dtype, stream=None):
    """``tensors``: dicts with the fsdp_mt_tensor fields.  Returns an opaque
    handle (int) to pass to fsdp_mt_step / fsdp_mt_plan_destroy."""
    n = len(tensors)
    arr = (MtTensor * max(n, 1))()
    tables = []  # host arrays of slice pointers, alive until the plan has copied them
    for i, t in enumerate(tensors):
        table = None
        if t.get("grad_slice_ptrs") is not None:
            ptrs = [_ptr(p) for p in t["grad_slice_ptrs"]]
            table = (ctypes.c_void_p * max(len(ptrs), 1))(*ptrs)
            tables.append(table)
        arr[i] = MtTensor(_ptr(t["param_fp32"]), _ptr(t["exp_avg"]), _ptr(t["exp_avg_sq"]),
                          _ptr(t.get("grad_slices")), int(t.get("slice_stride", 0)),
                          _ptr(t.get("unshard_bf16_out")), _ptr(t.get("grad_shard_out")),
                          int(t["shard_numel"]), int(t["valid"]), _ptr(t.get("unshard_fp8_out")),
                          ctypes.cast(table, ctypes.c_void_p) if table is not None else None)
    h = ctypes.c_void_p()
    _check(lib().fsdp_mt_plan_create(ctypes.byref(h), arr, n, int(n_slices), _dtype(slice_dtype),
                                     _stream(stream)))
    return h.value


def fsdp_mt_step(plan, hp, step, stream=None):
    h = _hparams(hp, step)
    _check(lib().fsdp_mt_step(plan, ctypes.byref(h), _stream(stream)))


def fsdp_mt_plan_get_info(plan):
    info = MtPlanInfo()
    _check(lib().fsdp_mt_plan_get_info(plan, ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in MtPlanInfo._fields_}


def fsdp_mt_plan_destroy(plan):
    _check(lib().fsdp_mt_plan_destroy(plan))


def fsdp_mt_reduce_sqnorm(plan, sqnorm_out, stream=None):
    _check(lib().fsdp_mt_reduce_sqnorm(plan, _ptr(sqnorm_out), _stream(stream)))


def fsdp_clip_coef(coef_out, norm_out, sqnorms, n_ranks, max_norm, stream=None):
    _check(lib().fsdp_clip_coef(_ptr(coef_out), _ptr(norm_out), _ptr(sqnorms), int(n_ranks),
                                float(max_norm), _stream(stream)))


def fsdp_mt_step_clipped(plan, hp, step, grad_scale, stream=None):
    h = _hparams(hp, step)
    _check(lib().fsdp_mt_step_clipped(plan, ctypes.byref(h), _ptr(grad_scale), _stream(stream)))


def fsdp_mt_step_capturable(plan, hp, step_dev, stream=None, lr_dev=None):
    """``step_dev``: device int64 [1], the steps taken so far (advanced by one);
    ``lr_dev``: None (hp's lr) or a device float64 [1] read in its place."""
    h = _hparams(hp, 1)
    _check(lib().fsdp_mt_step_capturable(plan, ctypes.byref(h), _ptr(step_dev), _ptr(lr_dev),
                                         _stream(stream)))


def fsdp_mt_step_clipped_capturable(plan, hp, step_dev, grad_scale, stream=None, lr_dev=None):
    h = _hparams(hp, 1)
    _check(lib().fsdp_mt_step_clipped_capturable(plan, ctypes.byref(h), _ptr(step_dev), _ptr(lr_dev),
                                                 _ptr(grad_scale), _stream(stream)))


def fsdp_mt_step_amax_capturable(plan, hp, step_dev, amax_out, stream=None, lr_dev=None):
    h = _hparams(hp, 1)
    _check(lib().fsdp_mt_step_amax_capturable(plan, ctypes.byref(h), _ptr(step_dev), _ptr(lr_dev),
                                              _ptr(amax_out), _stream(stream)))


def fsdp_mt_step_fp8_capturable(plan, hp, step_dev, scale_in, amax_out, stream=None, lr_dev=None):
    h = _hparams(hp, 1)
    _check(lib().fsdp_mt_step_fp8_capturable(plan, ctypes.byref(h), _ptr(step_dev), _ptr(lr_dev),
                                             _ptr(scale_in), _ptr(amax_out), _stream(stream)))


def fsdp_mt_step_amax(plan, hp, step, amax_out, stream=None):
    h = _hparams(hp, step)
    _check(lib().fsdp_mt_step_amax(plan, ctypes.byref(h), _ptr(amax_out), _stream(stream)))


def fsdp_mt_cast_fp8(plan, amax_ranks, n_ranks, scale_out=None, stream=None):
    _check(lib().fsdp_mt_cast_fp8(plan, _ptr(amax_ranks), int(n_ranks), _ptr(scale_out),
                                  _stream(stream)))


def fsdp_mt_step_fp8(plan, hp, step, scale_in, amax_out, stream=None):
    h = _hparams(hp, step)
    _check(lib().fsdp_mt_step_fp8(plan, ctypes.byref(h), _ptr(scale_in), _ptr(amax_out),
                                  _stream(stream)))


def fsdp_mt_reduce_accumulate(plan, accumulate, sqnorm_out=None, stream=None):
    _check(lib().fsdp_mt_reduce_accumulate(plan, int(bool(accumulate)), _ptr(sqnorm_out),
                                           _stream(stream)))


def fsdp_grad_accumulate(acc, micro, micro_dtype, numel, accumulate, stream=None):
    _check(lib().fsdp_grad_accumulate(_ptr(acc), _ptr(micro), _dtype(micro_dtype), int(numel),
                                      int(bool(accumulate)), _stream(stream)))


def fsdp_reduce_sqnorm_noalloc(grad_shard_out, sqnorm_out, grad_slices, slice_dtype, slice_stride,
                               n_slices, shard_numel, valid, stream=None):
    _check(lib().fsdp_reduce_sqnorm_noalloc(_ptr(grad_shard_out), _ptr(sqnorm_out), _ptr(grad_slices),
                                            _dtype(slice_dtype), int(slice_stride), int(n_slices),
                                            int(shard_numel), int(valid), _stream(stream)))


class MtPlan:
    """Owns one fsdp_mt_plan handle (and keeps the Python objects whose
    buffers it references alive)."""

    def __init__(self, tensors, n_slices, slice_dtype, stream=None):
        self.handle = None
        self._keep = tensors
        self.handle = fsdp_mt_plan_create(tensors, n_slices, slice_dtype, stream)

    def step(self, hp, step, stream=None):
        fsdp_mt_step(self.handle, hp, step, stream)

    def step_capturable(self, hp, step_dev, stream=None, lr_dev=None):
        fsdp_mt_step_capturable(self.handle, hp, step_dev, stream, lr_dev)

    def step_clipped_capturable(self, hp, step_dev, grad_scale, stream=None, lr_dev=None):
        fsdp_mt_step_clipped_capturable(self.handle, hp, step_dev, grad_scale, stream, lr_dev)

    def step_amax_capturable(self, hp, step_dev, amax_out, stream=None, lr_dev=None):
        fsdp_mt_step_amax_capturable(self.handle, hp, step_dev, amax_out, stream, lr_dev)

    def step_fp8_capturable(self, hp, step_dev, scale_in, amax_out, stream=None, lr_dev=None):
        fsdp_mt_step_fp8_capturable(self.handle, hp, step_dev, scale_in, amax_out, stream, lr_dev)

    def info(self):
        return fsdp_mt_plan_get_info(self.handle)

    def reduce_sqnorm(self, sqnorm_out, stream=None):
        fsdp_mt_reduce_sqnorm(self.handle, sqnorm_out, stream)

    def step_clipped(self, hp, step, grad_scale, stream=None):
        fsdp_mt_step_clipped(self.handle, hp, step, grad_scale, stream)

    def reduce_accumulate(self, accumulate, sqnorm_out=None, stream=None):
        fsdp_mt_reduce_accumulate(self.handle, accumulate, sqnorm_out, stream)

    def step_amax(self, hp, step, amax_out, stream=None):
        fsdp_mt_step_amax(self.handle, hp, step, amax_out, stream)

    def cast_fp8(self, amax_ranks, n_ranks, scale_out=None, stream=None):
        fsdp_mt_cast_fp8(self.handle, amax_ranks, n_ranks, scale_out, stream)

    def step_fp8(self, hp, step, scale_in, amax_out, stream=None):
        fsdp_mt_step_fp8(self.handle, hp, step, scale_in, amax_out, stream)

    def close(self):
        if self.handle is not None:
            fsdp_mt_plan_destroy(self.handle)
            self.handle = None
            self._keep = None

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
