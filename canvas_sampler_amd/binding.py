"""ctypes binding of libdgcanvas.so (include/dg_canvas.h): argument marshalling
only. Every step of the sampler runs in the library's HIP kernels; torch is
used for device memory (tensor data pointers) and streams.

The library must have been built (canvas_sampler_amd.build.build()); loading
fails loudly otherwise — there is no fallback implementation.
"""
import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdgcanvas.so")

DG_OK = 0
DG_ERR_INVALID_ARG = 1
DG_ERR_UNSUPPORTED = 2
DG_ERR_OUT_OF_MEMORY = 3
DG_ERR_DEVICE = 4
DG_ERR_CALLBACK = 5
DG_DTYPE_F32 = 0
DG_DTYPE_BF16 = 1

STATUS_NAMES = {0: "DG_OK", 1: "DG_ERR_INVALID_ARG", 2: "DG_ERR_UNSUPPORTED",
                3: "DG_ERR_OUT_OF_MEMORY", 4: "DG_ERR_DEVICE", 5: "DG_ERR_CALLBACK"}

# Every symbol include/dg_canvas.h declares.
EXPORTS = ["dg_params_default", "dg_params_check", "dg_create", "dg_destroy", "dg_last_error",
           "dg_get_params", "dg_temperature", "dg_set_stats_split", "dg_canvas_init",
           "dg_canvas_stats", "dg_accept_renoise", "dg_sampler_step", "dg_run_canvas",
           "dg_run_canvas_resident", "dg_generate", "dg_tokens_per_forward",
           "dg_self_condition", "dg_sampler_step_selfcond",
           "dg_lmhead_logits", "dg_lmhead_workspace_bytes", "dg_lmhead_sampler_step",
           "dg_sampler_step_noalloc", "dg_version"]


class DgParams(ctypes.Structure):
    _fields_ = [("canvas_len", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("entropy_bound", ctypes.c_float), ("temp_start", ctypes.c_float),
                ("temp_end", ctypes.c_float), ("temp_steps", ctypes.c_int32),
                ("max_steps", ctypes.c_int32), ("stop_mean_entropy", ctypes.c_float)]


class DgStepOut(ctypes.Structure):
    _fields_ = [("canvas_out", ctypes.c_void_p), ("argmax_out", ctypes.c_void_p),
                ("sample_out", ctypes.c_void_p), ("accept_out", ctypes.c_void_p),
                ("entropy_out", ctypes.c_void_p), ("n_accept_out", ctypes.c_void_p),
                ("mean_entropy_out", ctypes.c_void_p), ("stop_out", ctypes.c_void_p)]


DENOISE_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p)
BLOCK_DENOISE_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p)
CACHE_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                            ctypes.c_void_p)

_lib = None


class DgError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "canvas_sampler_amd.build.build() (no fallback exists)")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        sig = {
            "dg_params_default": [ctypes.POINTER(DgParams)],
            "dg_params_check": [ctypes.POINTER(DgParams)],
            "dg_create": [ctypes.POINTER(vp), ctypes.c_int, i32, ctypes.POINTER(DgParams)],
            "dg_destroy": [vp],
            "dg_get_params": [vp, ctypes.POINTER(DgParams)],
            "dg_temperature": [ctypes.POINTER(DgParams), i32, ctypes.POINTER(ctypes.c_float)],
            "dg_set_stats_split": [vp, i32],
            "dg_canvas_init": [vp, i32, vp, vp, vp],
            "dg_canvas_stats": [vp, i32, vp, ctypes.c_int, i64, vp, i32, vp, vp, vp, vp, vp, vp],
            "dg_accept_renoise": [vp, i32, vp, vp, vp, i32, vp, vp, vp, ctypes.POINTER(DgStepOut), vp],
            "dg_sampler_step": [vp, i32, vp, ctypes.c_int, i64, vp, i32, vp, vp, vp,
                                ctypes.POINTER(DgStepOut), vp],
            "dg_run_canvas": [vp, i32, vp, DENOISE_FN, vp, ctypes.c_int, vp, vp, vp, vp, vp],
            "dg_run_canvas_resident": [vp, i32, vp, DENOISE_FN, vp, ctypes.c_int, vp, vp, vp, vp,
                                       i32, vp],
            "dg_generate": [vp, i32, vp, i32, BLOCK_DENOISE_FN, CACHE_FN, vp, ctypes.c_int, vp, vp,
                            vp, vp, i32, vp],
            "dg_tokens_per_forward": [vp, i32, i32, i32, vp, vp],
            "dg_self_condition": [vp, i32, vp, ctypes.c_int, i64, vp, vp, vp, i32, vp, vp],
            "dg_sampler_step_selfcond": [vp, i32, vp, ctypes.c_int, i64, vp, i32, vp, vp, vp, vp, i32, vp,
                                         ctypes.POINTER(DgStepOut), vp],
            "dg_lmhead_logits": [vp, i32, vp, vp, i32, vp, i64, vp],
            "dg_lmhead_workspace_bytes": [vp, i32, ctypes.POINTER(ctypes.c_int64)],
            "dg_lmhead_sampler_step": [vp, i32, vp, vp, i32, vp, i64, vp, i32, vp, vp, vp, vp,
                                       ctypes.POINTER(DgStepOut), vp],
            "dg_sampler_step_noalloc": [ctypes.POINTER(DgParams), i32, vp, ctypes.c_int, i64, vp, i32, vp, vp,
                                        vp, ctypes.POINTER(DgStepOut), vp],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.dg_last_error.argtypes = [vp]
        L.dg_last_error.restype = ctypes.c_char_p
        L.dg_version.argtypes = []
        L.dg_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def tokens_per_forward(steps_used, canvas_len):
    """dg_tokens_per_forward on a host int32 array [n_canvases, B]; returns
    (per-stream TPF list, TPF over all streams)."""
    import numpy as np
    steps = np.ascontiguousarray(steps_used, dtype=np.int32)
    n, b = steps.shape
    per = (ctypes.c_double * b)()
    total = ctypes.c_double()
    _check(lib().dg_tokens_per_forward(steps.ctypes.data_as(ctypes.c_void_p), n, b, canvas_len,
                                       per, ctypes.byref(total)))
    return list(per), total.value


def _check(status, ctx=None):
    if status != DG_OK:
        raise DgError(status, lib().dg_last_error(ctx).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return DG_DTYPE_BF16
    if t.dtype == torch.float32:
        return DG_DTYPE_F32
    raise TypeError(f"logits dtype {t.dtype} is not float32 or bfloat16")


def params_default(**overrides):
    p = DgParams()
    _check(lib().dg_params_default(ctypes.byref(p)))
    for k, v in overrides.items():
        setattr(p, k, v)
    return p


def params_check(p):
    _check(lib().dg_params_check(ctypes.byref(p)))


def dg_temperature(p, step):
    out = ctypes.c_float()
    _check(lib().dg_temperature(ctypes.byref(p), step, ctypes.byref(out)))
    return out.value


class Context:
    """Owns a dg_ctx (device scratch for up to max_batch canvases)."""

    def __init__(self, params=None, max_batch=1, device=0):
        self.params = params if params is not None else params_default()
        h = ctypes.c_void_p()
        _check(lib().dg_create(ctypes.byref(h), device, max_batch, ctypes.byref(self.params)))
        self.handle = h
        self.max_batch = max_batch
        self.device = device

    def close(self):
        if self.handle:
            lib().dg_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _chk(self, status):
        _check(status, self.handle)

    @property
    def L(self):
        return self.params.canvas_len

    @property
    def V(self):
        return self.params.vocab

    def set_stats_split(self, nsplit):
        self._chk(lib().dg_set_stats_split(self.handle, nsplit))

    def dg_canvas_init(self, seeds, canvas, stream=None):
        self._chk(lib().dg_canvas_init(self.handle, seeds.shape[0], _ptr(seeds), _ptr(canvas),
                                       _stream(stream)))

    def dg_canvas_stats(self, logits, temperature, step, seeds, entropy, argmax, sample,
                        active=None, batch=None, row_stride=None, stream=None):
        B = batch if batch is not None else seeds.shape[0]
        stride = row_stride if row_stride is not None else logits.stride(0)
        self._chk(lib().dg_canvas_stats(self.handle, B, _ptr(logits), _dtype_code(logits), stride,
                                        _ptr(temperature), step, _ptr(seeds), _ptr(active),
                                        _ptr(entropy), _ptr(argmax), _ptr(sample),
                                        _stream(stream)))

    @staticmethod
    def step_out(canvas_out, argmax_out=None, sample_out=None, accept_out=None,
                 entropy_out=None, n_accept_out=None, mean_entropy_out=None, stop_out=None):
        o = DgStepOut()
        for name, t in (("canvas_out", canvas_out), ("argmax_out", argmax_out),
                        ("sample_out", sample_out), ("accept_out", accept_out),
                        ("entropy_out", entropy_out), ("n_accept_out", n_accept_out),
                        ("mean_entropy_out", mean_entropy_out), ("stop_out", stop_out)):
            setattr(o, name, None if t is None else t.data_ptr())
        return o

    def dg_accept_renoise(self, entropy, argmax, sample, step, seeds, out, prev_argmax=None,
                          active=None, batch=None, stream=None):
        B = batch if batch is not None else seeds.shape[0]
        self._chk(lib().dg_accept_renoise(self.handle, B, _ptr(entropy), _ptr(argmax),
                                          _ptr(sample), step, _ptr(seeds), _ptr(prev_argmax),
                                          _ptr(active), ctypes.byref(out), _stream(stream)))

    def dg_sampler_step(self, logits, temperature, step, seeds, out, prev_argmax=None,
                        active=None, batch=None, row_stride=None, stream=None):
        B = batch if batch is not None else seeds.shape[0]
        stride = row_stride if row_stride is not None else logits.stride(0)
        self._chk(lib().dg_sampler_step(self.handle, B, _ptr(logits), _dtype_code(logits), stride,
                                        _ptr(temperature), step, _ptr(seeds), _ptr(prev_argmax),
                                        _ptr(active), ctypes.byref(out), _stream(stream)))

    def dg_lmhead_logits(self, hidden, weight, logits, stream=None):
        """logits[:rows, :V] = hidden @ weight (bf16 operands, fp32 result)."""
        rows, k = hidden.shape
        self._chk(lib().dg_lmhead_logits(self.handle, rows, _ptr(hidden), _ptr(weight), k,
                                         _ptr(logits), logits.stride(0), _stream(stream)))

    def dg_lmhead_workspace_bytes(self, B):
        """Bytes of device workspace dg_lmhead_sampler_step needs for B canvases."""
        n = ctypes.c_int64()
        self._chk(lib().dg_lmhead_workspace_bytes(self.handle, B, ctypes.byref(n)))
        return n.value

    def dg_lmhead_sampler_step(self, hidden, weight, workspace, temperature, step, seeds, out,
                               steps=None, prev_argmax=None, active=None, stream=None,
                               workspace_bytes=None):
        """workspace: a device tensor of at least dg_lmhead_workspace_bytes(B) bytes."""
        B = seeds.shape[0]
        nbytes = workspace_bytes if workspace_bytes is not None else \
            workspace.numel() * workspace.element_size()
        self._chk(lib().dg_lmhead_sampler_step(self.handle, B, _ptr(hidden), _ptr(weight),
                                               hidden.shape[1], _ptr(workspace), nbytes,
                                               _ptr(temperature), step, _ptr(steps), _ptr(seeds),
                                               _ptr(prev_argmax), _ptr(active), ctypes.byref(out),
                                               _stream(stream)))

    def dg_run_canvas(self, seeds, denoise, logits_scratch, final_argmax, stream=None):
        """seeds: list of ints (host). denoise(step, canvas_ptr, active_ptr, logits, stream)
        must enqueue on `stream` the writing of `logits` (a tensor [B*L, V]);
        canvas_ptr / active_ptr are device addresses of the library's current
        canvas (int32 [B, L]) and active flags (uint8 [B]); copy_from_device()
        reads them. Returns (steps_used list, stopped list)."""
        B = len(seeds)
        seeds_arr = (ctypes.c_uint64 * B)(*[int(s) & (2**64 - 1) for s in seeds])
        steps = (ctypes.c_int32 * B)()
        stopped = (ctypes.c_uint8 * B)()
        errors = []

        def _cb(user, step, canvas_p, active_p, logits_p, stream_p):
            try:
                denoise(step, canvas_p, active_p, logits_scratch, stream)
                return 0
            except Exception as exc:  # reported through DG_ERR_CALLBACK
                errors.append(exc)
                return 1

        cb = DENOISE_FN(_cb)
        status = lib().dg_run_canvas(self.handle, B, seeds_arr, cb, None,
                                     _dtype_code(logits_scratch), _ptr(logits_scratch),
                                     _ptr(final_argmax), steps, stopped, _stream(stream))
        if errors and status == DG_ERR_CALLBACK:
            raise errors[0]
        self._chk(status)
        return list(steps), [bool(x) for x in stopped]

    def dg_self_condition(self, logits, temperature, argmax, embed, out, batch=None,
                          row_stride=None, stream=None):
        """out [B*L, d] fp32 = softmax(logits / T) @ embed ([V, d] fp32), with
        argmax the statistics pass's output for these logits."""
        B = batch if batch is not None else temperature.shape[0]
        stride = row_stride if row_stride is not None else logits.stride(0)
        self._chk(lib().dg_self_condition(self.handle, B, _ptr(logits), _dtype_code(logits), stride,
                                          _ptr(temperature), _ptr(argmax), _ptr(embed),
                                          embed.shape[1], _ptr(out), _stream(stream)))

    def dg_sampler_step_selfcond(self, logits, temperature, step, seeds, embed, selfcond_out, out,
                                 prev_argmax=None, active=None, batch=None, row_stride=None,
                                 stream=None):
        """dg_sampler_step with the self-conditioning matmul (embed [V, d]
        fp32 -> selfcond_out [B*L, d] fp32) after the statistics pass."""
        B = batch if batch is not None else seeds.shape[0]
        stride = row_stride if row_stride is not None else logits.stride(0)
        self._chk(lib().dg_sampler_step_selfcond(
            self.handle, B, _ptr(logits), _dtype_code(logits), stride, _ptr(temperature), step,
            _ptr(seeds), _ptr(prev_argmax), _ptr(active), _ptr(embed), embed.shape[1],
            _ptr(selfcond_out), ctypes.byref(out), _stream(stream)))

    def dg_generate(self, seeds, n_canvases, denoise, cache_update, logits_scratch, tokens,
                    steps_used, stopped, check_every=0, stream=None):
        """seeds: device uint64 tensor [B] (torch.int64); tokens int32
        [B, n_canvases * L], steps_used int32 [n_canvases, B] and stopped uint8
        [n_canvases, B] are device outputs. denoise(k, step, canvas_ptr,
        active_ptr, logits, stream) and cache_update(k, canvas_ptr, stream)
        (or None) enqueue their work on `stream`."""
        B = seeds.numel()
        errors = []

        def _den(user, k, step, canvas_p, active_p, logits_p, stream_p):
            try:
                denoise(k, step, canvas_p, active_p, logits_scratch, stream)
                return 0
            except Exception as exc:  # reported through DG_ERR_CALLBACK
                errors.append(exc)
                return 1

        def _cache(user, k, canvas_p, stream_p):
            try:
                cache_update(k, canvas_p, stream)
                return 0
            except Exception as exc:
                errors.append(exc)
                return 1

        den_cb = BLOCK_DENOISE_FN(_den)
        cache_cb = CACHE_FN(_cache) if cache_update is not None else CACHE_FN()
        self._generate_cbs = (den_cb, cache_cb)
        status = lib().dg_generate(self.handle, B, _ptr(seeds), n_canvases, den_cb, cache_cb, None,
                                   _dtype_code(logits_scratch), _ptr(logits_scratch), _ptr(tokens),
                                   _ptr(steps_used), _ptr(stopped), int(check_every),
                                   _stream(stream))
        if errors and status == DG_ERR_CALLBACK:
            raise errors[0]
        self._chk(status)

    def dg_run_canvas_resident(self, seeds, denoise, logits_scratch, final_argmax, steps_used,
                               stopped, check_every=0, stream=None):
        """seeds: device uint64 tensor [B] (torch.int64); steps_used (int32 [B])
        and stopped (uint8 [B]) are device outputs. denoise as for
        dg_run_canvas. With check_every == 0 nothing waits for the device, so
        the call may run under HIP graph capture; the callback object is kept
        on the context until the next call (a replayed graph does not call it)."""
        B = seeds.numel()
        errors = []

        def _cb(user, step, canvas_p, active_p, logits_p, stream_p):
            try:
                denoise(step, canvas_p, active_p, logits_scratch, stream)
                return 0
            except Exception as exc:  # reported through DG_ERR_CALLBACK
                errors.append(exc)
                return 1

        self._resident_cb = cb = DENOISE_FN(_cb)
        status = lib().dg_run_canvas_resident(self.handle, B, _ptr(seeds), cb, None,
                                              _dtype_code(logits_scratch), _ptr(logits_scratch),
                                              _ptr(final_argmax), _ptr(steps_used), _ptr(stopped),
                                              int(check_every), _stream(stream))
        if errors and status == DG_ERR_CALLBACK:
            raise errors[0]
        self._chk(status)


_hip = None


def sampler_step_noalloc(params, logits, temperature, step, seeds, out, prev_argmax=None, active=None,
                         batch=None, row_stride=None, stream=None):
    """dg_sampler_step_noalloc: one step with no context and no allocation
    (static device scratch); arguments as Context.dg_sampler_step plus the
    params of the step."""
    B = batch if batch is not None else seeds.shape[0]
    stride = row_stride if row_stride is not None else logits.stride(0)
    _check(lib().dg_sampler_step_noalloc(ctypes.byref(params), B, _ptr(logits), _dtype_code(logits), stride,
                                         _ptr(temperature), step, _ptr(seeds), _ptr(prev_argmax), _ptr(active),
                                         ctypes.byref(out), _stream(stream)))


def copy_from_device(dst, src_ptr, stream=None):
    """Enqueues a device-to-device copy of dst.numel() elements from the raw
    device address src_ptr into tensor dst (hipMemcpyAsync on `stream`)."""
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_int, ctypes.c_void_p]
        _hip.hipMemcpyAsync.restype = ctypes.c_int
    nbytes = dst.numel() * dst.element_size()
    err = _hip.hipMemcpyAsync(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src_ptr), nbytes,
                              3, _stream(stream))  # 3 = hipMemcpyDeviceToDevice
    if err != 0:
        raise RuntimeError(f"hipMemcpyAsync failed with error {err}")


def version():
    return lib().dg_version().decode()
