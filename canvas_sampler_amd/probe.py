"""ctypes binding of libdgprobe.so (include/dg_probe.h): the plain streaming
read used as the measured reference point for the statistics pass."""
import ctypes
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdgprobe.so")
EXPORTS = ["dg_probe_stream_read"]
_lib = None


def lib():
    """Loads the probe library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: run canvas_sampler_amd.build.build()")
        h = ctypes.CDLL(_LIB_PATH)
        h.dg_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        h.dg_probe_stream_read.restype = ctypes.c_int
        _lib = h
    return _lib


def stream_read(buf, grid, block, sink, stream):
    """Enqueues one read of the whole of `buf` (a CUDA tensor) on `stream`."""
    rc = lib().dg_probe_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), grid,
                                    block, sink.data_ptr(), stream.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"dg_probe_stream_read failed with status {rc}")
