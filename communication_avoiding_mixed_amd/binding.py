"""ctypes binding of libcasgd.so (the C ABI in include/casgd.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the method runs in the library's HIP kernels.  There is
no fallback: if the library has not been built, or no GPU is present, the
calls raise.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcasgd.so")

LOGISTIC, SQUARED, POISSON = 0, 1, 2
BF16, FP32, FP16, FP8 = 0, 1, 2, 3
OK, EINVAL, ENOMEM, EHIP = 0, -1, -2, -3
EXPORT_IDX, EXPORT_Y, EXPORT_YB, EXPORT_G, EXPORT_V, EXPORT_Z, EXPORT_R = range(7)
K_GATHER, K_GRAM, K_CHAIN, K_PIPE, K_TRAIN = range(5)
OPT_RECURRENCE, OPT_SPIN_LIMIT, OPT_MARGIN_BF16, OPT_CHAIN_LAYOUT, OPT_TRAIN_FORM, OPT_GRAM_BF16 = 0, 1, 2, 3, 4, 5
TRAIN_PERSISTENT, TRAIN_PER_STEP = 0, 1
LAYOUT_AUTO, LAYOUT_SPREAD, LAYOUT_ONE_XCD = 0, 1, 2
RECURRENCE_AUTO, RECURRENCE_ALL_TO_ALL, RECURRENCE_LOOKAHEAD = 0, 1, 2
KERNEL_NAMES = {K_GATHER: "gather", K_GRAM: "gram", K_CHAIN: "chain", K_PIPE: "pipe", K_TRAIN: "train"}

LOSS_IDS = {"logistic": LOGISTIC, "squared": SQUARED, "poisson": POISSON}
STORAGE_IDS = {"bf16": BF16, "fp32": FP32, "fp16": FP16, "fp8": FP8}

# every entry point declared in include/casgd.h: name -> (restype, argtypes)
_VP, _I64, _U64, _I, _F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int, ctypes.c_float
SIGNATURES = {
    "casgd_create": (_VP, [_VP, _VP, _I64, _I64, _I, _I]),
    "casgd_destroy": (None, [_VP]),
    "casgd_set_stream": (_I, [_VP, _VP]),
    "casgd_outer_step": (_I, [_VP, _I, _I, _F, _U64, _VP]),
    "casgd_outer_step_indices": (_I, [_VP, _I, _I, _F, _VP, _VP]),
    "casgd_train": (_I, [_VP, _I, _I, _F, _U64, _U64, _I, _VP]),
    "casgd_step_seed": (_U64, [_U64, _U64]),
    "casgd_loss": (_I, [_VP, _VP, ctypes.POINTER(ctypes.c_double)]),
    "casgd_debug_export": (_I, [_VP, _I, _VP, ctypes.c_size_t]),
    "casgd_export_rows": (_I, [_VP, _I64, _I64, _VP, ctypes.c_size_t]),
    "casgd_ld": (_I64, [_VP]),
    "casgd_fp8_exponent": (_I, [_VP]),
    "casgd_gram_bytes": (_I64, [_I, _I, _I]),
    "casgd_set_timing": (_I, [_VP, _I]),
    "casgd_get_timing": (_I, [_VP, _I, ctypes.POINTER(ctypes.c_double),
                              ctypes.POINTER(ctypes.c_int64), _I]),
    "casgd_last_error": (ctypes.c_char_p, []),
    "casgd_set_option": (_I, [_VP, _I, _I]),
    "casgd_loss_noalloc": (_I, [_VP, _VP, _VP]),
    "casgd_peak_copy": (_I, [_VP, _VP, _I64, _VP]),
    "casgd_peak_mfma": (_I, [_VP, _I, _I, _VP]),
    "casgd_peak_read": (_I, [_VP, _I64, _VP, _I, _VP]),
}

_lib = None


class CasgdError(RuntimeError):
    pass


def load(path: str = LIB_PATH):
    """Open libcasgd.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise CasgdError(f"{path} is missing: build it with "
                         "`python -m communication_avoiding_mixed_amd.build`")
    import torch  # noqa: F401  (loads the HIP runtime the library binds to)
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != OK:
        msg = load().casgd_last_error().decode(errors="replace")
        raise CasgdError(f"{what} failed ({rc}): {msg}")


def gram_bytes(s: int, b: int, packed: bool = True) -> int:
    return int(load().casgd_gram_bytes(s, b, 1 if packed else 0))


def step_seed(base_seed: int, k: int) -> int:
    return int(load().casgd_step_seed(base_seed, k))


def _stream_ptr():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev_f32(t, shape, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def peak_copy(src, dst):
    """Copy src into dst (same byte size) with the calibration copy kernel, on
    torch's current stream; returns the bytes read (= bytes written)."""
    import torch
    for t, name in ((src, "src"), (dst, "dst")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same byte size")
    _check(load().casgd_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                  nbytes, _stream_ptr()), "casgd_peak_copy")
    return nbytes


def peak_read(src, out, workgroups: int):
    """Stream src (a contiguous GPU tensor) with the read calibration kernel
    on torch's current stream; out: float32 GPU tensor of workgroups * 8.
    Returns the bytes read."""
    import torch
    if not isinstance(src, torch.Tensor) or not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    _dev_f32(out, (workgroups * 8,), "out")
    nbytes = src.numel() * src.element_size()
    _check(load().casgd_peak_read(ctypes.c_void_p(src.data_ptr()), nbytes, ctypes.c_void_p(out.data_ptr()),
                                  workgroups, _stream_ptr()), "casgd_peak_read")
    return nbytes


def peak_mfma(out, workgroups: int, iters: int):
    """Run the MFMA calibration loop on torch's current stream; out is a
    float32 GPU tensor of workgroups * 256 elements.  Returns its flops."""
    _dev_f32(out, (workgroups * 256,), "out")
    _check(load().casgd_peak_mfma(ctypes.c_void_p(out.data_ptr()), workgroups, iters, _stream_ptr()),
           "casgd_peak_mfma")
    return workgroups * 4 * 4 * iters * 2 * 32 * 32 * 16


class CASGD:
    """A handle over the stored data (X kept as bf16 or float32 on the GPU)."""

    def __init__(self, X, y, loss: str, storage: str = "bf16"):
        lib = load()
        if loss not in LOSS_IDS:
            raise ValueError(f"loss must be one of {sorted(LOSS_IDS)}")
        if storage not in STORAGE_IDS:
            raise ValueError(f"storage must be one of {sorted(STORAGE_IDS)}")
        if X.dim() != 2:
            raise ValueError("X must be 2-D")
        m, n = X.shape
        px = _dev_f32(X, (m, n), "X")
        py = _dev_f32(y, (m,), "y")
        self.m, self.n, self.loss, self.storage = int(m), int(n), loss, storage
        self._h = None
        # create on the null stream, after torch's pending work on its stream
        import torch
        torch.cuda.current_stream().synchronize()
        h = lib.casgd_create(px, py, self.m, self.n, LOSS_IDS[loss], STORAGE_IDS[storage])
        if not h:
            raise CasgdError("casgd_create failed: " + lib.casgd_last_error().decode(errors="replace"))
        self._h = ctypes.c_void_p(h)
        self.ld = int(lib.casgd_ld(self._h))
        self._last = None

    # -- lifetime
    def close(self):
        if self._h is not None:
            load().casgd_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _handle(self):
        if self._h is None:
            raise CasgdError("handle used after close()")
        _check(load().casgd_set_stream(self._h, _stream_ptr()), "casgd_set_stream")
        return self._h

    # -- the method
    def outer_step(self, s: int, b: int, eta: float, seed: int, w):
        h = self._handle()
        _check(load().casgd_outer_step(h, s, b, eta, seed, _dev_f32(w, (self.n,), "w")),
               "casgd_outer_step")
        self._last = (s, b)

    def outer_step_indices(self, s: int, b: int, eta: float, idx, w):
        import torch
        h = self._handle()
        if not (isinstance(idx, torch.Tensor) and idx.is_cuda and idx.dtype == torch.int32
                and idx.is_contiguous() and idx.numel() == s * b):
            raise ValueError("idx must be a contiguous int32 GPU tensor with s*b entries")
        _check(load().casgd_outer_step_indices(h, s, b, eta, ctypes.c_void_p(idx.data_ptr()),
                                               _dev_f32(w, (self.n,), "w")),
               "casgd_outer_step_indices")
        self._last = (s, b)

    def train(self, s: int, b: int, eta: float, base_seed: int, first_step: int, n_outer: int, w):
        h = self._handle()
        _check(load().casgd_train(h, s, b, eta, base_seed, first_step, n_outer,
                                  _dev_f32(w, (self.n,), "w")), "casgd_train")
        if n_outer > 0:
            self._last = (s, b)

    def loss_value(self, w) -> float:
        h = self._handle()
        out = ctypes.c_double(0.0)
        _check(load().casgd_loss(h, _dev_f32(w, (self.n,), "w"), ctypes.byref(out)), "casgd_loss")
        return float(out.value)

    # -- inspection
    @property
    def fp8_exponent(self) -> int:
        """k of fp8 storage (X stored as E4M3 of x * 2^k); 0 otherwise."""
        return int(load().casgd_fp8_exponent(self._handle()))

    def export(self, what: int) -> np.ndarray:
        if self._last is None:
            raise CasgdError("no outer step has run yet")
        s, b = self._last
        sb = s * b
        if what == EXPORT_IDX:
            arr = np.empty(sb, np.int32)
        elif what == EXPORT_Y:
            # gathered rows: bf16 bits for bf16 and fp8 storage, fp16 bits, or float32
            arr = np.empty((sb, self.ld), np.float32 if self.storage == "fp32" else np.uint16)
        elif what == EXPORT_G:
            arr = np.empty(b * b * s * (s - 1) // 2, np.float32)
        else:
            arr = np.empty(sb, np.float32)
        _check(load().casgd_debug_export(self._handle(), what, arr.ctypes.data_as(ctypes.c_void_p),
                                         arr.nbytes), "casgd_debug_export")
        return arr

    def export_rows(self, row0: int, nrows: int) -> np.ndarray:
        # stored rows: 16-bit patterns (bf16, fp16), E4M3 bytes (fp8) or float32
        arr = np.empty((nrows, self.ld), {"fp32": np.float32, "fp8": np.uint8}.get(self.storage, np.uint16))
        _check(load().casgd_export_rows(self._handle(), row0, nrows,
                                        arr.ctypes.data_as(ctypes.c_void_p), arr.nbytes),
               "casgd_export_rows")
        return arr

    def set_option(self, option: int, value: int):
        _check(load().casgd_set_option(self._handle(), option, value), "casgd_set_option")

    def set_timing(self, on, every: int = 1):
        """Stamp every `every`-th launch of each kernel (on), or stop (off)."""
        _check(load().casgd_set_timing(self._handle(), int(every) if on else 0), "casgd_set_timing")

    def timing(self, kernel: int, reset: bool = False):
        ms = ctypes.c_double(0.0)
        cnt = ctypes.c_int64(0)
        _check(load().casgd_get_timing(self._handle(), kernel, ctypes.byref(ms), ctypes.byref(cnt),
                                       1 if reset else 0), "casgd_get_timing")
        return float(ms.value), int(cnt.value)


def unpack_gram(G_packed: np.ndarray, s: int, b: int) -> dict:
    """Split the block-row packed strictly-lower Gram into {(j, t): b x b}."""
    out = {}
    for j in range(1, s):
        base = b * b * j * (j - 1) // 2
        rowblk = G_packed[base:base + b * j * b].reshape(b, j * b)
        for t in range(j):
            out[(j, t)] = rowblk[:, t * b:(t + 1) * b]
    return out
