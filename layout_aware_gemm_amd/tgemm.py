"""Thin ctypes binding over the tgemm C-ABI (``include/tgemm.h``).

Argument marshalling only: every step of the computation runs in the HIP
library.  There is no CPU or PyTorch fallback -- if the library is not built
the calls raise.

``run`` mirrors ``tgemm_run`` one to one.  The helpers derive layout flags
and leading dimensions from torch strides, so ``matmul(x, w.t())`` reads a
weight stored [N, K] in place (transB = 'T'), without a transposed copy.
"""

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libtgemm.so")
_lib = None

TGEMM_OK = 0
TGEMM_ERR_INVALID_ARG = -1
TGEMM_ERR_UNSUPPORTED = -2
TGEMM_ERR_HIP = -3
TGEMM_ERR_NO_MEMORY = -4
TGEMM_ERR_WORKSPACE_LIMIT = -5

EPI_STORE_BF16 = 0
EPI_STORE_F32 = 1
EPI_CE = 2
EPI_OUTER_F32 = 3
EPI_ROPE_COSSIN = 4

EXPORTS = ("tgemm_run", "tgemm_run_fp8", "tgemm_validate", "tgemm_validate_fp8",
           "tgemm_status_string", "tgemm_set_tile_config", "tgemm_set_split_k",
           "tgemm_set_fp8_cast_once", "tgemm_clock_probe", "tgemm_version",
           "tgemm_release_workspace", "tgemm_run_noalloc", "tgemm_noalloc_scratch_bytes",
           "tgemm_rope_region", "tgemm_validate_rope_region", "tgemm_run_ce_deferred",
           "tgemm_run_ce_grad", "tgemm_mfma_ceiling")


class TgemmError(RuntimeError):
    def __init__(self, status, what="tgemm_run"):
        self.status = status
        super().__init__(f"{what} failed: {status_string(status)} ({status})")


def library_path():
    return _LIB_PATH


def lib():
    """Load the shared library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"tgemm HIP library not found at {_LIB_PATH}; build it with "
                "`python -m layout_aware_gemm_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        L.tgemm_run.argtypes = [ctypes.c_char, ctypes.c_char, i64, i64, i64, vp, i64, vp, i64,
                                vp, i64, ctypes.c_int, vp, vp, vp, vp]
        L.tgemm_run.restype = ctypes.c_int
        L.tgemm_validate.argtypes = [ctypes.c_char, ctypes.c_char, i64, i64, i64, vp, i64, vp,
                                     i64, vp, i64, ctypes.c_int, vp, vp, vp]
        L.tgemm_validate.restype = ctypes.c_int
        L.tgemm_run_fp8.argtypes = [ctypes.c_char, ctypes.c_char, i64, i64, i64, vp, i64, vp,
                                    i64, vp, i64, ctypes.c_int, vp, vp]
        L.tgemm_run_fp8.restype = ctypes.c_int
        L.tgemm_validate_fp8.argtypes = [ctypes.c_char, ctypes.c_char, i64, i64, i64, vp, i64, vp,
                                         i64, vp, i64, ctypes.c_int, vp]
        L.tgemm_validate_fp8.restype = ctypes.c_int
        L.tgemm_status_string.argtypes = [ctypes.c_int]
        L.tgemm_status_string.restype = ctypes.c_char_p
        L.tgemm_set_tile_config.argtypes = [ctypes.c_int]
        L.tgemm_set_tile_config.restype = ctypes.c_int
        L.tgemm_set_split_k.argtypes = [ctypes.c_int]
        L.tgemm_set_split_k.restype = ctypes.c_int
        L.tgemm_set_fp8_cast_once.argtypes = [ctypes.c_int]
        L.tgemm_set_fp8_cast_once.restype = ctypes.c_int
        L.tgemm_clock_probe.argtypes = [i64, vp, vp]
        L.tgemm_clock_probe.restype = ctypes.c_int
        L.tgemm_mfma_ceiling.argtypes = [ctypes.c_int, i64, ctypes.c_int, vp, vp]
        L.tgemm_mfma_ceiling.restype = ctypes.c_int
        L.tgemm_version.argtypes = []
        L.tgemm_version.restype = ctypes.c_int
        L.tgemm_release_workspace.argtypes = [vp]
        L.tgemm_release_workspace.restype = ctypes.c_int
        L.tgemm_run_noalloc.argtypes = L.tgemm_run.argtypes
        L.tgemm_run_noalloc.restype = ctypes.c_int
        L.tgemm_noalloc_scratch_bytes.argtypes = []
        L.tgemm_noalloc_scratch_bytes.restype = ctypes.c_int64
        L.tgemm_run_ce_deferred.argtypes = [ctypes.c_char, ctypes.c_char, i64, i64, i64, vp, i64,
                                            vp, i64, vp, vp, vp, i64, vp, vp]
        L.tgemm_run_ce_deferred.restype = ctypes.c_int
        L.tgemm_run_ce_grad.argtypes = [ctypes.c_char, ctypes.c_char, i64, i64, i64, vp, i64, vp,
                                        vp, vp, i64, vp, i64, ctypes.c_int, vp]
        L.tgemm_run_ce_grad.restype = ctypes.c_int
        L.tgemm_rope_region.argtypes = [vp, i64, i64, i64, i64, vp, i64, vp, vp, vp, i64, vp, vp]
        L.tgemm_rope_region.restype = ctypes.c_int
        L.tgemm_validate_rope_region.argtypes = [vp, i64, i64, i64, i64, vp, i64, vp, vp, vp, i64,
                                                 vp]
        L.tgemm_validate_rope_region.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status):
    return lib().tgemm_status_string(int(status)).decode()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr() if x.numel() > 0 else None
    return int(x)


def _flag(t):
    t = t.encode() if isinstance(t, str) else bytes([t]) if isinstance(t, int) else t
    return ctypes.c_char(t[:1])


def _stream(stream, device=None):
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def run(transA, transB, M, N, K, A, lda, B, ldb, C, ldc, epilogue,
        labels=None, out_loss=None, out_grad=None, stream=None, check=True):
    """Call ``tgemm_run``.  Pointers may be tensors or integer addresses."""
    dev = A.device if isinstance(A, torch.Tensor) and A.is_cuda else None
    st = lib().tgemm_run(_flag(transA), _flag(transB), int(M), int(N), int(K), _ptr(A),
                         int(lda), _ptr(B), int(ldb), _ptr(C), int(ldc), int(epilogue),
                         _ptr(labels), _ptr(out_loss), _ptr(out_grad), _stream(stream, dev))
    if check and st != TGEMM_OK:
        raise TgemmError(st)
    return st


def run_noalloc(transA, transB, M, N, K, A, lda, B, ldb, C, ldc, epilogue,
                labels=None, out_loss=None, out_grad=None, stream=None, check=True):
    """Call ``tgemm_run_noalloc``: as ``run``, with every scratch buffer in
    the library's fixed per-device array (no device allocation)."""
    dev = A.device if isinstance(A, torch.Tensor) and A.is_cuda else None
    st = lib().tgemm_run_noalloc(_flag(transA), _flag(transB), int(M), int(N), int(K), _ptr(A),
                                 int(lda), _ptr(B), int(ldb), _ptr(C), int(ldc), int(epilogue),
                                 _ptr(labels), _ptr(out_loss), _ptr(out_grad),
                                 _stream(stream, dev))
    if check and st != TGEMM_OK:
        raise TgemmError(st, "tgemm_run_noalloc")
    return st


def noalloc_scratch_bytes():
    return int(lib().tgemm_noalloc_scratch_bytes())


def validate(transA, transB, M, N, K, A, lda, B, ldb, C, ldc, epilogue,
             labels=None, out_loss=None, out_grad=None):
    """Host-only ``tgemm_validate`` (no GPU needed)."""
    return lib().tgemm_validate(_flag(transA), _flag(transB), int(M), int(N), int(K), _ptr(A),
                                int(lda), _ptr(B), int(ldb), _ptr(C), int(ldc), int(epilogue),
                                _ptr(labels), _ptr(out_loss), _ptr(out_grad))


def run_fp8(transA, transB, M, N, K, A, lda, B, ldb, C, ldc, epilogue, scales, stream=None,
            check=True):
    """Call ``tgemm_run_fp8``: bf16 operands cast to e4m3fn as they are
    loaded; ``scales`` is a device fp32 [3] tensor {scale_a, scale_b,
    out_scale} (or its address)."""
    dev = A.device if isinstance(A, torch.Tensor) and A.is_cuda else None
    st = lib().tgemm_run_fp8(_flag(transA), _flag(transB), int(M), int(N), int(K), _ptr(A),
                             int(lda), _ptr(B), int(ldb), _ptr(C), int(ldc), int(epilogue),
                             _ptr(scales), _stream(stream, dev))
    if check and st != TGEMM_OK:
        raise TgemmError(st)
    return st


def validate_fp8(transA, transB, M, N, K, A, lda, B, ldb, C, ldc, epilogue, scales):
    """Host-only ``tgemm_validate_fp8`` (no GPU needed)."""
    return lib().tgemm_validate_fp8(_flag(transA), _flag(transB), int(M), int(N), int(K),
                                    _ptr(A), int(lda), _ptr(B), int(ldb), _ptr(C), int(ldc),
                                    int(epilogue), _ptr(scales))


def set_tile_config(cfg):
    """0 = automatic, 1 = 256x256, 2 = 128x128; returns the previous setting."""
    r = lib().tgemm_set_tile_config(int(cfg))
    if r < 0:
        raise TgemmError(r, "tgemm_set_tile_config")
    return r


def set_split_k(split):
    """0 = automatic; s > 0 forces s K chunks for 256x256-tile store GEMMs;
    returns the previous setting."""
    r = lib().tgemm_set_split_k(int(split))
    if r < 0:
        raise TgemmError(r, "tgemm_set_split_k")
    return r


def set_fp8_cast_once(enable):
    """1 (default): large fp8 products cast each operand once, in a pass of
    its own, before the GEMM; 0: always cast on load.  Returns the previous
    setting."""
    r = lib().tgemm_set_fp8_cast_once(int(enable))
    if r < 0:
        raise TgemmError(r, "tgemm_set_fp8_cast_once")
    return r


def release_workspace(stream=None, device=None):
    """Free (in stream order) the library's cached workspace of ``stream`` on
    the current device; the next call on that stream allocates afresh."""
    r = lib().tgemm_release_workspace(_stream(stream, device))
    if r != TGEMM_OK:
        raise TgemmError(r, "tgemm_release_workspace")


def clock_probe(ticks=2000, out=None, stream=None):
    """Enqueue the shader-clock probe (``tgemm_clock_probe``) and return the
    int64[3] device tensor it fills: shader cycles, constant-rate ticks and
    the constant rate in Hz.  ``clock_ghz`` reads the clock from it once the
    stream has reached it."""
    if out is None:
        out = torch.zeros(3, dtype=torch.int64, device="cuda")
    if out.dtype != torch.int64 or out.numel() < 3 or not out.is_cuda:
        raise ValueError("clock_probe: out must be a CUDA int64 tensor of 3 elements")
    r = lib().tgemm_clock_probe(int(ticks), _ptr(out), _stream(stream, out.device))
    if r != 0:
        raise TgemmError(r, "tgemm_clock_probe")
    return out


def mfma_ceiling(iters, out, kind=0, blocks=256, stream=None):
    """Enqueue the matrix-core ceiling kernel (``tgemm_mfma_ceiling``): MFMAs
    on register operands, kind 0 = 32x32x16 bf16 (524288 flop per wave and
    iteration), 1 = 32x32x64 fp8 e4m3fn (2097152); ``blocks * 4 * iters``
    wave-iterations; ``out`` a CUDA float32 tensor of at least ``blocks * 4``
    elements."""
    if out.dtype != torch.float32 or out.numel() < blocks * 4 or not out.is_cuda:
        raise ValueError("mfma_ceiling: out must be a CUDA float32 tensor of blocks * 4 elements")
    r = lib().tgemm_mfma_ceiling(int(kind), int(iters), int(blocks), _ptr(out),
                                 _stream(stream, out.device))
    if r != 0:
        raise TgemmError(r, "tgemm_mfma_ceiling")
    return out


def clock_ghz(probe_out):
    """Shader clock in GHz from a filled ``clock_probe`` tensor (synchronises)."""
    cyc, ticks, rate = (int(v) for v in probe_out.cpu().tolist()[:3])
    return cyc * rate / ticks / 1e9 if ticks > 0 else float("nan")


def layout_of(x):
    """(flag, ld) for a 2-D tensor viewed as the logical operand [R, C].

    Row-major storage (stride (ld, 1)) is 'N'; column-major storage
    (stride (1, ld)), e.g. ``w.t()`` of a row-major ``w``, is 'T'.
    """
    if x.dim() != 2:
        raise ValueError("operand must be 2-D")
    R, C = x.shape
    s0, s1 = x.stride()
    if s1 == 1 and (R == 1 or s0 >= C):
        return "N", (C if R == 1 else s0)
    if s0 == 1 and (C == 1 or s1 >= R):
        return "T", (R if C == 1 else s1)
    raise ValueError(f"operand with strides {x.stride()} is neither row- nor column-major")


def _check_dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tgemm operates on GPU tensors")


def _flatten_rows(a):
    """[..., K] -> [rows, K] as a view (the leading dims are flattened)."""
    if a.dim() == 2:
        return a
    if a.stride(-1) != 1:
        raise ValueError("batched operand needs a contiguous last dimension")
    return a.view(-1, a.shape[-1])


def matmul(a, b, out=None, out_dtype=torch.bfloat16, stream=None):
    """Y = a @ b for bf16 a [..., K] and b [K, N] (any row/column-major view).

    Leading dims of ``a`` are flattened as a view, and the result has shape
    [..., N].  ``out_dtype`` is torch.bfloat16 or torch.float32.
    """
    lead = a.shape[:-1]
    a2 = _flatten_rows(a)
    if a2.dtype != torch.bfloat16 or b.dtype != torch.bfloat16:
        raise TypeError("matmul expects bf16 operands")
    M, K = a2.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    _check_dev(a2, b)
    ta, lda = layout_of(a2)
    tb, ldb = layout_of(b)
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=a.device)
    if out.dim() != 2 or out.stride(1) != 1 or out.shape != (M, N):
        raise ValueError("out must be a row-major [M, N] tensor")
    epi = EPI_STORE_BF16 if out.dtype == torch.bfloat16 else EPI_STORE_F32
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bf16 or fp32")
    run(ta, tb, M, N, K, a2, lda, b, ldb, out, out.stride(0), epi, stream=stream)
    return out.view(*lead, N)


def matmul_fp8(a, b, scales, out=None, out_dtype=torch.bfloat16, stream=None):
    """out_scale * (e4m3(a * scale_a) @ e4m3(b * scale_b)) for bf16 a [..., K]
    and b [K, N] in any row/column-major view; ``scales`` is a device fp32
    tensor {scale_a, scale_b, out_scale}.  No fp8 copy of either operand is
    made, in either layout."""
    lead = a.shape[:-1]
    a2 = _flatten_rows(a)
    if a2.dtype != torch.bfloat16 or b.dtype != torch.bfloat16:
        raise TypeError("matmul_fp8 expects bf16 operands")
    if scales.dtype != torch.float32 or scales.numel() != 3 or not scales.is_contiguous():
        raise ValueError("scales must be a contiguous fp32 tensor of 3 values")
    M, K = a2.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    _check_dev(a2, b, scales)
    ta, lda = layout_of(a2)
    tb, ldb = layout_of(b)
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=a.device)
    if out.dim() != 2 or out.stride(1) != 1 or out.shape != (M, N):
        raise ValueError("out must be a row-major [M, N] tensor")
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bf16 or fp32")
    epi = EPI_STORE_BF16 if out.dtype == torch.bfloat16 else EPI_STORE_F32
    run_fp8(ta, tb, M, N, K, a2, lda, b, ldb, out, out.stride(0), epi, scales, stream=stream)
    return out.view(*lead, N)


def cross_entropy(h, w, labels, grad=False, stream=None):
    """Per-row loss of logits h @ w (fp32, never stored) against int32 labels.

    ``w`` is the logical [K, N] operand, usually ``W.t()`` of a weight stored
    [N, K].  Returns ``loss`` (fp32 [M]) or ``(loss, g)`` with g the bf16
    [M, N] softmax minus one-hot.
    """
    if h.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise TypeError("cross_entropy expects bf16 operands")
    M, K = h.shape
    K2, N = w.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    if labels.dtype != torch.int32 or labels.shape != (M,) or not labels.is_contiguous():
        raise ValueError("labels must be a contiguous int32 [M] tensor")
    _check_dev(h, w, labels)
    ta, lda = layout_of(h)
    tb, ldb = layout_of(w)
    loss = torch.empty(M, dtype=torch.float32, device=h.device)
    g = torch.empty(M, N, dtype=torch.bfloat16, device=h.device) if grad else None
    run(ta, tb, M, N, K, h, lda, w, ldb, None, N, EPI_CE, labels=labels, out_loss=loss,
        out_grad=g, stream=stream)
    return (loss, g) if grad else loss


def rope_cos_sin(pos, inv_freq, stream=None):
    """cos/sin tables bf16 [P, 2F] of fp32(pos)[:, None] * inv_freq[None, :].

    ``pos`` int64 [P], ``inv_freq`` fp32 [F]; the K=1 product is duplicated
    along the last dimension.
    """
    if pos.dtype != torch.int64 or inv_freq.dtype != torch.float32:
        raise TypeError("pos must be int64 and inv_freq fp32")
    if pos.dim() != 1 or inv_freq.dim() != 1:
        raise ValueError("pos and inv_freq must be 1-D")
    _check_dev(pos, inv_freq)
    P, F = pos.shape[0], inv_freq.shape[0]
    cos = torch.empty(P, 2 * F, dtype=torch.bfloat16, device=pos.device)
    sin = torch.empty(P, 2 * F, dtype=torch.bfloat16, device=pos.device)
    # A = positions as a [P, 1] column ('N', lda = element stride); B = the
    # frequencies as a [1, F] row ('N') or, when strided, an [F, 1] column ('T').
    if inv_freq.stride(0) == 1:
        tb, ldb = "N", F
    else:
        tb, ldb = "T", inv_freq.stride(0)
    run("N", tb, P, F, 1, pos, pos.stride(0), inv_freq, ldb, cos, 2 * F, EPI_ROPE_COSSIN,
        out_grad=sin, stream=stream)
    return cos, sin


def run_ce_deferred(transA, transB, M, N, K, A, lda, B, ldb, labels, out_loss, out_e, lde,
                    out_scale, stream=None, check=True):
    """Call ``tgemm_run_ce_deferred``."""
    dev = A.device if isinstance(A, torch.Tensor) and A.is_cuda else None
    st = lib().tgemm_run_ce_deferred(_flag(transA), _flag(transB), int(M), int(N), int(K),
                                     _ptr(A), int(lda), _ptr(B), int(ldb), _ptr(labels),
                                     _ptr(out_loss), _ptr(out_e), int(lde), _ptr(out_scale),
                                     _stream(stream, dev))
    if check and st != TGEMM_OK:
        raise TgemmError(st, "tgemm_run_ce_deferred")
    return st


def run_ce_grad(transA, transB, M, N, K, E, lde, scale, labels, B, ldb, C, ldc, epilogue,
                stream=None, check=True):
    """Call ``tgemm_run_ce_grad``."""
    dev = E.device if isinstance(E, torch.Tensor) and E.is_cuda else None
    st = lib().tgemm_run_ce_grad(_flag(transA), _flag(transB), int(M), int(N), int(K), _ptr(E),
                                 int(lde), _ptr(scale), _ptr(labels), _ptr(B), int(ldb), _ptr(C),
                                 int(ldc), int(epilogue), _stream(stream, dev))
    if check and st != TGEMM_OK:
        raise TgemmError(st, "tgemm_run_ce_grad")
    return st


def cross_entropy_deferred(h, w, labels, stream=None):
    """As ``cross_entropy(h, w, labels, grad=True)`` but with the gradient
    left unscaled: returns (loss fp32 [M], e bf16 [M, N], scale fp32
    [ceil(N/64), M]); ``ce_grad_matmul`` finishes the gradient on load."""
    if h.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise TypeError("cross_entropy_deferred expects bf16 operands")
    M, K = h.shape
    K2, N = w.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    if labels.dtype != torch.int32 or labels.shape != (M,) or not labels.is_contiguous():
        raise ValueError("labels must be a contiguous int32 [M] tensor")
    _check_dev(h, w, labels)
    ta, lda = layout_of(h)
    tb, ldb = layout_of(w)
    loss = torch.empty(M, dtype=torch.float32, device=h.device)
    e = torch.empty(M, N, dtype=torch.bfloat16, device=h.device)
    scale = torch.empty((N + 63) // 64, M, dtype=torch.float32, device=h.device)
    run_ce_deferred(ta, tb, M, N, K, h, lda, w, ldb, labels, loss, e, N, scale, stream=stream)
    return loss, e, scale


def ce_grad_matmul(g, scale, labels, b, out_dtype=torch.bfloat16, stream=None):
    """op(G) @ b where G is the gradient of ``cross_entropy_deferred``,
    finished as it is loaded.  ``g`` is its e tensor [T, V] for G, or
    ``e.t()`` for G^T; ``b`` any row/column-major view."""
    if g.dtype != torch.bfloat16 or b.dtype != torch.bfloat16:
        raise TypeError("ce_grad_matmul expects bf16 operands")
    _check_dev(g, b, scale, labels)
    M, K = g.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    ta, lda = layout_of(g)
    tb, ldb = layout_of(b)
    out = torch.empty(M, N, dtype=out_dtype, device=g.device)
    epi = EPI_STORE_BF16 if out_dtype == torch.bfloat16 else EPI_STORE_F32
    run_ce_grad(ta, tb, M, N, K, g, lda, scale, labels, b, ldb, out, N, epi, stream=stream)
    return out


def run_rope_region(q, ldq, P, H, D, pos, spos, inv_freq, cos, sin, ldc, q_out, stream=None,
                    check=True):
    """Call ``tgemm_rope_region`` (pointers may be tensors or addresses)."""
    dev = q.device if isinstance(q, torch.Tensor) and q.is_cuda else None
    st = lib().tgemm_rope_region(_ptr(q), int(ldq), int(P), int(H), int(D), _ptr(pos), int(spos),
                                 _ptr(inv_freq), _ptr(cos), _ptr(sin), int(ldc), _ptr(q_out),
                                 _stream(stream, dev))
    if check and st != TGEMM_OK:
        raise TgemmError(st, "tgemm_rope_region")
    return st


def validate_rope_region(q, ldq, P, H, D, pos, spos, inv_freq, cos, sin, ldc, q_out):
    """Host-only ``tgemm_validate_rope_region``."""
    return lib().tgemm_validate_rope_region(_ptr(q), int(ldq), int(P), int(H), int(D), _ptr(pos),
                                            int(spos), _ptr(inv_freq), _ptr(cos), _ptr(sin),
                                            int(ldc), _ptr(q_out))


def rope_region(q, pos, inv_freq, heads, stream=None):
    """The RoPE region in one launch: q bf16 [P, heads*D] (row-major, any
    row stride), pos int64 [P], inv_freq fp32 [D/2].  Returns (q_heads fp32
    [heads, P, D], cos bf16 [P, D], sin bf16 [P, D])."""
    if q.dtype != torch.bfloat16 or pos.dtype != torch.int64 or inv_freq.dtype != torch.float32:
        raise TypeError("q must be bf16, pos int64, inv_freq fp32")
    if q.dim() != 2 or q.stride(1) != 1 or pos.dim() != 1 or inv_freq.dim() != 1:
        raise ValueError("q must be a row-major [P, H*D] matrix, pos and inv_freq 1-D")
    if not inv_freq.is_contiguous():
        raise ValueError("inv_freq must be contiguous")
    _check_dev(q, pos, inv_freq)
    P, HD = q.shape
    D = 2 * inv_freq.shape[0]
    if pos.shape[0] != P or HD != heads * D:
        raise ValueError("shapes of q, pos, inv_freq and heads do not agree")
    q_out = torch.empty(heads, P, D, dtype=torch.float32, device=q.device)
    cos = torch.empty(P, D, dtype=torch.bfloat16, device=q.device)
    sin = torch.empty(P, D, dtype=torch.bfloat16, device=q.device)
    run_rope_region(q, q.stride(0), P, heads, D, pos, pos.stride(0), inv_freq, cos, sin, D, q_out,
                    stream=stream)
    return q_out, cos, sin


def outer_f32(a, b, stream=None):
    """C[m, n] = a[m] * b[n] for fp32 vectors (the K=1 matmul, exact)."""
    if a.dtype != torch.float32 or b.dtype != torch.float32 or a.dim() != 1 or b.dim() != 1:
        raise TypeError("outer_f32 expects 1-D fp32 tensors")
    _check_dev(a, b)
    M, N = a.shape[0], b.shape[0]
    c = torch.empty(M, N, dtype=torch.float32, device=a.device)
    if b.stride(0) == 1:
        run("N", "N", M, N, 1, a, a.stride(0), b, N, c, N, EPI_OUTER_F32, stream=stream)
    else:
        run("N", "T", M, N, 1, a, a.stride(0), b, b.stride(0), c, N, EPI_OUTER_F32,
            stream=stream)
    return c
