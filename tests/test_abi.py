"""CPU checks of the C-ABI boundary: the library loads, exports every symbol
``include/tgemm.h`` declares, and rejects invalid arguments before touching
the GPU (no compute call is made here).  Also the binding's stride -> layout
logic, which is host-only.
"""

import os
import re

import pytest
import torch

from layout_aware_gemm_amd import tgemm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tgemm.h")

OK, INV, UNS = tgemm.TGEMM_OK, tgemm.TGEMM_ERR_INVALID_ARG, tgemm.TGEMM_ERR_UNSUPPORTED
P = 0x1000  # a fake non-NULL address: validation never dereferences pointers


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"TGEMM_API\s+[\w\s\*]+?\b(tgemm_\w+)\s*\(", text)))


def test_header_declares_the_api():
    assert declared_functions() == sorted(tgemm.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = tgemm.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.tgemm_version() >= 100


def test_status_strings():
    assert tgemm.status_string(0) == "TGEMM_OK"
    assert tgemm.status_string(INV) == "TGEMM_ERR_INVALID_ARG"
    assert tgemm.status_string(UNS) == "TGEMM_ERR_UNSUPPORTED"
    assert tgemm.status_string(tgemm.TGEMM_ERR_HIP) == "TGEMM_ERR_HIP"
    assert tgemm.status_string(tgemm.TGEMM_ERR_NO_MEMORY) == "TGEMM_ERR_NO_MEMORY"
    assert tgemm.status_string(tgemm.TGEMM_ERR_WORKSPACE_LIMIT) == "TGEMM_ERR_WORKSPACE_LIMIT"
    assert tgemm.status_string(-99) == "TGEMM_ERR_UNKNOWN"


def v(ta="N", tb="T", M=768, N=5120, K=13824, A=P, lda=None, B=P, ldb=None, C=P, ldc=None,
      epi=0, labels=None, loss=None, grad=None):
    lda = (K if ta == "N" else M) if lda is None else lda
    ldb = (N if tb == "N" else K) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return tgemm.validate(ta, tb, M, N, K, A, lda, B, ldb, C, ldc, epi, labels, loss, grad)


def test_validate_accepts_the_workloads():
    assert v() == OK                                           # NT down-projection
    for ta in "NTnt":
        for tb in "NTnt":
            assert v(ta.upper(), tb.upper(), 4096, 4096, 4096) == OK
            assert v(ta, tb, 7, 3, 5) == OK
    assert v(M=4096, N=32000, K=4096, C=None, epi=2, labels=P, loss=P) == OK
    assert v(M=4096, N=32000, K=4096, C=None, epi=2, labels=P, loss=P, grad=P) == OK
    assert v("N", "N", 4096, 64, 1, lda=1, ldb=64, ldc=128, epi=4, grad=P) == OK
    assert v("N", "N", 10, 20, 1, lda=1, ldb=20, epi=3) == OK


@pytest.mark.parametrize("kw,expect", [
    (dict(ta="X"), INV), (dict(tb="q"), INV),
    (dict(M=0), INV), (dict(N=-1), INV), (dict(K=0), INV),
    (dict(M=1 << 31), UNS),
    (dict(lda=13823), INV), (dict(ldb=100), INV), (dict(ldc=5119), INV),
    (dict(ta="T", lda=767), INV), (dict(tb="N", ldb=5119), INV),
    (dict(A=None), INV), (dict(B=None), INV), (dict(C=None), INV),
    (dict(epi=5), INV), (dict(epi=-1), INV),
    (dict(epi=2, C=None, labels=None, loss=P), INV),
    (dict(epi=2, C=None, labels=P, loss=None), INV),
    (dict(epi=2, C=None, labels=P, loss=P, grad=P, ldc=10), INV),
    (dict(epi=3), UNS), (dict(epi=4, grad=P), UNS),
    (dict(ta="N", tb="N", K=1, lda=1, ldb=5120, epi=4, ldc=10240, grad=None), INV),
    (dict(ta="N", tb="N", K=1, lda=1, ldb=5120, epi=4, ldc=10239, grad=P), INV),
])
def test_validate_rejects(kw, expect):
    assert v(**kw) == expect


def test_run_rejects_before_touching_the_gpu():
    # invalid calls return the status without any HIP call (stream 0)
    st = tgemm.run("N", "T", 0, 5, 5, P, 5, P, 5, P, 5, 0, stream=0, check=False)
    assert st == INV
    with pytest.raises(tgemm.TgemmError):
        tgemm.run("Z", "T", 5, 5, 5, P, 5, P, 5, P, 5, 0, stream=0)


def test_set_tile_config_roundtrip():
    prev = tgemm.set_tile_config(2)
    assert tgemm.set_tile_config(prev) == 2
    prev = tgemm.set_tile_config(3)    # 192x256 (NT store products)
    assert tgemm.set_tile_config(prev) == 3
    for bad in (4, -1):
        with pytest.raises(tgemm.TgemmError):
            tgemm.set_tile_config(bad)


def test_set_split_k_roundtrip():
    prev = tgemm.set_split_k(4)
    assert tgemm.set_split_k(prev) == 4
    with pytest.raises(tgemm.TgemmError):
        tgemm.set_split_k(-1)


def test_layout_of_strides():
    w = torch.empty(5120, 13824, dtype=torch.bfloat16)
    assert tgemm.layout_of(w.t()) == ("T", 13824)               # weight read in place
    x = torch.empty(384, 2, 13824, dtype=torch.bfloat16).view(-1, 13824)
    assert tgemm.layout_of(x) == ("N", 13824)
    big = torch.empty(100, 300, dtype=torch.bfloat16)
    assert tgemm.layout_of(big[:, :200]) == ("N", 300)         # padded rows
    assert tgemm.layout_of(big[:, :200].t()) == ("T", 300)
    assert tgemm.layout_of(torch.empty(1, 7)) == ("N", 7)
    assert tgemm.layout_of(torch.empty(7, 1)) == ("N", 1)
    with pytest.raises(ValueError):
        tgemm.layout_of(big[:, ::2])


def test_binding_refuses_cpu_tensors():
    a = torch.zeros(4, 4, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tgemm.matmul(a, a)


def test_validate_fp8_rules():
    """fp8 calls: store epilogues only, scales required, else the bf16 rules."""
    ok = dict(transA="N", transB="T", M=64, N=32, K=48, A=16, lda=48, B=16, ldb=48, C=16, ldc=32,
              epilogue=tgemm.EPI_STORE_BF16, scales=16)
    assert tgemm.validate_fp8(**ok) == tgemm.TGEMM_OK
    assert tgemm.validate_fp8(**{**ok, "epilogue": tgemm.EPI_STORE_F32}) == tgemm.TGEMM_OK
    for bad in ({"epilogue": tgemm.EPI_CE}, {"epilogue": 4}, {"scales": None},
                {"lda": 47}, {"C": None}, {"K": 0}, {"transA": "X"}):
        assert tgemm.validate_fp8(**{**ok, **bad}) == tgemm.TGEMM_ERR_INVALID_ARG, bad


def test_run_fp8_rejects_before_touching_the_gpu():
    st = tgemm.run_fp8("N", "T", 64, 32, 48, 16, 48, 16, 48, 16, 32, tgemm.EPI_CE, 16, stream=0,
                       check=False)
    assert st == tgemm.TGEMM_ERR_INVALID_ARG


def test_clock_probe_rejects_before_touching_the_gpu():
    # ticks out of range, NULL or misaligned output: the status, no HIP call
    L = tgemm.lib()
    assert L.tgemm_clock_probe(2000, None, None) == tgemm.TGEMM_ERR_INVALID_ARG
    assert L.tgemm_clock_probe(0, 16, None) == tgemm.TGEMM_ERR_INVALID_ARG
    assert L.tgemm_clock_probe(10 ** 7 + 1, 16, None) == tgemm.TGEMM_ERR_INVALID_ARG
    assert L.tgemm_clock_probe(2000, 20, None) == tgemm.TGEMM_ERR_INVALID_ARG


def test_mfma_ceiling_rejects_before_touching_the_gpu():
    # kind, iteration count, block count, NULL or misaligned output
    L = tgemm.lib()
    assert L.tgemm_mfma_ceiling(2, 16, 256, 16, None) == tgemm.TGEMM_ERR_INVALID_ARG
    assert L.tgemm_mfma_ceiling(0, 0, 256, 16, None) == tgemm.TGEMM_ERR_INVALID_ARG
    assert L.tgemm_mfma_ceiling(1, 10 ** 8 + 1, 256, 16, None) == tgemm.TGEMM_ERR_INVALID_ARG
    assert L.tgemm_mfma_ceiling(0, 16, 0, 16, None) == tgemm.TGEMM_ERR_INVALID_ARG
    assert L.tgemm_mfma_ceiling(1, 16, 65537, 16, None) == tgemm.TGEMM_ERR_INVALID_ARG
    assert L.tgemm_mfma_ceiling(0, 16, 256, None, None) == tgemm.TGEMM_ERR_INVALID_ARG
    assert L.tgemm_mfma_ceiling(1, 16, 256, 18, None) == tgemm.TGEMM_ERR_INVALID_ARG


def test_set_fp8_cast_once_roundtrip():
    prev = tgemm.set_fp8_cast_once(0)
    assert prev == 1
    assert tgemm.set_fp8_cast_once(prev) == 0
    with pytest.raises(tgemm.TgemmError):
        tgemm.set_fp8_cast_once(2)


def test_rope_region_validation():
    P_ = 64  # any non-null address: validation never dereferences
    v = tgemm.validate_rope_region
    assert v(P_, 4096, 4096, 32, 128, P_, 1, P_, P_, P_, 128, P_) == OK
    assert v(P_, 4095, 4096, 32, 128, P_, 1, P_, P_, P_, 128, P_) == INV   # ldq < H*D
    assert v(P_, 4096, 4096, 32, 127, P_, 1, P_, P_, P_, 128, P_) == INV   # odd D
    assert v(P_, 4096, 0, 32, 128, P_, 1, P_, P_, P_, 128, P_) == INV      # no positions
    assert v(P_, 4096, 4096, 32, 128, P_, 1, P_, P_, P_, 127, P_) == INV   # ldc < D
    assert v(P_, 4096, 4096, 32, 128, P_, 0, P_, P_, P_, 128, P_) == INV   # position stride
    assert v(None, 4096, 4096, 32, 128, P_, 1, P_, P_, P_, 128, P_) == INV
    assert v(P_, 4096, 4096, 32, 128, P_, 1, P_, P_, P_, 128, None) == INV
    with pytest.raises(tgemm.TgemmError):
        tgemm.run_rope_region(P_, 4096, 4096, 32, 127, P_, 1, P_, P_, P_, 128, P_, stream=0)
