"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, and validates arguments before touching the GPU (these calls
return before any HIP runtime call, so they run without a GPU)."""

import ctypes
import os
import re

import pytest

import nested_int_matmul_amd as mq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mq.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mq_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mq.LIB_PATH):
        pytest.skip("libmq.so not built")
    return mq.lib()


def _exported_text_symbols(path):
    """Functions a shared library exports (nm -D), or None without nm."""
    import shutil
    import subprocess

    if not shutil.which("nm"):
        return None
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    return sorted(ln.split()[-1] for ln in out.splitlines() if " T " in ln)


def test_exports_every_declared_symbol(L):
    declared = _declared_functions()
    assert declared, "no declarations parsed"
    assert set(declared) == set(mq.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    # and nothing else: the library is built with hidden visibility
    exported = _exported_text_symbols(mq.LIB_PATH)
    if exported is not None:
        assert exported == declared


def test_peaks_library_exports_every_declared_symbol():
    """libmq_peaks.so (the measured-peak probes bench.py times) loads and
    exports what include/mq_peaks.h declares; its argument checks refuse bad
    input before any launch."""
    from nested_int_matmul_amd import build as b

    if not os.path.exists(b.PEAKS_LIB):
        pytest.skip("libmq_peaks.so not built")
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "mq_peaks.h")).read(),
                 flags=re.S)
    declared = sorted(set(re.findall(r"\b(mqp_[a-z_0-9]+)\s*\(", src)))
    assert declared == ["mqp_empty", "mqp_mfma_loop", "mqp_mfma_loop_flops", "mqp_stream_read"]
    exported = _exported_text_symbols(b.PEAKS_LIB)
    if exported is not None:
        assert exported == declared
    P = ctypes.CDLL(b.PEAKS_LIB)
    for name in declared:
        assert hasattr(P, name), name
    P.mqp_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_void_p]
    assert P.mqp_stream_read(None, 1024, 8, P16, None) == 1
    assert P.mqp_stream_read(P16, 1000, 8, P16, None) == 1      # not a multiple of 16
    assert P.mqp_stream_read(P1, 1024, 8, P16, None) == 1       # misaligned
    P.mqp_mfma_loop_flops.restype = ctypes.c_double
    assert P.mqp_mfma_loop_flops(2, 3) == 2 * 4 * 3 * 4 * 2 * 32 * 32 * 16


def test_status_strings_and_sizes(L):
    for code, name in mq.STATUS_NAMES.items():
        assert L.mq_status_string(code).decode().startswith(name)
    assert L.mq_status_string(99).decode() == "unknown mq_status"
    assert L.mq_version().decode().startswith("mq ")
    assert L.mq_packed_bytes(14336, 3584, 2) == 14336 * 3584 // 4
    assert L.mq_packed_bytes(10, 64, 3) == 10 * 64 * 3 // 8
    assert L.mq_packed_bytes(10, 64, 5) == 0
    assert L.mq_gemm_workspace_bytes(2048, 14336, 4096, 128) == 0


def test_split_k_plans(L):
    """K splits and their workspace (one fp32 [M, N] partial per slice) for
    M >= 65: tiles of 128 (M <= 128) or 256 rows by 256 columns, K in
    iterations of 64, split in powers of two while the tiles stay under 256
    workgroups and every slice keeps 8 iterations; slices hold whole groups
    (an even count of iterations)."""
    ws = L.mq_gemm_workspace_bytes
    # 4096 x 14336, M = 96: 16 tiles, 224 iterations -> 16 slices of 14
    assert ws(96, 4096, 14336, 14336) == 16 * 96 * 4096 * 4
    assert ws(96, 4096, 14336, 128) == 16 * 96 * 4096 * 4
    # 66 iterations over 2 tiles: 8-way split of 9, rounded to 10 -> 7 slices
    assert ws(100, 300, 4224, 4224) == 7 * 100 * 300 * 4
    assert ws(130, 300, 4224, 4224) == 7 * 130 * 300 * 4
    assert ws(256, 300, 4224, 4224) == 7 * 256 * 300 * 4
    # 14336 x 4096 at M = 200: prefill 56 tiles, 64 iterations -> 4 slices of 16
    assert ws(200, 14336, 4096, 4096) == 4 * 200 * 14336 * 4
    assert ws(200, 14336, 4096, 128) == 4 * 200 * 14336 * 4
    # 10 iterations of 64: no slice of 8 fits twice
    assert ws(130, 200, 640, 640) == 0
    assert ws(100, 200, 640, 640) == 0
    # prefill at M = 2048: 448 tiles fill the chip; the 4096-wide down
    # projection has 128 tiles -> 2 slices of 112 iterations
    assert ws(2048, 14336, 4096, 128) == 0
    assert ws(2048, 4096, 14336, 128) == 2 * 2048 * 4096 * 4
    assert ws(8, 4096, 14336, 128) == 0


NULL = None
P16 = ctypes.c_void_p(0x10000)  # a 16-byte-aligned dummy address: never dereferenced
P1 = ctypes.c_void_p(0x10001)


def test_pack_validation(L):
    assert L.mq_pack(NULL, 4, 64, 4, P16, NULL) == 1
    assert L.mq_pack(P16, 4, 64, 5, P16, NULL) == 3
    assert L.mq_pack(P16, 4, 65, 4, P16, NULL) == 2
    assert L.mq_pack(P16, 0, 64, 4, P16, NULL) == 2
    assert L.mq_pack(P1, 4, 64, 4, P16, NULL) == 5


def test_gemv_validation(L):
    args = lambda **kw: dict(dict(p=P16, r=4, a=P16, z=P16, g=64, N=4, K=64, x=P16, M=1, y=P16), **kw)

    def call(**kw):
        a = args(**kw)
        return L.mq_gemv(a["p"], a["r"], a["a"], a["z"], a["g"], a["N"], a["K"], a["x"], a["M"],
                         a["y"], NULL)

    assert call(p=NULL) == 1
    assert call(y=NULL) == 1
    assert call(r=5) == 3
    assert call(K=96, g=96) == 2
    assert call(g=32) == 4
    assert call(K=192, g=128) == 4
    assert call(M=0) == 2
    assert call(M=9) == 2
    assert call(x=P1) == 5


def test_gemm_and_grouped_validation(L):
    assert L.mq_gemm(P16, 5, P16, P16, 64, 4, 64, P16, 16, P16, NULL, 0, NULL) == 3
    assert L.mq_gemm(P16, 4, P16, P16, 64, 4, 64, P16, 0, P16, NULL, 0, NULL) == 2
    probs = (mq.GemvProblem * 2)()
    assert L.mq_gemv_grouped(probs, 2, 4, 1, NULL) == 1
    assert L.mq_gemv_grouped(probs, 0, 4, 1, NULL) == 2
    assert L.mq_gemv_grouped(probs, 17, 4, 1, NULL) == 2
    rs = (ctypes.c_int * 2)(4, 2)
    assert L.mq_gemv_mixed(probs, rs, 2, 1, NULL) == 1
    assert L.mq_gemv_mixed(probs, None, 2, 1, NULL) == 1
    assert L.mq_gemv_mixed(probs, rs, 0, 1, NULL) == 2
    assert L.mq_gemv_mixed(probs, rs, 17, 1, NULL) == 2


def _layer(H=64, Hkv=64, F=128, r=4, **override):
    """A Layer of dummy aligned pointers; override={"q": Linear(...)} etc."""
    lin = lambda n, k: mq.Linear(0x10000, 0x10000, 0x10000, n, k, k)
    shapes = {"q": (H, H), "k": (Hkv, H), "v": (Hkv, H), "o": (H, H), "up": (F, H),
              "gate": (F, H), "down": (H, F)}
    kw = {n: override.get(n, lin(*shapes[n])) for n in mq.LAYER_LINEARS}
    arr = (mq.Layer * 1)()
    arr[0] = mq.Layer(r=r, **kw)
    return arr


def test_mixnmatch_validation(L):
    empty = (mq.Layer * 1)()
    ws = 1 << 20
    # the bf16-input form (x -> h_out) and the in-place form
    assert L.mq_mixnmatch_forward(empty, 1, P16, 1, P16, P16, ws, NULL) == 1
    assert L.mq_mixnmatch_forward_inplace(empty, 1, P16, 1, P16, ws, NULL) == 1
    assert L.mq_mixnmatch_workspace_bytes(empty, 1, 1) == 0
    assert L.mq_mixnmatch_forward(empty, 0, P16, 1, P16, P16, ws, NULL) == 2
    ok = _layer()
    assert L.mq_mixnmatch_workspace_bytes(ok, 1, 1) > 0
    assert L.mq_mixnmatch_forward(ok, 1, NULL, 1, P16, P16, ws, NULL) == 1     # no x
    assert L.mq_mixnmatch_forward(ok, 1, P16, 1, NULL, P16, ws, NULL) == 1     # no h_out
    assert L.mq_mixnmatch_forward(ok, 1, P1, 1, P16, P16, ws, NULL) == 5       # x misaligned
    assert L.mq_mixnmatch_forward(ok, 1, P16, 1, P1, P16, ws, NULL) == 5       # h_out misaligned
    assert L.mq_mixnmatch_forward(ok, 1, P16, 9, P16, P16, ws, NULL) == 2      # M > 8
    assert L.mq_mixnmatch_forward(ok, 1, P16, 1, P16, NULL, ws, NULL) == 6     # no workspace
    assert L.mq_mixnmatch_forward(ok, 1, P16, 1, P16, P16, 16, NULL) == 6      # too small
    assert L.mq_mixnmatch_forward(_layer(r=5), 1, P16, 1, P16, P16, ws, NULL) == 3
    # a linear's scales must be 4-byte aligned, as for every product
    bad = mq.Linear(0x10000, 0x10002, 0x10000, 64, 64, 64)
    assert L.mq_mixnmatch_forward(_layer(q=bad), 1, P16, 1, P16, P16, ws, NULL) == 5
    bad = mq.Linear(0x10008, 0x10000, 0x10000, 64, 64, 64)                    # packed not 16-aligned
    assert L.mq_mixnmatch_forward(_layer(o=bad), 1, P16, 1, P16, P16, ws, NULL) == 5
    bad = mq.Linear(0x10000, 0x10000, 0x10000, 64, 128, 128)                   # down-shaped o
    assert L.mq_mixnmatch_forward(_layer(o=bad), 1, P16, 1, P16, P16, ws, NULL) == 2
    # the norm holds a row in registers: H up to 16384
    assert L.mq_mixnmatch_workspace_bytes(_layer(H=16384), 1, 1) > 0
    assert L.mq_mixnmatch_workspace_bytes(_layer(H=16448), 1, 1) == 0
    assert L.mq_mixnmatch_forward(_layer(H=16448), 1, P16, 1, P16, P16, ws, NULL) == 2


def test_gemm_noalloc_validation(L):
    """The no-workspace GEMM validates like mq_gemm and refuses shapes whose
    K-slice partials exceed its 64 MiB scratch, before touching the GPU."""
    call = lambda r=4, g=64, N=4, K=64, M=16, p=P16, y=P16: L.mq_gemm_noalloc(
        p, r, P16, P16, g, N, K, P16, M, y, NULL)
    assert call(p=NULL) == 1
    assert call(y=P1) == 5
    assert call(r=5) == 3
    assert call(M=0) == 2
    assert call(g=32) == 4
    # 64 slices of 64 x 14336 fp32 partials (235 MB) at K = 65536
    assert L.mq_gemm_workspace_bytes(64, 14336, 65536, 128) > mq.GEMM_NOALLOC_MAX_BYTES
    assert call(M=64, N=14336, K=65536, g=128) == 6
    # the prefill down projection at M = 2048 needs exactly the 64 MiB
    assert L.mq_gemm_workspace_bytes(2048, 4096, 14336, 128) == mq.GEMM_NOALLOC_MAX_BYTES


def test_quantize_validation(L):
    assert L.mq_quantize(NULL, 4, 64, 64, P16, P16, P16, NULL) == 1
    assert L.mq_quantize(P16, 4, 64, 32, P16, P16, P16, NULL) == 4
    assert L.mq_quantize(P16, 0, 64, 64, P16, P16, P16, NULL) == 2


def test_overflow_validation(L):
    assert L.mq_overflow_rows(NULL, 4, 64, 2, P16, NULL) == 1
    assert L.mq_overflow_rows(P16, 4, 64, 5, P16, NULL) == 3
    assert L.mq_overflow_rows(P16, 4, 96, 2, P16, NULL) == 2
    assert L.mq_overflow_cols(P16, 4, 64, 2, P16, NULL, NULL) == 1
    assert L.mq_overflow_cols(P16, 0, 64, 2, P16, P16, NULL) == 2
    assert L.mq_overflow_apply(P16, P16, 2, P16, 64, 4, 64, NULL, 1, P16, NULL) == 1
    assert L.mq_overflow_apply(P16, P16, 2, P16, 32, 4, 64, P16, 1, P16, NULL) == 4
    assert L.mq_overflow_apply(P16, P16, 2, P16, 64, 4, 64, P16, 0, P16, NULL) == 2
    assert L.mq_overflow_apply(P16, P16, 7, P16, 64, 4, 64, P16, 1, P16, NULL) == 3
    assert L.mq_overflow_apply(P16, P1, 2, P16, 64, 4, 64, P16, 1, P16, NULL) == 5  # 2-byte col_idx
    probs = (mq.OverflowProblem * 17)()
    assert L.mq_overflow_apply_grouped(probs, 2, 2, 1, NULL) == 1          # null members
    assert L.mq_overflow_apply_grouped(probs, 0, 2, 1, NULL) == 2
    assert L.mq_overflow_apply_grouped(probs, 17, 2, 1, NULL) == 2
    assert L.mq_overflow_apply_grouped(None, 1, 2, 1, NULL) == 1
    for i in range(2):
        probs[i] = mq.OverflowProblem(0x10000, 0x10000, 0x10000, 0x10000, 0x10000, 4, 64, 64)
    assert L.mq_overflow_apply_grouped(probs, 2, 5, 1, NULL) == 3
    probs[1].group = 32
    assert L.mq_overflow_apply_grouped(probs, 2, 2, 1, NULL) == 4


def test_bitplane_validation(L):
    assert L.mq_bitplanes_bytes(14336, 3584) == 14336 * 3584
    assert L.mq_bitplanes_bytes(4, 256) == 0          # K not a multiple of 512
    assert L.mq_bitplanes_bytes(1 << 16, 65536) == 0  # more than 2^31 codes
    assert L.mq_pack_bitplanes(NULL, 4, 512, P16, NULL) == 1
    assert L.mq_pack_bitplanes(P16, 4, 640, P16, NULL) == 2
    assert L.mq_pack_bitplanes(P16, 0, 512, P16, NULL) == 2
    assert L.mq_pack_bitplanes(P16, 4, 512, P1, NULL) == 5

    def gemv(p=P16, r=4, extra=0, a=P16, z=P16, g=512, N=4, K=512, x=P16, M=1, y=P16):
        return L.mq_gemv_bitplanes(p, r, extra, a, z, g, N, K, x, M, y, NULL)

    assert gemv(p=NULL) == 1
    assert gemv(r=0) == 3 and gemv(r=9) == 3
    assert gemv(extra=2) == 3
    assert gemv(K=1000, g=1000) == 2
    assert gemv(M=0) == 2 and gemv(M=9) == 2
    assert gemv(g=64) == 4
    assert gemv(y=P1) == 5


def test_mlp_validation(L):
    assert L.mq_mlp_workspace_bytes(1, 14336) == 2 * 57344 + 28672
    assert L.mq_mlp_workspace_bytes(9, 64) == 0
    lin = lambda n, k, g=None: mq.Linear(0x10000, 0x10000, 0x10000, n, k, g or k)
    up, gate, down = lin(128, 64), lin(128, 64), lin(64, 128)
    ws = 1 << 20

    def call(u=up, g=gate, d=down, r=4, act=0, x=P16, M=1, y=P16, w=P16):
        return L.mq_mlp_decode(ctypes.byref(u) if u else NULL, ctypes.byref(g), ctypes.byref(d),
                               r, act, x, M, y, w, ws, NULL)

    assert call(u=None) == 1
    assert call(x=NULL) == 1
    assert call(r=5) == 3
    assert call(act=3) == 3
    assert call(M=0) == 2 and call(M=9) == 2
    assert call(d=lin(64, 64)) == 2                # down's K must be up's N
    assert call(g=lin(128, 64, 128)) in (2, 4)     # group 128 needs K % 128 (shape) / differs from up
    assert call(u=lin(128, 256, 128), g=lin(128, 256, 256), d=lin(256, 128)) == 4
    assert call(w=NULL) == 6
    assert call(y=P1) == 5


def test_binding_checks_tensors_against_sizes(L):
    """The binding refuses, before any C call, tensors whose dtype or size
    disagrees with the integer arguments the library sizes its buffers from
    (CPU tensors: the checks come before the device check)."""
    torch = pytest.importorskip("torch")
    N, K, r, g = 8, 128, 4, 128
    packed = torch.zeros(N * K * r // 8, dtype=torch.uint8)
    alpha = torch.ones((N, K // g), dtype=torch.float32)
    zero = torch.zeros((N, K // g), dtype=torch.float32)
    x = torch.zeros((2, K), dtype=torch.bfloat16)
    y = torch.zeros((2, N), dtype=torch.float32)
    for f in (mq.gemv, mq.gemm):
        with pytest.raises(ValueError, match="packed"):
            f(packed[:-1], r, alpha, zero, g, N, K, x, out=y)
        with pytest.raises(ValueError, match="packed"):
            f(packed, 2, alpha, zero, g, N, K, x, out=y)        # plane of r = 4 served at r = 2
        with pytest.raises(ValueError, match="alpha"):
            f(packed, r, alpha[:, :0], zero, K, N, K, x, out=y)  # per-channel: N scales
        with pytest.raises(TypeError, match="alpha"):
            f(packed, r, alpha.double(), zero, g, N, K, x, out=y)
        with pytest.raises(ValueError, match="zero"):
            f(packed, r, alpha, zero[:4], g, N, K, x, out=y)
        with pytest.raises(ValueError, match="x"):
            f(packed, r, alpha, zero, g, N, K, x[:, :64], out=y)
        with pytest.raises(TypeError, match="out"):
            f(packed, r, alpha, zero, g, N, K, x, out=y.to(torch.bfloat16))
        with pytest.raises(ValueError, match="out"):
            f(packed, r, alpha, zero, g, N, K, x, out=y[:1])
    with pytest.raises(TypeError, match="activations"):
        mq.gemm(packed, r, alpha, zero, g, N, K, x.float(), out=y)
    with pytest.raises(ValueError, match="out"):
        mq.gemm_noalloc(packed, r, alpha, zero, g, N, K, x, y[:1])
    with pytest.raises(TypeError, match="w"):
        mq.quantize(torch.zeros((N, K), dtype=torch.bfloat16), g)
    with pytest.raises(ValueError, match="out"):
        mq.pack(torch.zeros((N, K), dtype=torch.uint8), r,
                out=torch.zeros(N * K * r // 8 - 16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="planes"):
        mq.gemv_bitplanes(torch.zeros(N * K - 1, dtype=torch.uint8), 2, alpha, zero, g, N, K, x,
                          out=y)
    with pytest.raises(ValueError, match="different devices"):
        mq._same_device(x, torch.zeros(1, device="meta"))
    lin = {"packed": packed, "alpha": alpha, "zero": zero, "N": N, "K": K, "group": g}
    with pytest.raises(ValueError, match="packed"):
        mq.make_layers([{"r": 2, **{n: lin for n in mq.LAYER_LINEARS}}])


def test_binding_rejects_host_tensors(L):
    """The binding passes only GPU tensors to the library: a host tensor is
    refused before any call (no silent host pointer)."""
    torch = pytest.importorskip("torch")
    codes = torch.zeros((4, 64), dtype=torch.uint8)
    with pytest.raises(ValueError):
        mq.pack(codes, 4, out=torch.zeros((4, 32), dtype=torch.uint8))
    with pytest.raises(ValueError):
        mq._ptr(torch.zeros(8))
