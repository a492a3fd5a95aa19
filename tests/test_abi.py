"""CPU checks of the C ABI: the library loads, exports every function that
``include/*.h`` declares, rejects invalid arguments on the host before
anything is enqueued (no GPU needed: these calls return before any HIP
call), and negotiates the scale layout between consumers (a host-only
helper; PRHub report of vLLM PR #56433, item 4)."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

import rmsnorm_fp8_block_amd as mi
from rmsnorm_fp8_block_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mi_\w+)\s*\(", text, re.M))
    return names


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail(f"{B.LIB_PATH} not built (run `python -m rmsnorm_fp8_block_amd.build`)")
    return mi.lib()


def test_header_declares_the_boundary():
    assert declared_functions() == set(B.EXPORTED)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(L, name)


def test_no_kernel_of_the_library_is_left_undefined():
    """A kernel whose launch stub the host compiler pass dropped shows up as
    an undefined symbol of the library's own namespace (the library would
    then fail to load on any machine with a GPU)."""
    out = subprocess.run(["nm", "-D", "--undefined-only", B.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    own = [line.split()[-1] for line in out.splitlines() if "_ZN2mi" in line]
    assert not own, own[:5]


def test_status_strings(L):
    for s in range(8):
        assert mi.mi_status_string(s).startswith(("MI_OK", "MI_ERR"))
    assert mi.mi_status_string(99) == "unknown mi_status"


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
NULL = ctypes.c_void_p(0)


def nq(L, **kw):
    a = dict(q=FAKE, qs=1536, kv=FAKE, ks=512, gq=FAKE, gk=FAKE, eps=1e-6, M=4, Nq=1536,
             Nkv=512, t=0, oq=FAKE, os_=FAKE, okv=FAKE)
    a.update(kw)
    return L.mi_fused_dual_rmsnorm_group_quant(a["q"], a["qs"], a["kv"], a["ks"], a["gq"], a["gk"],
                                               ctypes.c_float(a["eps"]), a["M"], a["Nq"], a["Nkv"],
                                               a["t"], a["oq"], a["os_"], a["okv"], NULL)


def test_normquant_validation(L):
    assert nq(L, M=-1) == B.MI_ERR_SHAPE
    assert nq(L, Nq=1500) == B.MI_ERR_SHAPE          # not a multiple of 128
    assert nq(L, Nq=0) == B.MI_ERR_SHAPE
    assert nq(L, Nq=4096 + 128) == B.MI_ERR_SHAPE
    assert nq(L, Nkv=0) == B.MI_ERR_SHAPE
    assert nq(L, Nkv=2049) == B.MI_ERR_SHAPE
    assert nq(L, M=0) == B.MI_OK                      # no-op, nothing enqueued
    assert nq(L, M=0, q=NULL, oq=NULL) == B.MI_OK
    for k in ("q", "kv", "gq", "gk", "oq", "os_", "okv"):
        assert nq(L, **{k: NULL}) == B.MI_ERR_NULL, k
    assert nq(L, qs=1535) == B.MI_ERR_STRIDE
    assert nq(L, ks=511) == B.MI_ERR_STRIDE


def single(L, normalize, **kw):
    a = dict(x=FAKE, xs=7168, g=FAKE, eps=1e-6, M=4, N=7168, t=0, oq=FAKE, os_=FAKE)
    a.update(kw)
    if normalize:
        return L.mi_rmsnorm_group_quant(a["x"], a["xs"], a["g"], ctypes.c_float(a["eps"]), a["M"], a["N"], a["t"],
                                        a["oq"], a["os_"], NULL)
    return L.mi_group_quant_1x128(a["x"], a["xs"], a["M"], a["N"], a["t"], a["oq"], a["os_"], NULL)


@pytest.mark.parametrize("normalize", [True, False])
def test_single_input_quant_validation(L, normalize):
    assert single(L, normalize, M=-1) == B.MI_ERR_SHAPE
    for n in (0, 100, 1500, 8192 + 128):
        assert single(L, normalize, N=n, xs=max(n, 1)) == B.MI_ERR_SHAPE, n
    assert single(L, normalize, M=0) == B.MI_OK
    assert single(L, normalize, M=0, x=NULL) == B.MI_OK
    for k in ("x", "oq", "os_"):
        assert single(L, normalize, **{k: NULL}) == B.MI_ERR_NULL, k
    # gamma is read only by the normalising form
    want = B.MI_ERR_NULL if normalize else B.MI_ERR_STRIDE
    assert single(L, normalize, g=NULL, xs=100) == want
    assert single(L, normalize, xs=7167) == B.MI_ERR_STRIDE


def gemm(L, **kw):
    a = dict(a=FAKE, As=FAKE, t=0, w=FAKE, Bs=FAKE, out=FAKE, M=4, N=1024, K=1536)
    a.update(kw)
    return L.mi_block_scaled_fp8_gemm(a["a"], a["As"], a["t"], a["w"], a["Bs"], a["out"],
                                      a["M"], a["N"], a["K"], NULL)


def test_gemm_validation(L):
    assert gemm(L, M=-1) == B.MI_ERR_SHAPE
    assert gemm(L, N=1000) == B.MI_ERR_SHAPE
    assert gemm(L, K=1000) == B.MI_ERR_SHAPE
    assert gemm(L, N=0) == B.MI_ERR_SHAPE
    assert gemm(L, M=0) == B.MI_OK
    for k in ("a", "As", "w", "Bs", "out"):
        assert gemm(L, **{k: NULL}) == B.MI_ERR_NULL, k
    assert gemm(L, a=ctypes.c_void_p(0x1008)) == B.MI_ERR_ALIGN
    assert gemm(L, w=ctypes.c_void_p(0x1004)) == B.MI_ERR_ALIGN
    assert gemm(L, out=ctypes.c_void_p(0x1002)) == B.MI_ERR_ALIGN
    assert gemm(L, As=ctypes.c_void_p(0x1002)) == B.MI_ERR_ALIGN


def gemm_pair(L, **kw):
    a = dict(a=FAKE, As=FAKE, t=0, w1=FAKE, Bs1=FAKE, out1=FAKE, N1=24576, w2=FAKE, Bs2=FAKE, out2=FAKE,
             N2=8192, M=4, K=1536)
    a.update(kw)
    return L.mi_block_scaled_fp8_gemm_pair(a["a"], a["As"], a["t"], a["w1"], a["Bs1"], a["out1"], a["N1"],
                                           a["w2"], a["Bs2"], a["out2"], a["N2"], a["M"], a["K"], NULL)


def test_gemm_pair_validation(L):
    assert gemm_pair(L, M=-1) == B.MI_ERR_SHAPE
    for k, v in (("N1", 1000), ("N2", 1000), ("K", 1000), ("N1", 0), ("N2", 0)):
        assert gemm_pair(L, **{k: v}) == B.MI_ERR_SHAPE, k
    assert gemm_pair(L, M=0) == B.MI_OK
    for k in ("a", "As", "w1", "Bs1", "out1", "w2", "Bs2", "out2"):
        assert gemm_pair(L, **{k: NULL}) == B.MI_ERR_NULL, k
    for k, v in (("a", 0x1008), ("w1", 0x1004), ("w2", 0x1004), ("out1", 0x1002), ("out2", 0x1002),
                 ("As", 0x1002), ("Bs1", 0x1002), ("Bs2", 0x1002)):
        assert gemm_pair(L, **{k: ctypes.c_void_p(v)}) == B.MI_ERR_ALIGN, k


def test_negotiate_scale_layout(L):
    assert mi.mi_negotiate_scale_layout([1, 1]) is True
    assert mi.mi_negotiate_scale_layout([0, 0, 0]) is False
    assert mi.mi_negotiate_scale_layout([1, 0]) is None
    assert mi.mi_negotiate_scale_layout([]) is None
    assert L.mi_negotiate_scale_layout(None, 2) == -1
    assert mi.mi_negotiate_scale_layout([5, 1]) is True    # any non-zero means "transposed"


def test_binding_raises_on_error_status():
    with pytest.raises(mi.MiError) as e:
        B._check("x", B.MI_ERR_SHAPE)
    assert e.value.status == B.MI_ERR_SHAPE


def relayout(L, **kw):
    a = dict(src=FAKE, fl=0, dst=ctypes.c_void_p(0x2000), tl=1, N=256, K=1536)
    a.update(kw)
    return L.mi_relayout_weight(a["src"], a["fl"], a["dst"], a["tl"], a["N"], a["K"], NULL)


def test_relayout_validation(L):
    for k, v in (("fl", 2), ("tl", -1)):
        assert relayout(L, **{k: v}) == B.MI_ERR_LAYOUT, k
    for k, v in (("N", 8), ("K", 100), ("N", -16)):
        assert relayout(L, **{k: v}) == B.MI_ERR_SHAPE, (k, v)
    assert relayout(L, N=0) == B.MI_OK
    for k in ("src", "dst"):
        assert relayout(L, **{k: NULL}) == B.MI_ERR_NULL, k
    assert relayout(L, dst=FAKE) == B.MI_ERR_ALIAS
    assert relayout(L, dst=ctypes.c_void_p(0x2008)) == B.MI_ERR_ALIGN


def test_gemm_ex_layout_validation(L):
    st = L.mi_block_scaled_fp8_gemm_ex(FAKE, FAKE, 0, FAKE, 2, FAKE, FAKE, 4, 1024, 1536, NULL)
    assert st == B.MI_ERR_LAYOUT
    st = L.mi_block_scaled_fp8_gemm_pair_ex(FAKE, FAKE, 0, 5, FAKE, FAKE, FAKE, 256, FAKE, FAKE, FAKE, 256, 4, 1536,
                                            NULL)
    assert st == B.MI_ERR_LAYOUT
    # a valid layout value goes on to the ordinary checks
    st = L.mi_block_scaled_fp8_gemm_ex(FAKE, FAKE, 0, FAKE, 1, FAKE, FAKE, 4, 1000, 1536, NULL)
    assert st == B.MI_ERR_SHAPE


def test_capabilities_and_preferred_layout(L):
    caps = mi.mi_gemm_capabilities()
    assert caps == B.MI_CAP_AS_ROW_MAJOR | B.MI_CAP_AS_COL_MAJOR | B.MI_CAP_WEIGHT_TILED | B.MI_CAP_SCALE_E8M0
    assert mi.mi_preferred_weight_layout(24576, 1536) in (B.MI_WEIGHT_ROW_MAJOR, B.MI_WEIGHT_TILED)
    for n, k in ((100, 1536), (256, 0), (-128, 128)):
        assert mi.mi_preferred_weight_layout(n, k) == -1


def test_binding_refuses_a_second_relayout():
    """The relayout is a permutation, not an involution: a TiledWeight is
    never relaid out again (checked before any device work)."""
    import torch
    tw = B.TiledWeight(torch.empty(0, dtype=torch.uint8), 128, 128)
    assert mi.weight_already_tiled(tw)
    with pytest.raises(TypeError):
        mi.relayout_weight(tw)
    with pytest.raises(TypeError):
        mi.untile_weight(torch.empty((128, 128), dtype=torch.uint8))


def test_e8m0_entry_validation(L):
    # dual norm-quant: same checks as the fp32-scale call, the byte scales required
    nq8 = lambda **kw: L.mi_fused_dual_rmsnorm_group_quant_e8m0(
        kw.get("q", FAKE), 1536, FAKE, 512, FAKE, FAKE, ctypes.c_float(1e-6), kw.get("M", 4), kw.get("Nq", 1536), 512,
        0, FAKE, kw.get("os_", FAKE), FAKE, NULL)
    assert nq8(Nq=1500) == B.MI_ERR_SHAPE
    assert nq8(os_=NULL) == B.MI_ERR_NULL
    assert nq8(os_=NULL, M=0) == B.MI_OK
    assert nq8(M=-1, os_=NULL) == B.MI_ERR_SHAPE
    # GEMMs
    g8 = lambda **kw: L.mi_block_scaled_fp8_gemm_e8m0(
        FAKE, kw.get("As", FAKE), 0, FAKE, kw.get("wl", 0), kw.get("Bs", FAKE), FAKE, 4, kw.get("N", 1024), 1536, NULL)
    assert g8(wl=3) == B.MI_ERR_LAYOUT
    assert g8(N=1000) == B.MI_ERR_SHAPE
    assert g8(As=NULL) == B.MI_ERR_NULL
    assert g8(As=ctypes.c_void_p(0x1002)) == B.MI_ERR_ALIGN
    assert g8(Bs=ctypes.c_void_p(0x1001)) == B.MI_ERR_ALIGN
    p8 = lambda **kw: L.mi_block_scaled_fp8_gemm_pair_e8m0(
        FAKE, FAKE, 0, kw.get("wl", 0), FAKE, kw.get("Bs1", FAKE), FAKE, 256, FAKE, FAKE, FAKE, kw.get("N2", 256), 4,
        1536, NULL)
    assert p8(wl=9) == B.MI_ERR_LAYOUT
    assert p8(N2=100) == B.MI_ERR_SHAPE
    assert p8(Bs1=NULL) == B.MI_ERR_NULL


def step(L, e8m0=False, **kw):
    a = dict(q=FAKE, qs=2048, kv=FAKE, ks=2048, gq=FAKE, gk=FAKE, eps=1e-6, M=4, Nq=1536, Nkv=512, t=1,
             oq=FAKE, os_=FAKE, okv=FAKE, wl=B.MI_WEIGHT_TILED, w1=FAKE, Bs1=FAKE, out1=FAKE, N1=24576,
             w2=FAKE, Bs2=FAKE, out2=FAKE, N2=8192)
    a.update(kw)
    fn = L.mi_fused_normquant_gemm_pair_e8m0 if e8m0 else L.mi_fused_normquant_gemm_pair
    return fn(
        a["q"], a["qs"], a["kv"], a["ks"], a["gq"], a["gk"], ctypes.c_float(a["eps"]), a["M"], a["Nq"], a["Nkv"],
        a["t"], a["oq"], a["os_"], a["okv"], a["wl"], a["w1"], a["Bs1"], a["out1"], a["N1"], a["w2"], a["Bs2"],
        a["out2"], a["N2"], NULL)


@pytest.mark.parametrize("e8m0", [False, True])
def test_fused_step_validation(L, e8m0):
    """The one-call decode step (fp32 or e8m0 scales) checks what both of
    its parts check."""
    assert step(L, e8m0, wl=2) == B.MI_ERR_LAYOUT
    for k, v in (("M", -1), ("Nq", 1500), ("Nkv", 0), ("N1", 1000), ("N2", 0)):
        assert step(L, e8m0, **{k: v}) == B.MI_ERR_SHAPE, k
    assert step(L, e8m0, M=0) == B.MI_OK
    assert step(L, e8m0, M=0, q=NULL) == B.MI_OK
    for k in ("q", "kv", "gq", "gk", "oq", "os_", "okv", "w1", "Bs1", "out1", "w2", "Bs2", "out2"):
        assert step(L, e8m0, **{k: NULL}) == B.MI_ERR_NULL, k
    assert step(L, e8m0, qs=1535) == B.MI_ERR_STRIDE
    for k, v in (("oq", 0x1008), ("w1", 0x1004), ("out2", 0x1002), ("os_", 0x1002), ("Bs2", 0x1001)):
        assert step(L, e8m0, **{k: ctypes.c_void_p(v)}) == B.MI_ERR_ALIGN, k


def test_fused_step_launch_count(L):
    """One launch for decode batches of the MLA shape over wide weights (the
    CU count taken as 256 where no GPU is visible); otherwise the
    norm-quant's launch plus the pair's one or two; 0 / -1 as documented."""
    f = mi.mi_fused_normquant_gemm_pair_launches
    assert f(0, 1536, 512, 24576, 8192) == 0
    for M in (1, 7, 16):
        assert f(M, 1536, 512, 24576, 8192) == 1, M
    for M in (17, 64):
        assert f(M, 1536, 512, 24576, 8192) == 2, M   # norm-quant, then the pair in one launch
    assert f(65, 1536, 512, 24576, 8192) == 3         # ... the pair as two GEMMs
    assert f(256, 1536, 512, 24576, 8192) == 3
    assert f(64, 2560, 512, 24576, 8192) == 3         # K / 128 = 20: two GEMMs
    assert f(1, 1536, 512, 3072, 1024) == 2       # narrow weights
    assert f(256, 1536, 512, 3072, 1024) == 2     # narrow pair above 64 rows: one launch
    assert f(256, 1536, 512, 6144, 2048) == 2
    assert f(256, 1536, 512, 12288, 4096) == 2    # TP-2 pair: 1024 subtiles, one launch
    assert f(257, 1536, 512, 3072, 1024) == 3     # beyond 256 rows: two GEMMs
    assert f(256, 2048, 512, 3072, 1024) == 3     # K / 128 = 16 above 64 rows: two GEMMs
    assert f(1, 1024, 512, 24576, 8192) == 2      # other latent width
    assert f(1, 1536, 448, 24576, 8192) == 2
    assert f(-1, 1536, 512, 24576, 8192) == -1
    assert f(1, 1500, 512, 24576, 8192) == -1
    assert f(1, 1536, 512, 1000, 8192) == -1


# ---- binding-side validation (CPU tensors: every check below raises before
# any library call, so no GPU is touched) ----

def _dual_cpu(M=4, Nq=1536, Nkv=512):
    import torch
    buf = torch.zeros((M, Nq + Nkv), dtype=torch.bfloat16)
    return dict(q=buf[:, :Nq], kv=buf[:, Nq:], gamma_q=torch.ones(Nq, dtype=torch.bfloat16),
                gamma_kv=torch.ones(Nkv, dtype=torch.bfloat16), eps=1e-6, transpose_scale=True,
                out_q=torch.empty((M, Nq), dtype=torch.uint8), out_scale=torch.empty(M * (Nq // 128)),
                out_kv=torch.empty((M, Nkv), dtype=torch.bfloat16))


def _e8m0(a):
    import torch
    a = dict(a)
    a["out_scale"] = torch.empty(a["out_scale"].numel(), dtype=torch.uint8)
    return a


DUAL_CALLS = (
    ("eager", lambda a: mi.mi_fused_dual_rmsnorm_group_quant(**a)),
    ("prepared", lambda a: mi.prepare_fused_dual_rmsnorm_group_quant(**a)),
    ("eager_e8m0", lambda a: mi.mi_fused_dual_rmsnorm_group_quant_e8m0(**_e8m0(a))),
    ("prepared_e8m0", lambda a: mi.prepare_fused_dual_rmsnorm_group_quant_e8m0(**_e8m0(a))),
)


@pytest.mark.parametrize("name,call", DUAL_CALLS, ids=[n for n, _ in DUAL_CALLS])
def test_dual_binding_checks(name, call):
    """Each form of the dual norm-quant (eager, prepared, fp32 and e8m0
    scales) runs the same checks: unit inner stride at every row count
    (a strided single row included), kv rows == q rows, gammas bf16,
    contiguous and of the row widths, contiguous outputs of the right type
    and size, and every tensor on the GPU of q."""
    import torch
    ok = _dual_cpu()
    with pytest.raises(ValueError, match="GPU tensor"):   # valid except for the device
        call(ok)
    one = _dual_cpu(M=1)
    one["q"] = torch.zeros((1, 3072), dtype=torch.bfloat16)[:, ::2]   # strides (3072, 2)
    with pytest.raises(ValueError, match="inner stride"):
        call(one)
    for key, value, msg in (
            ("kv", torch.zeros((3, 512), dtype=torch.bfloat16), "same number of rows"),
            ("gamma_q", torch.ones(1535, dtype=torch.bfloat16), "gamma_q"),
            ("gamma_kv", torch.ones(512, dtype=torch.float32), "gamma_kv"),
            ("gamma_q", torch.ones(3072, dtype=torch.bfloat16)[::2], "gamma_q"),
            ("out_q", torch.empty((1536, 4), dtype=torch.uint8).T, "contiguous"),
            ("out_kv", torch.empty((4, 511), dtype=torch.bfloat16), "too small"),
            ("out_kv", torch.empty((4, 512), dtype=torch.float16), "out_kv")):
        bad = _dual_cpu()
        bad[key] = value
        with pytest.raises(ValueError, match=msg):
            call(bad)
    if "e8m0" in name:
        with pytest.raises(ValueError, match="out_scale"):  # fp32 scales where bytes are written
            fn = (mi.mi_fused_dual_rmsnorm_group_quant_e8m0 if name == "eager_e8m0"
                  else mi.prepare_fused_dual_rmsnorm_group_quant_e8m0)
            fn(**_dual_cpu())
    else:
        bad = _dual_cpu()
        bad["out_scale"] = torch.empty(48, dtype=torch.uint8)
        with pytest.raises(ValueError, match="out_scale"):
            call(bad)


@pytest.mark.parametrize("prepared", [False, True])
@pytest.mark.parametrize("normalize", [False, True])
def test_single_input_binding_checks(prepared, normalize):
    import torch
    M, N = 4, 1536

    def call(x, gamma=None, out_q=None, out_scale=None):
        out_q = torch.empty((M, N), dtype=torch.uint8) if out_q is None else out_q
        out_scale = torch.empty(M * 12) if out_scale is None else out_scale
        gamma = torch.ones(N, dtype=torch.bfloat16) if gamma is None else gamma
        if normalize:
            f = mi.prepare_rmsnorm_group_quant if prepared else mi.mi_rmsnorm_group_quant
            return f(x, gamma, 1e-6, True, out_q, out_scale)
        f = mi.prepare_group_quant_1x128 if prepared else mi.mi_group_quant_1x128
        return f(x, True, out_q, out_scale)

    x = torch.zeros((M, N), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        call(x)
    with pytest.raises(ValueError, match="inner stride"):
        call(torch.zeros((1, 2 * N), dtype=torch.bfloat16)[:, ::2])
    with pytest.raises(ValueError, match="contiguous"):
        call(x, out_q=torch.empty((N, M), dtype=torch.uint8).T)
    with pytest.raises(ValueError, match="out_scale"):
        call(x, out_scale=torch.empty(M * 12, dtype=torch.float16))
    if normalize:
        with pytest.raises(ValueError, match="gamma"):
            call(x, gamma=torch.ones(N, dtype=torch.float32))
        with pytest.raises(ValueError, match="gamma"):
            call(x, gamma=torch.ones(N - 128, dtype=torch.bfloat16))


@pytest.mark.parametrize("prepared", [False, True])
def test_gemm_binding_checks(prepared):
    """The GEMM calls check operand types, shapes and the As strides, and
    that every tensor sits on the GPU of the activation."""
    import torch
    M, N, K = 4, 256, 1536
    a = torch.zeros((M, K), dtype=torch.uint8)
    a_s = torch.ones((M, K // 128))
    w = torch.zeros((N, K), dtype=torch.uint8)
    w_s = torch.ones((N // 128, K // 128))
    out = torch.empty((M, N), dtype=torch.bfloat16)

    def call(a=a, a_s=a_s, w=w, w_s=w_s, out=out):
        if prepared:
            return mi.prepare_block_scaled_fp8_gemm(a, a_s, w, w_s, out)
        return mi.mi_block_scaled_fp8_gemm(a, a_s, w, w_s, out)

    with pytest.raises(ValueError, match="GPU tensor"):
        call()
    with pytest.raises(ValueError, match="neither row- nor column-major"):
        call(a_s=torch.ones((M, 2 * K // 128))[:, ::2])
    with pytest.raises(ValueError, match="neither row- nor column-major"):
        call(a_s=torch.ones((1, 2 * K // 128))[:, ::2], a=a[:1], out=out[:1])
    with pytest.raises(ValueError, match="shape mismatch"):
        call(w_s=torch.ones((1, K // 128)))
    with pytest.raises(ValueError, match="out"):
        call(out=torch.empty((M, N), dtype=torch.float32))
    with pytest.raises(ValueError, match="out"):
        call(out=torch.empty((N, M), dtype=torch.bfloat16).T)
    assert B.scale_is_transposed(torch.ones((12, M)).T) is True
    assert B.scale_is_transposed(torch.ones((M, 12))) is False
    assert B.scale_is_transposed(torch.ones((1, 12))) is False


@pytest.mark.parametrize("prepared", [False, True])
def test_step_binding_checks(prepared):
    """The one-call step runs the dual norm-quant's checks (short kv, short
    gamma, device) and the weights' ones."""
    import torch
    base = _dual_cpu()
    W1 = torch.zeros((256, 1536), dtype=torch.uint8)
    W2 = torch.zeros((128, 1536), dtype=torch.uint8)
    S1, S2 = torch.ones((2, 12)), torch.ones((1, 12))
    out1 = torch.empty((4, 256), dtype=torch.bfloat16)
    out2 = torch.empty((4, 128), dtype=torch.bfloat16)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        args = (a["q"], a["kv"], a["gamma_q"], a["gamma_kv"], 1e-6, True, W1, a.get("S1", S1), W2, S2)
        outs = dict(out_q=a["out_q"], out_scale=a["out_scale"], out_kv=a["out_kv"], out1=out1, out2=out2)
        if prepared:
            return mi.prepare_fused_normquant_gemm_pair(*args, **outs)
        return mi.mi_fused_normquant_gemm_pair(*args, **outs)

    with pytest.raises(ValueError, match="GPU tensor"):
        call()
    with pytest.raises(ValueError, match="same number of rows"):
        call(kv=torch.zeros((2, 512), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="gamma_kv"):
        call(gamma_kv=torch.ones(100, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="w1"):
        call(S1=torch.ones((2, 12), dtype=torch.float64))


def test_init_reports_hip_errors_without_a_device(L):
    """mi_init needs a device: with none visible (this CPU host) it returns
    MI_ERR_HIP and the binding raises; it never crashes."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert L.mi_init() == B.MI_ERR_HIP
    with pytest.raises(mi.MiError):
        mi.mi_init()


def test_ceiling_library_loads_and_refuses_bad_arguments():
    """The benchmark's ceiling library (bench.py only; nothing in the hot
    path calls it) exports its three skeletons, and each refuses malformed
    sizes before touching the device (so this runs without a GPU)."""
    from rmsnorm_fp8_block_amd import build
    C = ctypes.CDLL(build.CEILING_LIB)
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    C.mi_ceiling_normquant_skeleton.argtypes = [p, i64, p, p, p, i64, p]
    C.mi_ceiling_weight_stream.argtypes = [p, i64, i64, p, p]
    C.mi_ceiling_mfma.argtypes = [i64, ctypes.c_int, i64, ctypes.c_int, ctypes.c_float, p, p, p]
    ok = 0
    assert C.mi_ceiling_normquant_skeleton(None, 2048, None, None, None, 0, None) == ok   # M = 0: nothing to launch
    for slab, blocks in ((4096 + 1, 1), (0, 1), (4096, 0), (4096, 1 << 31)):
        assert C.mi_ceiling_weight_stream(None, slab, blocks, None, None) != ok, (slab, blocks)
    for blocks, waves, per_wave, scale in ((0, 4, 96, 1.0), (1, 0, 96, 1.0), (1, 17, 96, 1.0), (1, 4, 95, 1.0),
                                           (1, 4, 0, 1.0), (1, 4, 96, 0.0), (1, 4, 96, -1.0)):
        assert C.mi_ceiling_mfma(blocks, waves, per_wave, 1, scale, None, None, None) != ok, \
            (blocks, waves, per_wave, scale)
