"""The C-ABI library on the host (no GPU needed): it loads, exports every
function include/specverify.h declares, and rejects bad arguments before
enqueuing anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")
LIB = os.path.join(ROOT, "lossless_verification_sampling_amd", "libspecverify.so")

SPEC_OK, SPEC_EINVAL, SPEC_EDTYPE, SPEC_EWORKSPACE, SPEC_EHIP, SPEC_EUNSUPPORTED = 0, -1, -2, -3, -4, -5
SPEC_ETOOLARGE = -6
NOALLOC_SCRATCH = 32 << 20


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    assert os.path.exists(LIB), "build the library first (__graft_entry__.build())"
    return ctypes.CDLL(LIB)


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in specverify.h but not exported"


def test_python_binding_names_match_header():
    import lossless_verification_sampling_amd as sv
    assert sorted(sv.EXPORTED) == declared_functions()
    for n in sv.EXPORTED:
        assert callable(getattr(sv, n))


def test_status_strings_and_version(lib):
    lib.spec_status_string.restype = ctypes.c_char_p
    for s in (SPEC_OK, SPEC_EINVAL, SPEC_EDTYPE, SPEC_EWORKSPACE, SPEC_EHIP, SPEC_EUNSUPPORTED,
              SPEC_ETOOLARGE):
        assert lib.spec_status_string(s).startswith(b"SPEC_")
    assert lib.spec_version() >= 100


def test_workspace_sizes(lib):
    f = lib.spec_verify_workspace_bytes
    f.restype = ctypes.c_size_t
    assert f(64, 7, 151936) > 0 and f(64, 7, 151936) % 256 == 0
    assert f(-1, 7, 100) == 0 and f(1, -1, 100) == 0 and f(1, 1, 0) == 0
    assert f(1, 65, 100) == 0                      # gamma above the supported maximum
    assert f(1, 1, 262144) > 0 and f(1, 1, 262145) == 0
    assert f(256, 7, 129280) >= f(64, 7, 129280)
    g = lib.spec_tv_workspace_bytes
    g.restype = ctypes.c_size_t
    assert g(10, 1000) > 0 and g(-1, 10) == 0
    m = lib.spec_markov_workspace_bytes
    m.restype = ctypes.c_size_t
    assert m(64, 7, 129280, 256) > 0 and m(64, 7, 129280, 128) == 0


def _verify(lib, **kw):
    p = ctypes.c_void_p
    fake = p(0x1000)
    args = dict(target=fake, t_dtype=1, draft=fake, d_dtype=1, tokens=fake, vlen=fake, temp=fake,
                ua=fake, us=fake, R=4, gamma=3, V=100, out_tok=fake, out_n=fake, cs=None,
                rs=None, lq=None, ws=p(0x10000), ws_bytes=1 << 30, stream=None)
    args.update(kw)
    f = lib.spec_verify_batch
    f.restype = ctypes.c_int
    f.argtypes = [p, ctypes.c_int, p, ctypes.c_int, p, p, p, p, p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, p, p, p, p, p, p, ctypes.c_size_t, p]
    return f(args["target"], args["t_dtype"], args["draft"], args["d_dtype"], args["tokens"],
             args["vlen"], args["temp"], args["ua"], args["us"], args["R"], args["gamma"],
             args["V"], args["out_tok"], args["out_n"], args["cs"], args["rs"], args["lq"],
             args["ws"], args["ws_bytes"], args["stream"])


def test_verify_argument_validation(lib):
    """Every case below must be rejected on the host before any HIP call."""
    assert _verify(lib, R=-1) == SPEC_EINVAL
    assert _verify(lib, V=0) == SPEC_EINVAL
    assert _verify(lib, gamma=-2) == SPEC_EINVAL
    assert _verify(lib, t_dtype=7) == SPEC_EDTYPE
    assert _verify(lib, d_dtype=-1) == SPEC_EDTYPE
    assert _verify(lib, gamma=65) == SPEC_EUNSUPPORTED
    assert _verify(lib, V=2097153) == SPEC_EUNSUPPORTED
    assert _verify(lib, target=None) == SPEC_EINVAL
    assert _verify(lib, us=None) == SPEC_EINVAL
    assert _verify(lib, out_n=None) == SPEC_EINVAL
    assert _verify(lib, draft=None) == SPEC_EINVAL
    assert _verify(lib, tokens=None) == SPEC_EINVAL
    assert _verify(lib, ws=None) == SPEC_EWORKSPACE
    assert _verify(lib, ws=ctypes.c_void_p(0x10010)) == SPEC_EWORKSPACE   # misaligned
    assert _verify(lib, ws_bytes=256) == SPEC_EWORKSPACE                  # too small
    assert _verify(lib, R=0) == SPEC_OK                                   # nothing to do


def test_markov_and_tv_argument_validation(lib):
    p = ctypes.c_void_p
    fake = p(0x1000)
    m = lib.spec_markov_draft_sample
    m.restype = ctypes.c_int
    m.argtypes = [p, ctypes.c_int, p, p, ctypes.c_int, p, p, p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, p, p, p, ctypes.c_size_t, p]

    def mk(**kw):
        a = dict(U=fake, ud=1, W1=fake, W2=fake, wd=1, anchor=fake, temp=fake, u=fake, R=2,
                 gamma=3, V=100, rank=256, tok=fake, lg=fake, ws=p(0x10000), wsb=1 << 30)
        a.update(kw)
        return m(a["U"], a["ud"], a["W1"], a["W2"], a["wd"], a["anchor"], a["temp"], a["u"],
                 a["R"], a["gamma"], a["V"], a["rank"], a["tok"], a["lg"], a["ws"], a["wsb"],
                 None)

    assert mk(rank=128) == SPEC_EUNSUPPORTED
    assert mk(wd=0) == SPEC_EDTYPE
    assert mk(ud=5) == SPEC_EDTYPE
    assert mk(R=-1) == SPEC_EINVAL
    assert mk(U=None) == SPEC_EINVAL
    assert mk(W1=p(0x1002)) == SPEC_EINVAL          # W1 must be 16-byte aligned
    assert mk(ws=None) == SPEC_EWORKSPACE
    assert mk(wsb=100) == SPEC_EWORKSPACE
    assert mk(R=0) == SPEC_OK and mk(gamma=0) == SPEC_OK

    t = lib.spec_tv_accept_rate
    t.restype = ctypes.c_int
    t.argtypes = [p, p, ctypes.c_int, p, ctypes.c_int, ctypes.c_int, p, p, p, ctypes.c_size_t, p]
    assert t(fake, fake, 3, fake, 4, 100, fake, None, p(0x10000), 1 << 30, None) == SPEC_EDTYPE
    assert t(None, fake, 0, fake, 4, 100, fake, None, p(0x10000), 1 << 30, None) == SPEC_EINVAL
    assert t(fake, fake, 0, fake, 4, 100, fake, None, None, 1 << 30, None) == SPEC_EWORKSPACE
    assert t(fake, fake, 0, fake, 0, 100, fake, None, None, 0, None) == SPEC_OK


def test_rnn_argument_validation(lib):
    p = ctypes.c_void_p
    fake = p(0x1000)
    f = lib.spec_rnn_draft_sample
    f.restype = ctypes.c_int
    i = ctypes.c_int
    f.argtypes = [p, i, p, p, i, p, i, p, p, p, p, p, i, i, i, i, p, p, p, p, ctypes.c_size_t, p]

    def rn(**kw):
        a = dict(U=fake, ud=1, W1=fake, W2=fake, wd=1, H=fake, hid=64, Wg=fake, bg=fake,
                 anchor=fake, temp=fake, u=fake, R=2, gamma=3, V=100, rank=256, tok=fake, lg=fake,
                 st=None, ws=p(0x10000), wsb=1 << 30)
        a.update(kw)
        return f(a["U"], a["ud"], a["W1"], a["W2"], a["wd"], a["H"], a["hid"], a["Wg"], a["bg"],
                 a["anchor"], a["temp"], a["u"], a["R"], a["gamma"], a["V"], a["rank"], a["tok"],
                 a["lg"], a["st"], a["ws"], a["wsb"], None)

    assert rn(rank=128) == SPEC_EUNSUPPORTED
    assert rn(hid=3073) == SPEC_EUNSUPPORTED
    assert rn(hid=0) == SPEC_EINVAL
    assert rn(wd=0) == SPEC_EDTYPE
    assert rn(H=None) == SPEC_EINVAL
    assert rn(Wg=None) == SPEC_EINVAL
    assert rn(bg=None) == SPEC_EINVAL
    assert rn(W2=p(0x1008)) == SPEC_EINVAL
    assert rn(ws=None) == SPEC_EWORKSPACE
    assert rn(wsb=100) == SPEC_EWORKSPACE
    assert rn(R=0) == SPEC_OK and rn(gamma=0) == SPEC_OK
    w = lib.spec_rnn_workspace_bytes
    w.restype = ctypes.c_size_t
    assert w(64, 7, 129280, 256, 1024) > 0 and w(64, 7, 129280, 256, 4000) == 0


def test_schedule_argument_validation(lib):
    p = ctypes.c_void_p
    fake = p(0x1000)
    f = lib.spec_schedule_verify_len
    f.restype = ctypes.c_int
    f.argtypes = [p, p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, p, p, p,
                  ctypes.c_size_t, p]
    w = lib.spec_schedule_workspace_bytes
    w.restype = ctypes.c_size_t
    assert w() == 256

    def sc(**kw):
        a = dict(c=fake, sps=fake, R=64, gamma=7, bmax=600, topk=-1, out=fake, th=None,
                 ws=p(0x10000), wsb=256)
        a.update(kw)
        return f(a["c"], a["sps"], a["R"], a["gamma"], a["bmax"], a["topk"], a["out"], a["th"],
                 a["ws"], a["wsb"], None)

    assert sc(R=-1) == SPEC_EINVAL
    assert sc(gamma=-1) == SPEC_EINVAL
    assert sc(bmax=-1) == SPEC_EINVAL
    assert sc(R=2048, gamma=5) == SPEC_EUNSUPPORTED    # pool of 10240 > 8192
    assert sc(c=None) == SPEC_EINVAL
    assert sc(sps=None) == SPEC_EINVAL
    assert sc(out=None) == SPEC_EINVAL
    assert sc(ws=None) == SPEC_EWORKSPACE
    assert sc(wsb=8) == SPEC_EWORKSPACE
    assert sc(ws=p(0x10004)) == SPEC_EWORKSPACE        # misaligned
    assert sc(R=0) == SPEC_OK


def test_sts_argument_validation(lib):
    p = ctypes.c_void_p
    fake = p(0x1000)
    i = ctypes.c_int
    w = lib.spec_sts_workspace_bytes
    w.restype = ctypes.c_size_t
    w.argtypes = [i, i, i, i]
    f = lib.spec_sts_calibrate
    f.restype = i
    f.argtypes = [p, p, p, i, i, i, i, p, p, p, p, ctypes.c_size_t, p]
    need = w(4096, 7, 64, 15)
    # a_prev (8 N) + tile sums (8 G bins tiles) + sums (8 G bins) + control
    assert need >= 8 * 4096 + 8 * 64 * 15 * 8 + 8 * 64 * 15 + 256
    assert w(4096, 7, 64, 25) == 0 and w(4096, 7, 1025, 15) == 0 and w(0, 7, 64, 15) == 0
    assert w((1 << 24) + 1, 7, 64, 15) == 0

    def sc(**kw):
        a = dict(z=fake, A=fake, g=fake, N=4096, gamma=7, G=64, bins=15, t=fake, e=fake,
                 curve=None, ws=p(0x10000), wsb=need)
        a.update(kw)
        return f(a["z"], a["A"], a["g"], a["N"], a["gamma"], a["G"], a["bins"], a["t"], a["e"],
                 a["curve"], a["ws"], a["wsb"], None)

    assert sc(N=-1) == SPEC_EINVAL
    assert sc(gamma=-1) == SPEC_EINVAL
    assert sc(G=0) == SPEC_EINVAL
    assert sc(bins=0) == SPEC_EINVAL
    assert sc(G=1025) == SPEC_EUNSUPPORTED
    assert sc(bins=25) == SPEC_EUNSUPPORTED
    assert sc(N=0) == SPEC_OK and sc(gamma=0) == SPEC_OK
    assert sc(z=None) == SPEC_EINVAL
    assert sc(A=None) == SPEC_EINVAL
    assert sc(g=None) == SPEC_EINVAL
    assert sc(t=None) == SPEC_EINVAL
    assert sc(e=None) == SPEC_EINVAL
    assert sc(ws=None) == SPEC_EWORKSPACE
    assert sc(ws=p(0x10008)) == SPEC_EWORKSPACE
    assert sc(wsb=need - 1) == SPEC_EWORKSPACE


def test_tree_argument_validation(lib):
    p = ctypes.c_void_p
    fake = p(0x1000)
    i = ctypes.c_int
    w = lib.spec_tree_workspace_bytes
    w.restype = ctypes.c_size_t
    w.argtypes = [i, i, i]
    f = lib.spec_tree_verify
    f.restype = i
    f.argtypes = [p, i, p, p, p, i, i, i, i, p, p, p, p, ctypes.c_size_t, p]
    need = w(64, 32, 151936)
    # status word, then per request and level: node, argmax word, fault flag
    assert need >= 256 + 64 * 32 * (4 + 8 + 4)
    assert w(64, 1025, 1000) == 0 and w(64, 32, 262145) == 0 and w(0, 32, 1000) == 0

    def tv(**kw):
        a = dict(L=fake, dt=1, P=fake, X=fake, n=fake, R=64, M=32, V=151936, D=6, acc=fake,
                 path=fake, tok=fake, ws=p(0x10000), wsb=need)
        a.update(kw)
        return f(a["L"], a["dt"], a["P"], a["X"], a["n"], a["R"], a["M"], a["V"], a["D"],
                 a["acc"], a["path"], a["tok"], a["ws"], a["wsb"], None)

    assert tv(R=-1) == SPEC_EINVAL
    assert tv(M=0) == SPEC_EINVAL
    assert tv(V=0) == SPEC_EINVAL
    assert tv(D=-1) == SPEC_EINVAL
    assert tv(dt=7) == SPEC_EDTYPE
    assert tv(M=1025) == SPEC_EUNSUPPORTED
    assert tv(V=262145) == SPEC_EUNSUPPORTED
    assert tv(D=32) == SPEC_EUNSUPPORTED          # a depth of M is impossible
    assert tv(R=0) == SPEC_OK
    for k in ("L", "P", "X", "n", "acc", "path", "tok"):
        assert tv(**{k: None}) == SPEC_EINVAL, k
    assert tv(ws=None) == SPEC_EWORKSPACE
    assert tv(ws=p(0x10010)) == SPEC_EWORKSPACE
    # max_depth 6 needs 7 levels: 256 + 64 * 7 * 16 + 256 bytes
    assert tv(wsb=256 + 64 * 7 * 16 + 255) == SPEC_EWORKSPACE


def test_workspace_init_validation(lib):
    f = lib.spec_workspace_init
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert f(None, 1024, None) == SPEC_EWORKSPACE
    assert f(ctypes.c_void_p(0x10010), 1024, None) == SPEC_EWORKSPACE
    assert f(ctypes.c_void_p(0x10000), 16, None) == SPEC_EWORKSPACE


def test_noalloc_size_limits(lib):
    """The no-allocation verify rejects, before any HIP call, sizes whose
    workspace exceeds its fixed scratch, and invalid sizes as spec_verify_batch
    does."""
    p = ctypes.c_void_p
    fake = p(0x1000)
    f = lib.spec_verify_batch_noalloc
    f.restype = ctypes.c_int
    f.argtypes = [p, ctypes.c_int, p, ctypes.c_int, p, p, p, p, p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, p, p, p, p, p, p]
    w = lib.spec_verify_workspace_bytes
    w.restype = ctypes.c_size_t

    def call(R, gamma, V):
        return f(fake, 1, fake, 1, fake, fake, fake, fake, fake, R, gamma, V, fake, fake, None,
                 None, None, None)

    # the largest batched shapes of the workloads fit; twice the 256-request
    # high-load batch at V = 151936 does not
    assert w(256, 7, 129280) <= NOALLOC_SCRATCH and w(64, 7, 151936) <= NOALLOC_SCRATCH
    assert w(512, 7, 151936) > NOALLOC_SCRATCH
    assert call(512, 7, 151936) == SPEC_ETOOLARGE
    assert call(64, 64, 262144) == SPEC_ETOOLARGE
    assert call(-1, 7, 100) == SPEC_EINVAL
    assert call(4, 7, 0) == SPEC_EINVAL
    assert call(4, 65, 100) == SPEC_EUNSUPPORTED
    assert call(0, 7, 100) == SPEC_OK


def test_timing_hook_arguments(lib):
    """spec_time_stats_launch validates its arguments on the host; n = 0 (stop)
    needs no arrays.  Nothing is recorded without a verification call."""
    p = ctypes.c_void_p
    f = lib.spec_time_stats_launch
    f.restype = ctypes.c_int
    f.argtypes = [p, p, ctypes.c_int]
    arr = (p * 2)(p(0x1000), p(0x2000))
    assert f(None, None, 0) == SPEC_OK
    assert f(arr, arr, -1) == SPEC_EINVAL
    assert f(None, arr, 2) == SPEC_EINVAL
    assert f(arr, None, 2) == SPEC_EINVAL
    assert f(arr, arr, 2) == SPEC_OK
    assert f(None, None, 0) == SPEC_OK


def test_verify_path_host_checks(lib):
    """spec_verify_path: invalid shapes are refused; fp32 rows, a vocabulary
    that is not a multiple of 8 and an empty batch take the split path (all
    decided before any HIP call)."""
    f = lib.spec_verify_path
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int] * 5
    F32, BF16 = 0, 1
    assert f(-1, 7, 151936, BF16, BF16) == -1
    assert f(64, 7, 0, BF16, BF16) == -1
    assert f(64, 7, 151936, 7, BF16) == -2
    assert f(64, 7, 262144 + 1, BF16, BF16) == -5   # past SPEC_MAX_VERIFY_VOCAB
    assert f(64, 7, 151936, F32, F32) == 0
    assert f(64, 7, 151936, BF16, F32) == 0
    assert f(64, 7, 151937, BF16, BF16) == 0
    assert f(0, 7, 151936, BF16, BF16) == 0
