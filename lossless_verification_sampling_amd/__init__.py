"""Python binding of libspecverify (batched lossless speculative-sampling
verification and the Markov-head draft on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/specverify.h.  The functions keep
the C names.  Tensors must be contiguous CUDA (HIP) tensors on one device;
logits are torch.float32 or torch.bfloat16.  Work is enqueued on the current
torch stream and nothing synchronises except spec_get_device_status.

The library must have been built (``python -m
lossless_verification_sampling_amd._build`` or ``__graft_entry__.build()``);
importing this module without it raises, there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecverify.so")

SPEC_F32, SPEC_BF16 = 0, 1
SPEC_OK = 0
SPEC_ETOOLARGE = -6
SPEC_NOALLOC_SCRATCH_BYTES = 32 << 20
SPEC_DEV_BAD_REQUEST = 0x1
SPEC_DEV_SPIN_TIMEOUT = 0x2
SPEC_MAX_VOCAB = 2097152
SPEC_MAX_VERIFY_VOCAB = 262144
SPEC_SCHED_MAX_POOL = 8192
SPEC_RNN_MAX_HIDDEN = 3072
SPEC_STS_MAX_BINS = 24
SPEC_STS_MAX_GRID = 1024
SPEC_STS_MAX_BLOCKS = 1 << 24
SPEC_TREE_MAX_NODES = 1024
SPEC_PATH_SPLIT, SPEC_PATH_HELD = 0, 1

EXPORTED = (
    "spec_version",
    "spec_status_string",
    "spec_verify_workspace_bytes",
    "spec_verify_path",
    "spec_workspace_init",
    "spec_verify_batch",
    "spec_verify_batch_noalloc",
    "spec_tv_workspace_bytes",
    "spec_tv_accept_rate",
    "spec_markov_workspace_bytes",
    "spec_rnn_workspace_bytes",
    "spec_rnn_draft_sample",
    "spec_schedule_workspace_bytes",
    "spec_schedule_verify_len",
    "spec_sts_workspace_bytes",
    "spec_sts_calibrate",
    "spec_tree_workspace_bytes",
    "spec_tree_verify",
    "spec_markov_draft_sample",
    "spec_get_device_status",
    "spec_time_stats_launch",
)


class SpecError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {spec_status_string(status)} ({status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                          "(python -m lossless_verification_sampling_amd._build)")
    lib = ctypes.CDLL(LIB_PATH)
    p, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.spec_version.restype = i
    lib.spec_version.argtypes = []
    lib.spec_status_string.restype = ctypes.c_char_p
    lib.spec_status_string.argtypes = [i]
    lib.spec_verify_workspace_bytes.restype = sz
    lib.spec_verify_workspace_bytes.argtypes = [i, i, i]
    lib.spec_verify_path.restype = i
    lib.spec_verify_path.argtypes = [i, i, i, i, i]
    lib.spec_tv_workspace_bytes.restype = sz
    lib.spec_tv_workspace_bytes.argtypes = [i, i]
    lib.spec_markov_workspace_bytes.restype = sz
    lib.spec_markov_workspace_bytes.argtypes = [i, i, i, i]
    lib.spec_workspace_init.restype = i
    lib.spec_workspace_init.argtypes = [p, sz, p]
    lib.spec_verify_batch.restype = i
    lib.spec_verify_batch.argtypes = [p, i, p, i, p, p, p, p, p, i, i, i, p, p, p, p, p, p, sz, p]
    lib.spec_time_stats_launch.restype = i
    lib.spec_time_stats_launch.argtypes = [p, p, i]
    lib.spec_verify_batch_noalloc.restype = i
    lib.spec_verify_batch_noalloc.argtypes = [p, i, p, i, p, p, p, p, p, i, i, i, p, p, p, p, p,
                                              p]
    lib.spec_tv_accept_rate.restype = i
    lib.spec_tv_accept_rate.argtypes = [p, p, i, p, i, i, p, p, p, sz, p]
    lib.spec_markov_draft_sample.restype = i
    lib.spec_markov_draft_sample.argtypes = [p, i, p, p, i, p, p, p, i, i, i, i, p, p, p, sz, p]
    lib.spec_rnn_workspace_bytes.restype = sz
    lib.spec_rnn_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.spec_rnn_draft_sample.restype = i
    lib.spec_rnn_draft_sample.argtypes = [p, i, p, p, i, p, i, p, p, p, p, p, i, i, i, i, p, p, p,
                                          p, sz, p]
    lib.spec_schedule_workspace_bytes.restype = sz
    lib.spec_schedule_workspace_bytes.argtypes = []
    lib.spec_schedule_verify_len.restype = i
    lib.spec_schedule_verify_len.argtypes = [p, p, i, i, i, i, p, p, p, sz, p]
    lib.spec_sts_workspace_bytes.restype = sz
    lib.spec_sts_workspace_bytes.argtypes = [i, i, i, i]
    lib.spec_sts_calibrate.restype = i
    lib.spec_sts_calibrate.argtypes = [p, p, p, i, i, i, i, p, p, p, p, sz, p]
    lib.spec_tree_workspace_bytes.restype = sz
    lib.spec_tree_workspace_bytes.argtypes = [i, i, i]
    lib.spec_tree_verify.restype = i
    lib.spec_tree_verify.argtypes = [p, i, p, p, p, i, i, i, i, p, p, p, p, sz, p]
    lib.spec_get_device_status.restype = i
    lib.spec_get_device_status.argtypes = [p, ctypes.POINTER(ctypes.c_uint32), i, p]
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib


def spec_version() -> int:
    return int(_lib.spec_version())


def spec_status_string(status: int) -> str:
    return _lib.spec_status_string(int(status)).decode()


def spec_verify_workspace_bytes(R: int, gamma: int, V: int) -> int:
    return int(_lib.spec_verify_workspace_bytes(R, gamma, V))


def spec_verify_path(R: int, gamma: int, V: int, target_dtype, draft_dtype) -> int:
    """SPEC_PATH_HELD or SPEC_PATH_SPLIT: the launch sequence a
    spec_verify_batch call of this shape takes on the current device (16-byte
    aligned rows); dtypes as torch dtypes or SPEC_F32 / SPEC_BF16."""
    def code(d):
        if isinstance(d, torch.dtype):
            return SPEC_BF16 if d == torch.bfloat16 else SPEC_F32
        return int(d)
    st = int(_lib.spec_verify_path(R, gamma, V, code(target_dtype), code(draft_dtype)))
    if st < 0:
        _raise(st, "spec_verify_path")
    return st


def spec_tv_workspace_bytes(N: int, V: int) -> int:
    return int(_lib.spec_tv_workspace_bytes(N, V))


def spec_markov_workspace_bytes(R: int, gamma: int, V: int, rank: int) -> int:
    return int(_lib.spec_markov_workspace_bytes(R, gamma, V, rank))


def spec_rnn_workspace_bytes(R: int, gamma: int, V: int, rank: int, hidden: int) -> int:
    return int(_lib.spec_rnn_workspace_bytes(R, gamma, V, rank, hidden))


def spec_schedule_workspace_bytes() -> int:
    return int(_lib.spec_schedule_workspace_bytes())


def spec_sts_workspace_bytes(N: int, gamma: int, G: int, bins: int) -> int:
    return int(_lib.spec_sts_workspace_bytes(N, gamma, G, bins))


def spec_tree_workspace_bytes(R: int, M: int, V: int) -> int:
    return int(_lib.spec_tree_workspace_bytes(R, M, V))


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _stream_ptr(stream: Optional[torch.cuda.Stream], device) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SPEC_F32
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _check(t: Optional[torch.Tensor], name: str, dtype=None, shape=None, device=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _raise(status: int, what: str):
    if status != SPEC_OK:
        raise SpecError(status, what)


class Workspace:
    """A device buffer for the library's cross-workgroup exchange, initialised
    once with spec_workspace_init and grown on demand.  Calls that share a
    workspace must be stream-ordered."""

    def __init__(self, device=None, nbytes: int = 0):
        self.device = torch.device(device if device is not None else "cuda")
        self.buf: Optional[torch.Tensor] = None
        if nbytes:
            self.ensure(nbytes)

    def ensure(self, nbytes: int, stream=None) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            n = max(int(nbytes), 1 << 16)
            n = (n + 255) // 256 * 256
            self.buf = torch.empty(n, dtype=torch.uint8, device=self.device)
            _raise(_lib.spec_workspace_init(_ptr(self.buf), n, _stream_ptr(stream, self.device)),
                   "spec_workspace_init")
        return self.buf

    @property
    def nbytes(self) -> int:
        return 0 if self.buf is None else self.buf.numel()


_default_ws = {}


def default_workspace(device) -> Workspace:
    device = torch.device(device)
    key = (device.type, device.index if device.index is not None else torch.cuda.current_device())
    ws = _default_ws.get(key)
    if ws is None:
        ws = Workspace(torch.device("cuda", key[1]))
        _default_ws[key] = ws
    return ws


def spec_workspace_init(workspace: Workspace, stream=None) -> None:
    buf = workspace.buf
    if buf is None:
        return
    _raise(_lib.spec_workspace_init(_ptr(buf), buf.numel(), _stream_ptr(stream, buf.device)),
           "spec_workspace_init")


def spec_get_device_status(workspace: Workspace, clear: bool = True, stream=None) -> int:
    """Synchronises the stream and returns the OR of SPEC_DEV_* bits."""
    bits = ctypes.c_uint32(0)
    buf = workspace.buf
    if buf is None:
        return 0
    _raise(_lib.spec_get_device_status(_ptr(buf), ctypes.byref(bits), int(clear),
                                       _stream_ptr(stream, buf.device)),
           "spec_get_device_status")
    return int(bits.value)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def _verify_io(target_logits, draft_logits, draft_tokens, verify_len, temperature, u_accept,
               u_sample, out, want_cstar, want_resid, want_logq):
    """Checks the inputs of a verification call and returns (R, gamma, V, outputs)
    with the missing output tensors allocated."""
    R, G1, V = target_logits.shape
    gamma = G1 - 1
    dev = target_logits.device
    _check(target_logits, "target_logits", device=dev)
    _check(draft_logits, "draft_logits", shape=(R, gamma, V), device=dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (R, gamma), dev)
    _check(verify_len, "verify_len", torch.int32, (R,), dev)
    _check(temperature, "temperature", torch.float32, (R,), dev)
    _check(u_accept, "u_accept", torch.float32, (R, gamma), dev)
    _check(u_sample, "u_sample", torch.float32, (R, G1), dev)
    if out is None:
        out = {}
    o_tok = out.get("tokens")
    if o_tok is None:
        o_tok = torch.empty((R, G1), dtype=torch.int32, device=dev)
    o_n = out.get("num_accepted")
    if o_n is None:
        o_n = torch.empty((R,), dtype=torch.int32, device=dev)
    o_cs = out.get("cstar")
    if o_cs is None and want_cstar:
        o_cs = torch.empty((R, gamma), dtype=torch.float32, device=dev)
    o_rs = out.get("resid_mass")
    if o_rs is None and want_resid:
        o_rs = torch.empty((R, gamma), dtype=torch.float32, device=dev)
    o_lq = out.get("logq")
    if o_lq is None and want_logq:
        o_lq = torch.empty((R, G1), dtype=torch.float32, device=dev)
    _check(o_tok, "out tokens", torch.int32, (R, G1), dev)
    _check(o_n, "out num_accepted", torch.int32, (R,), dev)
    _check(o_cs, "out cstar", torch.float32, (R, gamma), dev)
    _check(o_rs, "out resid_mass", torch.float32, (R, gamma), dev)
    _check(o_lq, "out logq", torch.float32, (R, G1), dev)
    return R, gamma, V, dict(tokens=o_tok, num_accepted=o_n, cstar=o_cs, resid_mass=o_rs,
                             logq=o_lq)


def spec_verify_batch(target_logits: torch.Tensor, draft_logits: Optional[torch.Tensor],
                      draft_tokens: Optional[torch.Tensor], verify_len: torch.Tensor,
                      temperature: torch.Tensor, u_accept: Optional[torch.Tensor],
                      u_sample: torch.Tensor, *, out: Optional[dict] = None,
                      want_cstar: bool = True, want_resid: bool = True, want_logq: bool = True,
                      workspace: Optional[Workspace] = None, stream=None) -> dict:
    """Batched verification.  target_logits [R, gamma+1, V], draft_logits
    [R, gamma, V] (float32 / bfloat16), draft_tokens [R, gamma] int32,
    verify_len [R] int32, temperature [R] float32, u_accept [R, gamma] and
    u_sample [R, gamma+1] float32.  Returns dict(tokens, num_accepted, cstar,
    resid_mass, logq); `out` may supply preallocated output tensors."""
    R, gamma, V, o = _verify_io(target_logits, draft_logits, draft_tokens, verify_len,
                                temperature, u_accept, u_sample, out, want_cstar, want_resid,
                                want_logq)
    dev = target_logits.device
    ws = workspace or default_workspace(dev)
    need = spec_verify_workspace_bytes(R, gamma, V)
    if need == 0:
        raise SpecError(-5, "spec_verify_workspace_bytes")
    buf = ws.ensure(need, stream)
    d_dtype = _dtype(draft_logits) if draft_logits is not None else SPEC_F32
    st = _lib.spec_verify_batch(_ptr(target_logits), _dtype(target_logits), _ptr(draft_logits),
                                d_dtype, _ptr(draft_tokens), _ptr(verify_len), _ptr(temperature),
                                _ptr(u_accept), _ptr(u_sample), R, gamma, V, _ptr(o["tokens"]),
                                _ptr(o["num_accepted"]), _ptr(o["cstar"]),
                                _ptr(o["resid_mass"]), _ptr(o["logq"]), _ptr(buf),
                                buf.numel(), _stream_ptr(stream, dev))
    _raise(st, "spec_verify_batch")
    return o


def spec_verify_batch_noalloc(target_logits: torch.Tensor, draft_logits: Optional[torch.Tensor],
                              draft_tokens: Optional[torch.Tensor], verify_len: torch.Tensor,
                              temperature: torch.Tensor, u_accept: Optional[torch.Tensor],
                              u_sample: torch.Tensor, *, out: dict, stream=None) -> dict:
    """spec_verify_batch on the library's fixed per-device scratch instead of
    a workspace (no allocation in the library).  `out` must hold every output
    tensor the call writes (tokens, num_accepted; cstar, resid_mass, logq or
    None), so that the call allocates nothing here either."""
    for k in ("tokens", "num_accepted", "cstar", "resid_mass", "logq"):
        if k not in out:
            raise ValueError(f"spec_verify_batch_noalloc: out[{k!r}] must be given "
                             "(a tensor, or None for an optional output)")
    R, gamma, V, o = _verify_io(target_logits, draft_logits, draft_tokens, verify_len,
                                temperature, u_accept, u_sample, out, False, False, False)
    dev = target_logits.device
    d_dtype = _dtype(draft_logits) if draft_logits is not None else SPEC_F32
    st = _lib.spec_verify_batch_noalloc(_ptr(target_logits), _dtype(target_logits),
                                        _ptr(draft_logits), d_dtype, _ptr(draft_tokens),
                                        _ptr(verify_len), _ptr(temperature), _ptr(u_accept),
                                        _ptr(u_sample), R, gamma, V, _ptr(o["tokens"]),
                                        _ptr(o["num_accepted"]), _ptr(o["cstar"]),
                                        _ptr(o["resid_mass"]), _ptr(o["logq"]),
                                        _stream_ptr(stream, dev))
    _raise(st, "spec_verify_batch_noalloc")
    return o


def spec_time_stats_launch(before, after) -> None:
    """Times the statistics launch of the calling thread's next len(before)
    verification calls: `before` and `after` are sequences of hipEvent_t
    handles (ints) that the library records around that launch.  The arrays
    are kept alive here until the next call of this function."""
    global _timing_arrays
    n = len(before)
    if len(after) != n:
        raise ValueError("spec_time_stats_launch: before and after differ in length")
    arr_t = ctypes.c_void_p * max(n, 1)
    _timing_arrays = (arr_t(*before), arr_t(*after))
    _raise(_lib.spec_time_stats_launch(_timing_arrays[0], _timing_arrays[1], n),
           "spec_time_stats_launch")


_timing_arrays = None


def spec_tv_accept_rate(draft_logits: torch.Tensor, target_logits: torch.Tensor,
                        temperature: torch.Tensor, *, want_resid: bool = True,
                        workspace: Optional[Workspace] = None, stream=None):
    """c* and Res of N row pairs [N, V]; returns (cstar [N], resid_mass [N] or None)."""
    N, V = target_logits.shape
    dev = target_logits.device
    _check(target_logits, "target_logits", device=dev)
    _check(draft_logits, "draft_logits", target_logits.dtype, (N, V), dev)
    _check(temperature, "temperature", torch.float32, (N,), dev)
    cs = torch.empty((N,), dtype=torch.float32, device=dev)
    rs = torch.empty((N,), dtype=torch.float32, device=dev) if want_resid else None
    ws = workspace or default_workspace(dev)
    need = spec_tv_workspace_bytes(N, V)
    if need == 0:
        raise SpecError(-5, "spec_tv_workspace_bytes")
    buf = ws.ensure(need, stream)
    st = _lib.spec_tv_accept_rate(_ptr(draft_logits), _ptr(target_logits), _dtype(target_logits),
                                  _ptr(temperature), N, V, _ptr(cs), _ptr(rs), _ptr(buf),
                                  buf.numel(), _stream_ptr(stream, dev))
    _raise(st, "spec_tv_accept_rate")
    return cs, rs


def spec_schedule_verify_len(confidence: torch.Tensor, sps: torch.Tensor, *, topk: int = -1,
                             out_len: Optional[torch.Tensor] = None,
                             out_theta: Optional[torch.Tensor] = None,
                             workspace: Optional[Workspace] = None, stream=None):
    """Confidence-scheduled verify lengths.  confidence [R, gamma] float32 in
    [0, 1], sps [bmax + 1] float32 (steps per second at batch size B).  topk < 0:
    greedy admission with early stop; topk >= 0: the top-K variant.  Returns
    (lengths [R] int32, theta [1] float64)."""
    R, gamma = confidence.shape
    dev = confidence.device
    _check(confidence, "confidence", torch.float32, (R, gamma), dev)
    _check(sps, "sps", torch.float32, None, dev)
    if sps.dim() != 1 or sps.numel() < 1:
        raise ValueError("sps must be a non-empty 1-D table")
    ln = out_len if out_len is not None else torch.empty((R,), dtype=torch.int32, device=dev)
    th = out_theta if out_theta is not None else torch.empty((1,), dtype=torch.float64, device=dev)
    _check(ln, "out_len", torch.int32, (R,), dev)
    _check(th, "out_theta", torch.float64, (1,), dev)
    ws = workspace or default_workspace(dev)
    buf = ws.ensure(spec_schedule_workspace_bytes(), stream)
    st = _lib.spec_schedule_verify_len(_ptr(confidence), _ptr(sps), R, gamma, sps.numel() - 1,
                                       int(topk), _ptr(ln), _ptr(th), _ptr(buf), buf.numel(),
                                       _stream_ptr(stream, dev))
    _raise(st, "spec_schedule_verify_len")
    return ln, th


def spec_sts_calibrate(conf_logits: torch.Tensor, accepted_len: torch.Tensor, grid: torch.Tensor,
                       *, bins: int = 15, want_curve: bool = False,
                       workspace: Optional[Workspace] = None, stream=None):
    """Sequential temperature scaling of the confidence head on a held-out
    set.  conf_logits [N, gamma] float32 raw logits, accepted_len [N] int32
    (accepted prefix length per block), grid [G] float64 candidate
    temperatures.  Returns (temperatures [gamma] float64, ece [gamma] float64,
    curves [gamma, G] float64 or None)."""
    N, gamma = conf_logits.shape
    G = grid.numel()
    dev = conf_logits.device
    _check(conf_logits, "conf_logits", torch.float32, (N, gamma), dev)
    _check(accepted_len, "accepted_len", torch.int32, (N,), dev)
    _check(grid, "grid", torch.float64, (G,), dev)
    temps = torch.empty((gamma,), dtype=torch.float64, device=dev)
    ece = torch.empty((gamma,), dtype=torch.float64, device=dev)
    curve = torch.empty((gamma, G), dtype=torch.float64, device=dev) if want_curve else None
    need = spec_sts_workspace_bytes(max(N, 1), gamma, G, bins)
    if need == 0:
        raise ValueError(f"spec_sts_calibrate: unsupported sizes N={N} G={G} bins={bins}")
    ws = workspace or default_workspace(dev)
    buf = ws.ensure(need, stream)
    st = _lib.spec_sts_calibrate(_ptr(conf_logits), _ptr(accepted_len), _ptr(grid), N, gamma, G,
                                 int(bins), _ptr(temps), _ptr(ece),
                                 _ptr(curve) if curve is not None else None, _ptr(buf),
                                 buf.numel(), _stream_ptr(stream, dev))
    _raise(st, "spec_sts_calibrate")
    return temps, ece, curve


def spec_tree_verify(logits: torch.Tensor, parent: torch.Tensor, tokens: torch.Tensor,
                     n_nodes: torch.Tensor, max_depth: int, *,
                     workspace: Optional[Workspace] = None, stream=None):
    """Greedy (T = 0) tree verification.  logits [R, M, V] float32 or
    bfloat16 (row v: the target's next-token logits after the path to node v),
    parent / tokens [R, M] int32, n_nodes [R] int32, max_depth a bound on every
    tree's depth (deeper trees are rejected).  Returns (accepted [R], path [R, M], committed tokens [R, M])
    as int32."""
    R, M, V = logits.shape
    dev = logits.device
    _check(logits, "logits", logits.dtype, (R, M, V), dev)
    for t, nm in ((parent, "parent"), (tokens, "tokens")):
        _check(t, nm, torch.int32, (R, M), dev)
    _check(n_nodes, "n_nodes", torch.int32, (R,), dev)
    acc = torch.empty((R,), dtype=torch.int32, device=dev)
    path = torch.empty((R, M), dtype=torch.int32, device=dev)
    tok = torch.empty((R, M), dtype=torch.int32, device=dev)
    need = spec_tree_workspace_bytes(max(R, 1), M, V)
    if need == 0:
        raise ValueError(f"spec_tree_verify: unsupported sizes M={M} V={V}")
    ws = workspace or default_workspace(dev)
    buf = ws.ensure(need, stream)
    st = _lib.spec_tree_verify(_ptr(logits), _dtype(logits), _ptr(parent), _ptr(tokens),
                               _ptr(n_nodes), R, M, V, int(max_depth), _ptr(acc), _ptr(path),
                               _ptr(tok), _ptr(buf), buf.numel(), _stream_ptr(stream, dev))
    _raise(st, "spec_tree_verify")
    return acc, path, tok


def spec_rnn_draft_sample(U: torch.Tensor, W1: torch.Tensor, W2: torch.Tensor,
                          hidden_states: torch.Tensor, Wg: torch.Tensor, bg: torch.Tensor,
                          anchor: torch.Tensor, temperature: torch.Tensor, u_draft: torch.Tensor,
                          *, want_state: bool = False, out_tokens: Optional[torch.Tensor] = None,
                          out_logits: Optional[torch.Tensor] = None,
                          workspace: Optional[Workspace] = None, stream=None):
    """RNN-head draft.  As spec_markov_draft_sample plus hidden_states
    [R, gamma, hidden] float32, Wg [2 rank + hidden, 2 rank] bfloat16, bg
    [2 rank] float32.  Returns (tokens, logits, states [R, gamma, rank] float32
    or None)."""
    R, gamma, V = U.shape
    rank = W1.shape[1]
    hidden = hidden_states.shape[2]
    dev = U.device
    _check(U, "U", device=dev)
    _check(W1, "W1", torch.bfloat16, (V, rank), dev)
    _check(W2, "W2", torch.bfloat16, (rank, V), dev)
    _check(hidden_states, "hidden_states", torch.float32, (R, gamma, hidden), dev)
    _check(Wg, "Wg", torch.bfloat16, (2 * rank + hidden, 2 * rank), dev)
    _check(bg, "bg", torch.float32, (2 * rank,), dev)
    _check(anchor, "anchor", torch.int32, (R,), dev)
    _check(temperature, "temperature", torch.float32, (R,), dev)
    _check(u_draft, "u_draft", torch.float32, (R, gamma), dev)
    tok = out_tokens if out_tokens is not None else torch.empty((R, gamma), dtype=torch.int32,
                                                                 device=dev)
    lg = out_logits if out_logits is not None else torch.empty((R, gamma, V),
                                                                dtype=torch.float32, device=dev)
    stt = torch.empty((R, gamma, rank), dtype=torch.float32, device=dev) if want_state else None
    _check(tok, "out_tokens", torch.int32, (R, gamma), dev)
    _check(lg, "out_logits", torch.float32, (R, gamma, V), dev)
    ws = workspace or default_workspace(dev)
    need = spec_rnn_workspace_bytes(R, gamma, V, rank, hidden)
    if need == 0:
        raise SpecError(-5, "spec_rnn_workspace_bytes")
    buf = ws.ensure(need, stream)
    st = _lib.spec_rnn_draft_sample(_ptr(U), _dtype(U), _ptr(W1), _ptr(W2), SPEC_BF16,
                                    _ptr(hidden_states), hidden, _ptr(Wg), _ptr(bg), _ptr(anchor),
                                    _ptr(temperature), _ptr(u_draft), R, gamma, V, rank, _ptr(tok),
                                    _ptr(lg), _ptr(stt), _ptr(buf), buf.numel(),
                                    _stream_ptr(stream, dev))
    _raise(st, "spec_rnn_draft_sample")
    return tok, lg, stt


def spec_markov_draft_sample(U: torch.Tensor, W1: torch.Tensor, W2: torch.Tensor,
                             anchor: torch.Tensor, temperature: torch.Tensor,
                             u_draft: torch.Tensor, *, out_tokens: Optional[torch.Tensor] = None,
                             out_logits: Optional[torch.Tensor] = None,
                             workspace: Optional[Workspace] = None, stream=None):
    """Markov-head draft.  U [R, gamma, V] (float32 / bfloat16), W1 [V, rank],
    W2 [rank, V] bfloat16, anchor [R] int32, temperature [R], u_draft
    [R, gamma] float32.  Returns (tokens [R, gamma] int32, logits [R, gamma, V]
    float32)."""
    R, gamma, V = U.shape
    rank = W1.shape[1]
    dev = U.device
    _check(U, "U", device=dev)
    _check(W1, "W1", torch.bfloat16, (V, rank), dev)
    _check(W2, "W2", torch.bfloat16, (rank, V), dev)
    _check(anchor, "anchor", torch.int32, (R,), dev)
    _check(temperature, "temperature", torch.float32, (R,), dev)
    _check(u_draft, "u_draft", torch.float32, (R, gamma), dev)
    tok = out_tokens if out_tokens is not None else torch.empty((R, gamma), dtype=torch.int32,
                                                                 device=dev)
    lg = out_logits if out_logits is not None else torch.empty((R, gamma, V),
                                                                dtype=torch.float32, device=dev)
    _check(tok, "out_tokens", torch.int32, (R, gamma), dev)
    _check(lg, "out_logits", torch.float32, (R, gamma, V), dev)
    ws = workspace or default_workspace(dev)
    need = spec_markov_workspace_bytes(R, gamma, V, rank)
    if need == 0:
        raise SpecError(-5, "spec_markov_workspace_bytes")
    buf = ws.ensure(need, stream)
    st = _lib.spec_markov_draft_sample(_ptr(U), _dtype(U), _ptr(W1), _ptr(W2), SPEC_BF16,
                                       _ptr(anchor), _ptr(temperature), _ptr(u_draft), R, gamma,
                                       V, rank, _ptr(tok), _ptr(lg), _ptr(buf), buf.numel(),
                                       _stream_ptr(stream, dev))
    _raise(st, "spec_markov_draft_sample")
    return tok, lg
