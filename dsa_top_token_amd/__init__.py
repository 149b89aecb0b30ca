"""MI355X (gfx950) DSA path: lightning indexer -> top-k -> sparse MQA attention.

A thin ctypes binding over libdsa.so (include/dsa.h). Every step of the path
runs in the library's HIP kernels; this module only checks tensors, builds
the dsa_problem description, allocates outputs and workspace through torch
and passes raw device pointers plus torch's current stream. There is no CPU
fallback: if libdsa.so is missing, every call raises.

Method: the DeepSeek-V3.2 DSA page (kwkr.cn/news/60693), sections 3.2
(indexer score), 3.3 (top-k then attention over the kept keys), 4.1-4.3
(precisions, shared K/V across heads, one fused chain).
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_OK = 0
STATUS = {0: "DSA_OK", -1: "DSA_E_NULL", -2: "DSA_E_SHAPE", -3: "DSA_E_UNSUPPORTED",
          -4: "DSA_E_ALIGN", -5: "DSA_E_WORKSPACE", -6: "DSA_E_HIP"}
IDX_FP8, IDX_BF16 = 0, 1
OP_TOPK, OP_ATTN, OP_FORWARD = 1, 2, 3
HEAD_DIM = 128

EXPORTS = ("dsa_workspace_size", "dsa_index_scores", "dsa_topk", "dsa_sparse_attn",
           "dsa_forward", "dsa_forward_ragged", "dsa_forward_paged", "dsa_forward_timed",
           "dsa_forward_ragged_timed", "dsa_forward_paged_timed", "dsa_forward_threshold",
           "dsa_forward_threshold_timed", "dsa_forward_ext", "dsa_forward_ext_timed",
           "dsa_index_project", "dsa_forward_noalloc", "dsa_status_str", "dsa_last_error")


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "n_q", "n_k", "q_pos0", "d_idx", "idx_dtype", "top_k",
                 "n_heads", "head_dim")]


class Pages(ctypes.Structure):
    """dsa_pages: a paged key layout (block table on the device)."""
    _fields_ = [("block_table", ctypes.c_void_p), ("page_size", ctypes.c_int32),
                ("pages_per_seq", ctypes.c_int32), ("n_pages", ctypes.c_int32)]


class Options(ctypes.Structure):
    """dsa_forward_options: layout and mode of dsa_forward_ext."""
    _fields_ = [("seq_pos", ctypes.c_void_p), ("pages", ctypes.POINTER(Pages)),
                ("threshold_mode", ctypes.c_int32), ("tau", ctypes.c_float)]


class DSAError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__("%s: %s" % (STATUS.get(status, status), detail))
        self.status = status


_lib = None
_lock = threading.Lock()


def load():
    """Load libdsa.so (built in-tree by build.py); raise if it is absent."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    "libdsa.so is not built (%s); run __graft_entry__.build() or "
                    "python dsa_top_token_amd/build.py" % LIB_PATH)
            lib = ctypes.CDLL(LIB_PATH)
            P, I, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
            PP = ctypes.POINTER(Problem)
            lib.dsa_workspace_size.argtypes = [PP, I, ctypes.POINTER(S)]
            lib.dsa_index_scores.argtypes = [PP, P, P, I, I, P, P]
            lib.dsa_topk.argtypes = [PP, P, I, I, P, P, S, P]
            lib.dsa_sparse_attn.argtypes = [PP, P, P, P, P, P, P, P, S, P]
            lib.dsa_forward.argtypes = [PP, P, P, P, P, P, P, P, P, P, S, P]
            lib.dsa_forward_noalloc.argtypes = [PP, P, P, P, P, P, P, P, P, P]
            lib.dsa_forward_ragged.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, S, P]
            lib.dsa_forward_timed.argtypes = [PP, P, P, P, P, P, P, P, P, P, S, P, P, P]
            lib.dsa_forward_ragged_timed.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, S, P, P,
                                                     P]
            PG = ctypes.POINTER(Pages)
            lib.dsa_forward_paged.argtypes = [PP, P, PG, P, P, P, P, P, P, P, P, P, S, P]
            lib.dsa_forward_paged_timed.argtypes = [PP, P, PG, P, P, P, P, P, P, P, P, P, S, P,
                                                    P, P]
            F = ctypes.c_float
            lib.dsa_forward_threshold.argtypes = [PP, F, P, P, P, P, P, P, P, P, P, S, P]
            lib.dsa_forward_threshold_timed.argtypes = [PP, F, P, P, P, P, P, P, P, P, P, S, P,
                                                        P, P]
            PO = ctypes.POINTER(Options)
            lib.dsa_forward_ext.argtypes = [PP, PO, P, P, P, P, P, P, P, P, P, S, P]
            lib.dsa_forward_ext_timed.argtypes = [PP, PO, P, P, P, P, P, P, P, P, P, S, P, P, P]
            lib.dsa_index_project.argtypes = [I, I, I, I, P, P, P, P, I, P]
            for f in (lib.dsa_index_project, lib.dsa_forward_ext, lib.dsa_forward_ext_timed,
                      lib.dsa_workspace_size, lib.dsa_index_scores, lib.dsa_topk,
                      lib.dsa_sparse_attn, lib.dsa_forward, lib.dsa_forward_ragged,
                      lib.dsa_forward_noalloc,
                      lib.dsa_forward_paged, lib.dsa_forward_timed,
                      lib.dsa_forward_ragged_timed, lib.dsa_forward_paged_timed,
                      lib.dsa_forward_threshold, lib.dsa_forward_threshold_timed):
                f.restype = I
            lib.dsa_status_str.argtypes = [I]
            lib.dsa_status_str.restype = ctypes.c_char_p
            lib.dsa_last_error.argtypes = []
            lib.dsa_last_error.restype = ctypes.c_char_p
            _lib = lib
    return _lib


def _check(rc):
    if rc != DSA_OK:
        raise DSAError(rc, load().dsa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def make_problem(batch, n_q, n_k, q_pos0, d_idx, idx_dtype, top_k, n_heads,
                 head_dim=HEAD_DIM) -> Problem:
    if isinstance(idx_dtype, torch.dtype):
        idx_dtype = IDX_FP8 if idx_dtype == torch.float8_e4m3fn else IDX_BF16
    elif isinstance(idx_dtype, str):
        idx_dtype = {"fp8": IDX_FP8, "bf16": IDX_BF16}[idx_dtype]
    return Problem(batch, n_q, n_k, q_pos0, d_idx, idx_dtype, top_k, n_heads, head_dim)


def workspace_size(p: Problem, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().dsa_workspace_size(ctypes.byref(p), op, ctypes.byref(n)))
    return n.value


def _dev_tensor(t, name, dtypes, ndim):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %d-d tensor" % (name, ndim))
    return t


_IDX_DTYPES = (torch.float8_e4m3fn, torch.bfloat16)


def selection_stats(p: Problem, ws, ws_bytes, seq_pos=None):
    """Diagnostics of the last forward call on this problem and workspace
    (dsa_internal_selection_stats, not part of the public interface; it
    synchronises the device): (rows longer than top_k, candidates kept for
    them, rows recomputed by a fallback, rows whose lists overflowed)."""
    lib = load()
    f = lib.dsa_internal_selection_stats
    f.argtypes = [ctypes.POINTER(Problem), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                  ctypes.c_void_p]
    f.restype = ctypes.c_int32
    out = (ctypes.c_int64 * 4)()
    _check(f(ctypes.byref(p), _ptr(ws), ws_bytes, _ptr(seq_pos), out))
    return tuple(int(v) for v in out)


def _workspace(p, op, dev):
    n = workspace_size(p, op)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=dev), n


def index_scores(q_idx, k_idx, q_pos0, q_begin=0, q_end=None, top_k=1, n_heads=1):
    """Indexer scores [B, q_end-q_begin, n_k] float32 (-inf past each query)."""
    _dev_tensor(q_idx, "q_idx", _IDX_DTYPES, 3)
    _dev_tensor(k_idx, "k_idx", (q_idx.dtype,), 3)
    B, n_q, d = q_idx.shape
    n_k = k_idx.shape[1]
    q_end = n_q if q_end is None else q_end
    p = make_problem(B, n_q, n_k, q_pos0, d, q_idx.dtype, top_k, n_heads)
    out = torch.empty((B, max(q_end - q_begin, 0), n_k), dtype=torch.float32,
                      device=q_idx.device)
    _check(load().dsa_index_scores(ctypes.byref(p), _ptr(q_idx), _ptr(k_idx), q_begin,
                                   q_end, _ptr(out), _stream(q_idx.device)))
    return out


def topk(scores, q_pos0, top_k, n_q=None, q_begin=0, d_idx=32):
    """Top-k indices [B, rows, top_k] int32 (ascending, -1 padded) of score rows
    belonging to queries q_begin.. of sequences with n_q queries at q_pos0."""
    _dev_tensor(scores, "scores", (torch.float32,), 3)
    B, rows, n_k = scores.shape
    n_q = q_begin + rows if n_q is None else n_q
    p = make_problem(B, n_q, n_k, q_pos0, d_idx, IDX_FP8, top_k, 1)
    idx = torch.empty((B, rows, top_k), dtype=torch.int32, device=scores.device)
    ws, n = _workspace(p, OP_TOPK, scores.device)
    _check(load().dsa_topk(ctypes.byref(p), _ptr(scores), q_begin, q_begin + rows,
                           _ptr(idx), _ptr(ws), n, _stream(scores.device)))
    return idx


def sparse_attn(Q, K, V, idx, want_lse=True, q_pos0=None):
    """O [B, n_q, H, 128] bf16 and lse [B, n_q, H] float32 (or None)."""
    _dev_tensor(Q, "Q", (torch.bfloat16,), 4)
    _dev_tensor(K, "K", (torch.bfloat16,), 3)
    _dev_tensor(V, "V", (torch.bfloat16,), 3)
    _dev_tensor(idx, "idx", (torch.int32,), 3)
    B, n_q, H, D = Q.shape
    n_k = K.shape[1]
    top_k = idx.shape[2]
    if q_pos0 is None:
        q_pos0 = n_k - n_q
    p = make_problem(B, n_q, n_k, q_pos0, 32, IDX_FP8, top_k, H, D)
    O = torch.empty_like(Q)
    lse = torch.empty((B, n_q, H), dtype=torch.float32, device=Q.device) if want_lse else None
    ws, n = _workspace(p, OP_ATTN, Q.device)
    _check(load().dsa_sparse_attn(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx),
                                  _ptr(O), _ptr(lse), _ptr(ws), n, _stream(Q.device)))
    return O, lse


def _options(seq_pos, pages, tau):
    """dsa_forward_options for a ragged and/or paged batch in threshold mode."""
    return Options(None if seq_pos is None else seq_pos.data_ptr(),
                   None if pages is None else ctypes.pointer(pages), 1, float(tau))


class Forward:
    """dsa_forward with its workspace allocated once for a fixed problem."""

    def __init__(self, problem: Problem, device):
        self.p = problem
        self.device = torch.device(device)
        self.ws, self.ws_bytes = _workspace(problem, OP_FORWARD, self.device)

    def __call__(self, q_idx, k_idx, Q, K, V, O, idx_out=None, lse=None, seq_pos=None,
                 pages=None, tau=None):
        """seq_pos (int32 [B] on the device): a ragged decode batch through
        dsa_forward_ragged (the problem has n_q = 1 and q_pos0 = 0); with
        pages (a Pages), k_idx, K and V are the page pools
        (dsa_forward_paged); with tau (a float), threshold-mode selection
        (dsa_forward_threshold)."""
        if tau is not None and (seq_pos is not None or pages is not None):
            opt = _options(seq_pos, pages, tau)
            _check(load().dsa_forward_ext(
                ctypes.byref(self.p), ctypes.byref(opt), _ptr(q_idx), _ptr(k_idx), _ptr(Q),
                _ptr(K), _ptr(V), _ptr(idx_out), _ptr(O), _ptr(lse), _ptr(self.ws), self.ws_bytes,
                _stream(self.device)))
            return
        if tau is not None:
            _check(load().dsa_forward_threshold(
                ctypes.byref(self.p), float(tau), _ptr(q_idx), _ptr(k_idx), _ptr(Q), _ptr(K),
                _ptr(V), _ptr(idx_out), _ptr(O), _ptr(lse), _ptr(self.ws), self.ws_bytes,
                _stream(self.device)))
            return
        if pages is not None:
            _check(load().dsa_forward_paged(
                ctypes.byref(self.p), _ptr(seq_pos), ctypes.byref(pages), _ptr(q_idx),
                _ptr(k_idx), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx_out), _ptr(O), _ptr(lse),
                _ptr(self.ws), self.ws_bytes, _stream(self.device)))
            return
        if seq_pos is not None:
            _check(load().dsa_forward_ragged(
                ctypes.byref(self.p), _ptr(seq_pos), _ptr(q_idx), _ptr(k_idx), _ptr(Q), _ptr(K),
                _ptr(V), _ptr(idx_out), _ptr(O), _ptr(lse), _ptr(self.ws), self.ws_bytes,
                _stream(self.device)))
            return
        _check(load().dsa_forward(ctypes.byref(self.p), _ptr(q_idx), _ptr(k_idx), _ptr(Q),
                                  _ptr(K), _ptr(V), _ptr(idx_out), _ptr(O), _ptr(lse),
                                  _ptr(self.ws), self.ws_bytes, _stream(self.device)))

    def timed(self, q_idx, k_idx, Q, K, V, O, idx_out=None, lse=None, seq_pos=None,
              pages=None, tau=None):
        """Run once through dsa_forward_timed (dsa_forward_ragged_timed with
        seq_pos, dsa_forward_paged_timed with pages,
        dsa_forward_threshold_timed with tau); returns ([indexer, top-k,
        attention] milliseconds, number of row slabs). Blocks until done."""
        ms = (ctypes.c_float * 3)()
        slabs = ctypes.c_int32(0)
        if tau is not None and (seq_pos is not None or pages is not None):
            opt = _options(seq_pos, pages, tau)
            _check(load().dsa_forward_ext_timed(
                ctypes.byref(self.p), ctypes.byref(opt), _ptr(q_idx), _ptr(k_idx), _ptr(Q),
                _ptr(K), _ptr(V), _ptr(idx_out), _ptr(O), _ptr(lse), _ptr(self.ws), self.ws_bytes,
                _stream(self.device), ms, ctypes.byref(slabs)))
            return list(ms), slabs.value
        if tau is not None:
            _check(load().dsa_forward_threshold_timed(
                ctypes.byref(self.p), float(tau), _ptr(q_idx), _ptr(k_idx), _ptr(Q), _ptr(K),
                _ptr(V), _ptr(idx_out), _ptr(O), _ptr(lse), _ptr(self.ws), self.ws_bytes,
                _stream(self.device), ms, ctypes.byref(slabs)))
            return list(ms), slabs.value
        if pages is not None:
            _check(load().dsa_forward_paged_timed(
                ctypes.byref(self.p), _ptr(seq_pos), ctypes.byref(pages), _ptr(q_idx),
                _ptr(k_idx), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx_out), _ptr(O), _ptr(lse),
                _ptr(self.ws), self.ws_bytes, _stream(self.device), ms, ctypes.byref(slabs)))
            return list(ms), slabs.value
        if seq_pos is not None:
            _check(load().dsa_forward_ragged_timed(
                ctypes.byref(self.p), _ptr(seq_pos), _ptr(q_idx), _ptr(k_idx), _ptr(Q), _ptr(K),
                _ptr(V), _ptr(idx_out), _ptr(O), _ptr(lse), _ptr(self.ws), self.ws_bytes,
                _stream(self.device), ms, ctypes.byref(slabs)))
            return list(ms), slabs.value
        _check(load().dsa_forward_timed(ctypes.byref(self.p), _ptr(q_idx), _ptr(k_idx),
                                        _ptr(Q), _ptr(K), _ptr(V), _ptr(idx_out), _ptr(O),
                                        _ptr(lse), _ptr(self.ws), self.ws_bytes,
                                        _stream(self.device), ms, ctypes.byref(slabs)))
        return list(ms), slabs.value


def forward(q_idx, k_idx, Q, K, V, q_pos0, top_k, want_idx=True, want_lse=True, seq_pos=None,
            tau=None):
    """The fused chain. Returns (idx [B,n_q,top_k] int32 or None,
    O [B,n_q,H,128] bf16, lse [B,n_q,H] float32 or None). With seq_pos (int32
    [B] on the device; n_q = 1, q_pos0 = 0) the batch is ragged: the query of
    sequence b sits at position seq_pos[b]. With tau the selection runs in
    threshold mode: the keys scoring above tau, at most top_k of them."""
    _dev_tensor(q_idx, "q_idx", _IDX_DTYPES, 3)
    _dev_tensor(k_idx, "k_idx", (q_idx.dtype,), 3)
    _dev_tensor(Q, "Q", (torch.bfloat16,), 4)
    _dev_tensor(K, "K", (torch.bfloat16,), 3)
    _dev_tensor(V, "V", (torch.bfloat16,), 3)
    B, n_q, d = q_idx.shape
    n_k = k_idx.shape[1]
    H = Q.shape[2]
    p = make_problem(B, n_q, n_k, q_pos0, d, q_idx.dtype, top_k, H, Q.shape[3])
    dev = Q.device
    idx = torch.empty((B, n_q, top_k), dtype=torch.int32, device=dev) if want_idx else None
    O = torch.empty_like(Q)
    lse = torch.empty((B, n_q, H), dtype=torch.float32, device=dev) if want_lse else None
    if seq_pos is not None:
        _dev_tensor(seq_pos, "seq_pos", (torch.int32,), 1)
        if seq_pos.shape[0] != B:
            raise ValueError("seq_pos must have one entry per sequence")
    Forward(p, dev)(q_idx, k_idx, Q, K, V, O, idx, lse, seq_pos=seq_pos, tau=tau)
    return idx, O, lse


def forward_noalloc(q_idx, k_idx, Q, K, V, q_pos0, top_k, O, idx=None, lse=None):
    """The fused chain through dsa_forward_noalloc: no workspace, the library's
    static device scratch instead. The caller passes the outputs (O
    [B,n_q,H,128] bf16; idx [B,n_q,top_k] int32 and lse [B,n_q,H] float32 may
    be None), so the call allocates nothing. Calls that overlap on one GPU
    share that scratch and must not run concurrently."""
    _dev_tensor(q_idx, "q_idx", _IDX_DTYPES, 3)
    _dev_tensor(k_idx, "k_idx", (q_idx.dtype,), 3)
    _dev_tensor(Q, "Q", (torch.bfloat16,), 4)
    _dev_tensor(K, "K", (torch.bfloat16,), 3)
    _dev_tensor(V, "V", (torch.bfloat16,), 3)
    _dev_tensor(O, "O", (torch.bfloat16,), 4)
    B, n_q, d = q_idx.shape
    p = make_problem(B, n_q, k_idx.shape[1], q_pos0, d, q_idx.dtype, top_k, Q.shape[2],
                     Q.shape[3])
    if O.shape != Q.shape:
        raise ValueError("O must have Q's shape")
    if idx is not None:
        _dev_tensor(idx, "idx", (torch.int32,), 3)
        if tuple(idx.shape) != (B, n_q, top_k):
            raise ValueError("idx must be [B, n_q, top_k]")
    if lse is not None:
        _dev_tensor(lse, "lse", (torch.float32,), 3)
        if tuple(lse.shape) != (B, n_q, Q.shape[2]):
            raise ValueError("lse must be [B, n_q, H]")
    _check(load().dsa_forward_noalloc(ctypes.byref(p), _ptr(q_idx), _ptr(k_idx), _ptr(Q), _ptr(K),
                                      _ptr(V), _ptr(idx), _ptr(O), _ptr(lse), _stream(Q.device)))
    return idx, O, lse


class Projection:
    """dsa_index_project for fixed sizes (the call needs no workspace)."""

    def __init__(self, rows, d_model, d_idx, device):
        self.rows, self.d_model, self.d_idx = rows, d_model, d_idx
        self.device = torch.device(device)

    def __call__(self, X, W, out, out_rows=None):
        """Encode X . W^T into out ([n_out, d_idx] float8_e4m3fn or bfloat16),
        row out_rows[r] (int32 on the device) or r."""
        dt = {torch.float8_e4m3fn: IDX_FP8, torch.bfloat16: IDX_BF16}[out.dtype]
        _check(load().dsa_index_project(
            self.rows, self.d_model, self.d_idx, dt, _ptr(X), _ptr(W), _ptr(out), _ptr(out_rows),
            out.shape[0], _stream(self.device)))


def index_project(X, W, out_dtype=torch.float8_e4m3fn, out=None, out_rows=None):
    """The indexer projection: encode(fl32(X . W^T)) for X [rows, d_model]
    and W [d_idx, d_model] (bfloat16, on the device), into a new
    [rows, d_idx] tensor or into rows out_rows of `out`. Returns the output."""
    _dev_tensor(X, "X", (torch.bfloat16,), 2)
    _dev_tensor(W, "W", (torch.bfloat16,), 2)
    rows, d_model = X.shape
    d_idx = W.shape[0]
    if W.shape[1] != d_model:
        raise ValueError("W must be [d_idx, d_model]")
    if out is None:
        out = torch.empty((rows, d_idx), dtype=out_dtype, device=X.device)
    _dev_tensor(out, "out", (torch.float8_e4m3fn, torch.bfloat16), 2)
    if out.shape[1] != d_idx:
        raise ValueError("out must have d_idx columns")
    if out_rows is not None:
        _dev_tensor(out_rows, "out_rows", (torch.int32,), 1)
        if out_rows.shape[0] != rows:
            raise ValueError("out_rows needs one entry per input row")
    Projection(rows, d_model, d_idx, X.device)(X, W, out, out_rows)
    return out


def make_pages(block_table, page_size, n_pages) -> Pages:
    """dsa_pages for a block table (int32 [B, pages_per_seq] on the device)."""
    _dev_tensor(block_table, "block_table", (torch.int32,), 2)
    return Pages(block_table.data_ptr(), page_size, block_table.shape[1], n_pages)


def forward_paged(q_idx, k_pool, Q, K_pool, V_pool, block_table, page_size, seq_pos, top_k,
                  want_idx=True, want_lse=True, tau=None):
    """The fused chain over a paged layout (dsa_forward_paged): one query per
    sequence at position seq_pos[b]; k_pool [n_pages, page_size, d_idx], K_pool
    and V_pool [n_pages, page_size, 128]; block_table int32 [B, pages_per_seq].
    With tau, threshold-mode selection (dsa_forward_ext). Returns (idx with
    logical key indices, O, lse) as forward()."""
    _dev_tensor(q_idx, "q_idx", _IDX_DTYPES, 3)
    _dev_tensor(k_pool, "k_pool", (q_idx.dtype,), 3)
    _dev_tensor(Q, "Q", (torch.bfloat16,), 4)
    _dev_tensor(K_pool, "K_pool", (torch.bfloat16,), 3)
    _dev_tensor(V_pool, "V_pool", (torch.bfloat16,), 3)
    _dev_tensor(seq_pos, "seq_pos", (torch.int32,), 1)
    B, n_q, d = q_idx.shape
    n_pages = k_pool.shape[0]
    if k_pool.shape[1] != page_size or K_pool.shape[:2] != (n_pages, page_size) or \
            V_pool.shape != K_pool.shape:
        raise ValueError("pools must be [n_pages, page_size, ...] alike")
    pages = make_pages(block_table, page_size, n_pages)
    n_k = block_table.shape[1] * page_size
    H = Q.shape[2]
    p = make_problem(B, n_q, n_k, 0, d, q_idx.dtype, top_k, H, Q.shape[3])
    dev = Q.device
    idx = torch.empty((B, n_q, top_k), dtype=torch.int32, device=dev) if want_idx else None
    O = torch.empty_like(Q)
    lse = torch.empty((B, n_q, H), dtype=torch.float32, device=dev) if want_lse else None
    Forward(p, dev)(q_idx, k_pool, Q, K_pool, V_pool, O, idx, lse, seq_pos=seq_pos, pages=pages,
                    tau=tau)
    return idx, O, lse
