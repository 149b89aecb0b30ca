"""CPU oracle for the DSA indexer -> top-k -> sparse MQA attention path.

TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers; the product path never imports this
package. The arithmetic lives in dsa_oracle.c (plain loops, double
accumulation); this module builds it with gcc and marshals numpy/torch arrays
through ctypes. It shares no code with the GPU library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

FP8, BF16 = 0, 1


def build(force: bool = False) -> str:
    """Compile dsa_oracle.c into liboracle.so (skipped when up to date)."""
    if (not force and os.path.exists(_LIB)
            and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC)):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-std=c11", "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            P, I = ctypes.c_void_p, ctypes.c_int
            lib.oracle_index_scale.argtypes = [I]
            lib.oracle_index_scale.restype = ctypes.c_float
            lib.oracle_index_scores.argtypes = [I, I, I, I, I, I, P, P, I, I, P]
            lib.oracle_topk.argtypes = [I, I, I, I, I, P, P]
            lib.oracle_sparse_attn.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P]
            lib.oracle_forward.argtypes = [I] * 9 + [P] * 5 + [I, I, P, P, P]
            lib.oracle_forward_seqpos.argtypes = [I, I, I, P] + [I] * 5 + [P] * 5 + [I, I, P,
                                                                                  P, P]
            lib.oracle_forward_rowlist.argtypes = [I] * 9 + [P] * 5 + [P, I, P, P, P]
            F = ctypes.c_float
            lib.oracle_select_threshold.argtypes = [I, I, I, I, I, F, P, P]
            lib.oracle_forward_threshold.argtypes = ([I] * 7 + [F, I, I] + [P] * 5 +
                                                     [I, I, P, P, P])
            lib.oracle_forward_seqpos_threshold.argtypes = ([I, I, I, P] + [I] * 3 + [F, I, I] +
                                                            [P] * 5 + [I, I, P, P, P])
            lib.oracle_index_project.argtypes = [I, I, I, I, P, P, P, I, P]
            lib.oracle_encode.argtypes = [I, I, P, P]
            lib.oracle_num_threads.argtypes = []
            for f in (lib.oracle_index_project, lib.oracle_encode,
                      lib.oracle_forward_seqpos_threshold,
                      lib.oracle_index_scores, lib.oracle_topk,
                      lib.oracle_sparse_attn, lib.oracle_forward,
                      lib.oracle_forward_seqpos, lib.oracle_select_threshold,
                      lib.oracle_forward_rowlist,
                      lib.oracle_forward_threshold, lib.oracle_num_threads):
                f.restype = I
            _lib = lib
    return _lib


def _raw(x):
    """Raw element bits of an fp8 / bf16 / int array as a contiguous numpy
    array (uint8 for 1-byte types, uint16 for 2-byte ones)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.element_size() == 1:
                return x.view(torch.uint8).numpy()
            if x.element_size() == 2:
                return x.view(torch.int16).numpy().view(np.uint16)
            return x.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(x)


def _dtype_code(x, dtype):
    if dtype is not None:
        return {"fp8": FP8, "bf16": BF16, FP8: FP8, BF16: BF16}[dtype]
    return FP8 if _raw(x).dtype.itemsize == 1 else BF16


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return _load().oracle_num_threads()


def index_scale(d: int) -> float:
    return float(np.float32(_load().oracle_index_scale(d)))


def encode(values, out_dtype: str) -> np.ndarray:
    """float32 values -> e4m3fn codes (uint8, round to nearest even, saturating
    at +-448) or bfloat16 codes (uint16, round to nearest even)."""
    v = np.ascontiguousarray(np.asarray(values, np.float32).reshape(-1))
    out = np.empty(v.shape, np.uint8 if out_dtype == "fp8" else np.uint16)
    rc = _load().oracle_encode(v.size, 0 if out_dtype == "fp8" else 1, _ptr(v), _ptr(out))
    assert rc == 0, rc
    return out


def index_project(X, W, out_dtype: str, out=None, out_rows=None) -> np.ndarray:
    """Indexer projection rows: encode(fl32(X[r] . W[o])) for X [rows, d_model]
    and W [d_idx, d_model] (bfloat16), written to row out_rows[r] (or r) of
    out [n_out, d_idx] (raw uint8 / uint16 codes; a fresh zeroed array of
    `rows` rows when out is None). Returns out."""
    x, wt = _raw(X), _raw(W)
    rows, d_model = x.shape
    d_idx = wt.shape[0]
    assert wt.shape == (d_idx, d_model)
    code = np.uint8 if out_dtype == "fp8" else np.uint16
    if out is None:
        out = np.zeros((rows, d_idx), code)
    assert out.dtype == code and out.shape[1] == d_idx and out.flags.c_contiguous
    dst = None
    if out_rows is not None:
        dst = np.ascontiguousarray(np.asarray(out_rows, np.int32).reshape(rows))
    rc = _load().oracle_index_project(rows, d_model, d_idx, 0 if out_dtype == "fp8" else 1,
                                      _ptr(x), _ptr(wt), _ptr(dst) if dst is not None else None,
                                      out.shape[0], _ptr(out))
    assert rc == 0, rc
    return out


def index_scores(q_idx, k_idx, q_pos0: int, q_begin: int = 0, q_end=None,
                 dtype=None) -> np.ndarray:
    """Scores [B, q_end-q_begin, n_k] float32; -inf past each query's position."""
    q, k = _raw(q_idx), _raw(k_idx)
    B, n_q, d = q.shape
    n_k = k.shape[1]
    assert k.shape == (B, n_k, d)
    q_end = n_q if q_end is None else q_end
    out = np.empty((B, q_end - q_begin, n_k), np.float32)
    rc = _load().oracle_index_scores(B, n_q, n_k, q_pos0, d,
                                     _dtype_code(q_idx, dtype), _ptr(q), _ptr(k),
                                     q_begin, q_end, _ptr(out))
    assert rc == 0, rc
    return out


def topk(scores: np.ndarray, pos_begin: int, k: int) -> np.ndarray:
    """Selected key indices [B, rows, k] int32, ascending, -1 padded."""
    s = np.ascontiguousarray(scores, dtype=np.float32)
    B, rows, n_k = s.shape
    out = np.empty((B, rows, k), np.int32)
    rc = _load().oracle_topk(B, rows, n_k, pos_begin, k, _ptr(s), _ptr(out))
    assert rc == 0, rc
    return out


def select_threshold(scores: np.ndarray, pos_begin: int, k: int, tau: float) -> np.ndarray:
    """Threshold-mode selection: per row the keys j <= pos scoring above tau
    (fp32 compare), at most k of them (the highest, ties to the lower index);
    [B, rows, k] int32, ascending, -1 padded."""
    s = np.ascontiguousarray(scores, dtype=np.float32)
    B, rows, n_k = s.shape
    out = np.empty((B, rows, k), np.int32)
    rc = _load().oracle_select_threshold(B, rows, n_k, pos_begin, k, float(np.float32(tau)),
                                         _ptr(s), _ptr(out))
    assert rc == 0, rc
    return out


def sparse_attn(Q, K, V, idx, want_lse: bool = True):
    """O [B, n_q, H, D] float32 and lse [B, n_q, H] float32 (or None)."""
    q, kk, vv = _raw(Q), _raw(K), _raw(V)
    ix = np.ascontiguousarray(_raw(idx), dtype=np.int32)
    B, n_q, H, D = q.shape
    n_k = kk.shape[1]
    k = ix.shape[2]
    assert kk.shape == (B, n_k, D) and vv.shape == (B, n_k, D)
    assert ix.shape == (B, n_q, k)
    O = np.empty((B, n_q, H, D), np.float32)
    lse = np.empty((B, n_q, H), np.float32) if want_lse else None
    rc = _load().oracle_sparse_attn(B, n_q, n_k, H, D, k, _ptr(q), _ptr(kk),
                                    _ptr(vv), _ptr(ix), _ptr(O),
                                    _ptr(lse) if want_lse else None)
    assert rc == 0, rc
    return O, lse


def forward(q_idx, k_idx, Q, K, V, q_pos0: int, k: int, q_begin: int = 0,
            q_end=None, dtype=None, seq_pos=None, tau=None):
    """All three stages for query rows [q_begin, q_end) of every sequence.
    With seq_pos (one int per sequence) query i of sequence b sits at
    seq_pos[b] + i instead of q_pos0 + i. With tau the selection runs in
    threshold mode (select_threshold) instead of top-k.

    Returns (idx [B, rows, k] int32, O [B, rows, H, D] float32,
    lse [B, rows, H] float32)."""
    qi, ki = _raw(q_idx), _raw(k_idx)
    q, kk, vv = _raw(Q), _raw(K), _raw(V)
    B, n_q, d = qi.shape
    n_k = ki.shape[1]
    H, D = q.shape[2], q.shape[3]
    q_end = n_q if q_end is None else q_end
    rows = q_end - q_begin
    idx = np.empty((B, rows, k), np.int32)
    O = np.empty((B, rows, H, D), np.float32)
    lse = np.empty((B, rows, H), np.float32)
    if tau is not None and seq_pos is not None:
        sp = np.ascontiguousarray(np.asarray(seq_pos, np.int32).reshape(B))
        rc = _load().oracle_forward_seqpos_threshold(
            B, n_q, n_k, _ptr(sp), d, _dtype_code(q_idx, dtype), k, float(np.float32(tau)), H, D,
            _ptr(qi), _ptr(ki), _ptr(q), _ptr(kk), _ptr(vv), q_begin, q_end, _ptr(idx), _ptr(O),
            _ptr(lse))
        assert rc == 0, rc
        return idx, O, lse
    if tau is not None:
        rc = _load().oracle_forward_threshold(B, n_q, n_k, q_pos0, d, _dtype_code(q_idx, dtype),
                                              k, float(np.float32(tau)), H, D, _ptr(qi),
                                              _ptr(ki), _ptr(q), _ptr(kk), _ptr(vv), q_begin,
                                              q_end, _ptr(idx), _ptr(O), _ptr(lse))
        assert rc == 0, rc
        return idx, O, lse
    if seq_pos is not None:
        sp = np.ascontiguousarray(np.asarray(seq_pos, np.int32).reshape(B))
        rc = _load().oracle_forward_seqpos(B, n_q, n_k, _ptr(sp), d,
                                           _dtype_code(q_idx, dtype), k, H, D, _ptr(qi),
                                           _ptr(ki), _ptr(q), _ptr(kk), _ptr(vv), q_begin,
                                           q_end, _ptr(idx), _ptr(O), _ptr(lse))
        assert rc == 0, rc
        return idx, O, lse
    rc = _load().oracle_forward(B, n_q, n_k, q_pos0, d, _dtype_code(q_idx, dtype),
                                k, H, D, _ptr(qi), _ptr(ki), _ptr(q), _ptr(kk),
                                _ptr(vv), q_begin, q_end, _ptr(idx), _ptr(O),
                                _ptr(lse))
    assert rc == 0, rc
    return idx, O, lse


def forward_rows(q_idx, k_idx, Q, K, V, q_pos0: int, k: int, rows, dtype=None):
    """forward() for a list of query rows (any order, repeats allowed) of
    every sequence: output entry t is query row rows[t]. One parallel call, so
    strided samples of a long prefill cost no more than a contiguous block.

    Returns (idx [B, len(rows), k] int32, O [B, len(rows), H, D] float32,
    lse [B, len(rows), H] float32)."""
    qi, ki = _raw(q_idx), _raw(k_idx)
    q, kk, vv = _raw(Q), _raw(K), _raw(V)
    B, n_q, d = qi.shape
    n_k = ki.shape[1]
    H, D = q.shape[2], q.shape[3]
    rl = np.ascontiguousarray(np.asarray(rows, np.int32).reshape(-1))
    n = rl.shape[0]
    idx = np.empty((B, n, k), np.int32)
    O = np.empty((B, n, H, D), np.float32)
    lse = np.empty((B, n, H), np.float32)
    rc = _load().oracle_forward_rowlist(B, n_q, n_k, q_pos0, d, _dtype_code(q_idx, dtype), k, H,
                                        D, _ptr(qi), _ptr(ki), _ptr(q), _ptr(kk), _ptr(vv),
                                        _ptr(rl), n, _ptr(idx), _ptr(O), _ptr(lse))
    assert rc == 0, rc
    return idx, O, lse
