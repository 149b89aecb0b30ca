"""Host-side checks of the C ABI: the library loads on a machine without a
GPU, exports every function include/dsa.h declares, sizes workspaces, and
rejects bad arguments before it touches the HIP runtime."""
import ctypes
import os
import re

import pytest

import dsa_top_token_amd as dsa
from dsa_top_token_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("dsa_index_scores", "dsa_topk", "dsa_sparse_attn", "dsa_forward",
              "dsa_workspace_size", "dsa_status_str", "dsa_last_error"):
        assert n in names


def test_header_compiles_as_c_and_matches_the_binding(tmp_path):
    # the boundary is plain C: the header compiles with a C99 compiler, and
    # the option structs have the sizes the ctypes binding assumes
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "t.c"
    src.write_text('#include "dsa.h"\n#include <stdio.h>\nint main(void) {\n'
                   '  printf("%d %d %d\\n", (int)sizeof(dsa_problem), (int)sizeof(dsa_pages),\n'
                   '         (int)sizeof(dsa_forward_options));\n  return 0;\n}\n')
    exe = tmp_path / "t"
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I" + os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    sizes = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                            check=True).stdout.split()]
    assert sizes == [ctypes.sizeof(dsa.Problem), ctypes.sizeof(dsa.Pages),
                     ctypes.sizeof(dsa.Options)]


def test_library_exports_every_declared_symbol():
    lib = dsa.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) <= set(dsa.EXPORTS)


def test_status_strings():
    lib = dsa.load()
    for code, name in dsa.STATUS.items():
        assert lib.dsa_status_str(code).decode() == name


def prob(**kw):
    base = dict(batch=1, n_q=64, n_k=64, q_pos0=0, d_idx=128, idx_dtype=0, top_k=8,
                n_heads=8, head_dim=128)
    base.update(kw)
    return dsa.Problem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), -2), (dict(n_q=0), -2), (dict(n_k=0), -2), (dict(q_pos0=-1), -2),
    (dict(q_pos0=1), -2), (dict(n_q=65), -2), (dict(n_k=1 << 23, n_q=1, q_pos0=0), -2),
    (dict(d_idx=0), -2), (dict(d_idx=100), -3), (dict(d_idx=288), -3),
    (dict(idx_dtype=2), -3), (dict(top_k=0), -2), (dict(top_k=4097), -3),
    (dict(n_heads=0), -2), (dict(n_heads=17), -3), (dict(head_dim=64), -3),
])
def test_bad_problems_are_rejected(kw, status):
    n = ctypes.c_size_t(0)
    p = prob(**kw)
    rc = dsa.load().dsa_workspace_size(ctypes.byref(p), dsa.OP_FORWARD, ctypes.byref(n))
    assert rc == status, dsa.load().dsa_last_error()
    assert dsa.load().dsa_last_error().decode() != ""


FAKE = ctypes.c_void_p(0x100000)       # never dereferenced: validation fails first
ODD = ctypes.c_void_p(0x100008)        # 8-byte aligned only


def test_null_and_misaligned_pointers():
    lib = dsa.load()
    p = prob()
    P = ctypes.byref(p)
    assert lib.dsa_index_scores(None, FAKE, FAKE, 0, 1, FAKE, None) == -1
    assert lib.dsa_index_scores(P, None, FAKE, 0, 1, FAKE, None) == -1
    assert lib.dsa_index_scores(P, FAKE, FAKE, 0, 1, None, None) == -1
    assert lib.dsa_index_scores(P, ODD, FAKE, 0, 1, FAKE, None) == -4
    assert lib.dsa_index_scores(P, FAKE, FAKE, 1, 1, FAKE, None) == -2
    assert lib.dsa_index_scores(P, FAKE, FAKE, 0, 65, FAKE, None) == -2
    assert lib.dsa_topk(P, None, 0, 1, FAKE, None, 0, None) == -1
    assert lib.dsa_topk(P, FAKE, 0, 1, ODD, None, 0, None) == -4
    assert lib.dsa_topk(P, FAKE, -1, 1, FAKE, None, 0, None) == -2
    assert lib.dsa_sparse_attn(P, FAKE, FAKE, None, FAKE, FAKE, None, None, 0, None) == -1
    assert lib.dsa_sparse_attn(P, FAKE, FAKE, FAKE, FAKE, FAKE, ODD, None, 0, None) == -4
    # forward needs its workspace
    assert lib.dsa_forward(P, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, 0,
                           None) == -5
    need = dsa.workspace_size(p, dsa.OP_FORWARD)
    assert lib.dsa_forward(P, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE,
                           need - 1, None) == -5
    assert lib.dsa_forward(P, FAKE, FAKE, FAKE, FAKE, FAKE, ODD, FAKE, None, FAKE,
                           need, None) == -4


def test_ragged_forward_arguments():
    lib = dsa.load()
    dec = prob(n_q=1, n_k=64, q_pos0=0)
    need = dsa.workspace_size(dec, dsa.OP_FORWARD)
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, need, None)
    assert lib.dsa_forward_ragged(ctypes.byref(dec), None, *args) == -1
    assert lib.dsa_forward_ragged(ctypes.byref(dec), ODD, *args) == -4
    # positions come from seq_pos only, one query per sequence
    assert lib.dsa_forward_ragged(ctypes.byref(prob(n_q=1, n_k=64, q_pos0=5)), FAKE, *args) == -2
    assert lib.dsa_forward_ragged(ctypes.byref(prob(n_q=2, n_k=64)), FAKE, *args) == -3
    # and the workspace of dsa_forward
    assert lib.dsa_forward_ragged(ctypes.byref(dec), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                  FAKE, None, FAKE, need - 1, None) == -5


def test_threshold_forward_arguments():
    lib = dsa.load()
    dec = prob(n_q=1, n_k=64, q_pos0=63)
    need = dsa.workspace_size(dec, dsa.OP_FORWARD)
    args = lambda ws=FAKE, n=need: (FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, ws, n, None)
    assert lib.dsa_forward_threshold(None, 0.5, *args()) == -1
    assert lib.dsa_forward_threshold(ctypes.byref(dec), 0.5, None, *args()[1:]) == -1
    assert lib.dsa_forward_threshold(ctypes.byref(prob(top_k=5000)), 0.5, *args()) == -3
    assert lib.dsa_forward_threshold(ctypes.byref(dec), 0.5, *args(n=need - 1)) == -5
    assert lib.dsa_forward_threshold(ctypes.byref(dec), 0.5, *args(ws=ODD)) == -4
    ms = (ctypes.c_float * 3)()
    assert lib.dsa_forward_threshold_timed(ctypes.byref(dec), 0.5, *args(), None, None) == -1
    assert lib.dsa_forward_threshold_timed(ctypes.byref(dec), 0.5, *args(n=need - 1), ms,
                                           None) == -5


def test_forward_ext_arguments():
    lib = dsa.load()
    dec = prob(n_q=1, n_k=512, q_pos0=0)
    need = dsa.workspace_size(dec, dsa.OP_FORWARD)
    tail = lambda n=need: (FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, n, None)
    pg = dsa.Pages(block_table=0x100000, page_size=256, pages_per_seq=2, n_pages=8)
    opt = lambda **kw: ctypes.byref(dsa.Options(**kw))
    # no options: the checks of dsa_forward
    assert lib.dsa_forward_ext(ctypes.byref(dec), None, *tail(need - 1)) == -5
    # pages need seq_pos; ragged and paged need one query per sequence at q_pos0 = 0
    assert lib.dsa_forward_ext(ctypes.byref(dec), opt(pages=ctypes.pointer(pg)), *tail()) == -1
    assert lib.dsa_forward_ext(ctypes.byref(prob(n_q=2, n_k=512)),
                               opt(seq_pos=0x100000, threshold_mode=1, tau=1.0), *tail()) == -3
    assert lib.dsa_forward_ext(ctypes.byref(dec), opt(seq_pos=0x100008), *tail()) == -4
    bad = dsa.Pages(block_table=0x100000, page_size=100, pages_per_seq=2, n_pages=8)
    assert lib.dsa_forward_ext(ctypes.byref(dec), opt(seq_pos=0x100000, pages=ctypes.pointer(bad)),
                               *tail()) == -2
    # valid layouts and modes get as far as the workspace check
    for o in (opt(threshold_mode=1, tau=0.5), opt(seq_pos=0x100000, threshold_mode=1, tau=0.5),
              opt(seq_pos=0x100000, pages=ctypes.pointer(pg), threshold_mode=1, tau=0.5)):
        assert lib.dsa_forward_ext(ctypes.byref(dec), o, *tail(need - 1)) == -5
    ms = (ctypes.c_float * 3)()
    assert lib.dsa_forward_ext_timed(ctypes.byref(dec), None, *tail(), None, None) == -1
    assert lib.dsa_forward_ext_timed(ctypes.byref(dec), None, *tail(need - 1), ms, None) == -5


def test_index_project_arguments():
    lib = dsa.load()
    call = lambda rows=64, dm=4096, di=128, dt=0, X=FAKE, W=FAKE, out=FAKE, orow=None, \
        n_out=64: lib.dsa_index_project(rows, dm, di, dt, X, W, out, orow, n_out, None)
    assert call(rows=0) == -2
    assert call(dm=100) == -3 and call(dm=0) == -3 and call(dm=1 << 20) == -3
    assert call(di=48) == -3 and call(di=512) == -3
    assert call(dt=2) == -3
    assert call(X=None) == -1 and call(W=None) == -1 and call(out=None) == -1
    assert call(X=ODD) == -4 and call(orow=ODD) == -4
    assert call(n_out=0) == -2
    assert call(n_out=10) == -2               # fewer output rows than inputs, no out_rows


def test_paged_forward_arguments():
    lib = dsa.load()
    dec = prob(n_q=1, n_k=512, q_pos0=0)
    need = dsa.workspace_size(dec, dsa.OP_FORWARD)
    tail = (FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, need, None)

    def call(pg, sp=FAKE, p=dec):
        return lib.dsa_forward_paged(ctypes.byref(p), sp, pg, *tail)

    ok = dict(block_table=0x100000, page_size=256, pages_per_seq=2, n_pages=8)
    pg = lambda **kw: ctypes.byref(dsa.Pages(**{**ok, **kw}))
    assert call(None) == -1
    assert call(pg(block_table=None)) == -1
    assert call(pg(block_table=0x100008)) == -4
    assert call(pg(page_size=0)) == -2
    assert call(pg(page_size=512)) == -2      # 2 x 512 != n_k
    assert call(pg(page_size=100)) == -2      # 2 x 100 != n_k
    assert call(pg(n_pages=0)) == -2
    assert call(pg(n_pages=1 << 16)) == -2    # K/V pools of 4 GiB
    assert call(pg(), sp=None) == -1
    assert call(pg(), p=prob(n_q=2, n_k=512)) == -3
    # valid arguments get as far as the workspace check
    assert lib.dsa_forward_paged(ctypes.byref(dec), FAKE, pg(), FAKE, FAKE, FAKE, FAKE, FAKE,
                                 None, FAKE, None, FAKE, need - 1, None) == -5


def test_attention_workspace_only_when_split():
    # decode-sized batches split each query's keys; prefill does not
    dec = synth.WORKLOADS["decode_128k_clustered"]
    p = dsa.make_problem(dec.batch, dec.n_q, dec.n_k, dec.q_pos0, dec.d_idx, dec.idx_dtype,
                         dec.top_k, dec.n_heads)
    assert dsa.workspace_size(p, dsa.OP_ATTN) > 0
    pre = synth.WORKLOADS["prefill_64k"]
    p = dsa.make_problem(pre.batch, pre.n_q, pre.n_k, pre.q_pos0, pre.d_idx, pre.idx_dtype,
                         pre.top_k, pre.n_heads)
    assert dsa.workspace_size(p, dsa.OP_ATTN) == 0


def test_topk_workspace_only_for_long_rows():
    # few long rows use the chunked schedule, which needs a workspace
    dec = synth.WORKLOADS["decode_128k_clustered"]
    p = dsa.make_problem(dec.batch, dec.n_q, dec.n_k, dec.q_pos0, dec.d_idx, dec.idx_dtype,
                         dec.top_k, dec.n_heads)
    assert dsa.workspace_size(p, dsa.OP_TOPK) > 0
    p = dsa.make_problem(4, 1, 4000, 3999, 128, "fp8", 64, 1)
    assert dsa.workspace_size(p, dsa.OP_TOPK) == 0


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_forward_workspace_fits(name):
    w = synth.WORKLOADS[name]
    p = dsa.make_problem(w.batch, w.n_q, w.n_k, w.q_pos0, w.d_idx, w.idx_dtype, w.top_k,
                         w.n_heads)
    n = dsa.workspace_size(p, dsa.OP_FORWARD)
    # score slab (<= 2 GiB) or candidate lists (<= 12 GiB), or the key-range
    # attention partials that reuse them (one 16-head fp16 row + 16 (lse,
    # scale) pairs per (row, 12288-key range) pair), + index lists + fallback
    # score rows (256 rows of n_k) + thresholds, counts and attention partials
    idx_bytes = w.batch * w.n_q * w.top_k * 4
    ranges = -(-w.n_k // 12288)
    big = max(12 << 30, w.batch * w.n_q * ranges * (16 * 128 * 2 + 16 * 8))
    assert idx_bytes <= n <= big + idx_bytes + 256 * w.n_k * 4 + (64 << 20)


def test_product_path_has_no_oracle_or_cpu_fallback():
    # the package never imports the oracle and has no CPU compute path
    pkg = os.path.join(ROOT, "dsa_top_token_amd")
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            src = open(os.path.join(pkg, f)).read()
            assert "import oracle" not in src and "from oracle" not in src, f
