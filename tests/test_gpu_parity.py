"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Indexer scores and top-k index lists must match bit for bit; attention
outputs must stay within max-abs 2e-2 and relative-L2 1e-2 of the oracle's
fp32 result (lse within 1e-3). Small cases are compared element by element;
full-size workloads in the benchmark's launch configuration are compared on
every query the oracle can afford (all decode queries, sampled prefill rows)
plus properties checked on every row.
"""
import numpy as np
import pytest
import torch

import oracle
import dsa_top_token_amd as dsa
from dsa_top_token_amd import synth
from dsa_top_token_amd.synth import Workload

pytestmark = pytest.mark.gpu

ATOL, RTOL_L2, LSE_TOL = 2e-2, 1e-2, 1e-3


def say(msg):
    print(msg, flush=True)


def bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def assert_attn_close(O_gpu, O_ref, lse_gpu=None, lse_ref=None, what=""):
    o = O_gpu.float().cpu().numpy()
    d = o - O_ref
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(O_ref), 1e-30))
    assert max_abs <= ATOL and rel <= RTOL_L2, "%s max_abs=%.3g rel_l2=%.3g" % (what, max_abs, rel)
    if lse_gpu is not None:
        l = lse_gpu.cpu().numpy()
        fin = np.isfinite(lse_ref)
        assert np.array_equal(fin, np.isfinite(l)), what
        if fin.any():
            err = float(np.max(np.abs(l[fin] - lse_ref[fin])))
            assert err <= LSE_TOL, "%s lse err %.3g" % (what, err)


def to_dev(x):
    return {k: v.to("cuda") for k, v in x.items()}


def set_prefill_direct(max_keys):
    """Sets the longest key rows with which a many-row problem takes the
    score-row path (an internal, non-ABI knob of the library; 0 never, a
    negative value the default). Returns the previous limit."""
    import ctypes
    f = dsa.load().dsa_internal_set_prefill_direct
    f.argtypes = [ctypes.c_int32]
    f.restype = ctypes.c_int32
    return f(max_keys)


@pytest.fixture(autouse=True)
def many_row_path():
    """Every test here runs small prefill problems through the many-row path
    (sampled threshold, candidate filter, select), which long contexts take;
    test_prefill_score_row_path covers the path short ones take by default."""
    prev = set_prefill_direct(0)
    yield
    set_prefill_direct(prev)


SMALL = [
    synth.WORKLOADS["prefill_1k"],
    Workload("prefill_bf16_d160_ragged", "prefill", 1, 777, 777, 0, 160, "bf16", 100, 16),
    Workload("decode_fp8_d96_ragged", "decode", 5, 1, 3001, 3000, 96, "fp8", 1024, 16),
    Workload("decode_clustered_small", "decode", 4, 1, 5000, 4999, 128, "fp8", 2048, 16,
             clustered=True),
    Workload("chunked_prefill", "prefill", 2, 50, 300, 250, 64, "fp8", 37, 3),
    Workload("single_key", "decode", 1, 1, 1, 0, 32, "fp8", 1, 1),
    Workload("topk_above_len_bf16_d256", "prefill", 2, 70, 70, 0, 256, "bf16", 4096, 4),
    Workload("prefill_d192_k1", "prefill", 1, 130, 130, 0, 192, "fp8", 1, 5),
    # long decode rows: chunked top-k with the histogram built by the indexer
    Workload("decode_chunked_20k", "decode", 3, 1, 20000, 19999, 128, "fp8", 2048, 16),
    Workload("decode_chunked_odd_len", "decode", 2, 1, 16390, 16389, 96, "fp8", 700, 8),
    Workload("decode_chunked_clustered", "decode", 2, 1, 40000, 39999, 128, "fp8", 1500, 16,
             clustered=True),
    Workload("decode_chunked_bf16", "decode", 2, 1, 9000, 8999, 160, "bf16", 4096, 4),
    Workload("decode_pos_inside_row", "decode", 2, 1, 30000, 25000, 128, "fp8", 900, 16),
    # LDS-staged decode filter at every row width it takes (16..160 bytes)
    Workload("decode_fp8_d32_8k", "decode", 2, 1, 8192, 8191, 32, "fp8", 256, 2),
    Workload("decode_fp8_d64_9k", "decode", 3, 1, 9000, 8999, 64, "fp8", 500, 4),
    Workload("decode_fp8_d160_10k", "decode", 2, 1, 10001, 10000, 160, "fp8", 1000, 8),
    Workload("decode_bf16_d32_12k", "decode", 2, 1, 12000, 11999, 32, "bf16", 600, 2),
    # a few long query rows (chunked top-k with its own histogram pass)
    Workload("chunked_prefill_long", "prefill", 2, 9, 12000, 11991, 64, "fp8", 333, 2),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_index_scores_bit_exact(gpu_lib, w):
    say("index_scores %s" % w.name)
    x = synth.make_inputs(w, seed=1, parts=("q_idx", "k_idx"))
    ref = oracle.index_scores(x["q_idx"], x["k_idx"], w.q_pos0)
    got = dsa.index_scores(x["q_idx"].cuda(), x["k_idx"].cuda(), w.q_pos0).cpu().numpy()
    assert np.array_equal(bits(got), bits(ref))
    if w.n_q > 3:  # a row slab in the middle
        a, b = w.n_q // 3, w.n_q // 3 + max(1, w.n_q // 4)
        got = dsa.index_scores(x["q_idx"].cuda(), x["k_idx"].cuda(), w.q_pos0, a, b)
        assert np.array_equal(bits(got.cpu().numpy()), bits(ref[:, a:b]))


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_topk_bit_exact_on_oracle_scores(gpu_lib, w):
    say("topk %s" % w.name)
    x = synth.make_inputs(w, seed=2, parts=("q_idx", "k_idx"))
    s = oracle.index_scores(x["q_idx"], x["k_idx"], w.q_pos0)
    ref = oracle.topk(s, w.q_pos0, w.top_k)
    got = dsa.topk(torch.from_numpy(s).cuda(), w.q_pos0, w.top_k).cpu().numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("n_k", [1000, 1024, 1025, 4097, 9999, 20000])
@pytest.mark.parametrize("levels", [1, 3, 40, 0])
@pytest.mark.parametrize("k", [1, 7, 600])
def test_topk_ties_and_ragged_rows(gpu_lib, n_k, levels, k):
    say("topk ties n_k=%d levels=%d k=%d" % (n_k, levels, k))
    g = np.random.default_rng(n_k * 7 + levels * 3 + k)
    rows = 6
    if levels:
        s = (g.integers(0, levels, (2, rows, n_k)) * 0.375).astype(np.float32)
    else:
        s = np.maximum(g.standard_normal((2, rows, n_k)), 0).astype(np.float32)
    pos_begin = n_k - rows - 3 if n_k > rows + 3 else 0
    for r in range(rows):
        s[:, r, pos_begin + r + 1:] = -np.inf
    ref = oracle.topk(s, pos_begin, k)
    got = dsa.topk(torch.from_numpy(s).cuda(), pos_begin, k, n_q=rows, q_begin=0)
    # dsa.topk takes q_pos0 of query 0; rows are queries 0..rows-1
    assert np.array_equal(got.cpu().numpy(), ref)


def random_selection(g, B, n_q, n_k, k, q_pos0, holes=True):
    idx = np.full((B, n_q, k), -1, np.int32)
    for b in range(B):
        for i in range(n_q):
            n = min(k, q_pos0 + i + 1)
            sel = np.sort(g.choice(q_pos0 + i + 1, n, replace=False))
            idx[b, i, :n] = sel
            if holes and n > 2:
                idx[b, i, g.integers(0, n)] = -1
                idx[b, i, g.integers(0, n)] = n_k + 5  # out of range: ignored
    return idx


@pytest.mark.parametrize("B,n_q,n_k,H,k,q_pos0", [
    (1, 300, 300, 8, 64, 0),       # one wave per query
    (2, 40, 2000, 16, 512, 1960),  # few queries: split keys + combine
    (3, 1, 6000, 16, 2048, 5999),  # decode-like
    (1, 17, 17, 1, 4096, 0),       # k far above the row length
    (2, 5, 900, 13, 96, 895),
    (4, 50, 3000, 16, 1000, 2950),  # two splits of 512 slots, the second ragged
    (1, 2047, 2100, 4, 64, 53),     # the most rows that still take the split path
])
def test_sparse_attn_vs_oracle(gpu_lib, B, n_q, n_k, H, k, q_pos0):
    say("sparse_attn B=%d n_q=%d n_k=%d H=%d k=%d" % (B, n_q, n_k, H, k))
    w = Workload("attn", "prefill", B, n_q, n_k, q_pos0, 32, "fp8", k, H)
    x = synth.make_inputs(w, seed=3, parts=("Q", "K", "V"))
    idx = random_selection(np.random.default_rng(B * n_k + k), B, n_q, n_k, k, q_pos0)
    O_ref, lse_ref = oracle.sparse_attn(x["Q"], x["K"], x["V"], idx)
    O, lse = dsa.sparse_attn(x["Q"].cuda(), x["K"].cuda(), x["V"].cuda(),
                             torch.from_numpy(idx).cuda(), q_pos0=q_pos0)
    assert_attn_close(O, O_ref, lse, lse_ref, "attn")


def test_sparse_attn_empty_selection(gpu_lib):
    w = Workload("attn", "decode", 2, 1, 64, 63, 32, "fp8", 32, 4)
    x = synth.make_inputs(w, seed=4, parts=("Q", "K", "V"))
    idx = np.full((2, 1, 32), -1, np.int32)
    idx[1, 0, :3] = [5, 9, 60]
    O_ref, lse_ref = oracle.sparse_attn(x["Q"], x["K"], x["V"], idx)
    O, lse = dsa.sparse_attn(x["Q"].cuda(), x["K"].cuda(), x["V"].cuda(),
                             torch.from_numpy(idx).cuda())
    assert torch.all(O[0].float() == 0)
    assert torch.all(torch.isneginf(lse[0]))
    assert_attn_close(O, O_ref, lse, lse_ref, "empty")


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_forward_small_vs_oracle(gpu_lib, w):
    say("forward %s" % w.name)
    x = synth.make_inputs(w, seed=5)
    idx_ref, O_ref, lse_ref = oracle.forward(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"],
                                             w.q_pos0, w.top_k)
    d = to_dev(x)
    idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], w.q_pos0,
                              w.top_k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert_attn_close(O, O_ref, lse, lse_ref, w.name)
    # deterministic: a second call gives identical bits
    idx2, O2, lse2 = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], w.q_pos0,
                                 w.top_k)
    assert torch.equal(idx, idx2) and torch.equal(O.view(torch.int16), O2.view(torch.int16))
    assert torch.equal(lse, lse2)


@pytest.mark.parametrize("n_k", [20000, 20001])
def test_decode_all_zero_query_overflows_candidates(gpu_lib, n_k):
    # every score is 0: the threshold bin holds the whole row, more than the
    # chunked schedule's candidate list, so the row falls back to the
    # per-row schedule; the k lowest indices win
    w = Workload("zeros_decode", "decode", 3, 1, n_k, n_k - 1, 128, "fp8", 300, 2)
    x = synth.make_inputs(w, seed=7)
    x["q_idx"][1] = 0
    d = to_dev(x)
    idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], w.q_pos0, 300)
    idx_ref, O_ref, lse_ref = oracle.forward(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"],
                                             w.q_pos0, 300)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert list(idx_ref[1, 0]) == list(range(300))
    assert_attn_close(O, O_ref, lse, lse_ref, "zeros decode")


def test_decode_threshold_misses_falls_back(gpu_lib):
    # Only every 32nd key (the ones the threshold pass samples) scores above
    # zero, so the sampled threshold keeps far fewer than k keys and the
    # select kernel must recompute the row.
    n_k, k = 20000, 300
    w = Workload("sampled_only", "decode", 2, 1, n_k, n_k - 1, 128, "fp8", k, 4)
    x = synth.make_inputs(w, seed=9)
    q = x["q_idx"].float()
    g = torch.Generator().manual_seed(9)
    noise = torch.randint(-1, 2, (2, n_k, 128), generator=g).float()
    kk = (-q).expand(2, n_k, 128).clone()
    kk[:, ::32] = (q + noise[:, ::32]).clamp(-5, 5)
    x["k_idx"] = kk.to(torch.float8_e4m3fn)
    d = to_dev(x)
    idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], w.q_pos0, k)
    idx_ref, O_ref, lse_ref = oracle.forward(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"],
                                             w.q_pos0, k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert np.all(idx_ref % 32 == 0)
    assert_attn_close(O, O_ref, lse, lse_ref, "sampled only")


def set_decode_select_min(n_k):
    """Sets the shortest key rows that take the sampled-threshold decode
    selection (an internal, non-ABI knob of the library; 0 restores the
    default). Returns the previous value."""
    import ctypes
    f = dsa.load().dsa_internal_set_decode_select_min
    f.argtypes = [ctypes.c_int32]
    f.restype = ctypes.c_int32
    return f(n_k)


# Decode batches long enough for the sampled-threshold selection, run through
# the score-row path instead (scores, then the chunked top-k schedule whose
# first histogram the indexer kernel builds), which shorter rows and top_k
# beyond the select's list take.
DECODE_SCORE_ROWS = [w for w in SMALL if w.mode == "decode" and w.n_k >= 8192]


@pytest.mark.parametrize("w", DECODE_SCORE_ROWS, ids=lambda w: w.name)
def test_forward_decode_score_rows(gpu_lib, w):
    say("decode score rows %s" % w.name)
    x = synth.make_inputs(w, seed=5)
    idx_ref, O_ref, lse_ref = oracle.forward(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"],
                                             w.q_pos0, w.top_k)
    d = to_dev(x)
    prev = set_decode_select_min(1 << 30)
    try:
        p = dsa.make_problem(w.batch, w.n_q, w.n_k, w.q_pos0, w.d_idx, w.idx_dtype, w.top_k,
                             w.n_heads)
        fwd = dsa.Forward(p, "cuda")
        idx = torch.empty(w.batch, 1, w.top_k, dtype=torch.int32, device="cuda")
        O = torch.empty_like(d["Q"])
        lse = torch.empty(w.batch, 1, w.n_heads, dtype=torch.float32, device="cuda")
        fwd(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], O, idx, lse)
        torch.cuda.synchronize()
        assert dsa.selection_stats(p, fwd.ws, fwd.ws_bytes)[1] == -1  # not the select path
    finally:
        set_decode_select_min(prev)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert_attn_close(O, O_ref, lse, lse_ref, "%s score rows" % w.name)


def test_forward_launch_log(gpu_lib, capfd, monkeypatch):
    # DSA_LOG=1: every forward call names its problem, selection path and
    # workspace on stderr; unset or "0" keeps the library silent.
    runs = [(Workload("log_decode", "decode", 2, 1, 9000, 8999, 128, "fp8", 300, 4),
             "decode selection"),
            (Workload("log_prefill", "prefill", 1, 600, 600, 0, 64, "fp8", 50, 2),
             "many-row selection")]
    for w, path in runs:
        d = to_dev(synth.make_inputs(w, seed=3))
        for on in ("1", "0"):
            monkeypatch.setenv("DSA_LOG", on)
            dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], w.q_pos0, w.top_k)
            torch.cuda.synchronize()
            err = capfd.readouterr().err
            if on == "1":
                assert "dsa: forward B=%d n_q=%d n_k=%d" % (w.batch, w.n_q, w.n_k) in err, err
                assert path in err, err
            else:
                assert "dsa: forward" not in err, err


def test_prefill_threshold_misses_fall_back(gpu_lib):
    # Only the keys the prefill threshold pass samples (every S-th key,
    # S = 2 top_k / 64 = 20) score above zero. Rows longer than 1280 keys have
    # more than m = 64 samples, so their threshold is positive and keeps only
    # the sampled keys, fewer than top_k: the fallback kernel recomputes them.
    n, k, S = 3000, 640, 20
    w = Workload("prefill_sampled_only", "prefill", 1, n, n, 0, 128, "fp8", k, 2)
    x = synth.make_inputs(w, seed=11)
    g = torch.Generator().manual_seed(11)
    x["q_idx"] = torch.ones(1, n, 128).to(torch.float8_e4m3fn)
    kk = -torch.ones(1, n, 128)
    kk[:, ::S] = torch.randint(1, 3, (1, (n + S - 1) // S, 128), generator=g).float()
    x["k_idx"] = kk.to(torch.float8_e4m3fn)
    d = to_dev(x)
    say("prefill threshold miss: n=%d k=%d" % (n, k))
    idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], 0, k)
    idx_ref, O_ref, lse_ref = oracle.forward(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"], 0, k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    # a long row (ascending indices): every sampled key plus the
    # lowest-index zero scores
    row = idx_ref[0, n - 1]
    zeros = [j for j in range(n) if j % S][: k - n // S]
    assert sorted(row.tolist()) == sorted(list(range(0, n, S)) + zeros)
    assert_attn_close(O, O_ref, lse, lse_ref, "prefill sampled only")


def test_prefill_equal_scores_overflow_falls_back(gpu_lib):
    # Every score is equal and positive: the threshold admits whole rows, more
    # than the candidate list holds (3 top_k + 768 = 960 entries) once a row
    # is longer than that, so those rows are recomputed by the fallback; the
    # k lowest indices win every row.
    n, k = 2500, 64
    w = Workload("prefill_equal", "prefill", 2, n, n, 0, 128, "fp8", k, 2)
    x = synth.make_inputs(w, seed=12)
    x["q_idx"] = torch.ones(2, n, 128).to(torch.float8_e4m3fn)
    x["k_idx"] = torch.ones(2, n, 128).to(torch.float8_e4m3fn)
    d = to_dev(x)
    say("prefill equal scores: n=%d k=%d" % (n, k))
    idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], 0, k)
    idx_ref, O_ref, lse_ref = oracle.forward(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"], 0, k)
    got = idx.cpu().numpy()
    assert np.array_equal(got, idx_ref)
    for i in (0, 63, 64, 959, 960, 2499):
        m = min(k, i + 1)
        assert list(got[1, i, :m]) == list(range(m)) and np.all(got[1, i, m:] == -1)
    assert_attn_close(O, O_ref, lse, lse_ref, "prefill equal scores")


RAGGED = [
    # decode select path (n_k >= 8192), positions short, at top_k, long,
    # empty (-1) and past the row (clamped to n_k - 1)
    (Workload("ragged_select", "decode", 7, 1, 20000, 0, 128, "fp8", 500, 4),
     [19999, 0, 499, 500, 7000, -1, 25000]),
    (Workload("ragged_select_clustered", "decode", 4, 1, 40000, 0, 128, "fp8", 1500, 16,
              clustered=True), [39999, 1499, 20000, 9001]),
    # wide bf16 rows (fragments straight from HBM)
    (Workload("ragged_select_bf16", "decode", 3, 1, 9000, 0, 160, "bf16", 1000, 4),
     [8999, 4000, 1200]),
    # short rows: score row + top-k schedule
    (Workload("ragged_topk", "decode", 4, 1, 3000, 0, 96, "fp8", 300, 8),
     [2999, 100, 1500, 299]),
]


@pytest.mark.parametrize("w,pos", RAGGED, ids=lambda v: v.name if hasattr(v, "name") else "")
def test_forward_ragged_decode(gpu_lib, w, pos):
    # Each sequence of a ragged batch equals the oracle's forward on that
    # sequence alone with its own query position.
    say("ragged %s %s" % (w.name, pos))
    x = synth.make_inputs(w, seed=13)
    d = to_dev(x)
    sp = torch.tensor(pos, dtype=torch.int32, device="cuda")
    idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], 0, w.top_k,
                              seq_pos=sp)
    idx = idx.cpu().numpy()
    for b, p in enumerate(pos):
        if p < 0:
            assert np.all(idx[b] == -1)
            assert torch.all(O[b].float() == 0) and torch.all(torch.isneginf(lse[b]))
            continue
        p = min(p, w.n_k - 1)
        sl = {k: v[b:b + 1] for k, v in x.items()}
        i_ref, O_ref, l_ref = oracle.forward(sl["q_idx"], sl["k_idx"], sl["Q"], sl["K"],
                                             sl["V"], p, w.top_k)
        assert np.array_equal(idx[b:b + 1], i_ref), (w.name, b, p)
        assert_attn_close(O[b:b + 1], O_ref, lse[b:b + 1], l_ref, "%s seq %d" % (w.name, b))


def to_pages(x, P, n_extra, seed):
    """A [B, n_k, ...] tensor as a shuffled pool of P-row pages plus its block
    table (n_extra unused pages hold noise)."""
    B, n_k = x.shape[:2]
    per = n_k // P
    n_pages = B * per + n_extra
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(n_pages, generator=g)[:B * per]
    pool = torch.randn((n_pages, P) + tuple(x.shape[2:]), generator=g).clamp(-4, 4).round()
    pool = pool.to(x.dtype)
    pool[perm] = x.reshape((B * per, P) + tuple(x.shape[2:]))
    return pool, perm.reshape(B, per).to(torch.int32)


PAGED = [
    # decode select path (256-key waves read pages of 256)
    (Workload("paged_select", "decode", 4, 1, 20480, 0, 128, "fp8", 500, 4), 256,
     [20479, 1000, 499, 12000]),
    # score-row path (short rows), pages of 512
    (Workload("paged_topk", "decode", 3, 1, 2048, 0, 96, "fp8", 300, 8), 512, [2047, 40, 1500]),
    # wide bf16 rows, pages of 1024
    (Workload("paged_bf16", "decode", 2, 1, 9216, 0, 160, "bf16", 1000, 4), 1024, [9215, 5000]),
    # pages smaller than a wave's 256-key run: translated key by key
    (Workload("paged16_select", "decode", 3, 1, 16384, 0, 128, "fp8", 700, 4), 16,
     [16383, 3000, 9999]),
    (Workload("paged64_select_d96", "decode", 2, 1, 8192, 0, 96, "fp8", 400, 2), 64,
     [8191, 5000]),
    (Workload("paged32_topk", "decode", 2, 1, 2048, 0, 64, "fp8", 200, 2), 32, [2047, 600]),
    (Workload("paged48_bf16", "decode", 2, 1, 9216, 0, 160, "bf16", 500, 2), 48, [9215, 4000]),
]


@pytest.mark.parametrize("w,P,pos", PAGED, ids=lambda v: v.name if hasattr(v, "name") else "")
def test_forward_paged_decode(gpu_lib, w, P, pos):
    # A paged layout gives exactly the results of the same batch laid out
    # contiguously (same arithmetic, rows read from other addresses), which
    # the ragged tests tie to the oracle; two sequences are checked against
    # the oracle directly as well.
    say("paged %s P=%d %s" % (w.name, P, pos))
    x = synth.make_inputs(w, seed=17)
    d = to_dev(x)
    sp = torch.tensor(pos, dtype=torch.int32, device="cuda")
    idx0, O0, lse0 = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], 0, w.top_k,
                                 seq_pos=sp)
    kp, table = to_pages(x["k_idx"], P, 5, 1)
    Kp, table_k = to_pages(x["K"], P, 5, 1)
    Vp, table_v = to_pages(x["V"], P, 5, 1)
    assert torch.equal(table, table_k) and torch.equal(table, table_v)
    idx, O, lse = dsa.forward_paged(d["q_idx"], kp.cuda(), d["Q"], Kp.cuda(), Vp.cuda(),
                                    table.cuda(), P, sp, w.top_k)
    assert torch.equal(idx, idx0)
    assert torch.equal(O.view(torch.int16), O0.view(torch.int16)) and torch.equal(lse, lse0)
    for b in (0, len(pos) - 1):
        sl = {k: v[b:b + 1] for k, v in x.items()}
        i_ref, O_ref, l_ref = oracle.forward(sl["q_idx"], sl["k_idx"], sl["Q"], sl["K"],
                                             sl["V"], pos[b], w.top_k)
        assert np.array_equal(idx[b:b + 1].cpu().numpy(), i_ref)
        assert_attn_close(O[b:b + 1], O_ref, lse[b:b + 1], l_ref, "%s seq %d" % (w.name, b))


def test_paged_threshold_miss_falls_back(gpu_lib):
    # As test_decode_threshold_misses_falls_back, over a paged layout: the
    # select kernel recomputes the rows from the page pool.
    n_k, k, P = 20480, 300, 512
    w = Workload("paged_sampled_only", "decode", 2, 1, n_k, 0, 128, "fp8", k, 4)
    x = synth.make_inputs(w, seed=19)
    q = x["q_idx"].float()
    g = torch.Generator().manual_seed(19)
    noise = torch.randint(-1, 2, (2, n_k, 128), generator=g).float()
    kk = (-q).expand(2, n_k, 128).clone()
    kk[:, ::32] = (q + noise[:, ::32]).clamp(-5, 5)
    x["k_idx"] = kk.to(torch.float8_e4m3fn)
    pos = [n_k - 1, 15000]
    d = to_dev(x)
    sp = torch.tensor(pos, dtype=torch.int32, device="cuda")
    kp, table = to_pages(x["k_idx"], P, 3, 2)
    Kp, _ = to_pages(x["K"], P, 3, 2)
    Vp, _ = to_pages(x["V"], P, 3, 2)
    idx, O, lse = dsa.forward_paged(d["q_idx"], kp.cuda(), d["Q"], Kp.cuda(), Vp.cuda(),
                                    table.cuda(), P, sp, k)
    for b, p in enumerate(pos):
        sl = {kk_: v[b:b + 1] for kk_, v in x.items()}
        i_ref, O_ref, l_ref = oracle.forward(sl["q_idx"], sl["k_idx"], sl["Q"], sl["K"],
                                             sl["V"], p, k)
        assert np.array_equal(idx[b:b + 1].cpu().numpy(), i_ref)
        assert np.all(i_ref % 32 == 0)
        assert_attn_close(O[b:b + 1], O_ref, lse[b:b + 1], l_ref, "paged miss seq %d" % b)


# Threshold mode: each workload at several tau, chosen from the oracle's
# scores so that rows keep fewer keys than top_k, more (cut to top_k), none,
# or all of them; a tau equal to a score checks the strict comparison.
THRESH_W = [
    synth.WORKLOADS["prefill_1k"],
    Workload("thr_prefill_bf16_d160", "prefill", 1, 777, 777, 0, 160, "bf16", 100, 16),
    Workload("thr_chunked_prefill", "prefill", 2, 50, 300, 250, 64, "fp8", 37, 3),
    Workload("thr_decode_fp8_d96", "decode", 5, 1, 3001, 3000, 96, "fp8", 1024, 16),
    Workload("thr_decode_20k", "decode", 3, 1, 20000, 19999, 128, "fp8", 2048, 16),
    Workload("thr_decode_clustered", "decode", 2, 1, 40000, 39999, 128, "fp8", 1500, 16,
             clustered=True),
    Workload("thr_k4096_bf16_d256", "prefill", 2, 70, 70, 0, 256, "bf16", 4096, 4),
]
THRESH_MODES = ["q50", "q97", "at_kth", "zero", "negative", "above_max", "nan"]


def pick_tau(s, mode, w):
    fin = np.sort(s[np.isfinite(s)])
    if mode == "q50":
        return float(fin[len(fin) // 2])
    if mode == "q97":
        return float(fin[int(0.97 * (len(fin) - 1))])
    if mode == "at_kth":
        # the k-th highest score of the last row: equal scores must not pass
        r = s[-1, -1][np.isfinite(s[-1, -1])]
        return float(np.sort(r)[::-1][min(w.top_k, len(r)) - 1])
    return {"zero": 0.0, "negative": -1.0, "above_max": float(fin[-1]),
            "nan": float("nan")}[mode]


@pytest.mark.parametrize("mode", THRESH_MODES)
@pytest.mark.parametrize("w", THRESH_W, ids=lambda w: w.name)
def test_forward_threshold_vs_oracle(gpu_lib, w, mode):
    say("threshold %s %s" % (w.name, mode))
    x = synth.make_inputs(w, seed=11)
    s = oracle.index_scores(x["q_idx"], x["k_idx"], w.q_pos0)
    tau = pick_tau(s, mode, w)
    idx_ref, O_ref, lse_ref = oracle.forward(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"],
                                             w.q_pos0, w.top_k, tau=tau)
    d = to_dev(x)
    idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], w.q_pos0,
                              w.top_k, tau=tau)
    assert np.array_equal(idx.cpu().numpy(), idx_ref), (w.name, mode, tau)
    assert_attn_close(O, O_ref, lse, lse_ref, "%s %s" % (w.name, mode))
    if mode == "negative":
        # every score is >= 0 > tau: the top-k forward, bit for bit
        i2, O2, l2 = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], w.q_pos0,
                                 w.top_k)
        assert torch.equal(idx, i2) and torch.equal(O.view(torch.int16), O2.view(torch.int16))
        assert torch.equal(lse, l2)
    if mode in ("above_max", "nan"):
        assert torch.all(idx == -1) and torch.all(O.float() == 0)
        assert torch.all(torch.isneginf(lse))


# Many query rows over short key rows: the score-row path (every causal
# score into the workspace, exact per-row selection), the default up to 4096
# keys.
DIRECT = [
    synth.WORKLOADS["prefill_1k"],
    Workload("direct_bf16_d160", "prefill", 1, 777, 777, 0, 160, "bf16", 100, 16),
    Workload("direct_chunked", "prefill", 2, 50, 300, 250, 64, "fp8", 37, 3),
    Workload("direct_k4096_bf16_d256", "prefill", 2, 70, 70, 0, 256, "bf16", 4096, 4),
    Workload("direct_d192_k1", "prefill", 1, 130, 130, 0, 192, "fp8", 1, 5),
    Workload("direct_4k_fp8", "prefill", 1, 4096, 4096, 0, 128, "fp8", 1024, 16),
    Workload("direct_b3_2k_fp8_d96", "prefill", 3, 2000, 2048, 48, 96, "fp8", 300, 4),
]


@pytest.mark.parametrize("tau_mode", [None, "q97", "at_kth"])
@pytest.mark.parametrize("w", DIRECT, ids=lambda w: w.name)
def test_prefill_score_row_path(gpu_lib, w, tau_mode):
    say("score-row path %s %s" % (w.name, tau_mode))
    set_prefill_direct(-1)
    p = dsa.make_problem(w.batch, w.n_q, w.n_k, w.q_pos0, w.d_idx, w.idx_dtype, w.top_k,
                         w.n_heads)
    st = dsa.selection_stats(p, *(lambda f: (f.ws, f.ws_bytes))(dsa.Forward(p, "cuda")))
    assert st[1] == -1, "problem does not take the score-row path: %s" % (st,)
    seed = 0 if w.name == "prefill_1k" else 17
    x = synth.make_inputs(w, seed=seed)
    tau = None
    if tau_mode is not None:
        tau = pick_tau(oracle.index_scores(x["q_idx"], x["k_idx"], w.q_pos0), tau_mode, w)
    idx_ref, O_ref, lse_ref = oracle.forward(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"],
                                             w.q_pos0, w.top_k, tau=tau)
    d = to_dev(x)
    idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], w.q_pos0,
                              w.top_k, tau=tau)
    assert np.array_equal(idx.cpu().numpy(), idx_ref), (w.name, tau_mode)
    assert_attn_close(O, O_ref, lse, lse_ref, "%s %s" % (w.name, tau_mode))


# Indexer projection: (rows, d_model, d_idx, out dtype, input range). "small"
# inputs keep |y| well inside the fp8 range; "wide" ones saturate often and
# land on rounding ties. Integer inputs keep every sum exact.
PROJ = [
    (1, 32, 32, "fp8", "small"),
    (17, 96, 128, "fp8", "small"),
    (64, 4096, 128, "fp8", "small"),      # a decode batch: the model width is split
    (64, 4096, 128, "bf16", "small"),
    (64, 4096, 128, "fp8", "wide"),
    (1000, 512, 160, "fp8", "wide"),
    (9000, 256, 256, "bf16", "wide"),     # two row tiles per wave
    (20000, 1024, 96, "fp8", "small"),
    (70001, 128, 64, "fp8", "wide"),
    # the LDS-staged many-rows kernel at each of its ring shapes, odd chunk
    # counts, and the register kernel for a model width not a multiple of 64
    (50000, 192, 128, "fp8", "wide"),
    (60001, 320, 96, "bf16", "small"),
    (52000, 64, 32, "fp8", "wide"),
    (50001, 160, 128, "fp8", "small"),
]


def proj_inputs(rows, d_model, d_idx, kind, seed):
    g = np.random.default_rng(seed)
    if kind == "small":
        X = g.integers(-3, 4, (rows, d_model))
        W = g.integers(-1, 2, (d_idx, d_model)) * (g.random((d_idx, d_model)) < 1 / 16)
    else:
        X = g.integers(-8, 9, (rows, d_model))
        W = g.integers(-2, 3, (d_idx, d_model)) * (g.random((d_idx, d_model)) < 1 / 4)
    return (torch.tensor(X, dtype=torch.bfloat16), torch.tensor(W, dtype=torch.bfloat16))


def raw_bytes(t):
    return t.view(torch.uint8).cpu().numpy() if t.element_size() == 1 else \
        t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("rows,d_model,d_idx,dt,kind", PROJ)
def test_index_project_bit_exact(gpu_lib, rows, d_model, d_idx, dt, kind):
    say("index_project rows=%d d_model=%d d_idx=%d %s %s" % (rows, d_model, d_idx, dt, kind))
    X, W = proj_inputs(rows, d_model, d_idx, kind, rows + d_model)
    ref = oracle.index_project(X, W, dt)
    cast = torch.float8_e4m3fn if dt == "fp8" else torch.bfloat16
    got = dsa.index_project(X.cuda(), W.cuda(), cast)
    assert np.array_equal(raw_bytes(got), ref)
    if kind == "wide" and dt == "fp8" and d_model >= 2048:
        assert (ref == 0x7e).any() and (ref == 0xfe).any()  # saturation was exercised


def test_index_project_appends_to_cache(gpu_lib):
    # one new key row per sequence into the k_idx cache at its position; a
    # destination outside the cache is skipped
    B, n_k, d_model, d_idx = 6, 1000, 2048, 128
    X, W = proj_inputs(B, d_model, d_idx, "small", 3)
    g = np.random.default_rng(4)
    cache0 = g.integers(0, 0x7e, (B * n_k, d_idx)).astype(np.uint8)
    pos = [0, 999, 500, 17, 3, 998]
    dst = [b * n_k + p for b, p in enumerate(pos)]
    dst_gpu = list(dst)
    dst_gpu[4] = B * n_k + 5  # outside the cache
    ref = oracle.index_project(X[[0, 1, 2, 3, 5]], W, "fp8", out=cache0.copy(),
                               out_rows=[dst[i] for i in (0, 1, 2, 3, 5)])
    cache = torch.from_numpy(cache0.copy()).cuda().view(torch.float8_e4m3fn)
    rows = torch.tensor(dst_gpu, dtype=torch.int32, device="cuda")
    dsa.index_project(X.cuda(), W.cuda(), out=cache, out_rows=rows)
    assert np.array_equal(raw_bytes(cache), ref)


@pytest.mark.parametrize("rows,d_model", [(64, 4096), (3000, 1024)])
def test_index_project_real_valued_within_one_step(gpu_lib, rows, d_model):
    # N(0, 1) inputs and N(0, 1/d_model) weights: sums are no longer exact, so
    # the fp32 accumulation order may move a value across a rounding
    # boundary; each code must be the oracle's or a neighbour
    g = torch.Generator().manual_seed(9)
    X = torch.randn((rows, d_model), generator=g).to(torch.bfloat16)
    W = (torch.randn((128, d_model), generator=g) / d_model ** 0.5).to(torch.bfloat16)
    ref = oracle.index_project(X, W, "fp8")
    got = raw_bytes(dsa.index_project(X.cuda(), W.cuda()))
    vr = torch.from_numpy(ref).view(torch.float8_e4m3fn).float().numpy()
    vg = torch.from_numpy(got).view(torch.float8_e4m3fn).float().numpy()
    step = np.maximum(np.abs(vr), np.abs(vg)) / 8 + 2.0 ** -9
    assert np.all(np.abs(vr - vg) <= step)
    assert np.mean(got == ref) > 0.99


def test_projected_decode_step(gpu_lib):
    # a decode step from hidden states: project the queries, append the new
    # keys to the k_idx cache at each sequence's last position, then the
    # forward; against the oracle's projection and forward
    w = Workload("proj_decode", "decode", 4, 1, 3000, 2999, 128, "fp8", 256, 16)
    x = synth.make_inputs(w, seed=13)
    d_model = 1024
    Xh, Wq = proj_inputs(w.batch, d_model, w.d_idx, "small", 21)
    _, Wk = proj_inputs(w.batch, d_model, w.d_idx, "small", 22)
    dst = [b * w.n_k + w.q_pos0 for b in range(w.batch)]
    q_ref = oracle.index_project(Xh, Wq, "fp8")
    k_ref = oracle.index_project(Xh, Wk, "fp8", out=raw_bytes(x["k_idx"]).reshape(-1, w.d_idx).copy(),
                                 out_rows=dst)
    q_ref_t = torch.from_numpy(q_ref).view(torch.float8_e4m3fn).reshape(w.batch, 1, w.d_idx)
    k_ref_t = torch.from_numpy(k_ref).view(torch.float8_e4m3fn).reshape(w.batch, w.n_k, w.d_idx)
    idx_ref, O_ref, lse_ref = oracle.forward(q_ref_t, k_ref_t, x["Q"], x["K"], x["V"], w.q_pos0,
                                             w.top_k)
    d = to_dev(x)
    q = dsa.index_project(Xh.cuda(), Wq.cuda()).reshape(w.batch, 1, w.d_idx)
    kc = d["k_idx"].reshape(-1, w.d_idx)
    dsa.index_project(Xh.cuda(), Wk.cuda(), out=kc,
                      out_rows=torch.tensor(dst, dtype=torch.int32, device="cuda"))
    idx, O, lse = dsa.forward(q, d["k_idx"], d["Q"], d["K"], d["V"], w.q_pos0, w.top_k)
    assert np.array_equal(raw_bytes(d["k_idx"]).reshape(-1, w.d_idx), k_ref)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert_attn_close(O, O_ref, lse, lse_ref, "projected decode")


@pytest.mark.parametrize("w,pos", RAGGED[:3], ids=lambda v: v.name if hasattr(v, "name") else "")
def test_forward_ragged_paged_threshold(gpu_lib, w, pos):
    # threshold mode in a ragged batch (dsa_forward_ext) against the oracle
    # at each sequence's position, then the same batch in 16- and 256-key
    # pages: identical results
    x = synth.make_inputs(w, seed=17)
    s = oracle.index_scores(x["q_idx"], x["k_idx"], 0)
    tau = float(np.quantile(s[np.isfinite(s)], 0.98))
    say("ragged threshold %s tau=%.3f" % (w.name, tau))
    idx_ref, O_ref, lse_ref = oracle.forward(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"], 0,
                                             w.top_k, seq_pos=pos, tau=tau)
    d = to_dev(x)
    sp = torch.tensor(pos, dtype=torch.int32, device="cuda")
    idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], 0, w.top_k,
                              seq_pos=sp, tau=tau)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert_attn_close(O, O_ref, lse, lse_ref, "ragged threshold")
    for P in (16, 256):
        if w.n_k % P:
            continue
        kp, table = to_pages(x["k_idx"], P, 3, P)
        Kp, _ = to_pages(x["K"], P, 3, P)
        Vp, _ = to_pages(x["V"], P, 3, P)
        i2, O2, l2 = dsa.forward_paged(d["q_idx"], kp.cuda(), d["Q"], Kp.cuda(), Vp.cuda(),
                                       table.cuda(), P, sp, w.top_k, tau=tau)
        assert torch.equal(i2, idx), P
        assert torch.equal(O2.view(torch.int16), O.view(torch.int16)) and torch.equal(l2, lse), P


def test_all_zero_query_selects_first_keys(gpu_lib):
    w = Workload("zeros", "prefill", 1, 600, 600, 0, 128, "fp8", 64, 2)
    x = synth.make_inputs(w, seed=6)
    x["q_idx"] = torch.zeros_like(x["q_idx"])
    d = to_dev(x)
    idx, _, _ = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], 0, 64)
    idx = idx.cpu().numpy()[0]
    for i in range(600):
        m = min(64, i + 1)
        assert list(idx[i, :m]) == list(range(m)) and np.all(idx[i, m:] == -1)


def test_prefill_1k_seed0_every_row(gpu_lib):
    # The 1K prefill exactly as the benchmark draws it (seed 0): scores of
    # every row bit for bit, every index list bit for bit, attention within
    # tolerance, all 1024 rows.
    w = synth.WORKLOADS["prefill_1k"]
    say("prefill_1k seed 0: every row")
    x = synth.make_inputs(w, seed=0)
    d = to_dev(x)
    idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], 0, w.top_k)
    idx_ref, O_ref, lse_ref = oracle.forward(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"], 0,
                                             w.top_k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert_attn_close(O, O_ref, lse, lse_ref, "prefill_1k seed 0")
    s = dsa.index_scores(d["q_idx"], d["k_idx"], 0).cpu().numpy()
    assert np.array_equal(bits(s), bits(oracle.index_scores(x["q_idx"], x["k_idx"], 0)))
    check_topk_every_row(d, w, idx)


# Many-row prefills whose top_k takes the larger select instantiations (list
# entries per thread: 14 for top_k 2048, 18 for 2800, 26 for 4096), on rows
# longer than top_k, every row against the oracle.
BIG_K = [
    Workload("prefill_bf16_d160_k2048", "prefill", 1, 12000, 12000, 0, 160, "bf16", 2048, 2),
    Workload("prefill_fp8_d128_k2800", "prefill", 1, 10000, 10000, 0, 128, "fp8", 2800, 2),
    Workload("prefill_fp8_d128_k4096", "prefill", 1, 10000, 10000, 0, 128, "fp8", 4096, 2),
]


@pytest.mark.parametrize("w", BIG_K, ids=lambda w: w.name)
def test_prefill_large_topk_every_row(gpu_lib, w):
    say("large top_k prefill %s" % w.name)
    x = synth.make_inputs(w, seed=21)
    d = to_dev(x)
    idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], 0, w.top_k)
    torch.cuda.synchronize()
    check_topk_every_row(d, w, idx)
    say("large top_k prefill %s: oracle" % w.name)
    idx_ref, O_ref, lse_ref = oracle.forward(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"], 0,
                                             w.top_k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert_attn_close(O, O_ref, lse, lse_ref, w.name)


@pytest.mark.parametrize("w", [
    # few query rows at the end of a long context: each row's keys are
    # scored in up to four key ranges by separate workgroups, into separate
    # sub-lists the select concatenates in order
    Workload("chunk_50k_fp8_ranges", "prefill", 2, 700, 50000, 49300, 128, "fp8", 512, 2),
    Workload("chunk_70k_bf16_ranges", "prefill", 1, 500, 70000, 69500, 160, "bf16", 2048, 2),
], ids=lambda w: w.name)
def test_prefill_key_ranges_every_row(gpu_lib, w):
    say("key-range prefill %s" % w.name)
    x = synth.make_inputs(w, seed=29)
    d = to_dev(x)
    idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], w.q_pos0, w.top_k)
    torch.cuda.synchronize()
    check_topk_every_row(d, w, idx)
    idx_ref, O_ref, lse_ref = oracle.forward(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"],
                                             w.q_pos0, w.top_k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert_attn_close(O, O_ref, lse, lse_ref, w.name)


@pytest.mark.parametrize("w,n_slabs", [
    (Workload("prefill_b2_slabs4", "prefill", 2, 6000, 6000, 0, 128, "fp8", 300, 2), 4),
    (Workload("prefill_bf16_slabs3_chunked", "prefill", 1, 3001, 5000, 1999, 96, "bf16", 500, 3),
     3),
], ids=lambda v: v.name if isinstance(v, Workload) else str(v))
def test_prefill_forced_slabs_every_row(gpu_lib, w, n_slabs):
    # A lowered slab budget splits the many-row path into strided slabs (rows
    # s, s + n, s + 2n, ... for slab s), each with its own threshold, filter,
    # select and fallback launches over the same workspace: every row against
    # the oracle, and identical to the one-slab result.
    x = synth.make_inputs(w, seed=23)
    d = to_dev(x)
    idx1, O1, lse1 = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], w.q_pos0,
                                 w.top_k)
    per = (w.n_q + n_slabs - 1) // n_slabs
    old = set_prefill_slab_rows(per)
    try:
        assert prefill_slab_count(d, w) == n_slabs
        say("forced slabs %s: %d slabs" % (w.name, n_slabs))
        idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], w.q_pos0,
                                  w.top_k)
        torch.cuda.synchronize()
    finally:
        set_prefill_slab_rows(old)
    idx_ref, O_ref, lse_ref = oracle.forward(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"],
                                             w.q_pos0, w.top_k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert_attn_close(O, O_ref, lse, lse_ref, w.name)
    assert torch.equal(idx, idx1)
    assert torch.equal(O.view(torch.int16), O1.view(torch.int16)) and torch.equal(lse, lse1)


@pytest.mark.parametrize("w,rows", [
    # every row reaches both 12288-key ranges; two sequences
    (Workload("ranged_chunked", "prefill", 2, 1100, 20000, 18900, 64, "fp8", 300, 16),
     [(0, 3), (517, 520), (1097, 1100)]),
    # rows below key 12288 finish in one range, the rest merge two partials;
    # 5 heads, and rows just past 12288 often select no key of range 1
    (Workload("ranged_prefill", "prefill", 1, 13000, 13000, 0, 32, "bf16", 200, 5),
     [(0, 13000)]),
], ids=lambda v: v.name if isinstance(v, Workload) else "")
def test_forward_key_range_attention(gpu_lib, w, rows):
    # Many sorted, causal rows over more than 12288 keys: the forward's
    # attention runs range by range and merges per-range partials. Every row
    # must agree with the one-pass attention call on the same selection, and
    # the sampled rows with the oracle.
    say("key-range attention %s" % w.name)
    x = synth.make_inputs(w, seed=11)
    d = to_dev(x)
    idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], w.q_pos0,
                              w.top_k)
    check_selection_properties(idx, w.q_pos0, w.top_k)
    O1, lse1 = dsa.sparse_attn(d["Q"], d["K"], d["V"], idx, q_pos0=w.q_pos0)
    assert_attn_close(O, O1.float().cpu().numpy(), lse, lse1.cpu().numpy(), "vs one pass")
    for (a, b) in rows:
        idx_ref, O_ref, lse_ref = oracle.forward(x["q_idx"], x["k_idx"], x["Q"], x["K"],
                                                 x["V"], w.q_pos0, w.top_k, a, b)
        assert np.array_equal(idx[:, a:b].cpu().numpy(), idx_ref), (a, b)
        assert_attn_close(O[:, a:b], O_ref, lse[:, a:b], lse_ref, "%s %d-%d" % (w.name, a, b))


def check_selection_properties(idx, q_pos0, k):
    """On the GPU, for every row: ascending, inside [0, pos], min(k, pos+1)
    entries, -1 padding."""
    B, n_q, _ = idx.shape
    pos = q_pos0 + torch.arange(n_q, device=idx.device)[None, :, None]
    n_sel = torch.clamp(pos + 1, max=k)
    slot = torch.arange(k, device=idx.device)[None, None, :]
    valid = slot < n_sel
    assert torch.all(torch.where(valid, idx >= 0, idx == -1))
    assert torch.all(torch.where(valid, idx <= pos, True))
    inc = idx[:, :, 1:] > idx[:, :, :-1]
    assert torch.all(torch.where(valid[:, :, 1:], inc, True))


def check_topk_every_row(d, w, idx, rows_per_slab=None):
    """Every row's index list against an independent top-k computed on the GPU
    with torch (neither the HIP path nor the oracle): the integer indexer
    inputs make the dot an exact integer |n| <= 2560, so an fp32 matmul gives
    it exactly; one fp32 multiply by fl32(d^-0.5) and ReLU give the score
    (the DSA page, section 3.2). The kept set is then the first min(k, pos+1)
    causal keys under (score desc, index asc) (section 3.3), found with a
    torch top-k over int64 keys (score bits << 32 | ~index) and listed in
    ascending index order, -1 padded."""
    torch.backends.cuda.matmul.allow_tf32 = False
    B, n_q, dq = d["q_idx"].shape
    n_k = d["k_idx"].shape[1]
    k = w.top_k
    scale = torch.tensor(np.float32(oracle.index_scale(dq)), device="cuda")
    if rows_per_slab is None:
        rows_per_slab = max(1, min(n_q, (1 << 26) // n_k))
    j = torch.arange(n_k, device="cuda", dtype=torch.int64)
    low = (0xFFFFFFFF - j)[None, :]
    for b in range(B):
        kf = d["k_idx"][b].float()
        kt = kf.t().contiguous()
        for r0 in range(0, n_q, rows_per_slab):
            r1 = min(n_q, r0 + rows_per_slab)
            qf = d["q_idx"][b, r0:r1].float()
            dots = torch.mm(qf, kt)
            # the dot must be an exact integer for this check to be the score
            assert torch.equal(dots, dots.round()) and float(dots.abs().max()) <= 2560.0
            sc = torch.relu(dots * scale)
            key = (sc.view(torch.int32).to(torch.int64) << 32) | low
            pos = w.q_pos0 + torch.arange(r0, r1, device="cuda", dtype=torch.int64)[:, None]
            key = torch.where(j[None, :] <= pos, key, torch.full_like(key, -1))
            kk = min(k, n_k)
            top = torch.topk(key, kk, dim=1, sorted=False).values
            sel = torch.where(top >= 0, 0xFFFFFFFF - (top & 0xFFFFFFFF), torch.full_like(top, n_k))
            sel = torch.sort(sel, dim=1).values
            sel = torch.where(sel < n_k, sel, torch.full_like(sel, -1)).to(torch.int32)
            if kk < k:
                sel = torch.cat([sel, torch.full((r1 - r0, k - kk), -1, dtype=torch.int32,
                                                 device="cuda")], 1)
            got = idx[b, r0:r1]
            if not torch.equal(got, sel):
                bad = (got != sel).any(1).nonzero()[:, 0]
                raise AssertionError("%s: %d rows of sequence %d differ from the torch top-k, "
                                     "first row %d" % (w.name, bad.numel(), b, r0 + int(bad[0])))
        del kf, kt


def strided_rows(n_q, k, n=1024, seed=0):
    """About n query rows spread over the prefill (a seeded offset, then a
    fixed stride) plus the rows around top_k and the last row."""
    step = max(1, n_q // n)
    off = int(np.random.default_rng(seed + n_q).integers(0, step))
    rows = set(range(off, n_q, step))
    rows.update(r for r in (0, 1, k - 2, k - 1, k, k + 1, 2 * k, n_q - 2, n_q - 1) if 0 <= r < n_q)
    return sorted(rows)


def oracle_rows_check(x, idx, O, lse, w, rows):
    """Oracle comparison of the listed query rows (one parallel oracle call)."""
    say("%s: oracle on %d rows" % (w.name, len(rows)))
    idx_ref, O_ref, lse_ref = oracle.forward_rows(x["q_idx"], x["k_idx"], x["Q"], x["K"],
                                                  x["V"], w.q_pos0, w.top_k, rows)
    rt = torch.tensor(rows, device=idx.device, dtype=torch.long)
    got = idx.index_select(1, rt).cpu().numpy()
    if not np.array_equal(got, idx_ref):
        bad = np.nonzero((got != idx_ref).any(-1))
        raise AssertionError("%s: rows %s differ from the oracle" %
                             (w.name, sorted(set(rows[i] for i in bad[1]))[:10]))
    assert_attn_close(O.index_select(1, rt), O_ref, lse.index_select(1, rt), lse_ref,
                      "%s %d rows" % (w.name, len(rows)))


def set_prefill_slab_rows(rows):
    """Caps the query rows of one many-row slab (an internal, non-ABI knob of
    the library; 0 restores the default). Returns the previous cap."""
    import ctypes
    f = dsa.load().dsa_internal_set_prefill_slab_rows
    f.argtypes = [ctypes.c_int32]
    f.restype = ctypes.c_int32
    return f(rows)


def prefill_slab_count(d, w):
    p = dsa.make_problem(w.batch, w.n_q, w.n_k, w.q_pos0, w.d_idx, w.idx_dtype, w.top_k,
                         w.n_heads)
    fwd = dsa.Forward(p, "cuda")
    O = torch.empty_like(d["Q"])
    _, slabs = fwd.timed(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], O)
    return slabs


def run_full(w, sample_rows, gen_device="cpu"):
    say("full-size %s: generating inputs" % w.name)
    x = synth.make_inputs(w, seed=0, device=gen_device)
    d = to_dev(x) if gen_device == "cpu" else x
    say("full-size %s: GPU forward" % w.name)
    idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], w.q_pos0,
                              w.top_k)
    torch.cuda.synchronize()
    check_selection_properties(idx, w.q_pos0, w.top_k)
    xc = x if gen_device == "cpu" else {k: v.cpu() for k, v in x.items()}
    for (a, b) in sample_rows:
        say("full-size %s: oracle rows [%d, %d)" % (w.name, a, b))
        idx_ref, O_ref, lse_ref = oracle.forward(xc["q_idx"], xc["k_idx"], xc["Q"], xc["K"],
                                                 xc["V"], w.q_pos0, w.top_k, a, b)
        assert np.array_equal(idx[:, a:b].cpu().numpy(), idx_ref), (a, b)
        assert_attn_close(O[:, a:b], O_ref, lse[:, a:b], lse_ref, "%s rows %d-%d" % (w.name, a, b))
    return x, d


def test_max_size_decode(gpu_lib):
    # The largest problem the library accepts in one dimension: a decode row
    # of 4194304 keys (past the sampled-threshold select's 1M keys, so the
    # chunked top-k path over written score rows) with the largest top_k.
    w = Workload("max_keys_decode", "decode", 1, 1, 4194304, 4194303, 128, "fp8", 4096, 16)
    say("max-size decode: generating inputs")
    x = synth.make_inputs(w, seed=2)
    d = to_dev(x)
    say("max-size decode: GPU forward")
    idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], w.q_pos0, w.top_k)
    torch.cuda.synchronize()
    say("max-size decode: oracle")
    idx_ref, O_ref, lse_ref = oracle.forward(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"],
                                             w.q_pos0, w.top_k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert_attn_close(O, O_ref, lse, lse_ref, "max-size decode")


def test_full_decode_32k(gpu_lib):
    w = synth.WORKLOADS["decode_32k"]
    run_full(w, [(0, 1)])


def test_full_decode_128k_clustered(gpu_lib):
    w = synth.WORKLOADS["decode_128k_clustered"]
    run_full(w, [(0, 1)])


def test_full_decode_128k_ragged(gpu_lib):
    # The benchmark's ragged batch: every fourth sequence against the oracle
    # at its own position (one decode query each), properties on all.
    w = synth.WORKLOADS["decode_128k_ragged"]
    pos = w.positions(0)
    say("full-size %s: generating inputs" % w.name)
    x = synth.make_inputs(w, seed=0)
    d = to_dev(x)
    sp = torch.tensor(pos, dtype=torch.int32, device="cuda")
    say("full-size %s: GPU forward" % w.name)
    idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], 0, w.top_k,
                              seq_pos=sp)
    torch.cuda.synchronize()
    for b in range(w.batch):
        check_selection_properties(idx[b:b + 1], pos[b], w.top_k)
    for b in range(0, w.batch, 4):
        say("full-size %s: oracle sequence %d (position %d)" % (w.name, b, pos[b]))
        sl = {k: v[b:b + 1] for k, v in x.items()}
        i_ref, O_ref, l_ref = oracle.forward(sl["q_idx"], sl["k_idx"], sl["Q"], sl["K"],
                                             sl["V"], pos[b], w.top_k)
        assert np.array_equal(idx[b:b + 1].cpu().numpy(), i_ref), (b, pos[b])
        assert_attn_close(O[b:b + 1], O_ref, lse[b:b + 1], l_ref, "ragged seq %d" % b)
    # the same batch over the benchmark's paged layouts (256- and 16-key
    # pages): identical results
    for wname in ("decode_128k_paged", "decode_128k_paged16"):
        wp = synth.WORKLOADS[wname]
        table, n_pages = wp.page_pool(0)
        P = wp.page_size
        per = w.n_k // P
        perm = table.reshape(-1).cuda().long()
        pools = {}
        for name in ("k_idx", "K", "V"):
            t = d[name]
            pool = torch.zeros((n_pages, P) + tuple(t.shape[2:]), dtype=t.dtype, device="cuda")
            pool[perm] = t.reshape((w.batch * per, P) + tuple(t.shape[2:]))
            pools[name] = pool
        say("full-size %s: paged forward" % wp.name)
        idx_p, O_p, lse_p = dsa.forward_paged(d["q_idx"], pools["k_idx"], d["Q"], pools["K"],
                                              pools["V"], table.cuda(), P, sp, w.top_k)
        assert torch.equal(idx_p, idx), wname
        assert torch.equal(O_p.view(torch.int16), O.view(torch.int16)), wname
        assert torch.equal(lse_p, lse), wname
        del pools, idx_p, O_p, lse_p


def test_full_decode_128k_threshold(gpu_lib):
    # The benchmark's threshold-mode batch, every sequence against the oracle.
    w = synth.WORKLOADS["decode_128k_threshold"]
    say("full-size %s: generating inputs" % w.name)
    x = synth.make_inputs(w, seed=0)
    d = to_dev(x)
    say("full-size %s: GPU forward" % w.name)
    idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], w.q_pos0,
                              w.top_k, tau=w.tau)
    torch.cuda.synchronize()
    kept = (idx >= 0).sum(-1).flatten().cpu().numpy()
    say("full-size %s: kept keys per query min %d mean %.0f max %d" %
        (w.name, kept.min(), kept.mean(), kept.max()))
    assert kept.min() < w.top_k and kept.max() == w.top_k  # both regimes occur
    for b0 in range(0, w.batch, 16):
        say("full-size %s: oracle sequences %d-%d" % (w.name, b0, b0 + 16))
        sl = {k: v[b0:b0 + 16] for k, v in x.items()}
        idx_ref, O_ref, lse_ref = oracle.forward(sl["q_idx"], sl["k_idx"], sl["Q"], sl["K"],
                                                 sl["V"], w.q_pos0, w.top_k, tau=w.tau)
        assert np.array_equal(idx[b0:b0 + 16].cpu().numpy(), idx_ref), b0
        assert_attn_close(O[b0:b0 + 16], O_ref, lse[b0:b0 + 16], lse_ref, "sequences %d+" % b0)


def prefill_samples(L, k):
    g = np.random.default_rng(L)
    rows = [(0, 3), (k - 3, k + 3), (2 * k - 1, 2 * k + 1), (L - 4, L)]
    for r in sorted(g.integers(2 * k + 1, L - 4, 6)):
        rows.append((int(r), int(r) + 2))
    return rows


def run_full_prefill(w):
    """The full-size prefill in the benchmark's launch configuration: every
    row's index list against the torch top-k, about 1024 strided rows (and
    the rows around top_k) against the oracle, properties on every row."""
    say("full-size %s: generating inputs" % w.name)
    x = synth.make_inputs(w, seed=0)
    d = to_dev(x)
    say("full-size %s: GPU forward" % w.name)
    idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], w.q_pos0,
                              w.top_k)
    torch.cuda.synchronize()
    check_selection_properties(idx, w.q_pos0, w.top_k)
    say("full-size %s: torch top-k of every row" % w.name)
    check_topk_every_row(d, w, idx)
    oracle_rows_check(x, idx, O, lse, w, strided_rows(w.n_q, w.top_k))
    return x, d


def test_full_prefill_64k(gpu_lib):
    w = synth.WORKLOADS["prefill_64k"]
    x, d = run_full_prefill(w)
    # indexer scores of sampled row slabs at full width, bit for bit
    for (a, b) in [(5, 9), (40000, 40006), (w.n_q - 3, w.n_q)]:
        got = dsa.index_scores(d["q_idx"], d["k_idx"], 0, a, b).cpu().numpy()
        ref = oracle.index_scores(x["q_idx"], x["k_idx"], 0, a, b)
        assert np.array_equal(bits(got), bits(ref)), (a, b)


def test_full_prefill_64k_threshold(gpu_lib):
    # The 64K prefill in threshold mode (tau 14) at full size: sampled rows
    # against the oracle, properties on every row.
    w = synth.WORKLOADS["prefill_64k"]
    tau = 14.0
    say("full-size %s threshold: generating inputs" % w.name)
    x = synth.make_inputs(w, seed=0)
    d = to_dev(x)
    say("full-size %s threshold: GPU forward" % w.name)
    idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], 0, w.top_k,
                              tau=tau)
    torch.cuda.synchronize()
    kept = (idx >= 0).sum(-1)
    pos = torch.arange(w.n_q, device=idx.device)[None, :, None]
    slot = torch.arange(w.top_k, device=idx.device)[None, None, :]
    valid = slot < kept[..., None]
    assert torch.all(torch.where(valid, (idx >= 0) & (idx <= pos), idx == -1))
    inc = idx[:, :, 1:] > idx[:, :, :-1]
    assert torch.all(torch.where(valid[:, :, 1:], inc, True))
    assert int(kept.min()) == 0 and int(kept.max()) == w.top_k  # both regimes occur
    for (a, b) in prefill_samples(w.n_q, w.top_k):
        say("full-size %s threshold: oracle rows [%d, %d)" % (w.name, a, b))
        idx_ref, O_ref, lse_ref = oracle.forward(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"],
                                                 0, w.top_k, a, b, tau=tau)
        assert np.array_equal(idx[:, a:b].cpu().numpy(), idx_ref), (a, b)
        assert_attn_close(O[:, a:b], O_ref, lse[:, a:b], lse_ref, "rows %d-%d" % (a, b))


def test_full_decode_128k_projected(gpu_lib):
    # The projected 128K decode step at full size: q rows and the appended
    # key rows byte for byte, then every sequence's forward against the
    # oracle's chain.
    w = synth.WORKLOADS["decode_128k_projected"]
    say("full-size %s: generating inputs" % w.name)
    x = synth.make_inputs(w, seed=0)
    d = to_dev(x)
    B, di = w.batch, w.d_idx
    dst = [b * w.n_k + w.q_pos0 for b in range(B)]
    say("full-size %s: GPU projections and forward" % w.name)
    q = dsa.index_project(d["X"], d["W_q"]).reshape(B, 1, di)
    dsa.index_project(d["X"], d["W_k"], out=d["k_idx"].view(-1, di),
                      out_rows=torch.tensor(dst, dtype=torch.int32, device="cuda"))
    idx, O, lse = dsa.forward(q, d["k_idx"], d["Q"], d["K"], d["V"], w.q_pos0, w.top_k)
    torch.cuda.synchronize()
    say("full-size %s: oracle projections" % w.name)
    q_ref = oracle.index_project(x["X"], x["W_q"], "fp8")
    k_new = oracle.index_project(x["X"], x["W_k"], "fp8")
    assert np.array_equal(raw_bytes(q).reshape(B, di), q_ref)
    kc = raw_bytes(d["k_idx"]).reshape(-1, di)
    assert np.array_equal(kc[dst], k_new)
    k_ref = raw_bytes(x["k_idx"]).reshape(-1, di).copy()
    k_ref[dst] = k_new
    assert np.array_equal(kc, k_ref)  # no other cache row changed
    q_t = torch.from_numpy(q_ref).view(torch.float8_e4m3fn).reshape(B, 1, di)
    k_t = torch.from_numpy(k_ref).view(torch.float8_e4m3fn).reshape(B, w.n_k, di)
    say("full-size %s: oracle forward" % w.name)
    idx_ref, O_ref, lse_ref = oracle.forward(q_t, k_t, x["Q"], x["K"], x["V"], w.q_pos0, w.top_k)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    assert_attn_close(O, O_ref, lse, lse_ref, w.name)


def test_full_prefill_64k_projection_rows(gpu_lib):
    # The 64K prefill's projections at full size (one launch over all 65536
    # hidden rows), sampled rows against the oracle byte for byte.
    w = synth.WORKLOADS["prefill_64k_projected"]
    say("full-size %s: generating hidden states" % w.name)
    x = synth.make_inputs(w, seed=0, parts=("X",))
    X = x["X"].cuda()
    for wname in ("W_q", "W_k"):
        say("full-size %s: projection %s" % (w.name, wname))
        out = dsa.index_project(X, x[wname].cuda())
        torch.cuda.synchronize()
        for (a, b) in [(0, 16), (31999, 32040), (w.n_q - 9, w.n_q)]:
            ref = oracle.index_project(x["X"][a:b], x[wname], "fp8")
            assert np.array_equal(raw_bytes(out[a:b]), ref), (wname, a, b)


def test_full_prefill_128k_bf16(gpu_lib):
    # two strided slabs of 65536 rows in the benchmark's configuration
    w = synth.WORKLOADS["prefill_128k"]
    x, d = run_full_prefill(w)
    for (a, b) in [(0, 4), (99999, 100003), (w.n_q - 2, w.n_q)]:
        got = dsa.index_scores(d["q_idx"], d["k_idx"], 0, a, b).cpu().numpy()
        ref = oracle.index_scores(x["q_idx"], x["k_idx"], 0, a, b)
        assert np.array_equal(bits(got), bits(ref)), (a, b)


def test_full_prefill_batch2_three_slabs(gpu_lib):
    # two sequences of 40000 rows as three strided slabs (a lowered slab
    # budget): every row against the torch top-k, sampled rows against the
    # oracle
    w = Workload("prefill_b2_40k", "prefill", 2, 40000, 40000, 0, 128, "fp8", 1024, 16)
    old = set_prefill_slab_rows(13334)
    try:
        say("full-size %s: generating inputs" % w.name)
        x = synth.make_inputs(w, seed=0)
        d = to_dev(x)
        assert prefill_slab_count(d, w) == 3
        idx, O, lse = dsa.forward(d["q_idx"], d["k_idx"], d["Q"], d["K"], d["V"], 0, w.top_k)
        torch.cuda.synchronize()
    finally:
        set_prefill_slab_rows(old)
    check_selection_properties(idx, 0, w.top_k)
    check_topk_every_row(d, w, idx)
    oracle_rows_check(x, idx, O, lse, w, strided_rows(w.n_q, w.top_k, n=256))


@pytest.mark.parametrize("name", ["decode_chunked_20k", "prefill_1k"])
def test_forward_timed_matches_forward(gpu_lib, name):
    w = [s for s in SMALL if s.name == name][0]
    x = to_dev(synth.make_inputs(w, seed=8))
    p = dsa.make_problem(w.batch, w.n_q, w.n_k, w.q_pos0, w.d_idx, w.idx_dtype, w.top_k,
                         w.n_heads)
    fwd = dsa.Forward(p, "cuda")
    outs = []
    for timed in (False, True):
        O = torch.empty_like(x["Q"])
        idx = torch.empty((w.batch, w.n_q, w.top_k), dtype=torch.int32, device="cuda")
        lse = torch.empty((w.batch, w.n_q, w.n_heads), dtype=torch.float32, device="cuda")
        if timed:
            ms, slabs = fwd.timed(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"], O, idx, lse)
            assert slabs == 1 and all(t > 0 for t in ms), ms
        else:
            fwd(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"], O, idx, lse)
        torch.cuda.synchronize()
        outs.append((idx, O, lse))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))
