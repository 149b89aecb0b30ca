"""Seeded synthetic inputs for the DSA indexer -> top-k -> sparse MQA attention path.

This module only draws random numbers and holds the workload shapes. It holds
none of the method's arithmetic, imports nothing else from this package, and
serves the GPU path, the oracle and the benchmark alike.

Workload shapes follow the DeepSeek-V3.2 DSA page (kwkr.cn/news/60693):
its parameter-tuning table (section 7.2) gives top_k / index_dim / precision
for 32K, 64K and 128K contexts, section 3.3 keeps 2048 keys per query at 128K,
and section 4.2 gives one K/V set shared by all query heads (MQA).

Recipe (every tensor has its own CPU generator seeded with seed*1000 + tid):
  * indexer inputs q_idx, k_idx: integers uniform in [-4, 4], stored as
    float8 e4m3fn (OCP) or bfloat16; both represent them exactly;
  * clustered keys: k_idx[b, j] = centroid[b, assign[b, j]] + noise[b, j],
    64 integer centroids per sequence in [-4, 4], integer noise in {-1, 0, 1},
    so values lie in [-5, 5] (still exact in e4m3fn);
  * Q [B, n_q, H, 128], K and V [B, n_k, 128]: N(0, 1) drawn in float32 and
    rounded to bfloat16;
  * ragged decode batches: each sequence's query position uniform in
    [n_k / 8, n_k - 1] (rows share the padded [B, n_k] layout);
  * paged layouts: the B * n_k / P pages of P keys placed at a seeded random
    permutation of a pool with 16 spare pages (page_pool()).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch

TID = {"q_idx": 1, "k_idx": 2, "Q": 3, "K": 4, "V": 5,
       "centroids": 6, "assign": 7, "noise": 8, "positions": 9, "pages": 10,
       "X": 11, "W_q": 12, "W_k": 13, "W_q_mask": 14, "W_k_mask": 15}

HEAD_DIM = 128
N_CENTROIDS = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    mode: str            # "prefill" or "decode"
    batch: int
    n_q: int
    n_k: int
    q_pos0: int          # query i of a sequence sits at position q_pos0 + i
    d_idx: int
    idx_dtype: str       # "fp8" (e4m3fn) or "bf16"
    top_k: int
    n_heads: int
    clustered: bool = False
    ragged: bool = False  # decode only: per-sequence query positions (positions())
    page_size: int = 0    # > 0: k_idx, K, V stored in shuffled pages of this many keys
    tau: Optional[float] = None  # threshold-mode selection: keys scoring above tau, <= top_k
    d_model: int = 0      # > 0: each step projects q_idx and the new k_idx rows from hidden
                          # states X [rows, d_model] (make_inputs parts "X", "W_q", "W_k")

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def torch_idx_dtype(self):
        return torch.float8_e4m3fn if self.idx_dtype == "fp8" else torch.bfloat16

    def positions(self, seed: int = 0):
        """Position of query 0 of every sequence: q_pos0, or for a ragged
        batch one seeded draw per sequence, uniform in [n_k / 8, n_k - 1]."""
        if not self.ragged:
            return [self.q_pos0] * self.batch
        g = _gen(seed, "positions", "cpu")
        return torch.randint(self.n_k // 8, self.n_k, (self.batch,), generator=g).tolist()

    def page_pool(self, seed: int = 0):
        """Physical page of every logical page, [B, n_k / P] (a seeded
        permutation of a pool of B * n_k / P + 16 pages), and the pool size."""
        per = self.n_k // self.page_size
        n_pages = self.batch * per + 16
        g = _gen(seed, "pages", "cpu")
        perm = torch.randperm(n_pages, generator=g)[: self.batch * per]
        return perm.reshape(self.batch, per).to(torch.int32), n_pages

    def n_selected(self, seed: int = 0) -> int:
        """Sum over queries of min(top_k, pos + 1): rows attended in total."""
        tot = 0
        for p0 in self.positions(seed):
            for i in range(self.n_q):
                tot += min(self.top_k, p0 + i + 1)
        return tot

    def n_causal_pairs(self, seed: int = 0) -> int:
        """Sum over queries of pos + 1: indexer scores computed in total."""
        n = self.n_q
        return sum(n * (p0 + 1) + n * (n - 1) // 2 for p0 in self.positions(seed))


def _prefill(name, L, d, dt, k, H, **kw):
    return Workload(name, "prefill", 1, L, L, 0, d, dt, k, H, **kw)


def _decode(name, B, L, d, dt, k, H, **kw):
    return Workload(name, "decode", B, 1, L, L - 1, d, dt, k, H, **kw)


# The five workloads: a 1K prefill small enough for the oracle, the pages'
# 32K / 64K / 128K settings, and a clustered-key 128K decode batch.
WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        _prefill("prefill_1k", 1024, 128, "fp8", 64, 8),
        _decode("decode_32k", 32, 32768, 96, "fp8", 1024, 16),
        _prefill("prefill_64k", 65536, 128, "fp8", 1536, 16),
        _prefill("prefill_128k", 131072, 160, "bf16", 2048, 16),
        _decode("decode_128k_clustered", 64, 131072, 128, "fp8", 2048, 16,
                clustered=True),
    ]
}
# A ragged 128K decode batch (sequence lengths spread over the context), and
# the same batch over paged layouts (256- and 16-key pages in shuffled pools).
WORKLOADS["decode_128k_ragged"] = Workload("decode_128k_ragged", "decode", 64, 1, 131072, 0,
                                           128, "fp8", 2048, 16, ragged=True)
WORKLOADS["decode_128k_paged"] = WORKLOADS["decode_128k_ragged"].replace(
    name="decode_128k_paged", page_size=256)
WORKLOADS["decode_128k_paged16"] = WORKLOADS["decode_128k_ragged"].replace(
    name="decode_128k_paged16", page_size=16)
# The clustered 128K decode batch and the 64K prefill with the indexer
# projection front-end (model width 4096, as the DSA page's "usual 4096
# dimensions"): a decode step projects each sequence's query and appends its
# new key row at the sequence's position; a prefill projects every token's
# query and key.
WORKLOADS["decode_128k_projected"] = WORKLOADS["decode_128k_clustered"].replace(
    name="decode_128k_projected", d_model=4096)
WORKLOADS["prefill_64k_projected"] = WORKLOADS["prefill_64k"].replace(
    name="prefill_64k_projected", d_model=4096)
# The clustered 128K decode batch in threshold mode: tau = 14 keeps from about
# 200 to several thousand keys per query on these inputs, so some rows keep
# all their passing keys and others are cut to the top_k highest.
WORKLOADS["decode_128k_threshold"] = WORKLOADS["decode_128k_clustered"].replace(
    name="decode_128k_threshold", tau=14.0)


def _gen(seed: int, tid: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + TID[tid])
    return g


def _ints(shape, lo, hi, seed, tid, device):
    return torch.randint(lo, hi + 1, shape, generator=_gen(seed, tid, device),
                         dtype=torch.int16, device=device)


def _normal_bf16(shape, seed, tid, device):
    x = torch.randn(shape, generator=_gen(seed, tid, device),
                    dtype=torch.float32, device=device)
    return x.to(torch.bfloat16)


def make_inputs(w: Workload, seed: int = 0, device: str = "cpu",
                parts: Optional[tuple] = None) -> Dict[str, torch.Tensor]:
    """Draw the inputs of workload `w`.

    device="cpu" is the canonical draw (the one parity tests use). A CUDA
    device draws the same distributions with the device's own generator,
    which gives different numbers; it exists so that large benchmark inputs
    need not cross PCIe.
    """
    want = set(parts) if parts else {"q_idx", "k_idx", "Q", "K", "V"}
    B, nq, nk, d = w.batch, w.n_q, w.n_k, w.d_idx
    out = {}
    if "q_idx" in want:
        out["q_idx"] = _ints((B, nq, d), -4, 4, seed, "q_idx", device).to(
            w.torch_idx_dtype)
    if "k_idx" in want:
        if w.clustered:
            cent = _ints((B, N_CENTROIDS, d), -4, 4, seed, "centroids", device)
            a = torch.randint(0, N_CENTROIDS, (B, nk), dtype=torch.int64,
                              generator=_gen(seed, "assign", device),
                              device=device)
            k = torch.empty((B, nk, d), dtype=w.torch_idx_dtype, device=device)
            step = 1 << 14
            g_noise = _gen(seed, "noise", device)
            for b in range(B):
                for j0 in range(0, nk, step):
                    j1 = min(nk, j0 + step)
                    noise = torch.randint(-1, 2, (j1 - j0, d), generator=g_noise,
                                          dtype=torch.int16, device=device)
                    k[b, j0:j1] = (cent[b][a[b, j0:j1]] + noise).to(
                        w.torch_idx_dtype)
            out["k_idx"] = k
        else:
            out["k_idx"] = _ints((B, nk, d), -4, 4, seed, "k_idx", device).to(
                w.torch_idx_dtype)
    if "Q" in want:
        out["Q"] = _normal_bf16((B, nq, w.n_heads, HEAD_DIM), seed, "Q", device)
    if "K" in want:
        out["K"] = _normal_bf16((B, nk, HEAD_DIM), seed, "K", device)
    if "V" in want:
        out["V"] = _normal_bf16((B, nk, HEAD_DIM), seed, "V", device)
    if w.d_model and (parts is None or "X" in want):
        # hidden states: integers in [-3, 3]; weights: {-1, 0, 1}, nonzero with
        # probability 1/16 (projected values stay exact and well inside fp8)
        rows = B * nq
        out["X"] = _ints((rows, w.d_model), -3, 3, seed, "X", device).to(torch.bfloat16)
        for name in ("W_q", "W_k"):
            wv = _ints((d, w.d_model), -1, 1, seed, name, device)
            keep = _ints((d, w.d_model), 0, 15, seed, name + "_mask", device) == 0
            out[name] = (wv * keep).to(torch.bfloat16)
    return out
