// C ABI of the DSA library: argument validation, workspace layout and the
// launch sequence of each call. Every check runs on the host before anything
// is enqueued; the library allocates no device memory.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/dsa.h"
#include "dsa_internal.h"

namespace {

thread_local std::string g_last_error;

dsa_status fail(dsa_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

dsa_status ok() {
    g_last_error.clear();
    return DSA_OK;
}

constexpr long long kMaxKeys = 4194304;
constexpr int kMaxTopK = 4096;
constexpr int kMaxHeads = 16;
constexpr int kMaxModelWidth = 65536;
constexpr int kHeadDim = 128;
constexpr size_t kAlign = 256;
constexpr size_t kScoreSlabBytes = size_t(2) << 30;  // score rows staged per forward pass
constexpr size_t kPrefillSlabBytes = size_t(12) << 30;  // candidate lists per forward pass
constexpr size_t kPartFloats = 16 * (kHeadDim + 4);   // attention partial per (task)

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

dsa_status check_problem(const dsa_problem* p) {
    if (!p) return fail(DSA_E_NULL, "problem is NULL");
    if (p->batch < 1 || p->n_q < 1 || p->n_k < 1 || p->q_pos0 < 0)
        return fail(DSA_E_SHAPE, "batch, n_q, n_k must be >= 1 and q_pos0 >= 0 "
                    "(got batch=%d n_q=%d n_k=%d q_pos0=%d)", p->batch, p->n_q, p->n_k, p->q_pos0);
    if (p->n_k > kMaxKeys)
        return fail(DSA_E_SHAPE, "n_k=%d exceeds %lld", p->n_k, kMaxKeys);
    if ((long long)p->q_pos0 + p->n_q > p->n_k)
        return fail(DSA_E_SHAPE, "q_pos0 + n_q = %lld exceeds n_k = %d",
                    (long long)p->q_pos0 + p->n_q, p->n_k);
    if (p->d_idx < 1) return fail(DSA_E_SHAPE, "d_idx=%d must be positive", p->d_idx);
    if (p->d_idx % 32 != 0 || p->d_idx > 256)
        return fail(DSA_E_UNSUPPORTED, "d_idx=%d must be a multiple of 32 in [32, 256]", p->d_idx);
    if (p->idx_dtype != DSA_IDX_FP8_E4M3FN && p->idx_dtype != DSA_IDX_BF16)
        return fail(DSA_E_UNSUPPORTED, "idx_dtype=%d is neither fp8 e4m3fn (0) nor bf16 (1)",
                    p->idx_dtype);
    if (p->top_k < 1) return fail(DSA_E_SHAPE, "top_k=%d must be >= 1", p->top_k);
    if (p->top_k > kMaxTopK)
        return fail(DSA_E_UNSUPPORTED, "top_k=%d exceeds %d", p->top_k, kMaxTopK);
    if (p->n_heads < 1) return fail(DSA_E_SHAPE, "n_heads=%d must be >= 1", p->n_heads);
    if (p->n_heads > kMaxHeads)
        return fail(DSA_E_UNSUPPORTED, "n_heads=%d exceeds %d", p->n_heads, kMaxHeads);
    if (p->head_dim != kHeadDim)
        return fail(DSA_E_UNSUPPORTED, "head_dim=%d must be %d", p->head_dim, kHeadDim);
    const long long rows = (long long)p->batch * p->n_q;
    if (rows * p->top_k > (1LL << 40) || rows > (1LL << 31))
        return fail(DSA_E_SHAPE, "batch * n_q = %lld is too large", rows);
    return DSA_OK;
}

dsa_status check_ptrs(std::initializer_list<const void*> ptrs, const char* names) {
    int i = 0;
    for (const void* q : ptrs) {
        if (!q) return fail(DSA_E_NULL, "required pointer #%d of (%s) is NULL", i, names);
        if (misaligned(q))
            return fail(DSA_E_ALIGN, "pointer #%d of (%s) is not 16-byte aligned", i, names);
        ++i;
    }
    return DSA_OK;
}

float index_scale(int d) { return (float)std::pow((double)d, -0.5); }

// Rows of each sequence whose scores one forward pass stages at a time.
int slab_rows(const dsa_problem* p) {
    const size_t row_bytes = (size_t)p->batch * p->n_k * sizeof(float);
    size_t r = kScoreSlabBytes / row_bytes;
    if (r < 1) r = 1;
    if (r > (size_t)p->n_q) r = (size_t)p->n_q;
    return (int)r;
}

// Attention workspace: per-(row, split) partials (none when every row is
// handled by one wave).
size_t attn_ws_bytes(const dsa_problem* p) {
    int ns, len;
    dsa::attn_split_plan(p->batch, p->n_q, p->top_k, &ns, &len);
    if ((long long)p->batch * p->n_q >= 2048) return 0;
    return align_up((size_t)p->batch * p->n_q * ns * kPartFloats * sizeof(float));
}


// Workspace of dsa_topk: the chunked schedule's buffers for the largest row
// slab that uses it (the schedule is chosen by batch * rows, so smaller slabs
// need less).
size_t topk_ws_bytes_max(const dsa_problem* p) {
    for (int rows = p->n_q < 256 ? p->n_q : 256; rows >= 1; --rows)
        if (dsa::topk_use_chunked(p->batch, rows, p->n_k))
            return align_up(dsa::topk_ws_bytes(p->batch, rows, p->n_k));
    return 0;
}

// Slabs of the many-row path: slab s holds query rows s, s + n, s + 2n, ...
// (n slabs), so every slab mixes short and long rows; the candidate lists of
// one slab stay within kPrefillSlabBytes.
// Tests can cap the rows of a slab instead (dsa_internal_set_prefill_slab_rows),
// so that small problems run as several slabs.
std::atomic<int> g_prefill_slab_rows{0};

int prefill_maxlen(const dsa_problem* p) {
    const long long m = (long long)p->q_pos0 + p->n_q;
    return (int)(m < p->n_k ? m : p->n_k);
}

// Shortest key rows that take the sampled-threshold decode selection beyond
// the kernels' own limit (tests raise it to run long rows on score rows).
std::atomic<int> g_select_min_keys{0};

bool decode_select_on(int rows, int n_k, int top_k) {
    return n_k >= g_select_min_keys.load() && dsa::decode_select_applies(rows, n_k, top_k);
}

// Many query rows per sequence over short key rows take the score-row path
// (scores of every causal pair into the workspace, exact per-row radix
// selection on them) when the whole score matrix fits one slab: with short
// rows the sampled threshold, candidate filter and select cost more launches
// and passes than writing and reading the scores. Tests move the limit
// (dsa_internal_set_prefill_direct) to run either path at small sizes.
constexpr int kPrefillDirectMaxKeys = 4096;  // faster at every size measured up to 4096 keys
std::atomic<int> g_prefill_direct_max{kPrefillDirectMaxKeys};

bool prefill_direct(const dsa_problem* p) {
    return p->n_q > 1 && p->n_k <= g_prefill_direct_max.load() &&
           (size_t)p->batch * p->n_q * p->n_k * sizeof(float) <= kScoreSlabBytes;
}

// The many-row path (sampled threshold, candidate filter, select).
bool prefill_many_row(const dsa_problem* p) { return p->n_q > 1 && !prefill_direct(p); }

// Key ranges per row of the many-row path, decided once for the problem.
int prefill_nr(const dsa_problem* p) {
    return dsa::prefill_nranges(prefill_maxlen(p), (long long)p->batch * p->n_q);
}

int prefill_slabs(const dsa_problem* p) {
    const size_t row_bytes =
        (size_t)p->batch * prefill_nr(p) * dsa::prefill_cap(p->top_k) * 8;
    size_t per = kPrefillSlabBytes / row_bytes > 0 ? kPrefillSlabBytes / row_bytes : 1;
    const int cap_rows = g_prefill_slab_rows.load();
    if (cap_rows > 0 && per > (size_t)cap_rows) per = (size_t)cap_rows;
    return (int)(((size_t)p->n_q + per - 1) / per);
}

int prefill_slab_rows(const dsa_problem* p) {
    const int n = prefill_slabs(p);
    return (p->n_q + n - 1) / n;
}

struct ForwardLayout {
    size_t scores, idx, topk, part, prow, done, total;
};

// Threshold mode's per-row flags (rows a select kernel finished) sit after
// everything else.
ForwardLayout with_done(ForwardLayout L, const dsa_problem* p) {
    L.done = L.total;
    L.total += align_up((size_t)p->batch * p->n_q * sizeof(uint32_t));
    return L;
}

ForwardLayout forward_layout_core(const dsa_problem* p) {
    ForwardLayout L;
    L.scores = 0;
    if (prefill_many_row(p)) {
        // many rows: candidate lists and thresholds, no score rows
        const size_t ib = align_up((size_t)p->batch * p->n_q * p->top_k * sizeof(int32_t));
        L.idx = 0;
        L.topk = ib;
        const size_t pw = align_up(dsa::prefill_ws_bytes(p->batch, prefill_slab_rows(p), p->n_k,
                                                         p->top_k, prefill_nr(p)));
        if (dsa::attn_ranged_applies(p->batch, p->n_q, p->n_k)) {
            // the key-range attention's partials reuse the select's buffers,
            // which are dead once the last slab's select has run
            const size_t rw =
                align_up(dsa::attn_ranged_ws_bytes(p->batch, p->n_q, p->n_k, p->q_pos0));
            L.part = L.topk;
            L.total = L.topk + (pw > rw ? pw : rw);
            return L;
        }
        L.part = L.topk + pw;
        L.total = L.part + attn_ws_bytes(p);
        return L;
    }
    const int R = slab_rows(p);
    const size_t sb = align_up((size_t)p->batch * R * p->n_k * sizeof(float));
    L.idx = sb;
    const size_t ib = align_up((size_t)p->batch * p->n_q * p->top_k * sizeof(int32_t));
    L.topk = L.idx + ib;
    size_t tb = align_up(dsa::topk_ws_bytes(p->batch, R, p->n_k));
    if (decode_select_on(R, p->n_k, p->top_k)) {
        const size_t db = align_up(dsa::decode_select_ws_bytes(p->batch, p->n_k, p->top_k));
        tb = db > tb ? db : tb;
    }
    L.part = L.topk + tb;
    // pool rows of the selection, for a paged layout's attention
    L.prow = L.part + align_up(attn_ws_bytes(p));
    L.total = L.prow + ib;
    return L;
}

ForwardLayout forward_layout(const dsa_problem* p) { return with_done(forward_layout_core(p), p); }

// Order key of a float (float order as unsigned order, -0.0 with +0.0), as
// the select kernels rank scores.
uint32_t order_key(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

dsa_status hip_fail(hipError_t e, const char* what) {
    return fail(DSA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

dsa::AttnArgs attn_args(const dsa_problem* p, const void* Q, const void* K, const void* V,
                        const int32_t* idx, void* O, float* lse, void* part) {
    dsa::AttnArgs a{};
    a.kv_bstride = p->n_k;
    a.kv_rows = p->n_k;
    a.Q = static_cast<const uint16_t*>(Q);
    a.K = static_cast<const uint16_t*>(K);
    a.V = static_cast<const uint16_t*>(V);
    a.idx = idx;
    a.O = static_cast<uint16_t*>(O);
    a.lse = lse;
    a.part = static_cast<float*>(part);
    a.B = p->batch;
    a.n_q = p->n_q;
    a.n_k = p->n_k;
    a.H = p->n_heads;
    a.k = p->top_k;
    dsa::attn_split_plan(p->batch, p->n_q, p->top_k, &a.n_split, &a.split_len);
    return a;
}

// HIP events recorded between the stages of a forward call (profiling).
// mark(s) starts a segment charged to stage s (0 indexer, 1 top-k,
// 2 attention; -1 ends the last segment).
struct StageTimer {
    hipStream_t st;
    std::vector<std::pair<int, hipEvent_t>> marks;
    hipError_t err = hipSuccess;
    void mark(int stage) {
        hipEvent_t e = nullptr;
        if (err == hipSuccess) err = hipEventCreate(&e);
        if (err == hipSuccess) err = hipEventRecord(e, st);
        if (err == hipSuccess) marks.push_back({stage, e});
    }
    hipError_t finish(float* ms) {
        if (err == hipSuccess && !marks.empty()) err = hipEventSynchronize(marks.back().second);
        for (size_t i = 0; err == hipSuccess && i + 1 < marks.size(); ++i) {
            float t = 0.f;
            err = hipEventElapsedTime(&t, marks[i].second, marks[i + 1].second);
            if (marks[i].first >= 0) ms[marks[i].first] += t;
        }
        for (auto& m : marks) hipEventDestroy(m.second);
        marks.clear();
        return err;
    }
};

// Host-side launch log: with DSA_LOG set to a non-empty value other than
// "0", every forward call prints one line to stderr naming the problem, the
// selection path it takes and the workspace it uses.
bool log_on() {
    const char* v = std::getenv("DSA_LOG");
    return v && v[0] && !(v[0] == '0' && v[1] == 0);
}

void log_forward(const dsa_problem* p, const char* path, int slabs, size_t ws_bytes,
                 const int32_t* seq_pos, const dsa::KeyPages* pages, const float* tau) {
    std::fprintf(stderr,
                 "dsa: forward B=%d n_q=%d n_k=%d q_pos0=%d d_idx=%d %s top_k=%d H=%d%s%s%s: %s, "
                 "%d slab(s), workspace %zu bytes\n",
                 p->batch, p->n_q, p->n_k, p->q_pos0, p->d_idx, p->idx_dtype ? "bf16" : "fp8",
                 p->top_k, p->n_heads, seq_pos ? ", ragged" : "", pages ? ", paged" : "",
                 tau ? ", threshold mode" : "", path, slabs, ws_bytes);
}

dsa_status forward_impl(const dsa_problem* p, const void* q_idx, const void* k_idx,
                        const void* Q, const void* K, const void* V, int32_t* idx_out, void* O,
                        float* lse, void* ws, size_t ws_bytes, void* stream, StageTimer* tm,
                        int32_t* n_slabs, const int32_t* seq_pos = nullptr,
                        const dsa::KeyPages* pages = nullptr, const float* tau = nullptr) {
    dsa_status s = check_problem(p);
    if (s != DSA_OK) return s;
    if ((s = check_ptrs({q_idx, k_idx, Q, K, V, O}, "q_idx, k_idx, Q, K, V, O")) != DSA_OK)
        return s;
    if (idx_out && misaligned(idx_out)) return fail(DSA_E_ALIGN, "idx_out is not 16-byte aligned");
    if (lse && misaligned(lse)) return fail(DSA_E_ALIGN, "lse is not 16-byte aligned");
    const ForwardLayout L = forward_layout(p);
    if (!ws || ws_bytes < L.total)
        return fail(DSA_E_WORKSPACE, "forward needs %zu workspace bytes (got %zu)", L.total,
                    ws ? ws_bytes : (size_t)0);
    if (misaligned(ws)) return fail(DSA_E_ALIGN, "workspace is not 16-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* w = static_cast<char*>(ws);
    float* scores = reinterpret_cast<float*>(w + L.scores);
    int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(w + L.idx);
    const int R = slab_rows(p);
    // Threshold mode: a negative tau keeps every key (the top-k result); else
    // the select kernels and the rescoring pass drop scores not above tau.
    dsa::ScoreFloor floor{};
    const bool floor_on = tau && !(*tau < 0.0f);
    if (floor_on) {
        floor.on = 1;
        floor.key = *tau != *tau ? 0xffffffffu : order_key(*tau);
        floor.done = reinterpret_cast<uint32_t*>(w + L.done);
        hipError_t e = dsa::launch_floor_reset(floor.done, (long long)p->batch * p->n_q, st);
        if (e != hipSuccess) return hip_fail(e, "threshold reset launch");
    }

    dsa::IndexArgs ia{};
    ia.q = q_idx;
    ia.k = k_idx;
    ia.scores = scores;
    ia.B = p->batch;
    ia.n_q = p->n_q;
    ia.n_k = p->n_k;
    ia.q_pos0 = p->q_pos0;
    ia.d = p->d_idx;
    ia.dtype = p->idx_dtype;
    ia.scale = index_scale(p->d_idx);
    ia.write_masked = 0;  // the selection never reads past a query's position
    ia.seq_pos = seq_pos;
    if (pages) ia.pages = *pages;
    dsa::TopkArgs ta{};
    ta.scores = scores;
    ta.idx = idx;
    ta.B = p->batch;
    ta.n_k = p->n_k;
    ta.k = p->top_k;
    ta.idx_rows = p->n_q;
    ta.seq_pos = seq_pos;
    ta.ws = w + L.topk;
    int slabs = 0;
    const bool many_row = prefill_many_row(p);
    if (many_row) {
        // Many query rows: threshold, indexer sweep keeping candidates,
        // per-row select and fallback, slab by slab.
        const int NS = prefill_slabs(p);
        for (int s0 = 0; s0 < NS; ++s0, ++slabs) {
            dsa::PrefillArgs pa{};
            pa.q = q_idx;
            pa.k = k_idx;
            pa.idx = idx;
            pa.B = p->batch;
            pa.n_q = p->n_q;
            pa.n_k = p->n_k;
            pa.q_pos0 = p->q_pos0;
            pa.d = p->d_idx;
            pa.dtype = p->idx_dtype;
            pa.top_k = p->top_k;
            pa.row0 = s0;
            pa.rstride = NS;
            pa.rows = (p->n_q - s0 + NS - 1) / NS;
            pa.scale = index_scale(p->d_idx);
            pa.nr = prefill_nr(p);
            pa.floor = floor;
            static const char* what[4] = {"prefill threshold launch", "prefill indexer launch",
                                          "prefill select launch", "prefill fallback launch"};
            static const int stage[4] = {1, 0, 1, 1};
            for (int part = 0; part < 4; ++part) {
                if (tm) tm->mark(stage[part]);
                hipError_t e = dsa::launch_prefill_select(pa, ta.ws, part, st);
                if (e != hipSuccess) return hip_fail(e, what[part]);
            }
        }
    }
    for (int r0 = 0; !many_row && r0 < p->n_q; r0 += R, ++slabs) {
        const int r1 = r0 + R < p->n_q ? r0 + R : p->n_q;
        ia.q_begin = r0;
        ia.q_end = r1;
        ta.rows = r1 - r0;
        ta.pos_begin = (long long)p->q_pos0 + r0;
        ta.idx_row0 = r0;
        if (decode_select_on(ta.rows, p->n_k, p->top_k)) {
            // One query row per sequence: sampled threshold, indexer that
            // keeps only candidates, exact select; no score row is written.
            dsa::DecodeArgs da{};
            da.q = q_idx;
            da.k = k_idx;
            da.idx = idx;
            da.B = p->batch;
            da.n_q = p->n_q;
            da.n_k = p->n_k;
            da.q_pos0 = p->q_pos0;
            da.d = p->d_idx;
            da.dtype = p->idx_dtype;
            da.top_k = p->top_k;
            da.q_row = r0;
            da.idx_rows = p->n_q;
            da.idx_row0 = r0;
            da.scale = index_scale(p->d_idx);
            da.fallback = scores;
            da.seq_pos = seq_pos;
            if (pages) da.pages = *pages;
            da.floor = floor;
            hipError_t e = hipSuccess;
            if (tm) tm->mark(1);
            if ((e = dsa::launch_decode_select(da, ta.ws, 0, st)) != hipSuccess)
                return hip_fail(e, "decode threshold launch");
            if (tm) tm->mark(0);
            if ((e = dsa::launch_decode_select(da, ta.ws, 1, st)) != hipSuccess)
                return hip_fail(e, "decode indexer launch");
            if (tm) tm->mark(1);
            if ((e = dsa::launch_decode_select(da, ta.ws, 2, st)) != hipSuccess)
                return hip_fail(e, "decode select launch");
            continue;
        }
        // One query per sequence on the chunked top-k schedule: the indexer
        // kernel builds the row histograms the selection starts from.
        const bool fuse = ta.rows == 1 && dsa::topk_use_chunked(p->batch, 1, p->n_k);
        ia.hist = fuse ? dsa::topk_hist_ptr(ta.ws) : nullptr;
        ta.hist_ready = fuse ? 1 : 0;
        hipError_t e = hipSuccess;
        if (tm) tm->mark(1);
        if (fuse && (e = dsa::launch_topk_prepare(ta, ta.ws, st)) != hipSuccess)
            return hip_fail(e, "topk prepare launch");
        if (tm) tm->mark(0);
        e = dsa::launch_index_scores(ia, st);
        if (e != hipSuccess) return hip_fail(e, "index_scores launch");
        if (tm) tm->mark(1);
        e = dsa::launch_topk(ta, st);
        if (e != hipSuccess) return hip_fail(e, "topk launch");
    }
    if (floor_on) {
        // threshold mode: drop the selected keys scoring at or below tau in
        // the rows no select kernel has finished
        dsa::FloorArgs fa{};
        fa.q = q_idx;
        fa.k = k_idx;
        fa.idx = idx;
        fa.B = p->batch;
        fa.n_q = p->n_q;
        fa.n_k = p->n_k;
        fa.d = p->d_idx;
        fa.dtype = p->idx_dtype;
        fa.top_k = p->top_k;
        fa.scale = index_scale(p->d_idx);
        fa.tau = *tau;
        fa.done = floor.done;
        if (pages) fa.pages = *pages;
        if (tm) tm->mark(1);
        hipError_t e = dsa::launch_threshold_floor(fa, st);
        if (e != hipSuccess) return hip_fail(e, "threshold launch");
    }
    if (tm) tm->mark(2);
    dsa::AttnArgs aa = attn_args(p, Q, K, V, idx, O, lse, w + L.part);
    if (pages) {
        // the attention reads pool rows: translate the selection
        int32_t* prow = reinterpret_cast<int32_t*>(w + L.prow);
        hipError_t e = dsa::launch_page_rows(idx, prow, p->batch, p->n_q * p->top_k, p->n_k,
                                             *pages, st);
        if (e != hipSuccess) return hip_fail(e, "page rows launch");
        aa.idx = prow;
        aa.kv_bstride = 0;
        aa.kv_rows = pages->n_pages * pages->page;
    }
    if (p->n_q > 1 && dsa::attn_ranged_applies(p->batch, p->n_q, p->n_k))
        dsa::attn_set_ranged(aa, p->q_pos0, w + L.part);  // idx rows are sorted and causal
    hipError_t e = dsa::launch_sparse_attn(aa, st);
    if (e != hipSuccess) return hip_fail(e, "sparse_attn launch");
    if (tm) tm->mark(-1);
    if (n_slabs) *n_slabs = slabs;
    if (log_on()) {
        const char* path;
        char buf[96];
        if (many_row) {
            std::snprintf(buf, sizeof buf, "many-row selection (%d key range(s), list cap %d)",
                          prefill_nr(p), dsa::prefill_cap(p->top_k));
            path = buf;
        } else if (p->n_q == 1 && decode_select_on(R, p->n_k, p->top_k)) {
            path = "decode selection (sampled threshold, candidate filter, select)";
        } else {
            path = "score rows and per-row selection";
        }
        log_forward(p, path, slabs, L.total, seq_pos, pages, tau);
    }
    return DSA_OK;
}

dsa_status check_project_sizes(int32_t rows, int32_t d_model, int32_t d_idx) {
    if (rows < 1) return fail(DSA_E_SHAPE, "rows=%d must be >= 1", rows);
    if (d_model < 32 || d_model % 32 != 0 || d_model > kMaxModelWidth)
        return fail(DSA_E_UNSUPPORTED, "d_model=%d must be a multiple of 32 in [32, %d]", d_model,
                    kMaxModelWidth);
    if (d_idx < 32 || d_idx % 32 != 0 || d_idx > 256)
        return fail(DSA_E_UNSUPPORTED, "d_idx=%d must be a multiple of 32 in [32, 256]", d_idx);
    if ((long long)rows * d_model > (1LL << 40))
        return fail(DSA_E_SHAPE, "rows * d_model = %lld is too large",
                    (long long)rows * d_model);
    return DSA_OK;
}

// Arguments a ragged batch adds to those of dsa_forward.
dsa_status check_ragged(const dsa_problem* p, const int32_t* seq_pos) {
    dsa_status s = check_problem(p);
    if (s != DSA_OK) return s;
    if (!seq_pos) return fail(DSA_E_NULL, "seq_pos is NULL");
    if (misaligned(seq_pos)) return fail(DSA_E_ALIGN, "seq_pos is not 16-byte aligned");
    if (p->q_pos0 != 0)
        return fail(DSA_E_SHAPE,
                    "a ragged batch takes its positions from seq_pos (q_pos0 = %d, need 0)",
                    p->q_pos0);
    if (p->n_q != 1)
        return fail(DSA_E_UNSUPPORTED, "ragged batches take one query per sequence (n_q = %d)",
                    p->n_q);
    return DSA_OK;
}

// A paged layout's description, checked and copied into kp.
dsa_status check_paged(const dsa_problem* p, const int32_t* seq_pos, const dsa_pages* pg,
                       dsa::KeyPages* kp) {
    dsa_status s = check_ragged(p, seq_pos);
    if (s != DSA_OK) return s;
    if (!pg || !pg->block_table) return fail(DSA_E_NULL, "pages or pages->block_table is NULL");
    if (misaligned(pg->block_table))
        return fail(DSA_E_ALIGN, "pages->block_table is not 16-byte aligned");
    if (pg->page_size < 1) return fail(DSA_E_SHAPE, "page_size = %d", pg->page_size);
    if (pg->pages_per_seq < 1 || (long long)pg->pages_per_seq * pg->page_size != p->n_k)
        return fail(DSA_E_SHAPE, "pages_per_seq * page_size must equal n_k (%d * %d != %d)",
                    pg->pages_per_seq, pg->page_size, p->n_k);
    // attention rows are addressed with 32-bit byte offsets into the K/V pools
    if (pg->n_pages < 1 || (long long)pg->n_pages * pg->page_size * 256 > 0xffffffffLL)
        return fail(DSA_E_SHAPE, "n_pages = %d: the K/V pools must hold 1 page and < 4 GiB",
                    pg->n_pages);
    kp->table = pg->block_table;
    kp->page = pg->page_size;
    kp->per_seq = pg->pages_per_seq;
    kp->n_pages = pg->n_pages;
    return DSA_OK;
}

// Scratch of dsa_forward_noalloc: a file-scope device array, so that the
// call needs neither an allocation nor a caller workspace. Every GPU the
// library runs on holds its own copy (at its own address) until the process
// ends; each call on a GPU overwrites that GPU's copy, so calls that overlap
// on one GPU race. In host code `scratch` names a host-side stand-in, never
// the device memory: kernels get the address hipGetSymbolAddress returns.
constexpr size_t kScratchBytes = DSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current GPU's scratch array, looked up once per
// device (with that device current) and kept. The stream must belong to the
// current device.
dsa_status scratch_address(hipStream_t st, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(DSA_E_UNSUPPORTED, "device %d is outside the %d devices this call tracks",
                    dev, kMaxDevices);
    if (st) {
        hipDevice_t sd = -1;
        e = hipStreamGetDevice(st, &sd);
        if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
        if ((int)sd != dev)
            return fail(DSA_E_UNSUPPORTED,
                        "the stream belongs to device %d while device %d is current; make the "
                        "stream's device current", (int)sd, dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(DSA_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return DSA_OK;
}

}  // namespace

extern "C" {

// Not part of the public interface: caps the query rows of one many-row slab
// (0 restores the default, set by a 12 GiB budget for the candidate lists)
// and returns the previous cap. Tests use it to run small prefill problems as
// several slabs; the workspace size of a forward call follows the cap in
// force when it is asked for, so a caller must not change it between sizing
// and calling.
int32_t dsa_internal_set_prefill_slab_rows(int32_t rows) {
    return g_prefill_slab_rows.exchange(rows > 0 ? rows : 0);
}

// Not part of the public interface: the longest key rows (n_k) with which a
// many-row problem takes the score-row path instead of the many-row path
// (0 never; a negative value restores the default). Returns the previous
// limit. The workspace size follows the limit in force when it is asked
// for, so a caller must not change it between sizing and calling.
int32_t dsa_internal_set_prefill_direct(int32_t max_keys) {
    return g_prefill_direct_max.exchange(max_keys < 0 ? kPrefillDirectMaxKeys : max_keys);
}

// Not part of the public interface: the shortest key rows (n_k) with which a
// one-query-per-sequence problem takes the sampled-threshold decode
// selection instead of score rows (0 restores the default). Returns the
// previous value; workspace sizes follow the value in force when asked for.
int32_t dsa_internal_set_decode_select_min(int32_t n_k) {
    return g_select_min_keys.exchange(n_k > 0 ? n_k : 0);
}

// Not part of the public interface: selection statistics of the last
// forward call on this problem and workspace (blocking: synchronises the
// device, then copies counters back). out[0] rows longer than top_k (the
// last slab's rows for a many-row problem), out[1] candidates the indexer
// kept for them, out[2] rows recomputed by a fallback, out[3] rows whose
// candidate lists overflowed. Problems on the score-row schedule report
// out[1..3] = -1. seq_pos: the ragged batch's device positions, or NULL.
dsa_status dsa_internal_selection_stats(const dsa_problem* p, const void* ws, size_t ws_bytes,
                                        const int32_t* seq_pos, int64_t* out) {
    dsa_status s = check_problem(p);
    if (s != DSA_OK) return s;
    if (!ws || !out) return fail(DSA_E_NULL, "ws and out must not be NULL");
    const ForwardLayout L = forward_layout(p);
    if (ws_bytes < L.total) return fail(DSA_E_WORKSPACE, "workspace smaller than the forward's");
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
    const char* w = static_cast<const char*>(ws);
    long long o[4] = {0, -1, -1, -1};
    if (prefill_many_row(p)) {
        const int NS = prefill_slabs(p);
        dsa::PrefillArgs pa{};
        pa.B = p->batch;
        pa.n_q = p->n_q;
        pa.n_k = p->n_k;
        pa.q_pos0 = p->q_pos0;
        pa.top_k = p->top_k;
        pa.row0 = NS - 1;
        pa.rstride = NS;
        pa.rows = (p->n_q - (NS - 1) + NS - 1) / NS;
        pa.nr = prefill_nr(p);
        e = dsa::prefill_stats(pa, w + L.topk, o);
    } else if (decode_select_on(slab_rows(p), p->n_k, p->top_k)) {
        std::vector<int32_t> sp;
        if (seq_pos) {
            sp.resize(p->batch);
            e = hipMemcpy(sp.data(), seq_pos, sp.size() * 4, hipMemcpyDeviceToHost);
        }
        if (e == hipSuccess)
            e = dsa::decode_stats(p->batch, p->n_k, p->q_pos0, seq_pos ? sp.data() : nullptr,
                                  p->top_k, w + L.topk, o);
    } else {
        o[0] = (long long)p->batch * p->n_q;
    }
    if (e != hipSuccess) return hip_fail(e, "selection statistics");
    for (int i = 0; i < 4; ++i) out[i] = o[i];
    return ok();
}

// Not part of the public interface: the many-row plan of a problem,
// out = {slabs, rows per slab, key ranges per row, keys per range,
// candidate-list capacity per (row, range), prefill workspace bytes}.
dsa_status dsa_internal_prefill_plan(const dsa_problem* p, int64_t* out) {
    dsa_status s = check_problem(p);
    if (s != DSA_OK) return s;
    if (!out) return fail(DSA_E_NULL, "out is NULL");
    const int nr = prefill_nr(p);
    out[0] = prefill_slabs(p);
    out[1] = prefill_slab_rows(p);
    out[2] = nr;
    out[3] = dsa::prefill_range_len(prefill_maxlen(p), nr);
    out[4] = dsa::prefill_cap(p->top_k);
    out[5] = (int64_t)dsa::prefill_ws_bytes(p->batch, prefill_slab_rows(p), p->n_k, p->top_k, nr);
    return ok();
}

dsa_status dsa_workspace_size(const dsa_problem* p, int32_t op, size_t* bytes) {
    if (!bytes) return fail(DSA_E_NULL, "bytes is NULL");
    dsa_status s = check_problem(p);
    if (s != DSA_OK) return s;
    switch (op) {
        case DSA_OP_TOPK: *bytes = topk_ws_bytes_max(p); break;
        case DSA_OP_ATTN: *bytes = attn_ws_bytes(p); break;
        case DSA_OP_FORWARD: *bytes = forward_layout(p).total; break;
        default: return fail(DSA_E_UNSUPPORTED, "unknown op %d", op);
    }
    return ok();
}

dsa_status dsa_index_scores(const dsa_problem* p, const void* q_idx, const void* k_idx,
                            int32_t q_begin, int32_t q_end, float* scores, void* stream) {
    dsa_status s = check_problem(p);
    if (s != DSA_OK) return s;
    if ((s = check_ptrs({q_idx, k_idx, scores}, "q_idx, k_idx, scores")) != DSA_OK) return s;
    if (q_begin < 0 || q_end > p->n_q || q_begin >= q_end)
        return fail(DSA_E_SHAPE, "need 0 <= q_begin < q_end <= n_q (got %d, %d, n_q=%d)",
                    q_begin, q_end, p->n_q);
    dsa::IndexArgs a{};
    a.q = q_idx;
    a.k = k_idx;
    a.scores = scores;
    a.B = p->batch;
    a.n_q = p->n_q;
    a.n_k = p->n_k;
    a.q_pos0 = p->q_pos0;
    a.d = p->d_idx;
    a.dtype = p->idx_dtype;
    a.q_begin = q_begin;
    a.q_end = q_end;
    a.scale = index_scale(p->d_idx);
    a.write_masked = 1;
    hipError_t e = dsa::launch_index_scores(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "index_scores launch");
    return ok();
}

dsa_status dsa_topk(const dsa_problem* p, const float* scores, int32_t q_begin, int32_t q_end,
                    int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
    dsa_status s = check_problem(p);
    if (s != DSA_OK) return s;
    if ((s = check_ptrs({scores, idx}, "scores, idx")) != DSA_OK) return s;
    if (q_begin < 0 || q_end > p->n_q || q_begin >= q_end)
        return fail(DSA_E_SHAPE, "need 0 <= q_begin < q_end <= n_q (got %d, %d, n_q=%d)",
                    q_begin, q_end, p->n_q);
    const size_t need = dsa::topk_ws_bytes(p->batch, q_end - q_begin, p->n_k);
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(DSA_E_WORKSPACE, "top-k needs %zu workspace bytes (got %zu)", need,
                    ws ? ws_bytes : (size_t)0);
    if (need > 0 && misaligned(ws)) return fail(DSA_E_ALIGN, "workspace is not 16-byte aligned");
    dsa::TopkArgs a{};
    a.scores = scores;
    a.idx = idx;
    a.B = p->batch;
    a.rows = q_end - q_begin;
    a.n_k = p->n_k;
    a.k = p->top_k;
    a.pos_begin = (long long)p->q_pos0 + q_begin;
    a.idx_rows = a.rows;
    a.idx_row0 = 0;
    a.ws = ws;
    a.hist_ready = 0;
    hipError_t e = dsa::launch_topk(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "topk launch");
    return ok();
}

dsa_status dsa_sparse_attn(const dsa_problem* p, const void* Q, const void* K, const void* V,
                           const int32_t* idx, void* O, float* lse, void* ws, size_t ws_bytes,
                           void* stream) {
    dsa_status s = check_problem(p);
    if (s != DSA_OK) return s;
    if ((s = check_ptrs({Q, K, V, idx, O}, "Q, K, V, idx, O")) != DSA_OK) return s;
    if (lse && misaligned(lse)) return fail(DSA_E_ALIGN, "lse is not 16-byte aligned");
    const size_t need = attn_ws_bytes(p);
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(DSA_E_WORKSPACE, "attention needs %zu workspace bytes (got %zu)", need,
                    ws ? ws_bytes : (size_t)0);
    if (need > 0 && misaligned(ws)) return fail(DSA_E_ALIGN, "workspace is not 16-byte aligned");
    dsa::AttnArgs a = attn_args(p, Q, K, V, idx, O, lse, ws);
    hipError_t e = dsa::launch_sparse_attn(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "sparse_attn launch");
    return ok();
}

dsa_status dsa_forward(const dsa_problem* p, const void* q_idx, const void* k_idx, const void* Q,
                       const void* K, const void* V, int32_t* idx_out, void* O, float* lse,
                       void* ws, size_t ws_bytes, void* stream) {
    dsa_status s = forward_impl(p, q_idx, k_idx, Q, K, V, idx_out, O, lse, ws, ws_bytes, stream,
                                nullptr, nullptr);
    return s == DSA_OK ? ok() : s;
}

dsa_status dsa_forward_noalloc(const dsa_problem* p, const void* q_idx, const void* k_idx,
                               const void* Q, const void* K, const void* V, int32_t* idx_out,
                               void* O, float* lse, void* stream) {
    dsa_status s = check_problem(p);
    if (s != DSA_OK) return s;
    const size_t need = forward_layout(p).total;
    if (need > kScratchBytes)
        return fail(DSA_E_WORKSPACE,
                    "dsa_forward_noalloc takes problems whose forward workspace fits its "
                    "%zu-byte static scratch; this one needs %zu bytes (call dsa_forward with a "
                    "workspace)", kScratchBytes, need);
    void* ws = nullptr;
    if ((s = scratch_address(static_cast<hipStream_t>(stream), &ws)) != DSA_OK) return s;
    s = forward_impl(p, q_idx, k_idx, Q, K, V, idx_out, O, lse, ws, kScratchBytes, stream,
                     nullptr, nullptr);
    return s == DSA_OK ? ok() : s;
}

dsa_status dsa_forward_ragged(const dsa_problem* p, const int32_t* seq_pos, const void* q_idx,
                              const void* k_idx, const void* Q, const void* K, const void* V,
                              int32_t* idx_out, void* O, float* lse, void* ws, size_t ws_bytes,
                              void* stream) {
    dsa_status s = check_ragged(p, seq_pos);
    if (s != DSA_OK) return s;
    s = forward_impl(p, q_idx, k_idx, Q, K, V, idx_out, O, lse, ws, ws_bytes, stream, nullptr,
                     nullptr, seq_pos);
    return s == DSA_OK ? ok() : s;
}

dsa_status dsa_forward_ragged_timed(const dsa_problem* p, const int32_t* seq_pos,
                                    const void* q_idx, const void* k_idx, const void* Q,
                                    const void* K, const void* V, int32_t* idx_out, void* O,
                                    float* lse, void* ws, size_t ws_bytes, void* stream,
                                    float* stage_ms, int32_t* n_slabs) {
    if (!stage_ms) return fail(DSA_E_NULL, "stage_ms is NULL");
    dsa_status s = check_ragged(p, seq_pos);
    if (s != DSA_OK) return s;
    StageTimer tm;
    tm.st = static_cast<hipStream_t>(stream);
    for (int i = 0; i < 3; ++i) stage_ms[i] = 0.f;
    s = forward_impl(p, q_idx, k_idx, Q, K, V, idx_out, O, lse, ws, ws_bytes, stream, &tm,
                     n_slabs, seq_pos);
    hipError_t e = tm.finish(stage_ms);
    if (s != DSA_OK) return s;
    if (e != hipSuccess) return hip_fail(e, "stage timing events");
    return ok();
}

dsa_status dsa_forward_paged(const dsa_problem* p, const int32_t* seq_pos, const dsa_pages* pg,
                             const void* q_idx, const void* k_pool, const void* Q,
                             const void* K_pool, const void* V_pool, int32_t* idx_out, void* O,
                             float* lse, void* ws, size_t ws_bytes, void* stream) {
    dsa::KeyPages kp{};
    dsa_status s = check_paged(p, seq_pos, pg, &kp);
    if (s != DSA_OK) return s;
    s = forward_impl(p, q_idx, k_pool, Q, K_pool, V_pool, idx_out, O, lse, ws, ws_bytes, stream,
                     nullptr, nullptr, seq_pos, &kp);
    return s == DSA_OK ? ok() : s;
}

dsa_status dsa_forward_paged_timed(const dsa_problem* p, const int32_t* seq_pos,
                                   const dsa_pages* pg, const void* q_idx, const void* k_pool,
                                   const void* Q, const void* K_pool, const void* V_pool,
                                   int32_t* idx_out, void* O, float* lse, void* ws,
                                   size_t ws_bytes, void* stream, float* stage_ms,
                                   int32_t* n_slabs) {
    if (!stage_ms) return fail(DSA_E_NULL, "stage_ms is NULL");
    dsa::KeyPages kp{};
    dsa_status s = check_paged(p, seq_pos, pg, &kp);
    if (s != DSA_OK) return s;
    StageTimer tm;
    tm.st = static_cast<hipStream_t>(stream);
    for (int i = 0; i < 3; ++i) stage_ms[i] = 0.f;
    s = forward_impl(p, q_idx, k_pool, Q, K_pool, V_pool, idx_out, O, lse, ws, ws_bytes, stream,
                     &tm, n_slabs, seq_pos, &kp);
    hipError_t e = tm.finish(stage_ms);
    if (s != DSA_OK) return s;
    if (e != hipSuccess) return hip_fail(e, "stage timing events");
    return ok();
}

dsa_status dsa_forward_threshold(const dsa_problem* p, float tau, const void* q_idx,
                                 const void* k_idx, const void* Q, const void* K, const void* V,
                                 int32_t* idx_out, void* O, float* lse, void* ws,
                                 size_t ws_bytes, void* stream) {
    dsa_status s = forward_impl(p, q_idx, k_idx, Q, K, V, idx_out, O, lse, ws, ws_bytes, stream,
                                nullptr, nullptr, nullptr, nullptr, &tau);
    return s == DSA_OK ? ok() : s;
}

dsa_status dsa_forward_threshold_timed(const dsa_problem* p, float tau, const void* q_idx,
                                       const void* k_idx, const void* Q, const void* K,
                                       const void* V, int32_t* idx_out, void* O, float* lse,
                                       void* ws, size_t ws_bytes, void* stream, float* stage_ms,
                                       int32_t* n_slabs) {
    if (!stage_ms) return fail(DSA_E_NULL, "stage_ms is NULL");
    StageTimer tm;
    tm.st = static_cast<hipStream_t>(stream);
    for (int i = 0; i < 3; ++i) stage_ms[i] = 0.f;
    dsa_status s = forward_impl(p, q_idx, k_idx, Q, K, V, idx_out, O, lse, ws, ws_bytes, stream,
                                &tm, n_slabs, nullptr, nullptr, &tau);
    hipError_t e = tm.finish(stage_ms);
    if (s != DSA_OK) return s;
    if (e != hipSuccess) return hip_fail(e, "stage timing events");
    return ok();
}

// Arguments of dsa_forward_ext: the layout (ragged, paged) and the mode.
dsa_status check_options(const dsa_problem* p, const dsa_forward_options* o, dsa::KeyPages* kp) {
    if (!o) return check_problem(p);
    if (o->pages) return check_paged(p, o->seq_pos, o->pages, kp);
    if (o->seq_pos) return check_ragged(p, o->seq_pos);
    return check_problem(p);
}

dsa_status forward_ext(const dsa_problem* p, const dsa_forward_options* o, const void* q_idx,
                       const void* k_idx, const void* Q, const void* K, const void* V,
                       int32_t* idx_out, void* O, float* lse, void* ws, size_t ws_bytes,
                       void* stream, StageTimer* tm, int32_t* n_slabs) {
    dsa::KeyPages kp{};
    dsa_status s = check_options(p, o, &kp);
    if (s != DSA_OK) return s;
    const float* tau = o && o->threshold_mode ? &o->tau : nullptr;
    return forward_impl(p, q_idx, k_idx, Q, K, V, idx_out, O, lse, ws, ws_bytes, stream, tm,
                        n_slabs, o ? o->seq_pos : nullptr, o && o->pages ? &kp : nullptr, tau);
}

dsa_status dsa_forward_ext(const dsa_problem* p, const dsa_forward_options* options,
                           const void* q_idx, const void* k_idx, const void* Q, const void* K,
                           const void* V, int32_t* idx_out, void* O, float* lse, void* ws,
                           size_t ws_bytes, void* stream) {
    dsa_status s = forward_ext(p, options, q_idx, k_idx, Q, K, V, idx_out, O, lse, ws, ws_bytes,
                               stream, nullptr, nullptr);
    return s == DSA_OK ? ok() : s;
}

dsa_status dsa_forward_ext_timed(const dsa_problem* p, const dsa_forward_options* options,
                                 const void* q_idx, const void* k_idx, const void* Q,
                                 const void* K, const void* V, int32_t* idx_out, void* O,
                                 float* lse, void* ws, size_t ws_bytes, void* stream,
                                 float* stage_ms, int32_t* n_slabs) {
    if (!stage_ms) return fail(DSA_E_NULL, "stage_ms is NULL");
    StageTimer tm;
    tm.st = static_cast<hipStream_t>(stream);
    for (int i = 0; i < 3; ++i) stage_ms[i] = 0.f;
    dsa_status s = forward_ext(p, options, q_idx, k_idx, Q, K, V, idx_out, O, lse, ws, ws_bytes,
                               stream, &tm, n_slabs);
    hipError_t e = tm.finish(stage_ms);
    if (s != DSA_OK) return s;
    if (e != hipSuccess) return hip_fail(e, "stage timing events");
    return ok();
}

dsa_status dsa_forward_timed(const dsa_problem* p, const void* q_idx, const void* k_idx,
                             const void* Q, const void* K, const void* V, int32_t* idx_out,
                             void* O, float* lse, void* ws, size_t ws_bytes, void* stream,
                             float* stage_ms, int32_t* n_slabs) {
    if (!stage_ms) return fail(DSA_E_NULL, "stage_ms is NULL");
    StageTimer tm;
    tm.st = static_cast<hipStream_t>(stream);
    for (int i = 0; i < 3; ++i) stage_ms[i] = 0.f;
    dsa_status s = forward_impl(p, q_idx, k_idx, Q, K, V, idx_out, O, lse, ws, ws_bytes, stream,
                                &tm, n_slabs);
    hipError_t e = tm.finish(stage_ms);
    if (s != DSA_OK) return s;
    if (e != hipSuccess) return hip_fail(e, "stage timing events");
    return ok();
}

dsa_status dsa_index_project(int32_t rows, int32_t d_model, int32_t d_idx, int32_t out_dtype,
                             const void* X, const void* W, void* out, const int32_t* out_rows,
                             int32_t n_out, void* stream) {
    dsa_status s = check_project_sizes(rows, d_model, d_idx);
    if (s != DSA_OK) return s;
    if (out_dtype != DSA_IDX_FP8_E4M3FN && out_dtype != DSA_IDX_BF16)
        return fail(DSA_E_UNSUPPORTED, "out_dtype=%d is neither fp8 e4m3fn (0) nor bf16 (1)",
                    out_dtype);
    if ((s = check_ptrs({X, W, out}, "X, W, out")) != DSA_OK) return s;
    if (out_rows && misaligned(out_rows))
        return fail(DSA_E_ALIGN, "out_rows is not 16-byte aligned");
    if (n_out < 1) return fail(DSA_E_SHAPE, "n_out=%d must be >= 1", n_out);
    if (!out_rows && n_out < rows)
        return fail(DSA_E_SHAPE, "without out_rows the output needs rows=%d rows (n_out=%d)",
                    rows, n_out);
    dsa::ProjectArgs a{};
    a.X = static_cast<const uint16_t*>(X);
    a.W = static_cast<const uint16_t*>(W);
    a.out = out;
    a.out_rows = out_rows;
    a.rows = rows;
    a.d_model = d_model;
    a.d_idx = d_idx;
    a.out_dtype = out_dtype;
    a.n_out = n_out;
    hipError_t e = dsa::launch_project(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "projection launch");
    return ok();
}

const char* dsa_status_str(int32_t status) {
    switch (status) {
        case DSA_OK: return "DSA_OK";
        case DSA_E_NULL: return "DSA_E_NULL";
        case DSA_E_SHAPE: return "DSA_E_SHAPE";
        case DSA_E_UNSUPPORTED: return "DSA_E_UNSUPPORTED";
        case DSA_E_ALIGN: return "DSA_E_ALIGN";
        case DSA_E_WORKSPACE: return "DSA_E_WORKSPACE";
        case DSA_E_HIP: return "DSA_E_HIP";
        default: return "DSA_E_UNKNOWN";
    }
}

const char* dsa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
