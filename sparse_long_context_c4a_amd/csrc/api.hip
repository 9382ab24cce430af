// The C ABI: host-side validation, workspace sizing and orchestration of the
// kernels for each entry point declared in dsa.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "common.h"
#include "internal.h"

namespace dsa {

namespace {
thread_local char g_err[512] = "";
thread_local dsa_timing_events g_hook = {};   // set by dsa_set_timing_events
thread_local TimingEvents g_active = {};      // the running call's events

// Moves the hook into the running call for its duration (one-shot).
struct TimingScope {
  TimingScope() {
    g_active = TimingEvents{static_cast<hipEvent_t>(g_hook.index_begin),
                            static_cast<hipEvent_t>(g_hook.index_end),
                            static_cast<hipEvent_t>(g_hook.attn_begin),
                            static_cast<hipEvent_t>(g_hook.attn_end)};
    g_hook = dsa_timing_events{};
  }
  ~TimingScope() { g_active = TimingEvents{}; }
};
}  // namespace

const TimingEvents& call_timing() { return g_active; }

dsa_status fail(dsa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

dsa_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return DSA_OK;
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

namespace {

#define REQUIRE(cond, ...)                                    \
  do {                                                        \
    if (!(cond)) return fail(DSA_ERR_INVALID_ARG, __VA_ARGS__); \
  } while (0)
#define SUPPORT(cond, ...)                                     \
  do {                                                         \
    if (!(cond)) return fail(DSA_ERR_UNSUPPORTED, __VA_ARGS__); \
  } while (0)

dsa_status check_geom(const dsa_geom& g, const char* who) {
  REQUIRE(g.stride >= 1 && g.span >= g.stride, "%s: need 1 <= stride <= span (got %d, %d)", who,
          g.stride, g.span);
  REQUIRE(g.dim >= 2 && g.dim % 2 == 0, "%s: dim %d must be even and >= 2", who, g.dim);
  REQUIRE(g.rope_dim >= 0 && g.rope_dim <= g.dim && g.rope_dim % 2 == 0,
          "%s: rope_dim %d must be even and in [0, dim]", who, g.rope_dim);
  REQUIRE(g.rope_dim == 0 || g.rope_base > 0.0, "%s: rope_base must be > 0", who);
  return DSA_OK;
}

bool is_dtype(int t) { return t == DSA_F32 || t == DSA_BF16 || t == DSA_FP8_E4M3; }

// The paging of a call: stride > 0 ties entries_per_block to the logical
// block (256 / stride); tiled: the compressed caches include 16-entry key
// tiles; max_pos_end bounds the positions the window table must cover.
dsa_status check_paging(const dsa_paging& p, int stride, int64_t e_cap, int64_t max_pos_end,
                        bool tiled, const char* who) {
  const bool any = p.block_table || p.swa_block_table;
  if (any) REQUIRE(p.blocks_per_seq >= 1, "%s: paging needs blocks_per_seq >= 1", who);
  if (p.block_table) {
    const int e = p.entries_per_block;
    REQUIRE(e >= 1 && (e & (e - 1)) == 0, "%s: entries_per_block %d must be a power of two", who, e);
    REQUIRE(stride <= 0 || static_cast<int64_t>(e) * stride == DSA_BLOCK_TOKENS,
            "%s: entries_per_block %d * stride %d must be %d raw positions", who, e, stride,
            DSA_BLOCK_TOKENS);
    REQUIRE(p.n_blocks >= 1, "%s: n_blocks < 1", who);
    REQUIRE(e_cap <= static_cast<int64_t>(p.blocks_per_seq) * e,
            "%s: e_cap %lld > blocks_per_seq * entries_per_block = %lld", who, (long long)e_cap,
            (long long)p.blocks_per_seq * e);
    SUPPORT(!tiled || e % 16 == 0, "%s: paged key tiles need entries_per_block a multiple of 16 "
            "(got %d)", who, e);
  }
  if (p.swa_block_table) {
    REQUIRE(p.n_swa_blocks >= 1, "%s: n_swa_blocks < 1", who);
    REQUIRE(static_cast<int64_t>(p.blocks_per_seq) * DSA_BLOCK_TOKENS >= max_pos_end,
            "%s: the window table covers %lld positions < max_pos_end %lld", who,
            (long long)p.blocks_per_seq * DSA_BLOCK_TOKENS, (long long)max_pos_end);
  }
  if (p.state_block) REQUIRE(p.n_state_blocks >= 1, "%s: n_state_blocks < 1", who);
  return DSA_OK;
}

dsa_status validate_compress(const dsa_compress_args* a) {
  REQUIRE(a, "dsa_compress: null args");
  dsa_status rc = check_geom(a->geom, "dsa_compress");
  if (rc != DSA_OK) return rc;
  REQUIRE(a->batch >= 1, "dsa_compress: batch %d < 1", a->batch);
  REQUIRE(a->raw_len >= 1, "dsa_compress: raw_len %lld < 1", (long long)a->raw_len);
  REQUIRE(a->raw && a->ring && a->raw_pos0 && a->logits && a->out,
          "dsa_compress: raw, ring, raw_pos0, logits and out must be non-null");
  REQUIRE(a->raw_dtype == DSA_F32 || a->raw_dtype == DSA_BF16,
          "dsa_compress: raw_dtype must be F32 or BF16");
  REQUIRE(is_dtype(a->out_dtype) || a->out_dtype == DSA_FP4_E2M1, "dsa_compress: bad out_dtype %d",
          a->out_dtype);
  REQUIRE(a->out_dtype != DSA_FP8_E4M3 || a->out_scale,
          "dsa_compress: FP8 output needs out_scale");
  REQUIRE(a->out_dtype != DSA_FP4_E2M1 || (a->out_mx_scale && a->geom.dim % 32 == 0),
          "dsa_compress: FP4 output needs out_mx_scale and dim a multiple of 32 (got %d)",
          a->geom.dim);
  REQUIRE(a->logits_rows >= ceil_div(a->raw_len, a->geom.stride),
          "dsa_compress: logits_rows %d < ceil(raw_len / stride) = %lld", a->logits_rows,
          (long long)ceil_div(a->raw_len, a->geom.stride));
  REQUIRE(a->e_cap >= 1, "dsa_compress: e_cap < 1");
  REQUIRE(a->max_pos_end >= a->raw_len, "dsa_compress: max_pos_end < raw_len");
  REQUIRE(a->rms_gamma == nullptr || a->rms_eps >= 0.f, "dsa_compress: rms_eps < 0");
  const bool tiled = (a->out_dtype == DSA_FP8_E4M3 || a->out_dtype == DSA_FP4_E2M1) &&
                     a->geom.dim == 128;
  return check_paging(a->paging, a->geom.stride, a->e_cap, a->max_pos_end, tiled, "dsa_compress");
}

dsa_status validate_index(const dsa_index_args* a) {
  REQUIRE(a, "dsa_index_topk: null args");
  REQUIRE(a->n_seqs >= 1 && a->queries_per_seq >= 1, "dsa_index_topk: n_seqs and "
          "queries_per_seq must be >= 1");
  REQUIRE(a->stride >= 1 && a->span >= a->stride, "dsa_index_topk: need 1 <= stride <= span");
  REQUIRE(a->k >= 1, "dsa_index_topk: k %d < 1", a->k);
  REQUIRE(a->q_pos && a->idx_out, "dsa_index_topk: q_pos and idx_out must be non-null");
  REQUIRE(a->e_cap >= 0 && a->max_pos_end >= 1, "dsa_index_topk: bad e_cap / max_pos_end");
  const int64_t nv_max = std::min<int64_t>(a->e_cap, n_complete(a->max_pos_end - 1, a->stride, a->span));
  if (a->keys == nullptr) {
    REQUIRE(nv_max <= a->k, "dsa_index_topk: keys may be NULL only when k >= n_vis for every "
            "position below max_pos_end (k %d, n_vis up to %lld)", a->k, (long long)nv_max);
    return DSA_OK;
  }
  REQUIRE(a->q && a->w, "dsa_index_topk: q and w must be non-null");
  REQUIRE(a->heads >= 1 && a->dim >= 1, "dsa_index_topk: heads and dim must be >= 1");
  REQUIRE(a->dtype == DSA_F32 || a->dtype == DSA_FP8_E4M3 || a->dtype == DSA_FP4_E2M1,
          "dsa_index_topk: dtype must be F32, FP8_E4M3 or FP4_E2M1");
  if (a->dtype == DSA_FP8_E4M3) REQUIRE(a->k_scale, "dsa_index_topk: FP8 keys need k_scale");
  if (a->dtype == DSA_FP4_E2M1) {
    REQUIRE(a->k_mx_scale, "dsa_index_topk: FP4 keys need k_mx_scale");
    SUPPORT(a->dim == 128 && a->heads <= 16,
            "dsa_index_topk: FP4 keys are built for dim 128 and at most 16 heads (got %d, %d)",
            a->dim, a->heads);
  }
  SUPPORT(a->heads * a->dim <= 16384, "dsa_index_topk: heads * dim %d too large", a->heads * a->dim);
  const bool tiled = (a->dtype == DSA_FP8_E4M3 || a->dtype == DSA_FP4_E2M1) && a->dim == 128;
  return check_paging(a->paging, a->stride, a->e_cap, a->max_pos_end, tiled, "dsa_index_topk");
}

dsa_status validate_attn(const dsa_attn_args* a) {
  REQUIRE(a, "dsa_sparse_attn: null args");
  REQUIRE(a->n_seqs >= 1 && a->queries_per_seq >= 1, "dsa_sparse_attn: bad batch");
  REQUIRE(a->heads >= 1, "dsa_sparse_attn: heads < 1");
  REQUIRE(a->dim >= 2 && a->dim % 2 == 0, "dsa_sparse_attn: dim %d must be even", a->dim);
  REQUIRE(a->rope_dim >= 0 && a->rope_dim <= a->dim && a->rope_dim % 2 == 0,
          "dsa_sparse_attn: bad rope_dim %d", a->rope_dim);
  REQUIRE(a->rope_dim == 0 || a->rope_base > 0.0, "dsa_sparse_attn: rope_base must be > 0");
  REQUIRE(a->dtype == DSA_F32 || a->dtype == DSA_BF16, "dsa_sparse_attn: dtype must be F32 or BF16");
  REQUIRE(a->q && a->q_pos && a->out, "dsa_sparse_attn: q, q_pos and out must be non-null");
  REQUIRE(a->k >= 0 && a->window_size >= 0, "dsa_sparse_attn: k and window_size must be >= 0");
  REQUIRE(a->k == 0 || (a->idx && a->cache && a->e_cap >= 1),
          "dsa_sparse_attn: k > 0 needs idx, cache and e_cap >= 1");
  REQUIRE(a->window_size == 0 ||
              (a->window && (a->paging.swa_block_table || a->w_cap >= a->window_size)),
          "dsa_sparse_attn: the window needs a ring with w_cap >= window_size (or a window table)");
  REQUIRE(a->chunk_win == nullptr || (a->chunk_pos0 && a->chunk_len >= 1),
          "dsa_sparse_attn: chunk_win needs chunk_pos0 and chunk_len >= 1");
  REQUIRE(a->k + a->window_size >= 1, "dsa_sparse_attn: empty attention set");
  REQUIRE(a->max_pos_end >= 1, "dsa_sparse_attn: max_pos_end < 1");
  REQUIRE(a->out_fp8 == 0 || a->out_fp8 == 1, "dsa_sparse_attn: out_fp8 must be 0 or 1");
  REQUIRE(!a->out_fp8 || a->out_scale, "dsa_sparse_attn: out_fp8 needs out_scale");
  REQUIRE(a->cache_fp8 == 0 || a->cache_fp8 == 1, "dsa_sparse_attn: cache_fp8 must be 0 or 1");
  REQUIRE(!a->cache_fp8 || a->k == 0 || a->cache_scale, "dsa_sparse_attn: cache_fp8 needs cache_scale");
  SUPPORT(!a->cache_fp8 || (a->dtype == DSA_BF16 && a->dim == 512),
          "dsa_sparse_attn: an fp8 cache needs dtype BF16 and dim 512");
  return check_paging(a->paging, 0, a->e_cap, a->max_pos_end, false, "dsa_sparse_attn");
}

dsa_status validate_layer(const dsa_layer_args* a, bool decode) {
  REQUIRE(a, "dsa_layer: null args");
  dsa_status rc = check_geom(a->main, "dsa_layer");
  if (rc != DSA_OK) return rc;
  REQUIRE(a->n_seqs >= 1 && a->chunk_len >= 1, "dsa_layer: n_seqs and chunk_len must be >= 1");
  REQUIRE(!decode || a->chunk_len == 1, "dsa_layer_decode: chunk_len must be 1 (got %d)",
          a->chunk_len);
  REQUIRE(a->heads >= 1 && a->k >= 1 && a->window_size >= 0, "dsa_layer: bad heads/k/window");
  REQUIRE(a->dtype == DSA_F32 || a->dtype == DSA_BF16, "dsa_layer: dtype must be F32 or BF16");
  REQUIRE(a->pos0 && a->x && a->logits_main && a->q && a->main_cache && a->main_ring &&
              a->window && a->out,
          "dsa_layer: pos0, x, logits_main, q, main_cache, main_ring, window, out must be non-null");
  REQUIRE(a->e_cap >= ceil_div(a->max_pos_end, a->main.stride),
          "dsa_layer: e_cap %lld < ceil(max_pos_end / stride) = %lld", (long long)a->e_cap,
          (long long)ceil_div(a->max_pos_end, a->main.stride));
  REQUIRE(a->paging.swa_block_table || (a->w_cap >= a->window_size && a->w_cap >= 1),
          "dsa_layer: w_cap < window_size");
  REQUIRE(a->max_pos_end >= a->chunk_len, "dsa_layer: max_pos_end < chunk_len");
  REQUIRE(a->out_fp8 == 0 || a->out_fp8 == 1, "dsa_layer: out_fp8 must be 0 or 1");
  REQUIRE(!a->out_fp8 || a->out_scale, "dsa_layer: out_fp8 needs out_scale");
  REQUIRE(a->main_fp8 == 0 || a->main_fp8 == 1, "dsa_layer: main_fp8 must be 0 or 1");
  REQUIRE(!a->main_fp8 || a->main_scale, "dsa_layer: main_fp8 needs main_scale");
  REQUIRE(a->q_norm_gamma == nullptr || a->rms_eps >= 0.f, "dsa_layer: rms_eps < 0");
  SUPPORT(!a->main_fp8 || (a->dtype == DSA_BF16 && a->main.dim == 512),
          "dsa_layer: an fp8 main cache is built for dtype BF16 and dim 512");
  if (a->main_fp8) {  // refused before the step writes any state
    rc = attn_fp8_cache_shape(a->k, a->heads, static_cast<int64_t>(a->n_seqs) * a->chunk_len);
    if (rc != DSA_OK) return rc;
  }
  if (a->idx_heads > 0) {
    REQUIRE(a->idx_dim >= 2 && a->idx_dim % 2 == 0, "dsa_layer: idx_dim must be even");
    REQUIRE(a->idx_rope_dim >= 0 && a->idx_rope_dim <= a->idx_dim && a->idx_rope_dim % 2 == 0,
            "dsa_layer: bad idx_rope_dim");
    REQUIRE(a->idx_dtype == DSA_F32 || a->idx_dtype == DSA_FP8_E4M3 ||
                a->idx_dtype == DSA_FP4_E2M1,
            "dsa_layer: idx_dtype must be F32, FP8_E4M3 or FP4_E2M1");
    REQUIRE(a->kx && a->logits_idx && a->qi && a->w && a->idx_cache && a->idx_ring,
            "dsa_layer: the indexer needs kx, logits_idx, qi, w, idx_cache and idx_ring");
    REQUIRE(a->idx_dtype != DSA_FP8_E4M3 || a->idx_scale,
            "dsa_layer: FP8 indexer cache needs idx_scale");
    REQUIRE(a->idx_dtype != DSA_FP4_E2M1 || a->idx_mx_scale,
            "dsa_layer: FP4 indexer cache needs idx_mx_scale");
    SUPPORT(a->idx_dtype != DSA_FP4_E2M1 || (a->idx_dim == 128 && a->idx_heads <= 16),
            "dsa_layer: an FP4 indexer cache is built for idx_dim 128 and at most 16 heads");
  } else {
    const int64_t nv_max = n_complete(a->max_pos_end - 1, a->main.stride, a->main.span);
    REQUIRE(nv_max <= a->k, "dsa_layer: without an indexer k (%d) must cover every visible entry "
            "(up to %lld)", a->k, (long long)nv_max);
  }
  const bool tiled = a->idx_heads > 0 && a->idx_dim == 128 &&
                     (a->idx_dtype == DSA_FP8_E4M3 || a->idx_dtype == DSA_FP4_E2M1);
  return check_paging(a->paging, a->main.stride, a->e_cap, a->max_pos_end, tiled, "dsa_layer");
}

// Workspace plan of a layer step: index/top-k scratch, attention scratch,
// the Top-k output (if the caller does not want it), the rotated chunk.
struct LayerWs {
  dsa_index_args ia;
  dsa_attn_args aa;
  size_t off_idx_ws, off_attn_ws, off_idx, off_rot, off_cs, off_qrot, total;
};

LayerWs layer_plan(const dsa_layer_args* a, void* ws) {
  LayerWs L{};
  const int64_t rows = static_cast<int64_t>(a->n_seqs) * a->chunk_len;
  char* base = static_cast<char*>(ws);
  dsa_index_args& ia = L.ia;
  ia.n_seqs = a->n_seqs;
  ia.queries_per_seq = a->chunk_len;
  ia.stride = a->main.stride;
  ia.span = a->main.span;
  ia.heads = a->idx_heads;
  ia.dim = a->idx_dim;
  ia.q = a->qi;
  ia.q_scale = a->idx_dtype != DSA_F32 ? a->qi_scale : nullptr;  // fp8 queries
  ia.w = a->w;
  ia.keys = a->idx_heads > 0 ? a->idx_cache : nullptr;
  ia.k_scale = a->idx_dtype == DSA_FP8_E4M3 ? a->idx_scale : nullptr;
  ia.k_mx_scale = a->idx_dtype == DSA_FP4_E2M1 ? a->idx_mx_scale : nullptr;
  ia.dtype = a->idx_dtype;
  ia.e_cap = a->e_cap;
  ia.max_pos_end = a->max_pos_end;
  ia.k = a->k;
  ia.score_out = nullptr;
  ia.status = a->status;
  ia.paging = a->paging;
  size_t off = 0;
  L.off_idx_ws = off;
  off = align_up(off + index_topk_ws_bytes(ia));
  L.off_idx = off;
  if (!a->idx_out) off = align_up(off + static_cast<size_t>(rows) * a->k * sizeof(int32_t));
  L.off_rot = off;
  off = align_up(off + static_cast<size_t>(rows) * a->main.dim * dtype_size(a->dtype));
  // decode: the (cos, sin) table of each row's position
  L.off_cs = off;
  if (a->chunk_len == 1) off = align_up(off + static_cast<size_t>(rows) * a->main.rope_dim * 4);
  // the prepared (normalised, rotated) queries: every decode step (the
  // prologue riding in the indexer's launch prepares them, so the attention
  // starts from rotated queries) and chunks with a Q-norm
  L.off_qrot = off;
  const bool qprep = a->q_norm_gamma != nullptr || a->chunk_len == 1;
  if (qprep)
    off = align_up(off + static_cast<size_t>(rows) * a->heads * a->main.dim * dtype_size(a->dtype));
  // q positions (one per row)
  dsa_attn_args& aa = L.aa;
  aa.n_seqs = a->n_seqs;
  aa.queries_per_seq = a->chunk_len;
  aa.heads = a->heads;
  aa.dim = a->main.dim;
  aa.rope_dim = a->main.rope_dim;
  aa.rope_base = a->main.rope_base;
  aa.rope_pos_offset = a->main.rope_pos_offset;
  aa.dtype = a->dtype;
  aa.q = a->q;
  aa.rotate_q = 1;
  aa.cache = a->main_cache;
  aa.e_cap = a->e_cap;
  aa.k = a->k;
  aa.window = a->window;
  aa.w_cap = a->w_cap;
  aa.window_size = a->window_size;
  aa.chunk_pos0 = a->pos0;
  aa.chunk_len = a->chunk_len;
  aa.softmax_scale = a->softmax_scale;
  aa.max_pos_end = a->max_pos_end;
  aa.out = a->out;
  aa.lse = a->lse;
  aa.out_fp8 = a->out_fp8;
  aa.out_scale = a->out_scale;
  aa.cache_fp8 = a->main_fp8;
  aa.cache_scale = a->main_scale;
  aa.status = a->status;
  aa.paging = a->paging;
  L.off_attn_ws = off;
  off = align_up(off + attn_ws_bytes(aa));
  // per-row positions
  size_t off_pos = off;
  off = align_up(off + static_cast<size_t>(rows) * sizeof(int64_t));
  L.total = off;
  if (base) {
    int32_t* idx = a->idx_out ? a->idx_out : reinterpret_cast<int32_t*>(base + L.off_idx);
    ia.idx_out = idx;
    aa.idx = idx;
    aa.chunk_win = base + L.off_rot;
    if (qprep) {  // attention reads the prepared queries
      aa.q = base + L.off_qrot;
      aa.rotate_q = 0;
    }
    int64_t* qpos = reinterpret_cast<int64_t*>(base + off_pos);
    ia.q_pos = qpos;
    aa.q_pos = qpos;
  }
  return L;
}

dsa_status run_layer(const dsa_layer_args* a, void* ws, size_t ws_bytes, hipStream_t st, bool decode) {
  dsa_status rc = validate_layer(a, decode);
  if (rc == DSA_OK && a->main_fp8 && !decode)
    rc = fail(DSA_ERR_UNSUPPORTED, "dsa_layer_prefill: an fp8 main cache is read by decode only");
  if (rc != DSA_OK) return rc;
  LayerWs L = layer_plan(a, nullptr);
  if (!ws || ws_bytes < L.total)
    return fail(DSA_ERR_WORKSPACE, "dsa_layer: workspace %zu < required %zu", ws_bytes, L.total);
  L = layer_plan(a, ws);
  const int B = a->n_seqs, T = a->chunk_len;
  char* base = static_cast<char*>(ws);
  if (T == 1) {
    // one token per sequence: fused prologue, indexer + Top-k, attention over
    // the selected entries and the window ring, window insert
    // slot m mod w_cap (a ring with a spare slot) or m's slot of its window
    // block (paged) is outside m's window
    const bool early = a->w_cap > a->window_size || a->paging.swa_block_table != nullptr;
    int64_t* qpos = const_cast<int64_t*>(L.ia.q_pos);
    L.ia.q_pos = a->pos0;  // one query per sequence, at pos0
    L.aa.q_pos = a->pos0;
    L.aa.chunk_win = nullptr;
    // the prologue leaves the (cos, sin) table of m for attention
    float* cs_tab = reinterpret_cast<float*>(base + L.off_cs);
    AttnLaunch lx;
    lx.ev0 = call_timing().attn0;
    lx.ev1 = call_timing().attn1;
    lx.cs_tab = cs_tab;
    rc = launch_decode_index_topk(L.ia, base + L.off_idx_ws, *a, qpos, early, cs_tab,
                                  base + L.off_qrot, st);
    if (rc != DSA_OK) return rc;
    rc = launch_attn(L.aa, base + L.off_attn_ws, st, lx);
    if (rc != DSA_OK) return rc;
    return early ? DSA_OK : launch_decode_window_insert(*a, st);
  }
  // S1: compress entries completing in the chunk (reads the old rings)
  const int rows_logits = static_cast<int>(ceil_div(T, a->main.stride));
  dsa_compress_args c{};
  c.geom = a->main;
  c.batch = B;
  c.raw = a->x;
  c.raw_dtype = a->dtype;
  c.raw_len = T;
  c.ring = a->main_ring;
  c.raw_pos0 = a->pos0;
  c.logits = a->logits_main;
  c.logits_rows = rows_logits;
  c.rms_gamma = a->rms_gamma;
  c.rms_eps = a->rms_eps;
  c.out = a->main_cache;
  c.out_dtype = a->dtype;
  c.out_scale = nullptr;
  c.e_cap = a->e_cap;
  c.max_pos_end = a->max_pos_end;
  c.status = a->status;
  c.paging = a->paging;
  const dsa_dtype raw_idx_dt = a->idx_dtype == DSA_F32 ? DSA_F32 : DSA_BF16;
  if (a->idx_heads == 0) {
    rc = launch_compress(c, st);
    if (rc != DSA_OK) return rc;
  } else {
    dsa_compress_args ci = c;
    ci.geom.dim = a->idx_dim;
    ci.geom.rope_dim = a->idx_rope_dim;
    ci.geom.rope_base = a->idx_rope_base;
    ci.raw = a->kx;
    ci.raw_dtype = raw_idx_dt;
    ci.ring = a->idx_ring;
    ci.logits = a->logits_idx;
    ci.rms_gamma = a->rms_gamma_idx;
    ci.out = a->idx_cache;
    ci.out_dtype = a->idx_dtype;
    ci.out_scale = a->idx_scale;
    ci.out_mx_scale = a->idx_mx_scale;
    rc = launch_compress_pair(c, ci, st);
    if (rc != DSA_OK) return rc;
  }
  // the rings take the chunk's raw tokens; the rows' positions (for the
  // indexer and attention) and, without a Q-norm, the chunk's tokens rotated
  // for the window, in the same launch
  rc = launch_chunk_tasks(a->x, a->dtype, a->main.dim, a->main_ring, a->kx, raw_idx_dt,
                          a->idx_dim, a->idx_heads > 0 ? a->idx_ring : nullptr, T, a->main.span,
                          a->pos0, B, a->max_pos_end, a->paging, a->status,
                          const_cast<int64_t*>(L.ia.q_pos),
                          a->q_norm_gamma ? nullptr : base + L.off_rot, a->main.rope_dim,
                          a->main.rope_base, a->main.rope_pos_offset, st);
  if (rc != DSA_OK) return rc;
  // S3 + S4
  rc = launch_index_topk(L.ia, base + L.off_idx_ws, st);
  if (rc != DSA_OK) return rc;
  // with a Q-norm: the queries prepared and the chunk's tokens rotated for
  // the window (the window of the chunk's own queries, then the ring) in one
  // launch
  if (a->q_norm_gamma) {
    rc = launch_qk_prep(*a, base + L.off_qrot, base + L.off_rot, st);
    if (rc != DSA_OK) return rc;
  }
  // S5
  AttnLaunch lx;
  lx.ev0 = call_timing().attn0;
  lx.ev1 = call_timing().attn1;
  rc = launch_attn(L.aa, base + L.off_attn_ws, st, lx);
  if (rc != DSA_OK) return rc;
  // window ring update after attention
  return launch_window_update(base + L.off_rot, a->dtype, a->main.dim, T, a->window, a->w_cap,
                              a->window_size, a->pos0, B, a->max_pos_end, a->paging, a->status,
                              st);
}

// ------------------------------------------------ allocation-free decode
// The scratch memory of dsa_layer_decode_noalloc: a file-scope device array
// (each GPU holds its own copy from the library's first use on it until the
// process ends).  In host code `scratch` only names the symbol; its device
// address on the current GPU comes from hipGetSymbolAddress, once per GPU.
constexpr size_t kScratchBytes = size_t{64} << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

dsa_status scratch_on_device(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DSA_ERR_UNSUPPORTED, "dsa_layer_decode_noalloc: device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    dsa_status rc = hip_check(hipGetDevice(&cur), "hipGetDevice");
    if (rc != DSA_OK) return rc;
    if (cur != dev && (rc = hip_check(hipSetDevice(dev), "hipSetDevice")) != DSA_OK) return rc;
    void* p = nullptr;
    rc = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (cur != dev) {
      const dsa_status rb = hip_check(hipSetDevice(cur), "hipSetDevice");
      if (rc == DSA_OK) rc = rb;
    }
    if (rc != DSA_OK) return rc;
    if (!p) return fail(DSA_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

dsa_status layer_decode_noalloc(const dsa_layer_args* a, hipStream_t st) {
  TimingScope ts;
  dsa_status rc = validate_layer(a, true);
  if (rc != DSA_OK) return rc;
  const size_t need = layer_plan(a, nullptr).total;
  if (need > kScratchBytes)
    return fail(DSA_ERR_WORKSPACE, "dsa_layer_decode_noalloc: this step needs %zu bytes of scratch, "
                "the static scratch holds %zu (use dsa_layer_decode with a workspace)", need,
                kScratchBytes);
  int dev = -1;
  rc = st ? hip_check(hipStreamGetDevice(st, &dev), "hipStreamGetDevice")
          : hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (rc != DSA_OK) return rc;
  void* ws = nullptr;
  rc = scratch_on_device(dev, &ws);
  if (rc != DSA_OK) return rc;
  return run_layer(a, ws, kScratchBytes, st, true);
}

}  // namespace
}  // namespace dsa

using namespace dsa;

extern "C" {

dsa_status dsa_compress(const dsa_compress_args* a, void* stream) {
  dsa_status rc = validate_compress(a);
  if (rc != DSA_OK) return rc;
  return launch_compress(*a, static_cast<hipStream_t>(stream));
}

size_t dsa_index_topk_workspace(const dsa_index_args* a) {
  if (validate_index(a) != DSA_OK) return 0;
  return index_topk_ws_bytes(*a);
}

dsa_status dsa_index_topk(const dsa_index_args* a, void* ws, size_t ws_bytes, void* stream) {
  TimingScope ts;
  dsa_status rc = validate_index(a);
  if (rc != DSA_OK) return rc;
  const size_t need = index_topk_ws_bytes(*a);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "dsa_index_topk: workspace %zu < required %zu", ws_bytes, need);
  return launch_index_topk(*a, ws, static_cast<hipStream_t>(stream));
}

size_t dsa_sparse_attn_workspace(const dsa_attn_args* a) {
  if (validate_attn(a) != DSA_OK) return 0;
  return attn_ws_bytes(*a);
}

dsa_status dsa_sparse_attn(const dsa_attn_args* a, void* ws, size_t ws_bytes, void* stream) {
  TimingScope ts;
  dsa_status rc = validate_attn(a);
  if (rc != DSA_OK) return rc;
  const size_t need = attn_ws_bytes(*a);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "dsa_sparse_attn: workspace %zu < required %zu", ws_bytes, need);
  AttnLaunch lx;
  lx.ev0 = call_timing().attn0;
  lx.ev1 = call_timing().attn1;
  return launch_attn(*a, ws, static_cast<hipStream_t>(stream), lx);
}

size_t dsa_layer_workspace(const dsa_layer_args* a) {
  if (validate_layer(a, false) != DSA_OK) return 0;
  return layer_plan(a, nullptr).total;
}

dsa_status dsa_layer_decode(const dsa_layer_args* a, void* ws, size_t ws_bytes, void* stream) {
  TimingScope ts;
  return run_layer(a, ws, ws_bytes, static_cast<hipStream_t>(stream), true);
}

dsa_status dsa_layer_decode_noalloc(const dsa_layer_args* a, void* stream) {
  return layer_decode_noalloc(a, static_cast<hipStream_t>(stream));
}

size_t dsa_layer_decode_noalloc_capacity(void) { return kScratchBytes; }

dsa_status dsa_layer_prefill(const dsa_layer_args* a, void* ws, size_t ws_bytes, void* stream) {
  TimingScope ts;
  return run_layer(a, ws, ws_bytes, static_cast<hipStream_t>(stream), false);
}

void dsa_set_timing_events(const dsa_timing_events* ev) { g_hook = ev ? *ev : dsa_timing_events{}; }

int dsa_device_supported(int device) {
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, device) != hipSuccess) return 0;
  return std::strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
}

const char* dsa_version(void) { return "dsa-mi355x 0.1.0 (gfx950)"; }

const char* dsa_last_error(void) { return g_err; }

size_t dsa_abi_sizeof(const char* name) {
  if (!name) return 0;
  if (!std::strcmp(name, "dsa_geom")) return sizeof(dsa_geom);
  if (!std::strcmp(name, "dsa_timing_events")) return sizeof(dsa_timing_events);
  if (!std::strcmp(name, "dsa_paging")) return sizeof(dsa_paging);
  if (!std::strcmp(name, "dsa_compress_args")) return sizeof(dsa_compress_args);
  if (!std::strcmp(name, "dsa_index_args")) return sizeof(dsa_index_args);
  if (!std::strcmp(name, "dsa_attn_args")) return sizeof(dsa_attn_args);
  if (!std::strcmp(name, "dsa_layer_args")) return sizeof(dsa_layer_args);
  return 0;
}

int64_t dsa_n_complete(int64_t L, int32_t stride, int32_t span) {
  if (stride < 1 || span < stride || L < 0) return -1;
  return n_complete(L, stride, span);
}

}  // extern "C"
