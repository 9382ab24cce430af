/*
 * dsa.h -- C ABI of the MI355X (gfx950) compressed sparse attention library.
 *
 * The layer (DeepSeek V4 attention as described in the pages
 * "DeepSeek DSA、DeepSeek V4与vLLM Hybrid KV Cache详解" [P1] and
 * "DeepSeek V4 稀疏注意力完全解剖" [P2]) runs five steps:
 *
 *   S1 compress   entry j = RoPE_{s j}( sum_{i<S} softmax(z_j)_i x_{s j + i} )
 *                 (c4a: S = 8 raw tokens at stride s = 4; c128a: S = s = 128)
 *                 [P1] 5.2, [P2] 机制二
 *   S2 visibility entry j is visible to query m iff s j + S - 1 < m;
 *                 window = raw tokens [m-W, m-1]          [P2] 机制四
 *   S3 indexer    I[m, j] = sum_h w[m,h] ReLU(q_idx[m,h] . k_idx[j])
 *                 over the visible entries                 [P1] 4.1
 *   S4 Top-k      keep the k highest-scoring entries       [P1] 4.2, [P2] 机制三
 *   S5 attention  MQA over {selected entries} U {window}, K = V, one softmax,
 *                 output rotated back by R_m^{-1}          [P1] 4.3 / 5.1,
 *                                                          [P2] 机制一, 深潜
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller, dense and
 *    row-major in the layout given per field.  The library never allocates,
 *    frees or synchronises; scratch memory comes in through the workspace
 *    argument (size from the matching *_workspace query, alignment 256 B),
 *    except for dsa_layer_decode_noalloc, whose scratch is a static device
 *    array of the library.
 *  - Each call validates its arguments on the host, enqueues kernels on
 *    `stream` (a hipStream_t; NULL = the default stream) and returns.  On a
 *    validation failure nothing is launched.
 *  - Per-sequence positions are device int64 arrays, so a call sequence can
 *    be captured in a HIP graph.  Host-side bounds (max_pos_end) size the
 *    grids; kernels clamp to them and never read or write outside the
 *    buffers described here.  A device-side precondition that fails (a
 *    position beyond max_pos_end, an entry beyond e_cap) sets bits in the
 *    optional device word `status` (see DSA_DEVERR_*), or is ignored if
 *    `status` is NULL; the affected outputs are then unspecified but all
 *    memory accesses stay in bounds.
 *  - Storage formats: DSA_F32 IEEE binary32; DSA_BF16 bfloat16;
 *    DSA_FP8_E4M3 OCP fp8 e4m3fn (bias 7, max 448, no infinities) with one
 *    fp32 scale per row (value = scale * code); DSA_FP4_E2M1 OCP MX FP4
 *    (indexer keys only): E2M1 codes (sign, 2 exponent bits with bias 1, one
 *    mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte with
 *    the lower nibble first, and one E8M0 scale byte e per 32 consecutive
 *    dims (value = 2^(e - 127) * code), the scales in their own row-major
 *    array [B, e_cap, dim / 32].  The pages store the indexer in fp4 ([P2]
 *    第三层, 机制三) without a format; MX FP4 is the reading taken.
 *  - Key tile layout: an FP8 cache of dim 128 (the indexer keys) is not
 *    row-major.  Each sequence holds e_pad = ceil(e_cap / 16) * 16 entries
 *    (allocate B * e_pad * 128 bytes) in tiles of 16 entries; tile t is 2048
 *    bytes: 8 chunks of 16 dims, chunk c holding the 16 entries' bytes
 *    16c .. 16c+15 in entry order.  Byte d of entry j of sequence b sits at
 *      ((b * e_pad + 16 * (j / 16)) * 128) + (d / 16) * 256 + (j % 16) * 16 + d % 16.
 *    This is the order in which the matrix-core operands are read, so each
 *    load instruction of the indexer streams 1 KiB of contiguous bytes.  The
 *    scales stay row-major [B, e_cap].  FP8 caches of other dims are
 *    row-major.  An FP4 cache of dim 128 uses the same 16-entry tiles at 64
 *    bytes per entry (allocate B * e_pad * 64 bytes): tile t is 1024 bytes,
 *    4 chunks of 32 dims (16 bytes), chunk c holding the 16 entries' bytes;
 *    the byte of dim d of entry j of sequence b (nibble d % 2) sits at
 *      ((b * e_pad + 16 * (j / 16)) * 64) + (d / 32) * 256 + (j % 16) * 16 + (d % 32) / 2.
 *  - RoPE acts on interleaved pairs of the last rope_dim dims of a vector,
 *    pair i rotated by angle (pos + rope_pos_offset) * rope_base^(-2i/rope_dim).
 *    rope_pos_offset shifts every rotation position and no index.
 *  - Calls hold no global mutable state (dsa_layer_decode_noalloc aside: one
 *    scratch array per GPU); errors are returned, never printed, and
 *    dsa_last_error() gives a thread-local message for the last failure.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = -1, /* null pointer, bad size, inconsistent shape   */
  DSA_ERR_UNSUPPORTED = -2, /* dtype / dim combination not built, not gfx950 */
  DSA_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than required       */
  DSA_ERR_HIP = -4          /* a HIP runtime call failed                     */
} dsa_status;

typedef enum dsa_dtype { DSA_F32 = 0, DSA_BF16 = 1, DSA_FP8_E4M3 = 2, DSA_FP4_E2M1 = 3 } dsa_dtype;

/* Bits OR-ed into the optional device status word by kernels. */
#define DSA_DEVERR_POSITION 1u  /* a position outside [0, max_pos_end)        */
#define DSA_DEVERR_CAPACITY 2u  /* an entry slot or n_vis beyond e_cap        */
#define DSA_DEVERR_NO_INDEX 4u  /* no indexer but n_vis(m) > k                */
#define DSA_DEVERR_BLOCK 8u     /* a block table entry outside its pool       */

/* ------------------------------------------------------------ paging ----
 * Paged caches ([P2] 第三层 设计 1 and 设计 2; [P1] 6.1 and 6.2).  A logical
 * block is DSA_BLOCK_TOKENS = 256 raw token positions of a sequence, whatever
 * the layer's compression, so every cache is addressed through the same
 * logical block numbers; each cache type decides how many of its own rows a
 * physical block holds.  A zeroed dsa_paging (every pointer NULL) keeps the
 * dense per-sequence layouts described with each field.
 *
 *  - block_table [B, blocks_per_seq]: the compressed caches (main_cache /
 *    cache, main_scale / cache_scale, idx_cache / keys, idx_scale / k_scale,
 *    idx_mx_scale / k_mx_scale / out_mx_scale) become pools of physical
 *    blocks of entries_per_block = 256 / stride entries (c4a 64, c128a 2).
 *    Entry j of sequence b is row  block_table[b, j / E] * E + j % E  (E =
 *    entries_per_block) of the pool, the pool laid out as the dense cache
 *    with (sequence, entry) replaced by that row: main [n_blocks * E, D],
 *    scales [n_blocks * E] and [n_blocks * E, Di / 32]; FP8 / FP4 keys of dim
 *    128 keep their 16-entry tiles (E a multiple of 16; rows n_blocks * E).
 *    e_cap stays the entries a sequence may hold (<= blocks_per_seq * E).
 *  - swa_block_table [B, blocks_per_seq]: the window.  Raw token n of
 *    sequence b is stored (rotated) in slot n % 256 of block
 *    swa_block_table[b, n / 256] of a pool [n_swa_blocks, 256, D]; w_cap is
 *    then not used, and blocks wholly before the window may be released
 *    (their entries are not read).
 *  - state_block [B]: the compressor states (rings of the last S raw tokens,
 *    [P2] 设计 2 treats them as sliding-window state): sequence b's rings are
 *    block state_block[b] of pools [n_state_blocks, S, D] and
 *    [n_state_blocks, S, Di].
 *
 * A block id outside [0, pool size) sets DSA_DEVERR_BLOCK in the status word;
 * reads through it then take block 0 and writes are dropped, so memory
 * accesses stay inside the pools.  Only entries a call reads or writes need
 * a valid block.
 */
#define DSA_BLOCK_TOKENS 256

typedef struct dsa_paging {
  const int32_t* block_table;      /* device [B, blocks_per_seq] or NULL      */
  const int32_t* swa_block_table;  /* device [B, blocks_per_seq] or NULL      */
  const int32_t* state_block;      /* device [B] or NULL                      */
  int32_t blocks_per_seq;          /* row stride of the two tables            */
  int32_t entries_per_block;       /* 256 / stride, a power of two            */
  int32_t n_blocks;                /* physical blocks of the entry pools      */
  int32_t n_swa_blocks;            /* physical blocks of the window pool      */
  int32_t n_state_blocks;          /* physical blocks of the ring pools       */
} dsa_paging;

/* Compressor / attention geometry. */
typedef struct dsa_geom {
  int32_t stride;          /* s: raw tokens between consecutive entries     */
  int32_t span;            /* S: raw tokens mixed into one entry (S >= s)   */
  int32_t dim;             /* D: vector length                              */
  int32_t rope_dim;        /* r: rotary tail dims, even, 0 <= r <= D        */
  double rope_base;        /* frequency base (> 0 when r > 0)               */
  int64_t rope_pos_offset; /* added to every rotation position              */
} dsa_geom;

/* ---------------------------------------------------------------- S1 ----
 * dsa_compress: write every compressed entry that completes inside a chunk
 * of raw tokens ([P1] 5.2; [P2] 机制二 c4a diagram T0 = t0..t7, T1 = t4..t11;
 * [P2] 融合点 1 for the fused order compress -> RMSNorm -> RoPE -> insert).
 *
 * For sequence b the chunk holds raw positions p0 = raw_pos0[b] ..
 * p0 + raw_len - 1.  Entries j with p0 <= s j + S - 1 < p0 + raw_len are
 * written, i.e. j = n_complete(p0) .. n_complete(p0 + raw_len) - 1 with
 * n_complete(L) = max(0, floor((L - S) / s) + 1).  Entry j reads raw tokens
 * s j .. s j + S - 1: those >= p0 from `raw`, those < p0 from `ring`.
 * Weights: softmax over logits[b, j - n_complete(p0), 0..S-1], one scalar per
 * raw token shared across D.  Optional RMSNorm (gamma != NULL):
 * c <- gamma * c / sqrt(mean(c^2) + eps).  Then RoPE at position s j.
 * FP8 output: scale = max|c| / 448 (fp32), codes round to nearest even.
 * FP4 output (MXFP4): per 32-dim block e = floor(log2(max|c|)) - 2 (clamped
 * to [-127, 127]; -127 for an all-zero block), codes = E2M1 of c / 2^e
 * rounded to nearest even and saturating at 6 (the OCP MX conversion).
 */
typedef struct dsa_compress_args {
  dsa_geom geom;
  int32_t batch;              /* B                                           */
  const void* raw;            /* [B, raw_len, D] raw tokens, raw_dtype       */
  dsa_dtype raw_dtype;        /* DSA_F32 or DSA_BF16                         */
  int64_t raw_len;            /* tokens per sequence in this chunk (>= 1)    */
  const void* ring;           /* [B, S, D] raw_dtype: the S raw tokens before
                                 the chunk, position p at slot p mod S        */
  const int64_t* raw_pos0;    /* device [B]: position of raw[b, 0]           */
  const float* logits;        /* [B, logits_rows, S]                         */
  int32_t logits_rows;        /* >= ceil(raw_len / s)                        */
  const float* rms_gamma;     /* [D] or NULL (no RMSNorm)                    */
  float rms_eps;
  void* out;                  /* [B, e_cap, D] cache, entry j at slot j
                                 (FP8 with D = 128: the key tile layout)     */
  dsa_dtype out_dtype;        /* DSA_F32, DSA_BF16 or DSA_FP8_E4M3           */
  float* out_scale;           /* [B, e_cap] for FP8 output, else ignored     */
  int64_t e_cap;              /* cache slots per sequence                    */
  int64_t max_pos_end;        /* host bound: raw_pos0[b] + raw_len <= this   */
  uint32_t* status;           /* optional device status word                 */
  uint8_t* out_mx_scale;      /* [B, e_cap, D / 32] E8M0 block scales for FP4
                                 output (D a multiple of 32), else ignored   */
  dsa_paging paging;          /* zeroed: dense caches (see paging above)  */
} dsa_compress_args;

dsa_status dsa_compress(const dsa_compress_args* a, void* stream);

/* ------------------------------------------------------------ S2-S4 ----
 * dsa_index_topk: lightning-indexer scores over the visible entries and
 * Top-k selection ([P1] 4.1, 4.2; [P2] 机制三).
 *
 * Queries are grouped per sequence: row i = b * queries_per_seq + t belongs
 * to sequence b and sits at position q_pos[i].  n_vis = n_complete(q_pos[i]).
 * I[i, j] = sum_h w[i,h] * qs[i,h] * ks[b,j] * ReLU(q[i,h] . k[b,j]) for
 * j < n_vis, where qs / ks are the fp8 scales (1 for F32).  The output holds
 * the min(k, n_vis) entries of highest score, ties to the lower index, in no
 * particular order, then -1 padding.  If k >= n_vis the selection is
 * 0 .. n_vis-1 and keys may be NULL.  Scores equal to within fp32 rounding
 * of the k-th may be exchanged with it.
 */
typedef struct dsa_index_args {
  int32_t n_seqs;             /* B                                           */
  int32_t queries_per_seq;    /* Tq (1 for decode)                           */
  const int64_t* q_pos;       /* device [B * Tq]                             */
  int32_t stride, span;       /* s, S of the compressor that made the keys   */
  int32_t heads, dim;         /* Hi, Di (DSA_FP8_E4M3 needs Di == 128)       */
  const void* q;              /* [B * Tq, Hi, Di]                            */
  const float* q_scale;       /* [B * Tq, Hi] (FP8; NULL means 1)            */
  const float* w;             /* [B * Tq, Hi] head weights                   */
  const void* keys;           /* [B, e_cap, Di]; FP8 Di = 128: tile layout   */
  const float* k_scale;       /* [B, e_cap] (FP8)                            */
  dsa_dtype dtype;            /* q and keys: DSA_F32 or DSA_FP8_E4M3; or
                                 DSA_FP4_E2M1: keys MXFP4 (Di == 128, tile
                                 layout, k_mx_scale), q fp8 with q_scale     */
  int64_t e_cap;
  int64_t max_pos_end;        /* host bound: q_pos[i] < max_pos_end          */
  int32_t k;                  /* >= 1                                        */
  int32_t* idx_out;           /* [B * Tq, k]                                 */
  float* score_out;           /* [B * Tq, k] or NULL (NaN for padding)       */
  uint32_t* status;
  const uint8_t* k_mx_scale;  /* [B, e_cap, Di / 32] E8M0 scales (FP4 keys)  */
  dsa_paging paging;          /* zeroed: dense caches (see paging above)  */
} dsa_index_args;

size_t dsa_index_topk_workspace(const dsa_index_args* a);
dsa_status dsa_index_topk(const dsa_index_args* a, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- S5 ----
 * dsa_sparse_attn: MQA attention over the selected entries and the raw
 * window, K = V, one joint softmax, inverse RoPE on the output ([P1] 4.3,
 * 5.1, 5.3; [P2] 机制一, 深潜 Inverse RoPE, 机制四).
 *
 * Row i (sequence b, position m = q_pos[i]) attends to
 *   { cache[b, j] : j in idx[i], j >= 0 }  U  { window vector of raw token n :
 *   max(0, m - W) <= n <= m - 1 }.
 * Window vectors are stored rotated: for n >= chunk_pos0[b] (if chunk_win is
 * given) at chunk_win[b, n - chunk_pos0[b]], otherwise at window[b, n mod
 * w_cap] (which the caller keeps current: w_cap >= W).
 * logits = scale * (R_m q_h) . v (q rotated here if rotate_q, else taken as
 * already rotated); out_h = R_m^{-1} sum_a softmax_a v_a; lse_h = natural-log
 * sum of exp(logits).  An empty set gives out = 0, lse = -inf.
 * With out_fp8 = 1 the output is stored token-wise in fp8, fused with the
 * R_m^{-1} epilogue ([P2] 融合点 2; the scale rule is the decode KV's
 * token-wise one, [P2] 第三层): per (row, head) sigma = max_d |out_h[d]| / 448
 * (f32, into out_scale), out = e4m3fn codes of out_h / sigma rounded to
 * nearest even; sigma = 0 gives zero codes.
 * With cache_fp8 = 1 the compressed entries are stored token-wise in fp8
 * ([P2] 第三层: decode KV in token-wise fp8): cache holds e4m3fn codes
 * [B, e_cap, D] (one byte per dim) and cache_scale one f32 scale per entry
 * [B, e_cap]; entry j's vector is cache_scale[b, j] * code.  The window
 * stays dtype.  Built for dtype BF16, D = 512, heads a multiple of 16 and
 * B * Tq * H / 16 <= 2048 (decode shapes); other shapes return
 * DSA_ERR_UNSUPPORTED.
 */
typedef struct dsa_attn_args {
  int32_t n_seqs;             /* B                                           */
  int32_t queries_per_seq;    /* Tq                                          */
  const int64_t* q_pos;       /* device [B * Tq]                             */
  int32_t heads;              /* H                                           */
  int32_t dim;                /* D (DSA_BF16 needs D == 512)                 */
  int32_t rope_dim;
  double rope_base;
  int64_t rope_pos_offset;
  dsa_dtype dtype;            /* q, cache, window, out: DSA_F32 or DSA_BF16  */
  const void* q;              /* [B * Tq, H, D]                              */
  int32_t rotate_q;           /* 1: rotate q at its position here            */
  const void* cache;          /* [B, e_cap, D]                               */
  int64_t e_cap;
  const int32_t* idx;         /* [B * Tq, k], -1 = none                      */
  int32_t k;
  const void* window;         /* [B, w_cap, D]                               */
  int32_t w_cap;
  int32_t window_size;        /* W (<= w_cap)                                */
  const void* chunk_win;      /* [B, chunk_len, D] or NULL                   */
  const int64_t* chunk_pos0;  /* device [B] (with chunk_win)                 */
  int64_t chunk_len;
  float softmax_scale;        /* 0 -> 1 / sqrt(D)                            */
  int64_t max_pos_end;        /* host bound: q_pos[i] < max_pos_end          */
  void* out;                  /* [B * Tq, H, D]                              */
  float* lse;                 /* [B * Tq, H] or NULL                         */
  uint32_t* status;
  int32_t out_fp8;            /* 0: out is dtype; 1: out is fp8 codes        */
  float* out_scale;           /* [B * Tq, H] (out_fp8)                       */
  int32_t cache_fp8;          /* 0: cache is dtype; 1: fp8 codes + scales    */
  const float* cache_scale;   /* [B, e_cap] (cache_fp8)                      */
  dsa_paging paging;          /* zeroed: dense caches (see paging above)  */
} dsa_attn_args;

size_t dsa_sparse_attn_workspace(const dsa_attn_args* a);
dsa_status dsa_sparse_attn(const dsa_attn_args* a, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ layer ----
 * dsa_layer_decode / dsa_layer_prefill: one layer step over a chunk of T raw
 * tokens per sequence at positions p0 = pos0[b] .. p0 + T - 1 ([P2] 全景图,
 * decode step C-E; [P1] 15 flowchart).  Decode is the T = 1 case.
 *
 *  1. S1 for every entry completing in the chunk, main (dtype) and indexer
 *     (idx_dtype) caches, reading raw tokens before the chunk from the
 *     compressor rings (state = last S raw tokens, [P2] 设计 2: c4a 8,
 *     c128a 128);
 *  2. the rings take the chunk's last S raw tokens;
 *  3. S3/S4 for each of the T queries (entries completed earlier in the same
 *     chunk are visible to later queries); with idx_heads == 0 every visible
 *     entry is selected, which needs k >= n_vis (the c128a case);
 *  4. S5 with the window [m - W, m - 1]; with q_norm_gamma each query head
 *     is first normalised, q <- gamma * q / sqrt(mean(q^2) + rms_eps).  The
 *     queries are normalised and rotated in one launch with the window
 *     tokens' rotation and insert (the pages' horizontally fused
 *     pre-attention step, [P2] 融合点 3): in decode always, riding in the
 *     indexer's launch; in a chunk when there is a Q-norm;
 *  5. the window ring takes the chunk's rotated tokens (after attention, so
 *     slot m mod w_cap is reused only once m's own query has run).
 * Raw indexer tokens kx are F32 when idx_dtype is F32 and BF16 when it is
 * FP8.  All state buffers are updated in place.
 */
typedef struct dsa_layer_args {
  dsa_geom main;              /* s, S, D, r, base, offset (main + window)    */
  int32_t heads;              /* H                                           */
  int32_t idx_heads;          /* Hi (0: no indexer)                          */
  int32_t idx_dim;            /* Di                                          */
  int32_t idx_rope_dim;
  double idx_rope_base;
  int32_t k;
  int32_t window_size;        /* W                                           */
  float softmax_scale;        /* 0 -> 1/sqrt(D)                              */
  int32_t n_seqs;             /* B                                           */
  int32_t chunk_len;          /* T                                           */
  const int64_t* pos0;        /* device [B]                                  */
  int64_t max_pos_end;        /* host bound: pos0[b] + T <= max_pos_end      */
  dsa_dtype dtype;            /* DSA_F32 or DSA_BF16                         */
  dsa_dtype idx_dtype;        /* DSA_F32, DSA_FP8_E4M3 or DSA_FP4_E2M1 (keys
                                 MXFP4 with Di == 128, queries qi fp8)       */
  const void* x;              /* [B, T, D] raw tokens                        */
  const void* kx;             /* [B, T, Di] raw indexer tokens               */
  const float* logits_main;   /* [B, ceil(T/s), S]                           */
  const float* logits_idx;    /* [B, ceil(T/s), S]                           */
  const void* q;              /* [B, T, H, D] (not rotated)                  */
  const void* qi;             /* [B, T, Hi, Di]                              */
  const float* qi_scale;      /* [B, T, Hi] (FP8)                            */
  const float* w;             /* [B, T, Hi]                                  */
  void* main_cache;           /* [B, e_cap, D]                               */
  void* idx_cache;            /* [B, e_cap, Di]; FP8 Di = 128: tile layout   */
  float* idx_scale;           /* [B, e_cap] (FP8)                            */
  int64_t e_cap;
  void* main_ring;            /* [B, S, D]                                   */
  void* idx_ring;             /* [B, S, Di]                                  */
  void* window;               /* [B, w_cap, D]                               */
  int32_t w_cap;
  const float* rms_gamma;     /* [D] or NULL                                 */
  const float* rms_gamma_idx; /* [Di] or NULL                                */
  float rms_eps;
  void* out;                  /* [B, T, H, D]                                */
  float* lse;                 /* [B, T, H] or NULL                           */
  int32_t* idx_out;           /* [B, T, k] or NULL                           */
  uint32_t* status;
  int32_t out_fp8;            /* 1: out as fp8 codes + out_scale (see S5)    */
  float* out_scale;           /* [B, T, H] (out_fp8)                         */
  int32_t main_fp8;           /* 1: main_cache holds token-wise fp8 codes    */
  float* main_scale;          /* [B, e_cap] (main_fp8); decode only, see S5  */
  const float* q_norm_gamma;  /* [D] or NULL: Q-norm of each query head      */
  uint8_t* idx_mx_scale;      /* [B, e_cap, Di / 32] (idx_dtype FP4)         */
  dsa_paging paging;          /* zeroed: dense caches (see paging above)  */
} dsa_layer_args;

size_t dsa_layer_workspace(const dsa_layer_args* a);
dsa_status dsa_layer_decode(const dsa_layer_args* a, void* ws, size_t ws_bytes, void* stream);
dsa_status dsa_layer_prefill(const dsa_layer_args* a, void* ws, size_t ws_bytes, void* stream);

/* dsa_layer_decode_noalloc: dsa_layer_decode for callers that cannot
 * allocate memory -- code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The same step with the same kernels and
 * results, but its scratch memory is a static device array inside the
 * library instead of a caller's workspace: the call allocates nothing and
 * calls no allocating routine.  The caller still passes every input, state
 * and output buffer in `a`.
 *  - Capacity: dsa_layer_decode_noalloc_capacity() bytes (64 MiB), which
 *    covers a decode step whose dsa_layer_workspace() fits in it (all of
 *    c4a B = 4 at 1M, B = 32 at 64K, c128a B = 16 at 1M); a larger step
 *    returns DSA_ERR_WORKSPACE before anything is launched.
 *  - Each GPU holds its own copy of the array from the first call on it
 *    until the process ends (its address is looked up once per device).
 *  - Every call on one GPU uses that GPU's one array: calls that overlap on
 *    one GPU (other streams, other threads) race and must be ordered by the
 *    caller.  The step writes every scratch byte it reads, so nothing needs
 *    clearing between calls.
 *  - Arguments, validation and errors as dsa_layer_decode. */
dsa_status dsa_layer_decode_noalloc(const dsa_layer_args* a, void* stream);
size_t dsa_layer_decode_noalloc_capacity(void);

/* ---------------------------------------------------------- measurement
 * dsa_set_timing_events: HIP events (hipEvent_t, NULL = none) that the NEXT
 * dsa_index_topk, dsa_sparse_attn or dsa_layer_* call made on this thread
 * attaches to its own kernels' dispatch packets (hipExtLaunchKernel, so no
 * extra packets sit between kernels): index_begin / index_end around the
 * scoring kernel, attn_begin / attn_end around the attention kernels (the
 * first one's start, the last one's end).  Benchmarks use it to time one
 * kernel inside a step.  One-shot and thread-local: that call consumes it,
 * whether it succeeds or not. */
typedef struct dsa_timing_events {
  void* index_begin;
  void* index_end;
  void* attn_begin;
  void* attn_end;
} dsa_timing_events;
void dsa_set_timing_events(const dsa_timing_events* ev);

/* ---------------------------------------------------------------- misc */
/* 1 if `device` is a gfx950 GPU this library was built for, else 0. */
int dsa_device_supported(int device);
const char* dsa_version(void);
const char* dsa_last_error(void);
/* n_complete(L) = max(0, floor((L - S) / s) + 1): entries whose S raw tokens
 * all lie in [0, L); also the visible-entry count of a query at position L. */
int64_t dsa_n_complete(int64_t L, int32_t stride, int32_t span);
/* sizeof of a struct declared here ("dsa_geom", "dsa_compress_args",
 * "dsa_index_args", "dsa_attn_args", "dsa_layer_args", "dsa_timing_events"),
 * 0 for other names.
 * Lets a binding check its mirror of the struct layouts. */
size_t dsa_abi_sizeof(const char* struct_name);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
