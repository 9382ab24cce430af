// S3 + S4: lightning indexer and Top-k selection.
//
// Score of query row i against visible entry j < n_vis(m_i):
//   I[i, j] = ks_j * sum_h (w_ih * qs_ih) * ReLU(q8_ih . k8_j)
// ("DeepSeek DSA、DeepSeek V4与vLLM Hybrid KV Cache详解" 4.1: a cheap score per
// (query, history entry), few heads, FP8).  The fp8 scales are positive, so
// they factor out of the ReLU and the dot products run on the e4m3 codes.
//
// Decode path (k_index_fp8_stream): the fp8 keys stream from HBM once per
// query.  The 16 indexer heads are the M side of the matrix-core product and
// 16 entries its N side; ReLU, the head weights and the head sum are a
// 4-value in-lane reduce plus two cross-lane adds on the accumulator.  The
// fp8 codes are widened to bf16 (exact: every e4m3fn value is a bf16 value)
// and multiplied on the bf16 MFMA (4 x v_mfma_f32_16x16x32_bf16 per 16
// entries): the gfx950 fp8 MFMA sums its 128 products with a shared
// alignment that drops low-order bits (measured up to ~2^-13 of the largest
// product), too coarse for Top-k near ties, while bf16 products are exact and
// sum in fp32.
//
// Top-k without cross-workgroup atomics: each wave (256 entries) keeps as
// candidates the entries with key above the wave's (cap+1)-th largest, t_w
// (found with wave-wide max reductions, no LDS and no barriers), and records
// t_w.  The final pass checks the certificate  k-th largest candidate key >=
// max_w t_w : every entry left out has a key below its wave's t_w, hence
// below the k-th, so the union's top k is the row's top k.  It
// then selects the exact top k of the union: one histogram over the
// candidates' key range, then the threshold bin resolved on (score key,
// complemented index), so ties go to the lower index.  If the certificate
// fails (adversarial score layouts, massive ties) the row falls back to an
// exact radix select over all of its scores, which the stream kernel also
// writes out.
//
// Row path (generic shapes, f32): scores go to memory and one workgroup per
// row runs the exact radix select.
//
// Many rows per sequence (a prefill chunk) take the matrix-core contraction
// of prefill_index.hip.
#include <type_traits>

#include "common.h"
#include "decode_impl.h"
#include "indexer_impl.h"
#include "internal.h"
#include "select_impl.h"

namespace dsa {
namespace {

// --------------------------------------------------- stream (decode) kernel
// Operand layout: lane l owns entry (or head) n = l % 16 and, within the
// 128-byte vector, bytes [16 g, 16 g + 16) and [64 + 16 g, 64 + 16 g + 16)
// with g = l / 16; MFMA c of the four takes the lane's bytes [8 c, 8 c + 8)
// of those 32.  A and B use the same byte-to-k assignment, so the four MFMAs
// sum every one of the 128 products exactly once.  With the keys' tile
// layout each of the two 16-byte loads of a wave reads 1 KiB of contiguous
// bytes.
template <bool kCand, int kEnt, int kFmt, bool kPaged>
__global__ __launch_bounds__(kThreads) void k_index_fp8_stream(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ keys, const float* __restrict__ k_scale,
    const uint8_t* __restrict__ k_mx, const int64_t* __restrict__ q_pos, int Tq, int Hi, int s,
    int S, int64_t e_cap, int64_t nv_cap, int64_t max_pos_end, float* __restrict__ scores,
    int64_t ld_scores, uint64_t* __restrict__ cand, uint32_t* __restrict__ meta, int cap,
    uint32_t* status, PageMap pm) {
  index_stream_block<kCand, kEnt, kFmt, kPaged>(blockIdx.x, gridDim.x, blockIdx.y, q, q_scale, w, keys,
                                        k_scale, k_mx, q_pos, Tq, Hi, s, S, e_cap, nv_cap,
                                        max_pos_end, scores, ld_scores, cand, meta, cap, status,
                                        pm);
}

// A decode step's indexer with the step's state updates riding along: the
// first kPrologueRoles x rows workgroups run the prologue roles (role id %
// kPrologueRoles of sequence id / kPrologueRoles), whose writes the indexer
// does not read (see decode_prologue_block), so they overlap the key stream
// instead of adding a launch and its latency in front of it; they come
// first so that they are dispatched with the first wave of workgroups, not
// after the stream has freed compute units.  The rest stream the keys: nb
// workgroups per row.
template <typename MainT, int kIdxOut, int kEnt, bool kMainFp8, bool kPaged>
__global__ __launch_bounds__(kThreads) void k_decode_index(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ keys, const float* __restrict__ k_scale,
    const uint8_t* __restrict__ k_mx, const int64_t* __restrict__ q_pos, int Hi, int s, int S,
    int64_t e_cap, int64_t nv_cap, int64_t max_pos_end, float* __restrict__ scores,
    int64_t ld_scores, uint64_t* __restrict__ cand, uint32_t* __restrict__ meta, int cap, int nb,
    PrologueArgs pa, uint32_t* status) {
  // the keys' paging is the layer's (the prologue's)
  pin_scalars(q, q_scale, w, keys, k_scale, k_mx, q_pos, Hi, s, S, e_cap, nv_cap, max_pos_end,
              scores, ld_scores, cand, meta, cap, nb, status, pa.B, pa.nq_roles, pa.pg.ent.table);
  const int rpr = kPrologueRoles + pa.nq_roles;  // prologue workgroups per sequence
  const int id = static_cast<int>(blockIdx.x), npro = pa.B * rpr;
  if (id < npro) {
    decode_prologue_block<MainT, kIdxOut, 1, kMainFp8>(id % rpr, id / rpr, pa);
  } else {
    const int sid = id - npro;
    index_stream_block<true, kEnt, kIdxOut, kPaged>(sid % nb, nb, sid / nb, q, q_scale, w, keys, k_scale,
                                            k_mx, q_pos, 1, Hi, s, S, e_cap, nv_cap, max_pos_end,
                                            scores, ld_scores, cand, meta, cap, status, pa.pg.ent);
  }
}

// ------------------------------------------------------------- generic VALU
// Any Hi, Di; q and keys f32 or fp8.  One entry per thread; scores only.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_index_generic(
    const T* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const T* __restrict__ keys, const float* __restrict__ k_scale, const int64_t* __restrict__ q_pos,
    int Tq, int Hi, int Di, int s, int S, int64_t e_cap, int64_t nv_cap, int64_t max_pos_end,
    float* __restrict__ scores, int64_t ld_scores, uint32_t* status, PageMap pm) {
  extern __shared__ float q_s[];  // [Hi * Di] then [Hi] weights
  const int row = blockIdx.y, b = row / Tq, tid = threadIdx.x;
  const RowInfo ri = row_info(q_pos, row, s, S, nv_cap, max_pos_end, status, blockIdx.x == 0 && tid == 0);
  const int64_t nv = ri.nv;
  float* w_s = q_s + Hi * Di;
  for (int i = tid; i < Hi * Di; i += blockDim.x) {
    const int64_t o = static_cast<int64_t>(row) * Hi * Di + i;
    if constexpr (sizeof(T) == 1) q_s[i] = fp8_to_f32(q[o]);
    else q_s[i] = q[o];
  }
  for (int h = tid; h < Hi; h += blockDim.x) {
    const int64_t o = static_cast<int64_t>(row) * Hi + h;
    w_s[h] = w[o] * ((sizeof(T) == 1 && q_scale) ? q_scale[o] : 1.0f);
  }
  __syncthreads();
  const int64_t ent = static_cast<int64_t>(blockIdx.x) * blockDim.x + tid;
  if (ent < nv) {
    // fp8 keys of dim 128 use the tile layout, everything else is row-major;
    // row: the entry's row (b * e_cap + ent dense, its pool row paged), trow
    // its tile row
    const bool tiled = sizeof(T) == 1 && Di == 128;
    const int64_t erow = entry_row(pm, b, ent, e_cap, status);
    const int64_t trow = pm.table ? erow : static_cast<int64_t>(b) * idx_e_pad(e_cap) + ent;
    const T* kr = keys + (tiled ? 0 : erow * Di);
    float tot = 0.f;
    for (int h = 0; h < Hi; ++h) {
      float d = 0.f;
      for (int i = 0; i < Di; ++i) {
        float kv;
        if constexpr (sizeof(T) == 1)
          kv = fp8_to_f32(tiled ? kr[idx_tile_off_row(trow, i)] : kr[i]);
        else kv = kr[i];
        d = fmaf(q_s[h * Di + i], kv, d);
      }
      tot += w_s[h] * fmaxf(d, 0.f);
    }
    if constexpr (sizeof(T) == 1) tot *= k_scale[erow];
    scores[static_cast<int64_t>(row) * ld_scores + ent] = tot;
  }
}

// ------------------------------------------------------------ final passes
// Waves of 256 entries the candidate pass scores again in full when their
// thresholds do not certify the candidates (LDS: 2 KiB each).
constexpr int kMaxF = 24;

// Candidate path: union of the waves' candidates (empty slots are 0), the
// certificate, and the exact top k; falls back to the full-row select when
// the certificate does not hold.  The candidates stay in registers (8 per
// thread) through one combined reduction pass, one histogram pass and the
// emit pass.
template <int kFmt>
__global__ __launch_bounds__(kSel) void k_topk_cand_final(
    float* __restrict__ scores, int64_t ld_scores, const int64_t* __restrict__ q_pos,
    int s, int S, int64_t nv_cap, int64_t max_pos_end, const uint64_t* __restrict__ cand,
    const uint32_t* __restrict__ meta, int nw, int cap, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out, int k, const uint8_t* __restrict__ q,
    const float* __restrict__ q_scale, const float* __restrict__ hw,
    const uint8_t* __restrict__ keys, const float* __restrict__ k_scale,
    const uint8_t* __restrict__ k_mx, int Tq, int Hi, int64_t e_cap, PageMap kpm,
    uint32_t* status) {
  __shared__ uint64_t cand_s[kFinalCap + 256 * kMaxF];
  __shared__ uint64_t tmp_s[kTmpCap];
  __shared__ __attribute__((aligned(16))) uint32_t h_s[kBins];
  __shared__ uint32_t red[3][kSelWaves];
  __shared__ uint32_t pos_bin, n_tmp;
  __shared__ uint32_t nu_s[kSelWaves];  // each wave's entries above the k-th bin
  __shared__ uint16_t f_s[kMaxF];        // waves scored again in full
  __shared__ uint32_t fbit_s[kSel / 32];  // the same as a bit set
  const int row = blockIdx.x, t = threadIdx.x, l = t & 63, w = t >> 6;
  // the candidates and wave thresholds do not depend on the row's position:
  // their loads go out with the position's, one memory round trip for all
  const int slots = nw * cap;  // <= kFinalCap by construction
  const uint32_t* mrow = meta + static_cast<int64_t>(row) * nw;
  const uint64_t* crow = cand + static_cast<int64_t>(row) * slots;
  // two candidates per 16-byte load: v[2 i + h] is slot 2 t + 2 kSel i + h
  // (slots is even: nw is a multiple of 4; the row's start is 16-byte aligned)
  constexpr int kPer = kFinalCap / kSel;
  uint64_t v[kPer];
#pragma unroll
  for (int i = 0; i < kPer / 2; ++i) {
    const int sl = 2 * t + 2 * kSel * i;
    uint4 w = {0u, 0u, 0u, 0u};
    if (sl < slots) w = *reinterpret_cast<const uint4*>(crow + sl);
    v[2 * i] = static_cast<uint64_t>(w.x) | (static_cast<uint64_t>(w.y) << 32);
    v[2 * i + 1] = static_cast<uint64_t>(w.z) | (static_cast<uint64_t>(w.w) << 32);
  }
  // wave thresholds: nw <= kSel (the plan's condition), one per thread
  const uint32_t mw = t < nw ? mrow[t] : 0u;
  uint32_t tm = mw;
  const RowInfo ri = row_info(q_pos, row, s, S, nv_cap, max_pos_end, nullptr, false);
  const int64_t nv = ri.nv;
  float* srow = scores + static_cast<int64_t>(row) * ld_scores;
  int32_t* irow = idx_out + static_cast<int64_t>(row) * k;
  float* orow = score_out ? score_out + static_cast<int64_t>(row) * k : nullptr;
  const int b = row / Tq;
  const KeySrc src = key_src<kFmt>(keys, k_scale, k_mx, kpm, b, e_cap, status);
  v8bf aq[4];
  float wv[4];
  if (nv <= k) {
    if (orow) {  // the visible entries' scores (the stream kept them in registers)
      exact_row_operands<kFmt>(q, q_scale, hw, row, Hi, aq, wv);
      score_row_exact<kFmt>(aq, wv, src, nv, srow, kSelWaves);
      __syncthreads();
    }
    emit_all_visible(srow, nv, k, irow, orow);
    return;
  }
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (v[u] != 0) {
      lo = min(lo, static_cast<uint32_t>(v[u] >> 32));
      hi = max(hi, static_cast<uint32_t>(v[u] >> 32));
    }
  // one combined block reduction: max t_w, min and max candidate key
  tm = wave_reduce_u32<0>(tm);
  lo = wave_reduce_u32<1>(lo);
  hi = wave_reduce_u32<0>(hi);
  if (l == 0) {
    red[0][w] = tm;
    red[1][w] = lo;
    red[2][w] = hi;
  }
  for (int i = t; i < 2048; i += kSel) h_s[i] = 0u;
  if (t == 0) pos_bin = n_tmp = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    tm = max(tm, red[0][i]);
    lo = min(lo, red[1][i]);
    hi = max(hi, red[2][i]);
  }
  // the histogram over the candidates' key range; its total is the number
  // of candidates
  const int shift = range_shift(hi - lo, 11);
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (v[u] != 0) atomicAdd(&h_s[(static_cast<uint32_t>(v[u] >> 32) - lo) >> shift], 1u);
  __syncthreads();
  uint32_t c_tot;
  const Bin br = find_bin_wave<2048>(h_s, static_cast<uint32_t>(k), &c_tot);  // barrier
  if (c_tot < static_cast<uint32_t>(k)) {
    // fewer candidates than k (ties at the wave thresholds): the whole row
    exact_row_operands<kFmt>(q, q_scale, hw, row, Hi, aq, wv);
    score_row_exact<kFmt>(aq, wv, src, nv, srow, kSelWaves);
    __syncthreads();
    row_select_from_scores(srow, nv, k, irow, orow, cand_s, h_s);
    return;
  }
  const uint32_t B = br.b, above = br.above, at = br.at;
  // The certificate: the k-th candidate lies in bin B, so its key is at
  // least kc = lo + B 2^shift.  An entry that is not a candidate has a key
  // below its wave's threshold t_w; where every t_w <= kc no such entry can
  // reach the k-th, and the candidates' top k is the row's.  Otherwise the
  // waves F with t_w > kc are scored again in full: with U = (candidates
  // of waves outside F) + (every entry of F), an entry outside U has a key
  // below t_w <= kc <= the k-th of U, so U's top k is exact.  Each wave of F
  // holds cap candidates above kc, so F stays small unless the scores are
  // laid out adversarially; beyond kMaxF waves the whole row is re-scored.
  const uint32_t kc = lo + (B << shift);
  if (tm > kc) {
    const bool in_f = mw > kc;
    const uint32_t nf = block_reduce_u32<2>(in_f ? 1u : 0u);  // barriers
    exact_row_operands<kFmt>(q, q_scale, hw, row, Hi, aq, wv);
    if (nf > static_cast<uint32_t>(kMaxF)) {
      score_row_exact<kFmt>(aq, wv, src, nv, srow, kSelWaves);
      __syncthreads();
      row_select_from_scores(srow, nv, k, irow, orow, cand_s, h_s);
      return;
    }
    if (t == 0) n_tmp = 0u;
    if (t < kSel / 32) fbit_s[t] = 0u;
    __syncthreads();
    if (in_f) {
      f_s[atomicAdd(&n_tmp, 1u)] = static_cast<uint16_t>(t);
      atomicOr(&fbit_s[t >> 5], 1u << (t & 31));
    }
    __syncthreads();
    // the candidates of waves outside F, in their slots
#pragma unroll
    for (int i = 0; i < kPer / 2; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int sl = 2 * t + 2 * kSel * i + h, wv_id = sl / cap;
        const bool drop = sl >= slots || ((fbit_s[wv_id >> 5] >> (wv_id & 31)) & 1u);
        cand_s[sl] = drop ? 0ull : v[2 * i + h];
      }
    // every entry of F, exactly, after them: tile ft = 16 entries of wave
    // f_s[ft / 16]; each wave takes every kSelWaves-th tile, the loads of
    // kBatch tiles in flight together
    constexpr int kBatch = 4;
    const int n = t & 15, g = (t & 63) >> 4, ntile = static_cast<int>(nf) * 16;
    for (int f0 = w; f0 < ntile; f0 += kBatch * kSelWaves) {
      int64_t jj[kBatch];
      float sc[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int ft = f0 + u * kSelWaves;
        jj[u] = ft < ntile ? static_cast<int64_t>(f_s[ft >> 4]) * 256 + (ft & 15) * 16 + n : nv;
      }
      exact_scores<kFmt, kBatch>(aq, wv, src, jj, nv, sc);
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int ft = f0 + u * kSelWaves;
        if (g == 0 && ft < ntile)
          cand_s[kFinalCap + ft * 16 + n] =
              jj[u] < nv ? composite(order_key(sc[u]), static_cast<uint32_t>(jj[u])) : 0ull;
      }
    }
    __syncthreads();
    select_topk_composites<kSel>(cand_s, kFinalCap + static_cast<int>(nf) * 256,
                                 static_cast<uint32_t>(k), irow, orow, tmp_s, h_s);
    return;
  }
  const bool fits = at <= static_cast<uint32_t>(kTmpCap);
  // places for the wave's entries above the bin and in it: the ballots of
  // all kPer values first; the bin's few members take places by an LDS
  // counter, the entries above it by the waves' counts (an exclusive sum
  // over the waves after the barrier below: no atomics on one address from
  // every wave)
  uint64_t bu[kPer], bm[kPer];
  uint32_t nu = 0, nm = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const uint32_t bin = (static_cast<uint32_t>(v[u] >> 32) - lo) >> shift;
    bu[u] = __ballot(v[u] != 0 && bin > B);
    bm[u] = __ballot(v[u] != 0 && bin == B);
    nu += static_cast<uint32_t>(__popcll(bu[u]));
    nm += static_cast<uint32_t>(__popcll(bm[u]));
  }
  uint32_t pm = 0;
  if (l == 0) {
    nu_s[w] = nu;
    if (nm) pm = atomicAdd(&n_tmp, nm);
  }
  pm = __builtin_amdgcn_readlane(pm, 0);
  const uint64_t below = (1ull << l) - 1ull;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const uint64_t x = v[u];
    const bool mid = (bm[u] >> l) & 1ull;
    const uint32_t q = pm + static_cast<uint32_t>(__popcll(bm[u] & below));
    if (mid && fits) tmp_s[q] = x;
    if (!fits) cand_s[t + u * kSel] = mid ? x : 0ull;  // only the bin's members
    pm += static_cast<uint32_t>(__popcll(bm[u]));
  }
  __syncthreads();
  uint32_t pu = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) pu += i < w ? nu_s[i] : 0u;
  const uint32_t need = static_cast<uint32_t>(k) - above;
  auto out_bin = [&](uint64_t x) {
    const uint32_t p = atomicAdd(&pos_bin, 1u);
    if (p < need) emit(irow, orow, above + p, comp_index(x), key_to_float(static_cast<uint32_t>(x >> 32)));
  };
  if (fits && at <= 64) {
    keep_largest_small(tmp_s, static_cast<int>(at), need, [&](uint64_t x, uint32_t slot) {
      emit(irow, orow, above + slot, comp_index(x), key_to_float(static_cast<uint32_t>(x >> 32)));
    });
  } else if (fits) {
    const uint64_t cut = kth_largest_composite(tmp_s, static_cast<int>(at), need,
                                               [](uint64_t) { return true; }, lo + (B << shift),
                                               shift);
    for (int i = t; i < static_cast<int>(at); i += kSel)
      if (tmp_s[i] >= cut) out_bin(tmp_s[i]);
  } else {
    const uint64_t cut = kth_largest_composite(cand_s, kFinalCap, need,
                                               [](uint64_t x) { return x != 0; },
                                               lo + (B << shift), shift);
    for (int i = t; i < kFinalCap; i += kSel)
      if (cand_s[i] != 0 && cand_s[i] >= cut) out_bin(cand_s[i]);
  }
  // the entries above the bin go out last, after every barrier: a barrier
  // waits for the workgroup's outstanding global stores
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const uint64_t x = v[u];
    const uint32_t p = pu + static_cast<uint32_t>(__popcll(bu[u] & below));
    if (((bu[u] >> l) & 1ull) && p < above)
      emit(irow, orow, p, comp_index(x), key_to_float(static_cast<uint32_t>(x >> 32)));
    pu += static_cast<uint32_t>(__popcll(bu[u]));
  }
}

// Row path: one workgroup per query row selects from the row's scores.
__global__ __launch_bounds__(kSel) void k_topk_rows(
    const float* __restrict__ scores, int64_t ld_scores, const int64_t* __restrict__ q_pos,
    int s, int S, int64_t nv_cap, int64_t max_pos_end, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out, int k, uint32_t* status) {
  __shared__ uint64_t cand_s[kFinalCap];
  __shared__ uint32_t h_s[kBins];
  const int row = blockIdx.x;
  const RowInfo ri = row_info(q_pos, row, s, S, nv_cap, max_pos_end, nullptr, false);
  const int64_t nv = ri.nv;
  const float* srow = scores ? scores + static_cast<int64_t>(row) * ld_scores : nullptr;
  int32_t* irow = idx_out + static_cast<int64_t>(row) * k;
  float* orow = score_out ? score_out + static_cast<int64_t>(row) * k : nullptr;
  if (nv <= k || scores == nullptr) {
    if (nv > k && threadIdx.x == 0) set_status(status, DSA_DEVERR_NO_INDEX);
    emit_all_visible(srow, std::min<int64_t>(nv, k), k, irow, orow);
    return;
  }
  row_select_from_scores(srow, nv, k, irow, orow, cand_s, h_s);
}

// Paged fp8 keys for the many-rows contraction: the visible tiles of each
// sequence (16 entries: 2 KiB of keys, contiguous in a block) and their
// scales copied to a dense per-sequence layout in the workspace, which the
// contraction's 16 KiB stages then stream as usual.  One workgroup per
// (tile, sequence).
__global__ __launch_bounds__(256) void k_densify_keys(const uint8_t* __restrict__ pool,
                                                      const float* __restrict__ ks_pool,
                                                      PageMap pm, int64_t e_cap,
                                                      uint8_t* __restrict__ keys,
                                                      float* __restrict__ ks,
                                                      uint32_t* status) {
  const int b = blockIdx.y, t = threadIdx.x;
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t R = paged_row(pm, b, j0, t == 0 ? status : nullptr);
  const int64_t d0 = static_cast<int64_t>(b) * idx_e_pad(e_cap) + j0;
  if (t < 128)
    reinterpret_cast<uint4*>(keys + d0 * 128)[t] = reinterpret_cast<const uint4*>(pool + R * 128)[t];
  else if (t < 144 && j0 + (t - 128) < e_cap)
    ks[static_cast<int64_t>(b) * e_cap + j0 + (t - 128)] = ks_pool[R + (t - 128)];
}

struct Plan {
  int64_t nv_cap, ld;
  bool mfma, cand, pre, dense_copy;
  int ent, nb, nw, cap;
  size_t off_scores, off_cand, off_meta, off_pre, off_dkeys, off_dks, total;
};

Plan plan(const dsa_index_args& a) {
  Plan p{};
  const int64_t rows = static_cast<int64_t>(a.n_seqs) * a.queries_per_seq;
  p.nv_cap = std::min<int64_t>(a.e_cap, n_complete(a.max_pos_end - 1, a.stride, a.span));
  if (p.nv_cap < 0) p.nv_cap = 0;
  p.ld = (p.nv_cap + 63) / 64 * 64;
  p.mfma = a.keys != nullptr && (a.dtype == DSA_FP8_E4M3 || a.dtype == DSA_FP4_E2M1) &&
           a.dim == 128 && a.heads <= 16;
  // entries per stream workgroup (1024: at 1M context 1024 workgroups of 4
  // waves keep every SIMD busy; 2048 halves the waves and loses more to
  // latency than it saves in candidate extraction)
  p.ent = 1024;
  p.nb = static_cast<int>(ceil_div(p.nv_cap, p.ent));
  p.nw = 4 * p.nb;  // waves per row, ent / 4 entries each
  // Candidates per wave: the union holds >= 2k and fits the final LDS pass
  // (one wave threshold per thread there: nw <= kSel).  A wave of 256
  // entries at 1M context holds ~0.5 of the row's top 512; more than 6 of
  // them has probability ~1e-6 per wave for unstructured scores (~1e-3 per
  // row), and such a wave is scored again in full by the final pass.
  p.cap = static_cast<int>(std::min<int64_t>(
      32, std::max<int64_t>(6, ceil_div(4 * static_cast<int64_t>(a.k), std::max(1, p.nw)))));
  p.cand = p.mfma && p.nv_cap > a.k && p.nw <= kSel &&
           static_cast<int64_t>(p.nw) * p.cap <= kFinalCap &&
           static_cast<int64_t>(p.nw) * p.cap >= 2 * static_cast<int64_t>(a.k);
  // many rows per sequence: the fp8 contraction with exact correction
  p.pre = prefill_index_applies(a, p.nv_cap);
  if (p.pre) p.cand = false;
  size_t off = 0;
  p.off_scores = off;
  off = align_up(off + static_cast<size_t>(rows) * p.ld * sizeof(float));
  p.off_cand = off;
  if (p.cand) off = align_up(off + static_cast<size_t>(rows) * p.nw * p.cap * sizeof(uint64_t));
  p.off_meta = off;
  if (p.cand) off = align_up(off + static_cast<size_t>(rows) * p.nw * sizeof(uint32_t));
  p.off_pre = off;
  if (p.pre) off = align_up(off + prefill_index_ws_bytes(a, p.nv_cap));
  // paged keys for the contraction: a dense copy of the visible tiles
  p.dense_copy = p.pre && a.paging.block_table != nullptr;
  p.off_dkeys = off;
  if (p.dense_copy) off = align_up(off + static_cast<size_t>(a.n_seqs) * idx_e_pad(a.e_cap) * 128);
  p.off_dks = off;
  if (p.dense_copy) off = align_up(off + static_cast<size_t>(a.n_seqs) * a.e_cap * sizeof(float));
  p.total = off;
  return p;
}

void launch_cand_final(const dsa_index_args& a, const Plan& P, float* scores, uint64_t* cand,
                       uint32_t* meta, int rows, int Tq, hipStream_t st) {
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(rows), dim3(kSel), 0, st, scores, P.ld, a.q_pos, a.stride,
                       a.span, P.nv_cap, a.max_pos_end, cand, meta, P.nw, P.cap, a.idx_out,
                       a.score_out, a.k, static_cast<const uint8_t*>(a.q), a.q_scale, a.w,
                       static_cast<const uint8_t*>(a.keys), a.k_scale, a.k_mx_scale, Tq, a.heads,
                       a.e_cap, make_paging(a.paging).ent, a.status);
  };
  if (a.dtype == DSA_FP4_E2M1) go(k_topk_cand_final<DSA_FP4_E2M1>);
  else go(k_topk_cand_final<DSA_FP8_E4M3>);
}

}  // namespace

size_t index_topk_ws_bytes(const dsa_index_args& a) { return plan(a).total; }

dsa_status launch_index_topk(const dsa_index_args& a, void* ws, hipStream_t st) {
  const Plan P = plan(a);
  const int rows = a.n_seqs * a.queries_per_seq;
  char* base = static_cast<char*>(ws);
  float* scores = reinterpret_cast<float*>(base + P.off_scores);
  uint64_t* cand = reinterpret_cast<uint64_t*>(base + P.off_cand);
  uint32_t* meta = reinterpret_cast<uint32_t*>(base + P.off_meta);
  const bool no_keys = a.keys == nullptr;  // only allowed when k >= every n_vis
  dsa_status rc;
  if (P.pre && P.dense_copy) {
    dsa_index_args d = a;
    d.keys = base + P.off_dkeys;
    d.k_scale = reinterpret_cast<float*>(base + P.off_dks);
    d.paging = dsa_paging{};
    if (P.nv_cap > 0) {
      hipLaunchKernelGGL(k_densify_keys, dim3(static_cast<unsigned>(ceil_div(P.nv_cap, 16)), a.n_seqs),
                         dim3(256), 0, st, static_cast<const uint8_t*>(a.keys), a.k_scale,
                         make_paging(a.paging).ent, a.e_cap, reinterpret_cast<uint8_t*>(base + P.off_dkeys),
                         reinterpret_cast<float*>(base + P.off_dks), a.status);
      rc = hip_check(hipGetLastError(), "k_densify_keys launch");
      if (rc != DSA_OK) return rc;
    }
    return launch_prefill_index_topk(d, P.nv_cap, scores, P.ld, base + P.off_pre, st);
  }
  if (P.pre) return launch_prefill_index_topk(a, P.nv_cap, scores, P.ld, base + P.off_pre, st);
  if (!no_keys && P.nv_cap > 0) {
    const hipEvent_t e0 = call_timing().index0, e1 = call_timing().index1;
    if (P.mfma) {
      dim3 grid(static_cast<unsigned>(P.nb), rows);
      auto go = [&](auto kern) {
        launch_timed(kern, grid, dim3(kThreads), 0, st, e0, e1, static_cast<const uint8_t*>(a.q),
                     a.q_scale, a.w, static_cast<const uint8_t*>(a.keys), a.k_scale, a.k_mx_scale,
                     a.q_pos, a.queries_per_seq, a.heads, a.stride, a.span, a.e_cap, P.nv_cap,
                     a.max_pos_end, scores, P.ld, cand, meta, P.cap, a.status,
                     make_paging(a.paging).ent);
      };
      const bool fp4 = a.dtype == DSA_FP4_E2M1, paged = a.paging.block_table != nullptr;
      auto by_fmt = [&](auto tag_cand) {
        constexpr bool kC = decltype(tag_cand)::value;
        if (fp4) {
          if (paged) go(k_index_fp8_stream<kC, 1024, DSA_FP4_E2M1, true>);
          else go(k_index_fp8_stream<kC, 1024, DSA_FP4_E2M1, false>);
        } else if (paged) {
          go(k_index_fp8_stream<kC, 1024, DSA_FP8_E4M3, true>);
        } else {
          go(k_index_fp8_stream<kC, 1024, DSA_FP8_E4M3, false>);
        }
      };
      if (P.cand) by_fmt(std::true_type{});
      else by_fmt(std::false_type{});
    } else {
      dim3 grid(static_cast<unsigned>(ceil_div(P.nv_cap, kThreads)), rows);
      const size_t shm = (static_cast<size_t>(a.heads) * a.dim + a.heads) * sizeof(float);
      if (a.dtype == DSA_F32)
        launch_timed(k_index_generic<float>, grid, dim3(kThreads), shm, st, e0, e1,
                           static_cast<const float*>(a.q), a.q_scale, a.w,
                           static_cast<const float*>(a.keys), a.k_scale, a.q_pos,
                           a.queries_per_seq, a.heads, a.dim, a.stride, a.span, a.e_cap, P.nv_cap,
                           a.max_pos_end, scores, P.ld, a.status, make_paging(a.paging).ent);
      else
        launch_timed(k_index_generic<uint8_t>, grid, dim3(kThreads), shm, st, e0, e1,
                           static_cast<const uint8_t*>(a.q), a.q_scale, a.w,
                           static_cast<const uint8_t*>(a.keys), a.k_scale, a.q_pos,
                           a.queries_per_seq, a.heads, a.dim, a.stride, a.span, a.e_cap, P.nv_cap,
                           a.max_pos_end, scores, P.ld, a.status, make_paging(a.paging).ent);
    }
    rc = hip_check(hipGetLastError(), "indexer launch");
    if (rc != DSA_OK) return rc;
  }
  if (P.cand && !no_keys) {
    launch_cand_final(a, P, scores, cand, meta, rows, a.queries_per_seq, st);
  } else {
    hipLaunchKernelGGL(k_topk_rows, dim3(rows), dim3(kSel), 0, st, no_keys ? nullptr : scores,
                       P.ld, a.q_pos, a.stride, a.span, P.nv_cap, a.max_pos_end, a.idx_out,
                       a.score_out, a.k, a.status);
  }
  return hip_check(hipGetLastError(), "top-k launch");
}

dsa_status launch_decode_index_topk(const dsa_index_args& a, void* ws, const dsa_layer_args& la,
                                    int64_t* qpos, bool insert_window, float* cs_tab, void* q_rot,
                                    hipStream_t st) {
  const Plan P = plan(a);
  const bool fused = P.cand && a.keys != nullptr && P.nv_cap > 0 && a.queries_per_seq == 1 &&
                     (a.dtype == DSA_FP8_E4M3 || a.dtype == DSA_FP4_E2M1) &&
                     la.dtype == DSA_BF16;
  if (!fused) {
    // no indexer keys (k >= every visible count): the selection is every
    // visible entry, written by the prologue (one launch fewer)
    const bool all_vis = a.keys == nullptr && a.score_out == nullptr && a.queries_per_seq == 1;
    dsa_status rc = launch_decode_prologue(la, qpos, insert_window, cs_tab, q_rot, st,
                                           all_vis ? a.idx_out : nullptr, a.k, P.nv_cap);
    if (rc != DSA_OK || all_vis) return rc;
    return launch_index_topk(a, ws, st);
  }
  const int rows = a.n_seqs;
  char* base = static_cast<char*>(ws);
  float* scores = reinterpret_cast<float*>(base + P.off_scores);
  uint64_t* cand = reinterpret_cast<uint64_t*>(base + P.off_cand);
  uint32_t* meta = reinterpret_cast<uint32_t*>(base + P.off_meta);
  const PrologueArgs pa = make_prologue_args(la, qpos, insert_window, cs_tab, q_rot);
  auto go = [&](auto kern) {
    launch_timed(kern, dim3((P.nb + kPrologueRoles + pa.nq_roles) * rows), dim3(kThreads), 0, st,
                 call_timing().index0, call_timing().index1,
                 static_cast<const uint8_t*>(a.q), a.q_scale, a.w,
                 static_cast<const uint8_t*>(a.keys), a.k_scale, a.k_mx_scale, a.q_pos, a.heads,
                 a.stride, a.span, a.e_cap, P.nv_cap, a.max_pos_end, scores, P.ld, cand, meta,
                 P.cap, P.nb, pa, a.status);
  };
  auto by_main = [&](auto tag_fmt, auto tag_paged) {
    constexpr int kF = decltype(tag_fmt)::value;
    constexpr bool kP = decltype(tag_paged)::value;
    if (la.main_fp8) go(k_decode_index<uint16_t, kF, 1024, true, kP>);
    else go(k_decode_index<uint16_t, kF, 1024, false, kP>);
  };
  const bool paged = a.paging.block_table != nullptr;
  using Fp4 = std::integral_constant<int, DSA_FP4_E2M1>;
  using Fp8 = std::integral_constant<int, DSA_FP8_E4M3>;
  if (a.dtype == DSA_FP4_E2M1) {
    if (paged) by_main(Fp4{}, std::true_type{});
    else by_main(Fp4{}, std::false_type{});
  } else if (paged) {
    by_main(Fp8{}, std::true_type{});
  } else {
    by_main(Fp8{}, std::false_type{});
  }
  dsa_status rc = hip_check(hipGetLastError(), "k_decode_index launch");
  if (rc != DSA_OK) return rc;
  launch_cand_final(a, P, scores, cand, meta, rows, 1, st);
  return hip_check(hipGetLastError(), "top-k launch");
}

}  // namespace dsa
