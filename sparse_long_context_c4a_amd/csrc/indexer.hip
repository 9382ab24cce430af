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
#include "common.h"
#include "decode_impl.h"
#include "indexer_impl.h"
#include "internal.h"

namespace dsa {
namespace {

constexpr int kBins = 4096;           // row select histogram bins
constexpr int kFinalCap = 8192;       // candidates resolved in LDS

// ------------------------------------------------------- block primitives
// The selection kernels run one workgroup of kSel threads (16 wave64s) per
// query row; every helper below assumes blockDim.x == kSel.
constexpr int kSel = 1024;
constexpr int kSelWaves = kSel / 64;

__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int o) {
  return static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o, 64));
}

// Block-wide max / min / sum over NT threads; every thread gets the result.
template <int kOp, int NT = kSel>  // 0 max, 1 min, 2 sum
__device__ __forceinline__ uint32_t block_reduce_u32(uint32_t v) {
  __shared__ uint32_t wv[NT / 64];
  const int t = threadIdx.x;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t y = shfl_xor_u32(v, o);
    v = kOp == 0 ? max(v, y) : kOp == 1 ? min(v, y) : v + y;
  }
  if ((t & 63) == 0) wv[t >> 6] = v;
  __syncthreads();
  uint32_t r = wv[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) r = kOp == 0 ? max(r, wv[i]) : kOp == 1 ? min(r, wv[i]) : r + wv[i];
  __syncthreads();
  return r;
}

// Exclusive prefix sum of one value per thread (in thread order) and the total.
template <int NT = kSel>
__device__ __forceinline__ uint32_t block_prefix_excl(uint32_t v, uint32_t* total) {
  __shared__ uint32_t wsum[NT / 64];
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = static_cast<uint32_t>(__shfl_up(static_cast<int>(x), o, 64));
    if (l >= o) x += y;
  }
  if (l == 63) wsum[w] = x;
  __syncthreads();
  uint32_t add = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    add += i < w ? wsum[i] : 0u;
    tot += wsum[i];
  }
  *total = tot;
  __syncthreads();
  return x - v + add;
}

// Position of this lane's item among the wave's items with `cond`, after a
// block-wide counter: one LDS atomic per wave.
__device__ __forceinline__ uint32_t wave_alloc(bool cond, uint32_t* ctr) {
  const uint64_t m = __ballot(cond);
  const int l = threadIdx.x & 63;
  uint32_t base = 0;
  if (l == 0 && m) base = atomicAdd(ctr, static_cast<uint32_t>(__popcll(m)));
  base = static_cast<uint32_t>(__shfl(static_cast<int>(base), 0, 64));
  return base + static_cast<uint32_t>(__popcll(m & ((1ull << l) - 1ull)));
}

// Smallest shift with (span >> shift) < 2^bits.
__device__ __forceinline__ int range_shift(uint32_t span, int bits) {
  const int used = span == 0u ? 0 : 32 - __clz(static_cast<int>(span));
  return used > bits ? used - bits : 0;
}

// For NT threads owning `per` consecutive bins each in descending order
// (thread 0 the highest): the bin B with count(bins above B) < need <=
// count(bins >= B), plus those two counts.  local[i] of thread t is bin
// top - (per * t + i).  Requires total >= need.
struct Bin {
  uint32_t b, above, at;
};

template <int per, int NT = kSel>
__device__ __forceinline__ Bin find_bin_desc(const uint32_t (&local)[per], uint32_t top,
                                             uint32_t need) {
  __shared__ Bin res;
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) sum += local[i];
  uint32_t total;
  const uint32_t before = block_prefix_excl<NT>(sum, &total);
  const int t = threadIdx.x;
  if (before < need && before + sum >= need) {
    uint32_t c = before;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      if (c < need && c + local[i] >= need) res = Bin{top - (per * t + i), c, local[i]};
      c += local[i];
    }
  }
  __syncthreads();
  const Bin r = res;
  __syncthreads();
  return r;
}

// Keep the `need` largest of the n distinct composites in v[] (LDS): each
// is kept iff fewer than `need` others exceed it.  For small n (one wave
// compares every pair through LDS broadcasts); calls f(v) for the kept.
template <typename F>
__device__ void keep_largest_small(const uint64_t* v, int n, uint32_t need, F f) {
  const int t = threadIdx.x;
  if (t < n) {
    const uint64_t x = v[t];
    uint32_t rank = 0;
    for (int i = 0; i < n; ++i) rank += v[i] > x ? 1u : 0u;
    if (rank < need) f(x);
  }
}

// Exact selection of the `need` largest of n distinct composites c[] (LDS)
// by radix passes of 8 bits, for the rare large tie groups; returns the
// smallest kept composite.  pred() filters which elements take part.
template <int NT = kSel, typename P>
__device__ uint64_t kth_largest_composite(const uint64_t* c, int n, uint32_t need, P pred) {
  static_assert(NT >= 256, "one thread per digit");
  __shared__ uint32_t cnt[256];
  __shared__ uint32_t res[3];
  const int t = threadIdx.x;
  uint64_t prefix = 0, mask = 0;
  for (int sh = 56; sh >= 0; sh -= 8) {
    if (t < 256) cnt[t] = 0;
    __syncthreads();
    for (int i = t; i < n; i += NT) {
      const uint64_t v = c[i];
      if (pred(v) && (v & mask) == prefix) atomicAdd(&cnt[(v >> sh) & 255u], 1u);
    }
    __syncthreads();
    // digit d: count(digits > d) < need <= count(digits >= d); thread t < 256
    // owns digit 255 - t (descending)
    const uint32_t mine = t < 256 ? cnt[255 - t] : 0u;
    uint32_t total;
    const uint32_t before = block_prefix_excl<NT>(mine, &total);
    if (t < 256 && before < need && before + mine >= need) {
      res[0] = 255u - t;
      res[1] = before;
      res[2] = mine;
    }
    __syncthreads();
    const uint32_t d = res[0], above = res[1], at = res[2];
    __syncthreads();
    prefix |= static_cast<uint64_t>(d) << sh;
    mask |= static_cast<uint64_t>(255u) << sh;
    need -= above;
    if (at == need) break;  // every composite with this prefix is kept
  }
  return prefix;
}

// Rows with n_vis <= k: every visible entry, in index order, then padding.
__device__ __forceinline__ void emit_all_visible(const float* srow, int64_t nv, int k, int32_t* idx_row,
                                 float* score_row) {
  for (int i = threadIdx.x; i < k; i += blockDim.x) {
    if (i < nv) emit(idx_row, score_row, i, i, srow ? srow[i] : 0.f);
    else {
      idx_row[i] = -1;
      if (score_row) score_row[i] = __uint_as_float(0x7fc00000u);
    }
  }
}

// The `k` largest (key, complemented index) composites among the n slots of
// c[] (LDS; 0 = empty slot), emitted to positions 0..k-1 in no particular
// order.  A 2048-bin histogram over the keys' own range finds the bin
// holding the k-th; entries above it go out directly, the bin's entries are
// resolved exactly.  tmp: kTmp u64 of LDS; hist: 2048 u32 of LDS.
constexpr int kTmpCap = 1024;

template <int NT = kSel, int kTmp = kTmpCap>
__device__ __forceinline__ void select_topk_composites(const uint64_t* c, int n, uint32_t k, int32_t* irow,
                                       float* orow, uint64_t* tmp, uint32_t* hist) {
  constexpr int kPer = 2048 / NT;
  __shared__ uint32_t pos_above, pos_bin, n_tmp;
  const int t = threadIdx.x;
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int i = t; i < n; i += NT) {
    const uint64_t v = c[i];
    if (v == 0) continue;
    lo = min(lo, static_cast<uint32_t>(v >> 32));
    hi = max(hi, static_cast<uint32_t>(v >> 32));
  }
  for (int i = t; i < 2048; i += NT) hist[i] = 0u;
  if (t == 0) pos_above = pos_bin = n_tmp = 0u;
  lo = block_reduce_u32<1, NT>(lo);  // has barriers
  hi = block_reduce_u32<0, NT>(hi);
  const int shift = range_shift(hi - lo, 11);
  for (int i = t; i < n; i += NT) {
    const uint64_t v = c[i];
    if (v != 0) atomicAdd(&hist[(static_cast<uint32_t>(v >> 32) - lo) >> shift], 1u);
  }
  __syncthreads();
  uint32_t local[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) local[i] = hist[2047 - (kPer * t + i)];
  const Bin br = find_bin_desc<kPer, NT>(local, 2047u, k);
  const uint32_t B = br.b, above = br.above, at = br.at;
  const bool fits = at <= static_cast<uint32_t>(kTmp);
  for (int i0 = 0; i0 < n; i0 += NT) {
    const int i = i0 + t;
    const uint64_t v = i < n ? c[i] : 0ull;
    const uint32_t bin = (static_cast<uint32_t>(v >> 32) - lo) >> shift;
    const bool up = v != 0 && bin > B;
    const uint32_t p = wave_alloc(up, &pos_above);
    if (up && p < above) emit(irow, orow, p, comp_index(v), key_to_float(static_cast<uint32_t>(v >> 32)));
    const bool mid = v != 0 && bin == B && fits;
    const uint32_t q = wave_alloc(mid, &n_tmp);
    if (mid) tmp[q] = v;
  }
  __syncthreads();
  const uint32_t need = k - above;
  auto out_bin = [&](uint64_t v) {
    const uint32_t p = atomicAdd(&pos_bin, 1u);
    if (p < need) emit(irow, orow, above + p, comp_index(v), key_to_float(static_cast<uint32_t>(v >> 32)));
  };
  if (fits && at <= 64) {
    keep_largest_small(tmp, static_cast<int>(at), need, out_bin);
  } else if (fits) {
    const uint64_t cut = kth_largest_composite<NT>(tmp, static_cast<int>(at), need,
                                                   [](uint64_t) { return true; });
    for (int i = t; i < static_cast<int>(at); i += NT)
      if (tmp[i] >= cut) out_bin(tmp[i]);
  } else {
    // very many keys in one bin: radix over the bin's composites in place
    const uint64_t bin_lo = (static_cast<uint64_t>(lo) + (static_cast<uint64_t>(B) << shift)) << 32;
    const uint64_t khi = static_cast<uint64_t>(lo) + (static_cast<uint64_t>(B + 1u) << shift);
    const uint64_t bin_hi = khi > 0xffffffffull ? ~0ull : (khi << 32);  // exclusive, or open
    auto in_bin = [=](uint64_t v) {
      return v != 0 && v >= bin_lo && (v < bin_hi || bin_hi == ~0ull);
    };
    const uint64_t cut = kth_largest_composite<NT>(c, n, need, in_bin);
    for (int i = t; i < n; i += NT)
      if (in_bin(c[i]) && c[i] >= cut) out_bin(c[i]);
  }
  __syncthreads();
}

// Visit the first nv scores of a row (read as float4; ld_scores is a
// multiple of 4 floats and entries past nv are skipped): f(j, score).
template <int NT = kSel, typename F>
__device__ __forceinline__ void for_row(const float* srow, int64_t nv, F f) {
  const float4* r4 = reinterpret_cast<const float4*>(srow);
  const int64_t n4 = (nv + 3) / 4;
  for (int64_t i = threadIdx.x; i < n4; i += 4 * NT) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t ii = i + u * NT;
      v[u] = ii < n4 ? r4[ii] : float4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = 4 * (i + u * NT);
      if (j + 0 < nv) f(j + 0, v[u].x);
      if (j + 1 < nv) f(j + 1, v[u].y);
      if (j + 2 < nv) f(j + 2, v[u].z);
      if (j + 3 < nv) f(j + 3, v[u].w);
    }
  }
}

// Exact top-k of one row from its scores in global memory (nv > k): a
// 4096-bin histogram over the row's own key range finds the bin holding the
// k-th score; entries above it go straight out and the bin's entries are
// resolved exactly on (key, complemented index).  cand_s: kCap u64 of LDS,
// h_s: kNB u32 of LDS (kNB = 2^kLogNB bins).
template <int kCap = kFinalCap, int NT = kSel, int kLogNB = 12>
__device__ __forceinline__ void row_select_from_scores(const float* srow, int64_t nv, int k, int32_t* irow,
                                       float* orow, uint64_t* cand_s, uint32_t* h_s) {
  constexpr int kNB = 1 << kLogNB, kPer = kNB / NT;
  __shared__ uint32_t cnt_above, cnt_cand, out_pos;
  const int t = threadIdx.x;
  uint32_t lo = 0xffffffffu, hi = 0u;
  for_row<NT>(srow, nv, [&](int64_t, float sc) {
    const uint32_t key = order_key(sc);
    lo = min(lo, key);
    hi = max(hi, key);
  });
  for (int i = t; i < kNB; i += NT) h_s[i] = 0;
  if (t == 0) cnt_above = cnt_cand = out_pos = 0;
  lo = block_reduce_u32<1, NT>(lo);
  hi = block_reduce_u32<0, NT>(hi);
  const int shift = range_shift(hi - lo, kLogNB);
  for_row<NT>(srow, nv, [&](int64_t, float sc) { atomicAdd(&h_s[(order_key(sc) - lo) >> shift], 1u); });
  __syncthreads();
  uint32_t local[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) local[i] = h_s[kNB - 1 - (kPer * t + i)];
  const Bin br = find_bin_desc<kPer, NT>(local, kNB - 1u, static_cast<uint32_t>(k));
  const uint32_t thr = br.b, above = br.above, at = br.at;
  const bool fits = at <= static_cast<uint32_t>(kCap);
  for_row<NT>(srow, nv, [&](int64_t j, float sc) {
    const uint32_t key = order_key(sc);
    const uint32_t bin = (key - lo) >> shift;
    if (bin > thr) {
      const uint32_t p = atomicAdd(&cnt_above, 1u);
      if (p < static_cast<uint32_t>(k)) emit(irow, orow, p, static_cast<uint32_t>(j), sc);
    } else if (bin == thr && fits) {
      const uint32_t p = atomicAdd(&cnt_cand, 1u);
      if (p < static_cast<uint32_t>(kCap)) cand_s[p] = composite(key, static_cast<uint32_t>(j));
    }
  });
  __syncthreads();
  const uint32_t need = static_cast<uint32_t>(k) - above;
  if (fits) {
    auto out_bin = [&](uint64_t v) {
      const uint32_t p = atomicAdd(&out_pos, 1u);
      if (p < need)
        emit(irow, orow, above + p, comp_index(v), key_to_float(static_cast<uint32_t>(v >> 32)));
    };
    if (at <= 64) {
      keep_largest_small(cand_s, static_cast<int>(at), need, out_bin);
    } else {
      const uint64_t cut = kth_largest_composite<NT>(cand_s, static_cast<int>(at), need,
                                                     [](uint64_t) { return true; });
      for (int i = t; i < static_cast<int>(at); i += NT)
        if (cand_s[i] >= cut) out_bin(cand_s[i]);
    }
  } else {
    // streaming radix over the bin's entries, composites built on the fly
    __shared__ uint32_t cnt[256];
    __shared__ uint32_t res[3];
    uint64_t prefix = 0, mask = 0;
    uint32_t rem = need;
    for (int sh = 56; sh >= 0; sh -= 8) {
      if (t < 256) cnt[t] = 0;
      __syncthreads();
      for_row<NT>(srow, nv, [&](int64_t j, float sc) {
        const uint32_t key = order_key(sc);
        if (((key - lo) >> shift) != thr) return;
        const uint64_t v = composite(key, static_cast<uint32_t>(j));
        if ((v & mask) == prefix) atomicAdd(&cnt[(v >> sh) & 255u], 1u);
      });
      __syncthreads();
      const uint32_t mine = t < 256 ? cnt[255 - t] : 0u;
      uint32_t total;
      const uint32_t before = block_prefix_excl<NT>(mine, &total);
      if (t < 256 && before < rem && before + mine >= rem) {
        res[0] = 255u - t;
        res[1] = before;
        res[2] = mine;
      }
      __syncthreads();
      const uint32_t d = res[0], ab = res[1], at2 = res[2];
      __syncthreads();
      prefix |= static_cast<uint64_t>(d) << sh;
      mask |= static_cast<uint64_t>(255u) << sh;
      rem -= ab;
      if (at2 == rem) break;
    }
    const uint64_t cut = prefix;
    for_row<NT>(srow, nv, [&](int64_t j, float sc) {
      const uint32_t key = order_key(sc);
      if (((key - lo) >> shift) != thr) return;
      const uint64_t v = composite(key, static_cast<uint32_t>(j));
      if (v >= cut) {
        const uint32_t p = atomicAdd(&out_pos, 1u);
        if (p < need) emit(irow, orow, above + p, comp_index(v), sc);
      }
    });
  }
  __syncthreads();
}

// --------------------------------------------------- stream (decode) kernel
// Operand layout: lane l owns entry (or head) n = l % 16 and, within the
// 128-byte vector, bytes [16 g, 16 g + 16) and [64 + 16 g, 64 + 16 g + 16)
// with g = l / 16; MFMA c of the four takes the lane's bytes [8 c, 8 c + 8)
// of those 32.  A and B use the same byte-to-k assignment, so the four MFMAs
// sum every one of the 128 products exactly once.  With the keys' tile
// layout each of the two 16-byte loads of a wave reads 1 KiB of contiguous
// bytes.
template <bool kCand, int kEnt>
__global__ __launch_bounds__(kThreads) void k_index_fp8_stream(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ keys, const float* __restrict__ k_scale,
    const int64_t* __restrict__ q_pos, int Tq, int Hi, int s, int S, int64_t e_cap,
    int64_t nv_cap, int64_t max_pos_end, float* __restrict__ scores, int64_t ld_scores,
    uint64_t* __restrict__ cand, uint32_t* __restrict__ meta, int cap, uint32_t* status) {
  index_stream_block<kCand, kEnt>(blockIdx.x, gridDim.x, blockIdx.y, q, q_scale, w, keys, k_scale, q_pos,
                            Tq, Hi, s, S, e_cap, nv_cap, max_pos_end, scores, ld_scores, cand,
                            meta, cap, status);
}

// A decode step's indexer with the step's state updates riding along: blocks
// x < nb stream the keys of row y; blocks nb, nb+1, nb+2 of row y (one
// sequence per row) run the prologue roles, whose writes the indexer does not
// read (see decode_prologue_block), so they overlap the key stream instead
// of adding a launch and its latency in front of it.
template <typename MainT, int kIdxOut, int kEnt>
__global__ __launch_bounds__(kThreads) void k_decode_index(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ keys, const float* __restrict__ k_scale,
    const int64_t* __restrict__ q_pos, int Hi, int s, int S, int64_t e_cap, int64_t nv_cap,
    int64_t max_pos_end, float* __restrict__ scores, int64_t ld_scores,
    uint64_t* __restrict__ cand, uint32_t* __restrict__ meta, int cap, int nb, PrologueArgs pa,
    uint32_t* status) {
  if (static_cast<int>(blockIdx.x) < nb)
    index_stream_block<true, kEnt>(blockIdx.x, nb, blockIdx.y, q, q_scale, w, keys, k_scale, q_pos, 1,
                             Hi, s, S, e_cap, nv_cap, max_pos_end, scores, ld_scores, cand, meta,
                             cap, status);
  else
    decode_prologue_block<MainT, kIdxOut>(blockIdx.x - nb, blockIdx.y, pa);
}

// ------------------------------------------------------------- generic VALU
// Any Hi, Di; q and keys f32 or fp8.  One entry per thread; scores only.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_index_generic(
    const T* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const T* __restrict__ keys, const float* __restrict__ k_scale, const int64_t* __restrict__ q_pos,
    int Tq, int Hi, int Di, int s, int S, int64_t e_cap, int64_t nv_cap, int64_t max_pos_end,
    float* __restrict__ scores, int64_t ld_scores, uint32_t* status) {
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
    // fp8 keys of dim 128 use the tile layout, everything else is row-major
    const bool tiled = sizeof(T) == 1 && Di == 128;
    const T* kr = keys + (tiled ? 0 : (static_cast<int64_t>(b) * e_cap + ent) * Di);
    const int64_t e_pad = idx_e_pad(e_cap);
    float tot = 0.f;
    for (int h = 0; h < Hi; ++h) {
      float d = 0.f;
      for (int i = 0; i < Di; ++i) {
        float kv;
        if constexpr (sizeof(T) == 1)
          kv = fp8_to_f32(tiled ? kr[idx_tile_off(b, e_pad, ent, i)] : kr[i]);
        else kv = kr[i];
        d = fmaf(q_s[h * Di + i], kv, d);
      }
      tot += w_s[h] * fmaxf(d, 0.f);
    }
    if constexpr (sizeof(T) == 1) tot *= k_scale[static_cast<int64_t>(b) * e_cap + ent];
    scores[static_cast<int64_t>(row) * ld_scores + ent] = tot;
  }
}

// ------------------------------------------------------------ final passes
// Candidate path: union of the waves' candidates (empty slots are 0), the
// certificate, and the exact top k; falls back to the full-row select when
// the certificate does not hold.  The candidates stay in registers (8 per
// thread) through one combined reduction pass, one histogram pass and the
// emit pass.
__global__ __launch_bounds__(kSel) void k_topk_cand_final(
    float* __restrict__ scores, int64_t ld_scores, const int64_t* __restrict__ q_pos,
    int s, int S, int64_t nv_cap, int64_t max_pos_end, const uint64_t* __restrict__ cand,
    const uint32_t* __restrict__ meta, int nw, int cap, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out, int k, const uint8_t* __restrict__ q,
    const float* __restrict__ q_scale, const float* __restrict__ hw,
    const uint8_t* __restrict__ keys, const float* __restrict__ k_scale, int Tq, int Hi,
    int64_t e_cap) {
  __shared__ uint64_t cand_s[kFinalCap];
  __shared__ uint64_t tmp_s[kTmpCap];
  __shared__ uint32_t h_s[kBins];
  __shared__ uint32_t red[3][kSelWaves];
  __shared__ uint32_t pos_above, pos_bin, n_tmp;
  const int row = blockIdx.x, t = threadIdx.x, l = t & 63, w = t >> 6;
  const RowInfo ri = row_info(q_pos, row, s, S, nv_cap, max_pos_end, nullptr, false);
  const int64_t nv = ri.nv;
  float* srow = scores + static_cast<int64_t>(row) * ld_scores;
  int32_t* irow = idx_out + static_cast<int64_t>(row) * k;
  float* orow = score_out ? score_out + static_cast<int64_t>(row) * k : nullptr;
  const int b = row / Tq;
  const uint8_t* kb = keys + static_cast<int64_t>(b) * idx_e_pad(e_cap) * 128;
  const float* ksb = k_scale + static_cast<int64_t>(b) * e_cap;
  v8bf aq[4];
  float wv[4];
  if (nv <= k) {
    if (orow) {  // the visible entries' scores (the stream kept them in registers)
      exact_row_operands(q, q_scale, hw, row, Hi, aq, wv);
      score_row_exact(aq, wv, kb, ksb, nv, srow, kSelWaves);
      __syncthreads();
    }
    emit_all_visible(srow, nv, k, irow, orow);
    return;
  }
  const int slots = nw * cap;  // <= kFinalCap by construction
  const uint32_t* mrow = meta + static_cast<int64_t>(row) * nw;
  const uint64_t* crow = cand + static_cast<int64_t>(row) * slots;
  constexpr int kPer = kFinalCap / kSel;
  uint64_t v[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) v[u] = t + u * kSel < slots ? crow[t + u * kSel] : 0ull;
  uint32_t tm = 0, lo = 0xffffffffu, hi = 0u;
  for (int b = t; b < nw; b += kSel) tm = max(tm, mrow[b]);
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (v[u] != 0) {
      lo = min(lo, static_cast<uint32_t>(v[u] >> 32));
      hi = max(hi, static_cast<uint32_t>(v[u] >> 32));
    }
  // one combined block reduction: max t_w, min and max candidate key
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    tm = max(tm, shfl_xor_u32(tm, o));
    lo = min(lo, shfl_xor_u32(lo, o));
    hi = max(hi, shfl_xor_u32(hi, o));
  }
  if (l == 0) {
    red[0][w] = tm;
    red[1][w] = lo;
    red[2][w] = hi;
  }
  for (int i = t; i < 2048; i += kSel) h_s[i] = 0u;
  if (t == 0) pos_above = pos_bin = n_tmp = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    tm = max(tm, red[0][i]);
    lo = min(lo, red[1][i]);
    hi = max(hi, red[2][i]);
  }
  // the certificate count (at least k candidates with key >= max_w t_w) and
  // the histogram over the candidates' key range, in one pass
  const int shift = range_shift(hi - lo, 11);
  uint32_t c_ge = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (v[u] != 0) {
      const uint32_t key = static_cast<uint32_t>(v[u] >> 32);
      c_ge += key >= tm ? 1u : 0u;
      atomicAdd(&h_s[(key - lo) >> shift], 1u);
    }
  const bool ok = block_reduce_u32<2>(c_ge) >= static_cast<uint32_t>(k);  // barriers
  if (!ok) {
    // the certificate failed: score the row exactly in full, then select
    exact_row_operands(q, q_scale, hw, row, Hi, aq, wv);
    score_row_exact(aq, wv, kb, ksb, nv, srow, kSelWaves);
    __syncthreads();
    row_select_from_scores(srow, nv, k, irow, orow, cand_s, h_s);
    return;
  }
  const uint32_t local[2] = {h_s[2047 - 2 * t], h_s[2046 - 2 * t]};
  const Bin br = find_bin_desc<2>(local, 2047u, static_cast<uint32_t>(k));
  const uint32_t B = br.b, above = br.above, at = br.at;
  const bool fits = at <= static_cast<uint32_t>(kTmpCap);
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const uint64_t x = v[u];
    const uint32_t bin = (static_cast<uint32_t>(x >> 32) - lo) >> shift;
    const bool up = x != 0 && bin > B;
    const uint32_t p = wave_alloc(up, &pos_above);
    if (up && p < above) emit(irow, orow, p, comp_index(x), key_to_float(static_cast<uint32_t>(x >> 32)));
    const bool mid = x != 0 && bin == B;
    const uint32_t q = wave_alloc(mid, &n_tmp);
    if (mid && fits) tmp_s[q] = x;
    if (!fits) cand_s[t + u * kSel] = mid ? x : 0ull;  // only the bin's members
  }
  __syncthreads();
  const uint32_t need = static_cast<uint32_t>(k) - above;
  auto out_bin = [&](uint64_t x) {
    const uint32_t p = atomicAdd(&pos_bin, 1u);
    if (p < need) emit(irow, orow, above + p, comp_index(x), key_to_float(static_cast<uint32_t>(x >> 32)));
  };
  if (fits && at <= 64) {
    keep_largest_small(tmp_s, static_cast<int>(at), need, out_bin);
  } else if (fits) {
    const uint64_t cut = kth_largest_composite(tmp_s, static_cast<int>(at), need,
                                               [](uint64_t) { return true; });
    for (int i = t; i < static_cast<int>(at); i += kSel)
      if (tmp_s[i] >= cut) out_bin(tmp_s[i]);
  } else {
    const uint64_t cut = kth_largest_composite(cand_s, kFinalCap, need,
                                               [](uint64_t x) { return x != 0; });
    for (int i = t; i < kFinalCap; i += kSel)
      if (cand_s[i] != 0 && cand_s[i] >= cut) out_bin(cand_s[i]);
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

// ------------------------------------------------------------ prefill path
// Many query rows against one sequence's keys is a dense contraction.  It
// runs on the matrix cores in two stages, with an exact correction so that
// the selection stays the exact Top-k:
//
//  k_pidx_prep  (one workgroup per kPQ rows of one sequence): nu_j = ks_j
//     ||k8_j|| over a slice of the sequence's entries (the slice's largest
//     value); per row the error scale beta (below) and the threshold theta,
//     the r-th largest approximate score over a sample of whole 16-entry
//     tiles (r = 2k scaled to the sample, plus 8), rounded down to 16 key
//     bits.
//  k_pidx_main  (one workgroup per kMRows rows and a range of entry tiles;
//     the range's keys pass through LDS once for all of those rows): per
//     row and 16-entry tile, the fp8 MFMA with an E8M0 scale of 2^-9 gives
//     2^-9 q8_h . k8_j for the 16 heads; ReLU and rounding to f16; an f16
//     MFMA contracts them with the row's head weights w'_h = w_h qs_h
//     (rounded to f16 after a per-row power-of-two scaling that puts the
//     largest |w'_h| in [2^14, 2^15)), two rows per 32-deep product.  An
//     entry whose approximate score reaches theta - beta nu_max sets its bit
//     in the row's candidate mask (16 bits per tile).
//  k_pidx_select (one workgroup of kPSelT threads per row): the candidates
//     from the masks, their exact scores (bf16 MFMA on exactly widened codes
//     and f32 weights, as the decode path), the certificate #{candidates with
//     exact score >= theta} >= k, then the exact Top-k of the candidates.  If
//     the certificate fails or the candidates overflow LDS, the row is scored
//     exactly in full and selected from its scores.
//
// Why the result is exact: |approx_j - exact_j| <= beta nu_j <= beta nu_max
// (below).  A non-candidate therefore has exact_j < theta, while at least k
// candidates reach theta, so the k-th largest exact score is >= theta and
// every entry of the Top-k (ties to the lower index) is a candidate.  The
// sample only steers theta (how many candidates); the certificate carries
// the guarantee.
//
// The bound, per head h with N_h = ||q8_h|| ||k8_j|| (code units) and W =
// max_h |w'_h|: the fp8 MFMA errs by at most 2^-10 N_h (its shared
// alignment drops low-order product bits: measured up to 2^-13.4 N_h on
// heavy-tailed codes and 2^-15.5 on uniform ones); its 2^-9 scale is exact
// (bit for bit the unscaled result times 2^-9) and keeps every value within
// 128 * 448^2 * 2^-9 = 50176 < 65504, the f16 range; rounding to f16 (to
// nearest) adds 2^-11 of the value plus 2^-25 absolute (subnormals), 2^-16 in
// code units; the f16 weights add 2^-11 |w'_h| plus 2^-39 W; the f16 MFMA
// sums its exact products in f32 (measured 2^-24.5 of the sum of |products|)
// and the exact path's own f32 rounding is of the same order.  ReLU is
// 1-Lipschitz.  Summed over the heads:
//   |approx_j - exact_j| <= ks_j (1.96e-3 sum_h |w'_h| N_h
//                                 + 2^-15.9 sum_h |w'_h| + 2^-38.9 W sum_h N_h).
// A non-zero key has ||k8_j|| >= 2^-9 (the smallest e4m3 magnitude) and a
// zero key scores exactly 0 on both paths, so with
//   beta = 2e-3 sum_h |w'_h| ||q8_h|| + 2^-6 sum_h |w'_h| + 2^-38 W sum_h ||q8_h||
// the error is at most beta nu_j.  The per-row threshold is computed in
// double with a relative margin of 2^-20 and rounded down, which covers the
// f32 rounding of the comparison.
constexpr int kPQ = 8;              // rows per prep workgroup
constexpr int kPSampleTiles = 128;  // sampled 16-entry tiles per row
constexpr int kPSample = kPSampleTiles * 16;
constexpr float kPEps = 2.0e-3f;
constexpr int kMR = 8;                               // rows per main wave
constexpr int kMRows = 4 * kMR;                      // rows per main workgroup
constexpr int kMStage = 8;                           // tiles per LDS stage
constexpr int kMKeyBytes = kMStage * 16 * 128;       // the stage's keys
constexpr int kMStageBytes = kMKeyBytes + kMStage * 16 * 4;  // + their scales
constexpr int kMTargetWGs = 768;                     // three per compute unit
constexpr int kMScaleOne = 127;                      // E8M0 code of 1
constexpr int kPSelT = 256;                          // select threads per row
constexpr int kPCandCap = 3072;                      // candidates held in LDS
constexpr int kPTmpCap = 512;

struct PArgs {
  const uint8_t* q;
  const float* q_scale;
  const float* w;
  const uint8_t* keys;
  const float* k_scale;
  const int64_t* q_pos;
  int Tq, Hi, s, S, k, tiles_per_seq;
  int rg_per_seq, rg_total, tps_split;
  int64_t e_cap, nv_cap, max_pos_end, ld_t;
  float* theta;
  float* beta;
  float* nu_part;
  float* kappa_part;
  uint16_t* masks;
  uint8_t* keys_rm;  // [B, nv_cap, 128] fp8 keys, one 128-byte run per entry
  uint32_t* status;
};

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v8i as_v8i(uint4 lo, uint4 hi) {
  return v8i{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z),
             static_cast<int>(lo.w), static_cast<int>(hi.x), static_cast<int>(hi.y),
             static_cast<int>(hi.z), static_cast<int>(hi.w)};
}

// Sum of squares of the 16 e4m3 codes in one uint4 (exact products, f32 sum).
__device__ __forceinline__ float fp8x16_sumsq(uint4 v) {
  float s = 0.f;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v2f a = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), false);
    const v2f b = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), true);
    s = fmaf(a[0], a[0], s);
    s = fmaf(a[1], a[1], s);
    s = fmaf(b[0], b[0], s);
    s = fmaf(b[1], b[1], s);
  }
  return s;
}

// The prep tile's rows: sequence b, rows row0 .. row0 + nq - 1.
struct PTile {
  int b, t0, nq;
  int64_t row0;
};
__device__ __forceinline__ PTile p_tile(const PArgs& a, int tile) {
  PTile t;
  t.b = tile / a.tiles_per_seq;
  t.t0 = (tile % a.tiles_per_seq) * kPQ;
  t.nq = min(kPQ, a.Tq - t.t0);
  t.row0 = static_cast<int64_t>(t.b) * a.Tq + t.t0;
  return t;
}

// Per-lane operands of the prep tile's rows for the fp8 MFMA: A_q (lane =
// head n, bytes [16g, 16g+16) and [64+16g, 64+16g+16) of the head's 128, the
// same byte-to-k assignment as the keys), and w'_q for heads 4g .. 4g+3.
struct PRows {
  v8i a[kPQ];
  float wv[kPQ][4];
  int64_t nv[kPQ];
};
__device__ __forceinline__ void p_load_rows(const PArgs& a, const PTile& t, PRows& r) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int q = 0; q < kPQ; ++q) {
    uint4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    r.nv[q] = 0;
    if (q < t.nq) {
      const int64_t row = t.row0 + q;
      if (n < a.Hi) {
        const uint4* qp = reinterpret_cast<const uint4*>(a.q + (row * a.Hi + n) * 128);
        lo = qp[g];
        hi = qp[4 + g];
      }
      const RowInfo ri = row_info(a.q_pos, static_cast<int>(row), a.s, a.S, a.nv_cap,
                                  a.max_pos_end, nullptr, false);
      r.nv[q] = ri.ok ? ri.nv : 0;
    }
    r.a[q] = as_v8i(lo, hi);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g + i;
      float wq = 0.f;
      if (q < t.nq && h < a.Hi) {
        const int64_t o = (t.row0 + q) * a.Hi + h;
        wq = a.w[o] * (a.q_scale ? a.q_scale[o] : 1.0f);
      }
      r.wv[q][i] = wq;
    }
  }
}

// Sum four rows' partials over the 4 head groups (16-lane rows of the
// wave) with the gfx950 lane swaps: permlane32_swap(x, y) gives
// ([x lanes 0-31, y lanes 0-31], [x lanes 32-63, y lanes 32-63]) and
// permlane16_swap(x, y) gives ([x r0, y r0, x r2, y r2], [x r1, y r1, x r3,
// y r3]) for 16-lane rows r.  The result's row g holds, for entry n, the
// full score of row kPerm[g] of the four.
constexpr int kPerm[4] = {0, 2, 1, 3};
__device__ __forceinline__ float p_reduce4(float p0, float p1, float p2, float p3) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
  const float z = __uint_as_float(a[0]) + __uint_as_float(a[1]);  // lanes 0-31: p0, 32-63: p1
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(p2), __float_as_uint(p3), false, false);
  const float w = __uint_as_float(b[0]) + __uint_as_float(b[1]);  // lanes 0-31: p2, 32-63: p3
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(z), __float_as_uint(w), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Approximate scores (before the key scale) of all kPQ rows against the
// tile's 16 entries, in f32 on the VALU: lane (g, n) of s[h] holds row
// 4h + kPerm[g], entry n.  (Used on the threshold sample only.)
__device__ __forceinline__ void p_scores(const PRows& r, const v8i& kb, float (&s)[kPQ / 4]) {
  v4f c[kPQ];
#pragma unroll
  for (int q = 0; q < kPQ; ++q)
    c[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(r.a[q], kb, v4f{0.f, 0.f, 0.f, 0.f},
                                                           0, 0, 0, 0, 0, 0);
  float p[kPQ];
#pragma unroll
  for (int q = 0; q < kPQ; ++q)
    p[q] = r.wv[q][0] * fmaxf(c[q][0], 0.f) + r.wv[q][1] * fmaxf(c[q][1], 0.f) +
           r.wv[q][2] * fmaxf(c[q][2], 0.f) + r.wv[q][3] * fmaxf(c[q][3], 0.f);
#pragma unroll
  for (int h = 0; h < kPQ / 4; ++h) s[h] = p_reduce4(p[4 * h], p[4 * h + 1], p[4 * h + 2], p[4 * h + 3]);
}

// Value of row 4h + kPerm[g] from a per-row array (selects, no dynamic
// register index).
template <typename T>
__device__ __forceinline__ T p_pick(const T (&v)[kPQ], int h, int g) {
  const T a = v[4 * h], b = v[4 * h + 2], c = v[4 * h + 1], d = v[4 * h + 3];
  return g == 0 ? a : g == 1 ? b : g == 2 ? c : d;
}

__global__ __launch_bounds__(kThreads) void k_pidx_prep(PArgs a) {
  __shared__ uint32_t skey[kPQ][kPSample];
  __shared__ uint32_t hist[kPQ][256];
  __shared__ float fred[kThreads / 64], kred[kThreads / 64];
  __shared__ int64_t ired[kThreads / 64];
  __shared__ uint32_t pick[kPQ][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, g = lane >> 4;
  const PTile t = p_tile(a, blockIdx.x);
  // the largest n_vis over the whole sequence (sets the slices of nu)
  int64_t nvs = 0;
  for (int i = tid; i < a.Tq; i += kThreads) {
    const RowInfo ri = row_info(a.q_pos, static_cast<int>(static_cast<int64_t>(t.b) * a.Tq + i),
                                a.s, a.S, a.nv_cap, a.max_pos_end, nullptr, false);
    if (ri.ok) nvs = max(nvs, ri.nv);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) nvs = max(nvs, static_cast<int64_t>(__shfl_xor(nvs, o, 64)));
  if (lane == 0) ired[wave] = nvs;
  __syncthreads();
  nvs = max(max(ired[0], ired[1]), max(ired[2], ired[3]));
  // nu over this tile's slice of [0, nvs): 4 threads per entry, 32 bytes each
  const int tps = a.tiles_per_seq, slice = blockIdx.x % tps;
  const int64_t per = (nvs + tps - 1) / tps;
  const int64_t e_lo = slice * per, e_hi = min(nvs, e_lo + per);
  const uint8_t* kb = a.keys + static_cast<int64_t>(t.b) * idx_e_pad(a.e_cap) * 128;
  const float* ksb = a.k_scale + static_cast<int64_t>(t.b) * a.e_cap;
  float nu = 0.f, kap = 0.f;
  for (int64_t e0 = e_lo; e0 < e_hi; e0 += kThreads / 4) {
    const int64_t e = e0 + tid / 4;
    float ss = 0.f;
    if (e < e_hi) {
      const uint4* kt = reinterpret_cast<const uint4*>(kb + (e & ~int64_t{15}) * 128);
      const int c = 2 * (tid & 3), en = static_cast<int>(e & 15);
      const uint4 x0 = kt[c * 16 + en], x1 = kt[(c + 1) * 16 + en];
      ss = fp8x16_sumsq(x0) + fp8x16_sumsq(x1);
      // the entry-contiguous copy the selection gathers from
      uint4* rm = reinterpret_cast<uint4*>(a.keys_rm + (static_cast<int64_t>(t.b) * a.nv_cap + e) * 128);
      rm[c] = x0;
      rm[c + 1] = x1;
    }
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    if (e < e_hi) {
      nu = fmaxf(nu, ksb[e] * sqrtf(ss));
      kap = fmaxf(kap, sqrtf(ss));
    }
  }
  nu = wave_max(nu);
  kap = wave_max(kap);
  if (lane == 0) {
    fred[wave] = nu;
    kred[wave] = kap;
  }
  // beta per row: thread -> row tid / 32, head (tid % 32) / 2, half tid % 2
  {
    const int q = tid / 32, h = (tid % 32) / 2, hf = tid % 2;
    float ss = 0.f, wabs = 0.f;
    if (q < t.nq && h < a.Hi) {
      const int64_t row = t.row0 + q;
      const uint4* qp = reinterpret_cast<const uint4*>(a.q + (row * a.Hi + h) * 128) + 4 * hf;
      ss = fp8x16_sumsq(qp[0]) + fp8x16_sumsq(qp[1]) + fp8x16_sumsq(qp[2]) + fp8x16_sumsq(qp[3]);
      const int64_t o = row * a.Hi + h;
      wabs = fabsf(a.w[o] * (a.q_scale ? a.q_scale[o] : 1.0f));
    }
    ss += __shfl_xor(ss, 1, 64);
    float c1 = hf == 0 ? wabs * sqrtf(ss) : 0.f;  // sum_h |w'_h| ||q8_h||
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) c1 += __shfl_xor(c1, o, 32);
    if (tid % 32 == 0 && q < t.nq) a.beta[t.row0 + q] = kPEps * c1;
  }
  __syncthreads();
  if (tid == 0) {
    a.nu_part[blockIdx.x] = fmaxf(fmaxf(fred[0], fred[1]), fmaxf(fred[2], fred[3]));
    a.kappa_part[blockIdx.x] = fmaxf(fmaxf(kred[0], kred[1]), fmaxf(kred[2], kred[3]));
  }
  // approximate scores of the sampled tiles T = st * i, i < ns_t (all 16
  // entries of each: 2 KiB of contiguous keys)
  PRows r;
  p_load_rows(a, t, r);
  int64_t nvt = 0;
#pragma unroll
  for (int q = 0; q < kPQ; ++q) nvt = max(nvt, r.nv[q]);
  const int64_t nst = (nvt + 15) / 16;
  const int64_t st = max<int64_t>(1, (nst + kPSampleTiles - 1) / kPSampleTiles);
  const int ns_t = static_cast<int>((nst + st - 1) / st);
  // sample tiles wave, wave + 4, ... with a ring of kPre tiles in flight;
  // the loads are unconditional (clamped to a valid tile) so that the
  // compiler can count them
  constexpr int kPre = 4;
  uint4 lo[kPre], hi[kPre];
  float ks[kPre];
  const int64_t tmax = max<int64_t>(0, static_cast<int64_t>(ns_t - 1) * st);
  const int64_t jks = max<int64_t>(0, nvt - 1);
  auto load = [&](int u, int ti) {
    const int64_t j = min<int64_t>(ti * st, tmax) * 16 + n;
    idx_load_chunks(kb, j, g, &lo[u], &hi[u]);
    ks[u] = ksb[min(j, jks)];
  };
  int64_t nvp[kPQ];
#pragma unroll
  for (int q = 0; q < kPQ; ++q) nvp[q] = r.nv[q];
  const int64_t nv0 = p_pick(nvp, 0, g), nv1 = p_pick(nvp, 1, g);
  if (ns_t > 0) {
#pragma unroll
    for (int u = 0; u < kPre; ++u) load(u, wave + 4 * u);
  }
  for (int t0 = wave; t0 < kPSampleTiles && ns_t > 0; t0 += 4 * kPre) {
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int ti = t0 + 4 * u;  // < kPSampleTiles: 16 | kPSampleTiles / 4
      const v8i bk = as_v8i(lo[u], hi[u]);
      const float ksc = ks[u];
      load(u, min(ti + 4 * kPre, kPSampleTiles - 1));
      const int64_t j = static_cast<int64_t>(ti) * st * 16 + n;
      const bool in = ti < ns_t;
      float sv[kPQ / 4];
      p_scores(r, bk, sv);
      // lane (g, n) holds rows qa and 4 + qa, qa = kPerm[g], of sample ti*16+n
      const int qa = g == 0 ? 0 : g == 1 ? 2 : g == 2 ? 1 : 3;
      const uint32_t k0 = order_key(sv[0] * ksc), k1 = order_key(sv[1] * ksc);
      skey[qa][ti * 16 + n] = (in & (j < nv0)) ? k0 : 0u;
      skey[4 + qa][ti * 16 + n] = (in & (j < nv1)) ? k1 : 0u;
    }
  }
  __syncthreads();
  // theta: the r-th largest sampled key of each row, to 16 bits (two 8-bit
  // histogram passes); 32 threads per row.  A valid key is never 0.
  const int q = tid / 32, l32 = tid % 32;
  int64_t nvq = 0;  // (r.nv is a register array: no dynamic index)
  if (q < t.nq) {
    const RowInfo ri = row_info(a.q_pos, static_cast<int>(t.row0 + q), a.s, a.S, a.nv_cap,
                                a.max_pos_end, nullptr, false);
    nvq = ri.ok ? ri.nv : 0;
  }
  uint32_t nsq = 0;
  for (int i = l32; i < kPSample; i += 32) nsq += skey[q][i] != 0u ? 1u : 0u;
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) nsq += static_cast<uint32_t>(__shfl_xor(static_cast<int>(nsq), o, 32));
  uint32_t need = static_cast<uint32_t>(min<int64_t>(
      nsq, (2 * static_cast<int64_t>(a.k) * nsq + nvq - 1) / max<int64_t>(nvq, 1) + 8));
  uint32_t prefix = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const int sh = 24 - 8 * pass;
    for (int i = l32; i < 256; i += 32) hist[q][i] = 0u;
    if (l32 == 0) pick[q][0] = pick[q][1] = 0u;
    __syncthreads();
    for (int i = l32; i < kPSample; i += 32) {
      const uint32_t key = skey[q][i];
      if (key != 0u && (pass == 0 || (key >> 24) == prefix)) atomicAdd(&hist[q][(key >> sh) & 255u], 1u);
    }
    __syncthreads();
    // lane l32 owns bins 255 - 8 l32 .. 248 - 8 l32 (descending)
    uint32_t c[8], sum = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      c[u] = hist[q][255 - 8 * l32 - u];
      sum += c[u];
    }
    uint32_t before = sum;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      const uint32_t x = static_cast<uint32_t>(__shfl_up(static_cast<int>(before), o, 32));
      if (l32 >= o) before += x;
    }
    before -= sum;  // exclusive
    if (need > 0 && before < need && before + sum >= need) {
      uint32_t acc = before;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (acc < need && acc + c[u] >= need) {
          pick[q][0] = 255u - 8u * l32 - u;
          pick[q][1] = acc;
        }
        acc += c[u];
      }
    }
    __syncthreads();
    const uint32_t bin = pick[q][0];
    need -= pick[q][1];
    prefix = pass == 0 ? bin : ((prefix << 8) | bin);
    __syncthreads();
  }
  if (l32 == 0 && q < t.nq) {
    const int64_t row = t.row0 + q;
    // rows that keep every visible entry (or none) need no candidates
    const bool sel = nvq > a.k && nsq > 0;
    a.theta[row] = sel ? key_to_float(prefix << 16) : INFINITY;
  }
}

// Two f32 values in [-1, 1] to a packed f16 pair (round to nearest even)
// with ReLU: one v_cvt_pk_f16_f32 with its clamp to [0, 1].
__device__ __forceinline__ v2h relu_f16x2(float x, float y) {
  const v2h h = {static_cast<_Float16>(x), static_cast<_Float16>(y)};
  const v2h z = {static_cast<_Float16>(0.f), static_cast<_Float16>(0.f)};
  const v2h o = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
  return __builtin_elementwise_min(__builtin_elementwise_max(h, z), o);
}
__device__ __forceinline__ v8h cat_f16(v2h a, v2h b, v2h c, v2h d) {
  const v4h ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const v4h cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Scaled fp8 product A B, A's per-row E8M0 code in byte `byte` of sa (a
// constant once the caller's loop is unrolled).
__device__ __forceinline__ v4f mfma_scaled(const v8i& A, const v8i& B, int sa, int byte) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  switch (byte) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, z, 0, 0, 0, sa, 0, kMScaleOne);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, z, 0, 0, 1, sa, 0, kMScaleOne);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, z, 0, 0, 2, sa, 0, kMScaleOne);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, z, 0, 0, 3, sa, 0, kMScaleOne);
  }
}

// v_writelane_b32: lane L of x takes the wave-uniform value v (no clang
// builtin here; the lane select is an immediate, so no lane-select hazard).
template <int L>
__device__ __forceinline__ void write_lane(uint32_t& x, uint32_t v) {
  asm("v_writelane_b32 %0, %1, %2" : "+v"(x) : "s"(v), "n"(L));
}
// Words wd[r] (r = row of the wave) to lanes 4 r + TP.
template <int TP>
__device__ __forceinline__ void put_words(uint32_t& x, const uint32_t (&wd)[8]) {
  write_lane<0 + TP>(x, wd[0]);
  write_lane<4 + TP>(x, wd[1]);
  write_lane<8 + TP>(x, wd[2]);
  write_lane<12 + TP>(x, wd[3]);
  write_lane<16 + TP>(x, wd[4]);
  write_lane<20 + TP>(x, wd[5]);
  write_lane<24 + TP>(x, wd[6]);
  write_lane<28 + TP>(x, wd[7]);
}

// A float rounded toward -inf (x finite).
__device__ __forceinline__ float round_down_f32(double x) {
  float f = static_cast<float>(x);
  if (static_cast<double>(f) > x) f = nextafterf(f, -INFINITY);
  return f;
}

__global__ __launch_bounds__(kThreads, 3) void k_pidx_main(PArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t stg[3][kMStageBytes];
  __shared__ float fred[kThreads / 64], kred[kThreads / 64];
  __shared__ int64_t nred[kThreads / 64];
  __shared__ int csh[kThreads / 64][kMR][16];  // per-head scale exponents
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, g = lane >> 4;
  // workgroup -> (tile range, row group): the workgroups of one XCD
  // (blockIdx mod 8) take consecutive linear ids, i.e. one tile range, so
  // that XCD's L2 holds only that range's keys
  const int G = gridDim.x;
  const int lin = (G & 7) == 0 ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  const int split = lin / a.rg_total, rg = lin % a.rg_total;
  const int b = rg / a.rg_per_seq, r0 = (rg % a.rg_per_seq) * kMRows;
  const int nq = min(kMRows, a.Tq - r0);
  const int64_t row0 = static_cast<int64_t>(b) * a.Tq + r0;
  // nu_max and kappa = max_j ||k8_j|| of the sequence; the workgroup's
  // largest n_vis
  float nu = 0.f, kap = 0.f;
  for (int i = tid; i < a.tiles_per_seq; i += kThreads) {
    nu = fmaxf(nu, a.nu_part[static_cast<int64_t>(b) * a.tiles_per_seq + i]);
    kap = fmaxf(kap, a.kappa_part[static_cast<int64_t>(b) * a.tiles_per_seq + i]);
  }
  nu = wave_max(nu);
  kap = wave_max(kap);
  int64_t nvm = 0;
  if (tid < nq) {
    const RowInfo ri = row_info(a.q_pos, static_cast<int>(row0 + tid), a.s, a.S, a.nv_cap,
                                a.max_pos_end, nullptr, false);
    nvm = ri.ok ? ri.nv : 0;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) nvm = max(nvm, static_cast<int64_t>(__shfl_xor(nvm, o, 64)));
  if (lane == 0) {
    fred[wave] = nu;
    kred[wave] = kap;
    nred[wave] = nvm;
  }
  __syncthreads();
  nu = fmaxf(fmaxf(fred[0], fred[1]), fmaxf(fred[2], fred[3]));
  kap = fmaxf(fmaxf(kred[0], kred[1]), fmaxf(kred[2], kred[3]));
  nvm = max(max(nred[0], nred[1]), max(nred[2], nred[3]));
  const int64_t t_lo = static_cast<int64_t>(split) * a.tps_split;
  const int64_t t_hi = min((nvm + 15) / 16, t_lo + a.tps_split);
  if (t_lo >= t_hi) return;  // the whole workgroup: no barrier follows
  const uint8_t* kb = a.keys + static_cast<int64_t>(b) * idx_e_pad(a.e_cap) * 128;
  const float* ksb = a.k_scale + static_cast<int64_t>(b) * a.e_cap;
  const int nst = static_cast<int>((t_hi - t_lo + kMStage - 1) / kMStage);
  // one stage: 16 KiB of keys (contiguous in the tile layout) and 128
  // scales, clamped to the range
  // (thread t loads bytes 16 (t % 128) of tiles 2u + t / 128; 32-bit
  // offsets: one sequence's keys are far below 4 GiB)
  const uint32_t lane_off = 16u * static_cast<uint32_t>(tid & 127);
  const int hb = tid >> 7;
  auto gload = [&](int s, u32x4 (&rk)[4], float& rks) {
    const int t0 = static_cast<int>(t_lo) + s * kMStage;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t tile = static_cast<uint32_t>(min(t0 + 2 * u + hb, static_cast<int>(t_hi) - 1));
      rk[u] = *reinterpret_cast<const u32x4*>(kb + (tile * 2048u + lane_off));
    }
    rks = ksb[min(static_cast<int64_t>(t0) * 16 + (tid & 127), a.e_cap - 1)];
  };
  auto swrite = [&](int buf, const u32x4 (&rk)[4], float rks) {
    uint8_t* d = stg[buf];
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<u32x4*>(d + 16 * (tid + kThreads * u)) = rk[u];
    if (tid < 128) reinterpret_cast<float*>(d + kMKeyBytes)[tid] = rks;
  };
  // the first two stages' loads are in flight while the operands are set up
  u32x4 rk0[4], rk1[4];
  float rks0, rks1;
  gload(0, rk0, rks0);
  gload(min(1, nst - 1), rk1, rks1);
  // the wave's rows wr0 .. wr0 + 7 of the workgroup
  const int wr0 = wave * kMR;
  // stage-1 operands: lane = head n, chunks g and 4 + g of each row, and the
  // E8M0 code of 2^-c for head n: 2^c >= 2 ||q8_n|| kappa (with a margin for
  // the f32 norms), so |2^-c q8_n . k8_j| <= 1/2 (1 + 2^-10) for every entry
  // even after the fp8 MFMA's error, and 2^c < 4 ||q8_n|| kappa
  v8i A[kMR];
  int sa[kMR / 4];  // four E8M0 codes per register, row q in byte q % 4
#pragma unroll
  for (int q = 0; q < kMR; ++q) {
    uint4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (wr0 + q < nq && n < a.Hi) {
      const uint4* qp = reinterpret_cast<const uint4*>(a.q + ((row0 + wr0 + q) * a.Hi + n) * 128);
      lo = qp[g];
      hi = qp[4 + g];
    }
    A[q] = as_v8i(lo, hi);
    float ss = fp8x16_sumsq(lo) + fp8x16_sumsq(hi);
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    int c = 0;
    const float x = 2.0f * sqrtf(ss) * kap * (1.0f + 0x1p-20f);
    if (x > 0.f) frexpf(x, &c);  // x = f 2^c, f in [0.5, 1)
    const int code = kMScaleOne - c;
    if ((q & 3) == 0) sa[q >> 2] = code;
    else sa[q >> 2] |= code << (8 * (q & 3));
    if (g == 0) csh[wave][q][n] = c;
  }
  // stage-2 operands: lane (g, m), m < 8, holds row m's weights for heads
  // 4g .. 4g+3 at k = 8g .. 8g+3 (m even) or 8g+4 .. 8g+7 (m odd) of pair
  // m / 2: w'_h 2^(c_h + e_m), with e_m putting the row's largest
  // |w'_h 2^c_h| in [2^14, 2^15)
  int e_row = 0;
  v8h a2m = {};
  if (n < kMR) {
    const int qr = wr0 + n;
    float wmax = 0.f, wq[4] = {0.f, 0.f, 0.f, 0.f};
    int cq[4] = {0, 0, 0, 0};
    if (qr < nq) {
      const int64_t o = (row0 + qr) * a.Hi;
#pragma unroll
      for (int h = 0; h < 16; ++h)  // (all loads in flight at once; Hi <= 16)
        if (h < a.Hi)
          wmax = fmaxf(wmax, ldexpf(fabsf(a.w[o + h] * (a.q_scale ? a.q_scale[o + h] : 1.0f)),
                                    csh[wave][n][h]));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * g + i;
        if (h < a.Hi) {
          wq[i] = a.w[o + h] * (a.q_scale ? a.q_scale[o + h] : 1.0f);
          cq[i] = csh[wave][n][h];
        }
      }
    }
    if (wmax > 0.f && wmax <= 3.0e38f) {
      int ex;
      frexpf(wmax, &ex);  // wmax = f 2^ex, f in [0.5, 1)
      e_row = 15 - ex;
    }
    v2h w01 = {static_cast<_Float16>(ldexpf(wq[0], cq[0] + e_row)),
               static_cast<_Float16>(ldexpf(wq[1], cq[1] + e_row))};
    v2h w23 = {static_cast<_Float16>(ldexpf(wq[2], cq[2] + e_row)),
               static_cast<_Float16>(ldexpf(wq[3], cq[3] + e_row))};
    const v2h z = {};
    a2m = (n & 1) ? cat_f16(z, z, w01, w23) : cat_f16(w01, w23, z, z);
  }
  v8h A2[kMR / 2];
#pragma unroll
  for (int p = 0; p < kMR / 2; ++p) A2[p] = (n < kMR && (n >> 1) == p) ? a2m : v8h{};
  // lane (g, n), g < 2, rows 4g + i, in units of 2^e per score unit: the
  // threshold (theta - beta nu_max, less a 2^-20 margin, rounded down) and
  // the stage-2 accumulator's start gamma kappa (rounded up), gamma = 2^-22 /
  // kPEps * beta, which covers the f16 subnormal error
  float thr[4], g0[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qd = 4 * (g & 1) + i;
    const int e_q = __shfl(e_row, qd, 64);
    thr[i] = INFINITY;
    g0[i] = 0.f;
    if (g < 2 && wr0 + qd < nq) {
      const float th = a.theta[row0 + wr0 + qd];
      const double be = static_cast<double>(a.beta[row0 + wr0 + qd]);
      if (th < INFINITY) {
        const double bn = be * nu;
        double d = static_cast<double>(th) - bn;
        d -= 0x1p-20 * (fabs(static_cast<double>(th)) + bn);
        thr[i] = round_down_f32(ldexp(d, e_q));
        g0[i] = -round_down_f32(-ldexp(be * (0x1p-22 / kPEps) * kap, e_q));
      }
    }
  }
  swrite(0, rk0, rks0);
  swrite(1, rk1, rks1);
  __syncthreads();
  // mask store: lane L < 32 writes row L / 4 of the wave, tiles 2 (L % 4)
  // and 2 (L % 4) + 1 of the stage (one u32)
  const bool st_ok = lane < 32 && wr0 + (lane >> 2) < nq;
  uint32_t* mst = reinterpret_cast<uint32_t*>(a.masks + (row0 + wr0 + (lane >> 2)) * a.ld_t);
  int buf = 0;
  for (int s = 0; s < nst; ++s) {
    u32x4 rk[4];
    float rks;
    gload(min(s + 2, nst - 1), rk, rks);
    const uint8_t* sb = stg[buf];
    uint32_t wout = 0u;
#pragma unroll
    for (int tp = 0; tp < kMStage / 2; ++tp) {
      uint64_t mk[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int tt = 2 * tp + h;
        const uint4 klo = *reinterpret_cast<const uint4*>(sb + tt * 2048 + 16 * lane);
        const uint4 khi = *reinterpret_cast<const uint4*>(sb + tt * 2048 + 1024 + 16 * lane);
        const float ksn = reinterpret_cast<const float*>(sb + kMKeyBytes)[tt * 16 + n];
        const v8i B = as_v8i(klo, khi);
        v4f c[kMR];
#pragma unroll
        for (int q = 0; q < kMR; ++q)
          c[q] = mfma_scaled(A[q], B, sa[q >> 2], q & 3);
        v4f c2 = {g0[0], g0[1], g0[2], g0[3]};
#pragma unroll
        for (int p = 0; p < kMR / 2; ++p) {
          const v8h b2 = cat_f16(relu_f16x2(c[2 * p][0], c[2 * p][1]), relu_f16x2(c[2 * p][2], c[2 * p][3]),
                                 relu_f16x2(c[2 * p + 1][0], c[2 * p + 1][1]),
                                 relu_f16x2(c[2 * p + 1][2], c[2 * p + 1][3]));
          c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A2[p], b2, c2, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) mk[h][i] = __ballot(c2[i] * ksn >= thr[i]);
      }
      // row i of the wave: bits 0-15 of mk[.][i]; row 4 + i: bits 16-31;
      // the words go to lanes 4 row + tp
      uint32_t wd[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wd[i] = static_cast<uint32_t>(mk[0][i] & 0xffffu) | (static_cast<uint32_t>(mk[1][i] & 0xffffu) << 16);
        wd[4 + i] = static_cast<uint32_t>((mk[0][i] >> 16) & 0xffffu) |
                    (static_cast<uint32_t>(mk[1][i]) & 0xffff0000u);
      }
      if (tp == 0) put_words<0>(wout, wd);
      if (tp == 1) put_words<1>(wout, wd);
      if (tp == 2) put_words<2>(wout, wd);
      if (tp == 3) put_words<3>(wout, wd);
    }
    if (st_ok) mst[((t_lo + static_cast<int64_t>(s) * kMStage) >> 1) + (lane & 3)] = wout;
    swrite(buf == 0 ? 2 : buf - 1, rk, rks);  // (s + 2) % 3
    __syncthreads();
    buf = buf == 2 ? 0 : buf + 1;
  }
}

__global__ __launch_bounds__(kPSelT) void k_pidx_select(PArgs a, float* __restrict__ scores,
                                                        int64_t ld_scores,
                                                        int32_t* __restrict__ idx_out) {
  __shared__ uint64_t cand_s[kPCandCap];
  __shared__ uint64_t tmp_s[kPTmpCap];
  __shared__ uint32_t h_s[2048];
  constexpr int kW = kPSelT / 64;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int b = row / a.Tq;
  const RowInfo ri = row_info(a.q_pos, row, a.s, a.S, a.nv_cap, a.max_pos_end, a.status, tid == 0);
  const int64_t nv = ri.ok ? ri.nv : 0;
  int32_t* irow = idx_out + static_cast<int64_t>(row) * a.k;
  if (nv <= a.k) {
    emit_all_visible(nullptr, nv, a.k, irow, nullptr);
    return;
  }
  const float theta = a.theta[row];
  // the candidates, in index order, from the row's masks: 8 tiles per
  // thread and pass, block prefix sums for the slots
  const uint16_t* mrow = a.masks + static_cast<int64_t>(row) * a.ld_t;
  const int64_t ntl = (nv + 15) / 16;
  const uint32_t tail = static_cast<uint32_t>(nv & 15);
  __shared__ uint32_t cnt_s;
  uint32_t cnt = 0;
  for (int64_t t0 = 0; t0 < ntl; t0 += 8 * kPSelT) {
    const int64_t tb = t0 + 8 * tid;
    uint32_t m[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if (tb < ntl) {
      const uint4 v = *reinterpret_cast<const uint4*>(mrow + tb);  // ld_t, tb multiples of 8
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m[2 * i] = w4[i] & 0xffffu;
        m[2 * i + 1] = w4[i] >> 16;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t tt = tb + i;
        if (tt >= ntl) m[i] = 0u;
        else if (tt == ntl - 1 && tail != 0u) m[i] &= (1u << tail) - 1u;
      }
    }
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) c += __popc(m[i]);
    uint32_t total;
    uint32_t pos = cnt + block_prefix_excl<kPSelT>(c, &total);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t mm = m[i];
      while (mm) {
        const int bit = __ffs(static_cast<int>(mm)) - 1;
        mm &= mm - 1u;
        if (pos < static_cast<uint32_t>(kPCandCap))
          cand_s[pos] = static_cast<uint64_t>((tb + i) * 16 + bit);
        ++pos;
      }
    }
    cnt += total;
  }
  if (tid == 0) cnt_s = cnt;
  __syncthreads();
  cnt = cnt_s;
  v8bf aq[4];
  float wv[4];
  exact_row_operands(a.q, a.q_scale, a.w, row, a.Hi, aq, wv);
  const uint8_t* kb = a.keys + static_cast<int64_t>(b) * idx_e_pad(a.e_cap) * 128;
  const uint8_t* krm = a.keys_rm + static_cast<int64_t>(b) * a.nv_cap * 128;
  const float* ksb = a.k_scale + static_cast<int64_t>(b) * a.e_cap;
  bool ok = cnt <= static_cast<uint32_t>(kPCandCap) && theta < INFINITY;
  if (ok) {
    const int ct = static_cast<int>((cnt + 15) / 16);
    uint32_t c_ge = 0;
    // four tiles per step: their indices, then their keys, then the math,
    // so that a step costs two memory round trips
    constexpr int kU = 4;
    for (int t0 = wave; t0 < ct; t0 += kU * kW) {
      int64_t j[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = (t0 + u * kW) * 16 + n;
        j[u] = i < static_cast<int>(cnt) ? static_cast<int64_t>(cand_s[i]) : -1;
      }
      uint4 blo[kU], bhi[kU];
      float ks[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t jj = j[u] >= 0 ? j[u] : 0;
        const uint4* rm = reinterpret_cast<const uint4*>(krm + jj * 128);
        blo[u] = rm[g];
        bhi[u] = rm[4 + g];
        ks[u] = ksb[jj];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = (t0 + u * kW) * 16 + n;
        const float sc = exact_tile_score(aq, wv, blo[u], bhi[u]) * ks[u];
        if (g == 0 && i < ct * 16) {
          cand_s[i] = j[u] >= 0 ? composite(order_key(sc), static_cast<uint32_t>(j[u])) : 0ull;
          c_ge += (j[u] >= 0 && sc >= theta) ? 1u : 0u;
        }
      }
    }
    ok = block_reduce_u32<2, kPSelT>(c_ge) >= static_cast<uint32_t>(a.k);  // barriers
  }
  if (ok) {
    select_topk_composites<kPSelT, kPTmpCap>(cand_s, static_cast<int>(cnt), static_cast<uint32_t>(a.k),
                                             irow, nullptr, tmp_s, h_s);
    return;
  }
  // fallback: score the whole row exactly, then select from the scores
  float* srow = scores + static_cast<int64_t>(row) * ld_scores;
  score_row_exact(aq, wv, kb, ksb, nv, srow, kW);
  __syncthreads();
  row_select_from_scores<kPCandCap, kPSelT, 11>(srow, nv, a.k, irow, nullptr, cand_s, h_s);
}

struct Plan {
  int64_t nv_cap, ld, ld_t;
  bool mfma, cand, pre;
  int ent, nb, nw, cap, tps, tiles, rg_per_seq, rg_total, nsplit, tps_split;
  size_t off_scores, off_cand, off_meta, off_theta, off_beta, off_nu, off_kappa, off_masks, off_krm,
      total;
};

Plan plan(const dsa_index_args& a) {
  Plan p{};
  const int64_t rows = static_cast<int64_t>(a.n_seqs) * a.queries_per_seq;
  p.nv_cap = std::min<int64_t>(a.e_cap, n_complete(a.max_pos_end - 1, a.stride, a.span));
  if (p.nv_cap < 0) p.nv_cap = 0;
  p.ld = (p.nv_cap + 63) / 64 * 64;
  p.mfma = a.keys != nullptr && a.dtype == DSA_FP8_E4M3 && a.dim == 128 && a.heads <= 16;
  // entries per stream workgroup (1024: at 1M context 1024 workgroups of 4
  // waves keep every SIMD busy; 2048 halves the waves and loses more to
  // latency than it saves in candidate extraction)
  p.ent = 1024;
  p.nb = static_cast<int>(ceil_div(p.nv_cap, p.ent));
  p.nw = 4 * p.nb;  // waves per row, ent / 4 entries each
  // Candidates per wave: the union holds >= 2k and fits the final LDS pass.
  // A wave of 256 entries at 1M context holds ~0.5 of the row's top 512;
  // more than 8 of them has probability ~3e-8 for unstructured scores.
  p.cap = static_cast<int>(std::min<int64_t>(
      32, std::max<int64_t>(8, ceil_div(4 * static_cast<int64_t>(a.k), std::max(1, p.nw)))));
  p.cand = p.mfma && p.nv_cap > a.k && static_cast<int64_t>(p.nw) * p.cap <= kFinalCap &&
           static_cast<int64_t>(p.nw) * p.cap >= 2 * static_cast<int64_t>(a.k);
  // many rows per sequence: the fp8 contraction with exact correction
  p.pre = p.mfma && a.score_out == nullptr && rows >= 512 && a.queries_per_seq >= 64 &&
          p.nv_cap > a.k;
  if (p.pre) p.cand = false;
  p.tps = static_cast<int>(ceil_div(a.queries_per_seq, kPQ));
  p.tiles = a.n_seqs * p.tps;
  // main: row groups of kMRows times tile ranges (multiples of one LDS
  // stage), aiming at two workgroups per compute unit with >= 8 stages each
  p.rg_per_seq = static_cast<int>(ceil_div(a.queries_per_seq, kMRows));
  p.rg_total = a.n_seqs * p.rg_per_seq;
  {
    const int64_t ntl = ceil_div(p.nv_cap, 16);
    p.ld_t = ceil_div(ntl, kMStage) * kMStage;
    const int64_t ns = std::max<int64_t>(
        1, std::min<int64_t>(ceil_div(kMTargetWGs, std::max(1, p.rg_total)), ntl / (8 * kMStage)));
    p.tps_split = static_cast<int>(ceil_div(ceil_div(ntl, ns), kMStage) * kMStage);
    p.nsplit = static_cast<int>(ceil_div(ntl, std::max(1, p.tps_split)));
  }
  size_t off = 0;
  p.off_scores = off;
  off = align_up(off + static_cast<size_t>(rows) * p.ld * sizeof(float));
  p.off_cand = off;
  if (p.cand) off = align_up(off + static_cast<size_t>(rows) * p.nw * p.cap * sizeof(uint64_t));
  p.off_meta = off;
  if (p.cand) off = align_up(off + static_cast<size_t>(rows) * p.nw * sizeof(uint32_t));
  p.off_theta = off;
  if (p.pre) off = align_up(off + static_cast<size_t>(rows) * sizeof(float));
  p.off_beta = off;
  if (p.pre) off = align_up(off + static_cast<size_t>(rows) * sizeof(float));
  p.off_nu = off;
  if (p.pre) off = align_up(off + static_cast<size_t>(p.tiles) * sizeof(float));
  p.off_kappa = off;
  if (p.pre) off = align_up(off + static_cast<size_t>(p.tiles) * sizeof(float));
  p.off_masks = off;
  if (p.pre) off = align_up(off + static_cast<size_t>(rows) * p.ld_t * sizeof(uint16_t));
  p.off_krm = off;
  if (p.pre) off = align_up(off + static_cast<size_t>(a.n_seqs) * p.nv_cap * 128);
  p.total = off;
  return p;
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
  if (P.pre) {
    PArgs pa{};
    pa.q = static_cast<const uint8_t*>(a.q);
    pa.q_scale = a.q_scale;
    pa.w = a.w;
    pa.keys = static_cast<const uint8_t*>(a.keys);
    pa.k_scale = a.k_scale;
    pa.q_pos = a.q_pos;
    pa.Tq = a.queries_per_seq;
    pa.Hi = a.heads;
    pa.s = a.stride;
    pa.S = a.span;
    pa.k = a.k;
    pa.tiles_per_seq = P.tps;
    pa.rg_per_seq = P.rg_per_seq;
    pa.rg_total = P.rg_total;
    pa.tps_split = P.tps_split;
    pa.e_cap = a.e_cap;
    pa.nv_cap = P.nv_cap;
    pa.max_pos_end = a.max_pos_end;
    pa.ld_t = P.ld_t;
    pa.theta = reinterpret_cast<float*>(base + P.off_theta);
    pa.beta = reinterpret_cast<float*>(base + P.off_beta);
    pa.nu_part = reinterpret_cast<float*>(base + P.off_nu);
    pa.kappa_part = reinterpret_cast<float*>(base + P.off_kappa);
    pa.masks = reinterpret_cast<uint16_t*>(base + P.off_masks);
    pa.keys_rm = reinterpret_cast<uint8_t*>(base + P.off_krm);
    pa.status = a.status;
    const hipEvent_t e0 = static_cast<hipEvent_t>(a.ev_index[0]);
    const hipEvent_t e1 = static_cast<hipEvent_t>(a.ev_index[1]);
    launch_timed(k_pidx_prep, dim3(P.tiles), dim3(kThreads), 0, st, e0, nullptr, pa);
    rc = hip_check(hipGetLastError(), "k_pidx_prep launch");
    if (rc != DSA_OK) return rc;
    hipLaunchKernelGGL(k_pidx_main, dim3(P.rg_total * P.nsplit), dim3(kThreads), 0, st, pa);
    rc = hip_check(hipGetLastError(), "k_pidx_main launch");
    if (rc != DSA_OK) return rc;
    launch_timed(k_pidx_select, dim3(rows), dim3(kPSelT), 0, st, nullptr, e1, pa, scores, P.ld,
                 a.idx_out);
    return hip_check(hipGetLastError(), "k_pidx_select launch");
  }
  if (!no_keys && P.nv_cap > 0) {
    const hipEvent_t e0 = static_cast<hipEvent_t>(a.ev_index[0]);
    const hipEvent_t e1 = static_cast<hipEvent_t>(a.ev_index[1]);
    if (P.mfma) {
      dim3 grid(static_cast<unsigned>(P.nb), rows);
      auto go = [&](auto kern) {
        launch_timed(kern, grid, dim3(kThreads), 0, st, e0, e1, static_cast<const uint8_t*>(a.q),
                     a.q_scale, a.w, static_cast<const uint8_t*>(a.keys), a.k_scale, a.q_pos,
                     a.queries_per_seq, a.heads, a.stride, a.span, a.e_cap, P.nv_cap,
                     a.max_pos_end, scores, P.ld, cand, meta, P.cap, a.status);
      };
      if (P.cand) go(k_index_fp8_stream<true, 1024>);
      else go(k_index_fp8_stream<false, 1024>);
    } else {
      dim3 grid(static_cast<unsigned>(ceil_div(P.nv_cap, kThreads)), rows);
      const size_t shm = (static_cast<size_t>(a.heads) * a.dim + a.heads) * sizeof(float);
      if (a.dtype == DSA_F32)
        launch_timed(k_index_generic<float>, grid, dim3(kThreads), shm, st, e0, e1,
                           static_cast<const float*>(a.q), a.q_scale, a.w,
                           static_cast<const float*>(a.keys), a.k_scale, a.q_pos,
                           a.queries_per_seq, a.heads, a.dim, a.stride, a.span, a.e_cap, P.nv_cap,
                           a.max_pos_end, scores, P.ld, a.status);
      else
        launch_timed(k_index_generic<uint8_t>, grid, dim3(kThreads), shm, st, e0, e1,
                           static_cast<const uint8_t*>(a.q), a.q_scale, a.w,
                           static_cast<const uint8_t*>(a.keys), a.k_scale, a.q_pos,
                           a.queries_per_seq, a.heads, a.dim, a.stride, a.span, a.e_cap, P.nv_cap,
                           a.max_pos_end, scores, P.ld, a.status);
    }
    rc = hip_check(hipGetLastError(), "indexer launch");
    if (rc != DSA_OK) return rc;
  }
  if (P.cand && !no_keys) {
    hipLaunchKernelGGL(k_topk_cand_final, dim3(rows), dim3(kSel), 0, st, scores, P.ld, a.q_pos,
                       a.stride, a.span, P.nv_cap, a.max_pos_end, cand, meta, P.nw, P.cap,
                       a.idx_out, a.score_out, a.k, static_cast<const uint8_t*>(a.q), a.q_scale,
                       a.w, static_cast<const uint8_t*>(a.keys), a.k_scale, a.queries_per_seq,
                       a.heads, a.e_cap);
  } else {
    hipLaunchKernelGGL(k_topk_rows, dim3(rows), dim3(kSel), 0, st, no_keys ? nullptr : scores,
                       P.ld, a.q_pos, a.stride, a.span, P.nv_cap, a.max_pos_end, a.idx_out,
                       a.score_out, a.k, a.status);
  }
  return hip_check(hipGetLastError(), "top-k launch");
}

dsa_status launch_decode_index_topk(const dsa_index_args& a, void* ws, const dsa_layer_args& la,
                                    int64_t* qpos, bool insert_window, float* cs_tab,
                                    hipStream_t st) {
  const Plan P = plan(a);
  const bool fused = P.cand && a.keys != nullptr && P.nv_cap > 0 && a.queries_per_seq == 1 &&
                     a.dtype == DSA_FP8_E4M3 && la.dtype == DSA_BF16;
  if (!fused) {
    dsa_status rc = launch_decode_prologue(la, qpos, insert_window, cs_tab, st);
    if (rc != DSA_OK) return rc;
    return launch_index_topk(a, ws, st);
  }
  const int rows = a.n_seqs;
  char* base = static_cast<char*>(ws);
  float* scores = reinterpret_cast<float*>(base + P.off_scores);
  uint64_t* cand = reinterpret_cast<uint64_t*>(base + P.off_cand);
  uint32_t* meta = reinterpret_cast<uint32_t*>(base + P.off_meta);
  const PrologueArgs pa = make_prologue_args(la, qpos, insert_window, cs_tab);
  auto go = [&](auto kern) {
    launch_timed(kern, dim3(P.nb + kPrologueRoles, rows), dim3(kThreads), 0, st,
                 static_cast<hipEvent_t>(a.ev_index[0]), static_cast<hipEvent_t>(a.ev_index[1]),
                 static_cast<const uint8_t*>(a.q), a.q_scale, a.w,
                 static_cast<const uint8_t*>(a.keys), a.k_scale, a.q_pos, a.heads, a.stride,
                 a.span, a.e_cap, P.nv_cap, a.max_pos_end, scores, P.ld, cand, meta, P.cap, P.nb,
                 pa, a.status);
  };
  go(k_decode_index<uint16_t, DSA_FP8_E4M3, 1024>);
  dsa_status rc = hip_check(hipGetLastError(), "k_decode_index launch");
  if (rc != DSA_OK) return rc;
  hipLaunchKernelGGL(k_topk_cand_final, dim3(rows), dim3(kSel), 0, st, scores, P.ld, a.q_pos,
                     a.stride, a.span, P.nv_cap, a.max_pos_end, cand, meta, P.nw, P.cap,
                     a.idx_out, a.score_out, a.k, static_cast<const uint8_t*>(a.q), a.q_scale,
                     a.w, static_cast<const uint8_t*>(a.keys), a.k_scale, 1, a.heads, a.e_cap);
  return hip_check(hipGetLastError(), "top-k launch");
}

}  // namespace dsa
