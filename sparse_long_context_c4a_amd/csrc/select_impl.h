// Block-level selection primitives shared by the Top-k kernels: exact
// Top-k by score with ties to the lower index, over composites (order key
// of the score, complemented index) held in LDS or over a row of scores in
// memory.  Every helper assumes blockDim.x == NT.
#pragma once

#include "common.h"
#include "indexer_impl.h"

namespace dsa {
namespace {

constexpr int kBins = 4096;           // row select histogram bins
constexpr int kFinalCap = 8192;       // candidates resolved in LDS

// ------------------------------------------------------- block primitives
// The selection kernels run one workgroup of kSel threads (16 wave64s) per
// query row; every helper below assumes blockDim.x == kSel.
constexpr int kSel = 1024;
constexpr int kSelWaves = kSel / 64;

// Lane exchanges within a wave without an LDS round trip: DPP moves inside
// each 16-lane row, the gfx950 row swaps across rows.
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(x), kCtrl, kRowMask, 0xf, false));
}

template <int kOp>  // 0 max, 1 min, 2 sum
__device__ __forceinline__ uint32_t op_u32(uint32_t a, uint32_t b) {
  return kOp == 0 ? max(a, b) : kOp == 1 ? min(a, b) : a + b;
}

// Max / min / sum over the wave, every lane getting the result: partners
// within quads (lane ^ 1, lane ^ 2), then the mirrored half-row and row
// (which pair each quad, then each half, with the other), then the row
// swaps.
template <int kOp>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v) {
  v = op_u32<kOp>(v, dpp_u32<0xb1>(v));   // quad_perm [1, 0, 3, 2]
  v = op_u32<kOp>(v, dpp_u32<0x4e>(v));   // quad_perm [2, 3, 0, 1]
  v = op_u32<kOp>(v, dpp_u32<0x141>(v));  // row_half_mirror
  v = op_u32<kOp>(v, dpp_u32<0x140>(v));  // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op_u32<kOp>(a[0], a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op_u32<kOp>(c[0], c[1]);
}

// Inclusive prefix sum over the wave's lanes (in lane order): shifts by 1,
// 2, 4 and 8 within each row, then the last lane of row 0 added to row 1
// and of row 2 to row 3, then lane 31 added to rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_u32<0x111>(x);  // row_shr:1 (lanes shifted in from outside the row read 0)
  x += dpp_u32<0x112>(x);
  x += dpp_u32<0x114>(x);
  x += dpp_u32<0x118>(x);
  x += dpp_u32<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_u32<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// Block-wide max / min / sum over NT threads; every thread gets the result.
template <int kOp, int NT = kSel>  // 0 max, 1 min, 2 sum
__device__ __forceinline__ uint32_t block_reduce_u32(uint32_t v) {
  __shared__ uint32_t wv[NT / 64];
  const int t = threadIdx.x;
  v = wave_reduce_u32<kOp>(v);
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
  const uint32_t x = wave_incl_scan(v);
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
  base = __builtin_amdgcn_readlane(base, 0);
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

// The same search over NB bins held in LDS (bin i at h[i], searched from the
// highest), done by the first wave alone: one barrier instead of the four of
// a block-wide scan.  Also gives the total count; the result is meaningful
// only when total >= need.  Every thread of the block must call it, once per
// kernel (its result slot is not guarded against a second call).
template <int NB>
__device__ __forceinline__ Bin find_bin_wave(const uint32_t* h, uint32_t need, uint32_t* total) {
  static_assert(NB % 256 == 0, "whole 16-byte reads per lane");
  constexpr int kL = NB / 64;  // bins per lane
  __shared__ Bin res;
  __shared__ uint32_t tot;
  const int t = threadIdx.x;
  if (t < 64) {
    // lane l: bins NB-1 - kL l down to NB - kL (l + 1), read upwards
    uint32_t up[kL];
    const uint4* src = reinterpret_cast<const uint4*>(h + (NB - kL * (t + 1)));
#pragma unroll
    for (int i = 0; i < kL / 4; ++i) {
      const uint4 v = src[i];
      up[4 * i] = v.x;
      up[4 * i + 1] = v.y;
      up[4 * i + 2] = v.z;
      up[4 * i + 3] = v.w;
    }
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < kL; ++i) sum += up[i];
    const uint32_t x = wave_incl_scan(sum);
    const uint32_t before = x - sum;
    if (t == 63) tot = x;
    // the lane whose range holds the bin, then the bin within it: lane i
    // takes that range's i-th bin from the top, a second wave scan
    const uint64_t hit = __ballot(before < need && x >= need);
    if (hit != 0) {
      const int L = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      const uint32_t bL = __builtin_amdgcn_readlane(before, L);
      const int bin = NB - 1 - (kL * L + (t < kL ? t : 0));
      const uint32_t c = t < kL ? h[bin] : 0u;
      const uint32_t y = wave_incl_scan(c);
      if (t < kL && bL + y - c < need && bL + y >= need)
        res = Bin{static_cast<uint32_t>(bin), bL + y - c, c};
    }
  }
  __syncthreads();
  *total = tot;
  return res;
}

// Keep the `need` largest of the n <= 64 distinct composites in v[] (LDS):
// each is kept iff fewer than `need` others exceed it.  The first wave holds
// one per lane and compares it with every other by lane broadcasts; calls
// f(v, slot) for the kept, slot = 0 .. kept-1 in lane order (no atomics).
template <typename F>
__device__ __forceinline__ void keep_largest_small(const uint64_t* v, int n, uint32_t need, F f) {
  const int t = threadIdx.x;
  if (t < 64) {
    const uint64_t x = t < n ? v[t] : 0ull;
    const uint32_t xlo = static_cast<uint32_t>(x), xhi = static_cast<uint32_t>(x >> 32);
    uint32_t rank = 0;
    for (int i = 0; i < n; ++i) {  // (n is uniform)
      // (readlane returns int: through uint32_t, no sign extension)
      const uint32_t yhi = static_cast<uint32_t>(__builtin_amdgcn_readlane(xhi, i));
      const uint32_t ylo = static_cast<uint32_t>(__builtin_amdgcn_readlane(xlo, i));
      const uint64_t y = (static_cast<uint64_t>(yhi) << 32) | ylo;
      rank += y > x ? 1u : 0u;
    }
    const bool keep = t < n && rank < need;
    const uint64_t km = __ballot(keep);
    if (keep) f(x, static_cast<uint32_t>(__popcll(km & ((1ull << t) - 1ull))));
  }
}

// Exact selection of the `need` largest of n distinct composites c[] (LDS)
// by radix passes of 8 bits, for the rare large tie groups; returns the
// smallest kept composite.  pred() filters which elements take part.  When
// every taking part has its key in [base_key, base_key + 2^key_bits) (one
// histogram bin), the passes run over the key's offset from base_key and
// then the index, so that no pass is spent on key bits the bin already
// fixes.
template <int NT = kSel, typename P>
__device__ uint64_t kth_largest_composite(const uint64_t* c, int n, uint32_t need, P pred,
                                          uint32_t base_key = 0u, int key_bits = 32) {
  static_assert(NT >= 256, "one thread per digit");
  __shared__ uint32_t cnt[256];
  __shared__ uint32_t res[3];
  const int t = threadIdx.x;
  // offset form: (key - base_key) above the 32 index bits (order-preserving
  // within the bin)
  auto off = [=](uint64_t v) {
    return (static_cast<uint64_t>(static_cast<uint32_t>(v >> 32) - base_key) << 32) |
           (v & 0xffffffffull);
  };
  uint64_t prefix = 0, mask = 0;
  for (int sh = ((key_bits + 32 + 7) / 8 - 1) * 8; sh >= 0; sh -= 8) {
    if (t < 256) cnt[t] = 0;
    __syncthreads();
    for (int i = t; i < n; i += NT) {
      const uint64_t v = c[i];
      if (!pred(v)) continue;
      const uint64_t o = off(v);
      if ((o & mask) == prefix) atomicAdd(&cnt[(o >> sh) & 255u], 1u);
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
  return (static_cast<uint64_t>(static_cast<uint32_t>(prefix >> 32) + base_key) << 32) |
         (prefix & 0xffffffffull);
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
// resolved exactly.  tmp: kTmp u64 of LDS; hist: 2048 u32 of LDS.  Ends
// without a barrier (its last stores are the emits): a caller that goes on
// to reuse c, tmp or hist synchronises first.
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
  // places: count the wave's entries above the bin and in it over all of
  // its passes, take them with one LDS counter update per kind, then emit
  const int l = t & 63;
  const uint64_t below = (1ull << l) - 1ull;
  auto classify = [&](int i, bool* up, bool* mid) {
    const uint64_t v = i < n ? c[i] : 0ull;
    const uint32_t bin = (static_cast<uint32_t>(v >> 32) - lo) >> shift;
    *up = v != 0 && bin > B;
    *mid = v != 0 && bin == B && fits;
    return v;
  };
  uint32_t nu = 0, nm = 0;
  for (int i0 = 0; i0 < n; i0 += NT) {
    bool up, mid;
    classify(i0 + t, &up, &mid);
    nu += static_cast<uint32_t>(__popcll(__ballot(up)));
    nm += static_cast<uint32_t>(__popcll(__ballot(mid)));
  }
  uint32_t pu = 0, pm = 0;
  if (l == 0) {
    if (nu) pu = atomicAdd(&pos_above, nu);
    if (nm) pm = atomicAdd(&n_tmp, nm);
  }
  pu = __builtin_amdgcn_readlane(pu, 0);
  pm = __builtin_amdgcn_readlane(pm, 0);
  for (int i0 = 0; i0 < n; i0 += NT) {
    bool up, mid;
    const uint64_t v = classify(i0 + t, &up, &mid);
    const uint64_t bm = __ballot(mid);
    const uint32_t q = pm + static_cast<uint32_t>(__popcll(bm & below));
    if (mid) tmp[q] = v;
    pm += static_cast<uint32_t>(__popcll(bm));
  }
  __syncthreads();
  const uint32_t need = k - above;
  auto out_bin = [&](uint64_t v) {
    const uint32_t p = atomicAdd(&pos_bin, 1u);
    if (p < need) emit(irow, orow, above + p, comp_index(v), key_to_float(static_cast<uint32_t>(v >> 32)));
  };
  if (fits && at <= 64) {
    keep_largest_small(tmp, static_cast<int>(at), need, [&](uint64_t v, uint32_t slot) {
      emit(irow, orow, above + slot, comp_index(v), key_to_float(static_cast<uint32_t>(v >> 32)));
    });
  } else if (fits) {
    const uint64_t cut = kth_largest_composite<NT>(tmp, static_cast<int>(at), need,
                                                   [](uint64_t) { return true; },
                                                   lo + (B << shift), shift);
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
    const uint64_t cut = kth_largest_composite<NT>(c, n, need, in_bin, lo + (B << shift), shift);
    for (int i = t; i < n; i += NT)
      if (in_bin(c[i]) && c[i] >= cut) out_bin(c[i]);
  }
  // the entries above the bin go out last, after every barrier: a barrier
  // waits for the workgroup's outstanding global stores
  for (int i0 = 0; i0 < n; i0 += NT) {
    bool up, mid;
    const uint64_t v = classify(i0 + t, &up, &mid);
    const uint64_t bu = __ballot(up);
    const uint32_t p = pu + static_cast<uint32_t>(__popcll(bu & below));
    if (up && p < above) emit(irow, orow, p, comp_index(v), key_to_float(static_cast<uint32_t>(v >> 32)));
    pu += static_cast<uint32_t>(__popcll(bu));
  }
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
      keep_largest_small(cand_s, static_cast<int>(at), need, [&](uint64_t v, uint32_t slot) {
        emit(irow, orow, above + slot, comp_index(v), key_to_float(static_cast<uint32_t>(v >> 32)));
      });
    } else {
      const uint64_t cut = kth_largest_composite<NT>(cand_s, static_cast<int>(at), need,
                                                     [](uint64_t) { return true; },
                                                     lo + (thr << shift), shift);
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

}  // namespace
}  // namespace dsa
