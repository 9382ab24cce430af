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
// Top-k without cross-workgroup atomics: each workgroup of 1024 entries keeps
// the entries whose key is above t_b = (cap+1)-th largest key of the
// workgroup (at most `cap` of them) as candidates and records t_b.  The final
// pass selects the exact top k of the union of candidates (radix select on
// (score key, complemented index), so ties go to the lower index) and checks
// the certificate  k-th key >= max_b t_b : every entry left out has a key
// below its workgroup's t_b, hence below the k-th, so the union's top k is
// the row's top k.  If the certificate fails (adversarial score layouts,
// massive ties) the row falls back to an exact radix select over all of its
// scores, which the stream kernel also writes out.
//
// Row path (generic shapes, f32): scores go to memory and one workgroup per
// row runs the exact radix select.
#include "common.h"
#include "internal.h"

namespace dsa {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kBins = 4096;           // row fallback histogram: top 12 key bits
constexpr int kBinShift = 20;
constexpr int kFinalCap = 8192;       // candidates resolved in LDS
constexpr int kStreamEntries = 1024;  // entries per workgroup in the stream kernel
constexpr int kThreads = 256;

// Four fp8 e4m3fn codes per dword -> eight bf16 values (exact widening).
__device__ __forceinline__ v8bf fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

struct RowInfo {
  int64_t nv;
  bool ok;
};

__device__ __forceinline__ RowInfo row_info(const int64_t* q_pos, int row, int s, int S,
                                            int64_t nv_cap, int64_t max_pos_end,
                                            uint32_t* status, bool report) {
  const int64_t m = q_pos[row];
  RowInfo r{0, true};
  if (m < 0 || m >= max_pos_end) {
    if (report) set_status(status, DSA_DEVERR_POSITION);
    r.ok = false;
    return r;
  }
  r.nv = n_complete(m, s, S);
  if (r.nv > nv_cap) {
    if (report) set_status(status, DSA_DEVERR_CAPACITY);
    r.nv = nv_cap;
  }
  return r;
}

// (key, complemented index): larger composite = larger score, then lower j.
__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t j) {
  return (static_cast<uint64_t>(key) << 32) | static_cast<uint64_t>(0xffffffffu - j);
}
__device__ __forceinline__ uint32_t comp_index(uint64_t c) {
  return 0xffffffffu - static_cast<uint32_t>(c);
}

__device__ __forceinline__ void emit(int32_t* idx_row, float* score_row, uint32_t pos, uint32_t j,
                                     float sc) {
  idx_row[pos] = static_cast<int32_t>(j);
  if (score_row) score_row[pos] = sc;
}

// ------------------------------------------------------- block primitives
// 256-thread inclusive suffix sums of cnt[0..255]: the digit d with
// sum(cnt[d+1..]) < need <= sum(cnt[d..]), the count above d, the count at
// d and the total.  If the total is below need, d = 0xffffffff.
struct Digit {
  uint32_t d, above, at, total;
};

__device__ Digit find_digit(const uint32_t* cnt, uint32_t need) {
  __shared__ uint32_t sfx[256];
  __shared__ Digit res;
  const int t = threadIdx.x;
  const uint32_t c = cnt[t];
  sfx[t] = c;
  if (t == 0) res.d = 0xffffffffu;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t add = (t + off < 256) ? sfx[t + off] : 0u;
    __syncthreads();
    sfx[t] += add;
    __syncthreads();
  }
  const uint32_t incl = sfx[t], excl = incl - c;
  if (excl < need && incl >= need) res = Digit{static_cast<uint32_t>(t), excl, c, 0u};
  __syncthreads();
  Digit r = res;
  r.total = sfx[0];
  __syncthreads();
  return r;
}

// rank-th largest (1-based) of the nonzero 32-bit keys in LDS; 0 if fewer.
__device__ uint32_t kth_largest_key(const uint32_t* keys, int n, uint32_t rank) {
  __shared__ uint32_t cnt[256];
  const int t = threadIdx.x;
  uint32_t prefix = 0, mask = 0, need = rank;
  for (int shift = 24; shift >= 0; shift -= 8) {
    cnt[t] = 0;
    __syncthreads();
    for (int i = t; i < n; i += kThreads) {
      const uint32_t k = keys[i];
      if (k != 0 && (k & mask) == prefix) atomicAdd(&cnt[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    const Digit dg = find_digit(cnt, need);
    if (dg.d == 0xffffffffu) return 0;
    prefix |= dg.d << shift;
    mask |= 255u << shift;
    need -= dg.above;
  }
  return prefix;
}

// Exact top-`need` among n distinct 64-bit composites in LDS: returns the
// smallest composite that is kept (keep every v >= result).
__device__ uint64_t kth_largest_composite(const uint64_t* c, int n, uint32_t need) {
  __shared__ uint32_t cnt[256];
  const int t = threadIdx.x;
  uint64_t prefix = 0, mask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    cnt[t] = 0;
    __syncthreads();
    for (int i = t; i < n; i += kThreads) {
      const uint64_t v = c[i];
      if ((v & mask) == prefix) atomicAdd(&cnt[(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    const Digit dg = find_digit(cnt, need);
    prefix |= static_cast<uint64_t>(dg.d) << shift;
    mask |= static_cast<uint64_t>(255u) << shift;
    need -= dg.above;
    if (dg.at == need) return prefix;  // every composite with this prefix is kept
  }
  return prefix;
}

// Rows with n_vis <= k: every visible entry, in index order, then padding.
__device__ void emit_all_visible(const float* srow, int64_t nv, int k, int32_t* idx_row,
                                 float* score_row) {
  for (int i = threadIdx.x; i < k; i += blockDim.x) {
    if (i < nv) emit(idx_row, score_row, i, i, srow ? srow[i] : 0.f);
    else {
      idx_row[i] = -1;
      if (score_row) score_row[i] = __uint_as_float(0x7fc00000u);
    }
  }
}

// Exact top-k of one row from its scores in global memory (nv > k):
// histogram of the top 12 key bits -> threshold bin; entries above it go
// straight out, the bin's entries are resolved exactly (in LDS when they
// fit, else by streaming radix passes).  cand_s: kFinalCap u64 of LDS,
// h_s: kBins u32 of LDS.
__device__ void row_select_from_scores(const float* srow, int64_t nv, int k, int32_t* irow,
                                       float* orow, uint64_t* cand_s, uint32_t* h_s) {
  __shared__ uint32_t cnt_above, cnt_cand, out_pos;
  __shared__ uint32_t part[kThreads];
  __shared__ uint32_t thr_s[3];
  __shared__ uint32_t cnt[256];
  const int t = threadIdx.x;
  for (int i = t; i < kBins; i += kThreads) h_s[i] = 0;
  if (t == 0) cnt_above = cnt_cand = out_pos = 0;
  __syncthreads();
  for (int64_t j = t; j < nv; j += kThreads) atomicAdd(&h_s[order_key(srow[j]) >> kBinShift], 1u);
  __syncthreads();
  // threshold bin: suffix counts over 4096 bins, 16 per thread
  uint32_t local[16], sum = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    local[i] = h_s[kBins - 1 - (16 * t + i)];
    sum += local[i];
  }
  part[t] = sum;
  __syncthreads();
  uint32_t before = 0;
  for (int i = 0; i < t; ++i) before += part[i];
  if (before < static_cast<uint32_t>(k) && before + sum >= static_cast<uint32_t>(k)) {
    uint32_t c = before;
    for (int i = 0; i < 16; ++i) {
      if (c + local[i] >= static_cast<uint32_t>(k)) {
        thr_s[0] = kBins - 1 - (16 * t + i);
        thr_s[1] = c;
        thr_s[2] = local[i];
        break;
      }
      c += local[i];
    }
  }
  __syncthreads();
  const uint32_t thr = thr_s[0], above = thr_s[1], at = thr_s[2];
  const bool fits = at <= static_cast<uint32_t>(kFinalCap);
  for (int64_t j = t; j < nv; j += kThreads) {
    const float sc = srow[j];
    const uint32_t key = order_key(sc);
    const uint32_t bin = key >> kBinShift;
    if (bin > thr) {
      const uint32_t p = atomicAdd(&cnt_above, 1u);
      if (p < static_cast<uint32_t>(k)) emit(irow, orow, p, static_cast<uint32_t>(j), sc);
    } else if (bin == thr && fits) {
      const uint32_t p = atomicAdd(&cnt_cand, 1u);
      if (p < static_cast<uint32_t>(kFinalCap)) cand_s[p] = composite(key, static_cast<uint32_t>(j));
    }
  }
  __syncthreads();
  const uint32_t need = static_cast<uint32_t>(k) - above;
  uint64_t cut;
  if (fits) {
    cut = kth_largest_composite(cand_s, static_cast<int>(at), need);
  } else {
    // streaming radix over the bin's entries, composites built on the fly
    uint64_t prefix = static_cast<uint64_t>(thr) << (32 + kBinShift);
    uint64_t mask = static_cast<uint64_t>(0xfffu) << (32 + kBinShift);
    uint32_t rem = need;
    for (int shift = 48; shift >= 0; shift -= 8) {
      cnt[t] = 0;
      __syncthreads();
      for (int64_t j = t; j < nv; j += kThreads) {
        const uint64_t v = composite(order_key(srow[j]), static_cast<uint32_t>(j));
        if ((v & mask) == prefix) atomicAdd(&cnt[(v >> shift) & 255u], 1u);
      }
      __syncthreads();
      const Digit dg = find_digit(cnt, rem);
      prefix |= static_cast<uint64_t>(dg.d) << shift;
      mask |= static_cast<uint64_t>(255u) << shift;
      rem -= dg.above;
      if (dg.at == rem) break;
    }
    cut = prefix;
  }
  // emit the threshold bin's kept entries
  if (fits) {
    for (int i = t; i < static_cast<int>(at); i += kThreads) {
      const uint64_t v = cand_s[i];
      if (v >= cut) {
        const uint32_t p = atomicAdd(&out_pos, 1u);
        if (p < need)
          emit(irow, orow, above + p, comp_index(v), key_to_float(static_cast<uint32_t>(v >> 32)));
      }
    }
  } else {
    for (int64_t j = t; j < nv; j += kThreads) {
      const uint64_t v = composite(order_key(srow[j]), static_cast<uint32_t>(j));
      if (v >= cut && (v >> (32 + kBinShift)) == thr) {
        const uint32_t p = atomicAdd(&out_pos, 1u);
        if (p < need) emit(irow, orow, above + p, comp_index(v), srow[j]);
      }
    }
  }
  __syncthreads();
}

// --------------------------------------------------- stream (decode) kernel
// Operand layout: lane l owns entry (or head) n = l % 16 and, within the
// 128-byte vector, bytes [16 g, 16 g + 16) and [64 + 16 g, 64 + 16 g + 16)
// with g = l / 16; MFMA c of the four takes the lane's bytes [8 c, 8 c + 8)
// of those 32.  A and B use the same byte-to-k assignment, so the four MFMAs
// sum every one of the 128 products exactly once; each of the two 16-byte
// loads of a wave covers 64 contiguous bytes of 16 entries.
template <bool kCand>
__global__ __launch_bounds__(kThreads) void k_index_fp8_stream(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ keys, const float* __restrict__ k_scale,
    const int64_t* __restrict__ q_pos, int Tq, int Hi, int s, int S, int64_t e_cap,
    int64_t nv_cap, int64_t max_pos_end, float* __restrict__ scores, int64_t ld_scores,
    uint64_t* __restrict__ cand, uint2* __restrict__ meta, int cap, uint32_t* status) {
  __shared__ uint32_t s_key[kCand ? kStreamEntries : 1];
  __shared__ uint32_t cand_cnt;
  const int row = blockIdx.y, b = row / Tq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const RowInfo ri = row_info(q_pos, row, s, S, nv_cap, max_pos_end, status, blockIdx.x == 0 && tid == 0);
  const int64_t nv = ri.nv;
  const int64_t e_begin = static_cast<int64_t>(blockIdx.x) * kStreamEntries;
  constexpr int kGroups = kStreamEntries / 4 / 16;  // 16-entry groups per wave
  constexpr int kUnroll = 4;
  if (e_begin < nv) {
    uint4 qlo = {0u, 0u, 0u, 0u}, qhi = {0u, 0u, 0u, 0u};
    if (n < Hi) {
      const uint4* qp = reinterpret_cast<const uint4*>(q + (static_cast<int64_t>(row) * Hi + n) * 128);
      qlo = qp[g];
      qhi = qp[4 + g];
    }
    const v8bf a0 = fp8x8_to_bf16(qlo.x, qlo.y), a1 = fp8x8_to_bf16(qlo.z, qlo.w);
    const v8bf a2 = fp8x8_to_bf16(qhi.x, qhi.y), a3 = fp8x8_to_bf16(qhi.z, qhi.w);
    float wv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g + i;
      wv[i] = 0.f;
      if (h < Hi) {
        const int64_t o = static_cast<int64_t>(row) * Hi + h;
        wv[i] = w[o] * (q_scale ? q_scale[o] : 1.0f);
      }
    }
    const uint8_t* kb = keys + static_cast<int64_t>(b) * e_cap * 128;
    const float* ksb = k_scale + static_cast<int64_t>(b) * e_cap;
    float* srow = scores + static_cast<int64_t>(row) * ld_scores;
    const int64_t wbase = e_begin + wave * (kStreamEntries / 4);
#pragma unroll 1
    for (int gi = 0; gi < kGroups; gi += kUnroll) {
      uint4 blo[kUnroll], bhi[kUnroll];
      float ks[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t ent = wbase + (gi + u) * 16 + n;
        if (ent < nv) {
          const uint4* kp = reinterpret_cast<const uint4*>(kb + ent * 128);
          blo[u] = kp[g];
          bhi[u] = kp[4 + g];
          ks[u] = ksb[ent];
        } else {
          blo[u] = bhi[u] = uint4{0u, 0u, 0u, 0u};
          ks[u] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, fp8x8_to_bf16(blo[u].x, blo[u].y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, fp8x8_to_bf16(blo[u].z, blo[u].w), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, fp8x8_to_bf16(bhi[u].x, bhi[u].y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a3, fp8x8_to_bf16(bhi[u].z, bhi[u].w), acc, 0, 0, 0);
        // lane holds rows (heads) 4g..4g+3 of column (entry) n
        float v = wv[0] * fmaxf(acc[0], 0.f) + wv[1] * fmaxf(acc[1], 0.f) +
                  wv[2] * fmaxf(acc[2], 0.f) + wv[3] * fmaxf(acc[3], 0.f);
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        const float sc = v * ks[u];
        const int local = wave * (kStreamEntries / 4) + (gi + u) * 16 + n;
        const int64_t ent = e_begin + local;
        if (g == 0) {
          if (ent < nv) srow[ent] = sc;
          if constexpr (kCand) s_key[local] = ent < nv ? order_key(sc) : 0u;
        }
      }
    }
  } else if constexpr (kCand) {
    for (int i = tid; i < kStreamEntries; i += kThreads) s_key[i] = 0u;
  }
  if constexpr (kCand) {
    // workgroup candidates: keys above the (cap+1)-th largest of this block
    if (tid == 0) cand_cnt = 0;
    __syncthreads();
    const uint32_t kth = kth_largest_key(s_key, kStreamEntries, static_cast<uint32_t>(cap) + 1u);
    const uint32_t tb = kth == 0 ? 1u : kth + 1u;  // fewer than cap+1 valid keys: take all
    uint64_t* crow = cand + (static_cast<int64_t>(row) * gridDim.x + blockIdx.x) * cap;
    for (int i = tid; i < kStreamEntries; i += kThreads) {
      const uint32_t key = s_key[i];
      if (key != 0u && key >= tb) {
        const uint32_t p = atomicAdd(&cand_cnt, 1u);
        if (p < static_cast<uint32_t>(cap))
          crow[p] = composite(key, static_cast<uint32_t>(e_begin + i));
      }
    }
    __syncthreads();
    if (tid == 0)
      meta[static_cast<int64_t>(row) * gridDim.x + blockIdx.x] =
          uint2{e_begin < nv ? tb : 0u, min(cand_cnt, static_cast<uint32_t>(cap))};
  }
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
    const T* kr = keys + (static_cast<int64_t>(b) * e_cap + ent) * Di;
    float tot = 0.f;
    for (int h = 0; h < Hi; ++h) {
      float d = 0.f;
      for (int i = 0; i < Di; ++i) {
        float kv;
        if constexpr (sizeof(T) == 1) kv = fp8_to_f32(kr[i]);
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
// Candidate path: union of the workgroups' candidates, exact top k, and the
// certificate; falls back to the full-row select when it does not hold.
__global__ __launch_bounds__(kThreads) void k_topk_cand_final(
    const float* __restrict__ scores, int64_t ld_scores, const int64_t* __restrict__ q_pos,
    int s, int S, int64_t nv_cap, int64_t max_pos_end, const uint64_t* __restrict__ cand,
    const uint2* __restrict__ meta, int nb, int cap, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out, int k) {
  __shared__ uint64_t cand_s[kFinalCap];
  __shared__ uint32_t h_s[kBins];  // block offsets here, then the fallback histogram
  __shared__ uint32_t part[kThreads];
  __shared__ uint32_t tmax_s, total_s, out_pos;
  const int row = blockIdx.x, t = threadIdx.x;
  const RowInfo ri = row_info(q_pos, row, s, S, nv_cap, max_pos_end, nullptr, false);
  const int64_t nv = ri.nv;
  const float* srow = scores + static_cast<int64_t>(row) * ld_scores;
  int32_t* irow = idx_out + static_cast<int64_t>(row) * k;
  float* orow = score_out ? score_out + static_cast<int64_t>(row) * k : nullptr;
  if (nv <= k) {
    emit_all_visible(srow, nv, k, irow, orow);
    return;
  }
  const uint2* mrow = meta + static_cast<int64_t>(row) * nb;
  if (t == 0) tmax_s = total_s = out_pos = 0;
  __syncthreads();
  // exclusive offsets of the per-block counts (nb <= kBins) and max t_b
  const int per = (nb + kThreads - 1) / kThreads;
  const int b0 = min(nb, t * per), b1 = min(nb, b0 + per);
  uint32_t sum = 0, tm = 0;
  for (int b = b0; b < b1; ++b) {
    const uint2 m = mrow[b];
    sum += m.y;
    tm = max(tm, m.x);
  }
  atomicMax(&tmax_s, tm);
  part[t] = sum;
  __syncthreads();
  uint32_t before = 0;
  for (int i = 0; i < t; ++i) before += part[i];
  for (int b = b0; b < b1; ++b) {
    h_s[b] = before;
    before += mrow[b].y;
  }
  if (t == kThreads - 1) total_s = before;
  __syncthreads();
  const uint32_t total = total_s, tmax = tmax_s;
  bool ok = total >= static_cast<uint32_t>(k) && total <= static_cast<uint32_t>(kFinalCap);
  uint64_t cut = 0;
  if (ok) {
    const int slots = nb * cap;
    const uint64_t* crow = cand + static_cast<int64_t>(row) * slots;
    for (int sl = t; sl < slots; sl += kThreads) {
      const int b = sl / cap, i = sl % cap;
      if (static_cast<uint32_t>(i) < mrow[b].y) cand_s[h_s[b] + i] = crow[sl];
    }
    __syncthreads();
    cut = kth_largest_composite(cand_s, static_cast<int>(total), static_cast<uint32_t>(k));
    ok = static_cast<uint32_t>(cut >> 32) >= tmax;  // the certificate
  }
  if (ok) {
    for (int i = t; i < static_cast<int>(total); i += kThreads) {
      const uint64_t v = cand_s[i];
      if (v >= cut) {
        const uint32_t p = atomicAdd(&out_pos, 1u);
        if (p < static_cast<uint32_t>(k))
          emit(irow, orow, p, comp_index(v), key_to_float(static_cast<uint32_t>(v >> 32)));
      }
    }
    return;
  }
  __syncthreads();
  row_select_from_scores(srow, nv, k, irow, orow, cand_s, h_s);
}

// Row path: one workgroup per query row selects from the row's scores.
__global__ __launch_bounds__(kThreads) void k_topk_rows(
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

struct Plan {
  int64_t nv_cap, ld;
  bool mfma, cand;
  int nb, cap;
  size_t off_scores, off_cand, off_meta, total;
};

Plan plan(const dsa_index_args& a) {
  Plan p{};
  const int64_t rows = static_cast<int64_t>(a.n_seqs) * a.queries_per_seq;
  p.nv_cap = std::min<int64_t>(a.e_cap, n_complete(a.max_pos_end - 1, a.stride, a.span));
  if (p.nv_cap < 0) p.nv_cap = 0;
  p.ld = (p.nv_cap + 63) / 64 * 64;
  p.mfma = a.keys != nullptr && a.dtype == DSA_FP8_E4M3 && a.dim == 128 && a.heads <= 16;
  p.nb = static_cast<int>(ceil_div(p.nv_cap, kStreamEntries));
  // candidates per workgroup: enough that the union is about 4k, at least 32
  p.cap = static_cast<int>(std::min<int64_t>(
      512, std::max<int64_t>(32, ceil_div(4 * static_cast<int64_t>(a.k), std::max(1, p.nb)))));
  p.cand = p.mfma && p.nv_cap > a.k && p.nb <= kBins;
  size_t off = 0;
  p.off_scores = off;
  off = align_up(off + static_cast<size_t>(rows) * p.ld * sizeof(float));
  p.off_cand = off;
  if (p.cand) off = align_up(off + static_cast<size_t>(rows) * p.nb * p.cap * sizeof(uint64_t));
  p.off_meta = off;
  if (p.cand) off = align_up(off + static_cast<size_t>(rows) * p.nb * sizeof(uint2));
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
  uint2* meta = reinterpret_cast<uint2*>(base + P.off_meta);
  const bool no_keys = a.keys == nullptr;  // only allowed when k >= every n_vis
  dsa_status rc;
  if (!no_keys && P.nv_cap > 0) {
    if (a.ev_index[0]) {
      rc = hip_check(hipEventRecord(static_cast<hipEvent_t>(a.ev_index[0]), st), "event record");
      if (rc != DSA_OK) return rc;
    }
    if (P.mfma) {
      dim3 grid(static_cast<unsigned>(P.nb), rows);
      if (P.cand)
        hipLaunchKernelGGL(k_index_fp8_stream<true>, grid, dim3(kThreads), 0, st,
                           static_cast<const uint8_t*>(a.q), a.q_scale, a.w,
                           static_cast<const uint8_t*>(a.keys), a.k_scale, a.q_pos,
                           a.queries_per_seq, a.heads, a.stride, a.span, a.e_cap, P.nv_cap,
                           a.max_pos_end, scores, P.ld, cand, meta, P.cap, a.status);
      else
        hipLaunchKernelGGL(k_index_fp8_stream<false>, grid, dim3(kThreads), 0, st,
                           static_cast<const uint8_t*>(a.q), a.q_scale, a.w,
                           static_cast<const uint8_t*>(a.keys), a.k_scale, a.q_pos,
                           a.queries_per_seq, a.heads, a.stride, a.span, a.e_cap, P.nv_cap,
                           a.max_pos_end, scores, P.ld, cand, meta, P.cap, a.status);
    } else {
      dim3 grid(static_cast<unsigned>(ceil_div(P.nv_cap, kThreads)), rows);
      const size_t shm = (static_cast<size_t>(a.heads) * a.dim + a.heads) * sizeof(float);
      if (a.dtype == DSA_F32)
        hipLaunchKernelGGL(k_index_generic<float>, grid, dim3(kThreads), shm, st,
                           static_cast<const float*>(a.q), a.q_scale, a.w,
                           static_cast<const float*>(a.keys), a.k_scale, a.q_pos,
                           a.queries_per_seq, a.heads, a.dim, a.stride, a.span, a.e_cap, P.nv_cap,
                           a.max_pos_end, scores, P.ld, a.status);
      else
        hipLaunchKernelGGL(k_index_generic<uint8_t>, grid, dim3(kThreads), shm, st,
                           static_cast<const uint8_t*>(a.q), a.q_scale, a.w,
                           static_cast<const uint8_t*>(a.keys), a.k_scale, a.q_pos,
                           a.queries_per_seq, a.heads, a.dim, a.stride, a.span, a.e_cap, P.nv_cap,
                           a.max_pos_end, scores, P.ld, a.status);
    }
    rc = hip_check(hipGetLastError(), "indexer launch");
    if (rc != DSA_OK) return rc;
    if (a.ev_index[1]) {
      rc = hip_check(hipEventRecord(static_cast<hipEvent_t>(a.ev_index[1]), st), "event record");
      if (rc != DSA_OK) return rc;
    }
  }
  if (P.cand && !no_keys) {
    hipLaunchKernelGGL(k_topk_cand_final, dim3(rows), dim3(kThreads), 0, st, scores, P.ld, a.q_pos,
                       a.stride, a.span, P.nv_cap, a.max_pos_end, cand, meta, P.nb, P.cap,
                       a.idx_out, a.score_out, a.k);
  } else {
    hipLaunchKernelGGL(k_topk_rows, dim3(rows), dim3(kThreads), 0, st, no_keys ? nullptr : scores,
                       P.ld, a.q_pos, a.stride, a.span, P.nv_cap, a.max_pos_end, a.idx_out,
                       a.score_out, a.k, a.status);
  }
  return hip_check(hipGetLastError(), "top-k launch");
}

}  // namespace dsa
