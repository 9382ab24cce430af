// S3 + S4: lightning indexer and Top-k selection.
//
// Score of query row i against visible entry j < n_vis(m_i):
//   I[i, j] = ks_j * sum_h (w_ih * qs_ih) * ReLU(q8_ih . k8_j)
// ("DeepSeek DSA、DeepSeek V4与vLLM Hybrid KV Cache详解" 4.1: a cheap score per
// (query, history entry), few heads, FP8).  The fp8 scales are positive, so
// they factor out of the ReLU: the dot products run on the raw e4m3 codes.
//
// Decode path (few query rows, long histories): k_index_fp8_stream streams
// the fp8 keys from HBM once per query.  The 16 indexer heads are the M side
// of one v_mfma_f32_16x16x128_f8f6f4 and 16 entries are its N side, so one
// MFMA scores 16 entries; ReLU, the head weights and the head sum are a
// 4-value in-lane reduce plus two cross-lane adds on the accumulator.  The
// same pass builds a 4096-bin histogram of the scores' top 12 key bits, and
// the last workgroup of a row picks the bin holding the k-th largest score.
// k_topk_collect then writes every entry above that bin straight to the
// output and gathers the bin's own entries as candidates, and
// k_topk_final resolves the candidates exactly (radix select on
// (score key, -index), so ties go to the lower index).
//
// Row path (many query rows, e.g. a prefill chunk): one workgroup per row
// histograms, collects and resolves its own row.
#include "common.h"
#include "internal.h"

namespace dsa {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBins = 4096;          // histogram on the top 12 bits of the key
constexpr int kBinShift = 20;
constexpr int kCtrl = 8;             // per-row control words
constexpr int kCandCap = 8192;       // candidates resolved in LDS
constexpr int kStreamEntries = 1024; // entries per workgroup in the stream kernel
constexpr int kStreamThreads = 256;

enum Ctrl { kDone = 0, kThrBin = 1, kAbove = 2, kAboveWritten = 3, kCandCount = 4, kBinCount = 5 };

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

// After all workgroups of a row have added their histogram, the last one
// finds the bin that holds the k-th largest key: count(bins > b1) < k <=
// count(bins >= b1).  Requires blockDim.x == 256.
__device__ void pick_threshold_bin(const uint32_t* hist, uint32_t* ctrl, int k) {
  __shared__ uint32_t part[256];
  __shared__ uint32_t found[3];
  const int t = threadIdx.x;
  // thread t owns bins [4095 - 16 t - 15, 4095 - 16 t] (descending)
  uint32_t local[16];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    local[i] = __hip_atomic_load(&hist[kBins - 1 - (16 * t + i)], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    sum += local[i];
  }
  part[t] = sum;
  if (t == 0) found[0] = 0xffffffffu;
  __syncthreads();
  // exclusive prefix over threads (descending bins)
  uint32_t before = 0;
  for (int i = 0; i < t; ++i) before += part[i];
  if (before < static_cast<uint32_t>(k) && before + sum >= static_cast<uint32_t>(k)) {
    uint32_t c = before;
    for (int i = 0; i < 16; ++i) {
      if (c + local[i] >= static_cast<uint32_t>(k)) {
        found[0] = kBins - 1 - (16 * t + i);
        found[1] = c;
        found[2] = local[i];
        break;
      }
      c += local[i];
    }
  }
  __syncthreads();
  if (t == 0) {
    ctrl[kThrBin] = found[0];
    ctrl[kAbove] = found[1];
    ctrl[kBinCount] = found[2];
  }
}

// Histogram flush + last-workgroup-done detection for the split path.
__device__ void finish_hist(uint32_t* h_s, uint32_t* hist, uint32_t* ctrl, int k) {
  __shared__ int is_last;
  __syncthreads();
  for (int i = threadIdx.x; i < kBins; i += blockDim.x) {
    const uint32_t v = h_s[i];
    if (v) atomicAdd(&hist[i], v);
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = atomicAdd(&ctrl[kDone], 1u);
    is_last = (prev == gridDim.x - 1);
  }
  __syncthreads();
  if (is_last) {
    __threadfence();
    pick_threshold_bin(hist, ctrl, k);
  }
}

// ---------------------------------------------------------------- fp8 MFMA
// Operand layout: lane l owns entry (or head) n = l % 16 and, within the
// 128-byte vector, bytes [16 g, 16 g + 16) and [64 + 16 g, 64 + 16 g + 16)
// with g = l / 16.  A and B use the same byte-to-k assignment, so the MFMA
// sums every one of the 128 products exactly once; each of the two 16-byte
// loads of a wave covers 64 contiguous bytes of 16 entries.
template <bool kHist>
__global__ __launch_bounds__(kStreamThreads) void k_index_fp8_stream(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ keys, const float* __restrict__ k_scale,
    const int64_t* __restrict__ q_pos, int Tq, int Hi, int s, int S, int64_t e_cap,
    int64_t nv_cap, int64_t max_pos_end, float* __restrict__ scores, int64_t ld_scores,
    uint32_t* __restrict__ hist, uint32_t* __restrict__ ctrl, int k, uint32_t* status) {
  __shared__ uint32_t h_s[kHist ? kBins : 1];
  const int row = blockIdx.y, b = row / Tq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const RowInfo ri = row_info(q_pos, row, s, S, nv_cap, max_pos_end, status, blockIdx.x == 0 && tid == 0);
  const int64_t nv = ri.nv;
  if constexpr (kHist) {
    for (int i = tid; i < kBins; i += kStreamThreads) h_s[i] = 0;
    __syncthreads();
  }
  const int64_t e_begin = static_cast<int64_t>(blockIdx.x) * kStreamEntries;
  if (e_begin < nv) {
    v8i a = {0, 0, 0, 0, 0, 0, 0, 0};
    if (n < Hi) {
      const uint4* qp = reinterpret_cast<const uint4*>(q + (static_cast<int64_t>(row) * Hi + n) * 128);
      const uint4 lo = qp[g], hi = qp[4 + g];
      a = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
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
    constexpr int kGroups = kStreamEntries / 4 / 16;  // 16-entry groups per wave
    constexpr int kUnroll = 4;
    const int64_t wbase = e_begin + wave * (kStreamEntries / 4);
#pragma unroll 1
    for (int gi = 0; gi < kGroups; gi += kUnroll) {
      v8i bk[kUnroll];
      float ks[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t ent = wbase + (gi + u) * 16 + n;
        if (ent < nv) {
          const uint4* kp = reinterpret_cast<const uint4*>(kb + ent * 128);
          const uint4 lo = kp[g], hi = kp[4 + g];
          bk[u] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          ks[u] = ksb[ent];
        } else {
          bk[u] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
          ks[u] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        // fp8 e4m3 x fp8 e4m3, scales unused (0) -> the plain MFMA
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bk[u], acc, 0, 0, 0, 0, 0, 0);
        // lane holds rows (heads) 4g..4g+3 of column (entry) n
        float v = wv[0] * fmaxf(acc[0], 0.f) + wv[1] * fmaxf(acc[1], 0.f) +
                  wv[2] * fmaxf(acc[2], 0.f) + wv[3] * fmaxf(acc[3], 0.f);
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        const float sc = v * ks[u];
        const int64_t ent = wbase + (gi + u) * 16 + n;
        if (g == 0 && ent < nv) {
          srow[ent] = sc;
          if constexpr (kHist) atomicAdd(&h_s[order_key(sc) >> kBinShift], 1u);
        }
      }
    }
  }
  if constexpr (kHist) finish_hist(h_s, hist + static_cast<int64_t>(row) * kBins,
                                   ctrl + static_cast<int64_t>(row) * kCtrl, k);
}

// ------------------------------------------------------------- generic VALU
// Any Hi, Di; q and keys f32 or fp8.  One entry per thread.
template <typename T, bool kHist>
__global__ __launch_bounds__(256) void k_index_generic(
    const T* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const T* __restrict__ keys, const float* __restrict__ k_scale, const int64_t* __restrict__ q_pos,
    int Tq, int Hi, int Di, int s, int S, int64_t e_cap, int64_t nv_cap, int64_t max_pos_end,
    float* __restrict__ scores, int64_t ld_scores, uint32_t* __restrict__ hist,
    uint32_t* __restrict__ ctrl, int k, uint32_t* status) {
  extern __shared__ float q_s[];  // [Hi * Di] then [Hi] weights
  __shared__ uint32_t h_s[kHist ? kBins : 1];
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
  if constexpr (kHist)
    for (int i = tid; i < kBins; i += blockDim.x) h_s[i] = 0;
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
    if constexpr (kHist) atomicAdd(&h_s[order_key(tot) >> kBinShift], 1u);
  }
  if constexpr (kHist) finish_hist(h_s, hist + static_cast<int64_t>(row) * kBins,
                                   ctrl + static_cast<int64_t>(row) * kCtrl, k);
}

// ------------------------------------------------------------------ Top-k
__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t j) {
  // low 20 bits of the key (the top 12 are the threshold bin), then the
  // complemented index so that, among equal scores, the lower index wins
  return (static_cast<uint64_t>(key & 0xfffffu) << 32) | static_cast<uint64_t>(0xffffffffu - j);
}

__device__ __forceinline__ void emit(int32_t* idx_row, float* score_row, int pos, uint32_t j,
                                     float sc) {
  idx_row[pos] = static_cast<int32_t>(j);
  if (score_row) score_row[pos] = sc;
}

// Block-wide (256 threads) search: digit d such that the count of elements
// with digit > d is < need <= count with digit >= d.  cnt[256] in LDS.
__device__ void find_digit(const uint32_t* cnt, uint32_t need, uint32_t* out_digit,
                           uint32_t* out_above, uint32_t* out_at) {
  __shared__ uint32_t sfx[256];
  const int t = threadIdx.x;
  // inclusive suffix sum over digits 255..t
  const uint32_t c = cnt[t];
  sfx[t] = c;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t add = (t + off < 256) ? sfx[t + off] : 0u;
    __syncthreads();
    sfx[t] += add;
    __syncthreads();
  }
  const uint32_t incl = sfx[t], excl = incl - c;
  if (excl < need && incl >= need) {
    *out_digit = t;
    *out_above = excl;
    *out_at = c;
  }
  __syncthreads();
}

// Select the `need` largest composites among the candidates of one row and
// emit them at positions base_pos .. base_pos + need - 1.  Candidates come
// either from an LDS array (n_lds of them) or, when they did not fit, from
// the row's scores in global memory filtered on the threshold bin.
// blockDim.x == 256.
__device__ void resolve_candidates(const uint64_t* cand, int n_lds, bool from_global,
                                   const float* srow, int64_t nv, uint32_t thr_bin, uint32_t need,
                                   int32_t* idx_row, float* score_row, int base_pos) {
  __shared__ uint32_t cnt[256];
  __shared__ uint32_t dig[3];
  __shared__ uint32_t out_pos;
  const int t = threadIdx.x;
  uint64_t prefix = 0, mask = 0;
  uint32_t remaining = need;
  bool take_all = false;
  for (int shift = 48; shift >= 0; shift -= 8) {
    cnt[t] = 0;
    __syncthreads();
    if (from_global) {
      for (int64_t j = t; j < nv; j += 256) {
        const uint32_t key = order_key(srow[j]);
        if ((key >> kBinShift) != thr_bin) continue;
        const uint64_t c = composite(key, static_cast<uint32_t>(j));
        if ((c & mask) == prefix) atomicAdd(&cnt[(c >> shift) & 255u], 1u);
      }
    } else {
      for (int i = t; i < n_lds; i += 256) {
        const uint64_t c = cand[i];
        if ((c & mask) == prefix) atomicAdd(&cnt[(c >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    find_digit(cnt, remaining, &dig[0], &dig[1], &dig[2]);
    const uint32_t d = dig[0], above = dig[1], at = dig[2];
    prefix |= static_cast<uint64_t>(d) << shift;
    mask |= static_cast<uint64_t>(255u) << shift;
    remaining -= above;
    if (at == remaining) {  // every element with this prefix is in: done
      take_all = true;
      break;
    }
    __syncthreads();
  }
  (void)take_all;
  // emit: composites above the prefix (on the resolved bits) or equal to it
  if (t == 0) out_pos = 0;
  __syncthreads();
  auto consider = [&](uint64_t c) {
    if ((c & mask) >= prefix) {
      const uint32_t p = atomicAdd(&out_pos, 1u);
      if (p >= need) return;  // cannot happen with distinct composites; keeps writes in bounds
      const uint32_t j = 0xffffffffu - static_cast<uint32_t>(c);
      const uint32_t key = (thr_bin << kBinShift) | static_cast<uint32_t>(c >> 32);
      emit(idx_row, score_row, base_pos + p, j, key_to_float(key));
    }
  };
  if (from_global) {
    for (int64_t j = t; j < nv; j += 256) {
      const uint32_t key = order_key(srow[j]);
      if ((key >> kBinShift) == thr_bin) consider(composite(key, static_cast<uint32_t>(j)));
    }
  } else {
    for (int i = t; i < n_lds; i += 256) consider(cand[i]);
  }
  __syncthreads();
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

// Split path, pass 2: entries above the threshold bin go straight out; the
// bin's own entries become candidates.
__global__ __launch_bounds__(256) void k_topk_collect(
    const float* __restrict__ scores, int64_t ld_scores, const int64_t* __restrict__ q_pos,
    int s, int S, int64_t nv_cap, int64_t max_pos_end, uint32_t* __restrict__ ctrl,
    uint64_t* __restrict__ cand, int32_t* __restrict__ idx_out, float* __restrict__ score_out,
    int k) {
  const int row = blockIdx.y;
  const RowInfo ri = row_info(q_pos, row, s, S, nv_cap, max_pos_end, nullptr, false);
  const int64_t nv = ri.nv;
  if (nv <= k) return;
  uint32_t* c = ctrl + static_cast<int64_t>(row) * kCtrl;
  const uint32_t thr = c[kThrBin];
  const float* srow = scores + static_cast<int64_t>(row) * ld_scores;
  int32_t* irow = idx_out + static_cast<int64_t>(row) * k;
  float* orow = score_out ? score_out + static_cast<int64_t>(row) * k : nullptr;
  uint64_t* crow = cand + static_cast<int64_t>(row) * kCandCap;
  for (int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; j < nv;
       j += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const float sc = srow[j];
    const uint32_t key = order_key(sc);
    const uint32_t bin = key >> kBinShift;
    if (bin > thr) {
      const uint32_t p = atomicAdd(&c[kAboveWritten], 1u);
      if (p < static_cast<uint32_t>(k)) emit(irow, orow, p, static_cast<uint32_t>(j), sc);
    } else if (bin == thr) {
      const uint32_t p = atomicAdd(&c[kCandCount], 1u);
      if (p < kCandCap) crow[p] = composite(key, static_cast<uint32_t>(j));
    }
  }
}

// Split path, pass 3: one workgroup per row resolves the threshold bin.
__global__ __launch_bounds__(256) void k_topk_final(
    const float* __restrict__ scores, int64_t ld_scores, const int64_t* __restrict__ q_pos,
    int s, int S, int64_t nv_cap, int64_t max_pos_end, const uint32_t* __restrict__ ctrl,
    const uint64_t* __restrict__ cand, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out, int k, uint32_t* status) {
  __shared__ uint64_t cand_s[kCandCap];
  const int row = blockIdx.x;
  const RowInfo ri = row_info(q_pos, row, s, S, nv_cap, max_pos_end, nullptr, false);
  const int64_t nv = ri.nv;
  const float* srow = scores + static_cast<int64_t>(row) * ld_scores;
  int32_t* irow = idx_out + static_cast<int64_t>(row) * k;
  float* orow = score_out ? score_out + static_cast<int64_t>(row) * k : nullptr;
  if (nv <= k || scores == nullptr) {
    if (nv > k && threadIdx.x == 0) set_status(status, DSA_DEVERR_NO_INDEX);
    emit_all_visible(nullptr, ri.ok ? std::min<int64_t>(nv, k) : 0, k, irow, orow);
    return;
  }
  const uint32_t* c = ctrl + static_cast<int64_t>(row) * kCtrl;
  const uint32_t thr = c[kThrBin], above = c[kAbove], at = c[kBinCount];
  const uint32_t need = static_cast<uint32_t>(k) - above;
  const bool fits = at <= static_cast<uint32_t>(kCandCap);
  if (fits) {
    const uint64_t* crow = cand + static_cast<int64_t>(row) * kCandCap;
    for (int i = threadIdx.x; i < static_cast<int>(at); i += blockDim.x) cand_s[i] = crow[i];
  }
  __syncthreads();
  resolve_candidates(cand_s, fits ? static_cast<int>(at) : 0, !fits, srow, nv, thr, need, irow,
                     orow, static_cast<int>(above));
}

// Row path: one workgroup (256 threads) per query row does all three passes.
__global__ __launch_bounds__(256) void k_topk_rows(
    const float* __restrict__ scores, int64_t ld_scores, const int64_t* __restrict__ q_pos,
    int s, int S, int64_t nv_cap, int64_t max_pos_end, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out, int k, uint32_t* status) {
  __shared__ uint32_t h_s[kBins];
  __shared__ uint64_t cand_s[kCandCap];
  __shared__ uint32_t above_cnt, cand_cnt;
  const int row = blockIdx.x, t = threadIdx.x;
  const RowInfo ri = row_info(q_pos, row, s, S, nv_cap, max_pos_end, nullptr, false);
  const int64_t nv = ri.nv;
  const float* srow = scores + static_cast<int64_t>(row) * ld_scores;
  int32_t* irow = idx_out + static_cast<int64_t>(row) * k;
  float* orow = score_out ? score_out + static_cast<int64_t>(row) * k : nullptr;
  if (nv <= k || scores == nullptr) {
    if (nv > k && t == 0) set_status(status, DSA_DEVERR_NO_INDEX);
    emit_all_visible(scores ? srow : nullptr, ri.ok ? std::min<int64_t>(nv, k) : 0, k, irow, orow);
    return;
  }
  for (int i = t; i < kBins; i += 256) h_s[i] = 0;
  if (t == 0) above_cnt = cand_cnt = 0;
  __syncthreads();
  for (int64_t j = t; j < nv; j += 256) atomicAdd(&h_s[order_key(srow[j]) >> kBinShift], 1u);
  __syncthreads();
  __shared__ uint32_t ctrl_s[kCtrl];
  {
    // same search as pick_threshold_bin, on the LDS histogram
    __shared__ uint32_t part[256];
    uint32_t local[16];
    uint32_t sum = 0;
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
          ctrl_s[kThrBin] = kBins - 1 - (16 * t + i);
          ctrl_s[kAbove] = c;
          ctrl_s[kBinCount] = local[i];
          break;
        }
        c += local[i];
      }
    }
    __syncthreads();
  }
  const uint32_t thr = ctrl_s[kThrBin], above = ctrl_s[kAbove], at = ctrl_s[kBinCount];
  const bool fits = at <= static_cast<uint32_t>(kCandCap);
  for (int64_t j = t; j < nv; j += 256) {
    const float sc = srow[j];
    const uint32_t key = order_key(sc);
    const uint32_t bin = key >> kBinShift;
    if (bin > thr) {
      const uint32_t p = atomicAdd(&above_cnt, 1u);
      if (p < static_cast<uint32_t>(k)) emit(irow, orow, p, static_cast<uint32_t>(j), sc);
    } else if (bin == thr && fits) {
      const uint32_t p = atomicAdd(&cand_cnt, 1u);
      if (p < static_cast<uint32_t>(kCandCap)) cand_s[p] = composite(key, static_cast<uint32_t>(j));
    }
  }
  __syncthreads();
  resolve_candidates(cand_s, fits ? static_cast<int>(at) : 0, !fits, srow, nv, thr,
                     static_cast<uint32_t>(k) - above, irow, orow, static_cast<int>(above));
}

struct WsLayout {
  int64_t nv_cap, ld;
  size_t off_scores, off_hist, off_ctrl, off_cand, total;
  bool split;
};

WsLayout layout(const dsa_index_args& a) {
  WsLayout L{};
  const int64_t rows = static_cast<int64_t>(a.n_seqs) * a.queries_per_seq;
  L.nv_cap = std::min<int64_t>(a.e_cap, n_complete(a.max_pos_end - 1, a.stride, a.span));
  if (L.nv_cap < 0) L.nv_cap = 0;
  L.ld = (L.nv_cap + 63) / 64 * 64;
  L.split = a.queries_per_seq < 8 || rows < 256;
  size_t off = 0;
  L.off_scores = off;
  off = align_up(off + static_cast<size_t>(rows) * L.ld * sizeof(float));
  L.off_hist = off;
  if (L.split) off = align_up(off + static_cast<size_t>(rows) * kBins * sizeof(uint32_t));
  L.off_ctrl = off;
  if (L.split) off = align_up(off + static_cast<size_t>(rows) * kCtrl * sizeof(uint32_t));
  L.off_cand = off;
  if (L.split) off = align_up(off + static_cast<size_t>(rows) * kCandCap * sizeof(uint64_t));
  L.total = off;
  return L;
}

}  // namespace

size_t index_topk_ws_bytes(const dsa_index_args& a) { return layout(a).total; }

dsa_status launch_index_topk(const dsa_index_args& a, void* ws, hipStream_t st) {
  const WsLayout L = layout(a);
  const int rows = a.n_seqs * a.queries_per_seq;
  char* base = static_cast<char*>(ws);
  float* scores = reinterpret_cast<float*>(base + L.off_scores);
  uint32_t* hist = reinterpret_cast<uint32_t*>(base + L.off_hist);
  uint32_t* ctrl = reinterpret_cast<uint32_t*>(base + L.off_ctrl);
  uint64_t* cand = reinterpret_cast<uint64_t*>(base + L.off_cand);
  const bool no_keys = a.keys == nullptr;  // only allowed when k >= every n_vis
  dsa_status rc;
  if (L.split && !no_keys) {
    rc = launch_zero(hist, L.off_cand - L.off_hist, st);
    if (rc != DSA_OK) return rc;
  }
  if (!no_keys && L.nv_cap > 0) {
    if (a.ev_index[0]) {
      rc = hip_check(hipEventRecord(static_cast<hipEvent_t>(a.ev_index[0]), st), "event record");
      if (rc != DSA_OK) return rc;
    }
    const bool mfma = a.dtype == DSA_FP8_E4M3 && a.dim == 128 && a.heads <= 16;
    if (mfma) {
      dim3 grid(static_cast<unsigned>(ceil_div(L.nv_cap, kStreamEntries)), rows);
      if (L.split)
        hipLaunchKernelGGL(k_index_fp8_stream<true>, grid, dim3(kStreamThreads), 0, st,
                           static_cast<const uint8_t*>(a.q), a.q_scale, a.w,
                           static_cast<const uint8_t*>(a.keys), a.k_scale, a.q_pos,
                           a.queries_per_seq, a.heads, a.stride, a.span, a.e_cap, L.nv_cap,
                           a.max_pos_end, scores, L.ld, hist, ctrl, a.k, a.status);
      else
        hipLaunchKernelGGL(k_index_fp8_stream<false>, grid, dim3(kStreamThreads), 0, st,
                           static_cast<const uint8_t*>(a.q), a.q_scale, a.w,
                           static_cast<const uint8_t*>(a.keys), a.k_scale, a.q_pos,
                           a.queries_per_seq, a.heads, a.stride, a.span, a.e_cap, L.nv_cap,
                           a.max_pos_end, scores, L.ld, hist, ctrl, a.k, a.status);
    } else {
      dim3 grid(static_cast<unsigned>(ceil_div(L.nv_cap, 256)), rows);
      const size_t shm = (static_cast<size_t>(a.heads) * a.dim + a.heads) * sizeof(float);
#define DSA_GENERIC(T, H)                                                                       \
  hipLaunchKernelGGL((k_index_generic<T, H>), grid, dim3(256), shm, st,                          \
                     static_cast<const T*>(a.q), a.q_scale, a.w, static_cast<const T*>(a.keys), \
                     a.k_scale, a.q_pos, a.queries_per_seq, a.heads, a.dim, a.stride, a.span,   \
                     a.e_cap, L.nv_cap, a.max_pos_end, scores, L.ld, hist, ctrl, a.k, a.status)
      if (a.dtype == DSA_F32) {
        if (L.split) DSA_GENERIC(float, true); else DSA_GENERIC(float, false);
      } else {
        if (L.split) DSA_GENERIC(uint8_t, true); else DSA_GENERIC(uint8_t, false);
      }
#undef DSA_GENERIC
    }
    rc = hip_check(hipGetLastError(), "indexer launch");
    if (rc != DSA_OK) return rc;
    if (a.ev_index[1]) {
      rc = hip_check(hipEventRecord(static_cast<hipEvent_t>(a.ev_index[1]), st), "event record");
      if (rc != DSA_OK) return rc;
    }
  }
  if (L.split) {
    if (!no_keys && L.nv_cap > static_cast<int64_t>(a.k)) {
      const unsigned cb = static_cast<unsigned>(std::min<int64_t>(64, ceil_div(L.nv_cap, 4096)));
      hipLaunchKernelGGL(k_topk_collect, dim3(std::max(1u, cb), rows), dim3(256), 0, st, scores,
                         L.ld, a.q_pos, a.stride, a.span, L.nv_cap, a.max_pos_end, ctrl, cand,
                         a.idx_out, a.score_out, a.k);
      rc = hip_check(hipGetLastError(), "k_topk_collect launch");
      if (rc != DSA_OK) return rc;
    }
    hipLaunchKernelGGL(k_topk_final, dim3(rows), dim3(256), 0, st, no_keys ? nullptr : scores,
                       L.ld, a.q_pos, a.stride, a.span, L.nv_cap, a.max_pos_end, ctrl, cand,
                       a.idx_out, a.score_out, a.k, a.status);
  } else {
    hipLaunchKernelGGL(k_topk_rows, dim3(rows), dim3(256), 0, st, no_keys ? nullptr : scores,
                       L.ld, a.q_pos, a.stride, a.span, L.nv_cap, a.max_pos_end, a.idx_out,
                       a.score_out, a.k, a.status);
  }
  return hip_check(hipGetLastError(), "top-k launch");
}

}  // namespace dsa
