// The decode indexer's streaming body (one workgroup = 1024 entries of one
// query row), shared by the indexer kernel and the fused decode kernel.
// See indexer.hip for the method.
#pragma once

#include "common.h"

namespace dsa {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

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

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o, 64)));
  return v;
}

template <bool kCand>
__device__ __forceinline__ void index_stream_block(
    int bx, int nbx, int row, const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ keys, const float* __restrict__ k_scale,
    const int64_t* __restrict__ q_pos, int Tq, int Hi, int s, int S, int64_t e_cap,
    int64_t nv_cap, int64_t max_pos_end, float* __restrict__ scores, int64_t ld_scores,
    uint64_t* __restrict__ cand, uint32_t* __restrict__ meta, int cap, uint32_t* status) {
  const int b = row / Tq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const RowInfo ri = row_info(q_pos, row, s, S, nv_cap, max_pos_end, status, bx == 0 && tid == 0);
  const int64_t nv = ri.nv;
  const int64_t e_begin = static_cast<int64_t>(bx) * kStreamEntries;
  constexpr int kGroups = kStreamEntries / 4 / 16;  // 16-entry groups per wave
  constexpr int kUnroll = 4;
  const int64_t wbase = e_begin + wave * (kStreamEntries / 4);
  // each lane keeps the keys of the groups gi + g (one per outer step)
  uint32_t kk[kGroups / kUnroll] = {};
  if (wbase < nv) {
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
#pragma unroll
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
        v += __shfl_xor(v, 32, 64);  // every lane of column n now holds its score
        const float sc = v * ks[u];
        const int64_t ent = wbase + (gi + u) * 16 + n;
        if (g == 0 && ent < nv) srow[ent] = sc;
        if constexpr (kCand)
          if (u == g) kk[gi / kUnroll] = ent < nv ? order_key(sc) : 0u;
      }
    }
  }
  if constexpr (kCand) {
    // wave candidates: the keys above the (cap+1)-th largest of the wave's 256
    uint32_t work[kGroups / kUnroll];
#pragma unroll
    for (int i = 0; i < kGroups / kUnroll; ++i) work[i] = kk[i];
    uint32_t next = 0;
    for (int it = 0; it <= cap; ++it) {
      uint32_t m = work[0];
#pragma unroll
      for (int i = 1; i < kGroups / kUnroll; ++i) m = max(m, work[i]);
      m = wave_max_u32(m);
      next = m;
      if (m == 0u || it == cap) break;
      // drop one instance of m (from the lowest lane that holds it)
      bool has = false;
#pragma unroll
      for (int i = 0; i < kGroups / kUnroll; ++i) has |= work[i] == m;
      const uint64_t bal = __ballot(has);
      if (lane == __ffsll(static_cast<long long>(bal)) - 1) {
        bool done = false;
#pragma unroll
        for (int i = 0; i < kGroups / kUnroll; ++i)
          if (!done && work[i] == m) {
            work[i] = 0u;
            done = true;
          }
      }
    }
    // threshold: strictly above the (cap+1)-th largest (1 if fewer keys)
    const uint32_t tw = next == 0u ? 1u : (next == 0xffffffffu ? next : next + 1u);
    const int64_t wave_id = static_cast<int64_t>(row) * (nbx * 4) + bx * 4 + wave;
    uint64_t* crow = cand + wave_id * cap;
    int base = 0;
#pragma unroll
    for (int i = 0; i < kGroups / kUnroll; ++i) {
      const bool in = kk[i] != 0u && kk[i] >= tw;
      const uint64_t bal = __ballot(in);
      const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
      if (in && pos < cap) {
        const int64_t ent = wbase + (kUnroll * i + g) * 16 + n;
        crow[pos] = composite(kk[i], static_cast<uint32_t>(ent));
      }
      base += __popcll(bal);
    }
    if (lane >= base && lane < cap) crow[lane] = 0ull;  // empty slots
    if (lane == 0) meta[wave_id] = wbase < nv ? tw : 0u;
  }
}


}  // namespace dsa
