// The decode indexer's streaming body (one workgroup = 1024 entries of one
// query row), shared by the indexer kernel and the fused decode kernel.
// See indexer.hip for the method.
#pragma once

#include "common.h"

namespace dsa {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

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
  // within 16-lane rows by DPP (row_ror 8, row_ror 4, quad xor 2, quad xor
  // 1), then across rows with the gfx950 lane swaps: short dependency chain,
  // no LDS traffic
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x128, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x124, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(static_cast<uint32_t>(a[0]), static_cast<uint32_t>(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(static_cast<uint32_t>(b[0]), static_cast<uint32_t>(b[1]));
}

// Exact score (before the key scale) of entry column n for one row: A = the
// row's 16 heads widened to bf16 (aq), f32 head weights wv for heads
// 4g .. 4g+3; B = the entry's operand chunks.  Every lane of column n gets
// the sum over heads.
__device__ __forceinline__ float exact_tile_score(const v8bf (&aq)[4], const float (&wv)[4],
                                                  uint4 blo, uint4 bhi) {
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[0], fp8x8_to_bf16(blo.x, blo.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[1], fp8x8_to_bf16(blo.z, blo.w), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[2], fp8x8_to_bf16(bhi.x, bhi.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[3], fp8x8_to_bf16(bhi.z, bhi.w), acc, 0, 0, 0);
  float v = wv[0] * fmaxf(acc[0], 0.f) + wv[1] * fmaxf(acc[1], 0.f) +
            wv[2] * fmaxf(acc[2], 0.f) + wv[3] * fmaxf(acc[3], 0.f);
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// A row's exact operands: its heads (lane = head n, chunks g and 4 + g)
// widened to bf16, and w * q_scale for heads 4g .. 4g+3.
__device__ __forceinline__ void exact_row_operands(const uint8_t* q, const float* q_scale,
                                                   const float* w, int64_t row, int Hi,
                                                   v8bf (&aq)[4], float (&wv)[4]) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  uint4 qlo = {0u, 0u, 0u, 0u}, qhi = {0u, 0u, 0u, 0u};
  if (n < Hi) {
    const uint4* qp = reinterpret_cast<const uint4*>(q + (row * Hi + n) * 128);
    qlo = qp[g];
    qhi = qp[4 + g];
  }
  aq[0] = fp8x8_to_bf16(qlo.x, qlo.y);
  aq[1] = fp8x8_to_bf16(qlo.z, qlo.w);
  aq[2] = fp8x8_to_bf16(qhi.x, qhi.y);
  aq[3] = fp8x8_to_bf16(qhi.z, qhi.w);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g + i;
    wv[i] = 0.f;
    if (h < Hi) {
      const int64_t o = row * Hi + h;
      wv[i] = w[o] * (q_scale ? q_scale[o] : 1.0f);
    }
  }
}

// Exact scores of a row's first nv entries into srow (every wave of the
// workgroup takes every nwaves-th tile of 16 entries).
__device__ __forceinline__ void score_row_exact(const v8bf (&aq)[4], const float (&wv)[4],
                                                const uint8_t* kb, const float* ksb, int64_t nv,
                                                float* srow, int nwaves) {
  // four tiles' loads in flight per wave and round
  constexpr int kBatch = 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 15, g = lane >> 4;
  for (int64_t t0 = wave; t0 * 16 < nv; t0 += kBatch * nwaves) {
    uint4 blo[kBatch], bhi[kBatch];
    float ks[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t j = (t0 + static_cast<int64_t>(u) * nwaves) * 16 + n;
      blo[u] = bhi[u] = uint4{0u, 0u, 0u, 0u};
      ks[u] = 0.f;
      if (j < nv) {
        idx_load_chunks(kb, j, g, &blo[u], &bhi[u]);
        ks[u] = ksb[j];
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t j = (t0 + static_cast<int64_t>(u) * nwaves) * 16 + n;
      const float sc = exact_tile_score(aq, wv, blo[u], bhi[u]) * ks[u];
      if (g == 0 && j < nv) srow[j] = sc;
    }
  }
}

// kEnt entries per workgroup, 4 waves of kEnt / 4.  With kCand the scores
// stay in registers (candidates and wave thresholds go out; a row whose
// certificate fails is re-scored by the final pass); without, every score
// is written to its row.
template <bool kCand, int kEnt>
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
  const int64_t e_begin = static_cast<int64_t>(bx) * kEnt;
  constexpr int kGroups = kEnt / 4 / 16;            // 16-entry groups per wave
  constexpr int kSteps = kGroups / 2;               // two groups per step
  constexpr int kKeep = kGroups / 4;                // keys kept per lane
  const int64_t wbase = e_begin + wave * (kEnt / 4);
  // each lane keeps the keys of groups 4i + 2 (g & 1) + (g >> 1), i < kKeep
  uint32_t kk[kKeep] = {};
  if (wbase < nv) {
    const uint8_t* kb = keys + static_cast<int64_t>(b) * idx_e_pad(e_cap) * 128;
    const float* ksb = k_scale + static_cast<int64_t>(b) * e_cap;
    // key loads: a ring of two slots of two groups; unconditional (clamped
    // to a visible entry, masked later) so the compiler can count them, and
    // the first slot issued before the query set-up
    const int64_t jmax = nv - 1;
    uint4 blo[2][2], bhi[2][2];
    float ks[2][2];
    auto load = [&](int slot, int gr) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t ent = min<int64_t>(wbase + (gr + u) * 16 + n, jmax);
        idx_load_chunks(kb, ent, g, &blo[slot][u], &bhi[slot][u]);
        ks[slot][u] = ksb[ent];
      }
    };
    load(0, 0);
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
    float* srow = scores + static_cast<int64_t>(row) * ld_scores;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int sl = st & 1;
      if (st + 1 < kSteps) load(sl ^ 1, 2 * (st + 1));
      float part[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, fp8x8_to_bf16(blo[sl][u].x, blo[sl][u].y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, fp8x8_to_bf16(blo[sl][u].z, blo[sl][u].w), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, fp8x8_to_bf16(bhi[sl][u].x, bhi[sl][u].y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a3, fp8x8_to_bf16(bhi[sl][u].z, bhi[sl][u].w), acc, 0, 0, 0);
        // lane holds rows (heads) 4g..4g+3 of column (entry) n
        part[u] = wv[0] * fmaxf(acc[0], 0.f) + wv[1] * fmaxf(acc[1], 0.f) +
                  wv[2] * fmaxf(acc[2], 0.f) + wv[3] * fmaxf(acc[3], 0.f);
      }
      // head-group sums of both groups with the gfx950 lane swaps:
      // permlane32_swap(x, y) -> ([x 0-31, y 0-31], [x 32-63, y 32-63]),
      // permlane16_swap(x, x) -> rows (r0, r0, r2, r2) and (r1, r1, r3, r3);
      // lanes 0-31 end with group 0's score of entry n, lanes 32-63 group 1's
      const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[1]), false, false);
      const float z = __uint_as_float(x32[0]) + __uint_as_float(x32[1]);
      const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(z), __float_as_uint(z), false, false);
      const float v = __uint_as_float(x16[0]) + __uint_as_float(x16[1]);
      const int u = g >> 1;
      const float sc = v * ks[sl][u];
      const int64_t ent = wbase + (2 * st + u) * 16 + n;
      const bool vis = ent < nv;
      if constexpr (!kCand)
        if ((g & 1) == 0 && vis) srow[ent] = sc;
      if constexpr (kCand)
        if ((g & 1) == (st & 1)) kk[st >> 1] = vis ? order_key(sc) : 0u;
    }
  }
  if constexpr (kCand) {
    // wave candidates: the keys above the (cap+1)-th largest of the wave's 256
    uint32_t work[kKeep];
#pragma unroll
    for (int i = 0; i < kKeep; ++i) work[i] = kk[i];
    uint32_t next = 0;
    for (int it = 0; it <= cap; ++it) {
      uint32_t m = work[0];
#pragma unroll
      for (int i = 1; i < kKeep; ++i) m = max(m, work[i]);
      m = wave_max_u32(m);
      next = m;
      if (m == 0u || it == cap) break;
      // drop one instance of m (from the lowest lane that holds it)
      bool has = false;
#pragma unroll
      for (int i = 0; i < kKeep; ++i) has |= work[i] == m;
      const uint64_t bal = __ballot(has);
      if (lane == __ffsll(static_cast<long long>(bal)) - 1) {
        bool done = false;
#pragma unroll
        for (int i = 0; i < kKeep; ++i)
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
    for (int i = 0; i < kKeep; ++i) {
      const bool in = kk[i] != 0u && kk[i] >= tw;
      const uint64_t bal = __ballot(in);
      const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
      if (in && pos < cap) {
        const int64_t ent = wbase + (4 * i + 2 * (g & 1) + (g >> 1)) * 16 + n;
        crow[pos] = composite(kk[i], static_cast<uint32_t>(ent));
      }
      base += __popcll(bal);
    }
    if (lane >= base && lane < cap) crow[lane] = 0ull;  // empty slots
    if (lane == 0) meta[wave_id] = wbase < nv ? tw : 0u;
  }
}


}  // namespace dsa
