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

// Eight fp4 (E2M1) codes per dword, times the block scale -> eight bf16
// values (exact: a code has two significant bits, the scale is a power of two).
__device__ __forceinline__ v8bf fp4x8_to_bf16(uint32_t w, float sc) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// E8M0 scale byte -> 2^(e - 127) as f32 (e = 0: the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return e == 0u ? __uint_as_float(0x00400000u) : __uint_as_float(e << 23);
}

// The key formats of the matrix-core indexer (dim 128, 16-entry tiles).
// Per lane (g, n) of a tile: its raw bytes of entry n, the four bf16 B
// operands widened from them exactly, and the entry's scale factor (fp8:
// the per-entry f32 scale; fp4: 1, the block scale is applied in the
// widening).  The query's A operands take the same dims: fp8 keys give lane
// g the 32 bytes 16g.. and 64 + 16g.. (two 16-byte chunks); fp4 keys give it
// dims 32g .. 32g + 31 (one chunk, one E8M0 scale).  Either way the four
// MFMAs of a tile sum each of the 128 products exactly once.
template <int kFmt>
struct KeyOps;

template <>
struct KeyOps<DSA_FP8_E4M3> {
  static constexpr int kBytes = 128;  // per entry
  struct Raw {
    uint4 lo, hi;
    float ks;
  };
  // kb: the sequence's keys; ksb: its per-entry scales; (msb unused)
  __device__ static Raw load(const uint8_t* kb, const float* ksb, const uint8_t*, int64_t j, int g) {
    Raw r;
    idx_load_chunks(kb, j, g, &r.lo, &r.hi);
    r.ks = ksb[j];
    return r;
  }
  __device__ static Raw zero() { return Raw{{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, 0.f}; }
  __device__ static void operands(const Raw& r, v8bf (&bo)[4]) {
    bo[0] = fp8x8_to_bf16(r.lo.x, r.lo.y);
    bo[1] = fp8x8_to_bf16(r.lo.z, r.lo.w);
    bo[2] = fp8x8_to_bf16(r.hi.x, r.hi.y);
    bo[3] = fp8x8_to_bf16(r.hi.z, r.hi.w);
  }
  __device__ static float scale(const Raw& r) { return r.ks; }
  // head n's fp8 query row (128 bytes) -> A operands for lane group g
  __device__ static void q_operands(const uint8_t* qrow, int g, v8bf (&a)[4]) {
    uint4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (qrow) {
      lo = reinterpret_cast<const uint4*>(qrow)[g];
      hi = reinterpret_cast<const uint4*>(qrow)[4 + g];
    }
    a[0] = fp8x8_to_bf16(lo.x, lo.y);
    a[1] = fp8x8_to_bf16(lo.z, lo.w);
    a[2] = fp8x8_to_bf16(hi.x, hi.y);
    a[3] = fp8x8_to_bf16(hi.z, hi.w);
  }
};

template <>
struct KeyOps<DSA_FP4_E2M1> {
  static constexpr int kBytes = 64;
  struct Raw {
    uint4 c;     // dims 32g .. 32g + 31 of the entry
    uint32_t e;  // their E8M0 scale byte
  };
  // kb: the sequence's keys; msb: its scale bytes [e_cap, 4]
  __device__ static Raw load(const uint8_t* kb, const float*, const uint8_t* msb, int64_t j, int g) {
    return Raw{idx4_load_chunk(kb, j, g), msb[j * 4 + g]};
  }
  __device__ static Raw zero() { return Raw{{0u, 0u, 0u, 0u}, 0u}; }
  __device__ static void operands(const Raw& r, v8bf (&bo)[4]) {
    const float sc = e8m0_to_f32(r.e);
    bo[0] = fp4x8_to_bf16(r.c.x, sc);
    bo[1] = fp4x8_to_bf16(r.c.y, sc);
    bo[2] = fp4x8_to_bf16(r.c.z, sc);
    bo[3] = fp4x8_to_bf16(r.c.w, sc);
  }
  __device__ static float scale(const Raw&) { return 1.f; }
  __device__ static void q_operands(const uint8_t* qrow, int g, v8bf (&a)[4]) {
    uint4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (qrow) {
      lo = reinterpret_cast<const uint4*>(qrow)[2 * g];
      hi = reinterpret_cast<const uint4*>(qrow)[2 * g + 1];
    }
    a[0] = fp8x8_to_bf16(lo.x, lo.y);
    a[1] = fp8x8_to_bf16(lo.z, lo.w);
    a[2] = fp8x8_to_bf16(hi.x, hi.y);
    a[3] = fp8x8_to_bf16(hi.z, hi.w);
  }
};

// Where a sequence's keys are: dense, its own tiles (kb), scales (ksb) and
// MX scale bytes (msb), entry j at row j; paged, the pools, entry j at its
// pool row.
struct KeySrc {
  const uint8_t* kb;
  const float* ksb;
  const uint8_t* msb;
  PageMap pm;
  int b;
  uint32_t* status;
  __device__ int64_t row(int64_t j) const { return pm.table ? paged_row(pm, b, j, status) : j; }
};

template <int kFmt>
__device__ __forceinline__ KeySrc key_src(const uint8_t* keys, const float* k_scale,
                                          const uint8_t* k_mx, const PageMap& pm, int b,
                                          int64_t e_cap, uint32_t* status) {
  if (pm.table) return KeySrc{keys, k_scale, k_mx, pm, b, status};
  return KeySrc{keys + static_cast<int64_t>(b) * idx_e_pad(e_cap) * KeyOps<kFmt>::kBytes,
                k_scale ? k_scale + static_cast<int64_t>(b) * e_cap : nullptr,
                k_mx ? k_mx + static_cast<int64_t>(b) * e_cap * 4 : nullptr, pm, b, status};
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
// 4g .. 4g+3; B = the entry's operands.  Every lane of column n gets the sum
// over heads.
__device__ __forceinline__ float exact_tile_score(const v8bf (&aq)[4], const float (&wv)[4],
                                                  const v8bf (&bo)[4]) {
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[c], bo[c], acc, 0, 0, 0);
  float v = wv[0] * fmaxf(acc[0], 0.f) + wv[1] * fmaxf(acc[1], 0.f) +
            wv[2] * fmaxf(acc[2], 0.f) + wv[3] * fmaxf(acc[3], 0.f);
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// A row's exact operands: its heads (lane = head n) widened to bf16 in the
// key format's dim assignment, and w * q_scale for heads 4g .. 4g+3.
template <int kFmt>
__device__ __forceinline__ void exact_row_operands(const uint8_t* q, const float* q_scale,
                                                   const float* w, int64_t row, int Hi,
                                                   v8bf (&aq)[4], float (&wv)[4]) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  KeyOps<kFmt>::q_operands(n < Hi ? q + (row * Hi + n) * 128 : nullptr, g, aq);
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

// The exact score of entry j (j < nv, else 0) for lane (g, n) of a tile:
// kBatch entries' loads go out before the first product.
template <int kFmt, int kBatch>
__device__ __forceinline__ void exact_scores(const v8bf (&aq)[4], const float (&wv)[4],
                                             const KeySrc& src, const int64_t (&j)[kBatch],
                                             int64_t nv, float (&sc)[kBatch]) {
  using K = KeyOps<kFmt>;
  const int g = (threadIdx.x & 63) >> 4;
  typename K::Raw r[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; ++u)
    r[u] = j[u] < nv ? K::load(src.kb, src.ksb, src.msb, src.row(j[u]), g) : K::zero();
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    v8bf bo[4];
    K::operands(r[u], bo);
    sc[u] = exact_tile_score(aq, wv, bo) * K::scale(r[u]);
  }
}

// Exact scores of a row's first nv entries into srow (every wave of the
// workgroup takes every nwaves-th tile of 16 entries).
template <int kFmt>
__device__ __forceinline__ void score_row_exact(const v8bf (&aq)[4], const float (&wv)[4],
                                                const KeySrc& src, int64_t nv, float* srow,
                                                int nwaves) {
  // four tiles' loads in flight per wave and round
  constexpr int kBatch = 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 15, g = lane >> 4;
  for (int64_t t0 = wave; t0 * 16 < nv; t0 += kBatch * nwaves) {
    int64_t j[kBatch];
    float sc[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) j[u] = (t0 + static_cast<int64_t>(u) * nwaves) * 16 + n;
    exact_scores<kFmt, kBatch>(aq, wv, src, j, nv, sc);
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (g == 0 && j[u] < nv) srow[j[u]] = sc[u];
  }
}

// kEnt entries per workgroup, 4 waves of kEnt / 4.  With kCand the scores
// stay in registers (candidates and wave thresholds go out; a row whose
// certificate fails is re-scored by the final pass); without, every score
// is written to its row.
template <bool kCand, int kEnt, int kFmt = DSA_FP8_E4M3, bool kPaged = false>
__device__ __forceinline__ void index_stream_block(
    int bx, int nbx, int row, const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ keys, const float* __restrict__ k_scale,
    const uint8_t* __restrict__ k_mx, const int64_t* __restrict__ q_pos, int Tq, int Hi, int s,
    int S, int64_t e_cap, int64_t nv_cap, int64_t max_pos_end, float* __restrict__ scores,
    int64_t ld_scores, uint64_t* __restrict__ cand, uint32_t* __restrict__ meta, int cap,
    uint32_t* status, PageMap pm) {
  using K = KeyOps<kFmt>;
  const int b = row / Tq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int64_t e_begin = static_cast<int64_t>(bx) * kEnt;
  constexpr int kGroups = kEnt / 4 / 16;            // 16-entry groups per wave
  constexpr int kSteps = kGroups / 2;               // two groups per step
  constexpr int kKeep = kGroups / 4;                // keys kept per lane
  const int64_t wbase = e_begin + wave * (kEnt / 4);
  const KeySrc src = key_src<kFmt>(keys, k_scale, k_mx, pm, b, e_cap, status);
  // key loads: a ring of two slots of two groups; unconditional (clamped to
  // an entry that exists, masked later) so the compiler can count them.
  // Dense keys: both slots go out before the row's visible count is known
  // (clamped to the cache's capacity), and so do the query and weight loads,
  // so their latency overlaps that of the position load
  typename K::Raw kr[2][2];
  int64_t jmax = e_cap - 1;
  int32_t gblk = 0;
  auto load = [&](int slot, int gr) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t ent = min<int64_t>(wbase + (gr + u) * 16 + n, jmax);
      int64_t rw = ent;
      if constexpr (kPaged)
        rw = (static_cast<int64_t>(__builtin_amdgcn_readlane(gblk, gr + u)) << pm.shift) |
             (ent & ((int64_t{1} << pm.shift) - 1));
      kr[slot][u] = K::load(src.kb, src.ksb, src.msb, rw, g);
    }
  };
  const bool early = !kPaged && e_cap > 0;
  if (early) {
    load(0, 0);
    load(1, 2);
  }
  v8bf aq[4];
  K::q_operands(n < Hi ? q + (static_cast<int64_t>(row) * Hi + n) * 128 : nullptr, g, aq);
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
  const RowInfo ri = row_info(q_pos, row, s, S, nv_cap, max_pos_end, status, bx == 0 && tid == 0);
  const int64_t nv = ri.nv;
  // each lane keeps the keys of groups 4i + 2 (g & 1) + (g >> 1), i < kKeep
  uint32_t kk[kKeep] = {};
  if (wbase < nv) {
    jmax = nv - 1;
    // paged: lane l < kGroups holds the block of the wave's group l (16
    // entries never straddle a block), read once per wave; each load takes
    // its group's block id from that lane (the table is read only for
    // visible entries)
    if constexpr (kPaged)
      if (lane < kGroups)
        gblk = static_cast<int32_t>(
            paged_row(pm, b, min<int64_t>(wbase + lane * 16, jmax), status) >> pm.shift);
    if (!early) load(0, 0);
    float* srow = scores + static_cast<int64_t>(row) * ld_scores;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int sl = st & 1;
      if (st + 1 < kSteps && !(early && st == 0)) load(sl ^ 1, 2 * (st + 1));
      float part[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        v8bf bo[4];
        K::operands(kr[sl][u], bo);
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[c], bo[c], acc, 0, 0, 0);
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
      // (a select, not an index by u: a lane-dependent index into kr would
      // put the whole ring in scratch memory)
      const float sc = v * (u ? K::scale(kr[sl][1]) : K::scale(kr[sl][0]));
      const int64_t ent = wbase + (2 * st + u) * 16 + n;
      const bool vis = ent < nv;
      if constexpr (!kCand)
        if ((g & 1) == 0 && vis) srow[ent] = sc;
      if constexpr (kCand)
        if ((g & 1) == (st & 1)) kk[st >> 1] = vis ? order_key(sc) : 0u;
    }
  }
  if constexpr (kCand) {
    // wave candidates: the keys above the (cap+1)-th largest of the wave's
    // 256.  Each lane sorts its keys (descending) once, so a lane holding
    // the wave's maximum holds it first; the maximum is then taken cap + 1
    // times, each time one instance leaving the lowest lane that has it
    // (its keys move up one place)
    uint32_t work[kKeep];
#pragma unroll
    for (int i = 0; i < kKeep; ++i) work[i] = kk[i];
#pragma unroll
    for (int i = 0; i < kKeep; ++i)
#pragma unroll
      for (int j = 0; j + 1 < kKeep - i; ++j) {
        const uint32_t hi = max(work[j], work[j + 1]), lo = min(work[j], work[j + 1]);
        work[j] = hi;
        work[j + 1] = lo;
      }
    uint32_t next = 0;
    for (int it = 0; it <= cap; ++it) {
      const uint32_t m =
          static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(wave_max_u32(work[0]))));
      next = m;
      if (m == 0u || it == cap) break;
      const uint64_t bal = __ballot(work[0] == m);
      const bool me = lane == __ffsll(static_cast<long long>(bal)) - 1;
#pragma unroll
      for (int i = 0; i + 1 < kKeep; ++i) work[i] = me ? work[i + 1] : work[i];
      work[kKeep - 1] = me ? 0u : work[kKeep - 1];
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
