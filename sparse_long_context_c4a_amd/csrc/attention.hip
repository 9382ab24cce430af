// S5: sparse MQA attention with K = V and the inverse-RoPE epilogue.
//
// Row i (sequence b, position m) attends to the set
//   A(m) = { cache[b, j] : j in idx[i], j >= 0 } U { window token n : m-W <= n <= m-1 }
// ("DeepSeek DSA、DeepSeek V4与vLLM Hybrid KV Cache详解" 4.2-4.3 and 5.3;
// "DeepSeek V4 稀疏注意力完全解剖" 机制三 / 机制四).  Every head shares the same
// vectors (MQA), each vector is both key and value (机制一), one softmax runs
// over the whole set, and the head output is rotated back by R_m^{-1}
// (深潜: 为什么必须做 Inverse RoPE).
//
// The set is walked as a virtual list of k + W slots: slot a < k is idx[a],
// slot k + t is window position m - W + t.  A workgroup takes one row, a
// group of 16 heads and a contiguous run of slots; each tile of 16 vectors
// is staged once in LDS and used by all 16 heads for both the logits and
// the weighted sum (online softmax).  Runs are merged by k_attn_combine
// (log-sum-exp) unless one run covers the row.
#include "common.h"
#include "internal.h"

namespace dsa {
namespace {

constexpr int kHG = 16;       // heads per workgroup
constexpr int kTile = 16;     // vectors per LDS tile
constexpr int kThreads = 256; // 16 threads per head
constexpr int kMaxD = 1024;

struct AttnGeom {
  const int64_t* q_pos;
  int Tq, H, D, r;
  double base;
  double theta1;  // base^(-2 / r): the rotation's frequencies are its powers
  int64_t off;
  const int32_t* idx;
  int k;
  int64_t e_cap;
  int w_cap, W;
  const int64_t* chunk_pos0;
  int64_t chunk_len;
  float scale;
  int64_t max_pos_end;
  int slots_per_run, n_runs;
  const float* cs_tab;  // optional (cos, sin) of R_m per row, r floats per row
  uint32_t* status;
  int rows;
  // true: the attention kernel writes the final output (one run per row and
  // a bf16 / f32 output); false: it leaves partials for a combine kernel
  bool direct;
  float* out_scale;  // fp8 output: one scale per (row, head), else nullptr
  const float* cache_scale;  // fp8 cache: one scale per entry [B, e_cap], else nullptr
  PageMap ent, swa;          // paged cache entries and window tokens (tables nullptr: dense)
};

// Row of cache entry j (0 <= j < e_cap) of sequence b, and of window token n.
__device__ __forceinline__ int64_t cache_row(const AttnGeom& g, int b, int64_t j) {
  return entry_row(g.ent, b, j, g.e_cap, g.status);
}
__device__ __forceinline__ int64_t win_row(const AttnGeom& g, int b, int64_t n) {
  return window_row(g.swa, b, n, g.w_cap, g.status);
}

// Source of slot a of row `row`; nullptr if the slot is empty.
template <typename T>
__device__ __forceinline__ const T* slot_ptr(const AttnGeom& g, int row, int b, int64_t m,
                                             int a, const T* cache, const T* window,
                                             const T* chunk_win) {
  if (a < g.k) {
    const int32_t j = g.idx[static_cast<int64_t>(row) * g.k + a];
    if (j < 0 || j >= g.e_cap) return nullptr;
    return cache + cache_row(g, b, j) * g.D;
  }
  const int64_t n = m - g.W + (a - g.k);
  if (n < 0 || n >= m) return nullptr;
  if (chunk_win) {
    const int64_t c0 = g.chunk_pos0[b];
    if (n >= c0 && n - c0 < g.chunk_len)
      return chunk_win + (static_cast<int64_t>(b) * g.chunk_len + (n - c0)) * g.D;
  }
  return window + win_row(g, b, n) * g.D;
}

// Max and sum over the four 16-lane rows of a wave (lanes n, n + 16, n + 32,
// n + 48, every lane getting the result) with the gfx950 lane swaps:
// permlane16_swap(x, x) gives rows (r0, r0, r2, r2) and (r1, r1, r3, r3),
// permlane32_swap(x, x) the two halves; no LDS round trip.
__device__ __forceinline__ float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Largest value of x over the workgroup's NT threads (every thread calls it
// once; red holds one float per wave).
template <int NT>
__device__ __forceinline__ float block_max(float x, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) m = fmaxf(m, red[w]);
  return m;
}

// Token-wise fp8 output of one head ([P2] 融合点 2, with the quantisation of
// the decode KV): scale = max|o| / 448 over the head's D dims, code =
// e4m3fn(o / scale) rounded to nearest even; an all-zero head gets scale 0
// and zero codes.
__device__ __forceinline__ uint32_t fp8_code(float v, float sc) {
  return sc > 0.f ? f32_to_fp8(v / sc) : 0u;
}

// Generic (any D <= 1024, f32 or bf16) attention run.  Output: either the
// final rotated result (g.direct) or an un-normalised partial
// (max, sum, acc[D]) per head for k_attn_combine.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_attn_generic(
    AttnGeom g, const T* __restrict__ q, int rotate_q, const T* __restrict__ cache,
    const T* __restrict__ window, const T* __restrict__ chunk_win, T* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_acc, float* __restrict__ part_ml) {
  extern __shared__ float smem[];
  float* q_s = smem;                     // [kHG][D]
  float* v_s = q_s + kHG * g.D;          // [kTile][D]
  __shared__ float p_s[kHG][kTile];
  __shared__ float cs_s[kMaxD / 2][2];   // rotation table for position m
  __shared__ int valid_s[kTile];
  const int row = blockIdx.y, hg = blockIdx.x, run = blockIdx.z;
  const int b = row / g.Tq, tid = threadIdx.x;
  const int h_loc = tid / 16, sub = tid % 16;
  const int64_t m = g.q_pos[row];
  const bool ok = m >= 0 && m < g.max_pos_end;
  if (!ok && tid == 0 && hg == 0 && run == 0) set_status(g.status, DSA_DEVERR_POSITION);
  const int D = g.D, half = g.r / 2, first_rot = (D - g.r) / 2;
  for (int i = tid; i < half; i += kThreads) {
    float c = 1.f, s = 0.f;
    if (ok) rope_cs1(m + g.off, i, g.theta1, &c, &s);
    cs_s[i][0] = c;
    cs_s[i][1] = s;
  }
  __syncthreads();
  // load (and rotate) the 16 query heads of this group
  for (int i = tid; i < kHG * D / 2; i += kThreads) {
    const int hh = i / (D / 2), pr = i % (D / 2);
    const int h = hg * kHG + hh;
    float a0 = 0.f, a1 = 0.f;
    if (h < g.H) {
      const int64_t o = (static_cast<int64_t>(row) * g.H + h) * D + 2 * pr;
      a0 = load_as_f32(q, o);
      a1 = load_as_f32(q, o + 1);
      if (rotate_q && pr >= first_rot) {
        const float c = cs_s[pr - first_rot][0], s = cs_s[pr - first_rot][1];
        const float t0 = a0 * c - a1 * s, t1 = a0 * s + a1 * c;
        a0 = t0;
        a1 = t1;
        if constexpr (sizeof(T) == 2) {  // the rotated query is held in bf16
          a0 = bf16_to_f32(f32_to_bf16(a0));
          a1 = bf16_to_f32(f32_to_bf16(a1));
        }
      }
    }
    q_s[hh * D + 2 * pr] = a0;
    q_s[hh * D + 2 * pr + 1] = a1;
  }
  const int total = g.k + g.W;
  const int a_begin = run * g.slots_per_run;
  const int a_end = min(total, a_begin + g.slots_per_run);
  const int dpt = D / 16;  // dims per thread in the accumulate phase
  float acc[kMaxD / 16];
#pragma unroll
  for (int i = 0; i < kMaxD / 16; ++i) acc[i] = 0.f;
  float run_max = -INFINITY, run_sum = 0.f;
  static_assert(kThreads == 16 * kTile, "one 16-thread group per staged vector");
  for (int a0 = a_begin; a0 < a_end; a0 += kTile) {
    __syncthreads();
    {
      // stage the tile: thread group e = tid / 16 fetches vector e (its slot's
      // index, then its D values, 16 threads side by side), so a tile costs
      // two memory round trips
      const int e = tid / 16, dl = tid % 16;
      const int a = a0 + e;
      const T* src = (ok && a < a_end) ? slot_ptr<T>(g, row, b, m, a, cache, window, chunk_win)
                                       : nullptr;
      if (dl == 0) valid_s[e] = src != nullptr;
#pragma unroll 8
      for (int d = dl; d < D; d += 16) v_s[e * D + d] = src ? load_as_f32(src, d) : 0.f;
    }
    __syncthreads();
    // logits: thread (h_loc, sub) -> head h_loc, vector sub
    float lg = -INFINITY;
    if (valid_s[sub]) {
      float d0 = 0.f;
      for (int d = 0; d < D; ++d) d0 = fmaf(q_s[h_loc * D + d], v_s[sub * D + d], d0);
      lg = d0 * g.scale;
    }
    float tmax = lg;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o, 16));
    const float new_max = fmaxf(run_max, tmax);
    const float p = (lg == -INFINITY) ? 0.f : expf(lg - new_max);
    const float corr = (run_max == -INFINITY) ? 0.f : expf(run_max - new_max);
    float psum = p;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) psum += __shfl_xor(psum, o, 16);
    run_sum = run_sum * corr + psum;
    run_max = new_max;
    p_s[h_loc][sub] = p;
    __syncthreads();
    // accumulate: thread (h_loc, sub) owns dims sub + 16 i
    for (int i = 0; i < dpt; ++i) {
      const int d = sub + 16 * i;
      float s = acc[i] * corr;
      for (int e = 0; e < kTile; ++e) s = fmaf(p_s[h_loc][e], v_s[e * D + d], s);
      acc[i] = s;
    }
  }
  const int h = hg * kHG + h_loc;
  const bool hv = h < g.H;
  if (g.direct) {
    const float inv = run_sum > 0.f ? 1.0f / run_sum : 0.f;
    const int64_t o = (static_cast<int64_t>(row) * g.H + h) * D;
    __syncthreads();
    for (int i = 0; i < dpt; ++i) v_s[h_loc * D + sub + 16 * i] = acc[i] * inv;  // reuse as staging
    __syncthreads();
    for (int pr = sub; pr < D / 2; pr += 16) {
      float a0 = v_s[h_loc * D + 2 * pr], a1 = v_s[h_loc * D + 2 * pr + 1];
      if (pr >= first_rot) {  // R_m^{-1}: rotate by -angle
        const float c = cs_s[pr - first_rot][0], s = cs_s[pr - first_rot][1];
        const float t0 = a0 * c + a1 * s, t1 = -a0 * s + a1 * c;
        a0 = t0;
        a1 = t1;
      }
      if (hv) {
        store_from_f32(out, o + 2 * pr, a0);
        store_from_f32(out, o + 2 * pr + 1, a1);
      }
    }
    if (lse && sub == 0 && hv)
      lse[static_cast<int64_t>(row) * g.H + h] = run_sum > 0.f ? run_max + logf(run_sum) : -INFINITY;
  } else if (hv) {
    const int64_t pi = (static_cast<int64_t>(row) * g.n_runs + run) * g.H + h;
    for (int i = 0; i < dpt; ++i) part_acc[pi * D + sub + 16 * i] = acc[i];
    if (sub == 0) {
      part_ml[2 * pi] = run_max;
      part_ml[2 * pi + 1] = run_sum;
    }
  }
}

// Merge the runs of one (row, head) and apply R_m^{-1}: thread -> dim pairs
// tid and tid + 256 (D <= 1024), the partials of up to kGCombR runs loaded
// per memory round trip, merged with a running log-sum-exp.
constexpr int kGCombR = 8;

template <typename T>
__global__ __launch_bounds__(256) void k_attn_combine(AttnGeom g, const float* __restrict__ part_acc,
                                                      const float* __restrict__ part_ml,
                                                      void* __restrict__ out_v,
                                                      float* __restrict__ lse) {
  __shared__ float red[4];
  const int row = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
  const int64_t m = g.q_pos[row];
  const bool ok = m >= 0 && m < g.max_pos_end;
  const int D = g.D, first_rot = (D - g.r) / 2, npairs = D / 2;
  const int64_t p0 = static_cast<int64_t>(row) * g.n_runs;
  float M = -INFINITY, L = 0.f;
  float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  for (int r0 = 0; r0 < g.n_runs; r0 += kGCombR) {
    float mr[kGCombR], lr[kGCombR], u[kGCombR][2][2];
#pragma unroll
    for (int q = 0; q < kGCombR; ++q) {
      // an empty run left max -inf, sum 0 and acc 0; runs past the end are empty
      mr[q] = -INFINITY;
      lr[q] = 0.f;
#pragma unroll
      for (int k = 0; k < 2; ++k) u[q][k][0] = u[q][k][1] = 0.f;
      if (r0 + q < g.n_runs) {
        const int64_t pi = (p0 + r0 + q) * g.H + h;
        mr[q] = part_ml[2 * pi];
        lr[q] = part_ml[2 * pi + 1];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int pr = tid + 256 * k;
          if (pr < npairs) {
            u[q][k][0] = part_acc[pi * D + 2 * pr];
            u[q][k][1] = part_acc[pi * D + 2 * pr + 1];
          }
        }
      }
    }
    float Mn = M;
#pragma unroll
    for (int q = 0; q < kGCombR; ++q) Mn = fmaxf(Mn, mr[q]);
    if (Mn == -INFINITY) continue;
    const float c = M == -INFINITY ? 0.f : expf(M - Mn);
    L *= c;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      acc[k][0] *= c;
      acc[k][1] *= c;
    }
#pragma unroll
    for (int q = 0; q < kGCombR; ++q) {
      const float wgt = mr[q] == -INFINITY ? 0.f : expf(mr[q] - Mn);
      L = fmaf(wgt, lr[q], L);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        acc[k][0] = fmaf(wgt, u[q][k][0], acc[k][0]);
        acc[k][1] = fmaf(wgt, u[q][k][1], acc[k][1]);
      }
    }
    M = Mn;
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  const int64_t o = (static_cast<int64_t>(row) * g.H + h) * D;
  float v[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int pr = tid + 256 * k;
    if (pr >= npairs) continue;
    float a0 = acc[k][0] * inv, a1 = acc[k][1] * inv;
    if (pr >= first_rot && ok) {
      float c, sn;
      rope_cs1(m + g.off, pr - first_rot, g.theta1, &c, &sn);
      const float t0 = a0 * c + a1 * sn, t1 = -a0 * sn + a1 * c;
      a0 = t0;
      a1 = t1;
    }
    v[k][0] = a0;
    v[k][1] = a1;
  }
  if (g.out_scale) {
    const float am = block_max<256>(
        fmaxf(fmaxf(fabsf(v[0][0]), fabsf(v[0][1])), fmaxf(fabsf(v[1][0]), fabsf(v[1][1]))), red);
    const float sc = am / 448.0f;
    uint8_t* out = static_cast<uint8_t*>(out_v);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int pr = tid + 256 * k;
      if (pr < npairs)
        *reinterpret_cast<uint16_t*>(out + o + 2 * pr) =
            static_cast<uint16_t>(fp8_code(v[k][0], sc) | (fp8_code(v[k][1], sc) << 8));
    }
    if (tid == 0) g.out_scale[static_cast<int64_t>(row) * g.H + h] = sc;
  } else {
    T* out = static_cast<T*>(out_v);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int pr = tid + 256 * k;
      if (pr >= npairs) continue;
      store_from_f32(out, o + 2 * pr, v[k][0]);
      store_from_f32(out, o + 2 * pr + 1, v[k][1]);
    }
  }
  if (lse && tid == 0)
    lse[static_cast<int64_t>(row) * g.H + h] = L > 0.f ? M + logf(L) : -INFINITY;
}

// ----------------------------------------------------------- MFMA path
// bf16, D = 512, heads in groups of 64.  A workgroup takes one row and a run
// of slots; each tile of 32 gathered vectors is staged once in LDS
// (row-major, 1056-byte pitch) and feeds both products:
//   S^T = K Q^T : A = 16 vectors x 32 dims (ds_read_b128 rows), B = the
//                 wave's rotated query heads held in registers;
//   O^T += V^T P^T : A = 16 dims x 32 vectors read with the gfx950 LDS
//                 transpose load (ds_read_b64_tr_b16), B = P straight from
//                 the S^T accumulator (each lane already holds, for its
//                 head, the probabilities of the entries it multiplies).
// K = V, so one staged copy serves both.  Online softmax per head; partial
// runs go to k_attn_combine, single runs apply R_m^{-1} and store.
constexpr int kMD = 512;
constexpr int kMTile = 32;
constexpr int kMPitch = 1056;  // bytes per staged vector (1024 + 32 of padding)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 10.0f;  // log2 headroom of the lazily raised running max
constexpr int kMRunSlots = 2048;
constexpr int kT8 = 64;  // vectors per staged tile of the eight-wave kernel  // slots per run of the MFMA path (indices held in LDS)

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;

__device__ __forceinline__ v8bf as_v8bf(uint4 v) { return __builtin_bit_cast(v8bf, v); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// Eight waves: wave w takes heads 16 (w % 4) .. +15 and dims 256 (w / 4) ..
// +255, so each wave holds half a head group's query and output registers
// (two waves per SIMD rather than one).  The logits are summed over the two
// dim halves through LDS (the two partners add the same two partial sums,
// so both see identical logits and probabilities); each wave then
// accumulates its half of the dims.  The run's cache indices are read into
// LDS once, so each tile's gather is one memory round trip; the next tile is
// gathered into registers while one computes.
template <bool kFinal>
__global__ __launch_bounds__(512) void k_attn_mfma8(
    AttnGeom g, const uint16_t* __restrict__ q, int rotate_q, const uint16_t* __restrict__ cache,
    const uint16_t* __restrict__ window, const uint16_t* __restrict__ chunk_win,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_acc,
    float* __restrict__ part_ml) {
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[kT8 * kMPitch];
  __shared__ float cs_s[kMD / 2][2];
  __shared__ int valid_s[kT8];
  __shared__ int32_t idx_s[kMRunSlots];
  __shared__ v4f spart[8][kT8 / 16][64];  // each wave's partial logits
  pin_scalars(g.q_pos, g.Tq, g.H, g.r, g.off, g.idx, g.k, g.e_cap, g.W, g.chunk_pos0, g.chunk_len,
              g.scale, g.max_pos_end, g.slots_per_run, g.n_runs, g.ent.table, g.swa.table, q,
              cache, window, chunk_win);
  const int row = blockIdx.y, hq = blockIdx.x, run = blockIdx.z;
  const int b = row / g.Tq, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, gq = lane >> 4, hgw = wave & 3, dh = wave >> 2;
  const int64_t m = g.q_pos[row];
  const bool ok = m >= 0 && m < g.max_pos_end;
  if (!ok && tid == 0 && hq == 0 && run == 0) set_status(g.status, DSA_DEVERR_POSITION);
  const int half = g.r / 2, rot0 = kMD - g.r;
  const int total = g.k + g.W;
  const int a_begin = run * g.slots_per_run;
  const int a_end = min(total, a_begin + g.slots_per_run);
  // the run's cache indices (at most kMRunSlots = 4 x 512) are loaded into
  // registers and stored to LDS after the rotation table's arithmetic, which
  // covers their latency
  int32_t ix[kMRunSlots / 512];
  const int a_idx = min(a_end, g.k);
#pragma unroll
  for (int u = 0; u < kMRunSlots / 512; ++u) {
    const int a = a_begin + tid + 512 * u;
    ix[u] = a < a_idx ? g.idx[static_cast<int64_t>(row) * g.k + a] : -1;
  }
  const int64_t c0 = chunk_win ? g.chunk_pos0[b] : 0;
  for (int i = tid; i < half; i += 512) {
    float c = 1.f, sn = 0.f;
    if (ok) rope_cs1(m + g.off, i, g.theta1, &c, &sn);
    cs_s[i][0] = c;
    cs_s[i][1] = sn;
  }
#pragma unroll
  for (int u = 0; u < kMRunSlots / 512; ++u) {
    const int a = a_begin + tid + 512 * u;
    if (a < a_idx) idx_s[a - a_begin] = ix[u];
  }
  __syncthreads();
  // query head h as the B operand, this wave's dim half: chunks c = 8 dh +
  // cc, dims 32 c + 8 gq + (0..7)
  const int h = hq * 64 + hgw * 16 + n;
  const uint16_t* qrow0 = q + (static_cast<int64_t>(row) * g.H + h) * kMD;
  v8bf qb[8];
  {
    const uint16_t* qrow = qrow0;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const int d0 = 32 * (8 * dh + cc) + 8 * gq;
      uint4 raw = *reinterpret_cast<const uint4*>(qrow + d0);
      if (rotate_q && d0 + 8 > rot0) {
        uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int d = d0 + 2 * p;
          if (d >= rot0) {
            const float a0 = bf16_to_f32(static_cast<uint16_t>(wd[p] & 0xffffu));
            const float a1 = bf16_to_f32(static_cast<uint16_t>(wd[p] >> 16));
            const float cc2 = cs_s[(d - rot0) / 2][0], ss = cs_s[(d - rot0) / 2][1];
            wd[p] = pack_bf16x2(a0 * cc2 - a1 * ss, a0 * ss + a1 * cc2);
          }
        }
        raw = uint4{wd[0], wd[1], wd[2], wd[3]};
      }
      qb[cc] = as_v8bf(raw);
    }
  }
  auto src_of = [&](int a) -> const uint16_t* {
    if (!ok || a >= a_end) return nullptr;
    if (a < g.k) {
      const int32_t j = idx_s[a - a_begin];
      if (j < 0 || j >= g.e_cap) return nullptr;
      return cache + cache_row(g, b, j) * kMD;
    }
    const int64_t nn = m - g.W + (a - g.k);
    if (nn < 0 || nn >= m) return nullptr;
    if (chunk_win && nn >= c0 && nn - c0 < g.chunk_len)
      return chunk_win + (static_cast<int64_t>(b) * g.chunk_len + (nn - c0)) * kMD;
    return window + win_row(g, b, nn) * kMD;
  };
  v4f o[16];
#pragma unroll
  for (int db = 0; db < 16; ++db) o[db] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float scale2 = g.scale * kLog2e;
  // staging: thread t -> vector t / 8 of the tile, 16-byte chunks 8 j + t % 8
  const int se = tid >> 3, sc = tid & 7;
  uint4 pre[8];
  int valid_next = 0;
  {
    const uint16_t* src = src_of(a_begin + se);
    valid_next = src != nullptr;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      pre[j] = src ? reinterpret_cast<const uint4*>(src)[j * 8 + sc] : uint4{0u, 0u, 0u, 0u};
  }
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const int te = (lane & 15) >> 2, tq = lane & 3;
  constexpr int kNB = kT8 / 16;  // 16-vector blocks per tile
  for (int a0 = a_begin; a0 < a_end; a0 += kT8) {
    __syncthreads();  // the previous tile is no longer read
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<uint4*>(v_lds + se * kMPitch + (j * 8 + sc) * 16) = pre[j];
    if (sc == 0) valid_s[se] = valid_next;
    // the next tile's gather goes out while this one computes, one load per
    // step of the logits products: issued together, the eight waves' loads
    // queue at the texture unit (64 bytes a cycle) and hold up the products.
    // Its sources are found while the barrier waits (idx_s is not written
    // again).
    // (after the last tile the loads read the query row and are dropped)
    const bool pf = a0 + kT8 < a_end;
    const uint16_t* nsrc = pf ? src_of(a0 + kT8 + se) : nullptr;
    if (pf) valid_next = nsrc != nullptr;
    const uint4* lsrc = reinterpret_cast<const uint4*>(nsrc ? nsrc : qrow0);
    __syncthreads();
    // partial S^T over this wave's dims: block i holds vectors 16 i .. +15
    v4f sv[kNB];
#pragma unroll
    for (int i = 0; i < kNB; ++i) sv[i] = v4f{0.f, 0.f, 0.f, 0.f};
    v8bf kv[8][kNB];
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const int off = (32 * (8 * dh + cc) + 8 * gq) * 2;
#pragma unroll
      for (int i = 0; i < kNB; ++i)
        kv[cc][i] = as_v8bf(*reinterpret_cast<const uint4*>(v_lds + (16 * i + n) * kMPitch + off));
    }
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const uint4 t = lsrc[cc * 8 + sc];
      pre[cc] = nsrc ? t : uint4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < kNB; ++i)
        sv[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv[cc][i], qb[cc], sv[i], 0, 0, 0);
    }
    // issue order: the K fragments two steps ahead of their products, one
    // gather load per step
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kNB, 0);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, kNB, 0);
      if (cc < 6) __builtin_amdgcn_sched_group_barrier(0x100, kNB, 0);
    }
    // the first weighted-sum step's V^T fragments (the tile stays in LDS
    // until the next tile's first barrier): read now, so that they land while
    // the partial logits are exchanged and the softmax runs
    lds_u8* const lds_base = (lds_u8*)v_lds;
    v4s lo0[16], hi0[16];
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      lo0[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4s_ptr)(lds_base + (4 * gq + te) * kMPitch + tq * 8 + dh * 512 + db * 32));
      hi0[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4s_ptr)(lds_base + (16 + 4 * gq + te) * kMPitch + tq * 8 + dh * 512 + db * 32));
    }
#pragma unroll
    for (int i = 0; i < kNB; ++i) spart[wave][i][lane] = sv[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kNB; ++i) sv[i] += spart[wave ^ 4][i][lane];
    // log2 units; the running max is raised lazily: the weights
    // exp2(x - m_run) may reach 2^kLazy before the accumulators are rescaled,
    // so most tiles need no rescale
    float x[4 * kNB];
#pragma unroll
    for (int i = 0; i < kNB; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        x[4 * i + e] = valid_s[16 * i + 4 * gq + e] ? sv[i][e] * scale2 : -INFINITY;
    float tmax = x[0];
#pragma unroll
    for (int i = 1; i < 4 * kNB; ++i) tmax = fmaxf(tmax, x[i]);
    tmax = rows_max(tmax);
    if (__any(tmax > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, tmax);
      const float corr = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= corr;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < 16; ++db) o[db] *= corr;
    }
    float p[4 * kNB], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4 * kNB; ++i) {
      p[i] = (x[i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(x[i] - m_run);
      psum += p[i];
    }
    psum = rows_sum(psum);
    l_run += psum;
    // O^T += V^T P^T over this wave's dims, 32 vectors per product: P of
    // blocks 2 u and 2 u + 1 is the B operand
#pragma unroll
    for (int u = 0; u < kNB / 2; ++u) {
      const v8bf pb = {static_cast<__bf16>(p[8 * u + 0]), static_cast<__bf16>(p[8 * u + 1]),
                       static_cast<__bf16>(p[8 * u + 2]), static_cast<__bf16>(p[8 * u + 3]),
                       static_cast<__bf16>(p[8 * u + 4]), static_cast<__bf16>(p[8 * u + 5]),
                       static_cast<__bf16>(p[8 * u + 6]), static_cast<__bf16>(p[8 * u + 7])};
      if (u == 0) {
#pragma unroll
        for (int db = 0; db < 16; ++db) {
          const v8bf va =
              __builtin_bit_cast(v8bf, __builtin_shufflevector(lo0[db], hi0[db], 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[db], 0, 0, 0);
        }
        continue;
      }
      lds_u8* r_lo = lds_base + (32 * u + 4 * gq + te) * kMPitch + tq * 8 + dh * 512;
      lds_u8* r_hi = lds_base + (32 * u + 16 + 4 * gq + te) * kMPitch + tq * 8 + dh * 512;
      v4s lo[16], hi[16];
#pragma unroll
      for (int db = 0; db < 16; ++db) {
        lo[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(r_lo + db * 32));
        hi[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(r_hi + db * 32));
      }
#pragma unroll
      for (int db = 0; db < 16; ++db) {
        const v8bf va = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo[db], hi[db], 0, 1, 2, 3, 4, 5, 6, 7));
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[db], 0, 0, 0);
      }
      // issue order: the V^T fragments four products ahead
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int db = 0; db < 16; ++db) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (db < 12) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
  }
  // lane holds O^T[dims 256 dh + 16 db + 4 gq + i][head h]
  if constexpr (kFinal) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    uint16_t* orow = out + (static_cast<int64_t>(row) * g.H + h) * kMD;
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      const int d = 256 * dh + 16 * db + 4 * gq;
      float v[4] = {o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv};
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const int dd = d + 2 * pr;
        if (dd >= rot0) {  // R_m^{-1}
          const float cc2 = cs_s[(dd - rot0) / 2][0], ss = cs_s[(dd - rot0) / 2][1];
          const float a0 = v[2 * pr], a1 = v[2 * pr + 1];
          v[2 * pr] = a0 * cc2 + a1 * ss;
          v[2 * pr + 1] = -a0 * ss + a1 * cc2;
        }
      }
      *reinterpret_cast<uint2*>(orow + d) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
    if (lse && gq == 0 && dh == 0)
      lse[static_cast<int64_t>(row) * g.H + h] =
          l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  } else {
    // the run's own attention output (normalised by its sum), rounded to
    // bf16 like the layer's output, and its (max, sum) in f32: half the
    // bytes of f32 accumulators for the merge to read
    const int64_t pi = (static_cast<int64_t>(row) * g.n_runs + run) * g.H + h;
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    uint16_t* prow = reinterpret_cast<uint16_t*>(part_acc) + pi * kMD;
#pragma unroll
    for (int db = 0; db < 16; ++db)
      *reinterpret_cast<uint2*>(prow + 256 * dh + 16 * db + 4 * gq) =
          uint2{pack_bf16x2(o[db][0] * inv, o[db][1] * inv), pack_bf16x2(o[db][2] * inv, o[db][3] * inv)};
    if (gq == 0 && dh == 0) {
      part_ml[2 * pi] = m_run * kLn2;  // natural-log units for the merge
      part_ml[2 * pi + 1] = l_run;
    }
  }
}

// ------------------------------------------------------ decode-shaped path
// bf16, D = 512, heads in groups of 16, few rows.  A workgroup takes one
// row, 16 heads and a run of slots; its kDecWaves waves take interleaved
// groups of 32 slots.  Each wave gathers its own 32 vectors (16 bytes per
// lane of each, through registers into its LDS tile) and computes S^T =
// K Q^T for the 16 heads; the waves agree on each step's max per head and
// leave their probabilities in LDS; then wave w accumulates O^T += V^T P^T
// over dims kWD w .. +kWD-1 for all the step's tiles, so the waves never
// merge.  A row whose slots span several runs leaves one un-normalised
// partial (max, sum, acc in f32) per run, merged by k_attn_dcombine with the
// R_m table the run-0 workgroup leaves.  (Merging in the same launch by the
// last workgroup to arrive needs agent-scope release/acquire fences, whose
// L2 write-back and invalidate cost more than the second launch.)
//
// Workgroup order: the head groups of one (row, run) read the same vectors,
// so they are placed on one XCD (workgroup ids congruent mod 8; the
// dispatcher deals ids round-robin over the 8 XCDs) and share its L2: a
// block of 8 G ids holds 8 (row, run) pairs x G head groups.
constexpr int kDH = 16;                       // heads per workgroup
constexpr int kDStep = 32;                    // vectors per wave step
constexpr int kDWaveBytes = kDStep * kMPitch; // 33,792 B of LDS per wave
// waves (32-slot steps) per workgroup: measured at the c4a decode B=4
// workload, 4 (80 workgroups, each wave 128 of the dims) and 2 (160, 256
// dims each) give the same step time; longer runs (fewer workgroups) are
// slower: 5 runs of 128 slots 51.8 us per step, 3 of 256 54.8, 2 59.3, 1
// 64.8
constexpr int kDecWaves = 4;

// Source of slot a of row `row` given its cache index j (read by the caller
// for a < k); nullptr if the slot is empty.
template <bool kFp8>
__device__ __forceinline__ const uint16_t* dslot_ptr(const AttnGeom& g, int b, int64_t m, int a,
                                                     int32_t j, const uint16_t* cache,
                                                     const uint16_t* window,
                                                     const uint16_t* chunk_win) {
  if (a < g.k) {
    if (j < 0 || j >= g.e_cap) return nullptr;
    if constexpr (kFp8)  // one byte per dim
      return reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(cache) +
                                               cache_row(g, b, j) * kMD);
    return cache + cache_row(g, b, j) * kMD;
  }
  const int64_t n = m - g.W + (a - g.k);
  if (n < 0 || n >= m) return nullptr;
  if (chunk_win) {
    const int64_t c0 = g.chunk_pos0[b];
    if (n >= c0 && n - c0 < g.chunk_len)
      return chunk_win + (static_cast<int64_t>(b) * g.chunk_len + (n - c0)) * kMD;
  }
  return window + win_row(g, b, n) * kMD;
}

// Cache index of slot a for lane-parallel prefetch (only slots a < k have one).
__device__ __forceinline__ int32_t dslot_index(const AttnGeom& g, int row, int a, int a_end) {
  return (a < a_end && a < g.k) ? g.idx[static_cast<int64_t>(row) * g.k + a] : -1;
}

// Load one wave step's vectors into registers: lane l holds bytes
// [16 l, 16 l + 16) of vector v < 32 in stg[v] (a stand-in vector, whose
// probability will be zero, for empty slots).  Plain loads: at a few
// workgroups per chip the LDS DMA load takes about twice as long to land as
// these do.  Returns the ballot of non-empty slots.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint64_t gather_load(const uint16_t* src, const uint16_t* dummy,
                                                int lane, u32x4 (&stg)[kDStep]) {
  const uint64_t vmask = __ballot(lane < kDStep && src != nullptr);
  if (vmask == 0) return 0;
  if (src == nullptr) src = dummy;
  const uint64_t sp = reinterpret_cast<uint64_t>(src);
  const uint32_t sp_lo = static_cast<uint32_t>(sp), sp_hi = static_cast<uint32_t>(sp >> 32);
#pragma unroll
  for (int v = 0; v < kDStep; ++v) {
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(sp_lo, v));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(sp_hi, v));
    const uint64_t base = (static_cast<uint64_t>(hi) << 32) | lo;
    typedef __attribute__((address_space(1))) const u32x4 g_u32x4;
    stg[v] = *reinterpret_cast<g_u32x4*>(base + static_cast<uint64_t>(lane) * 16);
  }
  return vmask;
}

// Write the staged vectors to the wave's LDS tile (vector v at row v).
__device__ __forceinline__ void gather_store(const u32x4 (&stg)[kDStep], int lane, uint8_t* wl) {
#pragma unroll
  for (int v = 0; v < kDStep; ++v) *reinterpret_cast<u32x4*>(wl + v * kMPitch + lane * 16) = stg[v];
}

// The same for a step of fp8 cache entries (512 bytes each): one 16-byte
// load covers two vectors, lanes 0-31 vector 2u and lanes 32-63 vector
// 2u + 1, lane l holding the codes of dims 16 (l % 32) .. +15 in stg[u].
__device__ __forceinline__ uint64_t gather_load8(const uint16_t* src, const uint16_t* dummy,
                                                 int lane, u32x4 (&stg)[kDStep]) {
  const uint64_t vmask = __ballot(lane < kDStep && src != nullptr);
  if (vmask == 0) return 0;
  if (src == nullptr) src = dummy;
  const uint64_t sp = reinterpret_cast<uint64_t>(src);
  const uint32_t sp_lo = static_cast<uint32_t>(sp), sp_hi = static_cast<uint32_t>(sp >> 32);
  const bool upper = lane >= 32;
  const uint64_t off = static_cast<uint64_t>(lane & 31) * 16;
#pragma unroll
  for (int u = 0; u < kDStep / 2; ++u) {
    const uint32_t lo0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(sp_lo, 2 * u));
    const uint32_t hi0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(sp_hi, 2 * u));
    const uint32_t lo1 = static_cast<uint32_t>(__builtin_amdgcn_readlane(sp_lo, 2 * u + 1));
    const uint32_t hi1 = static_cast<uint32_t>(__builtin_amdgcn_readlane(sp_hi, 2 * u + 1));
    const uint64_t base = upper ? ((static_cast<uint64_t>(hi1) << 32) | lo1)
                                : ((static_cast<uint64_t>(hi0) << 32) | lo0);
    typedef __attribute__((address_space(1))) const u32x4 g_u32x4;
    stg[u] = *reinterpret_cast<g_u32x4*>(base + off);
  }
  return vmask;
}

// Eight fp8 e4m3fn codes -> eight bf16 (exact: bf16 holds every e4m3 value).
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
               __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
}

// Stage an fp8 step: the codes widened to bf16 (the entries' scales go on
// their logits and probabilities); an empty slot, whose stand-in bytes need
// not be finite as fp8, is staged as zeros.
__device__ __forceinline__ void gather_store8(const u32x4 (&stg)[kDStep], int lane, uint8_t* wl,
                                              uint64_t vmask) {
  const int c = lane & 31, hv = lane >> 5;
#pragma unroll
  for (int u = 0; u < kDStep / 2; ++u) {
    const int v = 2 * u + hv;
    u32x4 lo = fp8x8_to_bf16x8(stg[u].x, stg[u].y), hi = fp8x8_to_bf16x8(stg[u].z, stg[u].w);
    if (!((vmask >> v) & 1ull)) lo = hi = u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(wl + v * kMPitch + c * 32) = lo;
    *reinterpret_cast<u32x4*>(wl + v * kMPitch + c * 32 + 16) = hi;
  }
}

// Normalise and apply R_m^{-1} to dims 4 d4 .. 4 d4 + 3 of one head.
__device__ __forceinline__ void head_dims4(float4 acc, float L, int d4, int rot0, const float* cs,
                                           float (&v)[4]) {
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  v[0] = acc.x * inv;
  v[1] = acc.y * inv;
  v[2] = acc.z * inv;
  v[3] = acc.w * inv;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int d = 4 * d4 + 2 * p;
    if (d >= rot0) {
      const float c = cs[d - rot0], s = cs[d - rot0 + 1];
      const float a0 = v[2 * p], a1 = v[2 * p + 1];
      v[2 * p] = a0 * c + a1 * s;
      v[2 * p + 1] = -a0 * s + a1 * c;
    }
  }
}

__device__ __forceinline__ void store_head_dims4(float4 acc, float L, int d4, int rot0,
                                                 const float* cs, uint16_t* orow) {
  float v[4];
  head_dims4(acc, L, d4, rot0, cs, v);
  *reinterpret_cast<uint2*>(orow + 4 * d4) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// The same as fp8 codes with the head's scale: the 128 threads of the
// workgroup each hold 4 of the head's 512 dims and all call it.
__device__ __forceinline__ void store_head_dims4_fp8(float4 acc, float L, int d4, int rot0,
                                                     const float* cs, uint8_t* orow, float* scale,
                                                     float* red) {
  float v[4];
  head_dims4(acc, L, d4, rot0, cs, v);
  const float am = block_max<128>(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))), red);
  const float sc = am / 448.0f;
  *reinterpret_cast<uint32_t*>(orow + 4 * d4) = fp8_code(v[0], sc) | (fp8_code(v[1], sc) << 8) |
                                                (fp8_code(v[2], sc) << 16) | (fp8_code(v[3], sc) << 24);
  if (d4 == 0) *scale = sc;
}

// kFp8: the cache holds fp8 e4m3fn codes with one scale per entry (the
// pages' token-wise fp8 decode KV; k a multiple of 32, so a wave step is all
// cache or all window); the window stays bf16.  An entry's scale multiplies
// its logit and its probability in the weighted sum of code vectors.
// LDS of one run of the decode attention (NW waves).
template <int NW>
struct DecSmem {
  uint8_t dsm[NW * kDWaveBytes];  // each wave's staged tile of 32 vectors
  uint8_t q_s[kDH * kMPitch];     // rotated q, head n at row n
  float cs_s[kMD];                // (cos, sin) of pair i at 2i, 2i+1
  v8bf p_s[NW][64];               // each wave's probabilities, as the PV B operand
  float mx_s[NW][kDH];            // each wave's step max per head (log2 units)
  float ps_s[NW][kDH];            // each wave's step sum per head
  int vm_s[NW];                   // whether the wave staged a vector this step
};

// Slot sources of a run (slots numbered 0 .. count()-1): index(a) gives the
// cache index of a cache slot for lane-parallel prefetch (-1 otherwise),
// ptr<kFp8>(a, j) its vector (nullptr for an empty slot), is_cache(a)
// whether slot a is a cache entry (else a bf16 window token).
//
// RunSlots: slots a_begin .. a_end-1 of the row's virtual list (k selected
// indices, then the W window positions).
struct RunSlots {
  const AttnGeom* g;
  int row, b, a_begin, a_end;
  int64_t m;
  const uint16_t *cache, *window, *chunk_win;
  __device__ int count() const { return a_end - a_begin; }
  __device__ int32_t index(int a) const { return dslot_index(*g, row, a_begin + a, a_end); }
  template <bool kFp8>
  __device__ const uint16_t* ptr(int a, int32_t j) const {
    return dslot_ptr<kFp8>(*g, b, m, a_begin + a, j, cache, window, chunk_win);
  }
  __device__ bool is_cache(int a) const { return a_begin + a < g->k; }
};

// One run of the decode attention (NW waves of a workgroup, 16 heads hg of
// row `row`): the run's slots in steps of NW x 32 vectors.  In a step wave w
// stages and scores its own 32 vectors; the waves agree on each head's
// running max and share their probabilities through LDS; then wave w
// accumulates dims kWD w .. +kWD-1 (kWD = 512 / NW) over all the step's
// vectors, so the run ends with no merge of the waves.  The run's partial (or, with g.direct,
// the final rotated output) goes out from registers.
template <int NW, bool kFp8, typename Src>
__device__ __forceinline__ void decode_attn_run(
    const AttnGeom& g, int row, int hg, int run, const Src& src, const uint16_t* __restrict__ q,
    int rotate_q, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_acc, float* __restrict__ part_ml, float* __restrict__ cs_out,
    DecSmem<NW>& sm) {
  constexpr int kWD = kMD / NW;  // dims each wave accumulates
  static_assert(kWD % 16 == 0, "whole 16-dim blocks per wave");
  constexpr int NT = NW * 64, kSlotsPerIter = NW * kDStep;
  constexpr int kQPer = kDH * 64 / NT;  // 16-byte pieces of the query tile per thread
  uint8_t* dsm = sm.dsm;
  uint8_t* q_s = sm.q_s;
  float* cs_s = sm.cs_s;
  const int G = g.H / kDH;
  const int b = row / g.Tq, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, gq = lane >> 4;
  const int a_end = src.count();
  int a0 = wave * kDStep;
  // independent loads first: the first step's cache indices, the query
  // position, the 16 heads' query rows (piece c = tid + NT i: head c / 64,
  // dims 8 (c % 64) .. +7) and, when given, the R_m table
  int32_t jn = lane < kDStep ? src.index(a0 + lane) : -1;
  const int64_t m = g.q_pos[row];
  uint4 qraw[kQPer];
  {
    const uint4* qrows = reinterpret_cast<const uint4*>(q + (static_cast<int64_t>(row) * g.H + hg * kDH) * kMD);
#pragma unroll
    for (int i = 0; i < kQPer; ++i) qraw[i] = qrows[tid + NT * i];
  }
  const int half = g.r / 2, rot0 = kMD - g.r;
  const bool ok = m >= 0 && m < g.max_pos_end;
  if (!ok && tid == 0 && hg == 0 && run == 0) set_status(g.status, DSA_DEVERR_POSITION);
  uint8_t* wl = dsm + wave * kDWaveBytes;
  const uint16_t* dummy = q + static_cast<int64_t>(row) * g.H * kMD;
  // the first step's gather goes out before the set-up below; later steps
  // load at the top of their iteration
  uint64_t vmask0 = 0;
  float sig0 = 1.f;
  u32x4 stg0[kDStep];
  // an fp8 cache slot's scale (1 for window slots and without kFp8)
  auto slot_scale = [&](int a, const uint16_t* sp, int32_t j) -> float {
    if constexpr (kFp8)
      if (sp != nullptr && src.is_cache(a)) return g.cache_scale[cache_row(g, b, j)];
    return 1.f;
  };
  if (a0 < a_end) {
    const uint16_t* sp = (ok && a0 + lane < a_end && lane < kDStep)
                             ? src.template ptr<kFp8>(a0 + lane, jn)
                             : nullptr;
    sig0 = slot_scale(a0 + lane, sp, jn);
    vmask0 = (kFp8 && src.is_cache(a0)) ? gather_load8(sp, dummy, lane, stg0)
                                        : gather_load(sp, dummy, lane, stg0);
  }
  // (after the gather: its loads wait on every load issued before them)
  if (g.cs_tab)
    for (int i = tid; i < 2 * half; i += NT) cs_s[i] = g.cs_tab[static_cast<int64_t>(row) * g.r + i];
  if (!g.cs_tab)
    for (int i = tid; i < half; i += NT) {
      float c = 1.f, sn = 0.f;
      if (ok) rope_cs1(m + g.off, i, g.theta1, &c, &sn);
      cs_s[2 * i] = c;
      cs_s[2 * i + 1] = sn;
    }
  __syncthreads();
  if (cs_out && !g.cs_tab && run == 0 && hg == 0)
    for (int i = tid; i < 2 * half; i += NT) cs_out[static_cast<int64_t>(row) * g.r + i] = cs_s[i];
#pragma unroll
  for (int i = 0; i < kQPer; ++i) {
    const int c = tid + NT * i, d0 = 8 * (c & 63);
    uint4 raw = qraw[i];
    if (rotate_q && d0 + 8 > rot0) {
      uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int d = d0 + 2 * p;
        if (d >= rot0) {
          const float x0 = bf16_to_f32(static_cast<uint16_t>(wd[p] & 0xffffu));
          const float x1 = bf16_to_f32(static_cast<uint16_t>(wd[p] >> 16));
          const float cc = cs_s[d - rot0], ss = cs_s[d - rot0 + 1];
          wd[p] = pack_bf16x2(x0 * cc - x1 * ss, x0 * ss + x1 * cc);
        }
      }
      raw = uint4{wd[0], wd[1], wd[2], wd[3]};
    }
    *reinterpret_cast<uint4*>(q_s + (c >> 6) * kMPitch + 2 * d0) = raw;
  }
  __syncthreads();
  v4f o[kWD / 16];  // O^T[dims kWD wave + 16 db + 4 gq + i][head n]
#pragma unroll
  for (int db = 0; db < kWD / 16; ++db) o[db] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float scale2 = g.scale * kLog2e;
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const int te = (lane & 15) >> 2, tq = lane & 3;
  // one step (every wave of the workgroup, barriers inside): the wave's
  // staged vectors to its tile and their logits; the step's max per head
  // agreed through LDS (raised lazily: the weights exp2(x - m_run) may reach
  // 2^kLazy before the accumulators are rescaled); the probabilities shared
  // through LDS; then this wave's dims over every tile of the step
  auto step = [&](const u32x4 (&stg)[kDStep], uint64_t vmask, bool st8, float sig) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = -INFINITY;
    // the scale of this lane's vector i (4 gq + i, then 16 + 4 gq + i)
    auto sgi = [&](int i) -> float {
      if constexpr (kFp8) return __shfl(sig, (i < 4 ? 4 * gq + i : 12 + 4 * gq + i), 64);
      return 1.f;
    };
    if (vmask != 0) {
      // (a tile's empty slots hold the stand-in vector: finite, weight 0)
      if (kFp8 && st8)
        gather_store8(stg, lane, wl, vmask);
      else
        gather_store(stg, lane, wl);
      v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const int off = (32 * c + 8 * gq) * 2;
        const v8bf k0 = as_v8bf(*reinterpret_cast<const uint4*>(wl + n * kMPitch + off));
        const v8bf k1 = as_v8bf(*reinterpret_cast<const uint4*>(wl + (16 + n) * kMPitch + off));
        const v8bf qb = as_v8bf(*reinterpret_cast<const uint4*>(q_s + n * kMPitch + off));
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qb, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qb, s1, 0, 0, 0);
      }
      // log2 units (the lane exchanges run on every lane: outside the
      // selects below)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sa = sgi(i) * scale2, sb = sgi(4 + i) * scale2;
        x[i] = ((vmask >> (4 * gq + i)) & 1) ? s0[i] * sa : -INFINITY;
        x[4 + i] = ((vmask >> (16 + 4 * gq + i)) & 1) ? s1[i] * sb : -INFINITY;
      }
    }
    float tmax = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, x[i]);
    tmax = rows_max(tmax);
    if (gq == 0) sm.mx_s[wave][n] = tmax;
    if (lane == 0) sm.vm_s[wave] = vmask != 0;
    __syncthreads();  // tiles staged, maxima out
    float ms = sm.mx_s[0][n];
#pragma unroll
    for (int w = 1; w < NW; ++w) ms = fmaxf(ms, sm.mx_s[w][n]);
    // (the same values in every wave, so the same decision)
    if (ms > m_run + kLazy) {
      const float m_new = fmaxf(m_run, ms);
      const float corr = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= corr;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < kWD / 16; ++db) o[db] *= corr;
    }
    float p[8], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = (x[i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(x[i] - m_run);
      psum += p[i];
    }
    psum = rows_sum(psum);
    if (gq == 0) sm.ps_s[wave][n] = psum;
    if constexpr (kFp8)
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] *= sgi(i);  // the weighted sum of code vectors
    sm.p_s[wave][lane] = v8bf{static_cast<__bf16>(p[0]), static_cast<__bf16>(p[1]),
                              static_cast<__bf16>(p[2]), static_cast<__bf16>(p[3]),
                              static_cast<__bf16>(p[4]), static_cast<__bf16>(p[5]),
                              static_cast<__bf16>(p[6]), static_cast<__bf16>(p[7])};
    __syncthreads();  // probabilities and sums out
#pragma unroll
    for (int w = 0; w < NW; ++w) l_run += sm.ps_s[w][n];
    // O^T += V^T P^T over this wave's dims, one 32-vector product per tile
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (!sm.vm_s[w]) continue;  // (uniform)
      const v8bf pb = sm.p_s[w][lane];
      lds_u8* tile = (lds_u8*)(dsm + w * kDWaveBytes) + wave * kWD * 2;
      lds_u8* r_lo = tile + (4 * gq + te) * kMPitch + tq * 8;
      lds_u8* r_hi = tile + (16 + 4 * gq + te) * kMPitch + tq * 8;
#pragma unroll
      for (int db = 0; db < kWD / 16; ++db) {
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(r_lo + db * 32));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(r_hi + db * 32));
        const v8bf va = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[db], 0, 0, 0);
      }
    }
  };
  // the same number of steps in every wave (a wave past the run's end
  // stages nothing)
  const int nsteps = (a_end + kSlotsPerIter - 1) / kSlotsPerIter;
  if (nsteps > 0) {
    // next step's cache indices in flight during this step
    jn = (a0 + kSlotsPerIter < a_end && lane < kDStep) ? src.index(a0 + kSlotsPerIter + lane) : -1;
    step(stg0, vmask0, src.is_cache(a0), sig0);
    for (int st = 1; st < nsteps; ++st) {
      a0 += kSlotsPerIter;
      u32x4 stg[kDStep];
      const uint16_t* sp = (ok && a0 + lane < a_end && lane < kDStep)
                               ? src.template ptr<kFp8>(a0 + lane, jn)
                               : nullptr;
      const float sig = slot_scale(a0 + lane, sp, jn);
      const bool st8 = kFp8 && src.is_cache(a0);
      const uint64_t vmask = st8 ? gather_load8(sp, dummy, lane, stg)
                                 : gather_load(sp, dummy, lane, stg);
      const int nxt = a0 + kSlotsPerIter;
      jn = (nxt < a_end && lane < kDStep) ? src.index(nxt + lane) : -1;
      __syncthreads();  // every wave done with the previous step's tiles
      step(stg, vmask, st8, sig);
    }
  }
  // lane holds O^T[dims kWD wave + 16 db + 4 gq + i][head n]; m_run (log2
  // units) and l_run are the run's max and sum for head n
  const float M = m_run * kLn2, L = l_run;
  const int hh = hg * kDH + n;
  if (g.direct) {
    uint16_t* orow = out + (static_cast<int64_t>(row) * g.H + hh) * kMD;
#pragma unroll
    for (int db = 0; db < kWD / 16; ++db)
      store_head_dims4(float4{o[db][0], o[db][1], o[db][2], o[db][3]}, L,
                       kWD / 4 * wave + 4 * db + gq, rot0, cs_s, orow);
    if (lse && wave == 0 && gq == 0)
      lse[static_cast<int64_t>(row) * g.H + hh] = L > 0.f ? M + logf(L) : -INFINITY;
  } else {
    const int64_t pi = ((static_cast<int64_t>(row) * G + hg) * g.n_runs + run) * kDH + n;
#pragma unroll
    for (int db = 0; db < kWD / 16; ++db)
      *reinterpret_cast<float4*>(part_acc + pi * kMD + kWD * wave + 16 * db + 4 * gq) =
          float4{o[db][0], o[db][1], o[db][2], o[db][3]};
    if (wave == 0 && gq == 0) {
      part_ml[2 * pi] = M;
      part_ml[2 * pi + 1] = L;
    }
  }
}

template <int NW, bool kFp8>
__global__ __launch_bounds__(NW * 64) void k_attn_decode(
    AttnGeom g, const uint16_t* __restrict__ q, int rotate_q, const uint16_t* __restrict__ cache,
    const uint16_t* __restrict__ window, const uint16_t* __restrict__ chunk_win,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_acc,
    float* __restrict__ part_ml, float* __restrict__ cs_out) {
  __shared__ __attribute__((aligned(16))) DecSmem<NW> sm;
  // the fields the set-up reads, loaded in one batch: left to itself the
  // compiler spreads these kernel-argument loads over a chain of dependent
  // waits ahead of the first index load
  pin_scalars(g.q_pos, g.Tq, g.H, g.r, g.off, g.idx, g.k, g.e_cap, g.w_cap, g.W, g.chunk_pos0,
              g.chunk_len, g.scale, g.max_pos_end, g.slots_per_run, g.n_runs, g.cs_tab, g.rows,
              g.ent.table, g.swa.table, g.cache_scale, q, cache, window, chunk_win);
  const int G = g.H / kDH;
  const int id = blockIdx.x;
  const int pair = 8 * (id / (8 * G)) + (id & 7), hg = (id >> 3) % G;
  if (pair >= g.rows * g.n_runs) return;
  const int row = pair / g.n_runs, run = pair % g.n_runs;
  const int a_begin = run * g.slots_per_run;
  const RunSlots src{&g, row, row / g.Tq, a_begin, min(g.k + g.W, a_begin + g.slots_per_run),
                     g.q_pos[row], cache, window, chunk_win};
  decode_attn_run<NW, kFp8>(g, row, hg, run, src, q, rotate_q, out, lse, part_acc, part_ml, cs_out,
                            sm);
}

// Merge the runs of one (row, head) pair of heads of the decode-shaped path
// and apply R_m^{-1} (table left by the run-0 workgroup).  Workgroup ->
// (head blockIdx.x, row blockIdx.y), thread -> dims 4 tid .. +3.  The
// partials of up to kCombR runs are loaded together (one memory round
// trip), then merged with a running log-sum-exp; longer rows take several
// such rounds.
constexpr int kCombR = 16;

__global__ __launch_bounds__(128) void k_attn_dcombine(AttnGeom g, const float* __restrict__ part_acc,
                                                       const float* __restrict__ part_ml,
                                                       const float* __restrict__ cs_in,
                                                       void* __restrict__ out,
                                                       float* __restrict__ lse) {
  __shared__ float cs_s[kMD];
  __shared__ float red[2];
  const int row = blockIdx.y, tid = threadIdx.x;
  const int h = blockIdx.x, d4 = tid;
  const int hg = h / kDH, ch = h % kDH, G = g.H / kDH;
  const float* cs_src = g.cs_tab ? g.cs_tab : cs_in;
  // the R_m table into registers now, into LDS after the partials' loads
  // are out (a store to LDS here would wait for it first)
  float csv[kMD / 128];
#pragma unroll
  for (int i = 0; i < kMD / 128; ++i)
    csv[i] = tid + 128 * i < g.r ? cs_src[static_cast<int64_t>(row) * g.r + tid + 128 * i] : 0.f;
  const int64_t p0 = (static_cast<int64_t>(row) * G + hg) * g.n_runs;
  float M = -INFINITY, L = 0.f;
  float4 t = {0.f, 0.f, 0.f, 0.f};
  for (int r0 = 0; r0 < g.n_runs; r0 += kCombR) {
    const int nr = min(kCombR, g.n_runs - r0);
    // the runs' (max, sum) in one vector load, lane q holding run r0 + q's
    // (loaded per run as scalars, each waited on before the next is issued)
    const int ql = (tid & 63) < nr ? (tid & 63) : 0;
    const float2 mlv = reinterpret_cast<const float2*>(part_ml)[(p0 + r0 + ql) * kDH + ch];
    // an empty run left max -inf, sum 0 and acc 0; runs past the end are
    // empty.  Every partial's load goes out before any result is used.
    float mr[kCombR], lr[kCombR];
    float4 u[kCombR];
#pragma unroll
    for (int q = 0; q < kCombR; ++q) {
      u[q] = float4{0.f, 0.f, 0.f, 0.f};
      if (q < nr) u[q] = reinterpret_cast<const float4*>(part_acc + ((p0 + r0 + q) * kDH + ch) * kMD)[d4];
    }
#pragma unroll
    for (int q = 0; q < kCombR; ++q) {
      const float mq = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(mlv.x), q));
      const float lq = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(mlv.y), q));
      mr[q] = q < nr ? mq : -INFINITY;
      lr[q] = q < nr ? lq : 0.f;
    }
    float Mn = M;
#pragma unroll
    for (int q = 0; q < kCombR; ++q) Mn = fmaxf(Mn, mr[q]);
    if (Mn == -INFINITY) continue;
    const float c = M == -INFINITY ? 0.f : expf(M - Mn);
    L *= c;
    t.x *= c;
    t.y *= c;
    t.z *= c;
    t.w *= c;
#pragma unroll
    for (int q = 0; q < kCombR; ++q) {
      const float wgt = mr[q] == -INFINITY ? 0.f : expf(mr[q] - Mn);
      L = fmaf(wgt, lr[q], L);
      t.x = fmaf(wgt, u[q].x, t.x);
      t.y = fmaf(wgt, u[q].y, t.y);
      t.z = fmaf(wgt, u[q].z, t.z);
      t.w = fmaf(wgt, u[q].w, t.w);
    }
    M = Mn;
  }
#pragma unroll
  for (int i = 0; i < kMD / 128; ++i)
    if (tid + 128 * i < g.r) cs_s[tid + 128 * i] = csv[i];
  __syncthreads();
  const int64_t oh = static_cast<int64_t>(row) * g.H + h;
  if (g.out_scale)
    store_head_dims4_fp8(t, L, d4, kMD - g.r, cs_s, static_cast<uint8_t*>(out) + oh * kMD,
                         g.out_scale + oh, red);
  else
    store_head_dims4(t, L, d4, kMD - g.r, cs_s, static_cast<uint16_t*>(out) + oh * kMD);
  if (lse && d4 == 0) lse[static_cast<int64_t>(row) * g.H + h] = L > 0.f ? M + logf(L) : -INFINITY;
}

// Merge the runs of one (row, head) of the matrix-core path (partials
// (row, run, head): each run's normalised output o_r in bf16 and its max
// m_r and sum l_r, so out = sum_r e^(m_r - M) l_r o_r / sum_r e^(m_r - M) l_r)
// and apply R_m^{-1}: workgroup -> (head blockIdx.x, row blockIdx.y),
// thread -> dims 4 tid .. +3, up to kCombR runs' partials loaded per memory
// round trip.  The (cos, sin) of R_m come from the
// step's table when the caller has one, else are computed here.
__global__ __launch_bounds__(128) void k_attn_mcombine(AttnGeom g, const float* __restrict__ part_acc,
                                                       const float* __restrict__ part_ml,
                                                       void* __restrict__ out,
                                                       float* __restrict__ lse) {
  __shared__ float cs_s[kMD];
  __shared__ float red[2];
  const int row = blockIdx.y, h = blockIdx.x, tid = threadIdx.x, d4 = tid;
  // the (cos, sin) pairs i = tid + 128 j this thread stages: the step's
  // table loaded now (into LDS after the partials' loads are out), or
  // computed after the merge
  float cv[kMD / 256], sv[kMD / 256];
#pragma unroll
  for (int j = 0; j < kMD / 256; ++j) {
    const int i = tid + 128 * j;
    cv[j] = 1.f;
    sv[j] = 0.f;
    if (g.cs_tab && g.r >= 2) {  // (uniform; pairs past r / 2 read the last one, unused)
      const int ii = min(i, g.r / 2 - 1);
      cv[j] = g.cs_tab[static_cast<int64_t>(row) * g.r + 2 * ii];
      sv[j] = g.cs_tab[static_cast<int64_t>(row) * g.r + 2 * ii + 1];
    }
  }
  const int64_t p0 = static_cast<int64_t>(row) * g.n_runs;
  float M = -INFINITY, L = 0.f;
  float4 t = {0.f, 0.f, 0.f, 0.f};
  for (int r0 = 0; r0 < g.n_runs; r0 += kCombR) {
    const int nr = min(kCombR, g.n_runs - r0);
    // the runs' (max, sum) in one vector load, lane q holding run r0 + q's
    const int ql = (tid & 63) < nr ? (tid & 63) : 0;
    const float2 mlv = reinterpret_cast<const float2*>(part_ml)[(p0 + r0 + ql) * g.H + h];
    // an empty run left max -inf, sum 0 and acc 0; runs past the end are
    // empty.  Every partial's load goes out before any result is used.
    float mr[kCombR], lr[kCombR];
    uint2 u[kCombR];
    const uint16_t* pacc = reinterpret_cast<const uint16_t*>(part_acc);
#pragma unroll
    for (int q = 0; q < kCombR; ++q) {
      u[q] = uint2{0u, 0u};
      if (q < nr) u[q] = reinterpret_cast<const uint2*>(pacc + ((p0 + r0 + q) * g.H + h) * kMD)[d4];
    }
#pragma unroll
    for (int q = 0; q < kCombR; ++q) {
      const float mq = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(mlv.x), q));
      const float lq = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(mlv.y), q));
      mr[q] = q < nr ? mq : -INFINITY;
      lr[q] = q < nr ? lq : 0.f;
    }
    float Mn = M;
#pragma unroll
    for (int q = 0; q < kCombR; ++q) Mn = fmaxf(Mn, mr[q]);
    if (Mn == -INFINITY) continue;
    const float c = M == -INFINITY ? 0.f : expf(M - Mn);
    L *= c;
    t.x *= c;
    t.y *= c;
    t.z *= c;
    t.w *= c;
#pragma unroll
    for (int q = 0; q < kCombR; ++q) {
      const float wl = mr[q] == -INFINITY ? 0.f : expf(mr[q] - Mn) * lr[q];
      L += wl;
      t.x = fmaf(wl, bf16_to_f32(static_cast<uint16_t>(u[q].x & 0xffffu)), t.x);
      t.y = fmaf(wl, bf16_to_f32(static_cast<uint16_t>(u[q].x >> 16)), t.y);
      t.z = fmaf(wl, bf16_to_f32(static_cast<uint16_t>(u[q].y & 0xffffu)), t.z);
      t.w = fmaf(wl, bf16_to_f32(static_cast<uint16_t>(u[q].y >> 16)), t.w);
    }
    M = Mn;
  }
  {
    const int64_t m = g.q_pos[row];
    const bool ok = m >= 0 && m < g.max_pos_end;
#pragma unroll
    for (int jj = 0; jj < kMD / 256; ++jj) {
      const int i = tid + 128 * jj;
      if (i < g.r / 2) {
        if (!g.cs_tab && ok) rope_cs1(m + g.off, i, g.theta1, &cv[jj], &sv[jj]);
        cs_s[2 * i] = cv[jj];
        cs_s[2 * i + 1] = sv[jj];
      }
    }
  }
  __syncthreads();
  const int64_t oh = static_cast<int64_t>(row) * g.H + h;
  if (g.out_scale)
    store_head_dims4_fp8(t, L, d4, kMD - g.r, cs_s, static_cast<uint8_t*>(out) + oh * kMD,
                         g.out_scale + oh, red);
  else
    store_head_dims4(t, L, d4, kMD - g.r, cs_s, static_cast<uint16_t*>(out) + oh * kMD);
  if (lse && d4 == 0) lse[static_cast<int64_t>(row) * g.H + h] = L > 0.f ? M + logf(L) : -INFINITY;
}

struct Plan {
  bool mfma, dec;
  bool part;  // partials and a combine launch (several runs, or an fp8 output)
  int slots_per_run, n_runs;
  size_t off_acc, off_ml, off_cs, total;
};

Plan plan(const dsa_attn_args& a) {
  Plan p{};
  const int64_t rows = static_cast<int64_t>(a.n_seqs) * a.queries_per_seq;
  const int total = std::max(1, a.k + a.window_size);
  const bool bf16_512 = a.dtype == DSA_BF16 && a.dim == kMD && a.rope_dim <= kMD;
  // The 16-head decode kernel for few rows with short sets (it spreads a row
  // over four head-group workgroups per run); otherwise the 64-head
  // matrix-core kernel, which stages each vector once for all heads.
  // Measured (c4a decode, 640 slots): 4 rows 56 vs 62 us per step, 32 rows
  // 78 vs 63 us (attention + combine 46 vs 31); c128a decode (16 rows of
  // 8320 slots) 146 vs 89 us.
  const bool mfma_ok = bf16_512 && a.heads % 64 == 0;
  const bool dec_ok = bf16_512 && a.heads % kDH == 0 && rows * (a.heads / kDH) <= 2048;
  // (an fp8 cache is read by the decode kernel only)
  p.dec = dec_ok && (a.cache_fp8 || !mfma_ok || (total < 4096 && rows * (a.heads / 64) < 16));
  p.mfma = !p.dec && mfma_ok;
  if (p.dec) {
    // about 1024 workgroups: runs of whole NW x 32-slot iterations
    const int64_t pairs = rows * (a.heads / kDH);
    const int64_t iters_total = ceil_div(total, kDecWaves * kDStep);
    const int64_t rmax = std::max<int64_t>(1, ceil_div(1024, pairs));
    const int64_t iters = ceil_div(iters_total, rmax);
    p.slots_per_run = static_cast<int>(iters * kDecWaves * kDStep);
    p.n_runs = static_cast<int>(ceil_div(total, p.slots_per_run));
  } else if (p.mfma) {
    // about 256 workgroups, one per compute unit (the kernel's LDS admits
    // one), at least two tiles per run: splitting a row further multiplies
    // the partials the combine reads (c128a decode, 16 rows of 8320 slots:
    // 89 us per step at 256, 110 at 512, 164 at 1024, 106 at 128)
    const int64_t hq = a.heads / 64;
    const int tiles = static_cast<int>(ceil_div(total, kMTile));
    int64_t runs = ceil_div(256, std::max<int64_t>(1, rows * hq));
    runs = std::max<int64_t>(1, std::min<int64_t>(runs, ceil_div(tiles, 2)));
    runs = std::max<int64_t>(runs, ceil_div(tiles, kMRunSlots / kMTile));  // indices fit LDS
    const int tpr = static_cast<int>(ceil_div(tiles, runs));
    p.slots_per_run = tpr * kMTile;
    p.n_runs = static_cast<int>(ceil_div(tiles, tpr));
  } else {
    const int64_t hgroups = ceil_div(a.heads, kHG);
    // enough workgroups to cover the chip (~1024), runs of whole 16-slot
    // tiles (a few rows: one tile per run, so the runs run side by side)
    int64_t want = ceil_div(1024, std::max<int64_t>(1, rows * hgroups));
    int spr = static_cast<int>(ceil_div(total, std::max<int64_t>(1, want)));
    spr = std::max(kTile, static_cast<int>(ceil_div(spr, kTile) * kTile));
    p.slots_per_run = spr;
    p.n_runs = static_cast<int>(ceil_div(total, spr));
  }
  p.part = p.n_runs > 1 || a.out_fp8;
  size_t off = 0;
  p.off_acc = off;
  // partial outputs: bf16 on the matrix-core path, f32 accumulators elsewhere
  const size_t acc_el = p.mfma ? 2 : 4;
  if (p.part) off = align_up(off + static_cast<size_t>(rows) * p.n_runs * a.heads * a.dim * acc_el);
  p.off_ml = off;
  if (p.part) off = align_up(off + static_cast<size_t>(rows) * p.n_runs * a.heads * 2 * 4);
  p.off_cs = off;
  if (p.dec && p.part) off = align_up(off + static_cast<size_t>(rows) * a.rope_dim * 4);
  p.total = off;
  return p;
}

template <typename T>
dsa_status launch_typed(const dsa_attn_args& a, const Plan& p, void* ws, hipStream_t st,
                        const AttnLaunch& lx) {
  AttnGeom g{};
  g.q_pos = a.q_pos;
  g.Tq = a.queries_per_seq;
  g.H = a.heads;
  g.D = a.dim;
  g.r = a.rope_dim;
  g.base = a.rope_base;
  g.theta1 = a.rope_dim > 0 ? std::pow(a.rope_base, -2.0 / a.rope_dim) : 1.0;
  g.off = a.rope_pos_offset;
  g.idx = a.idx;
  g.k = a.k;
  g.e_cap = a.e_cap;
  g.w_cap = a.w_cap;
  g.W = a.window_size;
  g.chunk_pos0 = a.chunk_pos0;
  g.chunk_len = a.chunk_len;
  g.scale = a.softmax_scale != 0.f ? a.softmax_scale : 1.0f / sqrtf(static_cast<float>(a.dim));
  g.max_pos_end = a.max_pos_end;
  g.slots_per_run = p.slots_per_run;
  g.n_runs = p.n_runs;
  g.cs_tab = lx.cs_tab;
  g.status = a.status;
  const int rows = a.n_seqs * a.queries_per_seq;
  g.rows = rows;
  g.direct = !p.part;
  g.out_scale = a.out_fp8 ? a.out_scale : nullptr;
  g.cache_scale = a.cache_fp8 ? a.cache_scale : nullptr;
  const Paging pg = make_paging(a.paging);
  g.ent = pg.ent;
  g.swa = pg.swa;
  char* base = static_cast<char*>(ws);
  float* part_acc = reinterpret_cast<float*>(base + p.off_acc);
  float* part_ml = reinterpret_cast<float*>(base + p.off_ml);
  const hipEvent_t ev0 = static_cast<hipEvent_t>(lx.ev0), ev1 = static_cast<hipEvent_t>(lx.ev1);
  const bool combine = p.part && !p.dec && !p.mfma;
  if constexpr (sizeof(T) == 2) {
    if (p.dec) {
      float* cs_ws = p.part ? reinterpret_cast<float*>(base + p.off_cs) : nullptr;
      const int64_t G = a.heads / kDH, pairs = static_cast<int64_t>(rows) * p.n_runs;
      const dim3 grid(static_cast<unsigned>(ceil_div(pairs, 8) * 8 * G));
      launch_timed(a.cache_fp8 ? k_attn_decode<kDecWaves, true> : k_attn_decode<kDecWaves, false>,
                   grid, dim3(kDecWaves * 64), 0, st, ev0, p.part ? nullptr : ev1, g,
                   static_cast<const uint16_t*>(a.q), a.rotate_q,
                   static_cast<const uint16_t*>(a.cache), static_cast<const uint16_t*>(a.window),
                   static_cast<const uint16_t*>(a.chunk_win), static_cast<uint16_t*>(a.out), a.lse,
                   part_acc, part_ml, cs_ws);
      dsa_status rc = hip_check(hipGetLastError(), "k_attn_decode launch");
      if (rc != DSA_OK || !p.part) return rc;
      launch_timed(k_attn_dcombine, dim3(a.heads, rows), dim3(128), 0, st, nullptr, ev1, g,
                   static_cast<const float*>(part_acc), static_cast<const float*>(part_ml),
                   static_cast<const float*>(cs_ws), a.out, a.lse);
      return hip_check(hipGetLastError(), "k_attn_dcombine launch");
    } else if (p.mfma) {
      dim3 grid(static_cast<unsigned>(a.heads / 64), rows, p.n_runs);
      if (!p.part)
        launch_timed(k_attn_mfma8<true>, grid, dim3(512), 0, st, ev0, ev1, g,
                     static_cast<const uint16_t*>(a.q), a.rotate_q,
                     static_cast<const uint16_t*>(a.cache), static_cast<const uint16_t*>(a.window),
                     static_cast<const uint16_t*>(a.chunk_win), static_cast<uint16_t*>(a.out),
                     a.lse, part_acc, part_ml);
      else {
        launch_timed(k_attn_mfma8<false>, grid, dim3(512), 0, st, ev0, nullptr, g,
                     static_cast<const uint16_t*>(a.q), a.rotate_q,
                     static_cast<const uint16_t*>(a.cache), static_cast<const uint16_t*>(a.window),
                     static_cast<const uint16_t*>(a.chunk_win), static_cast<uint16_t*>(a.out),
                     a.lse, part_acc, part_ml);
        dsa_status rc = hip_check(hipGetLastError(), "k_attn_mfma8 launch");
        if (rc != DSA_OK) return rc;
        launch_timed(k_attn_mcombine, dim3(a.heads, rows), dim3(128), 0, st, nullptr, ev1, g,
                     static_cast<const float*>(part_acc), static_cast<const float*>(part_ml),
                     a.out, a.lse);
        return hip_check(hipGetLastError(), "k_attn_mcombine launch");
      }
    }
  }
  if (!p.mfma && !p.dec) {
    dim3 grid(static_cast<unsigned>(ceil_div(a.heads, kHG)), rows, p.n_runs);
    const size_t shm = static_cast<size_t>(kHG + kTile) * a.dim * sizeof(float);
    launch_timed(k_attn_generic<T>, grid, dim3(kThreads), shm, st, ev0,
                 combine ? nullptr : ev1, g, static_cast<const T*>(a.q), a.rotate_q,
                 static_cast<const T*>(a.cache), static_cast<const T*>(a.window),
                 static_cast<const T*>(a.chunk_win), static_cast<T*>(a.out), a.lse, part_acc,
                 part_ml);
  }
  dsa_status rc = hip_check(hipGetLastError(), "attention launch");
  if (rc != DSA_OK || !combine) return rc;
  launch_timed(k_attn_combine<T>, dim3(a.heads, rows), dim3(256), 0, st, nullptr, ev1, g,
               static_cast<const float*>(part_acc), static_cast<const float*>(part_ml), a.out,
               a.lse);
  return hip_check(hipGetLastError(), "k_attn_combine launch");
}

}  // namespace

size_t attn_ws_bytes(const dsa_attn_args& a) { return plan(a).total; }

dsa_status attn_fp8_cache_shape(int k, int heads, int64_t rows) {
  if (k % kDStep != 0 || heads % kDH != 0 || rows * (heads / kDH) > 2048)
    return fail(DSA_ERR_UNSUPPORTED, "an fp8 cache needs bf16, dim 512, k a multiple of %d, heads "
                "a multiple of %d and rows * heads / %d <= 2048 (k %d, heads %d, rows %lld)",
                kDStep, kDH, kDH, k, heads, static_cast<long long>(rows));
  return DSA_OK;
}

dsa_status launch_attn(const dsa_attn_args& a, void* ws, hipStream_t st, const AttnLaunch& lx) {
  if (a.dim > kMaxD || a.dim % 16 != 0)
    return fail(DSA_ERR_UNSUPPORTED, "attention dim %d must be a multiple of 16, <= %d", a.dim, kMaxD);
  const size_t shm = static_cast<size_t>(kHG + kTile) * a.dim * sizeof(float);
  if (shm > 160 * 1024 - 8192) return fail(DSA_ERR_UNSUPPORTED, "attention dim %d too large", a.dim);
  const Plan p = plan(a);
  if (a.cache_fp8) {
    const dsa_status rc = attn_fp8_cache_shape(a.k, a.heads, static_cast<int64_t>(a.n_seqs) * a.queries_per_seq);
    if (rc != DSA_OK) return rc;
    if (!p.dec) return fail(DSA_ERR_UNSUPPORTED, "an fp8 cache is read by the decode kernel only");
  }
  return a.dtype == DSA_F32 ? launch_typed<float>(a, p, ws, st, lx)
                            : launch_typed<uint16_t>(a, p, ws, st, lx);
}

}  // namespace dsa
