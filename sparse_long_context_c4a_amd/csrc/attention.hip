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
  uint32_t* status;
};

// Source of slot a of row `row`; nullptr if the slot is empty.
template <typename T>
__device__ __forceinline__ const T* slot_ptr(const AttnGeom& g, int row, int b, int64_t m,
                                             int a, const T* cache, const T* window,
                                             const T* chunk_win) {
  if (a < g.k) {
    const int32_t j = g.idx[static_cast<int64_t>(row) * g.k + a];
    if (j < 0 || j >= g.e_cap) return nullptr;
    return cache + (static_cast<int64_t>(b) * g.e_cap + j) * g.D;
  }
  const int64_t n = m - g.W + (a - g.k);
  if (n < 0 || n >= m) return nullptr;
  if (chunk_win) {
    const int64_t c0 = g.chunk_pos0[b];
    if (n >= c0 && n - c0 < g.chunk_len)
      return chunk_win + (static_cast<int64_t>(b) * g.chunk_len + (n - c0)) * g.D;
  }
  return window + (static_cast<int64_t>(b) * g.w_cap + (n % g.w_cap)) * g.D;
}

// Generic (any D <= 1024, f32 or bf16) attention run.  Output: either the
// final rotated result (n_runs == 1) or an un-normalised partial
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
    if (ok) rope_cs(m + g.off, i, g.r, g.base, &c, &s);
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
  for (int a0 = a_begin; a0 < a_end; a0 += kTile) {
    __syncthreads();
    for (int e = 0; e < kTile; ++e) {
      const int a = a0 + e;
      const T* src = (ok && a < a_end) ? slot_ptr<T>(g, row, b, m, a, cache, window, chunk_win)
                                       : nullptr;
      if (tid == 0) valid_s[e] = src != nullptr;
      for (int d = tid; d < D; d += kThreads) v_s[e * D + d] = src ? load_as_f32(src, d) : 0.f;
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
  if (g.n_runs == 1) {
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

// Merge the runs of one (row, head) and apply R_m^{-1}.
template <typename T>
__global__ __launch_bounds__(256) void k_attn_combine(AttnGeom g, const float* __restrict__ part_acc,
                                                      const float* __restrict__ part_ml,
                                                      T* __restrict__ out, float* __restrict__ lse) {
  const int row = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
  const int64_t m = g.q_pos[row];
  const bool ok = m >= 0 && m < g.max_pos_end;
  float M = -INFINITY;
  for (int r = 0; r < g.n_runs; ++r)
    M = fmaxf(M, part_ml[2 * ((static_cast<int64_t>(row) * g.n_runs + r) * g.H + h)]);
  float L = 0.f;
  for (int r = 0; r < g.n_runs; ++r) {
    const int64_t pi = (static_cast<int64_t>(row) * g.n_runs + r) * g.H + h;
    const float mr = part_ml[2 * pi];
    if (mr != -INFINITY) L += part_ml[2 * pi + 1] * expf(mr - M);
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  const int D = g.D, first_rot = (D - g.r) / 2;
  const int64_t o = (static_cast<int64_t>(row) * g.H + h) * D;
  for (int pr = tid; pr < D / 2; pr += blockDim.x) {
    float a0 = 0.f, a1 = 0.f;
    for (int r = 0; r < g.n_runs; ++r) {
      const int64_t pi = (static_cast<int64_t>(row) * g.n_runs + r) * g.H + h;
      const float mr = part_ml[2 * pi];
      if (mr == -INFINITY) continue;
      const float wgt = expf(mr - M);
      a0 = fmaf(wgt, part_acc[pi * D + 2 * pr], a0);
      a1 = fmaf(wgt, part_acc[pi * D + 2 * pr + 1], a1);
    }
    a0 *= inv;
    a1 *= inv;
    if (pr >= first_rot && ok) {
      float c, s;
      rope_cs(m + g.off, pr - first_rot, g.r, g.base, &c, &s);
      const float t0 = a0 * c + a1 * s, t1 = -a0 * s + a1 * c;
      a0 = t0;
      a1 = t1;
    }
    store_from_f32(out, o + 2 * pr, a0);
    store_from_f32(out, o + 2 * pr + 1, a1);
  }
  if (lse && tid == 0)
    lse[static_cast<int64_t>(row) * g.H + h] = L > 0.f ? M + logf(L) : -INFINITY;
}

struct Plan {
  int slots_per_run, n_runs;
  size_t off_acc, off_ml, total;
};

Plan plan(const dsa_attn_args& a) {
  Plan p{};
  const int64_t rows = static_cast<int64_t>(a.n_seqs) * a.queries_per_seq;
  const int total = a.k + a.window_size;
  const int64_t hgroups = ceil_div(a.heads, kHG);
  // enough workgroups to cover the chip (~1024), runs of at least 64 slots
  int64_t want = ceil_div(1024, std::max<int64_t>(1, rows * hgroups));
  int spr = static_cast<int>(ceil_div(total, std::max<int64_t>(1, want)));
  spr = std::max(64, static_cast<int>(ceil_div(spr, kTile) * kTile));
  p.slots_per_run = spr;
  p.n_runs = static_cast<int>(ceil_div(total, spr));
  size_t off = 0;
  p.off_acc = off;
  if (p.n_runs > 1) off = align_up(off + static_cast<size_t>(rows) * p.n_runs * a.heads * a.dim * 4);
  p.off_ml = off;
  if (p.n_runs > 1) off = align_up(off + static_cast<size_t>(rows) * p.n_runs * a.heads * 2 * 4);
  p.total = off;
  return p;
}

template <typename T>
dsa_status launch_typed(const dsa_attn_args& a, const Plan& p, void* ws, hipStream_t st) {
  AttnGeom g{};
  g.q_pos = a.q_pos;
  g.Tq = a.queries_per_seq;
  g.H = a.heads;
  g.D = a.dim;
  g.r = a.rope_dim;
  g.base = a.rope_base;
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
  g.status = a.status;
  const int rows = a.n_seqs * a.queries_per_seq;
  char* base = static_cast<char*>(ws);
  float* part_acc = reinterpret_cast<float*>(base + p.off_acc);
  float* part_ml = reinterpret_cast<float*>(base + p.off_ml);
  dim3 grid(static_cast<unsigned>(ceil_div(a.heads, kHG)), rows, p.n_runs);
  const size_t shm = static_cast<size_t>(kHG + kTile) * a.dim * sizeof(float);
  hipLaunchKernelGGL(k_attn_generic<T>, grid, dim3(kThreads), shm, st, g,
                     static_cast<const T*>(a.q), a.rotate_q, static_cast<const T*>(a.cache),
                     static_cast<const T*>(a.window), static_cast<const T*>(a.chunk_win),
                     static_cast<T*>(a.out), a.lse, part_acc, part_ml);
  dsa_status rc = hip_check(hipGetLastError(), "k_attn_generic launch");
  if (rc != DSA_OK || p.n_runs == 1) return rc;
  hipLaunchKernelGGL(k_attn_combine<T>, dim3(a.heads, rows), dim3(256), 0, st, g, part_acc,
                     part_ml, static_cast<T*>(a.out), a.lse);
  return hip_check(hipGetLastError(), "k_attn_combine launch");
}

}  // namespace

size_t attn_ws_bytes(const dsa_attn_args& a) { return plan(a).total; }

dsa_status launch_attn(const dsa_attn_args& a, void* ws, hipStream_t st) {
  if (a.dim > kMaxD || a.dim % 16 != 0)
    return fail(DSA_ERR_UNSUPPORTED, "attention dim %d must be a multiple of 16, <= %d", a.dim, kMaxD);
  const size_t shm = static_cast<size_t>(kHG + kTile) * a.dim * sizeof(float);
  if (shm > 160 * 1024 - 8192) return fail(DSA_ERR_UNSUPPORTED, "attention dim %d too large", a.dim);
  const Plan p = plan(a);
  return a.dtype == DSA_F32 ? launch_typed<float>(a, p, ws, st)
                            : launch_typed<uint16_t>(a, p, ws, st);
}

}  // namespace dsa
