// Layer-state maintenance kernels: compressor rings, chunk rotation and the
// window ring.
//
// The compressor state is the last S raw tokens of each compressor (c4a 8,
// c128a 128: "DeepSeek V4 稀疏注意力完全解剖", 设计 2), raw position p at slot
// p mod S.  The window keeps the rotated raw tokens R_n x_n of the last w_cap
// positions (same page, 机制四), position n at slot n mod w_cap.  Paged
// (same page, 第三层 设计 1 and 2), a sequence's rings are one block of the
// ring pools and window token n sits in slot n mod 256 of its logical block's
// window block.
#include "common.h"
#include "compress_impl.h"
#include "decode_impl.h"
#include "internal.h"

namespace dsa {
namespace {

// One ring's copy source and destination (element size in 2-byte units).
struct RingCopy {
  const uint16_t* raw;
  uint16_t* ring;
  int units;
};

// The chunk's tokens rotated for the window: out[b, t] = R_{p0 + t + off}
// x[b, t] in the storage dtype.
template <typename T>
struct RotateJob {
  const T* x;
  T* out;
  int D, r;
  double theta1;  // base^(-2 / r): pair i turns by (p + off) theta1^i
  int64_t off;
};

template <typename T>
__device__ __forceinline__ void rotate_token(const RotateJob<T>& j, int b, int64_t t, int64_t Tn,
                                             int64_t p0) {
  const int64_t o = (static_cast<int64_t>(b) * Tn + t) * j.D;
  const int first_rot = (j.D - j.r) / 2;
  for (int pr = threadIdx.x; pr < j.D / 2; pr += blockDim.x) {
    float a0 = load_as_f32(j.x, o + 2 * pr), a1 = load_as_f32(j.x, o + 2 * pr + 1);
    if (pr >= first_rot) {
      float c, s;
      rope_cs1(p0 + t + j.off, pr - first_rot, j.theta1, &c, &s);
      const float t0 = a0 * c - a1 * s, t1 = a0 * s + a1 * c;
      a0 = t0;
      a1 = t1;
    }
    store_from_f32(j.out, o + 2 * pr, a0);
    store_from_f32(j.out, o + 2 * pr + 1, a1);
  }
}

// A chunk's bookkeeping after the compressor, in one launch, no role
// waiting on another (grid (X, B, roles)): for blockIdx.z < n_rings, ring z
// (0 the main ring, 1 the indexer's) takes the last min(T, S) raw tokens of
// the chunk (blocks x < min(T, S)); blockIdx.z = n_rings writes every row's
// position pos0[b] + t to qpos; with rot.out, blockIdx.z = n_rings + 1
// rotates the chunk's tokens for the window (token t by block t mod X).
template <typename RT>
__global__ void k_chunk_tasks(RingCopy r0, RingCopy r1, int n_rings, int64_t T, int S,
                              const int64_t* __restrict__ pos0, int B, int64_t max_pos_end,
                              Paging pg, uint32_t* status, int64_t* __restrict__ qpos,
                              RotateJob<RT> rot) {
  const int z = static_cast<int>(blockIdx.z);
  if (z == n_rings) {
    const int64_t nrow = static_cast<int64_t>(B) * T;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * gridDim.y * blockDim.x;
    for (int64_t i = (static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x) * blockDim.x +
                     threadIdx.x;
         i < nrow; i += stride)
      qpos[i] = pos0[i / T] + i % T;
    return;
  }
  if (z > n_rings) {
    const int b = blockIdx.y;
    const int64_t p0 = pos0[b];
    if (p0 < 0 || p0 + T > max_pos_end) return;
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) rotate_token(rot, b, t, T, p0);
    return;
  }
  const int64_t keep = T < S ? T : S;
  if (static_cast<int64_t>(blockIdx.x) >= keep) return;
  const uint16_t* raw = blockIdx.z == 0 ? r0.raw : r1.raw;
  uint16_t* ring = blockIdx.z == 0 ? r0.ring : r1.ring;
  const int units = blockIdx.z == 0 ? r0.units : r1.units;
  const int b = blockIdx.y;
  const int64_t p0 = pos0[b];
  if (p0 < 0 || p0 + T > max_pos_end) return;
  bool ok = true;
  const int64_t sq = state_seq(pg, b, threadIdx.x == 0 ? status : nullptr, &ok);
  if (!ok) return;
  const int64_t t = T - keep + blockIdx.x;  // chunk offset of the token
  const int64_t p = p0 + t;
  const uint16_t* src = raw + (static_cast<int64_t>(b) * T + t) * units;
  uint16_t* dst = ring + (sq * S + (p % S)) * units;
  for (int i = threadIdx.x; i < units; i += blockDim.x) dst[i] = src[i];
}

// The pre-attention step of a chunk, horizontally fused ("DeepSeek V4 稀疏注意力
// 完全解剖", 融合点 3): the first B T nq workgroups prepare the queries (Q-norm
// and rotation, four heads per workgroup, one per wave), the next B T rotate
// the chunk's raw tokens for the window (K RoPE; the window ring takes them
// after attention).  No workgroup waits on another.
template <typename T>
__global__ __launch_bounds__(256) void k_qk_prep(const T* __restrict__ q, T* __restrict__ q_rot,
                                                 int H, int nq, const float* __restrict__ gamma,
                                                 float eps, const T* __restrict__ x, T* __restrict__ rot,
                                                 int D, int64_t Tn, int r, double base, int64_t off,
                                                 const int64_t* __restrict__ pos0, int B,
                                                 int64_t max_pos_end) {
  const int64_t id = blockIdx.x, nqw = static_cast<int64_t>(B) * Tn * nq;
  if (id < nqw) {
    const int64_t row = id / nq;  // b * T + t
    const int b = static_cast<int>(row / Tn);
    const int64_t t = row % Tn, p0 = pos0[b];
    const int h = 4 * static_cast<int>(id % nq) + static_cast<int>(threadIdx.x >> 6);
    if (h >= H || p0 < 0 || p0 + Tn > max_pos_end) return;
    const int64_t o = (row * H + h) * D;
    q_prep_head(q + o, q_rot + o, D, r, base, p0 + t + off, gamma, eps);
    return;
  }
  const int64_t tk = id - nqw;
  const int b = static_cast<int>(tk / Tn);
  const int64_t t = tk % Tn, p0 = pos0[b];
  if (p0 < 0 || p0 + Tn > max_pos_end) return;
  const int64_t o = (static_cast<int64_t>(b) * Tn + t) * D;
  const int first_rot = (D - r) / 2;
  for (int pr = threadIdx.x; pr < D / 2; pr += blockDim.x) {
    float a0 = load_as_f32(x, o + 2 * pr), a1 = load_as_f32(x, o + 2 * pr + 1);
    if (pr >= first_rot) {
      float c, s;
      rope_cs(p0 + t + off, pr - first_rot, r, base, &c, &s);
      const float t0 = a0 * c - a1 * s, t1 = a0 * s + a1 * c;
      a0 = t0;
      a1 = t1;
    }
    store_from_f32(rot, o + 2 * pr, a0);
    store_from_f32(rot, o + 2 * pr + 1, a1);
  }
}

// The window takes the last min(T, keep_cap) rotated chunk tokens (ring:
// keep_cap = w_cap; paged: the window size, the tokens later steps read).
__global__ void k_window_update(const uint16_t* __restrict__ rot, int units, int64_t T,
                                uint16_t* __restrict__ win, int w_cap, int keep_cap,
                                const int64_t* __restrict__ pos0, int64_t max_pos_end,
                                PageMap swa, uint32_t* status) {
  const int b = blockIdx.y;
  const int64_t p0 = pos0[b];
  if (p0 < 0 || p0 + T > max_pos_end) return;
  const int64_t keep = T < keep_cap ? T : keep_cap;
  const int64_t t = T - keep + blockIdx.x;
  const int64_t n = p0 + t;
  bool ok = true;
  const int64_t wr = window_row(swa, b, n, w_cap, threadIdx.x == 0 ? status : nullptr, &ok);
  if (!ok) return;
  const uint16_t* src = rot + (static_cast<int64_t>(b) * T + t) * units;
  uint16_t* dst = win + wr * units;
  for (int i = threadIdx.x; i < units; i += blockDim.x) dst[i] = src[i];
}

template <typename MainT, int kIdxOut, bool kMainFp8 = false>
__global__ __launch_bounds__(kCompressThreads) void k_decode_prologue(PrologueArgs a) {
  decode_prologue_block<MainT, kIdxOut, kStandaloneSlices, kMainFp8>(blockIdx.x / a.B,
                                                                     blockIdx.x % a.B, a);
}

// Decode-step epilogue when the window ring has no spare slot: the rotated
// token m goes to slot m mod w_cap after the attention that read it.
template <typename MainT>
__global__ void k_decode_window_insert(const MainT* __restrict__ x, MainT* __restrict__ win, int D,
                                       int w_cap, int r, double base, int64_t off,
                                       const int64_t* __restrict__ pos0, int64_t max_pos_end,
                                       PageMap swa, uint32_t* status) {
  const int b = blockIdx.x;
  const int64_t m = pos0[b];
  if (m < 0 || m >= max_pos_end) return;
  bool ok = true;
  const int64_t wr = window_row(swa, b, m, w_cap, threadIdx.x == 0 ? status : nullptr, &ok);
  if (ok) rotate_store(x + static_cast<int64_t>(b) * D, win + wr * D, D, r, base, m + off);
}

}  // namespace

dsa_status launch_chunk_tasks(const void* raw0, dsa_dtype dt0, int D0, void* ring0,
                              const void* raw1, dsa_dtype dt1, int D1, void* ring1, int64_t T,
                              int S, const int64_t* pos0, int B, int64_t max_pos_end,
                              const dsa_paging& pg, uint32_t* status, int64_t* qpos,
                              void* rot_out, int rope_dim, double rope_base, int64_t rope_off,
                              hipStream_t st) {
  const RingCopy r0{static_cast<const uint16_t*>(raw0), static_cast<uint16_t*>(ring0),
                    static_cast<int>(D0 * dtype_size(dt0) / 2)};
  const RingCopy r1{static_cast<const uint16_t*>(raw1), static_cast<uint16_t*>(ring1),
                    ring1 ? static_cast<int>(D1 * dtype_size(dt1) / 2) : 0};
  const int n_rings = ring1 ? 2 : 1;
  const int64_t keep = T < S ? T : S;
  const int64_t rot_blocks = rot_out ? std::min<int64_t>(T, 2048) : 0;
  const double theta1 = rope_dim > 0 ? std::pow(rope_base, -2.0 / rope_dim) : 1.0;
  const dim3 grid(static_cast<unsigned>(std::max(keep, rot_blocks)), B, n_rings + 1 + (rot_out ? 1 : 0));
  if (dt0 == DSA_F32) {
    const RotateJob<float> rj{static_cast<const float*>(raw0), static_cast<float*>(rot_out), D0,
                              rope_dim, theta1, rope_off};
    hipLaunchKernelGGL(k_chunk_tasks<float>, grid, dim3(256), 0, st, r0, r1, n_rings, T, S, pos0, B,
                       max_pos_end, make_paging(pg), status, qpos, rj);
  } else {
    const RotateJob<uint16_t> rj{static_cast<const uint16_t*>(raw0), static_cast<uint16_t*>(rot_out),
                                 D0, rope_dim, theta1, rope_off};
    hipLaunchKernelGGL(k_chunk_tasks<uint16_t>, grid, dim3(256), 0, st, r0, r1, n_rings, T, S, pos0,
                       B, max_pos_end, make_paging(pg), status, qpos, rj);
  }
  return hip_check(hipGetLastError(), "k_chunk_tasks launch");
}

dsa_status launch_qk_prep(const dsa_layer_args& a, void* q_rot, void* rot_chunk, hipStream_t st) {
  const int B = a.n_seqs, H = a.heads, D = a.main.dim;
  const int64_t T = a.chunk_len;
  const int nq = (H + 3) / 4;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(B) * T * (nq + 1)));
  if (a.dtype == DSA_F32)
    hipLaunchKernelGGL(k_qk_prep<float>, grid, dim3(256), 0, st, static_cast<const float*>(a.q),
                       static_cast<float*>(q_rot), H, nq, a.q_norm_gamma, a.rms_eps,
                       static_cast<const float*>(a.x), static_cast<float*>(rot_chunk), D, T,
                       a.main.rope_dim, a.main.rope_base, a.main.rope_pos_offset, a.pos0, B,
                       a.max_pos_end);
  else
    hipLaunchKernelGGL(k_qk_prep<uint16_t>, grid, dim3(256), 0, st,
                       static_cast<const uint16_t*>(a.q), static_cast<uint16_t*>(q_rot), H, nq,
                       a.q_norm_gamma, a.rms_eps, static_cast<const uint16_t*>(a.x),
                       static_cast<uint16_t*>(rot_chunk), D, T, a.main.rope_dim, a.main.rope_base,
                       a.main.rope_pos_offset, a.pos0, B, a.max_pos_end);
  return hip_check(hipGetLastError(), "k_qk_prep launch");
}

dsa_status launch_window_update(const void* rot_chunk, dsa_dtype dt, int D, int64_t T, void* win,
                                int w_cap, int window_size, const int64_t* pos0, int B,
                                int64_t max_pos_end, const dsa_paging& pg, uint32_t* status,
                                hipStream_t st) {
  const int units = static_cast<int>(D * dtype_size(dt) / 2);
  const Paging P = make_paging(pg);
  const int keep_cap = P.swa.table ? window_size : w_cap;
  const int64_t keep = T < keep_cap ? T : keep_cap;
  if (keep <= 0) return DSA_OK;
  hipLaunchKernelGGL(k_window_update, dim3(static_cast<unsigned>(keep), B), dim3(256), 0, st,
                     static_cast<const uint16_t*>(rot_chunk), units, T,
                     static_cast<uint16_t*>(win), w_cap, keep_cap, pos0, max_pos_end, P.swa,
                     status);
  return hip_check(hipGetLastError(), "k_window_update launch");
}

}  // namespace dsa

namespace dsa {

PrologueArgs make_prologue_args(const dsa_layer_args& a, int64_t* qpos, bool insert_window,
                                float* cs_tab, void* q_rot) {
  PrologueArgs p{};
  p.H = a.heads;
  p.nq_roles = q_rot ? (a.heads + 3) / 4 : 0;
  p.q = a.q;
  p.q_rot = q_rot;
  p.q_gamma = a.q_norm_gamma;
  p.B = a.n_seqs;
  p.D = a.main.dim;
  p.Di = a.idx_dim;
  p.s = a.main.stride;
  p.S = a.main.span;
  p.r = a.main.rope_dim;
  p.r_idx = a.idx_rope_dim;
  p.w_cap = a.w_cap;
  p.base = a.main.rope_base;
  p.idx_base = a.idx_rope_base;
  p.off = a.main.rope_pos_offset;
  p.e_cap = a.e_cap;
  p.max_pos_end = a.max_pos_end;
  p.eps = a.rms_eps;
  p.has_idx = a.idx_heads > 0;
  p.insert_window = insert_window;
  p.pos0 = a.pos0;
  p.x = a.x;
  p.kx = a.kx;
  p.logits_main = a.logits_main;
  p.logits_idx = a.logits_idx;
  p.gamma = a.rms_gamma;
  p.gamma_idx = a.rms_gamma_idx;
  p.main_cache = a.main_cache;
  p.idx_cache = a.idx_cache;
  p.main_ring = a.main_ring;
  p.idx_ring = a.idx_ring;
  p.window = a.window;
  p.idx_scale = a.idx_scale;
  p.idx_mx = a.idx_dtype == DSA_FP4_E2M1 ? a.idx_mx_scale : nullptr;
  p.qpos = qpos;
  p.cs_tab = cs_tab;
  p.main_scale = a.main_fp8 ? a.main_scale : nullptr;
  p.status = a.status;
  p.pg = make_paging(a.paging);
  return p;
}

dsa_status launch_decode_prologue(const dsa_layer_args& a, int64_t* qpos, bool insert_window,
                                  float* cs_tab, void* q_rot, hipStream_t st, int32_t* all_idx,
                                  int all_k, int64_t all_nv_cap) {
  PrologueArgs p = make_prologue_args(a, qpos, insert_window, cs_tab, q_rot);
  p.all_idx = all_idx;
  p.all_k = all_k;
  p.all_nv_cap = all_nv_cap;
  const dim3 grid((prologue_roles<kStandaloneSlices>() + p.nq_roles) * a.n_seqs),
      block(kCompressThreads);
  // the indexer entry's output format picks the instantiation
  auto by_idx = [&](auto f32, auto fp8, auto fp4) {
    if (a.idx_dtype == DSA_F32) hipLaunchKernelGGL(f32, grid, block, 0, st, p);
    else if (a.idx_dtype == DSA_FP4_E2M1) hipLaunchKernelGGL(fp4, grid, block, 0, st, p);
    else hipLaunchKernelGGL(fp8, grid, block, 0, st, p);
  };
  if (a.dtype == DSA_F32)
    by_idx(k_decode_prologue<float, DSA_F32>, k_decode_prologue<float, DSA_FP8_E4M3>,
           k_decode_prologue<float, DSA_FP4_E2M1>);
  else if (p.main_scale)  // token-wise fp8 main cache
    by_idx(k_decode_prologue<uint16_t, DSA_F32, true>,
           k_decode_prologue<uint16_t, DSA_FP8_E4M3, true>,
           k_decode_prologue<uint16_t, DSA_FP4_E2M1, true>);
  else
    by_idx(k_decode_prologue<uint16_t, DSA_F32>, k_decode_prologue<uint16_t, DSA_FP8_E4M3>,
           k_decode_prologue<uint16_t, DSA_FP4_E2M1>);
  return hip_check(hipGetLastError(), "k_decode_prologue launch");
}

dsa_status launch_decode_window_insert(const dsa_layer_args& a, hipStream_t st) {
  if (a.dtype == DSA_F32)
    hipLaunchKernelGGL(k_decode_window_insert<float>, dim3(a.n_seqs), dim3(256), 0, st,
                       static_cast<const float*>(a.x), static_cast<float*>(a.window), a.main.dim,
                       a.w_cap, a.main.rope_dim, a.main.rope_base, a.main.rope_pos_offset, a.pos0,
                       a.max_pos_end, make_paging(a.paging).swa, a.status);
  else
    hipLaunchKernelGGL(k_decode_window_insert<uint16_t>, dim3(a.n_seqs), dim3(256), 0, st,
                       static_cast<const uint16_t*>(a.x), static_cast<uint16_t*>(a.window),
                       a.main.dim, a.w_cap, a.main.rope_dim, a.main.rope_base,
                       a.main.rope_pos_offset, a.pos0, a.max_pos_end, make_paging(a.paging).swa,
                       a.status);
  return hip_check(hipGetLastError(), "k_decode_window_insert launch");
}

}  // namespace dsa
