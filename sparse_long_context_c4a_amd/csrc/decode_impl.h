// Decode-step state updates (compressor entries, rings, window insert) as a
// device function, shared by the stand-alone prologue kernel and the fused
// decode indexer kernel.
#pragma once

#include <type_traits>

#include "common.h"
#include "compress_impl.h"

namespace dsa {

// Rotate raw token x (D dims of type T) at position pos and store it to dst.
template <typename T>
__device__ __forceinline__ void rotate_store(const T* __restrict__ x, T* __restrict__ dst, int D,
                                             int r, double base, int64_t pos) {
  const int first_rot = (D - r) / 2;
  for (int pr = threadIdx.x; pr < D / 2; pr += blockDim.x) {
    float a0 = load_as_f32(x, 2 * pr), a1 = load_as_f32(x, 2 * pr + 1);
    if (pr >= first_rot) {
      float c, sn;
      rope_cs(pos, pr - first_rot, r, base, &c, &sn);
      const float t0 = a0 * c - a1 * sn, t1 = a0 * sn + a1 * c;
      a0 = t0;
      a1 = t1;
    }
    store_from_f32(dst, 2 * pr, a0);
    store_from_f32(dst, 2 * pr + 1, a1);
  }
}

// Q-norm and rotation of one query head by one wave of 64 lanes (the pages'
// horizontally fused pre-attention step, "DeepSeek V4 稀疏注意力完全解剖"
// 融合点 3: each wave owns one head, no exchange between waves):
// q <- gamma * q / sqrt(mean(q^2) + eps) when gamma is given (the RMSNorm
// form of the compressor's), then R_pos on the tail r dims, stored in the
// storage dtype T.
template <typename T>
__device__ __forceinline__ void q_prep_head(const T* __restrict__ qh, T* __restrict__ dst, int D,
                                            int r, double base, int64_t pos,
                                            const float* __restrict__ gamma, float eps) {
  const int lane = threadIdx.x & 63;
  float rs = 1.f;
  if (gamma) {
    float ss = 0.f;
    for (int pr = lane; pr < D / 2; pr += 64) {
      const float a0 = load_as_f32(qh, 2 * pr), a1 = load_as_f32(qh, 2 * pr + 1);
      ss += a0 * a0 + a1 * a1;
    }
    rs = 1.0f / sqrtf(wave_sum(ss) / static_cast<float>(D) + eps);
  }
  const int first_rot = (D - r) / 2;
  for (int pr = lane; pr < D / 2; pr += 64) {
    float a0 = load_as_f32(qh, 2 * pr), a1 = load_as_f32(qh, 2 * pr + 1);
    if (gamma) {
      a0 *= gamma[2 * pr] * rs;
      a1 *= gamma[2 * pr + 1] * rs;
    }
    if (pr >= first_rot) {
      float c, sn;
      rope_cs(pos, pr - first_rot, r, base, &c, &sn);
      const float t0 = a0 * c - a1 * sn, t1 = a0 * sn + a1 * c;
      a0 = t0;
      a1 = t1;
    }
    store_from_f32(dst, 2 * pr, a0);
    store_from_f32(dst, 2 * pr + 1, a1);
  }
}

struct PrologueArgs {
  int B, D, Di, s, S, r, r_idx, w_cap;
  int H, nq_roles;             // query heads; workgroups of q preparation per sequence (0: none)
  const void* q;               // [B, H, D] queries
  void* q_rot;                 // [B, H, D] normalised, rotated queries
  const float* q_gamma;        // [D] Q-norm weight or nullptr
  double base, idx_base;
  int64_t off, e_cap, max_pos_end;
  float eps;
  bool has_idx, insert_window;
  const int64_t* pos0;
  const void *x, *kx;
  const float *logits_main, *logits_idx, *gamma, *gamma_idx;
  void *main_cache, *idx_cache, *main_ring, *idx_ring, *window;
  float* idx_scale;
  uint8_t* idx_mx;  // fp4 indexer cache: E8M0 block scales [B, e_cap, Di / 32]
  int64_t* qpos;
  float* cs_tab;  // role 3: (cos, sin) of R_m, r floats per sequence
  float* main_scale;  // fp8 main cache: one scale per entry [B, e_cap], else nullptr
  uint32_t* status;
  Paging pg;          // paged caches, window and rings (tables nullptr: dense)
  // the selection when it is every visible entry (no indexer, k >= every
  // visible count): [B, all_k] indices written by role 3, nullptr: none
  int32_t* all_idx;
  int all_k;
  int64_t all_nv_cap;
};

// Workgroups of the prologue: kSlices for the main entry, then three.
template <int kSlices>
constexpr int prologue_roles() { return kSlices + 3; }
// The prologue riding in the indexer's launch keeps the main entry in one
// workgroup (c4a: 8 raw tokens); the stand-alone prologue (c128a: 128 raw
// tokens of 1 KiB) splits it by dims over four, which puts the loads of the
// whole span in flight at once (c128a decode: 11.6 -> 7.7 us per launch;
// eight slices measured the same).  An RMSNorm needs the whole vector, so with
// gamma (or dims that do not split into 8-dim groups) the first slice does
// it all.
constexpr int kPrologueRoles = prologue_roles<1>();
constexpr int kStandaloneSlices = 4;

// Decode-step prologue, one role per workgroup (then, when the queries are
// prepared here, a.nq_roles roles of four query heads each): roles 0 .. kSlices-1
// write (their dims of) the main entry completing at m (if any); the next
// role the indexer entry; the next puts token m into the compressor rings,
// the row's query position, and -- when the window ring has a spare slot
// (w_cap > W) -- the rotated token m (slot m mod w_cap is not in m's window
// then); the last writes the (cos, sin) table of R_m for the attention's
// query rotation and inverse rotation.  For one token the ring slot written
// (m mod S) is not one the compressor reads (it reads positions m-S+1 ..
// m-1 from the ring and m from x), and nothing here is read by the same
// step's indexer or attention (the new entry is not visible to m), so these
// workgroups may run beside them.
// kMainFp8: the main entry goes out as token-wise fp8 (codes + a.main_scale),
// whole in the first workgroup since the scale needs the vector's max.
template <typename MainT, int kIdxOut, int kSlices, bool kMainFp8 = false>
__device__ __forceinline__ void decode_prologue_block(int role, int b, PrologueArgs a) {
  using IdxRawT = typename std::conditional<kIdxOut == DSA_F32, float, uint16_t>::type;
  constexpr int kMainOut = std::is_same<MainT, float>::value ? DSA_F32 : DSA_BF16;
  if (role >= prologue_roles<kSlices>()) {
    // query preparation: four heads per workgroup, one per wave
    const int h = 4 * (role - prologue_roles<kSlices>()) + static_cast<int>(threadIdx.x >> 6);
    const int64_t m = a.pos0[b];
    if (h >= a.H || m < 0 || m >= a.max_pos_end) return;
    const int64_t o = (static_cast<int64_t>(b) * a.H + h) * a.D;
    q_prep_head(static_cast<const MainT*>(a.q) + o, static_cast<MainT*>(a.q_rot) + o, a.D, a.r,
                a.base, m + a.off, a.q_gamma, a.eps);
    return;
  }
  if (kSlices == 1 ? role == 0 : static_cast<unsigned>(role) < static_cast<unsigned>(kSlices)) {
    int d0 = 0, dn = -1;  // all dims
    if constexpr (kMainFp8) {
      if (role == 0)
        compress_one<MainT, DSA_FP8_E4M3>(0, b, static_cast<const MainT*>(a.x),
                                          static_cast<const MainT*>(a.main_ring), a.pos0,
                                          a.logits_main, a.main_cache, a.main_scale, a.gamma,
                                          a.eps, 1, 1, a.s, a.S, a.D, a.r, a.base, a.off,
                                          a.e_cap, a.max_pos_end, a.status, 0, -1, nullptr,
                                          a.pg);
      return;
    }
    if constexpr (kSlices > 1) {
      const bool split = a.gamma == nullptr && a.D % (8 * kSlices) == 0;
      if (!split && role > 0) return;
      if (split) {
        dn = a.D / kSlices;
        d0 = role * dn;
      }
    }
    compress_one<MainT, kMainOut>(0, b, static_cast<const MainT*>(a.x),
                                  static_cast<const MainT*>(a.main_ring), a.pos0, a.logits_main,
                                  a.main_cache, nullptr, a.gamma, a.eps, 1, 1, a.s, a.S, a.D, a.r,
                                  a.base, a.off, a.e_cap, a.max_pos_end, a.status, d0, dn, nullptr,
                                  a.pg);
    return;
  }
  role -= kSlices - 1;  // 1: indexer entry, 2: rings and window, 3: (cos, sin) table
  if (role == 1) {
    if (a.has_idx)
      compress_one<IdxRawT, kIdxOut>(0, b, static_cast<const IdxRawT*>(a.kx),
                                     static_cast<const IdxRawT*>(a.idx_ring), a.pos0, a.logits_idx,
                                     a.idx_cache, a.idx_scale, a.gamma_idx, a.eps, 1, 1, a.s, a.S,
                                     a.Di, a.r_idx, a.idx_base, a.off, a.e_cap, a.max_pos_end,
                                     a.status, 0, -1, a.idx_mx, a.pg);
    return;
  }
  if (role == 3) {
    const int64_t m = a.pos0[b];
    const bool ok = m >= 0 && m < a.max_pos_end;
    if (a.cs_tab)
      for (int i = threadIdx.x; i < a.r / 2; i += blockDim.x) {
        float c = 1.f, s = 0.f;
        if (ok) rope_cs(m + a.off, i, a.r, a.base, &c, &s);
        a.cs_tab[static_cast<int64_t>(b) * a.r + 2 * i] = c;
        a.cs_tab[static_cast<int64_t>(b) * a.r + 2 * i + 1] = s;
      }
    if (a.all_idx) {
      // entries 0 .. nv-1 in index order, then -1 (the status bits of the
      // selection pass it replaces)
      int64_t nv = 0;
      if (!ok) {
        if (threadIdx.x == 0) set_status(a.status, DSA_DEVERR_POSITION);
      } else {
        nv = n_complete(m, a.s, a.S);
        if (nv > a.all_nv_cap) {
          if (threadIdx.x == 0) set_status(a.status, DSA_DEVERR_CAPACITY);
          nv = a.all_nv_cap;
        }
      }
      if (nv > a.all_k && threadIdx.x == 0) set_status(a.status, DSA_DEVERR_NO_INDEX);
      int32_t* irow = a.all_idx + static_cast<int64_t>(b) * a.all_k;
      for (int i = threadIdx.x; i < a.all_k; i += blockDim.x) irow[i] = i < nv ? i : -1;
    }
    return;
  }
  const int64_t m = a.pos0[b];
  if (threadIdx.x == 0) a.qpos[b] = m;
  if (m < 0 || m >= a.max_pos_end) return;
  const MainT* xb = static_cast<const MainT*>(a.x) + static_cast<int64_t>(b) * a.D;
  uint32_t* st0 = threadIdx.x == 0 ? a.status : nullptr;
  bool ring_ok = true;
  const int64_t sq = state_seq(a.pg, b, st0, &ring_ok);  // the rings' block
  if (ring_ok) {
    MainT* rb = static_cast<MainT*>(a.main_ring) + (sq * a.S + m % a.S) * a.D;
    for (int i = threadIdx.x; i < a.D; i += blockDim.x) rb[i] = xb[i];
    if (a.has_idx) {
      const IdxRawT* kb = static_cast<const IdxRawT*>(a.kx) + static_cast<int64_t>(b) * a.Di;
      IdxRawT* ib = static_cast<IdxRawT*>(a.idx_ring) + (sq * a.S + m % a.S) * a.Di;
      for (int i = threadIdx.x; i < a.Di; i += blockDim.x) ib[i] = kb[i];
    }
  }
  if (a.insert_window) {
    bool ok = true;
    const int64_t wr = window_row(a.pg.swa, b, m, a.w_cap, st0, &ok);
    if (ok)
      rotate_store(xb, static_cast<MainT*>(a.window) + wr * a.D, a.D, a.r, a.base, m + a.off);
  }
}


}  // namespace dsa
