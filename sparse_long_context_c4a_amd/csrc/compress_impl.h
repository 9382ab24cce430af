// S1 core: one compressed entry per call, by a workgroup of
// kCompressThreads threads (shared by the compressor kernel and the fused
// decode prologue).
//
// Entry j mixes raw tokens s*j .. s*j+S-1 with softmax weights over its S
// logits (one weight per token, shared across the D dims), is optionally
// RMS-normalised, rotated at position s*j (+offset) and written to slot j
// (f32, bf16, or fp8 e4m3fn with one fp32 scale per entry).  The pages fuse
// exactly this chain -- compress, RMSNorm, RoPE, cache insert -- into one
// kernel ("DeepSeek V4 稀疏注意力完全解剖", 融合点 1); here each thread owns
// one (even, odd) dim pair so the rotation stays in registers, and a raw
// token row is read as one coalesced D-vector per step.
#pragma once

#include <type_traits>

#include "common.h"

namespace dsa {

constexpr int kCompressThreads = 256;
constexpr int kCompressMaxSpan = 256;
constexpr int kCompressPairs = 4;  // D <= 2048

// Dims 8 c .. 8 c + 7 of a raw token row in one or two 16-byte loads (eight
// bf16, or two float4), widened to f32 when used.
template <typename T>
struct Dim8;
template <>
struct Dim8<uint16_t> {
  typedef uint4 type;
  static __device__ __forceinline__ type load(const uint16_t* row, int c) {
    return reinterpret_cast<const uint4*>(row)[c];
  }
  static __device__ __forceinline__ float at(const type& v, int e) {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <>
struct Dim8<float> {
  struct type {
    float4 lo, hi;
  };
  static __device__ __forceinline__ type load(const float* row, int c) {
    const float4* r = reinterpret_cast<const float4*>(row) + 2 * c;
    return type{r[0], r[1]};
  }
  static __device__ __forceinline__ float at(const type& v, int e) {
    const float4& h = e < 4 ? v.lo : v.hi;
    const int k = e & 3;
    return k == 0 ? h.x : k == 1 ? h.y : k == 2 ? h.z : h.w;
  }
};

template <typename RawT, int kOut>
__device__ __forceinline__ void compress_one(
    int e, int b, const RawT* __restrict__ raw, const RawT* __restrict__ ring,
    const int64_t* __restrict__ pos0v, const float* __restrict__ logits, void* __restrict__ out,
    float* __restrict__ out_scale, const float* __restrict__ gamma, float eps, int64_t T,
    int logits_rows, int s, int S, int D, int r, double base, int64_t off, int64_t e_cap,
    int64_t max_pos_end, uint32_t* status, int d0 = 0, int dn = -1, uint8_t* out_mx = nullptr,
    Paging pg = Paging{}) {
  // dims d0 .. d0 + dn - 1 only (dn = -1: all D); a slice is a multiple of 8
  // dims and needs neither gamma nor fp8 output, which take the whole vector
  if (dn < 0) dn = D;
  __shared__ float w_s[kCompressMaxSpan];
  __shared__ float red[16];
  __shared__ float red8[kCompressThreads * 8];  // token groups' partial sums
  const int tid = threadIdx.x;
  const int64_t p0 = pos0v[b];
  if (p0 < 0 || p0 + T > max_pos_end) {
    if (tid == 0 && e == 0) set_status(status, DSA_DEVERR_POSITION);
    return;
  }
  const int64_t j0 = n_complete(p0, s, S), j1 = n_complete(p0 + T, s, S);
  const int64_t j = j0 + e;
  if (j >= j1) return;  // uniform across the block
  if (j >= e_cap) {
    if (tid == 0) set_status(status, DSA_DEVERR_CAPACITY);
    return;
  }
  // the entry's row: b * e_cap + j, or its row in the paged pool (a block
  // outside the pool drops the entry; uniform across the block)
  bool ok = true;
  const int64_t erow = entry_row(pg.ent, b, j, e_cap, tid == 0 ? status : nullptr, &ok);
  if (!ok) return;
  // tile row of the key layouts: b * e_pad + j dense, the pool row paged
  const int64_t trow = pg.ent.table ? erow : static_cast<int64_t>(b) * idx_e_pad(e_cap) + j;

  // softmax weights of this entry
  const float* lg = logits + (static_cast<int64_t>(b) * logits_rows + e) * S;
  float mx = -INFINITY;
  for (int i = tid; i < S; i += kCompressThreads) mx = fmaxf(mx, lg[i]);
  mx = block_max(mx, red);
  float sum = 0.f;
  for (int i = tid; i < S; i += kCompressThreads) {
    const float v = expf(lg[i] - mx);
    w_s[i] = v;
    sum += v;
  }
  sum = block_sum(sum, red);  // contains a barrier: w_s is complete
  const float inv = 1.0f / sum;

  // weighted sum; thread owns pairs (2p, 2p+1) of the slice, p = tid + k*kCompressThreads
  const int npairs = dn / 2, pr0 = d0 / 2;
  float acc[kCompressPairs][2];
#pragma unroll
  for (int k = 0; k < kCompressPairs; ++k) acc[k][0] = acc[k][1] = 0.f;
  const RawT* rawb = raw + static_cast<int64_t>(b) * T * D;
  const RawT* ringb = ring + state_seq(pg, b, tid == 0 ? status : nullptr) * S * D;
  if (dn % 8 == 0 && d0 % 8 == 0 && dn / 8 <= kCompressThreads) {
    // 16-byte loads: thread (group gr, column c) sums dims 8c .. 8c+7 over
    // the tokens i = gr (mod ngrp) -- a token row is D/8 threads wide, and
    // the ngrp = 256 / (D/8) groups split the span -- kTok tokens per round
    // with all of their loads out before the first is used (unconditional:
    // past the span the last token is re-read with weight 0); the groups'
    // sums then meet in LDS.  (Four-byte loads, one dim pair per thread,
    // made the 128-token c128a entry bound by the load instruction rate.)
    constexpr int kTok = 8;
    using DV = Dim8<RawT>;
    const int tpr = dn / 8, ngrp = kCompressThreads / tpr;
    const int gr = tid / tpr, c = tid % tpr;
    const int64_t pj = static_cast<int64_t>(s) * j;  // the entry's first raw position
    const int ring0 = static_cast<int>(pj % S);
    float a8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (gr < ngrp) {
      for (int i0 = gr; i0 < S; i0 += ngrp * kTok) {
        typename DV::type xw[kTok];
#pragma unroll
        for (int u = 0; u < kTok; ++u) {
          const int i = min(i0 + u * ngrp, S - 1);
          const int64_t p = pj + i;
          const int slot = ring0 + i < S ? ring0 + i : ring0 + i - S;
          const RawT* row = (p >= p0) ? rawb + (p - p0) * D : ringb + static_cast<int64_t>(slot) * D;
          xw[u] = DV::load(row + d0, c);
        }
#pragma unroll
        for (int u = 0; u < kTok; ++u) {
          const float wi = i0 + u * ngrp < S ? w_s[i0 + u * ngrp] * inv : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) a8[e] = fmaf(wi, DV::at(xw[u], e), a8[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) red8[gr * dn + 8 * c + e] = a8[e];
    }
    __syncthreads();
    // back to the layout below: thread owns pairs tid + 256 k
#pragma unroll
    for (int k = 0; k < kCompressPairs; ++k) {
      const int pr = tid + k * kCompressThreads;
      if (pr < npairs) {
        float x0 = 0.f, x1 = 0.f;
        for (int g2 = 0; g2 < ngrp; ++g2) {
          x0 += red8[g2 * dn + 2 * pr];
          x1 += red8[g2 * dn + 2 * pr + 1];
        }
        acc[k][0] = x0;
        acc[k][1] = x1;
      }
    }
  } else {
    for (int i = 0; i < S; ++i) {
      const int64_t p = static_cast<int64_t>(s) * j + i;
      const RawT* row = (p >= p0) ? rawb + (p - p0) * D : ringb + (p % S) * D;
      const float wi = w_s[i] * inv;
#pragma unroll
      for (int k = 0; k < kCompressPairs; ++k) {
        const int pr = tid + k * kCompressThreads;
        if (pr < npairs) {
          acc[k][0] = fmaf(wi, load_as_f32(row, d0 + 2 * pr), acc[k][0]);
          acc[k][1] = fmaf(wi, load_as_f32(row, d0 + 2 * pr + 1), acc[k][1]);
        }
      }
    }
  }

  if (gamma) {  // RMSNorm: c <- gamma * c / sqrt(mean(c^2) + eps)
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < kCompressPairs; ++k)
      if (tid + k * kCompressThreads < npairs) ss += acc[k][0] * acc[k][0] + acc[k][1] * acc[k][1];
    ss = block_sum(ss, red);
    const float rs = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
#pragma unroll
    for (int k = 0; k < kCompressPairs; ++k) {
      const int pr = tid + k * kCompressThreads;
      if (pr < npairs) {
        acc[k][0] *= gamma[d0 + 2 * pr] * rs;
        acc[k][1] *= gamma[d0 + 2 * pr + 1] * rs;
      }
    }
  }

  // RoPE on the tail r dims at position s*j + off
  const int first_rot_pair = (D - r) / 2;
#pragma unroll
  for (int k = 0; k < kCompressPairs; ++k) {
    const int pr = tid + k * kCompressThreads;
    if (pr < npairs && pr0 + pr >= first_rot_pair) {
      float c, sn;
      rope_cs(static_cast<int64_t>(s) * j + off, pr0 + pr - first_rot_pair, r, base, &c, &sn);
      const float a0 = acc[k][0], a1 = acc[k][1];
      acc[k][0] = a0 * c - a1 * sn;
      acc[k][1] = a0 * sn + a1 * c;
    }
  }

  const int64_t o = erow * D;
  if constexpr (kOut == DSA_F32 || kOut == DSA_BF16) {
    using OT = typename std::conditional<kOut == DSA_F32, float, uint16_t>::type;
    OT* op = static_cast<OT*>(out) + o;
#pragma unroll
    for (int k = 0; k < kCompressPairs; ++k) {
      const int pr = tid + k * kCompressThreads;
      if (pr < npairs) {
        store_from_f32(op, d0 + 2 * pr, acc[k][0]);
        store_from_f32(op, d0 + 2 * pr + 1, acc[k][1]);
      }
    }
  } else if constexpr (kOut == DSA_FP4_E2M1) {
    // MXFP4: 32 dims (16 consecutive threads' pairs) share an E8M0 scale
    // 2^e, e = floor(log2(block max)) - 2, the elements the E2M1 codes of
    // c / 2^e (OCP MX conversion); dim 128 in the fp4 tile layout
    const bool tiled = D == 128;
    uint8_t* op = static_cast<uint8_t*>(out);
    const int64_t ro = erow;
#pragma unroll
    for (int k = 0; k < kCompressPairs; ++k) {
      const int pr = tid + k * kCompressThreads;
      const bool in = pr < npairs;
      float am = in ? fmaxf(fabsf(acc[k][0]), fabsf(acc[k][1])) : 0.f;
#pragma unroll
      for (int sh = 8; sh > 0; sh >>= 1) am = fmaxf(am, __shfl_xor(am, sh, 16));
      int se = -127;  // the block's scale exponent
      if (am > 0.f) {
        int ex;
        frexpf(am, &ex);  // am = f 2^ex, f in [0.5, 1)
        se = min(127, max(-127, ex - 3));
      }
      const float rsc = ldexpf(1.0f, -se);  // exact: a power of two
      if (in) {
        const uint32_t c0 = f32_to_fp4(acc[k][0] * rsc), c1 = f32_to_fp4(acc[k][1] * rsc);
        const int d = d0 + 2 * pr;
        const int64_t at = tiled ? idx4_tile_off_row(trow, d) : ro * (D / 2) + d / 2;
        op[at] = static_cast<uint8_t>(c0 | (c1 << 4));
        if ((d & 31) == 0) out_mx[ro * (D / 32) + d / 32] = static_cast<uint8_t>(se + 127);
      }
    }
  } else {  // fp8 e4m3fn, token-wise scale = amax / 448
    float am = 0.f;
#pragma unroll
    for (int k = 0; k < kCompressPairs; ++k)
      if (tid + k * kCompressThreads < npairs) am = fmaxf(am, fmaxf(fabsf(acc[k][0]), fabsf(acc[k][1])));
    am = block_max(am, red);
    const float sc = am / 448.0f;
    // dim 128: the 16-entry tile layout of the indexer keys; else row-major
    const bool tiled = D == 128;
    uint8_t* op = static_cast<uint8_t*>(out) + (tiled ? 0 : o);
#pragma unroll
    for (int k = 0; k < kCompressPairs; ++k) {
      const int pr = tid + k * kCompressThreads;
      if (pr < npairs) {
        const uint32_t c0 = sc > 0.f ? f32_to_fp8(acc[k][0] / sc) : 0u;
        const uint32_t c1 = sc > 0.f ? f32_to_fp8(acc[k][1] / sc) : 0u;
        const int64_t at = tiled ? idx_tile_off_row(trow, d0 + 2 * pr) : d0 + 2 * pr;
        *reinterpret_cast<uint16_t*>(op + at) = static_cast<uint16_t>(c0 | (c1 << 8));
      }
    }
    if (tid == 0) out_scale[erow] = sc;
  }
}


}  // namespace dsa
