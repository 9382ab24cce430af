// S3 + S4 for many query rows per sequence (a prefill chunk): the lightning
// indexer as a two-stage matrix-core contraction with an exact correction,
// and the per-row Top-k of the candidates it keeps.  The scores are those
// of "DeepSeek DSA、DeepSeek V4与vLLM Hybrid KV Cache详解" 4.1,
//   I[i, j] = ks_j * sum_h (w_ih * qs_ih) * ReLU(q8_ih . k8_j),
// and the result is the exact Top-k of them (ties to the lower index).
#include "common.h"
#include "indexer_impl.h"
#include "internal.h"
#include "select_impl.h"

namespace dsa {
namespace {

// ------------------------------------------------------------ prefill path
// Many query rows against one sequence's keys is a dense contraction.  It
// runs on the matrix cores in two stages, with an exact correction so that
// the selection stays the exact Top-k:
//
//  k_pidx_prep  (one workgroup per kPQ rows of one sequence): nu_j = ks_j
//     ||k8_j|| over a slice of the sequence's entries (the slice's largest
//     value); per row the error scale beta (below) and the threshold theta,
//     the r-th largest approximate score over a sample of whole 16-entry
//     tiles (r = 2k scaled to the sample, plus 8), rounded down to a 2^-16
//     fraction of the row's sampled key range.
//  k_pidx_main  (one workgroup per kMRows rows and a range of entry tiles;
//     the range's keys pass through LDS once for all of those rows): per
//     row and 16-entry tile, the fp8 MFMA with an E8M0 scale of 2^-9 gives
//     2^-9 q8_h . k8_j for the 16 heads; ReLU and rounding to f16; an f16
//     MFMA contracts them with the row's head weights w'_h = w_h qs_h
//     (rounded to f16 after a per-row power-of-two scaling that puts the
//     largest |w'_h| in [2^14, 2^15)), two rows per 32-deep product.  An
//     entry whose approximate score reaches theta - beta nu_max sets its bit
//     in the row's candidate mask (16 bits per tile).
//  k_pidx_select (one workgroup of kPSelT threads per row): the candidates
//     from the masks, their exact scores (bf16 MFMA on exactly widened codes
//     and f32 weights, as the decode path), the certificate #{candidates with
//     exact score >= theta} >= k, then the exact Top-k of the candidates.  If
//     the certificate fails or the candidates overflow LDS, the row is scored
//     exactly in full and selected from its scores.
//
// Why the result is exact: |approx_j - exact_j| <= beta nu_j <= beta nu_max
// (below).  A non-candidate therefore has exact_j < theta, while at least k
// candidates reach theta, so the k-th largest exact score is >= theta and
// every entry of the Top-k (ties to the lower index) is a candidate.  The
// sample only steers theta (how many candidates); the certificate carries
// the guarantee.
//
// The bound, per head h with N_h = ||q8_h|| ||k8_j|| (code units) and W =
// max_h |w'_h|: the fp8 MFMA errs by at most 2^-10 N_h (its shared
// alignment drops low-order product bits: measured up to 2^-13.4 N_h on
// heavy-tailed codes and 2^-15.5 on uniform ones); its 2^-9 scale is exact
// (bit for bit the unscaled result times 2^-9) and keeps every value within
// 128 * 448^2 * 2^-9 = 50176 < 65504, the f16 range; rounding to f16 (to
// nearest) adds 2^-11 of the value plus 2^-25 absolute (subnormals), 2^-16 in
// code units; the f16 weights add 2^-11 |w'_h| plus 2^-39 W; the f16 MFMA
// sums its exact products in f32 (measured 2^-24.5 of the sum of |products|)
// and the exact path's own f32 rounding is of the same order.  ReLU is
// 1-Lipschitz.  Summed over the heads:
//   |approx_j - exact_j| <= ks_j (1.96e-3 sum_h |w'_h| N_h
//                                 + 2^-15.9 sum_h |w'_h| + 2^-38.9 W sum_h N_h).
// A non-zero key has ||k8_j|| >= 2^-9 (the smallest e4m3 magnitude) and a
// zero key scores exactly 0 on both paths, so with
//   beta = 2e-3 sum_h |w'_h| ||q8_h|| + 2^-6 sum_h |w'_h| + 2^-38 W sum_h ||q8_h||
// the error is at most beta nu_j.  The per-row threshold is computed in
// double with a relative margin of 2^-20 and rounded down, which covers the
// f32 rounding of the comparison.
constexpr int kPQ = 8;              // rows per prep workgroup
constexpr int kPSampleTiles = 128;  // sampled 16-entry tiles per row
constexpr int kPSample = kPSampleTiles * 16;
constexpr float kPEps = 2.0e-3f;
constexpr int kMR = 8;                               // rows per main wave
constexpr int kMRows = 4 * kMR;                      // rows per main workgroup
constexpr int kMStage = 8;                           // tiles per LDS stage
constexpr int kMKeyBytes = kMStage * 16 * 128;       // the stage's keys
constexpr int kMStageBytes = kMKeyBytes + kMStage * 16 * 4;  // + their scales
constexpr int kMTargetWGs = 768;                     // three per compute unit
constexpr int kMScaleOne = 127;                      // E8M0 code of 1
constexpr int kPSelT = 256;                          // select threads per row
constexpr int kPCandCap = 3072;                      // candidates held in LDS
constexpr int kPTmpCap = 256;                        // threshold-bin members held in LDS
// (select's LDS stays under 40 KiB, so four rows run per compute unit)

struct PArgs {
  const uint8_t* q;
  const float* q_scale;
  const float* w;
  const uint8_t* keys;
  const float* k_scale;
  const int64_t* q_pos;
  int Tq, Hi, s, S, k, tiles_per_seq;
  int rg_per_seq, rg_total, tps_split;
  int64_t e_cap, nv_cap, max_pos_end, ld_t;
  float* theta;
  float* beta;
  float* nu_part;
  float* kappa_part;
  uint16_t* masks;
  uint8_t* keys_rm;  // [B, nv_cap, 128] fp8 keys, one 128-byte run per entry
  uint32_t* status;
};

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v8i as_v8i(uint4 lo, uint4 hi) {
  return v8i{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z),
             static_cast<int>(lo.w), static_cast<int>(hi.x), static_cast<int>(hi.y),
             static_cast<int>(hi.z), static_cast<int>(hi.w)};
}

// Sum of squares of the 16 e4m3 codes in one uint4 (exact products, f32 sum).
__device__ __forceinline__ float fp8x16_sumsq(uint4 v) {
  float s = 0.f;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v2f a = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), false);
    const v2f b = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), true);
    s = fmaf(a[0], a[0], s);
    s = fmaf(a[1], a[1], s);
    s = fmaf(b[0], b[0], s);
    s = fmaf(b[1], b[1], s);
  }
  return s;
}

// The prep tile's rows: sequence b, rows row0 .. row0 + nq - 1.
struct PTile {
  int b, t0, nq;
  int64_t row0;
};
__device__ __forceinline__ PTile p_tile(const PArgs& a, int tile) {
  PTile t;
  t.b = tile / a.tiles_per_seq;
  t.t0 = (tile % a.tiles_per_seq) * kPQ;
  t.nq = min(kPQ, a.Tq - t.t0);
  t.row0 = static_cast<int64_t>(t.b) * a.Tq + t.t0;
  return t;
}

// Per-lane operands of the prep tile's rows for the fp8 MFMA: A_q (lane =
// head n, bytes [16g, 16g+16) and [64+16g, 64+16g+16) of the head's 128, the
// same byte-to-k assignment as the keys), and w'_q for heads 4g .. 4g+3.
struct PRows {
  v8i a[kPQ];
  float wv[kPQ][4];
  int64_t nv[kPQ];
};
__device__ __forceinline__ void p_load_rows(const PArgs& a, const PTile& t, PRows& r) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int q = 0; q < kPQ; ++q) {
    uint4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    r.nv[q] = 0;
    if (q < t.nq) {
      const int64_t row = t.row0 + q;
      if (n < a.Hi) {
        const uint4* qp = reinterpret_cast<const uint4*>(a.q + (row * a.Hi + n) * 128);
        lo = qp[g];
        hi = qp[4 + g];
      }
      const RowInfo ri = row_info(a.q_pos, static_cast<int>(row), a.s, a.S, a.nv_cap,
                                  a.max_pos_end, nullptr, false);
      r.nv[q] = ri.ok ? ri.nv : 0;
    }
    r.a[q] = as_v8i(lo, hi);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g + i;
      float wq = 0.f;
      if (q < t.nq && h < a.Hi) {
        const int64_t o = (t.row0 + q) * a.Hi + h;
        wq = a.w[o] * (a.q_scale ? a.q_scale[o] : 1.0f);
      }
      r.wv[q][i] = wq;
    }
  }
}

// Sum four rows' partials over the 4 head groups (16-lane rows of the
// wave) with the gfx950 lane swaps: permlane32_swap(x, y) gives
// ([x lanes 0-31, y lanes 0-31], [x lanes 32-63, y lanes 32-63]) and
// permlane16_swap(x, y) gives ([x r0, y r0, x r2, y r2], [x r1, y r1, x r3,
// y r3]) for 16-lane rows r.  The result's row g holds, for entry n, the
// full score of row kPerm[g] of the four.
constexpr int kPerm[4] = {0, 2, 1, 3};
__device__ __forceinline__ float p_reduce4(float p0, float p1, float p2, float p3) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
  const float z = __uint_as_float(a[0]) + __uint_as_float(a[1]);  // lanes 0-31: p0, 32-63: p1
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(p2), __float_as_uint(p3), false, false);
  const float w = __uint_as_float(b[0]) + __uint_as_float(b[1]);  // lanes 0-31: p2, 32-63: p3
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(z), __float_as_uint(w), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Approximate scores (before the key scale) of all kPQ rows against the
// tile's 16 entries, in f32 on the VALU: lane (g, n) of s[h] holds row
// 4h + kPerm[g], entry n.  (Used on the threshold sample only.)
__device__ __forceinline__ void p_scores(const PRows& r, const v8i& kb, float (&s)[kPQ / 4]) {
  v4f c[kPQ];
#pragma unroll
  for (int q = 0; q < kPQ; ++q)
    c[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(r.a[q], kb, v4f{0.f, 0.f, 0.f, 0.f},
                                                           0, 0, 0, 0, 0, 0);
  float p[kPQ];
#pragma unroll
  for (int q = 0; q < kPQ; ++q)
    p[q] = r.wv[q][0] * fmaxf(c[q][0], 0.f) + r.wv[q][1] * fmaxf(c[q][1], 0.f) +
           r.wv[q][2] * fmaxf(c[q][2], 0.f) + r.wv[q][3] * fmaxf(c[q][3], 0.f);
#pragma unroll
  for (int h = 0; h < kPQ / 4; ++h) s[h] = p_reduce4(p[4 * h], p[4 * h + 1], p[4 * h + 2], p[4 * h + 3]);
}

// Value of row 4h + kPerm[g] from a per-row array (selects, no dynamic
// register index).
template <typename T>
__device__ __forceinline__ T p_pick(const T (&v)[kPQ], int h, int g) {
  const T a = v[4 * h], b = v[4 * h + 2], c = v[4 * h + 1], d = v[4 * h + 3];
  return g == 0 ? a : g == 1 ? b : g == 2 ? c : d;
}

__global__ __launch_bounds__(kThreads) void k_pidx_prep(PArgs a) {
  __shared__ uint32_t skey[kPQ][kPSample];
  __shared__ uint32_t hist[kPQ][256];
  __shared__ float fred[kThreads / 64], kred[kThreads / 64];
  __shared__ int64_t ired[kThreads / 64];
  __shared__ uint32_t pick[kPQ][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, g = lane >> 4;
  const PTile t = p_tile(a, blockIdx.x);
  // the largest n_vis over the whole sequence (sets the slices of nu)
  // (eight positions per thread and round, their loads out together)
  int64_t nvs = 0;
  for (int i0 = tid; i0 < a.Tq; i0 += 8 * kThreads) {
    int64_t mp[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kThreads;
      mp[u] = i < a.Tq ? a.q_pos[static_cast<int64_t>(t.b) * a.Tq + i] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (mp[u] >= 0 && mp[u] < a.max_pos_end) nvs = max(nvs, min(a.nv_cap, n_complete(mp[u], a.s, a.S)));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) nvs = max(nvs, static_cast<int64_t>(__shfl_xor(nvs, o, 64)));
  if (lane == 0) ired[wave] = nvs;
  __syncthreads();
  nvs = max(max(ired[0], ired[1]), max(ired[2], ired[3]));
  // nu over this tile's slice of [0, nvs): 4 threads per entry, 32 bytes each
  const int tps = a.tiles_per_seq, slice = blockIdx.x % tps;
  const int64_t per = (nvs + tps - 1) / tps;
  const int64_t e_lo = slice * per, e_hi = min(nvs, e_lo + per);
  const uint8_t* kb = a.keys + static_cast<int64_t>(t.b) * idx_e_pad(a.e_cap) * 128;
  const float* ksb = a.k_scale + static_cast<int64_t>(t.b) * a.e_cap;
  float nu = 0.f, kap = 0.f;
  for (int64_t e0 = e_lo; e0 < e_hi; e0 += kThreads / 4) {
    const int64_t e = e0 + tid / 4;
    float ss = 0.f;
    if (e < e_hi) {
      const uint4* kt = reinterpret_cast<const uint4*>(kb + (e & ~int64_t{15}) * 128);
      const int c = 2 * (tid & 3), en = static_cast<int>(e & 15);
      const uint4 x0 = kt[c * 16 + en], x1 = kt[(c + 1) * 16 + en];
      ss = fp8x16_sumsq(x0) + fp8x16_sumsq(x1);
      // the entry-contiguous copy the selection gathers from
      uint4* rm = reinterpret_cast<uint4*>(a.keys_rm + (static_cast<int64_t>(t.b) * a.nv_cap + e) * 128);
      rm[c] = x0;
      rm[c + 1] = x1;
    }
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    if (e < e_hi) {
      nu = fmaxf(nu, ksb[e] * sqrtf(ss));
      kap = fmaxf(kap, sqrtf(ss));
    }
  }
  nu = wave_max(nu);
  kap = wave_max(kap);
  if (lane == 0) {
    fred[wave] = nu;
    kred[wave] = kap;
  }
  // beta per row: thread -> row tid / 32, head (tid % 32) / 2, half tid % 2
  {
    const int q = tid / 32, h = (tid % 32) / 2, hf = tid % 2;
    float ss = 0.f, wabs = 0.f;
    if (q < t.nq && h < a.Hi) {
      const int64_t row = t.row0 + q;
      const uint4* qp = reinterpret_cast<const uint4*>(a.q + (row * a.Hi + h) * 128) + 4 * hf;
      ss = fp8x16_sumsq(qp[0]) + fp8x16_sumsq(qp[1]) + fp8x16_sumsq(qp[2]) + fp8x16_sumsq(qp[3]);
      const int64_t o = row * a.Hi + h;
      wabs = fabsf(a.w[o] * (a.q_scale ? a.q_scale[o] : 1.0f));
    }
    ss += __shfl_xor(ss, 1, 64);
    float c1 = hf == 0 ? wabs * sqrtf(ss) : 0.f;  // sum_h |w'_h| ||q8_h||
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) c1 += __shfl_xor(c1, o, 32);
    if (tid % 32 == 0 && q < t.nq) a.beta[t.row0 + q] = kPEps * c1;
  }
  __syncthreads();
  if (tid == 0) {
    a.nu_part[blockIdx.x] = fmaxf(fmaxf(fred[0], fred[1]), fmaxf(fred[2], fred[3]));
    a.kappa_part[blockIdx.x] = fmaxf(fmaxf(kred[0], kred[1]), fmaxf(kred[2], kred[3]));
  }
  // approximate scores of the sampled tiles T = st * i, i < ns_t (all 16
  // entries of each: 2 KiB of contiguous keys)
  PRows r;
  p_load_rows(a, t, r);
  int64_t nvt = 0;
#pragma unroll
  for (int q = 0; q < kPQ; ++q) nvt = max(nvt, r.nv[q]);
  const int64_t nst = (nvt + 15) / 16;
  const int64_t st = max<int64_t>(1, (nst + kPSampleTiles - 1) / kPSampleTiles);
  const int ns_t = static_cast<int>((nst + st - 1) / st);
  // sample tiles wave, wave + 4, ... with a ring of kPre tiles in flight;
  // the loads are unconditional (clamped to a valid tile) so that the
  // compiler can count them
  constexpr int kPre = 4;
  uint4 lo[kPre], hi[kPre];
  float ks[kPre];
  const int64_t tmax = max<int64_t>(0, static_cast<int64_t>(ns_t - 1) * st);
  const int64_t jks = max<int64_t>(0, nvt - 1);
  auto load = [&](int u, int ti) {
    const int64_t j = min<int64_t>(ti * st, tmax) * 16 + n;
    idx_load_chunks(kb, j, g, &lo[u], &hi[u]);
    ks[u] = ksb[min(j, jks)];
  };
  int64_t nvp[kPQ];
#pragma unroll
  for (int q = 0; q < kPQ; ++q) nvp[q] = r.nv[q];
  const int64_t nv0 = p_pick(nvp, 0, g), nv1 = p_pick(nvp, 1, g);
  if (ns_t > 0) {
#pragma unroll
    for (int u = 0; u < kPre; ++u) load(u, wave + 4 * u);
  }
  for (int t0 = wave; t0 < kPSampleTiles && ns_t > 0; t0 += 4 * kPre) {
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int ti = t0 + 4 * u;  // < kPSampleTiles: 4 kPre divides kPSampleTiles
      const v8i bk = as_v8i(lo[u], hi[u]);
      const float ksc = ks[u];
      load(u, min(ti + 4 * kPre, kPSampleTiles - 1));
      const int64_t j = static_cast<int64_t>(ti) * st * 16 + n;
      const bool in = ti < ns_t;
      float sv[kPQ / 4];
      p_scores(r, bk, sv);
      // lane (g, n) holds rows qa and 4 + qa, qa = kPerm[g], of sample ti*16+n
      const int qa = g == 0 ? 0 : g == 1 ? 2 : g == 2 ? 1 : 3;
      const uint32_t k0 = order_key(sv[0] * ksc), k1 = order_key(sv[1] * ksc);
      skey[qa][ti * 16 + n] = (in & (j < nv0)) ? k0 : 0u;
      skey[4 + qa][ti * 16 + n] = (in & (j < nv1)) ? k1 : 0u;
    }
  }
  __syncthreads();
  // theta: the r-th largest sampled key of each row, rounded down to a
  // 2^-16 fraction of the row's own key range [lo, hi] (two 8-bit histogram
  // passes over (key - lo), so the bins spread over the keys present rather
  // than over the few exponents they share); 32 threads per row.  A valid
  // key is never 0.
  const int q = tid / 32, l32 = tid % 32;
  int64_t nvq = 0;  // (r.nv is a register array: no dynamic index)
  if (q < t.nq) {
    const RowInfo ri = row_info(a.q_pos, static_cast<int>(t.row0 + q), a.s, a.S, a.nv_cap,
                                a.max_pos_end, nullptr, false);
    nvq = ri.ok ? ri.nv : 0;
  }
  uint32_t nsq = 0, klo = 0xffffffffu, khi = 0u;
#pragma unroll 8
  for (int i = l32; i < kPSample; i += 32) {
    const uint32_t key = skey[q][i];
    if (key != 0u) {
      ++nsq;
      klo = min(klo, key);
      khi = max(khi, key);
    }
  }
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) {
    nsq += static_cast<uint32_t>(__shfl_xor(static_cast<int>(nsq), o, 32));
    klo = min(klo, static_cast<uint32_t>(__shfl_xor(static_cast<int>(klo), o, 32)));
    khi = max(khi, static_cast<uint32_t>(__shfl_xor(static_cast<int>(khi), o, 32)));
  }
  uint32_t need = static_cast<uint32_t>(min<int64_t>(
      nsq, (2 * static_cast<int64_t>(a.k) * nsq + nvq - 1) / max<int64_t>(nvq, 1) + 8));
  // pass 0 bins (key - lo) >> s0, pass 1 the next (up to) 8 bits below
  const int s0 = nsq > 0 ? range_shift(khi - klo, 8) : 0;
  const int s1 = max(0, s0 - 8);
  uint32_t base = 0;  // (key - lo) of theta, bins resolved so far
  // (both passes run in every row: the barriers are workgroup-wide; a row
  // whose range fits 8 bits is resolved by pass 0 and skips pass 1's work)
  for (int pass = 0; pass < 2; ++pass) {
    const int sh = pass == 0 ? s0 : s1;
    const uint32_t bmask = pass == 0 ? 255u : (1u << (s0 - s1)) - 1u;
    const bool work = pass == 0 || s0 > 0;
    for (int i = l32; i < 256; i += 32) hist[q][i] = 0u;
    if (l32 == 0) pick[q][0] = pick[q][1] = 0u;
    __syncthreads();
    if (work) {
#pragma unroll 8
      for (int i = l32; i < kPSample; i += 32) {
        const uint32_t key = skey[q][i];
        const uint32_t d = key - klo;
        if (key != 0u && (pass == 0 || (d >> s0) == (base >> s0)))
          atomicAdd(&hist[q][(d >> sh) & bmask], 1u);
      }
    }
    __syncthreads();
    // lane l32 owns bins 255 - 8 l32 .. 248 - 8 l32 (descending)
    uint32_t c[8], sum = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      c[u] = hist[q][255 - 8 * l32 - u];
      sum += c[u];
    }
    uint32_t before = sum;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      const uint32_t x = static_cast<uint32_t>(__shfl_up(static_cast<int>(before), o, 32));
      if (l32 >= o) before += x;
    }
    before -= sum;  // exclusive
    if (work && need > 0 && before < need && before + sum >= need) {
      uint32_t acc = before;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (acc < need && acc + c[u] >= need) {
          pick[q][0] = 255u - 8u * l32 - u;
          pick[q][1] = acc;
        }
        acc += c[u];
      }
    }
    __syncthreads();
    base += pick[q][0] << sh;
    need -= pick[q][1];
    __syncthreads();
  }
  if (l32 == 0 && q < t.nq) {
    const int64_t row = t.row0 + q;
    // rows that keep every visible entry (or none) need no candidates
    const bool sel = nvq > a.k && nsq > 0;
    a.theta[row] = sel ? key_to_float(klo + base) : INFINITY;
  }
}

// Two f32 values in [-1, 1] to a packed f16 pair (round to nearest even)
// with ReLU: one v_cvt_pk_f16_f32 with its clamp to [0, 1].
__device__ __forceinline__ v2h relu_f16x2(float x, float y) {
  const v2h h = {static_cast<_Float16>(x), static_cast<_Float16>(y)};
  const v2h z = {static_cast<_Float16>(0.f), static_cast<_Float16>(0.f)};
  const v2h o = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
  return __builtin_elementwise_min(__builtin_elementwise_max(h, z), o);
}
__device__ __forceinline__ v8h cat_f16(v2h a, v2h b, v2h c, v2h d) {
  const v4h ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const v4h cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Scaled fp8 product A B, A's per-row E8M0 code in byte `byte` of sa (a
// constant once the caller's loop is unrolled).
__device__ __forceinline__ v4f mfma_scaled(const v8i& A, const v8i& B, int sa, int byte) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  switch (byte) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, z, 0, 0, 0, sa, 0, kMScaleOne);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, z, 0, 0, 1, sa, 0, kMScaleOne);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, z, 0, 0, 2, sa, 0, kMScaleOne);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, z, 0, 0, 3, sa, 0, kMScaleOne);
  }
}

// v_writelane_b32: lane L of x takes the wave-uniform value v (no clang
// builtin here; the lane select is an immediate, so no lane-select hazard).
template <int L>
__device__ __forceinline__ void write_lane(uint32_t& x, uint32_t v) {
  asm("v_writelane_b32 %0, %1, %2" : "+v"(x) : "s"(v), "n"(L));
}
// Words wd[r] (r = row of the wave) to lanes 4 r + TP.
template <int TP>
__device__ __forceinline__ void put_words(uint32_t& x, const uint32_t (&wd)[8]) {
  write_lane<0 + TP>(x, wd[0]);
  write_lane<4 + TP>(x, wd[1]);
  write_lane<8 + TP>(x, wd[2]);
  write_lane<12 + TP>(x, wd[3]);
  write_lane<16 + TP>(x, wd[4]);
  write_lane<20 + TP>(x, wd[5]);
  write_lane<24 + TP>(x, wd[6]);
  write_lane<28 + TP>(x, wd[7]);
}

// A float rounded toward -inf (x finite).
__device__ __forceinline__ float round_down_f32(double x) {
  float f = static_cast<float>(x);
  if (static_cast<double>(f) > x) f = nextafterf(f, -INFINITY);
  return f;
}

__global__ __launch_bounds__(kThreads, 3) void k_pidx_main(PArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t stg[3][kMStageBytes];
  __shared__ float fred[kThreads / 64], kred[kThreads / 64];
  __shared__ int64_t nred[kThreads / 64];
  __shared__ int csh[kThreads / 64][kMR][16];  // per-head scale exponents
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, g = lane >> 4;
  // workgroup -> (tile range, row group): the workgroups of one XCD
  // (blockIdx mod 8) take consecutive linear ids, i.e. one tile range, so
  // that XCD's L2 holds only that range's keys
  const int G = gridDim.x;
  const int lin = (G & 7) == 0 ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  const int split = lin / a.rg_total, rg = lin % a.rg_total;
  const int b = rg / a.rg_per_seq, r0 = (rg % a.rg_per_seq) * kMRows;
  const int nq = min(kMRows, a.Tq - r0);
  const int64_t row0 = static_cast<int64_t>(b) * a.Tq + r0;
  const int wr0 = wave * kMR;  // the wave's rows wr0 .. wr0 + 7 of the workgroup
  // every load of the set-up that depends on no other goes out first (one
  // memory round trip instead of a chain of four): the wave's rows' query
  // codes, their head weights (all heads of row n for lanes n < kMR) and the
  // thresholds and error scales of rows 4 (g & 1) + i (lanes g < 2); rows
  // past the group read row 0 of it and are masked below
  uint4 qlo_r[kMR], qhi_r[kMR];
#pragma unroll
  for (int q = 0; q < kMR; ++q) {
    const int64_t rq = row0 + (wr0 + q < nq ? wr0 + q : 0);
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + (rq * a.Hi + (n < a.Hi ? n : 0)) * 128);
    qlo_r[q] = qp[g];
    qhi_r[q] = qp[4 + g];
  }
  float wl_r[4];  // heads 4g .. 4g+3 of row n (lanes n < kMR)
  {
    const int64_t rq = row0 + (n < kMR && wr0 + n < nq ? wr0 + n : 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g + i;
      const int64_t o = rq * a.Hi + (h < a.Hi ? h : 0);
      wl_r[i] = a.w[o] * (a.q_scale ? a.q_scale[o] : 1.0f);
    }
  }
  float th_r[4], be_r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qd = 4 * (g & 1) + i;
    const int64_t rq = row0 + (wr0 + qd < nq ? wr0 + qd : 0);
    th_r[i] = a.theta[rq];
    be_r[i] = a.beta[rq];
  }
  // nu_max and kappa = max_j ||k8_j|| of the sequence; the workgroup's
  // largest n_vis
  float nu = 0.f, kap = 0.f;
  for (int i = tid; i < a.tiles_per_seq; i += kThreads) {
    nu = fmaxf(nu, a.nu_part[static_cast<int64_t>(b) * a.tiles_per_seq + i]);
    kap = fmaxf(kap, a.kappa_part[static_cast<int64_t>(b) * a.tiles_per_seq + i]);
  }
  nu = wave_max(nu);
  kap = wave_max(kap);
  int64_t nvm = 0;
  if (tid < nq) {
    const RowInfo ri = row_info(a.q_pos, static_cast<int>(row0 + tid), a.s, a.S, a.nv_cap,
                                a.max_pos_end, nullptr, false);
    nvm = ri.ok ? ri.nv : 0;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) nvm = max(nvm, static_cast<int64_t>(__shfl_xor(nvm, o, 64)));
  if (lane == 0) {
    fred[wave] = nu;
    kred[wave] = kap;
    nred[wave] = nvm;
  }
  __syncthreads();
  nu = fmaxf(fmaxf(fred[0], fred[1]), fmaxf(fred[2], fred[3]));
  kap = fmaxf(fmaxf(kred[0], kred[1]), fmaxf(kred[2], kred[3]));
  nvm = max(max(nred[0], nred[1]), max(nred[2], nred[3]));
  const int64_t t_lo = static_cast<int64_t>(split) * a.tps_split;
  const int64_t t_hi = min((nvm + 15) / 16, t_lo + a.tps_split);
  if (t_lo >= t_hi) return;  // the whole workgroup: no barrier follows
  const uint8_t* kb = a.keys + static_cast<int64_t>(b) * idx_e_pad(a.e_cap) * 128;
  const float* ksb = a.k_scale + static_cast<int64_t>(b) * a.e_cap;
  const int nst = static_cast<int>((t_hi - t_lo + kMStage - 1) / kMStage);
  // one stage: 16 KiB of keys (contiguous in the tile layout) and 128
  // scales, clamped to the range
  // (thread t loads bytes 16 (t % 128) of tiles 2u + t / 128; 32-bit
  // offsets: one sequence's keys are far below 4 GiB)
  const uint32_t lane_off = 16u * static_cast<uint32_t>(tid & 127);
  const int hb = tid >> 7;
  auto gload = [&](int s, u32x4 (&rk)[4], float& rks) {
    const int t0 = static_cast<int>(t_lo) + s * kMStage;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t tile = static_cast<uint32_t>(min(t0 + 2 * u + hb, static_cast<int>(t_hi) - 1));
      rk[u] = *reinterpret_cast<const u32x4*>(kb + (tile * 2048u + lane_off));
    }
    rks = ksb[min(static_cast<int64_t>(t0) * 16 + (tid & 127), a.e_cap - 1)];
  };
  auto swrite = [&](int buf, const u32x4 (&rk)[4], float rks) {
    uint8_t* d = stg[buf];
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<u32x4*>(d + 16 * (tid + kThreads * u)) = rk[u];
    if (tid < 128) reinterpret_cast<float*>(d + kMKeyBytes)[tid] = rks;
  };
  // the first two stages' loads are in flight while the operands are set up
  u32x4 rk0[4], rk1[4];
  float rks0, rks1;
  gload(0, rk0, rks0);
  gload(min(1, nst - 1), rk1, rks1);
  // stage-1 operands: lane = head n, chunks g and 4 + g of each row, and the
  // E8M0 code of 2^-c for head n: 2^c >= 2 ||q8_n|| kappa (with a margin for
  // the f32 norms), so |2^-c q8_n . k8_j| <= 1/2 (1 + 2^-10) for every entry
  // even after the fp8 MFMA's error, and 2^c < 4 ||q8_n|| kappa
  v8i A[kMR];
  int sa[kMR / 4];  // four E8M0 codes per register, row q in byte q % 4
#pragma unroll
  for (int q = 0; q < kMR; ++q) {
    uint4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (wr0 + q < nq && n < a.Hi) {
      lo = qlo_r[q];
      hi = qhi_r[q];
    }
    A[q] = as_v8i(lo, hi);
    float ss = fp8x16_sumsq(lo) + fp8x16_sumsq(hi);
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    int c = 0;
    const float x = 2.0f * sqrtf(ss) * kap * (1.0f + 0x1p-20f);
    if (x > 0.f) frexpf(x, &c);  // x = f 2^c, f in [0.5, 1)
    const int code = kMScaleOne - c;
    if ((q & 3) == 0) sa[q >> 2] = code;
    else sa[q >> 2] |= code << (8 * (q & 3));
    if (g == 0) csh[wave][q][n] = c;
  }
  // stage-2 operands: lane (g, m), m < 8, holds row m's weights for heads
  // 4g .. 4g+3 at k = 8g .. 8g+3 (m even) or 8g+4 .. 8g+7 (m odd) of pair
  // m / 2: w'_h 2^(c_h + e_m), with e_m putting the row's largest
  // |w'_h 2^c_h| in [2^14, 2^15)
  int e_row = 0;
  v8h a2m = {};
  // the row's largest |w'_h 2^c_h|: lane (g, n) takes heads 4g .. 4g+3 of
  // row n, then the max over the four head groups (lanes n, n+16, n+32, n+48)
  float wmax = 0.f, wq[4] = {0.f, 0.f, 0.f, 0.f};
  int cq[4] = {0, 0, 0, 0};
  if (n < kMR && wr0 + n < nq) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g + i;
      if (h < a.Hi) {  // (Hi <= 16)
        wq[i] = wl_r[i];
        cq[i] = csh[wave][n][h];
        wmax = fmaxf(wmax, ldexpf(fabsf(wq[i]), cq[i]));
      }
    }
  }
  wmax = fmaxf(wmax, __shfl_xor(wmax, 16, 64));
  wmax = fmaxf(wmax, __shfl_xor(wmax, 32, 64));
  if (n < kMR) {
    if (wmax > 0.f && wmax <= 3.0e38f) {
      int ex;
      frexpf(wmax, &ex);  // wmax = f 2^ex, f in [0.5, 1)
      e_row = 15 - ex;
    }
    v2h w01 = {static_cast<_Float16>(ldexpf(wq[0], cq[0] + e_row)),
               static_cast<_Float16>(ldexpf(wq[1], cq[1] + e_row))};
    v2h w23 = {static_cast<_Float16>(ldexpf(wq[2], cq[2] + e_row)),
               static_cast<_Float16>(ldexpf(wq[3], cq[3] + e_row))};
    const v2h z = {};
    a2m = (n & 1) ? cat_f16(z, z, w01, w23) : cat_f16(w01, w23, z, z);
  }
  v8h A2[kMR / 2];
#pragma unroll
  for (int p = 0; p < kMR / 2; ++p) A2[p] = (n < kMR && (n >> 1) == p) ? a2m : v8h{};
  // lane (g, n), g < 2, rows 4g + i, in units of 2^e per score unit: the
  // threshold (theta - beta nu_max, less a 2^-20 margin, rounded down) and
  // the stage-2 accumulator's start gamma kappa (rounded up), gamma = 2^-22 /
  // kPEps * beta, which covers the f16 subnormal error
  float thr[4], g0[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qd = 4 * (g & 1) + i;
    const int e_q = __shfl(e_row, qd, 64);
    thr[i] = INFINITY;
    g0[i] = 0.f;
    if (g < 2 && wr0 + qd < nq) {
      const float th = th_r[i];
      const double be = static_cast<double>(be_r[i]);
      if (th < INFINITY) {
        const double bn = be * nu;
        double d = static_cast<double>(th) - bn;
        d -= 0x1p-20 * (fabs(static_cast<double>(th)) + bn);
        thr[i] = round_down_f32(ldexp(d, e_q));
        g0[i] = -round_down_f32(-ldexp(be * (0x1p-22 / kPEps) * kap, e_q));
      }
    }
  }
  swrite(0, rk0, rks0);
  swrite(1, rk1, rks1);
  __syncthreads();
  // mask store: lane L < 32 writes row L / 4 of the wave, tiles 2 (L % 4)
  // and 2 (L % 4) + 1 of the stage (one u32)
  const bool st_ok = lane < 32 && wr0 + (lane >> 2) < nq;
  uint32_t* mst = reinterpret_cast<uint32_t*>(a.masks + (row0 + wr0 + (lane >> 2)) * a.ld_t);
  int buf = 0;
  for (int s = 0; s < nst; ++s) {
    // the three workgroups sharing a compute unit keep pace: a wave's
    // priority falls with each quarter of its stages (left alone, the
    // oldest workgroup takes most issue slots and the last one runs its
    // final stretch with one wave per SIMD)
    {
      const int qtr = (4 * s) / nst;
      if (qtr == 0) __builtin_amdgcn_s_setprio(3);
      else if (qtr == 1) __builtin_amdgcn_s_setprio(2);
      else if (qtr == 2) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    u32x4 rk[4];
    float rks;
    gload(min(s + 2, nst - 1), rk, rks);
    const uint8_t* sb = stg[buf];
    uint32_t wout = 0u;
#pragma unroll
    for (int tp = 0; tp < kMStage / 2; ++tp) {
      uint64_t mk[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int tt = 2 * tp + h;
        const uint4 klo = *reinterpret_cast<const uint4*>(sb + tt * 2048 + 16 * lane);
        const uint4 khi = *reinterpret_cast<const uint4*>(sb + tt * 2048 + 1024 + 16 * lane);
        const float ksn = reinterpret_cast<const float*>(sb + kMKeyBytes)[tt * 16 + n];
        const v8i B = as_v8i(klo, khi);
        v4f c[kMR];
#pragma unroll
        for (int q = 0; q < kMR; ++q)
          c[q] = mfma_scaled(A[q], B, sa[q >> 2], q & 3);
        v4f c2 = {g0[0], g0[1], g0[2], g0[3]};
#pragma unroll
        for (int p = 0; p < kMR / 2; ++p) {
          const v8h b2 = cat_f16(relu_f16x2(c[2 * p][0], c[2 * p][1]), relu_f16x2(c[2 * p][2], c[2 * p][3]),
                                 relu_f16x2(c[2 * p + 1][0], c[2 * p + 1][1]),
                                 relu_f16x2(c[2 * p + 1][2], c[2 * p + 1][3]));
          c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A2[p], b2, c2, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) mk[h][i] = __ballot(c2[i] * ksn >= thr[i]);
      }
      // row i of the wave: bits 0-15 of mk[.][i]; row 4 + i: bits 16-31;
      // the words go to lanes 4 row + tp
      uint32_t wd[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wd[i] = static_cast<uint32_t>(mk[0][i] & 0xffffu) | (static_cast<uint32_t>(mk[1][i] & 0xffffu) << 16);
        wd[4 + i] = static_cast<uint32_t>((mk[0][i] >> 16) & 0xffffu) |
                    (static_cast<uint32_t>(mk[1][i]) & 0xffff0000u);
      }
      if (tp == 0) put_words<0>(wout, wd);
      if (tp == 1) put_words<1>(wout, wd);
      if (tp == 2) put_words<2>(wout, wd);
      if (tp == 3) put_words<3>(wout, wd);
    }
    if (st_ok) mst[((t_lo + static_cast<int64_t>(s) * kMStage) >> 1) + (lane & 3)] = wout;
    swrite(buf == 0 ? 2 : buf - 1, rk, rks);  // (s + 2) % 3
    __syncthreads();
    buf = buf == 2 ? 0 : buf + 1;
  }
}

__global__ __launch_bounds__(kPSelT) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_pidx_select(PArgs a, float* __restrict__ scores,
                                                        int64_t ld_scores,
                                                        int32_t* __restrict__ idx_out) {
  __shared__ uint64_t cand_s[kPCandCap];
  __shared__ uint64_t tmp_s[kPTmpCap];
  __shared__ uint32_t h_s[2048];
  constexpr int kW = kPSelT / 64;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int b = row / a.Tq;
  const RowInfo ri = row_info(a.q_pos, row, a.s, a.S, a.nv_cap, a.max_pos_end, a.status, tid == 0);
  const int64_t nv = ri.ok ? ri.nv : 0;
  int32_t* irow = idx_out + static_cast<int64_t>(row) * a.k;
  if (nv <= a.k) {
    emit_all_visible(nullptr, nv, a.k, irow, nullptr);
    return;
  }
  const float theta = a.theta[row];
  // the candidates, in index order, from the row's masks: 8 tiles per
  // thread and pass, block prefix sums for the slots
  const uint16_t* mrow = a.masks + static_cast<int64_t>(row) * a.ld_t;
  const int64_t ntl = (nv + 15) / 16;
  const uint32_t tail = static_cast<uint32_t>(nv & 15);
  __shared__ uint32_t cnt_s;
  uint32_t cnt = 0;
  for (int64_t t0 = 0; t0 < ntl; t0 += 8 * kPSelT) {
    const int64_t tb = t0 + 8 * tid;
    uint32_t m[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if (tb < ntl) {
      const uint4 v = *reinterpret_cast<const uint4*>(mrow + tb);  // ld_t, tb multiples of 8
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m[2 * i] = w4[i] & 0xffffu;
        m[2 * i + 1] = w4[i] >> 16;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t tt = tb + i;
        if (tt >= ntl) m[i] = 0u;
        else if (tt == ntl - 1 && tail != 0u) m[i] &= (1u << tail) - 1u;
      }
    }
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) c += __popc(m[i]);
    uint32_t total;
    uint32_t pos = cnt + block_prefix_excl<kPSelT>(c, &total);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t mm = m[i];
      while (mm) {
        const int bit = __ffs(static_cast<int>(mm)) - 1;
        mm &= mm - 1u;
        if (pos < static_cast<uint32_t>(kPCandCap))
          cand_s[pos] = static_cast<uint64_t>((tb + i) * 16 + bit);
        ++pos;
      }
    }
    cnt += total;
  }
  if (tid == 0) cnt_s = cnt;
  __syncthreads();
  cnt = cnt_s;
  v8bf aq[4];
  float wv[4];
  exact_row_operands<DSA_FP8_E4M3>(a.q, a.q_scale, a.w, row, a.Hi, aq, wv);
  const uint8_t* kb = a.keys + static_cast<int64_t>(b) * idx_e_pad(a.e_cap) * 128;
  const uint8_t* krm = a.keys_rm + static_cast<int64_t>(b) * a.nv_cap * 128;
  const float* ksb = a.k_scale + static_cast<int64_t>(b) * a.e_cap;
  bool ok = cnt <= static_cast<uint32_t>(kPCandCap) && theta < INFINITY;
  if (ok) {
    const int ct = static_cast<int>((cnt + 15) / 16);
    uint32_t c_ge = 0;
    // six tiles per step: their indices, then their keys, then the math,
    // so that a step costs one memory round trip (the indices are in LDS);
    // six keeps the kernel within 128 VGPRs (four waves per SIMD)
    constexpr int kU = 6;
    for (int t0 = wave; t0 < ct; t0 += kU * kW) {
      int64_t j[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = (t0 + u * kW) * 16 + n;
        j[u] = i < static_cast<int>(cnt) ? static_cast<int64_t>(cand_s[i]) : -1;
      }
      uint4 blo[kU], bhi[kU];
      float ks[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t jj = j[u] >= 0 ? j[u] : 0;
        const uint4* rm = reinterpret_cast<const uint4*>(krm + jj * 128);
        blo[u] = rm[g];
        bhi[u] = rm[4 + g];
        ks[u] = 0.f;
      }
      // the score is whole in every lane and lanes g == 0 keep it, so only
      // they load the key scales (a gather's cost follows its active lanes)
      if (g == 0) {
#pragma unroll
        for (int u = 0; u < kU; ++u) ks[u] = ksb[j[u] >= 0 ? j[u] : 0];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = (t0 + u * kW) * 16 + n;
        v8bf bo[4];
        KeyOps<DSA_FP8_E4M3>::operands(KeyOps<DSA_FP8_E4M3>::Raw{blo[u], bhi[u], ks[u]}, bo);
        const float sc = exact_tile_score(aq, wv, bo) * ks[u];
        if (g == 0 && i < ct * 16) {
          cand_s[i] = j[u] >= 0 ? composite(order_key(sc), static_cast<uint32_t>(j[u])) : 0ull;
          c_ge += (j[u] >= 0 && sc >= theta) ? 1u : 0u;
        }
      }
    }
    ok = block_reduce_u32<2, kPSelT>(c_ge) >= static_cast<uint32_t>(a.k);  // barriers
  }
  if (ok) {
    select_topk_composites<kPSelT, kPTmpCap>(cand_s, static_cast<int>(cnt), static_cast<uint32_t>(a.k),
                                             irow, nullptr, tmp_s, h_s);
    return;
  }
  // fallback: score the whole row exactly, then select from the scores
  float* srow = scores + static_cast<int64_t>(row) * ld_scores;
  score_row_exact<DSA_FP8_E4M3>(aq, wv, KeySrc{kb, ksb, nullptr, PageMap{}, b, nullptr}, nv, srow,
                                kW);
  __syncthreads();
  row_select_from_scores<kPCandCap, kPSelT, 11>(srow, nv, a.k, irow, nullptr, cand_s, h_s);
}

// Workspace of the path (after the per-row scores it shares with the other
// paths as the fallback buffer).
struct PLayout {
  int tps, tiles, rg_per_seq, rg_total, nsplit, tps_split;
  int64_t ld_t;
  size_t off_theta, off_beta, off_nu, off_kappa, off_masks, off_krm, total;
};

PLayout playout(const dsa_index_args& a, int64_t nv_cap) {
  PLayout p{};
  const int64_t rows = static_cast<int64_t>(a.n_seqs) * a.queries_per_seq;
  p.tps = static_cast<int>(ceil_div(a.queries_per_seq, kPQ));
  p.tiles = a.n_seqs * p.tps;
  // main: row groups of kMRows times tile ranges (multiples of one LDS
  // stage), aiming at three workgroups per compute unit with >= 8 stages
  // each
  p.rg_per_seq = static_cast<int>(ceil_div(a.queries_per_seq, kMRows));
  p.rg_total = a.n_seqs * p.rg_per_seq;
  const int64_t ntl = ceil_div(nv_cap, 16);
  p.ld_t = ceil_div(ntl, kMStage) * kMStage;
  const int64_t ns = std::max<int64_t>(
      1, std::min<int64_t>(ceil_div(kMTargetWGs, std::max(1, p.rg_total)), ntl / (8 * kMStage)));
  p.tps_split = static_cast<int>(ceil_div(ceil_div(ntl, ns), kMStage) * kMStage);
  p.nsplit = static_cast<int>(ceil_div(ntl, std::max(1, p.tps_split)));
  size_t off = 0;
  p.off_theta = off;
  off = align_up(off + static_cast<size_t>(rows) * sizeof(float));
  p.off_beta = off;
  off = align_up(off + static_cast<size_t>(rows) * sizeof(float));
  p.off_nu = off;
  off = align_up(off + static_cast<size_t>(p.tiles) * sizeof(float));
  p.off_kappa = off;
  off = align_up(off + static_cast<size_t>(p.tiles) * sizeof(float));
  p.off_masks = off;
  off = align_up(off + static_cast<size_t>(rows) * p.ld_t * sizeof(uint16_t));
  p.off_krm = off;
  off = align_up(off + static_cast<size_t>(a.n_seqs) * nv_cap * 128);
  p.total = off;
  return p;
}

}  // namespace

bool prefill_index_applies(const dsa_index_args& a, int64_t nv_cap) {
  const int64_t rows = static_cast<int64_t>(a.n_seqs) * a.queries_per_seq;
  const bool mfma = a.keys != nullptr && a.dtype == DSA_FP8_E4M3 && a.dim == 128 && a.heads <= 16;
  return mfma && a.score_out == nullptr && rows >= 512 && a.queries_per_seq >= 64 && nv_cap > a.k;
}

size_t prefill_index_ws_bytes(const dsa_index_args& a, int64_t nv_cap) {
  return playout(a, nv_cap).total;
}

dsa_status launch_prefill_index_topk(const dsa_index_args& a, int64_t nv_cap, float* scores,
                                     int64_t ld, void* ws, hipStream_t st) {
  const PLayout P = playout(a, nv_cap);
  const int rows = a.n_seqs * a.queries_per_seq;
  char* base = static_cast<char*>(ws);
  PArgs pa{};
  pa.q = static_cast<const uint8_t*>(a.q);
  pa.q_scale = a.q_scale;
  pa.w = a.w;
  pa.keys = static_cast<const uint8_t*>(a.keys);
  pa.k_scale = a.k_scale;
  pa.q_pos = a.q_pos;
  pa.Tq = a.queries_per_seq;
  pa.Hi = a.heads;
  pa.s = a.stride;
  pa.S = a.span;
  pa.k = a.k;
  pa.tiles_per_seq = P.tps;
  pa.rg_per_seq = P.rg_per_seq;
  pa.rg_total = P.rg_total;
  pa.tps_split = P.tps_split;
  pa.e_cap = a.e_cap;
  pa.nv_cap = nv_cap;
  pa.max_pos_end = a.max_pos_end;
  pa.ld_t = P.ld_t;
  pa.theta = reinterpret_cast<float*>(base + P.off_theta);
  pa.beta = reinterpret_cast<float*>(base + P.off_beta);
  pa.nu_part = reinterpret_cast<float*>(base + P.off_nu);
  pa.kappa_part = reinterpret_cast<float*>(base + P.off_kappa);
  pa.masks = reinterpret_cast<uint16_t*>(base + P.off_masks);
  pa.keys_rm = reinterpret_cast<uint8_t*>(base + P.off_krm);
  pa.status = a.status;
  const hipEvent_t e0 = call_timing().index0, e1 = call_timing().index1;
  launch_timed(k_pidx_prep, dim3(P.tiles), dim3(kThreads), 0, st, e0, nullptr, pa);
  dsa_status rc = hip_check(hipGetLastError(), "k_pidx_prep launch");
  if (rc != DSA_OK) return rc;
  hipLaunchKernelGGL(k_pidx_main, dim3(P.rg_total * P.nsplit), dim3(kThreads), 0, st, pa);
  rc = hip_check(hipGetLastError(), "k_pidx_main launch");
  if (rc != DSA_OK) return rc;
  launch_timed(k_pidx_select, dim3(rows), dim3(kPSelT), 0, st, nullptr, e1, pa, scores, ld,
               a.idx_out);
  return hip_check(hipGetLastError(), "k_pidx_select launch");
}

}  // namespace dsa
