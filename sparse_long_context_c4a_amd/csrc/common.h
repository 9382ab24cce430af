// Device-side helpers shared by the gfx950 kernels: storage-format
// conversions, rotary angles, wave64 reductions, error words.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

constexpr int kWave = 64;

// ------------------------------------------------------------ formats

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even; NaN stays a quiet NaN, overflow becomes inf.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// OCP e4m3fn code -> float (exact).
__device__ __forceinline__ float fp8_to_f32(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 0xfu, m = c & 7u;
  if (e == 0) return __uint_as_float(sign | __float_as_uint(static_cast<float>(m) * 0x1p-9f));
  if (e == 15 && m == 7) return __uint_as_float(0x7fc00000u);
  return __uint_as_float(sign | ((e + 120u) << 23) | (m << 20));
}

// float -> OCP e4m3fn code, round to nearest even, saturating at +-448.
// Works on the binary32 bit pattern: below 2^-6 the grid is spaced 2^-9;
// above, the 23-bit fraction is rounded to 3 bits at bit 20.
__device__ __forceinline__ uint32_t f32_to_fp8(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t ua = u & 0x7fffffffu;
  if (ua > 0x7f800000u) return 0x7fu;             // NaN
  if (ua >= 0x43e80000u) return sign | 0x7eu;     // |x| >= 464 (incl. inf)
  if (ua < 0x3c800000u) {                          // |x| < 2^-6
    const float q = rintf(__uint_as_float(ua) * 512.0f);  // 0..8
    return sign | static_cast<uint32_t>(q);
  }
  const uint32_t r = (ua + 0x7ffffu + ((ua >> 20) & 1u)) & 0xfff00000u;
  const uint32_t ef = (r >> 23) - 120u;            // biased e4m3 exponent, 1..15
  const uint32_t m = (r >> 20) & 7u;
  if (ef > 15u || (ef == 15u && m == 7u)) return sign | 0x7eu;
  return sign | (ef << 3) | m;
}

// float -> OCP MX FP4 (E2M1) code: the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6
// with ties to the even code (mantissa bit 0), saturating at 6; the sign
// bit (8) is set for negative inputs.
__device__ __forceinline__ uint32_t f32_to_fp4(float x) {
  const float a = fabsf(x);
  uint32_t c;
  if (a <= 0.25f) c = 0u;
  else if (a < 0.75f) c = 1u;
  else if (a <= 1.25f) c = 2u;
  else if (a < 1.75f) c = 3u;
  else if (a <= 2.5f) c = 4u;
  else if (a < 3.5f) c = 5u;
  else if (a <= 5.0f) c = 6u;
  else c = 7u;
  return c | ((__float_as_uint(x) >> 28) & 8u);
}

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

template <typename T>
__device__ __forceinline__ void store_from_f32(T* p, int64_t i, float v);
template <>
__device__ __forceinline__ void store_from_f32<float>(float* p, int64_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void store_from_f32<uint16_t>(uint16_t* p, int64_t i, float v) {
  p[i] = f32_to_bf16(v);
}

// --------------------------------------------------------------- RoPE
// cos / sin of (pos * base^(-2i/r)).  The angle is formed and reduced modulo
// 2 pi in fp64 (two-term Cody-Waite with a double-double 2 pi), so that
// positions near 2^20 keep full accuracy; the reduced angle in [-pi, pi]
// then goes through fp32 sincos.
__device__ __forceinline__ void rope_cs(int64_t pos, int i, int r, double base, float* c,
                                        float* s) {
  const double theta = pow(base, -2.0 * static_cast<double>(i) / static_cast<double>(r));
  const double ang = static_cast<double>(pos) * theta;
  const double kq = rint(ang * 0.15915494309189533577);             // 1 / (2 pi)
  double red = fma(-kq, 6.28318530717958623200, ang);                // 2 pi, high part
  red = fma(-kq, 2.44929359829470635445e-16, red);                   // 2 pi, low part
  sincosf(static_cast<float>(red), s, c);
}

// The same from theta1 = base^(-2/r) computed once on the host: theta_i =
// theta1^i by repeated squaring (at most 2 log2(i) double products, relative
// error ~1e-15 against base^(-2i/r): an angle error of ~1e-8 rad at position
// 2^21, far below the single-precision sin/cos), instead of a double pow
// per pair on the kernel's critical path.
__device__ __forceinline__ void rope_cs1(int64_t pos, int i, double theta1, float* c, float* s) {
  double theta = 1.0, b = theta1;
  for (int e = i; e != 0; e >>= 1) {
    if (e & 1) theta *= b;
    b *= b;
  }
  const double ang = static_cast<double>(pos) * theta;
  const double kq = rint(ang * 0.15915494309189533577);             // 1 / (2 pi)
  double red = fma(-kq, 6.28318530717958623200, ang);                // 2 pi, high part
  red = fma(-kq, 2.44929359829470635445e-16, red);                   // 2 pi, low part
  sincosf(static_cast<float>(red), s, c);
}

// ------------------------------------------------ indexer key tile layout
// fp8 caches of dim 128 (the indexer keys) are stored in tiles of 16
// entries: tile t of sequence b holds entries 16t .. 16t+15 as 8 chunks of
// 16 dims, chunk-major, each chunk the 16 entries' 16 bytes in entry order.
// A wave that gives lane (g, n) chunk g (or 4 + g) of entry n -- the
// matrix-core operand layout -- then reads 1 KiB of contiguous bytes per
// load instruction.  Sequences are e_pad = ceil(e_cap / 16) * 16 entries
// apart.
__host__ __device__ __forceinline__ int64_t idx_e_pad(int64_t e_cap) { return (e_cap + 15) & ~int64_t{15}; }
// Byte offset of dim d of entry j of sequence b.
__host__ __device__ __forceinline__ int64_t idx_tile_off(int64_t b, int64_t e_pad, int64_t j, int d) {
  return (b * e_pad + (j & ~int64_t{15})) * 128 + (d >> 4) * 256 + (j & 15) * 16 + (d & 15);
}
// The same by tile row R (dense: b * e_pad + j; paged: the entry's pool row,
// blocks being whole tiles).
__host__ __device__ __forceinline__ int64_t idx_tile_off_row(int64_t R, int d) {
  return (R & ~int64_t{15}) * 128 + (d >> 4) * 256 + (R & 15) * 16 + (d & 15);
}
// The two 16-byte operand chunks of lane (g, n) for entry j (n = j mod 16
// in the operand layout): chunks g and 4 + g.
__device__ __forceinline__ void idx_load_chunks(const uint8_t* seq_keys, int64_t j, int g, uint4* lo,
                                                uint4* hi) {
  const uint4* t = reinterpret_cast<const uint4*>(seq_keys + (j & ~int64_t{15}) * 128);
  const int n = static_cast<int>(j & 15);
  *lo = t[g * 16 + n];
  *hi = t[(4 + g) * 16 + n];
}

// fp4 (MXFP4) caches of dim 128 use the same 16-entry tiles at 64 bytes per
// entry: tile t holds 4 chunks of 16 bytes (32 dims each, two codes per byte,
// the lower nibble first), chunk-major, each chunk the 16 entries' bytes in
// entry order.  Lane (g, n) reads chunk g of entry n, 1 KiB per wave load.
// Byte of dim d (its nibble: d % 2) of entry j of sequence b:
__host__ __device__ __forceinline__ int64_t idx4_tile_off(int64_t b, int64_t e_pad, int64_t j, int d) {
  return (b * e_pad + (j & ~int64_t{15})) * 64 + (d >> 5) * 256 + (j & 15) * 16 + ((d & 31) >> 1);
}
__host__ __device__ __forceinline__ int64_t idx4_tile_off_row(int64_t R, int d) {
  return (R & ~int64_t{15}) * 64 + (d >> 5) * 256 + (R & 15) * 16 + ((d & 31) >> 1);
}
__device__ __forceinline__ uint4 idx4_load_chunk(const uint8_t* seq_keys, int64_t j, int g) {
  const uint4* t = reinterpret_cast<const uint4*>(seq_keys + (j & ~int64_t{15}) * 64);
  return t[g * 16 + static_cast<int>(j & 15)];
}

// ------------------------------------------------------- counts / keys
__host__ __device__ __forceinline__ int64_t n_complete(int64_t L, int s, int S) {
  return L < S ? 0 : (L - S) / s + 1;  // L - S >= 0 here, so / is floor
}

// Monotone map float -> uint32 (larger float, larger key); -0 and +0 map to
// the same key so that equal scores tie.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ void set_status(uint32_t* st, uint32_t bits) {
  if (st) atomicOr(st, bits);
}

// ------------------------------------------------------ paged caches
// A logical block is 256 raw token positions; a cache type holds 2^shift of
// its rows per physical block (compressed entries: 256 / stride; window:
// 256 tokens).  With a table, row j of sequence b is
//   table[b, j >> shift] << shift | (j mod 2^shift);
// a block id outside [0, n_blocks) sets DSA_DEVERR_BLOCK and maps to block 0
// (ok = false: the caller drops a write).
struct PageMap {
  const int32_t* table;  // [B, stride] or nullptr (dense)
  int64_t stride;
  int shift;
  int32_t n_blocks;
};

__device__ __forceinline__ int64_t paged_row(const PageMap& p, int b, int64_t j, uint32_t* status,
                                             bool* ok = nullptr) {
  int32_t blk = p.table[b * p.stride + (j >> p.shift)];
  if (static_cast<uint32_t>(blk) >= static_cast<uint32_t>(p.n_blocks)) {
    set_status(status, DSA_DEVERR_BLOCK);
    blk = 0;
    if (ok) *ok = false;
  }
  return (static_cast<int64_t>(blk) << p.shift) | (j & ((int64_t{1} << p.shift) - 1));
}

// Row of entry j of sequence b: dense b * dense_rows + j, or its pool row.
__device__ __forceinline__ int64_t entry_row(const PageMap& p, int b, int64_t j, int64_t dense_rows,
                                             uint32_t* status, bool* ok = nullptr) {
  return p.table ? paged_row(p, b, j, status, ok) : b * dense_rows + j;
}

// The paging of a call: compressed caches, window, compressor rings.
struct Paging {
  PageMap ent;
  PageMap swa;
  const int32_t* state;  // [B] ring block of each sequence or nullptr
  int32_t n_state;
};

inline Paging make_paging(const dsa_paging& p) {
  Paging g{};
  int sh = 0;
  while (sh < 30 && (1 << sh) < p.entries_per_block) ++sh;
  g.ent = PageMap{p.block_table, p.blocks_per_seq, sh, p.n_blocks};
  g.swa = PageMap{p.swa_block_table, p.blocks_per_seq, 8, p.n_swa_blocks};  // 256 tokens
  g.state = p.state_block;
  g.n_state = p.n_state_blocks;
  return g;
}

// Row of window token n of sequence b: slot n mod w_cap of the sequence's
// ring, or slot n mod 256 of its window block.
__device__ __forceinline__ int64_t window_row(const PageMap& w, int b, int64_t n, int w_cap,
                                              uint32_t* status, bool* ok = nullptr) {
  return w.table ? paged_row(w, b, n, status, ok) : static_cast<int64_t>(b) * w_cap + n % w_cap;
}

// The compressor rings' block of sequence b (b itself when dense).
__device__ __forceinline__ int64_t state_seq(const Paging& pg, int b, uint32_t* status,
                                             bool* ok = nullptr) {
  if (!pg.state) return b;
  const int32_t s = pg.state[b];
  if (static_cast<uint32_t>(s) >= static_cast<uint32_t>(pg.n_state)) {
    set_status(status, DSA_DEVERR_BLOCK);
    if (ok) *ok = false;
    return 0;
  }
  return s;
}

// ------------------------------------------------------ reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Block-wide reductions (blockDim.x a multiple of 64, <= 1024).  `red` is a
// __shared__ float[16] scratch; all threads get the result.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave, nw = blockDim.x / kWave;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave, nw = blockDim.x / kWave;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int i = 0; i < nw; ++i) t = fmaxf(t, red[i]);
  return t;
}

// Holds each value in scalar registers at this point, so that the loads of
// kernel arguments feeding them are issued together (left to itself the
// compiler spreads them over a chain of dependent waits).
template <typename T>
__device__ __forceinline__ void pin_scalar(const T& v) {
  asm volatile("" ::"s"(v));
}
template <typename... T>
__device__ __forceinline__ void pin_scalars(const T&... v) {
  (pin_scalar(v), ...);
}

}  // namespace dsa
