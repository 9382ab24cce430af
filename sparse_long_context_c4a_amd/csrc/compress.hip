// S1: the compressor kernel, one workgroup per (entry slot e, sequence b);
// the per-entry work is compress_one (compress_impl.h).
#include "common.h"
#include "compress_impl.h"
#include "internal.h"

namespace dsa {
namespace {

template <typename RawT, int kOut>
__global__ __launch_bounds__(kCompressThreads) void k_compress(
    const RawT* __restrict__ raw, const RawT* __restrict__ ring, const int64_t* __restrict__ pos0v,
    const float* __restrict__ logits, void* __restrict__ out, float* __restrict__ out_scale,
    uint8_t* __restrict__ out_mx, const float* __restrict__ gamma, float eps, int64_t T,
    int logits_rows, int s, int S, int D, int r, double base, int64_t off, int64_t e_cap,
    int64_t max_pos_end, uint32_t* status, Paging pg) {
  compress_one<RawT, kOut>(blockIdx.x, blockIdx.y, raw, ring, pos0v, logits, out, out_scale, gamma,
                           eps, T, logits_rows, s, S, D, r, base, off, e_cap, max_pos_end, status,
                           0, -1, out_mx, pg);
}

// One of two compressions sharing a launch: what differs between them.
struct CompressJob {
  const void* raw;
  const void* ring;
  const float* logits;
  void* out;
  float* out_scale;
  uint8_t* out_mx;
  const float* gamma;
  int D, r;
  double base;
  int64_t off;
};

CompressJob job_of(const dsa_compress_args& a) {
  return CompressJob{a.raw, a.ring, a.logits, a.out, a.out_scale, a.out_mx_scale, a.rms_gamma,
                     a.geom.dim, a.geom.rope_dim, a.geom.rope_base, a.geom.rope_pos_offset};
}

// Two compressions of one chunk in one launch (blockIdx.z = 0: job a,
// 1: job b; the same entries, positions and paging), e.g. the main entries
// and the indexer keys: neither reads what the other writes.
template <typename RawA, int kOutA, typename RawB, int kOutB>
__global__ __launch_bounds__(kCompressThreads) void k_compress2(
    CompressJob ja, CompressJob jb, const int64_t* __restrict__ pos0v, float eps, int64_t T,
    int logits_rows, int s, int S, int64_t e_cap, int64_t max_pos_end, uint32_t* status,
    Paging pg) {
  if (blockIdx.z == 0)
    compress_one<RawA, kOutA>(blockIdx.x, blockIdx.y, static_cast<const RawA*>(ja.raw),
                              static_cast<const RawA*>(ja.ring), pos0v, ja.logits, ja.out,
                              ja.out_scale, ja.gamma, eps, T, logits_rows, s, S, ja.D, ja.r, ja.base,
                              ja.off, e_cap, max_pos_end, status, 0, -1, ja.out_mx, pg);
  else
    compress_one<RawB, kOutB>(blockIdx.x, blockIdx.y, static_cast<const RawB*>(jb.raw),
                              static_cast<const RawB*>(jb.ring), pos0v, jb.logits, jb.out,
                              jb.out_scale, jb.gamma, eps, T, logits_rows, s, S, jb.D, jb.r, jb.base,
                              jb.off, e_cap, max_pos_end, status, 0, -1, jb.out_mx, pg);
}

template <typename RawT>
dsa_status launch_typed(const dsa_compress_args& a, hipStream_t st) {
  dim3 grid(a.logits_rows, a.batch);
  const RawT* raw = static_cast<const RawT*>(a.raw);
  const RawT* ring = static_cast<const RawT*>(a.ring);
  const dsa_geom& g = a.geom;
  const Paging pg = make_paging(a.paging);
#define DSA_COMPRESS_LAUNCH(OUT)                                                                  \
  hipLaunchKernelGGL((k_compress<RawT, OUT>), grid, dim3(kCompressThreads), 0, st, raw, ring, a.raw_pos0, \
                     a.logits, a.out, a.out_scale, a.out_mx_scale, a.rms_gamma, a.rms_eps,       \
                     a.raw_len,                                                                  \
                     a.logits_rows, g.stride, g.span, g.dim, g.rope_dim, g.rope_base,            \
                     g.rope_pos_offset, a.e_cap, a.max_pos_end, a.status, pg)
  switch (a.out_dtype) {
    case DSA_F32: DSA_COMPRESS_LAUNCH(DSA_F32); break;
    case DSA_BF16: DSA_COMPRESS_LAUNCH(DSA_BF16); break;
    case DSA_FP4_E2M1: DSA_COMPRESS_LAUNCH(DSA_FP4_E2M1); break;
    default: DSA_COMPRESS_LAUNCH(DSA_FP8_E4M3); break;
  }
#undef DSA_COMPRESS_LAUNCH
  return hip_check(hipGetLastError(), "k_compress launch");
}

}  // namespace

dsa_status launch_compress(const dsa_compress_args& a, hipStream_t st) {
  if (a.geom.span > kCompressMaxSpan) return fail(DSA_ERR_UNSUPPORTED, "span %d > %d", a.geom.span, kCompressMaxSpan);
  if (a.geom.dim > 2 * kCompressThreads * kCompressPairs)
    return fail(DSA_ERR_UNSUPPORTED, "dim %d > %d", a.geom.dim, 2 * kCompressThreads * kCompressPairs);
  if (a.logits_rows == 0) return DSA_OK;
  return a.raw_dtype == DSA_F32 ? launch_typed<float>(a, st) : launch_typed<uint16_t>(a, st);
}

dsa_status launch_compress_pair(const dsa_compress_args& a, const dsa_compress_args& b,
                                hipStream_t st) {
  // one launch for a bf16 compression with bf16 output (a) and a bf16 one
  // with fp8 or MXFP4 output (b) over the same entries; other type pairs,
  // two launches
  const bool fused = a.raw_dtype == DSA_BF16 && a.out_dtype == DSA_BF16 &&
                     b.raw_dtype == DSA_BF16 &&
                     (b.out_dtype == DSA_FP8_E4M3 || b.out_dtype == DSA_FP4_E2M1) &&
                     a.logits_rows == b.logits_rows && a.batch == b.batch &&
                     a.geom.stride == b.geom.stride && a.geom.span == b.geom.span &&
                     a.raw_len == b.raw_len && a.raw_pos0 == b.raw_pos0 && a.e_cap == b.e_cap &&
                     a.max_pos_end == b.max_pos_end && a.rms_eps == b.rms_eps &&
                     a.status == b.status;
  if (!fused) {
    dsa_status rc = launch_compress(a, st);
    return rc != DSA_OK ? rc : launch_compress(b, st);
  }
  for (const dsa_compress_args* x : {&a, &b}) {
    if (x->geom.span > kCompressMaxSpan)
      return fail(DSA_ERR_UNSUPPORTED, "span %d > %d", x->geom.span, kCompressMaxSpan);
    if (x->geom.dim > 2 * kCompressThreads * kCompressPairs)
      return fail(DSA_ERR_UNSUPPORTED, "dim %d > %d", x->geom.dim, 2 * kCompressThreads * kCompressPairs);
  }
  if (a.logits_rows == 0) return DSA_OK;
  const dim3 grid(a.logits_rows, a.batch, 2);
  const Paging pg = make_paging(a.paging);
  if (b.out_dtype == DSA_FP8_E4M3)
    hipLaunchKernelGGL((k_compress2<uint16_t, DSA_BF16, uint16_t, DSA_FP8_E4M3>), grid,
                       dim3(kCompressThreads), 0, st, job_of(a), job_of(b), a.raw_pos0, a.rms_eps,
                       a.raw_len, a.logits_rows, a.geom.stride, a.geom.span, a.e_cap, a.max_pos_end,
                       a.status, pg);
  else
    hipLaunchKernelGGL((k_compress2<uint16_t, DSA_BF16, uint16_t, DSA_FP4_E2M1>), grid,
                       dim3(kCompressThreads), 0, st, job_of(a), job_of(b), a.raw_pos0, a.rms_eps,
                       a.raw_len, a.logits_rows, a.geom.stride, a.geom.span, a.e_cap, a.max_pos_end,
                       a.status, pg);
  return hip_check(hipGetLastError(), "k_compress2 launch");
}

}  // namespace dsa
