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

}  // namespace dsa
