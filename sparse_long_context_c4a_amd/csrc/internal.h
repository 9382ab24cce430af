// Host-side internals: launch helpers and the error channel behind the C ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstddef>
#include <cstdint>

#include "dsa.h"

namespace dsa {

dsa_status fail(dsa_status s, const char* fmt, ...);
dsa_status hip_check(hipError_t e, const char* what);

// A kernel launch with optional timing events attached to its own dispatch
// packet (no separate event packets, so no idle gap between kernels).
template <typename K, typename... Args>
void launch_timed(K kernel, dim3 grid, dim3 block, size_t shm, hipStream_t st, hipEvent_t ev0,
                  hipEvent_t ev1, Args... args) {
  if (ev0 || ev1)
    hipExtLaunchKernelGGL(kernel, grid, block, static_cast<uint32_t>(shm), st, ev0, ev1, 0u,
                          args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shm, st, args...);
}

// Timing events of the entry-point call running on this thread (taken from
// the one-shot dsa_set_timing_events hook for the call's duration; all null
// otherwise).
struct TimingEvents {
  hipEvent_t index0, index1, attn0, attn1;
};
const TimingEvents& call_timing();

inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Kernel launchers (one per step); arguments already validated.
dsa_status launch_compress(const dsa_compress_args& a, hipStream_t st);
// Two compressions of one chunk (the main entries a, the indexer keys b) in
// one launch where their types allow, else one after the other.
dsa_status launch_compress_pair(const dsa_compress_args& a, const dsa_compress_args& b,
                                hipStream_t st);

// Indexer + Top-k.  Workspace layout is owned by indexer.hip.
size_t index_topk_ws_bytes(const dsa_index_args& a);
dsa_status launch_index_topk(const dsa_index_args& a, void* ws, hipStream_t st);

// Indexer + Top-k for many rows per sequence (prefill): whether it applies,
// its workspace beyond the shared per-row scores (rows x ld floats, the
// fallback buffer), and its launch.  Owned by prefill_index.hip.
bool prefill_index_applies(const dsa_index_args& a, int64_t nv_cap);
size_t prefill_index_ws_bytes(const dsa_index_args& a, int64_t nv_cap);
dsa_status launch_prefill_index_topk(const dsa_index_args& a, int64_t nv_cap, float* scores,
                                     int64_t ld, void* ws, hipStream_t st);

// Attention.  Optional timing events ride on the first and last kernel's
// dispatch.
struct AttnLaunch {
  void* ev0 = nullptr;
  void* ev1 = nullptr;
  const float* cs_tab = nullptr;  // (cos, sin) of each row's position, rope_dim floats per row
};
size_t attn_ws_bytes(const dsa_attn_args& a);
// The shapes whose attention can read a token-wise fp8 cache (the decode
// kernel's): DSA_OK or DSA_ERR_UNSUPPORTED with the message set.
dsa_status attn_fp8_cache_shape(int k, int heads, int64_t rows);
dsa_status launch_attn(const dsa_attn_args& a, void* ws, hipStream_t st,
                       const AttnLaunch& lx = AttnLaunch{});

// Layer helpers: ring and window maintenance, chunk rotation.
// In one launch after the compressor: the chunk's tail into the main ring
// (raw0, ring0) and, with ring1, the indexer's ring; every row's position
// into qpos; with rot_out, the chunk's main tokens (raw0) rotated for the
// window.
dsa_status launch_chunk_tasks(const void* raw0, dsa_dtype dt0, int D0, void* ring0,
                              const void* raw1, dsa_dtype dt1, int D1, void* ring1, int64_t T,
                              int S, const int64_t* pos0, int B, int64_t max_pos_end,
                              const dsa_paging& pg, uint32_t* status, int64_t* qpos,
                              void* rot_out, int rope_dim, double rope_base, int64_t rope_off,
                              hipStream_t st);
dsa_status launch_window_update(const void* rot_chunk, dsa_dtype dt, int D, int64_t T, void* win,
                                int w_cap, int window_size, const int64_t* pos0, int B,
                                int64_t max_pos_end, const dsa_paging& pg, uint32_t* status,
                                hipStream_t st);

// Decode (one token per sequence): fused prologue and, when the window ring
// has no spare slot, the window insert after attention.
struct PrologueArgs;
PrologueArgs make_prologue_args(const dsa_layer_args& a, int64_t* qpos, bool insert_window,
                                float* cs_tab, void* q_rot);
// The indexer + Top-k of a decode step with the prologue's workgroups riding
// in the indexer's launch (or launched first when the indexer takes another
// path).
dsa_status launch_decode_index_topk(const dsa_index_args& a, void* ws, const dsa_layer_args& la,
                                    int64_t* qpos, bool insert_window, float* cs_tab, void* q_rot,
                                    hipStream_t st);
// all_idx (may be nullptr): the step's selection when it is every visible
// entry (no indexer keys), [B, all_k], written by the prologue itself.
dsa_status launch_decode_prologue(const dsa_layer_args& a, int64_t* qpos, bool insert_window,
                                  float* cs_tab, void* q_rot, hipStream_t st,
                                  int32_t* all_idx = nullptr, int all_k = 0,
                                  int64_t all_nv_cap = 0);
// The chunk's pre-attention step: queries normalised and rotated into q_rot,
// the raw tokens rotated into rot_chunk (one launch).
dsa_status launch_qk_prep(const dsa_layer_args& a, void* q_rot, void* rot_chunk, hipStream_t st);
dsa_status launch_decode_window_insert(const dsa_layer_args& a, hipStream_t st);

inline size_t dtype_size(dsa_dtype t) {
  return t == DSA_F32 ? 4 : t == DSA_BF16 ? 2 : 1;
}

}  // namespace dsa
