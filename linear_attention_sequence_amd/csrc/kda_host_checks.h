// kda_host_checks.h -- the host side of the C ABI that touches no GPU: the
// argument checks of every entry point (first violated condition first, the
// contract of fused_kda_unsupported_reason on page "nemo_automodel.components.
// models.kimi_k3.kda_fused") and the byte layout of each call's workspace.
//
// Plain C++ with no HIP headers, so that a host compiler can build it on its
// own, under AddressSanitizer and UndefinedBehaviorSanitizer, and drive it
// with extreme arguments (tests/test_host_sanitizers.py).  The library's
// entry points call these functions and then launch their kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "kda_status.h"

namespace kda_check {

// the outcome of a check: KDA_OK and "" or the first violated condition
struct Result {
  int code;
  const char* msg;
};

// Workgroups of a launch times their threads must stay below 2^32 work-items.
constexpr int64_t MAX_RECURRENT_UNITS = int64_t(1) << 25;  // n_docs * H (2 x 64 threads each)
constexpr int64_t MAX_BWD_CHAIN_UNITS = int64_t(1) << 21;  // n_docs * H (4 x 512 threads each)

Result chunk_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                 const void* cu_seqlens, int64_t T, int32_t H, int32_t chunk, float gate_bound,
                 const void* out);

Result chunk_fwd_state(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, const void* cu_seqlens, int32_t n_docs, int64_t T,
                       int32_t H, int32_t chunk, float gate_bound, const void* initial_state,
                       const void* final_state, const void* out);

Result recurrent_fwd(const void* q, const void* k, const void* v, const void* g,
                     const void* beta, const void* cu_seqlens, int32_t n_docs, int64_t T,
                     int32_t H, const void* initial_state, const void* final_state,
                     const void* out);

Result chunk_bwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                 const void* cu_seqlens, int32_t n_docs, int64_t T, int32_t H, int32_t chunk,
                 float gate_bound, const void* initial_state, const void* d_out,
                 const void* d_final_state, const void* dq, const void* dk, const void* dv,
                 const void* dg, const void* dbeta, const void* d_initial_state);

// True when a checked call has nothing to enqueue (T = 0 without a state to
// hand through).
bool fwd_is_noop(int64_t T, const void* final_state);
bool bwd_is_noop(int64_t T, const void* d_initial_state);

// ---- workspace of the forward: header | docs | doc_ids | split | pre_chunks | images
struct FwdLayout {
  size_t off_docs, off_ids, off_split, off_pre, off_img, bytes;
  size_t max_split;   // split-document slots
  size_t cap_chunks;  // chunks of split documents the images can hold
};
// n_exact < 0: self-delimiting cu_seqlens; split_allowed: the policy allows
// splitting; img_bytes: one chunk image; img_budget: the images' byte cap.
bool fwd_layout(int64_t T, int32_t H, int32_t n_exact, bool split_allowed, size_t img_bytes,
                size_t img_budget, int min_split_chunks, int max_split_docs, FwdLayout* out);

// ---- workspace of the backward: one slot per chunk (and per document), per
// head: state, state gradient, image, F^T and R, plus per-workgroup scratch
struct BwdLayout {
  size_t n_slots, items;
  size_t off_table, off_order, off_states, off_dstates, off_img, off_ft, off_r, off_sp, off_sc,
      off_o, bytes;
};
bool bwd_layout(int64_t T, int32_t H, int32_t n_docs, int grid, size_t chunk_desc_bytes,
                size_t img_floats, size_t sp_floats, size_t sc_floats, BwdLayout* out);

}  // namespace kda_check
