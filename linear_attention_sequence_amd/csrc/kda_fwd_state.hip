// kda_fwd_state.hip -- the main kernel of libkda with state input / output
// (each (document, head) unit starts from h0[doc][h] and stores its last
// state to ht[doc][h]), instantiated in a translation unit of its own; see
// kda_kernels.h.
#include "kda_kernels.h"

namespace kda_state_tu {

hipError_t launch_main_state(dim3 grid, hipStream_t stream, const void* q, const void* k,
                             const void* v, const float* g, const float* beta, void* out,
                             void* hdr, const void* docs, const void* split, const void* images,
                             int64_t T, int H, float gate_bound) {
  hipLaunchKernelGGL(kda_pc_kernel<true>, grid, dim3(NPC), 0, stream,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                     static_cast<const bf16*>(v), g, beta, static_cast<bf16*>(out),
                     static_cast<WorkHeader*>(hdr), static_cast<const int2*>(docs),
                     static_cast<const int2*>(split), static_cast<const uint8_t*>(images), T, H,
                     gate_bound);
  return hipGetLastError();
}

}  // namespace kda_state_tu
