/*
 * kda.h -- C ABI of the MI355X (gfx950) forward pass of Kimi Delta Attention
 * (KDA), chunked form, specialised to head dims K = V = 128 in packed layout.
 *
 * Operation (page "nemo_automodel.components.models.kimi_k3.kda_fused",
 * package docstring, fused_chunk_kda and fused_kda_unsupported_reason):
 * per document d and head h, a K x V fp32 state S starts at zero and, for
 * every token t of the document in order,
 *
 *     S  <- (I - beta_t kh_t kh_t^T) Diag(exp(g_t)) S + beta_t kh_t v_t^T
 *     o_t = 128**-0.5 * S^T qh_t
 *
 * where qh, kh are q, k scaled by 1/sqrt(sum(x*x) + 1e-6) (the in-kernel
 * l2 norm), g_t is the per-key-channel log decay (the bounded log gate) and
 * the state is dropped at the end of the document (no initial or final state).
 * Documents are delimited by int32 cu_seqlens (the packed, batch-1 layout);
 * a dense batch of B equal-length sequences is the same computation with
 * cu_seqlens = [0, T, 2T, ..., BT].  The result does not depend on the chunk
 * length; the library works in chunks of 64 tokens.
 *
 * All entry points are thread-safe.  Errors are returned, never hidden: there
 * is no fallback path (the pages' contract: a call either runs the fused
 * kernels or stops with the first violated condition).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "kda_status.h"

#ifdef __cplusplus
extern "C" {
#endif


/*
 * kda_chunk_fwd -- o = KDA(q, k, v, g, beta) over a packed token stream.
 *
 * Layouts (all contiguous, row-major, token-major "[1, T, H, D]" packed):
 *   q, k, v     bf16  [T][H][128]   device memory, 16-byte aligned
 *   g           fp32  [T][H][128]   device memory, 16-byte aligned; natural-log
 *                                   decay per token, head and key channel; the
 *                                   caller promises gate_bound <= g <= 0
 *   beta        fp32  [T][H]        device memory, 4-byte aligned; any finite value
 *   cu_seqlens  int32 [N+1]         device memory, 4-byte aligned, or NULL for a
 *                                   single document [0, T).  cu[0] = 0, entries
 *                                   non-decreasing, and the list ends at its first
 *                                   entry equal to T, at index N <= T.  Zero-length
 *                                   documents are allowed.  The library reads the
 *                                   list in aligned 4 KiB blocks up to the block
 *                                   that holds that entry (bytes past it in the same
 *                                   page are read and ignored).
 *   out         bf16  [T][H][128]   device memory, 16-byte aligned, fully
 *                                   overwritten (round to nearest even)
 *   T           tokens in the stream, 0 <= T <= INT32_MAX (T = 0 is a no-op)
 *   H           heads, 1 <= H <= KDA_MAX_HEADS (same H for q, k and v)
 *   chunk       must be 64
 *   gate_bound  L with -5.5 <= L < 0: the lower bound of the bounded log gate.
 *               It licenses the 16-token sub-block factorisation of the decay
 *               inside a chunk (no exp() argument beyond +-88); it is never used
 *               to clamp g.
 *   stream      HIP stream on the current device; all work is enqueued on it.
 *
 * Ownership: the caller owns every buffer and keeps it alive until the stream
 * has passed this call.  The library allocates one stream-ordered workspace
 * per call (hipMallocFromPoolAsync / hipFreeAsync on `stream`, from a memory
 * pool the library creates per device; it keeps up to 8 GiB reserved between
 * calls and leaves the device's default pool untouched) and never syncs the
 * host: a document list (8 B per token) and room for the intermediate chunk
 * images of long documents (up to about 1 KB per token and head, at most
 * 16 GiB).
 *
 * Errors: returns KDA_OK or the negative kda_status of the FIRST violated
 * condition, checked in this order: shape (T, H), then (unless T = 0) NULL
 * pointers, chunk and gate_bound, alignment.  kda_last_error() then names the
 * condition.  Violations only visible on the device (cu_seqlens contents,
 * g outside the promised range) are reported through kda_device_status().
 */
int kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                  const float* beta, const int32_t* cu_seqlens, int64_t T, int32_t H,
                  int32_t chunk, float gate_bound, void* out, hipStream_t stream);

/*
 * kda_chunk_fwd_noalloc -- kda_chunk_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, layouts, errors and output (bit for
 * bit); it calls no hipMalloc, hipFree or allocating routine.  Its workspace
 * is a fixed 64 MiB array per device that the library holds until the process
 * ends, so T is limited to what fits there: 8 bytes per token plus a few KiB
 * (about 8.3 million tokens); a larger T returns KDA_ERR_BAD_SHAPE before
 * anything is enqueued.  The images of long documents get only what the array
 * has left, so long documents may run slower than with kda_chunk_fwd.
 * Every call on a device shares that device's array: calls that overlap on
 * one device (on different streams, or from different threads without
 * ordering) race and must not be issued.
 */
int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const int32_t* cu_seqlens, int64_t T, int32_t H,
                          int32_t chunk, float gate_bound, void* out, hipStream_t stream);

/*
 * kda_chunk_fwd_state -- kda_chunk_fwd with a state carried into and out of
 * every document: document d starts from S = initial_state[d] (instead of
 * zero) and its last state is written to final_state[d].  This is the
 * initial_state / output_final_state convention of FLA's chunk_kda, for
 * which fused_chunk_kda (page "nemo_automodel.components.models.kimi_k3.
 * kda_fused", fused_chunk_kda entry) is the drop-in with the final state
 * switched off.  With initial_state = NULL and final_state = NULL the output
 * equals kda_chunk_fwd's bit for bit.
 *
 * Arguments as for kda_chunk_fwd, except:
 *   cu_seqlens     int32 [n_docs+1], or NULL for one document [0, T)
 *                  (then n_docs must be 1).  Read exactly: cu[0] = 0,
 *                  non-decreasing, cu[n_docs] = T.  Every entry delimits a
 *                  document, trailing empty ones included; an empty document
 *                  passes its initial state through unchanged.
 *   n_docs         number of documents, >= 1, n_docs * H <= INT32_MAX
 *   initial_state  fp32 [n_docs][H][128][128] (S[key channel][value channel]
 *                  of document d, head h), 16-byte aligned, or NULL for zero
 *   final_state    fp32 [n_docs][H][128][128], 16-byte aligned, or NULL (not
 *                  written).  May be the same buffer as initial_state (each
 *                  (document, head) slot is read before it is written, by the
 *                  same workgroup); any other overlap is undefined.
 *   T              may be 0: then q, k, v, g, beta and out are not read and
 *                  may be NULL, cu_seqlens must hold n_docs + 1 zeros, and
 *                  final_state (if given) receives initial_state (or zeros).
 *
 * Errors: as kda_chunk_fwd, in the same order, plus KDA_ERR_BAD_SHAPE for
 * n_docs (checked with T and H) and KDA_ERR_ALIGN for the two state buffers.
 * A cu_seqlens that breaks its contract is reported through
 * kda_device_status; out and final_state are then filled with NaN.
 */
int kda_chunk_fwd_state(const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const int32_t* cu_seqlens, int32_t n_docs,
                        int64_t T, int32_t H, int32_t chunk, float gate_bound,
                        const float* initial_state, float* final_state, void* out,
                        hipStream_t stream);

/*
 * kda_recurrent_fwd -- the same operator as kda_chunk_fwd_state, evaluated
 * token by token instead of in chunks: the recurrent mode that the K3 model
 * selects for decoding and short sequences (page "nemo_automodel.components.
 * models.kimi_k3.kda_fused", package docstring: the fused kernels cover the
 * chunk mode only; the mode is a model option).  Meant for one token (decode)
 * or a few tokens per document; the chunked entry points are faster beyond
 * that.  The result equals kda_chunk_fwd_state's within rounding.
 *
 * Arguments as for kda_chunk_fwd_state, without chunk and gate_bound (no
 * decay factorisation is used, so g only needs to be finite; g <= 0 keeps the
 * state bounded).  cu_seqlens [n_docs+1] is read exactly; n_docs * H <= 2^25
 * (the launch runs 2 x 64 work-items per document and head, below 2^32).
 * initial_state / final_state may be NULL or the same buffer (decode updates
 * the state in place).
 *
 * Ownership: as kda_chunk_fwd; the workspace is 256 bytes.
 * Errors: as kda_chunk_fwd_state (no chunk / gate_bound checks).  A
 * cu_seqlens that breaks its contract sets KDA_DEV_BAD_CU_SEQLENS and fills
 * out and final_state with NaN.
 */
int kda_recurrent_fwd(const void* q, const void* k, const void* v, const float* g,
                      const float* beta, const int32_t* cu_seqlens, int32_t n_docs, int64_t T,
                      int32_t H, const float* initial_state, float* final_state, void* out,
                      hipStream_t stream);

/*
 * kda_chunk_bwd -- gradients of the state-carrying forward (kda_chunk_fwd_state)
 * with respect to q, k, v, g, beta and the initial states, given d_out = dL/do
 * and d_final_state = dL/dS_end.  It recomputes every intermediate from the
 * raw inputs, as the backward of the pages' fused forward does (page
 * "nemo_automodel.components.models.kimi_k3.kda_fused", package docstring:
 * the autograd function saves only q, k, v, g, beta and cu_seqlens).
 *
 * Inputs as for kda_chunk_fwd_state (q, k, v, g, beta, cu_seqlens read exactly
 * with n_docs + 1 entries, initial_state or NULL), plus
 *   d_out          bf16 [T][H][128], 16-byte aligned
 *   d_final_state  fp32 [n_docs][H][128][128] or NULL (zero)
 * Outputs, all fp32, fully overwritten:
 *   dq, dk, dv, dg fp32 [T][H][128], 16-byte aligned
 *   dbeta          fp32 [T][H], 4-byte aligned
 *   d_initial_state fp32 [n_docs][H][128][128] or NULL (not written)
 * T = 0 is allowed (then the token tensors are not read and
 * d_initial_state, if given, receives d_final_state).
 *
 * Arithmetic: fp32 throughout (MFMA 16x16x4 fp32 products); the forward
 * states it differentiates around come from the forward kernels.
 * Ownership: as kda_chunk_fwd; the stream-ordered workspace holds, per chunk
 * and head, the state and its gradient at the chunk boundary, the fp32 chunk
 * image and its transition (about 400 KiB), plus a bf16 copy of the forward
 * output.  A call whose workspace would exceed a ceiling (16 GiB by default,
 * kda_debug_set_bwd_workspace_limit) reads cu_seqlens back to the host (the
 * call then waits for `stream`) and runs over consecutive groups of whole
 * documents, each group's workspace within the ceiling; a single document
 * larger than the ceiling is one group of its own.  Same result bit for bit.
 * Errors: as kda_chunk_fwd_state, plus KDA_ERR_NULL_PTR for d_out and the
 * gradient outputs and KDA_ERR_BAD_SHAPE when n_docs * H exceeds 2^21 (one
 * state-gradient chain of 512 work-items per document, head and quarter of
 * the value columns, below 2^32 work-items per launch); a cu_seqlens that
 * breaks its contract sets
 * KDA_DEV_BAD_CU_SEQLENS and fills every gradient output with NaN.
 */
int kda_chunk_bwd(const void* q, const void* k, const void* v, const float* g,
                  const float* beta, const int32_t* cu_seqlens, int32_t n_docs, int64_t T,
                  int32_t H, int32_t chunk, float gate_bound, const float* initial_state,
                  const void* d_out, const float* d_final_state, float* dq, float* dk, float* dv,
                  float* dg, float* dbeta, float* d_initial_state, hipStream_t stream);

/*
 * kda_last_error -- the first violated condition of the last non-zero return
 * of any entry point on the calling thread ("" if none), the counterpart of
 * fused_kda_unsupported_reason (page "nemo_automodel.components.models.
 * kimi_k3.kda_fused", function table: it names the first condition that keeps
 * a call off the fused kernels).  The string is owned by the library and stays
 * valid until the next call on the same thread.
 */
const char* kda_last_error(void);

/*
 * kda_device_status -- debug/test helper with no counterpart on the pages:
 * synchronises `stream`, returns the sticky kda_device_flags word of the
 * current device accumulated by all calls since the last kda_device_status,
 * and clears it.  Returns KDA_ERR_HIP if a HIP call fails.  Not for the hot
 * path (it blocks the host).
 */
int kda_device_status(hipStream_t stream);

/*
 * kda_debug_set_split_policy -- test hook with no counterpart on the pages:
 * forces the choice of the long documents whose chunks are prepared in
 * parallel before their sequential chain runs ("split" documents).
 * 0 = never split, 1 = automatic (the default), 2 = split every document the
 * workspace allows.  All three give the same output bit for bit; only the
 * speed differs.  Process-wide; returns the previous policy, or
 * KDA_ERR_UNSUPPORTED for another value.  Calls already enqueued keep the
 * policy they were enqueued with.
 */
int kda_debug_set_split_policy(int policy);

/*
 * kda_debug_set_bwd_workspace_limit -- test hook with no counterpart on the
 * pages: sets the ceiling of one backward pass's workspace in bytes (0
 * restores the default, 16 GiB), above which kda_chunk_bwd runs over groups of
 * documents.  Process-wide; returns the previous ceiling.
 */
uint64_t kda_debug_set_bwd_workspace_limit(uint64_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
