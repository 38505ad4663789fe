// kda_host_checks.cpp -- argument checks and workspace layouts of the C ABI
// (see kda_host_checks.h).  No GPU code, no HIP headers.
#include "kda_host_checks.h"

namespace kda_check {
namespace {

constexpr Result OK{KDA_OK, ""};

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

Result bad(int code, const char* msg) { return Result{code, msg}; }

// shape checks shared by every entry point (T, then H)
Result shape(int64_t T, int32_t H) {
  if (T < 0) return bad(KDA_ERR_BAD_SHAPE, "T must be >= 0");
  if (T > INT32_MAX) return bad(KDA_ERR_BAD_SHAPE, "T must be <= INT32_MAX");
  if (H < 1) return bad(KDA_ERR_BAD_SHAPE, "H must be >= 1");
  if (H > KDA_MAX_HEADS) return bad(KDA_ERR_BAD_SHAPE, "H must be <= KDA_MAX_HEADS");
  return OK;
}

Result chunk_and_gate(int32_t chunk, float gate_bound) {
  if (chunk != KDA_CHUNK) return bad(KDA_ERR_UNSUPPORTED, "chunk must be 64");
  if (!(gate_bound >= -5.5f && gate_bound < 0.f))
    return bad(KDA_ERR_UNSUPPORTED, "gate_bound must be finite and in [-5.5, 0)");
  return OK;
}

// the token tensors of a forward (T > 0): NULL pointers, chunk and gate bound,
// alignment
Result tokens(const void* q, const void* k, const void* v, const void* g, const void* beta,
              const void* out, int32_t chunk, float gate_bound) {
  if (!q) return bad(KDA_ERR_NULL_PTR, "q is NULL");
  if (!k) return bad(KDA_ERR_NULL_PTR, "k is NULL");
  if (!v) return bad(KDA_ERR_NULL_PTR, "v is NULL");
  if (!g) return bad(KDA_ERR_NULL_PTR, "g is NULL");
  if (!beta) return bad(KDA_ERR_NULL_PTR, "beta is NULL");
  if (!out) return bad(KDA_ERR_NULL_PTR, "out is NULL");
  const Result r = chunk_and_gate(chunk, gate_bound);
  if (r.code != KDA_OK) return r;
  if (!aligned(q, 16)) return bad(KDA_ERR_ALIGN, "q is not 16-byte aligned");
  if (!aligned(k, 16)) return bad(KDA_ERR_ALIGN, "k is not 16-byte aligned");
  if (!aligned(v, 16)) return bad(KDA_ERR_ALIGN, "v is not 16-byte aligned");
  if (!aligned(g, 16)) return bad(KDA_ERR_ALIGN, "g is not 16-byte aligned");
  if (!aligned(out, 16)) return bad(KDA_ERR_ALIGN, "out is not 16-byte aligned");
  if (!aligned(beta, 4)) return bad(KDA_ERR_ALIGN, "beta is not 4-byte aligned");
  return OK;
}

Result documents(const void* cu_seqlens, int32_t n_docs, int32_t H) {
  if (n_docs < 1) return bad(KDA_ERR_BAD_SHAPE, "n_docs must be >= 1");
  if ((int64_t)n_docs * H > INT32_MAX) return bad(KDA_ERR_BAD_SHAPE, "n_docs * H must be <= INT32_MAX");
  if (!cu_seqlens && n_docs != 1) return bad(KDA_ERR_BAD_SHAPE, "n_docs must be 1 when cu_seqlens is NULL");
  return OK;
}

Result states(const void* cu_seqlens, const void* s0, const void* s1, const char* m0, const char* m1) {
  if (cu_seqlens && !aligned(cu_seqlens, 4)) return bad(KDA_ERR_ALIGN, "cu_seqlens is not 4-byte aligned");
  if (s0 && !aligned(s0, 16)) return bad(KDA_ERR_ALIGN, m0);
  if (s1 && !aligned(s1, 16)) return bad(KDA_ERR_ALIGN, m1);
  return OK;
}

// overflow-checked size arithmetic
bool add(size_t a, size_t b, size_t* r) { return !__builtin_add_overflow(a, b, r); }
bool mul(size_t a, size_t b, size_t* r) { return !__builtin_mul_overflow(a, b, r); }
bool align256(size_t x, size_t* r) {
  if (!add(x, 255, r)) return false;
  *r &= ~size_t(255);
  return true;
}
// off = align256(off + n * elem); returns the offset the region starts at
bool region(size_t* off, size_t n, size_t elem, size_t* start) {
  size_t b = 0;
  *start = *off;
  return mul(n, elem, &b) && add(*off, b, off) && align256(*off, off);
}

}  // namespace

Result chunk_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                 const void* cu_seqlens, int64_t T, int32_t H, int32_t chunk, float gate_bound,
                 const void* out) {
  Result r = shape(T, H);
  if (r.code != KDA_OK || T == 0) return r;
  r = tokens(q, k, v, g, beta, out, chunk, gate_bound);
  if (r.code != KDA_OK) return r;
  if (cu_seqlens && !aligned(cu_seqlens, 4)) return bad(KDA_ERR_ALIGN, "cu_seqlens is not 4-byte aligned");
  return OK;
}

Result chunk_fwd_state(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, const void* cu_seqlens, int32_t n_docs, int64_t T,
                       int32_t H, int32_t chunk, float gate_bound, const void* initial_state,
                       const void* final_state, const void* out) {
  Result r = shape(T, H);
  if (r.code != KDA_OK) return r;
  r = documents(cu_seqlens, n_docs, H);
  if (r.code != KDA_OK || fwd_is_noop(T, final_state)) return r;
  r = T > 0 ? tokens(q, k, v, g, beta, out, chunk, gate_bound) : chunk_and_gate(chunk, -1.f);
  if (r.code != KDA_OK) return r;
  return states(cu_seqlens, initial_state, final_state, "initial_state is not 16-byte aligned",
                "final_state is not 16-byte aligned");
}

Result recurrent_fwd(const void* q, const void* k, const void* v, const void* g,
                     const void* beta, const void* cu_seqlens, int32_t n_docs, int64_t T,
                     int32_t H, const void* initial_state, const void* final_state,
                     const void* out) {
  Result r = shape(T, H);
  if (r.code != KDA_OK) return r;
  if (n_docs < 1) return bad(KDA_ERR_BAD_SHAPE, "n_docs must be >= 1");
  if ((int64_t)n_docs * H > MAX_RECURRENT_UNITS) return bad(KDA_ERR_BAD_SHAPE, "n_docs * H must be <= 2^25");
  if (!cu_seqlens && n_docs != 1) return bad(KDA_ERR_BAD_SHAPE, "n_docs must be 1 when cu_seqlens is NULL");
  if (fwd_is_noop(T, final_state)) return OK;
  if (T > 0) {
    if (!q) return bad(KDA_ERR_NULL_PTR, "q is NULL");
    if (!k) return bad(KDA_ERR_NULL_PTR, "k is NULL");
    if (!v) return bad(KDA_ERR_NULL_PTR, "v is NULL");
    if (!g) return bad(KDA_ERR_NULL_PTR, "g is NULL");
    if (!beta) return bad(KDA_ERR_NULL_PTR, "beta is NULL");
    if (!out) return bad(KDA_ERR_NULL_PTR, "out is NULL");
    if (!aligned(q, 16)) return bad(KDA_ERR_ALIGN, "q is not 16-byte aligned");
    if (!aligned(k, 16)) return bad(KDA_ERR_ALIGN, "k is not 16-byte aligned");
    if (!aligned(v, 16)) return bad(KDA_ERR_ALIGN, "v is not 16-byte aligned");
    if (!aligned(g, 16)) return bad(KDA_ERR_ALIGN, "g is not 16-byte aligned");
    if (!aligned(out, 16)) return bad(KDA_ERR_ALIGN, "out is not 16-byte aligned");
    if (!aligned(beta, 4)) return bad(KDA_ERR_ALIGN, "beta is not 4-byte aligned");
  }
  return states(cu_seqlens, initial_state, final_state, "initial_state is not 16-byte aligned",
                "final_state is not 16-byte aligned");
}

Result chunk_bwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                 const void* cu_seqlens, int32_t n_docs, int64_t T, int32_t H, int32_t chunk,
                 float gate_bound, const void* initial_state, const void* d_out,
                 const void* d_final_state, const void* dq, const void* dk, const void* dv,
                 const void* dg, const void* dbeta, const void* d_initial_state) {
  Result r = shape(T, H);
  if (r.code != KDA_OK) return r;
  if (n_docs < 1) return bad(KDA_ERR_BAD_SHAPE, "n_docs must be >= 1");
  if ((int64_t)n_docs * H > MAX_BWD_CHAIN_UNITS) return bad(KDA_ERR_BAD_SHAPE, "n_docs * H must be <= 2^21");
  if (!cu_seqlens && n_docs != 1) return bad(KDA_ERR_BAD_SHAPE, "n_docs must be 1 when cu_seqlens is NULL");
  if (bwd_is_noop(T, d_initial_state)) return OK;
  if (T > 0) {
    if (!q) return bad(KDA_ERR_NULL_PTR, "q is NULL");
    if (!k) return bad(KDA_ERR_NULL_PTR, "k is NULL");
    if (!v) return bad(KDA_ERR_NULL_PTR, "v is NULL");
    if (!g) return bad(KDA_ERR_NULL_PTR, "g is NULL");
    if (!beta) return bad(KDA_ERR_NULL_PTR, "beta is NULL");
    if (!d_out) return bad(KDA_ERR_NULL_PTR, "d_out is NULL");
    if (!dq || !dk || !dv || !dg || !dbeta) return bad(KDA_ERR_NULL_PTR, "a gradient output is NULL");
  }
  r = chunk_and_gate(chunk, gate_bound);
  if (r.code != KDA_OK) return r;
  if (T > 0) {
    if (!aligned(q, 16)) return bad(KDA_ERR_ALIGN, "q is not 16-byte aligned");
    if (!aligned(k, 16)) return bad(KDA_ERR_ALIGN, "k is not 16-byte aligned");
    if (!aligned(v, 16)) return bad(KDA_ERR_ALIGN, "v is not 16-byte aligned");
    if (!aligned(g, 16)) return bad(KDA_ERR_ALIGN, "g is not 16-byte aligned");
    if (!aligned(beta, 4)) return bad(KDA_ERR_ALIGN, "beta is not 4-byte aligned");
    if (!aligned(d_out, 16)) return bad(KDA_ERR_ALIGN, "d_out is not 16-byte aligned");
    if (!aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(dg, 16) || !aligned(dbeta, 4))
      return bad(KDA_ERR_ALIGN, "a gradient output is not aligned");
  }
  if (cu_seqlens && !aligned(cu_seqlens, 4)) return bad(KDA_ERR_ALIGN, "cu_seqlens is not 4-byte aligned");
  if (initial_state && !aligned(initial_state, 16)) return bad(KDA_ERR_ALIGN, "initial_state is not 16-byte aligned");
  if (d_final_state && !aligned(d_final_state, 16)) return bad(KDA_ERR_ALIGN, "d_final_state is not 16-byte aligned");
  if (d_initial_state && !aligned(d_initial_state, 16)) return bad(KDA_ERR_ALIGN, "d_initial_state is not 16-byte aligned");
  return OK;
}

bool fwd_is_noop(int64_t T, const void* final_state) { return T == 0 && final_state == nullptr; }
bool bwd_is_noop(int64_t T, const void* d_initial_state) { return T == 0 && d_initial_state == nullptr; }

bool fwd_layout(int64_t T, int32_t H, int32_t n_exact, bool split_allowed, size_t img_bytes,
                size_t img_budget, int min_split_chunks, int max_split_docs, FwdLayout* out) {
  if (T < 0 || H < 1 || img_bytes == 0 || min_split_chunks < 1 || max_split_docs < 1) return false;
  const size_t t = (size_t)T;
  const size_t n_list = t > (size_t)(n_exact > 0 ? n_exact : 0) ? t : (size_t)n_exact;
  // a split document has at least min_split_chunks chunks: (min - 1) 64 + 1 tokens
  size_t max_split = t / ((size_t)KDA_CHUNK * (size_t)(min_split_chunks - 1) + 1) + 1;
  if (max_split > (size_t)max_split_docs) max_split = (size_t)max_split_docs;
  size_t cap = 0;
  if (split_allowed) {
    cap = (t + KDA_CHUNK - 1) / KDA_CHUNK + max_split;
    const size_t fit = img_budget / ((size_t)H * img_bytes);
    if (cap > fit) cap = fit;
    if (cap < (size_t)min_split_chunks) cap = 0;
  }
  FwdLayout L{};
  size_t off = 256;
  size_t ids_n = n_exact >= 0 ? n_list : 0;
  if (!region(&off, n_list, 8, &L.off_docs) || !region(&off, ids_n, 4, &L.off_ids) ||
      !region(&off, max_split, 8, &L.off_split) || !region(&off, cap, 8, &L.off_pre))
    return false;
  L.off_img = off;
  size_t img = 0;
  if (!mul(cap, (size_t)H, &img) || !mul(img, img_bytes, &img) || !add(off, img, &L.bytes)) return false;
  L.max_split = max_split;
  L.cap_chunks = cap;
  *out = L;
  return true;
}

bool bwd_layout(int64_t T, int32_t H, int32_t n_docs, int grid, size_t chunk_desc_bytes,
                size_t img_floats, size_t sp_floats, size_t sc_floats, BwdLayout* out) {
  if (T < 0 || H < 1 || n_docs < 1 || grid < 1) return false;
  BwdLayout L{};
  // chunk slots: first token / 64 + document index + chunk index, all distinct
  if (!add((size_t)T / KDA_CHUNK, (size_t)n_docs + 1, &L.n_slots) || !mul(L.n_slots, (size_t)H, &L.items))
    return false;
  const size_t kv = (size_t)KDA_HEAD_DIM * KDA_HEAD_DIM;
  size_t off = 256, per = 0, o_bytes = 0;
  bool ok = region(&off, L.n_slots, chunk_desc_bytes, &L.off_table) &&
            region(&off, (size_t)n_docs, 4, &L.off_order) &&
            mul(L.items, kv, &per) &&
            region(&off, per, 4, &L.off_states) &&
            region(&off, per, 4, &L.off_dstates) &&
            mul(L.items, img_floats, &per) && region(&off, per, 4, &L.off_img) &&
            mul(L.items, kv, &per) && region(&off, per, 4, &L.off_ft) &&
            region(&off, per, 4, &L.off_r) &&
            region(&off, (size_t)grid, sp_floats * 4, &L.off_sp) &&
            region(&off, (size_t)grid, sc_floats * 4, &L.off_sc) &&
            mul((size_t)T * (size_t)H, (size_t)KDA_HEAD_DIM * 2, &o_bytes) &&
            region(&off, o_bytes, 1, &L.off_o);
  if (!ok) return false;
  L.bytes = off;
  *out = L;
  return true;
}

}  // namespace kda_check
