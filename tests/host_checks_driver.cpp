// Host-only driver of the library's argument checks and workspace layouts
// (linear_attention_sequence_amd/csrc/kda_host_checks.cpp), built with a plain
// C++ compiler under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py.  It feeds every check valid, invalid and
// extreme arguments (limits of T, H and n_docs, pointer alignments, the
// largest workspaces) and exits non-zero on the first unexpected result.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kda_host_checks.h"

using kda_check::Result;

static int g_failures = 0;

static void expect(const char* what, Result r, int code, const char* msg_part) {
  const bool ok = r.code == code && (msg_part == nullptr || strstr(r.msg, msg_part) != nullptr);
  if (!ok) {
    fprintf(stderr, "FAIL %s: got (%d, \"%s\"), want (%d, \"%s\")\n", what, r.code, r.msg, code,
            msg_part ? msg_part : "");
    ++g_failures;
  }
}

static void expect_true(const char* what, bool v) {
  if (!v) {
    fprintf(stderr, "FAIL %s\n", what);
    ++g_failures;
  }
}

// fake, 16-byte aligned addresses: the checks only look at their values
static const void* P(uintptr_t off = 0) { return reinterpret_cast<const void*>(uintptr_t(1) << 20 | off); }

static Result fwd(int64_t T, int32_t H, const void* q = P(), const void* cu = nullptr,
                  int32_t chunk = 64, float gb = -5.f, const void* beta = P(), const void* out = P()) {
  return kda_check::chunk_fwd(q, P(), P(), P(), beta, cu, T, H, chunk, gb, out);
}

int main() {
  // ---- kda_chunk_fwd
  expect("fwd ok", fwd(4096, 32), KDA_OK, "");
  expect("fwd T=0 no-op ignores pointers", fwd(0, 1, nullptr), KDA_OK, "");
  expect("fwd T<0", fwd(-1, 1), KDA_ERR_BAD_SHAPE, "T must be >= 0");
  expect("fwd T min", fwd(INT64_MIN, 1), KDA_ERR_BAD_SHAPE, "T must be >= 0");
  expect("fwd T max", fwd(INT64_MAX, 1), KDA_ERR_BAD_SHAPE, "INT32_MAX");
  expect("fwd T=INT32_MAX ok", fwd(INT32_MAX, KDA_MAX_HEADS), KDA_OK, "");
  expect("fwd H=0", fwd(1, 0), KDA_ERR_BAD_SHAPE, "H must be >= 1");
  expect("fwd H min", fwd(1, INT32_MIN), KDA_ERR_BAD_SHAPE, "H must be >= 1");
  expect("fwd H max", fwd(1, INT32_MAX), KDA_ERR_BAD_SHAPE, "KDA_MAX_HEADS");
  expect("fwd shape before null", fwd(-1, 0, nullptr), KDA_ERR_BAD_SHAPE, "T must be");
  expect("fwd null q", fwd(1, 1, nullptr), KDA_ERR_NULL_PTR, "q is NULL");
  expect("fwd null before chunk", fwd(1, 1, nullptr, nullptr, 32), KDA_ERR_NULL_PTR, "q is NULL");
  expect("fwd chunk", fwd(1, 1, P(), nullptr, 32), KDA_ERR_UNSUPPORTED, "chunk must be 64");
  expect("fwd gate 0", fwd(1, 1, P(), nullptr, 64, 0.f), KDA_ERR_UNSUPPORTED, "gate_bound");
  expect("fwd gate nan", fwd(1, 1, P(), nullptr, 64, NAN), KDA_ERR_UNSUPPORTED, "gate_bound");
  expect("fwd gate -inf", fwd(1, 1, P(), nullptr, 64, -INFINITY), KDA_ERR_UNSUPPORTED, "gate_bound");
  expect("fwd gate -5.5 ok", fwd(1, 1, P(), nullptr, 64, -5.5f), KDA_OK, "");
  expect("fwd gate before align", fwd(1, 1, P(8), nullptr, 64, 1.f), KDA_ERR_UNSUPPORTED, "gate_bound");
  expect("fwd align q", fwd(1, 1, P(8)), KDA_ERR_ALIGN, "q is not 16-byte aligned");
  expect("fwd align beta", fwd(1, 1, P(), nullptr, 64, -5.f, P(2)), KDA_ERR_ALIGN, "beta is not 4-byte");
  expect("fwd beta 4-aligned ok", fwd(1, 1, P(), nullptr, 64, -5.f, P(4)), KDA_OK, "");
  expect("fwd align out", fwd(1, 1, P(), nullptr, 64, -5.f, P(), P(2)), KDA_ERR_ALIGN, "out is not");
  expect("fwd align cu", fwd(1, 1, P(), P(2)), KDA_ERR_ALIGN, "cu_seqlens is not 4-byte aligned");

  // ---- kda_chunk_fwd_state
  auto st = [](int64_t T, int32_t H, int32_t n, const void* cu, const void* h0, const void* ht,
               const void* q = P(), int32_t chunk = 64) {
    return kda_check::chunk_fwd_state(q, P(), P(), P(), P(), cu, n, T, H, chunk, -5.f, h0, ht, P());
  };
  expect("state ok", st(100, 4, 3, P(), P(), P()), KDA_OK, "");
  expect("state n_docs 0", st(100, 4, 0, P(), P(), P()), KDA_ERR_BAD_SHAPE, "n_docs must be >= 1");
  expect("state n_docs*H", st(100, KDA_MAX_HEADS, INT32_MAX, P(), P(), P()), KDA_ERR_BAD_SHAPE, "n_docs * H");
  expect("state n_docs*H at INT32_MAX ok", st(100, 1, INT32_MAX, P(), P(), P()), KDA_OK, "");
  expect("state cu NULL", st(100, 4, 2, nullptr, P(), P()), KDA_ERR_BAD_SHAPE, "cu_seqlens is NULL");
  expect("state T=0 no final no-op", st(0, 4, 2, P(), P(8), nullptr, nullptr), KDA_OK, "");
  expect("state T=0 final checks chunk", st(0, 4, 2, P(), P(), P(), nullptr, 32), KDA_ERR_UNSUPPORTED, "chunk");
  expect("state T=0 final ok", st(0, 4, 2, P(), P(), P(), nullptr), KDA_OK, "");
  expect("state align h0", st(100, 4, 2, P(), P(8), P()), KDA_ERR_ALIGN, "initial_state");
  expect("state align ht", st(100, 4, 2, P(), P(), P(4)), KDA_ERR_ALIGN, "final_state");

  // ---- kda_recurrent_fwd
  auto rec = [](int64_t T, int32_t H, int32_t n, const void* cu, const void* h0, const void* ht) {
    return kda_check::recurrent_fwd(P(), P(), P(), P(), P(), cu, n, T, H, h0, ht, P());
  };
  expect("rec ok", rec(5, 32, 1024, P(), P(), P()), KDA_OK, "");
  expect("rec units at the limit", rec(5, 2, int32_t(1) << 24, P(), nullptr, nullptr), KDA_OK, "");
  expect("rec units over the limit", rec(5, 2, (int32_t(1) << 24) + 1, P(), nullptr, nullptr),
         KDA_ERR_BAD_SHAPE, "2^25");
  expect("rec units far over", rec(5, KDA_MAX_HEADS, INT32_MAX, P(), nullptr, nullptr), KDA_ERR_BAD_SHAPE, "2^25");
  expect("rec T=0 no-op", rec(0, 2, 1, nullptr, P(), nullptr), KDA_OK, "");
  expect("rec align", rec(5, 2, 1, nullptr, P(4), P()), KDA_ERR_ALIGN, "initial_state");

  // ---- kda_chunk_bwd
  auto bwd = [](int64_t T, int32_t H, int32_t n, const void* cu, const void* dg, const void* dh0,
                int32_t chunk = 64) {
    return kda_check::chunk_bwd(P(), P(), P(), P(), P(), cu, n, T, H, chunk, -5.f, nullptr, P(),
                                nullptr, P(), P(), P(), dg, P(), dh0);
  };
  expect("bwd ok", bwd(4096, 32, 1, nullptr, P(), nullptr), KDA_OK, "");
  expect("bwd units at the limit", bwd(64, 2, int32_t(1) << 20, P(), P(), nullptr), KDA_OK, "");
  expect("bwd units over the limit", bwd(64, 2, (int32_t(1) << 20) + 1, P(), P(), nullptr),
         KDA_ERR_BAD_SHAPE, "2^21");
  expect("bwd null grad", bwd(64, 2, 1, nullptr, nullptr, nullptr), KDA_ERR_NULL_PTR, "gradient output is NULL");
  expect("bwd null before chunk", bwd(64, 2, 1, nullptr, nullptr, nullptr, 16), KDA_ERR_NULL_PTR, "NULL");
  expect("bwd chunk", bwd(64, 2, 1, nullptr, P(), nullptr, 16), KDA_ERR_UNSUPPORTED, "chunk");
  expect("bwd align grad", bwd(64, 2, 1, nullptr, P(4), nullptr), KDA_ERR_ALIGN, "not aligned");
  expect("bwd T=0 no-op", bwd(0, 2, 1, nullptr, nullptr, nullptr), KDA_OK, "");
  expect("bwd T=0 dh0 align", bwd(0, 2, 1, nullptr, nullptr, P(8)), KDA_ERR_ALIGN, "d_initial_state");

  // ---- workspace layouts: ordered, aligned, and no overflow at the extremes
  kda_check::FwdLayout fl;
  const size_t img = 61968, budget = size_t(16) << 30;
  expect_true("fwd layout packed", kda_check::fwd_layout(32768, 32, -1, true, img, budget, 8, 1024, &fl));
  expect_true("fwd layout order", fl.off_docs >= 256 && fl.off_ids >= fl.off_docs + 8 * 32768 &&
                                      fl.off_split >= fl.off_ids &&
                                      fl.off_pre >= fl.off_split && fl.off_img >= fl.off_pre &&
                                      fl.off_img % 256 == 0 && fl.bytes >= fl.off_img);
  expect_true("fwd layout images within budget", fl.cap_chunks * 32 * img <= budget);
  expect_true("fwd layout no split", kda_check::fwd_layout(32768, 32, -1, false, img, budget, 8, 1024, &fl) &&
                                         fl.cap_chunks == 0 && fl.bytes == fl.off_img);
  expect_true("fwd layout largest", kda_check::fwd_layout(INT32_MAX, KDA_MAX_HEADS, INT32_MAX, true, img,
                                                          budget, 8, 1024, &fl));
  expect_true("fwd layout largest fits budget", fl.cap_chunks * (size_t)KDA_MAX_HEADS * img <= budget);
  expect_true("fwd layout tiny", kda_check::fwd_layout(1, 1, 1, true, img, budget, 8, 1024, &fl) &&
                                     fl.cap_chunks == 0);
  expect_true("fwd layout rejects T<0", !kda_check::fwd_layout(-1, 1, -1, true, img, budget, 8, 1024, &fl));
  // the image budget bounds the images whatever their size: no overflow
  expect_true("fwd layout huge images", kda_check::fwd_layout(INT32_MAX, KDA_MAX_HEADS, -1, true,
                                                              size_t(1) << 40, SIZE_MAX, 8, 1024, &fl) &&
                                            fl.bytes > fl.off_img &&
                                            (fl.bytes - fl.off_img) / KDA_MAX_HEADS / (size_t(1) << 40) ==
                                                fl.cap_chunks);
  kda_check::BwdLayout bl;
  expect_true("bwd layout", kda_check::bwd_layout(32768, 32, 21, 256, 16, 36992, 8192, 40000, &bl) &&
                                bl.n_slots == 32768 / 64 + 22 && bl.items == bl.n_slots * 32 &&
                                bl.off_o > bl.off_sc && bl.bytes > bl.off_o);
  expect_true("bwd layout largest", kda_check::bwd_layout(INT32_MAX, KDA_MAX_HEADS, 1 << 9, 256, 16, 36992,
                                                          8192, 40000, &bl));
  expect_true("bwd layout overflow is refused",
              !kda_check::bwd_layout(INT32_MAX, KDA_MAX_HEADS, INT32_MAX, 256, 16, SIZE_MAX / 4, 1, 1, &bl));

  if (g_failures) {
    fprintf(stderr, "%d failure(s)\n", g_failures);
    return 1;
  }
  printf("host checks: all cases passed\n");
  return 0;
}
