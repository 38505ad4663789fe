// kda_kernels.h -- device code of libkda shared by its two translation units:
// types, LDS layouts, the per-chunk stages (prepare_chunk, chain_chunk) and
// the main kernel template.  kda_fwd.hip instantiates the main kernel without
// state input/output and holds the scheduler, the pre kernel and the C ABI;
// kda_fwd_state.hip instantiates it with states.  The two instantiations
// live in separate translation units so that each is compiled exactly as if
// it were the only user of the shared stages.
//
// What is computed, and the chunk form the kernels use: see kda_fwd.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <string.h>
#include <stdlib.h>
#include <stddef.h>
#include <algorithm>
#include <stdio.h>
#include <string>
#include <mutex>
#include <vector>

#include "kda.h"

namespace {

constexpr int CH = 64;    // chunk length (tokens)
constexpr int DK = 128;   // key head dim
constexpr int DV = 128;   // value head dim
constexpr int NTHR = 256; // threads per workgroup (4 waves)
constexpr float L2_EPS = 1e-6f;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo_to_f32(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// swap bits 2 and 3: maps a 32x32 MFMA C-layout row to the token / channel it
// holds, chosen so that C fragments are directly reusable as B operands
__device__ __forceinline__ int swap23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// lane i of each 16-lane row receives x from lane i - N of the same row (0 if none)
template <int N>
__device__ __forceinline__ float dpp_row_shr(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xF, 0xF, false));
}

__device__ __forceinline__ f32x4 mfma16f(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16h(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32h(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// LDS layout (one chunk in flight, ~117 KB: one workgroup per CU)
//
// The leading part, Qt .. u.tb, is the chunk's "image": everything the chain
// reads that does not depend on the state.  For a split document the pre
// kernel builds it and copies it to global memory byte for byte; the main
// kernel copies it back instead of building it.  The per-channel state decay
// e^{G_c} travels in the row padding of Kt (see dvec).
// ---------------------------------------------------------------------------
struct alignas(16) Smem {
  bf16 Qt[CH][DK + 8];       // qh * e^G                      (A operand of Qt S)
  bf16 Kt[CH][DK + 8];       // -kh * e^G                     (A operand of X = V - Kt S)
  _Float16 KbT[DK][CH + 8];  // (kh * e^{G_c - G})^T <= 1     (A operand of the state update)
  _Float16 M[CH][CH + 8];    // M (|M| <= 1), lower incl.
  union {
    _Float16 tb[CH][CH + 8];  // Tb 2^-e (written after the solve; 2^e in tbscale)
    float A[CH][CH + 4];     // beta-scaled strictly lower A (fp32), input of the solve
  } u;
  // ---- end of the image
  union {
    f16x8 R[3][4][64];       // right operands of off-diagonal sub-blocks (fp16), lane order
    float T[CH][CH + 4];     // (I + A)^-1 (fp32)
    struct {
      union {
        unsigned short vt[32][CH + 8];  // this chunk's V, transposed (its 32 columns)
        unsigned short o[CH][32];       // then the bf16 O rows of those columns
      };
    } ws[4];                 // per-wave staging slices
  } u2;
  float etab[13][DK];        // per-channel decay factors of the chunk (see fill_tables)
  float tot[4][DK];          // per sub-block total decay (log2 domain)
  float beta[CH];
  float tbmax[8];            // per wave: largest |Tb| of the blocks it solved
  int unit;
  int gate_bad;
};


// e^{G_c} of channels c .. c + 3 (c a multiple of 4): the padding of Kt row c / 4
__device__ __forceinline__ float* dvec(Smem& sm, int c) {
  return reinterpret_cast<float*>(&sm.Kt[c >> 2][DK]);
}
// the power of two Tb was divided by: the padding of Kt row 32
__device__ __forceinline__ float* tbscale(Smem& sm) {
  return reinterpret_cast<float*>(&sm.Kt[32][DK]);
}

// byte offsets of the image parts
constexpr int OFF_QT = (int)offsetof(Smem, Qt);
constexpr int OFF_KT = (int)offsetof(Smem, Kt);
constexpr int OFF_KBT = (int)offsetof(Smem, KbT);
constexpr int OFF_TB = (int)offsetof(Smem, u);
constexpr int ROW_QK = (DK + 8) * 2;   // bytes per Qt / Kt row
constexpr int ROW_CC = (CH + 8) * 2;   // bytes per M / Tb row
static_assert(offsetof(Smem, M) == OFF_KBT + DK * ROW_CC, "KbT and M are contiguous");
static_assert(OFF_TB == (int)offsetof(Smem, M) + CH * ROW_CC, "Tb follows M");
static_assert(OFF_KT == OFF_QT + CH * ROW_QK, "Kt follows Qt");

// The image in global memory holds the tiles the chain reads, without the LDS
// row padding, in 16-byte pieces:
//   the Qt and Kt rows (16 pieces each);
//   the KbT rows (8 each);
//   the first 32 columns of rows 0..31 of M, then of Tb (4 each: the chain's
//   first row tile reads only those);
//   rows 32..63 of M, then of Tb (8 each);
//   one piece per Kt row padding for D (rows 0..31) and Tb's scale (row 32).
// Every part but the last fills whole rounds of NTHR pieces, so image_to_lds
// knows the part of each round at compile time.
constexpr int IMG_QK = 2 * CH * (DK / 8);          // Qt, Kt pieces
constexpr int IMG_KB = DK * (CH / 8);              // KbT pieces
constexpr int IMG_SHORT = 2 * 32 * 4;              // rows 0..31 of M and Tb, columns 0..31
constexpr int IMG_LONG = 32 * (CH / 8);            // rows 32..63 of M (or of Tb)
constexpr int IMG_PAD = DK / 4 + 1;                // Kt row paddings in use
constexpr int IMG_VEC = IMG_QK + IMG_KB + IMG_SHORT + 2 * IMG_LONG + IMG_PAD;
constexpr int IMG_BYTES = 16 * IMG_VEC;            // one image in global memory
constexpr int IMG_PER_THREAD = (IMG_VEC + NTHR - 1) / NTHR;  // pieces per thread (the last partial)
static_assert(ROW_QK == 17 * 16 && ROW_CC == 9 * 16, "rows are whole pieces plus one of padding");
static_assert(IMG_QK % NTHR == 0 && IMG_KB % NTHR == 0 && IMG_SHORT == NTHR && IMG_LONG == NTHR,
              "every part but the last fills whole rounds");
constexpr int OFF_M = OFF_KBT + DK * ROW_CC;       // LDS rows of M, then Tb
// global piece indices of the parts the pre kernel writes
constexpr int GP_KB = IMG_QK;
constexpr int GP_SHORT = GP_KB + IMG_KB;
constexpr int GP_MLONG = GP_SHORT + IMG_SHORT;
constexpr int GP_TLONG = GP_MLONG + IMG_LONG;
constexpr int GP_PAD = GP_TLONG + IMG_LONG;
// global piece of (row, 8-column piece cp) of M (t = 0) or Tb (t = 1); -1 for
// the pieces the chain never reads (rows 0..31, columns 32..63)
__device__ __forceinline__ int img_mt_piece(int t, int row, int cp) {
  if (row < 32) return cp < 4 ? GP_SHORT + 128 * t + 4 * row + cp : -1;
  return (t ? GP_TLONG : GP_MLONG) + 8 * (row - 32) + cp;
}

// LDS of the pre kernel (~70 KB: two workgroups per CU).  KbT and M are
// staged here in the image's own layout; Qt, Kt, Tb and D go straight from
// registers to the image in global memory.
struct alignas(16) PreSmem {
  _Float16 KbT[DK][CH + 8];
  _Float16 M[CH][CH + 8];
  struct {
    float A[CH][CH + 4];
  } u;
  union {
    f16x8 R[3][4][64];
    float T[CH][CH + 4];
  } u2;
  float etab[13][DK];
  float tot[4][DK];
  float beta[CH];
  float tbmax[8];
  int gate_bad;
};
// KbT and M rows staged in PreSmem (padded like Smem) go to the image piece by
// piece: KbT (whole rounds), then the M pieces the chain reads
static_assert(offsetof(PreSmem, M) == sizeof(((PreSmem*)nullptr)->KbT) && ROW_CC * DK == sizeof(((PreSmem*)nullptr)->KbT),
              "KbT and M rows are contiguous in the staging, ROW_CC apart");

// Store the 16x16 block (a, b) of M (lower incl., fp16) and of A
// (beta-scaled, strictly lower, fp32).  C layout of a 16x16 MFMA tile: lane l
// holds column l % 16 and rows 4 (l / 16) + 0..3.  beta_mine is beta of the
// token this lane holds in the prologue layout (token r = l % 16 of block a).
template <class Sm>
__device__ __forceinline__ void store_block(Sm& sm, const f32x4& accM, const f32x4& accA,
                                            int a, int b, int l, bool diag, float beta_mine) {
  const int col = l & 15;
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int row = 4 * (l >> 4) + qq;
    const int R = 16 * a + row, C = 16 * b + col;
    float mm = accM[qq], aa = accA[qq];
    if (diag) {
      if (col > row) mm = 0.f;
      if (col >= row) aa = 0.f;
    }
    aa *= __shfl(beta_mine, row);
    sm.u.A[R][C] = aa;
    sm.M[R][C] = (_Float16)mm;
  }
}

// ---------------------------------------------------------------------------
// work list: the scheduler's constants and the header it writes for the pre
// and main kernels
// ---------------------------------------------------------------------------
constexpr int SCHED_THREADS = 1024;
constexpr int NBUCKET = 1024;
constexpr int MIN_SPLIT_CHUNKS = 8;   // shorter documents are never split
constexpr int MAX_SPLIT_DOCS = 1024;  // split candidates examined (the longest documents)
// relative cost of one chunk of one head: fused (prepare + chain on one
// workgroup), prepare only (pre kernel), chain only (main kernel)
constexpr int COST_FUSED = 29, COST_PRE = 22, COST_CHAIN = 11;

enum SplitPolicy { SPLIT_NEVER = 0, SPLIT_AUTO = 1, SPLIT_ALWAYS = 2 };

struct WorkHeader {
  int counter;       // next unit of the main kernel
  int status;        // non-zero: cu_seqlens broke its contract
  int n_units;       // documents * heads
  int n_docs;        // listed documents
  int n_pre_units;   // split chunks * heads
  int n_split;       // split documents (the first n_split entries of the list)
  int n_state_docs;  // documents of h0 / ht (0 without states)
  int pad;
  // states in and out (null when absent) and the document index of each list
  // entry; kept here rather than in kernel arguments so that the main kernel
  // reads them only where it uses them
  const float* h0;
  float* ht;
  const int* doc_ids;
  int* status_word;  // the sticky device status word the main kernel reports to
  // with states: when not null, S at the start of every chunk is stored here,
  // fp32 [slot][H][K][V], slot = first token / 64 + document index + chunk
  // index in the document (distinct for all chunks of all documents)
  float* chunk_states;
};

// Sticky kda_device_flags of this device.  Every translation unit that
// includes this header has its own copy; the one of kda_fwd.hip is the one
// kda_device_status reads, and the scheduler passes its address on through
// WorkHeader::status_word.
__device__ int g_kda_status;

// ---------------------------------------------------------------------------
// per-chunk stages shared by the kernels
// ---------------------------------------------------------------------------
// ---- global memory through buffer descriptors.  A descriptor covers the
// rows of one chunk of one head; per-lane byte offsets (always in the VGPR
// offset, which the hardware range-checks) select token rows.  Rows at or past
// the end of the chunk are out of range: loads return 0, stores are dropped.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// bytes of the first n token rows of one head when a token row holds row_bytes
// for each of H heads (n <= 0: nothing)
__device__ __forceinline__ uint32_t chunk_bytes(int n, int H, uint32_t row_bytes) {
  return n > 0 ? ((uint32_t)(n - 1) * (uint32_t)H + 1u) * row_bytes : 0u;
}
__device__ __forceinline__ u32x4 bload(Rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ void bstore(u32x4 x, Rsrc r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(x, r, (int)off, 0, 0);
}

struct RawChunk {
  u32x4 q[4];    // 32 bf16 channels of one token (element 8 s + j = channel 32 s + 8 cg + j)
  u32x4 k[4];
  u32x4 g[8];    // the same 32 channels, fp32 bits
  float beta;
};

// per-lane byte offsets, fixed for the whole kernel
struct Offsets {
  uint32_t qk;    // token row of the prologue layout in q / k (g: twice this)
  uint32_t b;     // the same token in beta
  uint32_t v[4];  // V / O layout: row 16 i + l / 4, columns 32 w + 8 (l % 4) ..
};

__device__ __forceinline__ Offsets make_offsets(int H, int tok, int cg, int w, int l) {
  Offsets o;
  o.qk = (uint32_t)tok * (uint32_t)H * 256u + 16u * cg;
  o.b = (uint32_t)tok * (uint32_t)H * 4u;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o.v[i] = (uint32_t)(16 * i + (l >> 2)) * (uint32_t)H * 256u + 64u * w + 16u * (l & 3);
  return o;
}

// q, k, g, beta of the chunk of n tokens at token c0 (head h); tokens at or
// past n read as zero.  Element 8 s + j of this lane is channel 32 s + 8 cg + j:
// the four lanes of a token read one contiguous 64-byte (q, k) or 128-byte (g)
// span per load.  The loads are issued in three parts (q and k; the first and
// the second half of g, and beta) so that they can be spread over a chunk.
struct RawSrc {
  Rsrc q, k, g, b;
};

__device__ __forceinline__ RawSrc raw_src(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                          const float* __restrict__ g, const float* __restrict__ beta,
                                          int64_t c0, int n, int H, int h) {
  const size_t row = (size_t)c0 * H + h;
  const uint32_t nb = chunk_bytes(n, H, 256u);
  RawSrc src;
  src.q = make_rsrc(q + row * DK, nb);
  src.k = make_rsrc(k + row * DK, nb);
  src.g = make_rsrc(g + row * DK, 2u * nb);
  src.b = make_rsrc(beta + row, chunk_bytes(n, H, 4u));
  return src;
}

__device__ __forceinline__ void load_raw_part(RawChunk& rc, const RawSrc& src, const Offsets& of,
                                              int part) {
  if (part == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rc.q[i] = bload(src.q, of.qk + 64u * i);
      rc.k[i] = bload(src.k, of.qk + 64u * i);
    }
  } else if (part == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      rc.g[2 * i] = bload(src.g, 2u * of.qk + 128u * i);
      rc.g[2 * i + 1] = bload(src.g, 2u * of.qk + 128u * i + 16u);
    }
  } else {
#pragma unroll
    for (int i = 2; i < 4; ++i) {
      rc.g[2 * i] = bload(src.g, 2u * of.qk + 128u * i);
      rc.g[2 * i + 1] = bload(src.g, 2u * of.qk + 128u * i + 16u);
    }
    rc.beta = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(src.b, (int)of.b, 0, 0));
  }
}

__device__ __forceinline__ void load_raw(RawChunk& rc, const RawSrc& src, const Offsets& of) {
  load_raw_part(rc, src, of, 0);
  load_raw_part(rc, src, of, 1);
  load_raw_part(rc, src, of, 2);
}

// V of one chunk, the 32 value columns of wave w: load i, lane l holds 16 bytes
// of row 16 i + l / 4 (columns 32 w + 8 (l % 4) ..); rows past the end read 0.
struct VChunk {
  u32x4 r[4];
};

__device__ __forceinline__ VChunk load_v(const bf16* __restrict__ v, int64_t c0, int n, int H,
                                         int h, const Offsets& of) {
  const Rsrc rv = make_rsrc(v + ((size_t)c0 * H + h) * DV, chunk_bytes(n, H, 256u));
  VChunk vc;
#pragma unroll
  for (int i = 0; i < 4; ++i) vc.r[i] = bload(rv, of.v[i]);
  return vc;
}

// a chunk image in registers: thread tid holds pieces tid + NTHR i
struct Image {
  u32x4 p[IMG_PER_THREAD];
};

// pieces [i0, i1) of an image (the last round only covers the first waves)
__device__ __forceinline__ void load_image_part(Image& im, Rsrc r, int tid, int i0, int i1) {
#pragma unroll
  for (int i = 0; i < IMG_PER_THREAD; ++i)
    if (i >= i0 && i < i1 && tid + NTHR * i < IMG_VEC)
      im.p[i] = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * tid, 16 * NTHR * i, 0);
}

__device__ __forceinline__ void load_image(Image& im, const uint8_t* __restrict__ src, int tid) {
  load_image_part(im, make_rsrc(src, IMG_BYTES), tid, 0, IMG_PER_THREAD);
}

// each round of NTHR pieces lies in one part of the image: the part of round
// i is known at compile time
__device__ __forceinline__ void image_to_lds(Smem& sm, const Image& im, int tid) {
  uint8_t* dst = reinterpret_cast<uint8_t*>(&sm);
#pragma unroll
  for (int i = 0; i < IMG_PER_THREAD; ++i) {
    const int p = tid + NTHR * i;
    const int r0 = NTHR * i;  // first piece of the round
    int off;
    if (r0 < GP_KB) {
      off = OFF_QT + (p >> 4) * ROW_QK + (p & 15) * 16;
    } else if (r0 < GP_SHORT) {
      const int q = p - GP_KB;
      off = OFF_KBT + (q >> 3) * ROW_CC + (q & 7) * 16;
    } else if (r0 < GP_MLONG) {
      const int q = p - GP_SHORT;  // Tb rows follow M rows in LDS: row (q >> 2) + 64 (q >> 7)
      off = OFF_M + ((q & 127) >> 2) * ROW_CC + CH * ROW_CC * (q >> 7) + (q & 3) * 16;
    } else if (r0 < GP_PAD) {
      const int q = p - GP_MLONG;  // M rows 32..63, then Tb rows 32..63
      off = OFF_M + (32 + ((q & 255) >> 3)) * ROW_CC + CH * ROW_CC * (q >> 8) + (q & 7) * 16;
    } else {
      off = OFF_KT + (p - GP_PAD) * ROW_QK + 2 * DK;
    }
    if (p < IMG_VEC) *reinterpret_cast<u32x4*>(dst + off) = im.p[i];
  }
}

// Where prepare_chunk puts the image parts it holds in registers (Qt, Kt, Tb
// and D): the LDS image of the main kernel, or the global image.
struct LdsSink {
  Smem* sm;
  __device__ __forceinline__ void qk(int tok, int col, const bf16x8& qt, const bf16x8& kt) const {
    *reinterpret_cast<bf16x8*>(&sm->Qt[tok][col]) = qt;
    *reinterpret_cast<bf16x8*>(&sm->Kt[tok][col]) = kt;
  }
  __device__ __forceinline__ void dv(int c, float f) const { dvec(*sm, c)[c & 3] = f; }
  __device__ __forceinline__ void tb(int row, int col, const f16x8& x) const {
    *reinterpret_cast<f16x8*>(&sm->u.tb[row][col]) = x;
  }
  __device__ __forceinline__ void tbs(float f) const { *tbscale(*sm) = f; }
};

struct GlobalSink {
  Rsrc r;  // one image, IMG_BYTES (the layout above)
  __device__ __forceinline__ void qk(int tok, int col, const bf16x8& qt, const bf16x8& kt) const {
    const uint32_t o = (uint32_t)(tok * 2 * DK + 2 * col);
    bstore(__builtin_bit_cast(u32x4, qt), r, o);
    bstore(__builtin_bit_cast(u32x4, kt), r, 16 * CH * (DK / 8) + o);
  }
  __device__ __forceinline__ void dv(int c, float f) const {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(f), r, 16 * (GP_PAD + (c >> 2)) + 4 * (c & 3), 0, 0);
  }
  __device__ __forceinline__ void tb(int row, int col, const f16x8& x) const {
    const int pc = img_mt_piece(1, row, col >> 3);
    if (pc >= 0) bstore(__builtin_bit_cast(u32x4, x), r, 16 * pc);
  }
  __device__ __forceinline__ void tbs(float f) const {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(f), r, 16 * (GP_PAD + DK / 4), 0, 0);
  }
};

// lane i of each 16-lane row receives lane N of the same row
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + N, 0xF, 0xF, false));
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// largest value of a non-negative x over the wave (uniform result)
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_row_shr<1>(x));
  x = fmaxf(x, dpp_row_shr<2>(x));
  x = fmaxf(x, dpp_row_shr<4>(x));
  x = fmaxf(x, dpp_row_shr<8>(x));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// fp16 operands: the power of two e >= 0 that brings a largest magnitude m
// below 2^14 (e = 0 for m < 2^14), as the biased-exponent bits of 2^-e and 2^e
__device__ __forceinline__ int f16_exponent(float m) {
  const int ex = (__float_as_int(m) >> 23) & 0xFF;
  return max(0, ex - (127 + 13));
}
__device__ __forceinline__ float pow2i(int e) { return __int_as_float((127 + e) << 23); }
// the exponent for the wave's largest lane value m: 0 unless some lane has
// m >= 2^14 (the common case costs one compare and a ballot)
__device__ __forceinline__ int wave_f16_exponent(float m) {
  if (__builtin_amdgcn_ballot_w64(m >= 16384.f) == 0) return 0;
  return f16_exponent(wave_max(m));
}

__device__ __forceinline__ f32x4 mfma16k16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Per-channel decay factors of a chunk from the sub-block totals t_w (log2
// domain, so every factor is a bare exp2):
//   rows 0..3:  e^{G_end(w)}          = 2^{t_0 + .. + t_w}      (row 3 = e^{G_c} = D)
//   rows 4..6:  e^{G_c - G_end(w)}    = 2^{t_{w+1} + .. + t_3}, w = 0..2
//   rows 7..12: e^{G_end(w) - G_end(b)} = 2^{t_{b+1} + .. + t_w}, pair (w, b), b < w,
//               at row 7 + w (w - 1) / 2 + b
// D is also written to the image (sink.dv).
template <class Sm, class Sink>
__device__ __forceinline__ void fill_tables(Sm& sm, const Sink& sink, int tid) {
  // thread pair (c, half): channel c reads its four totals once; half 0 writes
  // rows 0..6, half 1 rows 7..12
  const int c = tid & (DK - 1);
  const float t0 = sm.tot[0][c], t1 = sm.tot[1][c], t2 = sm.tot[2][c], t3 = sm.tot[3][c];
  const float t12 = t1 + t2, t23 = t2 + t3, t123 = t12 + t3;
  if (tid < DK) {
    const float t01 = t0 + t1, t012 = t01 + t2;
    const float d = __builtin_amdgcn_exp2f(t012 + t3);
    sm.etab[0][c] = __builtin_amdgcn_exp2f(t0);
    sm.etab[1][c] = __builtin_amdgcn_exp2f(t01);
    sm.etab[2][c] = __builtin_amdgcn_exp2f(t012);
    sm.etab[3][c] = d;
    sink.dv(c, d);
    sm.etab[4][c] = __builtin_amdgcn_exp2f(t123);
    sm.etab[5][c] = __builtin_amdgcn_exp2f(t23);
    sm.etab[6][c] = __builtin_amdgcn_exp2f(t3);
  } else {
    sm.etab[7][c] = __builtin_amdgcn_exp2f(t1);     // (1, 0)
    sm.etab[8][c] = __builtin_amdgcn_exp2f(t12);    // (2, 0)
    sm.etab[9][c] = __builtin_amdgcn_exp2f(t2);     // (2, 1)
    sm.etab[10][c] = __builtin_amdgcn_exp2f(t123);  // (3, 0)
    sm.etab[11][c] = __builtin_amdgcn_exp2f(t23);   // (3, 1)
    sm.etab[12][c] = __builtin_amdgcn_exp2f(t3);    // (3, 2)
  }
}

// Off-diagonal blocks (W, b), b < W, of M and A on fp16 MFMA.  Left operand
// x_r e^{G_r - G_end(b)} = l{q,k} e^{G_end(W) - G_end(b)} <= 1; right operand
// kh_i e^{G_end(b) - G_i} <= 1 (R, written by wave b).
template <int W, class Sm>
__device__ __forceinline__ void offdiag_row(Sm& sm, const float (&lq)[32], const float (&lk)[32], int l,
                                            int cg, float beta_mine) {
#pragma unroll
  for (int b = 0; b < W; ++b) {
    const float* fr = sm.etab[7 + (W * (W - 1)) / 2 + b];
    f32x4 accM[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    f32x4 accA[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f16x8 rv = sm.u2.R[b][s][l];
      const float4 fa = *reinterpret_cast<const float4*>(&fr[32 * s + 8 * cg]);
      const float4 fb = *reinterpret_cast<const float4*>(&fr[32 * s + 8 * cg + 4]);
      const float f[8] = {fa.x, fa.y, fa.z, fa.w, fb.x, fb.y, fb.z, fb.w};
      f16x8 lqv, lkv;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        lqv[j] = (_Float16)(lq[8 * s + j] * f[j]);
        lkv[j] = (_Float16)(lk[8 * s + j] * f[j]);
      }
      accM[s & 1] = mfma16h(lqv, rv, accM[s & 1]);
      accA[s & 1] = mfma16h(lkv, rv, accA[s & 1]);
    }
    store_block(sm, accM[0] + accM[1], accA[0] + accA[1], W, b, l, false, beta_mine);
  }
}

// Column block B of T = (I + A)^-1 below the diagonal, on fp32 16x16x4 MFMA
// (the diagonal blocks T_aa are in LDS).  k-step s of lane group g = l / 16
// takes k = 4 g + s on both operands, so the C layout of one product (lane l:
// rows 4 g .. 4 g + 3 of column l % 16) is the B operand of the next: the
// blocks T_kB stay in registers.  Returns tmax updated with |T_aB beta_col|.
template <int B, class Sm>
__device__ __forceinline__ float levels_column(Sm& sm, int l, float tmax) {
  const int c = l & 15, g4 = 4 * (l >> 4);
  f32x4 tcol[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) tcol[B][i] = sm.u2.T[16 * B + g4 + i][16 * B + c];
  const float bc = fabsf(sm.beta[16 * B + c]);
#pragma unroll
  for (int a = B + 1; a < 4; ++a) {
    f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = B; kb < a; ++kb) {
      const float4 av = *reinterpret_cast<const float4*>(&sm.u.A[16 * a + c][16 * kb + g4]);
      Y = mfma16f(av.x, tcol[kb][0], Y);
      Y = mfma16f(av.y, tcol[kb][1], Y);
      Y = mfma16f(av.z, tcol[kb][2], Y);
      Y = mfma16f(av.w, tcol[kb][3], Y);
    }
    const float4 tv = *reinterpret_cast<const float4*>(&sm.u2.T[16 * a + c][16 * a + g4]);
    f32x4 Z = {0.f, 0.f, 0.f, 0.f};
    Z = mfma16f(tv.x, Y[0], Z);
    Z = mfma16f(tv.y, Y[1], Z);
    Z = mfma16f(tv.z, Y[2], Z);
    Z = mfma16f(tv.w, Y[3], Z);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tcol[a][i] = -Z[i];
      sm.u2.T[16 * a + g4 + i][16 * B + c] = -Z[i];
      tmax = fmaxf(tmax, fabsf(Z[i]) * bc);
    }
  }
  return tmax;
}

// lane coordinates inside the workgroup
struct Lane {
  int tid;
  int w;    // wave (scalar)
  int l;    // lane
  int r;    // prologue: token inside the 16-token sub-block
  int cg;   // prologue: channel group
  int m;    // chain: MFMA row / column lane index
  int hg;   // chain: lane half
  int tok;  // prologue: token of this lane inside the chunk
};

__device__ __forceinline__ Lane make_lane() {
  Lane ln;
  ln.tid = threadIdx.x;
  ln.w = __builtin_amdgcn_readfirstlane(ln.tid >> 6);
  ln.l = ln.tid & 63;
  ln.r = ln.l & 15;
  ln.cg = ln.l >> 4;
  ln.m = ln.l & 31;
  ln.hg = ln.l >> 5;
  ln.tok = 16 * ln.w + ln.r;
  return ln;
}

// Everything of a chunk that does not depend on the state: from the raw
// inputs `cur` (n valid tokens) to the image in LDS (Qt, Kt, KbT, M, Tb, D).
// hook(0..2) run at fixed points once `cur` has been consumed (they may
// refill it); the scheduling barriers keep the loads they issue spread out.
// Ends with a workgroup barrier after which the image is complete.
template <class Sm, class Sink, class Hook>
__device__ __forceinline__ void prepare_chunk(Sm& sm, const Sink& sink, const RawChunk& cur, int n,
                                              float gate_bound, const Lane& ln, Hook hook) {
  const int tid = ln.tid, w = ln.w, l = ln.l, r = ln.r, cg = ln.cg, tok = ln.tok;

  // ================= prologue: l2 norm, cumulative decay =================
  // lane (w, r, cg): token 16w + r of the chunk; element 8 s + j is channel
  // 32 s + 8 cg + j (k-step s of the 16x16x32 MFMAs takes elements 8 s .. 8 s + 7).
  // lq, lk: qh, kh times e^{G - G_end(w)} (>= 1); kr: kh e^{G_end(w) - G} (<= 1),
  // where G_end(w) is the cumulative decay at the last token of sub-block w.
  float lq[32], lk[32], kr[32];
  const float beta_mine = cur.beta;
  {
    float qh[32], kh[32], lg[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t qa[4] = {cur.q[i][0], cur.q[i][1], cur.q[i][2], cur.q[i][3]};
      const uint32_t ka[4] = {cur.k[i][0], cur.k[i][1], cur.k[i][2], cur.k[i][3]};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qh[8 * i + 2 * j] = bf16_lo_to_f32(qa[j]);
        qh[8 * i + 2 * j + 1] = bf16_hi_to_f32(qa[j]);
        kh[8 * i + 2 * j] = bf16_lo_to_f32(ka[j]);
        kh[8 * i + 2 * j + 1] = bf16_hi_to_f32(ka[j]);
      }
    }
    float gmin = 0.f, gmax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float ga[4] = {__uint_as_float(cur.g[i][0]), __uint_as_float(cur.g[i][1]),
                           __uint_as_float(cur.g[i][2]), __uint_as_float(cur.g[i][3])};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        gmin = fminf(gmin, ga[j]);
        gmax = fmaxf(gmax, ga[j]);
        lg[4 * i + j] = ga[j] * 1.4426950408889634f;  // log2 domain
      }
    }
    if (tok < n && !(gmin >= gate_bound && gmax <= 0.f)) sm.gate_bad = 1;
    if (cg == 0) sm.beta[tok] = cur.beta;
    __builtin_amdgcn_sched_barrier(0);
    hook(0);
    __builtin_amdgcn_sched_barrier(0);
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) { sq += qh[j] * qh[j]; sk += kh[j] * kh[j]; }
    sq += __shfl_xor(sq, 16);
    sq += __shfl_xor(sq, 32);
    sk += __shfl_xor(sk, 16);
    sk += __shfl_xor(sk, 32);
    const float rq = __builtin_amdgcn_rsqf(sq + L2_EPS);  // hardware 1/sqrt (~1 ulp)
    const float rk = __builtin_amdgcn_rsqf(sk + L2_EPS);
    // inclusive scan over the 16 tokens of the sub-block (one 16-lane row),
    // step-major so that no DPP read waits on the write just before it
#pragma unroll
    for (int j = 0; j < 32; ++j) lg[j] += dpp_row_shr<1>(lg[j]);
#pragma unroll
    for (int j = 0; j < 32; ++j) lg[j] += dpp_row_shr<2>(lg[j]);
#pragma unroll
    for (int j = 0; j < 32; ++j) lg[j] += dpp_row_shr<4>(lg[j]);
#pragma unroll
    for (int j = 0; j < 32; ++j) lg[j] += dpp_row_shr<8>(lg[j]);
    if (r == 15) {
#pragma unroll
      for (int j = 0; j < 32; j += 4)
        *reinterpret_cast<float4*>(&sm.tot[w][32 * (j >> 3) + 8 * cg + (j & 7)]) =
            make_float4(lg[j], lg[j + 1], lg[j + 2], lg[j + 3]);
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float ert = __builtin_amdgcn_exp2f(row_bcast<15>(lg[j]) - lg[j]);  // <= 1
      const float elt = __builtin_amdgcn_rcpf(ert);                             // >= 1
      const float qn = qh[j] * rq, kn = kh[j] * rk;
      lq[j] = qn * elt;
      lk[j] = kn * elt;
      kr[j] = kn * ert;
    }
  }

  // diagonal block (w, w) of M and A on fp32 MFMA: k-step s takes element s
  // from every lane (the same channel on both operands)
  {
    f32x4 accM[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    f32x4 accA[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      accM[s & 1] = mfma16f(lq[s], kr[s], accM[s & 1]);
      accA[s & 1] = mfma16f(lk[s], kr[s], accA[s & 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
    hook(1);
    __builtin_amdgcn_sched_barrier(0);
    store_block(sm, accM[0] + accM[1], accA[0] + accA[1], w, w, l, true, beta_mine);
    // the chain's MFMAs read the upper blocks (0, 1) and (2, 3) (inside the two
    // diagonal 32x32 tiles): zero them; the other upper blocks are never read
    if (w == 0 || w == 2) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) sm.M[16 * w + 4 * (l >> 4) + qq][16 * (w + 1) + (l & 15)] = (_Float16)0.f;
    }
    if (w < 3) {
      // right operand of the pairs (a > w, w): kh_i e^{G_end(w) - G_i} <= 1
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        f16x8 rv;
#pragma unroll
        for (int j = 0; j < 8; ++j) rv[j] = (_Float16)kr[8 * s + j];
        sm.u2.R[w][s][l] = rv;
      }
    }
  }
  __syncthreads();  // B1: tot, beta, R, diagonal A / M visible
  fill_tables(sm, sink, tid);
  __syncthreads();  // B2: decay tables visible

  // ---- operand tiles of the chain: Qt = lq e^{G_end(w)}, Kt = -lk e^{G_end(w)},
  //      KbT = kr e^{G_c - G_end(w)}
#pragma unroll
  for (int j0 = 0; j0 < 32; j0 += 8) {
    float fq[8], fk[8];
    {
      const float4 a = *reinterpret_cast<const float4*>(&sm.etab[w][4 * j0 + 8 * cg]);
      const float4 b = *reinterpret_cast<const float4*>(&sm.etab[w][4 * j0 + 8 * cg + 4]);
      fq[0] = a.x; fq[1] = a.y; fq[2] = a.z; fq[3] = a.w;
      fq[4] = b.x; fq[5] = b.y; fq[6] = b.z; fq[7] = b.w;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) fk[j] = 1.f;
    if (w < 3) {
      const float4 a = *reinterpret_cast<const float4*>(&sm.etab[4 + w][4 * j0 + 8 * cg]);
      const float4 b = *reinterpret_cast<const float4*>(&sm.etab[4 + w][4 * j0 + 8 * cg + 4]);
      fk[0] = a.x; fk[1] = a.y; fk[2] = a.z; fk[3] = a.w;
      fk[4] = b.x; fk[5] = b.y; fk[6] = b.z; fk[7] = b.w;
    }
    bf16x8 qt, kt;
    f16x8 kb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      qt[j] = (bf16)(lq[j0 + j] * fq[j]);
      kt[j] = (bf16)(-lk[j0 + j] * fq[j]);
      kb[j] = (_Float16)(kr[j0 + j] * fk[j]);
    }
    sink.qk(tok, 4 * j0 + 8 * cg, qt, kt);
    // KbT is the transpose of these rows: multiplying by the identity on
    // MFMA (exact) leaves lane l with channel 32 s + l % 16 (and + 16) of
    // tokens 4 (l / 16) .. + 3, one 8-byte LDS store each
    {
      const int s8 = j0 / 8;
      f16x8 id0, id1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        id0[j] = (_Float16)((8 * cg + j == r) ? 1.f : 0.f);
        id1[j] = (_Float16)((8 * cg + j == 16 + r) ? 1.f : 0.f);
      }
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      const f32x4 c0 = mfma16h(kb, id0, z);
      const f32x4 c1 = mfma16h(kb, id1, z);
      f16x4 t0, t1;
#pragma unroll
      for (int i = 0; i < 4; ++i) { t0[i] = (_Float16)c0[i]; t1[i] = (_Float16)c1[i]; }
      *reinterpret_cast<f16x4*>(&sm.KbT[32 * s8 + r][16 * w + 4 * cg]) = t0;
      *reinterpret_cast<f16x4*>(&sm.KbT[32 * s8 + 16 + r][16 * w + 4 * cg]) = t1;
    }
  }

  __builtin_amdgcn_sched_barrier(0);
  hook(2);
  __builtin_amdgcn_sched_barrier(0);
  // ---- off-diagonal blocks (w, b), b < w, on fp16 MFMA (fully unrolled per
  // wave).  Wave 0, which has none, meanwhile inverts the four diagonal
  // blocks of I + A (complete since B1): T = (I + A)^-1 by 16x16 blocks, by
  // forward substitution, lane l owning column l % 16 of diagonal block
  // l / 16.  tmax tracks the largest |Tb| = |T_ij beta_j| a wave produces.
  // T shares its space with R, which waves 1-3 still read: until B3 the
  // columns wait in an upper block of A (A is strictly lower; its upper
  // blocks are never written or read): block da in block (pr, pc).
  const int da = l >> 4, dj = l & 15;
  const int pr = da == 3 ? 1 : da, pc = da == 3 ? 3 : da + 1;
  float tmax = 0.f;
  if (w == 1) offdiag_row<1>(sm, lq, lk, l, cg, beta_mine);
  else if (w == 2) offdiag_row<2>(sm, lq, lk, l, cg, beta_mine);
  else if (w == 3) offdiag_row<3>(sm, lq, lk, l, cg, beta_mine);
  else {
    // column-oriented: once x_i is final, subtract its share from every later
    // row (dependency depth 16 instead of the 120 terms of row dot products);
    // A is read four columns at a time (off the critical path, few registers)
    float x[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) x[rr] = (rr == dj) ? 1.f : 0.f;
#pragma unroll
    for (int i0 = 0; i0 < 16; i0 += 4) {
      float4 ac[16];
#pragma unroll
      for (int rr = i0 + 1; rr < 16; ++rr)
        ac[rr] = *reinterpret_cast<const float4*>(&sm.u.A[16 * da + rr][16 * da + i0]);
#pragma unroll
      for (int i = i0; i < i0 + 4 && i < 15; ++i)
#pragma unroll
        for (int rr = i + 1; rr < 16; ++rr) {
          const float4 a = ac[rr];
          const float air = i == i0 ? a.x : i == i0 + 1 ? a.y : i == i0 + 2 ? a.z : a.w;
          x[rr] -= air * x[i];
        }
    }
    const float bj = fabsf(sm.beta[16 * da + dj]);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      sm.u.A[16 * pr + rr][16 * pc + dj] = x[rr];
      tmax = fmaxf(tmax, fabsf(x[rr]) * bj);
    }
  }

  __syncthreads();  // B3: A and M complete, R dead (T, which shares its space, may be written)
  if (w == 0) {
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) sm.u2.T[16 * da + rr][16 * da + dj] = sm.u.A[16 * pr + rr][16 * pc + dj];
    if (da == 0 || da == 2) {  // upper blocks (0, 1) and (2, 3): read by U = Tb X
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sm.u2.T[16 * da + rr][16 * (da + 1) + dj] = 0.f;
    }
  }
  __syncthreads();  // B4: diagonal blocks of T visible
  // off-diagonal blocks: wave b walks column block b downwards,
  // T_ab = -T_aa sum_{k=b}^{a-1} A_ak T_kb, on fp32 MFMA
  if (w == 0) tmax = levels_column<0>(sm, l, tmax);
  else if (w == 1) tmax = levels_column<1>(sm, l, tmax);
  else if (w == 2) tmax = levels_column<2>(sm, l, tmax);
  tmax = wave_max(tmax);
  if (l == 0) sm.tbmax[w] = tmax;
  __syncthreads();  // B5: T complete
  // Tb = T Diag(beta) 2^-e in fp16 (in LDS it overwrites A), e chosen so
  // that |Tb 2^-e| < 2^14 (e = 0 unless Tb is huge): thread tid converts row
  // tid / 4, columns 16 (tid % 4) .. + 15
  {
    const int e = f16_exponent(fmaxf(fmaxf(sm.tbmax[0], sm.tbmax[1]), fmaxf(sm.tbmax[2], sm.tbmax[3])));
    const float down = pow2i(-e);
    if (tid == 0) sink.tbs(pow2i(e));
    const int rr = tid >> 2;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int cc = 16 * (tid & 3) + 8 * half;
      const float4 t0 = *reinterpret_cast<const float4*>(&sm.u2.T[rr][cc]);
      const float4 t1 = *reinterpret_cast<const float4*>(&sm.u2.T[rr][cc + 4]);
      const float4 b0 = *reinterpret_cast<const float4*>(&sm.beta[cc]);
      const float4 b1 = *reinterpret_cast<const float4*>(&sm.beta[cc + 4]);
      const float x[8] = {t0.x * b0.x, t0.y * b0.y, t0.z * b0.z, t0.w * b0.w,
                          t1.x * b1.x, t1.y * b1.y, t1.z * b1.z, t1.w * b1.w};
      f16x8 th;
#pragma unroll
      for (int j = 0; j < 8; ++j) th[j] = (_Float16)(x[j] * down);
      sink.tb(rr, cc, th);
    }
  }
  __syncthreads();  // B6: the image is complete, T dead (its space stages O)
}

// The state-dependent part of a chunk of n tokens starting at token c0, from
// the image in LDS and this chunk's V (wave w owns value columns 32 w ..):
//   X = V - Kt S,  U = Tb X,  O = scale (Qt S + M U),  S <- D S + KbT U.
// hook(0..3) run at fixed points after V has been consumed (they may refill
// vcur): after the V staging, after X, after U and after O.
template <class Hook>
__device__ __forceinline__ void chain_chunk(Smem& sm, f32x16 (&S)[4], const VChunk& vcur, int n,
                                            int64_t c0, int H, int h, bf16* __restrict__ out,
                                            const Lane& ln, const Offsets& of, Hook hook) {
  const int w = ln.w, l = ln.l, m = ln.m, hg = ln.hg;
  const float scale = 0.08838834764831845f;  // 128^-1/2

  // this chunk's V, transposed into the wave's staging slice (rows past
  // the end were read as zero)
  unsigned short (*vt)[CH + 8] = sm.u2.ws[w].vt;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 16 * i + (l >> 2);
    const u32x4 u = vcur.r[i];
    const uint32_t uu[4] = {u[0], u[1], u[2], u[3]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // column c keeps token t at t ^ 8 (c / 8): columns 8 apart (whose rows
      // share banks) write different banks; 8-token groups stay contiguous
      vt[8 * (l & 3) + 2 * j][t ^ (8 * (l & 3))] = (unsigned short)(uu[j] & 0xFFFFu);
      vt[8 * (l & 3) + 2 * j + 1][t ^ (8 * (l & 3))] = (unsigned short)(uu[j] >> 16);
    }
  }
  wave_sync_lds();
  const int rowsel = swap23(m);
  // V in the C layout of the X tiles (packed bf16; added after the product)
  u32x4 vx[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      vx[mt][hh] = *reinterpret_cast<const u32x4*>(&vt[m][(32 * mt + 16 * hh + 8 * hg) ^ (8 * (m >> 3))]);
  wave_sync_lds();  // V read out before the slice stages O
  __builtin_amdgcn_sched_barrier(0);
  hook(0);
  __builtin_amdgcn_sched_barrier(0);

  bf16x8 Sb[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) Sb[s][j] = (bf16)S[s >> 1][8 * (s & 1) + j];

  // X = V - kh e^G S (A operands loaded two k-steps ahead; Kt holds -kh e^G)
  f32x16 X[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) X[mt][i] = 0.f;
  {
    bf16x8 ka[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        ka[mt][s] = *reinterpret_cast<const bf16x8*>(&sm.Kt[32 * mt + rowsel][16 * s + 8 * hg]);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        X[mt] = mfma32(ka[mt][s & 1], Sb[s], X[mt]);
        if (s + 2 < 8)
          ka[mt][s & 1] = *reinterpret_cast<const bf16x8*>(&sm.Kt[32 * mt + rowsel][16 * (s + 2) + 8 * hg]);
      }
    }
  }
  // X in fp16, divided by 2^eX when |X| would not fit (eX = 0 almost always)
  float xv[32];
  float xmax = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t vv = vx[s >> 1][s & 1][j];
      xv[8 * s + 2 * j] = X[s >> 1][8 * (s & 1) + 2 * j] + bf16_lo_to_f32(vv);
      xv[8 * s + 2 * j + 1] = X[s >> 1][8 * (s & 1) + 2 * j + 1] + bf16_hi_to_f32(vv);
      xmax = fmaxf(xmax, fmaxf(fabsf(xv[8 * s + 2 * j]), fabsf(xv[8 * s + 2 * j + 1])));
    }
  const int ex = wave_f16_exponent(xmax);
  if (ex != 0) {
    const float down = pow2i(-ex);
#pragma unroll
    for (int i = 0; i < 32; ++i) xv[i] *= down;
  }
  f16x8 Xh[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) Xh[s][j] = (_Float16)xv[8 * s + j];
  __builtin_amdgcn_sched_barrier(0);
  hook(1);
  __builtin_amdgcn_sched_barrier(0);

  // U = Tb X: the six lower-triangular (row tile, k-step) pairs, fp16 operands
  constexpr int PMT[6] = {0, 0, 1, 1, 1, 1};
  constexpr int PS[6] = {0, 1, 0, 1, 2, 3};
  f32x16 U[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) U[mt][i] = 0.f;
  {
    // order (1,0) (0,0) (1,1) (0,1) (1,2) (1,3): the two row tiles alternate;
    // operands are loaded two pairs ahead
    constexpr int ORD[6] = {2, 0, 3, 1, 4, 5};
    f16x8 th[2];
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const int p = ORD[o];
      th[o] = *reinterpret_cast<const f16x8*>(&sm.u.tb[32 * PMT[p] + rowsel][16 * PS[p] + 8 * hg]);
    }
#pragma unroll
    for (int o = 0; o < 6; ++o) {
      const int p = ORD[o];
      U[PMT[p]] = mfma32h(th[o & 1], Xh[PS[p]], U[PMT[p]]);
      if (o + 2 < 6) {
        const int pn = ORD[o + 2];
        th[o & 1] = *reinterpret_cast<const f16x8*>(&sm.u.tb[32 * PMT[pn] + rowsel][16 * PS[pn] + 8 * hg]);
      }
    }
  }
  // undo the scalings of Tb and X (powers of two, exact)
  {
    const float up = *tbscale(sm) * pow2i(ex);
    if (up != 1.f) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) U[mt][i] *= up;
    }
  }
  // U in fp16 (divided by 2^eu when needed) for M U and the state update
  f16x8 Uh[4];
  float umax = 0.f;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) umax = fmaxf(umax, fabsf(U[mt][i]));
  const int eu = wave_f16_exponent(umax);
  const float udown = pow2i(-eu);
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      Uh[s][j] = (_Float16)(U[s >> 1][8 * (s & 1) + j] * udown);
    }
  if (eu != 0) {
    // M U is computed as M (U 2^-eu): bring Qt S to the same scale
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) Sb[s][j] = (bf16)(S[s >> 1][8 * (s & 1) + j] * udown);
  }
  __builtin_amdgcn_sched_barrier(0);
  hook(2);
  __builtin_amdgcn_sched_barrier(0);

  // O = scale (qh e^G S + M U), staged through LDS for 16-byte stores;
  // one accumulator per row tile
  unsigned short (*ost)[32] = sm.u2.ws[w].o;
  {
    const float oscale = scale * pow2i(eu);
    f32x16 O[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[mt][i] = 0.f;
    bf16x8 qa[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        qa[mt][s] = *reinterpret_cast<const bf16x8*>(&sm.Qt[32 * mt + rowsel][16 * s + 8 * hg]);
    // M operands loaded two pairs ahead
    f16x8 mh[2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
      mh[p] = *reinterpret_cast<const f16x8*>(&sm.M[32 * PMT[p] + rowsel][16 * PS[p] + 8 * hg]);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        O[mt] = mfma32(qa[mt][s & 1], Sb[s], O[mt]);
        if (s + 2 < 8)
          qa[mt][s & 1] = *reinterpret_cast<const bf16x8*>(&sm.Qt[32 * mt + rowsel][16 * (s + 2) + 8 * hg]);
      }
      if (s < 6) {
        const int p = s;
        O[PMT[p]] = mfma32h(mh[p & 1], Uh[PS[p]], O[PMT[p]]);
        if (p + 2 < 6)
          mh[p & 1] = *reinterpret_cast<const f16x8*>(&sm.M[32 * PMT[p + 2] + rowsel][16 * PS[p + 2] + 8 * hg]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = 32 * mt + 16 * (i >> 3) + 8 * hg + (i & 7);
        const bf16 ob = (bf16)(O[mt][i] * oscale);
        ost[t][m] = __builtin_bit_cast(unsigned short, ob);
      }
  }

  __builtin_amdgcn_sched_barrier(0);
  hook(3);
  __builtin_amdgcn_sched_barrier(0);
  // S <- e^{G_c} S + (kh e^{G_c - G})^T U: the product accumulates from zero
  // (the four row tiles interleaved) and S takes it with one fma per element,
  // so S itself is only ever touched by vector ALU code
  {
    f32x16 dS[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) dS[kt][i] = 0.f;
    f16x8 kb[2][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      kb[0][kt] = *reinterpret_cast<const f16x8*>(&sm.KbT[32 * kt + rowsel][8 * hg]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        if (s + 1 < 4)
          kb[(s + 1) & 1][kt] = *reinterpret_cast<const f16x8*>(&sm.KbT[32 * kt + rowsel][16 * (s + 1) + 8 * hg]);
        dS[kt] = mfma32h(kb[s & 1][kt], Uh[s], dS[kt]);
      }
    }
    if (eu != 0) {  // the product took U 2^-eu (exact power of two)
      const float up = pow2i(eu);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) dS[kt][i] *= up;
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i0 = 0; i0 < 16; i0 += 8) {
        const int c = 32 * kt + 16 * (i0 >> 3) + 8 * hg;
        const float4 d0 = *reinterpret_cast<const float4*>(dvec(sm, c));
        const float4 d1 = *reinterpret_cast<const float4*>(dvec(sm, c + 4));
        const float d[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) S[kt][i0 + j] = fmaf(d[j], S[kt][i0 + j], dS[kt][i0 + j]);
      }
  }

  // O rows: lane l writes 16 bytes of row 16 it + l / 4 (rows past the end
  // are dropped by the descriptor's range)
  wave_sync_lds();
  const Rsrc ro = make_rsrc(out + ((size_t)c0 * H + h) * DV, chunk_bytes(n, H, 256u));
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int t = 16 * it + (l >> 2);
    bstore(*reinterpret_cast<const u32x4*>(&ost[t][8 * (l & 3)]), ro, of.v[it]);
  }
}

// ---------------------------------------------------------------------------
// state in and out.  In registers, S[kt][i] holds key channel
// 32 kt + 16 (i / 8) + 8 hg + i % 8 and value column 32 w + m (the C layout of
// the chain's 32x32 products); in memory one state is fp32 [K][V], so the 32
// lanes of a half-wave touch 128 contiguous bytes of one key row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t state_lane_offset(const Lane& ln) {
  return (uint32_t)((8 * ln.hg * DV + 32 * ln.w + ln.m) * 4);
}
__device__ __forceinline__ int state_row_offset(int kt, int i) {
  return (32 * kt + 16 * (i >> 3) + (i & 7)) * DV * 4;
}
__device__ __forceinline__ void load_state(f32x16 (&S)[4], const float* src, const Lane& ln) {
  const Rsrc r = make_rsrc(src, DK * DV * 4);
  const uint32_t lo = state_lane_offset(ln);
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      S[kt][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)lo, state_row_offset(kt, i), 0));
}
__device__ __forceinline__ void store_state(const f32x16 (&S)[4], float* dst, const Lane& ln) {
  const Rsrc r = make_rsrc(dst, DK * DV * 4);
  const uint32_t lo = state_lane_offset(ln);
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[kt][i]), r, (int)lo, state_row_offset(kt, i), 0);
}

// ---------------------------------------------------------------------------
// main kernel: one (document, head) unit at a time; fused documents prepare
// and chain each chunk, split documents chain precomputed images.  With
// h0 / ht (then doc_ids maps a unit's list entry to its document index), a
// unit starts from h0[doc][h] instead of zero and stores its last state to
// ht[doc][h]; each unit touches only its own slot, so ht may equal h0.
// ---------------------------------------------------------------------------
template <bool kState>
__global__ __launch_bounds__(NTHR, 1) void kda_chunk_fwd_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, bf16* __restrict__ out,
    WorkHeader* __restrict__ hdr, const int2* __restrict__ docs, const int2* __restrict__ split,
    const uint8_t* __restrict__ images, int64_t T, int H, float gate_bound) {
  __shared__ Smem sm;
  const Lane ln = make_lane();
  const int tid = ln.tid, w = ln.w, l = ln.l;

  if (hdr->status != 0) {
    // cu_seqlens was rejected on the device: make the failure visible
    const size_t total = (size_t)T * H * DV;
    const size_t stride = (size_t)gridDim.x * NTHR;
    unsigned short* o16 = reinterpret_cast<unsigned short*>(out);
    for (size_t i = (size_t)blockIdx.x * NTHR + tid; i < total; i += stride) o16[i] = 0x7FC0;
    if (kState && hdr->ht != nullptr) {
      float* ht = hdr->ht;
      const size_t nst = (size_t)hdr->n_state_docs * H * DK * DV;
      for (size_t i = (size_t)blockIdx.x * NTHR + tid; i < nst; i += stride) ht[i] = __builtin_nanf("");
    }
    return;
  }
  const int n_units = hdr->n_units;
  const Offsets of = make_offsets(H, ln.tok, ln.cg, w, l);
  if (tid == 0) sm.gate_bad = 0;

  for (;;) {
    __syncthreads();
    if (tid == 0) sm.unit = atomicAdd(&hdr->counter, 1);
    __syncthreads();
    const int unit = __builtin_amdgcn_readfirstlane(sm.unit);
    if (unit >= n_units) break;
    const int di = unit / H;
    const int h = unit - di * H;
    const int2 doc = docs[di];

    // S starts at zero or at h0[doc][h]; with states, the last S goes to
    // ht[doc][h].  Each branch below keeps its own S (its own registers).
    auto state_in = [&](f32x16 (&S)[4]) {
      const float* h0 = kState ? hdr->h0 : nullptr;
      if (h0 != nullptr) {
        load_state(S, h0 + ((size_t)hdr->doc_ids[di] * H + h) * (DK * DV), ln);
      } else {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) S[kt][i] = 0.f;
      }
    };
    // S at the start of the chunk that begins at token c0 (states only)
    auto save_chunk = [&](const f32x16 (&S)[4], int64_t c0) {
      if constexpr (kState) {
        float* cs = hdr->chunk_states;
        if (cs != nullptr) {
          const int u = __builtin_amdgcn_readfirstlane(sm.unit);
          const int d = u / H;
          const int2 dd = docs[d];
          const int64_t first = dd.x < 0 ? (int64_t)split[-dd.x - 1].x : (int64_t)dd.x;
          const int64_t slot = first / CH + hdr->doc_ids[d] + (c0 - first) / CH;
          store_state(S, cs + ((size_t)slot * H + (u - d * H)) * (DK * DV), ln);
        }
      }
    };
    auto state_out = [&](const f32x16 (&S)[4]) {
      if constexpr (kState) {
        // the unit's indices again, from LDS (nothing kept live across the chain)
        const int u = __builtin_amdgcn_readfirstlane(sm.unit);
        const int d = u / H;
        float* ht = hdr->ht;
        if (ht != nullptr) store_state(S, ht + ((size_t)hdr->doc_ids[d] * H + (u - d * H)) * (DK * DV), ln);
      }
    };

    if (doc.x < 0) {
      // ---- split document: chain over precomputed images
      const int2 sp = split[-doc.x - 1];
      const int64_t bos = sp.x, eos = (int64_t)sp.x + doc.y;
      const uint8_t* img = images + ((size_t)sp.y * H + h) * IMG_BYTES;
      const size_t img_stride = (size_t)H * IMG_BYTES;
      Image im;
      load_image(im, img, tid);
      VChunk vcur = load_v(v, bos, (int)min<int64_t>(CH, eos - bos), H, h, of);
      f32x16 S[4];
      state_in(S);
      for (int64_t c0 = bos; c0 < eos; c0 += CH) {
        const int n = (int)min<int64_t>(CH, eos - c0);
        save_chunk(S, c0);
        image_to_lds(sm, im, tid);
        __syncthreads();  // the image is in LDS
        img += img_stride;
        const int64_t c1 = c0 + CH;
        const int n1 = (int)min<int64_t>(CH, eos - c1);
        const Rsrc rimg = make_rsrc(img, c1 < eos ? IMG_BYTES : 0);
        chain_chunk(sm, S, vcur, n, c0, H, h, out, ln, of, [&](int stage) {
          static_assert(IMG_PER_THREAD == 16, "the four load parts cover the image");
          if (stage == 0) {
            vcur = load_v(v, c1, n1, H, h, of);
            load_image_part(im, rimg, tid, 0, 4);
          } else if (stage == 1) {
            load_image_part(im, rimg, tid, 4, 8);
          } else if (stage == 2) {
            load_image_part(im, rimg, tid, 8, 12);
          } else {
            load_image_part(im, rimg, tid, 12, IMG_PER_THREAD);
          }
        });
        __syncthreads();  // the next chunk overwrites the image
      }
      state_out(S);
    } else {
      // ---- fused document: prepare and chain each chunk here
      const int64_t bos = doc.x, eos = (int64_t)doc.x + doc.y;
      RawChunk cur;
      VChunk vcur;
      {
        const int n0 = (int)min<int64_t>(CH, eos - bos);
        load_raw(cur, raw_src(q, k, g, beta, bos, n0, H, h), of);
        vcur = load_v(v, bos, n0, H, h, of);
      }
      f32x16 S[4];
      state_in(S);
      for (int64_t c0 = bos; c0 < eos; c0 += CH) {
        const int n = (int)min<int64_t>(CH, eos - c0);
        const int64_t c1 = c0 + CH;
        const int n1 = (int)min<int64_t>(CH, eos - c1);
        const RawSrc src = raw_src(q, k, g, beta, c1, n1, H, h);
        save_chunk(S, c0);
        prepare_chunk(sm, LdsSink{&sm}, cur, n, gate_bound, ln,
                      [&](int part) { load_raw_part(cur, src, of, part); });
        chain_chunk(sm, S, vcur, n, c0, H, h, out, ln, of, [&](int stage) {
          if (stage == 0) vcur = load_v(v, c1, n1, H, h, of);
        });
        __syncthreads();  // the next chunk overwrites every LDS tile
      }
      state_out(S);
    }
  }
  __syncthreads();
  if (tid == 0 && sm.gate_bad) atomicOr(kState ? hdr->status_word : &g_kda_status, KDA_DEV_GATE_RANGE);
}

}  // namespace
