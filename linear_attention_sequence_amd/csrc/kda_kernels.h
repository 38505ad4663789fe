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
// kernel builds it and writes it to global memory; the main kernel copies it
// back instead of building it.  The per-channel state decay e^{G_c} travels in
// the row padding of KbT (see dvec), Tb's scale in that of Kt row 32.
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
    float T[CH][CH + 4];     // (I + A)^-1 (fp32)
    uint8_t o[4][CH][64];    // per wave: the bf16 O rows of its 32 columns (see chain_o)
  } u2;
  f16x8 R[3][4][64];         // right operands of off-diagonal sub-blocks (fp16), lane order
  // Qt of every other chunk (chunks alternate between Qt and Qt1, so that a
  // copied image can write its Qt while the chain still reads the previous
  // chunk's)
  bf16 Qt1[CH][DK + 8];
  unsigned short vt[4][32][CH + 8];  // per wave: V of the chunk chained next, transposed (its 32 columns)
  float etab[13][DK];        // per-channel decay factors of the chunk (see fill_tables)
  float tot[4][DK];          // per sub-block total decay (log2 domain)
  float beta[CH];
  float tbmax[8];            // per wave: largest |Tb| of the blocks it solved
  int unit;
  int gate_bad;
};


// e^{G_c} of channels c .. c + 3 (c a multiple of 4): the padding of KbT row c / 4
__device__ __forceinline__ float* dvec(Smem& sm, int c) {
  return reinterpret_cast<float*>(&sm.KbT[c >> 2][CH]);
}
// the Qt buffer of parity qb (0: Qt, 1: Qt1)
__device__ __forceinline__ bf16 (*qt_buf(Smem& sm, int qb))[DK + 8] { return qb ? sm.Qt1 : sm.Qt; }
// the power of two Tb was divided by: the padding of Kt row 32
__device__ __forceinline__ float* tbscale(Smem& sm) {
  return reinterpret_cast<float*>(&sm.Kt[32][DK]);
}

// byte offsets of the image parts
constexpr int OFF_QT = (int)offsetof(Smem, Qt);
constexpr int OFF_QT1 = (int)offsetof(Smem, Qt1);
constexpr int OFF_KT = (int)offsetof(Smem, Kt);
constexpr int OFF_KBT = (int)offsetof(Smem, KbT);
constexpr int OFF_TB = (int)offsetof(Smem, u);
constexpr int ROW_QK = (DK + 8) * 2;   // bytes per Qt / Kt row
constexpr int ROW_CC = (CH + 8) * 2;   // bytes per M / Tb row
static_assert(offsetof(Smem, M) == OFF_KBT + DK * ROW_CC, "KbT and M are contiguous");
static_assert(OFF_TB == (int)offsetof(Smem, M) + CH * ROW_CC, "Tb follows M");
static_assert(OFF_KT == OFF_QT + CH * ROW_QK, "Kt follows Qt");

// The image in global memory holds the tiles the chain reads, without the LDS
// row padding, in 16-byte pieces, in two groups: first what the chain's
// second part (O and the state update) reads, then what its first part (X and
// U) reads:
//   the Qt rows (16 pieces each), the KbT rows (8 each), rows 32..63 of M (8
//   each), the first 32 columns of rows 0..31 of M (4 each: the chain's first
//   row tile reads only those), D (channels 4 r .. 4 r + 3 in piece r,
//   r = 0..31);
//   the Kt rows (16 each), rows 32..63 of Tb, the first 32 columns of rows
//   0..31 of Tb, Tb's scale.
// The parts of each group fill rounds of NTHR pieces that lie in one group
// (the last round of each is partial), so that the copy into LDS moves whole
// rounds per group.
constexpr int IMG_ROW16 = CH * (DK / 8);           // Qt (or Kt) pieces
constexpr int IMG_KB = DK * (CH / 8);              // KbT pieces
constexpr int IMG_SHORT = 32 * 4;                  // rows 0..31 of M (or Tb), columns 0..31
constexpr int IMG_LONG = 32 * (CH / 8);            // rows 32..63 of M (or Tb)
constexpr int GP_QT = 0;                           // global piece indices of the parts
constexpr int GP_KB = GP_QT + IMG_ROW16;
constexpr int GP_MLONG = GP_KB + IMG_KB;
constexpr int GP_MSHORT = GP_MLONG + IMG_LONG;
constexpr int GP_D = GP_MSHORT + IMG_SHORT;
constexpr int GP_KT = GP_D + DK / 4;               // the second group
constexpr int GP_TLONG = GP_KT + IMG_ROW16;
constexpr int GP_TSHORT = GP_TLONG + IMG_LONG;
constexpr int GP_TBS = GP_TSHORT + IMG_SHORT;
constexpr int IMG_VEC = GP_TBS + 1;
constexpr int IMG_BYTES = 16 * IMG_VEC;            // one image in global memory
static_assert(ROW_QK == 17 * 16 && ROW_CC == 9 * 16, "rows are whole pieces plus one of padding");
constexpr int OFF_M = OFF_KBT + DK * ROW_CC;       // LDS rows of M, then Tb
// global piece of (row, 8-column piece cp) of M (t = 0) or Tb (t = 1); -1 for
// the pieces the chain never reads (rows 0..31, columns 32..63)
__device__ __forceinline__ int img_mt_piece(int t, int row, int cp) {
  if (row < 32) return cp < 4 ? (t ? GP_TSHORT : GP_MSHORT) + 4 * row + cp : -1;
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
  struct {
    float T[CH][CH + 4];
  } u2;
  // the sub-block totals are read (fill_tables) before R is written: two
  // workgroups per CU need the room
  union {
    f16x8 R[3][4][64];
    float tot[4][DK];
  };
  float etab[13][DK];
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
constexpr int MIN_SPLIT_CHUNKS = 2;   // a document of one chunk is never split
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

// wave-uniform copies of values every lane holds alike (read from LDS, or
// derived from such values where the compiler cannot see it), so that it
// keeps them, and what is derived from them (buffer descriptors among
// others), in scalar registers
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni64(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

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

// The raw inputs of a chunk, sixteen 16-byte pieces per lane (q: p[0..3],
// k: p[4..7], g: p[8..15]; element 8 s + j of q or k is channel 32 s + 8 cg + j,
// and g holds the same 32 channels as fp32 bits) with beta.
struct RawChunk {
  u32x4 p[16];
  float beta;
};
constexpr int RAW_Q = 0, RAW_K = 4, RAW_G = 8;

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
  // (every lane asks for the same chunk)
  const size_t row = (size_t)uni64(c0 * H + h);
  n = uni(n);
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
      rc.p[RAW_Q + i] = bload(src.q, of.qk + 64u * i);
      rc.p[RAW_K + i] = bload(src.k, of.qk + 64u * i);
    }
  } else if (part == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      rc.p[RAW_G + 2 * i] = bload(src.g, 2u * of.qk + 128u * i);
      rc.p[RAW_G + 2 * i + 1] = bload(src.g, 2u * of.qk + 128u * i + 16u);
    }
  } else {
#pragma unroll
    for (int i = 2; i < 4; ++i) {
      rc.p[RAW_G + 2 * i] = bload(src.g, 2u * of.qk + 128u * i);
      rc.p[RAW_G + 2 * i + 1] = bload(src.g, 2u * of.qk + 128u * i + 16u);
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

// ---- a precomputed image back into LDS, through registers.  Round i (0..15)
// of thread tid is piece img_round_base(i) + tid of the image, held in p[i];
// rounds 0..9 are the first group (Qt, KbT, M, D), rounds 10..15 the second
// (Kt, Tb, Tb's scale).  Phase 0, copied while the chain reads the previous
// image's Qt (in the other Qt buffer), KbT, M and D, is what the chain's
// first part reads and Qt: rounds 0..3 and 10..15; phase 1, copied once the
// chain is done with the previous image, is KbT, M and D: rounds 4..9.
constexpr int IMG_ROUNDS = 16;
constexpr int IMG_ROUNDS_P1 = 10;
__device__ __forceinline__ constexpr int img_round_base(int i) {
  return i < 4 ? GP_QT + NTHR * i : i < 8 ? GP_KB + NTHR * (i - 4) : i == 8 ? GP_MLONG : i == 9 ? GP_MSHORT
         : i < 14 ? GP_KT + NTHR * (i - 10) : i == 14 ? GP_TLONG : GP_TSHORT;
}
__device__ __forceinline__ constexpr int img_round_count(int i) {
  return i == 9 ? IMG_SHORT + DK / 4 : i == 15 ? IMG_SHORT + 1 : NTHR;
}
static_assert(IMG_ROW16 == 4 * NTHR && IMG_KB == 4 * NTHR && IMG_LONG == NTHR &&
                  img_round_base(9) + img_round_count(9) == GP_KT &&
                  img_round_base(15) + img_round_count(15) == IMG_VEC,
              "the rounds cover the image, each group in whole rounds");
__device__ __forceinline__ constexpr int image_round_phase(int i) { return i >= 4 && i < IMG_ROUNDS_P1 ? 1 : 0; }
// the rounds of phase kPhase (-1: all) into registers.  n_bytes is the
// image's size, or 0 to load zeros (a descriptor of size 0 reads nothing);
// lanes past a round's count read past the end, zeros as well.  Every load is
// unconditional, so that each round's registers are simply replaced.
template <int kPhase = -1>
__device__ __forceinline__ void load_image(RawChunk& im, const uint8_t* __restrict__ src, uint32_t n_bytes,
                                           int tid) {
  // (every lane asks for the same image)
  const Rsrc r = make_rsrc(reinterpret_cast<const uint8_t*>(uni64((int64_t)src)), (uint32_t)uni((int)n_bytes));
#pragma unroll
  for (int i = 0; i < IMG_ROUNDS; ++i)
    if (kPhase < 0 || image_round_phase(i) == kPhase)
      im.p[i] = __builtin_amdgcn_raw_buffer_load_b128(
          r, tid < img_round_count(i) ? 16 * (img_round_base(i) + tid) : IMG_BYTES, 0, 0);
}
// the rounds of phase kPhase (-1: all) from registers into the LDS image, Qt
// into the Qt buffer qb
template <int kPhase = -1>
__device__ __forceinline__ void image_to_lds(Smem& sm, const RawChunk& im, int tid, int qb) {
  uint8_t* dst = reinterpret_cast<uint8_t*>(&sm);
#pragma unroll
  for (int i = 0; i < IMG_ROUNDS; ++i) {
    if (kPhase >= 0 && image_round_phase(i) != kPhase) continue;
    int off;
    if (i < 4) {         // Qt rows
      const int q = NTHR * i + tid;
      off = (qb ? OFF_QT1 : OFF_QT) + (q >> 4) * ROW_QK + (q & 15) * 16;
    } else if (i < 8) {  // KbT rows
      const int q = NTHR * (i - 4) + tid;
      off = OFF_KBT + (q >> 3) * ROW_CC + (q & 7) * 16;
    } else if (i == 8 || i == 14) {  // rows 32..63 of M, of Tb
      off = (i == 8 ? OFF_M : OFF_TB) + (32 + (tid >> 3)) * ROW_CC + (tid & 7) * 16;
    } else if (i >= 10 && i < 14) {  // Kt rows
      const int q = NTHR * (i - 10) + tid;
      off = OFF_KT + (q >> 4) * ROW_QK + (q & 15) * 16;
    } else if (tid < IMG_SHORT) {  // columns 0..31 of rows 0..31 of M (round 9), of Tb (round 15)
      off = (i == 9 ? OFF_M : OFF_TB) + (tid >> 2) * ROW_CC + (tid & 3) * 16;
    } else if (i == 9) { // D: the padding of KbT row tid - IMG_SHORT
      off = OFF_KBT + (tid - IMG_SHORT) * ROW_CC + 2 * CH;
    } else {             // Tb's scale: the padding of Kt row 32
      off = OFF_KT + 32 * ROW_QK + 2 * DK;
    }
    if (tid < img_round_count(i)) *reinterpret_cast<u32x4*>(dst + off) = im.p[i];
  }
}

// Where prepare_chunk puts the image parts it holds in registers (Qt, Kt, Tb
// and D): the LDS image of the main kernel, or the global image.
struct LdsSink {
  Smem* sm;
  int qb;  // the Qt buffer
  __device__ __forceinline__ void qk(int tok, int col, const bf16x8& qt, const bf16x8& kt) const {
    *reinterpret_cast<bf16x8*>(&qt_buf(*sm, qb)[tok][col]) = qt;
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
    const uint32_t o = (uint32_t)(tok * 2 * DK + 2 * col);  // 16 * (16 tok + col / 8)
    bstore(__builtin_bit_cast(u32x4, qt), r, 16 * GP_QT + o);
    bstore(__builtin_bit_cast(u32x4, kt), r, 16 * GP_KT + o);
  }
  __device__ __forceinline__ void dv(int c, float f) const {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(f), r, 16 * (GP_D + (c >> 2)) + 4 * (c & 3), 0, 0);
  }
  __device__ __forceinline__ void tb(int row, int col, const f16x8& x) const {
    const int pc = img_mt_piece(1, row, col >> 3);
    if (pc >= 0) bstore(__builtin_bit_cast(u32x4, x), r, 16 * pc);
  }
  __device__ __forceinline__ void tbs(float f) const {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(f), r, 16 * GP_TBS, 0, 0);
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

// fp16 operands are stored as x 2^-e for a power of two 2^e chosen from the
// largest magnitude m of the values that share it: e = 0 when 2^-4 <= m < 2^14
// (then fp16 holds every value to its relative precision, or to an absolute
// 2^-25, far below m's rounding), and otherwise the e that brings m into
// [2^13, 2^14), in both directions: large values are scaled down so that they
// fit, small ones (v or beta near zero) up, out of the fp16 subnormal range.
// Multiplying by a power of two is exact, so the scaled and the unscaled
// products round the same wherever neither is subnormal.
__device__ __forceinline__ int f16_exponent(float m) {
  if (m >= 0.0625f && m < 16384.f) return 0;
  const int ex = (__float_as_int(m) >> 23) & 0xFF;
  if (ex == 0) return 0;                          // zero: nothing to scale
  return min(max(ex - (127 + 13), -100), 100);    // 2^+-e stays a normal float
}
__device__ __forceinline__ float pow2i(int e) { return __int_as_float((127 + e) << 23); }
// the exponent for the wave's largest lane value m: the common case (some
// lane at or above 2^-4, none at or above 2^14) costs two compares and two
// ballots; otherwise the wave's maximum picks it
__device__ __forceinline__ int wave_f16_exponent(float m) {
  if (__builtin_amdgcn_ballot_w64(m >= 16384.f) == 0 && __builtin_amdgcn_ballot_w64(m >= 0.0625f) != 0)
    return 0;
  return f16_exponent(wave_max(m));
}

// Per-channel decay factors of a chunk from the sub-block totals t_w (log2
// domain, so every factor is a bare exp2):
//   rows 0..3:  e^{G_end(w)}          = 2^{t_0 + .. + t_w}      (row 3 = e^{G_c} = D)
//   rows 4..6:  e^{G_c - G_end(w)}    = 2^{t_{w+1} + .. + t_3}, w = 0..2
//   rows 7..12: e^{G_end(w) - G_end(b)} = 2^{t_{b+1} + .. + t_w}, pair (w, b), b < w,
//               at row 7 + w (w - 1) / 2 + b
// Thread tid < DK writes row 3 of channel tid (D, which the caller hands on
// to the image).
template <class Sm>
__device__ __forceinline__ void fill_tables(Sm& sm, int tid) {
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
      const f16x8 rv = sm.R[b][s][l];
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

__device__ __forceinline__ Lane make_lane(int tid = threadIdx.x) {
  Lane ln;
  ln.tid = tid;
  ln.w = __builtin_amdgcn_readfirstlane(ln.tid >> 6);
  ln.l = ln.tid & 63;
  ln.r = ln.l & 15;
  ln.cg = ln.l >> 4;
  ln.m = ln.l & 31;
  ln.hg = ln.l >> 5;
  ln.tok = 16 * ln.w + ln.r;
  return ln;
}

// Tb = T Diag(beta) 2^-e in fp16 (in LDS it overwrites A), e chosen so that
// |Tb 2^-e| < 2^14 (e = 0 unless Tb is huge): thread tid (0 .. 255) converts
// row tid / 4, columns 16 (tid % 4) + 8 half .. + 7 for half in [H0, H1).
// Reads T, beta and the blocks' largest |Tb| (complete at B5).
template <int H0, int H1, class Sm, class Sink>
__device__ __forceinline__ void convert_tb(Sm& sm, const Sink& sink, int tid) {
  const int e = f16_exponent(fmaxf(fmaxf(sm.tbmax[0], sm.tbmax[1]), fmaxf(sm.tbmax[2], sm.tbmax[3])));
  const float down = pow2i(-e);
  if (H0 == 0 && tid == 0) sink.tbs(pow2i(e));
  const int rr = tid >> 2;
#pragma unroll
  for (int half = H0; half < H1; ++half) {
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

// Everything of a chunk that does not depend on the state: from the raw
// inputs `cur` (n valid tokens) to the image in LDS (Qt, Kt, KbT, M, Tb, D).
// hook(0..2) run at fixed points once `cur` has been consumed (they may
// refill it); the scheduling barriers keep the loads they issue spread out.
// hook(6) runs between B1 and B2, after this role's stores there; hook(3)
// runs right after the fourth workgroup barrier (B3), hook(4) just before
// B5, hook(5) between B5 and B6.
// Six workgroup barriers, B0 .. B3, B5 and B6 (there is no B4), the last of
// which ends the function; after it the image is complete (with kTbShared,
// once the other role has converted the second column half of Tb between B5
// and B6, convert_tb<1, 2>).  Until B1 the function writes to LDS only tot,
// beta, gate_bad and the decay tables, and computes the diagonal blocks of A
// and M in registers (so that another workgroup role may still read the
// previous image until then); until B2 not Qt, Kt or KbT; until B5 not Tb or
// its scale.
template <bool kTbShared = false, class Sm, class Sink, class Hook>
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
      const u32x4 qi = cur.p[RAW_Q + i], ki = cur.p[RAW_K + i];
      const uint32_t qa[4] = {qi[0], qi[1], qi[2], qi[3]};
      const uint32_t ka[4] = {ki[0], ki[1], ki[2], ki[3]};
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
      const u32x4 gi = cur.p[RAW_G + i];
      const float ga[4] = {__uint_as_float(gi[0]), __uint_as_float(gi[1]), __uint_as_float(gi[2]),
                           __uint_as_float(gi[3])};
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
  __syncthreads();  // B0
  // the decay tables (its own LDS space) meanwhile; D, which belongs to the
  // image, is handed on after B1
  fill_tables(sm, tid);
  __builtin_amdgcn_sched_barrier(0);
  hook(1);
  __builtin_amdgcn_sched_barrier(0);
  // diagonal block (w, w) of M and A on fp32 MFMA (the factors
  // e^{+-(G - G_end(w))} inside a sub-block need fp32's range): k-step s
  // takes element s from every lane (the same channel on both operands).
  // The products stay in registers until B1, so that they run while another
  // workgroup role still reads the previous image.
  f32x4 accM[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  f32x4 accA[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    accM[s & 1] = mfma16f(lq[s], kr[s], accM[s & 1]);
    accA[s & 1] = mfma16f(lk[s], kr[s], accA[s & 1]);
  }
  __syncthreads();  // B1: the previous image's Qt, M, KbT and D may still be read until here

  {
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
        sm.R[w][s][l] = rv;
      }
    }
    if (tid < DK) sink.dv(tid, sm.etab[3][tid]);  // written by this thread before B1
  }
  __builtin_amdgcn_sched_barrier(0);
  hook(6);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();  // B2: decay tables, R and the diagonal A / M blocks visible

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
  // blocks of I + A (complete since B2): T = (I + A)^-1 by 16x16 blocks, by
  // forward substitution, lane l owning column l % 16 of diagonal block
  // l / 16.  tmax tracks the largest |Tb| = |T_ij beta_j| a wave produces.
  const int da = l >> 4, dj = l & 15;
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
      sm.u2.T[16 * da + rr][16 * da + dj] = x[rr];
      tmax = fmaxf(tmax, fabsf(x[rr]) * bj);
    }
    if (da == 0 || da == 2) {  // upper blocks (0, 1) and (2, 3): read by U = Tb X
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sm.u2.T[16 * da + rr][16 * (da + 1) + dj] = 0.f;
    }
  }

  __syncthreads();  // B3: A and M complete, R dead, diagonal blocks of T visible
  __builtin_amdgcn_sched_barrier(0);
  hook(3);
  __builtin_amdgcn_sched_barrier(0);
  // off-diagonal blocks: wave b walks column block b downwards,
  // T_ab = -T_aa sum_{k=b}^{a-1} A_ak T_kb, on fp32 MFMA
  if (w == 0) tmax = levels_column<0>(sm, l, tmax);
  else if (w == 1) tmax = levels_column<1>(sm, l, tmax);
  else if (w == 2) tmax = levels_column<2>(sm, l, tmax);
  tmax = wave_max(tmax);
  if (l == 0) sm.tbmax[w] = tmax;
  __builtin_amdgcn_sched_barrier(0);
  hook(4);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();  // B5: T complete
  // Tb: both column halves here, or only the first when the caller's other
  // role (the main kernel's consumer waves, idle until B6) converts the second
  if constexpr (kTbShared) convert_tb<0, 1>(sm, sink, tid);
  else convert_tb<0, 2>(sm, sink, tid);
  __builtin_amdgcn_sched_barrier(0);
  hook(5);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();  // B6: the image is complete, T dead (its space stages O)
}

// The state-dependent part of a chunk of n tokens starting at token c0, from
// the image in LDS and this chunk's V (wave w owns value columns 32 w ..):
//   X = V - Kt S,  U = Tb X,  O = scale (Qt S + M U),  S <- D S + KbT U,
// in three parts.  chain_a computes X and U: it reads V (staged by stage_v),
// Kt, Tb and Tb's scale; chain_o computes O and stages it in LDS (write_o
// stores it, on the other role, after the next workgroup barrier): it reads
// Qt and M; chain_b updates S: it reads only KbT and D.  ChainMid carries U (fp16, 2^-eu) from chain_a to the others.
// Scheduling fences in chain_a (after the V staging, after X and after U)
// keep its stages in order.
struct ChainMid {
  f16x8 Uh[4];
  int eu;
};

// V of the chunk chained next (rows past its end were read as zero),
// transposed into the wave's part of vt, where chain_a reads it
__device__ __forceinline__ void stage_v(Smem& sm, const VChunk& vn, const Lane& ln) {
  const int l = ln.l;
  unsigned short (*vt)[CH + 8] = sm.vt[ln.w];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 16 * i + (l >> 2);
    const u32x4 u = vn.r[i];
    const uint32_t uu[4] = {u[0], u[1], u[2], u[3]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // column c keeps token t at t ^ 8 (c / 8): columns 8 apart (whose rows
      // share banks) write different banks; 8-token groups stay contiguous
      vt[8 * (l & 3) + 2 * j][t ^ (8 * (l & 3))] = (unsigned short)(uu[j] & 0xFFFFu);
      vt[8 * (l & 3) + 2 * j + 1][t ^ (8 * (l & 3))] = (unsigned short)(uu[j] >> 16);
    }
  }
}

__device__ __forceinline__ void chain_a(Smem& sm, const f32x16 (&S)[4], int n, int64_t c0, int H, int h,
                                        bf16* __restrict__ out, const Lane& ln, const Offsets& of,
                                        ChainMid& mid) {
  const int w = ln.w, l = ln.l, m = ln.m, hg = ln.hg;
  const float scale = 0.08838834764831845f;  // 128^-1/2

  // this chunk's V, staged transposed by stage_v
  const unsigned short (*vt)[CH + 8] = sm.vt[w];
  const int rowsel = swap23(m);
  // V in the C layout of the X tiles (packed bf16; added after the product)
  u32x4 vx[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      vx[mt][hh] = *reinterpret_cast<const u32x4*>(&vt[m][(32 * mt + 16 * hh + 8 * hg) ^ (8 * (m >> 3))]);
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
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < 4; ++s) mid.Uh[s] = Uh[s];
  mid.eu = eu;
}

// O = scale (Qt S + M U) of the chunk, from S and the U that chain_a left in
// mid, computed transposed: O^T = S^T Qt^T + U^T M^T, with the fragments of S
// and U as left operands (in their C layout a lane holds one value column
// and eight consecutive key channels or tokens per k-step, which is the left
// operand layout of S^T and U^T) and rows of Qt and M as right operands.  In
// the C layout of O^T lane (n, hg) then holds token 32 mt + n and value
// columns 8 q + 4 hg + 0..3 (q = 0..3): four 8-byte pieces of that token's
// row.  They go through the wave's slice of u2 (one 64-byte row per token,
// 16-byte piece q at q ^ (row / 4 % 4), so that neither the 8-byte writes nor
// the 16-byte reads of 16 lanes share a bank) and leave as 16-byte row
// pieces, four lanes to a row.  Reads Qt and M.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void chain_o(Smem& sm, const f32x16 (&S)[4], const ChainMid& mid,
                                        const Lane& ln, int qb) {
  const int w = ln.w, m = ln.m, hg = ln.hg;
  const bf16 (*Qt)[DK + 8] = qt_buf(sm, qb);
  const float scale = 0.08838834764831845f;  // 128^-1/2
  constexpr int PMT[6] = {0, 0, 1, 1, 1, 1};
  constexpr int PS[6] = {0, 1, 0, 1, 2, 3};
  const int eu = mid.eu;
  const float udown = pow2i(-eu);
  f16x8 Uh[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) Uh[s] = mid.Uh[s];
  bf16x8 Sb[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) Sb[s][j] = (bf16)S[s >> 1][8 * (s & 1) + j];
  if (eu > 0) {
    // M U is computed as M (U 2^-eu) with U scaled down: bring Qt S to the
    // same scale (S 2^-eu cannot overflow)
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) Sb[s][j] = (bf16)(S[s >> 1][8 * (s & 1) + j] * udown);
  }

  // one accumulator per token tile mt (tokens 32 mt .. 32 mt + 31)
  float oscale = scale * pow2i(eu);
  f32x16 O[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[mt][i] = 0.f;
  if (eu < 0) {
    // U was scaled up (small values): S 2^-eu could overflow, so (U 2^-eu)^T
    // M^T is taken first and brought back to scale (exactly) before S^T Qt^T
    // joins it in the same accumulator
#pragma unroll
    for (int p = 0; p < 6; ++p) {
      const f16x8 mv = *reinterpret_cast<const f16x8*>(&sm.M[32 * PMT[p] + m][16 * PS[p] + 8 * hg]);
      O[PMT[p]] = mfma32h(Uh[PS[p]], mv, O[PMT[p]]);
    }
    const float up = pow2i(eu);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[mt][i] *= up;
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 qv = *reinterpret_cast<const bf16x8*>(&Qt[32 * mt + m][16 * s + 8 * hg]);
        O[mt] = mfma32(Sb[s], qv, O[mt]);
      }
    oscale = scale;
  } else {
    bf16x8 qa[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        qa[mt][s] = *reinterpret_cast<const bf16x8*>(&Qt[32 * mt + m][16 * s + 8 * hg]);
    // M operands loaded two pairs ahead
    f16x8 mh[2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
      mh[p] = *reinterpret_cast<const f16x8*>(&sm.M[32 * PMT[p] + m][16 * PS[p] + 8 * hg]);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        O[mt] = mfma32(Sb[s], qa[mt][s & 1], O[mt]);
        if (s + 2 < 8)
          qa[mt][s & 1] = *reinterpret_cast<const bf16x8*>(&Qt[32 * mt + m][16 * (s + 2) + 8 * hg]);
      }
      if (s < 6) {
        const int p = s;
        O[PMT[p]] = mfma32h(Uh[PS[p]], mh[p & 1], O[PMT[p]]);
        if (p + 2 < 6)
          mh[p & 1] = *reinterpret_cast<const f16x8*>(&sm.M[32 * PMT[p + 2] + m][16 * PS[p + 2] + 8 * hg]);
      }
    }
  }
  // token 32 mt + m, value columns 8 q + 4 hg + 0..3 of the wave's 32 from
  // O[mt][4 q ..], into the slice
  uint8_t* ost = &sm.u2.o[w][0][0];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int row = 32 * mt + m;
    uint8_t* dst = ost + 64 * row + 8 * hg;
    const int sw = (row >> 2) & 3;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x2 pk;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const bf16 lo = (bf16)(O[mt][4 * q + 2 * e] * oscale);
        const bf16 hi = (bf16)(O[mt][4 * q + 2 * e + 1] * oscale);
        pk[e] = (uint32_t)__builtin_bit_cast(unsigned short, lo) |
                ((uint32_t)__builtin_bit_cast(unsigned short, hi) << 16);
      }
      *reinterpret_cast<u32x2*>(dst + 16 * (q ^ sw)) = pk;
    }
  }
}

// The O rows that chain_o staged (wave w's slice, 32 columns) out to memory,
// for the chunk of n tokens at token c0: lane l writes 16 bytes of row
// 16 it + l / 4 (rows past the end are dropped by the descriptor's range).
// Run by the producer wave of the same index, once a workgroup barrier has
// followed chain_o.
__device__ __forceinline__ void write_o(const Smem& sm, int n, int64_t c0, int H, int h, bf16* __restrict__ out,
                                        const Lane& ln, const Offsets& of) {
  const uint8_t* ost = &sm.u2.o[ln.w][0][0];
  const int l = ln.l;
  const Rsrc ro = make_rsrc(out + ((size_t)c0 * H + h) * DV, chunk_bytes(n, H, 256u));
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int t = 16 * it + (l >> 2);
    bstore(*reinterpret_cast<const u32x4*>(ost + 64 * t + 16 * ((l & 3) ^ ((t >> 2) & 3))), ro, of.v[it]);
  }
}

// S <- e^{G_c} S + (kh e^{G_c - G})^T U: the product accumulates from zero
// (the four row tiles interleaved) and S takes it with one fma per element,
// so S itself is only ever touched by vector ALU code
__device__ __forceinline__ void chain_b(Smem& sm, f32x16 (&S)[4], const ChainMid& mid, const Lane& ln) {
  const int hg = ln.hg;
  const int rowsel = swap23(ln.m);
  const int eu = mid.eu;
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
        dS[kt] = mfma32h(kb[s & 1][kt], mid.Uh[s], dS[kt]);
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
// main kernel: producer / consumer.  One workgroup of 8 waves per CU.  Waves
// 0-3 (the producer) build the image of chunk i (prepare_chunk, or a copy of
// a split chunk's image from the workspace) while waves 4-7 (the consumer)
// chain chunk i - 1 on the image in LDS: two waves per SIMD, one of each role.
//
// The image is single-buffered (all but Qt, which alternates between two
// buffers); workgroup barriers order the consumer's reads
// of image i - 1 before the producer's writes of image i.  An iteration in
// which the producer builds an image from raw inputs has the six barriers of
// prepare_chunk, B0 .. B3, B5, B6:
//   before B0:  producer: prologue (registers, its own tot / beta);
//               consumer: chain_a, X and U (reads Kt, Tb and Tb's scale;
//               stages V in its slice);
//   B0 .. B1:   producer: decay tables (its own LDS space), the diagonal
//               blocks of A and M (registers);
//               consumer: chain_o and chain_b, O and the state update (reads
//               Qt, M, KbT and D);
//   B1 .. B6:   producer: the rest of the image;
//               consumer: loads and stages the V of the chunk it chains
//               next, then waits.
// An iteration that copies a precomputed image (or prepares nothing) has two:
//   B0 .. B1:   producer: Kt, Tb and Tb's scale of image i, and its Qt (into
//               the Qt buffer of parity i; the chain reads image i - 1's in
//               the other);
//   after B1:   producer: KbT, M and D of image i;
//               consumer: chain_a of image i (the next iteration), which reads
//               only what was written before B1.
// The producer hands each chunk to the consumer through an item descriptor in
// LDS (two slots, by iteration parity), published before the iteration that
// prepares it; the consumer reads it after that iteration's B0 and from it
// knows the iteration's barrier count.
// ---------------------------------------------------------------------------
constexpr int NPC = 2 * NTHR;  // threads of the producer / consumer kernel

enum ItemFlags { ITEM_VALID = 1, ITEM_FIRST = 2, ITEM_LAST = 4, ITEM_SPLIT = 8 };

struct Item {
  int64_t c0;     // first token of the chunk
  int64_t first;  // first token of the unit's document
  int n;          // tokens in the chunk (0 for an empty document)
  int h;          // head
  int unit;       // work-list entry: list index * H + h
  int flags;      // ItemFlags (ITEM_SPLIT: the image is precomputed)
};

// a unit as the producer walks it (uniform values)
struct PUnit {
  int u;          // work-list entry (>= n_units: none)
  int h;
  int64_t bos;    // first token
  int len;        // tokens
  int nch;        // chunks (at least 1: an empty document is one item of 0 tokens)
  int img0;       // split document: index of its first chunk image; -1: fused
};

struct alignas(16) PCSmem {
  Smem s;
  Item items[2];
  int fetch;      // a unit index fetched from the counter
  int nu[5];      // the next unit: index, doc.x, doc.y, split.x, split.y
};

__device__ __forceinline__ PUnit make_punit(int u, int n_units, int H, int dx, int dy, int sx, int sy) {
  PUnit p;
  p.u = u;
  p.h = 0;
  p.bos = 0;
  p.len = 0;
  p.nch = 0;
  p.img0 = -1;
  if (u < n_units) {
    p.h = u % H;
    p.len = dy;
    if (dx < 0) {
      p.bos = sx;
      p.img0 = sy;
    } else {
      p.bos = dx;
    }
    p.nch = max(1, (dy + CH - 1) / CH);
  }
  return p;
}

__device__ __forceinline__ Item read_item(const Item& src) {
  Item it;
  it.c0 = uni64(src.c0);
  it.first = uni64(src.first);
  it.n = uni(src.n);
  it.h = uni(src.h);
  it.unit = uni(src.unit);
  it.flags = uni(src.flags);
  return it;
}

__device__ __forceinline__ Item make_item(const PUnit& p, int c) {
  Item it;
  it.first = p.bos;
  it.c0 = p.bos + (int64_t)CH * c;
  it.n = (int)min<int64_t>(CH, (int64_t)p.len - (int64_t)CH * c);
  if (it.n < 0) it.n = 0;
  it.h = p.h;
  it.unit = p.u;
  it.flags = ITEM_VALID | (c == 0 ? ITEM_FIRST : 0) | (c == p.nch - 1 ? ITEM_LAST : 0) |
             (p.img0 >= 0 ? ITEM_SPLIT : 0);
  return it;
}

template <bool kState>
__global__ __launch_bounds__(NPC, 1) void kda_pc_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, bf16* __restrict__ out,
    WorkHeader* __restrict__ hdr, const int2* __restrict__ docs, const int2* __restrict__ split,
    const uint8_t* __restrict__ images, int64_t T, int H, float gate_bound) {
  __shared__ PCSmem ps;
  Smem& sm = ps.s;
  const Lane ln = make_lane(threadIdx.x & (NTHR - 1));
  const int tid = ln.tid, w = ln.w, l = ln.l;

  if (hdr->status != 0) {
    // cu_seqlens was rejected on the device: make the failure visible
    const size_t total = (size_t)T * H * DV;
    const size_t stride = (size_t)gridDim.x * NPC;
    unsigned short* o16 = reinterpret_cast<unsigned short*>(out);
    for (size_t i = (size_t)blockIdx.x * NPC + threadIdx.x; i < total; i += stride) o16[i] = 0x7FC0;
    if (kState && hdr->ht != nullptr) {
      float* ht = hdr->ht;
      const size_t nst = (size_t)hdr->n_state_docs * H * DK * DV;
      for (size_t i = (size_t)blockIdx.x * NPC + threadIdx.x; i < nst; i += stride) ht[i] = __builtin_nanf("");
    }
    return;
  }
  const int n_units = hdr->n_units;
  const Offsets of = make_offsets(H, ln.tok, ln.cg, w, l);

  // the first unit
  if (threadIdx.x == 0) {
    sm.gate_bad = 0;
    ps.fetch = atomicAdd(&hdr->counter, 1);
  }
  __syncthreads();

  if (threadIdx.x < NTHR) {
    // ======================== producer (waves 0-3) ========================
    // a unit's description from the work list (uniform scalar loads)
    auto unit_of = [&](int u) -> PUnit {
      int dx = 0, dy = 0, sx = 0, sy = 0;
      if (u < n_units) {
        const int2 d = docs[u / H];
        dx = d.x;
        dy = d.y;
        if (dx < 0) {
          const int2 sp = split[-dx - 1];
          sx = sp.x;
          sy = sp.y;
        }
      }
      return make_punit(u, n_units, H, dx, dy, sx, sy);
    };
    auto raw_of = [&](const PUnit& p, int c) {
      const int64_t c0 = p.bos + (int64_t)CH * c;
      return raw_src(q, k, g, beta, c0, (int)min<int64_t>(CH, (int64_t)p.len - (int64_t)CH * c), H, p.h);
    };
    auto image_of = [&](const PUnit& p, int c) {
      return images + ((size_t)(p.img0 + c) * H + p.h) * IMG_BYTES;
    };
    // the inputs of item (p, c): raw q, k, g, beta (fused unit) or the
    // precomputed image (split unit); zeros when there is no item, so that
    // buf is redefined on every path
    auto load_inputs = [&](RawChunk& b, const PUnit& p, int c, const Offsets& o, int t) {
      if (p.u < n_units && p.img0 >= 0) {
        load_image(b, image_of(p, c), IMG_BYTES, t);
      } else if (p.u < n_units) {
        load_raw(b, raw_of(p, c), o);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) b.p[i] = u32x4{0u, 0u, 0u, 0u};
        b.beta = 0.f;
      }
    };
    PUnit pu = unit_of(uni(ps.fetch));  // the unit of the current item
    int pc = 0;                         // the chunk of the current item in pu
    RawChunk buf;                       // inputs of the current item
    if (tid == 0) {
      Item none{};
      ps.items[0] = pu.u < n_units ? make_item(pu, 0) : none;
      ps.items[1] = none;
    }
    load_inputs(buf, pu, 0, of, tid);
    __syncthreads();  // item 0 published

    bool cv = false;  // the consumer chains an item in this iteration
    for (int iter = 0;; ++iter) {
      // this iteration prepares chunk pc of pu; the consumer chains the
      // previous item
      const bool pv = pu.u < n_units;
      if (!pv && !cv) break;
      const int pn = pv ? (int)max<int64_t>(0, min<int64_t>(CH, (int64_t)pu.len - (int64_t)CH * pc)) : 0;
      // the lane coordinates again, from a value the compiler cannot see
      // through: what it derives from them (LDS addresses and the like) is
      // computed inside the iteration instead of being hoisted out of the
      // loop, where it would hold registers for the whole kernel
      int t = tid;
      asm volatile("" : "+v"(t));
      const Lane lnI = make_lane(t);
      const Offsets ofI = make_offsets(H, lnI.tok, lnI.cg, lnI.w, lnI.l);
      // between B0 and B1 of a unit's last chunk: wave 3 fetches the next
      // unit from the counter
      auto fetch_next = [&]() {
        if (lnI.w == 3 && lnI.l == 0) {
          const int u = atomicAdd(&hdr->counter, 1);
          int dx = 0, dy = 0, sx = 0, sy = 0;
          if (u < n_units) {
            const int2 d = docs[u / H];
            dx = d.x;
            dy = d.y;
            if (dx < 0) {
              const int2 sp = split[-dx - 1];
              sx = sp.x;
              sy = sp.y;
            }
          }
          ps.nu[0] = u;
          ps.nu[1] = dx;
          ps.nu[2] = dy;
          ps.nu[3] = sx;
          ps.nu[4] = sy;
        }
      };
      // after B1: the unit fetched between B0 and B1
      auto fetched = [&]() {
        return make_punit(uni(ps.nu[0]), n_units, H, uni(ps.nu[1]), uni(ps.nu[2]), uni(ps.nu[3]), uni(ps.nu[4]));
      };
      // hand item (p, c) to the consumer, which reads it after the next B0 of
      // iteration it + 1 (the slot it replaces was read before the B0 of
      // iteration it)
      auto publish = [&](int it, const PUnit& p, int c) {
        if (lnI.tid == 0) {
          Item none{};
          ps.items[(it + 1) & 1] = p.u < n_units ? make_item(p, c) : none;
        }
      };
      // O of the item the consumer chains in this iteration, which its
      // chain_o staged in LDS before B1: out to memory after B1, before
      // publish() reuses that item's slot
      auto store_o = [&]() {
        const Item it = read_item(ps.items[(iter + 1) & 1]);
        if ((it.flags & ITEM_VALID) && it.n > 0) write_o(sm, it.n, it.c0, H, it.h, out, lnI, ofI);
      };
      PUnit nu = pu;  // the next item: (nu, nc)
      int nc = pc + 1;
      if (pv && pn > 0 && pu.img0 < 0) {
        // fused unit: build the image (six barriers; the consumer, told by
        // the item, passes B2, B3, B5 and B6 with it).  The next chunk's inputs go
        // into buf as soon as it is free: the same unit's after B1, a new
        // unit's (zeros if none) once it is known, after B3, so that buf is
        // redefined on every path and nothing keeps it alive across the
        // prologue.
        const bool last = pc + 1 >= pu.nch;
        prepare_chunk<true>(sm, LdsSink{&sm, iter & 1}, buf, pn, gate_bound, lnI, [&](int part) {
          // the next chunk of the same unit arrives in three parts (q and k
          // after B0, g's two halves and beta after the tiles and after B3),
          // so that its loads do not all share the window in which V is
          // loaded and O stored (between B1 and B2, part 6)
          if (part == 1) {
            if (last) fetch_next();
            else load_raw_part(buf, raw_of(pu, pc + 1), ofI, 0);
          } else if (part == 2) {
            if (!last) load_raw_part(buf, raw_of(pu, pc + 1), ofI, 1);
          } else if (part == 3) {
            if (last) {
              nu = fetched();
              nc = 0;
              load_inputs(buf, nu, 0, ofI, lnI.tid);
            } else {
              load_raw_part(buf, raw_of(pu, pc + 1), ofI, 2);
            }
          } else if (part == 5) {
            publish(iter, nu, nc);
          } else if (part == 6) {
            store_o();
          }
        });
      } else if (pv && pn > 0) {
        // split unit: all its remaining chunks here, an iteration each with
        // two barriers (the consumer starts on an image right after its B1).
        // A chunk's image goes from registers into LDS, what the chain's
        // first part reads after B0 and the rest after B1 (the next B0 orders
        // it before the chain's second part), each phase's registers then
        // taking the next chunk's.  The image registers are this loop's own,
        // so that nothing is copied between iterations.
        RawChunk im = buf;
        for (;; ++iter, ++pc) {
          // wave-uniform, so that the last chunk's extra work is a scalar
          // branch: a lane-mask branch would merge its loads' registers
          // with this path and make every chunk wait for its own prefetch
          const bool last = uni(pc + 1 >= pu.nch ? 1 : 0) != 0;
          const uint8_t* nimg = image_of(pu, pc + 1);
          const uint32_t nbytes = last ? 0u : IMG_BYTES;  // the next chunk, or zeros
          // this chunk's V (the consumer's columns of wave w), in flight
          // while this role waits at B0; staged after it, where the
          // consumer's chain_a no longer reads the previous chunk's
          const int64_t vc0 = pu.bos + (int64_t)CH * pc;
          const VChunk vn = load_v(v, vc0, (int)min<int64_t>(CH, (int64_t)pu.len - (int64_t)CH * pc), H, pu.h, ofI);
          __syncthreads();  // B0: the consumer has read Kt, Tb and Tb's scale of the previous image, and V
          image_to_lds<0>(sm, im, lnI.tid, iter & 1);
          load_image<0>(im, nimg, nbytes, lnI.tid);
          if (last) fetch_next();
          stage_v(sm, vn, lnI);
          __syncthreads();  // B1: ... and M, KbT and D (its Qt is in the other buffer)
          store_o();
          image_to_lds<1>(sm, im, lnI.tid, iter & 1);
          load_image<1>(im, nimg, nbytes, lnI.tid);
          if (last) {
            nu = fetched();
            nc = 0;
            load_inputs(buf, nu, 0, ofI, lnI.tid);
            publish(iter, nu, nc);
            break;
          }
          publish(iter, pu, pc + 1);
        }
      } else {
        // nothing to prepare (no item, or an empty document): two barriers
        const bool last = pv;  // an empty document is its unit's only chunk
        __syncthreads();  // B0
        if (last) fetch_next();
        __syncthreads();  // B1
        store_o();
        if (last) {
          nu = fetched();
          nc = 0;
        } else {
          nu.u = n_units;
        }
        load_inputs(buf, nu, nc, ofI, lnI.tid);
        publish(iter, nu, nc);
      }
      pu = nu;
      pc = nc;
      cv = pv;
    }
  } else {
    // ======================== consumer (waves 4-7) ========================
    // The chain holds up the producer at B0 and B1 and is idle after them:
    // its waves take precedence over the producer's in instruction issue
    // (otherwise the older producer waves win it, and the chain's MFMAs wait
    // behind the producer's long runs of them).
    __builtin_amdgcn_s_setprio(2);
    f32x16 S[4];  // the state
    auto state_in = [&](const Item& it) {
      const float* h0 = kState ? hdr->h0 : nullptr;
      if (h0 != nullptr) {
        load_state(S, h0 + ((size_t)hdr->doc_ids[it.unit / H] * H + it.h) * (DK * DV), ln);
      } else {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) S[kt][i] = 0.f;
      }
    };
    auto save_chunk = [&](const Item& it) {
      if constexpr (kState) {
        float* cs = hdr->chunk_states;
        if (cs != nullptr) {
          const int64_t slot = it.first / CH + hdr->doc_ids[it.unit / H] + (it.c0 - it.first) / CH;
          store_state(S, cs + ((size_t)slot * H + it.h) * (DK * DV), ln);
        }
      }
    };
    auto state_out = [&](const Item& it) {
      if constexpr (kState) {
        float* ht = hdr->ht;
        if (ht != nullptr) store_state(S, ht + ((size_t)hdr->doc_ids[it.unit / H] * H + it.h) * (DK * DV), ln);
      }
    };
    __syncthreads();  // item 0 published
    const bool any = (uni(ps.items[0].flags) & ITEM_VALID) != 0;
    for (int iter = 0;; ++iter) {
      // this iteration chains `ci`, the item the producer prepared in the
      // previous one; once the producer has none, the next iteration has
      // none to prepare either and both roles stop
      const Item ci = read_item(ps.items[(iter + 1) & 1]);
      const bool cv = (ci.flags & ITEM_VALID) != 0;
      if (!cv && (iter > 0 || !any)) break;
      const bool active = cv && ci.n > 0;
      ChainMid mid;
      if (cv && (ci.flags & ITEM_FIRST)) state_in(ci);
      if (active) {
        save_chunk(ci);
        chain_a(sm, S, ci.n, ci.c0, H, ci.h, out, ln, of, mid);
      }
      __syncthreads();  // B0
      // the item the producer prepares in this iteration (published before
      // its B0): its V, one load site for every path, so that the wait for
      // it, in the next iteration, counts only what was issued after it
      const Item pi = read_item(ps.items[iter & 1]);
      const bool pv = (pi.flags & ITEM_VALID) != 0;
      // the producer builds this item's image from raw inputs until B6; the
      // V of a precomputed (split) item it stages itself before B1, and an
      // empty item needs none
      const bool pfused = pv && pi.n > 0 && !(pi.flags & ITEM_SPLIT);
      if (active) {
        chain_o(sm, S, mid, ln, (iter + 1) & 1);
        chain_b(sm, S, mid, ln);
      }
      if (cv && (ci.flags & ITEM_LAST)) state_out(ci);
      __syncthreads();  // B1
      if (pfused) {
        // V of a fused item is loaded and staged while the producer builds
        // the image (this role has nothing else to do until B5), away from
        // the window between B0 and B1 in which the O stores and the
        // producer's loads go out
        const VChunk vcur = load_v(v, pi.c0, pi.n, H, pi.h, of);
        stage_v(sm, vcur, ln);
        __syncthreads();  // B2
        __syncthreads();  // B3
        __syncthreads();  // B5
        convert_tb<1, 2>(sm, LdsSink{&sm, 0}, ln.tid);  // the second column half of Tb
        __syncthreads();  // B6
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && sm.gate_bad) atomicOr(kState ? hdr->status_word : &g_kda_status, KDA_DEV_GATE_RANGE);
}

}  // namespace
