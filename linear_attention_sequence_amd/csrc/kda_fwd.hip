// kda_fwd.hip -- chunked forward of Kimi Delta Attention for MI355X (gfx950).
//
// What is computed: see include/kda.h (page "nemo_automodel.components.models.
// kimi_k3.kda_fused", package docstring).  This file holds the device code and
// the C-ABI launcher.
//
// Chunk form used by the kernels (an exact restatement of the token recurrence).
// For one chunk of c <= 64 tokens r, i with state S at its start, per key
// channel G_r = g_1 + ... + g_r (cumulative log decay inside the chunk):
//
//   A_ri = beta_r sum_c kh_rc kh_ic exp(G_rc - G_ic)   (i < r, strictly lower)
//   M_ri =        sum_c qh_rc kh_ic exp(G_rc - G_ic)   (i <= r)
//   Tb   = (I + A)^-1 Diag(beta)                       (the WY / UT factor)
//   X    = V - (kh * e^G) S
//   U    = Tb X
//   O    = scale ((qh * e^G) S + M U)
//   S   <- Diag(e^{G_c}) S + (kh * e^{G_c - G})^T U
//
// Only the last four lines depend on S; they form the sequential chain of a
// (document, head) unit.  Everything above them depends only on the chunk's
// own q, k, g, beta.
//
// Work decomposition: one workgroup of 4 waves owns a (document, head) unit at
// a time and walks its chunks in order.  A persistent grid pulls units from a
// counter; a one-workgroup scheduler kernel orders units longest-document
// first so the long sequential chains start early.
//
// Matrix products run on bf16 MFMA with fp32 accumulation.  Products whose
// rounding dominates the error (the intra-chunk A and M blocks, Tb X, M U) use
// a two-term bf16 split x = hi + lo on the operands (three MFMAs: hi*hi +
// lo*hi + hi*lo), which keeps ~16 significant bits.  The state S stays fp32 in
// registers; its bf16 copy feeds the MFMAs.
//
// Decay factors inside a chunk can reach exp(+-64*5.5).  A and M are therefore
// built from 16-token sub-blocks: for a diagonal sub-block both factors are
// taken relative to the sub-block's 8th token (each factor <= exp(8|L|)); for
// an off-diagonal pair (a > b) the left factor is exp(G_r - G_end(b)) <= 1
// and the right exp(G_end(b) - G_i) <= 1.  With |L| <= 5.5 nothing overflows.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <string.h>
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
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// workspace written by the scheduler, read by the main kernel
// ---------------------------------------------------------------------------
struct WorkHeader {
  int counter;   // next unit to hand out
  int status;    // non-zero: cu_seqlens broke its contract
  int n_units;   // documents * heads
  int n_docs;    // non-empty documents
};

__device__ int g_kda_status;  // sticky kda_device_flags of this device

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

// x ~= hi + lo with both terms bf16 (about 16 significant bits)
#define SPLIT_BF16(x, HI, LO)          \
  do {                                 \
    const float x_ = (x);              \
    const bf16 h_ = (bf16)x_;          \
    (HI) = h_;                         \
    (LO) = (bf16)(x_ - (float)h_);     \
  } while (0)

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// LDS layout of the main kernel (one chunk in flight)
// ---------------------------------------------------------------------------
struct alignas(16) Smem {
  bf16 Qt[CH][DK + 8];       // qh * e^G                      (A operand of Qt S)
  bf16 Kt[CH][DK + 8];       // -kh * e^G                     (A operand of X = V - Kt S)
  bf16 KbT[DK][CH + 8];      // (kh * e^{G_c - G})^T          (A operand of the state update)
  bf16 Mhi[CH][CH + 8];      // M split into hi + lo
  bf16 Mlo[CH][CH + 8];
  bf16 Tbhi[CH][CH + 8];     // Tb split into hi + lo
  bf16 Tblo[CH][CH + 8];
  union {
    bf16x8 R[3][4][2][64];   // right operands of off-diagonal sub-blocks, lane order
    float A[CH][CH + 4];     // beta-scaled strictly lower A (fp32) for the solve
  } u;
  float T[CH][CH + 4];       // (I + A)^-1
  float D[DK];               // e^{G_c}
  float tot[4][DK];          // per sub-block total decay
  float beta[CH];
  float Y[4][16][17];        // per-wave scratch of the block solve
  int unit;
  int gate_bad;
};

// ---------------------------------------------------------------------------
// scheduler: validate cu_seqlens, emit non-empty documents longest first
// ---------------------------------------------------------------------------
constexpr int SCHED_THREADS = 1024;
constexpr int NBUCKET = 1024;

__global__ __launch_bounds__(SCHED_THREADS) void kda_schedule_kernel(
    const int32_t* __restrict__ cu, int T, int H, WorkHeader* __restrict__ hdr,
    int2* __restrict__ docs) {
  __shared__ int s_vals[SCHED_THREADS];
  __shared__ int s_term;
  __shared__ int s_bad;
  __shared__ int s_carry;
  __shared__ int s_hist[NBUCKET];
  __shared__ int s_count;
  const int tid = threadIdx.x;

  if (cu == nullptr) {
    if (tid == 0) {
      docs[0] = make_int2(0, T);
      hdr->counter = 0;
      hdr->status = 0;
      hdr->n_docs = 1;
      hdr->n_units = H;
    }
    return;
  }

  // ---- 1. find the terminating entry (first entry equal to T) and validate
  if (tid == 0) { s_term = INT32_MAX; s_bad = 0; s_carry = 0; }
  __syncthreads();
  const int32_t* page = reinterpret_cast<const int32_t*>(reinterpret_cast<uintptr_t>(cu) & ~uintptr_t(4095));
  const int64_t first_idx = page - cu;  // index of page[0] relative to cu (<= 0)
  for (int64_t step = 0;; ++step) {
    const int64_t idx = first_idx + step * SCHED_THREADS + tid;  // entry index of this thread
    const bool mine = idx >= 0 && idx <= (int64_t)T;
    int val = 0;
    if (mine) val = page[step * SCHED_THREADS + tid];
    s_vals[tid] = val;
    __syncthreads();
    if (mine) {
      if (val == T) atomicMin(&s_term, (int)idx);
    }
    __syncthreads();
    const int term = s_term;
    if (mine && idx <= (int64_t)term) {
      int prev = (tid > 0) ? s_vals[tid - 1] : s_carry;
      bool bad = false;
      if (idx == 0) bad = (val != 0);
      else bad = (val < prev) || (val > T) || (val < 0);
      if (bad) atomicOr(&s_bad, 1);
    }
    __syncthreads();
    if (s_bad || term != INT32_MAX) break;
    // no terminator in this block: continue only if entries remain allowed
    const int64_t last_idx = first_idx + (step + 1) * SCHED_THREADS - 1;
    if (last_idx >= (int64_t)T) { if (tid == 0) s_bad = 1; __syncthreads(); break; }
    if (tid == 0) s_carry = s_vals[SCHED_THREADS - 1];
    __syncthreads();
  }
  if (s_bad) {
    if (tid == 0) {
      hdr->counter = 0;
      hdr->status = 1;
      hdr->n_docs = 0;
      hdr->n_units = 0;
      atomicOr(&g_kda_status, KDA_DEV_BAD_CU_SEQLENS);
    }
    return;
  }
  const int n = s_term;  // number of documents (entries 0..n are valid)

  // ---- 2. histogram of chunk counts (descending order = longest first)
  for (int b = tid; b < NBUCKET; b += SCHED_THREADS) s_hist[b] = 0;
  if (tid == 0) s_count = 0;
  __syncthreads();
  for (int i = tid; i < n; i += SCHED_THREADS) {
    const int a = cu[i], len = cu[i + 1] - a;
    if (len > 0) {
      const int nch = min((len + CH - 1) / CH, NBUCKET - 1);
      atomicAdd(&s_hist[NBUCKET - 1 - nch], 1);
      atomicAdd(&s_count, 1);
    }
  }
  __syncthreads();
  // exclusive prefix sum over buckets (Hillis-Steele on s_vals)
  {
    const int x = (tid < NBUCKET) ? s_hist[tid] : 0;
    s_vals[tid] = x;
    __syncthreads();
    for (int d = 1; d < SCHED_THREADS; d <<= 1) {
      const int y = (tid >= d) ? s_vals[tid - d] : 0;
      __syncthreads();
      s_vals[tid] += y;
      __syncthreads();
    }
    if (tid < NBUCKET) s_hist[tid] = s_vals[tid] - x;  // exclusive
  }
  __syncthreads();
  for (int i = tid; i < n; i += SCHED_THREADS) {
    const int a = cu[i], len = cu[i + 1] - a;
    if (len > 0) {
      const int nch = min((len + CH - 1) / CH, NBUCKET - 1);
      const int pos = atomicAdd(&s_hist[NBUCKET - 1 - nch], 1);
      docs[pos] = make_int2(a, len);
    }
  }
  if (tid == 0) {
    hdr->counter = 0;
    hdr->status = 0;
    hdr->n_docs = s_count;
    hdr->n_units = s_count * H;
  }
}

// ---------------------------------------------------------------------------
// main kernel
// ---------------------------------------------------------------------------
struct RawChunk {
  uint4 q[4];    // 32 bf16 channels of one token
  uint4 k[4];
  float4 g[8];   // 32 fp32 channels
  float beta;
};

__device__ __forceinline__ void load_raw(RawChunk& rc, const bf16* __restrict__ q,
                                         const bf16* __restrict__ k, const float* __restrict__ g,
                                         const float* __restrict__ beta, int64_t tok_global,
                                         bool valid, int H, int h, int cg) {
  if (valid) {
    const size_t off = ((size_t)tok_global * H + h) * DK + 32 * cg;
    const uint4* qp = reinterpret_cast<const uint4*>(q + off);
    const uint4* kp = reinterpret_cast<const uint4*>(k + off);
    const float4* gp = reinterpret_cast<const float4*>(g + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) { rc.q[i] = qp[i]; rc.k[i] = kp[i]; }
#pragma unroll
    for (int i = 0; i < 8; ++i) rc.g[i] = gp[i];
    rc.beta = beta[(size_t)tok_global * H + h];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) { rc.q[i] = make_uint4(0, 0, 0, 0); rc.k[i] = make_uint4(0, 0, 0, 0); }
#pragma unroll
    for (int i = 0; i < 8; ++i) rc.g[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    rc.beta = 0.f;
  }
}

__global__ __launch_bounds__(NTHR, 1) void kda_chunk_fwd_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, bf16* __restrict__ out,
    WorkHeader* __restrict__ hdr, const int2* __restrict__ docs, int64_t T, int H,
    float gate_bound) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int w = tid >> 6;      // wave
  const int l = tid & 63;      // lane
  const int r = l & 15;        // prologue: token inside the 16-token sub-block
  const int cg = l >> 4;       // prologue: channel group (32 channels)
  const int m = l & 31;        // recurrence: MFMA row / column lane index
  const int hg = l >> 5;       // recurrence: lane half
  const float scale = 0.08838834764831845f;  // 128^-1/2

  if (hdr->status != 0) {
    // cu_seqlens was rejected on the device: make the failure visible
    const size_t total = (size_t)T * H * DV;
    const size_t stride = (size_t)gridDim.x * NTHR;
    unsigned short* o16 = reinterpret_cast<unsigned short*>(out);
    for (size_t i = (size_t)blockIdx.x * NTHR + tid; i < total; i += stride) o16[i] = 0x7FC0;
    return;
  }
  const int n_units = hdr->n_units;
  if (tid == 0) sm.gate_bad = 0;

  for (;;) {
    __syncthreads();
    if (tid == 0) sm.unit = atomicAdd(&hdr->counter, 1);
    __syncthreads();
    const int unit = sm.unit;
    if (unit >= n_units) break;
    const int di = unit / H;
    const int h = unit - di * H;
    const int2 doc = docs[di];
    const int64_t bos = doc.x, eos = (int64_t)doc.x + doc.y;

    f32x16 S[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) S[kt][i] = 0.f;

    RawChunk cur;
    {
      const int n0 = (int)min<int64_t>(CH, eos - bos);
      load_raw(cur, q, k, g, beta, bos + 16 * w + r, 16 * w + r < n0, H, h, cg);
    }

    for (int64_t c0 = bos; c0 < eos; c0 += CH) {
      const int n = (int)min<int64_t>(CH, eos - c0);
      const int tok = 16 * w + r;

      // ---- V of this chunk in the C layout of the X tiles (see swap23)
      unsigned short vreg[2][16];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = 32 * mt + 16 * (i >> 3) + 8 * hg + (i & 7);
          vreg[mt][i] = (t < n)
              ? reinterpret_cast<const unsigned short*>(v)[((size_t)(c0 + t) * H + h) * DV + 32 * w + m]
              : (unsigned short)0;
        }

      // ================= prologue: l2 norm, cumulative decay =================
      float qh[32], kh[32], loc[32];
      {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t qa[4] = {cur.q[i].x, cur.q[i].y, cur.q[i].z, cur.q[i].w};
          const uint32_t ka[4] = {cur.k[i].x, cur.k[i].y, cur.k[i].z, cur.k[i].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            qh[8 * i + 2 * j] = bf16_lo_to_f32(qa[j]);
            qh[8 * i + 2 * j + 1] = bf16_hi_to_f32(qa[j]);
            kh[8 * i + 2 * j] = bf16_lo_to_f32(ka[j]);
            kh[8 * i + 2 * j + 1] = bf16_hi_to_f32(ka[j]);
          }
        }
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int j = 0; j < 32; ++j) { sq += qh[j] * qh[j]; sk += kh[j] * kh[j]; }
        sq += __shfl_xor(sq, 16);
        sq += __shfl_xor(sq, 32);
        sk += __shfl_xor(sk, 16);
        sk += __shfl_xor(sk, 32);
        const float rq = 1.0f / sqrtf(sq + L2_EPS);
        const float rk = 1.0f / sqrtf(sk + L2_EPS);
#pragma unroll
        for (int j = 0; j < 32; ++j) { qh[j] *= rq; kh[j] *= rk; }

        bool gbad = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float ga[4] = {cur.g[i].x, cur.g[i].y, cur.g[i].z, cur.g[i].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            loc[4 * i + j] = ga[j];
            gbad |= !(ga[j] >= gate_bound && ga[j] <= 0.f) && (tok < n);
          }
        }
        if (gbad) sm.gate_bad = 1;
        // inclusive scan over the 16 tokens of the sub-block (one DPP row)
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) {
#pragma unroll
          for (int j = 0; j < 32; ++j) {
            const float y = __shfl_up(loc[j], d, 16);
            loc[j] += (r >= d) ? y : 0.f;
          }
        }
        if (r == 15) {
#pragma unroll
          for (int j = 0; j < 32; j += 4)
            *reinterpret_cast<float4*>(&sm.tot[w][32 * cg + j]) =
                make_float4(loc[j], loc[j + 1], loc[j + 2], loc[j + 3]);
        }
        if (cg == 0) sm.beta[tok] = cur.beta;
      }
      __syncthreads();  // tot, beta visible

      // next chunk's raw inputs: issue the loads now, consume next iteration
      {
        const int64_t c1 = c0 + CH;
        const int n1 = (int)min<int64_t>(CH, eos - c1);
        load_raw(cur, q, k, g, beta, c1 + tok, c1 < eos && tok < n1, H, h, cg);
      }

      // ---- prefix decays, operand tiles of the chain, right operands of A / M
      float ref[32];
      {
        float P[32], P4[32];
#pragma unroll
        for (int j = 0; j < 32; j += 4) {
          float4 p = make_float4(0.f, 0.f, 0.f, 0.f), a = p;
#pragma unroll
          for (int ww = 0; ww < 4; ++ww) {
            const float4 t4 = *reinterpret_cast<const float4*>(&sm.tot[ww][32 * cg + j]);
            if (ww < w) { p.x += t4.x; p.y += t4.y; p.z += t4.z; p.w += t4.w; }
            a.x += t4.x; a.y += t4.y; a.z += t4.z; a.w += t4.w;
          }
          P[j] = p.x; P[j + 1] = p.y; P[j + 2] = p.z; P[j + 3] = p.w;
          P4[j] = a.x; P4[j + 1] = a.y; P4[j + 2] = a.z; P4[j + 3] = a.w;
        }
#pragma unroll
        for (int j0 = 0; j0 < 32; j0 += 8) {
          bf16x8 qt, kt;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float G = P[j0 + j] + loc[j0 + j];
            const float e = __expf(G);
            qt[j] = (bf16)(qh[j0 + j] * e);
            kt[j] = (bf16)(-kh[j0 + j] * e);
            sm.KbT[32 * cg + j0 + j][tok] = (bf16)(kh[j0 + j] * __expf(P4[j0 + j] - G));
          }
          *reinterpret_cast<bf16x8*>(&sm.Qt[tok][32 * cg + j0]) = qt;
          *reinterpret_cast<bf16x8*>(&sm.Kt[tok][32 * cg + j0]) = kt;
        }
        if (w == 0 && r == 0) {
#pragma unroll
          for (int j = 0; j < 32; ++j) sm.D[32 * cg + j] = __expf(P4[j]);
        }
        // reference of the diagonal sub-block: G at its 8th token
#pragma unroll
        for (int j = 0; j < 32; ++j) ref[j] = __shfl(loc[j], (l & ~15) | 7);
        if (w < 3) {
          // kh_i * e^{G_end(w) - G_i} <= 1 (right operand of pairs (a > w, w))
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            bf16x8 hi, lo;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int jj = 8 * s + j;
              const float tw = __shfl(loc[jj], (l & ~15) | 15);
              SPLIT_BF16(kh[jj] * __expf(tw - loc[jj]), hi[j], lo[j]);
            }
            sm.u.R[w][s][0][l] = hi;
            sm.u.R[w][s][1][l] = lo;
          }
        }
      }

      // ================= intra-chunk A and M (16x16 sub-blocks) =================
      // accMd / accAd: diagonal block (w, w); accMo[b] / accAo[b]: block (w, b), b < w
      f32x4 accMd, accAd, accMo[4], accAo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        accMd[i] = 0.f;
        accAd[i] = 0.f;
#pragma unroll
        for (int b = 0; b < 4; ++b) { accMo[b][i] = 0.f; accAo[b][i] = 0.f; }
      }
      // diagonal block (w, w) from registers
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 lqh, lql, lkh, lkl, rh, rl;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int jj = 8 * s + j;
          const float el = __expf(loc[jj] - ref[jj]);
          const float er = __expf(ref[jj] - loc[jj]);
          SPLIT_BF16(qh[jj] * el, lqh[j], lql[j]);
          SPLIT_BF16(kh[jj] * el, lkh[j], lkl[j]);
          SPLIT_BF16(kh[jj] * er, rh[j], rl[j]);
        }
        accMd = mfma16(lqh, rh, accMd);
        accMd = mfma16(lql, rh, accMd);
        accMd = mfma16(lqh, rl, accMd);
        accAd = mfma16(lkh, rh, accAd);
        accAd = mfma16(lkl, rh, accAd);
        accAd = mfma16(lkh, rl, accAd);
      }
      __syncthreads();  // right operands R visible
      // off-diagonal blocks (w, b), b < w
#pragma unroll
      for (int b = 0; b < 3; ++b) {
        if (b < w) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const bf16x8 rh = sm.u.R[b][s][0][l];
            const bf16x8 rl = sm.u.R[b][s][1][l];
            bf16x8 lqh, lql, lkh, lkl;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int jj = 8 * s + j;
              float e = loc[jj];  // G_r - P_w
              for (int ww = b + 1; ww < w; ++ww) e += sm.tot[ww][32 * cg + jj];
              const float f = __expf(e);   // e^{G_r - G_end(b)} <= 1
              SPLIT_BF16(qh[jj] * f, lqh[j], lql[j]);
              SPLIT_BF16(kh[jj] * f, lkh[j], lkl[j]);
            }
            accMo[b] = mfma16(lqh, rh, accMo[b]);
            accMo[b] = mfma16(lql, rh, accMo[b]);
            accMo[b] = mfma16(lqh, rl, accMo[b]);
            accAo[b] = mfma16(lkh, rh, accAo[b]);
            accAo[b] = mfma16(lkl, rh, accAo[b]);
            accAo[b] = mfma16(lkh, rl, accAo[b]);
          }
        }
      }
      __syncthreads();  // all reads of R done (A aliases R)
      // write A (beta-scaled, strictly lower) and M (lower incl.) of row block w
      {
        const int col = l & 15;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const int row = 4 * (l >> 4) + qq;
            const int R = 16 * w + row, C = 16 * b + col;
            float a = 0.f, mm = 0.f;
            if (b < w) {
              a = accAo[b][qq];
              mm = accMo[b][qq];
            } else if (b == w) {
              a = (col < row) ? accAd[qq] : 0.f;
              mm = (col <= row) ? accMd[qq] : 0.f;
            }
            a *= sm.beta[R];
            sm.u.A[R][C] = a;
            bf16 hi, lo;
            SPLIT_BF16(mm, hi, lo);
            sm.Mhi[R][C] = hi;
            sm.Mlo[R][C] = lo;
          }
        }
      }
      __syncthreads();

      // ================= (I + A)^-1 by 16x16 blocks =================
      if (l < 16) {
        const int j = l;
        float x[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          float acc = (rr == j) ? 1.f : 0.f;
#pragma unroll
          for (int i = 0; i < rr; ++i) acc -= sm.u.A[16 * w + rr][16 * w + i] * x[i];
          x[rr] = acc;
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
#pragma unroll
          for (int b = 0; b < 4; ++b)
            sm.T[16 * w + rr][16 * b + j] = (b == w) ? x[rr] : 0.f;
        }
      }
      __syncthreads();
#pragma unroll
      for (int dlev = 1; dlev < 4; ++dlev) {
        const int a = w, b = w - dlev;
        const int j = l & 15, gq = l >> 4;
        if (b >= 0) {
          float y[4] = {0.f, 0.f, 0.f, 0.f};
          for (int kb = b; kb < a; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const float tv = sm.T[16 * kb + i][16 * b + j];
#pragma unroll
              for (int qq = 0; qq < 4; ++qq) y[qq] += sm.u.A[16 * a + 4 * gq + qq][16 * kb + i] * tv;
            }
          }
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) sm.Y[w][4 * gq + qq][j] = y[qq];
        }
        __syncthreads();
        if (b >= 0) {
          float t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float yv = sm.Y[w][i][j];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) t[qq] -= sm.T[16 * a + 4 * gq + qq][16 * a + i] * yv;
          }
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) sm.T[16 * a + 4 * gq + qq][16 * b + j] = t[qq];
        }
        __syncthreads();
      }
      // Tb = T Diag(beta), split into hi + lo
      for (int e = tid; e < CH * CH; e += NTHR) {
        const int rr = e >> 6, cc = e & 63;
        bf16 hi, lo;
        SPLIT_BF16(sm.T[rr][cc] * sm.beta[cc], hi, lo);
        sm.Tbhi[rr][cc] = hi;
        sm.Tblo[rr][cc] = lo;
      }
      __syncthreads();

      // ================= the chain: X, U, O, S (wave w owns V columns 32w..) ====
      {
        const int rowsel = swap23(m);
        bf16x8 Sb[8];
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
          for (int j = 0; j < 8; ++j) Sb[s][j] = (bf16)S[s >> 1][8 * (s & 1) + j];

        // X = V - kh e^G S
        f32x16 X[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
          for (int i = 0; i < 16; ++i) X[mt][i] = __uint_as_float((uint32_t)vreg[mt][i] << 16);
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.Kt[32 * mt + rowsel][16 * s + 8 * hg]);
            X[mt] = mfma32(a, Sb[s], X[mt]);
          }
        }
        bf16x8 Xb[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int j = 0; j < 8; ++j) Xb[s][j] = (bf16)X[s >> 1][8 * (s & 1) + j];

        // U = Tb X
        f32x16 U[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
          for (int i = 0; i < 16; ++i) U[mt][i] = 0.f;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            if (s < 2 * (mt + 1)) {
              const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&sm.Tbhi[32 * mt + rowsel][16 * s + 8 * hg]);
              const bf16x8 al = *reinterpret_cast<const bf16x8*>(&sm.Tblo[32 * mt + rowsel][16 * s + 8 * hg]);
              U[mt] = mfma32(ah, Xb[s], U[mt]);
              U[mt] = mfma32(al, Xb[s], U[mt]);
            }
          }
        }
        bf16x8 Ubh[4], Ubl[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int j = 0; j < 8; ++j) SPLIT_BF16(U[s >> 1][8 * (s & 1) + j], Ubh[s][j], Ubl[s][j]);

        // O = scale (qh e^G S + M U)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          f32x16 O;
#pragma unroll
          for (int i = 0; i < 16; ++i) O[i] = 0.f;
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.Qt[32 * mt + rowsel][16 * s + 8 * hg]);
            O = mfma32(a, Sb[s], O);
          }
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            if (s < 2 * (mt + 1)) {
              const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&sm.Mhi[32 * mt + rowsel][16 * s + 8 * hg]);
              const bf16x8 al = *reinterpret_cast<const bf16x8*>(&sm.Mlo[32 * mt + rowsel][16 * s + 8 * hg]);
              O = mfma32(ah, Ubh[s], O);
              O = mfma32(al, Ubh[s], O);
              O = mfma32(ah, Ubl[s], O);
            }
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int t = 32 * mt + 16 * (i >> 3) + 8 * hg + (i & 7);
            if (t < n) out[((size_t)(c0 + t) * H + h) * DV + 32 * w + m] = (bf16)(O[i] * scale);
          }
        }

        // S <- e^{G_c} S + (kh e^{G_c - G})^T U
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            S[kt][i] *= sm.D[32 * kt + 16 * (i >> 3) + 8 * hg + (i & 7)];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.KbT[32 * kt + rowsel][16 * s + 8 * hg]);
            S[kt] = mfma32(a, Ubh[s], S[kt]);
          }
        }
      }
      __syncthreads();  // the next chunk overwrites every LDS tile
    }
  }
  __syncthreads();
  if (tid == 0 && sm.gate_bad) atomicOr(&g_kda_status, KDA_DEV_GATE_RANGE);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
thread_local std::string t_last_error;

int fail(int code, const std::string& msg) {
  t_last_error = msg;
  return code;
}

struct DeviceInfo {
  int num_cu = 0;
  bool pool_ready = false;
};
std::mutex g_mu;
std::vector<DeviceInfo> g_devices;

int device_info(int dev, DeviceInfo** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  if ((int)g_devices.size() <= dev) g_devices.resize(dev + 1);
  DeviceInfo& d = g_devices[dev];
  if (d.num_cu == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return -1;
    d.num_cu = n;
  }
  if (!d.pool_ready) {
    hipMemPool_t pool;
    if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
      uint64_t thr = UINT64_MAX;
      (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
    }
    d.pool_ready = true;
  }
  *out = &d;
  return 0;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

extern "C" int kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const int32_t* cu_seqlens, int64_t T, int32_t H,
                             int32_t chunk, float gate_bound, void* out, hipStream_t stream) {
  t_last_error.clear();
  if (T < 0) return fail(KDA_ERR_BAD_SHAPE, "T must be >= 0");
  if (T > INT32_MAX) return fail(KDA_ERR_BAD_SHAPE, "T must be <= INT32_MAX");
  if (H < 1) return fail(KDA_ERR_BAD_SHAPE, "H must be >= 1");
  if (H > KDA_MAX_HEADS) return fail(KDA_ERR_BAD_SHAPE, "H must be <= KDA_MAX_HEADS");
  if (T == 0) return KDA_OK;
  if (!q) return fail(KDA_ERR_NULL_PTR, "q is NULL");
  if (!k) return fail(KDA_ERR_NULL_PTR, "k is NULL");
  if (!v) return fail(KDA_ERR_NULL_PTR, "v is NULL");
  if (!g) return fail(KDA_ERR_NULL_PTR, "g is NULL");
  if (!beta) return fail(KDA_ERR_NULL_PTR, "beta is NULL");
  if (!out) return fail(KDA_ERR_NULL_PTR, "out is NULL");
  if (chunk != KDA_CHUNK) return fail(KDA_ERR_UNSUPPORTED, "chunk must be 64");
  if (!(gate_bound >= -5.5f && gate_bound < 0.f))
    return fail(KDA_ERR_UNSUPPORTED, "gate_bound must be finite and in [-5.5, 0)");
  if (!aligned(q, 16)) return fail(KDA_ERR_ALIGN, "q is not 16-byte aligned");
  if (!aligned(k, 16)) return fail(KDA_ERR_ALIGN, "k is not 16-byte aligned");
  if (!aligned(v, 16)) return fail(KDA_ERR_ALIGN, "v is not 16-byte aligned");
  if (!aligned(g, 16)) return fail(KDA_ERR_ALIGN, "g is not 16-byte aligned");
  if (!aligned(out, 16)) return fail(KDA_ERR_ALIGN, "out is not 16-byte aligned");
  if (!aligned(beta, 4)) return fail(KDA_ERR_ALIGN, "beta is not 4-byte aligned");
  if (cu_seqlens && !aligned(cu_seqlens, 4)) return fail(KDA_ERR_ALIGN, "cu_seqlens is not 4-byte aligned");

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(KDA_ERR_HIP, "hipGetDevice failed");
  DeviceInfo* di = nullptr;
  if (device_info(dev, &di) != 0) return fail(KDA_ERR_HIP, "hipDeviceGetAttribute failed");

  const size_t ws_bytes = sizeof(WorkHeader) + sizeof(int2) * (size_t)T;
  void* ws = nullptr;
  if (hipMallocAsync(&ws, ws_bytes, stream) != hipSuccess || !ws)
    return fail(KDA_ERR_ALLOC, "hipMallocAsync of the workspace failed");
  WorkHeader* hdr = static_cast<WorkHeader*>(ws);
  int2* docs = reinterpret_cast<int2*>(hdr + 1);

  hipLaunchKernelGGL(kda_schedule_kernel, dim3(1), dim3(SCHED_THREADS), 0, stream, cu_seqlens,
                     (int)T, (int)H, hdr, docs);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) {
    hipLaunchKernelGGL(kda_chunk_fwd_kernel, dim3(di->num_cu), dim3(NTHR), 0, stream,
                       static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                       static_cast<const bf16*>(v), g, beta, static_cast<bf16*>(out), hdr, docs,
                       T, (int)H, gate_bound);
    e = hipGetLastError();
  }
  const hipError_t ef = hipFreeAsync(ws, stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  if (ef != hipSuccess) return fail(KDA_ERR_HIP, "hipFreeAsync of the workspace failed");
  return KDA_OK;
}

extern "C" const char* kda_last_error(void) { return t_last_error.c_str(); }

extern "C" int kda_device_status(hipStream_t stream) {
  if (hipStreamSynchronize(stream) != hipSuccess) return KDA_ERR_HIP;
  int st = 0;
  if (hipMemcpyFromSymbol(&st, HIP_SYMBOL(g_kda_status), sizeof(int), 0, hipMemcpyDeviceToHost) != hipSuccess)
    return KDA_ERR_HIP;
  const int zero = 0;
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_kda_status), &zero, sizeof(int), 0, hipMemcpyHostToDevice) != hipSuccess)
    return KDA_ERR_HIP;
  return st;
}
