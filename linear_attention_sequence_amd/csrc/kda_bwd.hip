// kda_bwd.hip -- chunked backward of the KDA forward (fp32).
//
// Gradients of L = sum_t <o_t, do_t> + sum_d <S_end(d), dS_end(d)> with
// respect to q, k, v, g, beta and the initial states, for the operator of
// include/kda.h.  Like the backward of the pages' fused forward (page
// "nemo_automodel.components.models.kimi_k3.kda_fused", package docstring),
// it recomputes every intermediate from q, k, v, g, beta and cu_seqlens.
//
// Per chunk (c <= 64 tokens r, i; S0 the state at its start, dSc = dL/dS at
// its end; Tb = T Diag(beta), T = (I + Diag(beta) Kk)^-1, Kk and M the
// decayed key-key and query-key products, Qt, Kt, Kbar, D the decayed tiles):
//
//   forward:   X = V - Kt S0,   U = Tb X
//   dS0 = F^T dSc + R  with  F^T = D - Kt^T Tb^T Kbar,
//                            R   = scale Qt^T dO - Kt^T Tb^T (scale M^T dO)
//   dU  = scale M^T dO + Kbar dSc,  dX = Tb^T dU (= dV)
//   dQt = scale dO S0^T, dKt = -dX S0^T, dKbar = U dSc^T, dD = rowsum(dSc * S0)
//   dM  = scale tril(dO U^T), dTb = tril(dU X^T), dbeta_i += sum_r dTb_ri T_ri
//   dA  = -T^T (dTb Diag(beta)) T^T (strict lower), dbeta_r += sum_i dA_ri Kk_ri,
//   dKk = Diag(beta) dA
// followed by the bilinear forms of M and Kk (exp(G_r - G_i) per channel,
// never above 1 for i <= r), the decayed tiles, the in-chunk cumsum of g and
// the l2 norms.  The same derivation, in fp64 numpy, is checked against an
// autograd oracle.
//
// Passes (all on the caller's stream):
//   1. the stateful forward with S stored at every chunk start (kda_fwd.hip);
//   2. kda_bwd_setup_kernel: cu_seqlens check and the chunk table;
//   3. kda_bwd_prep_kernel (parallel over chunks): qh, kh, G, T, Kk, M and
//      F^T, R of every chunk (through Z = Kt^T Tb^T: F^T = D - Z Kbar,
//      R = scale (Qt^T - Z M^T) dO);
//   4. kda_bwd_chain_kernel (per document, head and quarter of the value
//      columns, last chunk first): dS <- F^T dS + R, storing dS at every
//      chunk end;
//   5. kda_bwd_grads_kernel (parallel over chunks): all input gradients.
// Products run on fp32 MFMA (16x16x4) with operands staged through LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>
#include <type_traits>
#include <vector>
#include <atomic>

#include "kda.h"

#include "kda_host_checks.h"

namespace kda_host {
int fail(int code, const std::string& msg);
int device(int* num_cu, int** status_word);
hipError_t alloc_async(void** p, size_t bytes, hipStream_t stream);
int forward_with_chunk_states(const void* q, const void* k, const void* v, const float* g,
                              const float* beta, const int32_t* cu, int32_t n_docs, int64_t T,
                              int32_t H, float gate_bound, const float* h0, void* out,
                              float* chunk_states, hipStream_t stream);
}  // namespace kda_host

namespace {

constexpr int CH = 64;
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int NT = 512;                      // threads per workgroup: 8 waves, 2 per SIMD
constexpr int NW = NT / 64;                  // waves per workgroup
constexpr int TPT = NT / CH;                 // threads per token row (8)
constexpr int CPT = DK / TPT;                // channels per thread in a token row (16)
constexpr int RG = NT / DK;                  // row groups when a thread owns one channel (4)
constexpr int LD = 132;                      // padded row of a [64][128] LDS tile (= 4 mod 8: the two rows
                                             // of a half-wave's C-layout store hit different banks)
constexpr int LDC = 65;                      // padded row of a [64][64] LDS tile
constexpr int LDM = 68;                      // [64][64] LDS tile read in 16-byte row pieces
constexpr float SCALE = 0.08838834764831845f;  // 128^-1/2
constexpr float L2_EPS = 1e-6f;
constexpr int SROW = 20;                     // staged row: 16 k values + 4 padding (conflict-free b128)
constexpr int STAGE_FLOATS = SROW * (128 + 128);
typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// per (chunk, head) image written by the prep pass, fp32
constexpr int IMG_QH = 0;                    // [64][128] qh
constexpr int IMG_KH = IMG_QH + CH * DK;     // [64][128] kh
constexpr int IMG_G = IMG_KH + CH * DK;      // [64][128] in-chunk cumsum of g
constexpr int IMG_T = IMG_G + CH * DK;       // [64][64] (I + Diag(beta) Kk)^-1
constexpr int IMG_KK = IMG_T + CH * CH;      // [64][64] Kk (strictly lower)
constexpr int IMG_M = IMG_KK + CH * CH;      // [64][64] M (lower incl.)
constexpr int IMG_RQ = IMG_M + CH * CH;      // [64] 1/||q||
constexpr int IMG_RK = IMG_RQ + CH;          // [64] 1/||k||
constexpr int IMG_FLOATS = IMG_RK + CH;

// per-workgroup scratch of the gradient pass, fp32 (the [64][64] tiles dM,
// dTb and Z live in LDS the products have finished with)
constexpr int SC_DQK = 0;                    // [128][128]: rows 0..63 dQt, 64..127 dKt
constexpr int SC_DKB = SC_DQK + 2 * CH * DK;  // [64][128] dKbar
constexpr int SC_FLOATS = SC_DKB + CH * DK;

// per-workgroup scratch of the prep pass: none (its products stay in LDS)
constexpr int SP_FLOATS = 0;

struct ChunkDesc {
  int start;  // first token
  int len;    // tokens (0: unused slot)
  int doc;
  int pad;
};

__device__ __forceinline__ f32x4 mfma16f(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(bf16 x) { return (float)x; }

// x of another lane in the same row of 16, chosen by the DPP control CTRL
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// LDS written by the lanes of a wave visible to the same wave
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// C (M x N) = sum over K of la(m, k) lb(k, n), then out(m, n, value).
// fp32 MFMA 16x16x4; operands staged through LDS (stage) in k-tiles of 16,
// the next k-tiles loaded into registers while the current one multiplies.
// AK / BK: whether consecutive threads fetch consecutive k (operand stored
// along k) or consecutive m / n, so that global fetches are contiguous.
// out(m, n, value, old) receives old(m, n) as well (zero by default).
// Every thread of the workgroup calls it (tid = its thread index); it
// synchronises before returning results and before its first staging (so
// operands may live in LDS buffers that out() overwrites), and again after
// the last out().  Its first operand fetches come before any barrier: LDS
// operands written just before the call need a barrier from the caller.
struct NoOld {
  __device__ float operator()(int, int) const { return 0.f; }
};

// PFMAX: k-tiles in flight (at most); EARLY_OLD: old() is fetched before the
// first k-tile instead of after the last, so its loads overlap the product.
template <int M, int N, int K, bool AK, bool BK, int PFMAX = 3, bool EARLY_OLD = false, class LA,
          class LB, class OUT, class OLD = NoOld>
__device__ __forceinline__ void wg_gemm(LA la, LB lb, OUT out, float* stage, int tid,
                                        OLD old = OLD()) {
  static_assert(M % 16 == 0 && N % 16 == 0 && K % 16 == 0 && M <= 128 && N <= 128, "shape");
  constexpr int TM = M / 16, TN = N / 16, TILES = TM * TN;
  constexpr int PER = (TILES + NW - 1) / NW;  // output tiles per wave (the last round may be partial)
  constexpr int NA = (16 * M + NT - 1) / NT, NB = (16 * N + NT - 1) / NT;  // staged per thread
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  // An operand fetched along k is staged m-major, [M][SROW] (row m holds
  // k = k0 .. k0 + 15); one fetched along m (n) is staged k-major,
  // [16][M + 4], so that a wave's staging stores fill consecutive banks.
  constexpr int MP = M + 4, NP = N + 4;
  static_assert(16 * MP <= M * SROW && 16 * NP <= N * SROW, "k-major tile fits the stage");
  float* sa = stage;
  float* sb = stage + M * SROW;
  // (m or n, kk) of this thread's staged element j
  auto a_mk = [&](int j, int& m, int& kk) {
    const int idx = min(tid + NT * j, 16 * M - 1);
    if (AK) { m = idx >> 4; kk = idx & 15; } else { kk = idx / M; m = idx - kk * M; }
  };
  auto b_nk = [&](int j, int& n, int& kk) {
    const int idx = min(tid + NT * j, 16 * N - 1);
    if (BK) { n = idx >> 4; kk = idx & 15; } else { kk = idx / N; n = idx - kk * N; }
  };
  // up to PF k-tiles in flight: tile k is multiplied while tiles k+1 .. k+PF-1
  // are on their way (a load round trip is several tiles' worth of MFMA time)
  constexpr int KT = K / 16;
  constexpr int PF = KT < PFMAX ? KT : PFMAX;
  float ra[PF][NA], rb[PF][NB];
  auto fetch = [&](int set, int k0) {
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      int m, kk;
      a_mk(j, m, kk);
      ra[set][j] = la(m, k0 + kk);  // clamped index: always a valid element
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      int n, kk;
      b_nk(j, n, kk);
      rb[set][j] = lb(k0 + kk, n);
    }
  };
  f32x4 acc[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
  // old(m, n): values out() adds to, all fetched before the first out() so
  // that the loads are not ordered behind its stores
  f32x4 prev[PER];
  auto fetch_old = [&]() {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int t = w + NW * p, tm = t / TN, tn = t - tm * TN;
      if (TILES % NW != 0 && t >= TILES) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) prev[p][i] = old(16 * tm + 4 * (l >> 4) + i, 16 * tn + (l & 15));
    }
  };
  auto tile = [&](int set, int kt) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      int m, kk;
      a_mk(j, m, kk);
      if (NA * NT == 16 * M || tid + NT * j < 16 * M)
        sa[AK ? m * SROW + kk : kk * MP + m] = ra[set][j];
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      int n, kk;
      b_nk(j, n, kk);
      if (NB * NT == 16 * N || tid + NT * j < 16 * N)
        sb[BK ? n * SROW + kk : kk * NP + n] = rb[set][j];
    }
    __syncthreads();
    if (kt + PF < KT) fetch(set, 16 * (kt + PF));
    // k-step s pairs lane group g = l / 16 with k = 4 g + s on both operands,
    // so each lane reads its four k values of an m-major tile as one 16-byte
    // vector; of a k-major one, as four 4-byte reads whose lane groups start
    // 4 (M + 4) = 16 (mod 64) floats apart, so they read different banks
    const int kq = 4 * (l >> 4);
    auto rd = [&](const float* s_, int rowp, bool along_k, int i0) {
      if (along_k) return *reinterpret_cast<const float4*>(&s_[(i0 + (l & 15)) * SROW + kq]);
      const float* c = &s_[kq * rowp + i0 + (l & 15)];
      return float4{c[0], c[rowp], c[2 * rowp], c[3 * rowp]};
    };
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int t = w + NW * p, tm = t / TN, tn = t - tm * TN;
      if (TILES % NW != 0 && t >= TILES) break;  // wave-uniform
      const float4 av = rd(sa, MP, AK, 16 * tm);
      const float4 bv = rd(sb, NP, BK, 16 * tn);
      acc[p] = mfma16f(av.x, bv.x, acc[p]);
      acc[p] = mfma16f(av.y, bv.y, acc[p]);
      acc[p] = mfma16f(av.z, bv.z, acc[p]);
      acc[p] = mfma16f(av.w, bv.w, acc[p]);
    }
  };
#pragma unroll
  for (int set = 0; set < PF; ++set) fetch(set, 16 * set);
  if (EARLY_OLD) fetch_old();
#pragma unroll 1
  for (int kt = 0; kt < KT; kt += PF) {
#pragma unroll
    for (int set = 0; set < PF; ++set)
      if (kt + set < KT) tile(set, kt + set);
  }
  __syncthreads();
  if (!EARLY_OLD) fetch_old();
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int t = w + NW * p, tm = t / TN, tn = t - tm * TN;
    if (TILES % NW != 0 && t >= TILES) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) out(16 * tm + 4 * (l >> 4) + i, 16 * tn + (l & 15), acc[p][i], prev[p][i]);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// setup: cu_seqlens (exactly n_docs + 1 entries), the chunk table and the
// order in which the chain kernel takes the documents
// ---------------------------------------------------------------------------
constexpr int SETUP_RANK_DOCS = 1024;  // documents ranked by length (beyond: cu_seqlens order)

__global__ __launch_bounds__(1024) void kda_bwd_setup_kernel(const int32_t* __restrict__ cu,
                                                             int n_docs, int T, int n_slots,
                                                             ChunkDesc* __restrict__ table,
                                                             int* __restrict__ order,
                                                             int* __restrict__ bad,
                                                             int* __restrict__ status_word) {
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (cu != nullptr) {
    for (int i = tid; i <= n_docs; i += 1024) {
      const int val = cu[i];
      bool b = (i == 0) ? (val != 0) : (val < cu[i - 1] || val > T);
      if (i == n_docs && val != T) b = true;
      if (b) atomicOr(&s_bad, 1);
    }
  }
  for (int s = tid; s < n_slots; s += 1024) table[s] = ChunkDesc{0, 0, 0, 0};
  __syncthreads();
  if (tid == 0) {
    *bad = s_bad;
    if (s_bad) atomicOr(status_word, KDA_DEV_BAD_CU_SEQLENS);
  }
  if (s_bad) return;
  for (int d = tid; d < n_docs; d += 1024) {
    const int a = cu ? cu[d] : 0, b = cu ? cu[d + 1] : T;
    const int first = a / CH + d;
    for (int j = 0; CH * j < b - a; ++j)
      table[first + j] = ChunkDesc{a + CH * j, min(CH, b - a - CH * j), d, 0};
  }
  // longest document first (ties by index), so that the longest sequential
  // chains start first: order[rank] = document
  __shared__ int s_len[SETUP_RANK_DOCS];
  if (n_docs <= SETUP_RANK_DOCS) {
    for (int d = tid; d < n_docs; d += 1024) s_len[d] = cu ? cu[d + 1] - cu[d] : T;
    __syncthreads();
    for (int d = tid; d < n_docs; d += 1024) {
      const int len = s_len[d];
      int rank = 0;
      for (int e = 0; e < n_docs; ++e) {
        const int le = s_len[e];
        rank += (le > len || (le == len && e < d)) ? 1 : 0;
      }
      order[rank] = d;
    }
  } else {
    for (int d = tid; d < n_docs; d += 1024) order[d] = d;
  }
}

// ---------------------------------------------------------------------------
// prep: per (chunk, head) image and F^T, R
// ---------------------------------------------------------------------------
struct PrepSmem {
  float qh[CH][LD];
  float kh[CH][LD];
  float G[CH][LD];
  float m[CH][LDC];
  float t[CH][LDC];
  float beta[CH];
  union {
    float kk[CH][LDC];           // until T is built and the image written
    alignas(16) float stage[STAGE_FLOATS];  // then the products' staging
  };
};

// q, k l2-normalised, G = in-chunk cumsum of g (rows past len: qh = kh = 0,
// g = 0 so G stays at the last row), beta; into LDS and the image
__device__ __forceinline__ void load_chunk(PrepSmem& sm, float* img, const bf16* __restrict__ q,
                                           const bf16* __restrict__ k, const float* __restrict__ g,
                                           const float* __restrict__ beta, int start, int len,
                                           int H, int h, int tid) {
  // TPT threads per token, CPT channels each
  const int t = tid / TPT, c0 = CPT * (tid % TPT);
  float qv[CPT], kv[CPT], gv[CPT];
  float sq = 0.f, sk = 0.f;
  const size_t row = ((size_t)(start + t) * H + h) * DK;
  static_assert(CPT % 8 == 0, "whole 16-byte vectors");
  if (t < len) {
#pragma unroll
    for (int j = 0; j < CPT; j += 8) {
      const uint4 uq = *reinterpret_cast<const uint4*>(q + row + c0 + j);
      const uint4 uk = *reinterpret_cast<const uint4*>(k + row + c0 + j);
      const float4 g0 = *reinterpret_cast<const float4*>(g + row + c0 + j);
      const float4 g1 = *reinterpret_cast<const float4*>(g + row + c0 + j + 4);
      const uint32_t wq[4] = {uq.x, uq.y, uq.z, uq.w}, wk[4] = {uk.x, uk.y, uk.z, uk.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        qv[j + 2 * u] = __uint_as_float(wq[u] << 16);
        qv[j + 2 * u + 1] = __uint_as_float(wq[u] & 0xFFFF0000u);
        kv[j + 2 * u] = __uint_as_float(wk[u] << 16);
        kv[j + 2 * u + 1] = __uint_as_float(wk[u] & 0xFFFF0000u);
      }
      const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
      for (int u = 0; u < 8; ++u) gv[j + u] = gg[u];
    }
  } else {
#pragma unroll
    for (int j = 0; j < CPT; ++j) qv[j] = kv[j] = gv[j] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    sq += qv[j] * qv[j];
    sk += kv[j] * kv[j];
  }
#pragma unroll
  for (int o = 1; o < TPT; o <<= 1) {
    sq += __shfl_xor(sq, o);
    sk += __shfl_xor(sk, o);
  }
  const float rq = 1.f / sqrtf(sq + L2_EPS), rk = 1.f / sqrtf(sk + L2_EPS);
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    sm.qh[t][c0 + j] = qv[j] * rq;
    sm.kh[t][c0 + j] = kv[j] * rk;
    sm.G[t][c0 + j] = gv[j];
  }
  if (tid % TPT == 0) {
    img[IMG_RQ + t] = rq;
    img[IMG_RK + t] = rk;
    sm.beta[t] = t < len ? beta[(size_t)(start + t) * H + h] : 0.f;
  }
  __syncthreads();
  // cumsum over the rows of each channel: RG groups of CH / RG rows, the
  // group totals combined through LDS (sm.t is free until T is built)
  {
    constexpr int RR = CH / RG;
    const int c = tid % DK, part = tid / DK;
    float x[RR];
#pragma unroll
    for (int j = 0; j < RR; ++j) x[j] = sm.G[RR * part + j][c];
#pragma unroll
    for (int j = 1; j < RR; ++j) x[j] += x[j - 1];
    float* tot = &sm.t[0][0];
    tot[part * DK + c] = x[RR - 1];
    __syncthreads();
    float off = 0.f;
#pragma unroll
    for (int p2 = 0; p2 < RG - 1; ++p2)
      if (p2 < part) off += tot[p2 * DK + c];
#pragma unroll
    for (int j = 0; j < RR; ++j) sm.G[RR * part + j][c] = x[j] + off;
  }
  __syncthreads();
  for (int idx = tid; idx < CH * DK; idx += NT) {
    const int r = idx >> 7, c = idx & 127;
    img[IMG_QH + idx] = sm.qh[r][c];
    img[IMG_KH + idx] = sm.kh[r][c];
    img[IMG_G + idx] = sm.G[r][c];
  }
}

__global__ __launch_bounds__(NT, 1) void kda_bwd_prep_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ beta, const bf16* __restrict__ dout, const ChunkDesc* __restrict__ table,
    const int* __restrict__ bad, int n_items, int H, float* __restrict__ imgs, float* __restrict__ fts,
    float* __restrict__ rs) {
  __shared__ PrepSmem sm;
  if (*bad) return;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int slot = item / H, h = item - slot * H;
    const ChunkDesc cd = table[slot];
    if (cd.len == 0) continue;
    const int start = cd.start, len = cd.len;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));  // lane values are recomputed per item, not kept live
    float* img = imgs + (size_t)item * IMG_FLOATS;
    __syncthreads();
    load_chunk(sm, img, q, k, g, beta, start, len, H, h, tid);
    // Kk (strictly lower, to the image) and M (lower incl., LDS) in 16-token
    // blocks.  Blocks above the diagonal are zero.
    for (int idx = tid; idx < CH * CH; idx += NT) {
      const int r = idx >> 6, i = idx & 63;
      if ((i >> 4) > (r >> 4)) {
        img[IMG_KK + idx] = 0.f;
        sm.m[r][i] = 0.f;
      }
    }
    // Kk and M by 16x16 tiles (a, b), b <= a, one wave per tile pair on fp32
    // MFMA (the Kk and M tiles share the right operand).  The decay
    // exp(G_r - G_i) splits at rho = G of row 16a + 7: both factors stay within
    // e^{+-44} for the pairs of a diagonal tile (bounded gate, |g| <= 5.5 per
    // token), and for the tiles to the left they are <= 1 or underflow
    // harmlessly (the product is what underflows); entries above the diagonal
    // are discarded, never used.  k-step ks of lane group g takes channel
    // c = 4 ks + g on both operands.
    {
      const int w = tid >> 6, l = tid & 63, g = l >> 4, cl = l & 15;
      for (int p = w; p < 10; p += NW) {  // wave-uniform
        const int a = p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3, b = p - a * (a + 1) / 2;
        const int ra = 16 * a + cl, ib = 16 * b + cl;
        const float* rho = sm.G[16 * a + 7];
        f32x4 kk = {0.f, 0.f, 0.f, 0.f}, mm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int ks = 0; ks < DK / 4; ++ks) {
          const int c = 4 * ks + g;
          const float rc = rho[c];
          const float ea = __expf(sm.G[ra][c] - rc), eb = __expf(rc - sm.G[ib][c]);
          const float bop = sm.kh[ib][c] * eb;
          kk = mfma16f(sm.kh[ra][c] * ea, bop, kk);
          mm = mfma16f(sm.qh[ra][c] * ea, bop, mm);
        }
        // C layout: lane (g, cl) holds rows 16a + 4g + i of column 16b + cl
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * a + 4 * g + i, col = 16 * b + cl;
          img[IMG_KK + r * CH + col] = col < r ? kk[i] : 0.f;
          sm.m[r][col] = col <= r ? mm[i] : 0.f;
        }
      }
    }
    __syncthreads();
    // T = (I + B)^-1 with B = Diag(beta) Kk (strictly lower), in 16-row blocks.
    // Diagonal blocks T_aa = (I + B_aa)^-1 by forward substitution: eight
    // consecutive lanes share a column, lane j sums the terms m = j (mod 8) of a
    // row, DPP combines the eight partial sums (every lane ends with the same
    // total) and lane r % 8 keeps x_r.  Then the blocks below the diagonal,
    // T_ab = -T_aa sum_{b <= k < a} B_ak T_kb, by column block (one wave each)
    // on fp32 MFMA.  Blocks above the diagonal are zero.
    for (int idx = tid; idx < CH * CH; idx += NT) sm.kk[idx >> 6][idx & 63] = img[IMG_KK + idx];
    for (int idx = tid; idx < CH * CH; idx += NT) {
      const int r = idx >> 6, i = idx & 63;
      if ((i >> 4) > (r >> 4)) sm.t[r][i] = 0.f;
    }
    __syncthreads();
    {
      static_assert(NT == 8 * CH, "eight lanes per column");
      const int R0 = 16 * (tid >> 7), i = (tid >> 3) & 15, j = tid & 7;
      float x0 = 0.f, x1 = 0.f;  // x of rows R0 + j and R0 + 8 + j; zero until solved
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // terms m >= r vanish: Kk is strictly lower and x_m is still zero
        float acc = sm.kk[R0 + r][R0 + j] * x0;
        if (r > 8) acc = fmaf(sm.kk[R0 + r][R0 + 8 + j], x1, acc);
        acc += dpp_mov<0xB1>(acc);   // lanes k ^ 1
        acc += dpp_mov<0x4E>(acc);   // lanes k ^ 2
        acc += dpp_mov<0x141>(acc);  // lane 7 - k of the same eight
        const float xr = r < i ? 0.f : (r == i ? 1.f : -sm.beta[R0 + r] * acc);
        if (j == (r & 7)) {
          if (r < 8) x0 = xr;
          else x1 = xr;
        }
      }
      sm.t[R0 + j][R0 + i] = x0;
      sm.t[R0 + 8 + j][R0 + i] = x1;
    }
    __syncthreads();
    // Column block BC of T below the diagonal, wave BC.  MFMA 16x16x4: k-step s
    // of lane group g takes k = 4 g + s on both operands, so the C layout of a
    // product (lane l: rows 4 g .. 4 g + 3 of column l % 16) is the B operand
    // of the next and the blocks T_k,BC stay in registers.
    {
      const int w = tid >> 6, l = tid & 63, g = l >> 4, cl = l & 15;
      auto column = [&](auto bconst) {
        constexpr int BC = decltype(bconst)::value;
        f32x4 tcol[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) tcol[BC][i] = sm.t[16 * BC + 4 * g + i][16 * BC + cl];
#pragma unroll
        for (int a = BC + 1; a < 4; ++a) {
          const float ba = sm.beta[16 * a + cl];
          f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = BC; kb < a; ++kb)
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
              y = mfma16f(ba * sm.kk[16 * a + cl][16 * kb + 4 * g + s2], tcol[kb][s2], y);
          f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) z = mfma16f(sm.t[16 * a + cl][16 * a + 4 * g + s2], y[s2], z);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            tcol[a][i] = -z[i];
            sm.t[16 * a + 4 * g + i][16 * BC + cl] = -z[i];
          }
        }
      };
      if (w == 0) column(std::integral_constant<int, 0>());
      else if (w == 1) column(std::integral_constant<int, 1>());
      else if (w == 2) column(std::integral_constant<int, 2>());
    }
    __syncthreads();
    for (int idx = tid; idx < CH * CH; idx += NT) {
      const int r = idx >> 6, i = idx & 63;
      img[IMG_T + idx] = sm.t[r][i];
      img[IMG_M + idx] = sm.m[r][i];
    }
    const float* Gl = sm.G[CH - 1];
    const size_t drow0 = (size_t)start * H + h;
    // rows past the chunk read the last row, then select zero: no branch
    // around the load (so the loads can be waited for by count)
    auto dO = [&](int r, int v) -> float {
      const float x = bf16_to_f32(dout[(drow0 + (size_t)min(r, len - 1) * H) * DV + v]);
      return r < len ? x : 0.f;
    };
    // Z = Kt^T Tb^T  [c][r] (Z_cr = sum_t Kt_tc T_rt beta_t), over M and T,
    // which the image holds from here on: M and T are contiguous, 128 rows of
    // LDC floats
    static_assert(offsetof(PrepSmem, t) == offsetof(PrepSmem, m) + sizeof(PrepSmem::m),
                  "M and T contiguous");
    float (*const zb)[LDC] = reinterpret_cast<float (*)[LDC]>(&sm.m[0][0]);
    wg_gemm<DK, CH, CH, false, true, 4>(
        [&](int c, int t) { return sm.kh[t][c] * __expf(sm.G[t][c]); },
        [&](int t, int r) { return sm.t[r][t] * sm.beta[t]; },
        [&](int c, int r, float x, float) { zb[c][r] = x; }, sm.stage, tid);
    // F^T = D - Z Kbar  [c][c']
    float* ft = fts + (size_t)item * DK * DK;
    wg_gemm<DK, DK, CH, true, false, 4>(
        [&](int c, int r) { return zb[c][r]; },
        [&](int r, int c2) { return sm.kh[r][c2] * __expf(Gl[c2] - sm.G[r][c2]); },
        [&](int c, int c2, float x, float) { ft[c * DK + c2] = (c == c2 ? __expf(Gl[c]) : 0.f) - x; },
        sm.stage, tid);
    // W = scale (Qt^T - Z M^T)  [c][s], over kh (read last by F^T); M from
    // the image, which this workgroup wrote above
    float (*const wb)[LDC] = reinterpret_cast<float (*)[LDC]>(&sm.kh[0][0]);
    static_assert(DK * LDC <= CH * LD, "W fits over kh");
    const float* im = img + IMG_M;
    wg_gemm<DK, CH, CH, true, true, 4>(
        [&](int c, int r) { return zb[c][r]; },
        [&](int r, int s2) { return im[s2 * CH + r]; },
        [&](int c, int s2, float x, float) {
          wb[c][s2] = SCALE * (sm.qh[s2][c] * __expf(sm.G[s2][c]) - x);
        },
        sm.stage, tid);
    // R = W dO  [c][v]
    float* rr = rs + (size_t)item * DK * DV;
    wg_gemm<DK, DV, CH, true, false, 4>(
        [&](int c, int s2) { return wb[c][s2]; },
        [&](int s2, int v) { return dO(s2, v); },
        [&](int c, int v, float x, float) { rr[c * DV + v] = x; }, sm.stage, tid);
  }
}

// ---------------------------------------------------------------------------
// chain: per (document, head, quarter of the value columns), last chunk
// first: dS <- F^T dS + R.  F^T acts on the key index, so the value columns
// of dS evolve independently: each (document, head) chain is split over four
// workgroups of CV columns, which quarters the product on the sequential path
// of a chunk.  Workgroups take documents longest first (order, from the setup
// kernel), the four parts of a chain next to each other.
// ---------------------------------------------------------------------------
constexpr int CV = DV / 4;  // value columns per chain workgroup

constexpr int CHAIN_PF = 8;  // k-tiles of F^T in flight in a chain step

struct ChainSmem {
  float ds[DK][CV + 1];
  alignas(16) float stage[STAGE_FLOATS];
};

__global__ __launch_bounds__(NT, 1) void kda_bwd_chain_kernel(
    const int32_t* __restrict__ cu, int T, int H, const int* __restrict__ bad,
    const int* __restrict__ order, const float* __restrict__ fts, const float* __restrict__ rs,
    const float* __restrict__ dht, float* __restrict__ dstates, float* __restrict__ dh0) {
  __shared__ ChainSmem sm;
  if (*bad) return;
  const int tid = threadIdx.x;
  constexpr int NH = DV / CV;  // workgroups per chain
  const int rk = blockIdx.x / (H * NH), rem = blockIdx.x - rk * (H * NH);
  const int h = rem / NH, v0 = CV * (rem - h * NH);
  const int d = order[rk];
  const int a = cu ? cu[d] : 0, b = cu ? cu[d + 1] : T;
  const int first = a / CH + d;
  const int n = (b - a + CH - 1) / CH;
  const size_t dh = ((size_t)d * H + h) * DK * DV;
  for (int idx = tid; idx < DK * CV; idx += NT) {
    const int c = idx / CV, v = idx % CV;
    sm.ds[c][v] = dht ? dht[dh + c * DV + v0 + v] : 0.f;
  }
  for (int j = n - 1; j >= 0; --j) {
    const size_t item = (size_t)(first + j) * H + h;
    __syncthreads();
    float* dst = dstates + item * DK * DV;
    for (int idx = tid; idx < DK * CV; idx += NT) {
      const int c = idx / CV, v = idx % CV;
      dst[c * DV + v0 + v] = sm.ds[c][v];
    }
    const float* ft = fts + item * DK * DK;
    const float* rr = rs + item * DK * DV + v0;
    // all of F^T's k-tiles in flight at once and R fetched with them: one
    // memory round trip per step of the chain
    wg_gemm<DK, CV, DK, true, false, CHAIN_PF, true>(
        [&](int c, int c2) { return ft[c * DK + c2]; }, [&](int c2, int v) { return sm.ds[c2][v]; },
        [&](int c, int v, float x, float r) { sm.ds[c][v] = x + r; }, sm.stage, tid,
        [&](int c, int v) { return rr[c * DV + v]; });
  }
  __syncthreads();
  if (dh0 != nullptr)
    for (int idx = tid; idx < DK * CV; idx += NT) {
      const int c = idx / CV, v = idx % CV;
      dh0[dh + c * DV + v0 + v] = sm.ds[c][v];
    }
}

// ---------------------------------------------------------------------------
// gradients: per (chunk, head), in parallel
// ---------------------------------------------------------------------------
// Two phases share the big LDS area: the products (X, U, dU, dX) and then
// the bilinear terms (qh, kh, G, dM, dKk).
struct GradSmem {
  union {
    struct {
      float x[CH][LD];
      float u[CH][LD];
      float du[CH][LD];
      float dx[CH][LD];
    } a;
    struct {
      float qh[CH][LD];
      float kh[CH][LD];
      float G[CH][LD];
      float dm[CH][LDM];   // dM (lower incl.)
      float dkk[CH][LDM];  // dKk (strictly lower)
    } b;
    struct {               // after the bilinear sums: dqh over G, dkh over dM, dKk
      float qh[CH][LD];
      float kh[CH][LD];
      float dqh[CH][LD];
      float dkh[CH][LD];
    } c;
  };
  float beta[CH];
  float dbeta[CH];
  float dD[DK];
  float gl[DK];          // G of the last row
  union {
    float kbsum[RG][DK];
    float part[NT / CH][CH];  // per-row-group partial sums of dbeta
  };
  float dgtot[RG][DK];        // per-row-block totals of dG
  alignas(16) float stage[STAGE_FLOATS];
};

__global__ __launch_bounds__(NT, 1) void kda_bwd_grads_kernel(
    const bf16* __restrict__ v, const float* __restrict__ beta, const bf16* __restrict__ dout,
    const ChunkDesc* __restrict__ table, const int* __restrict__ bad, int n_items, int H,
    const float* __restrict__ imgs, const float* __restrict__ states,
    const float* __restrict__ dstates, float* __restrict__ wscratch, float* __restrict__ dq,
    float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dg,
    float* __restrict__ dbeta) {
  __shared__ GradSmem sm;
  if (*bad) return;
  float* sc = wscratch + (size_t)blockIdx.x * SC_FLOATS;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int slot = item / H, h = item - slot * H;
    const ChunkDesc cd = table[slot];
    if (cd.len == 0) continue;
    const int start = cd.start, len = cd.len;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));  // lane values are recomputed per item, not kept live
    const float* img = imgs + (size_t)item * IMG_FLOATS;
    const float* S0 = states + (size_t)item * DK * DV;
    const float* dSc = dstates + (size_t)item * DK * DV;
    const float* T = img + IMG_T;
    const float* Kk = img + IMG_KK;
    const float* Mm = img + IMG_M;
    __syncthreads();
    if (tid < CH) {
      sm.beta[tid] = tid < len ? beta[(size_t)(start + tid) * H + h] : 0.f;
    }
    if (tid < DK) sm.gl[tid] = img[IMG_G + (CH - 1) * DK + tid];
    __syncthreads();
    const size_t row0 = (size_t)start * H + h;
    const float* ikh = img + IMG_KH;
    const float* iG = img + IMG_G;
    // rows past the chunk read the last row, then select zero (no branch
    // around the loads)
    auto dO = [&](int r, int c) -> float {
      const float x = bf16_to_f32(dout[(row0 + (size_t)min(r, len - 1) * H) * DV + c]);
      return r < len ? x : 0.f;
    };
    auto Vv = [&](int r, int c) -> float {
      const float x = bf16_to_f32(v[(row0 + (size_t)min(r, len - 1) * H) * DV + c]);
      return r < len ? x : 0.f;
    };
    // ---- phase A: the products, X, U, dU, dX in LDS
    // X = V - Kt S0
    wg_gemm<CH, DV, DK, true, false, 4, true>(
        [&](int t, int c) { return ikh[t * DK + c] * __expf(iG[t * DK + c]); },
        [&](int c, int vv) { return S0[c * DV + vv]; },
        [&](int t, int vv, float x, float vt) { sm.a.x[t][vv] = vt - x; }, sm.stage, tid,
        [&](int t, int vv) { return Vv(t, vv); });
    // U = Tb X
    wg_gemm<CH, DV, CH, true, false, 4>(
        [&](int t, int i) { return T[t * CH + i] * sm.beta[i]; },
        [&](int i, int vv) { return sm.a.x[i][vv]; },
        [&](int t, int vv, float x, float) { sm.a.u[t][vv] = x; }, sm.stage, tid);
    // dU = scale M^T dO + Kbar dSc
    wg_gemm<CH, DV, CH, false, false, 4>(
        [&](int t, int r) { return SCALE * Mm[r * CH + t]; },
        [&](int r, int vv) { return dO(r, vv); },
        [&](int t, int vv, float x, float) { sm.a.du[t][vv] = x; }, sm.stage, tid);
    wg_gemm<CH, DV, DK, true, false, 4>(
        [&](int t, int c) { return ikh[t * DK + c] * __expf(sm.gl[c] - iG[t * DK + c]); },
        [&](int c, int vv) { return dSc[c * DV + vv]; },
        [&](int t, int vv, float x, float prev) { sm.a.du[t][vv] = prev + x; }, sm.stage, tid,
        [&](int t, int vv) { return sm.a.du[t][vv]; });
    // dX = Tb^T dU  (= dV)
    wg_gemm<CH, DV, CH, false, false, 4>(
        [&](int t, int r) { return T[r * CH + t] * sm.beta[t]; },
        [&](int r, int vv) { return sm.a.du[r][vv]; },
        [&](int t, int vv, float x, float) {
          sm.a.dx[t][vv] = x;
          if (t < len) dv[(row0 + (size_t)t * H) * DV + vv] = x;
        },
        sm.stage, tid);
    // dQt = scale dO S0^T (rows 0..63 of SC_DQK) and dKt = -dX S0^T (rows
    // 64..127) as one product: S0 is streamed once for both
    wg_gemm<2 * CH, DK, DV, true, true, 4>(
        [&](int t, int vv) {
          const float a = SCALE * dO(min(t, CH - 1), vv), b = -sm.a.dx[t & (CH - 1)][vv];
          return t < CH ? a : b;
        },
        [&](int vv, int c) { return S0[c * DV + vv]; },
        [&](int t, int c, float x, float) { sc[SC_DQK + t * DK + c] = x; }, sm.stage, tid);
    // dKbar = U dSc^T
    wg_gemm<CH, DK, DV, true, true, 4>(
        [&](int t, int vv) { return sm.a.u[t][vv]; },
        [&](int vv, int c) { return dSc[c * DV + vv]; },
        [&](int t, int c, float x, float) { sc[SC_DKB + t * DK + c] = x; }, sm.stage, tid);
    // dM = scale tril(dO U^T), straight into its phase-B place (over dX, which
    // no product reads any more)
    wg_gemm<CH, CH, DV, true, true, 4>(
        [&](int r, int vv) { return SCALE * dO(r, vv); },
        [&](int vv, int i) { return sm.a.u[i][vv]; },
        [&](int r, int i, float x, float) { sm.b.dm[r][i] = i <= r ? x : 0.f; }, sm.stage, tid);
    // dTb = tril(dU X^T), over U (read last by the product above); Z below goes
    // over X.  Both are read before phase B writes qh and kh over them.
    float (*const dtb)[LDM] = reinterpret_cast<float (*)[LDM]>(&sm.a.u[0][0]);
    float (*const zb)[LDM] = reinterpret_cast<float (*)[LDM]>(&sm.a.x[0][0]);
    static_assert(CH * LDM <= CH * LD, "a [64][64] tile fits in a [64][128] one");
    wg_gemm<CH, CH, DV, true, true, 4>(
        [&](int r, int vv) { return sm.a.du[r][vv]; },
        [&](int vv, int i) { return sm.a.x[i][vv]; },
        [&](int r, int i, float x, float) { dtb[r][i] = i <= r ? x : 0.f; }, sm.stage, tid);
    // ---- phase A's products are done: X, dU, dX are free, U holds dTb
    // dD[c] = sum_v dSc[c][v] S0[c][v] (32 threads per row, 16-byte loads);
    // dbeta_i = sum_r dTb_ri T_ri (both lower: the sum runs over all rows, in 8
    // row groups of 8 combined through LDS)
    {
      constexpr int P = DK * DV / 4 / NT;
      float4 a4[P], b4[P];
#pragma unroll
      for (int j = 0; j < P; ++j) {
        a4[j] = *reinterpret_cast<const float4*>(dSc + 4 * (tid + NT * j));
        b4[j] = *reinterpret_cast<const float4*>(S0 + 4 * (tid + NT * j));
      }
      const int i = tid & (CH - 1), part = tid / CH;
      float tv[8], dv8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        tv[j] = T[(8 * part + j) * CH + i];
        dv8[j] = dtb[8 * part + j][i];
      }
#pragma unroll
      for (int j = 0; j < P; ++j) {
        float acc = fmaf(a4[j].x, b4[j].x, fmaf(a4[j].y, b4[j].y, fmaf(a4[j].z, b4[j].z, a4[j].w * b4[j].w)));
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) acc += __shfl_xor(acc, o);
        if ((tid & 31) == 0) sm.dD[(tid >> 5) + (NT / 32) * j] = acc;
      }
      float db = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) db = fmaf(dv8[j], tv[j], db);
      sm.part[part][i] = db;
      __syncthreads();
      if (tid < CH) {
        float s = 0.f;
#pragma unroll
        for (int p = 0; p < NT / CH; ++p) s += sm.part[p][tid];
        sm.dbeta[tid] = s;
      }
    }
    // Z = (dTb Diag(beta)) T^T;  dA = -T^T Z (strictly lower)
    wg_gemm<CH, CH, CH, true, true, 4>(
        [&](int r, int m) { return dtb[r][m] * sm.beta[m]; },
        [&](int m, int i) { return T[i * CH + m]; },
        [&](int r, int i, float x, float) { zb[r][i] = x; }, sm.stage, tid);
    wg_gemm<CH, CH, CH, false, false, 4>(
        [&](int r, int m) { return -T[m * CH + r]; },
        [&](int m, int i) { return zb[m][i]; },
        [&](int r, int i, float x, float) { sm.b.dkk[r][i] = i < r ? x : 0.f; }, sm.stage, tid);
    // ---- phase B: qh, kh, G of the image into LDS (16-byte vectors, all
    // loads first; dM is in place already)
    {
      constexpr int PV = CH * DK / 4 / NT;  // float4 per thread per tile
      float4 vq[PV], vk[PV], vg[PV];
#pragma unroll
      for (int j = 0; j < PV; ++j) {
        const int e = 4 * (tid + NT * j);
        vq[j] = *reinterpret_cast<const float4*>(img + IMG_QH + e);
        vk[j] = *reinterpret_cast<const float4*>(img + IMG_KH + e);
        vg[j] = *reinterpret_cast<const float4*>(img + IMG_G + e);
      }
#pragma unroll
      for (int j = 0; j < PV; ++j) {
        const int e = 4 * (tid + NT * j), r = e >> 7, c = e & 127;
        const float q4[4] = {vq[j].x, vq[j].y, vq[j].z, vq[j].w};
        const float k4[4] = {vk[j].x, vk[j].y, vk[j].z, vk[j].w};
        const float g4[4] = {vg[j].x, vg[j].y, vg[j].z, vg[j].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          sm.b.qh[r][c + u] = q4[u];
          sm.b.kh[r][c + u] = k4[u];
          sm.b.G[r][c + u] = g4[u];
        }
      }
    }
    // dbeta_r += sum_i dA_ri Kk_ri (both strictly lower: all i, 8 threads per row)
    {
      const int r = tid / 8, i0 = 8 * (tid % 8);
      const float4 ka = *reinterpret_cast<const float4*>(Kk + r * CH + i0);
      const float4 kb = *reinterpret_cast<const float4*>(Kk + r * CH + i0 + 4);
      const float kv8[8] = {ka.x, ka.y, ka.z, ka.w, kb.x, kb.y, kb.z, kb.w};
      float db = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) db = fmaf(sm.b.dkk[r][i0 + j], kv8[j], db);
      db += __shfl_xor(db, 1);
      db += __shfl_xor(db, 2);
      db += __shfl_xor(db, 4);
      if (tid % 8 == 0) sm.dbeta[r] += db;
    }
    __syncthreads();
    // dKk = Diag(beta) dA
    for (int idx = tid; idx < CH * CH; idx += NT) {
      const int r = idx >> 6, i = idx & 63;
      sm.b.dkk[r][i] *= sm.beta[r];
    }
    if (tid < CH && tid < len) dbeta[row0 + (size_t)tid * H] = sm.dbeta[tid];
    __syncthreads();
    // Bilinear forms of M and Kk, for (r, c):
    //   Sa1 = sum_{i <= r} dM_ri kh_ic E_ric,  Sa2 = sum_{i < r} dKk_ri kh_ic E_ric,
    //   Sb  = sum_{rr >= r} (dM_rr,r qh_rr,c + dKk_rr,r kh_rr,c) E_rr,r,c
    // with E_ric = exp(G_rc - G_ic), then combined with the decayed tiles into
    // dqh, dkh and dG.  Thread (block bb, channel c) owns rows 16 bb .. 16 bb + 15
    // of channel c and keeps their sums in registers; bb is uniform over a
    // wave, so the in-block rows of dM and dKk it reads are broadcasts.
    static_assert(NT == 4 * DK, "one thread per (16-row block, channel)");
    asm volatile("" : "+v"(tid));  // lane values from here on are recomputed, not kept live
    const int bb = __builtin_amdgcn_readfirstlane(tid / DK), c = tid % DK, r0 = 16 * bb;
    float sa1[16], sa2[16], sb[16];
    // pairs inside the block: one exp per pair i <= r serves Sa1, Sa2 of row r
    // and Sb of row i
    {
      float Gv[16], kv[16], qv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        Gv[j] = sm.b.G[r0 + j][c];
        kv[j] = sm.b.kh[r0 + j][c];
        qv[j] = sm.b.qh[r0 + j][c];
        sa1[j] = sa2[j] = sb[j] = 0.f;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
#pragma unroll
        for (int i = 0; i <= r; ++i) {
          const float e = __expf(Gv[r] - Gv[i]);  // <= 1
          const float dmri = sm.b.dm[r0 + r][r0 + i], dkri = sm.b.dkk[r0 + r][r0 + i];
          const float ki = kv[i] * e;
          sa1[r] = fmaf(dmri, ki, sa1[r]);
          sa2[r] = fmaf(dkri, ki, sa2[r]);
          sb[i] = fmaf(fmaf(dmri, qv[r], dkri * kv[r]), e, sb[i]);
        }
      }
    }
    // Pairs across blocks, on fp32 MFMA (16x16x4).  The wave's rows are block
    // BB (uniform over the wave; the code is written per BB at compile time) and
    // its channels CW .. CW + 63, four 16-channel tiles.  In the MFMA C layout
    // lane l = 16 g + j holds rows 4 g + i (i = 0..3) of the block for channel
    // CW + 16 t + j of tile t; k-step s pairs lane group g with k = 4 g + s on
    // both operands.
    //   Sa1, Sa2 from column block b < BB: the decay splits at rho = G of the
    //   last row of block b; A = the (BB, b) block of dM / dKk, B = kh_i
    //   exp(rho - G_i) <= 1, the product scaled by exp(G_r - rho) <= 1.
    //   Sb from row blocks a > BB: the decay splits at rho = G of the last row of
    //   block BB; A = the (a, BB) block of dM / dKk transposed, B = qh_r | kh_r
    //   exp(G_r - rho) <= 1, the sum scaled by exp(rho - G_i) <= 1.
    // The sums then move to the thread layout through a per-wave slice of the
    // staging area (unused in this phase).
    {
      const int l = tid & 63, g = l >> 4, j = l & 15;
      const int CW = c - l;  // first channel of the wave
      static_assert(NW * 2 * 16 * 17 <= STAGE_FLOATS, "per-wave slices fit the staging area");
      float* xp = sm.stage + (tid >> 6) * (2 * 16 * 17);  // this wave's slice
      // C layout -> thread layout: dst[r] += x of (row r, channel c)
      auto to_rows = [&](const f32x4 (&x)[4], float (&dst)[16]) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          wave_sync_lds();
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) xp[(tt * 16 + 4 * g + i) * 17 + j] = x[2 * h + tt][i];
          wave_sync_lds();
          if ((l >> 5) == h) {
            const int tt = (l >> 4) & 1;
#pragma unroll
            for (int r = 0; r < 16; ++r) dst[r] += xp[(tt * 16 + r) * 17 + j];
          }
        }
      };
      auto cross = [&](auto bconst) {
        constexpr int BB = decltype(bconst)::value, R0 = 16 * BB;
        float Gc[4][4];  // G of the C layout's rows and channels
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) Gc[t][i] = sm.b.G[R0 + 4 * g + i][CW + 16 * t + j];
        if (BB > 0) {
          f32x4 acc1[4], acc2[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) acc1[t] = acc2[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int b = 0; b < BB; ++b) {
            const float4 am = *reinterpret_cast<const float4*>(&sm.b.dm[R0 + j][16 * b + 4 * g]);
            const float4 ak = *reinterpret_cast<const float4*>(&sm.b.dkk[R0 + j][16 * b + 4 * g]);
            const float amv[4] = {am.x, am.y, am.z, am.w}, akv[4] = {ak.x, ak.y, ak.z, ak.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int cc = CW + 16 * t + j;
              const float rho = sm.b.G[16 * b + 15][cc];
              f32x4 p1 = {0.f, 0.f, 0.f, 0.f}, p2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int s2 = 0; s2 < 4; ++s2) {
                const int ri = 16 * b + 4 * g + s2;
                const float kb = sm.b.kh[ri][cc] * __expf(rho - sm.b.G[ri][cc]);
                p1 = mfma16f(amv[s2], kb, p1);
                p2 = mfma16f(akv[s2], kb, p2);
              }
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float e = __expf(Gc[t][i] - rho);
                acc1[t][i] = fmaf(e, p1[i], acc1[t][i]);
                acc2[t][i] = fmaf(e, p2[i], acc2[t][i]);
              }
            }
          }
          to_rows(acc1, sa1);
          to_rows(acc2, sa2);
        }
        if (BB < 3) {
          f32x4 acc3[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) acc3[t] = f32x4{0.f, 0.f, 0.f, 0.f};
          float rho[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) rho[t] = sm.b.G[R0 + 15][CW + 16 * t + j];
#pragma unroll
          for (int a2 = BB + 1; a2 < 4; ++a2) {
            float amv[4], akv[4];
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
              amv[s2] = sm.b.dm[16 * a2 + 4 * g + s2][R0 + j];
              akv[s2] = sm.b.dkk[16 * a2 + 4 * g + s2][R0 + j];
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int cc = CW + 16 * t + j;
#pragma unroll
              for (int s2 = 0; s2 < 4; ++s2) {
                const int rr = 16 * a2 + 4 * g + s2;
                const float e = __expf(sm.b.G[rr][cc] - rho[t]);
                acc3[t] = mfma16f(amv[s2], sm.b.qh[rr][cc] * e, acc3[t]);
                acc3[t] = mfma16f(akv[s2], sm.b.kh[rr][cc] * e, acc3[t]);
              }
            }
          }
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc3[t][i] *= __expf(rho[t] - Gc[t][i]);
          to_rows(acc3, sb);
        }
      };
      if (bb == 0) cross(std::integral_constant<int, 0>());
      else if (bb == 1) cross(std::integral_constant<int, 1>());
      else if (bb == 2) cross(std::integral_constant<int, 2>());
      else cross(std::integral_constant<int, 3>());
    }
    float Gv[16], kv[16], qv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      Gv[j] = sm.b.G[r0 + j][c];
      kv[j] = sm.b.kh[r0 + j][c];
      qv[j] = sm.b.qh[r0 + j][c];
    }
    // combine with the decayed tiles (Qt = qh e^G, Kt = -kh e^G, Kbar = kh e^{G_last - G}):
    // dqh, dkh and dG of the thread's rows; dG is summed from the last row up
    const float gl = sm.gl[c];
    float dqt[16], dkt[16], dkb[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      dqt[j] = sc[SC_DQK + (r0 + j) * DK + c];
      dkt[j] = sc[SC_DQK + (CH + r0 + j) * DK + c];
      dkb[j] = sc[SC_DKB + (r0 + j) * DK + c];
    }
    float dqh[16], dkh[16], kbs = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float eg = __expf(Gv[j]), eb = __expf(gl - Gv[j]);
      const float qr = qv[j], kr = kv[j];
      kbs = fmaf(dkb[j], kr * eb, kbs);
      dqh[j] = sa1[j] + dqt[j] * eg;
      dkh[j] = sa2[j] + sb[j] + dkt[j] * eg + dkb[j] * eb;
      // dG, kept in sa1
      sa1[j] = qr * sa1[j] + kr * sa2[j] - kr * sb[j] + dqt[j] * qr * eg + dkt[j] * kr * eg - dkb[j] * kr * eb;
    }
#pragma unroll
    for (int j = 14; j >= 0; --j) sa1[j] += sa1[j + 1];
    __syncthreads();  // G, dM and dKk are read by every thread until here
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      sm.c.dqh[r0 + j][c] = dqh[j];
      sm.c.dkh[r0 + j][c] = dkh[j];
    }
    sm.kbsum[bb][c] = kbs;
    sm.dgtot[bb][c] = sa1[0];
    __syncthreads();
    // dg = reverse cumsum of dG within the chunk; the last row also gains
    // sum_r dKbar_r Kbar_r + dD D (G_last is the cumsum up to the last token)
    {
      float base = sm.dD[c] * __expf(gl);
#pragma unroll
      for (int g2 = 0; g2 < RG; ++g2) base += sm.kbsum[g2][c];
#pragma unroll
      for (int g2 = 1; g2 < RG; ++g2)
        if (g2 > bb) base += sm.dgtot[g2][c];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (r0 + j < len) dg[(row0 + (size_t)(r0 + j) * H) * DK + c] = base + sa1[j];
    }
    // l2 norms: dq = rq (dqh - qh (qh . dqh)), dk likewise; TPT threads per token
    {
      const int t = tid / TPT, c0 = CPT * (tid % TPT);
#pragma unroll 1
      for (int which = 0; which < 2; ++which) {
        const float (*dxh)[LD] = which == 0 ? sm.c.dqh : sm.c.dkh;
        const float (*xh)[LD] = which == 0 ? sm.c.qh : sm.c.kh;
        float sdot = 0.f;
#pragma unroll
        for (int j = 0; j < CPT; ++j) sdot = fmaf(xh[t][c0 + j], dxh[t][c0 + j], sdot);
#pragma unroll
        for (int o = 1; o < TPT; o <<= 1) sdot += __shfl_xor(sdot, o);
        if (t < len) {
          const float rn = img[(which == 0 ? IMG_RQ : IMG_RK) + t];
          float* dst = (which == 0 ? dq : dk) + (row0 + (size_t)t * H) * DK;
#pragma unroll
          for (int j = 0; j < CPT; ++j) dst[c0 + j] = rn * (dxh[t][c0 + j] - xh[t][c0 + j] * sdot);
        }
      }
    }
  }
}

__global__ void kda_bwd_nan_kernel(const int* __restrict__ bad, float* dq, float* dk, float* dv,
                                   float* dg, float* dbeta, float* dh0, size_t n_tok_ch,
                                   size_t n_tok, size_t n_state) {
  if (!*bad) return;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const float nan = __builtin_nanf("");
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_tok_ch; i += stride) {
    dq[i] = nan;
    dk[i] = nan;
    dv[i] = nan;
    dg[i] = nan;
  }
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_tok; i += stride) dbeta[i] = nan;
  if (dh0 != nullptr)
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_state; i += stride) dh0[i] = nan;
}

// cu_seqlens of documents b0 .. b0 + n - 1, rebased to start at token 0
__global__ void kda_cu_rebase_kernel(const int32_t* __restrict__ cu, int b0, int n,
                                     int32_t* __restrict__ out) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i <= n; i += gridDim.x * blockDim.x)
    out[i] = cu[b0 + i] - cu[b0];
}

}  // namespace

namespace {

// Ceiling of one pass's workspace: a call whose workspace would exceed it runs
// over consecutive groups of whole documents (documents are independent),
// each group's workspace within it.
constexpr size_t BWD_WS_LIMIT_DEFAULT = (size_t)16 << 30;
std::atomic<size_t> g_bwd_ws_limit{BWD_WS_LIMIT_DEFAULT};

// One backward pass over n_docs documents: the caller's cu_seqlens as given
// (cu_b0 < 0), or documents cu_b0 .. cu_b0 + n_docs - 1 of it, whose token
// tensors and states the caller has offset (their cu_seqlens entries are
// rebased into the workspace).
int bwd_run(const void* q, const void* k, const void* v, const float* g, const float* beta,
            const int32_t* cu_seqlens, int cu_b0, int32_t n_docs, int64_t T, int32_t H,
            float gate_bound, const float* initial_state, const void* d_out,
            const float* d_final_state, float* dq, float* dk, float* dv, float* dg, float* dbeta,
            float* d_initial_state, int num_cu, int* status_word, hipStream_t stream) {
  using kda_host::fail;
  // workspace: bad | table | order | states | dstates | images | F^T | R | prep scratch |
  //            grads scratch | o [| rebased cu_seqlens]
  const int grid = num_cu;
  kda_check::BwdLayout lay;
  if (!kda_check::bwd_layout(T, H, n_docs, grid, sizeof(ChunkDesc), IMG_FLOATS, SP_FLOATS, SC_FLOATS, &lay))
    return fail(KDA_ERR_BAD_SHAPE, "workspace size overflows");
  const size_t n_slots = lay.n_slots;
  const size_t items = lay.items;
  const size_t off_cu = (lay.bytes + 255) & ~(size_t)255;
  const size_t off = cu_b0 >= 0 ? off_cu + 4 * ((size_t)n_docs + 1) : lay.bytes;
  uint8_t* ws = nullptr;
  if (kda_host::alloc_async(reinterpret_cast<void**>(&ws), off, stream) != hipSuccess || !ws)
    return fail(KDA_ERR_ALLOC, "hipMallocAsync of the backward workspace failed");
  int* bad = reinterpret_cast<int*>(ws);
  ChunkDesc* table = reinterpret_cast<ChunkDesc*>(ws + lay.off_table);
  int* order = reinterpret_cast<int*>(ws + lay.off_order);
  float* states = reinterpret_cast<float*>(ws + lay.off_states);
  float* dstates = reinterpret_cast<float*>(ws + lay.off_dstates);
  float* imgs = reinterpret_cast<float*>(ws + lay.off_img);
  float* fts = reinterpret_cast<float*>(ws + lay.off_ft);
  float* rs = reinterpret_cast<float*>(ws + lay.off_r);
  float* sc = reinterpret_cast<float*>(ws + lay.off_sc);
  void* o_scratch = ws + lay.off_o;

  int rc = KDA_OK;
  hipError_t e = hipSuccess;
  if (cu_b0 >= 0) {
    int32_t* cu_b = reinterpret_cast<int32_t*>(ws + off_cu);
    hipLaunchKernelGGL(kda_cu_rebase_kernel, dim3((n_docs + 256) / 256), dim3(256), 0, stream,
                       cu_seqlens, cu_b0, (int)n_docs, cu_b);
    e = hipGetLastError();
    cu_seqlens = cu_b;
  }
  if (e == hipSuccess) {
    hipLaunchKernelGGL(kda_bwd_setup_kernel, dim3(1), dim3(1024), 0, stream, cu_seqlens, (int)n_docs,
                       (int)T, (int)n_slots, table, order, bad, status_word);
    e = hipGetLastError();
  }
  if (e == hipSuccess && T > 0) {
    rc = kda_host::forward_with_chunk_states(q, k, v, g, beta, cu_seqlens, n_docs, T, H,
                                             gate_bound, initial_state, o_scratch, states, stream);
    if (rc == KDA_OK && T > 0) {
      hipLaunchKernelGGL(kda_bwd_prep_kernel, dim3(grid), dim3(NT), 0, stream,
                         static_cast<const bf16*>(q), static_cast<const bf16*>(k), g, beta,
                         static_cast<const bf16*>(d_out), table, bad, (int)items, (int)H, imgs, fts,
                         rs);
      e = hipGetLastError();
    }
  }
  if (e == hipSuccess && rc == KDA_OK) {
    hipLaunchKernelGGL(kda_bwd_chain_kernel, dim3(n_docs * H * (DV / CV)), dim3(NT), 0, stream,
                       cu_seqlens, (int)T, (int)H, bad, order, fts, rs, d_final_state, dstates,
                       d_initial_state);
    e = hipGetLastError();
  }
  if (e == hipSuccess && rc == KDA_OK && T > 0) {
    hipLaunchKernelGGL(kda_bwd_grads_kernel, dim3(grid), dim3(NT), 0, stream,
                       static_cast<const bf16*>(v), beta, static_cast<const bf16*>(d_out), table,
                       bad, (int)items, (int)H, imgs, states, dstates, sc, dq, dk, dv, dg, dbeta);
    e = hipGetLastError();
  }
  if (e == hipSuccess && rc == KDA_OK) {
    hipLaunchKernelGGL(kda_bwd_nan_kernel, dim3(grid), dim3(NT), 0, stream, bad, dq, dk, dv, dg,
                       dbeta, d_initial_state, (size_t)T * H * DK, (size_t)T * H,
                       (size_t)n_docs * H * DK * DV);
    e = hipGetLastError();
  }
  const hipError_t ef = hipFreeAsync(ws, stream);
  if (rc != KDA_OK) return rc;
  if (e != hipSuccess) return fail(KDA_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  if (ef != hipSuccess) return fail(KDA_ERR_HIP, "hipFreeAsync of the backward workspace failed");
  return KDA_OK;
}

// A cu_seqlens the host found broken: the setup kernel flags it on the device
// (as a single pass would) and the NaN kernel fills every gradient output.
int bwd_reject(const int32_t* cu_seqlens, int32_t n_docs, int64_t T, int32_t H, float* dq,
               float* dk, float* dv, float* dg, float* dbeta, float* d_initial_state, int num_cu,
               int* status_word, hipStream_t stream) {
  using kda_host::fail;
  const size_t n_slots = (size_t)T / KDA_CHUNK + (size_t)n_docs + 1;
  const size_t off_table = 256, off_order = off_table + n_slots * sizeof(ChunkDesc);
  const size_t bytes = off_order + 4 * (size_t)n_docs;
  uint8_t* ws = nullptr;
  if (kda_host::alloc_async(reinterpret_cast<void**>(&ws), bytes, stream) != hipSuccess || !ws)
    return fail(KDA_ERR_ALLOC, "hipMallocAsync of the backward workspace failed");
  int* bad = reinterpret_cast<int*>(ws);
  hipLaunchKernelGGL(kda_bwd_setup_kernel, dim3(1), dim3(1024), 0, stream, cu_seqlens, (int)n_docs,
                     (int)T, (int)n_slots, reinterpret_cast<ChunkDesc*>(ws + off_table),
                     reinterpret_cast<int*>(ws + off_order), bad, status_word);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) {
    hipLaunchKernelGGL(kda_bwd_nan_kernel, dim3(num_cu), dim3(NT), 0, stream, bad, dq, dk, dv, dg,
                       dbeta, d_initial_state, (size_t)T * H * DK, (size_t)T * H,
                       (size_t)n_docs * H * DK * DV);
    e = hipGetLastError();
  }
  const hipError_t ef = hipFreeAsync(ws, stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  if (ef != hipSuccess) return fail(KDA_ERR_HIP, "hipFreeAsync of the backward workspace failed");
  return KDA_OK;
}

}  // namespace

extern "C" int kda_chunk_bwd(const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const int32_t* cu_seqlens, int32_t n_docs,
                             int64_t T, int32_t H, int32_t chunk, float gate_bound,
                             const float* initial_state, const void* d_out,
                             const float* d_final_state, float* dq, float* dk, float* dv,
                             float* dg, float* dbeta, float* d_initial_state, hipStream_t stream) {
  using kda_host::fail;
  fail(KDA_OK, "");
  const kda_check::Result r =
      kda_check::chunk_bwd(q, k, v, g, beta, cu_seqlens, n_docs, T, H, chunk, gate_bound,
                           initial_state, d_out, d_final_state, dq, dk, dv, dg, dbeta,
                           d_initial_state);
  if (r.code != KDA_OK) return fail(r.code, r.msg);
  if (kda_check::bwd_is_noop(T, d_initial_state)) return KDA_OK;

  int num_cu = 0;
  int* status_word = nullptr;
  if (kda_host::device(&num_cu, &status_word) != 0)
    return fail(KDA_ERR_HIP, "device query (CU count, status word) failed");

  kda_check::BwdLayout lay;
  if (!kda_check::bwd_layout(T, H, n_docs, num_cu, sizeof(ChunkDesc), IMG_FLOATS, SP_FLOATS, SC_FLOATS, &lay))
    return fail(KDA_ERR_BAD_SHAPE, "workspace size overflows");
  const size_t limit = g_bwd_ws_limit.load(std::memory_order_relaxed);
  if (lay.bytes <= limit || cu_seqlens == nullptr || n_docs == 1)
    return bwd_run(q, k, v, g, beta, cu_seqlens, -1, n_docs, T, H, gate_bound, initial_state, d_out,
                   d_final_state, dq, dk, dv, dg, dbeta, d_initial_state, num_cu, status_word, stream);

  // Too large for one pass: the document boundaries on the host (this waits
  // for the stream), then consecutive groups of documents.
  std::vector<int32_t> cu((size_t)n_docs + 1);
  if (hipMemcpyAsync(cu.data(), cu_seqlens, sizeof(int32_t) * cu.size(), hipMemcpyDeviceToHost, stream) !=
          hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return fail(KDA_ERR_HIP, "reading cu_seqlens for the batched backward failed");
  bool ok = cu[0] == 0 && cu[n_docs] == T;
  for (int32_t i = 1; ok && i <= n_docs; ++i) ok = cu[i] >= cu[i - 1] && cu[i] <= T;
  if (!ok)
    return bwd_reject(cu_seqlens, n_docs, T, H, dq, dk, dv, dg, dbeta, d_initial_state, num_cu,
                      status_word, stream);
  const size_t tok = (size_t)H * DK, st = (size_t)H * DK * DV;
  for (int32_t b0 = 0; b0 < n_docs;) {
    int32_t b1 = b0 + 1;  // at least one document per pass
    for (; b1 < n_docs; ++b1) {
      kda_check::BwdLayout l2;
      if (!kda_check::bwd_layout((int64_t)cu[b1 + 1] - cu[b0], H, b1 + 1 - b0, num_cu, sizeof(ChunkDesc),
                                 IMG_FLOATS, SP_FLOATS, SC_FLOATS, &l2) ||
          l2.bytes > limit)
        break;
    }
    const size_t t0 = (size_t)cu[b0];
    const int rc = bwd_run(
        static_cast<const bf16*>(q) + t0 * tok, static_cast<const bf16*>(k) + t0 * tok,
        static_cast<const bf16*>(v) + t0 * tok, g + t0 * tok, beta + t0 * H, cu_seqlens, b0, b1 - b0,
        (int64_t)cu[b1] - cu[b0], H, gate_bound, initial_state ? initial_state + b0 * st : nullptr,
        static_cast<const bf16*>(d_out) + t0 * tok, d_final_state ? d_final_state + b0 * st : nullptr,
        dq + t0 * tok, dk + t0 * tok, dv + t0 * tok, dg + t0 * tok, dbeta + t0 * H,
        d_initial_state ? d_initial_state + b0 * st : nullptr, num_cu, status_word, stream);
    if (rc != KDA_OK) return rc;
    b0 = b1;
  }
  return KDA_OK;
}

extern "C" uint64_t kda_debug_set_bwd_workspace_limit(uint64_t bytes) {
  return g_bwd_ws_limit.exchange(bytes == 0 ? BWD_WS_LIMIT_DEFAULT : (size_t)bytes);
}
