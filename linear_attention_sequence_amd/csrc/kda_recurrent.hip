// kda_recurrent.hip -- token-recurrent form of the KDA forward (decode and
// short documents).
//
// Same operator as kda_chunk_fwd_state (include/kda.h): per document and head
// a K x V fp32 state, for every token in order
//
//     S  <- Diag(exp g_t) S;   S <- S + beta_t kh_t (v_t - S^T kh_t)^T;
//     o_t = 128**-0.5 S^T qh_t
//
// computed one token at a time instead of in chunks: the recurrent mode of
// the KDA functions that the K3 model selects by sequence length (page
// "nemo_automodel.components.models.kimi_k3.kda_fused", package docstring:
// the fused path is the chunk mode; page "kimi_k3.model": the mode option).
//
// Every value column of S evolves on its own: column c needs only S[:, c],
// v_t[c] and the shared vectors kh_t, qh_t, exp(g_t).  So one lane owns one
// column (128 fp32 in VGPRs), a wave owns 64 columns, and a (document, head)
// unit is two single-wave workgroups with no communication between them.
// Per token a wave l2-normalises q_t and k_t itself (two elements per lane),
// puts kh, qh * scale and exp(g) into its own LDS slice, and every lane reads
// them back as broadcasts.  The state is read once (from initial_state or
// zero) and written once (to final_state), 256 contiguous bytes per wave
// instruction; for a one-token document (decode) that traffic is the cost.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "kda.h"

#include "kda_host_checks.h"

namespace kda_host {
int fail(int code, const std::string& msg);
int device(int* num_cu, int** status_word);
hipError_t alloc_async(void** p, size_t bytes, hipStream_t stream);
}  // namespace kda_host

namespace {

constexpr int DK = 128;
constexpr int DV = 128;
constexpr int CHECK_THREADS = 256;
constexpr float L2_EPS = 1e-6f;
typedef __bf16 bf16;

// cu_seqlens holds exactly n_docs + 1 entries: 0, non-decreasing, ending at T.
// One workgroup; writes the outcome of the check to *bad (0 or 1) and the sticky flag.
__global__ __launch_bounds__(CHECK_THREADS) void kda_recurrent_check_kernel(
    const int32_t* __restrict__ cu, int n_docs, int T, int* __restrict__ bad,
    int* __restrict__ status_word) {
  __shared__ int s_bad;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  if (cu != nullptr) {
    for (int i = threadIdx.x; i <= n_docs; i += CHECK_THREADS) {
      const int val = cu[i];
      bool b = (i == 0) ? (val != 0) : (val < cu[i - 1] || val > T);
      if (i == n_docs && val != T) b = true;
      if (b) atomicOr(&s_bad, 1);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    *bad = s_bad;
    if (s_bad) atomicOr(status_word, KDA_DEV_BAD_CU_SEQLENS);
  }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// One wave = value columns 64 * half .. + 63 of one (document, head) unit.
__global__ __launch_bounds__(64, 2) void kda_recurrent_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
    int T, int H, const float* __restrict__ h0, float* __restrict__ ht, bf16* __restrict__ out,
    int n_docs, const int* __restrict__ bad) {
  __shared__ float4 vec[3][DK / 4];  // kh, qh * scale, exp(g) of the current token
  const int lane = threadIdx.x;
  const int unit = blockIdx.x >> 1;
  const int col = 64 * (blockIdx.x & 1) + lane;
  const int d = unit / H;
  const int h = unit - d * H;

  if (*bad) {
    // cu_seqlens broke its contract: make the failure visible
    const size_t stride = (size_t)gridDim.x * 64;
    unsigned short* o16 = reinterpret_cast<unsigned short*>(out);
    for (size_t i = (size_t)blockIdx.x * 64 + lane; i < (size_t)T * H * DV; i += stride) o16[i] = 0x7FC0;
    if (ht != nullptr)
      for (size_t i = (size_t)blockIdx.x * 64 + lane; i < (size_t)n_docs * H * DK * DV; i += stride)
        ht[i] = __builtin_nanf("");
    return;
  }
  const int a = cu ? cu[d] : 0;
  const int b = cu ? cu[d + 1] : T;
  const size_t sbase = ((size_t)d * H + h) * DK * DV + col;

  float S[DK];
  if (h0 != nullptr) {
#pragma unroll
    for (int r = 0; r < DK; ++r) S[r] = h0[sbase + (size_t)r * DV];
  } else {
#pragma unroll
    for (int r = 0; r < DK; ++r) S[r] = 0.f;
  }

  const float scale = 0.08838834764831845f;  // 128^-1/2
  float* vflat = reinterpret_cast<float*>(&vec[0][0]);
  for (int t = a; t < b; ++t) {
    const size_t row = (size_t)t * H + h;
    // lane holds channels 2 lane, 2 lane + 1 of q, k, g
    const uint32_t qq = reinterpret_cast<const uint32_t*>(q + row * DK)[lane];
    const uint32_t kk = reinterpret_cast<const uint32_t*>(k + row * DK)[lane];
    const float2 gg = reinterpret_cast<const float2*>(g + row * DK)[lane];
    const float vc = (float)v[row * DV + col];
    const float bt = beta[row];
    const float q0 = __uint_as_float(qq << 16), q1 = __uint_as_float(qq & 0xFFFF0000u);
    const float k0 = __uint_as_float(kk << 16), k1 = __uint_as_float(kk & 0xFFFF0000u);
    const float rq = 1.f / sqrtf(wave_sum(q0 * q0 + q1 * q1) + L2_EPS);
    const float rk = 1.f / sqrtf(wave_sum(k0 * k0 + k1 * k1) + L2_EPS);
    __syncthreads();  // the previous token's vectors have been read
    vflat[2 * lane] = k0 * rk;
    vflat[2 * lane + 1] = k1 * rk;
    vflat[DK + 2 * lane] = q0 * rq * scale;
    vflat[DK + 2 * lane + 1] = q1 * rq * scale;
    vflat[2 * DK + 2 * lane] = expf(gg.x);
    vflat[2 * DK + 2 * lane + 1] = expf(gg.y);
    __syncthreads();
    // decay, then the prediction S^T kh (four partial sums)
    float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r4 = 0; r4 < DK / 4; ++r4) {
      const float4 kd = vec[0][r4];
      const float4 dd = vec[2][r4];
      const float kv[4] = {kd.x, kd.y, kd.z, kd.w};
      const float dv[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        S[4 * r4 + j] *= dv[j];
        p[j] = fmaf(kv[j], S[4 * r4 + j], p[j]);
      }
      // keep the broadcast reads close to their use (S already takes 128 VGPRs)
      if (r4 % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
    const float u = bt * (vc - ((p[0] + p[1]) + (p[2] + p[3])));
    // write, then the output S^T qh scale
    float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r4 = 0; r4 < DK / 4; ++r4) {
      const float4 kd = vec[0][r4];
      const float4 qd = vec[1][r4];
      const float kv[4] = {kd.x, kd.y, kd.z, kd.w};
      const float qv[4] = {qd.x, qd.y, qd.z, qd.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        S[4 * r4 + j] = fmaf(kv[j], u, S[4 * r4 + j]);
        o[j] = fmaf(qv[j], S[4 * r4 + j], o[j]);
      }
      if (r4 % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
    out[row * DV + col] = (bf16)((o[0] + o[1]) + (o[2] + o[3]));
  }

  if (ht != nullptr) {
#pragma unroll
    for (int r = 0; r < DK; ++r) ht[sbase + (size_t)r * DV] = S[r];
  }
}

}  // namespace

extern "C" int kda_recurrent_fwd(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const int32_t* cu_seqlens, int32_t n_docs,
                                 int64_t T, int32_t H, const float* initial_state,
                                 float* final_state, void* out, hipStream_t stream) {
  using kda_host::fail;
  fail(KDA_OK, "");
  const kda_check::Result r = kda_check::recurrent_fwd(q, k, v, g, beta, cu_seqlens, n_docs, T, H,
                                                       initial_state, final_state, out);
  if (r.code != KDA_OK) return fail(r.code, r.msg);
  if (kda_check::fwd_is_noop(T, final_state)) return KDA_OK;

  int num_cu = 0;
  int* status_word = nullptr;
  if (kda_host::device(&num_cu, &status_word) != 0)
    return fail(KDA_ERR_HIP, "device query (CU count, status word) failed");
  int* bad = nullptr;
  if (kda_host::alloc_async(reinterpret_cast<void**>(&bad), 256, stream) != hipSuccess || !bad)
    return fail(KDA_ERR_ALLOC, "hipMallocAsync of the workspace failed");
  hipLaunchKernelGGL(kda_recurrent_check_kernel, dim3(1), dim3(CHECK_THREADS), 0, stream,
                     cu_seqlens, (int)n_docs, (int)T, bad, status_word);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) {
    hipLaunchKernelGGL(kda_recurrent_kernel, dim3(2 * n_docs * H), dim3(64), 0, stream,
                       static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                       static_cast<const bf16*>(v), g, beta, cu_seqlens, (int)T, (int)H,
                       initial_state, final_state, static_cast<bf16*>(out), (int)n_docs, bad);
    e = hipGetLastError();
  }
  const hipError_t ef = hipFreeAsync(bad, stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  if (ef != hipSuccess) return fail(KDA_ERR_HIP, "hipFreeAsync of the workspace failed");
  return KDA_OK;
}
