// Gate: g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b).
// Elementwise over [T][Hv]; the backward's per-head token sums (dA_log,
// ddt_bias) go through per-block partials added in a fixed order.
#include "common.h"
#include "launch.h"

namespace gdn {

__device__ __forceinline__ float softplusf_(float x) {
  // log(1 + e^x) = max(x, 0) + log1p(e^-|x|): no overflow, no threshold
  return fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x)));
}

template <typename T>
__global__ void gate_fwd_kernel(const T* __restrict__ a, const T* __restrict__ b,
                                const float* __restrict__ A_log, const float* __restrict__ dt_bias,
                                int64_t n, int H, float* __restrict__ g, float* __restrict__ beta) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    int h = (int)(i % H);
    float xa = to_f(a[i]) + dt_bias[h];
    g[i] = -__expf(A_log[h]) * softplusf_(xa);
    beta[i] = sigmoidf_(to_f(b[i]));
  }
}

// Block = 256 threads covering GATE_TB tokens x all heads: thread (lt, h) with
// h = tid % H, lt = tid / H walks tokens lt, lt + nl, ...  Per-head partial
// sums are combined over lt in LDS in order.
template <typename T>
__global__ void __launch_bounds__(256) gate_bwd_kernel(
    const T* __restrict__ a, const T* __restrict__ b, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, const float* __restrict__ dg,
    const float* __restrict__ dbeta, int64_t T_tok, int H, T* __restrict__ da, T* __restrict__ db,
    float* __restrict__ partials) {
  __shared__ float sA[256], sD[256];
  const int tid = threadIdx.x;
  const int nl = 256 / H;
  const int h = tid % H, lt = tid / H;
  const int64_t t0 = (int64_t)blockIdx.x * GATE_TB;
  const int64_t t1 = t0 + GATE_TB < T_tok ? t0 + GATE_TB : T_tok;
  float accA = 0.f, accD = 0.f;
  if (lt < nl) {
    const float Aneg = -__expf(A_log[h]);
    const float bias = dt_bias[h];
    for (int64_t t = t0 + lt; t < t1; t += nl) {
      const int64_t i = t * H + h;
      float xa = to_f(a[i]) + bias;
      float gv = Aneg * softplusf_(xa);
      float dgi = dg[i];
      float dxa = dgi * Aneg * sigmoidf_(xa);
      da[i] = from_f<T>(dxa);
      accD += dxa;
      accA += dgi * gv;  // g is linear in exp(A_log): dg/dA_log = g
      float bt = sigmoidf_(to_f(b[i]));
      db[i] = from_f<T>(dbeta[i] * bt * (1.f - bt));
    }
  }
  sA[tid] = accA;
  sD[tid] = accD;
  __syncthreads();
  if (tid < H) {
    float pa = 0.f, pd = 0.f;
    for (int l = 0; l < nl; ++l) {
      pa += sA[l * H + tid];
      pd += sD[l * H + tid];
    }
    partials[(int64_t)blockIdx.x * 2 * H + tid] = pa;
    partials[(int64_t)blockIdx.x * 2 * H + H + tid] = pd;
  }
}

hipError_t launch_gate_fwd(const gdn_shape& s, const void* a, const void* b, const float* A_log,
                           const float* dt_bias, float* g, float* beta, hipStream_t st) {
  const int64_t n = s.total_tokens * s.hv;
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (s.dtype == GDN_BF16)
    hipLaunchKernelGGL(gate_fwd_kernel<bf16>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const bf16*)a, (const bf16*)b, A_log, dt_bias, n, s.hv, g, beta);
  else if (s.dtype == GDN_FP16)
    hipLaunchKernelGGL(gate_fwd_kernel<fp16>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const fp16*)a, (const fp16*)b, A_log, dt_bias, n, s.hv, g, beta);
  else
    hipLaunchKernelGGL(gate_fwd_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const float*)a, (const float*)b, A_log, dt_bias, n, s.hv, g, beta);
  return hipGetLastError();
}

hipError_t launch_gate_bwd(const gdn_shape& s, const void* a, const void* b, const float* A_log,
                           const float* dt_bias, const float* dg, const float* dbeta, void* da,
                           void* db, float* dA_log, float* ddt_bias, float* partials,
                           hipStream_t st) {
  const int64_t np = gate_partials(s.total_tokens);
  if (np > 0) {
    if (s.dtype == GDN_BF16)
      hipLaunchKernelGGL(gate_bwd_kernel<bf16>, dim3((unsigned)np), dim3(256), 0, st,
                         (const bf16*)a, (const bf16*)b, A_log, dt_bias, dg, dbeta, s.total_tokens,
                         s.hv, (bf16*)da, (bf16*)db, partials);
    else if (s.dtype == GDN_FP16)
      hipLaunchKernelGGL(gate_bwd_kernel<fp16>, dim3((unsigned)np), dim3(256), 0, st,
                         (const fp16*)a, (const fp16*)b, A_log, dt_bias, dg, dbeta, s.total_tokens,
                         s.hv, (fp16*)da, (fp16*)db, partials);
    else
      hipLaunchKernelGGL(gate_bwd_kernel<float>, dim3((unsigned)np), dim3(256), 0, st,
                         (const float*)a, (const float*)b, A_log, dt_bias, dg, dbeta,
                         s.total_tokens, s.hv, (float*)da, (float*)db, partials);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_reduce_partials(partials, np, 2 * (int64_t)s.hv, dA_log, s.hv, ddt_bias, st);
}

}  // namespace gdn
