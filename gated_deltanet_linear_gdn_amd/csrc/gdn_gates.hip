// gdn_prefill_gates: per-token log-gate and beta of a prefill batch.
//
// Math (pymllm `gdn_chunkwise` docs, `gdn_extend_chunkwise` parameters a, b,
// A_log, dt_bias; formulas from the regolith `gdn.metal` header comment):
//   g[t,h]    = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h])   (log-space)
//   beta[t,h] = 1 / (1 + exp(-b[t,h]))
// (gates_of in gdn_device.h).  Elementwise and HBM-bound (a few bytes per
// token and head); one thread per element, grid-stride.

#include "gdn_device.h"
#include "gdn_host.h"

namespace gdn {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void gdn_gates_kernel(
    const T* __restrict__ a, const T* __restrict__ b, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, float* __restrict__ g, float* __restrict__ beta,
    long n, int Hv) {
  const long stride = static_cast<long>(gridDim.x) * blockDim.x;
  for (long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int h = static_cast<int>(i % Hv);
    gates_of(Act<T>::load(a + i) + dt_bias[h], A_log[h], Act<T>::load(b + i), g[i], beta[i]);
  }
}

template <typename T>
int launch(const void* a, const void* b, const float* A_log, const float* dt_bias, float* g,
           float* beta, long n, int Hv, hipStream_t stream) {
  const long want = (n + 255) / 256;
  const unsigned blocks = static_cast<unsigned>(want < 65536 ? want : 65536);
  (void)hipGetLastError();
  hipLaunchKernelGGL((gdn_gates_kernel<T>), dim3(blocks), dim3(256), 0, stream,
                     static_cast<const T*>(a), static_cast<const T*>(b), A_log, dt_bias, g, beta,
                     n, Hv);
  return launch_status();
}

}  // namespace
}  // namespace gdn

extern "C" int gdn_prefill_gates(const void* a, const void* b, const float* A_log,
                                 const float* dt_bias, float* g, float* beta, int64_t T_tot,
                                 int Hv, gdn_dtype act, hipStream_t stream) {
  using namespace gdn;
  if (T_tot < 0 || Hv <= 0) return GDN_ERR_SHAPE;
  if (!is_act(act)) return GDN_ERR_DTYPE;
  if (T_tot == 0) return GDN_OK;
  if (!a || !b || !A_log || !dt_bias || !g || !beta) return GDN_ERR_NULL;
  const long n = static_cast<long>(T_tot) * Hv;
  const size_t nb = static_cast<size_t>(n) * sizeof(float);
  if (overlaps(g, nb, beta, nb)) return GDN_ERR_ALIAS;
  if (act == GDN_BF16) return launch<bf16>(a, b, A_log, dt_bias, g, beta, n, Hv, stream);
  return launch<float>(a, b, A_log, dt_bias, g, beta, n, Hv, stream);
}

extern "C" const char* gdn_status_string(int status) {
  switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: a size is negative or inconsistent";
    case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE: unknown activation dtype";
    case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: a pointer is not 16-byte aligned";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: head or chunk size not built";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
    case GDN_ERR_LAUNCH: return "GDN_ERR_LAUNCH: kernel launch failed";
    case GDN_ERR_DEVICE: return "GDN_ERR_DEVICE: no usable HIP device";
    case GDN_ERR_ALIAS: return "GDN_ERR_ALIAS: buffers overlap";
  }
  return "GDN_ERR_UNKNOWN";
}
