// gdn_stream_copy: a plain device-to-device copy, one 16-byte load and one
// 16-byte store per thread, used as the measured bandwidth ceiling of the
// streaming kernels.  The KBench `comba_decode_step` page (perf_md) asks for
// the roofline of a bandwidth-bound step to come from a large stream copy on
// the machine at hand rather than from a datasheet figure; the decode step
// moves its state the same way (non-temporal 16-byte loads and stores, every
// byte touched once), so this copy is the fair comparison.

#include "gdn_device.h"
#include "gdn_host.h"

namespace gdn {
namespace {

constexpr int kCopyThreads = 128;

__global__ __launch_bounds__(kCopyThreads) void gdn_copy_kernel(const float* __restrict__ src,
                                                                float* __restrict__ dst,
                                                                size_t n4) {
  const size_t i = static_cast<size_t>(blockIdx.x) * kCopyThreads + threadIdx.x;
  if (i < n4) store_stream(dst + 4 * i, load_stream(src + 4 * i));
}

}  // namespace
}  // namespace gdn

extern "C" int gdn_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  using namespace gdn;
  if (bytes == 0) return GDN_OK;
  if (!src || !dst) return GDN_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst)) return GDN_ERR_ALIGN;
  if (bytes % 16 != 0) return GDN_ERR_SHAPE;
  if (overlaps(src, bytes, dst, bytes)) return GDN_ERR_ALIAS;
  const size_t n4 = bytes / 16;
  const size_t blocks = (n4 + kCopyThreads - 1) / kCopyThreads;
  if (blocks > 0x7fffffffull) return GDN_ERR_UNSUPPORTED;  // one launch's grid
  (void)hipGetLastError();
  hipLaunchKernelGGL(gdn_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kCopyThreads), 0, stream,
                     static_cast<const float*>(src), static_cast<float*>(dst), n4);
  return launch_status();
}
