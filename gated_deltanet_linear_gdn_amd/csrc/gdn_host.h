// Host-side helpers for the libgdn C ABI: argument checks and launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool is_act(gdn_dtype act) { return act == GDN_F32 || act == GDN_BF16; }

inline size_t act_bytes(gdn_dtype act) { return act == GDN_BF16 ? 2 : 4; }

// True when [a, a+na) and [b, b+nb) share a byte.
inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

// A buffer as (address, bytes).
struct Span {
  const void* p;
  size_t n;
};

// True when a buffer that is only read shares a byte with one that is
// written (kernels read inputs while other workgroups write outputs).
template <int NI, int NO>
inline bool inputs_overlap_outputs(const Span (&in)[NI], const Span (&out)[NO]) {
  for (int i = 0; i < NI; ++i)
    for (int o = 0; o < NO; ++o)
      if (overlaps(in[i].p, in[i].n, out[o].p, out[o].n)) return true;
  return false;
}

// ceil(2^32 / G) for the decode kernels' multiply-high hk = hv / G; 0 for
// G == 1, whose reciprocal does not fit 32 bits.  Exact for every hv < 2^16:
// the reciprocal's rounding error m*G - 2^32 is below G <= 2^16.
inline unsigned hk_reciprocal(int G) {
  return G == 1 ? 0u : static_cast<unsigned>(((1ull << 32) + G - 1) / static_cast<unsigned>(G));
}

inline bool pow2_head(int d) { return d == 32 || d == 64 || d == 128 || d == 256; }

// Head sizes of the streaming kernels: a multiple of 32 up to 256.
inline bool valid_head(int d) { return d >= 32 && d <= 256 && d % 32 == 0; }

// The gated RMS norm epilogue (gdn_layer.hip), also used by the prefill
// when a value head spans several chunk-loop workgroups.
int gated_rmsnorm_launch(const void* o, const void* z, const float* gamma, float eps, long rows,
                         int Dv, void* y, gdn_dtype act, hipStream_t stream);

// Status of the launch just enqueued.
inline int launch_status() {
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

}  // namespace gdn
