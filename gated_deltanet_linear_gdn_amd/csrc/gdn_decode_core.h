// The single-token decode kernel and its launcher, shared by gdn_decode_step
// (gdn_decode.hip) and gdn_conv_decode_step (gdn_conv_decode.hip).  See
// gdn_decode.hip for the design.
#pragma once

#include <algorithm>

#include "gdn_device.h"
#include "gdn_host.h"

namespace gdn {
namespace {

constexpr int kThreads = 128;
constexpr int kRowsPerLane = 2;
// grid z holds at most this many sequences: larger batches launch in slices
constexpr int kMaxGridZ = 65535;

// T: the activations' type (q, k, v, beta); TY: y's.
template <int DK, int NV, bool FULL, typename T, typename TY = T>
__global__ __launch_bounds__(kThreads) void gdn_decode_kernel(
    const float* state_in, float* state_out, const T* __restrict__ q,
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ g,
    const T* __restrict__ beta, TY* __restrict__ y, int Hk, int Hv, int Dv,
    unsigned hk_mul) {
  constexpr int ACT = DK / 4;            // float4 columns of a row
  constexpr int LPR = row_lanes(ACT);    // lanes per row (ACT rounded up to a power of two)
  constexpr int RPS = kThreads / LPR;    // rows per register slot, whole workgroup
  constexpr int ROWS = RPS * NV;         // rows per workgroup

  // grid (part, hv, b): the same dispatch order as slice-major with parts
  // innermost, and no integer division on the way in (hk = hv / (Hv/Hk) as a
  // multiply-high by hk_mul, the host's hk_reciprocal(Hv/Hk)).
  const int part = blockIdx.x;
  const int hv = blockIdx.y;
  const int b = blockIdx.z;
  const int slice = b * Hv + hv;  // n = b * Hv + hv
  const int hk = hk_mul ? static_cast<int>(__umulhi(static_cast<unsigned>(hv), hk_mul)) : hv;
  const int tid = threadIdx.x;
  const int c4 = tid % LPR;                        // float4 column within the row
  const int row0 = part * ROWS + tid / LPR;
  // Lanes past the row's ACT columns (only when Dk is not a power of two)
  // load the last column again, count as zero in the sums, store nothing.
  const bool live = ACT == LPR || c4 < ACT;
  const int cc = ACT == LPR ? c4 : min(c4, ACT - 1);

  const size_t qk_off = (static_cast<size_t>(b) * Hk + hk) * DK + cc * 4;
  const size_t slice_off = static_cast<size_t>(slice) * Dv * DK;
  const float* sin = state_in + slice_off + cc * 4;
  float* sout = state_out + slice_off + cc * 4;
  // FULL: every row this workgroup covers exists (Dv % ROWS == 0) and the
  // body is branch-free.  Otherwise rows past Dv load the last row again
  // (a branch around a load makes it wait for the previous one) and only
  // their stores are skipped.
  auto rowc = [&](int n) { return FULL ? row0 + n * RPS : min(row0 + n * RPS, Dv - 1); };

  // Every load is issued before the first wait: the small activation loads
  // first (loads complete in issue order, so their first use does not wait
  // for the state rows), kept as stored, then the NV state rows.  Converting
  // bf16 activations right after their loads would make the compiler wait
  // for them before issuing the state loads: two memory round trips per
  // workgroup instead of one.  The barriers keep the scheduler from moving
  // any conversion (and its wait) between the loads.
  Raw4<T> kr, qr;
  kr.load(k + qk_off);
  qr.load(q + qk_off);
  const float graw = g[slice];
  const T btr = beta[slice];
  T vr[NV];
#pragma unroll
  for (int n = 0; n < NV; ++n) vr[n] = v[static_cast<size_t>(slice) * Dv + rowc(n)];
  __builtin_amdgcn_sched_barrier(0);
  f32x4 s[NV];
#pragma unroll
  for (int n = 0; n < NV; ++n) s[n] = load_stream(sin + static_cast<size_t>(rowc(n)) * DK);
  __builtin_amdgcn_sched_barrier(0);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const f32x4 kk = live ? kr.f() : zero4, qq = live ? qr.f() : zero4;
  const float bt = to_f32(btr);
  float vv[NV];
#pragma unroll
  for (int n = 0; n < NV; ++n) vv[n] = to_f32(vr[n]);
  const float gate = expf(graw);
  const float kq = group_sum<LPR>(dot4(kk, qq));

#pragma unroll
  for (int n = 0; n < NV; ++n) {
    const int row = row0 + n * RPS;
    const float sk = group_sum<LPR>(dot4(s[n], kk));
    const float sq = group_sum<LPR>(dot4(s[n], qq));
    const float d = bt * (vv[n] - gate * sk);
    const f32x4 sn = gate * s[n] + d * kk;
    if ((FULL || row < Dv) && live) {
      store_stream(sout + static_cast<size_t>(row) * DK, sn);
      if (c4 == 0) Act<TY>::store(y + static_cast<size_t>(slice) * Dv + row, gate * sq + d * kq);
    }
  }
}

template <int DK, typename T, typename TY = T>
int launch_decode_dk(const float* state_in, float* state_out, const void* q, const void* k,
                     const void* v, const float* g, const void* beta, void* y, int B, int Hk,
                     int Hv, int Dv, hipStream_t stream) {
  constexpr int NV = kRowsPerLane;
  constexpr int ROWS = kThreads / row_lanes(DK / 4) * NV;
  const int parts = (Dv + ROWS - 1) / ROWS;
  if (Hv > 65535) return GDN_ERR_SHAPE;  // grid y
  const unsigned hk_mul = hk_reciprocal(Hv / Hk);
  const T* qa = static_cast<const T*>(q);
  const T* ka = static_cast<const T*>(k);
  const T* va = static_cast<const T*>(v);
  const T* ba = static_cast<const T*>(beta);
  TY* ya = static_cast<TY*>(y);
  (void)hipGetLastError();
  for (int b0 = 0; b0 < B; b0 += kMaxGridZ) {
    const int nb = std::min(B - b0, kMaxGridZ);
    const size_t sv = static_cast<size_t>(b0) * Hv;  // value-head slices before this one
    const size_t sk = static_cast<size_t>(b0) * Hk * DK;
    const dim3 grid(static_cast<unsigned>(parts), static_cast<unsigned>(Hv), static_cast<unsigned>(nb));
    if (Dv % ROWS == 0)
      hipLaunchKernelGGL((gdn_decode_kernel<DK, NV, true, T, TY>), grid, dim3(kThreads), 0, stream,
                         state_in + sv * Dv * DK, state_out + sv * Dv * DK, qa + sk, ka + sk,
                         va + sv * Dv, g + sv, ba + sv, ya + sv * Dv, Hk, Hv, Dv, hk_mul);
    else
      hipLaunchKernelGGL((gdn_decode_kernel<DK, NV, false, T, TY>), grid, dim3(kThreads), 0, stream,
                         state_in + sv * Dv * DK, state_out + sv * Dv * DK, qa + sk, ka + sk,
                         va + sv * Dv, g + sv, ba + sv, ya + sv * Dv, Hk, Hv, Dv, hk_mul);
  }
  return launch_status();
}

}  // namespace
}  // namespace gdn
