// comba_decode_step: one Comba token (gated delta rule with a decoupled read
// key) for a dense batch.
//
// Math (KBench `comba_decode_step` spec, spec_md): for each (b, h) slice
// S [K, V] (V contiguous), gate a = exp(g):
//   u_j = beta (v_j - sum_i p_i a S[i,j]),  S'[i,j] = a S[i,j] + k_i u_j,
//   o_j = sum_i (scale q_i) S'[i,j].
//
// Design (gfx950, HBM-bound): the reductions run down K, across rows, so a
// workgroup (256 threads) holds the whole K x V slice in registers: a row of
// V floats is V/4 lanes x float4, the 256/(V/4) row groups each own K/RG
// consecutive rows.  One pass computes, per lane, partial column sums of
// p_i S[i,:] and (scale q_i) S[i,:] over its rows (and the scalar
// sum_i scale q_i k_i); the row groups of a wave combine them with cross-lane
// adds, the waves through LDS behind one barrier.  Then u = beta (v - a Sp), o = a Sq + (scale q . k) u (the exact
// identity for the readout from the updated state), and every lane writes
// its rows a S + k_i u once.  The state crosses HBM exactly twice.

#include "gdn_device.h"
#include "gdn_host.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;

// N consecutive activations (a thread's rows of p, q or k) -> fp32: 16-byte
// vector loads when the run is a whole number of them (the run then starts
// 16-byte aligned: the slice and row offsets are multiples of it), else
// element by element.
template <typename T, int N>
__device__ __forceinline__ void load_run(const T* src, float (&out)[N]) {
  if constexpr ((N * sizeof(T)) % 16 == 0) {
    constexpr int PER = 16 / sizeof(T);
#pragma unroll
    for (int c = 0; c < N / PER; ++c) {
      const uint4 w = reinterpret_cast<const uint4*>(src)[c];
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        if constexpr (sizeof(T) == 2)
          out[c * PER + e] = (e & 1) ? __uint_as_float(u[e >> 1] & 0xffff0000u) : __uint_as_float(u[e >> 1] << 16);
        else
          out[c * PER + e] = __uint_as_float(u[e]);
      }
    }
  } else {
#pragma unroll
    for (int n = 0; n < N; ++n) out[n] = Act<T>::load(src + n);
  }
}

template <int K, int V, typename T, int NT>
__global__ __launch_bounds__(NT) void comba_decode_kernel(
    const float* state, float* state_new, const T* __restrict__ q, const T* __restrict__ k,
    const T* __restrict__ v, const T* __restrict__ p, const T* __restrict__ beta,
    const float* __restrict__ g, T* __restrict__ o, float scale) {
  constexpr int ACT = V / 4;             // float4 columns of a row
  constexpr int LPR = row_lanes(ACT);    // lanes per row (ACT rounded up to a power of two)
  constexpr int RG = NT / LPR;           // row groups
  constexpr int RPT = K / RG;            // rows per thread (consecutive)
  static_assert(K % RG == 0 && RPT >= 1 && NT % 64 == 0 && LPR <= 64, "shape");

  constexpr int WAVES = NT / 64;
  __shared__ f32x4 red_p[WAVES][LPR];
  __shared__ f32x4 red_q[WAVES][LPR];
  __shared__ float red_kq[WAVES];

  const int slice = blockIdx.x;
  const int tid = threadIdx.x;
  const int c4 = tid % LPR;
  const int rg = tid / LPR;
  const int r0 = rg * RPT;
  // Lanes past the row's ACT columns (V not a power of two) load the last
  // column again, add nothing to the sums and store nothing.
  const bool live = ACT == LPR || c4 < ACT;
  const int cc = ACT == LPR ? c4 : min(c4, ACT - 1);

  const size_t soff = static_cast<size_t>(slice) * K * V + static_cast<size_t>(r0) * V + cc * 4;
  f32x4 s[RPT];
#pragma unroll
  for (int n = 0; n < RPT; ++n) s[n] = load_stream(state + soff + static_cast<size_t>(n) * V);

  const size_t koff = static_cast<size_t>(slice) * K + r0;
  float pr[RPT], qr[RPT], kr[RPT];
  load_run<T, RPT>(p + koff, pr);
  load_run<T, RPT>(q + koff, qr);
  load_run<T, RPT>(k + koff, kr);
#pragma unroll
  for (int n = 0; n < RPT; ++n) qr[n] *= scale;
  const f32x4 vv = Act<T>::load4(v + static_cast<size_t>(slice) * V + cc * 4);
  const float gate = expf(g[slice]);
  const float bt = Act<T>::load(beta + slice);

  f32x4 sp = {0.f, 0.f, 0.f, 0.f}, sq = {0.f, 0.f, 0.f, 0.f};
  float kq = 0.f;
#pragma unroll
  for (int n = 0; n < RPT; ++n) {
    sp += pr[n] * s[n];
    sq += qr[n] * s[n];
    kq += qr[n] * kr[n];
  }
  if (!live) sp = sq = f32x4{0.f, 0.f, 0.f, 0.f};
  // Row groups of one wave first: its lanes that hold the same columns
  // differ only in the lane bits from LPR up (cross-lane adds, no LDS), then
  // one partial per wave through LDS behind the single barrier.
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1) {
    sp.x += __shfl_xor(sp.x, m);
    sp.y += __shfl_xor(sp.y, m);
    sp.z += __shfl_xor(sp.z, m);
    sp.w += __shfl_xor(sp.w, m);
    sq.x += __shfl_xor(sq.x, m);
    sq.y += __shfl_xor(sq.y, m);
    sq.z += __shfl_xor(sq.z, m);
    sq.w += __shfl_xor(sq.w, m);
    kq += __shfl_xor(kq, m);
  }
  const int wave = tid / 64, lane = tid % 64;
  if (lane < LPR) {
    red_p[wave][lane] = sp;
    red_q[wave][lane] = sq;
  }
  if (lane == 0) red_kq[wave] = kq;
  __syncthreads();
  sp = red_p[0][c4];
  sq = red_q[0][c4];
  kq = red_kq[0];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) {
    sp += red_p[w][c4];
    sq += red_q[w][c4];
    kq += red_kq[w];
  }

  const f32x4 u = bt * (vv - gate * sp);
  if (rg == 0 && live) Act<T>::store4(o + static_cast<size_t>(slice) * V + cc * 4, gate * sq + kq * u);
  if (live) {
#pragma unroll
    for (int n = 0; n < RPT; ++n)
      store_stream(state_new + soff + static_cast<size_t>(n) * V, gate * s[n] + kr[n] * u);
  }
}

template <int K, int V, typename T>
int launch_kv(const float* state, float* state_new, const void* q, const void* k,
              const void* v, const void* p, const void* beta, const float* g, void* o,
              long slices, float scale, hipStream_t stream) {
  if (slices > 0x7fffffffL) return GDN_ERR_SHAPE;
  constexpr int NT = row_lanes(V / 4) * K < kThreads ? row_lanes(V / 4) * K : kThreads;
  (void)hipGetLastError();
  hipLaunchKernelGGL((comba_decode_kernel<K, V, T, NT>), dim3(static_cast<unsigned>(slices)),
                     dim3(NT), 0, stream, state, state_new, static_cast<const T*>(q),
                     static_cast<const T*>(k), static_cast<const T*>(v),
                     static_cast<const T*>(p), static_cast<const T*>(beta), g,
                     static_cast<T*>(o), scale);
  return launch_status();
}

template <int K, typename T>
int launch_k(const float* state, float* state_new, const void* q, const void* k,
             const void* v, const void* p, const void* beta, const float* g, void* o,
             long slices, int V, float scale, hipStream_t stream) {
  // at most 32 rows (128 state registers) per thread: K * row_lanes(V / 4) <= 8192
  switch (V) {
    case 32: return launch_kv<K, 32, T>(state, state_new, q, k, v, p, beta, g, o, slices, scale, stream);
    case 64: return launch_kv<K, 64, T>(state, state_new, q, k, v, p, beta, g, o, slices, scale, stream);
    case 96: return launch_kv<K, 96, T>(state, state_new, q, k, v, p, beta, g, o, slices, scale, stream);
    case 128: return launch_kv<K, 128, T>(state, state_new, q, k, v, p, beta, g, o, slices, scale, stream);
    case 160:
    case 192:
    case 224:
    case 256:
      if constexpr (K <= 128) {
        if (V == 160) return launch_kv<K, 160, T>(state, state_new, q, k, v, p, beta, g, o, slices, scale, stream);
        if (V == 192) return launch_kv<K, 192, T>(state, state_new, q, k, v, p, beta, g, o, slices, scale, stream);
        if (V == 224) return launch_kv<K, 224, T>(state, state_new, q, k, v, p, beta, g, o, slices, scale, stream);
        return launch_kv<K, 256, T>(state, state_new, q, k, v, p, beta, g, o, slices, scale, stream);
      }
      break;
  }
  return GDN_ERR_UNSUPPORTED;
}

template <typename T>
int launch(const float* state, float* state_new, const void* q, const void* k, const void* v,
           const void* p, const void* beta, const float* g, void* o, long slices, int K, int V,
           float scale, hipStream_t stream) {
  switch (K) {
    case 32: return launch_k<32, T>(state, state_new, q, k, v, p, beta, g, o, slices, V, scale, stream);
    case 64: return launch_k<64, T>(state, state_new, q, k, v, p, beta, g, o, slices, V, scale, stream);
    case 128: return launch_k<128, T>(state, state_new, q, k, v, p, beta, g, o, slices, V, scale, stream);
    case 256: return launch_k<256, T>(state, state_new, q, k, v, p, beta, g, o, slices, V, scale, stream);
    case 96: return launch_k<96, T>(state, state_new, q, k, v, p, beta, g, o, slices, V, scale, stream);
    case 160: return launch_k<160, T>(state, state_new, q, k, v, p, beta, g, o, slices, V, scale, stream);
    case 192: return launch_k<192, T>(state, state_new, q, k, v, p, beta, g, o, slices, V, scale, stream);
    case 224: return launch_k<224, T>(state, state_new, q, k, v, p, beta, g, o, slices, V, scale, stream);
  }
  return GDN_ERR_UNSUPPORTED;
}

}  // namespace
}  // namespace gdn

extern "C" int comba_decode_step(const float* state, float* state_new, const void* q,
                                 const void* k, const void* v, const void* p,
                                 const void* beta, const float* g, void* o, int B, int H,
                                 int K, int V, float scale, gdn_dtype act,
                                 hipStream_t stream) {
  using namespace gdn;
  if (B < 0 || H < 0 || K <= 0 || V <= 0) return GDN_ERR_SHAPE;
  if (!is_act(act)) return GDN_ERR_DTYPE;
  if (!valid_head(K) || !valid_head(V) || K * row_lanes(V / 4) > 8192) return GDN_ERR_UNSUPPORTED;
  if (B == 0 || H == 0) return GDN_OK;
  if (!state || !state_new || !q || !k || !v || !p || !beta || !g || !o) return GDN_ERR_NULL;
  if (!aligned16(state) || !aligned16(state_new) || !aligned16(q) || !aligned16(k) ||
      !aligned16(p) || !aligned16(v) || !aligned16(o))
    return GDN_ERR_ALIGN;
  const size_t state_bytes = static_cast<size_t>(B) * H * K * V * sizeof(float);
  if (state_new != state && overlaps(state, state_bytes, state_new, state_bytes))
    return GDN_ERR_ALIAS;
  const size_t o_bytes = static_cast<size_t>(B) * H * V * act_bytes(act);
  if (overlaps(o, o_bytes, state_new, state_bytes) || overlaps(o, o_bytes, state, state_bytes))
    return GDN_ERR_ALIAS;
  {
    const size_t qk = static_cast<size_t>(B) * H * K * act_bytes(act);
    const size_t bh = static_cast<size_t>(B) * H;
    const Span in[] = {{q, qk}, {k, qk}, {p, qk}, {v, o_bytes}, {beta, bh * act_bytes(act)}, {g, bh * sizeof(float)}};
    const Span out[] = {{o, o_bytes}, {state_new, state_bytes}};
    if (inputs_overlap_outputs(in, out)) return GDN_ERR_ALIAS;
  }
  if (!(scale > 0.0f)) scale = 1.0f / sqrtf(static_cast<float>(K));
  const long slices = static_cast<long>(B) * H;
  if (act == GDN_BF16)
    return launch<bf16>(state, state_new, q, k, v, p, beta, g, o, slices, K, V, scale, stream);
  return launch<float>(state, state_new, q, k, v, p, beta, g, o, slices, K, V, scale, stream);
}
