// The layer steps on either side of the recurrence (regolith `gdn.metal`,
// header comment and the conv/SiLU and output blocks of its kernel):
//
// gdn_conv_silu: the 4-tap causal convolution + SiLU of the q, k and v
//   channels of each token, with a rolling history of the last three inputs
//   per pool slot (oldest first), over packed variable-length sequences; a
//   decode step is the case of one token per sequence.  For channel c of a
//   sequence's token t, with the inputs before the sequence's first token
//   taken from the slot's history:
//     pre = x[t-3] W[c][0] + x[t-2] W[c][1] + x[t-1] W[c][2] + x[t] W[c][3]
//     out = pre / (1 + exp(-pre))
//   and the slot's history becomes the newest three of (history, inputs).
//   Two kernels on the caller's stream: the outputs (which read the old
//   history) and then the history update, so the in-place update needs no
//   ordering inside a kernel.
//
// gdn_gated_rmsnorm: y = o / sqrt(mean(o^2) + eps) * gamma * sigmoid(z) per
//   (token, value head) over its Dv outputs, gamma [Dv] shared by the heads.
//
// Both are elementwise-shaped and HBM-bound: 16-byte vector accesses along
// the contiguous channel axis, fp32 arithmetic.

#include "gdn_device.h"
#include "gdn_host.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8;  // channels per thread (16 bytes of bf16)

// Eight consecutive activations <-> fp32.
template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
  static __device__ __forceinline__ void load(const bf16* p, float (&x)[8]) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(u[i] << 16);
      x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
  // round to nearest even, two values per v_cvt_pk_bf16_f32
  static __device__ __forceinline__ void store(bf16* p, const float (&x)[8]) {
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 lo = static_cast<__bf16>(x[2 * i]), hi = static_cast<__bf16>(x[2 * i + 1]);
      u[i] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
    }
    *reinterpret_cast<uint4*>(p) = uint4{u[0], u[1], u[2], u[3]};
  }
};
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float (&x)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float (&x)[8]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
  }
};

// One input row of kVec channels kept as loaded (packed for bf16).
template <typename T> struct Row8;
template <> struct Row8<bf16> {
  uint32_t w[4];
  __device__ __forceinline__ void load(const bf16* p) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  }
  __device__ __forceinline__ float get(int i) const {
    return (i & 1) ? __uint_as_float(w[i >> 1] & 0xffff0000u) : __uint_as_float(w[i >> 1] << 16);
  }
};
template <> struct Row8<float> {
  float f[8];
  __device__ __forceinline__ void load(const float* p) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  __device__ __forceinline__ float get(int i) const { return f[i]; }
};

// e[k] for a run-time k in 0..2 without indexing a register array.
__device__ __forceinline__ float pick3(const float (&e)[3], int k) {
  return k == 0 ? e[0] : (k == 1 ? e[1] : e[2]);
}


// Sequence bounds clamped to [0, T): out-of-contract entries never index
// outside the buffers.
__device__ __forceinline__ void seq_range(const int64_t* cu, int s, int64_t T, int64_t& t0, int64_t& t1) {
  t0 = cu[s];
  t1 = cu[s + 1];
  t0 = t0 < 0 ? 0 : (t0 > T ? T : t0);
  t1 = t1 < t0 ? t0 : (t1 > T ? T : t1);
}

// Largest s with cu[s] <= t (the sequence holding token t when it is not
// empty).  Wave-uniform arguments, so this runs on scalar loads.
__device__ __forceinline__ int seq_of(const int64_t* cu, int N_s, int64_t t) {
  int lo = 0, hi = N_s;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// The 3 history entries of kVec channels: 24 consecutive floats, 16-byte
// aligned (C is a multiple of 8), as six 16-byte accesses.
struct Hist8 {
  float h[kVec][3];
  __device__ __forceinline__ void load(const float* p) {
    f32x4 a[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) a[i] = *reinterpret_cast<const f32x4*>(p + 4 * i);
#pragma unroll
    for (int e = 0; e < 24; ++e) h[e / 3][e % 3] = a[e / 4][e % 4];
  }
  __device__ __forceinline__ void store(float* p) const {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      f32x4 a;
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = h[(4 * i + e) / 3][(4 * i + e) % 3];
      *reinterpret_cast<f32x4*>(p + 4 * i) = a;
    }
  }
};

// Outputs for the TT tokens of one tile x kVec channels per thread.  The
// tile's input rows and the three before it are loaded up front; window
// entries before a sequence's first token come from the slot's history.
// A sequence lying wholly inside the tile has all its history reads in this
// thread, which then also writes its new history; the history of every
// other sequence is written by gdn_conv_history_kernel after this kernel.
template <typename T, int TT>
__global__ __launch_bounds__(kThreads) void gdn_conv_silu_kernel(
    const T* __restrict__ x, const float* __restrict__ W, float* __restrict__ hist,
    int64_t pool_size, const int64_t* __restrict__ cache_indices, const int64_t* __restrict__ cu,
    int N_s, int64_t T_tot, int C, int Cq, int Cv, int gx, T* __restrict__ q, T* __restrict__ k,
    T* __restrict__ v) {
  constexpr int R = TT + 3;  // rows ts-3 .. ts+TT-1
  const int tile = blockIdx.x / gx;
  const int c0 = ((blockIdx.x - tile * gx) * kThreads + threadIdx.x) * kVec;
  if (c0 >= C) return;
  const int64_t ts = static_cast<int64_t>(tile) * TT;
  const int64_t te = ts + TT < T_tot ? ts + TT : T_tot;

  // output row: q, k ([T, Cq]) or v ([T, Cv]) and the channel inside it
  T* orow;
  int oc, ostride;
  if (c0 < Cq) { orow = q; oc = c0; ostride = Cq; }
  else if (c0 < 2 * Cq) { orow = k; oc = c0 - Cq; ostride = Cq; }
  else { orow = v; oc = c0 - 2 * Cq; ostride = Cv; }

  int s = seq_of(cu, N_s, ts);
  int64_t t0, t1;
  seq_range(cu, s, T_tot, t0, t1);
  float w4[kVec][4];
#pragma unroll
  for (int i = 0; i < kVec; ++i) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(W + static_cast<size_t>(c0 + i) * 4);
    w4[i][0] = a.x; w4[i][1] = a.y; w4[i][2] = a.z; w4[i][3] = a.w;
  }
  if (te == ts + TT && t0 <= ts - 3 && t1 >= te) {
    // the common case: a full tile inside one sequence whose windows never
    // reach its history -- straight-line loads, products and stores
    Row8<T> rr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rr[r].load(x + static_cast<size_t>(ts - 3 + r) * C + c0);
    // every row load is issued before the first use (loads complete in order)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < TT; ++j) {
      float out[kVec];
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        float pre = rr[j].get(i) * w4[i][0];
        pre = fmaf(rr[j + 1].get(i), w4[i][1], pre);
        pre = fmaf(rr[j + 2].get(i), w4[i][2], pre);
        pre = fmaf(rr[j + 3].get(i), w4[i][3], pre);
        out[i] = silu_fast(pre);
      }
      Vec8<T>::store(orow + static_cast<size_t>(ts + j) * ostride + oc, out);
    }
    return;
  }
  // rows any window of this tile reads start at max(first sequence start, ts-3)
  const int64_t lo = t0 > ts - 3 ? t0 : ts - 3;
  Row8<T> rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t p = ts - 3 + r;
    if (p >= lo && p < te) rows[r].load(x + static_cast<size_t>(p) * C + c0);
  }

  Hist8 hs;      // the current sequence's old history (when it is needed)
  int hs_seq = -1;
#pragma clang loop unroll(full)
  for (int j = 0; j < TT; ++j) {
    const int64_t t = ts + j;
    while (t < te && t >= t1 && s + 1 < N_s) {  // next sequence holding t
      ++s;
      seq_range(cu, s, T_tot, t0, t1);
    }
    // (no token past the tile, none outside every sequence)
    if (t < te && t >= t0 && t < t1) {
      const int64_t slot = cache_indices[s];
      const bool slot_ok = slot >= 0 && slot < pool_size;
      const bool need_hist = t - 3 < t0;
      if (need_hist && hs_seq != s) {
        if (slot_ok) {
          hs.load(hist + (static_cast<size_t>(slot) * C + c0) * 3);
        } else {
#pragma unroll
          for (int i = 0; i < kVec; ++i) hs.h[i][0] = hs.h[i][1] = hs.h[i][2] = 0.f;
        }
        hs_seq = s;
      }
      float out[kVec];
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        float win[3];
#pragma unroll
        for (int m = 0; m < 3; ++m) {  // position t-3+m
          const int64_t p = t - 3 + m;
          win[m] = p >= t0 ? rows[j + m].get(i) : pick3(hs.h[i], static_cast<int>(p - t0 + 3));
        }
        float pre = win[0] * w4[i][0];
        pre = fmaf(win[1], w4[i][1], pre);
        pre = fmaf(win[2], w4[i][2], pre);
        pre = fmaf(rows[j + 3].get(i), w4[i][3], pre);
        out[i] = silu_fast(pre);
      }
      Vec8<T>::store(orow + static_cast<size_t>(t) * ostride + oc, out);
      // the whole sequence lies in this tile: its new history, from here
      if (t == t1 - 1 && t0 >= ts && slot_ok) {
        Hist8 nw;
#pragma unroll
        for (int m = 0; m < 3; ++m) {  // position t1-3+m = t-2+m
          const int64_t p = t - 2 + m;
#pragma unroll
          for (int i = 0; i < kVec; ++i)
            nw.h[i][m] = p >= t0 ? rows[j + 1 + m].get(i) : pick3(hs.h[i], static_cast<int>(p - t0 + 3));
        }
        nw.store(hist + (static_cast<size_t>(slot) * C + c0) * 3);
      }
    }
  }
}

// New history per (sequence, channel group) for the sequences that span
// more than one tile of TT tokens: the newest three of (old history, the
// sequence's inputs).  Runs after the outputs kernel.
template <typename T>
__global__ __launch_bounds__(kThreads) void gdn_conv_history_kernel(
    const T* __restrict__ x, float* __restrict__ hist, int64_t pool_size,
    const int64_t* __restrict__ cache_indices, const int64_t* __restrict__ cu, int N_s,
    int64_t T_tot, int C, int gx, int TT) {
  const int s = blockIdx.x / gx;
  const int c0 = ((blockIdx.x - s * gx) * kThreads + threadIdx.x) * kVec;
  if (c0 >= C || s >= N_s) return;
  int64_t t0, t1;
  seq_range(cu, s, T_tot, t0, t1);
  const int64_t slot = cache_indices[s];
  if (t1 == t0 || slot < 0 || slot >= pool_size) return;
  if (t0 / TT == (t1 - 1) / TT) return;  // written by the outputs kernel
  float* h = hist + (static_cast<size_t>(slot) * C + c0) * 3;
  Hist8 old, nw;
  old.load(h);
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    const int64_t p = t1 - 3 + m;
    if (p >= t0) {
      float r[kVec];
      Vec8<T>::load(x + static_cast<size_t>(p) * C + c0, r);
#pragma unroll
      for (int i = 0; i < kVec; ++i) nw.h[i][m] = r[i];
    } else {
#pragma unroll
      for (int i = 0; i < kVec; ++i) nw.h[i][m] = pick3(old.h[i], static_cast<int>(p - t0 + 3));
    }
  }
  nw.store(h);
}

template <typename T, int TT>
int launch_conv_tt(const void* x, const float* W, float* hist, int64_t pool_size, const int64_t* ci,
                   const int64_t* cu, int N_s, int64_t T_tot, int C, int Cq, int Cv, void* q, void* k,
                   void* v, hipStream_t stream) {
  const int gx = (C / kVec + kThreads - 1) / kThreads;  // workgroups per token row
  const int64_t tiles = (T_tot + TT - 1) / TT;
  if (tiles * gx > 0x7fffffff || static_cast<int64_t>(N_s) * gx > 0x7fffffff) return GDN_ERR_SHAPE;
  (void)hipGetLastError();
  hipLaunchKernelGGL((gdn_conv_silu_kernel<T, TT>), dim3(static_cast<unsigned>(tiles * gx)), dim3(kThreads), 0,
                     stream, static_cast<const T*>(x), W, hist, pool_size, ci, cu, N_s, T_tot, C, Cq, Cv, gx,
                     static_cast<T*>(q), static_cast<T*>(k), static_cast<T*>(v));
  if (launch_status() != GDN_OK) return GDN_ERR_LAUNCH;
  hipLaunchKernelGGL((gdn_conv_history_kernel<T>), dim3(static_cast<unsigned>(static_cast<int64_t>(N_s) * gx)),
                     dim3(kThreads), 0, stream, static_cast<const T*>(x), hist, pool_size, ci, cu, N_s, T_tot,
                     C, gx, TT);
  return launch_status();
}

template <typename T>
int launch_conv(const void* x, const float* W, float* hist, int64_t pool_size, const int64_t* ci,
                const int64_t* cu, int N_s, int64_t T_tot, int C, int Cq, int Cv, void* q, void* k,
                void* v, hipStream_t stream) {
  // a few tokens per thread amortise the weight loads; one keeps small
  // (decode-sized) batches spread over the CUs
  if (T_tot >= 8192)
    return launch_conv_tt<T, sizeof(T) == 2 ? 16 : 8>(x, W, hist, pool_size, ci, cu, N_s, T_tot, C, Cq, Cv, q, k,
                                                       v, stream);
  if (T_tot >= 2048)
    return launch_conv_tt<T, 4>(x, W, hist, pool_size, ci, cu, N_s, T_tot, C, Cq, Cv, q, k, v, stream);
  return launch_conv_tt<T, 1>(x, W, hist, pool_size, ci, cu, N_s, T_tot, C, Cq, Cv, q, k, v, stream);
}

// ------------------------------------------------------------ gated RMS norm

// G = Dv/8 lanes per row, 8 values per lane; a workgroup takes RPT groups
// of kThreads/G rows, and each lane issues the loads of its RPT rows before
// using any of them.
constexpr int kNormRPT = 4;

template <typename T, int G>
__global__ __launch_bounds__(kThreads) void gdn_gated_rmsnorm_kernel(
    const T* o, const T* __restrict__ z, const float* __restrict__ gamma, float eps, long rows,
    T* y) {
  constexpr int RPB = kThreads / G;  // rows per group
  const int lane_in_row = threadIdx.x % G;
  const f32x4 g0 = *reinterpret_cast<const f32x4*>(gamma + lane_in_row * kVec);
  const f32x4 g1 = *reinterpret_cast<const f32x4*>(gamma + lane_in_row * kVec + 4);
  const float gm[kVec] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
  float ov[kNormRPT][kVec], zv[kNormRPT][kVec];
  size_t base[kNormRPT];
  bool ok[kNormRPT];
#pragma unroll
  for (int u = 0; u < kNormRPT; ++u) {
    const long row = (static_cast<long>(blockIdx.x) * kNormRPT + u) * RPB + threadIdx.x / G;
    ok[u] = row < rows;
    const long r = ok[u] ? row : rows - 1;  // idle lanes repeat the last row (not stored)
    base[u] = static_cast<size_t>(r) * (G * kVec) + lane_in_row * kVec;
    Vec8<T>::load(o + base[u], ov[u]);
    Vec8<T>::load(z + base[u], zv[u]);
  }
#pragma unroll
  for (int u = 0; u < kNormRPT; ++u) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < kVec; ++i) ss = fmaf(ov[u][i], ov[u][i], ss);
    ss = group_sum<G>(ss);
    const float rs = __builtin_amdgcn_rsqf(ss * (1.0f / static_cast<float>(G * kVec)) + eps);
    float out[kVec];
#pragma unroll
    for (int i = 0; i < kVec; ++i) out[i] = ov[u][i] * rs * gm[i] * sigmoid_fast(zv[u][i]);
    if (ok[u]) Vec8<T>::store(y + base[u], out);
  }
}

template <typename T, int G>
int launch_norm_g(const void* o, const void* z, const float* gamma, float eps, long rows, void* y,
                  hipStream_t stream) {
  constexpr long RPW = static_cast<long>(kThreads / G) * kNormRPT;  // rows per workgroup
  const long blocks = (rows + RPW - 1) / RPW;
  if (blocks > 0x7fffffffL) return GDN_ERR_SHAPE;
  (void)hipGetLastError();
  hipLaunchKernelGGL((gdn_gated_rmsnorm_kernel<T, G>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                     0, stream, static_cast<const T*>(o), static_cast<const T*>(z), gamma, eps, rows,
                     static_cast<T*>(y));
  return launch_status();
}

template <typename T>
int launch_norm(const void* o, const void* z, const float* gamma, float eps, long rows, int Dv, void* y,
                hipStream_t stream) {
  switch (Dv) {
    case 32: return launch_norm_g<T, 4>(o, z, gamma, eps, rows, y, stream);
    case 64: return launch_norm_g<T, 8>(o, z, gamma, eps, rows, y, stream);
    case 128: return launch_norm_g<T, 16>(o, z, gamma, eps, rows, y, stream);
    case 256: return launch_norm_g<T, 32>(o, z, gamma, eps, rows, y, stream);
  }
  return GDN_ERR_UNSUPPORTED;
}

}  // namespace

int gated_rmsnorm_launch(const void* o, const void* z, const float* gamma, float eps, long rows,
                         int Dv, void* y, gdn_dtype act, hipStream_t stream) {
  if (act == GDN_BF16) return launch_norm<bf16>(o, z, gamma, eps, rows, Dv, y, stream);
  return launch_norm<float>(o, z, gamma, eps, rows, Dv, y, stream);
}

}  // namespace gdn

extern "C" int gdn_conv_silu(const void* qkv, const float* conv_w, float* conv_state,
                             int64_t pool_size, const int64_t* cache_indices,
                             const int64_t* cu_seqlens, int N_s, int64_t T_tot, int Hk, int Hv,
                             int Dk, int Dv, void* q, void* k, void* v, gdn_dtype act,
                             hipStream_t stream) {
  using namespace gdn;
  if (N_s < 0 || T_tot < 0 || pool_size < 0 || Hk <= 0 || Hv <= 0 || Dk <= 0 || Dv <= 0)
    return GDN_ERR_SHAPE;
  if (!is_act(act)) return GDN_ERR_DTYPE;
  if (Dk % kVec != 0 || Dv % kVec != 0) return GDN_ERR_UNSUPPORTED;
  const int64_t Cq64 = static_cast<int64_t>(Hk) * Dk, Cv64 = static_cast<int64_t>(Hv) * Dv;
  const int64_t C64 = 2 * Cq64 + Cv64;
  if (C64 > (int64_t{1} << 30)) return GDN_ERR_UNSUPPORTED;
  if (N_s == 0 || T_tot == 0) return GDN_OK;
  if (!qkv || !conv_w || !conv_state || !cache_indices || !cu_seqlens || !q || !k || !v)
    return GDN_ERR_NULL;
  if (!aligned16(qkv) || !aligned16(conv_w) || !aligned16(conv_state) || !aligned16(q) || !aligned16(k) ||
      !aligned16(v))
    return GDN_ERR_ALIGN;
  const size_t ab = act_bytes(act);
  const size_t xb = static_cast<size_t>(T_tot) * C64 * ab;
  const size_t qb = static_cast<size_t>(T_tot) * Cq64 * ab, vb = static_cast<size_t>(T_tot) * Cv64 * ab;
  const size_t hb = static_cast<size_t>(pool_size) * C64 * 3 * sizeof(float);
  const void* outs[3] = {q, k, v};
  const size_t ob[3] = {qb, qb, vb};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(outs[i], ob[i], qkv, xb) || overlaps(outs[i], ob[i], conv_state, hb)) return GDN_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], ob[i], outs[j], ob[j])) return GDN_ERR_ALIAS;
  }
  if (overlaps(qkv, xb, conv_state, hb)) return GDN_ERR_ALIAS;
  const int C = static_cast<int>(C64), Cq = static_cast<int>(Cq64), Cv = static_cast<int>(Cv64);
  if (act == GDN_BF16)
    return launch_conv<bf16>(qkv, conv_w, conv_state, pool_size, cache_indices, cu_seqlens, N_s, T_tot,
                             C, Cq, Cv, q, k, v, stream);
  return launch_conv<float>(qkv, conv_w, conv_state, pool_size, cache_indices, cu_seqlens, N_s, T_tot, C,
                            Cq, Cv, q, k, v, stream);
}

extern "C" int gdn_gated_rmsnorm(const void* o, const void* z, const float* gamma, float eps,
                                 void* y, int64_t T_tot, int Hv, int Dv, gdn_dtype act,
                                 hipStream_t stream) {
  using namespace gdn;
  if (T_tot < 0 || Hv <= 0 || Dv <= 0) return GDN_ERR_SHAPE;
  if (!is_act(act)) return GDN_ERR_DTYPE;
  if (!pow2_head(Dv)) return GDN_ERR_UNSUPPORTED;
  if (!(eps >= 0.0f)) return GDN_ERR_SHAPE;
  if (T_tot == 0) return GDN_OK;
  if (!o || !z || !gamma || !y) return GDN_ERR_NULL;
  if (!aligned16(o) || !aligned16(z) || !aligned16(gamma) || !aligned16(y)) return GDN_ERR_ALIGN;
  const long rows = static_cast<long>(T_tot) * Hv;
  const size_t nb = static_cast<size_t>(rows) * Dv * act_bytes(act);
  if (overlaps(y, nb, z, nb)) return GDN_ERR_ALIAS;
  if (y != o && overlaps(y, nb, o, nb)) return GDN_ERR_ALIAS;
  return gated_rmsnorm_launch(o, z, gamma, eps, rows, Dv, y, act, stream);
}
