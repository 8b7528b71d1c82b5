// gdn_conv_decode_step: one decode token of the layer front: 4-tap causal
// conv + SiLU of the token's q, k and v channels against a rolling history
// (updated in place), L2 norm of q and k with the query scale, the gates from
// the raw a, b, and the gated delta-rule step.
//
// Math (regolith `gdn.metal`, header comment and the conv/SiLU block of its
// kernel; metaltile-std `gated_delta.rs`, "Recurrence per step"): for
// sequence b, channel c of the C = 2 Hk Dk + Hv Dv input channels
// [q heads | k heads | v heads], history h[b][c][0..2] oldest first:
//   x'_c = SiLU(h0 w0 + h1 w1 + h2 w2 + x_c w3),   new history (h1, h2, x_c)
//   k^ = k' / sqrt(|k'|^2 + 1e-6),  q^ = scale q' / sqrt(|q'|^2 + 1e-6)
//   g = -exp(A_log[hv]) softplus(a + dt_bias[hv]),  beta = sigmoid(b)
//   then gdn_decode_step with (q^, k^, v', g, beta).
//
// Design: two kernels on the caller's stream.
// * gdn_layer_prologue_kernel, one workgroup per (sequence, key head): the
//   key head's q and k channels and the v channels of its Hv/Hk value heads,
//   each channel's history read and rewritten by the one thread that owns it
//   (nothing else reads it), the two norms (workgroup reduction) and the
//   gates of those value heads.  Results go to the workspace in fp32, in the
//   layouts of gdn_decode_step (q^, k^ [B,Hk,Dk], v' [B,Hv,Dv], g, beta
//   [B,Hv]): 10.5 MB at B=256, written and read back while it sits in the
//   caches.
// * the decode step's own kernel (gdn_decode_core.h) on those fp32 inputs,
//   y in the activation dtype.
// Measured and dropped: convolving in the decode kernel itself.  A key
// head's q and k feed 3 x 16 workgroups at Dk = Dv = 128: convolving them in
// each took 378 us per B=256 step (7.7 KB of inputs, history and weights
// loaded per 8 KB of state); with only the value rows convolved there (q, k
// from a prologue) 299 us, the ten extra loads per lane for a row's input,
// history and weights costing more than the separate conv kernel.

#include "gdn_decode_core.h"

namespace gdn {
namespace {

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

struct Hist {
  float h0, h1, h2;
};

__device__ __forceinline__ Hist load_hist(const float* p) { return Hist{p[0], p[1], p[2]}; }

// a channel's new history: the two newest old entries, then this token
__device__ __forceinline__ void store_hist(float* p, const Hist& h, float x) {
  p[0] = h.h1;
  p[1] = h.h2;
  p[2] = x;
}

__device__ __forceinline__ float conv4(const Hist& h, f32x4 w, float x) {
  return h.h0 * w.x + h.h1 * w.y + h.h2 * w.z + x * w.w;
}

// Where the prologue's fp32 results go: the gdn_decode_step layouts.
struct PrologueOut {
  float* q;     // [B, Hk, Dk]
  float* k;     // [B, Hk, Dk]
  float* v;     // [B, Hv, Dv]
  float* g;     // [B, Hv]
  float* beta;  // [B, Hv]
};

inline PrologueOut prologue_out(void* ws, int B, int Hk, int Hv, int Dk, int Dv) {
  float* f = static_cast<float*>(ws);
  PrologueOut o;
  o.q = f;
  o.k = o.q + static_cast<size_t>(B) * Hk * Dk;
  o.v = o.k + static_cast<size_t>(B) * Hk * Dk;
  o.g = o.v + static_cast<size_t>(B) * Hv * Dv;
  o.beta = o.g + static_cast<size_t>(B) * Hv;
  return o;
}

// One workgroup per (sequence b, key head hk), 128 threads.
template <int DK, typename T>
__global__ __launch_bounds__(kThreads) void gdn_layer_prologue_kernel(
    const T* __restrict__ qkv, const float* __restrict__ conv_w, float* __restrict__ conv_state,
    const T* __restrict__ a, const T* __restrict__ bg, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, PrologueOut out, int Hk, int Hv, int Dv, float scale, int l2) {
  constexpr int QKC = (DK + kThreads - 1) / kThreads;  // q (and k) channels per thread
  constexpr int NW = kThreads / 64;
  __shared__ float part_q[NW], part_k[NW];
  const int hk = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int G = Hv / Hk;
  const size_t C = static_cast<size_t>(2 * Hk) * DK + static_cast<size_t>(Hv) * Dv;
  const size_t xb = static_cast<size_t>(b) * C;
  const size_t qc0 = static_cast<size_t>(hk) * DK, kc0 = static_cast<size_t>(Hk + hk) * DK;

  // q and k: one channel of each per thread (two at Dk = 256)
  float qo[QKC], ko[QKC];
  float sq = 0.0f, sk = 0.0f;
#pragma unroll
  for (int i = 0; i < QKC; ++i) {
    const int ch = tid + i * kThreads;
    qo[i] = ko[i] = 0.0f;
    if (ch < DK) {
      const float xq = to_f32(qkv[xb + qc0 + ch]), xk = to_f32(qkv[xb + kc0 + ch]);
      float* hq = conv_state + (xb + qc0 + ch) * 3;
      float* hkk = conv_state + (xb + kc0 + ch) * 3;
      const Hist oq = load_hist(hq), ok = load_hist(hkk);
      qo[i] = silu(conv4(oq, *reinterpret_cast<const f32x4*>(conv_w + (qc0 + ch) * 4), xq));
      ko[i] = silu(conv4(ok, *reinterpret_cast<const f32x4*>(conv_w + (kc0 + ch) * 4), xk));
      store_hist(hq, oq, xq);
      store_hist(hkk, ok, xk);
      sq += qo[i] * qo[i];
      sk += ko[i] * ko[i];
    }
  }
  // v of the key head's value heads (consecutive channels), and their gates
  const size_t vc0 = static_cast<size_t>(2 * Hk) * DK + static_cast<size_t>(hk) * G * Dv;
  const size_t vo0 = (static_cast<size_t>(b) * Hv + static_cast<size_t>(hk) * G) * Dv;
  for (int c = tid; c < G * Dv; c += kThreads) {
    const float x = to_f32(qkv[xb + vc0 + c]);
    float* h = conv_state + (xb + vc0 + c) * 3;
    const Hist o = load_hist(h);
    out.v[vo0 + c] = silu(conv4(o, *reinterpret_cast<const f32x4*>(conv_w + (vc0 + c) * 4), x));
    store_hist(h, o, x);
  }
  for (int j = tid; j < G; j += kThreads) {
    const int hv = hk * G + j;
    const size_t n = static_cast<size_t>(b) * Hv + hv;
    gates_of(to_f32(a[n]) + dt_bias[hv], A_log[hv], to_f32(bg[n]), out.g[n], out.beta[n]);
  }
  float fq = scale, fk = 1.0f;
  if (l2) {
    sq = group_sum<64>(sq);
    sk = group_sum<64>(sk);
    if ((tid & 63) == 0) {
      part_q[tid >> 6] = sq;
      part_k[tid >> 6] = sk;
    }
    __syncthreads();
    sq = 0.0f;
    sk = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      sq += part_q[w];
      sk += part_k[w];
    }
    fq = scale / sqrtf(sq + 1e-6f);
    fk = 1.0f / sqrtf(sk + 1e-6f);
  }
  const size_t qo0 = (static_cast<size_t>(b) * Hk + hk) * DK;
#pragma unroll
  for (int i = 0; i < QKC; ++i) {
    const int ch = tid + i * kThreads;
    if (ch < DK) {
      out.q[qo0 + ch] = qo[i] * fq;
      out.k[qo0 + ch] = ko[i] * fk;
    }
  }
}

template <int DK, typename T>
int launch_layer_dk(const float* state_in, float* state_out, const void* qkv, const float* conv_w,
                    float* conv_state, void* ws, const void* a, const void* bg, const float* A_log,
                    const float* dt_bias, void* y, int B, int Hk, int Hv, int Dv, float scale, int l2,
                    hipStream_t stream) {
  const size_t C = static_cast<size_t>(2 * Hk) * DK + static_cast<size_t>(Hv) * Dv;
  const PrologueOut o = prologue_out(ws, B, Hk, Hv, DK, Dv);
  (void)hipGetLastError();
  for (int b0 = 0; b0 < B; b0 += kMaxGridZ) {
    const int nb = std::min(B - b0, kMaxGridZ);
    const size_t sv = static_cast<size_t>(b0) * Hv;
    PrologueOut ob = o;
    ob.q += static_cast<size_t>(b0) * Hk * DK;
    ob.k += static_cast<size_t>(b0) * Hk * DK;
    ob.v += sv * Dv;
    ob.g += sv;
    ob.beta += sv;
    hipLaunchKernelGGL((gdn_layer_prologue_kernel<DK, T>), dim3(static_cast<unsigned>(Hk), static_cast<unsigned>(nb)),
                       dim3(kThreads), 0, stream, static_cast<const T*>(qkv) + static_cast<size_t>(b0) * C, conv_w,
                       conv_state + static_cast<size_t>(b0) * C * 3, static_cast<const T*>(a) + sv,
                       static_cast<const T*>(bg) + sv, A_log, dt_bias, ob, Hk, Hv, Dv, scale, l2);
  }
  if (launch_status() != GDN_OK) return GDN_ERR_LAUNCH;
  return launch_decode_dk<DK, float, T>(state_in, state_out, o.q, o.k, o.v, o.g, o.beta, y, B, Hk, Hv, Dv, stream);
}

template <typename T>
int launch_layer(const float* state_in, float* state_out, const void* qkv, const float* conv_w, float* conv_state,
                 void* ws, const void* a, const void* bg, const float* A_log, const float* dt_bias, void* y, int B,
                 int Hk, int Hv, int Dk, int Dv, float scale, int l2, hipStream_t stream) {
  switch (Dk) {
    case 32:
      return launch_layer_dk<32, T>(state_in, state_out, qkv, conv_w, conv_state, ws, a, bg, A_log, dt_bias, y, B,
                                    Hk, Hv, Dv, scale, l2, stream);
    case 64:
      return launch_layer_dk<64, T>(state_in, state_out, qkv, conv_w, conv_state, ws, a, bg, A_log, dt_bias, y, B,
                                    Hk, Hv, Dv, scale, l2, stream);
    case 128:
      return launch_layer_dk<128, T>(state_in, state_out, qkv, conv_w, conv_state, ws, a, bg, A_log, dt_bias, y,
                                     B, Hk, Hv, Dv, scale, l2, stream);
    case 256:
      return launch_layer_dk<256, T>(state_in, state_out, qkv, conv_w, conv_state, ws, a, bg, A_log, dt_bias, y,
                                     B, Hk, Hv, Dv, scale, l2, stream);
    case 96:
      return launch_layer_dk<96, T>(state_in, state_out, qkv, conv_w, conv_state, ws, a, bg, A_log, dt_bias, y,
                                     B, Hk, Hv, Dv, scale, l2, stream);
    case 160:
      return launch_layer_dk<160, T>(state_in, state_out, qkv, conv_w, conv_state, ws, a, bg, A_log, dt_bias, y,
                                     B, Hk, Hv, Dv, scale, l2, stream);
    case 192:
      return launch_layer_dk<192, T>(state_in, state_out, qkv, conv_w, conv_state, ws, a, bg, A_log, dt_bias, y,
                                     B, Hk, Hv, Dv, scale, l2, stream);
    case 224:
      return launch_layer_dk<224, T>(state_in, state_out, qkv, conv_w, conv_state, ws, a, bg, A_log, dt_bias, y,
                                     B, Hk, Hv, Dv, scale, l2, stream);
  }
  return GDN_ERR_UNSUPPORTED;
}

}  // namespace
}  // namespace gdn

extern "C" size_t gdn_conv_decode_workspace(int B, int Hk, int Hv, int Dk, int Dv) {
  if (B < 0 || Hk <= 0 || Hv <= 0 || Dk <= 0 || Dv <= 0) return 0;
  return static_cast<size_t>(B) * (2 * static_cast<size_t>(Hk) * Dk + static_cast<size_t>(Hv) * Dv + 2 * Hv) *
         sizeof(float);
}

extern "C" int gdn_conv_decode_step(const float* state_in, float* state_out, const void* qkv,
                                    const float* conv_w, float* conv_state, const void* a, const void* b,
                                    const float* A_log, const float* dt_bias, void* y, int B, int Hk, int Hv,
                                    int Dk, int Dv, float scale, unsigned flags, gdn_dtype act, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  using namespace gdn;
  if (B < 0 || Hk <= 0 || Hv <= 0 || Dk <= 0 || Dv <= 0 || Hv % Hk != 0) return GDN_ERR_SHAPE;
  if (!is_act(act)) return GDN_ERR_DTYPE;
  if (!valid_head(Dk) || Dv % 32 != 0 || Dv > 256 || (flags & ~static_cast<unsigned>(GDN_QK_L2NORM)) != 0)
    return GDN_ERR_UNSUPPORTED;
  if (B == 0) return GDN_OK;
  if (!state_in || !state_out || !qkv || !conv_w || !conv_state || !a || !b || !A_log || !dt_bias || !y ||
      !workspace)
    return GDN_ERR_NULL;
  if (!aligned16(state_in) || !aligned16(state_out) || !aligned16(conv_w) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(conv_state) & 3u) != 0)
    return GDN_ERR_ALIGN;
  const size_t ws_bytes = gdn_conv_decode_workspace(B, Hk, Hv, Dk, Dv);
  if (workspace_bytes < ws_bytes) return GDN_ERR_WORKSPACE;
  const size_t state_bytes = static_cast<size_t>(B) * Hv * Dv * Dk * sizeof(float);
  if (state_out != state_in && overlaps(state_in, state_bytes, state_out, state_bytes)) return GDN_ERR_ALIAS;
  const size_t C = static_cast<size_t>(2 * Hk) * Dk + static_cast<size_t>(Hv) * Dv;
  const size_t hist_bytes = static_cast<size_t>(B) * C * 3 * sizeof(float);
  const size_t y_bytes = static_cast<size_t>(B) * Hv * Dv * act_bytes(act);
  {
    const size_t bv = static_cast<size_t>(B) * Hv;
    const Span in[] = {{qkv, static_cast<size_t>(B) * C * act_bytes(act)},
                       {conv_w, C * 4 * sizeof(float)},
                       {a, bv * act_bytes(act)},
                       {b, bv * act_bytes(act)},
                       {A_log, static_cast<size_t>(Hv) * sizeof(float)},
                       {dt_bias, static_cast<size_t>(Hv) * sizeof(float)},
                       {state_in, state_out == state_in ? 0 : state_bytes}};
    const Span out[] = {{y, y_bytes}, {state_out, state_bytes}, {conv_state, hist_bytes}, {workspace, ws_bytes}};
    if (inputs_overlap_outputs(in, out)) return GDN_ERR_ALIAS;
    for (int i = 0; i < 4; ++i)
      for (int j = i + 1; j < 4; ++j)
        if (overlaps(out[i].p, out[i].n, out[j].p, out[j].n)) return GDN_ERR_ALIAS;
  }
  if (!(scale > 0.0f)) scale = 1.0f / sqrtf(static_cast<float>(Dk));
  const int l2 = (flags & GDN_QK_L2NORM) ? 1 : 0;
  if (act == GDN_BF16)
    return launch_layer<bf16>(state_in, state_out, qkv, conv_w, conv_state, workspace, a, b, A_log, dt_bias, y, B,
                              Hk, Hv, Dk, Dv, scale, l2, stream);
  return launch_layer<float>(state_in, state_out, qkv, conv_w, conv_state, workspace, a, b, A_log, dt_bias, y, B,
                             Hk, Hv, Dk, Dv, scale, l2, stream);
}
