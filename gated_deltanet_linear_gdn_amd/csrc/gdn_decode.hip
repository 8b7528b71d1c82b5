// gdn_decode_step: one gated delta-rule token for a dense decode batch.
//
// Math (metaltile-std `gated_delta.rs`, module doc "Recurrence per step"):
// for each (b, hv) slice S [Dv, Dk] (Dk contiguous), gate a = exp(g):
//   kv_j = sum_i (a S[j,i]) k_i,  d_j = beta (v_j - kv_j),
//   S'[j,i] = a S[j,i] + d_j k_i,  y_j = sum_i S'[j,i] q_i.
//
// Design (gfx950, HBM-bound):
// * Every value row j of a slice is independent: it needs only its own 512 B
//   of state (Dk = 128), the shared k and q, and v_j.  A row is spread over
//   Dk/4 lanes, one float4 per lane, so each load/store instruction of a
//   wave moves whole rows with 16-byte accesses (global_load_dwordx4).
// * A workgroup of 128 threads (two waves) owns ROWS = (128 / (Dk/4)) * 2
//   rows of one slice, two per lane-row group: 4 KiB of state (8 rows at
//   Dk = 128, 16 workgroups per 64 KiB slice).  Each lane keeps its two
//   float4s in registers from the load to the store, so the state crosses
//   HBM exactly twice (read once, written once).  Measured on MI355X at
//   B=256, Hv=48, Dk=Dv=128 this fine grain streams within 2% of a one-load,
//   one-store copy kernel of the same bytes (6.44 vs 6.58 TB/s); one slice
//   per 512-thread workgroup with 8 rows per lane was 7% slower, and more
//   rows per lane or larger workgroups were slower still.
// * Both row reductions (S.k and S.q, before the update) run together as
//   lane-group sums; the readout then uses the exact identity
//   y_j = a (S_j . q) + d_j (k . q), so no second pass over the updated row
//   is needed.  k . q is one extra group sum per workgroup.
// * State traffic uses non-temporal loads and stores: each byte is touched
//   once per step and should not evict the activations from L2.
// * In-place (state_out == state_in) is safe: each element is read and then
//   written by the same lane.

#include "gdn_decode_core.h"

namespace gdn {
namespace {

template <typename T>
int launch(const float* state_in, float* state_out, const void* q, const void* k,
           const void* v, const float* g, const void* beta, void* y, int B, int Hk, int Hv,
           int Dk, int Dv, hipStream_t stream) {
  switch (Dk) {
    case 32: return launch_decode_dk<32, T>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dv, stream);
    case 64: return launch_decode_dk<64, T>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dv, stream);
    case 128: return launch_decode_dk<128, T>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dv, stream);
    case 256: return launch_decode_dk<256, T>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dv, stream);
    case 96: return launch_decode_dk<96, T>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dv, stream);
    case 160: return launch_decode_dk<160, T>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dv, stream);
    case 192: return launch_decode_dk<192, T>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dv, stream);
    case 224: return launch_decode_dk<224, T>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dv, stream);
  }
  return GDN_ERR_UNSUPPORTED;
}

// ------------------------------------------------------------ decode windows
//
// T tokens per sequence in one pass (metaltile `mt_gated_delta_chunk`: the
// state stays in registers across an inner token loop; regolith commit
// rule): the same per-token arithmetic as gdn_decode_kernel, token after
// token, on the lane's two state rows.  Every token's activations are
// loaded before the state (kept as loaded, converted on use); the state
// after the first `commit` tokens is kept in registers and stored at the
// end (commit 0: a verify window, no state write).  The state crosses HBM
// once per window instead of once per token.

template <int DK, int NV, bool FULL, typename T, int NT>
__global__ __launch_bounds__(kThreads) void gdn_window_kernel(
    const float* state_in, float* state_out, const T* __restrict__ q,
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ g,
    const T* __restrict__ beta, T* __restrict__ y, int Hk, int Hv, int Dv,
    unsigned hk_mul, int Tn, int commit) {
  constexpr int ACT = DK / 4;            // float4 columns of a row
  constexpr int LPR = row_lanes(ACT);    // lanes per row
  constexpr int RPS = kThreads / LPR;    // rows per register slot, whole workgroup
  constexpr int ROWS = RPS * NV;         // rows per workgroup

  // grid (part, hv, b) and the key head as in the single-step kernel
  const int part = blockIdx.x;
  const int hv = blockIdx.y;
  const int b = blockIdx.z;
  const int slice = b * Hv + hv;
  const int hk = hk_mul ? static_cast<int>(__umulhi(static_cast<unsigned>(hv), hk_mul)) : hv;
  const int tid = threadIdx.x;
  const int c4 = tid % LPR;
  const int row0 = part * ROWS + tid / LPR;
  auto rowc = [&](int n) { return FULL ? row0 + n * RPS : min(row0 + n * RPS, Dv - 1); };
  // idle lanes past the row's columns, as in the single-step kernel
  const bool live = ACT == LPR || c4 < ACT;
  const int cc = ACT == LPR ? c4 : min(c4, ACT - 1);

  const size_t slice_off = static_cast<size_t>(slice) * Dv * DK;
  const float* sin = state_in + slice_off + cc * 4;
  float* sout = state_out + slice_off + cc * 4;

  // every token's activations first (token t of sequence b is row b*Tn + t)
  Raw4<T> kr[NT], qr[NT];
  float vv[NT][NV], graw[NT], bt[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t < Tn) {
      const size_t bt_ = static_cast<size_t>(b) * Tn + t;
      const size_t qk_off = (bt_ * Hk + hk) * DK + cc * 4;
      kr[t].load(k + qk_off);
      qr[t].load(q + qk_off);
      graw[t] = g[bt_ * Hv + hv];
      bt[t] = Act<T>::load(beta + bt_ * Hv + hv);
#pragma unroll
      for (int n = 0; n < NV; ++n) vv[t][n] = Act<T>::load(v + (bt_ * Hv + hv) * Dv + rowc(n));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x4 s[NV], kept[NV];
#pragma unroll
  for (int n = 0; n < NV; ++n) s[n] = load_stream(sin + static_cast<size_t>(rowc(n)) * DK);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int n = 0; n < NV; ++n) kept[n] = s[n];

#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t < Tn) {
      const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
      const f32x4 kk = live ? kr[t].f() : zero4, qq = live ? qr[t].f() : zero4;
      const float gate = expf(graw[t]);
      const float kq = group_sum<LPR>(dot4(kk, qq));
      const size_t yrow = ((static_cast<size_t>(b) * Tn + t) * Hv + hv) * Dv;
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        const int row = row0 + n * RPS;
        const float sk = group_sum<LPR>(dot4(s[n], kk));
        const float sq = group_sum<LPR>(dot4(s[n], qq));
        const float d = bt[t] * (vv[t][n] - gate * sk);
        s[n] = gate * s[n] + d * kk;
        if ((FULL || row < Dv) && c4 == 0) Act<T>::store(y + yrow + row, gate * sq + d * kq);
      }
      if (t + 1 == commit) {
#pragma unroll
        for (int n = 0; n < NV; ++n) kept[n] = s[n];
      }
    }
  }
  if (commit > 0) {
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      const int row = row0 + n * RPS;
      if ((FULL || row < Dv) && live) store_stream(sout + static_cast<size_t>(row) * DK, kept[n]);
    }
  }
}

template <int DK, typename T, int NT>
int launch_window_nt(const float* state_in, float* state_out, const void* q, const void* k, const void* v,
                     const float* g, const void* beta, void* y, int B, int Hk, int Hv, int Dv, int Tn,
                     int commit, hipStream_t stream) {
  constexpr int NV = kRowsPerLane;
  constexpr int ROWS = kThreads / row_lanes(DK / 4) * NV;
  const int parts = (Dv + ROWS - 1) / ROWS;
  if (Hv > 65535) return GDN_ERR_SHAPE;  // grid y
  const unsigned hk_mul = hk_reciprocal(Hv / Hk);
  const T* qa = static_cast<const T*>(q);
  const T* ka = static_cast<const T*>(k);
  const T* va = static_cast<const T*>(v);
  const T* ba = static_cast<const T*>(beta);
  T* ya = static_cast<T*>(y);
  (void)hipGetLastError();
  for (int b0 = 0; b0 < B; b0 += kMaxGridZ) {
    const int nb = std::min(B - b0, kMaxGridZ);
    const size_t sv = static_cast<size_t>(b0) * Hv;        // state slices before this batch slice
    const size_t tv = static_cast<size_t>(b0) * Tn * Hv;   // token x value-head rows before it
    const size_t tk = static_cast<size_t>(b0) * Tn * Hk * DK;
    const dim3 grid(static_cast<unsigned>(parts), static_cast<unsigned>(Hv), static_cast<unsigned>(nb));
    if (Dv % ROWS == 0)
      hipLaunchKernelGGL((gdn_window_kernel<DK, NV, true, T, NT>), grid, dim3(kThreads), 0, stream,
                         state_in + sv * Dv * DK, state_out + sv * Dv * DK, qa + tk, ka + tk,
                         va + tv * Dv, g + tv, ba + tv, ya + tv * Dv, Hk, Hv, Dv, hk_mul, Tn, commit);
    else
      hipLaunchKernelGGL((gdn_window_kernel<DK, NV, false, T, NT>), grid, dim3(kThreads), 0, stream,
                         state_in + sv * Dv * DK, state_out + sv * Dv * DK, qa + tk, ka + tk,
                         va + tv * Dv, g + tv, ba + tv, ya + tv * Dv, Hk, Hv, Dv, hk_mul, Tn, commit);
  }
  return launch_status();
}

template <int DK, typename T>
int launch_window(const float* state_in, float* state_out, const void* q, const void* k, const void* v,
                  const float* g, const void* beta, void* y, int B, int Hk, int Hv, int Dv, int Tn,
                  int commit, hipStream_t stream) {
  // the smallest built token capacity that holds the window
  if (Tn <= 2)
    return launch_window_nt<DK, T, 2>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dv, Tn, commit, stream);
  if (Tn <= 4)
    return launch_window_nt<DK, T, 4>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dv, Tn, commit, stream);
  return launch_window_nt<DK, T, 8>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dv, Tn, commit, stream);
}

template <typename T>
int launch_window_dk(const float* state_in, float* state_out, const void* q, const void* k, const void* v,
                     const float* g, const void* beta, void* y, int B, int Hk, int Hv, int Dk, int Dv,
                     int Tn, int commit, hipStream_t stream) {
  switch (Dk) {
    case 32: return launch_window<32, T>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dv, Tn, commit, stream);
    case 64: return launch_window<64, T>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dv, Tn, commit, stream);
    case 128: return launch_window<128, T>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dv, Tn, commit, stream);
    case 256: return launch_window<256, T>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dv, Tn, commit, stream);
    case 96: return launch_window<96, T>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dv, Tn, commit, stream);
    case 160: return launch_window<160, T>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dv, Tn, commit, stream);
    case 192: return launch_window<192, T>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dv, Tn, commit, stream);
    case 224: return launch_window<224, T>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dv, Tn, commit, stream);
  }
  return GDN_ERR_UNSUPPORTED;
}

}  // namespace
}  // namespace gdn

extern "C" int gdn_decode_window(const float* state_in, float* state_out, const void* q,
                                 const void* k, const void* v, const float* g,
                                 const void* beta, void* y, int B, int T, int Hk, int Hv, int Dk,
                                 int Dv, int commit, gdn_dtype act, hipStream_t stream) {
  using namespace gdn;
  if (B < 0 || T < 1 || Hk <= 0 || Hv <= 0 || Dk <= 0 || Dv <= 0 || Hv % Hk != 0 || commit < 0 ||
      commit > T)
    return GDN_ERR_SHAPE;
  if (!is_act(act)) return GDN_ERR_DTYPE;
  if (!valid_head(Dk) || Dv % 32 != 0 || Dv > 256 || T > 8) return GDN_ERR_UNSUPPORTED;
  if (B == 0) return GDN_OK;
  if (!state_in || !q || !k || !v || !g || !beta || !y || (commit > 0 && !state_out)) return GDN_ERR_NULL;
  if (!aligned16(state_in) || (state_out && !aligned16(state_out)) || !aligned16(q) || !aligned16(k))
    return GDN_ERR_ALIGN;
  const size_t state_bytes = static_cast<size_t>(B) * Hv * Dv * Dk * sizeof(float);
  if (state_out && state_out != state_in && overlaps(state_in, state_bytes, state_out, state_bytes))
    return GDN_ERR_ALIAS;
  const size_t y_bytes = static_cast<size_t>(B) * T * Hv * Dv * act_bytes(act);
  if (overlaps(y, y_bytes, state_in, state_bytes) || (state_out && overlaps(y, y_bytes, state_out, state_bytes)))
    return GDN_ERR_ALIAS;
  {
    const size_t qk = static_cast<size_t>(B) * T * Hk * Dk * act_bytes(act);
    const size_t tv = static_cast<size_t>(B) * T * Hv;
    const Span in[] = {{q, qk}, {k, qk}, {v, y_bytes}, {g, tv * sizeof(float)}, {beta, tv * act_bytes(act)}};
    const Span out[] = {{y, y_bytes}, {state_out, commit > 0 ? state_bytes : 0}};
    if (inputs_overlap_outputs(in, out)) return GDN_ERR_ALIAS;
  }
  if (act == GDN_BF16)
    return launch_window_dk<bf16>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dk, Dv, T, commit, stream);
  return launch_window_dk<float>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dk, Dv, T, commit, stream);
}

extern "C" int gdn_decode_step(const float* state_in, float* state_out, const void* q,
                               const void* k, const void* v, const float* g,
                               const void* beta, void* y, int B, int Hk, int Hv, int Dk,
                               int Dv, gdn_dtype act, hipStream_t stream) {
  using namespace gdn;
  if (B < 0 || Hk <= 0 || Hv <= 0 || Dk <= 0 || Dv <= 0 || Hv % Hk != 0) return GDN_ERR_SHAPE;
  if (!is_act(act)) return GDN_ERR_DTYPE;
  if (!valid_head(Dk) || Dv % 32 != 0 || Dv > 256) return GDN_ERR_UNSUPPORTED;
  if (B == 0) return GDN_OK;
  if (!state_in || !state_out || !q || !k || !v || !g || !beta || !y) return GDN_ERR_NULL;
  if (!aligned16(state_in) || !aligned16(state_out) || !aligned16(q) || !aligned16(k))
    return GDN_ERR_ALIGN;
  const size_t state_bytes = static_cast<size_t>(B) * Hv * Dv * Dk * sizeof(float);
  if (state_out != state_in && overlaps(state_in, state_bytes, state_out, state_bytes))
    return GDN_ERR_ALIAS;
  const size_t y_bytes = static_cast<size_t>(B) * Hv * Dv * act_bytes(act);
  if (overlaps(y, y_bytes, state_out, state_bytes) || overlaps(y, y_bytes, state_in, state_bytes))
    return GDN_ERR_ALIAS;
  {
    const size_t qk = static_cast<size_t>(B) * Hk * Dk * act_bytes(act);
    const size_t bv = static_cast<size_t>(B) * Hv;
    const Span in[] = {{q, qk}, {k, qk}, {v, y_bytes}, {g, bv * sizeof(float)}, {beta, bv * act_bytes(act)}};
    const Span out[] = {{y, y_bytes}, {state_out, state_bytes}};
    if (inputs_overlap_outputs(in, out)) return GDN_ERR_ALIAS;
  }
  if (act == GDN_BF16)
    return launch<bf16>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dk, Dv, stream);
  return launch<float>(state_in, state_out, q, k, v, g, beta, y, B, Hk, Hv, Dk, Dv, stream);
}
