// gdn_chunk_prefill: variable-length chunkwise (WY) prefill over a state pool.
//
// Source: pymllm `gdn_chunkwise` docs, "Algorithm (per chunk of C tokens with
// initial state S_0)", steps 1-3, and the `gdn_extend_chunkwise` parameters.
// The chunk algebra is used in its division-free form (every exponent <= 0
// for log-gates g <= 0).  Per chunk of a sequence, with k^, q^ the
// L2-normalised keys/queries (q^ also scaled), G_t the inclusive in-chunk sum
// of the log-gates, gamma_t = exp(G_t), and the state S = S^T of the stored
// [Dv, Dk] slice (Dk x Dv):
//   A_ij  = beta_i exp(G_i - G_j) k^_i . k^_j   (j < i),   T = (I + A)^-1
//   R     = diag(beta) V - diag(beta gamma) K^ S
//   Delta = T R                                  (the WY "new values")
//   O     = diag(gamma) Q^ S + P Delta,  P_ij = exp(G_i - G_j) q^_i . k^_j (j <= i)
//   S    <- gamma_C S + (diag(exp(G_C - G)) K^)^T Delta
// which is the page's w/u~ construction, S_0 W, triu(K^T Q) and state update
// rescaled by the cumulative decay (no 1/gamma anywhere).
//
// Kernels (gfx950, wave64, v_mfma_f32_16x16x32_bf16 for the contractions):
//  1. The chunk map: scan over cu_seqlens -> first chunk of each sequence
//     and the order the chunk loop takes them in (device side, no host
//     sync); gdn_chunk_map_kernel, or with bf16 activations and up to 64
//     sequences one more workgroup of the WY launch.
//  2. The WY pass, all chunks of all sequences in parallel (nothing here
//     depends on the state): q/k row norms, G, the Gram blocks K K^T and
//     Q K^T on MFMA, A and P, T = (I + A)^-1, and per-token factors (the
//     gates themselves too when they come raw: gdn_chunk_prefill_raw).
//     bf16 activations: gdn_wy_wave_kernel (section 4), one wave per
//     (chunk, key head), blocked inverse.  fp32 activations: gdn_wy_kernel
//     (section 2), one wave per (chunk, value head), column-parallel forward
//     substitution.
//  3. The sequential chunk loop per (sequence, value head, value columns),
//     each wave keeping its Dk x 16 slice of S in MFMA accumulators:
//     X = K S, Y = Q S, Delta = T R, O = Y' + P Delta and the state update as
//     chained MFMAs (every product's right operand is the previous product's
//     accumulator converted to bf16, with the contraction index permuted
//     identically on both sides so no data moves between lanes).  Raw q/k/v
//     enter the MFMAs exactly; norms and decays scale fp32 accumulators;
//     operands that carry the state (S, R, Delta, T, and the scaled Delta of
//     the update) are split into bf16 hi + lo halves so the state and the
//     output keep fp32-grade accuracy.  bf16 activations: gdn_prefill_stream_kernel
//     (section 5), operands streamed through LDS by asynchronous copies.
//     fp32 activations: gdn_prefill_kernel (section 3), register fragments
//     from global memory, hi/lo on both sides of every product.

#include <atomic>
#include <mutex>
#include <type_traits>

#include "gdn_device.h"
#include "gdn_host.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8v __attribute__((__vector_size__(16)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNormEps = 1e-6f;

__device__ __forceinline__ f32x4 mma(bf16x8v a, bf16x8v b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pk(float a, float b) {
  bf16x2v v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Two fp32 values -> packed bf16 hi (round to nearest even) and lo =
// bf16(x - hi).  The hi halves come back to fp32 from the packed word (a
// shift and a mask), not from a second conversion.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& h, uint32_t& l) {
  h = pk(a, b);
  asm("" : "+v"(h));  // opaque: otherwise the low half is converted again on its own
  l = pk(a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xffff0000u));
}

// Eight fp32 values -> bf16 hi (and lo = bf16(x - hi)) operand vectors.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8v& hi, bf16x8v& lo) {
  u32x4 h, l;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t hp, lp;
    split_pair(x[2 * p], x[2 * p + 1], hp, lp);
    h[p] = hp;
    l[p] = lp;
  }
  hi = __builtin_bit_cast(bf16x8v, h);
  lo = __builtin_bit_cast(bf16x8v, l);
}

// Operand over the contraction index from two stacked 16x16 accumulator tiles
// (rows base..base+15 in t0, base+16..base+31 in t1): element e < 4 is row
// base + kg*4 + e, element e >= 4 is row base + 16 + kg*4 + (e-4).
__device__ __forceinline__ void acc_operand(f32x4 t0, f32x4 t1, bf16x8v& hi, bf16x8v& lo) {
  const float x[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
  split8(x, hi, lo);
}
__device__ __forceinline__ bf16x8v acc_operand_hi(f32x4 t0, f32x4 t1) {
  u32x4 h = {pk(t0.x, t0.y), pk(t0.z, t0.w), pk(t1.x, t1.y), pk(t1.z, t1.w)};
  return __builtin_bit_cast(bf16x8v, h);
}

__device__ __forceinline__ bf16x8v zero8() { return __builtin_bit_cast(bf16x8v, u32x4{0, 0, 0, 0}); }

// Memory fragments along a row.  "pi" order matches acc_operand: elements
// 0..3 = row[k0 + kg*4 + 0..3], 4..7 = row[k0 + 16 + kg*4 + 0..3].  "std"
// order: elements 0..7 = row[k0 + kg*8 + 0..7].
template <typename T> struct Frag;

template <> struct Frag<bf16> {
  static __device__ __forceinline__ void pi(const bf16* row, int k0, int kg, bf16x8v& hi, bf16x8v& lo) {
    const uint2 a = *reinterpret_cast<const uint2*>(row + k0 + kg * 4);
    const uint2 b = *reinterpret_cast<const uint2*>(row + k0 + 16 + kg * 4);
    hi = __builtin_bit_cast(bf16x8v, u32x4{a.x, a.y, b.x, b.y});
    lo = zero8();
  }
  static __device__ __forceinline__ void stdo(const bf16* row, int k0, int kg, bf16x8v& hi, bf16x8v& lo) {
    const uint4 a = *reinterpret_cast<const uint4*>(row + k0 + kg * 8);
    hi = __builtin_bit_cast(bf16x8v, u32x4{a.x, a.y, a.z, a.w});
    lo = zero8();
  }
  static __device__ __forceinline__ float sumsq(const bf16* row, int n) {
    float s = 0.f;
    for (int d = 0; d < n; d += 8) {
      const uint4 a = *reinterpret_cast<const uint4*>(row + d);
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float x = __uint_as_float(w[p] << 16), y = __uint_as_float(w[p] & 0xffff0000u);
        s += x * x + y * y;
      }
    }
    return s;
  }
};

template <> struct Frag<float> {
  static __device__ __forceinline__ void pi(const float* row, int k0, int kg, bf16x8v& hi, bf16x8v& lo) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(row + k0 + kg * 4);
    const f32x4 b = *reinterpret_cast<const f32x4*>(row + k0 + 16 + kg * 4);
    const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    split8(x, hi, lo);
  }
  static __device__ __forceinline__ void stdo(const float* row, int k0, int kg, bf16x8v& hi, bf16x8v& lo) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(row + k0 + kg * 8);
    const f32x4 b = *reinterpret_cast<const f32x4*>(row + k0 + kg * 8 + 4);
    const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    split8(x, hi, lo);
  }
  static __device__ __forceinline__ float sumsq(const float* row, int n) {
    float s = 0.f;
    for (int d = 0; d < n; d += 4) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(row + d);
      s += (a.x * a.x + a.y * a.y) + (a.z * a.z + a.w * a.w);
    }
    return s;
  }
};

// Raw A-operand fragments in "pi" order, kept as loaded so that every global
// load of a chunk can be issued before the first use; converted (and split
// into hi/lo for fp32 activations) when consumed.
template <typename T> struct Raw;
template <> struct Raw<bf16> {
  uint2 a, b;
  static __device__ __forceinline__ Raw load(const bf16* row, int k0, int kg) {
    return Raw{*reinterpret_cast<const uint2*>(row + k0 + kg * 4),
               *reinterpret_cast<const uint2*>(row + k0 + 16 + kg * 4)};
  }
  __device__ __forceinline__ void operand(bf16x8v& hi, bf16x8v& lo) const {
    hi = __builtin_bit_cast(bf16x8v, u32x4{a.x, a.y, b.x, b.y});
    lo = zero8();
  }
};
template <> struct Raw<float> {
  f32x4 a, b;
  static __device__ __forceinline__ Raw load(const float* row, int k0, int kg) {
    return Raw{*reinterpret_cast<const f32x4*>(row + k0 + kg * 4),
               *reinterpret_cast<const f32x4*>(row + k0 + 16 + kg * 4)};
  }
  __device__ __forceinline__ void operand(bf16x8v& hi, bf16x8v& lo) const {
    const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    split8(x, hi, lo);
  }
};

// ----------------------------------------------------------------------------
// 1. chunk map: scs[s] = sum_{s' < s} ceil(L_s' / C), scs[N_s] = total, and
// after it (scs + N_s + 1) the order in which the chunk loop takes the
// sequences: longest first, by the bit length of the chunk count (so a long
// sequence never waits for a whole round of short ones to finish before its
// chain starts), with the longest sequence itself first (the split test
// below compares against it); the order within a bit length is otherwise
// arbitrary, and no result depends on it.

// The layer prologue run inside the bf16 WY pass (gdn_conv_prefill): the raw
// channels x [T, C] of every token (C = 2 Hk Dk + Hv Dv, laid out as q heads
// | k heads | v heads), the conv weights W [C, 4] (tap 3 weighs the current
// token), the rolling history hist [pool_size, C, 3] (oldest first), and the
// convolved q, k [T, Hk, Dk] and v [T, Hv, Dv] that the rest of the WY pass
// and the chunk loop read.  x == nullptr: no prologue.
struct ConvIn {
  const bf16* x;
  const float* W;
  float* hist;
  const int64_t* ci;
  int64_t pool_size;
  bf16* q;
  bf16* k;
  bf16* v;
  bf16* trash;  // 16 bytes no one reads: the store of a row past the chunk
  int Dv;
  int keep;  // leave the history as it is (GDN_KEEP_STATE)
};

// Raw gate inputs of a prefill whose gates are formed inside the WY pass
// (gdn_chunk_prefill_raw); a, b in the bf16 activation dtype; and the conv
// prologue, when the pass runs it too.
struct RawGates {
  const bf16* a;
  const bf16* b;
  const float* A_log;
  const float* dt_bias;
  ConvIn cv;
};

__device__ __forceinline__ void seq_bounds(const int64_t* cu, int s, int64_t T_tot, int64_t& b0,
                                           int64_t& len) {
  int64_t a = cu[s], b = cu[s + 1];
  a = a < 0 ? 0 : (a > T_tot ? T_tot : a);
  b = b < a ? a : (b > T_tot ? T_tot : b);
  b0 = a;
  len = b - a;
}

// The fixed-T batch layout as a varlen batch: sequence s owns tokens
// s*T .. s*T + T - 1 and state slot s.
__global__ __launch_bounds__(256) void gdn_fixed_index_kernel(int64_t* __restrict__ cu,
                                                              int64_t* __restrict__ ci, int B,
                                                              int64_t T) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i <= B) cu[i] = static_cast<int64_t>(i) * T;
  if (i < B) ci[i] = i;
}

// A fixed-length batch with bf16 activations (gdn_chunk_prefill_fixed):
// every sequence is T tokens long and owns the state slot of its index.
// The WY launch then finds each chunk's sequence by division, and its last
// workgroup writes cu_seqlens and cache_indices (for the chunk loop) and
// the chunk map, so no index or map kernel runs ahead of it.
struct FixedBatch {
  int64_t T;     // tokens per sequence (0: a varlen batch)
  int64_t* cu;   // [N_s + 1], written by the WY launch
  int64_t* ci;   // [N_s], written by the WY launch
};

// The chunk map of a fixed-length batch, on the threads of one workgroup:
// what chunk_map_body computes when every sequence has the same length
// (the order is the identity, which is longest first; the sequences split
// in halves all together or not at all, since none is longer than another).
__device__ __forceinline__ void fixed_map_body(const FixedBatch& fb, int N_s, int C, int* __restrict__ scs,
                                               int wg_per_seq, int num_cu, int allow_split) {
  const int per = static_cast<int>((fb.T + C - 1) / C);
  const int64_t idle = static_cast<int64_t>(num_cu) - static_cast<int64_t>(N_s) * wg_per_seq;
  const bool all_split = allow_split && idle > 0 && idle / wg_per_seq >= N_s;
  const int wg = all_split ? 2 * wg_per_seq : wg_per_seq;
  int* ord = scs + N_s + 1;
  int* wgp = ord + N_s;
  for (int i = threadIdx.x; i <= N_s; i += blockDim.x) {
    fb.cu[i] = static_cast<int64_t>(i) * fb.T;
    scs[i] = i * per;
    wgp[i] = i * wg;
    if (i < N_s) {
      fb.ci[i] = i;
      ord[i] = i;
    }
  }
}

// LDS of the chunk map for NT threads.  The first NC sequences' chunk
// counts and the first NC positions of the order stay there after the pass
// that forms them (every later pass would otherwise wait on another round
// of global loads); beyond NC they are read again.
template <int NT>
struct MapLds {
  static constexpr int NC = 4 * NT;
  int part[NT];
  int ncache[NC], ocache[NC];
  int bucket[33];  // sequences per bit length of the chunk count (0..32)
  int split_n;
  unsigned long long top_key;  // the longest sequence (ties: the first)
};

// The chunk map on NT threads of one workgroup (all of them call it).
template <int NT>
__device__ __forceinline__ void chunk_map_body(MapLds<NT>& m, const int64_t* __restrict__ cu, int N_s,
                                               int64_t T_tot, int C, int* __restrict__ scs, int wg_per_seq,
                                               int num_cu, int allow_split) {
  constexpr int NC = MapLds<NT>::NC;
  int* part = m.part;
  int* ncache = m.ncache;
  int* ocache = m.ocache;
  int* bucket = m.bucket;
  unsigned long long& top_key = m.top_key;
  int& split_n = m.split_n;
  const int tid = threadIdx.x;
  auto nch_global = [&](int s) -> int {
    int64_t b0, len;
    seq_bounds(cu, s, T_tot, b0, len);
    return static_cast<int>((len + C - 1) / C);
  };
  auto nch = [&](int s) -> int { return s < NC ? ncache[s] : nch_global(s); };
  const int per_t = (N_s + NT - 1) / NT;  // sequences (positions) per thread
  const int s0 = tid * per_t;
  int local = 0;
  for (int s = s0; s < s0 + per_t && s < N_s; ++s) {
    const int n = nch_global(s);
    if (s < NC) ncache[s] = n;
    local += n;
  }
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {  // inclusive scan
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - local;  // exclusive prefix of this thread's range
  if (tid < 33) bucket[tid] = 0;
  if (tid == 0) top_key = 0ull;
  __syncthreads();
  for (int s = s0; s < s0 + per_t && s < N_s; ++s) {
    scs[s] = run;
    const int n = nch(s);
    run += n;
    atomicAdd(&bucket[32 - __clz(n)], 1);
    atomicMax(&top_key, (static_cast<unsigned long long>(n) << 32) | (0xffffffffu - static_cast<unsigned>(s)));
  }
  if (tid == NT - 1) scs[N_s] = part[NT - 1];
  __syncthreads();
  const int top_s = static_cast<int>(0xffffffffu - static_cast<unsigned>(top_key & 0xffffffffull));
  const int top_n = static_cast<int>(top_key >> 32);
  if (tid == 0) {  // first rank of each bit length, longest first
    int r = 0;
    for (int b = 32; b >= 0; --b) {
      const int cnt = bucket[b];
      bucket[b] = r;
      r += cnt;
    }
    bucket[32 - __clz(top_n)] = 1;  // its first rank (0) goes to the longest sequence itself
  }
  __syncthreads();
  int* ord = scs + N_s + 1;
  for (int s = s0; s < s0 + per_t && s < N_s; ++s) {
    const int r = s == top_s ? 0 : atomicAdd(&bucket[32 - __clz(nch(s))], 1);
    ord[r] = s;
    if (r < NC) ocache[r] = s;
  }
  __syncthreads();
  auto ord_at = [&](int r) -> int { return r < NC ? ocache[r] : ord[r]; };
  // wgp[r]: chunk-loop workgroups before position r of that order.  The
  // first sequences of the order get two per (value head, column block) --
  // each computing half of the columns with half of its waves, a shorter
  // step -- as far as CUs would otherwise sit idle (on a full machine the
  // half-capable kernel is not launched: its whole workgroups run a little
  // slower), and only if that shortens the batch: the longest sequence left
  // whole must be clearly shorter than the longest split one.
  int* wgp = ord + N_s;
  if (tid == 0) {
    const int64_t idle = static_cast<int64_t>(num_cu) - static_cast<int64_t>(N_s) * wg_per_seq;
    int kk = allow_split && idle > 0 ? static_cast<int>(min(idle / wg_per_seq, static_cast<int64_t>(N_s))) : 0;
    if (kk > 0 && kk < N_s && 20 * nch(ord_at(kk)) > 17 * nch(ord_at(0))) kk = 0;
    split_n = kk;
  }
  __syncthreads();
  const int room = split_n;  // positions that split
  int loc = 0;
  for (int r = s0; r < s0 + per_t && r < N_s; ++r) {
    const bool sp = r < room && nch(ord_at(r)) > 0;
    loc += sp ? 2 * wg_per_seq : wg_per_seq;
  }
  part[tid] = loc;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int wrun = part[tid] - loc;
  for (int r = s0; r < s0 + per_t && r < N_s; ++r) {
    wgp[r] = wrun;
    const bool sp = r < room && nch(ord_at(r)) > 0;
    wrun += sp ? 2 * wg_per_seq : wg_per_seq;
  }
  if (tid == NT - 1) wgp[N_s] = part[NT - 1];
}

template <int NT>
__global__ __launch_bounds__(NT) void gdn_chunk_map_kernel(const int64_t* __restrict__ cu,
                                                             int N_s, int64_t T_tot, int C,
                                                             int* __restrict__ scs, int wg_per_seq,
                                                             int num_cu, int allow_split) {
  __shared__ MapLds<NT> m;
  chunk_map_body<NT>(m, cu, N_s, T_tot, C, scs, wg_per_seq, num_cu, allow_split);
}

// ----------------------------------------------------------------------------
// 2. WY pre-pass: one wave per (chunk, value head).

template <typename T, int DK, int CT>
__global__ __launch_bounds__(64) void gdn_wy_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ beta, const int64_t* __restrict__ cu, const int* __restrict__ scs,
    int N_s, int64_t T_tot, int Hk, int Hv, int C, float scale, int l2norm,
    bf16* __restrict__ Th, bf16* __restrict__ Tl, bf16* __restrict__ Ph, bf16* __restrict__ Pl,
    float* __restrict__ fac) {
  constexpr bool PRECISE = std::is_same<T, float>::value;
  constexpr int MT = CT / 16, KB = DK / 32;
  __shared__ float sG[CT], srk[CT], srq[CT], sb[CT];
  __shared__ __attribute__((aligned(16))) float Am[CT][CT + 4];

  const int c = blockIdx.x / Hv;
  const int hv = blockIdx.x - c * Hv;
  if (c >= scs[N_s]) return;
  int lo = 0, hi = N_s;  // largest s with scs[s] <= c
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (scs[mid] <= c) lo = mid; else hi = mid;
  }
  const int s = lo;
  int64_t b0, len;
  seq_bounds(cu, s, T_tot, b0, len);
  const int64_t j0 = static_cast<int64_t>(c - scs[s]) * C;
  const int64_t t0 = b0 + j0;
  const int n = static_cast<int>(len - j0 < C ? len - j0 : C);
  const int hk = hv / (Hv / Hk);
  const int lane = threadIdx.x, l16 = lane & 15, kg = lane >> 4;
  const size_t mat = static_cast<size_t>(c) * Hv + hv;

  // All K and Q fragments of the chunk, issued at once: lane (l16, kg) holds
  // row I*16 + l16, elements kb*32 + kg*8 .. +7, for every row block I and
  // k-block kb.  They serve as both MFMA operands of every Gram tile and give
  // the row norms.  Rows past the last token read it again and get zero
  // factors below.
  bf16x8v kh[MT][KB], kl[MT][KB], qh[MT][KB], ql[MT][KB];
  float ssk[MT], ssq[MT];
#pragma unroll
  for (int I = 0; I < MT; ++I) {
    const size_t roff = (static_cast<size_t>(t0 + min(I * 16 + l16, n - 1)) * Hk + hk) * DK;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      Frag<T>::stdo(k + roff, kb * 32, kg, kh[I][kb], kl[I][kb]);
      Frag<T>::stdo(q + roff, kb * 32, kg, qh[I][kb], ql[I][kb]);
    }
  }
  float gl = 0.f, bt = 0.f;
  if (lane < CT) {
    const size_t th = static_cast<size_t>(t0 + min(lane, n - 1)) * Hv + hv;
    gl = g[th];
    bt = beta[th];
  }
  // row sums of squares: per-lane partials over its 8 elements of each k-block,
  // then across the four lanes kg = 0..3 of the row
#pragma unroll
  for (int I = 0; I < MT; ++I) {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const u32x4 wk = __builtin_bit_cast(u32x4, kh[I][kb]), wq = __builtin_bit_cast(u32x4, qh[I][kb]);
      const u32x4 vk = __builtin_bit_cast(u32x4, kl[I][kb]), vq = __builtin_bit_cast(u32x4, ql[I][kb]);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        // x = hi + lo exactly reconstructs fp32 inputs; lo is zero for bf16 inputs
        const float x0 = __uint_as_float(wk[p] << 16) + __uint_as_float(vk[p] << 16);
        const float x1 = __uint_as_float(wk[p] & 0xffff0000u) + __uint_as_float(vk[p] & 0xffff0000u);
        const float y0 = __uint_as_float(wq[p] << 16) + __uint_as_float(vq[p] << 16);
        const float y1 = __uint_as_float(wq[p] & 0xffff0000u) + __uint_as_float(vq[p] & 0xffff0000u);
        a += x0 * x0 + x1 * x1;
        b += y0 * y0 + y1 * y1;
      }
    }
    a += __shfl_xor(a, 16);
    a += __shfl_xor(a, 32);
    b += __shfl_xor(b, 16);
    b += __shfl_xor(b, 32);
    ssk[I] = a;
    ssq[I] = b;
  }
  if (kg == 0) {
#pragma unroll
    for (int I = 0; I < MT; ++I) {
      const int t = I * 16 + l16;
      const bool ok = t < n;
      srk[t] = ok ? (l2norm ? 1.0f / sqrtf(ssk[I] + kNormEps) : 1.0f) : 0.f;
      srq[t] = ok ? scale * (l2norm ? 1.0f / sqrtf(ssq[I] + kNormEps) : 1.0f) : 0.f;
    }
  }
  // inclusive prefix sum of the log-gates over the chunk (wave scan)
  float G = lane < n ? gl : 0.f;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float up = __shfl_up(G, off);
    if (lane >= off) G += up;
  }
  if (lane < CT) {
    sG[lane] = G;
    sb[lane] = lane < n ? bt : 0.f;
  }
  __syncthreads();
  // Per-token factors of the chunk loop (zero past the last token):
  //   beta, beta gamma / |k|, gamma scale / |q|, exp(G_C - G) / |k|,
  // and gamma_C = exp(G_C); G is flat past the last token, so G_C = G[CT-1].
  if (lane < CT) {
    float* fp = fac + mat * (4 * CT + 4);
    const float GC = sG[CT - 1];
    const float gam = __expf(G);
    fp[lane] = sb[lane];
    fp[CT + lane] = sb[lane] * gam * srk[lane];
    fp[2 * CT + lane] = gam * srq[lane];
    fp[3 * CT + lane] = __expf(GC - G) * srk[lane];
    if (lane == 0) fp[4 * CT] = __expf(GC);
  }
  // Gram K K^T and Q K^T tiles (I, J), J <= I; A and P from them.
  bf16* ph = Ph + mat * CT * CT;
  bf16* pl = Pl + mat * CT * CT;
#pragma unroll
  for (int I = 0; I < MT; ++I) {
#pragma unroll
    for (int J = 0; J < MT; ++J) {
      if (J > I) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ii = I * 16 + kg * 4 + r, jj = J * 16 + l16;
          ph[ii * CT + jj] = 0;
          if constexpr (PRECISE) pl[ii * CT + jj] = 0;
        }
        continue;
      }
      f32x4 gk = {0.f, 0.f, 0.f, 0.f}, gq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        gk = mma(kh[I][kb], kh[J][kb], gk);
        gq = mma(qh[I][kb], kh[J][kb], gq);
        if constexpr (PRECISE) {
          gk = mma(kh[I][kb], kl[J][kb], gk);
          gk = mma(kl[I][kb], kh[J][kb], gk);
          gq = mma(qh[I][kb], kl[J][kb], gq);
          gq = mma(ql[I][kb], kh[J][kb], gq);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ii = I * 16 + kg * 4 + r, jj = J * 16 + l16;
        const float dec = (jj <= ii) ? __expf(sG[ii] - sG[jj]) : 0.f;
        Am[ii][jj] = (jj < ii) ? sb[ii] * dec * srk[ii] * srk[jj] * gk[r] : 0.f;
        const float pv = (jj <= ii) ? dec * srq[ii] * srk[jj] * gq[r] : 0.f;
        const __bf16 h = (__bf16)pv;
        ph[ii * CT + jj] = __builtin_bit_cast(bf16, h);
        if constexpr (PRECISE) pl[ii * CT + jj] = __builtin_bit_cast(bf16, (__bf16)(pv - (float)h));
      }
    }
  }
  __syncthreads();

  // T = (I + A)^-1, unit lower triangular; lane c computes column c by
  // forward substitution, four partial sums per row.
  if (lane < CT) {
    float tr[CT];
#pragma unroll
    for (int i = 0; i < CT; ++i) {
      float a0 = (i == lane) ? 1.f : 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
      for (int j = 0; j + 3 < i; j += 4) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(&Am[i][j]);
        a0 -= a.x * tr[j];
        a1 -= a.y * tr[j + 1];
        a2 -= a.z * tr[j + 2];
        a3 -= a.w * tr[j + 3];
      }
#pragma unroll
      for (int j = i & ~3; j < i; ++j) a0 -= Am[i][j] * tr[j];
      tr[i] = (a0 + a1) + (a2 + a3);
    }
    bf16* th = Th + mat * CT * CT;
    bf16* tl = Tl + mat * CT * CT;
#pragma unroll
    for (int i = 0; i < CT; ++i) {
      const __bf16 h = (__bf16)tr[i];
      th[i * CT + lane] = __builtin_bit_cast(bf16, h);
      tl[i * CT + lane] = __builtin_bit_cast(bf16, (__bf16)(tr[i] - (float)h));
    }
  }
}

// ----------------------------------------------------------------------------
// 3. Sequential chunk loop per (sequence, value head, value block).

template <typename T, int DK, int CT, int NW>
__global__ __launch_bounds__(64 * NW) void gdn_prefill_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ beta, float* __restrict__ pool, int64_t pool_size,
    const int64_t* __restrict__ cache_indices, const int64_t* __restrict__ cu,
    const int* __restrict__ scs, int N_s, int64_t T_tot, int Hk, int Hv, int Dv, int C, int maxc,
    const bf16* __restrict__ Th, const bf16* __restrict__ Tl, const bf16* __restrict__ Ph,
    const bf16* __restrict__ Pl, const float* __restrict__ fac, T* __restrict__ y, int keep) {
  constexpr bool PRECISE = std::is_same<T, float>::value;
  constexpr int BV = 16 * NW, NT = 64 * NW;
  constexpr int MT = CT / 16, CKB = CT / 32, DT = DK / 16, KB = DK / 32;
  constexpr int KTP = CT + 8;  // K^T row pitch in elements
  __shared__ __attribute__((aligned(16))) T KT[DK][KTP];
  __shared__ float fB[CT], fK[CT], fQ[CT], fD[CT];
  __shared__ float sGC;

  const int nvb = Dv / BV;
  const int pos = blockIdx.x / (Hv * nvb);
  const int s = scs[N_s + 1 + pos];  // longest sequences first
  const int rem = blockIdx.x - pos * (Hv * nvb);
  const int hv = rem / nvb;
  const int vb = rem - hv * nvb;
  const int64_t slot = cache_indices[s];
  if (slot < 0 || slot >= pool_size) return;
  int64_t b0, len;
  seq_bounds(cu, s, T_tot, b0, len);
  if (len <= 0) return;
  const int cbase = scs[s];
  // chunks past the workspace bound only exist for cu_seqlens outside the
  // contract; they are skipped rather than read out of bounds
  const int nch_all = static_cast<int>((len + C - 1) / C);
  const int nch = cbase + nch_all > maxc ? (maxc > cbase ? maxc - cbase : 0) : nch_all;
  const int hk = hv / (Hv / Hk);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, kg = lane >> 4;
  const int dv = vb * BV + w * 16 + l16;

  float* Sp = pool + (static_cast<size_t>(slot) * Hv + hv) * Dv * DK + static_cast<size_t>(dv) * DK;
  f32x4 S[DT];
#pragma unroll
  for (int m = 0; m < DT; ++m) S[m] = *reinterpret_cast<const f32x4*>(Sp + m * 16 + kg * 4);

  for (int ci = 0; ci < nch; ++ci) {
    const int c = cbase + ci;
    const int64_t t0 = b0 + static_cast<int64_t>(ci) * C;
    const int n = static_cast<int>(len - static_cast<int64_t>(ci) * C < C ? len - static_cast<int64_t>(ci) * C : C);
    const size_t mat = static_cast<size_t>(c) * Hv + hv;

    // ---- every global load of the chunk, issued before any of them is used.
    // Rows past the chunk's last token read that token again (a branch
    // around each load would serialise the loads) and are zeroed or get zero
    // factors, so they contribute nothing.
    // K^T staging: CT * DK/8 items of 8 elements, NSTG per thread (the last
    // round may be partial for small tiles: surplus threads load an item
    // again and skip its LDS write)
    constexpr int NITEMS = CT * (DK / 8);
    constexpr int NSTG = (NITEMS + NT - 1) / NT;
    T kst[NSTG][8];
#pragma unroll
    for (int it = 0; it < NSTG; ++it) {
      const int idx = min(tid + it * NT, NITEMS - 1), t = idx % CT, d8 = idx / CT;
      const T* src = k + (static_cast<size_t>(t0 + min(t, n - 1)) * Hk + hk) * DK + d8 * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) kst[it][e] = src[e];
    }
    Raw<T> kf[MT][KB], qf[MT][KB];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const size_t roff = (static_cast<size_t>(t0 + min(mt * 16 + l16, n - 1)) * Hk + hk) * DK;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        kf[mt][kb] = Raw<T>::load(k + roff, kb * 32, kg);
        qf[mt][kb] = Raw<T>::load(q + roff, kb * 32, kg);
      }
    }
    float vv[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vv[mt][r] = Act<T>::load(
            v + (static_cast<size_t>(t0 + min(mt * 16 + kg * 4 + r, n - 1)) * Hv + hv) * Dv + dv);
    // T (hi, lo) and P rows for the lower-triangular (mt, cb) blocks
    Raw<bf16> thf[MT][CKB], tlf[MT][CKB], phf[MT][CKB], plf[MT][CKB];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const size_t roff = mat * CT * CT + static_cast<size_t>(mt * 16 + l16) * CT;
#pragma unroll
      for (int cb = 0; cb <= mt / 2; ++cb) {
        thf[mt][cb] = Raw<bf16>::load(Th + roff, cb * 32, kg);
        tlf[mt][cb] = Raw<bf16>::load(Tl + roff, cb * 32, kg);
        phf[mt][cb] = Raw<bf16>::load(Ph + roff, cb * 32, kg);
        if constexpr (PRECISE) plf[mt][cb] = Raw<bf16>::load(Pl + roff, cb * 32, kg);
      }
    }
    float fvB = 0.f, fvK = 0.f, fvQ = 0.f, fvD = 0.f, fvC = 0.f;
    if (tid < CT) {
      const float* fp = fac + mat * (4 * CT + 4);
      fvB = fp[tid];
      fvK = fp[CT + tid];
      fvQ = fp[2 * CT + tid];
      fvD = fp[3 * CT + tid];
      fvC = fp[4 * CT];
    }

    __syncthreads();  // the previous chunk no longer reads K^T or the factors
#pragma unroll
    for (int it = 0; it < NSTG; ++it) {
      const int idx = tid + it * NT, t = idx % CT, d8 = idx / CT;
      if (NITEMS % NT == 0 || idx < NITEMS) {
#pragma unroll
        for (int e = 0; e < 8; ++e) KT[d8 * 8 + e][t] = t < n ? kst[it][e] : T(0);
      }
    }
    if (tid < CT) {
      fB[tid] = fvB;
      fK[tid] = fvK;
      fQ[tid] = fvQ;
      fD[tid] = fvD;
      if (tid == 0) sGC = fvC;
    }
    __syncthreads();

    // state operand over dk (hi/lo)
    bf16x8v Sh[KB], Sl[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) acc_operand(S[2 * kb], S[2 * kb + 1], Sh[kb], Sl[kb]);

    // X = K S (state-grade), Y = Q S (output-grade)
    f32x4 X[MT], Y[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      X[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      Y[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        bf16x8v akh, akl, aqh, aql;
        kf[mt][kb].operand(akh, akl);
        qf[mt][kb].operand(aqh, aql);
        X[mt] = mma(akh, Sh[kb], X[mt]);
        X[mt] = mma(akh, Sl[kb], X[mt]);
        Y[mt] = mma(aqh, Sh[kb], Y[mt]);
        if constexpr (PRECISE) {
          X[mt] = mma(akl, Sh[kb], X[mt]);
          Y[mt] = mma(aqh, Sl[kb], Y[mt]);
          Y[mt] = mma(aql, Sh[kb], Y[mt]);
        }
      }
    }

    // R = diag(beta) V - diag(beta gamma / |k|) X   (fB = fK = 0 past the last token)
    f32x4 R[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = mt * 16 + kg * 4 + r;
        R[mt][r] = fB[t] * vv[mt][r] - fK[t] * X[mt][r];
      }
    bf16x8v Rh[CKB], Rl[CKB];
#pragma unroll
    for (int cb = 0; cb < CKB; ++cb) acc_operand(R[2 * cb], R[2 * cb + 1], Rh[cb], Rl[cb]);

    // Delta = T R (T lower triangular: skip blocks above the diagonal)
    f32x4 D[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      D[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cb = 0; cb <= mt / 2; ++cb) {
        bf16x8v th, tl, unused;
        thf[mt][cb].operand(th, unused);
        tlf[mt][cb].operand(tl, unused);
        D[mt] = mma(th, Rh[cb], D[mt]);
        D[mt] = mma(th, Rl[cb], D[mt]);
        D[mt] = mma(tl, Rh[cb], D[mt]);
      }
    }

    // O = diag(gamma scale / |q|) Y + P Delta -> y
    bf16x8v Dh[CKB], Dl[CKB];
#pragma unroll
    for (int cb = 0; cb < CKB; ++cb) acc_operand(D[2 * cb], D[2 * cb + 1], Dh[cb], Dl[cb]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 O;
#pragma unroll
      for (int r = 0; r < 4; ++r) O[r] = fQ[mt * 16 + kg * 4 + r] * Y[mt][r];
#pragma unroll
      for (int cb = 0; cb <= mt / 2; ++cb) {
        bf16x8v ph, pl, unused;
        phf[mt][cb].operand(ph, unused);
        O = mma(ph, Dh[cb], O);
        if constexpr (PRECISE) {
          plf[mt][cb].operand(pl, unused);
          O = mma(ph, Dl[cb], O);
          O = mma(pl, Dh[cb], O);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = mt * 16 + kg * 4 + r;
        if (t < n) Act<T>::store(y + (static_cast<size_t>(t0 + t) * Hv + hv) * Dv + dv, O[r]);
      }
    }

    // S <- gamma_C S + K^T diag(exp(G_C - G) / |k|) Delta
    f32x4 Dp[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) Dp[mt][r] = fD[mt * 16 + kg * 4 + r] * D[mt][r];
    bf16x8v Eh[CKB], El[CKB];
#pragma unroll
    for (int cb = 0; cb < CKB; ++cb) acc_operand(Dp[2 * cb], Dp[2 * cb + 1], Eh[cb], El[cb]);
    const float gC = sGC;
#pragma unroll
    for (int m = 0; m < DT; ++m) {
      S[m] *= gC;
      const T* ktrow = &KT[m * 16 + l16][0];
#pragma unroll
      for (int cb = 0; cb < CKB; ++cb) {
        bf16x8v ah, al;
        Frag<T>::pi(ktrow, cb * 32, kg, ah, al);
        S[m] = mma(ah, Eh[cb], S[m]);
        S[m] = mma(ah, El[cb], S[m]);
        if constexpr (PRECISE) S[m] = mma(al, Eh[cb], S[m]);
      }
    }
  }

#pragma unroll
  for (int m = 0; m < DT; ++m)
    if (!keep) *reinterpret_cast<f32x4*>(Sp + m * 16 + kg * 4) = S[m];  // keep: the slot is read only
}

// ----------------------------------------------------------------------------
// 3b. Helpers of the bf16 chunk loop (section 5): buffer descriptors,
// asynchronous buffer->LDS copies, LDS operand reads (fragment and
// transposing), hi/lo splits for 16x16x16 products.

typedef __attribute__((address_space(3))) void* lds_vptr;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4p;

// A copy offset beyond every bound used here: the copy fills zeros.
constexpr uint32_t kOOB = 0x7ffffff0u;

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor of `bytes` bytes at `base`: stride 0 (raw byte offsets),
// 32-bit data format; offsets at or past `bytes` read zero / drop the write.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{static_cast<int>(static_cast<uint32_t>(a)), static_cast<int>((a >> 32) & 0xffffu),
               static_cast<int>(bytes), 0x00020000};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_vptr)(const_cast<void*>(p))));
}

// Asynchronous 16-byte-per-lane copy from the buffer to LDS: lane i's bytes
// land at lds + 16 i.  Written as asm so that the compiler does not track
// it: every wait for these copies is explicit (handover below), and the
// compiler's own conservative waits would otherwise stall on them.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc) : "m0");
}

// Buffer resource for stores (and loads) dropped at or past `bytes`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(bytes), 0x00020000);
}

// A tile of ROWS rows; row r is ITEMS 16-byte items at byte offset
// r * src_stride of the source, stored in LDS with a pitch of PITCH bf16.
// SKEW: rows with bit 3 set start one 16-byte slot (8 bf16) later.
// The copy runs in 1 KiB blocks of 64 consecutive 16-byte LDS slots, dealt
// round-robin to the NW waves; each lane's source offset per block is fixed
// for the whole sequence (only the descriptor changes per chunk).
template <int ROWS, int ITEMS, int PITCH, int NW, bool SKEW = false>
struct TileCopy {
  static constexpr int SPR = PITCH / 8;                 // LDS slots per row
  static constexpr int NBLK = (ROWS * SPR + 63) / 64;
  static constexpr int ELEMS = NBLK * 512;              // LDS bf16 to reserve
  static constexpr int PER = (NBLK + NW - 1) / NW;      // blocks of the busiest wave
  static constexpr int MIN = NBLK / NW;                 // blocks of every wave
  static_assert(PITCH % 8 == 0 && PITCH >= 8 * (ITEMS + SKEW), "pitch");
  uint32_t off[PER];
  __device__ __forceinline__ void init(int w, int lane, uint32_t src_stride) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int slot = (j * NW + w) * 64 + lane;
      const int row = slot / SPR, item = slot - row * SPR - (SKEW ? (row >> 3) & 1 : 0);
      const bool copy = row < ROWS && item >= 0 && item < ITEMS;
      off[j] = copy ? static_cast<uint32_t>(row) * src_stride + item * 16 : kOOB;
    }
  }
  // the wave's j-th block (none past the tile)
  __device__ __forceinline__ void issue_one(i32x4 r, void* tile, int w, int j) const {
    if (j < MIN || (j < PER && j * NW + w < NBLK)) dma16(r, lds_addr(tile) + (j * NW + w) * 1024, off[j]);
  }
  __device__ __forceinline__ void issue(i32x4 r, void* tile, int w) const {
#pragma unroll
    for (int j = 0; j < PER; ++j) issue_one(r, tile, w, j);
  }
};

// Wait until at most `VM` of this wave's vector-memory operations are in
// flight and its LDS reads are done, then meet the workgroup.  The asm is a
// compiler memory barrier too, so no LDS access moves across it.
template <int VM>
__device__ __forceinline__ void handover() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VM) : "memory");
}
__device__ __forceinline__ void lds_handover() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// "pi"-order operand from row `row` of a padded LDS tile (see acc_operand).
// The two halves are separate 8-byte reads (volatile, so they are not fused
// into one paired read): on gfx950 a half-wave of single 8-byte reads over
// 16 rows at an odd 16-byte-slot pitch hits every bank once, while the
// paired form serves the two addresses of a lane together and conflicts.
template <int PITCH>
__device__ __forceinline__ bf16x8v lds_pi(const bf16* tile, int row, int k0, int kg) {
  const bf16* p = tile + row * PITCH + k0 + kg * 4;
  typedef const volatile __attribute__((address_space(3))) u32x2* lds_u32x2p;
  const u32x2 a = *(lds_u32x2p)(p);
  const u32x2 b = *(lds_u32x2p)(p + 16);
  return __builtin_bit_cast(bf16x8v, u32x4{a.x, a.y, b.x, b.y});
}

// Transposing read: for lane (l16, kg) whose address is
//   tile + (r0 + kg*4 + l16/4) * PITCH + c0 + 4*(l16%4),
// element e of the result is tile[r0 + kg*4 + e][c0 + l16].
__device__ __forceinline__ s16x4 lds_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4p)(p));
}

// "pi"-order operand of M^T from a tile holding M row-major: rows r and
// r + 16 of the tile (r = k0 + kg*4 + l16/4) at column c (= m0 + 4*(l16%4))
// give elements 0..3 and 4..7, i.e. M[k0 + kg*4 + e][m0 + l16] and
// M[k0 + 16 + kg*4 + e][m0 + l16].
template <int PITCH>
__device__ __forceinline__ bf16x8v lds_trT(const bf16* tile, int r, int c) {
  const bf16* p = tile + r * PITCH + c;
  const s16x4 lo4 = lds_tr(p), hi4 = lds_tr(p + 16 * PITCH);
  return __builtin_bit_cast(bf16x8v, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Compact upper-triangular storage of a CT x CT bf16 matrix (bf16
// activations): only the 16x16 blocks (a, b) with a <= b, block-row-major,
// each block 16 rows of 32 bytes.  Block (a, b) starts at element
// 256 * tri_block<CT>(a, b).
template <int CT>
__host__ __device__ constexpr int tri_blocks() { return (CT / 16) * (CT / 16 + 1) / 2; }
template <int CT>
__device__ __forceinline__ constexpr int tri_block(int a, int b) {
  return a * (CT / 16) - a * (a - 1) / 2 + (b - a);
}

// The same operand of M^T from M in compact upper-triangular blocks
// (tri_block): rows 32 cb + kg*4 + e and 32 cb + 16 + kg*4 + e of M at
// column 16 mt + l16; lane_off = (kg*4 + l16/4) * 16 + 4*(l16%4).  The second
// half is zero when block (2cb + 1, mt) lies below the diagonal.  Within a
// block, the 8 rows of a half-wave's read are 256 contiguous bytes.
template <int CT>
__device__ __forceinline__ bf16x8v tri_trT(const bf16* tile, int cb, int mt, int lane_off) {
  const s16x4 lo4 = lds_tr(tile + tri_block<CT>(2 * cb, mt) * 256 + lane_off);
  s16x4 hi4 = {0, 0, 0, 0};
  if (2 * cb + 1 <= mt) hi4 = lds_tr(tile + tri_block<CT>(2 * cb + 1, mt) * 256 + lane_off);
  return __builtin_bit_cast(bf16x8v, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ float bf16_bits_to_f32(short x) {
  return __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(x)) << 16);
}

// 16x16x16 products of fp32 fragments split into bf16 hi + lo, three per
// product (the lo x lo term is below fp32 rounding).
// A: row l16, k = kg*4 + e;  B and C: column l16, k/row = kg*4 + e.
__device__ __forceinline__ void split4(f32x4 x, s16x4& h, s16x4& l) {
  uint32_t h0, l0, h1, l1;
  split_pair(x[0], x[1], h0, l0);
  split_pair(x[2], x[3], h1, l1);
  h = __builtin_bit_cast(s16x4, u32x2{h0, h1});
  l = __builtin_bit_cast(s16x4, u32x2{l0, l1});
}
// C += A B with the right operand already split (bh, bl).
__device__ __forceinline__ f32x4 mm3_rb(f32x4 a, s16x4 bh, s16x4 bl, f32x4 c) {
  s16x4 ah, al;
  split4(a, ah, al);
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, c, 0, 0, 0);
  return c;
}
// A B with the left operand already split (ah, al), from a zero accumulator.
__device__ __forceinline__ f32x4 mm3_la(s16x4 ah, s16x4 al, f32x4 b) {
  s16x4 bh, bl;
  split4(b, bh, bl);
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, c, 0, 0, 0);
  return c;
}

// ----------------------------------------------------------------------------
// The conv prologue of one chunk inside its WY wave (regolith `gdn.metal`,
// header comment and the conv/SiLU block of its kernel): for every channel c
// of key head hk's q and k heads and of the v heads of its group, and every
// token t of the chunk,
//   pre = x[t-3] W[c][0] + x[t-2] W[c][1] + x[t-1] W[c][2] + x[t] W[c][3],
//   out = pre sigmoid(pre),
// with inputs before the sequence's first token taken from the slot's
// history -- the formula, operation order and SiLU of gdn_conv_silu, so the
// outputs are the same bits.  Channels go in groups of 8 (one 16-byte load
// or store per lane and row), consecutive lanes on consecutive groups.  With
// 64 groups or more, lane l first takes group l through all of the chunk's
// rows (the window rolls on, the weights load once); the remaining groups
// (all of them below 64) go as (group, run of 16 rows) items dealt over the
// lanes.  Both loops are software pipelined: the next run's rows (and an
// item's window rows and weights) load while the current run computes, so
// the wave's loads stay in flight through its arithmetic (the kernel holds
// two waves per SIMD, too few to hide a load's latency otherwise).  The wave
// of a sequence's first chunk is the only one that reads the slot's history
// for these channels; after those reads it writes the new history (the
// newest three of history and inputs), so no later kernel is needed for it.
struct ConvItem {
  int ch;       // first channel of the group in the raw row
  int ostride;  // elements per output row
  int r0;       // first row of the run in the chunk
  bf16* out;    // the group's output column
};

template <int DK>
__device__ __forceinline__ void conv_chunk(const ConvIn& cv, int s, int64_t b0, int64_t len, int64_t t0, int n,
                                           int Hk, int Hv, int hk, int HG) {
  constexpr int NGQ = DK / 8;                 // 8-channel groups of one q (or k) head
  const int NG = 2 * NGQ + HG * cv.Dv / 8;    // groups of the key head's channels
  const int C = 2 * Hk * DK + Hv * cv.Dv;
  const bool first = t0 == b0;
  const int64_t slot = cv.ci[s];
  const bool slot_ok = first && slot >= 0 && slot < cv.pool_size;

  auto describe = [&](int gi, int r0) __attribute__((always_inline)) {
    ConvItem d;
    d.r0 = r0;
    if (gi < NGQ) {
      d.ch = hk * DK + gi * 8;
      d.out = cv.q + hk * DK + gi * 8;
      d.ostride = Hk * DK;
    } else if (gi < 2 * NGQ) {
      d.ch = (Hk + hk) * DK + (gi - NGQ) * 8;
      d.out = cv.k + hk * DK + (gi - NGQ) * 8;
      d.ostride = Hk * DK;
    } else {
      const int vc = hk * HG * cv.Dv + (gi - 2 * NGQ) * 8;
      d.ch = 2 * Hk * DK + vc;
      d.out = cv.v + vc;
      d.ostride = Hv * cv.Dv;
    }
    return d;
  };
  auto row = [&](int64_t p, int ch) __attribute__((always_inline)) {
    return *reinterpret_cast<const uint4*>(cv.x + static_cast<size_t>(p) * C + ch);
  };
  // eight rows of the run from row r (clamped to the chunk's last token)
  auto load8 = [&](const ConvItem& d, int r, uint4 (&X)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) X[j] = row(t0 + min(d.r0 + r + j, n - 1), d.ch);
  };
  // the three window rows before the run.  Only a sequence's first run has
  // rows before the sequence (all three, as a chunk holds at least 8 rows);
  // its loads are clamped to a row of the sequence and replaced below, so
  // that no select waits for them here.
  auto load_win = [&](const ConvItem& d, uint4 (&Wr)[3]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      const int64_t p = t0 + d.r0 - 3 + m;
      Wr[m] = row(p > b0 ? p : b0, d.ch);
    }
  };
  auto load_w = [&](const ConvItem& d, f32x4 (&w)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = *reinterpret_cast<const f32x4*>(cv.W + static_cast<size_t>(d.ch + i) * 4);
  };
  auto unpack = [](const uint4& x, float (&f)[8]) __attribute__((always_inline)) {
    const uint32_t u[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(u[i] << 16);
      f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  };
  // rows r .. r+7 of the run from X, the window rolling along
  auto compute8 = [&](const ConvItem& d, int r, const uint4 (&X)[8], const f32x4 (&w)[8], float (&win)[3][8])
      __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float cur[8];
      unpack(X[j], cur);
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float y2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int c8 = 2 * i + e;
          float pre = win[0][c8] * w[c8][0];
          pre = fmaf(win[1][c8], w[c8][1], pre);
          pre = fmaf(win[2][c8], w[c8][2], pre);
          pre = fmaf(cur[c8], w[c8][3], pre);
          y2[e] = silu_fast(pre);
        }
        o[i] = pk(y2[0], y2[1]);  // both to bf16 (nearest even) in one conversion
      }
      // rows past the chunk (computed from repeated inputs) go to the trash
      // slot: a select, not a branch, whose join would make the compiler
      // wait for every load in flight
      const int rr = d.r0 + r + j;
      bf16* dst = rr < n ? d.out + static_cast<size_t>(t0 + rr) * d.ostride : cv.trash;
      *reinterpret_cast<uint4*>(dst) = uint4{o[0], o[1], o[2], o[3]};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        win[0][i] = win[1][i];
        win[1][i] = win[2][i];
        win[2][i] = cur[i];
      }
    }
  };

  // HIST: a sequence's first chunk (history reads and the new history).
  // The loop is built twice so that the other chunks carry no history loads:
  // under a lane-dependent branch those would make the compiler wait for
  // every load in flight (the next item's rows too) where the branches join.
  // the slot's new history for channel group ch: inputs b0+len-3 ..
  // b0+len-1, entries before the sequence from the old history (read
  // before by this lane, and again here before the store)
  auto new_history = [&](int ch) __attribute__((always_inline)) {
    float nh[8][3];
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      const int64_t p = b0 + len - 3 + m;
      float f[8];
      if (p >= b0) {
        unpack(row(p, ch), f);
      } else {
        const float* h = cv.hist + (static_cast<size_t>(slot) * C + ch) * 3 + (p - b0 + 3);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = h[3 * i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) nh[i][m] = f[i];
    }
    float* h = cv.hist + (static_cast<size_t>(slot) * C + ch) * 3;
#pragma unroll
    for (int q4 = 0; q4 < 6; ++q4)
      *reinterpret_cast<f32x4*>(h + 4 * q4) =
          f32x4{nh[(4 * q4) / 3][(4 * q4) % 3], nh[(4 * q4 + 1) / 3][(4 * q4 + 1) % 3],
                nh[(4 * q4 + 2) / 3][(4 * q4 + 2) % 3], nh[(4 * q4 + 3) / 3][(4 * q4 + 3) % 3]};
  };
  // the window of a sequence's first run: the slot's history (zeros for a
  // slot out of range)
  auto history_window = [&](int ch, float (&win)[3][8]) __attribute__((always_inline)) {
    const float* h = cv.hist + (static_cast<size_t>(slot) * C + ch) * 3;
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
      for (int i = 0; i < 8; ++i) win[m][i] = slot_ok ? h[3 * i + m] : 0.f;
  };

  // Groups 0..63 when the key head has at least 64: lane = group, all of
  // the chunk's rows in order, the window rolling from run to run and the
  // weights loaded once; the next run's eight-row halves load while the
  // current ones compute.
  const int g_roll = NG >= 64 ? 64 : 0;
  auto rolling = [&](auto hist_tag) __attribute__((always_inline)) {
    constexpr bool HIST = decltype(hist_tag)::value;
    ConvItem d = describe(threadIdx.x, 0);
    uint4 A[8], B[8], Wr[3];
    f32x4 w[8];
    if constexpr (!HIST) load_win(d, Wr);
    load8(d, 0, A);
    load_w(d, w);
    load8(d, 8, B);
    float win[3][8];
    if constexpr (HIST) {
      history_window(d.ch, win);
    } else {
#pragma unroll
      for (int m = 0; m < 3; ++m) unpack(Wr[m], win[m]);
    }
    for (int r0 = 0; r0 < n; r0 += 16) {
      d.r0 = r0;
      const bool more = r0 + 16 < n;
      compute8(d, 0, A, w, win);
      if (more) {
        ConvItem nx = d;
        nx.r0 = r0 + 16;
        load8(nx, 0, A);
      }
      compute8(d, 8, B, w, win);
      if (more) {
        ConvItem nx = d;
        nx.r0 = r0 + 16;
        load8(nx, 8, B);
      }
    }
    if (HIST && slot_ok && !cv.keep) new_history(d.ch);
  };

  // The other groups (all of them below 64) as (group, run of 16 rows)
  // items dealt over the lanes, pipelined one item ahead.
  const int NGr = NG - g_roll;
  const int total = NGr * ((n + 15) >> 4);
  auto item_of = [&](int it) __attribute__((always_inline)) {
    const int sg = it / NGr;
    return describe(g_roll + (it - sg * NGr), sg * 16);
  };
  auto items = [&](auto hist_tag) __attribute__((always_inline)) {
  constexpr bool HIST = decltype(hist_tag)::value;
  int it = threadIdx.x;
  ConvItem cur{};
  uint4 A[8], B[8], Wr[3];
  f32x4 w[8];
  if (it < total) {
    cur = item_of(it);
    load_win(cur, Wr);
    load8(cur, 0, A);
    load_w(cur, w);
    load8(cur, 8, B);
  }
  for (; it < total; it += 64) {
    const bool more = it + 64 < total;
    const ConvItem nxt = more ? item_of(it + 64) : cur;
    // the window of this run: inputs, or (a sequence's first rows) history
    float win[3][8];
#pragma unroll
    for (int m = 0; m < 3; ++m) unpack(Wr[m], win[m]);
    const bool hist_rows = HIST && cur.r0 == 0;  // t0 - 3 + m < b0 = t0 for every m
    if (hist_rows) history_window(cur.ch, win);
    uint4 Wr2[3];
    f32x4 w2[8];
    compute8(cur, 0, A, w, win);
    if (more) {
      load_win(nxt, Wr2);
      load8(nxt, 0, A);
      load_w(nxt, w2);
    }
    compute8(cur, 8, B, w, win);
    if (more) load8(nxt, 8, B);
    if (hist_rows && slot_ok && !cv.keep) new_history(cur.ch);
    if (more) {
      cur = nxt;
#pragma unroll
      for (int m = 0; m < 3; ++m) Wr[m] = Wr2[m];
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = w2[i];
    }
  }
  };
  if (first) {
    if (g_roll) rolling(std::true_type{});
    items(std::true_type{});
  } else {
    if (g_roll) rolling(std::false_type{});
    items(std::false_type{});
  }
}

// ----------------------------------------------------------------------------
// 4. bf16 WY pass: one independent wave per (chunk, key head).
//
// The wave holds every K and Q fragment of the chunk in registers (rows past
// the last token read it again; their factors are zero), takes the row norms
// from them and the Gram blocks K K^T and Q K^T on MFMA, once for the value
// heads of the key head.  Then, per value head: the gate scan (lane = token),
// the record [gamma/|k| | gamma scale/|q| | exp(G_C - G)/|k| | gamma_C,0,0,0],
// A and P from the Gram blocks, and T = (I + A)^-1 built blockwise: the
// 16x16 diagonal blocks D_b by forward substitution in fp32 (lane = (block,
// column)), then level by level
//   T_jj = D_j,   T_ij = -D_i sum_{k=j}^{i-1} A_ik T_kj   (i > j)
// with 16x16x16 MFMA on hi/lo-split operands.  T diag(beta) is written, so
// that Delta = T diag(beta) (V - diag(gamma/|k|) K S) needs no beta in the
// chunk loop: transposed as bf16 hi/lo, and P transposed as bf16 (each
// lane's four accumulator rows are then one 8-byte store), blocks on and
// below the diagonal only, in the compact upper-triangular form of the
// transposes (tri_block).  The lanes of the one wave hand each other data
// through LDS (norms and gates, A, the diagonal inverses): a __syncthreads()
// at each hand-off waits for no other wave but keeps the compiler from
// serving a lane's read from what that lane itself stored earlier.  The LDS
// footprint (19 KB) and a register budget of 256 (two waves per SIMD,
// requested from the compiler) let eight waves share a CU.
//
// COMBA: the Comba forward (read key p, write key k; KBench
// `comba_decode_step` spec run over every token).  Its chunk form is the
// same with A_ij = beta_i exp(G_i - G_j) p_i . k_j (the read key of the
// later token against the write key of the earlier one) and the read term
// R = V - diag(gamma) P S; keys are taken as given (no norms) and q is only
// scaled.  The Gram blocks are then P K^T instead of K K^T, and beta comes
// in the activation dtype.

__device__ __forceinline__ float ld_beta(const float* b, size_t i) { return b[i]; }
__device__ __forceinline__ float ld_beta(const bf16* b, size_t i) { return bf16_to_f32(b[i]); }

// RAW: the gates come from the raw inputs a, b [T, Hv] (bf16), A_log and
// dt_bias [Hv] (gates_of), formed where the gate scan needs them, instead
// of from g and beta.
//
// CONV (with RAW): the wave first runs the conv prologue of its chunk's
// channels (conv_chunk), writing the q, k and v the chunk loop reads, and
// then takes its K and Q fragments from those rows (written by this wave,
// so a workgroup barrier orders them).
template <int DK, int CT, bool COMBA = false, typename BT = float, bool RAW = false, bool CONV = false>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void gdn_wy_wave_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ pr,
    const float* __restrict__ g, const BT* __restrict__ beta, const int64_t* __restrict__ cu,
    const int* __restrict__ scs,
    int N_s, int64_t T_tot, int Hk, int Hv, int C, float scale, int l2norm, bf16* __restrict__ Th,
    bf16* __restrict__ Tl, bf16* __restrict__ Ph, float* __restrict__ fac, RawGates rg, int own_map,
    int* __restrict__ map_out, int wg_per_seq, int num_cu, int allow_split, FixedBatch fb) {
  static_assert(!RAW || !COMBA, "raw gates: GDN only");
  static_assert(!CONV || RAW, "the conv prologue comes with raw gates");
  constexpr int MT = CT / 16, KB = DK / 32;
  constexpr int NPAIR = MT * (MT + 1) / 2, FSTR = 3 * CT + 4;
  __shared__ __attribute__((aligned(16))) float sG[CT], sRK[CT], sRQ[CT], sB[CT];
  // 16x16 fp32 blocks with a row pitch of 20; a block stride of 324 floats
  // puts the four diagonal blocks (read together by lane groups of the
  // diagonal solve) on distinct banks
  __shared__ __attribute__((aligned(16))) float sA[NPAIR][324];
  __shared__ __attribute__((aligned(16))) float sD[MT][324];

  const int c = blockIdx.x / Hk;
  const int hk = blockIdx.x - c * Hk;
  int lo = 0, cbase;  // the sequence holding chunk c and its first chunk
  if (own_map) {
    // This launch also makes the chunk map the chunk loop reads (its last
    // workgroup, in the storage of sA); every other wave finds its chunk
    // itself: by division in a fixed-length batch (whose cu_seqlens the last
    // workgroup is still writing), else from cu_seqlens, N_s <= 64, a lane
    // per sequence.
    static_assert(sizeof(MapLds<64>) <= sizeof(sA), "the chunk map's LDS lives in sA");
    if (blockIdx.x == gridDim.x - 1) {
      if (fb.T > 0)
        fixed_map_body(fb, N_s, C, map_out, wg_per_seq, num_cu, allow_split);
      else
        chunk_map_body<64>(*reinterpret_cast<MapLds<64>*>(&sA[0][0]), cu, N_s, T_tot, C, map_out, wg_per_seq,
                           num_cu, allow_split);
      return;
    }
  }
  if (own_map && fb.T > 0) {
    const int per = static_cast<int>((fb.T + C - 1) / C);
    lo = c / per;
    if (lo >= N_s) return;
    cbase = lo * per;
  } else if (own_map) {
    const int ln = threadIdx.x;
    int nl = 0;
    if (ln < N_s) {
      int64_t bx, lx;
      seq_bounds(cu, ln, T_tot, bx, lx);
      nl = static_cast<int>((lx + C - 1) / C);
    }
    int incl = nl;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(incl, off);
      if (ln >= off) incl += u;
    }
    const int excl = incl - nl;
    if (c >= __shfl(incl, 63)) return;
    lo = 63 - __clzll(__ballot(ln < N_s && excl <= c));  // largest such s
    cbase = __shfl(excl, lo);
  } else {
    if (c >= scs[N_s]) return;
    int hi = N_s;  // largest s with scs[s] <= c
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (scs[mid] <= c) lo = mid; else hi = mid;
    }
    cbase = scs[lo];
  }
  int64_t b0, len;
  if (fb.T > 0) {
    b0 = static_cast<int64_t>(lo) * fb.T;
    len = fb.T;
  } else {
    seq_bounds(cu, lo, T_tot, b0, len);
  }
  const int64_t j0 = static_cast<int64_t>(c - cbase) * C;
  const int64_t t0 = b0 + j0;
  const int n = static_cast<int>(len - j0 < C ? len - j0 : C);
  const int HG = Hv / Hk;
  const int lane = threadIdx.x, l16 = lane & 15, kg = lane >> 4;
  const bool ok = lane < n;
  const size_t tg = static_cast<size_t>(t0 + min(lane, n - 1)) * Hv + hk * HG;  // gates of token `lane`
  if constexpr (CONV) {
    conv_chunk<DK>(rg.cv, lo, b0, len, t0, n, Hk, Hv, hk, HG);
    __syncthreads();  // the convolved rows, stored by other lanes, before the fragment loads below
  }
  // where the fragments come from: the inputs, or the rows just convolved
  const bf16* const qsrc = CONV ? rg.cv.q : q;
  const bf16* const ksrc = CONV ? rg.cv.k : k;

  // gates of the first value head, then the K fragments: lane (l16, kg)
  // holds row I*16 + l16, elements kb*32 + kg*8 .. +7 (the same order on
  // both sides of every Gram product); Q fragments follow one row block at a
  // time, as the Q K^T blocks of that row need them
  // gates of value head hk*HG + j for this lane's token
  auto gates = [&](int j, float& gv, float& bv) __attribute__((always_inline)) {
    if constexpr (RAW) {
      const int h = hk * HG + j;
      gates_of(bf16_to_f32(rg.a[tg + j]) + rg.dt_bias[h], rg.A_log[h], bf16_to_f32(rg.b[tg + j]), gv, bv);
    } else {
      gv = g[tg + j];
      bv = ld_beta(beta, tg + j);
    }
  };
  float gl, bl;
  gates(0, gl, bl);
  auto row_off = [&](int I) __attribute__((always_inline)) {
    return (static_cast<size_t>(t0 + min(I * 16 + l16, n - 1)) * Hk + hk) * DK + kg * 8;
  };
  bf16x8v kf[MT][KB];
#pragma unroll
  for (int I = 0; I < MT; ++I)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      kf[I][kb] = __builtin_bit_cast(bf16x8v, *reinterpret_cast<const uint4*>(ksrc + row_off(I) + kb * 32));
  // row sums of squares: 8 elements per lane and k-block, then over kg
  auto sumsq = [&](const bf16x8v (&f)[KB]) __attribute__((always_inline)) {
    float a = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const u32x4 wv = __builtin_bit_cast(u32x4, f[kb]);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float x0 = __uint_as_float(wv[p] << 16), x1 = __uint_as_float(wv[p] & 0xffff0000u);
        a += x0 * x0 + x1 * x1;
      }
    }
    a += __shfl_xor(a, 16);
    return a + __shfl_xor(a, 32);
  };
  // Gram blocks (I >= J), kept for every value head of the group; lane
  // t = kg*16 + l16 takes row t's sums of squares from row block kg
  f32x4 gk[NPAIR], gq[NPAIR];
  float mk = 0.f, mq = 0.f;
  // the Q (and Comba's P) fragments of row block I + 1 are in flight while
  // the Gram blocks of row block I run
  bf16x8v qn[KB], pn[KB];
  auto load_qp = [&](int I) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      qn[kb] = __builtin_bit_cast(bf16x8v, *reinterpret_cast<const uint4*>(qsrc + row_off(I) + kb * 32));
      if constexpr (COMBA)
        pn[kb] = __builtin_bit_cast(bf16x8v, *reinterpret_cast<const uint4*>(pr + row_off(I) + kb * 32));
    }
  };
  load_qp(0);
#pragma unroll
  for (int I = 0; I < MT; ++I) {
    bf16x8v qf[KB], lf[KB];  // lf: the left factor of the A Gram blocks (k, or Comba's p)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      qf[kb] = qn[kb];
      lf[kb] = COMBA ? pn[kb] : kf[I][kb];
    }
    if (I + 1 < MT) load_qp(I + 1);
    if constexpr (!COMBA) {
      const float sk = sumsq(kf[I]), sq = sumsq(qf);
      mk = kg == I ? sk : mk;
      mq = kg == I ? sq : mq;
    }
#pragma unroll
    for (int J = 0; J <= I; ++J) {
      const int pidx = I * (I + 1) / 2 + J;
      gk[pidx] = f32x4{0.f, 0.f, 0.f, 0.f};
      gq[pidx] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        gk[pidx] = mma(lf[kb], kf[J][kb], gk[pidx]);
        gq[pidx] = mma(qf[kb], kf[J][kb], gq[pidx]);
      }
    }
  }
  const bool nrm = !COMBA && l2norm;
  const float rk = ok ? (nrm ? 1.0f / sqrtf(mk + kNormEps) : 1.0f) : 0.f;
  const float rq = ok ? scale * (nrm ? 1.0f / sqrtf(mq + kNormEps) : 1.0f) : 0.f;
  if (lane < CT) {
    sRK[lane] = rk;
    sRQ[lane] = rq;
  }

  for (int j = 0; j < HG; ++j) {
    const int hv = hk * HG + j;
    const size_t mat = static_cast<size_t>(c) * Hv + hv;
    float G = ok ? gl : 0.f;
    const float bt = ok ? bl : 0.f;
    if (j + 1 < HG) gates(j + 1, gl, bl);  // the next head's gates, in flight during this head
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float up = __shfl_up(G, off);
      if (lane >= off) G += up;
    }
    // the prefix in base 2 (G log2 e), so that each decay below is one exp2
    const float G2 = G * 1.44269504088896341f;
    const float GC2 = __shfl(G2, CT - 1);
    if (lane < CT) {
      const float gam = __builtin_amdgcn_exp2f(G2);
      float* r = fac + mat * FSTR;
      r[lane] = gam * rk;
      r[CT + lane] = gam * rq;
      r[2 * CT + lane] = __builtin_amdgcn_exp2f(GC2 - G2) * rk;
      if (lane < 4) r[3 * CT + lane] = lane == 0 ? __builtin_amdgcn_exp2f(GC2) : 0.f;
      sG[lane] = G2;
      sB[lane] = bt;
    }
    __syncthreads();  // norms and gates -> every lane

    // ---- A (LDS, fp32) and P (global, bf16, transposed) from the Gram blocks
    bf16* th = Th + mat * NPAIR * 256;
    bf16* tl = Tl + mat * NPAIR * 256;
    bf16* ph = Ph + mat * NPAIR * 256;
    // A_ij = beta_i/|k_i| (k_i . k_j)/|k_j| e^(G_i - G_j) below the diagonal;
    // P_ij = scale/|q_i| (q_i . k_j)/|k_j| e^(G_i - G_j) on and below it
#pragma unroll
    for (int I = 0; I < MT; ++I) {
      const f32x4 Gi = *reinterpret_cast<const f32x4*>(sG + I * 16 + kg * 4);
      const f32x4 rki = *reinterpret_cast<const f32x4*>(sRK + I * 16 + kg * 4);
      const f32x4 rqi = *reinterpret_cast<const f32x4*>(sRQ + I * 16 + kg * 4);
      const f32x4 bki = *reinterpret_cast<const f32x4*>(sB + I * 16 + kg * 4) * rki;
#pragma unroll
      for (int J = 0; J <= I; ++J) {
        const int pidx = I * (I + 1) / 2 + J;
        const int jj = J * 16 + l16;
        const float Gj = sG[jj], rkj = sRK[jj];
        s16x4 pv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ii = I * 16 + kg * 4 + r;
          const float t = jj <= ii ? __builtin_amdgcn_exp2f(Gi[r] - Gj) * rkj : 0.f;  // decay / |k_j|
          sA[pidx][(kg * 4 + r) * 20 + l16] = jj < ii ? bki[r] * t * gk[pidx][r] : 0.f;
          pv[r] = __builtin_bit_cast(short, (__bf16)(rqi[r] * t * gq[pidx][r]));
        }
        // P^T row jj, columns I*16 + kg*4 .. +3: block (J, I), row l16
        *reinterpret_cast<s16x4*>(ph + tri_block<CT>(J, I) * 256 + l16 * 16 + kg * 4) = pv;
      }
    }

    __syncthreads();  // A -> the solving lanes

    // ---- diagonal blocks: lane (b, cc) solves column cc of (I + A_bb)^-1
    {
      const int b = lane >> 4, cc = l16;
      if (b < MT) {
        const float* Ab = sA[b * (b + 1) / 2 + b];
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float a0 = (i == cc) ? 1.f : 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
          for (int jx = 0; jx + 3 < i; jx += 4) {
            const f32x4 ar = *reinterpret_cast<const f32x4*>(Ab + i * 20 + jx);
            a0 -= ar.x * x[jx];
            a1 -= ar.y * x[jx + 1];
            a2 -= ar.z * x[jx + 2];
            a3 -= ar.w * x[jx + 3];
          }
#pragma unroll
          for (int jx = i & ~3; jx < i; ++jx) a0 -= Ab[i * 20 + jx] * x[jx];
          x[i] = (a0 + a1) + (a2 + a3);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sD[b][i * 20 + cc] = x[i];
      }
    }

    __syncthreads();  // D -> every lane

    // ---- block columns of T diag(beta), the form the chunk loop reads.  The
    // block recurrence T_i,jb = -D_i sum_kk A_i,kk T_kk,jb is linear in each
    // block column, so scaling the diagonal blocks D_jb by the column's beta
    // scales the whole column; each block's hi/lo split, made once for its
    // store, is then also its operand in the later products of the column.
    s16x4 Th_[MT][MT], Tl_[MT][MT];  // accumulator layout: column l16, rows kg*4 .. +3
    auto put_T = [&](int i, int jb, f32x4 t) __attribute__((always_inline)) {
      split4(t, Th_[i][jb], Tl_[i][jb]);
      const int off = tri_block<CT>(jb, i) * 256 + l16 * 16 + kg * 4;  // T^T row jb*16 + l16
      *reinterpret_cast<s16x4*>(th + off) = Th_[i][jb];
      *reinterpret_cast<s16x4*>(tl + off) = Tl_[i][jb];
    };
#pragma unroll
    for (int jb = 0; jb < MT; ++jb) {
      // D_jb diag(beta) in accumulator layout
      const float bc = sB[jb * 16 + l16];
      f32x4 t;
#pragma unroll
      for (int r = 0; r < 4; ++r) t[r] = sD[jb][(kg * 4 + r) * 20 + l16] * bc;
      put_T(jb, jb, t);
    }
    // D_i as the left operand (row l16, k = kg*4 + e), split once per block
    s16x4 Dh_[MT], Dl_[MT];
#pragma unroll
    for (int i = 1; i < MT; ++i) split4(*reinterpret_cast<const f32x4*>(&sD[i][l16 * 20 + kg * 4]), Dh_[i], Dl_[i]);
    // level by level (i - jb = 1, 2, ...) so the columns' chains interleave
#pragma unroll
    for (int d = 1; d < MT; ++d)
#pragma unroll
      for (int jb = 0; jb + d < MT; ++jb) {
        const int i = jb + d;
        f32x4 M = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = jb; kk < i; ++kk)
          M = mm3_rb(*reinterpret_cast<const f32x4*>(&sA[i * (i + 1) / 2 + kk][l16 * 20 + kg * 4]), Th_[kk][jb],
                     Tl_[kk][jb], M);
        put_T(i, jb, -mm3_la(Dh_[i], Dl_[i], M));
      }
    __syncthreads();  // this head's reads of A, D and the gates before the next head's writes
  }
}

// ----------------------------------------------------------------------------
// 5. bf16 chunk loop: one workgroup per (sequence, value head, BV = 16 * NW
// value columns), a wave per 16 columns, state in MFMA accumulators.
//
// Chunk operands reach LDS by asynchronous buffer->LDS copies.  K, Q, T
// hi/lo, P and the factor record are double-buffered and copied for chunk
// ci+1 when step ci starts; V is copied right after the phase that reads it.
// Per step (products that do not depend on each other share a phase, so
// their MFMA chains interleave):
//   A: X = K S and Y = Q S (S as hi + lo);  R = V - (gamma/|k|) X
//      -- barrier, copy V (ci+1)
//   B: Delta = (T diag(beta)) R                 (lower triangular)
//   C: O = (gamma scale/|q|) Y + P Delta;  S <- gamma_C S + K^T diag(exp(G_C - G)/|k|) Delta
//      -- wait for every copy, barrier, O -> LDS (bf16, row-major)
// and the previous chunk's y leaves LDS after barrier b of the next step,
// each wave storing whole rows (16-byte pieces, 4 rows per instruction).
// Copies are bounded by a buffer descriptor per chunk: rows past the chunk's
// last token (and whole chunks past the sequence) read as zero, and y rows
// past it are dropped the same way.  K^T, T^T, P^T and V are read with the
// transposing LDS load.
//
// COMBA (the Comba forward): phase A reads the state with the read keys
// (X = Pr S, Pr the chunk's p rows) and phase C writes it with k.  Pr has
// one single-buffered tile (it is only read in phase A) copied beside V.
// The state slot is stored [K, V] (value index contiguous), the Comba
// layout, instead of [Dv, Dk].

template <int DK, int CT, int NW, int CW>
struct StreamTiles {
  static constexpr int BV = 16 * CW * NW;
  // LDS layouts (bf16), chosen so that each half-wave of reads touches
  // every bank once (64 banks of 4 bytes, i.e. 16 slots of 16 bytes):
  // * Q rows take 8-byte fragment reads, 16 rows by one slot: an odd slot
  //   pitch (DK + 8) spreads them.
  // * V takes transposing reads, 8 rows by 2 slots: a pitch of twice an odd
  //   number of slots (BV + 16) spreads them.
  // * T^T hi/lo and P^T arrive as their compact upper-triangular blocks
  //   (tri_block), one linear copy each; a transposing read stays inside
  //   one block, whose rows are 32 contiguous bytes.
  // * K takes both kinds of read.  Its pitch is DK + 16 (2 x odd slots) and
  //   rows with bit 3 set start one slot later, which moves rows 8..15 of
  //   every 16 onto the odd slots the even pitch leaves free: fragment
  //   reads cover 16 distinct slots and transposing reads (rows 0..7 or
  //   8..15 of a block) 8 distinct slot pairs.
  // * y waits in sY (CT rows of BV + 8): 16-byte row reads for the stores.
  static constexpr int KP = DK + 16, QP = DK + 8, VP = BV + 16, YP = BV + 8;
  static constexpr int FSTR = 3 * CT + 4;  // floats per record
  static constexpr int NTB = tri_blocks<CT>();
  using Kcopy = TileCopy<CT, DK / 8, KP, NW, true>;
  using Qcopy = TileCopy<CT, DK / 8, QP, NW>;
  using Tcopy = TileCopy<1, NTB * 32, NTB * 256, NW>;  // NTB blocks of 32 16-byte items
  using Vcopy = TileCopy<CT, BV / 8, VP, NW>;
  using Fcopy = TileCopy<1, FSTR / 4, 2 * FSTR, NW>;  // the record as 16-byte items
  struct __attribute__((aligned(16))) Set {
    bf16 K[Kcopy::ELEMS];
    bf16 Q[Qcopy::ELEMS];
    bf16 Th[Tcopy::ELEMS];
    bf16 Tl[Tcopy::ELEMS];
    bf16 P[Tcopy::ELEMS];
    bf16 F[Fcopy::ELEMS];
  };
};

template <int DK, int CT, int NW, int CW, bool GATED = false, bool COMBA = false, bool HALVES = false,
          bool SINGLE = false>
__global__ __launch_bounds__(64 * NW) void gdn_prefill_stream_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ pr,
    const bf16* __restrict__ v,
    float* __restrict__ pool, int64_t pool_size, const int64_t* __restrict__ cache_indices,
    const int64_t* __restrict__ cu, const int* __restrict__ scs, int N_s, int64_t T_tot, int Hk,
    int Hv, int Dv, int C, int maxc, const bf16* __restrict__ Th, const bf16* __restrict__ Tl,
    const bf16* __restrict__ Ph, const float* __restrict__ fac, bf16* __restrict__ y,
    const bf16* __restrict__ z, const float* __restrict__ gamma, float eps, int keep) {
  using Tiles = StreamTiles<DK, CT, NW, CW>;
  using Set = typename Tiles::Set;
  constexpr int BV = Tiles::BV, KP = Tiles::KP, QP = Tiles::QP, VP = Tiles::VP, YP = Tiles::YP,
                FSTR = Tiles::FSTR, NTB = Tiles::NTB;
  constexpr int MT = CT / 16, CKB = CT / 32, DT = DK / 16, KB = DK / 32;
  // Two distinct sets (not an indexed pair): reads of one never depend on
  // copies into the other.
  // SINGLE (every sequence is one chunk long): no chunk ci+1 to copy ahead,
  // so one operand set and none of the copies the double-buffered loop
  // issues for the (empty) next chunk
  static_assert(!SINGLE || (!GATED && !COMBA && !HALVES), "single-set variant: plain GDN only");
  __shared__ Set setA;
  __shared__ std::conditional_t<SINGLE, char, Set> setB_mem;
  Set& setB = [&]() -> Set& {
    if constexpr (SINGLE) return setA;
    else return setB_mem;
  }();
  __shared__ __attribute__((aligned(16))) bf16 sV[Tiles::Vcopy::ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 sY[CT * YP];
  // the gated epilogue's z tile and Comba's read-key tile (8 elements when unused)
  static_assert(!(GATED && COMBA), "no fused epilogue for the Comba forward");
  __shared__ __attribute__((aligned(16))) bf16 sZ[GATED ? CT * BV : 8];
  __shared__ __attribute__((aligned(16))) bf16 sPr[COMBA ? Tiles::Qcopy::ELEMS : 8];

  const int nvb = Dv / BV;
  // workgroup -> (position in the longest-first order, value head, column
  // block, half).  HALVES (launched when CUs would otherwise sit idle): wgp
  // (after the order) counts the workgroups before each position, and a
  // split sequence has two per (head, block), each computing BV/2 columns on
  // waves 0..NW/2-1 (half 0 or 1; -1: not split).
  constexpr bool SPLIT = HALVES && NW == 8 && CW == 1 && !GATED;
  const int* ord = scs + N_s + 1;
  const int* wgp = ord + N_s;
  const int bid = blockIdx.x;
  int pos, local;
  if constexpr (SPLIT) {
    if (bid >= wgp[N_s]) return;
    int lo = 0, hi = N_s;  // largest position r with wgp[r] <= bid (wgp strictly increases)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (wgp[mid] <= bid) lo = mid; else hi = mid;
    }
    pos = lo;
    local = bid - wgp[pos];
  } else {
    pos = bid / (Hv * nvb);
    local = bid - pos * (Hv * nvb);
  }
  const int s = ord[pos];
  int hv, vb, half = -1;
  if (SPLIT && wgp[pos + 1] - wgp[pos] == 2 * Hv * nvb) {
    hv = local / (2 * nvb);
    const int r2 = local - hv * 2 * nvb;
    vb = r2 >> 1;
    half = r2 & 1;
  } else {
    hv = local / nvb;
    vb = local - hv * nvb;
  }
  const int hoff = half < 0 ? 0 : half * (BV / 2);  // first column of this half in the block
  const int64_t slot = cache_indices[s];
  if (slot < 0 || slot >= pool_size) return;
  int64_t b0, len;
  seq_bounds(cu, s, T_tot, b0, len);
  if (len <= 0) return;
  const int cbase = scs[s];
  const int nch_all = static_cast<int>((len + C - 1) / C);
  const int nch = cbase + nch_all > maxc ? (maxc > cbase ? maxc - cbase : 0) : nch_all;
  if (nch <= 0 || (SINGLE && nch != 1)) return;
  const int hk = hv / (Hv / Hk);
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, kg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wave w owns value columns (w*CW + t)*16 + l16 of the block (of the half),
  // t < CW; in a half only waves 0..NW/2-1 compute, the others take their
  // share of the copies, barriers and y stores
  auto dvl = [&](int t) __attribute__((always_inline)) { return (w * CW + t) * 16 + l16; };
  const bool act = !SPLIT || half < 0 || w < NW / 2;

  const uint32_t kstride = static_cast<uint32_t>(Hk) * DK * 2;  // bytes between tokens
  const uint32_t vstride = static_cast<uint32_t>(Hv) * Dv * 2;
  typename Tiles::Kcopy cK;
  typename Tiles::Qcopy cQ;
  typename Tiles::Tcopy cT;
  typename Tiles::Vcopy cV;
  typename Tiles::Fcopy cF;
  typename Tiles::Qcopy cPr;  // Comba's read keys (same layout as Q)
  cK.init(w, lane, kstride);
  if constexpr (COMBA) cPr.init(w, lane, kstride);
  cQ.init(w, lane, kstride);
  cT.init(w, lane, 0);
  cV.init(w, lane, vstride);
  cF.init(w, lane, 0);

  // rows of chunk ci that exist (0 past the sequence)
  auto rows = [&](int ci) __attribute__((always_inline)) -> int {
    if (ci >= nch) return 0;
    const int64_t left = len - static_cast<int64_t>(ci) * C;
    return static_cast<int>(left < C ? left : C);
  };
  auto tok0 = [&](int ci) __attribute__((always_inline)) -> int64_t {
    return b0 + static_cast<int64_t>(ci) * C;
  };
  auto matix = [&](int ci) __attribute__((always_inline)) -> size_t {
    return static_cast<size_t>(cbase + ci) * Hv + hv;
  };
  auto kq_rsrc = [&](const bf16* base, int ci) __attribute__((always_inline)) {
    const int n = rows(ci);
    return make_rsrc(base + (static_cast<size_t>(tok0(ci)) * Hk + hk) * DK,
                     n > 0 ? (n - 1) * kstride + DK * 2 : 0u);
  };
  auto ws_rsrc = [&](const bf16* base, int ci) __attribute__((always_inline)) {
    return make_rsrc(base + matix(ci) * NTB * 256, rows(ci) > 0 ? NTB * 512 : 0u);
  };
  auto vy_off = [&](int ci) __attribute__((always_inline)) -> size_t {
    return (static_cast<size_t>(tok0(ci)) * Hv + hv) * Dv + vb * BV + hoff;
  };
  // (a half's range ends at its own columns: copies of the rest of a row
  // read the next row's first columns, or zero past the last row)
  auto vy_bytes = [&](int ci) __attribute__((always_inline)) -> uint32_t {
    const int n = rows(ci);
    return n > 0 ? (n - 1) * vstride + (half < 0 ? BV : BV / 2) * 2 : 0u;
  };
  // The copies of chunk ci's set are a per-wave list of single 1 KiB copies
  // (K, the record, T hi, T lo, Q, P); a step issues them one at a time
  // between its products, so no wave stalls on a burst of memory
  // instructions while its MFMAs wait.
  using Tiles_ = Tiles;
  constexpr int J0 = Tiles_::Kcopy::PER, J1 = J0 + Tiles_::Fcopy::PER, J2 = J1 + Tiles_::Tcopy::PER,
                J3 = J2 + Tiles_::Tcopy::PER, J4 = J3 + Tiles_::Qcopy::PER, NJOBS = J4 + Tiles_::Tcopy::PER;
  struct Rsrc {
    i32x4 K, F, Th, Tl, Q, P;
  };
  auto set_rsrc = [&](int ci) __attribute__((always_inline)) {
    return Rsrc{kq_rsrc(k, ci), make_rsrc(fac + matix(ci) * FSTR, rows(ci) > 0 ? FSTR * 4 : 0u),
                ws_rsrc(Th, ci), ws_rsrc(Tl, ci), kq_rsrc(q, ci), ws_rsrc(Ph, ci)};
  };
  auto copy_job = [&](const Rsrc& r, Set& d, int n) __attribute__((always_inline)) {
    if (n < J0) cK.issue_one(r.K, d.K, w, n);
    else if (n < J1) cF.issue_one(r.F, d.F, w, n - J0);
    else if (n < J2) cT.issue_one(r.Th, d.Th, w, n - J1);
    else if (n < J3) cT.issue_one(r.Tl, d.Tl, w, n - J2);
    else if (n < J4) cQ.issue_one(r.Q, d.Q, w, n - J3);
    else if (n < NJOBS) cT.issue_one(r.P, d.P, w, n - J4);
  };
  auto v_rsrc = [&](int ci) __attribute__((always_inline)) { return make_rsrc(v + vy_off(ci), vy_bytes(ci)); };

  // S[t][m][r] is the state at key index m*16 + kg*4 + r, value column dvl(t)
  float* Sp = pool + (static_cast<size_t>(slot) * Hv + hv) * Dv * DK +
              (COMBA ? static_cast<size_t>(vb * BV + hoff) : static_cast<size_t>(vb * BV + hoff) * DK);
  auto s_at = [&](int t, int m, int r) __attribute__((always_inline)) -> float* {
    return COMBA ? Sp + static_cast<size_t>(m * 16 + kg * 4 + r) * Dv + dvl(t)
                 : Sp + static_cast<size_t>(dvl(t)) * DK + m * 16 + kg * 4 + r;
  };
  f32x4 S[CW][DT];
  if (!act) {
#pragma unroll
    for (int t = 0; t < CW; ++t)
#pragma unroll
      for (int m = 0; m < DT; ++m) S[t][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  } else if constexpr (COMBA) {
#pragma unroll
    for (int t = 0; t < CW; ++t)
#pragma unroll
      for (int m = 0; m < DT; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[t][m][r] = *s_at(t, m, r);
  } else if (keep || !SINGLE) {
    // plain cache policy, as buffer loads so that the compiler cannot merge
    // them with the other branch's loads of the same addresses and drop the
    // non-temporal hint: for a slot that is only read (verify windows of 4
    // tokens 4% faster than with non-temporal loads), and in the
    // double-buffered loop (one workgroup per CU; non-temporal loads made
    // committed windows of 64 tokens 8% slower there and the varlen batch no
    // faster)
    const __amdgpu_buffer_rsrc_t srs = buf_rsrc(Sp, static_cast<uint32_t>(BV) * DK * sizeof(float));
#pragma unroll
    for (int t = 0; t < CW; ++t)
#pragma unroll
      for (int m = 0; m < DT; ++m)
        S[t][m] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                srs, static_cast<int>((s_at(t, m, 0) - Sp) * sizeof(float)), 0, 0));
  } else {
    // the single-set loop (three workgroups per CU) on a slot it writes
    // back: non-temporal (committed windows of 4-8 tokens 5% faster)
#pragma unroll
    for (int t = 0; t < CW; ++t)
#pragma unroll
      for (int m = 0; m < DT; ++m) S[t][m] = load_stream(s_at(t, m, 0));
  }

  // lane parts of the transposing reads
  const int tr_row = kg * 4 + (l16 >> 2), tr_col = 4 * (l16 & 3);
  // the skew of K rows read by this lane: fragment reads take row l16 of a
  // block, transposing reads rows kg*4 + l16/4 (+16)
  const int kfrag = ((l16 >> 3) & 1) * 8, ktr = (kg >> 1) * 8;
  const int tri_off = tr_row * 16 + tr_col;  // lane part of tri_trT
  f32x4 O[CW][MT];  // the chunk's outputs, staged after the step's last wait

  // O -> sY as bf16 rows (token, value column)
  auto stage_y = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < CW; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          // one conversion for two rows: low half to row r, high half to r + 1
          uint32_t p = pk(O[t][mt][r], O[t][mt][r + 1]);
          asm("" : "+v"(p));
          sY[(mt * 16 + kg * 4 + r) * YP + dvl(t)] = static_cast<bf16>(p);
          sY[(mt * 16 + kg * 4 + r + 1) * YP + dvl(t)] = static_cast<bf16>(p >> 16);
        }
  };
  // sY -> y rows of chunk ci: wave w stores CT/NW whole rows, 16 bytes per
  // lane, in NYS instructions
  constexpr int SPR = BV / 8;              // 16-byte pieces per row
  constexpr int PIECES = CT * SPR / NW;    // per wave, a multiple of 64
  constexpr int NYS = PIECES / 64;
  static_assert(PIECES % 64 == 0, "y pieces");
  auto y_off = [&](int it) __attribute__((always_inline)) -> uint32_t {
    const int pc = w * PIECES + it * 64 + lane;
    const int row = pc / SPR, col = (pc - row * SPR) * 8;
    return static_cast<uint32_t>(row) * vstride + col * 2;
  };
  // GATED: y = o / sqrt(mean(o^2) + eps) * gamma * sigmoid(z) over the
  // head's BV = Dv columns, i.e. over the 16 lanes that store one row.  Each
  // wave copies the z pieces of its own y pieces into sZ when the step
  // starts (so no other wave is involved); gamma for the lane's 8 columns is
  // loaded once.
  static_assert(!GATED || SPR == 16, "the gated epilogue needs one 128-column head per workgroup");
  float gm[8];
  if constexpr (GATED) {
    const f32x4 g0 = *reinterpret_cast<const f32x4*>(gamma + (lane % SPR) * 8);
    const f32x4 g1 = *reinterpret_cast<const f32x4*>(gamma + (lane % SPR) * 8 + 4);
    gm[0] = g0.x; gm[1] = g0.y; gm[2] = g0.z; gm[3] = g0.w;
    gm[4] = g1.x; gm[5] = g1.y; gm[6] = g1.z; gm[7] = g1.w;
  }
  auto store_y_one = [&](__amdgpu_buffer_rsrc_t yr, int it) __attribute__((always_inline)) {
    const int pc = w * PIECES + it * 64 + lane;
    const int row = pc / SPR, col = (pc - row * SPR) * 8;
    if (half >= 0 && col >= BV / 2) return;  // a half stores its own columns only
    u32x4 d = *reinterpret_cast<const u32x4*>(sY + row * YP + col);
    if constexpr (GATED) {
      float o8[8], ss = 0.f;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        o8[2 * p] = __uint_as_float(d[p] << 16);
        o8[2 * p + 1] = __uint_as_float(d[p] & 0xffff0000u);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(o8[i], o8[i], ss);
      ss = group_sum<16>(ss);
      const float rs = __builtin_amdgcn_rsqf(ss * (1.0f / BV) + eps);
      const u32x4 zv = *reinterpret_cast<const u32x4*>(sZ + pc * 8);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float z0 = __uint_as_float(zv[p] << 16), z1 = __uint_as_float(zv[p] & 0xffff0000u);
        // sigmoid on the hardware exponential and reciprocal (a few ulp)
        d[p] = pk(o8[2 * p] * rs * gm[2 * p] * __builtin_amdgcn_rcpf(1.0f + __expf(-z0)),
                  o8[2 * p + 1] * rs * gm[2 * p + 1] * __builtin_amdgcn_rcpf(1.0f + __expf(-z1)));
      }
    }
    __builtin_amdgcn_raw_buffer_store_b128(d, yr, y_off(it), 0, 0);
  };
  // z pieces of chunk ci -> sZ slot pc (one 1 KiB copy per y instruction).
  // The reads wait with vmcnt(N): at most N of this wave's later loads
  // outstanding (loads complete in order), which covers z without waiting
  // for the copies issued after it.
  auto z_load = [&](int ci) __attribute__((always_inline)) {
    const i32x4 zr = make_rsrc(z + vy_off(ci), vy_bytes(ci));
#pragma unroll
    for (int it = 0; it < NYS; ++it) dma16(zr, lds_addr(sZ) + (w * PIECES + it * 64) * 16, y_off(it));
  };

  // Every operand fragment read from LDS feeds the CW column tiles of the
  // wave; the tiles' MFMA chains are independent and interleave.
  // a waiting wave of a half: the same copies, y stores and barriers as a
  // step, no products
  auto idle_step = [&](int ci, Set& nx) __attribute__((always_inline)) {
    const Rsrc rn = set_rsrc(ci + 1);
    {
#pragma unroll
      for (int n = 0; n < NJOBS; ++n) copy_job(rn, nx, n);
      lds_handover();
      const i32x4 rv = v_rsrc(ci + 1);
#pragma unroll
      for (int j = 0; j < Tiles_::Vcopy::PER; ++j) cV.issue_one(rv, sV, w, j);
      if constexpr (COMBA) {
        const i32x4 rp = kq_rsrc(pr, ci + 1);
#pragma unroll
        for (int j = 0; j < Tiles_::Qcopy::PER; ++j) cPr.issue_one(rp, sPr, w, j);
      }
      if (ci > 0) {
        const __amdgpu_buffer_rsrc_t yr = buf_rsrc(y + vy_off(ci - 1), vy_bytes(ci - 1));
#pragma unroll
        for (int it = 0; it < NYS; ++it) store_y_one(yr, it);
      }
      handover<0>();
    }
  };

  auto step = [&](int ci, const Set& c, Set& nx) __attribute__((always_inline)) {
    const float* F = reinterpret_cast<const float*>(c.F);
    const Rsrc rn = set_rsrc(ci + 1);
    if constexpr (GATED) {
      if (ci > 0) z_load(ci - 1);
    }

    // ---- A: X = K S and Y = Q S (S as hi + lo: a row of y whose state-side
    // term nearly cancels the in-chunk term would otherwise carry 2^-9 of
    // that term as error), R, and O's first term
    f32x4 X[CW][MT], Y[CW][MT];
#pragma unroll
    for (int t = 0; t < CW; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        X[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        Y[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      bf16x8v Sh[CW], Sl[CW];
#pragma unroll
      for (int t = 0; t < CW; ++t) acc_operand(S[t][2 * kb], S[t][2 * kb + 1], Sh[t], Sl[t]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8v a = COMBA ? lds_pi<QP>(sPr, mt * 16 + l16, kb * 32, kg)
                                : lds_pi<KP>(c.K + kfrag, mt * 16 + l16, kb * 32, kg);
        const bf16x8v aq = lds_pi<QP>(c.Q, mt * 16 + l16, kb * 32, kg);
#pragma unroll
        for (int t = 0; t < CW; ++t) {
          X[t][mt] = mma(a, Sh[t], X[t][mt]);
          Y[t][mt] = mma(aq, Sh[t], Y[t][mt]);
          X[t][mt] = mma(a, Sl[t], X[t][mt]);
          Y[t][mt] = mma(aq, Sl[t], Y[t][mt]);
        }
        if constexpr (!SINGLE) copy_job(rn, nx, kb * MT + mt);  // chunk ci+1's set, one copy per product group
      }
    }
    if constexpr (!SINGLE) {
#pragma unroll
      for (int n = KB * MT; n < NJOBS; ++n) copy_job(rn, nx, n);
    }
    f32x4 R[CW][MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const f32x4 fk = *reinterpret_cast<const f32x4*>(F + mt * 16 + kg * 4);
      const f32x4 fq = *reinterpret_cast<const f32x4*>(F + CT + mt * 16 + kg * 4);
#pragma unroll
      for (int t = 0; t < CW; ++t) {
        const s16x4 vv = lds_tr(sV + (mt * 16 + tr_row) * VP + (w * CW + t) * 16 + tr_col);
        O[t][mt] = fq * Y[t][mt];
#pragma unroll
        for (int r = 0; r < 4; ++r) R[t][mt][r] = bf16_bits_to_f32(vv[r]) - fk[r] * X[t][mt][r];
      }
    }
    lds_handover();  // V (and Comba's Pr) is free; every wave staged chunk ci-1's y
    const i32x4 rv = v_rsrc(ci + 1);
    i32x4 rp;
    if constexpr (COMBA) rp = kq_rsrc(pr, ci + 1);
    const __amdgpu_buffer_rsrc_t yr = buf_rsrc(y + vy_off(ci > 0 ? ci - 1 : 0), ci > 0 ? vy_bytes(ci - 1) : 0u);

    // ---- B: Delta = T R (blocks above the diagonal skipped)
    bf16x8v Rh[CW][CKB], Rl[CW][CKB];
#pragma unroll
    for (int t = 0; t < CW; ++t)
#pragma unroll
      for (int cb = 0; cb < CKB; ++cb) acc_operand(R[t][2 * cb], R[t][2 * cb + 1], Rh[t][cb], Rl[t][cb]);
    f32x4 D[CW][MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int t = 0; t < CW; ++t) D[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cb = 0; cb <= mt / 2; ++cb) {
        const bf16x8v th = tri_trT<CT>(c.Th, cb, mt, tri_off);
        const bf16x8v tl = tri_trT<CT>(c.Tl, cb, mt, tri_off);
#pragma unroll
        for (int t = 0; t < CW; ++t) {
          D[t][mt] = mma(th, Rh[t][cb], D[t][mt]);
          D[t][mt] = mma(th, Rl[t][cb], D[t][mt]);
          D[t][mt] = mma(tl, Rh[t][cb], D[t][mt]);
        }
      }
      if constexpr (!SINGLE) cV.issue_one(rv, sV, w, mt);  // chunk ci+1's V
      if constexpr (COMBA) cPr.issue_one(rp, sPr, w, mt);
    }
    if constexpr (!SINGLE) {
#pragma unroll
      for (int j = MT; j < Tiles_::Vcopy::PER; ++j) cV.issue_one(rv, sV, w, j);
    }
    if constexpr (COMBA) {
#pragma unroll
      for (int j = MT; j < Tiles_::Qcopy::PER; ++j) cPr.issue_one(rp, sPr, w, j);
    }

    // ---- C: O += P Delta (hi parts);  S <- gamma_C S + K^T diag(fD) Delta
    bf16x8v Dh[CW][CKB], Eh[CW][CKB], El[CW][CKB];
#pragma unroll
    for (int t = 0; t < CW; ++t) {
#pragma unroll
      for (int cb = 0; cb < CKB; ++cb) Dh[t][cb] = acc_operand_hi(D[t][2 * cb], D[t][2 * cb + 1]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        D[t][mt] *= *reinterpret_cast<const f32x4*>(F + 2 * CT + mt * 16 + kg * 4);
#pragma unroll
      for (int cb = 0; cb < CKB; ++cb) acc_operand(D[t][2 * cb], D[t][2 * cb + 1], Eh[t][cb], El[t][cb]);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int cb = 0; cb <= mt / 2; ++cb) {
        const bf16x8v pa = tri_trT<CT>(c.P, cb, mt, tri_off);
#pragma unroll
        for (int t = 0; t < CW; ++t) O[t][mt] = mma(pa, Dh[t][cb], O[t][mt]);
      }
    const float gC = F[3 * CT];
#pragma unroll
    for (int m = 0; m < DT; ++m) {
#pragma unroll
      for (int t = 0; t < CW; ++t) S[t][m] *= gC;
#pragma unroll
      for (int cb = 0; cb < CKB; ++cb) {
        const bf16x8v a = lds_trT<KP>(c.K + ktr, cb * 32 + tr_row, m * 16 + tr_col);
#pragma unroll
        for (int t = 0; t < CW; ++t) {
          S[t][m] = mma(a, Eh[t][cb], S[t][m]);
          S[t][m] = mma(a, El[t][cb], S[t][m]);
        }
      }
      // chunk ci-1's y, spread over the update
      if constexpr (GATED) {
        // every wave issued at least these copies after its z loads
        constexpr int VMZ = Tiles_::Kcopy::MIN + Tiles_::Fcopy::MIN + 3 * Tiles_::Tcopy::MIN +
                            Tiles_::Qcopy::MIN + Tiles_::Vcopy::MIN;
        static_assert(VMZ < 64, "z wait");
        if (m == 0 && ci > 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(VMZ) : "memory");
      }
      if (m % (DT / NYS) == 0 && m / (DT / NYS) < NYS && ci > 0) store_y_one(yr, m / (DT / NYS));
    }
    handover<0>();  // every copy of chunk ci+1 landed; this chunk's set and sY are free
    stage_y();
  };

  // prologue: all operands of chunk 0
  {
    const Rsrc r0 = set_rsrc(0);
#pragma unroll
    for (int n = 0; n < NJOBS; ++n) copy_job(r0, setA, n);
    cV.issue(v_rsrc(0), sV, w);
    if constexpr (COMBA) cPr.issue(kq_rsrc(pr, 0), sPr, w);
  }
  handover<0>();
  if constexpr (SINGLE) {
    step(0, setA, setB);
  } else if (act) {
    for (int ci = 0; ci < nch; ci += 2) {
      step(ci, setA, setB);
      if (ci + 1 < nch) step(ci + 1, setB, setA);
    }
  } else {
    for (int ci = 0; ci < nch; ci += 2) {
      idle_step(ci, setB);
      if (ci + 1 < nch) idle_step(ci + 1, setA);
    }
  }
  // (every copy has landed: each step ends waiting for all of them)
  lds_handover();
  {
    if constexpr (GATED) {
      z_load(nch - 1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    const __amdgpu_buffer_rsrc_t yr = buf_rsrc(y + vy_off(nch - 1), vy_bytes(nch - 1));
#pragma unroll
    for (int it = 0; it < NYS; ++it) store_y_one(yr, it);
  }

  if (!act || keep) return;  // keep: the slot is read only
#pragma unroll
  for (int t = 0; t < CW; ++t)
#pragma unroll
    for (int m = 0; m < DT; ++m) {
      if constexpr (COMBA) {
#pragma unroll
        for (int r = 0; r < 4; ++r) *s_at(t, m, r) = S[t][m][r];
      } else {
        *reinterpret_cast<f32x4*>(s_at(t, m, 0)) = S[t][m];
      }
    }
}

// ----------------------------------------------------------------------------
// host side

constexpr size_t kAlign = 256;
inline size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline int chunk_tile(int chunk) { return chunk <= 32 ? 32 : 64; }

// Workspace: the chunk map, then per (chunk, value head) T hi/lo and P (hi;
// plus P lo for fp32 activations) and the factor record.  The matrices are
// CT x CT bf16 for fp32 activations and compact upper-triangular blocks
// (tri_block) for bf16 activations.
struct Layout {
  size_t scs, th, tl, ph, pl, fac, total;
};

// Compute units of the current device (cached per device; 256 if the query
// fails): the chunk map's test for "every sequence split still fits".
inline int cu_count() {
  static std::atomic<int> cache[64];  // 0: not looked up yet (calls may come from several threads)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Options of one prefill call, passed down to the launches.
constexpr unsigned kOneChunk = 1u;   // every sequence is one chunk long (the host knows it)
constexpr unsigned kKeepState = 2u;  // the state slots are read, never written

// The chunk map on one workgroup: a single wave for up to 64 sequences (one
// per lane; its barriers are then nearly free), else 1,024 threads (a wave
// scanning several sequences per lane measured slower than that).
inline void chunk_map(const int64_t* cu, int N_s, int64_t T_tot, int chunk, int* scs, int per_seq,
                      bool split, hipStream_t stream) {
  if (N_s <= 64)
    hipLaunchKernelGGL(gdn_chunk_map_kernel<64>, dim3(1), dim3(64), 0, stream, cu, N_s, T_tot, chunk, scs,
                       per_seq, cu_count(), split ? 1 : 0);
  else
    hipLaunchKernelGGL(gdn_chunk_map_kernel<1024>, dim3(1), dim3(1024), 0, stream, cu, N_s, T_tot, chunk, scs,
                       per_seq, cu_count(), split ? 1 : 0);
}

inline Layout layout(int64_t T_tot, int N_s, int Hv, int chunk, bool bf16_act) {
  const int CT = chunk_tile(chunk);
  const size_t maxc = static_cast<size_t>(T_tot / chunk) + static_cast<size_t>(N_s);
  const size_t mats = maxc * static_cast<size_t>(Hv);
  const size_t per = bf16_act ? static_cast<size_t>(CT / 16) * (CT / 16 + 1) / 2 * 256 : static_cast<size_t>(CT) * CT;
  const size_t tile = up(mats * per * sizeof(bf16));
  Layout L;
  size_t off = 0;
  L.scs = off; off += up(sizeof(int) * (3 * static_cast<size_t>(N_s) + 2));  // chunk map, order, workgroup prefix
  L.th = off; off += tile;
  L.tl = off; off += tile;
  L.ph = off; off += tile;
  L.pl = off; off += bf16_act ? 0 : tile;
  L.fac = off; off += up(mats * ((bf16_act ? 3 : 4) * CT + 4) * sizeof(float));
  L.total = off;
  return L;
}

// The optional gated RMS norm of y (gdn_chunk_prefill_gated).
struct Epilogue {
  const void* z;
  const float* gamma;
  float eps;
};

template <typename T, int DK, int CT, int NW, int CW = 1>
int launch_all(const void* q, const void* k, const void* v, const float* g, const float* beta,
               float* pool, int64_t pool_size, const int64_t* ci, const int64_t* cu, int N_s,
               int64_t T_tot, int Hk, int Hv, int Dv, int chunk, float scale, int l2norm, void* y,
               char* ws, const Layout& L, const Epilogue* epi, const RawGates* raw, const FixedBatch* fixb,
               hipStream_t stream, unsigned opts) {
  const bool one_chunk = (opts & kOneChunk) != 0;
  const int keep = (opts & kKeepState) ? 1 : 0;
  int* scs = reinterpret_cast<int*>(ws + L.scs);
  bf16* Th = reinterpret_cast<bf16*>(ws + L.th);
  bf16* Tl = reinterpret_cast<bf16*>(ws + L.tl);
  bf16* Ph = reinterpret_cast<bf16*>(ws + L.ph);
  bf16* Pl = reinterpret_cast<bf16*>(ws + L.pl);
  float* fac = reinterpret_cast<float*>(ws + L.fac);
  // chunks of the batch: at most T_tot/chunk + N_s (the layout's bound);
  // exactly N_s ceil(T/chunk) in a fixed-length batch, whose WY launch then
  // has no waves without a chunk
  const size_t maxc = fixb ? static_cast<size_t>(N_s) * static_cast<size_t>((fixb->T + chunk - 1) / chunk)
                           : static_cast<size_t>(T_tot / chunk) + static_cast<size_t>(N_s);
  const size_t wy_blocks = maxc * static_cast<size_t>(Hv);
  const int per_seq = Hv * (Dv / (16 * NW * CW));  // chunk-loop workgroups per sequence, unsplit
  // when CUs would sit idle, the longest sequences run as two half-width
  // workgroups each (bf16, eight waves, no fused norm)
  const bool split = std::is_same<T, bf16>::value && NW == 8 && CW == 1 && !(epi && Dv == 128) &&
                     static_cast<int64_t>(N_s) * per_seq < cu_count();
  const size_t main_blocks = static_cast<size_t>(N_s) * per_seq * (split ? 2 : 1);
  if (wy_blocks > 0x7fffffffu || main_blocks > 0x7fffffffu) return GDN_ERR_SHAPE;
  (void)hipGetLastError();
  if constexpr (std::is_same<T, bf16>::value) {
    // up to 64 sequences, or a fixed-length batch (whose cu_seqlens and
    // cache_indices it writes as well): the WY launch makes the chunk map
    // too (one more workgroup)
    const int own = N_s <= 64 || fixb ? 1 : 0;
    if (!own) chunk_map(cu, N_s, T_tot, chunk, scs, per_seq, split, stream);
    const FixedBatch fb = fixb ? *fixb : FixedBatch{0, nullptr, nullptr};
    const int64_t* wy_cu = fixb ? nullptr : cu;  // not read in a fixed-length batch
    const dim3 wy_grid(static_cast<unsigned>(maxc * static_cast<size_t>(Hk) + own));
    if (raw && raw->cv.x)  // the conv prologue and the gates inside the WY pass (q, k: its outputs)
      hipLaunchKernelGGL((gdn_wy_wave_kernel<DK, CT, false, float, true, true>), wy_grid, dim3(64), 0, stream,
                         static_cast<const bf16*>(nullptr), static_cast<const bf16*>(nullptr),
                         static_cast<const bf16*>(nullptr), static_cast<const float*>(nullptr),
                         static_cast<const float*>(nullptr), wy_cu, scs, N_s, T_tot, Hk, Hv, chunk, scale, l2norm, Th,
                         Tl, Ph, fac, *raw, own, scs, per_seq, cu_count(), split ? 1 : 0, fb);
    else if (raw)  // the gates formed inside the WY pass
      hipLaunchKernelGGL((gdn_wy_wave_kernel<DK, CT, false, float, true>), wy_grid, dim3(64), 0, stream,
                         static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(nullptr),
                         static_cast<const float*>(nullptr), static_cast<const float*>(nullptr), wy_cu, scs, N_s,
                         T_tot, Hk, Hv, chunk, scale, l2norm, Th, Tl, Ph, fac, *raw, own, scs, per_seq, cu_count(),
                         split ? 1 : 0, fb);
    else
      hipLaunchKernelGGL((gdn_wy_wave_kernel<DK, CT>), wy_grid, dim3(64), 0, stream, static_cast<const bf16*>(q),
                         static_cast<const bf16*>(k), static_cast<const bf16*>(nullptr), g, beta, wy_cu, scs, N_s,
                         T_tot, Hk, Hv, chunk, scale, l2norm, Th, Tl, Ph, fac, RawGates{}, own, scs, per_seq,
                         cu_count(), split ? 1 : 0, fb);
    // the epilogue is fused when one workgroup covers a whole 128-column head
    if constexpr (NW == 8 && CW == 1) {
      if (epi && Dv == 128) {
        hipLaunchKernelGGL((gdn_prefill_stream_kernel<DK, CT, NW, CW, true>), dim3(static_cast<unsigned>(main_blocks)),
                           dim3(64 * NW), 0, stream, static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                           static_cast<const bf16*>(nullptr), static_cast<const bf16*>(v), pool, pool_size, ci, cu, scs, N_s, T_tot, Hk, Hv, Dv,
                           chunk, static_cast<int>(maxc), Th, Tl, Ph, fac, static_cast<bf16*>(y),
                           static_cast<const bf16*>(epi->z), epi->gamma, epi->eps, keep);
        return launch_status();
      }
    }
    // every sequence one chunk long (the host knows it for fixed-length
    // batches): the single-set variant, more workgroups per CU
    if constexpr (CT == 32 && NW == 8 && CW == 1) {
      if (one_chunk && !split) {
        hipLaunchKernelGGL((gdn_prefill_stream_kernel<DK, CT, NW, CW, false, false, false, true>),
                           dim3(static_cast<unsigned>(main_blocks)), dim3(64 * NW), 0, stream,
                           static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(nullptr),
                           static_cast<const bf16*>(v), pool, pool_size, ci, cu, scs, N_s, T_tot, Hk, Hv, Dv, chunk,
                           static_cast<int>(maxc), Th, Tl, Ph, fac, static_cast<bf16*>(y),
                           static_cast<const bf16*>(nullptr), static_cast<const float*>(nullptr), 0.0f, keep);
        return launch_status();
      }
    }
    if (split)
      hipLaunchKernelGGL((gdn_prefill_stream_kernel<DK, CT, NW, CW, false, false, true>),
                         dim3(static_cast<unsigned>(main_blocks)), dim3(64 * NW), 0, stream,
                         static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(nullptr),
                         static_cast<const bf16*>(v), pool, pool_size, ci, cu, scs, N_s, T_tot, Hk, Hv, Dv, chunk,
                         static_cast<int>(maxc), Th, Tl, Ph, fac, static_cast<bf16*>(y),
                         static_cast<const bf16*>(nullptr), static_cast<const float*>(nullptr), 0.0f, keep);
    else
      hipLaunchKernelGGL((gdn_prefill_stream_kernel<DK, CT, NW, CW>), dim3(static_cast<unsigned>(main_blocks)),
                         dim3(64 * NW), 0, stream, static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                         static_cast<const bf16*>(nullptr), static_cast<const bf16*>(v), pool, pool_size, ci, cu,
                         scs, N_s, T_tot, Hk, Hv, Dv, chunk, static_cast<int>(maxc), Th, Tl, Ph, fac,
                         static_cast<bf16*>(y), static_cast<const bf16*>(nullptr),
                         static_cast<const float*>(nullptr), 0.0f, keep);
  } else {
    if (raw) return GDN_ERR_UNSUPPORTED;  // fp32 activations take their gates from gdn_prefill_gates
    chunk_map(cu, N_s, T_tot, chunk, scs, per_seq, split, stream);
    hipLaunchKernelGGL((gdn_wy_kernel<T, DK, CT>), dim3(static_cast<unsigned>(wy_blocks)), dim3(64), 0,
                       stream, static_cast<const T*>(q), static_cast<const T*>(k), g, beta, cu, scs, N_s,
                       T_tot, Hk, Hv, chunk, scale, l2norm, Th, Tl, Ph, Pl, fac);
    hipLaunchKernelGGL((gdn_prefill_kernel<T, DK, CT, NW>), dim3(static_cast<unsigned>(main_blocks)),
                       dim3(64 * NW), 0, stream, static_cast<const T*>(q), static_cast<const T*>(k),
                       static_cast<const T*>(v), beta, pool, pool_size, ci, cu, scs, N_s, T_tot, Hk, Hv,
                       Dv, chunk, static_cast<int>(maxc), Th, Tl, Ph, Pl, fac, static_cast<T*>(y), keep ? 1 : 0);
  }
  if (launch_status() != GDN_OK) return GDN_ERR_LAUNCH;
  // otherwise the separate norm kernel, in place on y
  if (epi)
    return gated_rmsnorm_launch(y, epi->z, epi->gamma, epi->eps, static_cast<long>(T_tot) * Hv, Dv, y,
                                std::is_same<T, bf16>::value ? GDN_BF16 : GDN_F32, stream);
  return GDN_OK;
}

template <typename T, int DK, int CT>
int dispatch_nw(int Dv, const void* q, const void* k, const void* v, const float* g,
                const float* beta, float* pool, int64_t pool_size, const int64_t* ci,
                const int64_t* cu, int N_s, int64_t T_tot, int Hk, int Hv, int chunk, float scale,
                int l2norm, void* y, char* ws, const Layout& L, const Epilogue* epi, const RawGates* raw,
                const FixedBatch* fixb, hipStream_t stream, unsigned opts) {
  // bf16: the streamed LDS kernel, up to 128 value columns (eight waves) per
  // workgroup so each chunk operand is fetched once per 128 columns.  fp32
  // activations: the register-fragment kernel, 64 (four waves, up to 512
  // registers each) or 32 columns per workgroup.
  if constexpr (std::is_same<T, bf16>::value) {
    if (Dv % 128 == 0)
      return launch_all<T, DK, CT, 8, 1>(q, k, v, g, beta, pool, pool_size, ci, cu, N_s, T_tot, Hk, Hv, Dv,
                                         chunk, scale, l2norm, y, ws, L, epi, raw, fixb, stream, opts);
  }
  if (Dv % 64 == 0)
    return launch_all<T, DK, CT, 4>(q, k, v, g, beta, pool, pool_size, ci, cu, N_s, T_tot, Hk, Hv, Dv,
                                    chunk, scale, l2norm, y, ws, L, epi, raw, fixb, stream, opts);
  return launch_all<T, DK, CT, 2>(q, k, v, g, beta, pool, pool_size, ci, cu, N_s, T_tot, Hk, Hv, Dv,
                                  chunk, scale, l2norm, y, ws, L, epi, raw, fixb, stream, opts);
}

template <typename T, int DK>
int dispatch_ct(int CT, int Dv, const void* q, const void* k, const void* v, const float* g,
                const float* beta, float* pool, int64_t pool_size, const int64_t* ci,
                const int64_t* cu, int N_s, int64_t T_tot, int Hk, int Hv, int chunk, float scale,
                int l2norm, void* y, char* ws, const Layout& L, const Epilogue* epi, const RawGates* raw,
                const FixedBatch* fixb, hipStream_t stream, unsigned opts) {
  if constexpr (DK > 128) {  // 32-row tiles only (effective_chunk)
    return dispatch_nw<T, DK, 32>(Dv, q, k, v, g, beta, pool, pool_size, ci, cu, N_s, T_tot, Hk, Hv,
                                  chunk, scale, l2norm, y, ws, L, epi, raw, fixb, stream, opts);
  } else {
    if (CT == 32)
      return dispatch_nw<T, DK, 32>(Dv, q, k, v, g, beta, pool, pool_size, ci, cu, N_s, T_tot, Hk, Hv,
                                    chunk, scale, l2norm, y, ws, L, epi, raw, fixb, stream, opts);
    return dispatch_nw<T, DK, 64>(Dv, q, k, v, g, beta, pool, pool_size, ci, cu, N_s, T_tot, Hk, Hv,
                                  chunk, scale, l2norm, y, ws, L, epi, raw, fixb, stream, opts);
  }
}

template <typename T>
int dispatch_dk(int Dk, int CT, int Dv, const void* q, const void* k, const void* v,
                const float* g, const float* beta, float* pool, int64_t pool_size,
                const int64_t* ci, const int64_t* cu, int N_s, int64_t T_tot, int Hk, int Hv,
                int chunk, float scale, int l2norm, void* y, char* ws, const Layout& L,
                const Epilogue* epi, const RawGates* raw, const FixedBatch* fixb, hipStream_t stream,
                unsigned opts) {
  switch (Dk) {
    case 32: return dispatch_ct<T, 32>(CT, Dv, q, k, v, g, beta, pool, pool_size, ci, cu, N_s, T_tot, Hk, Hv, chunk, scale, l2norm, y, ws, L, epi, raw, fixb, stream, opts);
    case 64: return dispatch_ct<T, 64>(CT, Dv, q, k, v, g, beta, pool, pool_size, ci, cu, N_s, T_tot, Hk, Hv, chunk, scale, l2norm, y, ws, L, epi, raw, fixb, stream, opts);
    case 128: return dispatch_ct<T, 128>(CT, Dv, q, k, v, g, beta, pool, pool_size, ci, cu, N_s, T_tot, Hk, Hv, chunk, scale, l2norm, y, ws, L, epi, raw, fixb, stream, opts);
    case 96: return dispatch_ct<T, 96>(CT, Dv, q, k, v, g, beta, pool, pool_size, ci, cu, N_s, T_tot, Hk, Hv, chunk, scale, l2norm, y, ws, L, epi, raw, fixb, stream, opts);
  }
  // wider heads: bf16 activations only (the fp32 kernels would spill at these widths)
  if constexpr (std::is_same<T, bf16>::value) {
    switch (Dk) {
      case 160: return dispatch_ct<T, 160>(CT, Dv, q, k, v, g, beta, pool, pool_size, ci, cu, N_s, T_tot, Hk, Hv, chunk, scale, l2norm, y, ws, L, epi, raw, fixb, stream, opts);
      case 192: return dispatch_ct<T, 192>(CT, Dv, q, k, v, g, beta, pool, pool_size, ci, cu, N_s, T_tot, Hk, Hv, chunk, scale, l2norm, y, ws, L, epi, raw, fixb, stream, opts);
      case 224: return dispatch_ct<T, 224>(CT, Dv, q, k, v, g, beta, pool, pool_size, ci, cu, N_s, T_tot, Hk, Hv, chunk, scale, l2norm, y, ws, L, epi, raw, fixb, stream, opts);
      case 256: return dispatch_ct<T, 256>(CT, Dv, q, k, v, g, beta, pool, pool_size, ci, cu, N_s, T_tot, Hk, Hv, chunk, scale, l2norm, y, ws, L, epi, raw, fixb, stream, opts);
    }
  }
  return GDN_ERR_UNSUPPORTED;
}

inline bool valid_chunk(int chunk) { return chunk == 8 || chunk == 16 || chunk == 32 || chunk == 64; }

// Key heads wider than 128 run chunks of at most 32 tokens: two 64-row K
// and Q tiles of that width (plus their double buffers) do not fit in a
// CU's LDS, 32-row ones do.  The chunk size changes results only through
// rounding.
inline int effective_chunk(int Dk, int chunk) { return Dk > 128 && chunk > 32 ? 32 : chunk; }

// The Comba forward (bf16 activations): the WY pass on P K^T Gram blocks and
// the chunk loop reading with p, over a [K, V] state pool; one key head per
// value head.
struct CombaArgs {
  const bf16 *q, *k, *v, *p, *beta;
  const float* g;
  float* pool;
  int64_t pool_size;
  const int64_t *ci, *cu;
  int N_s;
  int64_t T_tot;
  int H, V, chunk;
  float scale;
  bf16* o;
};

template <int DK, int CT, int NW>
int comba_launch(const CombaArgs& a, char* ws, const Layout& L, hipStream_t stream) {
  int* scs = reinterpret_cast<int*>(ws + L.scs);
  bf16* Th = reinterpret_cast<bf16*>(ws + L.th);
  bf16* Tl = reinterpret_cast<bf16*>(ws + L.tl);
  bf16* Ph = reinterpret_cast<bf16*>(ws + L.ph);
  float* fac = reinterpret_cast<float*>(ws + L.fac);
  const size_t maxc = static_cast<size_t>(a.T_tot / a.chunk) + static_cast<size_t>(a.N_s);
  const size_t wy_blocks = maxc * static_cast<size_t>(a.H);
  const int per_seq = a.H * (a.V / (16 * NW));
  // when CUs would sit idle, the longest sequences run as two half-width workgroups
  const bool split = NW == 8 && static_cast<int64_t>(a.N_s) * per_seq < cu_count();
  const size_t main_blocks = static_cast<size_t>(a.N_s) * per_seq * (split ? 2 : 1);
  if (wy_blocks > 0x7fffffffu || main_blocks > 0x7fffffffu) return GDN_ERR_SHAPE;
  (void)hipGetLastError();
  // up to 64 sequences: the WY launch makes the chunk map too (one more workgroup)
  const int own = a.N_s <= 64 ? 1 : 0;
  if (!own) chunk_map(a.cu, a.N_s, a.T_tot, a.chunk, scs, per_seq, split, stream);
  hipLaunchKernelGGL((gdn_wy_wave_kernel<DK, CT, true, bf16>), dim3(static_cast<unsigned>(wy_blocks + own)), dim3(64),
                     0, stream, a.q, a.k, a.p, a.g, a.beta, a.cu, scs, a.N_s, a.T_tot, a.H, a.H, a.chunk, a.scale, 0,
                     Th, Tl, Ph, fac, RawGates{}, own, scs, per_seq, cu_count(), split ? 1 : 0,
                     FixedBatch{0, nullptr, nullptr});
  if (split)
    hipLaunchKernelGGL((gdn_prefill_stream_kernel<DK, CT, NW, 1, false, true, true>),
                       dim3(static_cast<unsigned>(main_blocks)), dim3(64 * NW), 0, stream, a.q, a.k, a.p, a.v, a.pool,
                       a.pool_size, a.ci, a.cu, scs, a.N_s, a.T_tot, a.H, a.H, a.V, a.chunk, static_cast<int>(maxc),
                       Th, Tl, Ph, fac, a.o, static_cast<const bf16*>(nullptr), static_cast<const float*>(nullptr),
                       0.0f, 0);
  else
    hipLaunchKernelGGL((gdn_prefill_stream_kernel<DK, CT, NW, 1, false, true>), dim3(static_cast<unsigned>(main_blocks)),
                       dim3(64 * NW), 0, stream, a.q, a.k, a.p, a.v, a.pool, a.pool_size, a.ci, a.cu, scs, a.N_s,
                       a.T_tot, a.H, a.H, a.V, a.chunk, static_cast<int>(maxc), Th, Tl, Ph, fac, a.o,
                       static_cast<const bf16*>(nullptr), static_cast<const float*>(nullptr), 0.0f, 0);
  return launch_status();
}

template <int DK, int CT>
int comba_dispatch_nw(const CombaArgs& a, char* ws, const Layout& L, hipStream_t stream) {
  if (a.V % 128 == 0) return comba_launch<DK, CT, 8>(a, ws, L, stream);
  if (a.V % 64 == 0) return comba_launch<DK, CT, 4>(a, ws, L, stream);
  return comba_launch<DK, CT, 2>(a, ws, L, stream);
}

template <int DK>
int comba_dispatch_ct(int CT, const CombaArgs& a, char* ws, const Layout& L, hipStream_t stream) {
  if constexpr (DK > 128)  // 32-row tiles only (effective_chunk)
    return comba_dispatch_nw<DK, 32>(a, ws, L, stream);
  else
    return CT == 32 ? comba_dispatch_nw<DK, 32>(a, ws, L, stream) : comba_dispatch_nw<DK, 64>(a, ws, L, stream);
}

}  // namespace
}  // namespace gdn

extern "C" size_t gdn_chunk_prefill_workspace(int64_t T_tot, int N_s, int Hk, int Hv, int Dk, int Dv,
                                              int chunk, gdn_dtype act) {
  (void)Dv;
  if (T_tot < 0 || N_s < 0 || Hk <= 0 || Hv <= 0 || Dk <= 0 || !gdn::valid_chunk(chunk) ||
      !gdn::is_act(act))
    return 0;
  return gdn::layout(T_tot, N_s, Hv, gdn::effective_chunk(Dk, chunk), act == GDN_BF16).total;
}

namespace gdn {
namespace {

// Every host-side check, then (unless check_only) the launches.  With
// no_ws_checks (a check-only pass for the library's own scratch) the checks
// of the workspace pointer, size and overlaps are left out.
int chunk_prefill(const void* q, const void* k, const void* v, const float* g, const float* beta,
                  float* state_pool, int64_t pool_size, const int64_t* cache_indices,
                  const int64_t* cu_seqlens, int N_s, int64_t T_tot, int Hk, int Hv, int Dk, int Dv,
                  int chunk, float scale, unsigned flags, void* y, gdn_dtype act, void* workspace,
                  size_t workspace_bytes, const Epilogue* epi, hipStream_t stream,
                  bool check_only = false, int64_t max_len = 0, bool no_ws_checks = false,
                  const RawGates* raw = nullptr, const FixedBatch* fixb = nullptr) {
  if (N_s < 0 || T_tot < 0 || pool_size < 0 || Hk <= 0 || Hv <= 0 || Dk <= 0 || Dv <= 0 ||
      Hv % Hk != 0)
    return GDN_ERR_SHAPE;
  if (!is_act(act)) return GDN_ERR_DTYPE;
  if (!(valid_head(Dk) && (Dk <= 128 || act == GDN_BF16)) || Dv % 32 != 0 ||
      Dv > 256 || !valid_chunk(chunk) || (flags & ~static_cast<unsigned>(GDN_QK_L2NORM | GDN_KEEP_STATE)) != 0)
    return GDN_ERR_UNSUPPORTED;
  chunk = effective_chunk(Dk, chunk);
  if (N_s == 0) return GDN_OK;
  if (!cache_indices || !cu_seqlens || !state_pool || (!workspace && !no_ws_checks)) return GDN_ERR_NULL;
  if (T_tot > 0 && (!q || !k || !v || !y || (raw ? (!raw->a || !raw->b || !raw->A_log || !raw->dt_bias)
                                                     : (!g || !beta))))
    return GDN_ERR_NULL;
  if (raw && act != GDN_BF16) return GDN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(state_pool) ||
      (!aligned16(workspace) && !no_ws_checks))
    return GDN_ERR_ALIGN;
  // per-chunk copy offsets are 32-bit: 64 token rows of q/k/v must span < 1 GiB
  if (static_cast<uint64_t>(Hk) * Dk * 2 * 64 >= (1ull << 30) ||
      static_cast<uint64_t>(Hv) * Dv * 2 * 64 >= (1ull << 30))
    return GDN_ERR_UNSUPPORTED;
  const Layout L = layout(T_tot, N_s, Hv, chunk, act == GDN_BF16);
  if (workspace_bytes < L.total && !no_ws_checks) return GDN_ERR_WORKSPACE;
  const size_t ws_bytes = no_ws_checks ? 0 : L.total;  // an empty span overlaps nothing
  const size_t pool_bytes = static_cast<size_t>(pool_size) * Hv * Dv * Dk * sizeof(float);
  const size_t y_bytes = static_cast<size_t>(T_tot) * Hv * Dv * act_bytes(act);
  if (overlaps(y, y_bytes, state_pool, pool_bytes) || overlaps(workspace, ws_bytes, state_pool, pool_bytes) ||
      overlaps(workspace, ws_bytes, y, y_bytes))
    return GDN_ERR_ALIAS;
  if (epi && (overlaps(epi->z, y_bytes, state_pool, pool_bytes) || overlaps(epi->z, y_bytes, workspace, ws_bytes)))
    return GDN_ERR_ALIAS;
  {
    const size_t qk_bytes = static_cast<size_t>(T_tot) * Hk * Dk * act_bytes(act);
    const size_t v_bytes = static_cast<size_t>(T_tot) * Hv * Dv * act_bytes(act);
    const size_t gb_bytes = static_cast<size_t>(T_tot) * Hv * sizeof(float);
    const Span out[] = {{y, y_bytes}, {state_pool, pool_bytes}, {workspace, ws_bytes}};
    if (raw) {
      const size_t ab_bytes = static_cast<size_t>(T_tot) * Hv * act_bytes(act);
      const size_t h_bytes = static_cast<size_t>(Hv) * sizeof(float);
      const Span in[] = {{q, qk_bytes}, {k, qk_bytes}, {v, v_bytes}, {raw->a, ab_bytes}, {raw->b, ab_bytes},
                         {raw->A_log, h_bytes}, {raw->dt_bias, h_bytes}};
      if (inputs_overlap_outputs(in, out)) return GDN_ERR_ALIAS;
    } else {
      const Span in[] = {{q, qk_bytes}, {k, qk_bytes}, {v, v_bytes}, {g, gb_bytes}, {beta, gb_bytes}};
      if (inputs_overlap_outputs(in, out)) return GDN_ERR_ALIAS;
    }
  }
  if (check_only) return GDN_OK;
  if (!(scale > 0.0f)) scale = 1.0f / sqrtf(static_cast<float>(Dk));
  const int l2 = (flags & GDN_QK_L2NORM) ? 1 : 0;
  const int CT = chunk_tile(chunk);
  char* ws = static_cast<char*>(workspace);
  // max_len > 0: no sequence is longer (the caller knows it); then whether
  // every sequence fits one chunk
  const bool one_chunk = max_len > 0 && max_len <= chunk;
  const unsigned opts = (one_chunk ? kOneChunk : 0u) | ((flags & GDN_KEEP_STATE) ? kKeepState : 0u);
  if (act == GDN_BF16)
    return dispatch_dk<bf16>(Dk, CT, Dv, q, k, v, g, beta, state_pool, pool_size, cache_indices,
                             cu_seqlens, N_s, T_tot, Hk, Hv, chunk, scale, l2, y, ws, L, epi, raw, fixb, stream, opts);
  return dispatch_dk<float>(Dk, CT, Dv, q, k, v, g, beta, state_pool, pool_size, cache_indices,
                            cu_seqlens, N_s, T_tot, Hk, Hv, chunk, scale, l2, y, ws, L, epi, raw, fixb, stream, opts);
}

}  // namespace
}  // namespace gdn

extern "C" int gdn_chunk_prefill(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, float* state_pool, int64_t pool_size,
                                 const int64_t* cache_indices, const int64_t* cu_seqlens, int N_s,
                                 int64_t T_tot, int Hk, int Hv, int Dk, int Dv, int chunk,
                                 float scale, unsigned flags, void* y, gdn_dtype act,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return gdn::chunk_prefill(q, k, v, g, beta, state_pool, pool_size, cache_indices, cu_seqlens, N_s,
                            T_tot, Hk, Hv, Dk, Dv, chunk, scale, flags, y, act, workspace, workspace_bytes,
                            nullptr, stream);
}

// ------------------------------------------------- prefill from raw gates
//
// gdn_chunk_prefill_raw: the gates from the raw inputs in the same call.
// bf16 activations form them inside the WY pass (the only kernel that reads
// them); fp32 activations run gdn_prefill_gates into the workspace's tail
// first.  Either way the gates are those gdn_prefill_gates writes, bit for
// bit (gates_of).

extern "C" size_t gdn_chunk_prefill_raw_workspace(int64_t T_tot, int N_s, int Hk, int Hv, int Dk, int Dv,
                                                  int chunk, gdn_dtype act) {
  const size_t base = gdn_chunk_prefill_workspace(T_tot, N_s, Hk, Hv, Dk, Dv, chunk, act);
  if (base == 0 || act == GDN_BF16) return base;
  return base + gdn::up(2 * static_cast<size_t>(T_tot) * static_cast<size_t>(Hv) * sizeof(float));
}

extern "C" int gdn_chunk_prefill_raw(const void* q, const void* k, const void* v, const void* a,
                                     const void* b, const float* A_log, const float* dt_bias,
                                     float* state_pool, int64_t pool_size, const int64_t* cache_indices,
                                     const int64_t* cu_seqlens, int N_s, int64_t T_tot, int Hk, int Hv,
                                     int Dk, int Dv, int chunk, float scale, unsigned flags, void* y,
                                     gdn_dtype act, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  using namespace gdn;
  if (act == GDN_BF16) {
    const RawGates rg{static_cast<const bf16*>(a), static_cast<const bf16*>(b), A_log, dt_bias};
    return chunk_prefill(q, k, v, nullptr, nullptr, state_pool, pool_size, cache_indices, cu_seqlens, N_s, T_tot,
                         Hk, Hv, Dk, Dv, chunk, scale, flags, y, act, workspace, workspace_bytes, nullptr, stream,
                         false, 0, false, &rg);
  }
  if (!is_act(act)) return GDN_ERR_DTYPE;
  if (N_s < 0 || T_tot < 0 || Hv <= 0) return GDN_ERR_SHAPE;
  if (N_s == 0) return chunk_prefill(q, k, v, nullptr, nullptr, state_pool, pool_size, cache_indices, cu_seqlens,
                                     N_s, T_tot, Hk, Hv, Dk, Dv, chunk, scale, flags, y, act, workspace,
                                     workspace_bytes, nullptr, stream);
  const size_t base = gdn_chunk_prefill_workspace(T_tot, N_s, Hk, Hv, Dk, Dv, chunk, act);
  const size_t need = gdn_chunk_prefill_raw_workspace(T_tot, N_s, Hk, Hv, Dk, Dv, chunk, act);
  if (!workspace) return GDN_ERR_NULL;
  if (need == 0 || workspace_bytes < need) return base == 0 ? GDN_ERR_UNSUPPORTED : GDN_ERR_WORKSPACE;
  if (T_tot > 0 && (!a || !b || !A_log || !dt_bias)) return GDN_ERR_NULL;
  float* g = reinterpret_cast<float*>(static_cast<char*>(workspace) + base);
  float* beta = g + static_cast<size_t>(T_tot) * Hv;
  {  // the raw inputs must not overlap the gates' scratch or the outputs
    const size_t ab = static_cast<size_t>(T_tot) * Hv * act_bytes(act), hb = static_cast<size_t>(Hv) * 4;
    const size_t yb = static_cast<size_t>(T_tot) * Hv * Dv * act_bytes(act);
    const size_t pb = static_cast<size_t>(pool_size < 0 ? 0 : pool_size) * Hv * Dv * Dk * sizeof(float);
    const Span in[] = {{a, ab}, {b, ab}, {A_log, hb}, {dt_bias, hb}};
    const Span out[] = {{workspace, need}, {y, yb}, {state_pool, pb}};
    if (inputs_overlap_outputs(in, out)) return GDN_ERR_ALIAS;
  }
  // every other check before any launch
  int rc = chunk_prefill(q, k, v, g, beta, state_pool, pool_size, cache_indices, cu_seqlens, N_s, T_tot, Hk, Hv,
                         Dk, Dv, chunk, scale, flags, y, act, workspace, base, nullptr, stream, true);
  if (rc != GDN_OK) return rc;
  rc = gdn_prefill_gates(a, b, A_log, dt_bias, g, beta, T_tot, Hv, act, stream);
  if (rc != GDN_OK) return rc;
  return chunk_prefill(q, k, v, g, beta, state_pool, pool_size, cache_indices, cu_seqlens, N_s, T_tot, Hk, Hv, Dk,
                       Dv, chunk, scale, flags, y, act, workspace, base, nullptr, stream);
}

extern "C" int gdn_chunk_prefill_gated(const void* q, const void* k, const void* v, const float* g,
                                       const float* beta, float* state_pool, int64_t pool_size,
                                       const int64_t* cache_indices, const int64_t* cu_seqlens, int N_s,
                                       int64_t T_tot, int Hk, int Hv, int Dk, int Dv, int chunk,
                                       float scale, unsigned flags, const void* z, const float* gamma,
                                       float eps, void* y, gdn_dtype act, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  using namespace gdn;
  if (N_s < 0 || T_tot < 0 || Hv <= 0 || Dv <= 0) return GDN_ERR_SHAPE;
  if (!(eps >= 0.0f)) return GDN_ERR_SHAPE;
  if (!pow2_head(Dv)) return GDN_ERR_UNSUPPORTED;
  if (N_s > 0 && T_tot > 0) {
    if (!z || !gamma) return GDN_ERR_NULL;
    if (!aligned16(z) || !aligned16(gamma)) return GDN_ERR_ALIGN;
    if (is_act(act)) {
      const size_t nb = static_cast<size_t>(T_tot) * Hv * Dv * act_bytes(act);
      if (y && overlaps(z, nb, y, nb)) return GDN_ERR_ALIAS;
    }
  }
  const Epilogue epi{z, gamma, eps};
  return chunk_prefill(q, k, v, g, beta, state_pool, pool_size, cache_indices, cu_seqlens, N_s, T_tot, Hk,
                       Hv, Dk, Dv, chunk, scale, flags, y, act, workspace, workspace_bytes, &epi, stream);
}

// ------------------------------------------- prefill with the conv prologue
//
// gdn_conv_prefill: the layer's prefill from its raw channels.  The WY pass
// runs the conv prologue of its chunk (conv_chunk) and the gates from the raw
// inputs; the convolved q, k, v go to the workspace's tail, which the chunk
// loop reads; the gated norm, when z is given, as gdn_chunk_prefill_gated.

namespace gdn {
namespace {

struct ConvLayout {
  size_t base, q, k, v, trash, total;
};

inline ConvLayout conv_layout(size_t base, int64_t T_tot, int Hk, int Hv, int Dk, int Dv) {
  ConvLayout c;
  c.base = base;
  c.q = base;
  c.k = c.q + up(static_cast<size_t>(T_tot) * Hk * Dk * sizeof(bf16));
  c.v = c.k + up(static_cast<size_t>(T_tot) * Hk * Dk * sizeof(bf16));
  c.trash = c.v + up(static_cast<size_t>(T_tot) * Hv * Dv * sizeof(bf16));
  c.total = c.trash + kAlign;
  return c;
}

}  // namespace
}  // namespace gdn

extern "C" size_t gdn_conv_prefill_workspace(int64_t T_tot, int N_s, int Hk, int Hv, int Dk, int Dv, int chunk) {
  const size_t base = gdn_chunk_prefill_workspace(T_tot, N_s, Hk, Hv, Dk, Dv, chunk, GDN_BF16);
  if (base == 0 || Dv <= 0) return 0;
  return gdn::conv_layout(base, T_tot, Hk, Hv, Dk, Dv).total;
}

extern "C" int gdn_conv_prefill(const void* qkv, const float* conv_w, float* conv_state, const void* a,
                                const void* b, const float* A_log, const float* dt_bias, float* state_pool,
                                int64_t pool_size, const int64_t* cache_indices, const int64_t* cu_seqlens,
                                int N_s, int64_t T_tot, int Hk, int Hv, int Dk, int Dv, int chunk, float scale,
                                unsigned flags, const void* z, const float* gamma, float eps, void* y,
                                gdn_dtype act, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace gdn;
  if (N_s < 0 || T_tot < 0 || pool_size < 0 || Hk <= 0 || Hv <= 0 || Dk <= 0 || Dv <= 0 || Hv % Hk != 0)
    return GDN_ERR_SHAPE;
  if (!is_act(act)) return GDN_ERR_DTYPE;
  if (act != GDN_BF16) return GDN_ERR_UNSUPPORTED;
  if (z && !(eps >= 0.0f)) return GDN_ERR_SHAPE;
  if (z && !pow2_head(Dv)) return GDN_ERR_UNSUPPORTED;
  const size_t base = gdn_chunk_prefill_workspace(T_tot, N_s, Hk, Hv, Dk, Dv, chunk, act);
  if (base == 0) return GDN_ERR_UNSUPPORTED;
  const ConvLayout cl = conv_layout(base, T_tot, Hk, Hv, Dk, Dv);
  if (N_s == 0) return GDN_OK;
  if (!workspace) return GDN_ERR_NULL;
  if (workspace_bytes < cl.total) return GDN_ERR_WORKSPACE;
  const size_t C = 2 * static_cast<size_t>(Hk) * Dk + static_cast<size_t>(Hv) * Dv;
  const size_t x_bytes = static_cast<size_t>(T_tot) * C * sizeof(bf16);
  const size_t w_bytes = C * 4 * sizeof(float);
  const size_t h_bytes = static_cast<size_t>(pool_size) * C * 3 * sizeof(float);
  const size_t y_bytes = static_cast<size_t>(T_tot) * Hv * Dv * sizeof(bf16);
  const size_t p_bytes = static_cast<size_t>(pool_size) * Hv * Dv * Dk * sizeof(float);
  if (T_tot > 0) {
    if (!qkv || !conv_w || !conv_state || (z && !gamma)) return GDN_ERR_NULL;
    if (!aligned16(qkv) || !aligned16(conv_w) || !aligned16(conv_state) || (z && (!aligned16(z) || !aligned16(gamma))))
      return GDN_ERR_ALIGN;
    const size_t ab_bytes = static_cast<size_t>(T_tot) * Hv * sizeof(bf16);
    const size_t hv_bytes = static_cast<size_t>(Hv) * sizeof(float);
    const Span in[] = {{qkv, x_bytes}, {conv_w, w_bytes}, {z, z ? y_bytes : 0}, {a, ab_bytes},
                       {b, ab_bytes}, {A_log, hv_bytes}, {dt_bias, hv_bytes}};
    const Span out[] = {{conv_state, h_bytes}, {y, y_bytes}, {state_pool, p_bytes}, {workspace, cl.total}};
    if (inputs_overlap_outputs(in, out)) return GDN_ERR_ALIAS;
    if (overlaps(conv_state, h_bytes, y, y_bytes) || overlaps(conv_state, h_bytes, state_pool, p_bytes) ||
        overlaps(conv_state, h_bytes, workspace, cl.total) || overlaps(y, y_bytes, workspace, cl.total) ||
        overlaps(state_pool, p_bytes, workspace, cl.total))
      return GDN_ERR_ALIAS;
  }
  char* ws = static_cast<char*>(workspace);
  bf16* cq = reinterpret_cast<bf16*>(ws + cl.q);
  bf16* ck = reinterpret_cast<bf16*>(ws + cl.k);
  bf16* cv = reinterpret_cast<bf16*>(ws + cl.v);
  RawGates rg{static_cast<const bf16*>(a), static_cast<const bf16*>(b), A_log, dt_bias,
              ConvIn{static_cast<const bf16*>(qkv), conv_w, conv_state, cache_indices, pool_size, cq, ck, cv,
                     reinterpret_cast<bf16*>(ws + cl.trash), Dv, (flags & GDN_KEEP_STATE) ? 1 : 0}};
  const Epilogue epi{z, gamma, eps};
  // the prefill's own checks (the convolved rows lie past its workspace span)
  return chunk_prefill(cq, ck, cv, nullptr, nullptr, state_pool, pool_size, cache_indices, cu_seqlens, N_s, T_tot,
                       Hk, Hv, Dk, Dv, chunk, scale, flags, y, act, workspace, base, z ? &epi : nullptr, stream,
                       false, 0, false, &rg);
}

extern "C" int gdn_validate_varlen(const int64_t* cu_seqlens, const int64_t* cache_indices, int N_s,
                                   int64_t T_tot, int64_t pool_size, hipStream_t stream) {
  using namespace gdn;
  if (N_s < 0 || T_tot < 0 || pool_size < 0) return GDN_ERR_SHAPE;
  if (N_s == 0) return T_tot == 0 ? GDN_OK : GDN_ERR_SHAPE;
  if (!cu_seqlens || !cache_indices) return GDN_ERR_NULL;
  const size_t n = static_cast<size_t>(N_s);
  int64_t* h = static_cast<int64_t*>(malloc(sizeof(int64_t) * (2 * n + 1)));
  if (!h) return GDN_ERR_DEVICE;
  int rc = GDN_OK;
  if (hipMemcpyAsync(h, cu_seqlens, sizeof(int64_t) * (n + 1), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipMemcpyAsync(h + n + 1, cache_indices, sizeof(int64_t) * n, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    rc = GDN_ERR_DEVICE;
  } else {
    const int64_t* cu = h;
    const int64_t* ci = h + n + 1;
    if (cu[0] != 0 || cu[n] != T_tot) rc = GDN_ERR_SHAPE;
    for (size_t s = 0; rc == GDN_OK && s < n; ++s)
      if (cu[s + 1] < cu[s] || ci[s] < 0 || ci[s] >= pool_size) rc = GDN_ERR_SHAPE;
    for (size_t a = 0; rc == GDN_OK && a < n; ++a)
      for (size_t b = a + 1; b < n; ++b)
        if (ci[a] == ci[b]) { rc = GDN_ERR_SHAPE; break; }
  }
  free(h);
  return rc;
}

extern "C" size_t comba_chunk_prefill_workspace(int64_t T_tot, int N_s, int H, int K, int V, int chunk,
                                                gdn_dtype act) {
  (void)V;
  if (T_tot < 0 || N_s < 0 || H <= 0 || K <= 0 || !gdn::valid_chunk(chunk) || act != GDN_BF16) return 0;
  return gdn::layout(T_tot, N_s, H, gdn::effective_chunk(K, chunk), true).total;
}

extern "C" int comba_chunk_prefill(const void* q, const void* k, const void* v, const void* p,
                                   const void* beta, const float* g, float* state_pool, int64_t pool_size,
                                   const int64_t* cache_indices, const int64_t* cu_seqlens, int N_s,
                                   int64_t T_tot, int H, int K, int V, int chunk, float scale, void* o,
                                   gdn_dtype act, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  using namespace gdn;
  if (N_s < 0 || T_tot < 0 || pool_size < 0 || H <= 0 || K <= 0 || V <= 0) return GDN_ERR_SHAPE;
  if (!is_act(act)) return GDN_ERR_DTYPE;
  if (act != GDN_BF16 || !valid_head(K) || V % 32 != 0 || V > 256 ||
      !valid_chunk(chunk))
    return GDN_ERR_UNSUPPORTED;
  chunk = effective_chunk(K, chunk);
  if (N_s == 0) return GDN_OK;
  if (!cache_indices || !cu_seqlens || !state_pool || !workspace) return GDN_ERR_NULL;
  if (T_tot > 0 && (!q || !k || !v || !p || !beta || !g || !o)) return GDN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(p) || !aligned16(state_pool) ||
      !aligned16(workspace))
    return GDN_ERR_ALIGN;
  // per-chunk copy offsets are 32-bit: 64 token rows of q/k/p/v must span < 1 GiB
  if (static_cast<uint64_t>(H) * K * 2 * 64 >= (1ull << 30) || static_cast<uint64_t>(H) * V * 2 * 64 >= (1ull << 30))
    return GDN_ERR_UNSUPPORTED;
  const Layout L = layout(T_tot, N_s, H, chunk, true);
  if (workspace_bytes < L.total) return GDN_ERR_WORKSPACE;
  const size_t pool_bytes = static_cast<size_t>(pool_size) * H * K * V * sizeof(float);
  const size_t o_bytes = static_cast<size_t>(T_tot) * H * V * sizeof(bf16);
  if (overlaps(o, o_bytes, state_pool, pool_bytes) || overlaps(workspace, L.total, state_pool, pool_bytes) ||
      overlaps(workspace, L.total, o, o_bytes))
    return GDN_ERR_ALIAS;
  {
    const size_t qk_bytes = static_cast<size_t>(T_tot) * H * K * sizeof(bf16);
    const size_t tb = static_cast<size_t>(T_tot) * H;
    const Span in[] = {{q, qk_bytes}, {k, qk_bytes}, {p, qk_bytes}, {v, o_bytes},
                       {beta, tb * sizeof(bf16)}, {g, tb * sizeof(float)}};
    const Span out[] = {{o, o_bytes}, {state_pool, pool_bytes}, {workspace, L.total}};
    if (inputs_overlap_outputs(in, out)) return GDN_ERR_ALIAS;
  }
  if (!(scale > 0.0f)) scale = 1.0f / sqrtf(static_cast<float>(K));
  const CombaArgs a{static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(v),
                    static_cast<const bf16*>(p), static_cast<const bf16*>(beta), g, state_pool, pool_size,
                    cache_indices, cu_seqlens, N_s, T_tot, H, V, chunk, scale, static_cast<bf16*>(o)};
  char* ws = static_cast<char*>(workspace);
  const int CT = chunk_tile(chunk);
  switch (K) {
    case 32: return comba_dispatch_ct<32>(CT, a, ws, L, stream);
    case 64: return comba_dispatch_ct<64>(CT, a, ws, L, stream);
    case 96: return comba_dispatch_ct<96>(CT, a, ws, L, stream);
    case 128: return comba_dispatch_ct<128>(CT, a, ws, L, stream);
    case 160: return comba_dispatch_ct<160>(CT, a, ws, L, stream);
    case 192: return comba_dispatch_ct<192>(CT, a, ws, L, stream);
    case 224: return comba_dispatch_ct<224>(CT, a, ws, L, stream);
    default: return comba_dispatch_ct<256>(CT, a, ws, L, stream);
  }
}

// ---------------------------------------------------------------------------
// Fixed-T batch layout: q, k [B, T, Hk, Dk], v, y [B, T, Hv, Dv], g, beta
// [B, T, Hv], state [B, Hv, Dv, Dk] -- the packed varlen layout with B
// sequences of T tokens and state slot b for sequence b.  The index arrays
// go to the end of the workspace (written by a small kernel on the stream),
// then the varlen path runs.

namespace gdn {
namespace {
inline size_t fixed_index_bytes(int B) { return up(sizeof(int64_t) * (2 * static_cast<size_t>(B) + 1)); }
}  // namespace
}  // namespace gdn

extern "C" size_t gdn_chunk_prefill_fixed_workspace(int B, int64_t T, int Hk, int Hv, int Dk, int Dv,
                                                    int chunk, gdn_dtype act) {
  if (B < 0 || T < 0 || (T > 0 && B > INT64_MAX / T)) return 0;
  const size_t main = gdn_chunk_prefill_workspace(static_cast<int64_t>(B) * T, B, Hk, Hv, Dk, Dv, chunk, act);
  return main ? main + gdn::fixed_index_bytes(B) : 0;
}

extern "C" int gdn_chunk_prefill_fixed(const void* q, const void* k, const void* v, const float* g,
                                       const float* beta, float* state, int B, int64_t T, int Hk,
                                       int Hv, int Dk, int Dv, int chunk, float scale, unsigned flags,
                                       void* y, gdn_dtype act, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  using namespace gdn;
  if (B < 0 || T < 0 || (T > 0 && B > INT64_MAX / T) || Hk <= 0 || Hv <= 0 || Dk <= 0 || Dv <= 0 ||
      Hv % Hk != 0)
    return GDN_ERR_SHAPE;
  if (!is_act(act)) return GDN_ERR_DTYPE;
  if (B == 0 || T == 0) return GDN_OK;
  if (!workspace) return GDN_ERR_NULL;
  const size_t total = gdn_chunk_prefill_fixed_workspace(B, T, Hk, Hv, Dk, Dv, chunk, act);
  if (total == 0) return GDN_ERR_UNSUPPORTED;
  if (workspace_bytes < total) return GDN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GDN_ERR_ALIGN;
  const size_t main = total - fixed_index_bytes(B);
  int64_t* cu = reinterpret_cast<int64_t*>(static_cast<char*>(workspace) + main);
  int64_t* ci = cu + B + 1;
  // the index arrays must not overlap the state or y (the varlen call checks the rest)
  const size_t state_bytes = static_cast<size_t>(B) * Hv * Dv * Dk * sizeof(float);
  const size_t y_bytes = static_cast<size_t>(B) * T * Hv * Dv * act_bytes(act);
  const size_t qk_bytes = static_cast<size_t>(B) * T * Hk * Dk * act_bytes(act);
  const size_t gb_bytes = static_cast<size_t>(B) * T * Hv * sizeof(float);
  {
    const Span in[] = {{q, qk_bytes}, {k, qk_bytes}, {v, y_bytes}, {g, gb_bytes}, {beta, gb_bytes}};
    const Span out[] = {{cu, total - main}};
    if (overlaps(cu, total - main, state, state_bytes) || overlaps(cu, total - main, y, y_bytes) ||
        inputs_overlap_outputs(in, out))
      return GDN_ERR_ALIAS;
  }
  // everything the varlen call checks, before the index kernel touches the device
  const int rc = chunk_prefill(q, k, v, g, beta, state, B, ci, cu, B, static_cast<int64_t>(B) * T, Hk, Hv, Dk,
                               Dv, chunk, scale, flags, y, act, workspace, main, nullptr, stream, true);
  if (rc != GDN_OK) return rc;
  if (act == GDN_BF16) {  // the WY launch writes the index arrays and the chunk map
    const FixedBatch fb{T, cu, ci};
    return chunk_prefill(q, k, v, g, beta, state, B, ci, cu, B, static_cast<int64_t>(B) * T, Hk, Hv, Dk, Dv,
                         chunk, scale, flags, y, act, workspace, main, nullptr, stream, false, T, false, nullptr,
                         &fb);
  }
  (void)hipGetLastError();
  hipLaunchKernelGGL(gdn_fixed_index_kernel, dim3(static_cast<unsigned>((B + 1 + 255) / 256)), dim3(256), 0,
                     stream, cu, ci, B, T);
  if (launch_status() != GDN_OK) return GDN_ERR_LAUNCH;
  return chunk_prefill(q, k, v, g, beta, state, B, ci, cu, B, static_cast<int64_t>(B) * T, Hk, Hv, Dk, Dv,
                       chunk, scale, flags, y, act, workspace, main, nullptr, stream, false, T);
}

// ------------------------------------------------- allocation-free prefill
//
// gdn_chunk_prefill_noalloc: the same call with the workspace in a static
// device array of this library instead of caller memory, for callers that
// cannot allocate (code under graph capture, tight serving loops).  Every
// GPU the library runs on holds its own copy of the array until the process
// ends.  Nothing in the workspace needs to start at zero: the chunk-map
// kernel writes every index the later kernels read, and the WY pass writes
// every plane and factor record the chunk loop reads.

namespace gdn {
namespace {

constexpr size_t kScratchBytes = size_t{128} << 20;
constexpr int kScratchDevices = 64;

std::mutex scratch_mutex;
void* scratch_address[kScratchDevices];

}  // namespace
}  // namespace gdn

static __device__ __align__(256) unsigned char scratch[gdn::kScratchBytes];

namespace gdn {
namespace {

// Device address of `scratch` on the current device, looked up on the first
// call there and kept.  The array's name in host code stands for a host-side
// shadow, never for device memory: only this address reaches a kernel.
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return GDN_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_address[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return GDN_ERR_DEVICE;
    }
    scratch_address[dev] = p;
  }
  *out = scratch_address[dev];
  return GDN_OK;
}

}  // namespace
}  // namespace gdn

extern "C" int gdn_chunk_prefill_noalloc(const void* q, const void* k, const void* v, const float* g,
                                         const float* beta, float* state_pool, int64_t pool_size,
                                         const int64_t* cache_indices, const int64_t* cu_seqlens, int N_s,
                                         int64_t T_tot, int Hk, int Hv, int Dk, int Dv, int chunk,
                                         float scale, unsigned flags, void* y, gdn_dtype act,
                                         hipStream_t stream) {
  using namespace gdn;
  // every check of the caller's arguments first, before any HIP call
  const int pre = chunk_prefill(q, k, v, g, beta, state_pool, pool_size, cache_indices, cu_seqlens, N_s, T_tot,
                                Hk, Hv, Dk, Dv, chunk, scale, flags, y, act, nullptr, 0, nullptr, stream, true, 0,
                                true);
  if (pre != GDN_OK || N_s == 0) return pre;
  const size_t need = gdn_chunk_prefill_workspace(T_tot, N_s, Hk, Hv, Dk, Dv, chunk, act);
  if (need == 0 || need > kScratchBytes) return GDN_ERR_WORKSPACE;
  void* ws = nullptr;
  const int st = scratch_on_current_device(&ws);
  if (st != GDN_OK) return st;
  return chunk_prefill(q, k, v, g, beta, state_pool, pool_size, cache_indices, cu_seqlens, N_s, T_tot, Hk, Hv,
                       Dk, Dv, chunk, scale, flags, y, act, ws, kScratchBytes, nullptr, stream);
}
