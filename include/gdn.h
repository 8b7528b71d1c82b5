/*
 * gdn.h - C ABI of libgdn: the gated delta-rule (Gated DeltaNet) recurrence
 * on AMD Instinct MI355X (gfx950), as hand-written HIP kernels.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument is a device pointer (memory the caller allocated
 *   on the current HIP device).  The library never allocates or frees memory,
 *   keeps no pointer after returning and never synchronises: all work is
 *   enqueued on `stream` (0 = the null stream) and finishes asynchronously.
 * - The recurrent state is always float32 and every state computation is
 *   done in float32.  Activations (q, k, v, p, beta, y, o, a, b) have the
 *   dtype `act`: GDN_F32 (float32) or GDN_BF16 (bfloat16 bits, values are
 *   rounded to nearest-even when written).  The log-space gate g is always
 *   float32; the gate applied to the state is exp(g).
 * - All tensors are dense, row-major, with the last dimension contiguous.
 * - Return value: GDN_OK (0) or a negative GDN_ERR_* code.  Argument checks
 *   (null pointers, shapes, dtype, alignment, aliasing, workspace size) are
 *   made on the host before any HIP call, so an invalid call touches no
 *   device state.  GDN_ERR_LAUNCH reports a failed kernel launch; faults
 *   inside a kernel surface at the caller's next synchronisation.
 * - Calls on one stream run in order; calls that write the same memory from
 *   different streams race, as with any HIP kernel.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_NULL = -1,        /* a required pointer is NULL                      */
  GDN_ERR_SHAPE = -2,       /* a size is negative or inconsistent             */
  GDN_ERR_DTYPE = -3,       /* `act` is not a gdn_dtype                        */
  GDN_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned where required */
  GDN_ERR_UNSUPPORTED = -5, /* a head size or chunk size this build lacks      */
  GDN_ERR_WORKSPACE = -6,   /* workspace missing or smaller than required      */
  GDN_ERR_LAUNCH = -7,      /* the kernel launch failed                        */
  GDN_ERR_DEVICE = -8,      /* no usable HIP device                            */
  GDN_ERR_ALIAS = -9        /* two buffers overlap in a way that is not allowed */
};

/*
 * gdn_decode_step - one single-token gated delta-rule step for a dense decode
 * batch.  Source: metaltile-std `gated_delta.rs` (docs.rs), module doc
 * sections "Recurrence per step" and "Layouts", and the DISPATCH INVARIANTS
 * of `mt_gated_delta_step`.  For every sequence b and value head hv, with
 * key head hk = hv / (Hv / Hk) (consecutive value heads share a key head) and
 * S the [Dv, Dk] state slice of (b, hv):
 *     S    <- exp(g) * S
 *     kv_j  = sum_i S[j, i] k[i]
 *     d_j   = beta * (v_j - kv_j)
 *     S[j, i] <- S[j, i] + d_j k[i]
 *     y_j   = sum_i S[j, i] q[i]        (no query scale: pre-scale q)
 *
 * state_in  [B, Hv, Dv, Dk] float32, read only.
 * state_out [B, Hv, Dv, Dk] float32, written.  May equal state_in exactly
 *           (in-place update); any other overlap is GDN_ERR_ALIAS.
 * q, k      [B, Hk, Dk] act.     v, y [B, Hv, Dv] act.
 * g         [B, Hv] float32 (log-space gate).   beta [B, Hv] act.
 * Requirements: Hk >= 1, Hv % Hk == 0, Dk a multiple of 32 in [32, 256],
 * Dv a multiple of 32 in [32, 256], B >= 0 (B == 0 is a no-op);
 * state_in, state_out, q and k 16-byte aligned.  y overlaps neither state;
 * no input (q, k, v, g, beta) overlaps y or state_out (GDN_ERR_ALIAS).
 */
int gdn_decode_step(const float* state_in, float* state_out, const void* q,
                    const void* k, const void* v, const float* g,
                    const void* beta, void* y, int B, int Hk, int Hv, int Dk,
                    int Dv, gdn_dtype act, hipStream_t stream);

/*
 * gdn_decode_window - T decode tokens per sequence in one pass, with the
 * state kept on chip across them (metaltile `mt_gated_delta_chunk`: the
 * recurrent state lives in registers across an inner token loop; regolith
 * `gdn.metal` commit rule for verify windows).  Token t of sequence b is
 * the gdn_decode_step above applied to the state after tokens 0..t-1.
 * q, k          [B, T, Hk, Dk] act.     v, y: [B, T, Hv, Dv] act.
 * g, beta       [B, T, Hv] (g float32 log-space, beta act).
 * state_in      [B, Hv, Dv, Dk] float32, read.
 * state_out     [B, Hv, Dv, Dk] float32: receives the state after the first
 *               `commit` tokens (0 <= commit <= T); commit == 0 is a verify
 *               window (state_out not written, may be NULL); may equal
 *               state_in; every token's y is written in all cases.
 * Requirements: 1 <= T <= 8 and the gdn_decode_step sizes; q, k,
 * state_in, state_out 16-byte aligned; the aliasing rules of
 * gdn_decode_step (state_out counts as written only when commit > 0).
 * A committed window (commit == T) is also gdn_chunk_prefill_fixed with
 * flags 0 and scale 1 on the same layouts (in place on the state, with a
 * workspace), and a verify window (commit == 0) the same call with flags
 * GDN_KEEP_STATE; from T = 4 on that MFMA path is the faster of the two.
 */
int gdn_decode_window(const float* state_in, float* state_out, const void* q,
                      const void* k, const void* v, const float* g,
                      const void* beta, void* y, int B, int T, int Hk, int Hv,
                      int Dk, int Dv, int commit, gdn_dtype act,
                      hipStream_t stream);

/*
 * comba_decode_step - one Comba step (gated delta rule with a decoupled read
 * key) for a dense batch.  Source: KBench `comba_decode_step` spec, sections
 * spec_md and contract_md.  For every (b, h), S the [K, V] state slice:
 *     S    <- exp(g) * S
 *     u_j   = beta * (v_j - sum_i p[i] S[i, j])       (read with p)
 *     S[i, j] <- S[i, j] + k[i] u_j                    (write with k)
 *     o_j   = sum_i (scale q[i]) S[i, j]               (updated state)
 *
 * state     [B, H, K, V] float32, read only.
 * state_new [B, H, K, V] float32, written; may equal `state` exactly.
 * q, k, p   [B, H, K] act.   v, o [B, H, V] act.   beta [B, H] act.
 * g         [B, H] float32 (log-decay, <= 0 in practice).
 * scale     query scale; a value <= 0 selects K^-1/2.
 * Requirements: K and V multiples of 32 in [32, 256] with at most 32 state
 * rows per thread: K * L <= 8192, L = V/4 rounded up to a power of two
 * (every K with V <= 128; K <= 128 with V > 128); B, H >= 0;
 * state, state_new, q, k, p, v and o 16-byte aligned.  o overlaps neither
 * state; no input (q, k, p, v, beta, g) overlaps o or state_new
 * (GDN_ERR_ALIAS).
 */
int comba_decode_step(const float* state, float* state_new, const void* q,
                      const void* k, const void* v, const void* p,
                      const void* beta, const float* g, void* o, int B, int H,
                      int K, int V, float scale, gdn_dtype act,
                      hipStream_t stream);

/*
 * gdn_prefill_gates - per-token gates of a prefill batch from raw inputs.
 * Source: pymllm `gdn_chunkwise` docs, `gdn_extend_chunkwise` parameters
 * (a, b, A_log, dt_bias), with the formulas of the regolith `gdn.metal`
 * header comment:
 *     g[t, h]    = -exp(A_log[h]) * softplus(a[t, h] + dt_bias[h])
 *     beta[t, h] = sigmoid(b[t, h])
 * a, b [T_tot, Hv] act; A_log, dt_bias [Hv] float32;
 * g, beta [T_tot, Hv] float32, written (g is the log-space gate).
 * Requirements: T_tot >= 0, Hv >= 1.
 */
int gdn_prefill_gates(const void* a, const void* b, const float* A_log,
                      const float* dt_bias, float* g, float* beta,
                      int64_t T_tot, int Hv, gdn_dtype act, hipStream_t stream);

/* gdn_chunk_prefill flag: L2-normalise q and k per token inside the kernel
 * (x / sqrt(sum x^2 + 1e-6)), as the pymllm page's q is "not pre-normalised"
 * and the regolith kernel normalises both. */
#define GDN_QK_L2NORM 1u

/* gdn_chunk_prefill flag: the state slots are read but never written, and
 * every y is still produced - a verify window of speculative decoding (the
 * regolith `gdn.metal` commit rule with nothing committed), run on the
 * chunked path. */
#define GDN_KEEP_STATE 2u

/*
 * gdn_chunk_prefill_workspace - bytes of device workspace gdn_chunk_prefill
 * needs for these sizes and activation dtype (0 for invalid arguments).  It
 * depends only on T_tot, N_s, Hv, chunk, act and (through the chunk of at
 * most 32 tokens that Dk > 128 runs) Dk; the other sizes are accepted for a
 * stable signature.
 */
size_t gdn_chunk_prefill_workspace(int64_t T_tot, int N_s, int Hk, int Hv,
                                   int Dk, int Dv, int chunk, gdn_dtype act);

/*
 * gdn_chunk_prefill - variable-length chunkwise (WY) prefill that advances a
 * pool of recurrent states in place.  Source: pymllm `gdn_chunkwise` docs,
 * module doc "Algorithm (per chunk of C tokens with initial state S_0)" steps
 * 1-3, and the `gdn_extend_chunkwise` parameter list.  Sequence s owns the
 * packed tokens cu_seqlens[s] .. cu_seqlens[s+1]-1 and the state slot
 * state_pool[cache_indices[s]]; for every value head hv (key head
 * hk = hv / (Hv/Hk)) the result equals running, token by token,
 *     k^ = k / sqrt(|k|^2 + 1e-6),  q^ = scale * q / sqrt(|q|^2 + 1e-6)
 *     (no normalisation without GDN_QK_L2NORM, q^ = scale * q)
 *     S <- exp(g) S;  d = beta (v - S k^);  S <- S + d k^T;  y = S q^
 * from the slot's current contents, then writing the final S back to the
 * slot.  The work is arranged in chunks of `chunk` tokens (the last one of a
 * sequence may be shorter); results depend on `chunk` only through rounding.
 *
 * q, k          [T_tot, Hk, Dk] act (raw; not normalised).
 * v             [T_tot, Hv, Dv] act.
 * g, beta       [T_tot, Hv] float32: log-space gate (<= 0 expected; the
 *               chunk form is exact for any g but may overflow for g > 0)
 *               and beta, e.g. from gdn_prefill_gates.
 * state_pool    [pool_size, Hv, Dv, Dk] float32, read and written in place.
 * cache_indices [N_s] int64, cu_seqlens [N_s + 1] int64: device arrays,
 *               not checked by this call.  Contract: cu_seqlens[0] == 0,
 *               non-decreasing, cu_seqlens[N_s] == T_tot; cache_indices
 *               distinct and in [0, pool_size).  Zero-length sequences leave
 *               their slot untouched; slots not named are never accessed.
 *               Entries outside the contract are skipped or clamped (no
 *               out-of-bounds access) but give unspecified results;
 *               gdn_validate_varlen checks the contract.
 * y             [T_tot, Hv, Dv] act, written.
 * chunk         8, 16, 32 or 64 tokens.     scale: <= 0 selects Dk^-1/2.
 * flags         0, or GDN_QK_L2NORM and/or GDN_KEEP_STATE (then state_pool is
 *               only read).
 * workspace     device memory of at least gdn_chunk_prefill_workspace()
 *               bytes, 16-byte aligned; its contents are scratch.
 * Requirements: Dk a multiple of 32 up to 256 (above 128 with bf16
 * activations only, and in chunks of at most 32 tokens whatever `chunk`
 * asks for: two 64-row operand tiles of that width do not fit in LDS); Dv a
 * multiple of 32,
 * <= 256; Hv % Hk == 0; q, k, v, state_pool 16-byte aligned; 64 tokens of q/k
 * (64 * Hk * Dk elements) and of v (64 * Hv * Dv) each under 1 GiB, else
 * GDN_ERR_UNSUPPORTED.  y, state_pool and the workspace overlap neither
 * each other nor any input (q, k, v, g, beta), else GDN_ERR_ALIAS.
 * N_s == 0 is a no-op.
 * On an in-kernel failure the referenced slots are unspecified (the update
 * is in place): callers that need to retry keep a copy of those slots.
 */
int gdn_chunk_prefill(const void* q, const void* k, const void* v,
                      const float* g, const float* beta, float* state_pool,
                      int64_t pool_size, const int64_t* cache_indices,
                      const int64_t* cu_seqlens, int N_s, int64_t T_tot,
                      int Hk, int Hv, int Dk, int Dv, int chunk, float scale,
                      unsigned flags, void* y, gdn_dtype act, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * gdn_chunk_prefill_raw_workspace - bytes of workspace gdn_chunk_prefill_raw
 * needs: gdn_chunk_prefill_workspace(), plus 8 bytes per (token, value head)
 * with fp32 activations (the gates' scratch).  0 for invalid arguments.
 */
size_t gdn_chunk_prefill_raw_workspace(int64_t T_tot, int N_s, int Hk, int Hv,
                                       int Dk, int Dv, int chunk, gdn_dtype act);

/*
 * gdn_chunk_prefill_raw - gdn_prefill_gates and gdn_chunk_prefill in one
 * call, from the raw gate inputs the pymllm `gdn_extend_chunkwise`
 * parameter list names (a, b, A_log, dt_bias; the formulas of
 * gdn_prefill_gates).  With bf16 activations the gates are formed inside the
 * prefill's WY pass, the one kernel that reads them, so no [T_tot, Hv] g
 * and beta pass through memory; with fp32 activations gdn_prefill_gates
 * writes them into the workspace's tail first.  Results equal those of the
 * two calls bit for bit.
 * a, b          [T_tot, Hv] act.   A_log, dt_bias [Hv] float32.
 * Every other argument as for gdn_chunk_prefill (flags GDN_QK_L2NORM and/or
 * GDN_KEEP_STATE); workspace: at least gdn_chunk_prefill_raw_workspace()
 * bytes, 16-byte aligned, scratch.  a, b, A_log and dt_bias must not overlap
 * y, the pool or the workspace (GDN_ERR_ALIAS); otherwise the errors of
 * gdn_chunk_prefill.
 */
int gdn_chunk_prefill_raw(const void* q, const void* k, const void* v,
                          const void* a, const void* b, const float* A_log,
                          const float* dt_bias, float* state_pool,
                          int64_t pool_size, const int64_t* cache_indices,
                          const int64_t* cu_seqlens, int N_s, int64_t T_tot,
                          int Hk, int Hv, int Dk, int Dv, int chunk, float scale,
                          unsigned flags, void* y, gdn_dtype act, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * gdn_chunk_prefill_gated - gdn_chunk_prefill followed by the layer's gated
 * RMS norm of every output row (gdn_gated_rmsnorm below): y receives
 *     o_j / sqrt(mean_j(o_j^2) + eps) * gamma[j] * sigmoid(z_j)
 * per (token, value head), o being what gdn_chunk_prefill writes.  Source:
 * regolith `gdn.metal` output block, fused into the recurrence's output as
 * that kernel does.  With bf16 activations and Dv == 128 the norm runs inside
 * the chunk loop's store of y (o is not written to memory); otherwise the
 * norm kernel runs afterwards on y in place (o rounded to act first).
 * z [T_tot, Hv, Dv] act; gamma [Dv] float32; eps >= 0.  Requirements: those
 * of gdn_chunk_prefill, Dv in {32, 64, 128, 256}, z and gamma 16-byte
 * aligned, z overlapping none of y, state_pool and the workspace.
 */
int gdn_chunk_prefill_gated(const void* q, const void* k, const void* v,
                            const float* g, const float* beta,
                            float* state_pool, int64_t pool_size,
                            const int64_t* cache_indices,
                            const int64_t* cu_seqlens, int N_s, int64_t T_tot,
                            int Hk, int Hv, int Dk, int Dv, int chunk,
                            float scale, unsigned flags, const void* z,
                            const float* gamma, float eps, void* y,
                            gdn_dtype act, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * gdn_validate_varlen - debug/test helper: copies cu_seqlens and
 * cache_indices to the host (synchronising `stream`) and checks the
 * gdn_chunk_prefill contract above.  GDN_OK, or GDN_ERR_SHAPE if violated.
 */
int gdn_validate_varlen(const int64_t* cu_seqlens,
                        const int64_t* cache_indices, int N_s, int64_t T_tot,
                        int64_t pool_size, hipStream_t stream);

/*
 * gdn_conv_silu - the layer prologue: 4-tap causal convolution + SiLU of the
 * q, k and v channels of every token, with a rolling history per state slot.
 * Source: regolith `gdn.metal`, header comment and the conv/SiLU block of its
 * kernel (4 taps, history [channels][3] oldest first).  Per token the
 * C = 2*Hk*Dk + Hv*Dv input channels are [q heads | k heads | v heads].
 * For sequence s (packed tokens cu_seqlens[s] .. cu_seqlens[s+1]-1, slot
 * cache_indices[s]) and channel c, with inputs before the sequence's first
 * token read from the slot's history (conv_state[slot][c][0] the oldest):
 *     pre = x[t-3] w[c][0] + x[t-2] w[c][1] + x[t-1] w[c][2] + x[t] w[c][3]
 *     out[t][c] = pre / (1 + exp(-pre))
 * and afterwards the slot's history holds the newest three of (history,
 * the sequence's inputs).  A decode step is one token per sequence
 * (cu_seqlens = 0, 1, ..., B).
 *
 * qkv           [T_tot, C] act, read.
 * conv_w        [C, 4] float32 (tap 3 weighs the current token).
 * conv_state    [pool_size, C, 3] float32, read and written in place; only
 *               the slots of non-empty sequences are accessed.
 * cache_indices, cu_seqlens: as for gdn_chunk_prefill (device arrays, same
 *               contract, not checked here).
 * q, k          [T_tot, Hk, Dk] act, written (channels 0 .. 2*Hk*Dk-1).
 * v             [T_tot, Hv, Dv] act, written.
 * Requirements: Dk and Dv multiples of 8; qkv, conv_w, conv_state, q, k, v
 * 16-byte aligned; no two of qkv, conv_state, q, k, v overlap.  Two kernels
 * are enqueued (outputs, then the history update of the longer sequences).
 */
int gdn_conv_silu(const void* qkv, const float* conv_w, float* conv_state,
                  int64_t pool_size, const int64_t* cache_indices,
                  const int64_t* cu_seqlens, int N_s, int64_t T_tot, int Hk,
                  int Hv, int Dk, int Dv, void* q, void* k, void* v,
                  gdn_dtype act, hipStream_t stream);

/*
 * gdn_gated_rmsnorm - the layer epilogue: per (token, value head), over its
 * Dv outputs o_j,
 *     y_j = o_j / sqrt(mean_j(o_j^2) + eps) * gamma[j] * sigmoid(z_j)
 * Source: regolith `gdn.metal`, header comment and the kernel's output block
 * (gamma indexed by the column only, shared by every head).
 * o, z, y       [T_tot, Hv, Dv] act; y may equal o (in place), nothing else
 *               may overlap.   gamma: [Dv] float32.   eps >= 0.
 * Requirements: Dv in {32, 64, 128, 256}; o, z, gamma, y 16-byte aligned.
 */
int gdn_gated_rmsnorm(const void* o, const void* z, const float* gamma,
                      float eps, void* y, int64_t T_tot, int Hv, int Dv,
                      gdn_dtype act, hipStream_t stream);

/*
 * gdn_chunk_prefill_fixed_workspace - bytes of device workspace
 * gdn_chunk_prefill_fixed needs (0 for invalid arguments): that of
 * gdn_chunk_prefill for B sequences of T tokens, plus the index arrays.
 */
size_t gdn_chunk_prefill_fixed_workspace(int B, int64_t T, int Hk, int Hv,
                                         int Dk, int Dv, int chunk,
                                         gdn_dtype act);

/*
 * gdn_chunk_prefill_fixed - gdn_chunk_prefill over a fixed-length batch in
 * the metaltile layouts (metaltile-std `gated_delta.rs`, "Layouts" of
 * `mt_gated_delta_chunk`): B sequences of T tokens each, the state one slice
 * per (b, hv) updated in place.  The same computation as gdn_chunk_prefill
 * with cu_seqlens = {0, T, 2T, ..., BT} and cache_indices = {0, ..., B-1}.
 *
 * q, k          [B, T, Hk, Dk] act.     v, y [B, T, Hv, Dv] act (y written).
 * g, beta       [B, T, Hv] float32.
 * state         [B, Hv, Dv, Dk] float32 (the gdn_decode_step layout), read
 *               and written in place (only read with GDN_KEEP_STATE).
 * chunk, scale, flags: as for gdn_chunk_prefill.
 * workspace     device memory of at least gdn_chunk_prefill_fixed_workspace()
 *               bytes, 16-byte aligned; its contents are scratch (the call
 *               writes the index arrays into its end: with bf16 activations
 *               the first kernel does, which also finds each chunk's
 *               sequence by division; with fp32 ones a small kernel first).
 * Requirements: those of gdn_chunk_prefill.  B == 0 or T == 0 is a no-op.
 * When T fits one chunk (after the Dk > 128 cap) the call knows every
 * sequence is a single chunk and runs a chunk loop without next-chunk
 * prefetch (same results, bit for bit; faster for decode windows).
 */
int gdn_chunk_prefill_fixed(const void* q, const void* k, const void* v,
                            const float* g, const float* beta, float* state,
                            int B, int64_t T, int Hk, int Hv, int Dk, int Dv,
                            int chunk, float scale, unsigned flags, void* y,
                            gdn_dtype act, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * comba_chunk_prefill_workspace - bytes of device workspace
 * comba_chunk_prefill needs (0 for invalid arguments or act != GDN_BF16).
 * Depends only on T_tot, N_s, H, chunk and (K > 128 runs chunks of at most
 * 32 tokens) K.
 */
size_t comba_chunk_prefill_workspace(int64_t T_tot, int N_s, int H, int K,
                                     int V, int chunk, gdn_dtype act);

/*
 * comba_chunk_prefill - the Comba forward over a variable-length batch,
 * chunkwise (WY), advancing a pool of [K, V] states in place.  Source: KBench
 * `comba_decode_step` spec, spec_md (the step, and the forward task as that
 * step run over every token) and contract_md (argument order and dtypes).
 * Sequence s owns the packed tokens cu_seqlens[s] .. cu_seqlens[s+1]-1 and
 * the slot state_pool[cache_indices[s]]; for every head the result equals
 * running comba_decode_step token by token from the slot's contents:
 *     S <- exp(g) S;  u = beta (v - S^T p);  S <- S + k u^T;  o = S^T (scale q)
 * and writing the final S back.  In chunk form the WY factor is
 * (I + A)^-1 with A_ij = beta_i exp(G_i - G_j) (p_i . k_j), j < i, G the
 * in-chunk cumulative log-gate.  Results depend on `chunk` only through
 * rounding.  Keys are used as given (no normalisation).
 *
 * q, k, p       [T_tot, H, K] bf16.   v, o [T_tot, H, V] bf16 (o written).
 * beta          [T_tot, H] bf16.      g [T_tot, H] float32 (log-decay, <= 0
 *               expected; the chunk form may overflow for g > 0).
 * state_pool    [pool_size, H, K, V] float32 (value index contiguous, the
 *               comba_decode_step layout), read and written in place.
 * cache_indices [N_s] int64, cu_seqlens [N_s + 1] int64: device arrays with
 *               the contract of gdn_chunk_prefill (gdn_validate_varlen
 *               checks it); zero-length sequences leave their slot untouched.
 * chunk         8, 16, 32 or 64 tokens.   scale: <= 0 selects K^-1/2.
 * workspace     device memory of at least comba_chunk_prefill_workspace()
 *               bytes, 16-byte aligned; its contents are scratch.
 * Requirements: act == GDN_BF16 (else GDN_ERR_UNSUPPORTED); K a multiple of
 * 32 up to 256 (above 128 in chunks of at most 32 tokens); V a multiple of 32,
 * <= 256; q, k, p, v, state_pool 16-byte aligned;
 * 64 tokens of q (64 * H * K elements) and of v each under 1 GiB.
 * o, state_pool and the workspace overlap neither each other nor any input
 * (q, k, p, v, beta, g), else GDN_ERR_ALIAS.
 * N_s == 0 is a no-op.  On an in-kernel failure the referenced slots are
 * unspecified (the update is in place).
 */
int comba_chunk_prefill(const void* q, const void* k, const void* v,
                        const void* p, const void* beta, const float* g,
                        float* state_pool, int64_t pool_size,
                        const int64_t* cache_indices, const int64_t* cu_seqlens,
                        int N_s, int64_t T_tot, int H, int K, int V, int chunk,
                        float scale, void* o, gdn_dtype act, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * gdn_conv_decode_workspace - bytes of device workspace gdn_conv_decode_step
 * needs: B * (2*Hk*Dk + Hv*Dv + 2*Hv) floats (the convolved, normalised
 * q, k, v and the gates of the token, fp32); 0 for invalid sizes.
 */
size_t gdn_conv_decode_workspace(int B, int Hk, int Hv, int Dk, int Dv);

/*
 * gdn_conv_decode_step - one decode token of the layer front: the 4-tap
 * causal conv + SiLU of the token's q, k and v channels with the history
 * updated in place (gdn_conv_silu), the L2 norm of q and k with the query
 * scale and the gates from raw a, b (gdn_prefill_gates), then the gated
 * delta-rule step (gdn_decode_step).  Two kernels: a prologue writes the
 * token's convolved, normalised q, k, v and its gates to the workspace in
 * fp32 (never rounded to the activation dtype), the decode kernel reads them.
 * Source: regolith `gdn.metal`, header comment and the conv/SiLU block of
 * its kernel (conv, SiLU, norms and gates ahead of the recurrence);
 * metaltile-std `gated_delta.rs`, "Recurrence per step".  For sequence b:
 *     x'_c = SiLU(h[c][0] w[c][0] + h[c][1] w[c][1] + h[c][2] w[c][2] + x_c w[c][3])
 *            over the C = 2*Hk*Dk + Hv*Dv channels [q heads | k heads | v heads],
 *            after which conv_state[b][c] = (h[c][1], h[c][2], x_c)
 *     k^ = k' / sqrt(|k'|^2 + 1e-6),  q^ = scale q' / sqrt(|q'|^2 + 1e-6)
 *            (with GDN_QK_L2NORM; without it k^ = k', q^ = scale q')
 *     g = -exp(A_log[hv]) softplus(a + dt_bias[hv]),  beta = sigmoid(b)
 *     then for every value head hv (key head hv / (Hv/Hk)) the decode step
 *     on state slice (b, hv) with (q^, k^, v', g, beta), y its readout.
 *
 * state_in, state_out  [B, Hv, Dv, Dk] float32; state_out may equal state_in.
 * qkv          [B, C] act, this token's raw channels (before the conv).
 * conv_w       [C, 4] float32 (tap 3 weighs the current token).
 * conv_state   [B, C, 3] float32, the history (oldest first), read and
 *              updated in place.
 * a, b         [B, Hv] act (raw gate inputs).   A_log, dt_bias [Hv] float32.
 * y            [B, Hv, Dv] act, written.
 * scale        query scale; <= 0 selects Dk^-1/2.  flags: 0 or GDN_QK_L2NORM.
 * workspace    device memory of at least gdn_conv_decode_workspace() bytes,
 *              16-byte aligned; scratch.  Two kernels run on `stream`.
 * Requirements: those of gdn_decode_step (Dk a multiple of 32 up to 256, Dv a
 * multiple of 32 up to 256, Hv % Hk == 0); state_in, state_out, conv_w and
 * the workspace 16-byte aligned, conv_state 4-byte aligned; y, state_out,
 * conv_state and the workspace overlap no input and each other
 * (GDN_ERR_ALIAS).  B == 0 is a no-op.
 */
int gdn_conv_decode_step(const float* state_in, float* state_out,
                         const void* qkv, const float* conv_w,
                         float* conv_state, const void* a, const void* b,
                         const float* A_log, const float* dt_bias, void* y,
                         int B, int Hk, int Hv, int Dk, int Dv, float scale,
                         unsigned flags, gdn_dtype act, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * gdn_conv_prefill_workspace - bytes of device workspace gdn_conv_prefill
 * needs (bf16 activations): gdn_chunk_prefill_workspace() plus the convolved
 * q, k [T_tot, Hk, Dk] and v [T_tot, Hv, Dv] in bf16, each rounded up to 256
 * bytes, plus 256 bytes.  0 for invalid arguments.
 */
size_t gdn_conv_prefill_workspace(int64_t T_tot, int N_s, int Hk, int Hv,
                                  int Dk, int Dv, int chunk);

/*
 * gdn_conv_prefill - the layer's prefill from its raw channels: the conv
 * prologue of gdn_conv_silu, the gates of gdn_prefill_gates, the recurrence
 * of gdn_chunk_prefill and, when z is given, the gated norm of
 * gdn_chunk_prefill_gated, in one call.  Source: regolith `gdn.metal`,
 * header comment (conv, SiLU, norms and gates ahead of the recurrence, the
 * gated norm after it) and the pymllm `gdn_extend_chunkwise` parameter list
 * (raw gates, varlen batch, state pool).  The conv runs inside the prefill's
 * WY pass, one chunk of one key head per wave (its q and k heads and the v
 * heads of its group); the convolved q, k, v are written once, to the
 * workspace, for the chunk loop.  Every result equals the separate calls
 * (gdn_conv_silu, then gdn_chunk_prefill_raw, or gdn_chunk_prefill_gated
 * with the gates of gdn_prefill_gates) bit for bit.
 * qkv          [T_tot, C] bf16, C = 2*Hk*Dk + Hv*Dv channels per token laid
 *              out as [q heads | k heads | v heads], read.
 * conv_w       [C, 4] float32 (tap 3 weighs the current token), read.
 * conv_state   [pool_size, C, 3] float32, the history (oldest first) per
 *              state slot: read, then updated in place to the newest three of
 *              (history, the sequence's inputs); left as it is with
 *              GDN_KEEP_STATE.  Only the slots of non-empty sequences are
 *              accessed.
 * a, b         [T_tot, Hv] bf16.   A_log, dt_bias [Hv] float32.
 * z, gamma     NULL: y is the recurrence's output.  Else z [T_tot, Hv, Dv]
 *              bf16 and gamma [Dv] float32, eps >= 0, Dv in {32, 64, 128,
 *              256}: y is the gated norm of it.
 * Every other argument as for gdn_chunk_prefill (flags GDN_QK_L2NORM and/or
 * GDN_KEEP_STATE, which then also keeps conv_state); act must be GDN_BF16
 * (GDN_ERR_UNSUPPORTED otherwise).  workspace: at least
 * gdn_conv_prefill_workspace() bytes, 16-byte aligned, scratch.
 * Requirements: those of gdn_chunk_prefill; qkv, conv_w, conv_state, z and
 * gamma 16-byte aligned (GDN_ERR_ALIGN); conv_state overlapping none of y,
 * state_pool and the workspace, and no input (qkv, conv_w, z, a, b, A_log,
 * dt_bias) overlapping an output (GDN_ERR_ALIAS).  N_s == 0 is a no-op.
 * On an in-kernel failure the referenced state slots and histories are
 * unspecified (both are updated in place).
 */
int gdn_conv_prefill(const void* qkv, const float* conv_w, float* conv_state,
                     const void* a, const void* b, const float* A_log,
                     const float* dt_bias, float* state_pool, int64_t pool_size,
                     const int64_t* cache_indices, const int64_t* cu_seqlens,
                     int N_s, int64_t T_tot, int Hk, int Hv, int Dk, int Dv,
                     int chunk, float scale, unsigned flags, const void* z,
                     const float* gamma, float eps, void* y, gdn_dtype act,
                     void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * gdn_chunk_prefill_noalloc - gdn_chunk_prefill without a caller workspace,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * workspace lives in a static 128 MiB device array of the library (one per
 * GPU, held until the process ends); the call allocates nothing and calls
 * no allocating routine.  Arguments, results and requirements: those of
 * gdn_chunk_prefill, minus workspace and workspace_bytes.
 * Limit: gdn_chunk_prefill_workspace() for these sizes must be at most
 * 134,217,728 bytes (e.g. about 8,000 tokens at 48 value heads, chunk 64,
 * bf16), else GDN_ERR_WORKSPACE and nothing is launched.
 * Every call on one GPU uses that GPU's one array: calls that can overlap in
 * time on the same GPU (different streams, or host threads without ordering)
 * race and give unspecified results; calls ordered on one stream are safe.
 * The first call on each device looks the array's address up (no device
 * memory is touched); GDN_ERR_DEVICE if that fails.
 */
int gdn_chunk_prefill_noalloc(const void* q, const void* k, const void* v,
                              const float* g, const float* beta,
                              float* state_pool, int64_t pool_size,
                              const int64_t* cache_indices,
                              const int64_t* cu_seqlens, int N_s,
                              int64_t T_tot, int Hk, int Hv, int Dk, int Dv,
                              int chunk, float scale, unsigned flags, void* y,
                              gdn_dtype act, hipStream_t stream);

/*
 * gdn_stream_copy - measurement helper: copies `bytes` bytes from src to dst
 * with one 16-byte non-temporal load and one 16-byte non-temporal store per
 * thread, the access pattern of the decode step's state stream.  Source:
 * KBench `comba_decode_step` page, perf_md (a bandwidth-bound step is
 * compared with a large stream copy measured on the same machine).  Its rate over
 * 2 * bytes is the measured ceiling the streaming kernels are compared with.
 * src, dst: device memory, 16-byte aligned, not overlapping (GDN_ERR_ALIAS).
 * bytes: a multiple of 16 (else GDN_ERR_SHAPE); 0 is a no-op; at most
 * 2^31 - 1 workgroups of 2 KiB (GDN_ERR_UNSUPPORTED beyond).
 */
int gdn_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

/* Human-readable name of a gdn_status value (static string, never NULL). */
const char* gdn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
