/*
 * libraceattn — RACE Attention (soft-LSH sketch attention) on AMD MI355X (gfx950).
 *
 * The operation (arXiv 2510.04008, "RACE Attention: A Strictly Linear-Time
 * Attention for Long-Sequence Training", as summarised on gist.science and
 * fugumt.com):
 *   - the similarity of a query and a key is a sharpened angular kernel of
 *     their normalised dot product (Japanese gist.science page, section 2.1;
 *     Italian page, Sommario tecnico section 2, Concetti Chiave 1);
 *   - queries and keys are unit-normalised and projected on L tables of P
 *     random hyperplanes, softened with tanh and assigned to the R = 2^P
 *     hypercube corners by a softmax with temperature beta (Italian page,
 *     section 2, Concetti Chiave 2; Korean page, 기술 요약 section 2;
 *     Japanese page, section 2.2);
 *   - keys accumulate per-bucket mass and value sums; each query reads its
 *     own soft buckets and the output is the normalised weighted average over
 *     the tables (Italian page, section 2, Algoritmo; Japanese page,
 *     section 2.1);
 *   - the causal variant restricts the sums to keys at or before the query
 *     through prefix sums (Japanese page, section 2.2);
 *   - the layer is trained end to end, so the library also returns the
 *     gradients with respect to Q, K and V (Japanese page, section 2.2;
 *     fugumt.com abstract: forward-backward pass).
 *
 * Per query i and table l (a = soft assignment, c_r = corner signs):
 *   a_l(x) = softmax_r( beta * <c_r, tanh(W_l x / |x|)> )
 *   O_i    = sum_l sum_r a_l(q_i)[r] S_l[r]  /  sum_l sum_r a_l(q_i)[r] z_l[r]
 *   S_l[r] = sum_{j in scope(i)} a_l(k_j)[r] v_j,   z_l[r] = sum_{j in scope(i)} a_l(k_j)[r]
 * scope(i) = all keys (non-causal) or keys j <= i (causal).
 * Corner r has sign +1 on plane p when bit p of r is set. Hard-hash id of a
 * table = sum_p [h_p > 0] 2^p.
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers unless stated otherwise; the caller
 *     owns all memory; the library allocates nothing. Its only mutable
 *     global state is the calling thread's profiling hook
 *     (race_attn_profile_events, thread-local) and, for
 *     race_attn_fwd_noalloc, its fixed per-GPU scratch array and the cached
 *     device address of it; every other entry point is thread-safe
 *     (concurrent calls on different streams with different buffers are
 *     independent).
 *   - Q, K, V, O, dO, dQ, dK, dV: [B, H, N, d] contiguous row-major, element
 *     type `dtype`. W: [L, P, d] contiguous, element type `dtype`, shared by
 *     queries, keys, batches and heads, or [H, L, P, d] (one set per head)
 *     when RACE_W_PER_HEAD is or'ed into `dtype`; it is a fixed random
 *     projection and receives no gradient.
 *   - Every tensor pointer (and ws, saved) must be 16-byte aligned, else
 *     RACE_ERR_INVALID_ARG.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream). Argument errors are reported synchronously, before any
 *     device work is enqueued. Device faults surface at the caller's next
 *     synchronisation.
 *   - Supported: d = 32, 64 or 128; 1 <= P <= 6; L >= 1
 *     with L * 2^P <= 65536; N >= 1; B, H >= 1 with B * H <= 65535;
 *     1 <= chunk <= 2^20; dtype RACE_F32 or RACE_BF16. Other shapes return
 *     RACE_ERR_UNSUPPORTED. Many tables run as consecutive groups of at most
 *     256 features (P = 4, causal: 16 tables; P = 5: 8; P = 6: 4; otherwise
 *     128 projection rows), one launch per group and pass, whose partial
 *     outputs add up in float32 before the last group finishes them. At
 *     d = 128 the plane values come from the whole rows and every sketch pass
 *     runs once per half of 64 value columns.
 *   - Numerics: bf16 inputs are multiplied on bf16 matrix cores with float32
 *     accumulation; float32 inputs use float32 matrix cores throughout.
 *     Running sums and all reductions are float32. Between passes the chunk
 *     sketch states are float32 for RACE_F32 inputs; for RACE_BF16 inputs
 *     their value sums are stored in bf16 (the precision of the matrix-core
 *     operands they feed), their masses and the empty subset's value sums in
 *     float32. No atomics are used on the attention path, so results are
 *     bitwise reproducible run to run. The read-out sums monomial terms that
 *     cancel for a query whose soft collisions with the keys are nearly
 *     zero (sharp temperatures with few tables); such rows lose accuracy in
 *     proportion to the operand precision over their denominator, most with
 *     RACE_BF16 inputs, where RACE_F32 keeps it.
 *   - `chunk` is the number of tokens a workgroup owns; per-chunk sketch
 *     states are published and prefix-scanned at that granularity. Results do
 *     not depend on it beyond float32 rounding.
 *   - No C++ exception crosses this interface.
 */
#ifndef RACE_ATTN_H
#define RACE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RACE_OK = 0,
    RACE_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, bad dtype, overflow */
    RACE_ERR_UNSUPPORTED = 2,   /* valid but outside the supported shape set */
    RACE_ERR_WORKSPACE = 3,     /* ws_bytes smaller than required */
    RACE_ERR_HIP = 4            /* a HIP launch or query failed */
} race_status_t;

typedef enum { RACE_F32 = 0, RACE_BF16 = 1 } race_dtype_t;

/* Or'ed into the dtype argument of any entry point (and into for_backward of
 * race_attn_workspace_bytes): W is [H, L, P, d], one set of hyperplanes per
 * head (head h of every batch uses W[h]), instead of one [L, P, d] for all
 * heads. */
#define RACE_W_PER_HEAD 0x100

/* Bytes of device workspace `ws` for this shape. Writes *bytes.
 *   for_backward = 0: race_attn_fwd with saved = NULL;
 *   for_backward = 3: race_attn_fwd with a `saved` buffer;
 *   for_backward = 1: race_attn_bwd given O and `saved` from the forward;
 *   for_backward = 2: race_attn_bwd with O = saved = NULL (it then recomputes
 *                     the forward into this workspace);
 * any other value gives RACE_ERR_INVALID_ARG; or'ed with RACE_W_PER_HEAD, the
 * size for per-head hyperplanes. The size depends on dtype only
 * through element sizes, so it is computed for RACE_F32, an upper bound for
 * both dtypes. */
race_status_t race_attn_workspace_bytes(int64_t B, int64_t H, int64_t N, int d, int P, int L,
                                        int causal, int chunk, int for_backward, size_t *bytes);

/* Bytes of the optional `saved` buffer a forward call fills for the backward,
 * per (batch, head): the sketch state at the start of every chunk (causal)
 * or the whole-sequence sketch (non-causal), sized as float32 (bf16 value
 * sums for RACE_BF16, see Numerics above); the float32 per-token
 * softmax denominators D_i = sum_l sum_r a_l(q_i)[r] z_l[r] (the quantity
 * the output divides by); and, for queries and for keys, each token's
 * per-plane u = tanh of the normalised projection (float16 for RACE_BF16,
 * float32 for RACE_F32) with 1 / max(|x|, 1e-12) in float32, so that the
 * backward rebuilds the soft assignments without projecting again.
 * Layout is private to the library. */
race_status_t race_attn_saved_bytes(int64_t B, int64_t H, int64_t N, int d, int P, int L,
                                    int causal, int chunk, size_t *bytes);

/* Forward: O = RACE-Attention(Q, K, V; W, P, L, temperature, causal).
 * `temperature` is the pages' beta: it multiplies the corner logits, so a
 * larger value gives harder bucket assignments. +INFINITY selects the hard
 * buckets (one-hot of the sign pattern of the projections; the discrete hash
 * the temperature softens: Japanese gist.science page, section 2.2); a
 * query that shares no bucket with any key it attends to then gets O = 0.
 * The denominators are exact collision counts (bf16 inputs feed the masses
 * to the matrix cores in three bf16 parts) while F * N < 2^24, F = the
 * number of features over all table groups (2^P * L rounded up to whole
 * projection tiles); beyond that +INFINITY gives RACE_ERR_UNSUPPORTED. The
 * backward takes finite temperatures only. NaN and -INFINITY give
 * RACE_ERR_INVALID_ARG. `saved` may be NULL; if not
 * NULL it receives the sketch states, denominators and plane values
 * (race_attn_saved_bytes). `ws` must hold race_attn_workspace_bytes(...,
 * for_backward = 0), or (..., for_backward = 3) when `saved` is given. */
race_status_t race_attn_fwd(const void *Q, const void *K, const void *V, const void *W,
                            int64_t B, int64_t H, int64_t N, int d, int P, int L,
                            float temperature, int causal, int chunk, race_dtype_t dtype,
                            void *O, void *saved, void *ws, size_t ws_bytes, void *stream);

/* Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): race_attn_fwd with the same arguments minus `ws`; its workspace
 * is a fixed device array inside the library, RACE_NOALLOC_SCRATCH_BYTES
 * (64 MiB) on each GPU it runs on, held until the process ends. A shape whose
 * workspace (race_attn_workspace_bytes, for_backward = 0, or 3 when `saved` is
 * given) exceeds it returns RACE_ERR_WORKSPACE before any device work. The
 * call allocates nothing (no hipMalloc, no allocating library routine). Every
 * call on one GPU uses that GPU's one array and leaves its last contents
 * there (the forward writes every workspace byte it reads, so no clearing is
 * needed): calls that overlap on one GPU (other streams, other host threads)
 * race and must be serialised by the caller. */
#define RACE_NOALLOC_SCRATCH_BYTES (64u << 20)
race_status_t race_attn_fwd_noalloc(const void *Q, const void *K, const void *V, const void *W,
                                    int64_t B, int64_t H, int64_t N, int d, int P, int L,
                                    float temperature, int causal, int chunk, race_dtype_t dtype,
                                    void *O, void *saved, void *stream);

/* Backward: given dO = dLoss/dO, writes dQ, dK, dV (the exact gradients of
 * the forward above; the pages train the layer end to end, Japanese
 * gist.science page, section 2.2). With g_i = dO_i / D_i and
 * e_i = -<dO_i, O_i> / D_i, the query side reads the key sketch with [g | e]
 * and the key side reads the reverse sketch sum_i a(q_i)^T [g_i | e_i].
 * O (the forward's output) and `saved` (the buffer that forward call filled,
 * with identical arguments) are given together, or both NULL: then the
 * forward is recomputed inside the call. Exactly one of them NULL gives
 * RACE_ERR_INVALID_ARG. `ws` must hold race_attn_workspace_bytes(...,
 * for_backward = 1) when they are given, (..., for_backward = 2) when not. */
race_status_t race_attn_bwd(const void *Q, const void *K, const void *V, const void *W,
                            const void *O, const void *dO, const void *saved, int64_t B,
                            int64_t H, int64_t N, int d, int P, int L, float temperature,
                            int causal, int chunk, race_dtype_t dtype, void *dQ, void *dK,
                            void *dV, void *ws, size_t ws_bytes, void *stream);

/* Hard-hash diagnostic (the beta -> infinity limit of the soft assignment):
 * bucket_ids[row, l] = sum_p [<W_lp, x_row / |x_row|> > 0] 2^p for the
 * rows of X ([B, H, N, d], dtype), written as int32 [B, H, N, L].
 * *near_zero (a device counter, added to, not reset) receives the number of
 * projections with |<W_lp, x/|x|>| < 1e-5, whose sign is not reliable. */
race_status_t race_attn_hash(const void *X, const void *W, int64_t B, int64_t H, int64_t N,
                             int d, int P, int L, race_dtype_t dtype, int32_t *bucket_ids,
                             unsigned long long *near_zero, void *stream);

/* ---- Decoding: the sketch as a constant-size key-value cache --------------
 * Efficient key-value caching at inference is the pages' named next use of
 * the sketch (Japanese gist.science page, section 6; Korean page, section 5).
 * The running state of one (batch, head) is the key sketch of every token so
 * far: per feature, the sum of the keys' feature value times v (float32) and
 * the sum of the feature values, the mass (float64, so that counts of more
 * than 2^24 keys stay exact): L * 2^P * (64 * 4 + 8) bytes (d = 32 or 64;
 * d = 128: L * 2^P * (128 * 4 + 8); padded to whole projection tiles)
 * whatever the length. Its layout is private to the
 * library; all-zero bytes are the state of an empty sequence. `temperature` = +INFINITY selects the hard
 * buckets (the discrete hash that the temperature softens: Japanese
 * gist.science page, section 2.2): each table then adds [v | 1] to exactly
 * one bucket, and a query that shares no bucket with any key outputs zeros.
 * Finite temperatures give the soft assignment of race_attn_fwd. NaN and
 * -INFINITY give RACE_ERR_INVALID_ARG. */

/* Bytes of a running state for B * H heads, [B * H][state bytes], 16-byte
 * aligned per head. Same shape checks as race_attn_fwd. */
race_status_t race_attn_state_bytes(int64_t B, int64_t H, int d, int P, int L, size_t *bytes);

/* Prefill: state = the key sketch of the N tokens of K, V ([B, H, N, d],
 * dtype) with hyperplanes W ([L, P, d]); overwrites `state` (device float32,
 * race_attn_state_bytes, 16-byte aligned). `chunk` only tiles the work (any
 * value in 1..2^20; 1024 is a good choice); the result does not depend on it
 * beyond float32 rounding order. `ws` must hold race_attn_workspace_bytes(B,
 * H, N, d, P, L, causal = 0, chunk, for_backward = 0, ...). The outputs of the
 * prompt itself come from race_attn_fwd with causal = 1. */
race_status_t race_attn_prefill(const void *K, const void *V, const void *W, int64_t B, int64_t H,
                                int64_t N, int d, int P, int L, float temperature, int chunk,
                                race_dtype_t dtype, float *state, void *ws, size_t ws_bytes,
                                void *stream);

/* Causal decode of T new tokens for every (batch, head): q, k, v are their
 * rows ([B, H, T, d], dtype). In token order, each token's k and v join
 * `state` (in and out), then its q reads it, so o ([B, H, T, d], dtype) holds
 * the causal output of each token, diagonal included (Japanese gist.science
 * page, section 2.2, causal prefix sums): T = 1 is one generation step, T > 1
 * extends the sequence by several tokens (a draft to verify, a prompt piece)
 * while reading and writing the state once. T >= 1. W and `state` must be
 * 16-byte aligned (RACE_ERR_INVALID_ARG otherwise). One workgroup per head;
 * no workspace. Calls on one stream run in order; two calls that update the
 * same state concurrently race. */
race_status_t race_attn_decode(const void *q, const void *k, const void *v, const void *W, int64_t B,
                               int64_t H, int64_t T, int d, int P, int L, float temperature,
                               race_dtype_t dtype, float *state, void *o, void *stream);

/* Profiling aid (not needed for computation). For the CALLING THREAD only:
 * `events` is an array of `capacity` (>= 2) caller-created hipEvent_t handles.
 * Each subsequent race_attn_fwd / _bwd / _hash / _prefill / _decode call on this
 * thread records events[i] on its stream just before its i-th kernel launch and one more
 * event after the last launch, so stage i took elapsed(events[i], events[i+1]).
 * Pass events = NULL to stop. race_attn_profile_count() gives the number of
 * events the last call recorded; race_attn_profile_stage(i) the name of the
 * kernel launched after event i ("end" for the last). Calls on other threads
 * are unaffected. */
race_status_t race_attn_profile_events(void **events, int capacity);
int race_attn_profile_count(void);
const char *race_attn_profile_stage(int i);

/* Static, human-readable name of a status code. */
const char *race_attn_status_string(race_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* RACE_ATTN_H */
