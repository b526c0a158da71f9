/*
 * gdr.h -- C ABI of libgdr.so: the gated-delta-rule state recurrence on MI355X (gfx950).
 *
 * The recurrence (FlashQLA PR #1 "Fused recurrent GDN decode + SGLang DFlash verify
 * kernel (TileLang, SM90)", core decode-kernel commit): per value head h the state
 * S[V][K] (fp32, row v over key channels c) takes, for every token t,
 *
 *     decay    S[v][c] *= exp(g[t,h])          scalar gate (GDN), or
 *              S[v][c] *= exp(gk[t,h,c])       per-key-channel gate (KDA)
 *     read     kS[v]    = sum_c S[v][c] * k[t,hk,c]
 *     delta    nu[v]    = beta[t,h] * (v[t,h,v] - kS[v])
 *     write    S[v][c] += nu[v] * k[t,hk,c]
 *     output   o[t,h,v] = scale * sum_c S[v][c] * q[t,hk,c]    (post-update state)
 *
 * with key/query head hk = h / (HV / HK) (grouped-query mapping, same page, review
 * commit).  For gdr_recurrent_fwd, gdr_chunk_fwd and gdr_decode_paged, q and k arrive
 * l2-normalised per (token, head) and g, beta arrive already activated (same page,
 * verify-kernel commit); those entry points never re-normalise.  g is the natural-log
 * decay and must be finite and <= 0.  The gated entry points (gdr_gating_prepass,
 * gdr_decode_paged_gated) take the raw inputs instead; see gdr_gating below.
 *
 * Layouts (all tensors contiguous, row-major, packed variable-length batch):
 *   q, k           [T, HK, K]          io_dtype
 *   v, o           [T, HV, V]          io_dtype
 *   beta           [T, HV]             io_dtype
 *   g              [T, HV]             fp32 (GDR_GATE_SCALAR)
 *   gk             [T, HV, K]          fp32 (GDR_GATE_PER_K)
 *   cu_seqlens     [N + 1]             int32, cu_seqlens[0] = 0, non-decreasing,
 *                                      cu_seqlens[N] = T; sequence n owns tokens
 *                                      cu_seqlens[n] .. cu_seqlens[n+1]-1
 *   states         [.., HV, V, K]      V-major ("state_v_first"): row v contiguous over K
 * Supported: K, V in {64, 128}; HV % HK == 0; io_dtype fp32 or bf16; every
 * fp32 -> bf16 store rounds to nearest even.
 *
 * Ownership and behaviour common to every entry point (the graph-safe entry that neither
 * allocates nor synchronises: FlashQLA PR #1, verify integration spec commit, shared
 * infrastructure; the caller-preallocated path that avoids any allocation and the default
 * that never validates device contents or synchronises: cuLA PR #113, final-source
 * validation section):
 *   - every pointer is device memory owned by the caller; the library never
 *     allocates, frees, retains or synchronises: it validates metadata on the host,
 *     enqueues kernels on `hip_stream` (NULL = the legacy default stream) and returns,
 *     so every call can be captured into a HIP graph;
 *   - validation covers metadata only (null pointers, sizes, enums) and happens
 *     before any launch; device contents (slot ids, cu_seqlens values, NaN, g > 0,
 *     duplicate slots) are NOT checked and are undefined behaviour when invalid;
 *   - N == 0 returns GDR_SUCCESS without launching anything; so does T == 0 unless a
 *     final state is requested (the dense entry points then copy the initial state);
 *   - outputs must not alias inputs, except where stated;
 *   - the library keeps no mutable global state and is thread-safe.
 */
#ifndef GDR_H_
#define GDR_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define GDR_API __attribute__((visibility("default")))
#else
#define GDR_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdr_status {
    GDR_SUCCESS = 0,
    GDR_ERROR_INVALID_VALUE = 1,   /* bad metadata: null pointer, size, enum, workspace */
    GDR_ERROR_NOT_SUPPORTED = 2,   /* valid but unsupported: head dim, dtype combo, device */
    GDR_ERROR_LAUNCH_FAILED = 3,   /* hipGetLastError reported a failure after a launch */
    GDR_ERROR_SCRATCH_LIMIT = 4    /* gdr_chunk_fwd_noalloc: the problem needs more scratch than
                                      GDR_NOALLOC_SCRATCH_BYTES                              */
} gdr_status;

/* Size of the fixed device scratch array behind gdr_chunk_fwd_noalloc (per GPU). */
#define GDR_NOALLOC_SCRATCH_BYTES (64u << 20)

typedef enum gdr_dtype { GDR_F32 = 0, GDR_BF16 = 1 } gdr_dtype;

typedef enum gdr_gate {
    GDR_GATE_SCALAR = 0,  /* g  [T, HV]     one log-decay per token and value head (GDN) */
    GDR_GATE_PER_K = 1    /* gk [T, HV, K]  one log-decay per key channel (KDA)          */
} gdr_gate;

typedef struct gdr_problem {
    int64_t total_tokens;   /* T (host value; equals cu_seqlens[N] on the device)        */
    int32_t num_seqs;       /* N                                                          */
    int32_t num_k_heads;    /* HK                                                         */
    int32_t num_v_heads;    /* HV, a multiple of HK                                       */
    int32_t head_dim_k;     /* K in {64, 128}                                             */
    int32_t head_dim_v;     /* V in {64, 128}                                             */
    float scale;            /* multiplies o only (1/sqrt(K) in the usual setting)         */
    gdr_gate gate;
    gdr_dtype io_dtype;     /* dtype of q, k, v, beta, o; gates are always fp32            */
} gdr_problem;

/*
 * gdr_recurrent_fwd -- the recurrence token by token over a packed varlen batch.
 * (FlashQLA PR #1: the fused recurrent decode kernel and its multi-step q_len loop.)
 *
 *   cu_seqlens     int32 [N+1]; may be NULL only when N == 1 (one sequence of T tokens)
 *   initial_state  fp32 [N, HV, V, K] or NULL (zeros)
 *   o              [T, HV, V] io_dtype (written)
 *   final_state    fp32 [N, HV, V, K] or NULL (not written); may alias initial_state
 * Empty sequences are allowed: their final state equals their initial state.
 */
GDR_API gdr_status gdr_recurrent_fwd(const gdr_problem* p,
                             const void* q, const void* k, const void* v,
                             const float* g, const void* beta,
                             const int32_t* cu_seqlens,
                             const float* initial_state,
                             void* o, float* final_state,
                             void* hip_stream);

/*
 * gdr_chunk_workspace_size -- bytes of device workspace gdr_chunk_fwd needs for this
 * problem (depends on T, N, HV, K, V and io_dtype).  Returns 0 for invalid metadata.
 * The workspace follows the caller-preallocated path of the chunked forward (cuLA PR #113,
 * final-source validation section: the preallocated path issues no allocation); here it
 * holds the segment table, per-segment offsets and linear maps and the chained start states
 * of the context-parallel route for a few long sequences (FlashQLA PR #1, decode design
 * commit: occupancy by splitting work, the decode analogue of automatic context
 * parallelism), and is 0 when that route is not taken.
 */
GDR_API size_t gdr_chunk_workspace_size(const gdr_problem* p, int32_t chunk_size);

/*
 * gdr_chunk_fwd -- the same result as gdr_recurrent_fwd computed chunk-parallel: 64-token
 * chunks counted from each sequence's first token (the last chunk of a sequence may be
 * short), an intra-chunk WY/UT transform (cumulative gate, A = (I + strictly-lower
 * beta*KK^T*decay)^-1, w, u), a sequential inter-chunk state pass
 * (v_new = u - w h, h <- decayed h + (decayed k)^T v_new) and a chunk output stage.
 * (cuLA PR #113 "[GDN2] Add Hopper SM90 CuTe DSL prefill"; attention-gym PR #344 "Replace
 * the KDA inter-chunk recurrence with a warp-specialized kernel".)  No factor of the form
 * exp(-prefix) is ever formed, so every finite g <= 0 is safe (cuLA PR #113 review).
 *
 *   chunk_size     must be 64
 *   cu_seqlens, initial_state, o, final_state: as gdr_recurrent_fwd
 *   workspace      device buffer of at least gdr_chunk_workspace_size(p, 64) bytes,
 *                  caller-owned, contents need not be initialised, 256-byte aligned, or NULL.
 *                  A non-zero size means the problem has few, long sequences for the number of
 *                  heads; with the workspace the call cuts every sequence into segments that run
 *                  in parallel (segment offsets and linear maps, a scan over each sequence's
 *                  segments, then every segment from its true start state), with NULL it runs
 *                  every sequence's chunks in one pass.  A non-NULL workspace smaller than the
 *                  size returns GDR_ERROR_INVALID_VALUE.
 * Every K, V in {64, 128} and both I/O dtypes are accepted with either gate.  fp32 I/O with the
 * per-key-channel gate at K = 128 runs the token-serial recurrence kernel of gdr_recurrent_fwd (the
 * chunk kernel's fp32 per-channel operands do not fit the LDS): its result equals gdr_recurrent_fwd
 * bitwise, it needs no workspace (gdr_chunk_workspace_size returns 0) and its time grows with the
 * longest sequence token by token.  Every other configuration runs the chunked method, and its
 * result matches gdr_recurrent_fwd to the chunked method's rounding, not bitwise.
 */
GDR_API gdr_status gdr_chunk_fwd(const gdr_problem* p, int32_t chunk_size,
                         const void* q, const void* k, const void* v,
                         const float* g, const void* beta,
                         const int32_t* cu_seqlens,
                         const float* initial_state,
                         void* o, float* final_state,
                         void* workspace, size_t workspace_bytes,
                         void* hip_stream);

/*
 * gdr_chunk_fwd_noalloc -- gdr_chunk_fwd for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, and harnesses that forbid hipMalloc.  Same
 * arguments and result as gdr_chunk_fwd, minus the workspace: the scratch that
 * gdr_chunk_workspace_size reports comes from a fixed device array inside the library,
 * GDR_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, reserved on each GPU the library runs on until
 * the process ends.  The call allocates nothing (no hipMalloc, no allocating library routine).
 *   - a problem whose workspace exceeds GDR_NOALLOC_SCRATCH_BYTES returns
 *     GDR_ERROR_SCRATCH_LIMIT without launching anything;
 *   - every call on one GPU shares that GPU's array, which keeps the last call's contents (each
 *     call writes every scratch byte it reads before reading it); calls that overlap on one GPU
 *     (concurrent streams or host threads) race on the array and give undefined results.
 */
GDR_API gdr_status gdr_chunk_fwd_noalloc(const gdr_problem* p, int32_t chunk_size,
                                 const void* q, const void* k, const void* v,
                                 const float* g, const void* beta,
                                 const int32_t* cu_seqlens,
                                 const float* initial_state,
                                 void* o, float* final_state,
                                 void* hip_stream);

/*
 * gdr_decode_paged -- decode (q_len 1) and speculative verify (q_len up to 12) against a
 * paged state pool.  (FlashQLA PR #1: verify kernel -- in-kernel paged gather/scatter via
 * state_indices, V-major pool, per-token intermediate states, no-commit mode, varlen
 * cu_seqlens; deployment-facts commit -- PAD_SLOT_ID = -1, slot 0 valid, intermediate rows
 * gated by the pool slot mask.)
 *
 *   max_q_len            1..12, an upper bound on every sequence length
 *   cu_seqlens           int32 [N+1], or NULL: every sequence has exactly one token (T == N)
 *   pool                 [num_slots, HV, V, K] pool_dtype (fp32 or bf16), updated in place
 *   state_indices        int32 [N]; sequence b starts from pool[state_indices[b]];
 *                        a negative index marks a padded sequence, which is skipped
 *                        entirely: no pool read or write, no intermediate write, and its
 *                        o rows are left untouched.  Non-negative indices must be distinct
 *                        and < num_slots.
 *   commit               1: write the state after the last token back to pool[slot]
 *                        0: the pool is not written (verify)
 *   inter_states         NULL, or [num_cache_slots, cache_steps, HV, V, K] inter_dtype:
 *                        the post-update state after token t (t < len_b) of sequence b goes
 *                        to [inter_state_indices[b], t]; rows t >= len_b are untouched
 *   inter_state_indices  int32 [N] (required when inter_states is set), values <
 *                        num_cache_slots
 *   cache_steps          >= max_q_len when inter_states is set
 *   o                    [T, HV, V] io_dtype
 * The gate must be GDR_GATE_SCALAR or GDR_GATE_PER_K as declared in p.
 */
GDR_API gdr_status gdr_decode_paged(const gdr_problem* p, int32_t max_q_len,
                            const void* q, const void* k, const void* v,
                            const float* g, const void* beta,
                            const int32_t* cu_seqlens,
                            void* pool, gdr_dtype pool_dtype, int32_t num_slots,
                            const int32_t* state_indices, int32_t commit,
                            void* inter_states, gdr_dtype inter_dtype,
                            int32_t num_cache_slots, int32_t cache_steps,
                            const int32_t* inter_state_indices,
                            void* o, void* hip_stream);

/*
 * Gating front (FlashQLA PR #1: host-gating wrapper commit, in-kernel gated verify commit,
 * verify pre-pass commit, and the pull-request description for softplus 1.0 / 20.0).  The
 * entry points below take the raw inputs of the usual GDN layer instead of activated ones:
 *
 *     g[t,h]    = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h])
 *                 softplus(x) = x for x > 20, log(1 + exp(x)) otherwise
 *     beta[t,h] = sigmoid(b[t,h]), times 2 when allow_neg_eigval
 *     q, k      <- x / sqrt(sum_c x_c^2 + l2norm_eps) per (token, key head), when qk_l2norm
 *
 * The pages give no epsilon for the normalisation; it is the caller's (0 allowed, 1e-6 is
 * the binding's default).  Only the scalar gate (GDR_GATE_SCALAR) has a gating front;
 * a per-K-channel problem returns GDR_ERROR_NOT_SUPPORTED.
 */
typedef struct gdr_gating {
    const void*  a;                 /* [T, HV] io_dtype: decay input before softplus        */
    const void*  b;                 /* [T, HV] io_dtype: beta input before the sigmoid       */
    const float* A_log;             /* [HV] fp32                                            */
    const float* dt_bias;           /* [HV] fp32                                            */
    float        l2norm_eps;        /* finite, >= 0                                         */
    int32_t      qk_l2norm;         /* 1: normalise q and k; 0: take them as given          */
    int32_t      allow_neg_eigval;  /* 1: beta = 2 sigmoid(b)                               */
} gdr_gating;

/*
 * gdr_gating_prepass -- the gating front as one pass over the batch (the pre-pass design of
 * the verify pre-pass commit): writes normalised q, k and activated g, beta for every token,
 * ready for gdr_recurrent_fwd, gdr_chunk_fwd or gdr_decode_paged.
 *
 *   q, k           [T, HK, K] io_dtype, raw (read only when gating->qk_l2norm)
 *   q_out, k_out   [T, HK, K] io_dtype (written when qk_l2norm; may be NULL otherwise);
 *                  q_out may equal q and k_out may equal k (in place)
 *   g_out          [T, HV] fp32;  beta_out [T, HV] io_dtype
 * T == 0 returns GDR_SUCCESS without a launch.  p->num_seqs and p->head_dim_v are not used
 * beyond validation.
 */
GDR_API gdr_status gdr_gating_prepass(const gdr_problem* p,
                              const void* q, const void* k,
                              const gdr_gating* gating,
                              void* q_out, void* k_out,
                              float* g_out, void* beta_out,
                              void* hip_stream);

/*
 * gdr_decode_paged_gated -- gdr_decode_paged with the gating front inside the token loop
 * (the fused design of the in-kernel gated verify commit): q and k are the raw inputs, and
 * g and beta are formed from gating->a, gating->b per token.  Every other argument, the
 * padded-slot rule, commit and the intermediate states behave exactly as in
 * gdr_decode_paged.  Equivalent, up to rounding, to gdr_gating_prepass followed by
 * gdr_decode_paged.
 */
GDR_API gdr_status gdr_decode_paged_gated(const gdr_problem* p, int32_t max_q_len,
                                  const void* q, const void* k, const void* v,
                                  const gdr_gating* gating,
                                  const int32_t* cu_seqlens,
                                  void* pool, gdr_dtype pool_dtype, int32_t num_slots,
                                  const int32_t* state_indices, int32_t commit,
                                  void* inter_states, gdr_dtype inter_dtype,
                                  int32_t num_cache_slots, int32_t cache_steps,
                                  const int32_t* inter_state_indices,
                                  void* o, void* hip_stream);

/*
 * Fused KDA decode front (tokenspeed PR #834 "[WIP] perf(k3): optimize decode": the commit that
 * rewrites the single-launch KDA decode -- causal convolution with SiLU, the gate projection, q/k
 * l2 normalisation and the delta-rule recurrence against the paged fp32 state -- and the commit
 * that folds rmsnorm(o) * w * sigmoid(gate) into its epilogue).  The page names the steps but
 * not their formulas; the readings taken here, per token t of sequence n and head h (one key head
 * per value head, HK == HV):
 *
 *     conv     y[c] = silu(bias[c] + sum_{i<W} w[c][i] x_{t-(W-1)+i}[c]) for every channel c of
 *              q, k and v (raw projections), with the tokens before the call taken from the
 *              slot's window (the W-1 latest raw inputs, oldest first); silu(z) = z sigmoid(z)
 *     gate     gk[h][c] = -exp(A_log[h]) softplus((gate_weight gate_in[t])[h K + c] + dt_bias[h K + c])
 *              (softplus with threshold 20, as gdr_gating)
 *     norm     q, k <- y / sqrt(sum y^2 + l2norm_eps) per (token, head)
 *     beta     sigmoid(b[t, h])
 *     state    the recurrence of gdr_decode_paged with the per-key-channel gate
 *     epilogue optional: o <- o / sqrt(mean_v o^2 + norm_eps) * norm_weight[v] * sigmoid(norm_gate[t,h,v])
 */
typedef struct gdr_kda_front {
    int32_t      conv_width;   /* W in 1..4                                                      */
    const void*  conv_weight;  /* [C, W] io_dtype, C = 2*HV*K + HV*V channels: q | k | v, each   */
                               /* head-major (q channel h*K + c, then k, then v); taps oldest first */
    const void*  conv_bias;    /* [C] io_dtype, or NULL (no bias)                                */
    void*        conv_state;   /* [num_slots, C, W-1] io_dtype: each slot's window, oldest first;  */
                               /* rewritten in place on commit; may be NULL when W == 1            */
    const void*  gate_in;      /* [T, R] io_dtype: the low-rank gate input of each token           */
    const void*  gate_weight;  /* [HV*K, R] io_dtype: the gate projection                          */
    int32_t      gate_rank;    /* R, a positive multiple of 8, at most 4096                        */
    const float* A_log;        /* [HV] fp32                                                        */
    const float* dt_bias;      /* [HV*K] fp32                                                      */
    const void*  b;            /* [T, HV] io_dtype: beta input before the sigmoid                  */
    float        l2norm_eps;   /* finite, >= 0                                                     */
    const void*  norm_weight;  /* [V] io_dtype, or NULL: no epilogue                               */
    const void*  norm_gate;    /* [T, HV, V] io_dtype (required with norm_weight)                  */
    float        norm_eps;     /* finite, >= 0                                                     */
} gdr_kda_front;

/*
 * gdr_kda_decode_fused -- decode (q_len 1) and multi-token decode (q_len up to 12) of the KDA layer
 * from the raw projections, in one launch.  q, k [T, HV, K] and v [T, HV, V] are the raw inputs of
 * the convolution; p->gate must be GDR_GATE_PER_K and p->num_k_heads == p->num_v_heads (otherwise
 * GDR_ERROR_NOT_SUPPORTED).  cu_seqlens, pool, pool_dtype, num_slots, state_indices (-1 = padded:
 * the sequence is skipped, its o rows untouched), commit and o behave as in gdr_decode_paged;
 * commit also writes each active slot's convolution window back, and commit = 0 leaves both the
 * pool and the windows unchanged.  There is no per-token intermediate-state buffer here.
 * The workgroup of a (sequence, head) owns every convolution channel of that head, so the window
 * update does not race between heads or sequences; distinct slots are required as in
 * gdr_decode_paged.
 */
GDR_API gdr_status gdr_kda_decode_fused(const gdr_problem* p, int32_t max_q_len,
                                const void* q, const void* k, const void* v,
                                const gdr_kda_front* front,
                                const int32_t* cu_seqlens,
                                void* pool, gdr_dtype pool_dtype, int32_t num_slots,
                                const int32_t* state_indices, int32_t commit,
                                void* o, void* hip_stream);

/* Human-readable name of a status code (static string, never NULL; unknown codes map to
 * "GDR_ERROR_UNKNOWN").  The codes stand for the loud contract checks of the pages' entry
 * points: a device-capability check (cuLA PR #113, review thread on SM90 availability) and a
 * wrapper that rejects unsupported dtypes, shapes and capabilities while empty inputs return
 * early on the host (attention-gym PR #344, pull-request description). */
GDR_API const char* gdr_status_string(gdr_status s);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H_ */
