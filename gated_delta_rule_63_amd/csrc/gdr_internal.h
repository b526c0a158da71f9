// Internal (non-exported) declarations shared by the host side of libgdr:
// kernel argument blocks and launchers.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <type_traits>

namespace gdr {

// Token-loop kernel (dense recurrent, paged decode, verify).
struct RecurrentArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const void* beta;
    void* o;
    const int32_t* cu_seqlens;   // NULL: see one_token_per_seq
    int32_t one_token_per_seq;   // with cu_seqlens NULL: 1 -> sequence n is token n; 0 -> one sequence of T tokens
    int32_t prefetch;            // 1: load token t+1's inputs while token t computes (multi-token sequences)
    int64_t T;
    const void* src;             // state source [*, HV, V, K] (pool or initial state), NULL = zeros
    void* dst;                   // state destination (pool on commit, final state), NULL = none
    const int32_t* slots;        // state_indices (paged) or NULL (dense: slot = sequence)
    void* ibuf;                  // per-token states [*, cache_steps, HV, V, K] or NULL
    const int32_t* ibuf_idx;
    int32_t cache_steps;
    int32_t N, HK, HV, V;
    float scale;
    // gating front, read only by the gated instantiation: g and beta are formed per token from
    // the raw inputs a, b and the per-head A_log, dt_bias; q and k are l2-normalised when asked
    const void* ga;              // a [T, HV] io dtype
    const void* gb;              // b [T, HV] io dtype
    const float* A_log;          // [HV]
    const float* dt_bias;        // [HV]
    float l2_eps;
    int32_t qk_l2norm;
    float beta_mul;              // 1, or 2 when negative eigenvalues are allowed
};

// Copy n fp32 values src -> dst (zeros when src is NULL); nothing when src == dst.
hipError_t launch_state_copy(const float* src, float* dst, int64_t n, hipStream_t stream);

// dtype codes: 0 = fp32, 1 = bf16; ib_dtype -1 = no intermediate buffer.  gated needs !per_k.
// Requires a.T >= 1.
hipError_t launch_recurrent(const RecurrentArgs& a, int K, int io_dtype, int st_dtype, int ib_dtype,
                            bool per_k, bool gated, hipStream_t stream);

// Gating front as a pass of its own: normalised q, k and activated g, beta for every token.
struct GatingArgs {
    const void* q;
    const void* k;
    void* q_out;                 // may equal q (each row is read whole before it is written)
    void* k_out;
    const void* a;
    const void* b;
    const float* A_log;
    const float* dt_bias;
    float* g_out;                // [T, HV] fp32
    void* beta_out;              // [T, HV] io dtype
    int64_t T;
    int32_t HK, HV;
    float l2_eps;
    int32_t qk_l2norm;
    float beta_mul;
};

hipError_t launch_gating(const GatingArgs& a, int K, int io_dtype, hipStream_t stream);

// Chunked path (64-token chunks).
struct ChunkArgs {
    const void* q;
    const void* k;
    const void* v;               // NULL reads as zeros
    const float* g;
    const void* beta;
    const int32_t* cu_seqlens;   // NULL only when N == 1
    const float* h0;             // [N, HV, V, K] or NULL (zeros)
    void* o;                     // NULL: outputs not written
    float* ht;                   // [N, HV, V, K] or NULL; may equal h0 (each thread reads its part first)
    // non-NULL selects the paired run of the segmented route (bf16, K = V, either gate): besides
    // ht, map [N, HV, K, K] receives the end state from the identity with v = 0; q and o are unused
    float* map;
    int64_t T;
    int32_t N, HK, HV, K, V;
    float scale;
};

hipError_t launch_chunk(const ChunkArgs& a, int io_dtype, bool per_k, hipStream_t stream);

// Fused KDA decode front (gdr_kda.hip): convolution + SiLU, gate projection, q/k l2 norm, beta,
// per-key-channel recurrence against the paged state, optional gated RMSNorm epilogue.
struct KdaArgs {
    const void* q;               // [T, HV, K] io dtype, raw (before the convolution)
    const void* k;               // [T, HV, K]
    const void* v;               // [T, HV, V]
    const int32_t* cu_seqlens;   // [N + 1] or NULL (one token per sequence)
    void* pool;                  // [slots, HV, V, K] state dtype
    const int32_t* slots;        // [N]; negative = padded sequence
    int32_t commit;              // write the state and the convolution windows back
    void* o;                     // [T, HV, V] io dtype
    int32_t conv_width;          // 1..4
    const void* conv_weight;     // [C, W] io dtype, C = 2 HV K + HV V (q | k | v)
    const void* conv_bias;       // [C] or NULL
    void* conv_state;            // [slots, C, W - 1] io dtype
    const void* gate_in;         // [T, R] io dtype
    const void* gate_weight;     // [HV K, R] io dtype
    int32_t gate_rank;           // R, a multiple of 8
    const float* A_log;          // [HV]
    const float* dt_bias;        // [HV K]
    const void* b;               // [T, HV] io dtype
    float l2_eps;
    const void* norm_weight;     // [V] io dtype, or NULL: no epilogue
    const void* norm_gate;       // [T, HV, V] io dtype
    float norm_eps;
    float scale;
    int32_t N, HV;
};

hipError_t launch_kda(const KdaArgs& a, int K, int V, int io_dtype, int st_dtype, hipStream_t stream);

// Context parallelism for a few long sequences (gdr_cp.hip): every sequence is cut into segments of
// seg_tokens tokens (a multiple of 64; a sequence's last segment may be shorter) that run as the
// sequences of three chunk-kernel launches.
constexpr int kCpWorkgroups = 256;   // target chunk-kernel workgroups per run: one per CU of the part
constexpr int kCpMinChunks = 8;      // at least this many chunks per segment
constexpr int kCpMinSegments = 4;    // segments per sequence; below this the three runs cost more than they save

struct CpPlan {
    int P;                           // segments the workspace holds (an upper bound on the real count); 1 = no CP
    int N;                           // sequences
    int64_t seg_tokens;
    size_t cu_seg, seg_first, B, M, S, total;   // workspace offsets (256-byte aligned) and size
};

CpPlan cp_plan(int64_t T, int32_t N, int32_t HV, int32_t K, int32_t V, int io_bytes);
// identity: also set every segment map to the identity (the start state of the separate map run)
hipError_t launch_cp_setup(const CpPlan& pl, char* ws, const int32_t* cu, int64_t T, int32_t HV, int32_t K,
                           bool identity, hipStream_t stream);
hipError_t launch_cp_scan(const CpPlan& pl, char* ws, const float* h0, int32_t HV, int32_t K, int32_t V,
                          hipStream_t stream);
hipError_t launch_cp_final(const CpPlan& pl, const char* ws, float* out, int32_t HV, int32_t K, int32_t V,
                           hipStream_t stream);

}  // namespace gdr
