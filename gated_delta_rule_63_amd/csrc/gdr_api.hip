// C ABI of libgdr (declared in include/gdr.h): metadata validation on the host,
// then kernel launches on the caller's stream.  No allocation, no synchronisation.
#include <atomic>
#include <cstring>

#include "../../include/gdr.h"
#include "gdr_internal.h"

namespace {

using gdr::RecurrentArgs;

// Scratch of gdr_chunk_fwd_noalloc: a fixed device array instead of a caller's workspace, for
// callers that cannot allocate.  Each GPU the library runs on holds its own copy until the process
// ends.  In host code the array's name is only a stand-in for the symbol: its device address, per
// device, comes from hipGetSymbolAddress and is the only form ever passed to a kernel.
static __device__ __align__(256) char scratch[GDR_NOALLOC_SCRATCH_BYTES];

std::atomic<char*> g_scratch_ptr[64];

// Device address of this device's scratch array (looked up once per device, with it current).
gdr_status scratch_address(char** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return GDR_ERROR_NOT_SUPPORTED;
    char* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        void* sym = nullptr;
        if (hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch)) != hipSuccess || !sym) return GDR_ERROR_LAUNCH_FAILED;
        ptr = static_cast<char*>(sym);
        g_scratch_ptr[dev].store(ptr, std::memory_order_release);  // every thread finds the same address
    }
    *out = ptr;
    return GDR_SUCCESS;
}

bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }

bool dtype_ok(int d) { return d == GDR_F32 || d == GDR_BF16; }

// gfx950 check, cached per device (written once, idempotent).
std::atomic<int> g_arch_ok[64];

gdr_status check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GDR_ERROR_NOT_SUPPORTED;
    if (dev < 0 || dev >= 64) return GDR_ERROR_NOT_SUPPORTED;
    int cached = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (cached == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GDR_ERROR_NOT_SUPPORTED;
        cached = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_arch_ok[dev].store(cached, std::memory_order_relaxed);
    }
    return cached == 1 ? GDR_SUCCESS : GDR_ERROR_NOT_SUPPORTED;
}

// Metadata shared by every entry point.
gdr_status check_problem(const gdr_problem* p) {
    if (!p) return GDR_ERROR_INVALID_VALUE;
    if (p->total_tokens < 0 || p->num_seqs < 0) return GDR_ERROR_INVALID_VALUE;
    if (p->num_k_heads <= 0 || p->num_v_heads <= 0) return GDR_ERROR_INVALID_VALUE;
    if (p->num_v_heads % p->num_k_heads != 0) return GDR_ERROR_INVALID_VALUE;
    if (p->gate != GDR_GATE_SCALAR && p->gate != GDR_GATE_PER_K) return GDR_ERROR_INVALID_VALUE;
    if (!dtype_ok(p->io_dtype)) return GDR_ERROR_INVALID_VALUE;
    if (p->head_dim_k <= 0 || p->head_dim_v <= 0) return GDR_ERROR_INVALID_VALUE;
    if (!head_dim_ok(p->head_dim_k) || !head_dim_ok(p->head_dim_v)) return GDR_ERROR_NOT_SUPPORTED;
    if (p->num_seqs > 65535 || p->num_v_heads > 65535) return GDR_ERROR_NOT_SUPPORTED;  // grid y/z limits
    return GDR_SUCCESS;
}

bool token_inputs_ok(const gdr_problem* p, const void* q, const void* k, const void* v, const float* g,
                     const void* beta) {
    if (p->total_tokens == 0) return true;
    return q && k && v && g && beta;
}

gdr_status status_of(hipError_t e) { return e == hipSuccess ? GDR_SUCCESS : GDR_ERROR_LAUNCH_FAILED; }

// fp32 operands with the per-key-channel gate at K = 128: the chunk kernel's fp32 per-channel tables
// and operands do not fit the LDS, so gdr_chunk_fwd runs the token-serial recurrence kernel instead
// (the same launch as gdr_recurrent_fwd, the exact recurrence rather than the chunked rounding)
bool token_serial_chunk(const gdr_problem* p) {
    return p->io_dtype == GDR_F32 && p->gate == GDR_GATE_PER_K && p->head_dim_k == 128;
}

// Gating-front metadata: scalar decay only, flags 0/1, eps finite and >= 0, pointers present.
gdr_status check_gating(const gdr_problem* p, const gdr_gating* gt) {
    if (!gt) return GDR_ERROR_INVALID_VALUE;
    if (p->gate != GDR_GATE_SCALAR) return GDR_ERROR_NOT_SUPPORTED;
    if (gt->qk_l2norm != 0 && gt->qk_l2norm != 1) return GDR_ERROR_INVALID_VALUE;
    if (gt->allow_neg_eigval != 0 && gt->allow_neg_eigval != 1) return GDR_ERROR_INVALID_VALUE;
    if (!(gt->l2norm_eps >= 0.0f) || gt->l2norm_eps > 3.0e38f) return GDR_ERROR_INVALID_VALUE;  // NaN fails too
    if (p->total_tokens > 0 && !(gt->a && gt->b && gt->A_log && gt->dt_bias)) return GDR_ERROR_INVALID_VALUE;
    return GDR_SUCCESS;
}

// Shared body of the paged entry points; either (g, beta) or gating is set, and the token
// inputs have been checked by the caller.
gdr_status decode_paged_impl(const gdr_problem* p, int32_t max_q_len, const void* q, const void* k, const void* v,
                             const float* g, const void* beta, const gdr_gating* gating,
                             const int32_t* cu_seqlens, void* pool, gdr_dtype pool_dtype, int32_t num_slots,
                             const int32_t* state_indices, int32_t commit, void* inter_states,
                             gdr_dtype inter_dtype, int32_t num_cache_slots, int32_t cache_steps,
                             const int32_t* inter_state_indices, void* o, void* hip_stream) {
    if (max_q_len < 1 || max_q_len > 12) return GDR_ERROR_INVALID_VALUE;
    if (!pool || num_slots <= 0 || !state_indices) return GDR_ERROR_INVALID_VALUE;
    if (!dtype_ok(pool_dtype)) return GDR_ERROR_INVALID_VALUE;
    if (commit != 0 && commit != 1) return GDR_ERROR_INVALID_VALUE;
    if (p->total_tokens > 0 && !o) return GDR_ERROR_INVALID_VALUE;
    if (!cu_seqlens && p->total_tokens != p->num_seqs) return GDR_ERROR_INVALID_VALUE;
    if (p->total_tokens > (int64_t)p->num_seqs * max_q_len) return GDR_ERROR_INVALID_VALUE;
    if (inter_states) {
        if (!inter_state_indices || num_cache_slots <= 0 || cache_steps < max_q_len) return GDR_ERROR_INVALID_VALUE;
        if (!dtype_ok(inter_dtype)) return GDR_ERROR_INVALID_VALUE;
    }
    if (p->num_seqs == 0 || p->total_tokens == 0) return GDR_SUCCESS;
    gdr_status st = check_device();
    if (st != GDR_SUCCESS) return st;

    RecurrentArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = o;
    a.cu_seqlens = cu_seqlens;
    a.one_token_per_seq = cu_seqlens ? 0 : 1;
    a.prefetch = max_q_len > 1;
    a.T = p->total_tokens;
    a.src = pool;
    a.dst = commit ? pool : nullptr;
    a.slots = state_indices;
    a.ibuf = inter_states;
    a.ibuf_idx = inter_state_indices;
    a.cache_steps = cache_steps;
    a.N = p->num_seqs; a.HK = p->num_k_heads; a.HV = p->num_v_heads; a.V = p->head_dim_v;
    a.scale = p->scale;
    if (gating) {
        a.ga = gating->a; a.gb = gating->b; a.A_log = gating->A_log; a.dt_bias = gating->dt_bias;
        a.l2_eps = gating->l2norm_eps;
        a.qk_l2norm = gating->qk_l2norm;
        a.beta_mul = gating->allow_neg_eigval ? 2.0f : 1.0f;
    }
    return status_of(gdr::launch_recurrent(a, p->head_dim_k, p->io_dtype, pool_dtype,
                                           inter_states ? (int)inter_dtype : -1, p->gate == GDR_GATE_PER_K,
                                           gating != nullptr, static_cast<hipStream_t>(hip_stream)));
}

}  // namespace

extern "C" {

const char* gdr_status_string(gdr_status s) {
    switch (s) {
        case GDR_SUCCESS: return "GDR_SUCCESS";
        case GDR_ERROR_INVALID_VALUE: return "GDR_ERROR_INVALID_VALUE";
        case GDR_ERROR_NOT_SUPPORTED: return "GDR_ERROR_NOT_SUPPORTED";
        case GDR_ERROR_LAUNCH_FAILED: return "GDR_ERROR_LAUNCH_FAILED";
        case GDR_ERROR_SCRATCH_LIMIT: return "GDR_ERROR_SCRATCH_LIMIT";
        default: return "GDR_ERROR_UNKNOWN";
    }
}

gdr_status gdr_recurrent_fwd(const gdr_problem* p, const void* q, const void* k, const void* v, const float* g,
                             const void* beta, const int32_t* cu_seqlens, const float* initial_state, void* o,
                             float* final_state, void* hip_stream) {
    gdr_status st = check_problem(p);
    if (st != GDR_SUCCESS) return st;
    if (!token_inputs_ok(p, q, k, v, g, beta)) return GDR_ERROR_INVALID_VALUE;
    if (p->total_tokens > 0 && !o) return GDR_ERROR_INVALID_VALUE;
    if (p->num_seqs > 1 && !cu_seqlens) return GDR_ERROR_INVALID_VALUE;
    if (p->num_seqs == 0 && p->total_tokens > 0) return GDR_ERROR_INVALID_VALUE;
    if (p->num_seqs == 0) return GDR_SUCCESS;
    // all sequences empty and no final state requested: nothing to compute
    if (p->total_tokens == 0 && !final_state) return GDR_SUCCESS;
    if ((st = check_device()) != GDR_SUCCESS) return st;
    if (p->total_tokens == 0) {  // every sequence empty: final state = initial state (or zeros)
        const int64_t n = (int64_t)p->num_seqs * p->num_v_heads * p->head_dim_v * p->head_dim_k;
        return status_of(gdr::launch_state_copy(initial_state, final_state, n, static_cast<hipStream_t>(hip_stream)));
    }

    RecurrentArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = o;
    a.cu_seqlens = cu_seqlens;
    a.one_token_per_seq = 0;
    a.prefetch = 1;
    a.T = p->total_tokens;
    a.src = initial_state;
    a.dst = final_state;
    a.slots = nullptr;
    a.ibuf = nullptr; a.ibuf_idx = nullptr; a.cache_steps = 0;
    a.N = p->num_seqs; a.HK = p->num_k_heads; a.HV = p->num_v_heads; a.V = p->head_dim_v;
    a.scale = p->scale;
    return status_of(gdr::launch_recurrent(a, p->head_dim_k, p->io_dtype, GDR_F32, -1,
                                           p->gate == GDR_GATE_PER_K, false, static_cast<hipStream_t>(hip_stream)));
}

gdr_status gdr_decode_paged(const gdr_problem* p, int32_t max_q_len, const void* q, const void* k, const void* v,
                            const float* g, const void* beta, const int32_t* cu_seqlens, void* pool,
                            gdr_dtype pool_dtype, int32_t num_slots, const int32_t* state_indices, int32_t commit,
                            void* inter_states, gdr_dtype inter_dtype, int32_t num_cache_slots,
                            int32_t cache_steps, const int32_t* inter_state_indices, void* o, void* hip_stream) {
    gdr_status st = check_problem(p);
    if (st != GDR_SUCCESS) return st;
    if (!token_inputs_ok(p, q, k, v, g, beta)) return GDR_ERROR_INVALID_VALUE;
    return decode_paged_impl(p, max_q_len, q, k, v, g, beta, nullptr, cu_seqlens, pool, pool_dtype, num_slots,
                             state_indices, commit, inter_states, inter_dtype, num_cache_slots, cache_steps,
                             inter_state_indices, o, hip_stream);
}

gdr_status gdr_decode_paged_gated(const gdr_problem* p, int32_t max_q_len, const void* q, const void* k,
                                  const void* v, const gdr_gating* gating, const int32_t* cu_seqlens, void* pool,
                                  gdr_dtype pool_dtype, int32_t num_slots, const int32_t* state_indices,
                                  int32_t commit, void* inter_states, gdr_dtype inter_dtype,
                                  int32_t num_cache_slots, int32_t cache_steps,
                                  const int32_t* inter_state_indices, void* o, void* hip_stream) {
    gdr_status st = check_problem(p);
    if (st != GDR_SUCCESS) return st;
    if ((st = check_gating(p, gating)) != GDR_SUCCESS) return st;
    if (p->total_tokens > 0 && !(q && k && v)) return GDR_ERROR_INVALID_VALUE;
    return decode_paged_impl(p, max_q_len, q, k, v, nullptr, nullptr, gating, cu_seqlens, pool, pool_dtype,
                             num_slots, state_indices, commit, inter_states, inter_dtype, num_cache_slots,
                             cache_steps, inter_state_indices, o, hip_stream);
}

gdr_status gdr_kda_decode_fused(const gdr_problem* p, int32_t max_q_len, const void* q, const void* k, const void* v,
                                const gdr_kda_front* f, const int32_t* cu_seqlens, void* pool, gdr_dtype pool_dtype,
                                int32_t num_slots, const int32_t* state_indices, int32_t commit, void* o,
                                void* hip_stream) {
    gdr_status st = check_problem(p);
    if (st != GDR_SUCCESS) return st;
    if (!f) return GDR_ERROR_INVALID_VALUE;
    if (p->gate != GDR_GATE_PER_K || p->num_k_heads != p->num_v_heads) return GDR_ERROR_NOT_SUPPORTED;
    if (max_q_len < 1 || max_q_len > 12) return GDR_ERROR_INVALID_VALUE;
    if (!pool || num_slots <= 0 || !state_indices) return GDR_ERROR_INVALID_VALUE;
    if (!dtype_ok(pool_dtype)) return GDR_ERROR_INVALID_VALUE;
    if (commit != 0 && commit != 1) return GDR_ERROR_INVALID_VALUE;
    if (!cu_seqlens && p->total_tokens != p->num_seqs) return GDR_ERROR_INVALID_VALUE;
    if (p->total_tokens > (int64_t)p->num_seqs * max_q_len) return GDR_ERROR_INVALID_VALUE;
    if (f->conv_width < 1 || f->conv_width > 4) return GDR_ERROR_INVALID_VALUE;
    if (f->conv_width > 1 && !f->conv_state) return GDR_ERROR_INVALID_VALUE;
    if (f->gate_rank <= 0 || f->gate_rank > 4096 || f->gate_rank % 8 != 0) return GDR_ERROR_INVALID_VALUE;
    if (!(f->l2norm_eps >= 0.0f) || f->l2norm_eps > 3.0e38f) return GDR_ERROR_INVALID_VALUE;
    if (f->norm_weight && (!f->norm_gate || !(f->norm_eps >= 0.0f) || f->norm_eps > 3.0e38f))
        return GDR_ERROR_INVALID_VALUE;
    if (p->total_tokens > 0 && !(q && k && v && o && f->conv_weight && f->gate_in && f->gate_weight && f->A_log &&
                                 f->dt_bias && f->b))
        return GDR_ERROR_INVALID_VALUE;
    if (p->num_seqs == 0 || p->total_tokens == 0) return GDR_SUCCESS;
    if ((st = check_device()) != GDR_SUCCESS) return st;
    gdr::KdaArgs a{};
    a.q = q; a.k = k; a.v = v; a.cu_seqlens = cu_seqlens; a.pool = pool; a.slots = state_indices;
    a.commit = commit; a.o = o;
    a.conv_width = f->conv_width; a.conv_weight = f->conv_weight; a.conv_bias = f->conv_bias;
    a.conv_state = f->conv_state; a.gate_in = f->gate_in; a.gate_weight = f->gate_weight;
    a.gate_rank = f->gate_rank; a.A_log = f->A_log; a.dt_bias = f->dt_bias; a.b = f->b;
    a.l2_eps = f->l2norm_eps; a.norm_weight = f->norm_weight; a.norm_gate = f->norm_gate; a.norm_eps = f->norm_eps;
    a.scale = p->scale; a.N = p->num_seqs; a.HV = p->num_v_heads;
    return status_of(gdr::launch_kda(a, p->head_dim_k, p->head_dim_v, p->io_dtype, pool_dtype,
                                     static_cast<hipStream_t>(hip_stream)));
}

gdr_status gdr_gating_prepass(const gdr_problem* p, const void* q, const void* k, const gdr_gating* gating,
                              void* q_out, void* k_out, float* g_out, void* beta_out, void* hip_stream) {
    gdr_status st = check_problem(p);
    if (st != GDR_SUCCESS) return st;
    if ((st = check_gating(p, gating)) != GDR_SUCCESS) return st;
    if (p->total_tokens > 0) {
        if (!g_out || !beta_out) return GDR_ERROR_INVALID_VALUE;
        if (gating->qk_l2norm && !(q && k && q_out && k_out)) return GDR_ERROR_INVALID_VALUE;
    }
    if (p->total_tokens == 0) return GDR_SUCCESS;
    if ((st = check_device()) != GDR_SUCCESS) return st;
    gdr::GatingArgs a{};
    a.q = q; a.k = k; a.q_out = q_out; a.k_out = k_out;
    a.a = gating->a; a.b = gating->b; a.A_log = gating->A_log; a.dt_bias = gating->dt_bias;
    a.g_out = g_out; a.beta_out = beta_out;
    a.T = p->total_tokens; a.HK = p->num_k_heads; a.HV = p->num_v_heads;
    a.l2_eps = gating->l2norm_eps;
    a.qk_l2norm = gating->qk_l2norm;
    a.beta_mul = gating->allow_neg_eigval ? 2.0f : 1.0f;
    return status_of(gdr::launch_gating(a, p->head_dim_k, p->io_dtype, static_cast<hipStream_t>(hip_stream)));
}

size_t gdr_chunk_workspace_size(const gdr_problem* p, int32_t chunk_size) {
    if (check_problem(p) != GDR_SUCCESS || chunk_size != 64) return 0;
    if (token_serial_chunk(p)) return 0;  // no segmented route for this configuration
    const gdr::CpPlan pl = gdr::cp_plan(p->total_tokens, p->num_seqs, p->num_v_heads, p->head_dim_k,
                                        p->head_dim_v, p->io_dtype == GDR_BF16 ? 2 : 4);
    return pl.P > 1 ? pl.total : 0;
}

}  // extern "C"

namespace {

// Metadata checks of gdr_chunk_fwd that do not involve the workspace.
gdr_status check_chunk(const gdr_problem* p, int32_t chunk_size, const void* q, const void* k, const void* v,
                       const float* g, const void* beta, const int32_t* cu_seqlens, const void* o) {
    gdr_status st = check_problem(p);
    if (st != GDR_SUCCESS) return st;
    if (chunk_size != 64) return GDR_ERROR_INVALID_VALUE;
    if (!token_inputs_ok(p, q, k, v, g, beta)) return GDR_ERROR_INVALID_VALUE;
    if (p->total_tokens > 0 && !o) return GDR_ERROR_INVALID_VALUE;
    if (p->num_seqs > 1 && !cu_seqlens) return GDR_ERROR_INVALID_VALUE;
    if (p->num_seqs == 0 && p->total_tokens > 0) return GDR_ERROR_INVALID_VALUE;
    return GDR_SUCCESS;
}

// Body of gdr_chunk_fwd after validation; `workspace` holds at least gdr_chunk_workspace_size bytes.
gdr_status chunk_fwd_impl(const gdr_problem* p, const void* q, const void* k, const void* v, const float* g,
                          const void* beta, const int32_t* cu_seqlens, const float* initial_state, void* o,
                          float* final_state, void* workspace, void* hip_stream) {
    gdr_status st;
    if (p->num_seqs == 0) return GDR_SUCCESS;
    if (p->total_tokens == 0) {
        // every sequence is empty: final state = initial state
        return gdr_recurrent_fwd(p, q, k, v, g, beta, cu_seqlens, initial_state, o, final_state, hip_stream);
    }
    if (token_serial_chunk(p))
        return gdr_recurrent_fwd(p, q, k, v, g, beta, cu_seqlens, initial_state, o, final_state, hip_stream);
    if ((st = check_device()) != GDR_SUCCESS) return st;

    const bool per_k = p->gate == GDR_GATE_PER_K;
    const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    gdr::ChunkArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.cu_seqlens = cu_seqlens;
    a.h0 = initial_state;
    a.o = o;
    a.ht = final_state;
    a.T = p->total_tokens;
    a.N = p->num_seqs; a.HK = p->num_k_heads; a.HV = p->num_v_heads; a.K = p->head_dim_k; a.V = p->head_dim_v;
    a.scale = p->scale;

    const gdr::CpPlan pl = gdr::cp_plan(p->total_tokens, p->num_seqs, p->num_v_heads, p->head_dim_k,
                                        p->head_dim_v, p->io_dtype == GDR_BF16 ? 2 : 4);
    // the segmented route needs its workspace; without one the call runs the single-pass route
    if (pl.P <= 1 || !workspace) return status_of(gdr::launch_chunk(a, p->io_dtype, per_k, stream));

    // Few long sequences, few heads: cut every sequence into segments that run in parallel.
    //   0. segment table from cu_seqlens (device side), identity maps
    //   1. B_s = end state of segment s from zero; M_s = end state of segment s from the identity
    //      with v = 0 (the K x K linear part of its map); outputs discarded
    //   2. scan per sequence: S_first = initial state, S_{s+1} = S_s M_s + B_s
    //   3. every segment from its true start state: outputs, and the end state in place
    //   4. each sequence's final state = the end state of its last segment
    char* ws = static_cast<char*>(workspace);
    const int32_t* cu_seg = reinterpret_cast<const int32_t*>(ws + pl.cu_seg);
    float* Bs = reinterpret_cast<float*>(ws + pl.B);
    float* Ms = reinterpret_cast<float*>(ws + pl.M);
    float* Ss = reinterpret_cast<float*>(ws + pl.S);
    // bf16 with K = V forms B_s and M_s in one paired run, M_s from an identity it holds itself
    const bool paired = p->io_dtype == GDR_BF16 && p->head_dim_k == p->head_dim_v;
    hipError_t e = gdr::launch_cp_setup(pl, ws, cu_seqlens, p->total_tokens, p->num_v_heads, p->head_dim_k, !paired,
                                        stream);
    if (e != hipSuccess) return status_of(e);

    gdr::ChunkArgs b = a;  // 1a: offsets B_s
    b.cu_seqlens = cu_seg; b.N = pl.P; b.h0 = nullptr; b.o = nullptr; b.ht = Bs;
    if (paired) {
        // 1: one paired run forms B_s and M_s, sharing every chunk's reads and intra-chunk transform
        b.q = nullptr; b.map = Ms;
        if ((e = gdr::launch_chunk(b, p->io_dtype, per_k, stream)) != hipSuccess) return status_of(e);
    } else {
        if ((e = gdr::launch_chunk(b, p->io_dtype, per_k, stream)) != hipSuccess) return status_of(e);
        gdr::ChunkArgs m = a;  // 1b: linear parts M_s (a K-row state, v = 0), in place from the identity
        m.cu_seqlens = cu_seg; m.N = pl.P; m.v = nullptr; m.V = p->head_dim_k; m.h0 = Ms; m.o = nullptr; m.ht = Ms;
        if ((e = gdr::launch_chunk(m, p->io_dtype, per_k, stream)) != hipSuccess) return status_of(e);
    }

    e = gdr::launch_cp_scan(pl, ws, initial_state, p->num_v_heads, p->head_dim_k, p->head_dim_v, stream);
    if (e != hipSuccess) return status_of(e);

    gdr::ChunkArgs f = a;  // 3: outputs from the true start states; end states in place
    f.cu_seqlens = cu_seg; f.N = pl.P; f.h0 = Ss; f.ht = Ss;
    if ((e = gdr::launch_chunk(f, p->io_dtype, per_k, stream)) != hipSuccess) return status_of(e);
    if (final_state) e = gdr::launch_cp_final(pl, ws, final_state, p->num_v_heads, p->head_dim_k, p->head_dim_v, stream);
    return status_of(e);
}

}  // namespace

extern "C" {

gdr_status gdr_chunk_fwd(const gdr_problem* p, int32_t chunk_size, const void* q, const void* k, const void* v,
                         const float* g, const void* beta, const int32_t* cu_seqlens, const float* initial_state,
                         void* o, float* final_state, void* workspace, size_t workspace_bytes, void* hip_stream) {
    gdr_status st = check_chunk(p, chunk_size, q, k, v, g, beta, cu_seqlens, o);
    if (st != GDR_SUCCESS) return st;
    const size_t need = gdr_chunk_workspace_size(p, chunk_size);
    if (need > 0 && workspace && workspace_bytes < need) return GDR_ERROR_INVALID_VALUE;
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return GDR_ERROR_INVALID_VALUE;
    return chunk_fwd_impl(p, q, k, v, g, beta, cu_seqlens, initial_state, o, final_state, need > 0 ? workspace : nullptr,
                          hip_stream);
}

gdr_status gdr_chunk_fwd_noalloc(const gdr_problem* p, int32_t chunk_size, const void* q, const void* k,
                                 const void* v, const float* g, const void* beta, const int32_t* cu_seqlens,
                                 const float* initial_state, void* o, float* final_state, void* hip_stream) {
    gdr_status st = check_chunk(p, chunk_size, q, k, v, g, beta, cu_seqlens, o);
    if (st != GDR_SUCCESS) return st;
    const size_t need = gdr_chunk_workspace_size(p, chunk_size);
    if (need > (size_t)GDR_NOALLOC_SCRATCH_BYTES) return GDR_ERROR_SCRATCH_LIMIT;
    char* ws = nullptr;
    if (need > 0 && p->num_seqs > 0 && p->total_tokens > 0) {
        if ((st = check_device()) != GDR_SUCCESS) return st;
        if ((st = scratch_address(&ws)) != GDR_SUCCESS) return st;
    }
    return chunk_fwd_impl(p, q, k, v, g, beta, cu_seqlens, initial_state, o, final_state, ws, hip_stream);
}

}  // extern "C"
