// Chunked path (placeholder while the kernels are written).
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

ChunkWorkspaceLayout chunk_workspace_layout(int64_t T, int32_t N, int32_t HV, int32_t K, int32_t V, int io_bytes,
                                            bool per_k) {
    ChunkWorkspaceLayout L{};
    const int64_t max_chunks = T / 64 + N;
    size_t off = 0;
    L.chunk_seq = off; off = align256(off + sizeof(int32_t) * (size_t)max_chunks);
    L.chunk_first = off; off = align256(off + sizeof(int32_t) * (size_t)(N + 1));
    L.gcum = off; off = align256(off + sizeof(float) * (size_t)T * HV * (per_k ? K : 1));
    L.w = off; off = align256(off + (size_t)io_bytes * T * HV * K);
    L.u = off; off = align256(off + (size_t)io_bytes * T * HV * V);
    L.vnew = off; off = align256(off + (size_t)io_bytes * T * HV * V);
    L.hc = off; off = align256(off + (size_t)io_bytes * max_chunks * HV * V * K);
    L.total = off;
    return L;
}

hipError_t launch_chunk(const ChunkArgs&, int, bool, hipStream_t) { return hipErrorNotSupported; }

}  // namespace gdr
