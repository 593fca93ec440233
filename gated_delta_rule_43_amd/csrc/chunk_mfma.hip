// chunk_mfma.hip -- bf16-input chunked KDA forward on the matrix cores (gfx950).
#include "kda_common.hpp"

namespace kda {

bool chunk_mfma_supported(int K, int V, int C) { (void)K; (void)V; (void)C; return false; }

hipError_t launch_chunk_mfma(const void *, const void *, const void *, const void *,
                             const void *, const float *, void *, float *, const int32_t *,
                             int, int, int, int, bool, hipStream_t) {
    return hipErrorInvalidValue;
}

}  // namespace kda
