// MFMA kernels (placeholder until the bf16 tiles land).
#include "launch.hpp"

namespace ssd {
bool mfma_supported(const ScanShape &) { return false; }
void launch_chunk_state_mfma(const ScanShape &, const void *, const void *, const float *,
                             const float *, float *, hipStream_t) {}
void launch_chunk_scan_mfma(const ScanShape &, const void *, const float *, const void *,
                            const void *, const float *, const float *, const float *, void *,
                            hipStream_t) {}
}  // namespace ssd
