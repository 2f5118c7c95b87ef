// Shape table and dispatch of the matrix-core split kernel (the kernel
// itself is in tsw_mfma_impl.h, instantiated per shape by tsw_mfma_inst.hip).
#include "tsw_internal.h"

namespace tsw {

#define TSW_SHAPES(X) X(1, 1) X(1, 2) X(1, 3) X(1, 4) X(2, 3) X(2, 4) X(2, 5) X(4, 3) X(4, 4) X(4, 5)
#define TSW_DECLARE(r, nb) \
    hipError_t launch_mfma_##r##_##nb(bool gather, const SplitArgs& a, int n_kv_heads, hipStream_t stream);
TSW_SHAPES(TSW_DECLARE)

bool mfma_config_for(int M, MfmaConfig* cfg) {
    // Blocks of 16 query rows per kv head, dealt to R row groups so that
    // every wave owns NB or NB-1 blocks.
    const int nblk = (M + 15) / 16;
    if (nblk <= 0) return false;
    if (nblk <= 4) *cfg = {4, 1, nblk};
    else if (nblk <= 6) *cfg = {4, 2, 3};
    else if (nblk <= 8) *cfg = {4, 2, 4};
    else if (nblk <= 10) *cfg = {4, 2, 5};
    else if (nblk <= 12) *cfg = {4, 4, 3};
    else if (nblk <= 16) *cfg = {4, 4, 4};
    else if (nblk <= 20) *cfg = {4, 4, 5};
    else return false;
    return true;
}

hipError_t launch_split_mfma(const MfmaConfig& cfg, bool gather, const SplitArgs& a, int n_kv_heads,
                             hipStream_t stream) {
#define TSW_CASE(R_, NB_) \
    if (cfg.rgroups == R_ && cfg.nb == NB_) return launch_mfma_##R_##_##NB_(gather, a, n_kv_heads, stream);
    TSW_SHAPES(TSW_CASE)
#undef TSW_CASE
    return hipErrorInvalidValue;
}

}  // namespace tsw
