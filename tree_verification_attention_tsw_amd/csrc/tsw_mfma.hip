// Shape table and dispatch of the matrix-core split kernel (the kernel
// itself is in tsw_mfma_impl.h, instantiated per shape by tsw_mfma_inst.hip).
#include "tsw_internal.h"

namespace tsw {

// (the shapes mfma_config_for picks; every one is built)
#define TSW_SHAPES(X) X(4, 1, 1) X(4, 1, 2) X(8, 2, 2) X(8, 4, 2) X(8, 4, 3) X(8, 8, 2) X(8, 8, 3)
#define TSW_DECLARE(w, r, nb) \
    hipError_t launch_mfma_##w##_##r##_##nb(int mode, const SplitArgs& a, int n_kv_heads, hipStream_t stream);
TSW_SHAPES(TSW_DECLARE)

bool mfma_config_for(int M, MfmaConfig* cfg) {
    // Blocks of 16 query rows per kv head, dealt to R row groups so that
    // every wave owns NB or NB-1 blocks.  From three blocks on, eight waves
    // (two per SIMD) share the work so one wave's exponentials overlap the
    // other's matrix products; the pairs on a SIMD own NB + (NB or NB-1)
    // blocks between them.
    const int nblk = (M + 15) / 16;
    if (nblk <= 0) return false;
    if (nblk <= 2) *cfg = {4, 1, nblk};
    else if (nblk <= 4) *cfg = {8, 2, 2};
    else if (nblk <= 8) *cfg = {8, 4, 2};
    else if (nblk <= 12) *cfg = {8, 4, 3};
    else if (nblk <= 16) *cfg = {8, 8, 2};
    else if (nblk <= 24) *cfg = {8, 8, 3};
    else return false;
    return true;
}

hipError_t launch_split_mfma(const MfmaConfig& cfg, int mode, const SplitArgs& a, int n_kv_heads,
                             hipStream_t stream) {
#define TSW_CASE(W_, R_, NB_)                                  \
    if (cfg.waves == W_ && cfg.rgroups == R_ && cfg.nb == NB_) \
        return launch_mfma_##W_##_##R_##_##NB_(mode, a, n_kv_heads, stream);
    TSW_SHAPES(TSW_CASE)
#undef TSW_CASE
    return hipErrorInvalidValue;
}

}  // namespace tsw
