// One instantiation of the matrix-core split kernel, selected at compile
// time with -DTSW_W=<waves> -DTSW_R=<row groups> -DTSW_NB=<query blocks per
// wave>; the build compiles this file once per shape so the shapes build in
// parallel.
#include "tsw_mfma_impl.h"

#if !defined(TSW_W) || !defined(TSW_R) || !defined(TSW_NB)
#error "compile with -DTSW_W=... -DTSW_R=... -DTSW_NB=..."
#endif

#define TSW_LAUNCH_NAME2(w, r, nb) launch_mfma_##w##_##r##_##nb
#define TSW_LAUNCH_NAME(w, r, nb) TSW_LAUNCH_NAME2(w, r, nb)

namespace tsw {

hipError_t TSW_LAUNCH_NAME(TSW_W, TSW_R, TSW_NB)(int mode, const SplitArgs& a, int n_kv_heads, hipStream_t stream) {
    return mfma::launch<TSW_W, TSW_R, TSW_NB>(mode, a, n_kv_heads, stream);
}

}  // namespace tsw
