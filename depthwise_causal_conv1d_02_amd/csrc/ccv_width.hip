// ccv_width.hip — the kernels of one filter width.  The build compiles this
// file once per width with -DCCV_WIDTH=<W>, so the widths compile in parallel.
#include "ccv_dispatch.h"

#ifndef CCV_WIDTH
#error "compile with -DCCV_WIDTH=<filter width>"
#endif

#define CCV_CAT2(a, b) a##b
#define CCV_CAT(a, b) CCV_CAT2(a, b)

namespace ccv {

hipError_t CCV_CAT(fwd_dispatch_w, CCV_WIDTH)(const FwdArgs &a, int vec, int silu, int rows,
                                               hipStream_t s, int64_t *cap) {
    return fwd_dispatch<CCV_WIDTH>(a, vec, silu, rows, s, cap);
}

hipError_t CCV_CAT(bwd_dispatch_w, CCV_WIDTH)(const BwdArgs &a, int vec, int silu, int rows,
                                               hipStream_t s, int64_t *cap) {
    return bwd_dispatch<CCV_WIDTH>(a, vec, silu, rows, s, cap);
}

hipError_t CCV_CAT(update_dispatch_w, CCV_WIDTH)(const UpdArgs &a, int vec, int silu,
                                                  hipStream_t s) {
    return update_dispatch<CCV_WIDTH>(a, vec, silu, s);
}

}  // namespace ccv
