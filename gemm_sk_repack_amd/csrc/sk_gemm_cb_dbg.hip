// sk_gemm_cb_dbg.hip -- GEMM kernels for 4-bit codebook weights, with the test hook's debug exports.
#include "sk_gemm_kernel.h"

namespace sk {

KernelFn pick_kernel_cb_dbg(int pro, int xt, int gs, bool dot4, bool wide) {
    return pick_format<FMT_CB, true>(pro, xt, gs, dot4, wide);
}

}  // namespace sk
