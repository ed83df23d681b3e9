// sk_gemm_w6_dbg.hip -- GEMM kernels for 6-bit weights, with the test hook's debug exports.
#include "sk_gemm_kernel.h"

namespace sk {

KernelFn pick_kernel_w6_dbg(int pro, int xt, int gs, bool dot4, bool wide) {
    return pick_format<FMT_W6, true>(pro, xt, gs, dot4, wide);
}

}  // namespace sk
