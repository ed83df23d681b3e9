// sk_gemm_cb.hip -- GEMM kernels for 4-bit codebook weights, production instances (no debug exports).
#include "sk_gemm_kernel.h"

namespace sk {

KernelFn pick_kernel_cb(int pro, int xt, int gs, bool dot4, bool wide) {
    return pick_format<FMT_CB, false>(pro, xt, gs, dot4, wide);
}

}  // namespace sk
