// sk_gemm_w6.hip -- GEMM kernels for 6-bit weights, production instances (no debug exports).
#include "sk_gemm_kernel.h"

namespace sk {

KernelFn pick_kernel_w6(int pro, int xt, int gs, bool dot4, bool wide) {
    return pick_format<FMT_W6, false>(pro, xt, gs, dot4, wide);
}

}  // namespace sk
