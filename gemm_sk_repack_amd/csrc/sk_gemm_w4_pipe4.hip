// sk_gemm_w4_pipe4.hip -- GEMM kernels for 4-bit weights without a prologue
// with a 4-slot register pipeline (production instances).
#include "sk_gemm_kernel.h"

namespace sk {

KernelFn pick_kernel_w4_pipe4(int xt, int gs, bool dot4, bool wide) { return pick_pipe<4>(xt, gs, dot4, wide); }

}  // namespace sk
