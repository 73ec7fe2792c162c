// gemvn_swiglu.hip -- multi-column GEMV instantiations, SwiGLU epilogue.
#include "gemvn_kernels.h"

using namespace mak;

const void* mak_gemvn_fn_swiglu(int rr, int nc)
{
#define X(RR, NC) \
    if (rr == RR && nc == NC) return reinterpret_cast<const void*>(&k_gemvn<RR, NC, EPI_SWIGLU>);
    MAK_GEMVN_PAIR_SHAPES(X)
#undef X
    return nullptr;
}
