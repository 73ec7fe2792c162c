// gemv1_swiglu.hip -- compiled batch-1 GEMV tile shapes, SwiGLU epilogue.
#include "gemv_kernels.h"

using namespace mak;

const void* mak_gemv1_fn_swiglu(int r, int j, int ks)
{
#define X(R, J) \
    if (ks == 1 && r == R && j == J) return reinterpret_cast<const void*>(&k_gemv1<R, J, EPI_SWIGLU>);
    MAK_GEMV1_PAIR_SHAPES(X)
#undef X
#define X(R, J) \
    if (ks == 2 && r == R && j == J) return reinterpret_cast<const void*>(&k_gemv1<R, J, EPI_SWIGLU, 2>);
    MAK_GEMV1_KS_PAIR_SHAPES(X)
#undef X
    return nullptr;
}
