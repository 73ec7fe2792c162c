// gemv1_residual.hip -- compiled batch-1 GEMV tile shapes, residual-add epilogue.
#include "gemv_kernels.h"

using namespace mak;

const void* mak_gemv1_fn_residual(int r, int j, int ks)
{
#define X(R, J) \
    if (ks == 1 && r == R && j == J) return reinterpret_cast<const void*>(&k_gemv1<R, J, EPI_RESIDUAL>);
    MAK_GEMV1_SHAPES(X)
#undef X
#define X(R, J) \
    if (ks == 2 && r == R && j == J) return reinterpret_cast<const void*>(&k_gemv1<R, J, EPI_RESIDUAL, 2>);
    MAK_GEMV1_KS_SHAPES(X)
#undef X
    return nullptr;
}
