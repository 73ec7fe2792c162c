// gemv1_logits.hip -- compiled batch-1 GEMV tile shapes, fp32-logits + argmax epilogue.
#include "gemv_kernels.h"

using namespace mak;

const void* mak_gemv1_fn_logits(int r, int j, int ks)
{
#define X(R, J) \
    if (ks == 1 && r == R && j == J) return reinterpret_cast<const void*>(&k_gemv1<R, J, EPI_LOGITS>);
    MAK_GEMV1_SHAPES(X)
#undef X
    return nullptr;
}
