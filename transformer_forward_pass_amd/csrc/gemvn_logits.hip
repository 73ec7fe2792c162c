// gemvn_logits.hip -- multi-column GEMV instantiations, fp32 logits + greedy argmax epilogue.
#include "gemvn_kernels.h"

using namespace mak;

const void* mak_gemvn_fn_logits(int rr, int nc)
{
#define X(RR, NC) \
    if (rr == RR && nc == NC) return reinterpret_cast<const void*>(&k_gemvn<RR, NC, EPI_LOGITS>);
    MAK_GEMVN_SHAPES(X)
#undef X
    return nullptr;
}
