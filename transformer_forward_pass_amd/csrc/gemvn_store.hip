// gemvn_store.hip -- multi-column GEMV instantiations, bf16 store epilogue.
#include "gemvn_kernels.h"

using namespace mak;

const void* mak_gemvn_fn_store(int rr, int nc)
{
#define X(RR, NC) \
    if (rr == RR && nc == NC) return reinterpret_cast<const void*>(&k_gemvn<RR, NC, EPI_STORE>);
    MAK_GEMVN_SHAPES(X)
#undef X
    return nullptr;
}
