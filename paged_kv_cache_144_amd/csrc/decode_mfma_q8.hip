// Matrix-core decode kernel instances for 8-bit caches (one fp16 scale per 32 values) with
// fp16 or bf16 queries: head_dim 64 / 128 / 256, groups of 4 or 8 query heads per KV head.
#include "decode_mfma.h"

namespace pa {

const void* decode_kernel_ptr_mfma_q8(int dtype, int head_dim, int group) {
#define PA_CASE(DT, D, G) \
    if (dtype == DT && head_dim == D && group == G) return (const void*)&decode_mfma_kernel<DT, D, G>;
#define PA_CASES(DT, D) PA_CASE(DT, D, 4) PA_CASE(DT, D, 8)
    PA_CASES(DT_Q8F16, 64) PA_CASES(DT_Q8F16, 128) PA_CASES(DT_Q8F16, 256)
    PA_CASES(DT_Q8BF16, 64) PA_CASES(DT_Q8BF16, 128) PA_CASES(DT_Q8BF16, 256)
#undef PA_CASES
#undef PA_CASE
    return nullptr;
}

}  // namespace pa
