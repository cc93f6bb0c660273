// Matrix-core decode kernel instances that take the step's new rows
// (pa_decode_write_attend): fp16 / bf16 caches with 16-token blocks, head_dim 64 / 128 / 256,
// groups of 4 or 8 query heads per KV head.
#include "decode_mfma.h"

namespace pa {

const void* decode_kernel_ptr_mfma_new(int dtype, int head_dim, int group) {
#define PA_CASE(DT, D, G) \
    if (dtype == DT && head_dim == D && group == G) \
        return (const void*)&decode_mfma_kernel<DT, D, G, true>;
#define PA_CASES(DT, D) PA_CASE(DT, D, 4) PA_CASE(DT, D, 8)
    PA_CASES(DT_F16, 64) PA_CASES(DT_F16, 128) PA_CASES(DT_F16, 256)
    PA_CASES(DT_BF16, 64) PA_CASES(DT_BF16, 128) PA_CASES(DT_BF16, 256)
#undef PA_CASES
#undef PA_CASE
    return nullptr;
}

}  // namespace pa
