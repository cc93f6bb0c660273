// Group-mode decode kernel instances for 8-bit caches (sliding-window decode batches):
// fp16 / bf16 activations, head_dim 64 / 128 / 256, group 1 / 2 / 4 / 8.
#include "decode_group.h"

namespace pa {

const void* decode_group_ptr_q8(int dtype, int head_dim, int group) {
#define PA_CASE(DT, D, G) \
    if (dtype == DT && head_dim == D && group == G) \
        return (const void*)&decode_group_kernel<DT, D, G, false>;
#define PA_CASES(DT, D) PA_CASE(DT, D, 1) PA_CASE(DT, D, 2) PA_CASE(DT, D, 4) PA_CASE(DT, D, 8)
    PA_CASES(DT_Q8F16, 64) PA_CASES(DT_Q8F16, 128) PA_CASES(DT_Q8F16, 256)
    PA_CASES(DT_Q8BF16, 64) PA_CASES(DT_Q8BF16, 128) PA_CASES(DT_Q8BF16, 256)
#undef PA_CASES
#undef PA_CASE
    return nullptr;
}

}  // namespace pa
