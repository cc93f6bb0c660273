// Group-mode decode kernel instances for f16 caches (sliding-window decode batches):
// head_dim 64 / 128 / 256, group 1 / 2 / 4 / 8, with and without the step's new rows.
#include "decode_group.h"

namespace pa {

const void* decode_group_ptr_f16(int head_dim, int group, bool new_rows) {
#define PA_CASE(D, G) \
    if (head_dim == D && group == G) \
        return new_rows ? (const void*)&decode_group_kernel<DT_F16, D, G, true> \
                        : (const void*)&decode_group_kernel<DT_F16, D, G, false>;
#define PA_CASES(D) PA_CASE(D, 1) PA_CASE(D, 2) PA_CASE(D, 4) PA_CASE(D, 8)
    PA_CASES(64) PA_CASES(128) PA_CASES(256)
#undef PA_CASES
#undef PA_CASE
    return nullptr;
}

}  // namespace pa
