// Paged decode kernel instances for f32 caches that take the step's new rows
// (pa_decode_write_attend): head_dim 64 / 128 / 256, group 1 / 2 / 4 / 8.
#include "decode_impl.h"

namespace pa {

const void* decode_kernel_ptr_f32_new(int head_dim, int group) {
#define PA_CASE(D, G) \
    if (head_dim == D && group == G) return (const void*)&decode_kernel<DT_F32, D, G, kBlock, true>;
#define PA_CASES(D) PA_CASE(D, 1) PA_CASE(D, 2) PA_CASE(D, 4) PA_CASE(D, 8)
    PA_CASES(64) PA_CASES(128) PA_CASES(256)
#undef PA_CASES
#undef PA_CASE
    return nullptr;
}

}  // namespace pa
