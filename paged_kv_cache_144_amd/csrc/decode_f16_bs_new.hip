// Paged decode kernel instances for f16 caches with 8- and 32-token blocks that take the
// step's new rows (pa_decode_write_attend): head_dim 64 / 128 / 256, group 1 / 2 / 4 / 8.
#include "decode_impl.h"

namespace pa {

const void* decode_kernel_ptr_f16_bs_new(int head_dim, int group, int block_size) {
#define PA_CASE(D, G, BS) \
    if (head_dim == D && group == G && block_size == BS) \
        return (const void*)&decode_kernel<DT_F16, D, G, BS, true>;
#define PA_CASES(D, BS) PA_CASE(D, 1, BS) PA_CASE(D, 2, BS) PA_CASE(D, 4, BS) PA_CASE(D, 8, BS)
    PA_CASES(64, 8) PA_CASES(128, 8) PA_CASES(256, 8)
    PA_CASES(64, 32) PA_CASES(128, 32) PA_CASES(256, 32)
#undef PA_CASES
#undef PA_CASE
    return nullptr;
}

}  // namespace pa
