// Chunk-row MFMA kernel instances for bf16 caches: head_dim 64 / 128 / 256, group 1 / 2 / 4 / 8.
#include "chunk_impl.h"

namespace pa {

const void* chunk_kernel_ptr_bf16(int head_dim, int group) {
#define PA_CASE(D, G) \
    if (head_dim == D && group == G) return (const void*)&chunk_kernel<DT_BF16, D, G>;
#define PA_CASES(D) PA_CASE(D, 1) PA_CASE(D, 2) PA_CASE(D, 4) PA_CASE(D, 8)
    PA_CASES(64) PA_CASES(128) PA_CASES(256)
#undef PA_CASES
#undef PA_CASE
    return nullptr;
}

}  // namespace pa
