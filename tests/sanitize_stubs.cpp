// Stand-ins for the device half of libpa.so, linked only into the CPU sanitizer build of the
// host code (tests/test_sanitizers.py).  The host half - argument checks, kernel selection,
// workspace layout, the block ledger - is compiled unchanged with AddressSanitizer and
// UndefinedBehaviorSanitizer; everything it would ask of the HIP runtime or of a kernel is
// answered here by a pretend device: 256 compute units, two workgroups of every kernel
// resident per compute unit, and launches that succeed without running anything.  Each
// launch is counted, so a driver can check that a refused call launched nothing.
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace {
int g_launches = 0;
const char g_kernel = 0;   // any non-null address stands for "this instance exists"

bool group_ok(int group) { return group == 1 || group == 2 || group == 4 || group == 8; }
}  // namespace

extern "C" int pa_stub_launches() { return g_launches; }

hipError_t hipGetDevice(int* dev) {
    *dev = 0;
    return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int) {
    *value = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
    return hipSuccess;
}

hipError_t hipOccupancyMaxActiveBlocksPerMultiprocessor(int* groups, const void*, int, size_t) {
    *groups = 2;
    return hipSuccess;
}

hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }

hipError_t hipGetLastError() { return hipSuccess; }

// every pointer counts as device memory
hipError_t hipPointerGetAttributes(hipPointerAttribute_t* attr, const void* p) {
    *attr = hipPointerAttribute_t{};
    attr->type = hipMemoryTypeDevice;
    attr->devicePointer = const_cast<void*>(p);
    return hipSuccess;
}

namespace pa {

// the pretend device's fixed workspace of pa_decode_noalloc: an address the stubbed
// launches never dereference
pa_status noalloc_scratch(void** out, size_t* bytes) {
    *out = reinterpret_cast<void*>(uintptr_t(1) << 40);
    *bytes = PA_NOALLOC_SCRATCH_BYTES;
    return PA_OK;
}

const void* decode_kernel_ptr(int, int, int group, int, bool) {
    return group_ok(group) ? &g_kernel : nullptr;
}
const void* decode_group_ptr(int, int, int group, bool) {
    return group_ok(group) ? &g_kernel : nullptr;
}
bool decode_uses_mfma(int dtype, int group, int block_size) {
    return block_size == kBlock && dtype != PA_F32 && (group == 4 || group == 8);
}
const void* chunk_kernel_ptr(int dtype, int, int group, int block_size) {
    return (dtype == PA_F16 || dtype == PA_BF16) && block_size == kBlock && group_ok(group)
               ? &g_kernel
               : nullptr;
}

hipError_t launch_write_kv(const void*, const void*, const int64_t*, int32_t, void*, void*,
                           int32_t, int32_t, int32_t, int32_t, int32_t, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_write_kv_q8(const void*, const void*, const int64_t*, int32_t, void*, void*,
                              int32_t, int32_t, int32_t, int, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_copy_blocks(void*, void*, const int32_t*, int32_t, int32_t, int32_t, int32_t,
                              int32_t, int32_t, int32_t*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_swap_blocks(const void*, const void*, void*, void*, const int32_t*, int32_t,
                              int32_t, int32_t, int32_t, int32_t, int32_t*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_plan(const DecodeArgs&, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_stream_read(const void*, size_t, uint32_t*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_decode(const DecodeArgs&, int, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_merge(const DecodeArgs&, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_chunk(const DecodeArgs&, int, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}

}  // namespace pa
