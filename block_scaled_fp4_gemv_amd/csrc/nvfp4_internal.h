// Library-internal declarations shared by the HIP sources of libnvfp4gemv.so
// (not exported from the shared library).
#ifndef NVFP4_INTERNAL_H
#define NVFP4_INTERNAL_H

// Records the hipError_t that nvfp4_last_hip_error reports for this thread.
__attribute__((visibility("hidden"))) void nvfp4_record_hip_error(int error);

#endif
