// Launch interface of the test decoder and the grouping kernel (k_misc.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qmoe {

hipError_t launch_dequant(int fmt, const uint8_t* packed, int64_t rows, int64_t kp, const int8_t* codebook,
                          float* out, hipStream_t s);
size_t group_lds(int E);
hipError_t launch_read(const void* src, size_t bytes, uint32_t* out, int blocks, hipStream_t s);
hipError_t launch_group(const int32_t* topk_idx, int n_slots, int E, int32_t* offsets, int32_t* sorted_slots,
                        int32_t* slot_pos, int* err_count, hipStream_t s);

}  // namespace qmoe
