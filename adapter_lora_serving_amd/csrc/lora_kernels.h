// Internal launch interface between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lora {

constexpr int kDtypeF32 = 0;
constexpr int kDtypeBF16 = 1;
constexpr int kMaxSlices = 8;

// Fused-output layout passed by value: slice i covers output columns
// [off[i], off[i+1]) and reads h columns [i*R, i*R + R).
struct SliceTable {
  int n;
  int off[kMaxSlices + 1];
};

hipError_t launch_build_addressing(const int32_t* token_slot, int T, int slots,
                                   int32_t* token_order, int32_t* slot_indptr,
                                   hipStream_t stream);

hipError_t launch_gather_shrink(int dtype, const int32_t* ids, int T, int64_t vocab,
                                const void* a, int slots, int R, const int32_t* token_order,
                                const int32_t* indptr, const int32_t* ranks, float* h,
                                hipStream_t stream);

hipError_t launch_shrink(int dtype, const void* x, int T, int in, const void* a, int slots,
                         int S, int R, const int32_t* token_order, const int32_t* indptr,
                         const int32_t* ranks, float* h, hipStream_t stream);

hipError_t launch_expand(int dtype, void* y, int T, const SliceTable& st, const float* h,
                         const void* b, int slots, int R, const int32_t* token_order,
                         const int32_t* indptr, const int32_t* ranks, const float* scalings,
                         hipStream_t stream);

}  // namespace lora
