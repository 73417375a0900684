// gather_shrink: the shrink of an embedding target.
//
// Follows the mstar lora.backend page, LoraBackend.gather_shrink: x @ A^T of
// a token id's one-hot is A's column for that id, so h[t, j] =
// a[slot(t), j, ids[t]] for j < rank; an id outside [0, vocab) contributes
// nothing. Every other entry of h is written 0. Each value is an exact
// widening of one element of A, so the result is bit-exact.
//
// Work mapping: one thread per (position p of token_order, rank column j),
// consecutive threads over j, so the h writes of one token are one
// contiguous run. The column of A for one (slot, id) has stride vocab, so
// each thread's read is its own 2- or 4-byte access: that is the nature of
// the gather and costs ~one 64-byte sector per element.
#include "lora_common.h"
#include "lora_kernels.h"

namespace lora {

template <typename E>
__global__ __launch_bounds__(256) void k_gather_shrink(const int32_t* __restrict__ ids, int T,
                                                       int64_t vocab, const void* __restrict__ a_,
                                                       int slots, int R,
                                                       const int32_t* __restrict__ token_order,
                                                       const int32_t* __restrict__ indptr,
                                                       const int32_t* __restrict__ ranks,
                                                       float* __restrict__ h) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= (int64_t)T * R) return;
  const int p = (int)(g / R);
  const int j = (int)(g - (int64_t)p * R);
  const int t = token_at(token_order, p, T);
  const int s = slot_of_position(indptr, slots, p);
  float v = 0.0f;
  if (s < slots) {
    const int r = clamp_rank(ranks[s], R);
    const int id = ids[t];
    if (j < r && id >= 0 && (int64_t)id < vocab) {
      const int64_t off = ((int64_t)s * R + j) * vocab + id;
      if constexpr (E::kBytes == 2) {
        const uint16_t* a = (const uint16_t*)a_;
        v = __uint_as_float((uint32_t)a[off] << 16);
      } else {
        v = ((const float*)a_)[off];
      }
    }
  }
  h[(int64_t)t * R + j] = v;
}

hipError_t launch_gather_shrink(int dtype, const int32_t* ids, int T, int64_t vocab,
                                const void* a, int slots, int R, const int32_t* token_order,
                                const int32_t* indptr, const int32_t* ranks, float* h,
                                hipStream_t stream) {
  const int64_t n = (int64_t)T * R;
  if (n == 0) return hipSuccess;
  const int block = 256;
  const int64_t grid = (n + block - 1) / block;
  if (dtype == kDtypeBF16)
    hipLaunchKernelGGL(k_gather_shrink<BF16>, dim3((unsigned)grid), dim3(block), 0, stream, ids,
                       T, vocab, a, slots, R, token_order, indptr, ranks, h);
  else
    hipLaunchKernelGGL(k_gather_shrink<F32>, dim3((unsigned)grid), dim3(block), 0, stream, ids, T,
                       vocab, a, slots, R, token_order, indptr, ranks, h);
  return hipGetLastError();
}

}  // namespace lora
