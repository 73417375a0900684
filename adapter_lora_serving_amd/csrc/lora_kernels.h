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

// Column chunks of the fused output handed to decode work items: chunk k
// covers columns [c0[k], c1[k]) of slice slice[k].
constexpr int kMaxChunks = 64;
struct ChunkTable {
  int n;
  int per_slice[kMaxSlices];   // chunks of each slice
  int first[kMaxSlices];       // index of each slice's first chunk
  int slice[kMaxChunks];
  int c0[kMaxChunks];
  int c1[kMaxChunks];
};

// Workspace bytes for the two-pass path of the addressing (0: one pass).
size_t addressing_workspace_bytes(int64_t T, int slots);
hipError_t launch_build_addressing(const int32_t* token_slot, int T, int slots,
                                   int32_t* token_order, int32_t* slot_indptr, void* ws,
                                   size_t ws_bytes, hipStream_t stream);

// Addressing of an expert-sorted batch (rows grouped by expert, bounds in
// offs[0..E]) over the composite key expert * slots + slot; the workspace
// holds the keys, then the addressing's own workspace.
size_t expert_addressing_workspace_bytes(int64_t rows, int E, int slots);
hipError_t launch_build_addressing_experts(const int32_t* row_slot, const int32_t* offs, int E,
                                           int rows, int slots, int32_t* token_order,
                                           int32_t* slot_indptr, void* ws, size_t ws_bytes,
                                           hipStream_t stream);

hipError_t launch_gather_shrink(int dtype, const int32_t* ids, int T, int64_t vocab,
                                const void* a, int slots, int R, const int32_t* token_order,
                                const int32_t* indptr, const int32_t* ranks, float* h,
                                hipStream_t stream);

// VALU (BGMV) shrink / expand; segments longer than max_seg are skipped
// (the SGMV kernels take them).
constexpr int kNoMaxSeg = 0x7fffffff;
hipError_t launch_shrink(int dtype, const void* x, int T, int in, const void* a, int slots,
                         int S, int R, const int32_t* token_order, const int32_t* indptr,
                         const int32_t* ranks, float* h, int max_seg, hipStream_t stream);

hipError_t launch_expand(int dtype, void* y, int T, const SliceTable& st, const float* h,
                         const void* b, int slots, int R, const int32_t* token_order,
                         const int32_t* indptr, const int32_t* ranks, const float* scalings,
                         int max_seg, hipStream_t stream);

// SGMV (bf16 MFMA) shrink / expand over the segments longer than min_len
// tokens (kLongSegment next to the decode tiles; 0 takes every segment).
constexpr int kLongSegment = 16;
bool sgmv_supported(int dtype, const SliceTable& st, int R, int T, int in);
// kparts > 1 splits K: the parts go to `parts` (kparts * T * S * R floats)
// and are summed into h in part order.
int sgmv_kparts(int in);
// K parts to launch for a batch of T tokens over `slots`, S slices of
// rank R (at most sgmv_kparts(in), which sizes the workspace).
int sgmv_kparts_for(int T, int in, int slots, int S, int R);
// Rank tiles of the shrink kernel launched for such a batch.
int sgmv_shrink_rt(int T, int slots, int S, int R);
hipError_t launch_sgmv_shrink(const void* x, int T, int in, const void* a, int slots, int S,
                              int R, const int32_t* order, const int32_t* indptr,
                              const int32_t* ranks, float* h, float* parts, int kparts,
                              int min_len, hipStream_t stream);
hipError_t launch_sgmv_expand(void* y, int T, const SliceTable& st, const float* h, const void* b,
                              int slots, int R, const int32_t* order, const int32_t* indptr,
                              const int32_t* ranks, const float* scalings, int min_len,
                              hipStream_t stream);

// Fused shrink + expand (bf16, MFMA). fused_supported() tells whether the
// shapes qualify (bf16, every slice width a multiple of 16, R <= 256, every
// buffer below 2 GiB).
bool fused_supported(int dtype, const SliceTable& st, int R, int T, int in);
// Workspace layout of lora_apply_linear: [counters | body]. The counters (a
// {count, base} int pair per (slot, chunk index), a fixed 4 MiB region) are
// used only by the fused kernel and stay consistent across calls of any
// shape. The body holds the fused path's fp32 partial h tiles or the other
// path's h.
size_t counter_bytes(int slots, int S);
size_t fused_partial_bytes(int slots, int S, int R, int in);
// Standalone bf16 shrink / expand for segments of at most 16 tokens on the
// decode tiles (MFMA): lora_shrink writes h's columns below the rank of those
// tokens (the zeros come from launch_shrink with max_seg 0), lora_expand
// reads h from memory. Supported where fused_supported() holds.
hipError_t launch_decode_shrink(const void* x, int T, int in, const void* a, int slots, int S,
                                int R, const int32_t* token_order, const int32_t* indptr,
                                const int32_t* ranks, float* h, hipStream_t stream);
hipError_t launch_decode_expand(void* y, int T, const SliceTable& st, const float* h,
                                const void* b, int slots, int R, const int32_t* token_order,
                                const int32_t* indptr, const int32_t* ranks,
                                const float* scalings, hipStream_t stream);

// The fused kernel for a small batch: decode pieces for segments of at most
// 16 tokens, 16-token prefill items over every column for longer ones.
// With token_slot (the one-launch form, where fused_from_slots_supported
// holds), the kernel builds the addressing itself: order_out / indptr_out
// receive what launch_build_addressing writes, and token_order / indptr are
// not read.
hipError_t launch_apply_fused(const void* x, void* y, int T, int in, const SliceTable& st,
                              const void* a, const void* b, int slots, int R,
                              const int32_t* token_order, const int32_t* indptr,
                              const int32_t* ranks, const float* scalings, void* workspace,
                              hipStream_t stream, const int32_t* token_slot = nullptr,
                              int32_t* order_out = nullptr, int32_t* indptr_out = nullptr,
                              const int32_t* expert_offs = nullptr, int E = 0, int eslots = 0);
bool fused_from_slots_supported(int T, int slots);
// With expert_offs as well, token_slot holds each row's slot within its
// expert and `slots` = E * eslots pool entries (the expert addressing).
bool fused_from_experts_supported(int T, int E, int eslots);

// The base projection y = x @ W^T of a fused linear layer (W [out, in], the
// shards stacked along out) with the LoRA delta of h (fp32 [T, S*R], from
// the shrink; nullptr: no delta) added before y is stored. Supported: bf16,
// every slice width a multiple of 256, `in` a multiple of 8, every buffer
// below 2 GiB.
bool linear_lora_supported(int dtype, const SliceTable& st, int R, int T, int in);
hipError_t launch_linear_lora(const void* x, const void* w, void* y, int T, int in,
                              const SliceTable& st, const float* h, const void* b, int slots,
                              int R, const int32_t* token_order, const int32_t* indptr,
                              const int32_t* ranks, const float* scalings, hipStream_t stream);

}  // namespace lora
