// C ABI of the batched multi-LoRA delta: argument validation on the host
// (scalars, pointers and alignment only; device data is never read here) and
// kernel launches on the caller's stream. Nothing is allocated and nothing
// synchronises, so every entry point can be recorded in a hipGraph.
#include "lora_mi355x.h"

#include <hip/hip_runtime.h>

#include "lora_kernels.h"

namespace {

using lora::SliceTable;

constexpr int64_t kMaxI32 = 0x7fffffff;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int dtype) { return dtype == LORA_BF16 ? 2 : 4; }
int vec_elems(int dtype) { return 16 / elem_bytes(dtype); }

lora_status check_common(int dtype, int64_t T, int32_t slots, int32_t R) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_UNSUPPORTED;
  if (T < 0 || T > kMaxI32) return LORA_ERR_INVALID_ARG;
  if (slots < 1 || slots > 8192) return LORA_ERR_UNSUPPORTED;
  if (R < 1 || R > 256) return LORA_ERR_UNSUPPORTED;
  if (R % vec_elems(dtype) != 0) return LORA_ERR_ALIGNMENT;
  return LORA_OK;
}

lora_status check_addr(const int32_t* token_order, const int32_t* slot_indptr,
                       const int32_t* ranks) {
  if (!token_order || !slot_indptr || !ranks) return LORA_ERR_INVALID_ARG;
  return LORA_OK;
}

lora_status make_slices(int dtype, const int64_t* out_slices, int32_t num_slices, int32_t R,
                        SliceTable* st) {
  if (num_slices < 1 || num_slices > lora::kMaxSlices) return LORA_ERR_UNSUPPORTED;
  if (!out_slices) return LORA_ERR_INVALID_ARG;
  if ((int64_t)num_slices * R > 1024) return LORA_ERR_UNSUPPORTED;
  int64_t off = 0;
  st->n = num_slices;
  st->off[0] = 0;
  for (int i = 0; i < num_slices; ++i) {
    const int64_t w = out_slices[i];
    if (w < 1) return LORA_ERR_INVALID_ARG;
    if (w % vec_elems(dtype) != 0) return LORA_ERR_ALIGNMENT;
    off += w;
    if (off > (1 << 30)) return LORA_ERR_INVALID_ARG;
    st->off[i + 1] = (int)off;
  }
  return LORA_OK;
}

lora_status hip_status(hipError_t e) { return e == hipSuccess ? LORA_OK : LORA_ERR_HIP; }

size_t ws_h_bytes(int64_t T, int32_t S, int32_t R) {
  return (((size_t)T * S * R * sizeof(float)) + 255) & ~(size_t)255;
}

size_t partial_bytes(int32_t slots, int32_t S, int32_t R, int64_t in) {
  return (lora::fused_partial_bytes(slots, S, R, (int)in) + 255) & ~(size_t)255;
}

// Batches of at least this many tokens (bf16) run every segment on the SGMV
// tiles; smaller ones use the fused kernel (apply) or the decode tiles for
// segments of at most kLongSegment tokens (shrink, expand).
constexpr int64_t kLargeBatch = 1024;

// Whether lora_shrink's products run on the MFMA kernels (the shapes only
// matter, not the output widths: a slice table of num_slices 16-wide slices
// stands in for them).
bool shrink_on_mfma(int dtype, int64_t T, int64_t in, int32_t S, int32_t R) {
  SliceTable st;
  st.n = S;
  for (int i = 0; i <= S; ++i) st.off[i] = 16 * i;
  return lora::sgmv_supported(dtype, st, R, (int)T, (int)in) &&
         lora::fused_supported(dtype, st, R, (int)T, (int)in);
}

// Kernel family of lora_apply_linear for these shapes (LORA_PATH_*).
int apply_path(int dtype, int64_t T, int64_t in, const SliceTable& st, int32_t R) {
  if (!lora::fused_supported(dtype, st, R, (int)T, (int)in)) return LORA_PATH_VALU;
  if (T < kLargeBatch) return LORA_PATH_FUSED;
  return lora::sgmv_supported(dtype, st, R, (int)T, (int)in) ? LORA_PATH_SEGMENT
                                                              : LORA_PATH_VALU;
}

}  // namespace

extern "C" {

const char* lora_status_string(int status) {
  switch (status) {
    case LORA_OK: return "ok";
    case LORA_ERR_INVALID_ARG: return "invalid argument";
    case LORA_ERR_UNSUPPORTED: return "unsupported dtype or size";
    case LORA_ERR_ALIGNMENT: return "pointer or row width not 16-byte aligned";
    case LORA_ERR_WORKSPACE: return "workspace missing or too small";
    case LORA_ERR_HIP: return "HIP launch failed";
    case LORA_ERR_SCRATCH_LIMIT:
      return "sizes need more than the static scratch array of lora_apply_linear_noalloc";
    default: return "unknown status";
  }
}

const char* lora_version(void) { return "lora_mi355x 0.1 (gfx950)"; }

size_t lora_build_addressing_workspace_bytes(int64_t T, int32_t slots) {
  if (T < 0 || T > kMaxI32 || slots < 1 || slots > 8192) return 0;
  return lora::addressing_workspace_bytes(T, slots);
}

lora_status lora_build_addressing(const int32_t* token_slot, int64_t T, int32_t slots,
                                  int32_t* token_order, int32_t* slot_indptr, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (T < 0 || T > kMaxI32) return LORA_ERR_INVALID_ARG;
  if (slots < 1 || slots > 8192) return LORA_ERR_UNSUPPORTED;
  if (!slot_indptr) return LORA_ERR_INVALID_ARG;
  if (T > 0 && (!token_slot || !token_order)) return LORA_ERR_INVALID_ARG;
  if (workspace) {
    if (workspace_bytes < lora_build_addressing_workspace_bytes(T, slots))
      return LORA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return LORA_ERR_ALIGNMENT;
  }
  return hip_status(lora::launch_build_addressing(token_slot, (int)T, slots, token_order,
                                                  slot_indptr, workspace, workspace_bytes,
                                                  (hipStream_t)stream));
}

size_t lora_build_addressing_experts_workspace_bytes(int64_t rows, int32_t num_experts,
                                                     int32_t slots) {
  if (rows < 0 || rows > kMaxI32 || num_experts < 1 || slots < 1 ||
      (int64_t)num_experts * slots > 8192)
    return 0;
  return lora::expert_addressing_workspace_bytes(rows, num_experts, slots);
}

lora_status lora_build_addressing_experts(const int32_t* row_slot, const int32_t* expert_offsets,
                                          int32_t num_experts, int64_t rows, int32_t slots,
                                          int32_t* token_order, int32_t* slot_indptr,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  if (rows < 0 || rows > kMaxI32) return LORA_ERR_INVALID_ARG;
  if (num_experts < 1 || slots < 1 || (int64_t)num_experts * slots > 8192)
    return LORA_ERR_UNSUPPORTED;
  if (!slot_indptr || !expert_offsets) return LORA_ERR_INVALID_ARG;
  if (rows > 0 && (!row_slot || !token_order)) return LORA_ERR_INVALID_ARG;
  if (!workspace ||
      workspace_bytes < lora_build_addressing_experts_workspace_bytes(rows, num_experts, slots))
    return LORA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LORA_ERR_ALIGNMENT;
  return hip_status(lora::launch_build_addressing_experts(
      row_slot, expert_offsets, num_experts, (int)rows, slots, token_order, slot_indptr,
      workspace, workspace_bytes, (hipStream_t)stream));
}

size_t lora_shrink_workspace_bytes(int64_t T, int64_t in_features, int32_t num_slices,
                                   int32_t R) {
  if (T < 0 || T > kMaxI32 || num_slices < 1 || num_slices > lora::kMaxSlices || R < 1 ||
      R > 256 || in_features < 1 || in_features > kMaxI32)
    return 0;
  const int kp = lora::sgmv_kparts((int)in_features);
  return kp > 1 ? ws_h_bytes(T, num_slices, R) * kp : 0;
}

}  // extern "C"

namespace {

// lora_shrink's body. zeros: whether the columns of h that no expand reads
// (past each slot's rank, rows of dead tokens and rank-0 slots) are written
// as zeros, as lora_shrink promises its callers; an internal h that only
// the fused GEMM's epilogue reads (below each slot's rank) skips them.
lora_status shrink_impl(int dtype, const void* x, int64_t T, int64_t in_features, const void* a,
                        int32_t slots, int32_t num_slices, int32_t R,
                        const int32_t* token_order, const int32_t* slot_indptr,
                        const int32_t* ranks, float* h, void* workspace,
                        size_t workspace_bytes, void* stream, bool zeros) {
  lora_status st = check_common(dtype, T, slots, R);
  if (st != LORA_OK) return st;
  if (num_slices < 1 || num_slices > lora::kMaxSlices) return LORA_ERR_UNSUPPORTED;
  if ((int64_t)num_slices * R > 1024) return LORA_ERR_UNSUPPORTED;
  if (in_features < 1 || in_features > kMaxI32) return LORA_ERR_INVALID_ARG;
  if (T == 0) return LORA_OK;
  if (!x || !a || !h) return LORA_ERR_INVALID_ARG;
  if ((st = check_addr(token_order, slot_indptr, ranks)) != LORA_OK) return st;
  if (!aligned16(x) || !aligned16(a) || !aligned16(h)) return LORA_ERR_ALIGNMENT;
  if (in_features % vec_elems(dtype) != 0) return LORA_ERR_ALIGNMENT;
  // K parts of the long segments when the caller lends a workspace
  int kparts = 1;
  if (workspace) {
    const size_t need = lora_shrink_workspace_bytes(T, in_features, num_slices, R);
    if (workspace_bytes < need) return LORA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LORA_ERR_ALIGNMENT;
    if (need > 0) kparts = lora::sgmv_kparts_for((int)T, (int)in_features, slots, num_slices, R);
  }
  // per-segment choice on the device. bf16: in a small batch, segments of at
  // most kLongSegment tokens on the decode tiles and longer ones on the SGMV
  // tiles, in a large batch every segment on the SGMV tiles, and the VALU
  // kernel writes only the zeros; otherwise (fp32, or sizes the MFMA kernels
  // do not take) the VALU kernel computes every segment.
  const bool mfma = shrink_on_mfma(dtype, T, in_features, num_slices, R);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (!mfma || zeros)
    e = lora::launch_shrink(dtype, x, (int)T, (int)in_features, a, slots, num_slices, R,
                            token_order, slot_indptr, ranks, h, mfma ? 0 : lora::kNoMaxSeg, s);
  const bool large = T >= kLargeBatch;
  if (e == hipSuccess && mfma && !large)
    e = lora::launch_decode_shrink(x, (int)T, (int)in_features, a, slots, num_slices, R,
                                   token_order, slot_indptr, ranks, h, s);
  if (e == hipSuccess && mfma)
    e = lora::launch_sgmv_shrink(x, (int)T, (int)in_features, a, slots, num_slices, R,
                                 token_order, slot_indptr, ranks, h,
                                 kparts > 1 ? static_cast<float*>(workspace) : nullptr, kparts,
                                 large ? 0 : lora::kLongSegment, s);
  return hip_status(e);
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// The kernels of lora_apply_linear once its arguments are checked.
lora_status run_apply(int dtype, const void* x, void* y, int64_t T, int64_t in_features,
                      const SliceTable& tab, int32_t num_slices, const void* a, const void* b,
                      int32_t slots, int32_t R, const int32_t* token_order,
                      const int32_t* slot_indptr, const int32_t* ranks, const float* scalings,
                      void* workspace, hipStream_t s) {
  float* h = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                      lora::counter_bytes(slots, num_slices) +
                                      partial_bytes(slots, num_slices, R, in_features));
  const int path = apply_path(dtype, T, in_features, tab, R);
  if (path != LORA_PATH_VALU) {
    // The host picks the kernel family from the shapes only (fixed per
    // captured graph): small batches run everything in the fused kernel
    // (decode pieces for segments of at most 16 tokens, 16-token prefill
    // items for longer ones); larger batches run every segment through the
    // SGMV shrink and expand, which write and read their h in the
    // workspace. There the few-token segments are pure weight streaming,
    // which the SGMV tiles' shared, deeper loads serve better than the
    // decode pieces.
    hipError_t e;
    if (path == LORA_PATH_FUSED) {
      e = lora::launch_apply_fused(x, y, (int)T, (int)in_features, tab, a, b, slots, R,
                                   token_order, slot_indptr, ranks, scalings, workspace, s);
    } else {
      const int kp = lora::sgmv_kparts_for((int)T, (int)in_features, slots, num_slices, R);
      float* parts = h + ws_h_bytes(T, num_slices, R) / sizeof(float);
      e = lora::launch_sgmv_shrink(x, (int)T, (int)in_features, a, slots, num_slices, R,
                                   token_order, slot_indptr, ranks, h, parts, kp, 0, s);
      if (e == hipSuccess)
        e = lora::launch_sgmv_expand(y, (int)T, tab, h, b, slots, R, token_order, slot_indptr,
                                     ranks, scalings, 0, s);
    }
    return hip_status(e);
  }
  hipError_t e = lora::launch_shrink(dtype, x, (int)T, (int)in_features, a, slots, num_slices, R,
                                     token_order, slot_indptr, ranks, h, lora::kNoMaxSeg, s);
  if (e != hipSuccess) return LORA_ERR_HIP;
  return hip_status(lora::launch_expand(dtype, y, (int)T, tab, h, b, slots, R, token_order,
                                        slot_indptr, ranks, scalings, lora::kNoMaxSeg, s));
}

}  // namespace

extern "C" {

lora_status lora_shrink(int dtype, const void* x, int64_t T, int64_t in_features, const void* a,
                        int32_t slots, int32_t num_slices, int32_t R,
                        const int32_t* token_order, const int32_t* slot_indptr,
                        const int32_t* ranks, float* h, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return shrink_impl(dtype, x, T, in_features, a, slots, num_slices, R, token_order, slot_indptr,
                     ranks, h, workspace, workspace_bytes, stream, true);
}

lora_status lora_gather_shrink(int dtype, const int32_t* ids, int64_t T, int64_t vocab,
                               const void* a, int32_t slots, int32_t R,
                               const int32_t* token_order, const int32_t* slot_indptr,
                               const int32_t* ranks, float* h, void* stream) {
  lora_status st = check_common(dtype, T, slots, R);
  if (st != LORA_OK) return st;
  if (vocab < 1 || vocab > kMaxI32) return LORA_ERR_INVALID_ARG;
  if (T == 0) return LORA_OK;
  if (!ids || !a || !h) return LORA_ERR_INVALID_ARG;
  if ((st = check_addr(token_order, slot_indptr, ranks)) != LORA_OK) return st;
  if (!aligned16(a) || !aligned16(h)) return LORA_ERR_ALIGNMENT;
  return hip_status(lora::launch_gather_shrink(dtype, ids, (int)T, vocab, a, slots, R,
                                               token_order, slot_indptr, ranks, h,
                                               (hipStream_t)stream));
}

lora_status lora_expand(int dtype, void* y, int64_t T, const int64_t* out_slices,
                        int32_t num_slices, const float* h, const void* b, int32_t slots,
                        int32_t R, const int32_t* token_order, const int32_t* slot_indptr,
                        const int32_t* ranks, const float* scalings, void* stream) {
  lora_status st = check_common(dtype, T, slots, R);
  if (st != LORA_OK) return st;
  SliceTable tab;
  if ((st = make_slices(dtype, out_slices, num_slices, R, &tab)) != LORA_OK) return st;
  if (T == 0) return LORA_OK;
  if (!y || !h || !b || !scalings) return LORA_ERR_INVALID_ARG;
  if ((st = check_addr(token_order, slot_indptr, ranks)) != LORA_OK) return st;
  if (!aligned16(y) || !aligned16(h) || !aligned16(b)) return LORA_ERR_ALIGNMENT;
  // bf16: in a small batch, segments of at most kLongSegment tokens on the
  // decode tiles and longer ones on the SGMV tiles, in a large batch every
  // segment on the SGMV tiles; otherwise the VALU kernel takes all
  const bool mfma = lora::sgmv_supported(dtype, tab, R, (int)T, 8) &&
                    lora::fused_supported(dtype, tab, R, (int)T, 8);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (mfma) {
    const bool large = T >= kLargeBatch;
    if (!large)
      e = lora::launch_decode_expand(y, (int)T, tab, h, b, slots, R, token_order, slot_indptr,
                                     ranks, scalings, s);
    if (e == hipSuccess)
      e = lora::launch_sgmv_expand(y, (int)T, tab, h, b, slots, R, token_order, slot_indptr,
                                   ranks, scalings, large ? 0 : lora::kLongSegment, s);
  } else {
    e = lora::launch_expand(dtype, y, (int)T, tab, h, b, slots, R, token_order, slot_indptr,
                            ranks, scalings, lora::kNoMaxSeg, s);
  }
  return hip_status(e);
}

size_t lora_fused_column_linear_workspace_bytes(int64_t T, int64_t in_features,
                                                int32_t num_slices, int32_t R) {
  if (T < 0 || T > kMaxI32 || num_slices < 1 || num_slices > lora::kMaxSlices || R < 1 ||
      R > 256 || in_features < 1 || in_features > kMaxI32)
    return 0;
  // h, then the shrink's K parts
  return ws_h_bytes(T, num_slices, R) +
         lora_shrink_workspace_bytes(T, in_features, num_slices, R);
}

lora_status lora_column_linear(int dtype, const void* x, const void* w, void* y, int64_t T,
                               int64_t in_features, const int64_t* out_slices,
                               int32_t num_slices, void* stream) {
  if (dtype != LORA_BF16) return LORA_ERR_UNSUPPORTED;
  if (T < 0 || T > kMaxI32 || in_features < 1 || in_features > kMaxI32)
    return LORA_ERR_INVALID_ARG;
  SliceTable tab;
  lora_status st = make_slices(dtype, out_slices, num_slices, 8, &tab);
  if (st != LORA_OK) return st;
  if (!lora::linear_lora_supported(dtype, tab, 8, (int)T, (int)in_features))
    return LORA_ERR_UNSUPPORTED;
  if (T == 0) return LORA_OK;
  if (!x || !w || !y) return LORA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return LORA_ERR_ALIGNMENT;
  // no delta: the token order is the identity, so no addressing is needed
  return hip_status(lora::launch_linear_lora(x, w, y, (int)T, (int)in_features, tab, nullptr,
                                             nullptr, 1, 8, nullptr, nullptr, nullptr, nullptr,
                                             (hipStream_t)stream));
}

lora_status lora_fused_column_linear(int dtype, const void* x, const void* w, void* y, int64_t T,
                                     int64_t in_features, const int64_t* out_slices,
                                     int32_t num_slices, const void* a, const void* b,
                                     int32_t slots, int32_t R, const int32_t* token_order,
                                     const int32_t* slot_indptr, const int32_t* ranks,
                                     const float* scalings, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (dtype != LORA_BF16) return LORA_ERR_UNSUPPORTED;
  lora_status st = check_common(dtype, T, slots, R);
  if (st != LORA_OK) return st;
  SliceTable tab;
  if ((st = make_slices(dtype, out_slices, num_slices, R, &tab)) != LORA_OK) return st;
  if (in_features < 1 || in_features > kMaxI32) return LORA_ERR_INVALID_ARG;
  if (!lora::linear_lora_supported(dtype, tab, R, (int)T, (int)in_features))
    return LORA_ERR_UNSUPPORTED;
  if (T == 0) return LORA_OK;
  if (!x || !w || !y || !a || !b || !scalings) return LORA_ERR_INVALID_ARG;
  if ((st = check_addr(token_order, slot_indptr, ranks)) != LORA_OK) return st;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || !aligned16(a) || !aligned16(b))
    return LORA_ERR_ALIGNMENT;
  if (in_features % vec_elems(dtype) != 0) return LORA_ERR_ALIGNMENT;
  const size_t need = lora_fused_column_linear_workspace_bytes(T, in_features, num_slices, R);
  if (!workspace || workspace_bytes < need) return LORA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LORA_ERR_ALIGNMENT;
  // h of the adapted tokens (below each slot's rank: the only columns the
  // epilogue uses), then the base projection with the delta of h in its
  // epilogue
  float* h = static_cast<float*>(workspace);
  const size_t hb = ws_h_bytes(T, num_slices, R);
  const size_t pb = workspace_bytes - hb;
  st = shrink_impl(dtype, x, T, in_features, a, slots, num_slices, R, token_order, slot_indptr,
                   ranks, h, pb > 0 ? static_cast<char*>(workspace) + hb : nullptr, pb, stream,
                   false);
  if (st != LORA_OK) return st;
  return hip_status(lora::launch_linear_lora(x, w, y, (int)T, (int)in_features, tab, h, b, slots,
                                             R, token_order, slot_indptr, ranks, scalings,
                                             (hipStream_t)stream));
}

int lora_apply_linear_path(int dtype, int64_t T, int64_t in_features, const int64_t* out_slices,
                           int32_t num_slices, int32_t R) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return -LORA_ERR_UNSUPPORTED;
  if (T < 0 || T > kMaxI32 || in_features < 1 || in_features > kMaxI32 || R < 1 || R > 256)
    return -LORA_ERR_INVALID_ARG;
  SliceTable tab;
  const lora_status st = make_slices(dtype, out_slices, num_slices, R, &tab);
  if (st != LORA_OK) return -st;
  return apply_path(dtype, T, in_features, tab, R);
}

size_t lora_apply_linear_workspace_bytes(int64_t T, int64_t in_features, int32_t slots,
                                         int32_t num_slices, int32_t R) {
  if (T < 0 || T > kMaxI32 || num_slices < 1 || num_slices > lora::kMaxSlices || R < 1 ||
      R > 256 || slots < 1 || slots > 8192 || in_features < 1 || in_features > kMaxI32)
    return 0;
  // counters, the fused path's partial tiles, then h for the long segments
  // (or for the whole batch on the shrink-then-expand path)
  // and the K parts of the SGMV shrink
  return lora::counter_bytes(slots, num_slices) + partial_bytes(slots, num_slices, R, in_features) +
         ws_h_bytes(T, num_slices, R) * (1 + lora::sgmv_kparts((int)in_features));
}

lora_status lora_apply_linear(int dtype, const void* x, void* y, int64_t T, int64_t in_features,
                              const int64_t* out_slices, int32_t num_slices, const void* a,
                              const void* b, int32_t slots, int32_t R,
                              const int32_t* token_order, const int32_t* slot_indptr,
                              const int32_t* ranks, const float* scalings, void* workspace,
                              size_t workspace_bytes, void* stream) {
  lora_status st = check_common(dtype, T, slots, R);
  if (st != LORA_OK) return st;
  SliceTable tab;
  if ((st = make_slices(dtype, out_slices, num_slices, R, &tab)) != LORA_OK) return st;
  if (in_features < 1 || in_features > kMaxI32) return LORA_ERR_INVALID_ARG;
  if (T == 0) return LORA_OK;
  if (!x || !y || !a || !b || !scalings) return LORA_ERR_INVALID_ARG;
  if ((st = check_addr(token_order, slot_indptr, ranks)) != LORA_OK) return st;
  if (!aligned16(x) || !aligned16(y) || !aligned16(a) || !aligned16(b)) return LORA_ERR_ALIGNMENT;
  if (in_features % vec_elems(dtype) != 0) return LORA_ERR_ALIGNMENT;
  const size_t need = lora_apply_linear_workspace_bytes(T, in_features, slots, num_slices, R);
  if (!workspace || workspace_bytes < need) return LORA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LORA_ERR_ALIGNMENT;
  return run_apply(dtype, x, y, T, in_features, tab, num_slices, a, b, slots, R, token_order,
                   slot_indptr, ranks, scalings, workspace, (hipStream_t)stream);
}

int lora_apply_linear_from_slots_one_launch(int dtype, int64_t T, int64_t in_features,
                                            const int64_t* out_slices, int32_t num_slices,
                                            int32_t slots, int32_t R) {
  const int path = lora_apply_linear_path(dtype, T, in_features, out_slices, num_slices, R);
  if (path < 0) return path;
  if (slots < 1 || slots > 8192) return -LORA_ERR_UNSUPPORTED;
  return path == LORA_PATH_FUSED && T > 0 && lora::fused_from_slots_supported((int)T, slots);
}

size_t lora_apply_linear_from_slots_workspace_bytes(int64_t T, int64_t in_features,
                                                    int32_t slots, int32_t num_slices,
                                                    int32_t R) {
  const size_t a = lora_apply_linear_workspace_bytes(T, in_features, slots, num_slices, R);
  if (a == 0) return 0;
  // the apply's region, then the addressing's (the two-pass sort of a large batch)
  return align256(a) + lora::addressing_workspace_bytes(T, slots);
}

lora_status lora_apply_linear_from_slots(int dtype, const void* x, void* y, int64_t T,
                                         int64_t in_features, const int64_t* out_slices,
                                         int32_t num_slices, const void* a, const void* b,
                                         int32_t slots, int32_t R, const int32_t* token_slot,
                                         int32_t* token_order, int32_t* slot_indptr,
                                         const int32_t* ranks, const float* scalings,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  lora_status st = check_common(dtype, T, slots, R);
  if (st != LORA_OK) return st;
  SliceTable tab;
  if ((st = make_slices(dtype, out_slices, num_slices, R, &tab)) != LORA_OK) return st;
  if (in_features < 1 || in_features > kMaxI32) return LORA_ERR_INVALID_ARG;
  if (!slot_indptr) return LORA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (T == 0)   // the addressing of an empty batch: slot_indptr all zeros
    return hip_status(lora::launch_build_addressing(nullptr, 0, slots, nullptr, slot_indptr,
                                                    nullptr, 0, s));
  if (!x || !y || !a || !b || !scalings || !token_slot) return LORA_ERR_INVALID_ARG;
  if ((st = check_addr(token_order, slot_indptr, ranks)) != LORA_OK) return st;
  if (!aligned16(x) || !aligned16(y) || !aligned16(a) || !aligned16(b)) return LORA_ERR_ALIGNMENT;
  if (in_features % vec_elems(dtype) != 0) return LORA_ERR_ALIGNMENT;
  const size_t apply_need = align256(
      lora_apply_linear_workspace_bytes(T, in_features, slots, num_slices, R));
  const size_t need =
      lora_apply_linear_from_slots_workspace_bytes(T, in_features, slots, num_slices, R);
  if (!workspace || workspace_bytes < need) return LORA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LORA_ERR_ALIGNMENT;
  if (lora_apply_linear_from_slots_one_launch(dtype, T, in_features, out_slices, num_slices,
                                              slots, R) == 1)
    return hip_status(lora::launch_apply_fused(x, y, (int)T, (int)in_features, tab, a, b, slots,
                                               R, nullptr, nullptr, ranks, scalings, workspace,
                                               s, token_slot, token_order, slot_indptr));
  const hipError_t e = lora::launch_build_addressing(
      token_slot, (int)T, slots, token_order, slot_indptr,
      static_cast<char*>(workspace) + apply_need, need - apply_need, s);
  if (e != hipSuccess) return LORA_ERR_HIP;
  return run_apply(dtype, x, y, T, in_features, tab, num_slices, a, b, slots, R, token_order,
                   slot_indptr, ranks, scalings, workspace, s);
}

int lora_apply_linear_from_experts_one_launch(int dtype, int64_t rows, int64_t in_features,
                                              const int64_t* out_slices, int32_t num_slices,
                                              int32_t num_experts, int32_t slots, int32_t R) {
  if (num_experts < 1 || slots < 1 || (int64_t)num_experts * slots > 8192)
    return -LORA_ERR_UNSUPPORTED;
  const int path = lora_apply_linear_path(dtype, rows, in_features, out_slices, num_slices, R);
  if (path < 0) return path;
  return path == LORA_PATH_FUSED && rows > 0 &&
         lora::fused_from_experts_supported((int)rows, num_experts, slots);
}

size_t lora_apply_linear_from_experts_workspace_bytes(int64_t rows, int64_t in_features,
                                                      int32_t num_experts, int32_t slots,
                                                      int32_t num_slices, int32_t R) {
  if (num_experts < 1 || slots < 1 || (int64_t)num_experts * slots > 8192) return 0;
  const size_t a =
      lora_apply_linear_workspace_bytes(rows, in_features, num_experts * slots, num_slices, R);
  const size_t b = lora_build_addressing_experts_workspace_bytes(rows, num_experts, slots);
  if (a == 0) return 0;
  // the apply's region, then the expert addressing's (keys and the sort)
  return align256(a) + b;
}

lora_status lora_apply_linear_from_experts(
    int dtype, const void* x, void* y, int64_t rows, int64_t in_features,
    const int64_t* out_slices, int32_t num_slices, const void* a, const void* b,
    int32_t num_experts, int32_t slots, int32_t R, const int32_t* row_slot,
    const int32_t* expert_offsets, int32_t* token_order, int32_t* slot_indptr,
    const int32_t* ranks, const float* scalings, void* workspace, size_t workspace_bytes,
    void* stream) {
  if (num_experts < 1 || slots < 1 || (int64_t)num_experts * slots > 8192)
    return LORA_ERR_UNSUPPORTED;
  const int32_t K = num_experts * slots;   // pool entries
  lora_status st = check_common(dtype, rows, K, R);
  if (st != LORA_OK) return st;
  SliceTable tab;
  if ((st = make_slices(dtype, out_slices, num_slices, R, &tab)) != LORA_OK) return st;
  if (in_features < 1 || in_features > kMaxI32) return LORA_ERR_INVALID_ARG;
  if (!slot_indptr || !expert_offsets) return LORA_ERR_INVALID_ARG;
  const size_t need = lora_apply_linear_from_experts_workspace_bytes(rows, in_features,
                                                                     num_experts, slots,
                                                                     num_slices, R);
  if (!workspace || workspace_bytes < need) return LORA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LORA_ERR_ALIGNMENT;
  hipStream_t s = (hipStream_t)stream;
  const size_t apply_need =
      align256(lora_apply_linear_workspace_bytes(rows, in_features, K, num_slices, R));
  char* ws_addr = static_cast<char*>(workspace) + apply_need;
  if (rows == 0)   // the addressing of an empty batch: slot_indptr all zeros
    return hip_status(lora::launch_build_addressing_experts(
        nullptr, expert_offsets, num_experts, 0, slots, nullptr, slot_indptr, ws_addr,
        need - apply_need, s));
  if (!x || !y || !a || !b || !scalings || !row_slot) return LORA_ERR_INVALID_ARG;
  if ((st = check_addr(token_order, slot_indptr, ranks)) != LORA_OK) return st;
  if (!aligned16(x) || !aligned16(y) || !aligned16(a) || !aligned16(b)) return LORA_ERR_ALIGNMENT;
  if (in_features % vec_elems(dtype) != 0) return LORA_ERR_ALIGNMENT;
  if (lora_apply_linear_from_experts_one_launch(dtype, rows, in_features, out_slices,
                                                num_slices, num_experts, slots, R) == 1)
    return hip_status(lora::launch_apply_fused(
        x, y, (int)rows, (int)in_features, tab, a, b, K, R, nullptr, nullptr, ranks, scalings,
        workspace, s, row_slot, token_order, slot_indptr, expert_offsets, num_experts, slots));
  const hipError_t e = lora::launch_build_addressing_experts(
      row_slot, expert_offsets, num_experts, (int)rows, slots, token_order, slot_indptr,
      ws_addr, need - apply_need, s);
  if (e != hipSuccess) return LORA_ERR_HIP;
  return run_apply(dtype, x, y, rows, in_features, tab, num_slices, a, b, K, R, token_order,
                   slot_indptr, ranks, scalings, workspace, s);
}

}  // extern "C"
