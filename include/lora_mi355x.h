/*
 * lora_mi355x.h: C ABI of the batched multi-LoRA delta for MI355X (gfx950).
 *
 * One step of multi-adapter LoRA serving adds, for every token t of a batch,
 * the low-rank update of the adapter slot the token is routed to:
 *
 *   shrink   h[t] = x[t] @ A[slot(t)]^T                  (a gather of A's column
 *                                                         for an embedding target)
 *   expand   y[t, slice i] += scaling[slot(t)] * h[t, slice i] @ B[slot(t), slice i]^T
 *
 * Source: the mstar.engine.resources.lora.backend page (module overview and
 * LoraBackend.shrink / gather_shrink / expand_fused / apply_linear_), with
 * the fused-output layout of mstar.model.components.linear (FusedColumnLinear:
 * shards along the output dimension, in order).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers are DEVICE pointers unless marked (host). The caller owns every
 * buffer; the library keeps no pointer past a call and allocates nothing.
 * Every call only enqueues work on `stream` (a hipStream_t; NULL is the null
 * stream): no host synchronisation, no device-to-host copy, no allocation, so
 * every call may be recorded under hipStreamBeginCapture. A return of
 * LORA_OK means the work was enqueued.
 *
 * Layouts (all row-major, contiguous):
 *   x        [T, in]                 dtype            (linear target)
 *   ids      [T]                     int32            (embedding target)
 *   y        [T, out]                dtype, updated in place; out = sum(out_slices)
 *   a        [slots, S*R, in]        dtype            (S = num_slices; rows i*R..i*R+R-1
 *                                                      belong to slice i)
 *   a (emb.) [slots, R, vocab]       dtype
 *   b        [slots, out, R]         dtype            (rows off_i..off_i+w_i-1 belong to
 *                                                      slice i, off_i = sum of widths before i)
 *   h        [T, S*R]                float32
 *   ranks    [slots]                 int32, clamped to [0, R] on the device
 *   scalings [slots]                 float32
 *   token_slot [T]                   int32; a value outside [0, slots) marks a token
 *                                    with no adapter ("dead")
 *   token_order [T], slot_indptr [slots+1]: the addressing (see
 *                                    lora_build_addressing)
 * dtype is LORA_F32 or LORA_BF16 and applies to x, a, b and y together;
 * h, scalings and all accumulation are float32.
 *
 * What is never read: rows of A at or past a slot's rank, columns of B at or
 * past it, all of A and B for a rank-0 slot, x rows of dead tokens and of
 * rank-0 slots. Results never depend on those values (NaN there is harmless).
 *
 * Invalid device DATA never traps: a slot outside [0, slots) is a dead token,
 * an id outside [0, vocab) contributes nothing, a rank is clamped to [0, R].
 * Invalid HOST arguments return an error before anything is enqueued.
 *
 * Limits checked on the host: 1 <= slots <= 8192, 1 <= R <= 256,
 * 1 <= num_slices <= 8, S*R <= 1024, 0 <= T < 2^31, 1 <= in < 2^31.
 * Alignment: x, a, b, y, h must be 16-byte aligned; `in` (linear targets),
 * R and every out_slices width must be multiples of 8 elements for bf16 and
 * of 4 for f32 (so every row starts on a 16-byte boundary).
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lora_status {
  LORA_OK = 0,
  LORA_ERR_INVALID_ARG = 1, /* null pointer with work to do, negative or out-of-range size */
  LORA_ERR_UNSUPPORTED = 2, /* dtype, R, num_slices or slots outside the supported set */
  LORA_ERR_ALIGNMENT = 3,   /* a pointer or a row width breaks the 16-byte rule above */
  LORA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
  LORA_ERR_HIP = 5,         /* a kernel launch failed (hipGetLastError after launch) */
  LORA_ERR_SCRATCH_LIMIT = 6 /* the sizes need more than the static scratch array of
                                lora_apply_linear_noalloc holds */
} lora_status;

typedef enum lora_dtype { LORA_F32 = 0, LORA_BF16 = 1 } lora_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* lora_status_string(int status);

/* Version string of the library build (static string). */
const char* lora_version(void);

/*
 * lora_build_addressing: group the batch's tokens by adapter slot.
 *
 * Source: lora.backend module overview (the shrink and the expand take
 * their slot addressing from the adapter pool's per-step addressing object,
 * not from an index the model keeps, which is what lets an eager step and a
 * captured graph address slots the same way) and shrink_reference /
 * expand_reference_, which take token_order and slot_indptr.
 *
 * Output: token_order is a permutation of [0, T). For each slot s the
 * segment token_order[slot_indptr[s] .. slot_indptr[s+1]) holds the tokens
 * with token_slot == s in ascending token index (stable); dead tokens follow
 * slot_indptr[slots], ascending. slot_indptr[0] = 0 and slot_indptr[slots] is
 * the number of live tokens. Deterministic and bit-exact.
 * token_slot [T] (read), token_order [T], slot_indptr [slots+1] (written).
 * T == 0 writes slot_indptr = 0 and nothing else.
 * workspace (device, optional): with at least
 * lora_build_addressing_workspace_bytes(T, slots) bytes (nonzero only for a
 * batch of more than 1024 tokens over at most 1023 slots), 16-byte aligned,
 * the batch is sorted by one workgroup per 1024 tokens in two passes; NULL
 * (with workspace_bytes 0) sorts it in one workgroup. The result is the
 * same. Contents need no initialisation; calls sharing one workspace must
 * not overlap in time. A non-NULL workspace that is too small is
 * LORA_ERR_WORKSPACE.
 */
lora_status lora_build_addressing(const int32_t* token_slot, int64_t T, int32_t slots,
                                  int32_t* token_order, int32_t* slot_indptr, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Workspace bytes lora_build_addressing can use (0: it would not use one,
 * or bad input, which the call itself reports). */
size_t lora_build_addressing_workspace_bytes(int64_t T, int32_t slots);

/*
 * lora_build_addressing_experts: the addressing of a routed-expert batch.
 *
 * Source: page "spark_model/lora/expert_apply.rs", the experts injection
 * shape (apply_expert_lora_sorted): the expert LoRA delta is applied to the
 * rows of the base grouped GEMM, which are sorted by expert, each row
 * carrying its token's adapter slot. Here the (expert, slot) pair is one
 * composite key, expert * slots + slot, and the rows are grouped by it with
 * the same stable counting sort as lora_build_addressing, on the device.
 * row_slot       device int32 [rows]: adapter slot of each row; outside
 *                [0, slots) the row is dead.
 * expert_offsets device int32 [num_experts + 1], non-decreasing: rows
 *                [expert_offsets[e], expert_offsets[e+1]) belong to expert
 *                e; rows outside [expert_offsets[0], expert_offsets[E]) are
 *                dead. A malformed array gives wrong keys, never an access
 *                out of bounds.
 * token_order    device int32 [rows] (out), rows grouped by key, stable.
 * slot_indptr    device int32 [num_experts * slots + 1] (out): the rows of
 *                (expert e, slot s) are token_order[slot_indptr[k] ..
 *                slot_indptr[k+1]) with k = e * slots + s.
 * The result is the addressing of the same rows with token_slot = key, for
 * num_experts * slots virtual slots (<= 8192), whose adapter weights and
 * ranks / scalings the apply entry points then index by k.
 * workspace (device, required): at least
 * lora_build_addressing_experts_workspace_bytes(rows, num_experts, slots)
 * bytes, 256-byte aligned; contents need no initialisation; calls sharing
 * one workspace must not overlap in time. Missing or too small:
 * LORA_ERR_WORKSPACE.
 */
lora_status lora_build_addressing_experts(const int32_t* row_slot, const int32_t* expert_offsets,
                                          int32_t num_experts, int64_t rows, int32_t slots,
                                          int32_t* token_order, int32_t* slot_indptr,
                                          void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes lora_build_addressing_experts needs (0 on bad input). */
size_t lora_build_addressing_experts_workspace_bytes(int64_t rows, int32_t num_experts,
                                                     int32_t slots);

/*
 * lora_shrink: h[t, i*R + j] = x[t] . a[slot(t), i*R + j] for j < rank(slot(t)).
 *
 * Source: lora.backend, LoraBackend.shrink (h[t] = x[t] @ a[slot(t)]^T) and
 * shrink_reference (zeros where the expand does not read).
 * Writes ALL of h [T, num_slices*R]: every entry the expand does not read
 * (dead tokens, rank-0 slots, columns at or past a slot's rank) is 0.
 * bf16: in a batch of fewer than 1024 tokens, segments of at most 16 tokens
 * run on the MFMA decode tiles and longer ones on the MFMA segment tiles; in
 * a larger batch every segment runs on the segment tiles; a VALU kernel
 * writes the zeros. fp32 runs on the VALU kernel. Which segment goes where
 * is decided on the device.
 * workspace (device, optional): with at least
 * lora_shrink_workspace_bytes(...) bytes, 256-byte aligned, the long
 * segments' products are split along in_features into parts that are summed
 * in a fixed order (the same h bit for bit on every call, and more
 * workgroups for a large batch); NULL (with workspace_bytes 0) runs them in
 * one part. Contents need no initialisation; calls sharing one workspace
 * must not overlap in time. A non-NULL workspace that is too small is
 * LORA_ERR_WORKSPACE.
 */
lora_status lora_shrink(int dtype, const void* x, int64_t T, int64_t in_features,
                        const void* a, int32_t slots, int32_t num_slices, int32_t R,
                        const int32_t* token_order, const int32_t* slot_indptr,
                        const int32_t* ranks, float* h, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Workspace bytes lora_shrink can use for these sizes; 0 when it would not
 * split (or on bad input, which the call itself reports). */
size_t lora_shrink_workspace_bytes(int64_t T, int64_t in_features, int32_t num_slices,
                                   int32_t R);

/*
 * lora_gather_shrink: h[t, j] = a[slot(t), j, ids[t]] for j < rank(slot(t)).
 *
 * Source: lora.backend, LoraBackend.gather_shrink (the shrink of a token's
 * one-hot is A's column for it; an id outside [0, in) contributes nothing)
 * and gather_shrink_reference. An embedding has one output, so S = 1 and h is
 * [T, R]. Every other entry of h (dead tokens, invalid ids, j >= rank) is 0.
 * Bit-exact: each entry is a widened copy of one element of a.
 */
lora_status lora_gather_shrink(int dtype, const int32_t* ids, int64_t T, int64_t vocab,
                               const void* a, int32_t slots, int32_t R,
                               const int32_t* token_order, const int32_t* slot_indptr,
                               const int32_t* ranks, float* h, void* stream);

/*
 * lora_expand: y[t, off_i + o] += scalings[slot(t)] *
 *              sum_{j < rank} h[t, i*R + j] * b[slot(t), off_i + o, j].
 *
 * Source: lora.backend, LoraBackend.expand_fused and expand_reference_; the
 * slice offsets follow FusedColumnLinear's shard layout.
 * out_slices (host) [num_slices]: the widths. y is updated in place with one
 * rounding per element (float32 accumulate, then round-to-nearest-even to
 * bf16 for bf16 y). Rows of dead tokens and of rank-0 slots are not touched;
 * columns of h and b at or past a slot's rank are not read.
 */
lora_status lora_expand(int dtype, void* y, int64_t T, const int64_t* out_slices,
                        int32_t num_slices, const float* h, const void* b, int32_t slots,
                        int32_t R, const int32_t* token_order, const int32_t* slot_indptr,
                        const int32_t* ranks, const float* scalings, void* stream);

/*
 * lora_apply_linear: shrink then expand into y for a linear target.
 *
 * Source: lora.backend, LoraBackend.apply_linear_ (the shrink and the
 * expand of one linear target, which a backend is free to run as one
 * kernel). Same result as lora_shrink followed by lora_expand (h kept in
 * float32 inside the workspace, never rounded). workspace must be at least
 * lora_apply_linear_workspace_bytes(...) bytes, 256-byte aligned, and zero-
 * filled before its FIRST use. Its first 4 MiB hold synchronisation
 * counters that stay consistent from call to call, so one workspace can be
 * reused across calls of any shape (and replayed from a captured graph)
 * without clearing; clearing it again between calls is also allowed. Calls
 * that share one workspace must not overlap in time (one workspace per
 * stream).
 */
lora_status lora_apply_linear(int dtype, const void* x, void* y, int64_t T,
                              int64_t in_features, const int64_t* out_slices,
                              int32_t num_slices, const void* a, const void* b,
                              int32_t slots, int32_t R, const int32_t* token_order,
                              const int32_t* slot_indptr, const int32_t* ranks,
                              const float* scalings, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Workspace bytes lora_apply_linear needs for these sizes (0 on bad input). */
size_t lora_apply_linear_workspace_bytes(int64_t T, int64_t in_features, int32_t slots,
                                         int32_t num_slices, int32_t R);

/*
 * lora_apply_linear_path: which kernel family lora_apply_linear runs for
 * these shapes (host-only query; touches no device memory).
 * Returns LORA_PATH_FUSED (the one-launch fused kernel of a small bf16
 * batch), LORA_PATH_SEGMENT (the MFMA segment-tiled shrink and expand of a
 * large bf16 batch, h in the workspace) or LORA_PATH_VALU (the vector
 * kernels: fp32, or sizes whose buffers the MFMA kernels' 32-bit offsets
 * cannot reach: x, y, h or one slot's A or B of 2 GiB or more), or a
 * negated lora_status for bad arguments. out_slices (host) as in
 * lora_apply_linear.
 */
enum { LORA_PATH_VALU = 0, LORA_PATH_FUSED = 1, LORA_PATH_SEGMENT = 2 };
int lora_apply_linear_path(int dtype, int64_t T, int64_t in_features, const int64_t* out_slices,
                           int32_t num_slices, int32_t R);

/*
 * lora_apply_linear_from_slots: lora_build_addressing followed by
 * lora_apply_linear, for the first linear target of a step.
 *
 * Source: lora.backend, module overview (the addressing is made once per
 * step from each token's slot, and every target's shrink and expand then
 * use it) and LoraBackend.apply_linear_. Arguments as lora_apply_linear,
 * except that token_slot (device, int32 [T]: each token's slot; a value
 * outside [0, slots) means no adapter) replaces the addressing, which this
 * call writes instead: token_order (device, int32 [T]) and slot_indptr
 * (device, int32 [slots + 1]) receive exactly what lora_build_addressing
 * writes, for the step's later targets, and y receives exactly (bit for bit)
 * what lora_apply_linear gives with that addressing.
 * Where lora_apply_linear_from_slots_one_launch(...) is 1 (the fused path of
 * a small bf16 batch, T <= 1024, slots <= 63) it is one kernel launch: each
 * piece finds its slot's tokens from token_slot itself and one workgroup
 * writes the addressing, which nothing in that launch reads. Elsewhere the
 * addressing kernel runs first, then lora_apply_linear's kernels.
 * workspace: at least lora_apply_linear_from_slots_workspace_bytes(...)
 * bytes, under lora_apply_linear's rules (256-byte aligned, zero-filled
 * before its first use, one per stream; shared with lora_apply_linear calls
 * on the same stream). T == 0 writes slot_indptr (all zeros) only.
 */
lora_status lora_apply_linear_from_slots(int dtype, const void* x, void* y, int64_t T,
                                         int64_t in_features, const int64_t* out_slices,
                                         int32_t num_slices, const void* a, const void* b,
                                         int32_t slots, int32_t R, const int32_t* token_slot,
                                         int32_t* token_order, int32_t* slot_indptr,
                                         const int32_t* ranks, const float* scalings,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes lora_apply_linear_from_slots needs (0 on bad input). */
size_t lora_apply_linear_from_slots_workspace_bytes(int64_t T, int64_t in_features,
                                                    int32_t slots, int32_t num_slices,
                                                    int32_t R);

/*
 * lora_apply_linear_from_slots_one_launch: 1 when lora_apply_linear_from_slots
 * runs as one kernel launch for these sizes, 0 when the addressing kernel runs
 * first, a negated lora_status for bad arguments (host-only query).
 */
int lora_apply_linear_from_slots_one_launch(int dtype, int64_t T, int64_t in_features,
                                            const int64_t* out_slices, int32_t num_slices,
                                            int32_t slots, int32_t R);

/*
 * lora_apply_linear_from_experts: lora_build_addressing_experts followed by
 * lora_apply_linear over the num_experts * slots pool entries, for the first
 * expert target of a step.
 *
 * Source: spark_model/lora/expert_apply.rs, experts injection shape (the
 * expert delta of each routed row, per expert and adapter slot) with the
 * addressing and apply of lora.backend, LoraBackend.apply_linear_. rows
 * tokens (rows of the expert-sorted batch) with row_slot (device, int32
 * [rows]: each row's adapter slot; outside [0, slots): no adapter) and
 * expert_offsets (device, int32 [num_experts + 1]: expert e owns rows
 * [offsets[e], offsets[e + 1])); a, b, ranks and scalings are laid out per
 * pool entry e * slots + slot, as for lora_apply_linear with num_experts *
 * slots slots. token_order (device, int32 [rows]) and slot_indptr (device,
 * int32 [num_experts * slots + 1]) receive exactly what
 * lora_build_addressing_experts writes, and y, for non-decreasing
 * expert_offsets, exactly what lora_apply_linear gives with that addressing
 * (other offsets keep every access in bounds but leave y unspecified).
 * Where lora_apply_linear_from_experts_one_launch(...) is 1 (the fused path
 * of a small bf16 batch: rows <= 1024, num_experts <= 63, num_experts *
 * slots <= 1023) it is one kernel launch; elsewhere the addressing kernels
 * run first, then lora_apply_linear's. workspace: at least
 * lora_apply_linear_from_experts_workspace_bytes(...) bytes under
 * lora_apply_linear's rules. rows == 0 writes slot_indptr (all zeros) only.
 */
lora_status lora_apply_linear_from_experts(
    int dtype, const void* x, void* y, int64_t rows, int64_t in_features,
    const int64_t* out_slices, int32_t num_slices, const void* a, const void* b,
    int32_t num_experts, int32_t slots, int32_t R, const int32_t* row_slot,
    const int32_t* expert_offsets, int32_t* token_order, int32_t* slot_indptr,
    const int32_t* ranks, const float* scalings, void* workspace, size_t workspace_bytes,
    void* stream);

/* Workspace bytes lora_apply_linear_from_experts needs (0 on bad input). */
size_t lora_apply_linear_from_experts_workspace_bytes(int64_t rows, int64_t in_features,
                                                      int32_t num_experts, int32_t slots,
                                                      int32_t num_slices, int32_t R);

/*
 * lora_apply_linear_from_experts_one_launch: 1 when
 * lora_apply_linear_from_experts runs as one kernel launch for these sizes,
 * 0 when the addressing kernels run first, a negated lora_status for bad
 * arguments (host-only query).
 */
int lora_apply_linear_from_experts_one_launch(int dtype, int64_t rows, int64_t in_features,
                                              const int64_t* out_slices, int32_t num_slices,
                                              int32_t num_experts, int32_t slots, int32_t R);

/*
 * lora_column_linear: the base projection of a fused column-parallel linear
 * layer, y = x @ W^T, on the library's bf16 MFMA GEMM.
 *
 * Source: page "mstar.model.components.linear", FusedColumnLinear (the
 * shards of the fused projection, e.g. q, k, v or gate, up, are stacked
 * along the output dimension in order and computed as one product).
 * x [T, in], W [out, in], y [T, out] (written, not accumulated), all bf16,
 * out = sum(out_slices) (host array, num_slices widths, each a multiple of
 * 256); fp32 accumulation, one round-to-nearest-even per output. This is the
 * same kernel lora_fused_column_linear runs, without a delta; it is the base
 * half of "base projection, then lora_apply_linear".
 * Errors: LORA_ERR_UNSUPPORTED for fp32, a width not a multiple of 256, `in`
 * not a multiple of 8 or a buffer of 2 GiB or more.
 */
lora_status lora_column_linear(int dtype, const void* x, const void* w, void* y, int64_t T,
                               int64_t in_features, const int64_t* out_slices,
                               int32_t num_slices, void* stream);

/*
 * lora_fused_column_linear: the base projection with the LoRA delta fused
 * into its epilogue:
 *   y[t, :] = x[t] @ W^T  +  (for each slice i) scalings[s] * h[t, slice i]
 *             @ B[s, slice i]^T,  h = shrink(x) as lora_shrink, s = slot(t).
 *
 * Source: page "mstar.model.components.linear", FusedColumnLinear (the base
 * product over the stacked shards), page "mstar.engine.resources.lora.
 * backend", LoraBackend.apply_linear_ (the delta), and page
 * "spark_model/lora/target.rs", module overview (kernels that fuse the delta
 * into the base projection's epilogue). The delta is added to the product's
 * fp32 accumulators before the single rounding of y, so y is written once
 * and never read: the same result as lora_column_linear followed by
 * lora_apply_linear up to that one rounding, without the delta's
 * read-modify-write of y.
 * Arguments as lora_column_linear plus those of lora_apply_linear (a, b,
 * slots, R, the addressing, ranks, scalings); dead tokens and rank-0 slots
 * get the base projection only. workspace (device, required, 256-byte
 * aligned, no initialisation needed): at least
 * lora_fused_column_linear_workspace_bytes(T, in, num_slices, R) bytes
 * (h and the shrink's K parts). Calls sharing a workspace must not overlap.
 */
lora_status lora_fused_column_linear(int dtype, const void* x, const void* w, void* y, int64_t T,
                                     int64_t in_features, const int64_t* out_slices,
                                     int32_t num_slices, const void* a, const void* b,
                                     int32_t slots, int32_t R, const int32_t* token_order,
                                     const int32_t* slot_indptr, const int32_t* ranks,
                                     const float* scalings, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Workspace bytes lora_fused_column_linear needs (0 on bad input). */
size_t lora_fused_column_linear_workspace_bytes(int64_t T, int64_t in_features,
                                                int32_t num_slices, int32_t R);

/*
 * lora_apply_linear_noalloc: lora_apply_linear without a workspace argument,
 * for callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid the allocator).
 *
 * Same arguments, semantics, result and kernels as lora_apply_linear, minus
 * workspace / workspace_bytes: the workspace is a static device array of
 * LORA_NOALLOC_SCRATCH_BYTES (128 MiB) that the library holds on every GPU it
 * runs on until the process ends. The call allocates nothing (no hipMalloc,
 * no allocating library routine); the first call on a device looks the
 * array's address up once (hipGetSymbolAddress), so make that first call
 * outside graph capture where possible.
 * Sizes whose lora_apply_linear_workspace_bytes(...) exceed the array are
 * refused with LORA_ERR_SCRATCH_LIMIT before anything else is done.
 * stream must belong to the current device (else LORA_ERR_INVALID_ARG).
 * All calls on one GPU share the array: calls that overlap in time on one
 * GPU race and must not be issued. The array keeps the last call's
 * contents; nothing in it needs clearing between calls.
 */
#define LORA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
lora_status lora_apply_linear_noalloc(int dtype, const void* x, void* y, int64_t T,
                                      int64_t in_features, const int64_t* out_slices,
                                      int32_t num_slices, const void* a, const void* b,
                                      int32_t slots, int32_t R, const int32_t* token_order,
                                      const int32_t* slot_indptr, const int32_t* ranks,
                                      const float* scalings, void* stream);

/* Size in bytes of lora_apply_linear_noalloc's static scratch array. */
size_t lora_noalloc_scratch_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* LORA_MI355X_H */
