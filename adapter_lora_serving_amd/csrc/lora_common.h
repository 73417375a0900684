// Device helpers shared by the LoRA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Element tags: BF16 data is handled as raw 16-bit patterns packed two per
// 32-bit word; F32 data as floats. Both move in 16-byte vectors.
struct BF16 {
  static constexpr int kVec = 8;    // elements per 16-byte vector
  static constexpr int kBytes = 2;
};
struct F32 {
  static constexpr int kVec = 4;
  static constexpr int kBytes = 4;
};

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return to_bf16_bits(lo) | (to_bf16_bits(hi) << 16);
}

// Two-term bf16 dot product accumulated in fp32 (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// D[16x16] += A[16 x 16] . B[16 x 16]^T in fp32 (v_mfma_f32_16x16x16_bf16):
// lane (m = lane & 15, g = lane >> 4) supplies row m, k in [4g, 4g+4) of
// both operands; it receives D[4g + i][m] in element i.
__device__ __forceinline__ f32x4 mfma_k16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// D[16x16] += A[16 x 32] . B[16 x 32]^T in fp32, where lane (m, g) supplies
// row m, k in [8g, 8g+8) of both operands (the 16x16x32 operand layout).
// Issued as two 16x16x16 products over the two halves of each lane's eight
// k values: A and B are split alike, so every k meets its partner once. The
// single v_mfma_f32_16x16x32_bf16 is not used because the compiler spaces a
// vector read of its result as for a 4-pass op, and such a read was measured
// to return the last accumulator register stale on gfx950.
__device__ __forceinline__ f32x4 mfma_k32(bf16x8 a, bf16x8 b, f32x4 c) {
  const u32x4 au = __builtin_bit_cast(u32x4, a);
  const u32x4 bu = __builtin_bit_cast(u32x4, b);
  c = mfma_k16(__builtin_bit_cast(s16x4, u32x2{au.x, au.y}),
               __builtin_bit_cast(s16x4, u32x2{bu.x, bu.y}), c);
  return mfma_k16(__builtin_bit_cast(s16x4, u32x2{au.z, au.w}),
                  __builtin_bit_cast(s16x4, u32x2{bu.z, bu.w}), c);
}

// Index of the calling wave in its workgroup, in a scalar register: every
// lane of a wave has the same value, and saying so lets the compiler keep
// per-wave loops as scalar loops instead of masked vector ones.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / 64u));
}

__device__ __forceinline__ int clamp_rank(int r, int R) { return r < 0 ? 0 : (r > R ? R : r); }

// Inclusive prefix sum across the wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  return v;
}

// Exclusive prefix sum across the block; `scratch` holds >= 17 ints of LDS.
// Every thread of the block must call it.
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int nw = (blockDim.x + kWave - 1) / kWave;
  int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) scratch[w] = inc;
  __syncthreads();
  if (w == 0) {
    int s = lane < nw ? scratch[lane] : 0;
    int si = wave_inclusive_scan(s);
    if (lane < nw) scratch[lane] = si - s;
    if (lane == nw - 1) scratch[16] = si;
  }
  __syncthreads();
  int r = inc - v + scratch[w];
  if (total) *total = scratch[16];
  __syncthreads();
  return r;
}

// Slot of position p of token_order: the s with slot_indptr[s] <= p <
// slot_indptr[s+1]; `slots` when p is in the dead region.
__device__ __forceinline__ int slot_of_position(const int32_t* __restrict__ indptr, int slots,
                                                int p) {
  if (p >= indptr[slots]) return slots;
  int lo = 0, hi = slots;  // invariant: indptr[lo] <= p < indptr[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (indptr[mid] <= p) lo = mid; else hi = mid;
  }
  return lo;
}

// Segment [beg, beg + n) of slot s in token_order, clamped to [0, T] so a
// malformed addressing can give wrong values but never an access outside the
// buffers.
__device__ __forceinline__ void segment_of(const int32_t* __restrict__ indptr, int s, int T,
                                           int& beg, int& n) {
  int b = indptr[s], e = indptr[s + 1];
  b = min(max(b, 0), T);
  e = min(max(e, b), T);
  beg = b;
  n = e - b;
}

// Token index read from token_order, clamped into [0, T).
__device__ __forceinline__ int token_at(const int32_t* __restrict__ order, int p, int T) {
  const int t = order[p];
  return min(max(t, 0), T - 1);
}

// Work-item location: given per-slot item counts count(s), find the slot
// owning `item` and the item's index inside that slot. Block-cooperative:
// every thread of the block must call it; the result is uniform.
struct SlotItem {
  int slot;   // -1 when item >= total
  int local;
  int total;  // items over all slots
};

template <typename CountFn>
__device__ __forceinline__ SlotItem locate_item(int item, int slots, CountFn count,
                                                int* scratch /* >= 20 ints LDS */) {
  const int nthreads = blockDim.x;
  const int chunk = (slots + nthreads - 1) / nthreads;
  const int s0 = threadIdx.x * chunk;
  const int s1 = min(slots, s0 + chunk);
  int local = 0;
  for (int s = s0; s < s1; ++s) local += count(s);
  int total = 0;
  int excl = block_exclusive_scan(local, scratch, &total);
  if (threadIdx.x == 0) { scratch[18] = -1; scratch[19] = 0; }
  __syncthreads();
  if (item >= excl && item < excl + local) {
    int run = excl;
    for (int s = s0; s < s1; ++s) {
      int c = count(s);
      if (item < run + c) { scratch[18] = s; scratch[19] = item - run; break; }
      run += c;
    }
  }
  __syncthreads();
  SlotItem r{scratch[18], scratch[19], total};
  __syncthreads();
  return r;
}

// Work-item location in two steps, for a workgroup that locates one item or
// several (a grid-stride loop). scan_slots loads each slot's values once
// (info(s, v): segment begin, length, rank) and forms the block-wide
// exclusive prefix of the per-slot item counts (count_of(v)); pick_item then
// finds any item's slot and the slot's values without another scan. When
// slots <= blockDim.x every thread holds at most one slot, in registers, so
// a pick makes no memory access.
struct SlotScan {
  int s0, s1;    // this thread's slots [s0, s1)
  int excl;      // items before slot s0
  int local;     // items of this thread's slots
  int first;     // items of slot s0
  int v0[3];     // values of slot s0
  int total;     // items over all slots
};

template <typename InfoFn, typename CountFn>
__device__ __forceinline__ SlotScan scan_slots(int slots, InfoFn info, CountFn count_of,
                                               int* scratch /* >= 24 ints LDS */) {
  SlotScan sc;
  const int nthreads = blockDim.x;
  const int chunk = (slots + nthreads - 1) / nthreads;
  sc.s0 = threadIdx.x * chunk;
  sc.s1 = min(slots, sc.s0 + chunk);
  sc.v0[0] = sc.v0[1] = sc.v0[2] = 0;
  sc.local = 0;
  sc.first = 0;
  for (int s = sc.s0; s < sc.s1; ++s) {
    int v[3];
    info(s, v);
    const int c = count_of(v);
    if (s == sc.s0) {
      sc.first = c;
      sc.v0[0] = v[0]; sc.v0[1] = v[1]; sc.v0[2] = v[2];
    }
    sc.local += c;
  }
  sc.excl = block_exclusive_scan(sc.local, scratch, &sc.total);
  sc.total = __builtin_amdgcn_readfirstlane(sc.total);
  return sc;
}

// Slot of `item` (< sc.total): fills it (slot, local, total) and v (the
// slot's values). Every thread of the block must call it; the caller keeps
// a __syncthreads() between one call's return and the next call.
template <typename InfoFn, typename CountFn>
__device__ __forceinline__ void pick_item(const SlotScan& sc, int item, InfoFn info,
                                          CountFn count_of, int* scratch, SlotItem& it,
                                          int* v) {
  if (threadIdx.x == 0) scratch[18] = -1;
  __syncthreads();
  if (item >= sc.excl && item < sc.excl + sc.local) {
    int run = sc.excl;
    for (int s = sc.s0; s < sc.s1; ++s) {
      int u[3] = {sc.v0[0], sc.v0[1], sc.v0[2]};
      if (s != sc.s0) info(s, u);
      const int c = s == sc.s0 ? sc.first : count_of(u);
      if (item < run + c) {
        scratch[18] = s;
        scratch[19] = item - run;
        scratch[20] = u[0];
        scratch[21] = u[1];
        scratch[22] = u[2];
        break;
      }
      run += c;
    }
  }
  __syncthreads();
  // uniform values: held in scalar registers
  it = SlotItem{__builtin_amdgcn_readfirstlane(scratch[18]),
                __builtin_amdgcn_readfirstlane(scratch[19]), sc.total};
  v[0] = __builtin_amdgcn_readfirstlane(scratch[20]);
  v[1] = __builtin_amdgcn_readfirstlane(scratch[21]);
  v[2] = __builtin_amdgcn_readfirstlane(scratch[22]);
}

// Raw buffer access. A resource covers [base, base + bytes); a load at an
// offset outside it returns zero without touching memory and a store there is
// dropped, so predicated accesses need no branches (kOOB is such an offset
// for every resource smaller than 2 GiB).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kRsrcWord3 = 0x00020000;   // gfx9-family raw buffer, range checked

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
// Streamed (nt) load, for data this kernel reads exactly once.
__device__ __forceinline__ u32x4 bload16_once(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
}
__device__ __forceinline__ u32x2 bload8(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ void bstore8(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void bstore16(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void bstore4(rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
}
// Stores of y, which the kernel writes once and never reads back: cache
// policy sc1 | nt (streamed toward memory). Measured on the decode apply
// (24 MB per launch): 12.9 -> 12.5 us against plain stores; nt or sc1 alone,
// or streamed loads of x, A, B or y there, gave nothing or lost time. The
// h written for the next kernel stays on the default policy (streaming it
// cost the prefill expand 4-5 us).
constexpr int kStreamOut = 18;
__device__ __forceinline__ void bstore8_out(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, kStreamOut);
}
__device__ __forceinline__ void bstore16_out(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kStreamOut);
}

// ---- buffer-to-LDS rings (the SGMV shrink, the base-projection GEMM) ----
typedef __attribute__((address_space(3))) void lds_void;

// One 16-byte global -> LDS transfer per lane (buffer_load ... lds): the
// wave's 64 lanes fill the 1 KB at dst, lane L at byte 16 L. dst must be
// uniform across the wave. An offset outside the resource writes zeros.
__device__ __forceinline__ void dma16(rsrc_t r, char* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, (int)off, 0, 0, 0);
}

// s_waitcnt operand that waits until at most n vector memory operations are
// outstanding (vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at
// their maxima, i.e. not waited for). Transfers into LDS count as vector
// memory operations.
constexpr int vmcnt_le(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Byte offset of logical 16-byte chunk c (0..3) of row `row` in an LDS tile
// of 64-byte rows: stored at chunk c ^ ((row >> 1) & 3), so that the operand
// reads of 16 consecutive rows (one chunk each) spread over the banks.
__device__ __forceinline__ int swz4(int row, int c) {
  return row * 64 + ((c ^ ((row >> 1) & 3)) << 4);
}

// Workgroup barrier with no memory fence. __syncthreads()'s release fence
// waits for every vector memory operation in flight, which would empty a
// ring of transfers that are meant to stay in flight across it; the empty
// asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


// ---------------------------------------------------------------------------
// Slot addressing pieces shared by the addressing kernels and the fused
// kernel's one-launch form (which builds the addressing in one workgroup of
// the same launch).

// Lanes of a wave holding the same key: dead tokens (slot outside
// [0, slots)) take key `slots`, after every live slot.
struct GroupMatch {
  int key;      // -1 for a lane past the range
  int rank;     // lanes below this one with the same key
  int count;    // lanes with this key
  bool leader;  // lowest lane with this key
};

// raw: the token's slot as stored (ignored when !valid). One ballot per key
// bit (nbits = bits of `slots`), independent of how many distinct keys the
// wave holds.
__device__ __forceinline__ GroupMatch match_raw(int raw, bool valid, int slots, int nbits) {
  GroupMatch g;
  int k = -1;
  if (valid) k = (raw >= 0 && raw < slots) ? raw : slots;
  uint64_t eq = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (k >> b) & 1;
    const uint64_t bal = __ballot(valid && bit);
    eq &= bit ? bal : ~bal;
  }
  const uint64_t below = eq & ((1ull << lane_id()) - 1ull);
  g.key = k;
  g.rank = __popcll(below);
  g.count = __popcll(eq);
  g.leader = valid && below == 0;
  return g;
}

// Stable counting sort of tokens [0, T) by slot in one wave, for T <= G * 64
// and slots + 1 <= 64 keys, with no workgroup barrier: token_order lists each
// slot's tokens in ascending index (dead tokens last), slot_indptr[s] is
// where slot s begins (slots + 1 entries). Per group of 64 tokens, a lane's
// offset within its key is the key's count so far (an LDS histogram, `hist`:
// 64 ints) plus its rank among equal keys in the group; lane k then holds
// key k for the scan that gives slot_indptr, and the scatter adds the key's
// start.
template <int G>
__device__ __forceinline__ void addressing_one_wave(const int32_t* __restrict__ token_slot, int T,
                                                    int slots, int32_t* __restrict__ token_order,
                                                    int32_t* __restrict__ slot_indptr,
                                                    int* hist) {
  const int lane = lane_id();
  const int nbits = 32 - __clz(slots);
  int raw[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int t = g * kWave + lane;
    raw[g] = t < T ? token_slot[t] : -1;
  }
  hist[lane] = 0;
  __builtin_amdgcn_wave_barrier();
  int key[G], off[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int t = g * kWave + lane;
    const GroupMatch m = match_raw(raw[g], t < T, slots, nbits);
    key[g] = m.key < 0 ? 0 : m.key;   // lanes past T: any valid index, never used
    off[g] = hist[key[g]] + m.rank;
    __builtin_amdgcn_wave_barrier();
    if (m.leader) hist[m.key] += m.count;   // distinct keys: no two leaders collide
    __builtin_amdgcn_wave_barrier();
  }
  const int c = lane <= slots ? hist[lane] : 0;
  const int start = wave_inclusive_scan(c) - c;
  if (lane <= slots) slot_indptr[lane] = start;
  __builtin_amdgcn_wave_barrier();
  hist[lane] = start;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int t = g * kWave + lane;
    if (t < T) token_order[hist[key[g]] + off[g]] = t;
  }
}


// Expert of row r of an expert-sorted batch: the e with offs[e] <= r <
// offs[e + 1] (binary search over the E + 1 bounds); its key e * slots +
// row_slot, or -1 (dead) for a slot outside [0, slots) or a row outside
// [offs[0], offs[E]). Malformed bounds give wrong keys but no access out of
// bounds.
__device__ __forceinline__ int expert_key(int r, int s, const int32_t* offs, int E, int slots) {
  int key = -1;
  if (r >= offs[0] && r < offs[E]) {
    int lo = 0, hi = E;   // invariant: offs[lo] <= r < offs[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (offs[mid] <= r) lo = mid; else hi = mid;
    }
    if (s >= 0 && s < slots) key = lo * slots + s;
  }
  return key;
}

// The one-wave sort over up to 1023 live keys (K), for a batch of at most
// G * 64 tokens: raw_of(t) gives token t's key (outside [0, K): dead). As
// addressing_one_wave, with the count histogram of every key in LDS (`hist`:
// K + 1 ints) and the scan over the K + 1 counts taken in per-lane runs of
// consecutive keys. Same output as the sort of those keys.
template <int G, class RawFn>
__device__ __forceinline__ void addressing_one_wave_keys(RawFn raw_of, int T, int K,
                                                         int32_t* __restrict__ token_order,
                                                         int32_t* __restrict__ slot_indptr,
                                                         int* hist) {
  const int lane = lane_id();
  for (int i = lane; i <= K; i += kWave) hist[i] = 0;
  int raw[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int t = g * kWave + lane;
    raw[g] = t < T ? raw_of(t) : -1;
  }
  __builtin_amdgcn_wave_barrier();
  const int nbits = 32 - __clz(K);
  int key[G], off[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int t = g * kWave + lane;
    const GroupMatch m = match_raw(raw[g], t < T, K, nbits);
    key[g] = m.key < 0 ? 0 : m.key;   // lanes past T: any valid index, never used
    off[g] = hist[key[g]] + m.rank;
    __builtin_amdgcn_wave_barrier();
    if (m.leader) hist[m.key] += m.count;   // distinct keys: no two leaders collide
    __builtin_amdgcn_wave_barrier();
  }
  // exclusive scan of the K + 1 counts: lane i takes keys [i C, (i + 1) C)
  const int C = (K + 1 + kWave - 1) / kWave;
  int sum = 0;
  for (int j = 0; j < C; ++j) {
    const int k = lane * C + j;
    if (k <= K) sum += hist[k];
  }
  int run = wave_inclusive_scan(sum) - sum;
  __builtin_amdgcn_wave_barrier();
  for (int j = 0; j < C; ++j) {
    const int k = lane * C + j;
    if (k <= K) {
      const int c = hist[k];
      slot_indptr[k] = run;
      hist[k] = run;
      run += c;
    }
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int t = g * kWave + lane;
    if (t < T) token_order[hist[key[g]] + off[g]] = t;
  }
}

}  // namespace lora
