// Segment-tiled (SGMV) shrink and expand on bf16 MFMA, for the slot segments
// longer than a given length (min_len): 16 tokens next to the decode tiles,
// or 0 (every segment) for a large batch, where the long segments' products
// are real dense contractions and the short ones stream their adapter
// weights through the same tiles.
//
// Follows the mstar lora.backend page: LoraBackend.shrink (h[t] =
// x[t] @ a[slot(t)]^T) and LoraBackend.expand_fused (y[t, slice i] +=
// scalings[slot(t)] * h[t, slice i] @ b[slot(t), slice i]^T); the slice
// layout follows mstar.model.components.linear, FusedColumnLinear.
//
// Shrink item: (slot, block of 128 tokens of its segment, slice group, K
//   part). Eight waves; wave w owns token tile w against the item's rank
//   tiles. The x block and the A rows stream through a ring of LDS stages
//   that buffer-to-LDS loads fill a few K steps ahead. A slot whose rank
//   needs fewer rank tiles than the kernel holds takes several slices in one
//   item (their tiles side by side), so its x block is read once for all of
//   them. Rows of A at or past the rank read as zeros without a memory
//   access. With several K parts each item writes a partial h and a second
//   kernel sums the parts.
// Expand item: (slot, block of 64 tokens, 256 output columns of one slice).
//   The block's h rows are scaled and split into bf16 hi + lo in LDS; every
//   wave prefetches its 4 column tiles of B and y in one round trip, then
//   y^T tile = B_tile . H^T with two v_mfma_f32_16x16x16_bf16 per 16 ranks
//   and 4 token tiles, one rounding of y.
// Items run in block order (blocks are dealt to the 8 XCDs round robin), and
// consecutive items sweep along token rows: an expand item's column chunks
// are innermost, so the workgroups resident at one time read and write y in
// long row-major runs; the chunk count per token block is padded to a
// multiple of 8 so chunk ck always runs on XCD ck % 8 and its B tile stays in
// that XCD's L2. A shrink item's K parts are innermost for the same reason.
// For a batch of mostly short segments the expand launches one resident
// round of workgroups (a multiple of 8) that walk the items with a grid
// stride, so item i still runs on XCD i % 8.
#include "lora_common.h"
#include "lora_kernels.h"

#include <algorithm>
#include <map>
#include <mutex>
#include <type_traits>

namespace lora {

namespace {

constexpr int kBMe = 64;      // tokens per expand item
constexpr int kCC = 256;      // output columns per expand item

}  // namespace

// ---------------------------------------------------------------------------
// shrink
// ---------------------------------------------------------------------------
// Item: (slot, block of 128 tokens, slice group, K part). A slot of rank r
// uses ntr = ceil(r / 16) rank tiles per slice; a group packs g = min(S,
// RT / ntr, gmax) slices, slice j of the group on tiles [j * ntr, (j + 1) *
// ntr), so a slot of small rank reads its x block once for several slices.
// gmax keeps a group's A rows below 2 GiB.
// K runs in steps of 32 through a ring of LDS stages, each holding the
// block's x rows (128 x 32 bf16) and the group's A rows (NT tiles x 16 rows x
// 32 bf16, NT = the item's live tiles rounded up to a power of two). Buffer
// loads write the ring directly (no registers), kStages - 1 steps ahead of
// the step being multiplied, so an item keeps several steps of loads in
// flight without holding them in registers; rows past the rank, padding
// tokens and K past `in` arrive as zeros (out-of-range offsets).
// Eight waves; wave w owns token tile w against the NT rank tiles and skips
// its products when the tile holds no token. The product is formed as
// A_rows . x_rows^T, so each lane ends with 4 consecutive ranks of one token
// and stores them as one 16-byte vector.
// With kparts > 1 each item writes its partial h to its own buffer
// (hout + kp * part_stride); k_sum_parts adds them in kp order. Every item
// writes the columns of its slices below 16 * ntr.
constexpr int kBMs = 128;

// Slices per item for a slot of rank r (r > 0) in a kernel of RT rank tiles.
__device__ __forceinline__ int shrink_group(int r, int RT, int S, int gmax) {
  const int ntr = (r + 15) / 16;
  return max(1, min(min(S, RT / ntr), gmax));
}

// LDS ring of the shrink (dynamic shared memory). A stage covers KS
// elements of K: 128 B rows up to 4 rank tiles, so that x is read in whole
// 128-byte lines; 64 B rows above, where a deeper stage would leave room for
// one workgroup per CU. Stage s at s * kStage: [x rows: 128 x RB][A rows: RT
// * 16 x RB]; then a 1 KB landing block for the empty transfers of waves with
// no A rows to load.
template <int RT>
struct ShrinkRing {
  static constexpr int KS = RT <= 4 ? 64 : 32;   // K elements per stage
  static constexpr int RB = KS * 2;              // bytes per row
  static constexpr int CH = RB / 16;             // 16-byte chunks per row
  static constexpr int RPB = 1024 / RB;          // rows per 1 KB transfer block
  static constexpr int kX = kBMs * RB;
  static constexpr int kA = RT * 16 * RB;
  static constexpr int kStage = kX + kA;
  // stages: as many as leave room for two workgroups per CU
  static constexpr int kStages = (RT == 1 || RT == 8) ? 4 : 3;
  static constexpr int kFill = kStages * kStage;
  static constexpr int kBytes = kFill + 1024;
  // byte offset of logical chunk c of row `row` in a tile: rows of 4 chunks
  // store chunk c at c ^ ((row >> 1) & 3), rows of 8 at c ^ (row & 7), so
  // that the operand reads of 16 consecutive rows spread over the banks
  static __device__ __forceinline__ int swz(int row, int c) {
    if constexpr (CH == 4) return swz4(row, c);
    return row * 128 + ((c ^ (row & 7)) << 4);
  }
};

template <int RT>
// two workgroups per CU (the ring's LDS)
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void k_sgmv_shrink(
    const void* __restrict__ x_, int T, int in, const void* __restrict__ a_, int slots, int S,
    int R, const int32_t* __restrict__ order, const int32_t* __restrict__ indptr,
    const int32_t* __restrict__ ranks, float* __restrict__ hout, int kparts,
    int64_t part_stride, int min_len, int gmax) {
  using Ring = ShrinkRing<RT>;
  constexpr int KS = Ring::KS;
  constexpr int CH = Ring::CH;
  extern __shared__ __attribute__((aligned(16))) char ring[];
  __shared__ int scratch[24];
  __shared__ int tok[kBMs];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = wave_id();
  auto info = [&](int ss, int* v) {
    segment_of(indptr, ss, T, v[0], v[1]);
    v[2] = clamp_rank(ranks[ss], R);
  };
  auto count_of = [&](const int* v) {
    if (v[1] <= min_len || v[2] <= 0) return 0;
    const int g = shrink_group(v[2], RT, S, gmax);
    return (S + g - 1) / g * kparts * ((v[1] + kBMs - 1) / kBMs);
  };
  const SlotScan sc = scan_slots(slots, info, count_of, scratch);
  if ((int)blockIdx.x >= sc.total) return;
  __syncthreads();   // the scan's scratch is reused by the pick
  SlotItem it;
  int sv[3];
  pick_item(sc, (int)blockIdx.x, info, count_of, scratch, it, sv);
  const int s = it.slot;
  const int seg0 = sv[0];
  const int n = sv[1];
  const int r = sv[2];
  const int nmb = (n + kBMs - 1) / kBMs;
  const int kp = it.local % kparts;
  const int rest = it.local / kparts;
  const int mb = rest % nmb;
  const int ntr = (r + 15) / 16;   // rank tiles of one slice
  const int g = shrink_group(r, RT, S, gmax);
  const int i0 = (rest / nmb) * g;  // first slice of the group
  const int gsz = min(g, S - i0);   // slices in the group
  const int live = gsz * ntr;       // rank tiles holding rows below r
  const int ntok = min(kBMs, n - mb * kBMs);
  if (tid < kBMs) tok[tid] = tid < ntok ? token_at(order, seg0 + mb * kBMs + tid, T) : -1;
  __syncthreads();

  const rsrc_t x_r = make_rsrc(x_, (uint32_t)T * (uint32_t)in * 2u);
  // the group's A rows: slices i0 .. i0 + gsz - 1 of the slot
  const rsrc_t a_r = make_rsrc((const char*)a_ + ((int64_t)s * S + i0) * R * in * 2,
                               (uint32_t)gsz * (uint32_t)R * (uint32_t)in * 2u);
  const uint32_t rowG = (uint32_t)in * 2u;
  const int steps = (in + KS - 1) / KS;
  const int s0 = (int)((int64_t)steps * kp / kparts);
  const int nst = (int)((int64_t)steps * (kp + 1) / kparts) - s0;

  // Transfers: one instruction of a wave fills a 1 KB block of a stage, RPB
  // rows, lane L at byte 16 L (row L / CH, physical chunk L % CH); the lane
  // fetches the logical chunk stored there (the swizzle is undone on the
  // global side). Wave w fills x blocks w (+ 8) and A blocks w (+ 8 j); a
  // wave past the item's A blocks sends an empty transfer to the landing
  // block, so every wave counts the same transfers per stage.
  constexpr int XB = kBMs / Ring::RPB / 8;   // x blocks per wave per stage
  const int pr = lane / CH;
  const int pc = CH == 4 ? (lane & 3) ^ ((pr >> 1) & 3) : (lane & 7) ^ (pr & 7);
  uint32_t xoff[XB];
#pragma unroll
  for (int j = 0; j < XB; ++j) {
    const int xt = tok[(w + 8 * j) * Ring::RPB + pr];
    xoff[j] = xt >= 0 ? (uint32_t)xt * rowG + (uint32_t)pc * 16u : kOOB;
  }
  auto a_off = [&](int blk) -> uint32_t {
    const int v = blk * Ring::RPB + pr;
    const int j = v / (16 * ntr);
    const int rr = v - j * 16 * ntr;
    return (j < gsz && rr < r) ? (uint32_t)(j * R + rr) * rowG + (uint32_t)pc * 16u : kOOB;
  };
  const bool prod = w * 16 < ntok;   // this wave's token tile holds tokens
  const int m = lane & 15;
  const int kg = lane >> 4;
  const int SR = S * R;
  float* hp = hout + (int64_t)kp * part_stride;

  f32x4 acc[RT];
#pragma unroll
  for (int nt = 0; nt < RT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the K loop and the store for NT rank tiles (a compile-time count)
  auto run = [&](auto ntc) {
    constexpr int NT = decltype(ntc)::value;
    constexpr int NAB = NT * 16 / Ring::RPB;     // A blocks per stage
    constexpr int AB = NAB >= 8 ? NAB / 8 : 1;   // A transfers per wave per stage
    constexpr int LW = XB + AB;                  // transfers per wave per stage
    uint32_t aoff[AB];
#pragma unroll
    for (int j = 0; j < AB; ++j) aoff[j] = a_off(w + 8 * j);
    auto issue = [&](int st) {
      char* sb = ring + (st % Ring::kStages) * Ring::kStage;
      const uint32_t kb = (uint32_t)(s0 + st) * (uint32_t)Ring::RB;   // the step's bytes in a row
      const bool kv = (s0 + st) * KS + pc * 8 < in;
#pragma unroll
      for (int j = 0; j < XB; ++j)
        dma16(x_r, sb + (w + 8 * j) * 1024, kv && xoff[j] != kOOB ? xoff[j] + kb : kOOB);
      if constexpr (NAB >= 8) {
#pragma unroll
        for (int j = 0; j < AB; ++j)
          dma16(a_r, sb + Ring::kX + (w + 8 * j) * 1024,
                kv && aoff[j] != kOOB ? aoff[j] + kb : kOOB);
      } else {
        char* dst = w < NAB ? sb + Ring::kX + w * 1024 : ring + Ring::kFill;
        dma16(a_r, dst, (w < NAB && kv && aoff[0] != kOOB) ? aoff[0] + kb : kOOB);
      }
    };
    for (int st = 0; st < Ring::kStages - 1 && st < nst; ++st) issue(st);
    for (int st = 0; st < nst; ++st) {
      // this step's transfers are done once at most the later steps' are
      // outstanding; the barrier then makes every wave's transfers visible
      // and frees the buffer read in the previous step
      const int ahead = min(nst - 1 - st, Ring::kStages - 2);
      if (ahead >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_le(2 * LW));
      else if (ahead == 1) __builtin_amdgcn_s_waitcnt(vmcnt_le(LW));
      else __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
      barrier_no_fence();
      if (st + Ring::kStages - 1 < nst) issue(st + Ring::kStages - 1);
      if (prod) {
        const char* sb = ring + (st % Ring::kStages) * Ring::kStage;
#pragma unroll
        for (int h = 0; h < KS / 32; ++h) {   // 32-element MFMA steps of the stage
          const int c = 4 * h + kg;            // the lane's logical chunk
          const bf16x8 xo = *(const bf16x8*)(sb + Ring::swz(w * 16 + m, c));
          // tiles in groups of 8: all reads of a group, then its products
#pragma unroll
          for (int n0 = 0; n0 < NT; n0 += 8) {
            constexpr int NG = NT < 8 ? NT : 8;
            bf16x8 ao[NG];
#pragma unroll
            for (int q = 0; q < NG; ++q)
              ao[q] = *(const bf16x8*)(sb + Ring::kX + Ring::swz((n0 + q) * 16 + m, c));
#pragma unroll
            for (int q = 0; q < NG; ++q) acc[n0 + q] = mfma_k32(ao[q], xo, acc[n0 + q]);
          }
        }
      }
    }
    // lane (m, kg) holds h[token tile w, row m][tile nt, ranks 4 kg .. 4 kg + 3]
    const int t = tok[w * 16 + m];
    if (!prod || t < 0) return;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int j = nt / ntr;
      const int rr = (nt - j * ntr) * 16 + 4 * kg;
      if (nt < live && rr < R)
        *(f32x4*)(hp + (int64_t)t * SR + (i0 + j) * R + rr) = acc[nt];
    }
  };
  const int ntp = live <= 1 ? 1 : live <= 2 ? 2 : live <= 4 ? 4 : live <= 8 ? 8 : 16;
  if constexpr (RT >= 16) {
    if (ntp == 16) return run(std::integral_constant<int, 16>{});
  }
  if constexpr (RT >= 8) {
    if (ntp == 8) return run(std::integral_constant<int, 8>{});
  }
  if constexpr (RT >= 4) {
    if (ntp == 4) return run(std::integral_constant<int, 4>{});
  }
  if constexpr (RT >= 2) {
    if (ntp == 2) return run(std::integral_constant<int, 2>{});
  }
  run(std::integral_constant<int, 1>{});
  // columns [16 ntr, R) of each slice are not written: lora_shrink's VALU
  // kernel writes the zeros of h, and lora_apply_linear's h is read only
  // below the rank
}

// h[t, :] = sum over kp (in order) of part[kp][t, :], for the tokens of
// segments longer than min_len (the only rows the parts hold), over each
// slice's columns below the slot's last rank tile.
__global__ __launch_bounds__(256) void k_sum_parts(const float* __restrict__ part, int kparts,
                                                   int64_t part_stride, float* __restrict__ h,
                                                   int T, int SR, int slots, int R,
                                                   const int32_t* __restrict__ order,
                                                   const int32_t* __restrict__ indptr,
                                                   const int32_t* __restrict__ ranks,
                                                   int min_len) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (position, 4 columns)
  const int cq = SR / 4;
  if (g >= (int64_t)T * cq) return;
  const int p = (int)(g / cq);
  const int c = (int)(g - (int64_t)p * cq) * 4;
  const int s = slot_of_position(indptr, slots, p);
  if (s >= slots) return;
  int b0, n;
  segment_of(indptr, s, T, b0, n);
  const int r = clamp_rank(ranks[s], R);
  // columns at or past the slot's last rank tile are neither in the parts
  // nor written (see the shrink)
  if (n <= min_len || r == 0 || c % R >= 16 * ((r + 15) / 16)) return;
  const int64_t off = (int64_t)token_at(order, p, T) * SR + c;
  // each part is read once: streamed (the skewed mix -1.2 us)
  f32x4 v = __builtin_nontemporal_load((const f32x4*)(part + off));
  for (int k = 1; k < kparts; ++k) {
    const f32x4 u =
        __builtin_nontemporal_load((const f32x4*)(part + (int64_t)k * part_stride + off));
    v = f32x4{v.x + u.x, v.y + u.y, v.z + u.z, v.w + u.w};
  }
  *(f32x4*)(h + off) = v;
}

// ---------------------------------------------------------------------------
// expand
// ---------------------------------------------------------------------------
// Item: (slot, block of 64 tokens, 256 output columns of one slice). Wave w
// owns columns [lo + 64w, lo + 64w + 64) for the 64 tokens. Every global
// access is 16 bytes per lane: B rows as 8 consecutive ranks (two
// 16x16x16 products per 32 ranks), h rows as 4 consecutive ranks, and y
// row-major. The MFMA result comes out as 4 columns of one token per lane;
// it is staged through a per-wave LDS tile so that y is read and written
// row-major: one instruction covers 8 token rows x 128 contiguous bytes,
// full cache lines, so HBM never sees partial-line writes.
// PERSIST: a workgroup runs items blockIdx.x, blockIdx.x + gridDim.x, ...
// (the grid is about one resident round, a multiple of 8, so an item's XCD
// is still item % 8). The slot scan is done once; while an item runs, the
// next item's slot is picked and its token ids are loaded, so an item starts
// with its B, h and y requests instead of two dependent round trips. That
// pays where most items are short (many short segments); otherwise one item
// per workgroup lets the dispatcher balance the load.
template <int RT, bool PERSIST>
__global__ __launch_bounds__(256) void k_sgmv_expand(void* __restrict__ y_, int T, SliceTable st,
                                                     const float* __restrict__ h,
                                                     const void* __restrict__ b_, int slots,
                                                     int R, const int32_t* __restrict__ order,
                                                     const int32_t* __restrict__ indptr,
                                                     const int32_t* __restrict__ ranks,
                                                     const float* __restrict__ scalings,
                                                     int min_len) {
  constexpr int RP = RT * 16;
  constexpr int RPS = RP + 8;         // LDS h row (bf16), 16-byte aligned rows
  constexpr int MT = kBMe / 16;       // token tiles
  constexpr int TPW = kCC / 16 / 4;   // column tiles per wave (4: 64 columns)
  constexpr int SRW = 64 + 4;         // staged row (floats), padded
  constexpr bool K32 = RT >= 2;       // 32 ranks per step (8 per lane)
  constexpr int KS = K32 ? RT / 2 : RT;
  constexpr int KW = K32 ? 32 : 16;
  __shared__ int scratch[24];
  __shared__ int tok[kBMe];
  __shared__ __attribute__((aligned(16))) uint16_t hhi[kBMe * RPS];
  __shared__ __attribute__((aligned(16))) uint16_t hlo[kBMe * RPS];
  __shared__ __attribute__((aligned(16))) float stage[4][16 * SRW];

  const int tid = threadIdx.x;
  const int w = wave_id();
  const int S = st.n;
  const int out = st.off[S];
  // column chunks: slice i holds ceil(w_i / kCC) chunks
  int nck = 0;
  for (int i = 0; i < S; ++i) nck += (st.off[i + 1] - st.off[i] + kCC - 1) / kCC;
  const int nck8 = (nck + 7) & ~7;   // chunk slots per token block (padding items idle)
  auto info = [&](int ss, int* v) {
    segment_of(indptr, ss, T, v[0], v[1]);
    v[2] = clamp_rank(ranks[ss], R);
  };
  auto count_of = [&](const int* v) {
    return (v[1] > min_len && v[2] > 0) ? nck8 * ((v[1] + kBMe - 1) / kBMe) : 0;
  };
  const SlotScan sc = scan_slots(slots, info, count_of, scratch);
  int item = blockIdx.x;
  if (item >= sc.total) return;
  __syncthreads();   // the scan's scratch is reused by the picks

  // the token id of thread tid (< 64) of an item: -1 past the item's tokens
  auto token_of = [&](const SlotItem& it, const int* v) {
    const int ntok = min(kBMe, v[1] - (it.local / nck8) * kBMe);
    return tid < ntok ? token_at(order, v[0] + (it.local / nck8) * kBMe + tid, T) : -1;
  };
  SlotItem it;
  int sv[3];
  pick_item(sc, item, info, count_of, scratch, it, sv);
  int tv = token_of(it, sv);

  const rsrc_t y_r = make_rsrc(y_, (uint32_t)T * (uint32_t)out * 2u);
  const int SR = S * R;
  const rsrc_t h_r = make_rsrc(h, (uint32_t)T * (uint32_t)SR * 4u);
  float* sw = stage[w];

  for (;;) {
    // lane-derived offsets are formed again in every item: kept across the
    // loop they would hold registers the item's loads need
    int ltid = tid;
    asm volatile("" : "+v"(ltid));
    const int lane_i = ltid & 63;
    const int m = lane_i & 15;
    const int kg = lane_i >> 4;
    const int prow = lane_i >> 3;
    const int ppc = lane_i & 7;
    const int s = it.slot;
    const int n = sv[1];
    const int r = sv[2];
    const int mb = it.local / nck8;
    int ck = it.local % nck8;
    // the next item's slot (no memory access for up to 256 slots)
    const int nitem = item + (int)gridDim.x;
    SlotItem nit;
    int nsv[3];
    if (PERSIST && nitem < sc.total) {
      __syncthreads();   // this item's pick was read by every thread
      pick_item(sc, nitem, info, count_of, scratch, nit, nsv);
    }
    if (ck < nck) {
      int i = 0;
      for (; i < S; ++i) {
        const int c = (st.off[i + 1] - st.off[i] + kCC - 1) / kCC;
        if (ck < c) break;
        ck -= c;
      }
      const int lo = st.off[i] + ck * kCC;
      const int hi = min(lo + kCC, st.off[i + 1]);
      const int ntok = min(kBMe, n - mb * kBMe);
      const rsrc_t b_r = make_rsrc((const char*)b_ + (int64_t)s * out * R * 2,
                                   (uint32_t)out * (uint32_t)R * 2u);
      const int ntiles = (hi - lo) >> 4;
      const int cw = lo + w * 64;         // this wave's first column
      const int ntr = (r + KW - 1) / KW;  // rank steps holding ranks below r
      // lane (m, kg) holds B[column][ranks kk, kk + KW/4) of each of its tiles
      u32x4 bq[TPW][KS];
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int tile = w * TPW + u;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int kk = ks * KW + kg * (KW / 4);
          const uint32_t off = (tile < ntiles && kk < r)
                                   ? ((uint32_t)(cw + u * 16 + m) * (uint32_t)R + kk) * 2u
                                   : kOOB;
          if constexpr (K32) {
            bq[u][ks] = bload16(b_r, off);
          } else {
            const u32x2 v = bload8(b_r, off);
            bq[u][ks] = u32x4{v.x, v.y, 0u, 0u};
          }
        }
      }
      if (tid < kBMe) tok[tid] = tv;
      __syncthreads();

      // row-major y access: lane -> rows (lane >> 3) and 8 + (lane >> 3) of a
      // token tile, 16-byte piece (lane & 7) of the wave's 128-byte column span
      const bool pcol = (w * TPW + (ppc >> 1)) < ntiles;   // piece inside the chunk
      u32x4 yv[MT][2];
#pragma unroll
      for (int q = 0; q < MT; ++q)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int t = tok[q * 16 + prow + 8 * hh];
          // y rows are read once (streamed: gate/up -4.5 us; the decode's
          // y prefetch lost time with it)
          yv[q][hh] = bload16_once(y_r, (pcol && t >= 0)
                                       ? ((uint32_t)t * (uint32_t)out + cw + 8 * ppc) * 2u
                                       : kOOB);
        }

      // h rows of the block, 4 ranks per load (ranks at or past r are set to
      // zero; they are the block's own h columns, not adapter weights), scaled
      // and split hi + lo; all of a thread's loads are issued before any is used
      const float scale = scalings[s];
      constexpr int RQ = RP / 4;                    // 16-byte pieces per h row
      constexpr int HQ = (kBMe * RQ + 255) / 256;   // pieces per thread
      u32x4 hv[HQ];
#pragma unroll
      for (int k = 0; k < HQ; ++k) {
        const int idx = ltid + 256 * k;
        const int q = idx / RQ;
        const int j = (idx - q * RQ) * 4;
        const int t = q < kBMe ? tok[q] : -1;
        hv[k] = bload16(h_r, (t >= 0 && j < r) ? ((uint32_t)t * (uint32_t)SR + i * R + j) * 4u
                                               : kOOB);
      }
      // the next item's token ids: in flight while this item computes
      if (PERSIST && nitem < sc.total) tv = token_of(nit, nsv);
#pragma unroll
      for (int k = 0; k < HQ; ++k) {
        const int idx = ltid + 256 * k;
        const int q = idx / RQ;
        const int j = (idx - q * RQ) * 4;
        uint32_t hb[4], lb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = (j + e < r) ? __uint_as_float(hv[k][e]) * scale : 0.f;
          hb[e] = to_bf16_bits(v);
          lb[e] = to_bf16_bits(v - __uint_as_float(hb[e] << 16));
        }
        if (q < kBMe) {
          *(u32x2*)(hhi + q * RPS + j) = u32x2{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
          *(u32x2*)(hlo + q * RPS + j) = u32x2{lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16)};
        }
      }
      __syncthreads();

      // ranks past r in a live step are never used
#pragma unroll
      for (int u = 0; u < TPW; ++u)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int kk = ks * KW + kg * (KW / 4);
#pragma unroll
          for (int e = 0; e < (K32 ? 4 : 2); ++e) {
            const uint32_t mlo = (kk + 2 * e < r) ? 0xffffu : 0u;
            const uint32_t mhi = (kk + 2 * e + 1 < r) ? 0xffff0000u : 0u;
            bq[u][ks][e] &= mlo | mhi;
          }
        }

      auto half = [](u32x4 v, int p) {   // bf16 quadruple p (0 or 1) of a 16-byte piece
        return __builtin_bit_cast(s16x4, p ? u32x2{v.z, v.w} : u32x2{v.x, v.y});
      };
      const int mtl = (ntok + 15) / 16;   // token tiles holding tokens
#pragma unroll
      for (int q = 0; q < MT; ++q) {
        if (q >= mtl) break;
        u32x4 hq[KS], lq[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks >= ntr) break;
          const int off = (q * 16 + m) * RPS + ks * KW + kg * (KW / 4);
          if constexpr (K32) {
            hq[ks] = *(const u32x4*)(hhi + off);
            lq[ks] = *(const u32x4*)(hlo + off);
          } else {
            const u32x2 a = *(const u32x2*)(hhi + off);
            const u32x2 c = *(const u32x2*)(hlo + off);
            hq[ks] = u32x4{a.x, a.y, 0u, 0u};
            lq[ks] = u32x4{c.x, c.y, 0u, 0u};
          }
        }
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
          f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            if (ks >= ntr) break;
#pragma unroll
            for (int p = 0; p < (K32 ? 2 : 1); ++p) {
              o = mfma_k16(half(bq[u][ks], p), half(hq[ks], p), o);
              o = mfma_k16(half(bq[u][ks], p), half(lq[ks], p), o);
            }
          }
          // o[ii] = delta[token m][column 16u + 4kg + ii]
          *(f32x4*)(sw + m * SRW + u * 16 + kg * 4) = o;
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int row = prow + 8 * hh;
          const f32x4 d0 = *(const f32x4*)(sw + row * SRW + 8 * ppc);
          const f32x4 d1 = *(const f32x4*)(sw + row * SRW + 8 * ppc + 4);
          const u32x4 yy = yv[q][hh];
          const int t = tok[q * 16 + row];
          bstore16_out(y_r,
                       (pcol && t >= 0) ? ((uint32_t)t * (uint32_t)out + cw + 8 * ppc) * 2u
                                        : kOOB,
                       u32x4{pack_bf16x2(bf16lo(yy.x) + d0.x, bf16hi(yy.x) + d0.y),
                             pack_bf16x2(bf16lo(yy.y) + d0.z, bf16hi(yy.y) + d0.w),
                             pack_bf16x2(bf16lo(yy.z) + d1.x, bf16hi(yy.z) + d1.y),
                             pack_bf16x2(bf16lo(yy.w) + d1.z, bf16hi(yy.w) + d1.w)});
        }
        __builtin_amdgcn_wave_barrier();
      }
    } else if (PERSIST && nitem < sc.total) {
      tv = token_of(nit, nsv);   // a padding item: only the next item's tokens
    }
    if (!PERSIST || nitem >= sc.total) break;
    __syncthreads();   // tok, h and the staging tiles are reused
    item = nitem;
    it = nit;
    sv[0] = nsv[0];
    sv[1] = nsv[1];
    sv[2] = nsv[2];
  }
}

namespace {

// Workgroups of `threads` threads of `kernel` resident at once on the current
// device (all CUs), at least 8.
template <typename K>
int64_t resident_blocks(K kernel, int threads) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
    return 8;
  return std::max<int64_t>(8, (int64_t)cus * per_cu);
}

int rt_of(int R) {
  const int RT = (R + 15) / 16;
  return RT <= 1 ? 1 : RT <= 2 ? 2 : RT <= 4 ? 4 : RT <= 8 ? 8 : 16;
}

}  // namespace

bool sgmv_supported(int dtype, const SliceTable& st, int R, int T, int in) {
  if (dtype != kDtypeBF16 || R > 256) return false;
  const int64_t lim = (int64_t)1 << 31;
  const int64_t out = st.off[st.n];
  // x, y, one slot's A and B, and h (read through a buffer resource by the
  // expand) must each stay below 2 GiB
  if ((int64_t)T * in * 2 >= lim || (int64_t)T * out * 2 >= lim ||
      (int64_t)out * R * 2 >= lim || (int64_t)R * in * 2 >= lim ||
      (int64_t)T * st.n * R * 4 >= lim)
    return false;
  for (int i = 0; i < st.n; ++i)
    if ((st.off[i + 1] - st.off[i]) % 16 != 0) return false;
  return true;
}

int sgmv_kparts(int in) {
  // ~1024-deep parts, but at least 4 (each >= 256 deep) for a shallow `in`,
  // where one part per token block leaves too few items to fill the GPU:
  // measured on a TP=8 down share (in 1792, 8192 tokens): 1 part 66 us,
  // 4 parts 55 us, 8 parts 58 us. The workspace is sized for this count;
  // sgmv_kparts_for may launch fewer.
  const int kp = std::max(in / 1024, std::min(4, in / 256));
  return kp < 1 ? 1 : kp > 16 ? 16 : kp;
}

namespace {

// Compute units of the current device (cached per device); 0 if the runtime
// cannot say.
int device_cus() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  const auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 0;
  cache[dev] = cus;
  return cus;
}

}  // namespace

int sgmv_shrink_rt(int T, int slots, int S, int R) {
  // The rank tiles of R, or, for a batch of long segments (two or more
  // 128-token blocks per slot on average) whose slices fit one item together
  // (S x ceil(R / 16) <= 8 tiles), enough tiles for all of them: an item then
  // reads its x block once for every slice, and the items per K part are
  // the token blocks. Measured with 3 K parts (240 items) on the TP=8
  // gate/up share (two slices of rank 64): 70.7-71.5 us against 73.4-74.9
  // us with one item per slice (4 parts); prefill gate/up 217-223 against
  // 223 us.
  const int rt = rt_of(R);
  if ((int64_t)T < (int64_t)2 * kBMs * slots || S <= 1) return rt;
  const int tiles = S * ((R + 15) / 16);
  if (tiles > 8) return rt;
  int p = 1;
  while (p < tiles) p *= 2;
  return std::max(rt, p);
}

int sgmv_kparts_for(int T, int in, int slots, int S, int R) {
  // A batch of long segments whose items per K part (token blocks, bounded
  // by ceil(T / 128) + slots, times the slice groups of an item) number at
  // most half the compute units: as many K parts as keep every item on a
  // compute unit of its own (at most sgmv_kparts(in)). A few more items than
  // compute units leaves a second, short round on a few of them. Measured
  // at 8192 tokens over 16 slots (<= 80 blocks, so 3 parts on 256 compute
  // units), apply per launch: down (in 14336) 95.6-96.3 us against
  // 101.0-101.6 us with 14 parts (4 parts 111 us, 6 parts 97.4 us); in 1792
  // (the TP=8 down share) 52.3-52.5 against 54.7-54.9 us with 4; in 4096 to
  // 12288 3 parts best too. With two slices in separate items (480 items at
  // 3 parts) the TP=8 gate/up share lost 1 us against 4 parts.
  const int kmax = sgmv_kparts(in);
  if ((int64_t)T < (int64_t)2 * kBMs * slots) return kmax;
  const int cus = device_cus();
  const int rt = sgmv_shrink_rt(T, slots, S, R);
  const int ntr = (R + 15) / 16;
  const int groups = rt >= S * ntr ? 1 : S;
  const int64_t per_part = (((int64_t)T + kBMs - 1) / kBMs + slots) * groups;
  if (cus <= 0 || 2 * per_part > cus) return kmax;
  return (int)std::min<int64_t>(kmax, cus / per_part);
}

hipError_t launch_sgmv_shrink(const void* x, int T, int in, const void* a, int slots, int S,
                              int R, const int32_t* order, const int32_t* indptr,
                              const int32_t* ranks, float* h, float* parts, int kparts,
                              int min_len, hipStream_t stream) {
  if (T <= min_len) return hipSuccess;   // no segment can be long enough
  if (kparts < 1 || (kparts > 1 && !parts)) return hipErrorInvalidValue;
  const int64_t stride = (int64_t)T * S * R;
  const int64_t items = (int64_t)S * kparts * ((T + kBMs - 1) / kBMs + slots);
  const int64_t grid = 8 * ((items + 7) / 8);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  float* dst = kparts > 1 ? parts : h;
  // slices per item at most: their A rows must stay below 2 GiB
  const int64_t slice_bytes = (int64_t)R * in * 2;
  const int gmax = (int)std::max<int64_t>(1, std::min<int64_t>(S, (((int64_t)1 << 31) - 1) /
                                                                       slice_bytes));
#define L(RTV)                                                                                 \
  do {                                                                                         \
    constexpr int lds = ShrinkRing<RTV>::kBytes;                                               \
    if (lds > 65536) {                                                                         \
      const hipError_t e = hipFuncSetAttribute((const void*)k_sgmv_shrink<RTV>,                \
                                               hipFuncAttributeMaxDynamicSharedMemorySize, lds); \
      if (e != hipSuccess) return e;                                                           \
    }                                                                                          \
    hipLaunchKernelGGL(k_sgmv_shrink<RTV>, dim3((unsigned)grid), dim3(512), lds, stream, x, T, \
                       in, a, slots, S, R, order, indptr, ranks, dst, kparts, stride, min_len, \
                       gmax);                                                                  \
  } while (0)
  switch (sgmv_shrink_rt(T, slots, S, R)) {
    case 1: L(1); break;
    case 2: L(2); break;
    case 4: L(4); break;
    case 8: L(8); break;
    default: L(16); break;
  }
#undef L
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || kparts == 1) return e;
  const int64_t n = (int64_t)T * (S * R / 4);
  hipLaunchKernelGGL(k_sum_parts, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, parts,
                     kparts, stride, h, T, S * R, slots, R, order, indptr, ranks, min_len);
  return hipGetLastError();
}

hipError_t launch_sgmv_expand(void* y, int T, const SliceTable& st, const float* h, const void* b,
                              int slots, int R, const int32_t* order, const int32_t* indptr,
                              const int32_t* ranks, const float* scalings, int min_len,
                              hipStream_t stream) {
  if (T <= min_len) return hipSuccess;
  int nck = 0;
  for (int i = 0; i < st.n; ++i) nck += (st.off[i + 1] - st.off[i] + kCC - 1) / kCC;
  const int64_t items = (int64_t)((nck + 7) & ~7) * ((T + kBMe - 1) / kBMe + slots);
  if (items > 0x7fffffff) return hipErrorInvalidValue;
  // fewer than two token blocks per slot on average: most items are short and
  // one resident round of workgroups (a multiple of 8) loops over them
  const bool persist = (int64_t)T < (int64_t)2 * kBMe * slots;
#define L(RTV)                                                                                 \
  do {                                                                                         \
    if (persist) {                                                                             \
      const int64_t grid =                                                                     \
          8 * ((std::min<int64_t>(items, resident_blocks(k_sgmv_expand<RTV, true>, 256)) + 7) / \
               8);                                                                             \
      hipLaunchKernelGGL((k_sgmv_expand<RTV, true>), dim3((unsigned)grid), dim3(256), 0,       \
                         stream, y, T, st, h, b, slots, R, order, indptr, ranks, scalings,     \
                         min_len);                                                             \
    } else {                                                                                   \
      hipLaunchKernelGGL((k_sgmv_expand<RTV, false>), dim3((unsigned)(8 * ((items + 7) / 8))),  \
                         dim3(256), 0, stream, y, T, st, h, b, slots, R, order, indptr, ranks,  \
                         scalings, min_len);                                                   \
    }                                                                                          \
  } while (0)
  switch (rt_of(R)) {
    case 1: L(1); break;
    case 2: L(2); break;
    case 4: L(4); break;
    case 8: L(8); break;
    default: L(16); break;
  }
#undef L
  return hipGetLastError();
}

}  // namespace lora
