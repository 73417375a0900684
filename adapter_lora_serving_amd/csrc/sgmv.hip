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
//   part). Eight waves; wave w owns token tile w against every rank tile.
//   Its x rows go straight from HBM into registers a few 64-element chunks
//   ahead; A's chunk is shared through a double-buffered LDS tile. A slot
//   whose rank needs fewer rank tiles than the kernel holds takes several
//   slices in one item (their tiles side by side), so its x block is read
//   once for all of them. Rows of A at or past the rank read as zeros
//   without a memory access. With several K parts each item writes a
//   partial h and a second kernel sums the parts.
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

namespace lora {

namespace {

constexpr int kBMe = 64;      // tokens per expand item
constexpr int kCC = 256;      // output columns per expand item
constexpr int kKC = 64;       // K elements per staged chunk
constexpr int kRowB = kKC * 2 + 16;   // padded LDS row (bytes)

}  // namespace

// ---------------------------------------------------------------------------
// shrink
// ---------------------------------------------------------------------------
// Item: (slot, block of 128 tokens, slice group, K part). Eight waves, wave w
// owns token tile w (16 tokens) against every rank tile, so its x rows are
// its own (read into registers D chunks ahead) and only A is shared: A's
// chunk [RP x 64] goes through a register ring D chunks ahead into a
// double-buffered LDS tile. A is thus re-read from L2 once per 128 tokens.
// A slot of rank r uses ntr = ceil(r / 16) rank tiles per slice; a group
// packs g = min(S, RT / ntr, gmax) slices, slice j of the group on tiles
// [j * ntr, (j + 1) * ntr). gmax keeps a group's A rows below 2 GiB.
// With kparts > 1 each item writes its partial h to its own buffer
// (hout + kp * part_stride); k_sum_parts adds them in kp order. Every item
// writes the columns of its slices below 16 * ntr.
constexpr int kBMs = 128;
constexpr int kD = 4;

// Slices per item for a slot of rank r (r > 0) in a kernel of RT rank tiles.
__device__ __forceinline__ int shrink_group(int r, int RT, int S, int gmax) {
  const int ntr = (r + 15) / 16;
  return max(1, min(min(S, RT / ntr), gmax));
}

template <int RT>
// Six waves per SIMD (three workgroups per CU) keep a prefill batch's items
// resident in one round, so no item starts after the first round ends; at 16
// rank tiles the LDS allows two workgroups per CU, so four waves per SIMD
// (128 VGPRs) are enough and keep the accumulators in registers.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(RT >= 16 ? 4 : 6))) void k_sgmv_shrink(
    const void* __restrict__ x_, int T, int in, const void* __restrict__ a_, int slots, int S,
    int R, const int32_t* __restrict__ order, const int32_t* __restrict__ indptr,
    const int32_t* __restrict__ ranks, float* __restrict__ hout, int kparts,
    int64_t part_stride, int min_len, int gmax) {
  constexpr int RP = RT * 16;
  constexpr int AL = RP >= 64 ? RP / 64 : 1;   // A pieces per thread per chunk
  // chunks in flight: 2 from 4 rank tiles up (measured at 4: prefill down
  // 106 -> 101 us against 3; at 8 a third chunk more than doubled the skewed
  // mix's time)
  constexpr int D = RT >= 4 ? 2 : kD;
  // XL: x rows are loaded as 8 rows x 128 contiguous bytes per instruction
  // and turned into the MFMA operand layout through a per-wave LDS tile
  // (16 rows x 64 bytes per instruction otherwise); the tile's 18 KB would
  // cost a workgroup per CU at the largest ranks, so those load directly
  constexpr bool XL = RT <= 4;
  __shared__ int scratch[24];
  __shared__ int tok[kBMs];
  __shared__ __attribute__((aligned(16))) char as[2][RP * kRowB];
  __shared__ __attribute__((aligned(16))) char xs[XL ? 8 : 1][XL ? 16 * kRowB : 16];

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
  // the token ids are the oldest loads in flight; the first A chunks (which
  // do not depend on them) are issued next, then the ids are waited for
  const int tv = token_at(order, seg0 + mb * kBMs + min(tid, ntok - 1), T);

  const rsrc_t x_r = make_rsrc(x_, (uint32_t)T * (uint32_t)in * 2u);
  // the group's A rows: slices i0 .. i0 + gsz - 1 of the slot
  const rsrc_t a_r = make_rsrc((const char*)a_ + ((int64_t)s * S + i0) * R * in * 2,
                               (uint32_t)gsz * (uint32_t)R * (uint32_t)in * 2u);
  const uint32_t rowG = (uint32_t)in * 2u;
  const int nchT = (in + kKC - 1) / kKC;
  const int cbeg = (int)((int64_t)nchT * kp / kparts);
  const int cend = (int)((int64_t)nchT * (kp + 1) / kparts);
  const int nch = cend - cbeg;

  const int m = lane & 15;
  const int kg = lane >> 4;
  const int arow = tid >> 3;        // 0..63 (+64 per extra piece)
  const int apc = tid & 7;
  // LDS tile row v holds row v % (16 ntr) of slice v / (16 ntr) of the group
  uint32_t abase[AL];
#pragma unroll
  for (int q = 0; q < AL; ++q) {
    const int v = arow + 64 * q;
    const int j = v / (16 * ntr);
    const int rr = v - j * 16 * ntr;
    abase[q] = (v < RP && j < gsz && rr < r) ? (uint32_t)(j * R + rr) * rowG : kOOB;
  }

  u32x4 xr[D][2];
  u32x4 ar[D][AL];
  auto issue_a = [&](int slot, int c) {   // A loads of chunk c (relative) into ring slot
    const bool cv = c < nch;
    const uint32_t kb = (uint32_t)(cbeg + c) * (kKC * 2u);
#pragma unroll
    for (int q = 0; q < AL; ++q) {
      const uint32_t e = (uint32_t)((cbeg + c) * kKC + apc * 8);
      ar[slot][q] = bload16(a_r, (cv && abase[q] != kOOB && e < (uint32_t)in)
                                     ? abase[q] + kb + apc * 16u
                                     : kOOB);
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) issue_a(d, d);
  if (tid < kBMs) tok[tid] = tid < ntok ? tv : -1;
  __syncthreads();
  // x rows of this lane: XL: rows xq and xq + 8 of the wave's 16 tokens,
  // 16-byte piece xp of the chunk; else row m, pieces kg and 4 + kg
  const int xq = lane >> 3;
  const int xp = lane & 7;
  uint32_t xrow[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int t = tok[w * 16 + (XL ? xq + 8 * hh : m)];
    xrow[hh] = t >= 0 ? (uint32_t)t * rowG : kOOB;
  }
  auto issue_x = [&](int slot, int c) {   // x loads of chunk c (relative) into ring slot
    const bool cv = c < nch;
    const uint32_t kb = (uint32_t)(cbeg + c) * (kKC * 2u);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int ke = XL ? xp * 8 : hh * 32 + kg * 8;   // element offset in the chunk
      const uint32_t e = (uint32_t)((cbeg + c) * kKC + ke);
      xr[slot][hh] = bload16(x_r, (cv && xrow[hh] != kOOB && e < (uint32_t)in)
                                      ? xrow[hh] + kb + (uint32_t)ke * 2u
                                      : kOOB);
    }
  };
  auto stage = [&](int slot, int buf) {   // A chunk in ring slot -> LDS buffer
#pragma unroll
    for (int q = 0; q < AL; ++q) {
      const int row = arow + 64 * q;
      if (row < RP) *(u32x4*)(as[buf] + row * kRowB + apc * 16) = ar[slot][q];
    }
  };

  f32x4 acc[RT];
#pragma unroll
  for (int nt = 0; nt < RT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int d = 0; d < D; ++d) issue_x(d, d);
  stage(0, 0);
  __syncthreads();
#pragma unroll 1
  for (int c0 = 0; c0 < nch; c0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int c = c0 + d;
      if (c < nch) {
        if (c + 1 < nch) stage((d + 1) % D, (c + 1) & 1);
        const char* ab = as[c & 1];
        if constexpr (XL) {
          *(u32x4*)(xs[w] + xq * kRowB + xp * 16) = xr[d][0];
          *(u32x4*)(xs[w] + (xq + 8) * kRowB + xp * 16) = xr[d][1];
          __builtin_amdgcn_wave_barrier();
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 xa;
          if constexpr (XL)
            xa = __builtin_bit_cast(bf16x8,
                                    *(const u32x4*)(xs[w] + m * kRowB + (ks * 32 + kg * 8) * 2));
          else
            xa = __builtin_bit_cast(bf16x8, xr[d][ks]);
#pragma unroll
          for (int nt = 0; nt < RT; ++nt) {
            // tiles past the group's rows hold only zeros (16 tiles take a
            // guard instead of an early exit, so that the loop unrolls)
            if (RT < 16 && nt >= live) break;
            if (nt < live) {
              const bf16x8 av = __builtin_bit_cast(
                  bf16x8, *(const u32x4*)(ab + (nt * 16 + m) * kRowB + (ks * 32 + kg * 8) * 2));
              acc[nt] = mfma_k32(xa, av, acc[nt]);
            }
          }
        }
        issue_a(d, c + D);
        issue_x(d, c + D);
        __syncthreads();
      }
    }
  }

  // lane (m, kg) holds h[token w*16 + 4kg + ii][slice i0 + nt / ntr, rank
  // (nt % ntr) * 16 + m]
  const int SR = S * R;
  float* hp = hout + (int64_t)kp * part_stride;
  if constexpr (RT < 16) {
#pragma unroll
    for (int nt = 0; nt < RT; ++nt) {
      if (nt >= live) break;
      const int j = nt / ntr;
      const int rr = (nt - j * ntr) * 16 + m;
      if (rr < R) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int tt = tok[w * 16 + 4 * kg + ii];
          if (tt >= 0) hp[(int64_t)tt * SR + (i0 + j) * R + rr] = acc[nt][ii];
        }
      }
    }
  } else {   // 16 tiles: no early exit, so that the loop unrolls
    int j = 0, rt = 0;   // slice in the group and rank tile of tile nt
#pragma unroll
    for (int nt = 0; nt < RT; ++nt) {
      const int rr = rt * 16 + m;
      if (nt < live && rr < R) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int tt = tok[w * 16 + 4 * kg + ii];
          if (tt >= 0) hp[(int64_t)tt * SR + (i0 + j) * R + rr] = acc[nt][ii];
        }
      }
      if (++rt == ntr) { rt = 0; ++j; }
    }
  }
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
  // 4 parts 55 us, 8 parts 58 us
  const int kp = std::max(in / 1024, std::min(4, in / 256));
  return kp < 1 ? 1 : kp > 16 ? 16 : kp;
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
  hipLaunchKernelGGL(k_sgmv_shrink<RTV>, dim3((unsigned)grid), dim3(512), 0, stream, x, T, in, \
                     a, slots, S, R, order, indptr, ranks, dst, kparts, stride, min_len, gmax)
  switch (rt_of(R)) {
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
