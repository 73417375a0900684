// Fused shrink + expand for bf16 targets (lora_apply_linear) of a small
// batch (fewer than 1024 tokens; larger batches run the segment-tiled
// kernels), on bf16 MFMA.
//
// Follows the mstar lora.backend page, LoraBackend.apply_linear_ ("a backend
// may fuse them"): the result is that of shrink (h = x @ A^T, per token's
// slot) followed by expand (y += scaling * h @ B^T per fused slice), with h
// kept in fp32 and never written to memory.
//
// Work (one 512-thread workgroup per piece or item):
//  * decode pieces, for segments of at most 16 tokens. A shrink piece
//    (slot, slice, K part) forms the partial product of the slot's tokens
//    with the slice's A rows over its part of `in` and stores it as a 16 x RP
//    fp32 tile in the workspace; an expand piece (slot, column chunk of one
//    slice) prefetches its B tile and y rows, waits for the slice's KP
//    partial tiles (a counter handoff, described below), adds them in a
//    fixed order, and expands its chunk. No byte of A or B is read twice.
//  * prefill items, for longer segments: (slot, block of 16 tokens) over
//    every slice and output column; h of the block stays in LDS.
// Shrink: K is split across the 8 waves; each wave accumulates a 16x16 tile
//   (tokens x A rows) per 16 rank rows on bf16 MFMA, and the waves' partial
//   tiles are added in a fixed order through LDS. Rows of A at or past the
//   rank, padding tokens and a partial last K step read as zeros through the
//   buffer range check.
// Expand: y^T tile [16 columns x 16 tokens] = B_tile [16 x r] . H^T, with H
//   (already multiplied by the slot's scaling) split into bf16 hi + lo parts,
//   two v_mfma_f32_16x16x16_bf16 per 16 ranks and fp32 accumulation, so h is
//   effectively fp32. Each lane then owns 4 consecutive columns of one token
//   and rounds y once (nearest-even). B ranks at or past the rank are zeroed
//   in registers.
#include "lora_common.h"
#include "lora_kernels.h"

#include <stdlib.h>

namespace lora {

namespace {


constexpr int kMT = 16;               // tokens per block (MFMA M / N tile)


// LDS layout of one workgroup of NW waves (bytes):
//   [0, 64)        tok[16]     token index per block row, -1 for padding
//   [64, 160)      scratch[24] block scan scratch
//   [256, ...)     red[NW][16][RP] fp32   per-wave partial h tiles
//   then           hhi[16][RPS], hlo[16][RPS] bf16 (RPS = RP + 4)
template <int RT, int NW>
struct Lds {
  static constexpr int RP = RT * 16;
  static constexpr int RPS = RP + 4;
  static constexpr int kRed = 256;
  static constexpr int kHhi = kRed + NW * kMT * RP * 4;
  static constexpr int kHlo = kHhi + kMT * RPS * 2;
  static constexpr int kBytes = kHlo + kMT * RPS * 2;
};

// Sum the NW partial tiles in a fixed order, apply the scaling and split into
// bf16 hi + lo parts (hi = RNE(v), lo = RNE(v - hi)).
template <int RT, int NW>
__device__ __forceinline__ void reduce_split(const float* red, float scale, uint16_t* hhi,
                                             uint16_t* hlo, int tid) {
  constexpr int RP = RT * 16;
  constexpr int RPS = RP + 4;
  for (int idx = tid; idx < kMT * RP; idx += NW * kWave) {
    float v = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) v += red[ww * kMT * RP + idx];
    v *= scale;
    const uint32_t hb = to_bf16_bits(v);
    const uint32_t lb = to_bf16_bits(v - __uint_as_float(hb << 16));
    const int q = idx / RP;
    const int j = idx - q * RP;
    hhi[q * RPS + j] = (uint16_t)hb;
    hlo[q * RPS + j] = (uint16_t)lb;
  }
}

// Load the 4 B ranks kk..kk+3 of column c, the A operand of the expand MFMA
// (zero when the whole group is at or past r). The value is not inspected
// here, so no wait is forced at the load; mask_b4 clears ranks at or past r
// where the operand is used.
__device__ __forceinline__ s16x4 load_b4(const char* __restrict__ bslot, int64_t brow, int c,
                                         int kk, int r) {
  s16x4 v = s16x4{0, 0, 0, 0};
  if (kk < r) v = *(const s16x4*)(bslot + (int64_t)c * brow + kk * 2);
  return v;
}
__device__ __forceinline__ s16x4 mask_b4(s16x4 v, int kk, int r) {
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (kk + e < r) ? v[e] : (short)0;   // never used past r
  return v;
}

// y[t][c .. c+3] += acc (one rounding to bf16), the lane's 4 columns of a tile.
__device__ __forceinline__ void update_y4(char* __restrict__ y, int64_t off, u32x2 yv, f32x4 acc) {
  const float y0 = bf16lo(yv.x) + acc[0];
  const float y1 = bf16hi(yv.x) + acc[1];
  const float y2 = bf16lo(yv.y) + acc[2];
  const float y3 = bf16hi(yv.y) + acc[3];
  *(u32x2*)(y + off) = u32x2{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
}

// y[tok][c] += sum_j B[c][j] * (hhi + hlo)[tok][j] for columns [lo, hi) of the
// current slice (lo, hi multiples of 16).
template <int RT, int NW>
__device__ __forceinline__ void expand_range(char* __restrict__ y, int out, const int* tok,
                                             const char* __restrict__ bslot, int R, int r, int lo,
                                             int hi, const uint16_t* hhi, const uint16_t* hlo,
                                             int lane, int w) {
  constexpr int RPS = RT * 16 + 4;
  constexpr int U = RT <= 4 ? 4 : RT <= 8 ? 2 : 1;   // column tiles in flight per wave
  const int m = lane & 15;
  const int kg = lane >> 4;
  const int t = tok[m];
  s16x4 hb[RT], lb[RT];
#pragma unroll
  for (int ks = 0; ks < RT; ++ks) {
    hb[ks] = *(const s16x4*)(hhi + m * RPS + ks * 16 + kg * 4);
    lb[ks] = *(const s16x4*)(hlo + m * RPS + ks * 16 + kg * 4);
  }
  const int64_t brow = (int64_t)R * 2;
  const int64_t yrow = (int64_t)out * 2;
  const int ntiles = (hi - lo) / 16;
  for (int tile0 = w * U; tile0 < ntiles; tile0 += NW * U) {
    s16x4 bv[U][RT];
    u32x2 yv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = lo + (tile0 + u) * 16;
      const bool tv = (tile0 + u) < ntiles;
#pragma unroll
      for (int ks = 0; ks < RT; ++ks)
        bv[u][ks] = tv ? load_b4(bslot, brow, c + m, ks * 16 + kg * 4, r) : s16x4{0, 0, 0, 0};
      yv[u] = u32x2{0u, 0u};
      if (tv && t >= 0) yv[u] = *(const u32x2*)(y + (int64_t)t * yrow + (int64_t)(c + 4 * kg) * 2);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if ((tile0 + u) >= ntiles) break;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < RT; ++ks) {
        if (ks * 16 >= r) break;
        const s16x4 b4 = mask_b4(bv[u][ks], ks * 16 + kg * 4, r);
        acc = mfma_k16(b4, hb[ks], acc);
        acc = mfma_k16(b4, lb[ks], acc);
      }
      if (t >= 0) {
        const int c = lo + (tile0 + u) * 16;
        update_y4(y, (int64_t)t * yrow + (int64_t)(c + 4 * kg) * 2, yv[u], acc);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// decode path (segments of at most 16 tokens)
//
// Work is split so that no byte is read twice and every CU gets a share:
//  * shrink pieces (slot s, slice i, K part kp): the partial product of the
//    slot's <= 16 tokens with A's rows of slice i over one part of `in`,
//    written as a 16 x RP fp32 tile to the workspace;
//  * expand pieces (slot s, column chunk c of slice i): prefetch their B
//    tiles and y rows, wait until the KP partial tiles of (s, i) are there,
//    add them in kp order (deterministic), scale, split into bf16 hi + lo and
//    expand.
// Handoff: every expand piece (s, c) owns a counter pair {count, base}. Each
// shrink piece of (s, i), once its partial tile is stored, adds 1 to the
// count of every chunk of slice i; the expand piece waits until
// count - base >= KP and then advances base by KP, so nothing is ever reset
// and the pairs stay consistent across calls of any shape (count and base of
// a chunk advance by the same KP in every call that uses it).
// Memory ordering: the partial tiles are written and read only with
// agent-scope atomic stores and loads, which are coherent across the XCDs
// (they are performed at the device coherence point, not in an XCD's L2);
// each producer waits for its stores to complete (s_waitcnt vmcnt(0)) before
// the workgroup barrier that precedes the count update, and consumers issue
// the tile loads only after observing the count. No L2 writeback is needed
// because no plain (non-atomic) store is read across workgroups.
// The wait is bounded: a piece that times out (its producers not resident,
// e.g. the GPU shared with other work) computes the slice's h itself and
// still advances its base, so the kernel always finishes with the right
// result and the counters stay consistent.
// ---------------------------------------------------------------------------

struct DecodeArgs {
  rsrc_t x_r, y_r;
  const int32_t* tokp;
  int T, in, out, R;
  int KP;
  int spin_limit;
};

// Token id of lane row m: one vector load per lane (index clamped into the
// array). Issued before the bulk A / B loads, it is the oldest load in
// flight, so the first use of the id waits for it alone (vector loads
// complete in order), not for the bulk loads issued after it.
__device__ __forceinline__ int lane_token(const int32_t* __restrict__ tokp, int T, int seg0,
                                          int m) {
  return tokp[min(seg0 + m, T - 1)];
}

// acc[nt] += x_block . A_rows(nt)^T for the first NT rank tiles, over K
// steps [s0, s1) of 32 elements; this wave takes steps s0 + w*U + (NW*U)*j + u.
// All U*(NT+1) loads of an iteration are issued before its products, and
// none is conditional: rows at or past the rank, padding tokens and k past
// `in` read as zeros through the buffer range check (kOOB).
template <int NT, int NW, class XRow>
__device__ __forceinline__ void shrink_steps_n(rsrc_t x_r, rsrc_t a_r, uint32_t rowA, int in,
                                               XRow xrow_of, int s0, int s1, f32x4* acc,
                                               int m, int kg, int w) {
  // K steps in flight per wave; 2 or more below 16 tiles, so the two
  // 64-byte halves of a 128-byte line of a row are read by the same wave
  // (16 tiles would not fit the registers twice)
  constexpr int U = NT <= 1 ? 8 : NT <= 2 ? 4 : NT <= 8 ? 2 : 1;
  int st0 = s0 + w * U;
  if (st0 >= s1) return;
  bf16x8 av[U][NT];
  bf16x8 xa[U];
  auto load_a = [&](int st) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (st + u) * 32 + kg * 8;
      const bool kv = (st + u) < s1 && k < in;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        av[u][nt] = __builtin_bit_cast(
            bf16x8, bload16(a_r, kv ? (uint32_t)(nt * 16 + m) * rowA + (uint32_t)k * 2u : kOOB));
    }
  };
  auto load_x = [&](int st, uint32_t xrow) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (st + u) * 32 + kg * 8;
      const bool kv = (st + u) < s1 && k < in && xrow != kOOB;
      xa[u] = __builtin_bit_cast(bf16x8, bload16(x_r, kv ? xrow + (uint32_t)k * 2u : kOOB));
    }
  };
  auto products = [&]() {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma_k32(xa[u], av[u][nt], acc[nt]);
  };
  // first iteration: A is requested before the x row offset is formed, so
  // the token id's latency overlaps the A loads
  load_a(st0);
  const uint32_t xrow = xrow_of();
  load_x(st0, xrow);
  products();
  for (st0 += NW * U; st0 < s1; st0 += NW * U) {
    load_a(st0);
    load_x(st0, xrow);
    products();
  }
}

// acc[nt] += x_block . A_rows(nt)^T over K steps [s0, s1) for the rank tiles
// that hold rows below r, rounded up to a power of two (so at most twice the
// products are formed, and tiles past r add zeros). One loop per tile count:
// the tile count is uniform, so the choice is a scalar branch taken once, and
// the loop bodies hold no per-tile conditions. xrow() gives the byte offset of
// the lane's x row, or kOOB for a padding token.
template <int RT, int NW, class XRow>
__device__ __forceinline__ void shrink_steps(rsrc_t x_r, rsrc_t a_r, uint32_t rowA, int in,
                                             int r, XRow xrow, int s0, int s1,
                                             f32x4 (&acc)[RT], int m, int kg, int w) {
  const int ntr = (r + 15) >> 4;
  if constexpr (RT >= 16) {
    if (ntr > 8) return shrink_steps_n<16, NW>(x_r, a_r, rowA, in, xrow, s0, s1, acc, m, kg, w);
  }
  if constexpr (RT >= 8) {
    if (ntr > 4) return shrink_steps_n<8, NW>(x_r, a_r, rowA, in, xrow, s0, s1, acc, m, kg, w);
  }
  if constexpr (RT >= 4) {
    if (ntr > 2) return shrink_steps_n<4, NW>(x_r, a_r, rowA, in, xrow, s0, s1, acc, m, kg, w);
  }
  if constexpr (RT >= 2) {
    if (ntr > 1) return shrink_steps_n<2, NW>(x_r, a_r, rowA, in, xrow, s0, s1, acc, m, kg, w);
  }
  shrink_steps_n<1, NW>(x_r, a_r, rowA, in, xrow, s0, s1, acc, m, kg, w);
}

template <int RT>
__device__ __forceinline__ void store_partial(float* dst, const f32x4 (&acc)[RT], int m,
                                              int kg) {
  constexpr int RP = RT * 16;
#pragma unroll
  for (int nt = 0; nt < RT; ++nt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) dst[(4 * kg + ii) * RP + nt * 16 + m] = acc[nt][ii];
}

// Loads of group g of a chunk's expand tiles: wave w takes tiles
// w + NW*(g*PT + u), u < PT; B ranks at or past r and tiles past the chunk
// read as zeros (kOOB), y rows of padding tokens too.
template <int RT, int NW, int PT>
__device__ __forceinline__ void load_expand_group(rsrc_t b_r, rsrc_t y_r, int R, int r, int lo,
                                                  int ntiles, bool live, uint32_t yrow, int g,
                                                  s16x4 (&bv)[PT][RT], u32x2 (&yv)[PT], int m,
                                                  int kg, int w) {
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int tile = w + NW * (g * PT + u);
#pragma unroll
    for (int ks = 0; ks < RT; ++ks) {
      const int kk = ks * 16 + kg * 4;
      const uint32_t off = (tile < ntiles && kk < r)
                               ? ((uint32_t)(lo + tile * 16 + m) * (uint32_t)R + kk) * 2u
                               : kOOB;
      bv[u][ks] = __builtin_bit_cast(s16x4, bload8(b_r, off));
    }
  }
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int tile = w + NW * (g * PT + u);
    yv[u] = bload8(y_r, (live && tile < ntiles) ? yrow + (uint32_t)(lo + tile * 16 + 4 * kg) * 2u
                                                : kOOB);
  }
}

// Products and y update of group g from its loaded tiles.
template <int RT, int NW, int PT>
__device__ __forceinline__ void expand_group(rsrc_t y_r, int r, int lo, int ntiles, bool live,
                                             uint32_t yrow, int g, const s16x4 (&bv)[PT][RT],
                                             const u32x2 (&yv)[PT], const s16x4 (&hb)[RT],
                                             const s16x4 (&lb)[RT], int kg, int w) {
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int tile = w + NW * (g * PT + u);
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < RT; ++ks) {
      if (ks * 16 >= r) break;
      const s16x4 b4 = mask_b4(bv[u][ks], ks * 16 + kg * 4, r);
      o = mfma_k16(b4, hb[ks], o);
      o = mfma_k16(b4, lb[ks], o);
    }
    const uint32_t off = (live && tile < ntiles)
                             ? yrow + (uint32_t)(lo + tile * 16 + 4 * kg) * 2u
                             : kOOB;
    const u32x2 yy = yv[u];
    bstore8_out(y_r, off,
            u32x2{pack_bf16x2(bf16lo(yy.x) + o[0], bf16hi(yy.x) + o[1]),
                  pack_bf16x2(bf16lo(yy.y) + o[2], bf16hi(yy.y) + o[3])});
  }
}

// Expand of a whole chunk once hhi / hlo hold the block's h: group 0 is
// already loaded (bv0, yv0); each later group's loads are issued before the
// products of the group before it (two register sets in turn), so a wide
// chunk costs one load latency, not one per group.
template <int RT, int NW, int PT>
__device__ __forceinline__ void expand_chunk(rsrc_t b_r, rsrc_t y_r, int R, int r, int lo,
                                             int ntiles, bool live, uint32_t yrow,
                                             s16x4 (&bv0)[PT][RT], u32x2 (&yv0)[PT],
                                             const uint16_t* hhi, const uint16_t* hlo, int m,
                                             int kg, int w) {
  constexpr int RPS = RT * 16 + 4;
  s16x4 hb[RT], lb[RT];
#pragma unroll
  for (int ks = 0; ks < RT; ++ks) {
    hb[ks] = *(const s16x4*)(hhi + m * RPS + ks * 16 + kg * 4);
    lb[ks] = *(const s16x4*)(hlo + m * RPS + ks * 16 + kg * 4);
  }
  const int ngroups = (ntiles + NW * PT - 1) / (NW * PT);
  if constexpr (RT <= 2) {
    // small ranks: a decode chunk is one group (NW * PT tiles); a wider one
    // (a tuning override) takes its further groups one after another
    expand_group<RT, NW, PT>(y_r, r, lo, ntiles, live, yrow, 0, bv0, yv0, hb, lb, kg, w);
    for (int g = 1; g < ngroups; ++g) {
      load_expand_group<RT, NW, PT>(b_r, y_r, R, r, lo, ntiles, live, yrow, g, bv0, yv0, m, kg,
                                    w);
      expand_group<RT, NW, PT>(y_r, r, lo, ntiles, live, yrow, g, bv0, yv0, hb, lb, kg, w);
    }
    return;
  }
  s16x4 bv1[PT][RT];
  u32x2 yv1[PT];
  for (int g = 0; g < ngroups; g += 2) {
    if (g + 1 < ngroups)
      load_expand_group<RT, NW, PT>(b_r, y_r, R, r, lo, ntiles, live, yrow, g + 1, bv1, yv1, m,
                                    kg, w);
    expand_group<RT, NW, PT>(y_r, r, lo, ntiles, live, yrow, g, bv0, yv0, hb, lb, kg, w);
    if (g + 1 < ngroups) {
      if (g + 2 < ngroups)
        load_expand_group<RT, NW, PT>(b_r, y_r, R, r, lo, ntiles, live, yrow, g + 2, bv0, yv0, m,
                                      kg, w);
      expand_group<RT, NW, PT>(y_r, r, lo, ntiles, live, yrow, g + 1, bv1, yv1, hb, lb, kg, w);
    }
  }
}

// Shrink piece (s, i, kp).
template <int RT, int NW>
__device__ __forceinline__ void shrink_piece(const DecodeArgs& d, rsrc_t a_r, int r, int seg0,
                                             int n, float* part_out, int2* pairs, int nchunks,
                                             int kp, float* red, int lane, int w, int tid) {
  constexpr int RP = RT * 16;
  const int m = lane & 15;
  const int kg = lane >> 4;
  const int t = lane_token(d.tokp, d.T, seg0, m);
  const bool live = m < n;
  const uint32_t rowA = (uint32_t)d.in * 2u;
  const int steps = (d.in + 31) / 32;
  const int s0 = (int)((int64_t)steps * kp / d.KP);
  const int s1 = (int)((int64_t)steps * (kp + 1) / d.KP);
  f32x4 acc[RT];
#pragma unroll
  for (int nt = 0; nt < RT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  shrink_steps<RT, NW>(
      d.x_r, a_r, rowA, d.in, r, [&] { return live ? (uint32_t)t * rowA : kOOB; }, s0, s1, acc,
      m, kg, w);
  store_partial<RT>(red + w * kMT * RP, acc, m, kg);
  __syncthreads();
  for (int idx = tid; idx < kMT * RP; idx += NW * kWave) {
    float v = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) v += red[ww * kMT * RP + idx];
    __hip_atomic_store(part_out + idx, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);   // this thread's tile stores have completed
  __syncthreads();
  if (tid < nchunks)
    __hip_atomic_fetch_add(&pairs[tid].x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Expand piece (s, chunk [lo, hi) of slice i).
template <int RT, int NW>
__device__ __forceinline__ void expand_piece(const DecodeArgs& d, rsrc_t a_r, rsrc_t b_r, int r,
                                             float scale, int seg0, int n, int lo, int hi,
                                             const float* part_in, int2* pair, float* red,
                                             uint16_t* hhi, uint16_t* hlo, int* flag, int lane,
                                             int w, int tid) {
  constexpr int RP = RT * 16;
  constexpr int RPS = RP + 4;
  constexpr int PT = RT <= 2 ? 8 : RT <= 4 ? 4 : RT <= 8 ? 2 : 1;   // tiles per wave in flight
  const int m = lane & 15;
  const int kg = lane >> 4;
  const int t = lane_token(d.tokp, d.T, seg0, m);   // oldest load in flight
  const bool live = m < n;
  const int ntiles = (hi - lo) >> 4;
  const int R = d.R;

  // group 0 of the chunk: B tiles, then the y rows (which need the token id)
  s16x4 bv[PT][RT];
  u32x2 yv[PT];
  const uint32_t yrow = (uint32_t)t * (uint32_t)d.out * 2u;
  load_expand_group<RT, NW, PT>(b_r, d.y_r, R, r, lo, ntiles, live, yrow, 0, bv, yv, m, kg, w);

  if (tid == 0) {
    const int base = __hip_atomic_load(&pair->y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int it = 0;
    while ((int)((uint32_t)__hip_atomic_load(&pair->x, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT) -
                 (uint32_t)base) < d.KP &&
           it < d.spin_limit) {
      __builtin_amdgcn_s_sleep(1);
      ++it;
    }
    *flag = (it < d.spin_limit) ? 1 : 0;
    __hip_atomic_store(&pair->y, (int)((uint32_t)base + (uint32_t)d.KP), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (*flag) {
    for (int idx = tid; idx < kMT * RP; idx += NW * kWave) {
      float v = 0.0f;
      for (int kp = 0; kp < d.KP; ++kp)
        v += __hip_atomic_load(part_in + kp * kMT * RP + idx, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      v *= scale;
      const uint32_t hb = to_bf16_bits(v);
      const uint32_t lb = to_bf16_bits(v - __uint_as_float(hb << 16));
      const int q = idx / RP;
      const int j = idx - q * RP;
      hhi[q * RPS + j] = (uint16_t)hb;
      hlo[q * RPS + j] = (uint16_t)lb;
    }
  } else {
    // producers not seen in time: compute this slice's h here
    const uint32_t rowA = (uint32_t)d.in * 2u;
    f32x4 acc[RT];
#pragma unroll
    for (int nt = 0; nt < RT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    shrink_steps<RT, NW>(
        d.x_r, a_r, rowA, d.in, r, [&] { return live ? (uint32_t)t * rowA : kOOB; }, 0,
        (d.in + 31) / 32, acc, m, kg, w);
    store_partial<RT>(red + w * kMT * RP, acc, m, kg);
    __syncthreads();
    reduce_split<RT, NW>(red, scale, hhi, hlo, tid);
  }
  __syncthreads();

  expand_chunk<RT, NW, PT>(b_r, d.y_r, R, r, lo, ntiles, live, yrow, bv, yv, hhi, hlo, m, kg,
                           w);
}

// ---------------------------------------------------------------------------
// standalone decode kernels (lora_shrink / lora_expand on segments of at most
// 16 tokens): the same tiles as the decode pieces, with h in memory
// ---------------------------------------------------------------------------

// h rows of one (slot, slice) for the slot's <= 16 tokens: K split across the
// NW waves, partial tiles added in a fixed order; columns below r written
// (the columns at or past r, and the rows of other tokens, are left to the
// zero-writing kernel).
template <int RT, int NW>
__device__ __forceinline__ void shrink_rows(rsrc_t x_r, rsrc_t a_r, const int32_t* tokp, int T,
                                            int in, int seg0, int n, int r, float* h, int SR,
                                            int col0, float* red, int* tok, int lane, int w,
                                            int tid) {
  constexpr int RP = RT * 16;
  const int m = lane & 15;
  const int kg = lane >> 4;
  const int t = lane_token(tokp, T, seg0, m);
  const bool live = m < n;
  const uint32_t rowA = (uint32_t)in * 2u;
  f32x4 acc[RT];
#pragma unroll
  for (int nt = 0; nt < RT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  shrink_steps<RT, NW>(x_r, a_r, rowA, in, r, [&] { return live ? (uint32_t)t * rowA : kOOB; },
                       0, (in + 31) / 32, acc, m, kg, w);
  store_partial<RT>(red + w * kMT * RP, acc, m, kg);
  if (w == 0 && kg == 0) tok[m] = live ? t : -1;
  __syncthreads();
  for (int idx = tid; idx < kMT * RP; idx += NW * kWave) {
    const int q = idx / RP;
    const int j = idx - q * RP;
    const int tq = tok[q];
    if (tq < 0 || j >= r) continue;
    float v = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) v += red[ww * kMT * RP + idx];
    h[(int64_t)tq * SR + col0 + j] = v;
  }
}

// expand of column chunk [lo, hi) of slice i for the slot's <= 16 tokens,
// with the slice's h rows read from memory
template <int RT, int NW>
__device__ __forceinline__ void expand_rows(const DecodeArgs& d, rsrc_t b_r, const float* h,
                                            int SR, int col0, int r, float scale, int seg0,
                                            int n, int lo, int hi, uint16_t* hhi, uint16_t* hlo,
                                            int* tok, int lane, int w, int tid) {
  constexpr int RP = RT * 16;
  constexpr int RPS = RP + 4;
  constexpr int PT = RT <= 2 ? 8 : RT <= 4 ? 4 : RT <= 8 ? 2 : 1;   // tiles per wave in flight
  const int m = lane & 15;
  const int kg = lane >> 4;
  const int t = lane_token(d.tokp, d.T, seg0, m);   // oldest load in flight
  const bool live = m < n;
  const int ntiles = (hi - lo) >> 4;
  const int R = d.R;
  const uint32_t yrow = (uint32_t)t * (uint32_t)d.out * 2u;

  s16x4 bv[PT][RT];
  u32x2 yv[PT];
  load_expand_group<RT, NW, PT>(b_r, d.y_r, R, r, lo, ntiles, live, yrow, 0, bv, yv, m, kg, w);
  if (w == 0 && kg == 0) tok[m] = live ? t : -1;
  __syncthreads();
  // h rows: scaled, split into bf16 hi + lo (ranks at or past r read as 0)
  const rsrc_t h_r = make_rsrc(h, (uint32_t)d.T * (uint32_t)SR * 4u);
  for (int idx = tid; idx < kMT * RP; idx += NW * kWave) {
    const int q = idx / RP;
    const int j = idx - q * RP;
    const int tq = tok[q];
    const float v =
        __uint_as_float(bload4(h_r, (tq >= 0 && j < r)
                                        ? ((uint32_t)tq * (uint32_t)SR + col0 + j) * 4u
                                        : kOOB)) *
        scale;
    const uint32_t hb = to_bf16_bits(v);
    const uint32_t lb = to_bf16_bits(v - __uint_as_float(hb << 16));
    hhi[q * RPS + j] = (uint16_t)hb;
    hlo[q * RPS + j] = (uint16_t)lb;
  }
  __syncthreads();

  expand_chunk<RT, NW, PT>(b_r, d.y_r, R, r, lo, ntiles, live, yrow, bv, yv, hhi, hlo, m, kg,
                           w);
}

}  // namespace

template <int RT, int NW>
__global__ __launch_bounds__(NW * 64) void k_apply_fused(
    const void* __restrict__ x_, void* __restrict__ y_, int T, int in, SliceTable st,
    const void* __restrict__ a_, const void* __restrict__ b_, int slots, int R,
    const int32_t* __restrict__ token_order, const int32_t* __restrict__ indptr,
    const int32_t* __restrict__ ranks, const float* __restrict__ scalings, ChunkTable ct,
    int n_shrink, int n_expand, int nclass, int KP, float* __restrict__ part,
    int2* __restrict__ pairs, int spin_limit) {
  using L = Lds<RT, NW>;
  constexpr int RP = RT * 16;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int* tok = (int*)lds;
  int* scratch = (int*)(lds + 64);
  float* red = (float*)(lds + L::kRed);
  uint16_t* hhi = (uint16_t*)(lds + L::kHhi);
  uint16_t* hlo = (uint16_t*)(lds + L::kHlo);

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = wave_id();
  const int S = st.n;
  const int SR = S * R;
  const int out = st.off[S];
  const int bid = blockIdx.x;

  if (bid < n_shrink + n_expand) {
    // decode pieces; block bid = 8*k + xcd runs on XCD `xcd`, and every piece
    // of slot s = 8*q + xcd is placed there, so they share that XCD's L2
    // With nclass > 1 each region (shrink, expand) is laid out once per rank
    // class, largest ranks first, and a piece runs in the pass of its slot's
    // class: the dispatcher, which starts blocks in order, then begins the
    // longest pieces first.
    const bool is_shrink = bid < n_shrink;
    const int per_slot = is_shrink ? S * KP : ct.n;
    int b = is_shrink ? bid : bid - n_shrink;
    int cls = 0;
    if (nclass > 1) {
      const int pass = 8 * ((slots + 7) / 8) * per_slot;
      cls = b / pass;
      b -= cls * pass;
    }
    const int xcd = b & 7;
    const int k = b >> 3;
    const int q = k / per_slot;
    const int rem = k - q * per_slot;
    const int s = q * 8 + xcd;
    if (s >= slots) return;
    // the three loads are issued together; reading the rank first keeps the
    // compiler from waiting on the segment bounds before requesting it
    const int r_raw = __builtin_nontemporal_load(ranks + s);
    int seg0, n;
    segment_of(indptr, s, T, seg0, n);
    const int r = clamp_rank(r_raw, R);
    if (r == 0 || n == 0 || n > kMT) return;
    if (nclass > 1 && cls != (2 * r > R ? 0 : 4 * r > R ? 1 : 2)) return;
    const int i = is_shrink ? rem / KP : ct.slice[rem];
    DecodeArgs d;
    d.x_r = make_rsrc(x_, (uint32_t)T * (uint32_t)in * 2u);
    d.y_r = make_rsrc(y_, (uint32_t)T * (uint32_t)out * 2u);
    d.tokp = token_order;
    d.T = T;
    d.in = in;
    d.out = out;
    d.R = R;
    d.KP = KP;
    d.spin_limit = spin_limit;
    const rsrc_t a_r = make_rsrc((const char*)a_ + ((int64_t)s * SR + (int64_t)i * R) * in * 2,
                                 (uint32_t)r * (uint32_t)in * 2u);
    float* pbase = part + ((int64_t)s * S + i) * KP * kMT * RP;
    int2* slot_pairs = pairs + (int64_t)s * kMaxChunks;
    if (is_shrink) {
      const int kp = rem - i * KP;
      shrink_piece<RT, NW>(d, a_r, r, seg0, n, pbase + kp * kMT * RP,
                           slot_pairs + ct.first[i], ct.per_slice[i], kp, red, lane, w, tid);
    } else {
      const rsrc_t b_r =
          make_rsrc((const char*)b_ + (int64_t)s * out * R * 2, (uint32_t)out * (uint32_t)R * 2u);
      expand_piece<RT, NW>(d, a_r, b_r, r, scalings[s], seg0, n, ct.c0[rem], ct.c1[rem], pbase,
                           slot_pairs + rem, red, hhi, hlo, scratch + 20, lane, w, tid);
    }
    return;
  }

  // prefill item: a block of 16 tokens of a long segment, every slice and column
  auto count = [&](int ss) -> int {
    int b0, nn;
    segment_of(indptr, ss, T, b0, nn);
    const int rr = clamp_rank(ranks[ss], R);
    return (nn > kMT && rr > 0) ? (nn + kMT - 1) / kMT : 0;
  };
  const SlotItem it = locate_item(bid - n_shrink - n_expand, slots, count, scratch);
  if (it.slot < 0) return;
  const int s = it.slot;
  int seg0, n;
  segment_of(indptr, s, T, seg0, n);
  const int r = clamp_rank(ranks[s], R);
  const int mb = it.local;
  const int ntok = min(kMT, n - mb * kMT);
  if (tid < kMT) tok[tid] = tid < ntok ? token_at(token_order, seg0 + mb * kMT + tid, T) : -1;
  __syncthreads();
  const float scale = scalings[s];
  const char* ab = (const char*)a_ + (int64_t)s * SR * in * 2;
  const char* bb = (const char*)b_ + (int64_t)s * out * R * 2;
  const rsrc_t x_r = make_rsrc(x_, (uint32_t)T * (uint32_t)in * 2u);
  const uint32_t rowA = (uint32_t)in * 2u;
  const int m = lane & 15;
  const int kg = lane >> 4;
  const int t = tok[m];
  const uint32_t xrow = t >= 0 ? (uint32_t)t * rowA : kOOB;
  for (int i = 0; i < S; ++i) {
    const rsrc_t a_r = make_rsrc(ab + (int64_t)i * R * in * 2, (uint32_t)r * rowA);
    f32x4 acc[RT];
#pragma unroll
    for (int nt = 0; nt < RT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    shrink_steps<RT, NW>(x_r, a_r, rowA, in, r, [&] { return xrow; }, 0, (in + 31) / 32, acc, m,
                         kg, w);
    store_partial<RT>(red + w * kMT * RT * 16, acc, m, kg);
    __syncthreads();
    reduce_split<RT, NW>(red, scale, hhi, hlo, tid);
    __syncthreads();
    expand_range<RT, NW>((char*)y_, out, tok, bb, R, r, st.off[i], st.off[i + 1], hhi, hlo, lane,
                         w);
    __syncthreads();
  }
}

template <int RT, int NW>
__global__ __launch_bounds__(NW * 64) void k_decode_shrink(
    const void* __restrict__ x_, int T, int in, const void* __restrict__ a_, int slots, int S,
    int R, const int32_t* __restrict__ token_order, const int32_t* __restrict__ indptr,
    const int32_t* __restrict__ ranks, float* __restrict__ h) {
  using L = Lds<RT, NW>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int* tok = (int*)lds;
  float* red = (float*)(lds + L::kRed);
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = wave_id();
  // block bid = 8*k + xcd runs on XCD xcd; slot s = 8*q + xcd
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int k = bid >> 3;
  const int q = k / S;
  const int i = k - q * S;
  const int s = q * 8 + xcd;
  if (s >= slots) return;
  int seg0, n;
  segment_of(indptr, s, T, seg0, n);
  const int r = clamp_rank(ranks[s], R);
  if (n == 0 || r == 0 || n > kMT) return;
  const rsrc_t x_r = make_rsrc(x_, (uint32_t)T * (uint32_t)in * 2u);
  const rsrc_t a_r = make_rsrc((const char*)a_ + ((int64_t)s * S * R + (int64_t)i * R) * in * 2,
                               (uint32_t)r * (uint32_t)in * 2u);
  shrink_rows<RT, NW>(x_r, a_r, token_order, T, in, seg0, n, r, h, S * R, i * R, red, tok, lane,
                      w, tid);
}

template <int RT, int NW>
__global__ __launch_bounds__(NW * 64) void k_decode_expand(
    void* __restrict__ y_, int T, SliceTable st, const float* __restrict__ h,
    const void* __restrict__ b_, int slots, int R, const int32_t* __restrict__ token_order,
    const int32_t* __restrict__ indptr, const int32_t* __restrict__ ranks,
    const float* __restrict__ scalings, ChunkTable ct) {
  using L = Lds<RT, NW>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int* tok = (int*)lds;
  uint16_t* hhi = (uint16_t*)(lds + L::kHhi);
  uint16_t* hlo = (uint16_t*)(lds + L::kHlo);
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = wave_id();
  const int S = st.n;
  const int out = st.off[S];
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int k = bid >> 3;
  const int q = k / ct.n;
  const int c = k - q * ct.n;
  const int s = q * 8 + xcd;
  if (s >= slots) return;
  int seg0, n;
  segment_of(indptr, s, T, seg0, n);
  const int r = clamp_rank(ranks[s], R);
  if (n == 0 || r == 0 || n > kMT) return;
  const int i = ct.slice[c];
  DecodeArgs d;
  d.y_r = make_rsrc(y_, (uint32_t)T * (uint32_t)out * 2u);
  d.tokp = token_order;
  d.T = T;
  d.in = 0;
  d.out = out;
  d.R = R;
  d.KP = 1;
  d.spin_limit = 0;
  const rsrc_t b_r =
      make_rsrc((const char*)b_ + (int64_t)s * out * R * 2, (uint32_t)out * (uint32_t)R * 2u);
  expand_rows<RT, NW>(d, b_r, h, S * R, i * R, r, scalings[s], seg0, n, ct.c0[c], ct.c1[c], hhi,
                      hlo, tok, lane, w, tid);
}

namespace {

int rt_bucket(int R) {
  const int RT = (R + 15) / 16;
  return RT <= 1 ? 1 : RT <= 2 ? 2 : RT <= 4 ? 4 : RT <= 8 ? 8 : 16;
}
constexpr int kNW = 8;

size_t lds_bytes(int rt, int nw) {
  const int RP = rt * 16;
  return 256 + (size_t)nw * kMT * RP * 4 + 2 * (size_t)kMT * (RP + 4) * 2;
}

int env_int(const char* name, int dflt) {
  const char* e = getenv(name);
  return e ? atoi(e) : dflt;
}

int decode_chunk_cols(int R) {
  // columns per decode expand piece; overridable for tuning experiments
  const int env = env_int("LORA_DECODE_CHUNK", 0);
  if (env >= 16 && env % 16 == 0) return env;
  return R <= 32 ? 1024 : 2048;
}

int k_parts(int in, int out) {
  // K parts of a decode shrink: ~2048 deep, or ~1024 when the output is
  // narrower than one expand chunk (a router's logits: then every slot has a
  // single expand piece, and more, shorter shrink pieces shorten the chain:
  // measured at 64 outputs, 9.5 -> 8.1 us for 2 -> 4 parts; 8 parts 9.4 us);
  // overridable for tuning
  const int env = env_int("LORA_KPARTS", 0);
  int kp = env > 0 ? env : in / (out < 1024 ? 1024 : 2048);
  return kp < 1 ? 1 : kp > 8 ? 8 : kp;
}

// Expand chunks: each slice cut into pieces of at most `cols` columns (a
// multiple of 16), at most kMaxChunks in all.
ChunkTable make_chunks(const SliceTable& st, int R) {
  ChunkTable ct;
  int cols = decode_chunk_cols(R);
  for (;;) {
    int n = 0;
    for (int i = 0; i < st.n; ++i) {
      const int w = st.off[i + 1] - st.off[i];
      n += (w + cols - 1) / cols;
    }
    if (n <= kMaxChunks) break;
    cols *= 2;
  }
  ct.n = 0;
  for (int i = 0; i < st.n; ++i) {
    ct.per_slice[i] = 0;
    ct.first[i] = ct.n;
    for (int c = st.off[i]; c < st.off[i + 1]; c += cols) {
      ct.slice[ct.n] = i;
      ct.c0[ct.n] = c;
      ct.c1[ct.n] = min(c + cols, st.off[i + 1]);
      ++ct.n;
      ++ct.per_slice[i];
    }
  }
  return ct;
}

}  // namespace

size_t counter_bytes(int slots, int S) {
  // fixed size (a {count, base} pair for every slot and chunk index), so
  // calls of different shapes share one workspace without their regions
  // overlapping
  (void)slots;
  (void)S;
  return (size_t)8192 * kMaxChunks * 2 * sizeof(int);
}

size_t fused_partial_bytes(int slots, int S, int R, int in) {
  const int RP = rt_bucket(R) * 16;
  // room for the most parts any output width takes
  return (size_t)slots * S * k_parts(in, 0) * kMT * RP * 4;
}

bool fused_supported(int dtype, const SliceTable& st, int R, int T, int in) {
  if (dtype != kDtypeBF16) return false;
  // buffer offsets are 32-bit: every resource must stay below 2 GiB
  const int64_t lim = (int64_t)1 << 31;
  const int64_t out = st.off[st.n];
  if ((int64_t)T * in * 2 >= lim || (int64_t)T * out * 2 >= lim ||
      (int64_t)out * R * 2 >= lim || (int64_t)R * in * 2 >= lim)
    return false;
  for (int i = 0; i < st.n; ++i)
    if ((st.off[i + 1] - st.off[i]) % 16 != 0) return false;
  const int rt = rt_bucket(R);
  return R <= 256 && lds_bytes(rt, kNW) <= 160 * 1024;
}

hipError_t launch_apply_fused(const void* x, void* y, int T, int in, const SliceTable& st,
                              const void* a, const void* b, int slots, int R,
                              const int32_t* token_order, const int32_t* indptr,
                              const int32_t* ranks, const float* scalings, void* workspace,
                              hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const ChunkTable ct = make_chunks(st, R);
  const int KP = k_parts(in, st.off[st.n]);
  const int64_t slots8 = 8 * (int64_t)((slots + 7) / 8);
  // rank classes (largest first) where ranks differ enough to matter
  const int nclass = rt_bucket(R) >= 4 ? 3 : 1;
  const int64_t n_shrink = nclass * slots8 * st.n * KP;
  const int64_t n_expand = nclass * slots8 * ct.n;
  const int64_t n_prefill = (T + kMT - 1) / kMT + slots;
  const int64_t grid = n_shrink + n_expand + n_prefill;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  int2* pairs = (int2*)workspace;
  float* part = (float*)((char*)workspace + counter_bytes(slots, st.n));
  // bound of the wait of an expand piece (iterations of ~0.1-1 us); 0 makes
  // every expand piece compute h itself (used by the tests of that path)
  const int spin_limit = env_int("LORA_SPIN_LIMIT", 1 << 13);
  const int rt = rt_bucket(R);
  const size_t lds = lds_bytes(rt, kNW);
#define LAUNCH(RTV)                                                                             \
  do {                                                                                          \
    if (lds > 65536) {                                                                          \
      hipError_t e = hipFuncSetAttribute((const void*)k_apply_fused<RTV, kNW>,                  \
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);  \
      if (e != hipSuccess) return e;                                                            \
    }                                                                                           \
    hipLaunchKernelGGL((k_apply_fused<RTV, kNW>), dim3((unsigned)grid), dim3(kNW * 64), lds,    \
                       stream, x, y, T, in, st, a, b, slots, R, token_order, indptr, ranks,     \
                       scalings, ct, (int)n_shrink, (int)n_expand, nclass, KP, part, pairs,      \
                       spin_limit);                                                             \
  } while (0)
  switch (rt) {
    case 1: LAUNCH(1); break;
    case 2: LAUNCH(2); break;
    case 4: LAUNCH(4); break;
    case 8: LAUNCH(8); break;
    default: LAUNCH(16); break;
  }
#undef LAUNCH
  return hipGetLastError();
}


hipError_t launch_decode_shrink(const void* x, int T, int in, const void* a, int slots, int S,
                                int R, const int32_t* token_order, const int32_t* indptr,
                                const int32_t* ranks, float* h, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int64_t grid = 8 * (int64_t)((slots + 7) / 8) * S;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const int rt = rt_bucket(R);
  const size_t lds = lds_bytes(rt, kNW);
#define LAUNCH(RTV)                                                                             \
  do {                                                                                          \
    if (lds > 65536) {                                                                          \
      hipError_t e = hipFuncSetAttribute((const void*)k_decode_shrink<RTV, kNW>,                \
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);  \
      if (e != hipSuccess) return e;                                                            \
    }                                                                                           \
    hipLaunchKernelGGL((k_decode_shrink<RTV, kNW>), dim3((unsigned)grid), dim3(kNW * 64), lds,  \
                       stream, x, T, in, a, slots, S, R, token_order, indptr, ranks, h);         \
  } while (0)
  switch (rt) {
    case 1: LAUNCH(1); break;
    case 2: LAUNCH(2); break;
    case 4: LAUNCH(4); break;
    case 8: LAUNCH(8); break;
    default: LAUNCH(16); break;
  }
#undef LAUNCH
  return hipGetLastError();
}

hipError_t launch_decode_expand(void* y, int T, const SliceTable& st, const float* h,
                                const void* b, int slots, int R, const int32_t* token_order,
                                const int32_t* indptr, const int32_t* ranks,
                                const float* scalings, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const ChunkTable ct = make_chunks(st, R);
  const int64_t grid = 8 * (int64_t)((slots + 7) / 8) * ct.n;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const int rt = rt_bucket(R);
  const size_t lds = lds_bytes(rt, kNW);
#define LAUNCH(RTV)                                                                             \
  do {                                                                                          \
    if (lds > 65536) {                                                                          \
      hipError_t e = hipFuncSetAttribute((const void*)k_decode_expand<RTV, kNW>,                \
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);  \
      if (e != hipSuccess) return e;                                                            \
    }                                                                                           \
    hipLaunchKernelGGL((k_decode_expand<RTV, kNW>), dim3((unsigned)grid), dim3(kNW * 64), lds,  \
                       stream, y, T, st, h, b, slots, R, token_order, indptr, ranks, scalings,   \
                       ct);                                                                     \
  } while (0)
  switch (rt) {
    case 1: LAUNCH(1); break;
    case 2: LAUNCH(2); break;
    case 4: LAUNCH(4); break;
    case 8: LAUNCH(8); break;
    default: LAUNCH(16); break;
  }
#undef LAUNCH
  return hipGetLastError();
}

}  // namespace lora
