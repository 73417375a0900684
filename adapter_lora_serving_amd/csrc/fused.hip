// Fused shrink + expand for bf16 targets (lora_apply_linear) of a small
// batch (fewer than 1024 tokens; larger batches run the segment-tiled
// kernels), on bf16 MFMA.
//
// Follows the mstar lora.backend page, LoraBackend.apply_linear_ (the shrink
// and the expand of one target, which a backend is free to run as one
// kernel): the result is that of shrink (h = x @ A^T, per token's slot)
// followed by expand (y += scaling * h @ B^T per fused slice), with h kept in
// fp32.
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
// Rank 16 and below (one rank tile): a decode shrink piece stages its A rows
//   and an expand piece of a 1024- or 2048-column chunk its y rows through
//   LDS as rows of 128 bytes (buffer-to-LDS transfers), since the MFMA
//   operand layout would read 16 rows x 64 (A) or x 32 (y) bytes per load,
//   far below the HBM rate (shrink_steps_staged, stage_y_run).
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
// One-launch form (lora_apply_linear_from_slots, at most 1024 tokens over at
//   most 63 slots): the kernel takes each token's slot instead of the
//   addressing, which the page builds once per step before the first
//   target. A decode piece finds its slot's tokens itself (each wave loads
//   the slot ids, one ballot per 64 tokens, and lane row m takes the m-th
//   match: the same tokens in the same order as the stable grouping gives,
//   so the result is bit-identical), a prefill item counts the slots in LDS
//   to locate its item, and one workgroup writes the addressing for the
//   step's later targets. A separate addressing kernel costs a whole launch
//   (about 3.5 us of a 16 us step); finding the tokens per piece costs
//   ~0.25 us of this kernel, because its vector loads queue behind the
//   start-up flood of x and A loads where the addressing form's scalar
//   reads of slot_indptr and token_order do not. (Reading the ids through
//   scalar loads, 32 per wave, with one workgroup barrier, was slower.)
#include "lora_common.h"
#include "lora_kernels.h"

#include <stdlib.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <utility>

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
  // one-tile kernels: per wave, the A rows of its 8 K steps staged by
  // buffer-to-LDS transfers (8 blocks of 1 KB), after the regions above
  static constexpr int kStage = (kBytes + 1023) & ~1023;
  static constexpr int kStageBytes = RT == 1 ? NW * 8 * 1024 : 0;
  static constexpr int kTotal = kStage + kStageBytes;
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
// Handoff: every partial tile (s, i, kp) has a ticket counter in the
// workspace, and every entry of the tile is one 64-bit word holding the fp32
// value and a 32-bit tag. Each call touching tile j adds exactly kTicket to
// its counter: the producer adds kTicket - nc and each of the nc expand pieces
// of slice i adds 1, all at their start, off the critical path. Every
// participant's fetch_add returns a value in [C, C + kTicket) where C, the
// counter at the call's start, is a multiple of kTicket, so all of them
// derive the same epoch E = C / kTicket + 1 without talking to each other.
// The producer stores each entry as {value, tag(E)} in one agent-scope
// atomic 64-bit store; an expand piece polls one entry per tile until it
// carries tag(E), then loads the whole tile and takes each entry whose tag
// matches (re-polling any that has not landed yet). Data and flag travel in
// the same word, so the chain from the producer's last product to the
// consumer's use is one store and one load (the earlier design stored the
// tile, waited for the stores to complete, bumped a count, polled the count
// and only then loaded the tile).
// Why a stale entry is never taken for a new one: the tile's address and
// size depend only on its index j and the rank bucket RT (16 x 16*RT
// entries), the tag holds log2(RT) in its low 3 bits, and the counter of j
// only grows, so an entry left at the same address by an earlier call either
// has another rank bucket or an older epoch. (The epoch field holds 29 bits
// and the counter 32: a stale entry could match again only after 2^25 calls
// touching tile j, none of them in its rank bucket.)
// Memory ordering: entries are written and read only with agent-scope
// atomic 64-bit accesses, coherent across the XCDs; no other memory carries
// the handoff, so no fence is needed. The counters need a zero-filled
// workspace before its first use (any multiple of kTicket works).
// The wait is bounded: a piece that times out (its producers not resident,
// e.g. the GPU shared with other work) computes the slice's h itself, so the
// kernel always finishes with the right result; its ticket was taken at the
// start, so the counters stay multiples of kTicket.
// ---------------------------------------------------------------------------

constexpr uint32_t kTicket = 128;   // > 1 producer + the most expand pieces of a slice

struct DecodeArgs {
  rsrc_t x_r, y_r;
  const int32_t* tokp;
  int T, in, out, R;
  int KP;
  int spin_limit;
  int early;     // 1: read the partial entries once with the prefetch
  bool tok_given;  // the lane's token id is tok_m (found from token_slot), not token_order's
  int tok_m;
  uint32_t lg;   // log2 of the rank bucket RT: the low 3 bits of every tag
};

__device__ __forceinline__ uint32_t epoch_tag(uint32_t ticket, uint32_t lg) {
  return ((ticket / kTicket + 1u) << 3) | lg;
}

// Token id of lane row m: one vector load per lane (index clamped into the
// array). Issued before the bulk A / B loads, it is the oldest load in
// flight, so the first use of the id waits for it alone (vector loads
// complete in order), not for the bulk loads issued after it.
__device__ __forceinline__ int lane_token(const int32_t* __restrict__ tokp, int T, int seg0,
                                          int m) {
  return tokp[min(seg0 + m, T - 1)];
}

// The same token id read through the scalar path: the slot's (at most 16)
// ids are 16 consecutive entries of token_order from a uniform base, loaded
// into scalar registers (s_load), and lane row m picks entry seg0 - base + m.
// Scalar loads are counted apart from vector memory (lgkmcnt, not vmcnt), so
// the x and y row addresses do not wait behind the vector loads and the
// ticket atomic a piece issues first.
__device__ __forceinline__ int lane_token_s(const int32_t* __restrict__ tokp, int T, int seg0,
                                            int m) {
  const int base = __builtin_amdgcn_readfirstlane(T >= kMT ? min(seg0, T - kMT) : 0);
  int ids[kMT];
  if (T >= kMT) {
#pragma unroll
    for (int k = 0; k < kMT; ++k) ids[k] = tokp[base + k];
  } else {   // a batch of fewer than 16 tokens: T >= 1 whenever a piece runs
#pragma unroll
    for (int k = 0; k < kMT; ++k) ids[k] = tokp[min(k, T - 1)];
  }
  const int j = min(seg0 - base + m, kMT - 1);
  int t = ids[0];
#pragma unroll
  for (int k = 1; k < kMT; ++k) t = j == k ? ids[k] : t;
  return t;
}

// The tokens t in [lo, hi) with ids[t] == s, in ascending index, found
// from the ids themselves (the one-launch forms, hi - lo <= 2 * NW * 64):
// the ones at positions [first, first + kMT) of that list go to
// tok[0..kMT), `fill` past its end; the return value is their count. This is the segment that the
// addressing gives slot s (a stable grouping by slot), found with one
// coalesced load and a ballot per 64 tokens instead of the two dependent
// reads of slot_indptr and token_order. `cnt`: 2 * NW ints of LDS. Every
// thread of the block calls it; the result is uniform.
template <int NW>
__device__ __forceinline__ int slot_tokens(const int32_t* __restrict__ ids, int lo, int hi,
                                           int s, int first, int fill, int* tok, int* cnt, int tid,
                                           int lane, int w) {
  constexpr int NT = NW * kWave;
  const int t0 = lo + tid;
  const int t1 = lo + tid + NT;
  const bool m0 = t0 < hi && ids[t0] == s;
  const bool m1 = t1 < hi && ids[t1] == s;
  const uint64_t b0 = __ballot(m0);
  const uint64_t b1 = __ballot(m1);
  if (lane == 0) {
    cnt[w] = __popcll(b0);        // tokens [64w, 64w + 64)
    cnt[NW + w] = __popcll(b1);   // tokens [NT + 64w, NT + 64w + 64)
  }
  if (tid < kMT) tok[tid] = fill;
  __syncthreads();
  int before0 = 0, before1 = 0, total = 0;
#pragma unroll
  for (int c = 0; c < 2 * NW; ++c) {
    const int v = cnt[c];
    before0 += c < w ? v : 0;
    before1 += c < NW + w ? v : 0;
    total += v;
  }
  const uint64_t below = (1ull << lane) - 1ull;
  const int p0 = before0 + __popcll(b0 & below) - first;
  const int p1 = before1 + __popcll(b1 & below) - first;
  if (m0 && p0 >= 0 && p0 < kMT) tok[p0] = t0;
  if (m1 && p1 >= 0 && p1 < kMT) tok[p1] = t1;
  __syncthreads();
  return total;
}

// Position of the k-th set bit (k from 0, k < popcount) of a 64-bit mask,
// by halving: six popcounts.
__device__ __forceinline__ int nth_set_bit(uint64_t mask, int k) {
  int pos = 0;
#pragma unroll
  for (int width = 32; width >= 1; width >>= 1) {
    const uint64_t low = mask & ((1ull << width) - 1ull);
    const int c = __popcll(low);
    if (k >= c) {
      k -= c;
      mask >>= width;
      pos += width;
    }
  }
  return pos;
}

// The decode pieces' form of slot_tokens, per wave and with no workgroup
// barrier (each wave starts its loads as soon as it has its tokens, as with
// token_order): the wave reads ids[lo, hi) (at most 1024, one 64-token group
// per load), takes one ballot per group, and lane row m picks the m-th t with
// ids[t] == s (0 when there are m or fewer: such rows are not live). n
// receives the count (uniform).
__device__ __forceinline__ int wave_slot_token(const int32_t* __restrict__ ids, int lo, int hi,
                                               int s, int m, int& n) {
  constexpr int kMaxGroups = 16;
  const int lane = lane_id();
  const int ng = (hi - lo + kWave - 1) / kWave;
  int v[kMaxGroups];
#pragma unroll
  for (int g = 0; g < kMaxGroups; ++g) {
    v[g] = -1;
    if (g < ng) {
      const int t = lo + g * kWave + lane;
      v[g] = t < hi ? ids[t] : -1;
    }
  }
  int count = 0;
  int tok = 0;
#pragma unroll
  for (int g = 0; g < kMaxGroups; ++g) {
    if (g < ng) {
      const uint64_t mask = __ballot(v[g] == s);
      const int c = __popcll(mask);
      if (m >= count && m < count + c) tok = lo + g * kWave + nth_set_bit(mask, m - count);
      count += c;
    }
  }
  n = count;
  return tok;
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

// shrink_steps_n for one rank tile with the A rows staged through LDS: per
// K-step pair a wave fetches rows 0-7 and 8-15 as two 1 KB blocks of 8 rows
// x 128 bytes (buffer-to-LDS, lane L: row L / 8, 16-byte chunk L % 8 holding
// the logical chunk (L % 8) ^ row, so that the operand reads spread over the
// banks), instead of 16 rows x 64 bytes per load into registers; the operand
// of lane (m, kg) for step u is then read back from LDS. x is read into
// registers as in shrink_steps_n. Same products, same order. Measured on
// the 32-slot qkv decode: step 12.05 -> 11.41 us.
template <int NW, class XRow>
__device__ __forceinline__ void shrink_steps_staged(rsrc_t x_r, rsrc_t a_r, uint32_t rowA,
                                                    int in, XRow xrow_of, int s0, int s1,
                                                    f32x4* acc, int m, int kg, int w,
                                                    char* stage) {
  constexpr int U = 8;
  int st0 = s0 + w * U;
  if (st0 >= s1) return;
  char* wst = stage + w * (U * 1024);
  const int lane = (kg << 4) | m;
  const int rl = lane >> 3;            // row of the lane's transfers within a block
  const int lc = (lane & 7) ^ rl;      // logical chunk the lane fetches
  bf16x8 xa[U];
  auto issue_a = [&](int st) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = ((u & 1) << 3) | rl;
      const int stp = st + (u & ~1);            // first step of the pair
      const int k = stp * 32 + lc * 8;          // element of the lane's chunk
      const bool kv = stp + (lc >> 2) < s1 && k < in;
      dma16(a_r, wst + u * 1024, kv ? (uint32_t)row * rowA + (uint32_t)k * 2u : kOOB);
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
    __builtin_amdgcn_s_waitcnt(vmcnt_le(0));   // the transfers into LDS have landed
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = ((u & 1) << 2) | kg;       // logical chunk of step u in its pair
      const int blk = (u & ~1) | (m >> 3);
      const int r7 = m & 7;
      const bf16x8 av = *(const bf16x8*)(wst + blk * 1024 + r7 * 128 + ((c ^ r7) << 4));
      acc[0] = mfma_k32(xa[u], av, acc[0]);
    }
  };
  issue_a(st0);
  const uint32_t xrow = xrow_of();
  load_x(st0, xrow);
  products();
  for (st0 += NW * U; st0 < s1; st0 += NW * U) {
    // the operand reads of the previous steps are done before their blocks
    // are refilled
    __builtin_amdgcn_s_waitcnt(0xc07f);
    asm volatile("" ::: "memory");
    issue_a(st0);
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
                                             f32x4 (&acc)[RT], int m, int kg, int w,
                                             char* stage = nullptr) {
  if constexpr (RT == 1) {
    if (stage) return shrink_steps_staged<NW>(x_r, a_r, rowA, in, xrow, s0, s1, acc, m, kg, w,
                                              stage);
  }
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

// Tile of group g that wave w handles as its u-th (u < PT). contig: the PT
// adjacent tiles (g*NW + w)*PT + u, so that a wave's y of a token row is one
// contiguous run (staged through LDS, stage_y_run); else dealt round robin,
// w + NW*(g*PT + u). Adjacent runs are taken for chunks of one or two full
// groups at one rank tile: alone (y in registers) they took the 32-slot qkv
// decode step from 12.31 to 12.05 us; with y staged, to 10.8 us. A narrow
// slice keeps round robin, which leaves no wave without a tile.
template <int NW, int PT>
__device__ __forceinline__ int tile_of(int g, int w, int u, bool contig) {
  return contig ? (g * NW + w) * PT + u : w + NW * (g * PT + u);
}

// Loads of group g of a chunk's expand tiles (tile_of); B ranks at or past r
// and tiles past the chunk read as zeros (kOOB), y rows of padding tokens too.
template <int RT, int NW, int PT>
__device__ __forceinline__ void load_expand_group(rsrc_t b_r, rsrc_t y_r, int R, int r, int lo,
                                                  int ntiles, bool live, uint32_t yrow, bool contig,
                                                  int g,
                                                  s16x4 (&bv)[PT][RT], u32x2 (&yv)[PT], int m,
                                                  int kg, int w, bool load_y = true) {
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int tile = tile_of<NW, PT>(g, w, u, contig);
#pragma unroll
    for (int ks = 0; ks < RT; ++ks) {
      const int kk = ks * 16 + kg * 4;
      const uint32_t off = (tile < ntiles && kk < r)
                               ? ((uint32_t)(lo + tile * 16 + m) * (uint32_t)R + kk) * 2u
                               : kOOB;
      bv[u][ks] = __builtin_bit_cast(s16x4, bload8(b_r, off));
    }
  }
  if (!load_y) return;
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int tile = tile_of<NW, PT>(g, w, u, contig);
    yv[u] = bload8(y_r, (live && tile < ntiles) ? yrow + (uint32_t)(lo + tile * 16 + 4 * kg) * 2u
                                                : kOOB);
  }
}

// y rows of a wave's run of 8 adjacent tiles (128 columns, 256 bytes per
// token row) for up to 16 tokens, staged through LDS: 4 buffer-to-LDS
// transfers of 8 rows x 128 bytes (block 2h + row group: half h of the
// span, rows 0-7 or 8-15; lane L fetches row L / 8 and the logical chunk
// (L % 8) ^ row into its 16-byte slot) instead of 8 loads of 16 rows x 32
// bytes into registers. yrow is the lane's own token row offset (rows m < n
// live); col0 the run's first column.
__device__ __forceinline__ void stage_y_run(rsrc_t y_r, uint32_t yrow, int n, int col0,
                                            char* ys, int lane) {
  const int rl = lane >> 3;
  const int lc = (lane & 7) ^ rl;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = j >> 1;
    const int row = ((j & 1) << 3) | rl;
    const uint32_t yr = (uint32_t)__shfl((int)yrow, row);
    dma16(y_r, ys + j * 1024,
          row < n ? yr + (uint32_t)col0 * 2u + (uint32_t)(h * 128 + lc * 16) : kOOB);
  }
}
// Products and y update of a wave's staged run (one rank tile): each tile's
// new y values go back into the staged blocks in place, then leave in 4
// stores of 8 rows x 128 bytes (each lane the 16 bytes it fetched), instead
// of 8 stores of 16 rows x 32 bytes.
template <int PT>
__device__ __forceinline__ void expand_run_staged(rsrc_t y_r, uint32_t yrow, int n, int col0,
                                                  int r, char* ys, const s16x4 (&bv)[PT][1],
                                                  s16x4 hb, s16x4 lb, int lane) {
  const int m = lane & 15;
  const int kg = lane >> 4;
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
    const s16x4 b4 = mask_b4(bv[u][0], kg * 4, r);
    o = mfma_k16(b4, hb, o);
    o = mfma_k16(b4, lb, o);
    const int blk = ((u >> 2) << 1) | (m >> 3);
    const int r7 = m & 7;
    const int ch = ((u & 3) << 1) | (kg >> 1);
    u32x2* p = (u32x2*)(ys + blk * 1024 + r7 * 128 + ((ch ^ r7) << 4) + (kg & 1) * 8);
    const u32x2 yy = *p;
    *p = u32x2{pack_bf16x2(bf16lo(yy.x) + o[0], bf16hi(yy.x) + o[1]),
               pack_bf16x2(bf16lo(yy.y) + o[2], bf16hi(yy.y) + o[3])};
  }
  // a wave's LDS accesses complete in order: the reads below see the writes
  const int rl = lane >> 3;
  const int lc = (lane & 7) ^ rl;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = j >> 1;
    const int row = ((j & 1) << 3) | rl;
    const uint32_t yr = (uint32_t)__shfl((int)yrow, row);
    const u32x4 v = *(const u32x4*)(ys + j * 1024 + lane * 16);
    bstore16_out(y_r, row < n ? yr + (uint32_t)col0 * 2u + (uint32_t)(h * 128 + lc * 16) : kOOB,
                 v);
  }
}

// Products and y update of group g from its loaded tiles.
template <int RT, int NW, int PT>
__device__ __forceinline__ void expand_group(rsrc_t y_r, int r, int lo, int ntiles, bool live,
                                             uint32_t yrow, bool contig, int g, const s16x4 (&bv)[PT][RT],
                                             const u32x2 (&yv)[PT], const s16x4 (&hb)[RT],
                                             const s16x4 (&lb)[RT], int kg, int w) {
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int tile = tile_of<NW, PT>(g, w, u, contig);
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
                                             int ntiles, bool live, uint32_t yrow, bool contig,
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
    expand_group<RT, NW, PT>(y_r, r, lo, ntiles, live, yrow, contig, 0, bv0, yv0, hb, lb, kg, w);
    for (int g = 1; g < ngroups; ++g) {
      load_expand_group<RT, NW, PT>(b_r, y_r, R, r, lo, ntiles, live, yrow, contig, g, bv0, yv0, m, kg,
                                    w);
      expand_group<RT, NW, PT>(y_r, r, lo, ntiles, live, yrow, contig, g, bv0, yv0, hb, lb, kg, w);
    }
    return;
  }
  s16x4 bv1[PT][RT];
  u32x2 yv1[PT];
  for (int g = 0; g < ngroups; g += 2) {
    if (g + 1 < ngroups)
      load_expand_group<RT, NW, PT>(b_r, y_r, R, r, lo, ntiles, live, yrow, contig, g + 1, bv1, yv1, m,
                                    kg, w);
    expand_group<RT, NW, PT>(y_r, r, lo, ntiles, live, yrow, contig, g, bv0, yv0, hb, lb, kg, w);
    if (g + 1 < ngroups) {
      if (g + 2 < ngroups)
        load_expand_group<RT, NW, PT>(b_r, y_r, R, r, lo, ntiles, live, yrow, contig, g + 2, bv0, yv0, m,
                                      kg, w);
      expand_group<RT, NW, PT>(y_r, r, lo, ntiles, live, yrow, contig, g + 1, bv1, yv1, hb, lb, kg, w);
    }
  }
}

// Shrink piece (s, i, kp): its partial tile goes to `tile` (16 x RP tagged
// entries); `cnt` is the tile's ticket counter, nc the expand pieces of
// slice i.
template <int RT, int NW>
__device__ __forceinline__ void shrink_piece(const DecodeArgs& d, rsrc_t a_r, int r, int seg0,
                                             int n, uint64_t* tile, uint32_t* cnt, int nc,
                                             int kp, float* red, int* lds_tag, int lane, int w,
                                             int tid, char* stage) {
  constexpr int RP = RT * 16;
  uint32_t ticket = 0;
  if (tid == 0)   // the oldest load in flight: its return is not waited for until the store
    ticket = __hip_atomic_fetch_add(cnt, kTicket - (uint32_t)nc, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
  const int m = lane & 15;
  const int kg = lane >> 4;
  const int t = d.tok_given ? d.tok_m : lane_token_s(d.tokp, d.T, seg0, m);
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
      m, kg, w, stage);
  // the ticket is first used here: the empty statement keeps the compiler
  // from consuming it (and so waiting for the atomic's return) before the
  // bulk loads above are issued
  asm volatile("" : "+v"(ticket));
  store_partial<RT>(red + w * kMT * RP, acc, m, kg);
  if (tid == 0) *lds_tag = (int)epoch_tag(ticket, d.lg);
  __syncthreads();
  const uint64_t tag = (uint64_t)(uint32_t)*lds_tag << 32;
  for (int idx = tid; idx < kMT * RP; idx += NW * kWave) {
    float v = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) v += red[ww * kMT * RP + idx];
    __hip_atomic_store(tile + idx, tag | __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Expand piece (s, chunk [lo, hi) of slice i): `tiles` are the KP partial
// tiles of (s, i), `cnts` their ticket counters. CONTIG: the tile order of
// tile_of, a compile-time choice so that each order's addresses fold.
template <int RT, int NW, bool CONTIG>
__device__ __forceinline__ void expand_piece(const DecodeArgs& d, rsrc_t a_r, rsrc_t b_r, int r,
                                             float scale, int seg0, int n, int lo, int hi,
                                             const uint64_t* tiles, uint32_t* cnts, float* red,
                                             uint16_t* hhi, uint16_t* hlo, int* lds_tag, int lane,
                                             int w, int tid, char* stage) {
  constexpr int RP = RT * 16;
  constexpr int RPS = RP + 4;
  constexpr int PT = RT <= 2 ? 8 : RT <= 4 ? 4 : RT <= 8 ? 2 : 1;   // tiles per wave in flight
  // one rank tile, adjacent runs (one full group of 8 tiles per wave): y
  // staged through LDS (stage_y_run), 4 KB per wave
  constexpr bool kStagedY = CONTIG && RT == 1 && PT == 8;
  static_assert(!CONTIG || kStagedY, "adjacent runs are taken only with y staged");
  uint32_t ticket = 0;
  if (tid < d.KP)   // one ticket per partial tile, taken first
    ticket = __hip_atomic_fetch_add(cnts + tid, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int m = lane & 15;
  const int kg = lane >> 4;
  const int t = d.tok_given ? d.tok_m : lane_token_s(d.tokp, d.T, seg0, m);
  const bool live = m < n;
  const int ntiles = (hi - lo) >> 4;
  const int R = d.R;
  const bool contig = CONTIG;

  // group 0 of the chunk: B tiles, then the y rows (which need the token id)
  s16x4 bv[PT][RT];
  u32x2 yv[PT];
  const uint32_t yrow = (uint32_t)t * (uint32_t)d.out * 2u;
  // staged: one or two full groups (chunks of 1024 or 2048 columns), each
  // wave's run of group g at stage + 8 KB w + 4 KB g; the B tiles of a second
  // group are prefetched too
  char* ys = stage + w * 8192;
  const int ngs = kStagedY ? ntiles / (NW * PT) : 1;
  s16x4 bv1[PT][RT];
  load_expand_group<RT, NW, PT>(b_r, d.y_r, R, r, lo, ntiles, live, yrow, contig, 0, bv, yv, m, kg,
                                w, !kStagedY);
  if constexpr (kStagedY) {
    if (ngs > 1)
      load_expand_group<RT, NW, PT>(b_r, d.y_r, R, r, lo, ntiles, live, yrow, contig, 1, bv1, yv,
                                    m, kg, w, false);
    for (int gg = 0; gg < ngs; ++gg)
      stage_y_run(d.y_r, yrow, n, lo + (gg * NW + w) * PT * 16, ys + gg * 4096, lane);
  }
  // With d.early, one read of this thread's first entry of each tile is
  // issued with the prefetch: when the producers are already done (a piece
  // that starts after them, in a grid larger than the chip holds at once)
  // the values come back with the prefetch and the wait below needs no
  // second round trip; an older value only fails its tag check. In a grid
  // that runs all at once the read comes too soon and only adds loads.
  constexpr int kMaxKP = 8;   // k_parts never returns more
  uint64_t early[kMaxKP];
#pragma unroll
  for (int kp = 0; kp < kMaxKP; ++kp) {
    early[kp] = 0;
    if (d.early && kp < d.KP && tid < kMT * RP)
      early[kp] = __hip_atomic_load(tiles + (size_t)kp * kMT * RP + tid, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
  }
  // first use of the ticket: not before the prefetch above is issued
  asm volatile("" : "+v"(ticket));

  // Every thread polls its own entries of the KP tiles (bounded) and takes
  // each one once it carries this call's tag. Beyond the early read above,
  // polling starts once this piece's own prefetch has returned: by then the
  // producers, whose loads were issued at the same time, are close to done,
  // and fewer polls load the memory system while it still streams A and x.
  // (A first stage in which one lane per tile polled a single entry cost a
  // further load round trip, ~0.5 us of the kernel's span.)
  if (tid < d.KP) lds_tag[tid] = (int)epoch_tag(ticket, d.lg);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  bool ok = true;
  for (int idx = tid; idx < kMT * RP; idx += NW * kWave) {
    float v = 0.0f;
#pragma unroll
    for (int kp = 0; kp < kMaxKP; ++kp) {
      if (kp >= d.KP) break;
      const uint64_t* e = tiles + (size_t)kp * kMT * RP + idx;
      const uint32_t tag = (uint32_t)lds_tag[kp];
      uint64_t word = d.early && idx == tid ? early[kp]
                                 : __hip_atomic_load(e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int it = 0;
      while ((uint32_t)(word >> 32) != tag && it < d.spin_limit) {
        __builtin_amdgcn_s_sleep(2);
        word = __hip_atomic_load(e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ++it;
      }
      ok = ok && (uint32_t)(word >> 32) == tag;
      v += __uint_as_float((uint32_t)word);
    }
    v *= scale;
    const uint32_t hb = to_bf16_bits(v);
    const uint32_t lb = to_bf16_bits(v - __uint_as_float(hb << 16));
    const int q = idx / RP;
    const int j = idx - q * RP;
    hhi[q * RPS + j] = (uint16_t)hb;
    hlo[q * RPS + j] = (uint16_t)lb;
  }
  if (!__syncthreads_and(ok)) {
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

  if constexpr (kStagedY) {
    // the transfers were waited for with the prefetch, before the partials
    const s16x4 hb = *(const s16x4*)(hhi + m * RPS + kg * 4);
    const s16x4 lb = *(const s16x4*)(hlo + m * RPS + kg * 4);
    expand_run_staged<PT>(d.y_r, yrow, n, lo + w * PT * 16, r, ys, bv, hb, lb, lane);
    if (ngs > 1)
      expand_run_staged<PT>(d.y_r, yrow, n, lo + (NW + w) * PT * 16, r, ys + 4096, bv1, hb, lb,
                            lane);
    return;
  }
  expand_chunk<RT, NW, PT>(b_r, d.y_r, R, r, lo, ntiles, live, yrow, contig, bv, yv, hhi, hlo, m, kg,
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
  const bool contig = n >= 4 && ntiles == NW * PT;
  const uint32_t yrow = (uint32_t)t * (uint32_t)d.out * 2u;

  s16x4 bv[PT][RT];
  u32x2 yv[PT];
  load_expand_group<RT, NW, PT>(b_r, d.y_r, R, r, lo, ntiles, live, yrow, contig, 0, bv, yv, m, kg, w);
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

  expand_chunk<RT, NW, PT>(b_r, d.y_r, R, r, lo, ntiles, live, yrow, contig, bv, yv, hhi, hlo, m, kg,
                           w);
}

}  // namespace

// MODE kFromSlots / kFromExperts (the one-launch forms): the slot
// addressing is built in this launch. Workgroup 0 runs a one-wave sort into
// order_out / indptr_out for later calls on the same batch (workgroups 1-7
// leave at once, so that the pieces keep their XCD placement), and every
// piece finds its tokens from the ids itself; nothing in the launch reads
// the addressing it writes.
//  * kFromSlots: token_slot holds each token's slot. Needs T <= 2 * NW * 64
//    and slots + 1 <= 64.
//  * kFromExperts: token_slot holds each row's slot within its expert
//    (row_slot) and expert_offs the E + 1 bounds of the expert-sorted rows;
//    pool entry (virtual slot) e * eslots + s, of `slots` = E * eslots. A
//    piece of entry (e, s) scans rows [offs[e], offs[e + 1]) for row_slot ==
//    s: for non-decreasing bounds exactly the rows the keys (expert_key) give
//    the entry. Needs T <= 2 * NW * 64, E + 1 <= 64 and slots + 1 <= 1024.
constexpr int kFromAddr = 0;
constexpr int kFromSlots = 1;
constexpr int kFromExperts = 2;

template <int RT, int NW, int MODE>
__global__ __launch_bounds__(NW * 64) void k_apply_fused(
    const void* __restrict__ x_, void* __restrict__ y_, int T, int in, SliceTable st,
    const void* __restrict__ a_, const void* __restrict__ b_, int slots, int R,
    const int32_t* __restrict__ token_order, const int32_t* __restrict__ indptr,
    const int32_t* __restrict__ ranks, const float* __restrict__ scalings, ChunkTable ct,
    int n_shrink, int n_expand, int nclass, int KP, uint64_t* __restrict__ part,
    uint32_t* __restrict__ tickets, int spin_limit, int early,
    const int32_t* __restrict__ token_slot, int32_t* __restrict__ order_out,
    int32_t* __restrict__ indptr_out, const int32_t* __restrict__ expert_offs, int E,
    int eslots) {
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
  int bid = blockIdx.x;
  // LDS while red is free (before any product): kFromSlots: the slot
  // histogram [64], then slot_tokens' counts; kFromExperts: the key
  // histogram [1024], the expert bounds [64], then the counts
  int* tcnt = (int*)red + (MODE == kFromExperts ? 1088 : kWave);
  int* soffs = (int*)red + 1024;
  if constexpr (MODE != kFromAddr) {
    if (bid < 8) {
      if (bid == 0 && w == 0) {
        if constexpr (MODE == kFromSlots) {
          if (T <= 4 * kWave)
            addressing_one_wave<4>(token_slot, T, slots, order_out, indptr_out, (int*)red);
          else
            addressing_one_wave<2 * NW>(token_slot, T, slots, order_out, indptr_out, (int*)red);
        } else {
          for (int i = lane; i <= E; i += kWave) soffs[i] = expert_offs[i];
          __builtin_amdgcn_s_waitcnt(0xc07f);
          __builtin_amdgcn_wave_barrier();
          auto raw_of = [&](int t) { return expert_key(t, token_slot[t], soffs, E, eslots); };
          if (T <= 4 * kWave)
            addressing_one_wave_keys<4>(raw_of, T, slots, order_out, indptr_out, (int*)red);
          else
            addressing_one_wave_keys<2 * NW>(raw_of, T, slots, order_out, indptr_out,
                                             (int*)red);
        }
      }
      return;
    }
    bid -= 8;
  }

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
    int seg0 = 0, n, tm = 0;
    if constexpr (MODE == kFromSlots) {
      tm = wave_slot_token(token_slot, 0, T, s, lane & 15, n);
    } else if constexpr (MODE == kFromExperts) {
      const int e = s / eslots;
      int lo = expert_offs[e], hi = expert_offs[e + 1];
      lo = min(max(lo, 0), T);
      hi = min(max(hi, lo), T);
      tm = wave_slot_token(token_slot, lo, hi, s - e * eslots, lane & 15, n);
    } else {
      segment_of(indptr, s, T, seg0, n);
    }
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
    d.early = early;
    d.tok_given = MODE != kFromAddr;
    d.tok_m = tm;
    d.lg = RT == 1 ? 0u : RT == 2 ? 1u : RT == 4 ? 2u : RT == 8 ? 3u : 4u;
    const rsrc_t a_r = make_rsrc((const char*)a_ + ((int64_t)s * SR + (int64_t)i * R) * in * 2,
                                 (uint32_t)r * (uint32_t)in * 2u);
    // the KP partial tiles of (s, i) and their ticket counters: tile index
    // j = (s * S + i) * KP + kp
    const int64_t j0 = ((int64_t)s * S + i) * KP;
    uint64_t* tiles = part + j0 * kMT * RP;
    uint32_t* cnts = tickets + j0;
    if (is_shrink) {
      const int kp = rem - i * KP;
      shrink_piece<RT, NW>(d, a_r, r, seg0, n, tiles + kp * kMT * RP, cnts + kp,
                           ct.per_slice[i], kp, red, scratch, lane, w, tid,
                           RT == 1 ? lds + L::kStage : nullptr);
    } else {
      const rsrc_t b_r =
          make_rsrc((const char*)b_ + (int64_t)s * out * R * 2, (uint32_t)out * (uint32_t)R * 2u);
      // tile order (tile_of): adjacent runs per wave, y through LDS, for a
      // chunk of one or two full groups of tiles at one rank tile
      const int cw = ct.c1[rem] - ct.c0[rem];
      if constexpr (RT == 1) {
        if (cw == 16 * NW * 8 || cw == 32 * NW * 8) {
          expand_piece<RT, NW, true>(d, a_r, b_r, r, scalings[s], seg0, n, ct.c0[rem],
                                     ct.c1[rem], tiles, cnts, red, hhi, hlo, scratch, lane, w,
                                     tid, lds + L::kStage);
          return;
        }
      }
      expand_piece<RT, NW, false>(d, a_r, b_r, r, scalings[s], seg0, n, ct.c0[rem], ct.c1[rem],
                                  tiles, cnts, red, hhi, hlo, scratch, lane, w, tid,
                                  lds + L::kStage);
    }
    return;
  }

  // prefill item: a block of 16 tokens of a long segment, every slice and column
  int* hist = (int*)red;   // one-launch forms: per-slot token counts of the batch
  if constexpr (MODE == kFromSlots) {
    if (tid < kWave) hist[tid] = 0;
    __syncthreads();
    for (int t = tid; t < T; t += NW * kWave) {
      const int v = token_slot[t];
      if (v >= 0 && v < slots) atomicAdd(hist + v, 1);
    }
    __syncthreads();
  } else if constexpr (MODE == kFromExperts) {
    for (int i = tid; i <= slots; i += NW * kWave) hist[i] = 0;
    for (int i = tid; i <= E; i += NW * kWave) soffs[i] = expert_offs[i];
    __syncthreads();
    for (int t = tid; t < T; t += NW * kWave) {
      const int v = expert_key(t, token_slot[t], soffs, E, eslots);
      if (v >= 0) atomicAdd(hist + v, 1);
    }
    __syncthreads();
  }
  auto count = [&](int ss) -> int {
    int b0, nn;
    if constexpr (MODE != kFromAddr)
      nn = hist[ss];
    else
      segment_of(indptr, ss, T, b0, nn);
    const int rr = clamp_rank(ranks[ss], R);
    return (nn > kMT && rr > 0) ? (nn + kMT - 1) / kMT : 0;
  };
  const SlotItem it = locate_item(bid - n_shrink - n_expand, slots, count, scratch);
  if (it.slot < 0) return;
  const int s = it.slot;
  const int r = clamp_rank(ranks[s], R);
  const int mb = it.local;
  if constexpr (MODE == kFromSlots) {
    slot_tokens<NW>(token_slot, 0, T, s, mb * kMT, -1, tok, tcnt, tid, lane, w);
  } else if constexpr (MODE == kFromExperts) {
    const int e = s / eslots;
    int lo = soffs[e], hi = soffs[e + 1];
    lo = min(max(lo, 0), T);
    hi = min(max(hi, lo), T);
    slot_tokens<NW>(token_slot, lo, hi, s - e * eslots, mb * kMT, -1, tok, tcnt, tid, lane, w);
  } else {
    int seg0, n;
    segment_of(indptr, s, T, seg0, n);
    const int ntok = min(kMT, n - mb * kMT);
    if (tid < kMT) tok[tid] = tid < ntok ? token_at(token_order, seg0 + mb * kMT + tid, T) : -1;
    __syncthreads();
  }
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
  d.early = 0;
  d.tok_given = false;
  d.tok_m = 0;
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

// k_apply_fused: the regions above, then (one rank tile) the staged A rows
// of the decode shrink pieces (Lds::kStage, Lds::kStageBytes)
size_t fused_lds_bytes(int rt) {
  static_assert(Lds<1, kNW>::kBytes == 256 + kNW * kMT * 16 * 4 + 2 * kMT * 20 * 2,
                "host and device LDS layouts");
  return rt == 1 ? (size_t)Lds<1, kNW>::kTotal : lds_bytes(rt, kNW);
}

int env_int(const char* name, int dflt) {
  const char* e = getenv(name);
  return e ? atoi(e) : dflt;
}

const void* fused_kernel(int rt, int mode) {
#define K(RTV)                                                                  \
  (mode == kFromExperts ? (const void*)k_apply_fused<RTV, kNW, kFromExperts>   \
   : mode == kFromSlots ? (const void*)k_apply_fused<RTV, kNW, kFromSlots>     \
                        : (const void*)k_apply_fused<RTV, kNW, kFromAddr>)
  switch (rt) {
    case 1: return K(1);
    case 2: return K(2);
    case 4: return K(4);
    case 8: return K(8);
    default: return K(16);
  }
#undef K
}

// Workgroups of a kernel instance that the current device holds at once
// (occupancy per CU x CUs), cached per instance and device; 0 if the
// runtime cannot say.
int64_t resident_blocks(const void* fn, int threads, size_t lds) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int64_t> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(fn, dev);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds) != hipSuccess)
    per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 0;
  const int64_t r = (int64_t)per_cu * cus;
  cache[key] = r;
  return r;
}

int decode_chunk_cols(int R, int out, int slots) {
  // columns per decode expand piece: 1024 up to rank 32, else 2048; twice
  // that when a batch of many slots would otherwise make more than 512
  // expand pieces, whose fixed cost (ticket, token ids, wait) then dominates
  // (measured on the routed-expert gate/up, 256 pool entries x 28672
  // outputs: 103.6 -> 93.5 us; on the routed-expert down, 1024 pieces of
  // 1024 columns, with y staged: 36.1 -> 34.3-34.7 us; the 32-slot qkv
  // decode, 192 pieces, keeps 1024: 2048 took 11.8 against 10.7 us);
  // overridable for tuning experiments
  const int env = env_int("LORA_DECODE_CHUNK", 0);
  if (env >= 16 && env % 16 == 0) return env;
  int cols = R <= 32 ? 1024 : 2048;
  if ((int64_t)slots * ((out + cols - 1) / cols) > 512) cols *= 2;
  return cols;
}

int k_parts(int in, int out, int slots, int S) {
  // K parts of a decode shrink: ~2048 deep, or ~1024 when the output is
  // narrower than one expand chunk (a router's logits: then every slot has a
  // single expand piece, and more, shorter shrink pieces shorten the chain:
  // measured at 64 outputs, 9.5 -> 8.1 us for 2 -> 4 parts; 8 parts 9.4 us);
  // then fewer while the shrink pieces (slots x slices x parts) would number
  // more than 512 (the routed-expert down product, 256 pool entries, in
  // 14336: 7 parts 41.1 us, 4 parts 39.0 us before A was staged; staged,
  // 7 / 4 / 3 / 2 parts 39.3 / 36.1 / 36.0 / 35.0 us; its gate/up, 2 slices,
  // 1 part as fast as 2); overridable for tuning
  const int env = env_int("LORA_KPARTS", 0);
  int kp = env > 0 ? env : in / (out < 1024 ? 1024 : 2048);
  kp = kp < 1 ? 1 : kp > 8 ? 8 : kp;
  if (env <= 0)
    while (kp > 1 && (int64_t)slots * S * kp > 512) --kp;
  return kp;
}

// Expand chunks: each slice cut into pieces of at most `cols` columns (a
// multiple of 16), at most kMaxChunks in all.
ChunkTable make_chunks(const SliceTable& st, int R, int slots) {
  ChunkTable ct;
  int cols = decode_chunk_cols(R, st.off[st.n], slots);
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
  // fixed size: a ticket counter for every partial tile index any call can
  // use (8192 slots x 8 slices x 8 K parts = 2^19; 2^20 reserved), so calls
  // of different shapes share one workspace without their regions
  // overlapping
  (void)slots;
  (void)S;
  return (size_t)1 << 22;
}

size_t fused_partial_bytes(int slots, int S, int R, int in) {
  const int RP = rt_bucket(R) * 16;
  // room for the most parts any output width takes; 8 bytes per entry
  // (value and tag)
  return (size_t)slots * S * k_parts(in, 0, 1, 1) * kMT * RP * sizeof(uint64_t);
}

bool fused_from_slots_supported(int T, int slots) {
  // slot_tokens covers 2 * 512 tokens; the one-wave sort 64 keys
  return T <= 2 * kNW * kWave && slots + 1 <= kWave;
}

bool fused_from_experts_supported(int T, int E, int eslots) {
  // slot_tokens covers 2 * 512 rows; the bounds (64) and the key histogram
  // (1024) share the first 1088 words of the reduction area
  return T <= 2 * kNW * kWave && E >= 1 && eslots >= 1 && E + 1 <= kWave &&
         (int64_t)E * eslots + 1 <= 1024;
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
                              hipStream_t stream, const int32_t* token_slot, int32_t* order_out,
                              int32_t* indptr_out, const int32_t* expert_offs, int E,
                              int eslots) {
  if (T == 0) return hipSuccess;
  const int mode = token_slot == nullptr ? kFromAddr
                   : expert_offs != nullptr ? kFromExperts : kFromSlots;
  const bool fs = mode != kFromAddr;
  if (mode == kFromSlots && !fused_from_slots_supported(T, slots)) return hipErrorInvalidValue;
  if (mode == kFromExperts &&
      (!fused_from_experts_supported(T, E, eslots) || slots != E * eslots))
    return hipErrorInvalidValue;
  const ChunkTable ct = make_chunks(st, R, slots);
  const int rt = rt_bucket(R);
  const size_t lds = fused_lds_bytes(rt);
  const void* fn = fused_kernel(rt, mode);
  if (lds > 65536) {
    hipError_t e =
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  int KP = k_parts(in, st.off[st.n], slots, st.n);
  // One rank tile stages A (8 K steps of 32 per wave, 2048 per workgroup):
  // a part shallower than that leaves waves without steps, so the count
  // stays at the ~2048-deep rule there (32-slot qkv decode, in 4096: 2 parts
  // 10.39-10.47 us per step against 10.73 with 3 and 13.2 with 4).
  if (env_int("LORA_KPARTS", 0) <= 0 && rt != 1) {
    // More K parts while every live piece (one per slot, slice and part, and
    // one per slot and column chunk) still fits on the chip at once, and each
    // part stays at least 1024 deep: more shrink pieces put more loads in
    // flight (the 32-slot qkv decode, 2 -> 3 parts: 480 pieces, 12.46 ->
    // 12.29 us per step; 4 parts make 576, more than the 512 the chip holds,
    // and take 16.9 us)
    const int64_t resident = resident_blocks(fn, kNW * kWave, lds);
    const int64_t live_expand = (int64_t)slots * ct.n;
    while (KP < 8 && in / (KP + 1) >= 1024 &&
           (int64_t)slots * st.n * (KP + 1) + live_expand <= resident)
      ++KP;
  }
  const int64_t slots8 = 8 * (int64_t)((slots + 7) / 8);
  // rank classes (largest first) where ranks differ enough to matter
  const int nclass = rt_bucket(R) >= 4 ? 3 : 1;
  const int64_t n_shrink = nclass * slots8 * st.n * KP;
  const int64_t n_expand = nclass * slots8 * ct.n;
  // prefill items: only slots with more than kMT tokens have any, at most
  // T / (kMT + 1) of them, each ceil(n / kMT) < n / kMT + 1 items, so at
  // most ceil(T / kMT) + min(slots, T / (kMT + 1)) in all (items past the
  // total leave at once)
  const int64_t n_prefill =
      (T + kMT - 1) / kMT + std::min<int64_t>(slots, (int64_t)T / (kMT + 1));
  const int64_t grid = n_shrink + n_expand + n_prefill + (fs ? 8 : 0);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  uint32_t* tickets = (uint32_t*)workspace;
  uint64_t* part = (uint64_t*)((char*)workspace + counter_bytes(slots, st.n));
  // bound of the wait of an expand piece (iterations of ~0.1-1 us); 0 makes
  // every expand piece compute h itself (used by the tests of that path)
  const int spin_limit = env_int("LORA_SPIN_LIMIT", 1 << 13);
  // early partial-entry reads only where the shrink and expand pieces
  // outnumber four per CU (about twice what the chip holds at once), so
  // that most expand pieces start after their producers: measured on the
  // routed-expert rows (thousands of pieces) 93.0 -> 90.7 us (gate/up) and
  // 38.8 -> 37.4 us (down); on grids that run at once (the 32-slot decode,
  // a router's logits) the reads cost ~0.3 us
  const int early = n_shrink + n_expand > 1024 ? 1 : 0;
#define LAUNCH(RTV, MV)                                                                         \
  do {                                                                                          \
    hipLaunchKernelGGL((k_apply_fused<RTV, kNW, MV>), dim3((unsigned)grid), dim3(kNW * 64),     \
                       lds, stream, x, y, T, in, st, a, b, slots, R, token_order, indptr,       \
                       ranks, scalings, ct, (int)n_shrink, (int)n_expand, nclass, KP, part,     \
                       tickets, spin_limit, early, token_slot, order_out, indptr_out,           \
                       expert_offs, E, eslots);                                                 \
  } while (0)
#define LAUNCH_RT(MV)                 \
  switch (rt) {                       \
    case 1: LAUNCH(1, MV); break;     \
    case 2: LAUNCH(2, MV); break;     \
    case 4: LAUNCH(4, MV); break;     \
    case 8: LAUNCH(8, MV); break;     \
    default: LAUNCH(16, MV); break;   \
  }
  if (mode == kFromExperts) {
    LAUNCH_RT(kFromExperts)
  } else if (mode == kFromSlots) {
    LAUNCH_RT(kFromSlots)
  } else {
    LAUNCH_RT(kFromAddr)
  }
#undef LAUNCH_RT
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
  const ChunkTable ct = make_chunks(st, R, slots);
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
