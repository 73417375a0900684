// The base projection of a fused linear layer with the LoRA delta added in
// its epilogue (lora_fused_column_linear), bf16 on MFMA.
//
// Follows page "mstar.model.components.linear", FusedColumnLinear (the
// shards of a fused projection are one product whose output columns hold the
// shards in order: y = x @ W^T with W = [W_0; W_1; ...] stacked along the
// output dimension) and page "mstar.engine.resources.lora.backend",
// LoraBackend.apply_linear_ (the delta: y[t, slice i] += scaling * h[t, slice
// i] @ B[slot(t), slice i]^T with h = x @ A[slot(t)]^T). Page
// "spark_model/lora/target.rs" (module overview) names kernels that fuse the
// delta into the base projection's epilogue as the step after grouped
// shrink / expand kernels: here y = x @ W^T + delta is formed in registers
// and stored once, so the delta costs no read-modify-write of y.
//
// Work: one 512-thread workgroup (8 waves) per 256 x 256 tile of y (256
// positions of token_order x 256 output columns); wave (wm, wn) owns 128
// rows x 64 columns of it as 4 x 8 tiles of v_mfma_f32_16x16x32_bf16 with
// fp32 accumulators. The product is formed transposed (the W rows are the A
// operand, the x rows the B operand), so each lane ends with 4 consecutive
// output columns of one token. Rows are taken in token_order (tokens grouped
// by slot): x rows are gathered and y rows scattered by token id, and the
// rows of one tile belong to few slots.
// Main loop: K in steps of 32 through a ring of 4 LDS stages, each holding
// the x and W tiles (256 x 32 bf16 each); buffer loads write the ring
// directly (no registers), three stages ahead of the one being multiplied.
// The 16-byte chunks of a 64-byte row are stored at chunk ^ ((row >> 1) & 3)
// so that the operand reads of 16 rows spread over the LDS banks.
// Epilogue, per slot q with rows in the tile and rank r_q > 0, per 32 ranks:
// s_q * h of the rows of q (others zero), split into bf16 hi + lo, and the
// slot's B rows of the tile's columns are staged in LDS, and the delta is
// accumulated by two more MFMA K-steps (hi, lo) into the same accumulators
// (h is thus effectively fp32). A tile lies in one out slice (every slice
// width is a multiple of 256), so its h columns are that slice's.
// The result is rounded once to bf16 (nearest even) and stored.
#include "lora_common.h"
#include "lora_kernels.h"

namespace lora {

namespace {

constexpr int kGT = 256;         // tile rows and columns
constexpr int kGK = 32;          // K per stage
constexpr int kStages = 4;       // LDS ring: the stage being read + 3 in flight
constexpr int kGThreads = 512;
constexpr int kStageBytes = kGT * kGK * 2;   // one operand tile of one stage, bf16 (16 KB)
// LDS: stage s holds [x tile][W tile] at s * 2 * kStageBytes; then token ids
constexpr int kLdsTok = kStages * 2 * kStageBytes;
constexpr int kGemmLds = kLdsTok + kGT * 4 + 64;
// D[16x16] += A[16 x 32] . B[16 x 32]^T (v_mfma_f32_16x16x32_bf16): lane
// (m, g) gives row m, k in [8g, 8g + 8) of both operands and receives
// D[4g + i][m] in element i.
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace

// y = x @ W^T (+ the LoRA delta when h != nullptr), 256 x 256 tiles.
__global__ __launch_bounds__(kGThreads) void k_linear_lora(
    const void* __restrict__ x_, const void* __restrict__ w_, void* __restrict__ y_, int T,
    int in, int out, SliceTable st, const float* __restrict__ h, const void* __restrict__ b_,
    int slots, int R, const int32_t* __restrict__ token_order,
    const int32_t* __restrict__ indptr, const int32_t* __restrict__ ranks,
    const float* __restrict__ scalings, int mtiles, int ntiles) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int* tok = (int*)(lds + kLdsTok);
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = wave_id();
  const int wm = w >> 2;   // token half of the tile (128 rows)
  const int wn = w & 3;    // column quarter (64 columns)
  const int m = lane & 15;
  const int g = lane >> 4;

  // tile order: block b runs on XCD b % 8 and takes position
  // (b % 8) * per + b / 8 of a grouped order (8 token blocks at a time, the
  // token block varying fastest), so the ~32 tiles an XCD runs at once are
  // 8 token blocks x 4 column blocks: each x block is read by 4 of them and
  // each W block by 8 from the XCD's L2 (a single column block against 32
  // token blocks would stream 33 operand blocks per window instead of 12)
  const int G = mtiles * ntiles;
  const int per = (G + 7) / 8;
  const int bid = blockIdx.x;
  const int L = (bid & 7) * per + (bid >> 3);
  if (L >= G) return;
  constexpr int kGroupM = 8;
  const int grp = L / (kGroupM * ntiles);
  const int fm = grp * kGroupM;
  const int gsz = min(kGroupM, mtiles - fm);
  const int li = L - grp * kGroupM * ntiles;
  const int tm = fm + li % gsz;
  const int tn = li / gsz;
  const int m0 = tm * kGT;
  const int n0 = tn * kGT;

  // token id of every tile row (position m0 + row of token_order; the
  // identity without an addressing), -1 past T
  if (tid < kGT) {
    const int p = m0 + tid;
    tok[tid] = p >= T ? -1 : token_order ? min(max(token_order[p], 0), T - 1) : p;
  }
  __syncthreads();

  const rsrc_t x_r = make_rsrc(x_, (uint32_t)T * (uint32_t)in * 2u);
  const rsrc_t w_r = make_rsrc(w_, (uint32_t)out * (uint32_t)in * 2u);
  const uint32_t rowb = (uint32_t)in * 2u;

  // global -> LDS without registers (buffer_load ... lds): one instruction
  // of a wave fills a contiguous 1 KB block of LDS, lane L at byte 16 L, i.e.
  // rows 16 blk + L / 4, physical chunk L & 3 of a 64-byte row; the lane
  // fetches the logical chunk stored there (the swizzle is undone on the
  // global side). Wave w fills blocks w and w + 8 of both the x and the W
  // tile of a stage: 4 instructions per wave per stage.
  const int pr = lane >> 2;                          // row within the block
  const int pc = (lane & 3) ^ ((pr >> 1) & 3);       // logical chunk of the lane
  uint32_t xoff[2], woff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = (w + 8 * j) * 16 + pr;
    const int t = tok[row];
    xoff[j] = t >= 0 ? (uint32_t)t * rowb + (uint32_t)pc * 16u : kOOB;
    woff[j] = n0 + row < out ? (uint32_t)(n0 + row) * rowb + (uint32_t)pc * 16u : kOOB;
  }
  auto issue = [&](int stage, int k0) {
    const bool kv = k0 + pc * 8 < in;
    char* sb = lds + (stage % kStages) * 2 * kStageBytes;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int blk = w + 8 * j;
      dma16(x_r, sb + blk * 1024, kv && xoff[j] != kOOB ? xoff[j] + (uint32_t)k0 * 2u : kOOB);
      dma16(w_r, sb + kStageBytes + blk * 1024,
            kv && woff[j] != kOOB ? woff[j] + (uint32_t)k0 * 2u : kOOB);
    }
  };

  f32x4 acc[4][8];   // [column tile][token tile]
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kt = (in + kGK - 1) / kGK;
  // three stages in flight before the loop
  for (int st0 = 0; st0 < kStages - 1 && st0 < kt; ++st0) issue(st0, st0 * kGK);
  for (int it = 0; it < kt; ++it) {
    // this stage's loads are done once at most the later stages' (4 per
    // stage per wave) are outstanding; then the barrier makes every wave's
    // part visible, and frees the buffer read in the previous iteration
    const int ahead = min(kt - 1 - it, kStages - 2);
    if (ahead >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_le(8));
    else if (ahead == 1) __builtin_amdgcn_s_waitcnt(vmcnt_le(4));
    else __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
    barrier_no_fence();
    if (it + kStages - 1 < kt) issue(it + kStages - 1, (it + kStages - 1) * kGK);
    const char* xb = lds + (it % kStages) * 2 * kStageBytes;
    const char* wb = xb + kStageBytes;
    bf16x8 wo[4], xo[8];
#pragma unroll
    for (int a = 0; a < 4; ++a)
      wo[a] = *(const bf16x8*)(wb + swz4(wn * 64 + a * 16 + m, g));
#pragma unroll
    for (int a = 0; a < 8; ++a)
      xo[a] = *(const bf16x8*)(xb + swz4(wm * 128 + a * 16 + m, g));
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int bq = 0; bq < 8; ++bq) acc[a][bq] = mfma32(wo[a], xo[bq], acc[a][bq]);
    // all 12 operand reads first, then the 32 products (each waits only for
    // its own operands), instead of a full LDS wait before every few products
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 32, 0);
  }
  __syncthreads();   // the epilogue reuses the ring

  // ---- LoRA epilogue ----------------------------------------------------
  if (h != nullptr && m0 < T) {
    // the tile's slice (it lies in one) and the slots of its rows
    int si = 0;
    while (si + 1 < st.n && st.off[si + 1] <= n0) ++si;
    const int SR = st.n * R;
    const int pend = min(m0 + kGT, T);
    const int live_end = indptr[slots];   // positions past it are dead tokens
    int s = slot_of_position(indptr, slots, m0);
    const rsrc_t h_r = make_rsrc(h, (uint32_t)T * (uint32_t)SR * 4u);
    char* hb = lds;                        // [256 tokens][32 ranks] bf16 hi
    char* hl = lds + kGT * 64;             // lo
    char* bb = lds + 2 * kGT * 64;         // [256 columns][32 ranks] bf16
    for (; s < slots; ++s) {
      int seg0, n;
      segment_of(indptr, s, T, seg0, n);
      if (seg0 >= pend || seg0 >= live_end) break;
      const int r = clamp_rank(ranks[s], R);
      if (n == 0 || r == 0 || seg0 + n <= m0) continue;
      const float scale = scalings[s];
      const int p0 = max(seg0, m0) - m0;   // tile rows [p0, p1) belong to slot s
      const int p1 = min(seg0 + n, pend) - m0;
      const rsrc_t b_r = make_rsrc((const char*)b_ + (int64_t)s * out * R * 2,
                                   (uint32_t)out * (uint32_t)R * 2u);
      for (int c0 = 0; c0 < r; c0 += 32) {
        // stage s * h (rows of slot s; zeros elsewhere and past the rank),
        // split into hi + lo, one token row per thread of the first 256, and
        // B rows of the tile's columns, one column per thread of the rest
        if (tid < kGT) {
          const int row = tid;
          const int t = tok[row];
          const bool mine = row >= p0 && row < p1 && t >= 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {   // 8 ranks per chunk
            const int j0 = c0 + q * 8;
            u32x4 hv0 = u32x4{0u, 0u, 0u, 0u}, hv1 = u32x4{0u, 0u, 0u, 0u};
            if (mine) {
              const uint32_t off = ((uint32_t)t * (uint32_t)SR + (uint32_t)(si * R + j0)) * 4u;
              hv0 = bload16(h_r, off);
              hv1 = bload16(h_r, off + 16u);
            }
            // ranks j0 .. j0 + 7 in order, scaled; past r (never read) zero
            const uint32_t raw[8] = {hv0.x, hv0.y, hv0.z, hv0.w, hv1.x, hv1.y, hv1.z, hv1.w};
            uint32_t hbits[8], lbits[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float v = (j0 + e < r) ? __uint_as_float(raw[e]) * scale : 0.0f;
              hbits[e] = to_bf16_bits(v);
              lbits[e] = to_bf16_bits(v - __uint_as_float(hbits[e] << 16));
            }
            const u32x4 hp = u32x4{hbits[0] | (hbits[1] << 16), hbits[2] | (hbits[3] << 16),
                                   hbits[4] | (hbits[5] << 16), hbits[6] | (hbits[7] << 16)};
            const u32x4 lp = u32x4{lbits[0] | (lbits[1] << 16), lbits[2] | (lbits[3] << 16),
                                   lbits[4] | (lbits[5] << 16), lbits[6] | (lbits[7] << 16)};
            *(u32x4*)(hb + swz4(row, q)) = hp;
            *(u32x4*)(hl + swz4(row, q)) = lp;
          }
        } else {
          // B[s, n0 + row, c0 .. c0 + 32): ranks past r read as zero
          const int row = tid - kGT;
          const int col = n0 + row;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int j0 = c0 + q * 8;
            u32x4 bv = u32x4{0u, 0u, 0u, 0u};
            if (col < out && j0 < r) {
              bv = bload16(b_r, ((uint32_t)col * (uint32_t)R + (uint32_t)j0) * 2u);
              // clear ranks j0 + e >= r inside the chunk
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (j0 + e >= r) {
                  const uint32_t keep = (e & 1) ? 0x0000ffffu : 0xffff0000u;
                  if (e < 2) bv.x &= keep; else if (e < 4) bv.y &= keep;
                  else if (e < 6) bv.z &= keep; else bv.w &= keep;
                }
            }
            *(u32x4*)(bb + swz4(row, q)) = bv;
          }
        }
        __syncthreads();
        // two K steps over the 32 ranks: s * h hi, then lo
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const char* hsrc = part == 0 ? hb : hl;
          bf16x8 bo[4], ho[8];
#pragma unroll
          for (int a = 0; a < 4; ++a)
            bo[a] = *(const bf16x8*)(bb + swz4(wn * 64 + a * 16 + m, g));
#pragma unroll
          for (int a = 0; a < 8; ++a)
            ho[a] = *(const bf16x8*)(hsrc + swz4(wm * 128 + a * 16 + m, g));
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int bq = 0; bq < 8; ++bq) acc[a][bq] = mfma32(bo[a], ho[bq], acc[a][bq]);
        }
        __syncthreads();
      }
    }
  }

  // ---- store: one rounding to bf16 --------------------------------------
  // wait states between the last MFMA and the first vector read of its result
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  const rsrc_t y_r = make_rsrc(y_, (uint32_t)T * (uint32_t)out * 2u);
#pragma unroll
  for (int bq = 0; bq < 8; ++bq) {
    const int t = tok[wm * 128 + bq * 16 + m];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int col = n0 + wn * 64 + a * 16 + 4 * g;
      const f32x4 v = acc[a][bq];
      const uint32_t off = (t >= 0 && col < out) ? ((uint32_t)t * (uint32_t)out + (uint32_t)col) * 2u
                                                 : kOOB;
      bstore8(y_r, off, u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
    }
  }
}

bool linear_lora_supported(int dtype, const SliceTable& st, int R, int T, int in) {
  if (dtype != kDtypeBF16 || R > 256) return false;
  const int64_t lim = (int64_t)1 << 31;
  const int64_t out = st.off[st.n];
  if ((int64_t)T * in * 2 >= lim || (int64_t)T * out * 2 >= lim || out * (int64_t)in * 2 >= lim ||
      out * (int64_t)R * 2 >= lim || (int64_t)T * st.n * R * 4 >= lim)
    return false;
  for (int i = 0; i < st.n; ++i)
    if ((st.off[i + 1] - st.off[i]) % kGT != 0) return false;
  return in % 8 == 0;
}

hipError_t launch_linear_lora(const void* x, const void* w, void* y, int T, int in,
                              const SliceTable& st, const float* h, const void* b, int slots,
                              int R, const int32_t* token_order, const int32_t* indptr,
                              const int32_t* ranks, const float* scalings, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int out = st.off[st.n];
  const int mt = (T + kGT - 1) / kGT;
  const int nt = (out + kGT - 1) / kGT;
  const int64_t G = (int64_t)mt * nt;
  const int64_t grid = 8 * ((G + 7) / 8);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute((const void*)k_linear_lora,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_linear_lora, dim3((unsigned)grid), dim3(kGThreads), kGemmLds, stream, x, w,
                     y, T, in, out, st, h, b, slots, R, token_order, indptr, ranks, scalings, mt,
                     nt);
  return hipGetLastError();
}

}  // namespace lora
