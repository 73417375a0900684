// expand: y[t, off_i + o] += scalings[slot(t)] *
//         sum_{j < rank} h[t, i*R + j] * b[slot(t), off_i + o, j], in place.
//
// Follows the mstar lora.backend page, LoraBackend.expand_fused and
// expand_reference_; slice i's columns start at the sum of the widths before
// it (mstar.model.components.linear, FusedColumnLinear shard layout).
//
// VALU path: one workgroup of 256 threads per item (slot, block of 8 tokens
// of the slot's segment, chunk of 256 16-byte column vectors). Each lane owns
// the output columns of one 16-byte vector of y (8 bf16 or 4 f32), so every y
// access is a 16-byte load or store and a wave covers 1 KiB of a y row per
// token. Widths are multiples of the vector, so a lane never straddles two
// slices or runs past the row. The block's h rows (only
// columns below the rank, the rest are set to 0 without reading) sit in LDS
// and are read as broadcasts. B rows are read 8 ranks (16 bytes) at a time;
// ranks at or past the slot's rank are masked to 0 in registers, never used.
// Accumulation is fp32; y is rounded once (bf16: nearest-even).
#include "lora_common.h"
#include "lora_kernels.h"

namespace lora {

namespace {

constexpr int kTG = 8;    // tokens per item
constexpr int kBlock = 256;

// One 16-byte vector <-> E::kVec floats.
template <typename E>
__device__ __forceinline__ void load_vec(const char* p, float (&v)[E::kVec]) {
  if constexpr (E::kBytes == 2) {
    const u32x4 u = *(const u32x4*)p;
    v[0] = bf16lo(u.x); v[1] = bf16hi(u.x); v[2] = bf16lo(u.y); v[3] = bf16hi(u.y);
    v[4] = bf16lo(u.z); v[5] = bf16hi(u.z); v[6] = bf16lo(u.w); v[7] = bf16hi(u.w);
  } else {
    const f32x4 a = *(const f32x4*)p;
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  }
}

template <typename E>
__device__ __forceinline__ void store_vec(char* p, const float (&v)[E::kVec]) {
  if constexpr (E::kBytes == 2) {
    u32x4 u;
    u.x = pack_bf16x2(v[0], v[1]);
    u.y = pack_bf16x2(v[2], v[3]);
    u.z = pack_bf16x2(v[4], v[5]);
    u.w = pack_bf16x2(v[6], v[7]);
    *(u32x4*)p = u;
  } else {
    *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
  }
}

}  // namespace

template <typename E>
__global__ __launch_bounds__(kBlock) void k_expand_valu(void* __restrict__ y_, int T, SliceTable st,
                                                        const float* __restrict__ h,
                                                        const void* __restrict__ b_, int slots,
                                                        int R, const int32_t* __restrict__ token_order,
                                                        const int32_t* __restrict__ indptr,
                                                        const int32_t* __restrict__ ranks,
                                                        const float* __restrict__ scalings,
                                                        int max_seg) {
  __shared__ int scratch[24];
  extern __shared__ float hl[];  // [kTG][S*R]
  const int S = st.n;
  const int SR = S * R;
  const int out = st.off[S];
  constexpr int CPL = E::kVec;           // output columns per lane
  constexpr int kCols = kBlock * CPL;    // output columns per item
  const int nchunk = (out + kCols - 1) / kCols;
  auto count = [&](int s) -> int {
    int b0, n;
    segment_of(indptr, s, T, b0, n);
    const int r = clamp_rank(ranks[s], R);
    return (n > 0 && n <= max_seg && r > 0) ? nchunk * ((n + kTG - 1) / kTG) : 0;
  };
  const SlotItem it = locate_item(blockIdx.x, slots, count, scratch);
  if (it.slot < 0) return;
  const int s = it.slot;
  int seg0, n;
  segment_of(indptr, s, T, seg0, n);
  const int r = clamp_rank(ranks[s], R);
  const int nmb = (n + kTG - 1) / kTG;
  const int m = it.local % nmb;
  const int cc = it.local / nmb;
  const int ntok = min(kTG, n - m * kTG);
  const float scale = scalings[s];

  int tok[kTG];
#pragma unroll
  for (int q = 0; q < kTG; ++q) tok[q] = q < ntok ? token_at(token_order, seg0 + m * kTG + q, T) : 0;

  for (int idx = threadIdx.x; idx < kTG * SR; idx += kBlock) {
    const int q = idx / SR;
    const int c = idx - q * SR;
    float v = 0.0f;
    if (q < ntok && (c % R) < r) v = h[(int64_t)token_at(token_order, seg0 + m * kTG + q, T) * SR + c];
    hl[idx] = v;
  }
  __syncthreads();

  const int col0 = cc * kCols + threadIdx.x * CPL;
  if (col0 >= out) return;
  int i = 0;
  while (i + 1 < S && st.off[i + 1] <= col0) ++i;

  // ranks are read one 16-byte vector (RV ranks) at a time; R is a multiple
  // of RV, so the vector never leaves the row
  constexpr int RV = E::kVec;
  const int64_t brow = (int64_t)R * E::kBytes;
  const char* bb = (const char*)b_ + ((int64_t)s * out + col0) * brow;
  float acc[kTG][CPL];
#pragma unroll
  for (int q = 0; q < kTG; ++q)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[q][c] = 0.0f;

  for (int j0 = 0; j0 < r; j0 += RV) {
    float bv[CPL][RV];
#pragma unroll
    for (int c = 0; c < CPL; ++c) load_vec<E>(bb + c * brow + (int64_t)j0 * E::kBytes, bv[c]);
#pragma unroll
    for (int jj = 0; jj < RV; ++jj) {
      if (j0 + jj >= r) break;   // ranks past the slot's rank are never used
#pragma unroll
      for (int q = 0; q < kTG; ++q) {
        const float hv = hl[q * SR + i * R + j0 + jj];
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[q][c] = fmaf(hv, bv[c][jj], acc[q][c]);
      }
    }
  }

  char* yb = (char*)y_;
  const int64_t yrow = (int64_t)out * E::kBytes;
#pragma unroll
  for (int q = 0; q < kTG; ++q) {
    if (q >= ntok) break;
    char* p = yb + tok[q] * yrow + (int64_t)col0 * E::kBytes;
    float v[CPL];
    load_vec<E>(p, v);
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c] = fmaf(scale, acc[q][c], v[c]);
    store_vec<E>(p, v);
  }
}

hipError_t launch_expand(int dtype, void* y, int T, const SliceTable& st, const float* h,
                         const void* b, int slots, int R, const int32_t* token_order,
                         const int32_t* indptr, const int32_t* ranks, const float* scalings,
                         int max_seg, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int out = st.off[st.n];
  const int cols = kBlock * (dtype == kDtypeBF16 ? BF16::kVec : F32::kVec);
  const int64_t nchunk = (out + cols - 1) / cols;
  const int64_t grid = nchunk * ((T + kTG - 1) / kTG + slots);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const size_t lds = (size_t)kTG * st.n * R * sizeof(float);
  if (dtype == kDtypeBF16)
    hipLaunchKernelGGL(k_expand_valu<BF16>, dim3((unsigned)grid), dim3(kBlock), lds, stream, y, T,
                       st, h, b, slots, R, token_order, indptr, ranks, scalings, max_seg);
  else
    hipLaunchKernelGGL(k_expand_valu<F32>, dim3((unsigned)grid), dim3(kBlock), lds, stream, y, T, st,
                       h, b, slots, R, token_order, indptr, ranks, scalings, max_seg);
  return hipGetLastError();
}

}  // namespace lora
