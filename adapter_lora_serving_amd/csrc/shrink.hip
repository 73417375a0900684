// shrink: h[t, i*R + j] = x[t] . a[slot(t), i*R + j] for j < rank(slot(t)).
//
// Follows the mstar lora.backend page, LoraBackend.shrink and
// shrink_reference (zeros where the expand does not read: dead tokens, rank-0
// slots, columns at or past a slot's rank).
//
// VALU path (BGMV-shaped): one workgroup of 4 waves per item
// (slot, slice, group of 8 A rows, block of 8 tokens of the slot's segment).
// The reduction dimension `in` is split across the waves and lanes: lane l of
// wave w reads the 16-byte vector at element (c*64 + l)*VEC of K-chunk c,
// c = w, w+4, ...; every A row and every x row is therefore streamed with
// fully coalesced 16-byte loads, each A vector is used for 8 tokens and each
// x vector for 8 rows. bf16 products use v_dot2_f32_bf16 (two bf16 products
// summed in fp32). At the end each wave folds its 64 (token, row) partial sums
// across the 64 lanes with a transpose-reduction (63 exchanges instead of
// 64*6) and the 4 waves are added in a fixed order through LDS, so results
// are deterministic run to run.
//
// Extra workgroups after the compute items write the zeros: one thread per
// (position, column) with column % R >= rank(slot). Segments longer than
// max_seg are left to the SGMV kernel (their zeros are still written here).
#include "lora_common.h"
#include "lora_kernels.h"

namespace lora {

namespace {

constexpr int kRG = 8;  // A rows per item
constexpr int kTG = 8;  // tokens per item

template <typename E>
__device__ __forceinline__ float dot16(const u32x4& x, const u32x4& a, float acc) {
  if constexpr (E::kBytes == 2) {
    acc = dot2_bf16(x.x, a.x, acc);
    acc = dot2_bf16(x.y, a.y, acc);
    acc = dot2_bf16(x.z, a.z, acc);
    acc = dot2_bf16(x.w, a.w, acc);
  } else {
    acc = fmaf(__uint_as_float(x.x), __uint_as_float(a.x), acc);
    acc = fmaf(__uint_as_float(x.y), __uint_as_float(a.y), acc);
    acc = fmaf(__uint_as_float(x.z), __uint_as_float(a.z), acc);
    acc = fmaf(__uint_as_float(x.w), __uint_as_float(a.w), acc);
  }
  return acc;
}

// On entry each lane holds 64 partial sums v[0..63]; on exit lane l returns
// the sum over all lanes of v[l]. Each halving step keeps the half of the
// values selected by one lane bit and swaps the other half with the partner.
__device__ __forceinline__ float wave_transpose_reduce64(float (&v)[64]) {
  const int lane = lane_id();
#pragma unroll
  for (int half = 32; half >= 1; half >>= 1) {
    const bool upper = (lane & half) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float keep = upper ? v[i + half] : v[i];
      const float send = upper ? v[i] : v[i + half];
      v[i] = keep + __shfl_xor(send, half);
    }
  }
  return v[0];
}

}  // namespace

template <typename E>
__global__ __launch_bounds__(256) void k_shrink_valu(const void* __restrict__ x_, int T, int in,
                                                     const void* __restrict__ a_, int slots, int S,
                                                     int R, const int32_t* __restrict__ token_order,
                                                     const int32_t* __restrict__ indptr,
                                                     const int32_t* __restrict__ ranks,
                                                     float* __restrict__ h, int n_compute,
                                                     int max_seg) {
  __shared__ int scratch[24];
  __shared__ float part[4][64];
  const int SR = S * R;
  const int tid = threadIdx.x;

  if ((int)blockIdx.x >= n_compute) {
    // zero-fill: every (position, column) the compute items do not write
    const int64_t g = (int64_t)(blockIdx.x - n_compute) * blockDim.x + tid;
    if (g >= (int64_t)T * SR) return;
    const int p = (int)(g / SR);
    const int c = (int)(g - (int64_t)p * SR);
    const int s = slot_of_position(indptr, slots, p);
    const int r = s < slots ? clamp_rank(ranks[s], R) : 0;
    if (c % R >= r) h[(int64_t)token_at(token_order, p, T) * SR + c] = 0.0f;
    return;
  }

  auto count = [&](int s) -> int {
    int b0, n;
    segment_of(indptr, s, T, b0, n);
    const int r = clamp_rank(ranks[s], R);
    return (n > 0 && n <= max_seg && r > 0) ? S * ((r + kRG - 1) / kRG) * ((n + kTG - 1) / kTG) : 0;
  };
  const SlotItem it = locate_item(blockIdx.x, slots, count, scratch);
  if (it.slot < 0) return;
  const int s = it.slot;
  int seg0, n;
  segment_of(indptr, s, T, seg0, n);
  const int r = clamp_rank(ranks[s], R);
  const int nmb = (n + kTG - 1) / kTG;
  const int ng = (r + kRG - 1) / kRG;
  const int m = it.local % nmb;
  const int rest = it.local / nmb;
  const int g = rest % ng;
  const int i = rest / ng;

  const int lane = lane_id();
  const int w = tid / kWave;
  constexpr int VEC = E::kVec;
  const int64_t rowbytes = (int64_t)in * E::kBytes;
  const char* xb = (const char*)x_;
  const char* ab = (const char*)a_ + ((int64_t)s * SR + (int64_t)i * R + g * kRG) * rowbytes;

  int tok[kTG];
  const int ntok = min(kTG, n - m * kTG);
  const int nrow = min(kRG, r - g * kRG);
#pragma unroll
  for (int q = 0; q < kTG; ++q) tok[q] = q < ntok ? token_at(token_order, seg0 + m * kTG + q, T) : 0;

  float acc[64];
#pragma unroll
  for (int k = 0; k < 64; ++k) acc[k] = 0.0f;

  const int CK = kWave * VEC;
  const int nchunks = (in + CK - 1) / CK;
  for (int c = w; c < nchunks; c += 4) {
    const int e = c * CK + lane * VEC;
    const bool kv = e < in;
    u32x4 av[kRG], xv[kTG];
#pragma unroll
    for (int rr = 0; rr < kRG; ++rr) {
      av[rr] = u32x4{0, 0, 0, 0};
      if (rr < nrow && kv) av[rr] = *(const u32x4*)(ab + rr * rowbytes + (int64_t)e * E::kBytes);
    }
#pragma unroll
    for (int q = 0; q < kTG; ++q) {
      xv[q] = u32x4{0, 0, 0, 0};
      if (q < ntok && kv) xv[q] = *(const u32x4*)(xb + tok[q] * rowbytes + (int64_t)e * E::kBytes);
    }
#pragma unroll
    for (int q = 0; q < kTG; ++q)
#pragma unroll
      for (int rr = 0; rr < kRG; ++rr) acc[q * kRG + rr] = dot16<E>(xv[q], av[rr], acc[q * kRG + rr]);
  }

  const float mine = wave_transpose_reduce64(acc);
  part[w][lane] = mine;
  __syncthreads();
  if (w == 0) {
    const float v = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
    const int q = lane / kRG;
    const int rr = lane % kRG;
    if (q < ntok && rr < nrow) h[(int64_t)tok[q] * SR + i * R + g * kRG + rr] = v;
  }
}

hipError_t launch_shrink(int dtype, const void* x, int T, int in, const void* a, int slots,
                         int S, int R, const int32_t* token_order, const int32_t* indptr,
                         const int32_t* ranks, float* h, int max_seg, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  // upper bound of compute items: sum over slots of S*ceil(r/8)*ceil(n/8)
  // (none when max_seg is 0: then only the zeros are written)
  const int64_t n_compute =
      max_seg > 0 ? (int64_t)S * ((R + kRG - 1) / kRG) * ((T + kTG - 1) / kTG + slots) : 0;
  const int64_t n_zero = ((int64_t)T * S * R + 255) / 256;
  const int64_t grid = n_compute + n_zero;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (dtype == kDtypeBF16)
    hipLaunchKernelGGL(k_shrink_valu<BF16>, dim3((unsigned)grid), dim3(256), 0, stream, x, T, in,
                       a, slots, S, R, token_order, indptr, ranks, h, (int)n_compute, max_seg);
  else
    hipLaunchKernelGGL(k_shrink_valu<F32>, dim3((unsigned)grid), dim3(256), 0, stream, x, T, in, a,
                       slots, S, R, token_order, indptr, ranks, h, (int)n_compute, max_seg);
  return hipGetLastError();
}

}  // namespace lora
