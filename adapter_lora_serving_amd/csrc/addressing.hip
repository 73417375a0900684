// Device-side slot addressing: token_slot -> (token_order, slot_indptr).
//
// Follows the mstar lora.backend page (module overview: both kernels read the
// step's LoraAddressing, so eager and captured paths address slots alike).
// The grouping is a stable counting sort keyed by slot, dead tokens (slot
// outside [0, slots)) keyed after every live slot. One workgroup of up to 16
// waves does the whole batch, with no host round trip, so a serving step can
// be captured in a hipGraph:
//   1. wave w owns the contiguous token range [w*per, (w+1)*per) and counts
//      its keys into its own LDS histogram row;
//   2. per key, the rows are turned into per-wave starting offsets and a key
//      total; a block-wide exclusive scan of the totals gives slot_indptr;
//   3. each wave walks its range 64 tokens at a time; inside a group, lanes
//      sharing a key are ranked with ballots, so the order inside a segment is
//      ascending token index (stable) with no sorting network.
#include "lora_common.h"
#include "lora_kernels.h"

namespace lora {

__global__ __launch_bounds__(1024) void k_build_addressing(const int32_t* __restrict__ token_slot,
                                                           int T, int slots,
                                                           int32_t* __restrict__ token_order,
                                                           int32_t* __restrict__ slot_indptr) {
  extern __shared__ int smem[];
  const int nw = blockDim.x / kWave;
  const int S1 = slots + 1;
  int* cnt = smem;              // [nw][S1]: counts, then running write cursors
  int* tot = smem + nw * S1;    // [S1]: per-key totals, then segment starts
  int* scratch = tot + S1;      // [20]
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid / kWave;

  for (int i = tid; i < nw * S1; i += blockDim.x) cnt[i] = 0;
  __syncthreads();

  const int per = (T + nw - 1) / nw;
  const int t0 = min(T, w * per);
  const int t1 = min(T, t0 + per);
  for (int t = t0 + lane; t < t1; t += kWave) {
    int s = token_slot[t];
    int k = (s >= 0 && s < slots) ? s : slots;
    atomicAdd(&cnt[w * S1 + k], 1);
  }
  __syncthreads();

  for (int k = tid; k < S1; k += blockDim.x) {
    int run = 0;
    for (int q = 0; q < nw; ++q) {
      int c = cnt[q * S1 + k];
      cnt[q * S1 + k] = run;
      run += c;
    }
    tot[k] = run;
  }
  __syncthreads();

  // exclusive scan of the key totals: each thread owns a contiguous run of keys
  const int chunk = (S1 + blockDim.x - 1) / blockDim.x;
  const int k0 = min(S1, tid * chunk);
  const int k1 = min(S1, k0 + chunk);
  int local = 0;
  for (int k = k0; k < k1; ++k) local += tot[k];
  int run = block_exclusive_scan(local, scratch, nullptr);
  for (int k = k0; k < k1; ++k) {
    int c = tot[k];
    tot[k] = run;
    run += c;
  }
  __syncthreads();

  for (int k = tid; k < S1; k += blockDim.x) {
    const int start = tot[k];
    slot_indptr[k] = start;
    for (int q = 0; q < nw; ++q) cnt[q * S1 + k] += start;
  }
  __syncthreads();

  // stable scatter: only wave w touches row w of cnt, so no atomics here
  int* cur = cnt + w * S1;
  for (int base = t0; base < t1; base += kWave) {
    const int t = base + lane;
    const bool valid = t < t1;
    int k = -1;
    if (valid) {
      int s = token_slot[t];
      k = (s >= 0 && s < slots) ? s : slots;
    }
    uint64_t active = __ballot(valid);
    while (active) {
      const int leader = __ffsll((unsigned long long)active) - 1;
      const int kl = __shfl(k, leader);
      const uint64_t m = __ballot(valid && k == kl) & active;
      int pos0 = 0;
      if (lane == leader) pos0 = cur[kl];
      pos0 = __shfl(pos0, leader);
      if ((m >> lane) & 1ull) {
        const int rank = __popcll(m & ((1ull << lane) - 1ull));
        token_order[pos0 + rank] = t;
      }
      if (lane == leader) cur[kl] = pos0 + __popcll(m);
      active &= ~m;
    }
  }
}

int addressing_waves(int64_t T, int slots) {
  int nw = (int)((T + kWave - 1) / kWave);
  if (nw < 1) nw = 1;
  if (nw > 16) nw = 16;
  // keep the LDS footprint (nw + 1) * (slots + 1) ints within 64 KiB
  const int max_nw = (int)(65536 / (4 * (int64_t)(slots + 1))) - 1;
  if (nw > max_nw) nw = max_nw;
  return nw < 1 ? 1 : nw;
}

size_t addressing_lds_bytes(int nw, int slots) {
  return (size_t)((nw + 1) * (slots + 1) + 20) * sizeof(int);
}

hipError_t launch_build_addressing(const int32_t* token_slot, int T, int slots,
                                   int32_t* token_order, int32_t* slot_indptr,
                                   hipStream_t stream) {
  const int nw = addressing_waves(T, slots);
  const size_t lds = addressing_lds_bytes(nw, slots);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)k_build_addressing,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_build_addressing, dim3(1), dim3(nw * kWave), lds, stream, token_slot, T,
                     slots, token_order, slot_indptr);
  return hipGetLastError();
}

}  // namespace lora
