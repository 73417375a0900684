// Device-side slot addressing: token_slot -> (token_order, slot_indptr).
//
// Follows the mstar lora.backend page (module overview: the shrink and the
// expand take their slot addressing from the pool's per-step addressing
// object, so an eager step and a captured graph address slots the same way).
// The grouping is a stable counting sort keyed by slot, dead tokens (slot
// outside [0, slots)) keyed after every live slot. One workgroup of up to 16
// waves does the whole batch, with no host round trip, so a serving step can
// be captured in a hipGraph (a batch of at most 1024 tokens over at most 63
// slots takes the one-wave kernel below instead):
//   1. wave w owns the contiguous token range [w*per, (w+1)*per); for every
//      group of 64 tokens each lane finds the lanes holding the same key with
//      one ballot per key bit (log2(slots+1) ballots, independent of how many
//      distinct keys the group has), which gives its rank among equal keys
//      and the group's count; the group leaders add the counts into the
//      wave's own LDS histogram row;
//   2. per key, the rows are turned into per-wave starting offsets and a key
//      total; a block-wide exclusive scan of the totals gives slot_indptr;
//   3. each wave walks its groups again: position = the wave's cursor for the
//      key + the lane's rank, so a segment lists its tokens in ascending
//      index (stable). Keys and ranks of the first kCache groups stay in
//      registers between the passes.
#include "lora_common.h"
#include "lora_kernels.h"

namespace lora {

namespace {

constexpr int kCache = 8;   // 64-token groups per wave kept in registers

__device__ __forceinline__ GroupMatch match_group(const int32_t* __restrict__ token_slot, int t,
                                                  bool valid, int slots, int nbits) {
  return match_raw(valid ? token_slot[t] : -1, valid, slots, nbits);
}

}  // namespace

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
  const int nbits = 32 - __clz(slots);   // bits of the largest key (= slots)

  for (int i = tid; i < nw * S1; i += blockDim.x) cnt[i] = 0;
  __syncthreads();

  const int per = (T + nw - 1) / nw;
  const int t0 = min(T, w * per);
  const int t1 = min(T, t0 + per);
  int* row = cnt + w * S1;
  const int ng = (t1 - t0 + kWave - 1) / kWave;   // this wave's groups (uniform)
  // the first kCache groups are unrolled (their matches stay in registers,
  // indexed at compile time); any further ones loop
  GroupMatch cache[kCache];
#pragma unroll
  for (int c = 0; c < kCache; ++c) {
    const int t = t0 + c * kWave + lane;
    cache[c] = c < ng ? match_group(token_slot, t, t < t1, slots, nbits)
                      : GroupMatch{-1, 0, 0, false};
  }
#pragma unroll
  for (int c = 0; c < kCache; ++c)   // distinct keys: no two leaders of a group collide
    if (cache[c].leader) row[cache[c].key] += cache[c].count;
  for (int c = kCache; c < ng; ++c) {
    const int t = t0 + c * kWave + lane;
    const GroupMatch g = match_group(token_slot, t, t < t1, slots, nbits);
    if (g.leader) row[g.key] += g.count;
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

  // stable scatter: only wave w touches row w of cnt
  auto scatter = [&](const GroupMatch& g, int t) {
    int pos = 0;
    if (t < t1) pos = row[g.key] + g.rank;
    __builtin_amdgcn_wave_barrier();
    if (g.leader) row[g.key] += g.count;
    if (t < t1) token_order[pos] = t;
  };
#pragma unroll
  for (int c = 0; c < kCache; ++c)
    if (c < ng) scatter(cache[c], t0 + c * kWave + lane);
  for (int c = kCache; c < ng; ++c) {
    const int t = t0 + c * kWave + lane;
    scatter(match_group(token_slot, t, t < t1, slots, nbits), t);
  }
}

// Small batches over at most 63 slots: one wave sorts the whole batch (G
// groups of 64 tokens, all slots loaded at once) with no workgroup barrier
// (addressing_one_wave).
template <int G>
__global__ __launch_bounds__(64) void k_build_addressing_wave(
    const int32_t* __restrict__ token_slot, int T, int slots, int32_t* __restrict__ token_order,
    int32_t* __restrict__ slot_indptr) {
  __shared__ int hist[kWave];
  addressing_one_wave<G>(token_slot, T, slots, token_order, slot_indptr, hist);
}

// Large batches with a workspace: two passes over blocks of 1024 tokens
// (16 waves x one group each). Pass 1 writes each block's per-key counts to
// the workspace; pass 2 gives every block the count of each key in the
// blocks before it and the key totals (so the segment starts), and scatters
// its tokens: position = segment start + count in earlier blocks + count in
// earlier waves of the block + rank in the group. Stable, like the
// one-workgroup kernel, and spread over ceil(T/1024) workgroups.
constexpr int kBlockTok = 16 * kWave;

__global__ __launch_bounds__(1024) void k_addr_block_hist(const int32_t* __restrict__ token_slot,
                                                          int T, int slots,
                                                          int32_t* __restrict__ ws) {
  extern __shared__ int smem[];   // [16][S1] per-wave counts
  const int S1 = slots + 1;
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int nbits = 32 - __clz(slots);
  for (int i = tid; i < 16 * S1; i += kBlockTok) smem[i] = 0;
  const int t = blockIdx.x * kBlockTok + tid;
  const GroupMatch g = match_group(token_slot, t, t < T, slots, nbits);
  __syncthreads();
  if (g.leader) smem[w * S1 + g.key] += g.count;   // distinct keys: no collision
  __syncthreads();
  for (int k = tid; k < S1; k += kBlockTok) {
    int c = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) c += smem[q * S1 + k];
    ws[(int64_t)blockIdx.x * S1 + k] = c;
  }
}

__global__ __launch_bounds__(1024) void k_addr_block_scatter(
    const int32_t* __restrict__ token_slot, int T, int slots, const int32_t* __restrict__ ws,
    int nb, int32_t* __restrict__ token_order, int32_t* __restrict__ slot_indptr) {
  extern __shared__ int smem[];
  const int S1 = slots + 1;
  int* cnt = smem;              // [16][S1]: per-wave counts, then offsets in the block
  int* base = cnt + 16 * S1;    // [S1]: segment start + count in earlier blocks
  int* scratch = base + S1;     // [20]
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int nbits = 32 - __clz(slots);
  const int b = blockIdx.x;
  for (int i = tid; i < 16 * S1; i += kBlockTok) cnt[i] = 0;
  const int t = b * kBlockTok + tid;
  const GroupMatch g = match_group(token_slot, t, t < T, slots, nbits);
  __syncthreads();
  if (g.leader) cnt[w * S1 + g.key] += g.count;
  __syncthreads();
  // key k = tid (S1 <= 1024): total over all blocks, count in earlier ones,
  // and the offsets of the block's waves
  int tot = 0, pre = 0;
  if (tid < S1) {
    for (int bb = 0; bb < nb; ++bb) {
      const int c = ws[(int64_t)bb * S1 + tid];
      tot += c;
      pre += bb < b ? c : 0;
    }
    int run = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int c = cnt[q * S1 + tid];
      cnt[q * S1 + tid] = run;
      run += c;
    }
  }
  const int start = block_exclusive_scan(tid < S1 ? tot : 0, scratch, nullptr);
  if (tid < S1) {
    base[tid] = start + pre;
    if (b == 0) slot_indptr[tid] = start;
  }
  __syncthreads();
  if (t < T) token_order[base[g.key] + cnt[w * S1 + g.key] + g.rank] = t;
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

// Composite key of each row of an expert-sorted batch (expert_key).
__global__ __launch_bounds__(256) void k_expert_keys(const int32_t* __restrict__ row_slot,
                                                     const int32_t* __restrict__ offs, int E,
                                                     int rows, int slots,
                                                     int32_t* __restrict__ keys) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  keys[r] = expert_key(r, row_slot[r], offs, E, slots);
}

size_t addressing_workspace_bytes(int64_t T, int slots) {
  // the two-pass path: batches past one block, keys within one per thread
  if (T <= kBlockTok || slots + 1 > kBlockTok) return 0;
  const int64_t nb = (T + kBlockTok - 1) / kBlockTok;
  return (size_t)nb * (slots + 1) * sizeof(int32_t);
}

hipError_t launch_build_addressing(const int32_t* token_slot, int T, int slots,
                                   int32_t* token_order, int32_t* slot_indptr, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
  const size_t need = addressing_workspace_bytes(T, slots);
  if (ws && need > 0 && ws_bytes >= need) {
    const int nb = (T + kBlockTok - 1) / kBlockTok;
    const int S1 = slots + 1;
    const size_t lds1 = (size_t)16 * S1 * sizeof(int);
    const size_t lds2 = ((size_t)17 * S1 + 20) * sizeof(int);
    if (lds2 > 65536) {
      hipError_t e = hipFuncSetAttribute((const void*)k_addr_block_hist,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1);
      if (e == hipSuccess)
        e = hipFuncSetAttribute((const void*)k_addr_block_scatter,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds2);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_addr_block_hist, dim3(nb), dim3(kBlockTok), lds1, stream, token_slot, T,
                       slots, (int32_t*)ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_addr_block_scatter, dim3(nb), dim3(kBlockTok), lds2, stream, token_slot,
                       T, slots, (const int32_t*)ws, nb, token_order, slot_indptr);
    return hipGetLastError();
  }
  if (slots + 1 <= kWave && T <= 16 * kWave) {
    const int groups = (T + kWave - 1) / kWave;
#define W(GV)                                                                                    \
  hipLaunchKernelGGL(k_build_addressing_wave<GV>, dim3(1), dim3(kWave), 0, stream, token_slot, T, \
                     slots, token_order, slot_indptr)
    if (groups <= 1)
      W(1);
    else if (groups <= 2)
      W(2);
    else if (groups <= 4)
      W(4);
    else if (groups <= 8)
      W(8);
    else
      W(16);
#undef W
    return hipGetLastError();
  }
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

size_t expert_addressing_workspace_bytes(int64_t rows, int E, int slots) {
  const size_t keys = ((size_t)rows * sizeof(int32_t) + 255) & ~(size_t)255;
  return keys + addressing_workspace_bytes(rows, E * slots);
}

hipError_t launch_build_addressing_experts(const int32_t* row_slot, const int32_t* offs, int E,
                                           int rows, int slots, int32_t* token_order,
                                           int32_t* slot_indptr, void* ws, size_t ws_bytes,
                                           hipStream_t stream) {
  const size_t kb = ((size_t)rows * sizeof(int32_t) + 255) & ~(size_t)255;
  int32_t* keys = (int32_t*)ws;
  if (rows > 0) {
    hipLaunchKernelGGL(k_expert_keys, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream,
                       row_slot, offs, E, rows, slots, keys);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_build_addressing(keys, rows, E * slots, token_order, slot_indptr,
                                 (char*)ws + kb, ws_bytes - kb, stream);
}

}  // namespace lora
