// Coordinated noise initialization of a new chunk (DualParal write-up,
// section 三, second improvement): the new chunk's noise frames come from a
// shared pool, leaving out the frames the tail chunk's last n_excl latent
// frames used (its temporal neighbour), in a random order.
//
// The draw is given as one 32-bit key per pool frame.  The candidates (pool
// frames not excluded) ranked by (key, pool index) give the new chunk's frames:
// frame f is the candidate of rank f, for f < n_frames.  Two launches:
//   noise_select  one workgroup: each candidate counts the candidates ranked
//                 before it (keys and exclusion flags in LDS); ranks below
//                 n_frames write their pool index.  P^2 comparisons, P <= 4096.
//   noise_gather  copies pool frame idx[f] to out frame f, 16 bytes per lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace chunkattn {

constexpr int kMaxNoisePool = 4096;

__global__ __launch_bounds__(256) void noise_select(const uint32_t* keys, int pool,
                                                    const int* prev_idx, int n_prev, int n_excl,
                                                    int n_frames, int* idx_out) {
  __shared__ uint32_t skey[kMaxNoisePool];
  __shared__ uint8_t excl[kMaxNoisePool];
  for (int p = threadIdx.x; p < pool; p += blockDim.x) {
    skey[p] = keys[p];
    excl[p] = 0;
  }
  __syncthreads();
  // the tail chunk's last n_excl frames (indices outside the pool exclude nothing)
  for (int j = n_prev - n_excl + (int)threadIdx.x; j < n_prev; j += blockDim.x) {
    const int p = prev_idx[j];
    if (p >= 0 && p < pool) excl[p] = 1;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < pool; p += blockDim.x) {
    if (excl[p]) continue;
    const uint32_t kp = skey[p];
    int rank = 0;
    for (int q = 0; q < pool; ++q)
      rank += !excl[q] && (skey[q] < kp || (skey[q] == kp && q < p));
    if (rank < n_frames) idx_out[rank] = p;
  }
}

// grid (ceil(frame_vecs / 256), n_frames): out frame f, 16-byte vector i
__global__ __launch_bounds__(256) void noise_gather(const uint4* pool, int64_t frame_vecs,
                                                    const int* idx, uint4* out) {
  const int f = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= frame_vecs) return;
  const int64_t src = (int64_t)idx[f];
  out[(int64_t)f * frame_vecs + i] = pool[src * frame_vecs + i];
}

}  // namespace chunkattn
