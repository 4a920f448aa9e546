// invert.hip -- q2k -> k2q index inversion on gfx950 (row a1 of the path).
//
// Definition (FastVideo backward test page, the invert_indices_torch helper; launch header, the
// k2q fields of the argument struct): k2q_num[b, h, kb] counts the q blocks whose first
// q2k_num[b, h, qb] entries contain kb; k2q_idx[b, h, kb, :] lists those q blocks in ascending
// order and holds 0 past the count. The page's Triton kernel compacts with atomics, so its row
// order varies from call to call; this one is bit-exact and deterministic:
//   1. zero a per-(b, h) bitmap [nkv][ceil(nq / 32)] of 32-bit words;
//   2. every counted q2k entry sets bit (kb, qb) with atomicOr (order-free; a duplicate entry
//      sets the same bit, so it counts once; entries with kb outside [0, nkv) are skipped);
//   3. one workgroup per k2q row turns the row's bits into ascending q ids with a popcount
//      prefix sum, and writes 0 to the rest of the row.
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace vsa {

size_t invert_bitmap_bytes(int BH, int nq, int nkv) {
  return (size_t)BH * nkv * (size_t)((nq + 31) / 32) * sizeof(uint32_t);
}

__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

__global__ void __launch_bounds__(256) invert_scatter_kernel(const int32_t* __restrict__ q2k_idx,
                                                             const int32_t* __restrict__ q2k_num,
                                                             int nq, int topk, int nkv, size_t total,
                                                             uint32_t* __restrict__ bitmap) {
  const int W = (nq + 31) / 32;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    const size_t row = e / topk;  // (bh, qb)
    const int t = (int)(e - row * topk);
    int num = q2k_num[row];
    num = num > topk ? topk : num;
    if (t >= num) continue;
    const int kb = q2k_idx[e];
    if (kb < 0 || kb >= nkv) continue;
    const int bh = (int)(row / nq);
    const int qb = (int)(row - (size_t)bh * nq);
    atomicOr(bitmap + ((size_t)bh * nkv + kb) * W + (qb >> 5), 1u << (qb & 31));
  }
}

// grid = BH * nkv rows, 256 threads.
__global__ void __launch_bounds__(256) invert_compact_kernel(const uint32_t* __restrict__ bitmap,
                                                             int nq, int32_t* __restrict__ k2q_idx,
                                                             int32_t* __restrict__ k2q_num) {
  __shared__ int wave_tot[4];
  const size_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int W = (nq + 31) / 32;
  const uint32_t* bits = bitmap + row * W;
  int32_t* out = k2q_idx + row * (size_t)nq;
  int base = 0;
  for (int w0 = 0; w0 < W; w0 += 256) {
    const int wi = w0 + tid;
    const uint32_t word = wi < W ? bits[wi] : 0u;
    const int cnt = __popc(word);
    // inclusive scan inside the wave
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d, 64);
      if (lane >= d) incl += y;
    }
    if (lane == 63) wave_tot[w] = incl;
    __syncthreads();
    int before = 0, chunk = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      before += k < w ? wave_tot[k] : 0;
      chunk += wave_tot[k];
    }
    __syncthreads();
    int pos = base + before + incl - cnt;
    uint32_t x = word;
    while (x) {
      const int b = __ffs(x) - 1;
      out[pos++] = wi * 32 + b;
      x &= x - 1;
    }
    base += chunk;
  }
  for (int i = base + tid; i < nq; i += 256) out[i] = 0;
  if (tid == 0) k2q_num[row] = base;
}

void launch_invert(const int32_t* q2k_idx, const int32_t* q2k_num, int BH, int nq, int topk,
                   int nkv, int32_t* k2q_idx, int32_t* k2q_num, uint32_t* bitmap,
                   hipStream_t stream) {
  const size_t words = invert_bitmap_bytes(BH, nq, nkv) / sizeof(uint32_t);
  size_t blocks = (words + 255) / 256;
  blocks = blocks > 16384 ? 16384 : (blocks == 0 ? 1 : blocks);
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, bitmap, words);
  const size_t total = (size_t)BH * nq * topk;
  if (total > 0) {
    size_t sb = (total + 255) / 256;
    sb = sb > 16384 ? 16384 : sb;
    hipLaunchKernelGGL(invert_scatter_kernel, dim3((unsigned)sb), dim3(256), 0, stream, q2k_idx,
                       q2k_num, nq, topk, nkv, total, bitmap);
  }
  hipLaunchKernelGGL(invert_compact_kernel, dim3((unsigned)((size_t)BH * nkv)), dim3(256), 0, stream,
                     bitmap, nq, k2q_idx, k2q_num);
}

}  // namespace vsa
