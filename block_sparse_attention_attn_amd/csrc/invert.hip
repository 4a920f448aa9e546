// invert.hip -- q2k -> k2q index inversion on gfx950 (row a1 of the path).
//
// Definition (FastVideo backward test page, the invert_indices_torch helper; launch header, the
// k2q fields of the argument struct): k2q_num[b, h, kb] counts the q blocks whose first
// q2k_num[b, h, qb] entries contain kb; k2q_idx[b, h, kb, :] lists those q blocks in ascending
// order and holds 0 past the count. The page's Triton kernel compacts with atomics, so its row
// order varies from call to call; this one is bit-exact and deterministic. Both steps go through
// a per-(b, h) bitmap [nkv][ceil(nq / 32)] of 32-bit words, bit qb % 32 of word (kb, qb / 32)
// saying that q block qb selects kv block kb:
//   1. one workgroup per (b, h, group of 32 q blocks) sets the bits of its q blocks' counted q2k
//      entries in an LDS column of nkv words (LDS atomicOr: order-free, a duplicate entry sets the
//      same bit, entries with kb outside [0, nkv) are skipped) and then stores the whole column,
//      so every word of the bitmap is written once with no global atomics and no clearing pass.
//      Beyond INVERT_LDS_MAX_KV kv blocks the column does not fit LDS; the bitmap is then zeroed
//      and set with global atomicOr instead;
//   2. one wave per k2q row turns the row's bits into ascending q ids with a popcount prefix sum
//      and writes 0 to the rest of the row.
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

constexpr int INVERT_LDS_MAX_KV = 16384;  // one LDS column of nkv words: 64 KiB

// grid = BH * ceil(nq / 32) workgroups of 256 threads, nkv * 4 bytes of dynamic LDS.
__global__ void __launch_bounds__(256) invert_columns_kernel(const int32_t* __restrict__ q2k_idx,
                                                             const int32_t* __restrict__ q2k_num,
                                                             int nq, int topk, int nkv,
                                                             uint32_t* __restrict__ bitmap) {
  extern __shared__ uint32_t column[];
  __shared__ int counts[32];
  const int W = (nq + 31) / 32;
  const int bh = blockIdx.x / W;
  const int qg = blockIdx.x - bh * W;
  const int tid = threadIdx.x;
  const int q0 = 32 * qg;
  const int nrow = nq - q0 < 32 ? nq - q0 : 32;
  const size_t row0 = (size_t)bh * nq + q0;
  for (int i = tid; i < nkv; i += 256) column[i] = 0u;
  if (tid < nrow) {
    const int c = q2k_num[row0 + tid];
    counts[tid] = c > topk ? topk : c;
  }
  __syncthreads();
  // the group's q2k rows are contiguous: entry e is row e / topk, position e % topk
  const int32_t* src = q2k_idx + row0 * topk;
  auto set = [&](int r, int t, int kb) {
    if (t < counts[r] && kb >= 0 && kb < nkv) atomicOr(&column[kb], 1u << r);
  };
  const long long total = (long long)nrow * topk;
  if (total < (1LL << 30)) {
    // eight loads in flight per thread before their bits are set
    constexpr int U = 8;
    const int tot = (int)total;
    for (int e0 = 0; e0 < tot; e0 += 256 * U) {
      int kb[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + 256 * u + tid;
        kb[u] = e < tot ? src[e] : -1;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + 256 * u + tid;
        if (e < tot) {
          const int r = e / topk;
          set(r, e - r * topk, kb[u]);
        }
      }
    }
  } else {
    for (int r = 0; r < nrow; ++r)
      for (long long t = tid; t < topk; t += 256) set(r, (int)t, src[(size_t)r * topk + t]);
  }
  __syncthreads();
  uint32_t* out = bitmap + (size_t)bh * nkv * W + qg;
  for (int kb = threadIdx.x; kb < nkv; kb += 256) out[(size_t)kb * W] = column[kb];
}

// grid = ceil(BH * nkv / 4) workgroups of 256 threads: one wave per k2q row.
__global__ void __launch_bounds__(256) invert_compact_kernel(const uint32_t* __restrict__ bitmap,
                                                             int nq, size_t nrows,
                                                             int32_t* __restrict__ k2q_idx,
                                                             int32_t* __restrict__ k2q_num) {
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= nrows) return;
  const int lane = threadIdx.x & 63;
  const int W = (nq + 31) / 32;
  const uint32_t* bits = bitmap + row * W;
  int32_t* out = k2q_idx + row * (size_t)nq;
  int base = 0;
  for (int w0 = 0; w0 < W; w0 += 64) {
    const int wi = w0 + lane;
    const uint32_t word = wi < W ? bits[wi] : 0u;
    const int cnt = __popc(word);
    int incl = cnt;  // inclusive scan over the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d, 64);
      if (lane >= d) incl += y;
    }
    int pos = base + incl - cnt;
    uint32_t x = word;
    while (x) {
      const int b = __ffs(x) - 1;
      out[pos++] = wi * 32 + b;
      x &= x - 1;
    }
    base += __shfl(incl, 63, 64);
  }
  for (int i = base + lane; i < nq; i += 64) out[i] = 0;
  if (lane == 0) k2q_num[row] = base;
}

void launch_invert(const int32_t* q2k_idx, const int32_t* q2k_num, int BH, int nq, int topk,
                   int nkv, int32_t* k2q_idx, int32_t* k2q_num, uint32_t* bitmap,
                   hipStream_t stream) {
  const int W = (nq + 31) / 32;
  if (nkv <= INVERT_LDS_MAX_KV) {
    hipLaunchKernelGGL(invert_columns_kernel, dim3((unsigned)((size_t)BH * W)), dim3(256),
                       (size_t)nkv * sizeof(uint32_t), stream, q2k_idx, q2k_num, nq, topk, nkv,
                       bitmap);
  } else {
    const size_t words = invert_bitmap_bytes(BH, nq, nkv) / sizeof(uint32_t);
    size_t blocks = (words + 255) / 256;
    blocks = blocks > 16384 ? 16384 : (blocks == 0 ? 1 : blocks);
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, bitmap,
                       words);
    const size_t total = (size_t)BH * nq * topk;
    size_t sb = (total + 255) / 256;
    sb = sb > 16384 ? 16384 : sb;
    hipLaunchKernelGGL(invert_scatter_kernel, dim3((unsigned)sb), dim3(256), 0, stream, q2k_idx,
                       q2k_num, nq, topk, nkv, total, bitmap);
  }
  const size_t rows = (size_t)BH * nkv;
  hipLaunchKernelGGL(invert_compact_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                     bitmap, nq, rows, k2q_idx, k2q_num);
}

}  // namespace vsa
