// bwd_aux.hip -- the streaming kernels around the backward's main kernel (gfx950):
//   preprocess  Delta = rowsum(bf16(o) * dO) in fp32, and the exact-zero dK/dV rows of kv blocks
//               that no q block selects (FastVideo sm_100a backward commit message, the
//               preprocess sentence; launch header, the delta field of the argument struct).
//               Delta is stored in a 512-byte record per q block: -lse/scale_log2 of its 64
//               rows, then -Delta of its 64 rows, the initial accumulator values of the
//               kv-major kernel's S and dP MFMAs;
//   order       the per-(b, h) length-binned permutation of work items that the launch header
//               computes on device from 1024 kv blocks on (its order-kernel launch and the
//               ORDER_MIN_KV_BLOCKS comment); used for the kv-major and the q-major kernel.
// The preprocess streams with 16-byte accesses, consecutive lanes on consecutive 16-byte chunks
// of a row. (The pages' dQ postprocess -- scale by sm_scale, round to bf16 -- is fused into the
// q-major dQ kernel's epilogue here.)
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace vsa {

// grid (nb, BH), 256 threads; each pass covers 16 rows x 16 chunks of 8 elements.
__global__ void __launch_bounds__(256) bwd_pre_kernel(BwdPreParams p) {
  const int blk = blockIdx.x;
  const int bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int rr = tid >> 4;  // row inside the pass
  const int c = tid & 15;   // 16-byte chunk of the row (8 bf16 / 8 fp32 halves)
  const size_t row0 = (size_t)bh * p.S + (size_t)blk * BLOCK;
  const bool empty = p.k2q_num[(size_t)bh * p.nb + blk] == 0;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const size_t row = row0 + pass * 16 + rr;
    const bf16x8 o = *(const bf16x8*)(p.o + row * HEAD_DIM + c * 8);
    const bf16x8 d = *(const bf16x8*)(p.dout + row * HEAD_DIM + c * 8);
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)o[e], (float)d[e], acc);
    // fixed-order reduction over the 16 lanes of the row
    acc += __shfl_xor(acc, 8, 64);
    acc += __shfl_xor(acc, 4, 64);
    acc += __shfl_xor(acc, 2, 64);
    acc += __shfl_xor(acc, 1, 64);
    if (c == 0) {
      float* rec = p.lse_delta + ((size_t)bh * p.nb + blk) * LD_RECORD_FLOATS;
      const int r = pass * 16 + rr;
      rec[r] = -(p.lse[row] / p.scale_log2);  // IEEE division: a fixed, testable rounding
      rec[BLOCK + r] = -acc;
    }
    if (empty) {
      *(bf16x8*)(p.dk + row * HEAD_DIM + c * 8) = bf16x8{};
      *(bf16x8*)(p.dv + row * HEAD_DIM + c * 8) = bf16x8{};
    }
  }
}

void launch_bwd_pre(const BwdPreParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(bwd_pre_kernel, dim3(p.nb, p.BH), dim3(256), 0, stream, p);
}

// One workgroup per (b, h): bitonic sort of 32-bit keys (inverted bin << 14 | kv) in LDS, so the
// result is larger bins first and ascending kv inside a bin -- a deterministic permutation.
// bin = k2q_num / bin_width, clamped to 18 bits.
__global__ void __launch_bounds__(1024) bwd_order_kernel(const int32_t* __restrict__ num_in, int nb,
                                                         int bin_width, int32_t* __restrict__ order) {
  __shared__ uint32_t keys[ORDER_MAX_KV_BLOCKS];
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  int P = 1;
  while (P < nb) P <<= 1;
  for (int i = tid; i < P; i += 1024) {
    uint32_t key = 0xFFFFFFFFu;
    if (i < nb) {
      int num = num_in[(size_t)bh * nb + i];
      num = num < 0 ? 0 : num;
      uint32_t bin = (uint32_t)(num / bin_width);
      bin = bin > 0x3FFFFu ? 0x3FFFFu : bin;
      key = ((0x3FFFFu - bin) << 14) | (uint32_t)i;
    }
    keys[i] = key;
  }
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = tid; i < P; i += 1024) {
        const int ixj = i ^ jj;
        if (ixj > i) {
          const uint32_t a = keys[i], b = keys[ixj];
          const bool up = (i & k) == 0;
          if ((a > b) == up) {
            keys[i] = b;
            keys[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int r = tid; r < nb; r += 1024)
    order[(size_t)bh * nb + r] = bh * nb + (int)(keys[r] & 0x3FFFu);
}

void launch_bwd_order(const int32_t* num, int BH, int nb, int bin_width, int32_t* order,
                      hipStream_t stream) {
  hipLaunchKernelGGL(bwd_order_kernel, dim3(BH), dim3(1024), 0, stream, num, nb, bin_width, order);
}

}  // namespace vsa
