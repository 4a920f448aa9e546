// bwd_aux.hip -- the streaming kernels around the backward's main kernel (gfx950):
//   preprocess  Delta = rowsum(bf16(o) * dO) in fp32, zero the fp32 dQ accumulator, and write the
//               exact-zero dK/dV rows of kv blocks that no q block selects (FastVideo sm_100a
//               backward commit message, the preprocess sentence; launch header, the delta and
//               dqaccum fields of the argument struct);
//   order       the per-(b, h) length-binned permutation of kv work items that the launch header
//               computes on device from 1024 kv blocks on (its order-kernel launch and the
//               ORDER_MIN_KV_BLOCKS comment);
//   postprocess dq = bf16(sm_scale * dQ accumulator) (commit message: dQ postprocess + sm_scale).
// All three are HBM-streaming; they use 16-byte accesses with consecutive lanes on consecutive
// 16-byte chunks of a row.
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
    if (c == 0) p.delta[row] = acc;
    f32x4* dq = (f32x4*)(p.dqaccum + row * HEAD_DIM + c * 8);
    dq[0] = f32x4{};
    dq[1] = f32x4{};
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
__global__ void __launch_bounds__(1024) bwd_order_kernel(const int32_t* __restrict__ k2q_num, int nb,
                                                         int bin_width, int32_t* __restrict__ order) {
  __shared__ uint32_t keys[ORDER_MAX_KV_BLOCKS];
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  int P = 1;
  while (P < nb) P <<= 1;
  for (int i = tid; i < P; i += 1024) {
    uint32_t key = 0xFFFFFFFFu;
    if (i < nb) {
      int num = k2q_num[(size_t)bh * nb + i];
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

void launch_bwd_order(const int32_t* k2q_num, int BH, int nb, int bin_width, int32_t* order,
                      hipStream_t stream) {
  hipLaunchKernelGGL(bwd_order_kernel, dim3(BH), dim3(1024), 0, stream, k2q_num, nb, bin_width,
                     order);
}

// 8 fp32 accumulator values -> 8 bf16 per thread, grid-stride.
__global__ void __launch_bounds__(256) bwd_post_kernel(const float* __restrict__ acc,
                                                       bf16* __restrict__ dq, size_t n8,
                                                       float sm_scale) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (size_t)gridDim.x * 256) {
    const f32x4 a = ((const f32x4*)acc)[2 * i];
    const f32x4 b = ((const f32x4*)acc)[2 * i + 1];
    ((bf16x8*)dq)[i] = pack8(a[0] * sm_scale, a[1] * sm_scale, a[2] * sm_scale, a[3] * sm_scale,
                             b[0] * sm_scale, b[1] * sm_scale, b[2] * sm_scale, b[3] * sm_scale);
  }
}

void launch_bwd_post(const float* dqaccum, bf16* dq, size_t n_elems, float sm_scale,
                     hipStream_t stream) {
  const size_t n8 = n_elems / 8;
  size_t blocks = (n8 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) return;
  hipLaunchKernelGGL(bwd_post_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dqaccum, dq, n8,
                     sm_scale);
}

}  // namespace vsa
