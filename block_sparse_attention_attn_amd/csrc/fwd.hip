// fwd.hip -- block-sparse attention forward on gfx950 (row a2: produces o and lse for the
// backward).
//
// What it computes (FastVideo pages: the sm_100a forward module docstring -- it returns (out,
// lse) with lse = max(qk * qk_scale) + log2(l), [B, H, S] fp32, the "M form"; the backward test
// page's reference -- keys of the selected kv blocks at or past variable_block_sizes are masked):
// for every (b, h, q block i), over the kv blocks j in its q2k list,
//     x = (q k^T) * sm_scale * log2(e)   for kv rows < vbs[j], -inf otherwise
//     o = sum_j softmax_2(x) v,  lse = max(x) + log2(sum 2^(x - max))
// with a base-2 online softmax (v_exp_f32 is 2^x natively). A row with no valid key gets o = 0
// and lse = -inf.
//
// gfx950 layout: one 256-thread workgroup per (b, h, q block); wave w owns q rows 16*w..16*w+15
// and keeps them in registers as the B operand of S^T = K Q^T (v_mfma_f32_16x16x32_bf16). K_j and
// V_j tiles stream through swizzled LDS (global_load_lds_dwordx4, double-buffered). The column
// statistics of S^T are lane-local plus a 4-group exchange; P^T (bf16) feeds O^T += V^T P^T
// directly as the B operand, with V^T from ds_read_b64_tr_b16 transposed reads.
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace vsa {

__global__ void __launch_bounds__(256) fwd_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(1024))) char k_s0[16384];
  __shared__ __attribute__((aligned(1024))) char k_s1[16384];
  __shared__ __attribute__((aligned(1024))) char v_s0[16384];
  __shared__ __attribute__((aligned(1024))) char v_s1[16384];

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int g = lane >> 4;    // 16-lane group = k group of the 16x16x32 layout
  const int l16 = lane & 15;

  const int item = blockIdx.x;  // (bh, q block)
  const int bh = item / p.nb;
  const int qb = item - bh * p.nb;
  int n = ld_const(p.q2k_num, item);
  n = n < 0 ? 0 : (n > p.q2k_stride ? p.q2k_stride : n);
  const int32_t* list = p.q2k_idx + (size_t)item * p.q2k_stride;
  const size_t head = (size_t)bh * p.S * HEAD_DIM;


  // Q^T fragment: lane holds q row 16*w + l16, d = 32*s + 8*g + 0..7.
  const int qrow = qb * BLOCK + 16 * w + l16;
  bf16x8 qf[4];
  {
    const bf16x8* qr = (const bf16x8*)(p.q + head + (size_t)qrow * HEAD_DIM);
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = qr[4 * s + g];
  }

  f32x4 oacc[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) oacc[mt] = f32x4{};
  float m_run = -__builtin_inff();
  float l_run = 0.0f;
  const float scale_log2 = p.scale_log2;

  // skip out-of-range kv ids (a caller contract violation) instead of reading out of bounds
  auto kv_of = [&](int t) {
    const int kb = ld_const(list, t);
    return (kb >= 0 && kb < p.nb) ? kb : -1;
  };

  if (n > 0) {
    const int kb0 = kv_of(0);
    if (kb0 >= 0) {
      tile_load_async<4>(p.k + head + (size_t)kb0 * BLOCK * HEAD_DIM, (VSA_LDS char*)k_s0, lane, w);
      tile_load_async<4>(p.v + head + (size_t)kb0 * BLOCK * HEAD_DIM, (VSA_LDS char*)v_s0, lane, w);
    }
  }
  auto step = [&](int t, VSA_LDS char* kt, VSA_LDS char* vt, VSA_LDS char* kn_s,
                  VSA_LDS char* vn_s) __attribute__((always_inline)) {
    const int kb = kv_of(t);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this block's K/V tiles have landed
    __syncthreads();
    if (t + 1 < n) {
      const int kn = kv_of(t + 1);
      if (kn >= 0) {
        tile_load_async<4>(p.k + head + (size_t)kn * BLOCK * HEAD_DIM, kn_s, lane, w);
        tile_load_async<4>(p.v + head + (size_t)kn * BLOCK * HEAD_DIM, vn_s, lane, w);
      }
    }
    if (kb < 0) return;
    const int vb = ld_const(p.vbs, kb);

    // S^T tiles: element i of tile mt is kv 16*mt + 4*g + i, q 16*w + l16
    f32x4 sacc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      sacc[mt] = f32x4{};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 ka = *(const VSA_LDS bf16x8*)(kt + tile_byte(16 * mt + l16, 4 * s + g));
        sacc[mt] = mfma16(ka, qf[s], sacc[mt]);
      }
    }
    float x[16];
    float mx = -__builtin_inff();
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kv = 16 * mt + 4 * g + i;
        const float xi = kv < vb ? sacc[mt][i] * scale_log2 : -__builtin_inff();
        x[4 * mt + i] = xi;
        mx = fmaxf(mx, xi);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -__builtin_inff() ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float ps[16];
    float rs = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ps[i] = __builtin_amdgcn_exp2f(x[i] - m_use);
      rs += ps[i];
    }
    rs += __shfl_xor(rs, 16, 64);
    rs += __shfl_xor(rs, 32, 64);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      oacc[mt][0] *= alpha;
      oacc[mt][1] *= alpha;
      oacc[mt][2] *= alpha;
      oacc[mt][3] *= alpha;
    }
    // O^T[d][q] += V^T[d][kv] P^T[kv][q]; k slot jj of step s2 is kv 32*s2 + 16*(jj/4) + 4*g + jj%4
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const bf16x8 pb = pack8(ps[8 * s2 + 0], ps[8 * s2 + 1], ps[8 * s2 + 2], ps[8 * s2 + 3],
                              ps[8 * s2 + 4], ps[8 * s2 + 5], ps[8 * s2 + 6], ps[8 * s2 + 7]);
      const int kv0 = 32 * s2 + 4 * g + (l16 >> 2);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const int col = 16 * mt + 4 * (l16 & 3);
        const bf16x8 va = join(lds_read_tr(vt + tile_elem_byte(kv0, col)),
                               lds_read_tr(vt + tile_elem_byte(kv0 + 16, col)));
        oacc[mt] = mfma16(va, pb, oacc[mt]);
      }
    }
  };
  for (int t = 0; t < n; t += 2) {
    step(t, (VSA_LDS char*)k_s0, (VSA_LDS char*)v_s0, (VSA_LDS char*)k_s1, (VSA_LDS char*)v_s1);
    if (t + 1 < n)
      step(t + 1, (VSA_LDS char*)k_s1, (VSA_LDS char*)v_s1, (VSA_LDS char*)k_s0, (VSA_LDS char*)v_s0);
  }

  // o row q = 16*w + l16; tile mt holds d = 16*mt + 4*g + 0..3
  const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  bf16* orow = p.o + head + (size_t)qrow * HEAD_DIM;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    union {
      bf16 b[4];
      s16x4 s;
    } u;
#pragma unroll
    for (int i = 0; i < 4; ++i) u.b[i] = (bf16)(oacc[mt][i] * inv_l);
    *(s16x4*)(orow + 16 * mt + 4 * g) = u.s;
  }
  if (g == 0) {
    const float lse = l_run > 0.0f ? m_run + __builtin_log2f(l_run) : -__builtin_inff();
    p.lse[(size_t)bh * p.S + qrow] = lse;
  }
}

void launch_fwd(const FwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(fwd_kernel, dim3((unsigned)(p.BH * p.nb)), dim3(256), 0, stream, p);
}

}  // namespace vsa
