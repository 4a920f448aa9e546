// bwd_dkdv.hip -- dK and dV of the 64-token block-sparse attention backward on gfx950 (the kv-major
// half of the backward's main step).
//
// What it computes (FastVideo sm_100a backward commit message: one work item per (batch, head,
// kv64 block); launch header argument struct: k2q lists, variable_block_sizes, dk carries
// sm_scale and dv does not; the gradient is the textbook softmax-attention gradient of the
// backward test page's reference): for one item (b, h, kv block j) and every q block i in its
// k2q list,
//     S    = Q_i K_j^T                       (recomputed scores, 64 x 64)
//     P    = exp2(S * scale_log2 - lse_i)     (lse in base-2 "M form"; kv rows >= vbs[j] -> 0)
//     dP   = dO_i V_j^T
//     dS   = P * (dP - Delta_i)
//     dV_j += P^T dO_i,   dK_j += dS^T Q_i
// then dk_j = bf16(sm_scale * dK_j), dv_j = bf16(dV_j). Items with an empty list do no work here:
// the preprocess wrote their zero rows. dQ is computed by the q-major kernel (bwd_dq.hip), so
// this kernel issues no atomics and its results are bitwise reproducible.
//
// gfx950 design:
//   * one 256-thread workgroup (4 waves, one per SIMD) per item; wave w owns q rows 32*(w&1)..
//     of every q block and kv rows 32*(w>>1).. of the item, so each 64x64x128 GEMM is eight
//     v_mfma_f32_32x32x16_bf16 per wave;
//   * K_j and V_j fragments (the B operands of S and dP) live in registers for the whole item,
//     with padded kv rows zeroed there;
//   * Q_i, dO_i (and lse_i, Delta_i) stream through XOR-swizzled LDS tiles filled by
//     global_load_lds_dwordx4, double-buffered: the next q block loads while this one computes;
//   * P and dS never leave registers: the D layout of S/dP feeds the A operand of dV/dK directly
//     (the contraction index is permuted to match), the partner operands dO_i^T and Q_i^T come
//     from ds_read_b64_tr_b16 transposed reads;
//   * dV and dK are accumulated per q half and the halves are summed through LDS once per item;
//   * work ids map XCD-first: workgroup ids go round-robin over the 8 XCDs, so XCD x runs a
//     contiguous slice of the (ordered) item list -- one head per XCD when B*H = 8 -- and that
//     head's Q/dO traffic stays in one XCD's L2.
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace vsa {

namespace {

__device__ __forceinline__ void barrier_lds() {
  // Wait for this wave's LDS traffic, then meet the other waves. Vector memory traffic (the next
  // tile's DMA) stays in flight across the barrier.
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct Pipe {
  VSA_LDS char* q;
  VSA_LDS char* d;
  VSA_LDS float* ld;
};

__device__ __forceinline__ void prefetch(const bf16* __restrict__ qh, const bf16* __restrict__ doh,
                                         const float* __restrict__ lseh,
                                         const float* __restrict__ deltah, int qb, Pipe p, int lane,
                                         int w) {
  const size_t off = (size_t)qb * BLOCK * HEAD_DIM;
  tile_load_async<4>(qh + off, p.q, lane, w);
  tile_load_async<4>(doh + off, p.d, lane, w);
  if (w == 0 && lane < 32) {
    const float* src = lane < 16 ? lseh + qb * BLOCK + lane * 4 : deltah + qb * BLOCK + (lane - 16) * 4;
    dma16(src, lds_addr(p.ld));
  }
}

}  // namespace

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_dkdv_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) char q_s0[16384];
  __shared__ __attribute__((aligned(1024))) char q_s1[16384];
  __shared__ __attribute__((aligned(1024))) char do_s0[16384];
  __shared__ __attribute__((aligned(1024))) char do_s1[16384];
  __shared__ __attribute__((aligned(16))) float ld_s0[128];
  __shared__ __attribute__((aligned(16))) float ld_s1[128];

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int wq = w & 1;   // q half of every q block
  const int wk = w >> 1;  // kv half of the item
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int grp = lane >> 4;  // 16-lane group
  const int t16 = lane & 15;  // lane inside the group

  // XCD-first work id: blockIdx.x % 8 is the XCD the dispatcher sends the workgroup to.
  const int wid = (blockIdx.x & 7) * p.items_per_xcd + (blockIdx.x >> 3);
  if (wid >= p.total_items) return;
  const int item = p.kv_order ? ld_const(p.kv_order, wid) : wid;
  if (item < 0 || item >= p.total_items) return;  // a malformed order entry: skip, never fault
  int n = ld_const(p.k2q_num, item);
  n = n > p.k2q_stride ? p.k2q_stride : n;
  if (n <= 0) return;
  const int bh = item / p.nb;
  const int j = item - bh * p.nb;
  const int vb = ld_const(p.vbs, j);
  const size_t head = (size_t)bh * p.S * HEAD_DIM;
  const bf16* __restrict__ qh = p.q + head;
  const bf16* __restrict__ doh = p.dout + head;
  const float* __restrict__ lseh = p.lse + (size_t)bh * p.S;
  const float* __restrict__ deltah = p.delta + (size_t)bh * p.S;
  const int* __restrict__ list = p.k2q_idx + (size_t)item * p.k2q_stride;
  // q block ids outside [0, nb) violate the caller contract; clamp them so no access leaves the
  // tensors (the result is then unspecified, but nothing faults)
  auto qblock = [&](int t) {
    const int qb = ld_const(list, t);
    return qb < 0 ? 0 : (qb >= p.nb ? p.nb - 1 : qb);
  };

  // the two pipeline stages; the loop below is unrolled by two so every LDS access names its
  // buffer statically
  const Pipe pipe0{(VSA_LDS char*)q_s0, (VSA_LDS char*)do_s0, (VSA_LDS float*)ld_s0};
  const Pipe pipe1{(VSA_LDS char*)q_s1, (VSA_LDS char*)do_s1, (VSA_LDS float*)ld_s1};
  prefetch(qh, doh, lseh, deltah, qblock(0), pipe0, lane, w);

  // B operand of S = Q K^T and dP = dO V^T: lane holds kv row 32*wk + l32, d = 16*s + 8*g + 0..7.
  const int kv_l = 32 * wk + l32;
  const bool kv_valid = kv_l < vb;
  bf16x8 kf[8], vf[8];
  {
    const bf16* kj = p.k + head + (size_t)j * BLOCK * HEAD_DIM;
    const bf16* vj = p.v + head + (size_t)j * BLOCK * HEAD_DIM;
    const bf16x8* kr = (const bf16x8*)(kj + (size_t)kv_l * HEAD_DIM);
    const bf16x8* vr = (const bf16x8*)(vj + (size_t)kv_l * HEAD_DIM);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      kf[s] = kr[2 * s + g];
      vf[s] = vr[2 * s + g];
    }
    if (!kv_valid) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        kf[s] = bf16x8{};
        vf[s] = bf16x8{};
      }
    }
  }

  f32x16 dv_acc[4], dk_acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    dv_acc[nt] = f32x16{};
    dk_acc[nt] = f32x16{};
  }

  const float scale_log2 = p.scale_log2;

  auto step = [&](int t, const Pipe cu, const Pipe nx) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this q block's tiles have landed (own DMAs)
    barrier_lds();                               // ... and everyone else's; buffer nx is free
    if (t + 1 < n) prefetch(qh, doh, lseh, deltah, qblock(t + 1), nx, lane, w);
    VSA_LDS char* qt = cu.q;
    VSA_LDS char* dt = cu.d;
    VSA_LDS float* ld = cu.ld;

    // ---- S = Q K^T and dP = dO V^T for q rows 32*wq.. x kv rows 32*wk.. ----
    f32x16 sacc = f32x16{}, pacc = f32x16{};
    const int qrow = 32 * wq + l32;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 qa = *(const VSA_LDS bf16x8*)(qt + tile_byte(qrow, 2 * s + g));
      const bf16x8 da = *(const VSA_LDS bf16x8*)(dt + tile_byte(qrow, 2 * s + g));
      sacc = mfma32(qa, kf[s], sacc);
      pacc = mfma32(da, vf[s], pacc);
    }

    // ---- P and dS in registers; element i is q row 32*wq + 8*(i/4) + 4*g + i%4, kv kv_l ----
    float pv[16], dsv[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int qr = 32 * wq + 8 * c + 4 * g;
      const f32x4 lse4 = *(const VSA_LDS f32x4*)(ld + qr);
      const f32x4 del4 = *(const VSA_LDS f32x4*)(ld + 64 + qr);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * c + e;
        const float pe = __builtin_amdgcn_exp2f(sacc[i] * scale_log2 - lse4[e]);
        pv[i] = kv_valid ? pe : 0.0f;
        dsv[i] = pv[i] * (pacc[i] - del4[e]);
      }
    }

    // ---- dV += P^T dO and dK += dS^T Q over this wave's q half ----
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const bf16x8 pa = pack8(pv[8 * s2 + 0], pv[8 * s2 + 1], pv[8 * s2 + 2], pv[8 * s2 + 3],
                              pv[8 * s2 + 4], pv[8 * s2 + 5], pv[8 * s2 + 6], pv[8 * s2 + 7]);
      const bf16x8 sa = pack8(dsv[8 * s2 + 0], dsv[8 * s2 + 1], dsv[8 * s2 + 2], dsv[8 * s2 + 3],
                              dsv[8 * s2 + 4], dsv[8 * s2 + 5], dsv[8 * s2 + 6], dsv[8 * s2 + 7]);
      const int q0 = 32 * wq + 16 * s2 + 4 * (grp >> 1) + (t16 >> 2);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int col = 32 * nt + 16 * (grp & 1) + 4 * (t16 & 3);
        const bf16x8 db = join(lds_read_tr(dt + tile_elem_byte(q0, col)),
                               lds_read_tr(dt + tile_elem_byte(q0 + 8, col)));
        const bf16x8 qbv = join(lds_read_tr(qt + tile_elem_byte(q0, col)),
                                lds_read_tr(qt + tile_elem_byte(q0 + 8, col)));
        dv_acc[nt] = mfma32(pa, db, dv_acc[nt]);
        dk_acc[nt] = mfma32(sa, qbv, dk_acc[nt]);
      }
    }
  };
  for (int t = 0; t < n; t += 2) {
    step(t, pipe0, pipe1);
    if (t + 1 < n) step(t + 1, pipe1, pipe0);
  }

  // ---- sum the two q halves of dV/dK through LDS, scale, round, store ----
  barrier_lds();  // every wave is past its last LDS read of the q/dO buffers
  // wave wq=1 hands over its dV half, wave wq=0 its dK half (16 KiB each, lane-native order);
  // kv half 0 uses the q buffers, kv half 1 the dO buffers
  VSA_LDS f32x4* dv_x = (VSA_LDS f32x4*)(wk == 0 ? (VSA_LDS char*)q_s0 : (VSA_LDS char*)do_s0);
  VSA_LDS f32x4* dk_x = (VSA_LDS f32x4*)(wk == 0 ? (VSA_LDS char*)q_s1 : (VSA_LDS char*)do_s1);
  VSA_LDS f32x4* mine_out = wq == 1 ? dv_x : dk_x;
  VSA_LDS f32x4* theirs = wq == 1 ? dk_x : dv_x;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x16& src = wq == 1 ? dv_acc[nt] : dk_acc[nt];
      mine_out[(nt * 4 + c) * 64 + lane] = f32x4{src[4 * c], src[4 * c + 1], src[4 * c + 2], src[4 * c + 3]};
    }
  }
  barrier_lds();
  bf16* outp = (wq == 0 ? p.dv : p.dk) + head + (size_t)j * BLOCK * HEAD_DIM;
  const float oscale = wq == 0 ? 1.0f : p.sm_scale;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int d = 32 * nt + l32;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 o = theirs[(nt * 4 + c) * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float mine = wq == 0 ? dv_acc[nt][4 * c + e] : dk_acc[nt][4 * c + e];
        const int kv = 32 * wk + 8 * c + 4 * g + e;
        outp[(size_t)kv * HEAD_DIM + d] = (bf16)((mine + o[e]) * oscale);
      }
    }
  }
}

void launch_bwd_dkdv(const BwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(p.items_per_xcd * 8), dim3(256), 0, stream, p);
}

}  // namespace vsa
