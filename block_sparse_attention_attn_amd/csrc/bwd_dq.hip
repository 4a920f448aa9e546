// bwd_dq.hip -- dQ of the 64-token block-sparse attention backward on gfx950 (the q-major half of
// the backward's main step, with the dQ scale/convert epilogue fused).
//
// What it computes (the gradient of the FastVideo backward test page's masked-dense reference;
// launch header argument struct: dq carries sm_scale, lse is the base-2 "M form"): for one q block
// i of (b, h) and every kv block j in its q2k list,
//     S^T  = K_j Q_i^T,   P^T = exp2(S^T * scale_log2 - lse_i)   (kv rows >= vbs[j] -> 0)
//     dP^T = V_j dO_i^T,  dS^T = P^T * (dP^T - Delta_i)
//     dQ_i += dS K_j
// and dq_i = bf16(sm_scale * dQ_i). A q block with an empty list gets zero rows.
//
// The pages reduce per-pair dQ partials into an fp32 accumulator with bulk asynchronous
// reductions. On MI355X the equivalent, global_atomic_add_f32, sustains about 3.4e11 lane adds/s
// whatever the address pattern (measured), i.e. >= 12.6 ms for the 4.3e9 adds of a 32k-token,
// 25 %-dense head-8 backward; so dQ is instead accumulated in registers here, walking each q
// block's own list and recomputing S and dP (two extra GEMMs per pair, no atomics, no fp32
// accumulator, bitwise-reproducible dq).
//
// gfx950 layout: one 256-thread workgroup per q block; wave w owns q rows 32*(w&1).. and kv rows
// 32*(w>>1).. of every kv block. Q_i and dO_i live in registers as the B operands of S^T = K Q^T
// and dP^T = V dO^T (v_mfma_f32_32x32x16_bf16), so lse and Delta are one scalar per lane. K_j,
// V_j stream through swizzled, double-buffered LDS tiles (global_load_lds_dwordx4). dS^T stays in
// registers as the B operand of dQ^T += K^T dS^T, with K^T from ds_read_b64_tr_b16. The two kv
// halves' partial dQ^T are summed through LDS once per q block.
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace vsa {

namespace {

__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_dq_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) char k_s0[16384];
  __shared__ __attribute__((aligned(1024))) char k_s1[16384];
  __shared__ __attribute__((aligned(1024))) char v_s0[16384];
  __shared__ __attribute__((aligned(1024))) char v_s1[16384];

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int wq = w & 1;   // q half of the q block
  const int wk = w >> 1;  // kv half of every kv block
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int grp = lane >> 4;
  const int t16 = lane & 15;

  const int wid = (blockIdx.x & 7) * p.items_per_xcd + (blockIdx.x >> 3);
  if (wid >= p.total_items) return;
  const int item = p.q_order ? ld_const(p.q_order, wid) : wid;  // (b, h, q block)
  if (item < 0 || item >= p.total_items) return;
  int n = ld_const(p.q2k_num, item);
  n = n < 0 ? 0 : (n > p.q2k_stride ? p.q2k_stride : n);
  const int bh = item / p.nb;
  const int i = item - bh * p.nb;
  const size_t head = (size_t)bh * p.S * HEAD_DIM;
  const int* __restrict__ list = p.q2k_idx + (size_t)item * p.q2k_stride;
  auto kvblock = [&](int t) {
    const int kb = ld_const(list, t);
    return kb < 0 ? 0 : (kb >= p.nb ? p.nb - 1 : kb);
  };

  // B operands: lane holds q row 32*wq + l32, d = 16*s + 8*g + 0..7
  const int qrow = i * BLOCK + 32 * wq + l32;
  bf16x8 qf[8], df[8];
  {
    const bf16x8* qr = (const bf16x8*)(p.q + head + (size_t)qrow * HEAD_DIM);
    const bf16x8* dr = (const bf16x8*)(p.dout + head + (size_t)qrow * HEAD_DIM);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qf[s] = qr[2 * s + g];
      df[s] = dr[2 * s + g];
    }
  }
  const float lse_q = p.lse[(size_t)bh * p.S + qrow];
  const float delta_q = p.delta[(size_t)bh * p.S + qrow];
  const float scale_log2 = p.scale_log2;

  // dQ^T tiles: element e of tile mt is d = 32*mt + 8*(e/4) + 4*g + e%4, q = 32*wq + l32
  f32x16 dq_acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) dq_acc[mt] = f32x16{};

  if (n > 0) {
    const size_t off = (size_t)kvblock(0) * BLOCK * HEAD_DIM;
    tile_load_async<4>(p.k + head + off, (VSA_LDS char*)k_s0, lane, w);
    tile_load_async<4>(p.v + head + off, (VSA_LDS char*)v_s0, lane, w);
  }

  auto step = [&](int t, VSA_LDS char* kt, VSA_LDS char* vt, VSA_LDS char* kn_s,
                  VSA_LDS char* vn_s) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    barrier_lds();
    if (t + 1 < n) {
      const size_t off = (size_t)kvblock(t + 1) * BLOCK * HEAD_DIM;
      tile_load_async<4>(p.k + head + off, kn_s, lane, w);
      tile_load_async<4>(p.v + head + off, vn_s, lane, w);
    }
    const int vb = ld_const(p.vbs, kvblock(t));

    // ---- S^T = K Q^T and dP^T = V dO^T: kv rows 32*wk.., q columns 32*wq.. ----
    f32x16 sacc = f32x16{}, pacc = f32x16{};
    const int kvrow = 32 * wk + l32;
    bf16x8 ka[8], va[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      ka[s] = *(const VSA_LDS bf16x8*)(kt + tile_byte(kvrow, 2 * s + g));
      va[s] = *(const VSA_LDS bf16x8*)(vt + tile_byte(kvrow, 2 * s + g));
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      sacc = mfma32(ka[s], qf[s], sacc);
      pacc = mfma32(va[s], df[s], pacc);
    }

    // ---- dS^T; element e is kv 32*wk + 8*(e/4) + 4*g + e%4. Masked kv rows are selected to 0
    // (never multiplied: a padded V row may hold anything) ----
    float dsv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int kv = 32 * wk + 8 * (e >> 2) + 4 * g + (e & 3);
      const float pe = __builtin_amdgcn_exp2f(sacc[e] * scale_log2 - lse_q);
      const float ds = pe * (pacc[e] - delta_q);
      dsv[e] = kv < vb ? ds : 0.0f;
    }

    // ---- dQ^T += K^T dS^T; k slot jj of step s2 is kv 32*wk + 16*s2 + 8*(jj/4) + 4*g + jj%4 ----
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const bf16x8 b = pack8(dsv[8 * s2 + 0], dsv[8 * s2 + 1], dsv[8 * s2 + 2], dsv[8 * s2 + 3],
                             dsv[8 * s2 + 4], dsv[8 * s2 + 5], dsv[8 * s2 + 6], dsv[8 * s2 + 7]);
      const int kv0 = 32 * wk + 16 * s2 + 4 * (grp >> 1) + (t16 >> 2);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int col = 32 * mt + 16 * (grp & 1) + 4 * (t16 & 3);
        bf16x8 a = join(lds_read_tr(kt + tile_elem_byte(kv0, col)),
                        lds_read_tr(kt + tile_elem_byte(kv0 + 8, col)));
        if (vb < BLOCK) {  // padded K rows may hold anything: zero them (0 * NaN = NaN)
          const int kvb = 32 * wk + 16 * s2 + 4 * g;
#pragma unroll
          for (int jj = 0; jj < 8; ++jj)
            if (kvb + 8 * (jj >> 2) + (jj & 3) >= vb) a[jj] = (bf16)0.0f;
        }
        dq_acc[mt] = mfma32(a, b, dq_acc[mt]);
      }
    }
  };
  for (int t = 0; t < n; t += 2) {
    step(t, (VSA_LDS char*)k_s0, (VSA_LDS char*)v_s0, (VSA_LDS char*)k_s1, (VSA_LDS char*)v_s1);
    if (t + 1 < n)
      step(t + 1, (VSA_LDS char*)k_s1, (VSA_LDS char*)v_s1, (VSA_LDS char*)k_s0, (VSA_LDS char*)v_s0);
  }

  // ---- sum the two kv halves: wave wk=0 finishes d tiles 0,1, wave wk=1 tiles 2,3 ----
  barrier_lds();  // all LDS reads of the K/V tiles are done
  VSA_LDS f32x4* xch = (VSA_LDS f32x4*)(wq == 0 ? (VSA_LDS char*)k_s0 : (VSA_LDS char*)k_s1);
  // region r holds the tiles that wave (wq, r) finishes, written by its partner (wq, 1 - r)
  VSA_LDS f32x4* give = xch + (wk == 0 ? 512 : 0);
  VSA_LDS f32x4* take = xch + (wk == 0 ? 0 : 512);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int mt = (wk == 0 ? 2 : 0) + u;  // the partner's tiles
#pragma unroll
    for (int c = 0; c < 4; ++c)
      give[(u * 4 + c) * 64 + lane] =
          f32x4{dq_acc[mt][4 * c], dq_acc[mt][4 * c + 1], dq_acc[mt][4 * c + 2], dq_acc[mt][4 * c + 3]};
  }
  barrier_lds();
  bf16* dqrow = p.dq + head + (size_t)qrow * HEAD_DIM;
  const float sc = p.sm_scale;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int mt = (wk == 0 ? 0 : 2) + u;  // my tiles
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 o = take[(u * 4 + c) * 64 + lane];
      union {
        bf16 b[4];
        s16x4 s;
      } r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r.b[e] = (bf16)((dq_acc[mt][4 * c + e] + o[e]) * sc);
      *(s16x4*)(dqrow + 32 * mt + 8 * c + 4 * g) = r.s;
    }
  }
}

void launch_bwd_dq(const BwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(bwd_dq_kernel, dim3(p.items_per_xcd * 8), dim3(256), 0, stream, p);
}

}  // namespace vsa
