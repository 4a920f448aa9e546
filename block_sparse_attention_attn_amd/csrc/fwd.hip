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
// and lse = -inf; kv ids outside [0, nb) in a list contribute nothing.
//
// gfx950 design: one 256-thread workgroup per (b, h, q block), two per CU. The four waves form a
// 2 x 2 grid, q half x kv half: wave (wq, wk) takes q rows 32wq .. 32wq+31 and, of every kv
// block, kv rows 32wk .. 32wk+31. Each wave runs its own online softmax over its kv halves (its
// own running max, sum and O^T), and the two kv halves of a q half are merged once at the end
// (max of the two maxima, each side rescaled to it). So no statistic crosses waves inside the
// loop, and each wave reads only its half of every K and V tile from LDS.
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = K rows from the swizzled LDS tile
//     (ds_read_b128), B = Q^T fragments held in registers for the whole item.
//   * A q column's 32 scores sit in one lane pair (l, l ^ 32): the max and the sum are lane-local
//     plus one v_permlane32_swap.
//   * The running max is only raised when a block's max exceeds it by more than 8 (in log2
//     units): the exponentials then stay below 2^8, O^T and the sum are rescaled rarely, and the
//     final o = O / l and lse = max + log2(l) are unchanged in exact arithmetic.
//   * P^T is the B operand of O^T += V^T P^T straight from the D layout of S^T (the kv
//     contraction index is permuted to match); V^T comes from ds_read_b64_tr_b16. That product
//     runs in fp16 (v_mfma_f32_32x32x16_f16, the bf16 rate): P < 2^8 fits, and fp16's 11-bit
//     significand rounds P 8x finer than bf16 would. V^T comes from an fp16 copy of V made by a
//     pre-pass, each head scaled by a power of two 2^-e into [2^14, 2^15) at its largest |v|, so
//     the copy is exact (bf16's 8 bits fit) for every |v| >= 2^-28 max; the epilogue multiplies
//     o by 2^e exactly.
//   * K and V tiles arrive by global_load_lds_dwordx4 into two-stage LDS rings, K two blocks and
//     V one block ahead: the S^T MFMAs of block t+1 run under the softmax of block t.
//   * The loop is unrolled by two so the ring stages are constants: each lane's LDS operand
//     addresses are computed once, and the stage rides as an immediate offset. Scores stay
//     unscaled: the block max is taken on raw scores and each exponent is one fma.
//   * Long lists run in kv-range chunks, one launch each, each wave carrying its running O^T,
//     max and sum to the next launch exactly: the workgroups on an XCD then share one window of
//     K/V tiles at a time, and the results are those of one launch, bit for bit. Before each
//     chunk the items are ordered by the length of their list's part in it (length bins), so the
//     items that run together on an XCD walk parts of equal length.
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace vsa {

namespace {

constexpr int TILE = 16384;         // one [64][128] bf16 tile
constexpr float RESCALE_GAP = 8.f;  // raise the running max only when exceeded by this much

__device__ __forceinline__ bf16x8 neg8(bf16x8 v) {  // exact: flips the eight sign bits
  union {
    bf16x8 b;
    uint32_t u[4];
  } r;
  r.b = v;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.u[i] ^= 0x80008000u;
  return r.b;
}

}  // namespace

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_kernel(FwdParams p) {
  // K stage s at s * TILE, V stage s at (2 + s) * TILE (s = 0, 1)
  __shared__ __attribute__((aligned(1024))) char kv_s[4 * TILE];

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int wq = w & 1;   // q half
  const int wk = w >> 1;  // kv half
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int grp = lane >> 4;
  const int t16 = lane & 15;

  int item = (blockIdx.x & 7) * p.items_per_xcd + (blockIdx.x >> 3);  // (bh, q block)
  if (item >= p.BH * p.nb) return;
  if (p.order) {  // the launch's work order (kv-range chunks: items binned per chunk)
    item = ld_const(p.order, item);
    if (item < 0 || item >= p.BH * p.nb) return;  // a malformed entry: skip, never fault
  }
  const int bh = item / p.nb;
  const int qb = item - bh * p.nb;
  int n = ld_const(p.q2k_num, item);
  n = n < 0 ? 0 : (n > p.q2k_stride ? p.q2k_stride : n);
  // kv-range chunk: this launch walks list positions [start, start + n), resuming (unless first)
  // from the state the chunk before left, and finishing (if last) or saving it
  int start = 0;
  bool first = true, last = true;
  if (p.nchunks > 0) {
    const int32_t* cb = p.chunk_bounds + (size_t)item * (p.nchunks + 1) + p.chunk;
    int b0 = ld_const(cb, 0), b1 = ld_const(cb, 1);
    b0 = b0 < 0 ? 0 : (b0 > n ? n : b0);
    b1 = b1 < b0 ? b0 : (b1 > n ? n : b1);
    start = b0;
    n = b1 - b0;
    first = p.chunk == 0;
    last = p.chunk == p.nchunks - 1;
    if (n == 0 && !first && !last) return;  // the state passes through unchanged
  }
  const int32_t* list = p.q2k_idx + (size_t)item * p.q2k_stride + start;
  const size_t head = (size_t)bh * p.S * HEAD_DIM;
  const int qrow = qb * BLOCK + 32 * wq + l32;  // this lane's q row (a column of S^T)

  // B operand of S^T = K Q^T: lane holds Q[qrow][16s + 8g + 0..7], s = 0..7
  bf16x8 qf[8];
  {
    const bf16x8* qr = (const bf16x8*)(p.q + head + (size_t)qrow * HEAD_DIM);
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = qr[2 * s + g];
  }
  // The softmax below wants a positive scale. A negative one is moved into Q (negating a bf16 is
  // exact, and so is the negated MFMA sum, so every score s * scale keeps its value); a zero one
  // becomes the least normal float, which changes every finite score by at most 2^-126 |s|.
  float scale_log2 = p.scale_log2;
  if (scale_log2 < 0.f) {
    scale_log2 = -scale_log2;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = neg8(qf[s]);
  }
  scale_log2 = fmaxf(scale_log2, 1.17549435e-38f);

  // list entry t (clamped to the list; an out-of-range kv id is read as block 0, masked entirely)
  auto kv_raw = [&](int t) { return ld_const(list, t < n ? t : n - 1); };
  auto kv_ok = [&](int kb) { return kb >= 0 && kb < p.nb; };
  auto vb_of = [&](int kb) { return kv_ok(kb) ? ld_const(p.vbs, kb) : 0; };
  uint32_t toff[4];
  tile_offsets_wave(toff, lane, w);
  const uint32_t lds0 = lds_addr((VSA_LDS char*)kv_s) + 4096 * w;
  auto tile_of = [&](int kb) { return (size_t)(kv_ok(kb) ? kb : 0) * BLOCK * HEAD_DIM; };
  auto issue_k = [&](int kb, int st) __attribute__((always_inline)) {
    dma_tile(p.k + head + tile_of(kb), toff, lds0 + st * TILE);
  };
  auto issue_v = [&](int kb, int st) __attribute__((always_inline)) {
    dma_tile(p.v16 + head + tile_of(kb), toff, lds0 + (2 + st) * TILE);
  };
  const int kv_l = 32 * wk + l32;  // this lane's kv row of the A operand of S^T
  // LDS byte addresses of this lane's operand reads in stage 0 of the rings: the K rows (A operand
  // of S^T: chunk 2s + g of kv row kv_l) and the V^T operands of k-step 0 (d tile dt, row half h).
  // The stage (one tile further) and the V^T k-step (16 rows = 4 KiB further, where the swizzle
  // repeats) differ by constants, which the reads carry as immediate offsets; the loop is unrolled
  // by two so the stage is a constant. The empty asm keeps the addresses in registers.
  uint32_t ka_at[8], va_at[4][2];
  {
    const uint32_t base = lds_addr((VSA_LDS char*)kv_s);
#pragma unroll
    for (int s = 0; s < 8; ++s) ka_at[s] = base + tile_byte(kv_l, 2 * s + g);
    const int r0 = 32 * wk + 4 * g + (t16 >> 2);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int col = 32 * dt + 16 * (grp & 1) + 4 * (t16 & 3);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        va_at[dt][h] = base + 2 * TILE + tile_elem_byte(r0 + 8 * h, col);
        asm volatile("" : "+v"(va_at[dt][h]));
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) asm volatile("" : "+v"(ka_at[s]));
  }
  // A operand of S^T (K rows) from K stage st
  auto read_k = [&](int st, bf16x8 (&ka)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 8; ++s)
      ka[s] = *(const VSA_LDS bf16x8*)(uintptr_t)(ka_at[s] + st * TILE);
  };

  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};
  float m_run = -__builtin_inff();  // of this lane's q column over this wave's kv halves
  float l_run = 0.f;
  // this wave's state in the chunk workspace: O^T element rows 0..63, then max, sum (lane-major)
  float* state = p.state ? p.state + ((size_t)item * 4 + w) * FWD_STATE_FLOATS + lane : nullptr;
  if (!first) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][i] = state[(16 * dt + i) * 64];
    m_run = state[64 * 64];
    l_run = state[65 * 64];
  }

  // Block t: K in K stage t % 2, V in V stage t % 2. The S^T tile of block t is computed during
  // step t-1 (the prologue for t = 0), so step t overlaps the softmax of t with the S^T MFMAs of
  // t+1. Step t issues K of block t+2 (into the K stage block t used) and V of block t+1 (into
  // the V stage block t-1 used); past the end of the list the last block is repeated, so no
  // branch splits the step (the extra S^T tile is never used).
  // The list entries of blocks t, t+1, t+2 (e0, e1, e2) and block t's valid rows (vb0) are loaded
  // at the end of the step before, so no scalar-load wait sits inside a step.
  f32x16 sacc = f32x16{};
  int e0 = 0, e1 = 0, e2 = 0, vb0 = 0;
  if (n > 0) {
    e0 = kv_raw(0);
    e1 = kv_raw(1);
    e2 = kv_raw(2);
    vb0 = vb_of(e0);
    issue_k(e0, 0);
    issue_v(e0, 0);
    issue_k(e1, 1);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), visible to the compiler
    asm volatile("s_barrier" ::: "memory");
    bf16x8 ka[8];
    read_k(0, ka);
#pragma unroll
    for (int s = 0; s < 8; ++s) sacc = mfma32(ka[s], qf[s], sacc);
  }
  auto step = [&](int t, int st) __attribute__((always_inline)) {
    // K of t+1 and V of t landed (own DMAs, then the barrier: everyone's); everyone is done with
    // K of t and V of t-1
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), visible to the compiler
    asm volatile("s_barrier" ::: "memory");
    const int vb = vb0;
    // Raised wave priority from here to the rescale test: of the two waves sharing a SIMD, the one
    // issuing its operand reads, DMAs and first S^T MFMAs goes first, the other's exponentials
    // fill in behind (5 % faster than no priority, 1.155 against 1.219 ms at 32768 tokens).
    __builtin_amdgcn_s_setprio(1);

    // Each DMA follows the LDS reads of its kind (the asm keeps its place among them), so the
    // reads of this step are requested first and the two DMA groups reach the address unit
    // apart: about 1.5 % faster than both groups right after the barrier.
    bf16x8 ka[8];
    read_k(st ^ 1, ka);
    issue_k(e2, st);
    // V^T operands of O^T += V^T P^T: k-step c, slot j is kv 32wk + 16c + 8(j/4) + 4g + j%4 (the
    // D-layout order of S^T); d tile dt, lane's d = 32dt + l32
    f16x8 va[4][2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t o = st * TILE + c * 4096;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        va[dt][c] = join_f16(lds_read_tr((const VSA_LDS void*)(uintptr_t)(va_at[dt][0] + o)),
                             lds_read_tr((const VSA_LDS void*)(uintptr_t)(va_at[dt][1] + o)));
    }
    issue_v(e1, st ^ 1);

    // softmax of block t. S^T element i is kv 32wk + 8(i/4) + 4g + i%4, q = this lane's column.
    // The scores stay unscaled (the scale is positive, see above): the block max of s * scale is
    // the max of s times scale (rounding is monotone), and each exponent is one fma(s, scale, -m).
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = sacc[i];
    if (vb < BLOCK) {  // ragged or invalid block: mask kv rows >= vb
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kv = 32 * wk + 8 * (i / 4) + 4 * g + (i & 3);
        x[i] = kv < vb ? x[i] : -__builtin_inff();
      }
    }
    // the first half of the S^T MFMAs of t+1 under the block max, the second half under the
    // exponentials (no MFMA-free stretch while the max and the rescale test run)
    f32x16 snext = f32x16{};
#pragma unroll
    for (int s = 0; s < 4; ++s) snext = mfma32(ka[s], qf[s], snext);
    float mx = x[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, x[i]);
    mx = pair_max32(mx);
    mx *= scale_log2;
    // raise the running max (and rescale) only when this block's max exceeds it by the gap;
    // both lanes of a q column decide alike, and the branch is taken by the whole wave
    const bool raise = mx > m_run + RESCALE_GAP;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float m_new = raise ? mx : m_run;
      const float alpha = m_run == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
    }
    __builtin_amdgcn_s_setprio(0);
    const float m_use = m_run == -__builtin_inff() ? 0.f : m_run;
    // exponentials of t under the S^T MFMAs of t+1, then the O^T MFMAs of t
#pragma unroll
    for (int s = 4; s < 8; ++s) snext = mfma32(ka[s], qf[s], snext);
    float pv[16];
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], scale_log2, -m_use));
      rs += pv[i];
    }
    l_run += pair_sum32(rs);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const f16x8 pb = pack8_f16(pv[8 * c + 0], pv[8 * c + 1], pv[8 * c + 2], pv[8 * c + 3],
                                 pv[8 * c + 4], pv[8 * c + 5], pv[8 * c + 6], pv[8 * c + 7]);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) oacc[dt] = mfma32_f16(va[dt][c], pb, oacc[dt]);
    }
    // the next step's entry and row count: issued after every LDS read of this step is consumed
    // (a scalar load in flight would make the compiler wait for all LDS reads at once)
    __builtin_amdgcn_sched_barrier(0);
    const int e3 = kv_raw(t + 3), vb1 = vb_of(e1);
    sacc = snext;
    e0 = e1;
    e1 = e2;
    e2 = e3;
    vb0 = vb1;
  };
  int t = 0;
  for (; t + 1 < n; t += 2) {
    step(t, 0);
    step(t + 1, 1);
  }
  if (t < n) step(t, 0);

  if (!last) {  // save the state for the next chunk, exactly
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // no DMA may still write this workgroup's LDS
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) state[(16 * dt + i) * 64] = oacc[dt][i];
    state[64 * 64] = m_run;
    state[65 * 64] = l_run;
    return;
  }

  // ---- merge the two kv halves of each q half through LDS, normalise, store ----
  // The wave with kv half wk finalises d tiles 2wk, 2wk+1 and hands the other two over.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __builtin_amdgcn_s_waitcnt(0xc07f);
  asm volatile("s_barrier" ::: "memory");  // every wave is done with the rings
  VSA_LDS f32x4* xo = (VSA_LDS f32x4*)(kv_s + (2 * wq + wk) * 9216);      // my hand-over
  VSA_LDS f32x4* po = (VSA_LDS f32x4*)(kv_s + (2 * wq + (wk ^ 1)) * 9216);  // the partner's
  VSA_LDS float* xs = (VSA_LDS float*)(xo + 8 * 64);
  VSA_LDS float* ps = (VSA_LDS float*)(po + 8 * 64);
  auto hand_over = [&](const f32x16& a, const f32x16& b) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      xo[c * 64 + lane] = f32x4{a[4 * c], a[4 * c + 1], a[4 * c + 2], a[4 * c + 3]};
      xo[(4 + c) * 64 + lane] = f32x4{b[4 * c], b[4 * c + 1], b[4 * c + 2], b[4 * c + 3]};
    }
  };
  if (wk == 0)  // uniform: constant register indices in each branch
    hand_over(oacc[2], oacc[3]);
  else
    hand_over(oacc[0], oacc[1]);
  xs[lane] = m_run;
  xs[64 + lane] = l_run;
  __builtin_amdgcn_s_waitcnt(0xc07f);
  asm volatile("s_barrier" ::: "memory");
  const float m_o = ps[lane], l_o = ps[64 + lane];
  const float m = fmaxf(m_run, m_o);
  const float a_me = m_run == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
  const float a_o = m_o == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_o - m);
  const float l = a_me * l_run + a_o * l_o;
  const float inv_l = l > 0.f ? 1.0f / l : 0.f;
  // O^T accumulated P v16 = P v * 2^-e: scale back exactly after normalising
  const int vexp = f16_head_exponent(ld_const(p.v_amax, bh));
  bf16* orow = p.o + head + (size_t)qrow * HEAD_DIM;
  auto finish = [&](const f32x16& mine, int u, int dt) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 o2 = po[(u * 4 + c) * 64 + lane];
      union {
        bf16 b[4];
        s16x4 s;
      } r;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        r.b[e] = (bf16)__builtin_ldexpf((a_me * mine[4 * c + e] + a_o * o2[e]) * inv_l, vexp);
      // element 4c + e of tile dt is d = 32dt + 8c + 4g + e
      *(s16x4*)(orow + 32 * dt + 8 * c + 4 * g) = r.s;
    }
  };
  if (wk == 0) {
    finish(oacc[0], 0, 0);
    finish(oacc[1], 1, 1);
  } else {
    finish(oacc[2], 0, 2);
    finish(oacc[3], 1, 3);
  }
  if (wk == 0 && g == 0)
    p.lse[(size_t)bh * p.S + qrow] = l > 0.f ? m + __builtin_log2f(l) : -__builtin_inff();
}

namespace {

// One workgroup per (bh, 64-row tile): each thread takes four 16-byte chunks of the 16 KiB tile.
// |x| of a bf16 is its bit pattern with the sign cleared, and for non-negative values the bit
// patterns order like the values, so the max is an integer max (fp32 bits = bf16 bits << 16). The
// tile's max goes to tmax[tile]; no atomics (thousands of them on one word per head serialise).
__global__ void __launch_bounds__(256) v_tile_absmax_kernel(const bf16* __restrict__ v,
                                                            uint32_t* __restrict__ tmax) {
  __shared__ uint32_t wmax[4];
  const i32x4* src = (const i32x4*)(v + (size_t)blockIdx.x * BLOCK * HEAD_DIM);
  uint32_t m = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const i32x4 x = src[c * 256 + threadIdx.x];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = (uint32_t)x[e];
      m = max(m, max(u & 0x7FFFu, (u >> 16) & 0x7FFFu));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    tmax[blockIdx.x] = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])) << 16;
}

// One workgroup per head: amax[bh] = max over the head's tile maxima.
__global__ void __launch_bounds__(256) v_head_absmax_kernel(const uint32_t* __restrict__ tmax,
                                                            int tiles_per_head,
                                                            uint32_t* __restrict__ amax) {
  __shared__ uint32_t wmax[4];
  const uint32_t* t = tmax + (size_t)blockIdx.x * tiles_per_head;
  uint32_t m = 0;
  for (int i = threadIdx.x; i < tiles_per_head; i += 256) m = max(m, t[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) amax[blockIdx.x] = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
}

__global__ void __launch_bounds__(256) v16_convert_kernel(const bf16* __restrict__ v,
                                                          int tiles_per_head,
                                                          const uint32_t* __restrict__ amax,
                                                          f16* __restrict__ v16) {
  const int tile = blockIdx.x;
  const int e = f16_head_exponent(ld_const(amax, tile / tiles_per_head));
  const size_t base = (size_t)tile * BLOCK * HEAD_DIM;
  const bf16x8* src = (const bf16x8*)(v + base);
  f16x8* dst = (f16x8*)(v16 + base);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const bf16x8 x = src[c * 256 + threadIdx.x];
    f16x8 y;
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = (f16)__builtin_ldexpf((float)x[k], -e);
    dst[c * 256 + threadIdx.x] = y;
  }
}

}  // namespace

void launch_v16(const bf16* v, int BH, int S, uint32_t* amax, uint32_t* tmax, f16* v16,
               hipStream_t stream) {
  const int tiles_per_head = S / BLOCK;
  hipLaunchKernelGGL(v_tile_absmax_kernel, dim3(BH * tiles_per_head), dim3(256), 0, stream, v,
                     tmax);
  hipLaunchKernelGGL(v_head_absmax_kernel, dim3(BH), dim3(256), 0, stream,
                     (const uint32_t*)tmax, tiles_per_head, amax);
  hipLaunchKernelGGL(v16_convert_kernel, dim3(BH * tiles_per_head), dim3(256), 0, stream, v,
                     tiles_per_head, (const uint32_t*)amax, v16);
}

void launch_fwd(const FwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(fwd_kernel, dim3((unsigned)(p.items_per_xcd * 8)), dim3(256), 0, stream, p);
}

}  // namespace vsa
