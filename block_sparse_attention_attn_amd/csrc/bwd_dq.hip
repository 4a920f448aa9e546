// bwd_dq.hip -- dQ of the 64-token block-sparse attention backward on gfx950 (the q-major half of
// the backward's main step, with the dQ scale/convert epilogue fused).
//
// What it computes (the gradient of the FastVideo backward test page's masked-dense reference;
// launch header argument struct: dq carries sm_scale, lse is the base-2 "M form"): for one q block
// i of (b, h) and every kv block j in its q2k list,
//     S^T  = K_j Q_i^T,   P^T = exp2(S^T * scale_log2 - lse_i)   (kv rows >= vbs[j] -> 0)
//     dP^T = V_j dO_i^T,  dS^T = P^T * (dP^T - Delta_i)
//     dQ_i += dS K_j
// and dq_i = bf16(sm_scale * dQ_i). A q block with an empty list gets zero rows. The GEMMs run on
// the preprocess's scaled fp16 copies (v_mfma_f32_32x32x16_f16): S' = S 2^-(eq+ek),
// dP' = dP 2^-(eo+ev), P' = P 2^pp = exp2(c S' + pp - lse), dS' = P' (dP' - Delta') = dS 2^es,
// and the sum dS' k16 = dQ 2^(es-ek) is scaled back in the epilogue.
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
// and dP^T = V dO^T (v_mfma_f32_32x32x16_f16), so lse and Delta are one scalar per lane. K_j,
// V_j stream through a four-stage ring of swizzled LDS tiles fetched three kv blocks ahead
// (global_load_lds_dwordx4). Step t runs the S^T/dP^T MFMAs of kv block t+1 interleaved with the
// exp2/convert work of kv block t and its K^T transposed reads (ds_read_b64_tr_b16), then the
// dQ^T += K^T dS^T MFMAs of kv block t interleaved with the K/V row reads of kv block t+2: every
// MFMA's LDS operands are requested a phase before it issues. dS^T stays in registers as the B
// operand. The two kv halves' partial dQ^T are summed through LDS once per q block. On request the
// lists run in kv-range chunks, one launch each, dQ carried between launches as fp32 partial sums.
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace vsa {

namespace {

constexpr int STAGES = 4;
constexpr int STAGE_BYTES = 16384;

__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_dq_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) char k_ring[STAGES * STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_ring[STAGES * STAGE_BYTES];

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
  // kv-range chunk: this launch walks list positions [start, start + n) and adds to (first:
  // starts) the fp32 partial dQ of the chunks before, which the last chunk turns into dq
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
    if (n == 0 && !first && !last) return;  // nothing to add, nothing to finish
  }
  const int bh = item / p.nb;
  const int i = item - bh * p.nb;
  const size_t head = (size_t)bh * p.S * HEAD_DIM;
  const bf16* __restrict__ kh = (const bf16*)(p.k16 + head);  // fp16 tiles (the DMA moves bytes)
  const bf16* __restrict__ vh = (const bf16*)(p.v16 + head);
  const int32_t* __restrict__ hs = p.scales + (size_t)bh * HEAD_SCALE_WORDS;
  const int* __restrict__ list = p.q2k_idx + (size_t)item * p.q2k_stride + start;
  auto kvblock = [&](int t) {
    const int kb = ld_const(list, t);
    return kb < 0 ? 0 : (kb >= p.nb ? p.nb - 1 : kb);
  };
  VSA_LDS char* const kr = (VSA_LDS char*)k_ring;
  VSA_LDS char* const vr = (VSA_LDS char*)v_ring;
  uint32_t toff[4];
  tile_offsets<4>(toff, lane, w);
  auto issue = [&](int t, int st) __attribute__((always_inline)) {
    const size_t tile = (size_t)kvblock(t) * BLOCK * HEAD_DIM;
    tile_load_async_off<4>(kh + tile, kr + st * STAGE_BYTES, toff, w);
    tile_load_async_off<4>(vh + tile, vr + st * STAGE_BYTES, toff, w);
  };
  if (n > 0) issue(0, 0);
  if (n > 1) issue(1, 1);
  if (n > 2) issue(2, 2);

  // B operands: lane holds q row 32*wq + l32, d = 16*s + 8*g + 0..7
  const int qrow = i * BLOCK + 32 * wq + l32;
  f16x8 qf[8], df[8];
  {
    const f16x8* qrp = (const f16x8*)(p.q16 + head + (size_t)qrow * HEAD_DIM);
    const f16x8* drp = (const f16x8*)(p.do16 + head + (size_t)qrow * HEAD_DIM);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qf[s] = qrp[2 * s + g];
      df[s] = drp[2 * s + g];
    }
  }
  // a q row with no valid key has lse = -inf; +inf makes its P exactly 0 (no inf * 0)
  float lse_q = p.lse[(size_t)bh * p.S + qrow];
  lse_q = lse_q == -__builtin_inff() ? __builtin_inff() : lse_q;
  // P' = exp2(c S' + (pp - lse))
  const float off_q = (float)ld_const(hs, SC_PP) - lse_q;
  // -Delta' of this q row, from the preprocess record of q block i
  const float ndelta_q =
      p.lse_delta[((size_t)bh * p.nb + i) * LD_RECORD_FLOATS + BLOCK + 32 * wq + l32];
  const float cexp = __uint_as_float((uint32_t)ld_const(hs, SC_C));

  // dQ^T tiles: element e of tile mt is d = 32*mt + 8*(e/4) + 4*g + e%4, q = 32*wq + l32
  f32x16 dq_acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) dq_acc[mt] = f32x16{};

  const int kvrow = 32 * wk + l32;
  // A operands of S^T = K Q^T and dP^T = V dO^T: kv row 32*wk + l32, d = 16*s + 8*g + 0..7
  auto load_rows = [&](int st, f16x8* ka, f16x8* va) __attribute__((always_inline)) {
    VSA_LDS char* kt = kr + st * STAGE_BYTES;
    VSA_LDS char* vt = vr + st * STAGE_BYTES;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      ka[s] = *(const VSA_LDS f16x8*)(kt + tile_byte(kvrow, 2 * s + g));
      va[s] = *(const VSA_LDS f16x8*)(vt + tile_byte(kvrow, 2 * s + g));
    }
  };

  // A kv block with padded rows (vbs < 64): once its tiles have landed, zero those K and V rows
  // in LDS (they may hold anything), then meet at a barrier before anyone reads them. Rare: a
  // uniform branch taken only for ragged blocks. Returns the block's vbs (its step masks dS^T).
  auto zero_padding = [&](int t, int st) __attribute__((always_inline)) {
    const int vb = ld_const(p.vbs, kvblock(t));
    if (vb < BLOCK) {
      const int first = vb < 0 ? 0 : vb;
      for (int c = first * 16 + (int)threadIdx.x; c < BLOCK * 16; c += 256) {
        *(VSA_LDS i32x4*)(kr + st * STAGE_BYTES + c * 16) = i32x4{};
        *(VSA_LDS i32x4*)(vr + st * STAGE_BYTES + c * 16) = i32x4{};
      }
      barrier_lds();
    }
    return vb;
  };

  if (n > 0) {
    f32x16 s0, p0, s1, p1;
    f16x8 ka0[8], va0[8], ka1[8], va1[8];
    // vbs of the kv block in each ring stage (set when its padding is zeroed, two steps ahead)
    int vbs0 = BLOCK, vbs1 = BLOCK, vbs2 = BLOCK, vbs3 = BLOCK;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // stages 0..2 landed (own DMAs)
    barrier_lds();
    vbs0 = zero_padding(0, 0);
    if (n > 1) vbs1 = zero_padding(1, 1);
    load_rows(0, ka0, va0);
    s0 = f32x16{};
    p0 = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      s0 = mfma32_f16(ka0[s], qf[s], s0);
      p0 = mfma32_f16(va0[s], df[s], p0);
    }
    load_rows(1, ka1, va1);  // stale but in bounds when n == 1

    // Step t (kv block t in stage st, t+2 in st2; kv block t+3 is fetched into st3): on entry
    // S^T/dP^T of t are in (sc, pc) and the row operands of t+1 in (ka, va). The last steps use
    // stale (in-bounds, quiescent) stages for throwaway work, keeping the body branch-free.
    auto step = [&](int t, int st, int st2, int st3, f32x16& sc, f32x16& pc, f32x16& sn,
                    f32x16& pn, f16x8* ka, f16x8* va, f16x8* kn, f16x8* vn, int vb_t,
                    int& vb_ahead) __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // stage t+2 landed (own DMAs)
      barrier_lds();  // ... everyone's; everyone is done with stage st3 (kv block t-1)
      if (t + 3 < n) issue(t + 3, st3);
      if (t + 2 < n) vb_ahead = zero_padding(t + 2, st2);  // before anyone reads kv block t+2
      VSA_LDS char* kt = kr + st * STAGE_BYTES;

      // ---- phase B: S^T/dP^T of kv block t+1; dS^T of kv block t; K^T reads of t ----
      // K^T A operand of dQ: lane holds d = 32*mt + l32, k slot jj of step s2 is kv
      // 32*wk + 16*s2 + 8*(jj/4) + 4*g + jj%4, matching the D layout of S^T
      f16x8 kt_op[2][4];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int kv0 = 32 * wk + 16 * s2 + 4 * (grp >> 1) + (t16 >> 2);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int col = 32 * mt + 16 * (grp & 1) + 4 * (t16 & 3);
          kt_op[s2][mt] = join_f16(lds_read_tr(kt + tile_elem_byte(kv0, col)),
                                   lds_read_tr(kt + tile_elem_byte(kv0 + 8, col)));
        }
      }
      sn = f32x16{};
      pn = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        sn = mfma32_f16(ka[s], qf[s], sn);
        pn = mfma32_f16(va[s], df[s], pn);
      }
      // dS'^T of kv block t. A padded kv row has a zero K row, so its score is 0 and its P' is
      // exp2(pp - lse_q): infinite once lse_q <= pp - 128 (every valid score far below), and inf
      // times the zero K^T row would put NaN into dQ. So a ragged block (a uniform branch, rare)
      // sets the dS^T of its padded rows to exactly 0. Element e is kv row
      // 32*wk + 8*(e/4) + 4*g + e%4.
      float dsv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], cexp, off_q));
        dsv[e] = pe * (pc[e] + ndelta_q);
      }
      if (vb_t < BLOCK) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          dsv[e] = 32 * wk + 8 * (e >> 2) + 4 * g + (e & 3) < vb_t ? dsv[e] : 0.0f;
      }
      f16x8 b[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        b[s2] = pack8_f16(dsv[8 * s2 + 0], dsv[8 * s2 + 1], dsv[8 * s2 + 2], dsv[8 * s2 + 3],
                      dsv[8 * s2 + 4], dsv[8 * s2 + 5], dsv[8 * s2 + 6], dsv[8 * s2 + 7]);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one transposed read
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
      }
      __builtin_amdgcn_sched_barrier(0);

      // ---- phase C: dQ^T += K^T dS^T of kv block t; row reads of kv block t+2 ----
      load_rows(st2, kn, vn);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) dq_acc[mt] = mfma32_f16(kt_op[s2][mt], b[s2], dq_acc[mt]);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two row reads
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int t = 0; t < n; t += 4) {
      step(t, 0, 2, 3, s0, p0, s1, p1, ka1, va1, ka0, va0, vbs0, vbs2);
      if (t + 1 < n) step(t + 1, 1, 3, 0, s1, p1, s0, p0, ka0, va0, ka1, va1, vbs1, vbs3);
      if (t + 2 < n) step(t + 2, 2, 0, 1, s0, p0, s1, p1, ka1, va1, ka0, va0, vbs2, vbs0);
      if (t + 3 < n) step(t + 3, 3, 1, 2, s1, p1, s0, p0, ka0, va0, ka1, va1, vbs3, vbs1);
    }
  }

  // ---- sum the two kv halves: wave wk=0 finishes d tiles 0,1, wave wk=1 tiles 2,3 ----
  barrier_lds();  // all LDS reads of the K/V ring are done
  VSA_LDS f32x4* xch = (VSA_LDS f32x4*)(kr + wq * STAGE_BYTES);
  // region r holds the tiles that wave (wq, r) finishes, written by its partner (wq, 1 - r)
  VSA_LDS f32x4* give = xch + (wk == 0 ? 512 : 0);
  VSA_LDS f32x4* take = xch + (wk == 0 ? 0 : 512);
  // (tiles are picked with selects, not a runtime index: that would move dq_acc to scratch)
#pragma unroll
  for (int u = 0; u < 2; ++u) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = wk == 0 ? dq_acc[2 + u][4 * c + e] : dq_acc[u][4 * c + e];
      give[(u * 4 + c) * 64 + lane] = v;  // the partner's tiles
    }
  }
  barrier_lds();
  bf16* dqrow = p.dq + head + (size_t)qrow * HEAD_DIM;
  // this lane's q row of the chunk partial sums: [64][128] fp32 per q block
  float* prow = p.part ? p.part + (size_t)item * (BLOCK * HEAD_DIM) +
                             (size_t)(32 * wq + l32) * HEAD_DIM
                       : nullptr;
  const float sc = p.sm_scale;
  const int oexp = ld_const(hs, SC_EK) - ld_const(hs, SC_ES);  // dq = sm_scale dQ' 2^(ek - es)
  // the chunks before: this lane's partial sums, all loaded before any store below (a store may
  // alias a later load, which would otherwise wait for it)
  f32x4 prev[2][4];
  if (!first) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        prev[u][c] = *(const f32x4*)(prow + 32 * ((wk == 0 ? 0 : 2) + u) + 8 * c + 4 * g);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int mt = (wk == 0 ? 0 : 2) + u;  // my tiles
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 o = take[(u * 4 + c) * 64 + lane];
      f32x4 sum;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sum[e] = (wk == 0 ? dq_acc[u][4 * c + e] : dq_acc[2 + u][4 * c + e]) + o[e];
      const int d0 = 32 * mt + 8 * c + 4 * g;
      if (!first) sum += prev[u][c];
      if (last) {
        union {
          bf16 b[4];
          s16x4 s;
        } r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r.b[e] = (bf16)__builtin_ldexpf(sum[e] * sc, oexp);
        *(s16x4*)(dqrow + d0) = r.s;
      } else {
        *(f32x4*)(prow + d0) = sum;
      }
    }
  }
}

void launch_bwd_dq(const BwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(bwd_dq_kernel, dim3(p.items_per_xcd * 8), dim3(256), 0, stream, p);
}

}  // namespace vsa
