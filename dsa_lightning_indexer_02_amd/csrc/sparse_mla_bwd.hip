// Backward of the sparse MLA forward (DeepSeek-V3.2-Exp summary page, section "Method": in the
// sparse training stage the main model trains with top-k selection on, its attention reading only
// the selected latent rows; AMD MI355X article, section "Training Approach", sparse stage).
//
// For query row t, head h and the valid entries i of its list (0 <= idx_i < n_t), with the
// forward's z_i = sm_scale q . k_i, p_i = exp(z_i - lse), out = sum_i p_i v_i and g = dL/dout:
//   dp_i = g . v_i,   D = g . out,   ds_i = p_i (dp_i - D),
//   dq      = sm_scale sum_i ds_i k_i                          (all D_qk columns)
//   dkv[s] += sm_scale ds_i q  +  p_i g (first D_v columns)   for each entry i with idx_i = s.
//
// D = g . out is formed here as sum_i p_i dp_i from the same fp32 p and dp as ds (not from the
// forward's rounded output: where one key dominates the softmax, ds is a small difference and a
// rounded D would swamp it).
//
// Kernels (H heads in halves of 64 per workgroup, 4 waves, one per SIMD; wave (g, f) serves the 32
// heads of group g and contraction half f, as in the forward):
//  - sparse_mla_bwd_kernel<DKV = false>: per block of 32 gathered rows (DMA into LDS, XOR-swizzled as
//    the forward), partial S^T = K Q^T and dP^T = V G^T over the wave's half (bf16 32x32x16 MFMA),
//    summed with the partner's through LDS; p in fp32 on the accumulator layout (lane = head).  Pass
//    0 sums p dp into D (written for the dKV kernel); pass 1 forms ds = p (dp - D) and
//    dQ^T += K^T dS^T with K^T from transposing LDS reads of the gathered rows and ds split into a
//    bf16 high part and a bf16 remainder (two MFMAs; 16 significant bits), accumulated over all
//    blocks in registers, written once;
//  - sparse_mla_bwd_kernel<DKV = true>: the same scores and D, then sm_scale ds and p as fp16 tiles
//    [head][key] in LDS; each wave forms the dKV rows of the block for its share of the columns,
//    contracting over the 64 heads (fp16 16x16x32 MFMA; Q^T and G^T fragments converted from bf16
//    once per workgroup and kept in registers), and adds them to dkv with fp32 atomic adds (the two
//    head halves and every query row selecting a key add into the same row).
#include "dsa_internal.hpp"

namespace dsa {

constexpr int BW_THREADS = 256;     // 4 waves
constexpr int BWM_KB = 32;          // gathered rows per block
constexpr int BWM_HEADS = 64;       // heads per workgroup
constexpr int BWM_MAX_K = 2048;
constexpr float BWM_LOG2E = 1.4426950408889634f;

// Geometry of the 576 / 512 latent rows (the only width the backward is built for).
struct BwmCfg {
  static constexpr int DQK = 576, DV = 512;
  static constexpr int DH = 288;            // q.k columns per wave of a pair
  static constexpr int NKS = DH / 16;       // 32x32x16 steps of the partial S^T
  static constexpr int DVH = 256;           // value columns per wave of a pair
  static constexpr int NVS = DVH / 16;      // steps of the partial dP^T
  static constexpr int NQT = DH / 32;       // 32-wide dQ tiles per wave
  static constexpr int RC = DQK / 8;        // 16-byte chunks per row (72)
  static constexpr int SLOTS = BWM_KB * RC;
  static constexpr int K_BYTES = SLOTS * 16;
  static constexpr int DMA_INSTR = SLOTS / WAVE;          // 36 wave-wide transfers per block
  static constexpr int DMA_PW = DMA_INSTR / 4;            // 9 per wave
  static constexpr int SX_BYTES = 4 * 2 * WAVE * 16 * 4;  // partial S^T and dP^T of every wave
  // dKV mode: columns per wave (dK over 576, dV over 512) in 16-wide MFMA tiles
  static constexpr int KC = DQK / 4, VC = DV / 4;         // 144, 128
  static constexpr int NKC = KC / 16, NVC = VC / 16;      // 9, 8
  static constexpr int TILE_STRIDE = BWM_KB * 2 + 16;     // bytes per head row of an fp16 [head][key] tile
  static constexpr int TILE_BYTES = BWM_HEADS * TILE_STRIDE;
  static constexpr int STAGE_Q_STRIDE = DQK * 2 + 16;     // row stride of the staged Q / G (bf16)
  static_assert(DMA_INSTR % 4 == 0 && 2 * DMA_PW <= WAVE, "gather transfers split evenly over 4 waves");
  // chunk XOR of gathered row r (the forward's swizzle: conflict-free fragment and transposing reads)
  static __host__ __device__ __forceinline__ constexpr int swz(int r) {
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
  static __device__ __forceinline__ int slot(int r, int c) { return r * RC + (c ^ swz(r)); }
};

constexpr size_t bwm_smem_bytes(bool dkv) {
  using C = BwmCfg;
  const size_t base = 2 * (size_t)C::K_BYTES + C::SX_BYTES + (size_t)(BWM_MAX_K + 4 + BWM_MAX_K / BWM_KB) * 4;
  const size_t tiles = 2 * (size_t)C::TILE_BYTES;
  const size_t stage = (size_t)BWM_HEADS * C::STAGE_Q_STRIDE;  // Q / G staging before the block loop
  const size_t loop = base + (dkv ? tiles : 0);
  return dkv && stage > loop ? stage : loop;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) reinterpret_cast<v4f*>(p)[i] = (v4f){0.f, 0.f, 0.f, 0.f};
}

__device__ __forceinline__ short f32_to_f16_bits(float x) { return __builtin_bit_cast(short, (_Float16)x); }

// bf16 round to nearest even of x (high part) and of the remainder x - high (16 significant bits
// together), as 16-bit patterns
__device__ __forceinline__ short bf16_hi(float x) { return (short)f32_to_bf16(x); }
__device__ __forceinline__ short bf16_lo(float x) {
  return (short)f32_to_bf16(x - __uint_as_float((uint32_t)f32_to_bf16(x) << 16));
}

template <bool DKV>
__global__ __launch_bounds__(BW_THREADS, 1) void sparse_mla_bwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    const float* __restrict__ lse, float* __restrict__ delta, const uint16_t* __restrict__ dout, int64_t S,
    int64_t q_start, int32_t H, int32_t k, float scale_log2, float sm_scale, float* __restrict__ dq,
    float* __restrict__ dkv) {
  using C = BwmCfg;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* Kbuf = smem;                                            // [2][SLOTS] x 16 B
  v4f* Sx = reinterpret_cast<v4f*>(smem + 2 * C::K_BYTES);          // [wave][S, dP][4][64] x v4f
  int32_t* phys = reinterpret_cast<int32_t*>(smem + 2 * C::K_BYTES + C::SX_BYTES);
  uint32_t* vmask = reinterpret_cast<uint32_t*>(phys + BWM_MAX_K + 4);
  uint8_t* tiles = reinterpret_cast<uint8_t*>(vmask + BWM_MAX_K / BWM_KB);  // DKV: fp16 [head][key] ds, p

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 1, hf = wave & 1;
  const int l32 = lane & 31, lh = lane >> 5;
  const int64_t t = (int64_t)gridDim.x - 1 - blockIdx.x;  // latest rows first (longest lists)
  const int h0 = blockIdx.y * BWM_HEADS;
  const int head = h0 + g * 32 + l32;
  const bool hv = head < H;
  const int64_t n = min(S, q_start + t + 1);

  // ---- index list: physical rows (-1: skipped entry) and per-block validity words
  for (int i = tid; i < k; i += BW_THREADS) {
    const int32_t li = idx[t * k + i];
    phys[i] = (li >= 0 && li < n) ? li : -1;
  }
  for (int base = wave * WAVE; base < (k + 63) / 64 * 64; base += 4 * WAVE) {
    const int i = base + lane;
    bool v = false;
    if (i < k) {
      const int32_t li = idx[t * k + i];
      v = li >= 0 && li < n;
    }
    const uint64_t bits = __ballot(v);
    if (lane == 0) {
      vmask[base / 32] = (uint32_t)bits;
      if (base + 32 < k) vmask[base / 32 + 1] = (uint32_t)(bits >> 32);
    }
  }

  // ---- resident operands: queries and output gradients of this wave's heads and half, as the
  // B operands of S^T = K Q^T and dP^T = V G^T
  s16x8 Qf[C::NKS], Gf[C::NVS];
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) {
    s16x8 v = *reinterpret_cast<const s16x8*>(q + (t * H + (hv ? head : 0)) * (int64_t)C::DQK + hf * C::DH +
                                              ks * 16 + lh * 8);
    if (!hv) v = (s16x8){0, 0, 0, 0, 0, 0, 0, 0};
    Qf[ks] = v;
  }
#pragma unroll
  for (int ks = 0; ks < C::NVS; ++ks) {
    s16x8 v = *reinterpret_cast<const s16x8*>(dout + (t * H + (hv ? head : 0)) * (int64_t)C::DV + hf * C::DVH +
                                              ks * 16 + lh * 8);
    if (!hv) v = (s16x8){0, 0, 0, 0, 0, 0, 0, 0};
    Gf[ks] = v;
  }
  // heads past H get p = 0 (exp2(-inf)) and ds = 0
  const float lse2 = hv ? lse[t * H + head] * BWM_LOG2E : INFINITY;
  float dlt = 0.f;  // D of this lane's head: summed in pass 0 (dQ kernel) or read (dKV kernel)
  if constexpr (DKV) dlt = hv ? delta[t * H + head] : 0.f;

  // ---- DKV: B operands of the head contraction, Q^T and G^T fragments (lane = column, eight heads
  // per lane group), staged through LDS once and converted bf16 -> fp16 (exact for |x| in
  // [2^-14, 65504])
  constexpr int NKC = DKV ? C::NKC : 1, NVC = DKV ? C::NVC : 1;
  s16x8 QT[NKC][2], GT[NVC][2];
  if constexpr (DKV) {
    const int a = lane & 15, grp = lane >> 4;
    auto stage_rows = [&](const uint16_t* src, int width) {
      // rows h0 .. h0 + 63 of [t][h][width] into LDS, row stride STAGE_Q_STRIDE (zeros past H)
      const int chunks = width / 8;
      for (int p = tid; p < BWM_HEADS * chunks; p += BW_THREADS) {
        const int r = p / chunks, c = p % chunks;
        v4i v = {0, 0, 0, 0};
        if (h0 + r < H) v = *reinterpret_cast<const v4i*>(src + (t * H + h0 + r) * (int64_t)width + c * 8);
        *reinterpret_cast<v4i*>(smem + r * C::STAGE_Q_STRIDE + c * 16) = v;
      }
    };
    // fragment (column tile col0, heads 32 kk .. 32 kk + 31): two transposing reads of rows
    // 32 kk + 8 grp + {0..3}, {4..7}, columns col0 + 4 (a % 4)
    auto frag = [&](int col0, int kk) {
      s16x8 r;
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        const int row = 32 * kk + 8 * grp + 4 * hlf + (a >> 2);
        const s16x4 w = lds_transpose_read16(smem + row * C::STAGE_Q_STRIDE + (col0 + 4 * (a & 3)) * 2);
#pragma unroll
        for (int e = 0; e < 4; ++e) r[4 * hlf + e] = f32_to_f16_bits(bf16_to_f32((uint16_t)w[e]));
      }
      return r;
    };
    stage_rows(q, C::DQK);
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < NKC; ++ct)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) QT[ct][kk] = frag(wave * C::KC + ct * 16, kk);
    __syncthreads();
    stage_rows(dout, C::DV);
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < NVC; ++ct)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) GT[ct][kk] = frag(wave * C::VC + ct * 16, kk);
  }
  __syncthreads();  // list, masks and staging done before the gathers overwrite the LDS

  const int32_t safe_row = 0;  // skipped entries gather row 0 (masked out)
  const uint32_t kbuf_lds = lds_offset(Kbuf);
  // gather of block blk into stage blk % 2: transfer i (this wave's j-th) covers slots [64 i, 64 i + 64)
  auto gather = [&](int blk) {
    const uint32_t base = kbuf_lds + (uint32_t)((blk & 1) * C::K_BYTES);
    int32_t prow = -1;
    {
      const int j = lane >> 1, i = wave + j * 4;
      const int rr = (i * WAVE + (lane & 1) * (WAVE - 1)) / C::RC;
      const int e = blk * BWM_KB + rr;
      if (j < C::DMA_PW && e < k) prow = phys[e];
      prow = prow >= 0 ? prow : safe_row;
    }
#pragma unroll
    for (int j = 0; j < C::DMA_PW; ++j) {
      const int i = wave + j * 4;
      const int s = i * WAVE + lane;
      const int rr = s / C::RC;
      const int c = (s % C::RC) ^ C::swz(rr);
      const int first = (i * WAVE) / C::RC;
      const int32_t pa = __builtin_amdgcn_readlane(prow, 2 * j), pb = __builtin_amdgcn_readlane(prow, 2 * j + 1);
      lds_dma_16B(kv + (int64_t)(rr == first ? pa : pb) * C::DQK + c * 8, base + (uint32_t)(i * WAVE * 16));
    }
  };

  // K fragment (A operand of S^T): row l32, chunk (hf DH / 8) + 2 ks + lh; V fragment (A operand of
  // dP^T): row l32, chunk (hf DVH / 8) + 2 ks + lh.  Steps 4 apart share a per-lane base.
  const int kx = C::swz(l32);
  int kb[4], vb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    kb[u] = (l32 * C::RC + ((hf * (C::DH / 8) + lh + 2 * u) ^ kx)) * 16;
    vb[u] = (l32 * C::RC + ((hf * (C::DVH / 8) + lh + 2 * u) ^ kx)) * 16;
  }
  // K^T fragment (A operand of dQ^T, tile dt, key step m): two transposing reads, rows
  // 16 m + 4 lh' + (a >> 2) (+ 8), columns hf DH + 32 dt + 16 (grp & 1) + 4 (a & 3), lh' = grp >> 1.
  // The chunk is hf 36 + 4 dt + low; its XOR with the row swizzle depends on (dt + hf) & 1 and the
  // read half only, so four per-lane bases plus compile-time offsets cover every fragment.
  int kt_base[2][2];
  {
    const int a = lane & 15, grp = lane >> 4;
    const int low = 2 * (grp & 1) + ((a & 3) >> 1);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int odd = 0; odd < 2; ++odd) {
        const int r = 4 * (grp >> 1) + (a >> 2) + 8 * j;
        const int par = odd ^ hf;
        const int c = 32 * hf + 8 * (hf & odd) + ((4 * par + low) ^ C::swz(r));
        kt_base[j][odd] = (r * C::RC + c) * 16 + (a & 1) * 8;
      }
  }

  v16f acc[DKV ? 1 : C::NQT];
  if constexpr (!DKV) {
#pragma unroll
    for (int dt = 0; dt < C::NQT; ++dt) acc[dt] = (v16f){};
  }

  const int nblk_all = (k + BWM_KB - 1) / BWM_KB;
  const uint64_t live = __ballot(lane < nblk_all && vmask[lane] != 0u);
  const int nblk = live ? 64 - __clzll(live) : 0;
  const v4f* Sx_peer = Sx + ((wave ^ 1) * 2) * 4 * WAVE + lane;
  v4f* Sx_mine = Sx + (wave * 2) * 4 * WAVE + lane;

  // the dQ kernel walks the blocks twice (pass 0: D; pass 1: dQ), the dKV kernel once
  for (int pass = DKV ? 1 : 0; pass < 2; ++pass) {
  if (nblk > 0) gather(0);
  float dsum = 0.f;  // pass 0: this lane's part of sum_i p_i dp_i
  for (int blk = 0; blk < nblk; ++blk) {
    const uint8_t* Kst = Kbuf + (blk & 1) * C::K_BYTES;
    vm_wait<0>();
    __syncthreads();  // stage blk complete; every wave done with block blk - 1
    if (blk + 1 < nblk) gather(blk + 1);

    // ---- partial S^T[key][head] and dP^T[key][head] over this wave's halves
    v16f sc = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      const s16x8 A = *reinterpret_cast<const s16x8*>(Kst + kb[ks % 4] + (ks / 4) * 128);
      sc = mfma_bf16_32x32x16(A, Qf[ks], sc);
    }
#pragma unroll
    for (int ks = 0; ks < C::NVS; ++ks) {
      const s16x8 A = *reinterpret_cast<const s16x8*>(Kst + vb[ks % 4] + (ks / 4) * 128);
      dp = mfma_bf16_32x32x16(A, Gf[ks], dp);
    }
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      Sx_mine[qd * WAVE] = (v4f){sc[4 * qd], sc[4 * qd + 1], sc[4 * qd + 2], sc[4 * qd + 3]};
      Sx_mine[(4 + qd) * WAVE] = (v4f){dp[4 * qd], dp[4 * qd + 1], dp[4 * qd + 2], dp[4 * qd + 3]};
    }
    __syncthreads();  // both partials posted

    // ---- full scores, probabilities and ds on the accumulator layout (lane = head, 16 keys)
    const uint32_t vt = vmask[blk] >> (4 * lh);
    const uint32_t vbits = (vt & 0xFu) | ((vt >> 4) & 0xF0u) | ((vt >> 8) & 0xF00u) | ((vt >> 12) & 0xF000u);
    float pr[16], ds[16];
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const v4f ps = Sx_peer[qd * WAVE], pd = Sx_peer[(4 + qd) * WAVE];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = 4 * qd + e;
        const bool valid = (vbits >> rr) & 1u;
        const float s2 = (sc[rr] + ps[e]) * scale_log2;
        const float p = valid ? __builtin_amdgcn_exp2f(s2 - lse2) : 0.f;
        const float dpf = dp[rr] + pd[e];
        pr[rr] = p;
        dsum = fmaf(p, dpf, dsum);
        ds[rr] = p * (dpf - dlt);
      }
    }
    if (pass == 0) continue;  // D only

    if constexpr (!DKV) {
      // dQ^T[d][head] += K^T[d][key] dS^T[key][head]: B = ds (hi, lo) for key steps m = 0, 1
      s16x8 Bh[2], Bl[2];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        Bh[rr >> 3][rr & 7] = bf16_hi(ds[rr]);
        Bl[rr >> 3][rr & 7] = bf16_lo(ds[rr]);
      }
#pragma unroll
      for (int dt = 0; dt < C::NQT; ++dt)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int off = (dt >> 1) * 128 + m * 16 * C::RC * 16;
          const s16x4 x0 = lds_transpose_read16(Kst + kt_base[0][dt & 1] + off);
          const s16x4 x1 = lds_transpose_read16(Kst + kt_base[1][dt & 1] + off);
          const s16x8 A = (s16x8){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          acc[dt] = mfma_bf16_32x32x16(A, Bh[m], acc[dt]);
          acc[dt] = mfma_bf16_32x32x16(A, Bl[m], acc[dt]);
        }
    } else {
      // ---- ds (times sm_scale) and p as fp16 tiles [head][key]; wave f = 0 writes ds, f = 1 p
      uint8_t* tile = tiles + hf * C::TILE_BYTES + (g * 32 + l32) * C::TILE_STRIDE;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {  // keys 8 qd + 4 lh + 0..3
        s16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = f32_to_f16_bits(hf == 0 ? ds[4 * qd + e] * sm_scale : pr[4 * qd + e]);
        *reinterpret_cast<s16x4*>(tile + (8 * qd + 4 * lh) * 2) = v;
      }
      __syncthreads();  // both tiles complete
      // A operands (16 keys x 32 heads): two transposing reads of head rows 32 kk + 8 grp + {0..3},
      // {4..7}, key columns 16 kt + 4 (a % 4)
      const int a = lane & 15, grp = lane >> 4;
      auto afrag = [&](int which, int kt, int kk) {
        s16x8 r;
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
          const int row = 32 * kk + 8 * grp + 4 * hlf + (a >> 2);
          const s16x4 w = lds_transpose_read16(tiles + which * C::TILE_BYTES + row * C::TILE_STRIDE +
                                                (16 * kt + 4 * (a & 3)) * 2);
#pragma unroll
          for (int e = 0; e < 4; ++e) r[4 * hlf + e] = w[e];
        }
        return r;
      };
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const s16x8 Ad0 = afrag(0, kt, 0), Ad1 = afrag(0, kt, 1);
        const s16x8 Ap0 = afrag(1, kt, 0), Ap1 = afrag(1, kt, 1);
        // accumulator lane l: column l % 16, keys 16 kt + 4 (l / 16) + r
        int32_t pk[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pk[r] = phys[blk * BWM_KB + 16 * kt + 4 * grp + r];
#pragma unroll
        for (int ct = 0; ct < C::NKC; ++ct) {
          v4f c = mfma_f16_16x16x32(Ad0, QT[ct][0], (v4f){0.f, 0.f, 0.f, 0.f});
          c = mfma_f16_16x16x32(Ad1, QT[ct][1], c);
          const int col = wave * C::KC + ct * 16 + a;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (pk[r] >= 0) atomicAdd(dkv + (int64_t)pk[r] * C::DQK + col, c[r]);
        }
#pragma unroll
        for (int ct = 0; ct < C::NVC; ++ct) {
          v4f c = mfma_f16_16x16x32(Ap0, GT[ct][0], (v4f){0.f, 0.f, 0.f, 0.f});
          c = mfma_f16_16x16x32(Ap1, GT[ct][1], c);
          const int col = wave * C::VC + ct * 16 + a;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (pk[r] >= 0) atomicAdd(dkv + (int64_t)pk[r] * C::DQK + col, c[r]);
        }
      }
    }
  }
  if (pass == 0) {
    // D of this lane's head: its 16 keys plus the other lane half's (both waves of a pair hold
    // the same sums)
    dlt = dsum + __shfl_xor(dsum, 32);
    if (hv && hf == 0 && lh == 0) delta[t * H + head] = dlt;
  }
  }
  vm_wait<0>();

  if constexpr (!DKV) {
    if (!hv) return;
    // accumulator element r of tile dt: column hf DH + 32 dt + 8 (r / 4) + 4 lh + r % 4 of the head
    float* drow = dq + (t * H + head) * (int64_t)C::DQK + hf * C::DH;
#pragma unroll
    for (int dt = 0; dt < C::NQT; ++dt)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *reinterpret_cast<v4f*>(drow + dt * 32 + 8 * qd + 4 * lh) =
            (v4f){acc[dt][4 * qd], acc[dt][4 * qd + 1], acc[dt][4 * qd + 2], acc[dt][4 * qd + 3]} * sm_scale;
  }
}

// ---------------------------------------------------------------------------------------------
bool mla_bwd_supported(int32_t D_qk, int32_t D_v, int32_t H, int32_t k) {
  return D_qk == BwmCfg::DQK && D_v == BwmCfg::DV && H >= 1 && H <= 128 && k >= 1 && k <= BWM_MAX_K;
}

size_t mla_bwd_workspace_bytes(int64_t T, int32_t H) { return (size_t)T * H * sizeof(float); }

hipError_t launch_sparse_mla_bwd(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const float* lse,
                                 const uint16_t* dout, int64_t T, int64_t S, int32_t H, int32_t k, int64_t q_start,
                                 float sm_scale, float* dq, float* dkv, void* workspace, hipStream_t stream) {
  using C = BwmCfg;
  const int64_t n4 = S * C::DQK / 4;
  hipError_t e = launch("fill_zero_kernel", fill_zero_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0,
                        stream, dkv, n4);
  if (e != hipSuccess || T <= 0) return e;
  float* delta = reinterpret_cast<float*>(workspace);
  for (const void* kern : {(const void*)sparse_mla_bwd_kernel<false>, (const void*)sparse_mla_bwd_kernel<true>}) {
    e = set_max_dynamic_lds(kern);
    if (e != hipSuccess) return e;
  }
  const float scale_log2 = sm_scale * BWM_LOG2E;
  const dim3 grid((unsigned)T, (unsigned)((H + BWM_HEADS - 1) / BWM_HEADS));
  e = launch("sparse_mla_bwd_kernel<dq>", sparse_mla_bwd_kernel<false>, grid, dim3(BW_THREADS), bwm_smem_bytes(false),
             stream, q, kv, idx, lse, delta, dout, S, q_start, H, k, scale_log2, sm_scale, dq, dkv);
  if (e != hipSuccess) return e;
  return launch("sparse_mla_bwd_kernel<dkv>", sparse_mla_bwd_kernel<true>, grid, dim3(BW_THREADS),
                bwm_smem_bytes(true), stream, q, kv, idx, lse, delta, dout, S, q_start, H, k, scale_log2, sm_scale,
                dq, dkv);
}

}  // namespace dsa
