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
// Kernels, per chunk of up to 512 query rows (the chunk's buffers live in the caller's workspace):
//  - sparse_mla_bwd_dq_kernel: H heads in halves of 64 per workgroup, 4 waves, one per SIMD; wave
//    (g, f) serves the 32 heads of group g and contraction half f, as in the forward.  Per block of
//    32 gathered rows (DMA into LDS, XOR-swizzled as the forward), partial S^T = K Q^T and
//    dP^T = V G^T over the wave's half (bf16 32x32x16 MFMA), summed with the partner's through LDS;
//    p in fp32 on the accumulator layout (lane = head).  Pass 0 sums p dp into D; pass 1 forms
//    ds = p (dp - D) and dQ^T += K^T dS^T with K^T from transposing LDS reads of the gathered rows
//    and ds split into a bf16 high part and a bf16 remainder (two MFMAs; 16 significant bits),
//    accumulated over all blocks in registers and written once.  Pass 1 also writes sm_scale ds
//    and p as fp16 [head][entry] tiles of the chunk (the dKV kernels' input).
//  - mla_bwd_pos_kernel: per chunk, the first entry of each (key, row) pair (atomic minimum into
//    a key-major map, so repeated keys of a list resolve to their first entry).
//  - mla_bwd_dkv_contrib_kernel: one workgroup per row, all heads.  Q^T and G^T fragments (16
//    columns x 32 heads, fp16) of the wave's 144 columns stay in registers; per block, the ds and p
//    tiles are read from the chunk buffer into LDS and every entry's 576-wide dKV contribution
//    sum_h sm_scale ds q_h + p g_h (fp16 16x16x32 MFMA, accumulator lane = four columns of one
//    entry) is stored to its own slot with plain 16-byte stores.  Entries repeating an earlier key
//    of the list are then added into that key's first slot, in entry order.
//  - mla_bwd_dkv_reduce_kernel: one wave per key, adding the slots the map names in row order and
//    the sum into dkv.  Every sum has a fixed order, so dkv is deterministic.
#include "dsa_internal.hpp"

namespace dsa {

constexpr int BW_THREADS = 256;     // 4 waves
constexpr int BWM_KB = 32;          // gathered rows per block
constexpr int BWM_HEADS = 64;       // heads per dq workgroup
constexpr int BWM_MAX_K = 2048;
constexpr int BWM_CHUNK_ROWS = 512; // query rows per chunk of the dKV buffers
constexpr int32_t BWM_NO_ENTRY = INT32_MAX;
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
  // dKV contribution kernel: wave w owns columns [144 w, 144 w + 144): 9 tiles of 16 of dK, and the
  // dV tiles among them (columns below 512: 9, 9, 9, 5)
  static constexpr int CW = DQK / 4, NCT = CW / 16;       // 144, 9
  static constexpr int STAGE_Q_STRIDE = DQK * 2 + 16;     // row stride of the staged Q / G (bf16)
  static constexpr int STAGE_BYTES = 128 * STAGE_Q_STRIDE;
  static_assert(DMA_INSTR % 4 == 0 && 2 * DMA_PW <= WAVE, "gather transfers split evenly over 4 waves");
  // chunk XOR of gathered row r (the forward's swizzle: conflict-free fragment and transposing reads)
  static __host__ __device__ __forceinline__ constexpr int swz(int r) {
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
  static __device__ __forceinline__ int slot(int r, int c) { return r * RC + (c ^ swz(r)); }
};

constexpr size_t bwm_dq_smem_bytes() {
  using C = BwmCfg;
  return 2 * (size_t)C::K_BYTES + C::SX_BYTES + (size_t)(BWM_MAX_K + 4 + BWM_MAX_K / BWM_KB) * 4 +
         4 * BWM_KB * 32 * 2;  // + the waves' transpose tiles
}
constexpr size_t bwm_contrib_smem_bytes() {
  return (size_t)BwmCfg::STAGE_BYTES + (BWM_MAX_K / BWM_KB) * 4 + (size_t)BWM_MAX_K * 4;
}
static_assert(bwm_dq_smem_bytes() <= kLdsPerWorkgroupMax && bwm_contrib_smem_bytes() <= kLdsPerWorkgroupMax,
              "LDS budget");

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) reinterpret_cast<v4f*>(p)[i] = (v4f){0.f, 0.f, 0.f, 0.f};
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

__device__ __forceinline__ short f32_to_f16_bits(float x) { return __builtin_bit_cast(short, (_Float16)x); }

// bf16 round to nearest even of x (high part) and of the remainder x - high (16 significant bits
// together), as 16-bit patterns
__device__ __forceinline__ short bf16_hi(float x) { return (short)f32_to_bf16(x); }
__device__ __forceinline__ short bf16_lo(float x) {
  return (short)f32_to_bf16(x - __uint_as_float((uint32_t)f32_to_bf16(x) << 16));
}

// Validity words of a list (bit e of word b: entry 32 b + e names a key in [0, n)), into LDS.
__device__ __forceinline__ void list_validity(const int32_t* __restrict__ list, int32_t k, int64_t n,
                                              uint32_t* vmask, int wave, int lane) {
  for (int base = wave * WAVE; base < (k + 63) / 64 * 64; base += 4 * WAVE) {
    const int i = base + lane;
    bool v = false;
    if (i < k) {
      const int32_t li = list[i];
      v = li >= 0 && li < n;
    }
    const uint64_t bits = __ballot(v);
    if (lane == 0) {
      vmask[base / 32] = (uint32_t)bits;
      if (base + 32 < k) vmask[base / 32 + 1] = (uint32_t)(bits >> 32);
    }
  }
}

// dq of rows t0 .. t0 + R - 1 (latest first) and the chunk's fp16 ds / p tiles
// dsp [R][2][kpad][Hp] (which 0: sm_scale ds, 1: p; heads past H and invalid entries hold 0).
__global__ __launch_bounds__(BW_THREADS, 1) void sparse_mla_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    const float* __restrict__ lse, const uint16_t* __restrict__ dout, int64_t S, int64_t q_start, int32_t H,
    int32_t k, float scale_log2, float sm_scale, float* __restrict__ dq, int64_t t0, int32_t Hp, int32_t kpad,
    uint16_t* __restrict__ dsp) {
  using C = BwmCfg;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* Kbuf = smem;                                            // [2][SLOTS] x 16 B
  v4f* Sx = reinterpret_cast<v4f*>(smem + 2 * C::K_BYTES);          // [wave][S, dP][4][64] x v4f
  int32_t* phys = reinterpret_cast<int32_t*>(smem + 2 * C::K_BYTES + C::SX_BYTES);
  uint32_t* vmask = reinterpret_cast<uint32_t*>(phys + BWM_MAX_K + 4);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 1, hf = wave & 1;
  const int l32 = lane & 31, lh = lane >> 5;
  // this wave's [32 entries][32 heads] fp16 transpose tile
  uint16_t* ttile = reinterpret_cast<uint16_t*>(vmask + BWM_MAX_K / BWM_KB) + wave * BWM_KB * 32;
  const int r = (int)gridDim.x - 1 - (int)blockIdx.x;  // latest rows first (longest lists)
  const int64_t t = t0 + r;
  const int h0 = blockIdx.y * BWM_HEADS;
  const int head = h0 + g * 32 + l32;
  const bool hv = head < H;
  const int64_t n = min(S, q_start + t + 1);

  // ---- index list: physical rows (-1: skipped entry) and per-block validity words
  for (int i = tid; i < k; i += BW_THREADS) {
    const int32_t li = idx[t * k + i];
    phys[i] = (li >= 0 && li < n) ? li : -1;
  }
  list_validity(idx + t * k, k, n, vmask, wave, lane);

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
  float dlt = 0.f;  // D of this lane's head, summed in pass 0
  __syncthreads();  // list and masks done before the gathers overwrite the LDS

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
        const int rr = 4 * (grp >> 1) + (a >> 2) + 8 * j;
        const int par = odd ^ hf;
        const int c = 32 * hf + 8 * (hf & odd) + ((4 * par + low) ^ C::swz(rr));
        kt_base[j][odd] = (rr * C::RC + c) * 16 + (a & 1) * 8;
      }
  }

  v16f acc[C::NQT];
#pragma unroll
  for (int dt = 0; dt < C::NQT; ++dt) acc[dt] = (v16f){};

  const int nblk_all = (k + BWM_KB - 1) / BWM_KB;
  const uint64_t live = __ballot(lane < nblk_all && vmask[lane] != 0u);
  const int nblk = live ? 64 - __clzll(live) : 0;
  const v4f* Sx_peer = Sx + ((wave ^ 1) * 2) * 4 * WAVE + lane;
  v4f* Sx_mine = Sx + (wave * 2) * 4 * WAVE + lane;
  // this wave's ds (f = 0) or p (f = 1) tile: lane L stores heads 16 (L % 2) .. + 15 of the wave's
  // group, entry L / 2 of the block
  uint16_t* tile_dst = dsp + ((int64_t)(r * 2 + hf) * kpad + (lane >> 1)) * Hp + h0 + g * 32 + 16 * (lane & 1);

  // the blocks are walked twice (pass 0: D; pass 1: dQ and the tiles)
  for (int pass = 0; pass < 2; ++pass) {
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

    // ---- the fp16 tile of this wave (entry 8 (rr / 4) + 4 lh + rr % 4 of the block, head l32),
    // transposed through LDS to head-contiguous rows and stored 16 bytes per lane twice
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
      ttile[(8 * (rr >> 2) + 4 * lh + (rr & 3)) * 32 + l32] =
          (uint16_t)f32_to_f16_bits(hf == 0 ? ds[rr] * sm_scale : pr[rr]);
    {
      const v4i* src = reinterpret_cast<const v4i*>(ttile + (lane >> 1) * 32 + 16 * (lane & 1));
      const v4i w0 = src[0], w1 = src[1];
      v4i* dst = reinterpret_cast<v4i*>(tile_dst + (int64_t)blk * BWM_KB * Hp);
      dst[0] = w0;
      dst[1] = w1;
    }

    // ---- dQ^T[d][head] += K^T[d][key] dS^T[key][head]: B = ds (hi, lo) for key steps m = 0, 1
    s16x8 Bh[2], Bl[2];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      Bh[rr >> 3][rr & 7] = bf16_hi(ds[rr]);
      Bl[rr >> 3][rr & 7] = bf16_lo(ds[rr]);
    }
    // A fragment of step i = (tile dt, key step m) = (i / 2, i % 2), read LA - 1 steps ahead so that
    // each pair of products waits for its own fragment only
    auto afrag = [&](int i) {
      const int dt = i >> 1, m = i & 1;
      const int off = (dt >> 1) * 128 + m * 16 * C::RC * 16;
      const s16x4 x0 = lds_transpose_read16(Kst + kt_base[0][dt & 1] + off);
      const s16x4 x1 = lds_transpose_read16(Kst + kt_base[1][dt & 1] + off);
      return (s16x8){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    };
    constexpr int NSTEP = 2 * C::NQT, LA = 3;
    s16x8 Af[LA];
#pragma unroll
    for (int i = 0; i < LA - 1; ++i) Af[i] = afrag(i);
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
      if (i + LA - 1 < NSTEP) Af[(i + LA - 1) % LA] = afrag(i + LA - 1);
      __builtin_amdgcn_sched_barrier(0);
      const int dt = i >> 1, m = i & 1;
      acc[dt] = mfma_bf16_32x32x16(Af[i % LA], Bh[m], acc[dt]);
      acc[dt] = mfma_bf16_32x32x16(Af[i % LA], Bl[m], acc[dt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (pass == 0) {
    // D of this lane's head: its 16 keys plus the other lane half's (both waves of a pair hold
    // the same sums)
    dlt = dsum + __shfl_xor(dsum, 32);
  }
  }
  vm_wait<0>();

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

// First entry of each (key, row) of the chunk: pos [keys][Rs] (BWM_NO_ENTRY where no entry).
__global__ __launch_bounds__(256) void mla_bwd_pos_kernel(const int32_t* __restrict__ idx, int64_t t0, int32_t Rs,
                                                          int64_t S, int64_t q_start, int32_t k,
                                                          int32_t* __restrict__ pos) {
  const int r = blockIdx.x;
  const int64_t t = t0 + r;
  const int64_t n = min(S, q_start + t + 1);
  for (int i = threadIdx.x; i < k; i += 256) {
    const int32_t s = idx[t * k + i];
    if (s >= 0 && s < n) atomicMin(pos + (int64_t)s * Rs + r, i);
  }
}

// The dKV contribution of every entry of row t0 + blockIdx.x: contrib [Rs][kpad][576] f32.
template <int NHS>  // 32-head steps of the contraction (Hp / 32)
__global__ __launch_bounds__(BW_THREADS, 1) void mla_bwd_dkv_contrib_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout, const int32_t* __restrict__ idx,
    const uint16_t* __restrict__ dsp, const int32_t* __restrict__ pos, int64_t t0, int32_t Rs, int64_t S,
    int64_t q_start, int32_t H, int32_t k, int32_t kpad, float* __restrict__ contrib) {
  using C = BwmCfg;
  constexpr int HP = NHS * 32;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* stage = smem;  // Q / G staging
  uint32_t* vmask = reinterpret_cast<uint32_t*>(smem + C::STAGE_BYTES);
  int32_t* prim = reinterpret_cast<int32_t*>(vmask + BWM_MAX_K / BWM_KB);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int a = lane & 15, grp = lane >> 4;
  const int r = blockIdx.x;
  const int64_t t = t0 + r;
  const int64_t n = min(S, q_start + t + 1);

  // ---- each valid entry's first entry of its key (itself unless the key repeats), validity words
  int dup = 0;
  for (int i = tid; i < k; i += BW_THREADS) {
    const int32_t s = idx[t * k + i];
    int32_t first = -1;
    if (s >= 0 && s < n) {
      first = pos[(int64_t)s * Rs + r];
      dup |= first != i;
    }
    prim[i] = first;
  }
  list_validity(idx + t * k, k, n, vmask, wave, lane);

  // ---- A operands of the head contraction: Q^T and G^T fragments (16 columns x 32 heads; lane =
  // column, eight heads per lane group), staged through LDS and converted bf16 -> fp16 (exact for
  // |x| in [2^-14, 65504])
  auto stage_rows = [&](const uint16_t* src, int width) {
    // rows 0 .. HP - 1 of [t][h][width] into LDS, row stride STAGE_Q_STRIDE (zeros past H)
    const int chunks = width / 8;
    for (int p = tid; p < HP * chunks; p += BW_THREADS) {
      const int h = p / chunks, c = p % chunks;
      v4i v = {0, 0, 0, 0};
      if (h < H) v = *reinterpret_cast<const v4i*>(src + (t * H + h) * (int64_t)width + c * 8);
      *reinterpret_cast<v4i*>(stage + h * C::STAGE_Q_STRIDE + c * 16) = v;
    }
  };
  // fragment (columns col0 .. col0 + 15, heads 32 kk .. 32 kk + 31): two transposing reads of rows
  // 32 kk + 8 grp + {0..3}, {4..7}, columns col0 + 4 (a % 4)
  auto frag = [&](int col0, int kk) {
    s16x8 v;
#pragma unroll
    for (int hlf = 0; hlf < 2; ++hlf) {
      const int row = 32 * kk + 8 * grp + 4 * hlf + (a >> 2);
      const s16x4 w = lds_transpose_read16(stage + row * C::STAGE_Q_STRIDE + (col0 + 4 * (a & 3)) * 2);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * hlf + e] = f32_to_f16_bits(bf16_to_f32((uint16_t)w[e]));
    }
    return v;
  };
  const int col_w = wave * C::CW;
  const int nv = wave < 3 ? C::NCT : (C::DV - 3 * C::CW) / 16;  // dV tiles among the wave's columns
  s16x8 QT[C::NCT][NHS], GT[C::NCT][NHS];
  stage_rows(q, C::DQK);
  __syncthreads();
#pragma unroll
  for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
    for (int kk = 0; kk < NHS; ++kk) QT[ct][kk] = frag(col_w + ct * 16, kk);
  __syncthreads();
  stage_rows(dout, C::DV);
  __syncthreads();
#pragma unroll
  for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
    for (int kk = 0; kk < NHS; ++kk)
      GT[ct][kk] = ct < nv ? frag(col_w + ct * 16, kk) : (s16x8){0, 0, 0, 0, 0, 0, 0, 0};
  const bool has_dup = __syncthreads_or(dup);

  // B operands: (entries 16 kt .. + 15) x (heads 32 kk .. + 31) of tile `which`: lane l reads the
  // eight heads 32 kk + 8 (l / 16) .. + 7 of entry 16 kt + l % 16, one 16-byte load
  const uint16_t* tiles_g = dsp + (int64_t)r * 2 * kpad * HP + (int64_t)a * HP + 8 * grp;
  auto load_frags = [&](int blk, s16x8 (&F)[2][2][NHS]) {
#pragma unroll
    for (int which = 0; which < 2; ++which)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int kk = 0; kk < NHS; ++kk)
          F[which][kt][kk] = *reinterpret_cast<const s16x8*>(
              tiles_g + ((int64_t)which * kpad + blk * BWM_KB + 16 * kt) * HP + 32 * kk);
  };
  const int nblk = (k + BWM_KB - 1) / BWM_KB;
  // live blocks (at least one valid entry) in order; the rest contribute nothing
  auto next_live = [&](int b) {
    while (b < nblk && vmask[b] == 0u) ++b;
    return b;
  };
  s16x8 F[2][2][NHS];
  int blk = next_live(0);
  if (blk < nblk) load_frags(blk, F);
  while (blk < nblk) {
    s16x8 cur[2][2][NHS];
#pragma unroll
    for (int which = 0; which < 2; ++which)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int kk = 0; kk < NHS; ++kk) cur[which][kt][kk] = F[which][kt][kk];
    const int nxt = next_live(blk + 1);
    if (nxt < nblk) load_frags(nxt, F);  // in flight during this block's MFMAs and stores
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      // accumulator lane l: columns 4 (l / 16) + 0..3 of the tile, entry 16 kt + l % 16
      float* dst = contrib + ((int64_t)r * kpad + blk * BWM_KB + 16 * kt + a) * C::DQK + col_w + 4 * grp;
#pragma unroll
      for (int ct = 0; ct < C::NCT; ++ct) {
        v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NHS; ++kk) c = mfma_f16_16x16x32(QT[ct][kk], cur[0][kt][kk], c);
        if (ct < nv) {
#pragma unroll
          for (int kk = 0; kk < NHS; ++kk) c = mfma_f16_16x16x32(GT[ct][kk], cur[1][kt][kk], c);
        }
        *reinterpret_cast<v4f*>(dst + ct * 16) = c;
      }
    }
    blk = nxt;
  }

  if (has_dup) {
    // entries repeating an earlier key of the list: added into the key's first slot in entry
    // order (agent-scope accesses: the slots were stored by other waves)
    __threadfence();
    __syncthreads();
    for (int i = 0; i < k; ++i) {
      const int32_t j = prim[i];
      if (j < 0 || j == i) continue;  // workgroup-uniform
      if (tid < C::DQK / 4) {
        float* dj = contrib + ((int64_t)r * kpad + j) * C::DQK + 4 * tid;
        const float* di = contrib + ((int64_t)r * kpad + i) * C::DQK + 4 * tid;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = __hip_atomic_load(dj + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const float y = __hip_atomic_load(di + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(dj + e, x + y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}

// dkv[s] += the slots the map names for key s, in row order (one wave per key; lane c holds the
// 16-byte column chunks c, c + 64 and, below 16, c + 128).  The slots are read once: streaming loads.
__global__ __launch_bounds__(256) void mla_bwd_dkv_reduce_kernel(const int32_t* __restrict__ pos, int32_t Rs,
                                                                 int32_t Rc, const float* __restrict__ contrib,
                                                                 int32_t kpad, int64_t nkeys, float* __restrict__ dkv) {
  constexpr int NC = BwmCfg::DQK / 4;  // 144 chunks per row
  const int lane = threadIdx.x & 63;
  const int64_t s = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= nkeys) return;
  const bool third = lane + 128 < NC;
  const int32_t* ps = pos + s * Rs;
  const v4f* cv = reinterpret_cast<const v4f*>(contrib);
  v4f a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0;
  // the key's map entries of every row of the chunk, all requested at once
  constexpr int NJ = BWM_CHUNK_ROWS / WAVE;
  int32_t v[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) v[j] = j * WAVE + lane < Rc ? ps[j * WAVE + lane] : BWM_NO_ENTRY;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    uint64_t m = __ballot(v[j] != BWM_NO_ENTRY);
    while (m) {
      // up to four slots in flight, added in row order
      int64_t off[4];
      int cnt = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        off[u] = 0;
        if (m) {
          const int b = __builtin_ctzll(m);
          m &= m - 1;
          const int32_t i = __shfl(v[j], b);
          off[u] = ((int64_t)(j * WAVE + b) * kpad + i) * NC;
          cnt = u + 1;
        }
      }
      v4f x0[4], x1[4], x2[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (u < cnt) {
          x0[u] = __builtin_nontemporal_load(cv + off[u] + lane);
          x1[u] = __builtin_nontemporal_load(cv + off[u] + 64 + lane);
          x2[u] = third ? __builtin_nontemporal_load(cv + off[u] + 128 + lane) : a2;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (u < cnt) {
          a0 += x0[u];
          a1 += x1[u];
          if (third) a2 += x2[u];
        }
      }
    }
  }
  v4f* d = reinterpret_cast<v4f*>(dkv + s * BwmCfg::DQK);
  d[lane] += a0;
  d[lane + 64] += a1;
  if (third) d[lane + 128] += a2;
}

// ---------------------------------------------------------------------------------------------
bool mla_bwd_supported(int32_t D_qk, int32_t D_v, int32_t H, int32_t k) {
  return D_qk == BwmCfg::DQK && D_v == BwmCfg::DV && H >= 1 && H <= 128 && k >= 1 && k <= BWM_MAX_K;
}

namespace {
struct BwmLayout {
  int32_t Rs, Hp, kpad;
  size_t dsp, contrib, pos, total;  // byte offsets and size
};
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
BwmLayout bwm_layout(int64_t T, int64_t S, int32_t H, int32_t k) {
  BwmLayout L{};
  L.Rs = (int32_t)std::min<int64_t>(T, BWM_CHUNK_ROWS);
  L.Hp = H <= 64 ? 64 : 128;
  L.kpad = (k + BWM_KB - 1) / BWM_KB * BWM_KB;
  L.dsp = 0;
  L.contrib = align256((size_t)L.Rs * 2 * L.Hp * L.kpad * sizeof(uint16_t));
  L.pos = L.contrib + align256((size_t)L.Rs * L.kpad * BwmCfg::DQK * sizeof(float));
  L.total = L.pos + align256((size_t)S * L.Rs * sizeof(int32_t));
  return L;
}
}  // namespace

size_t mla_bwd_workspace_bytes(int64_t T, int64_t S, int32_t H, int32_t k) {
  if (T <= 0 || S <= 0 || H <= 0 || k <= 0) return 0;
  return bwm_layout(T, S, H, k).total;
}

hipError_t launch_sparse_mla_bwd(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const float* lse,
                                 const uint16_t* dout, int64_t T, int64_t S, int32_t H, int32_t k, int64_t q_start,
                                 float sm_scale, float* dq, float* dkv, void* workspace, hipStream_t stream) {
  using C = BwmCfg;
  const int64_t n4 = S * C::DQK / 4;
  hipError_t e = launch("fill_zero_kernel", fill_zero_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0,
                        stream, dkv, n4);
  if (e != hipSuccess || T <= 0) return e;
  const BwmLayout L = bwm_layout(T, S, H, k);
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  uint16_t* dsp = reinterpret_cast<uint16_t*>(ws + L.dsp);
  float* contrib = reinterpret_cast<float*>(ws + L.contrib);
  int32_t* pos = reinterpret_cast<int32_t*>(ws + L.pos);
  const void* contrib_kernel =
      L.Hp == 64 ? (const void*)mla_bwd_dkv_contrib_kernel<2> : (const void*)mla_bwd_dkv_contrib_kernel<4>;
  for (const void* kern : {(const void*)sparse_mla_bwd_dq_kernel, contrib_kernel}) {
    e = set_max_dynamic_lds(kern);
    if (e != hipSuccess) return e;
  }
  const float scale_log2 = sm_scale * BWM_LOG2E;
  for (int64_t t0 = 0; t0 < T; t0 += L.Rs) {
    const int32_t Rc = (int32_t)std::min<int64_t>(L.Rs, T - t0);
    const int64_t nkeys = std::min<int64_t>(S, q_start + t0 + Rc);  // keys any row of the chunk can name
    e = launch("sparse_mla_bwd_dq_kernel", sparse_mla_bwd_dq_kernel, dim3((unsigned)Rc, (unsigned)(L.Hp / BWM_HEADS)),
               dim3(BW_THREADS), bwm_dq_smem_bytes(), stream, q, kv, idx, lse, dout, S, q_start, H, k, scale_log2,
               sm_scale, dq, t0, L.Hp, L.kpad, dsp);
    if (e != hipSuccess) return e;
    const int64_t npos = nkeys * L.Rs;
    e = launch("fill_i32_kernel", fill_i32_kernel, dim3((unsigned)((npos + 255) / 256)), dim3(256), 0, stream, pos,
               npos, BWM_NO_ENTRY);
    if (e != hipSuccess) return e;
    e = launch("mla_bwd_pos_kernel", mla_bwd_pos_kernel, dim3((unsigned)Rc), dim3(256), 0, stream, idx, t0, L.Rs, S,
               q_start, k, pos);
    if (e != hipSuccess) return e;
    if (L.Hp == 64)
      e = launch("mla_bwd_dkv_contrib_kernel", mla_bwd_dkv_contrib_kernel<2>, dim3((unsigned)Rc), dim3(BW_THREADS),
                 bwm_contrib_smem_bytes(), stream, q, dout, idx, dsp, pos, t0, L.Rs, S, q_start, H, k, L.kpad, contrib);
    else
      e = launch("mla_bwd_dkv_contrib_kernel", mla_bwd_dkv_contrib_kernel<4>, dim3((unsigned)Rc), dim3(BW_THREADS),
                 bwm_contrib_smem_bytes(), stream, q, dout, idx, dsp, pos, t0, L.Rs, S, q_start, H, k, L.kpad, contrib);
    if (e != hipSuccess) return e;
    e = launch("mla_bwd_dkv_reduce_kernel", mla_bwd_dkv_reduce_kernel, dim3((unsigned)((nkeys + 3) / 4)), dim3(256),
               0, stream, pos, L.Rs, Rc, contrib, L.kpad, nkeys, dkv);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dsa
