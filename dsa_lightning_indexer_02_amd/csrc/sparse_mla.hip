// Sparse MLA forward in MQA mode (DeepSeek-V3.2-Exp summary page, section "Method": the main
// attention reads only the top-k indexed latent KV rows, one row shared by every query head of
// a token; AMD MI355X article, section "Computational Efficiency": O(L k) core attention).
//
// For query row t, head h and the valid entries i of its index list (0 <= idx < n_t):
//   z_i = sm_scale * q[t,h,:] . kv[idx_i, :D_qk],  p = softmax(z),
//   out[t,h,:] = sum_i p_i kv[idx_i, :D_v],        lse[t,h] = log sum_i exp(z_i).
//
// One workgroup (4 waves) per query row (or per row and index split in decode).  Each wave owns
// 32 heads: their queries stay in registers, their fp32 output accumulators in the accumulation
// registers.  Blocks of 32 selected rows are gathered from HBM/L2 into LDS twice: row-major bf16
// for S^T = K Q^T (bf16 MFMA) and transposed fp16 for out^T = V^T P^T (fp16 MFMA).  The S^T
// accumulator layout of one 16x16 tile is exactly the B-operand layout the P^T V^T product
// needs, so probabilities never leave registers.  P is rounded to fp16 (11-bit significand)
// instead of bf16; V is converted bf16 -> fp16 once per row in LDS, exact for |v| in
// [2^-14, 65504].  Softmax is online with a lazy rescale: the running reference maximum only
// moves when a block's maximum exceeds it by more than 2^8 in probability.
#include "dsa_internal.hpp"

namespace dsa {

constexpr int MLA_WAVES = 4;
constexpr int MLA_THREADS = MLA_WAVES * WAVE;
constexpr int MLA_KB = 32;             // selected rows per block
constexpr int MLA_HEADS_PER_WAVE = 32;
constexpr float MLA_TAU = 8.0f;        // lazy-rescale threshold, log2 units

template <int DQK, int DV>
struct MlaCfg {
  static constexpr int DQK_PAD = (DQK + 31) / 32 * 32;
  static constexpr int NKS = DQK_PAD / 32;          // k-steps of the QK^T product
  static constexpr int NDT = DV / 16;               // 16-wide value tiles
  static constexpr int K_STRIDE = DQK_PAD * 2 + 16; // bytes per gathered bf16 row
  static constexpr int VT_STRIDE = MLA_KB * 2 + 8;  // bytes per fp16 value column
  static constexpr int K_BYTES = MLA_KB * K_STRIDE;
  static constexpr int VT_BYTES = DV * VT_STRIDE;
  static constexpr int NCH = DV / 8;                // 16-byte chunks of the value part
  static constexpr int MAIN_ITEMS = NCH * (MLA_KB / 4);
  static constexpr int MAIN_PER_THREAD = (MAIN_ITEMS + MLA_THREADS - 1) / MLA_THREADS;
  static constexpr int NR = (DQK - DV) / 8;         // 16-byte chunks of the rope part
  static constexpr int ROPE_ITEMS = NR * MLA_KB;
  static constexpr int ROPE_PER_THREAD = (ROPE_ITEMS + MLA_THREADS - 1) / MLA_THREADS;
  static_assert(DQK % 8 == 0 && DV % 16 == 0 && DV <= DQK, "unsupported MLA dims");
};

template <int DQK, int DV>
size_t mla_smem_bytes(int32_t keys_per_wg) {
  using C = MlaCfg<DQK, DV>;
  return (size_t)C::K_BYTES + C::VT_BYTES + (size_t)keys_per_wg * sizeof(int32_t);
}

template <int DQK, int DV>
__global__ __launch_bounds__(MLA_THREADS, 1) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ table, int64_t max_blocks, int32_t block_shift, int32_t per_row_table,
    const int32_t* __restrict__ seq_lens, int64_t S, int64_t q_start, int32_t H, int32_t k,
    float scale_log2, int32_t nsplit, int32_t keys_per_split, uint16_t* __restrict__ out,
    float* __restrict__ out_f32, float* __restrict__ lse, float* __restrict__ part_out,
    float* __restrict__ part_lse) {
  using C = MlaCfg<DQK, DV>;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* Kl = smem;                                           // [32][K_STRIDE] bf16
  uint8_t* Vt = smem + C::K_BYTES;                              // [DV][VT_STRIDE] fp16
  int32_t* phys = reinterpret_cast<int32_t*>(smem + C::K_BYTES + C::VT_BYTES);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j16 = lane & 15, g = lane >> 4;
  const int64_t r = blockIdx.y;
  const int sp = blockIdx.x;
  const int64_t n = seq_lens ? min((int64_t)max(seq_lens[r], 0), S) : min(S, q_start + r + 1);
  const int i0 = sp * keys_per_split;
  const int i1 = min(k, i0 + keys_per_split);
  const int cnt = max(i1 - i0, 0);
  const RowMap map{table ? (per_row_table ? table + r * max_blocks : table) : nullptr, block_shift};

  if (n <= 0) {  // nothing visible: out = 0, lse = -inf
    for (int p = tid; p < H * DV; p += MLA_THREADS) {
      const int64_t h = p / DV, d = p % DV;
      if (nsplit == 1) {
        out[(r * H + h) * DV + d] = 0;
        if (out_f32) out_f32[(r * H + h) * DV + d] = 0.f;
        if (lse && d == 0) lse[r * H + h] = -INFINITY;
      } else {
        part_out[((r * nsplit + sp) * (int64_t)H + h) * DV + d] = 0.f;
        if (d == 0) part_lse[(r * nsplit + sp) * (int64_t)H + h] = -INFINITY;
      }
    }
    return;
  }
  // physical rows of this workgroup's index entries (-1: skipped entry)
  for (int i = tid; i < cnt; i += MLA_THREADS) {
    const int32_t li = idx[r * k + i0 + i];
    phys[i] = (li >= 0 && li < n) ? (int32_t)map(li) : -1;
  }
  // skipped entries are gathered from a row that certainly holds finite data (the sequence's
  // first key) and masked out of the softmax, so no load needs a branch
  const int32_t safe_row = (int32_t)map(0);
  // zero the K padding columns once; they are never overwritten
  if (C::DQK_PAD > DQK) {
    for (int p = tid; p < MLA_KB * (C::DQK_PAD - DQK) / 8; p += MLA_THREADS) {
      const int row = p / ((C::DQK_PAD - DQK) / 8), c = p % ((C::DQK_PAD - DQK) / 8);
      *reinterpret_cast<v4i*>(Kl + row * C::K_STRIDE + (DQK + 8 * c) * 2) = (v4i){0, 0, 0, 0};
    }
  }

  // queries of this wave's 32 heads, as B operands of S^T = K Q^T
  const bool active = wave * MLA_HEADS_PER_WAVE < H;
  s16x8 Qf[2][C::NKS];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const int h = wave * MLA_HEADS_PER_WAVE + ht * 16 + j16;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      const int col = ks * 32 + g * 8;
      const bool ok = h < H && col < DQK;
      s16x8 v = *reinterpret_cast<const s16x8*>(q + (r * H + (ok ? h : 0)) * (int64_t)DQK + (ok ? col : 0));
      if (!ok) v = (s16x8){0, 0, 0, 0, 0, 0, 0, 0};
      Qf[ht][ks] = v;
    }
  }
  __syncthreads();

  v4f O[C::NDT][2];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) O[dt][0] = O[dt][1] = (v4f){0.f, 0.f, 0.f, 0.f};
  float mref[2] = {-INFINITY, -INFINITY};
  float lsum[2] = {0.f, 0.f};

  v4i mreg[C::MAIN_PER_THREAD][4];
  v4i rreg[C::ROPE_PER_THREAD];
  auto stage_load = [&](int blk) {
#pragma unroll
    for (int it = 0; it < C::MAIN_PER_THREAD; ++it) {
      const int p = tid + it * MLA_THREADS;
      const int c8 = p % C::NCH, kg = p / C::NCH;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int e = blk * MLA_KB + kg * 4 + kk;
        const int32_t pr = (p < C::MAIN_ITEMS && e < cnt) ? phys[e] : -1;
        mreg[it][kk] = *reinterpret_cast<const v4i*>(kv + (int64_t)(pr >= 0 ? pr : safe_row) * DQK + c8 * 8);
      }
    }
#pragma unroll
    for (int it = 0; it < C::ROPE_PER_THREAD; ++it) {
      const int p = tid + it * MLA_THREADS;
      const int row = p / (C::NR > 0 ? C::NR : 1), c = p % (C::NR > 0 ? C::NR : 1);
      const int e = blk * MLA_KB + row;
      const int32_t pr = (p < C::ROPE_ITEMS && e < cnt) ? phys[e] : -1;
      rreg[it] = *reinterpret_cast<const v4i*>(kv + (int64_t)(pr >= 0 ? pr : safe_row) * DQK + DV + c * 8);
    }
  };
  auto stage_store = [&]() {
#pragma unroll
    for (int it = 0; it < C::MAIN_PER_THREAD; ++it) {
      const int p = tid + it * MLA_THREADS;
      if (p < C::MAIN_ITEMS) {
        const int c8 = p % C::NCH, kg = p / C::NCH;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          *reinterpret_cast<v4i*>(Kl + (kg * 4 + kk) * C::K_STRIDE + c8 * 16) = mreg[it][kk];
        // transpose 4 keys x 8 columns into fp16 V^T
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          s16x4 col;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const uint32_t word = (uint32_t)mreg[it][kk][i >> 1];
            const uint16_t b = (i & 1) ? (uint16_t)(word >> 16) : (uint16_t)(word & 0xFFFFu);
            const _Float16 hv = (_Float16)bf16_to_f32(b);
            col[kk] = __builtin_bit_cast(short, hv);
          }
          *reinterpret_cast<s16x4*>(Vt + (c8 * 8 + i) * C::VT_STRIDE + kg * 8) = col;
        }
      }
    }
#pragma unroll
    for (int it = 0; it < C::ROPE_PER_THREAD; ++it) {
      const int p = tid + it * MLA_THREADS;
      if (p < C::ROPE_ITEMS) {
        const int row = p / (C::NR > 0 ? C::NR : 1), c = p % (C::NR > 0 ? C::NR : 1);
        *reinterpret_cast<v4i*>(Kl + row * C::K_STRIDE + (DV + c * 8) * 2) = rreg[it];
      }
    }
  };

  const int nblk = (cnt + MLA_KB - 1) / MLA_KB;
  if (nblk > 0) stage_load(0);
  for (int blk = 0; blk < nblk; ++blk) {
    __syncthreads();
    stage_store();
    __syncthreads();
    if (blk + 1 < nblk) stage_load(blk + 1);
    if (!active) continue;

    // ---- S^T[key][head] for 2 key tiles x 2 head tiles
    v4f s[2][2];
#pragma unroll
    for (int c = 0; c < 2; ++c) s[c][0] = s[c][1] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const s16x8 A = *reinterpret_cast<const s16x8*>(Kl + (c * 16 + j16) * C::K_STRIDE + (ks * 32 + g * 8) * 2);
        s[c][0] = mfma_bf16_16x16x32(A, Qf[0][ks], s[c][0]);
        s[c][1] = mfma_bf16_16x16x32(A, Qf[1][ks], s[c][1]);
      }
    }
    // ---- mask, scale, block maximum per head
    float x[2][2][4];
    float mb[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int e = blk * MLA_KB + c * 16 + 4 * g + rr;
        const bool valid = e < cnt && phys[e] >= 0;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          const float v = valid ? s[c][ht][rr] * scale_log2 : -INFINITY;
          x[c][ht][rr] = v;
          mb[ht] = fmaxf(mb[ht], v);
        }
      }
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      mb[ht] = fmaxf(mb[ht], __shfl_xor(mb[ht], 16));
      mb[ht] = fmaxf(mb[ht], __shfl_xor(mb[ht], 32));
    }
    const bool need0 = mb[0] > mref[0] + MLA_TAU, need1 = mb[1] > mref[1] + MLA_TAU;
    if (__any(need0 || need1)) {
      float f[2];
      f[0] = need0 ? exp2f(mref[0] - mb[0]) : 1.0f;
      f[1] = need1 ? exp2f(mref[1] - mb[1]) : 1.0f;
      if (need0) mref[0] = mb[0];
      if (need1) mref[1] = mb[1];
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) O[dt][ht] *= f[ht];
      lsum[0] *= f[0];
      lsum[1] *= f[1];
    }
    // ---- probabilities (fp16) packed as the B operand of out^T = V^T P^T
    s16x8 Bp[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float xv = x[c][ht][rr];
          const float p = xv == -INFINITY ? 0.0f : exp2f(xv - mref[ht]);
          const _Float16 ph = (_Float16)p;
          lsum[ht] += (float)ph;
          Bp[ht][c * 4 + rr] = __builtin_bit_cast(short, ph);
        }
    }
    // ---- out^T[d][head] += V^T[d][key] P^T[key][head]
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
      const uint8_t* vrow = Vt + (dt * 16 + j16) * C::VT_STRIDE;
      const s16x4 lo = *reinterpret_cast<const s16x4*>(vrow + g * 8);
      const s16x4 hi = *reinterpret_cast<const s16x4*>(vrow + 32 + g * 8);
      const s16x8 A = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      O[dt][0] = mfma_f16_16x16x32(A, Bp[0], O[dt][0]);
      O[dt][1] = mfma_f16_16x16x32(A, Bp[1], O[dt][1]);
    }
  }
  if (!active) return;

  // ---- normalise and store
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const float l = wave_sum_xor16_32(lsum[ht]);
    const int h = wave * MLA_HEADS_PER_WAVE + ht * 16 + j16;
    if (h >= H) continue;
    const float inv = l > 0.f ? 1.0f / l : 0.0f;
    const float lse_v = l > 0.f ? (mref[ht] + log2f(l)) * 0.69314718055994531f : -INFINITY;
    if (nsplit == 1) {
      uint16_t* orow = out + (r * H + h) * (int64_t)DV;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) {
        const int d = dt * 16 + 4 * g;
        v4f o = O[dt][ht] * inv;
        s16x4 ob;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) ob[rr] = (short)f32_to_bf16(o[rr]);
        *reinterpret_cast<s16x4*>(orow + d) = ob;
        if (out_f32) *reinterpret_cast<v4f*>(out_f32 + (r * H + h) * (int64_t)DV + d) = o;
      }
      if (g == 0 && lse) lse[r * H + h] = lse_v;
    } else {
      float* prow = part_out + ((r * nsplit + sp) * (int64_t)H + h) * DV;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
        *reinterpret_cast<v4f*>(prow + dt * 16 + 4 * g) = O[dt][ht] * inv;
      if (g == 0) part_lse[(r * nsplit + sp) * (int64_t)H + h] = lse_v;
    }
  }
}

// Re-reduction of split partials in fp32: out = sum_s w_s out_s / sum_s w_s, w_s = exp(lse_s - max).
template <int DV>
__global__ __launch_bounds__(256) void mla_combine_kernel(const float* __restrict__ part_out,
                                                          const float* __restrict__ part_lse, int32_t nsplit,
                                                          int32_t H, uint16_t* __restrict__ out,
                                                          float* __restrict__ out_f32, float* __restrict__ lse) {
  const int64_t r = blockIdx.x;
  for (int h = threadIdx.x / (DV / 4); h < H; h += 256 / (DV / 4)) {
    const int d = (threadIdx.x % (DV / 4)) * 4;
    float m = -INFINITY;
    for (int s = 0; s < nsplit; ++s) m = fmaxf(m, part_lse[(r * nsplit + s) * (int64_t)H + h]);
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (m != -INFINITY) {
      for (int s = 0; s < nsplit; ++s) {
        const float ls = part_lse[(r * nsplit + s) * (int64_t)H + h];
        const float wgt = ls == -INFINITY ? 0.f : expf(ls - m);
        wsum += wgt;
        const v4f v = *reinterpret_cast<const v4f*>(part_out + ((r * nsplit + s) * (int64_t)H + h) * DV + d);
        acc += wgt * v;
      }
    }
    const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
    const v4f o = acc * inv;
    s16x4 ob;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) ob[rr] = (short)f32_to_bf16(o[rr]);
    *reinterpret_cast<s16x4*>(out + (r * H + h) * (int64_t)DV + d) = ob;
    if (out_f32) *reinterpret_cast<v4f*>(out_f32 + (r * H + h) * (int64_t)DV + d) = o;
    if (d == 0 && lse) lse[r * H + h] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------------------------
template <int DQK, int DV>
static hipError_t launch_mla_t(const MlaArgs& a, hipStream_t stream) {
  const int nsplit = a.nsplit;
  const int kps = (a.k + nsplit - 1) / nsplit;
  const size_t smem = mla_smem_bytes<DQK, DV>(kps);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)sparse_mla_kernel<DQK, DV>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const float scale_log2 = a.sm_scale * 1.4426950408889634f;
  dim3 grid((unsigned)nsplit, (unsigned)a.R);
  hipLaunchKernelGGL((sparse_mla_kernel<DQK, DV>), grid, dim3(MLA_THREADS), smem, stream, a.q, a.kv,
                     a.idx, a.table, a.max_blocks, a.block_shift, a.per_row_table, a.seq_lens, a.S,
                     a.q_start, a.H, a.k, scale_log2, nsplit, kps, a.out, a.out_f32, a.lse, a.part_out,
                     a.part_lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  hipLaunchKernelGGL(mla_combine_kernel<DV>, dim3((unsigned)a.R), dim3(256), 0, stream, a.part_out,
                     a.part_lse, nsplit, a.H, a.out, a.out_f32, a.lse);
  return hipGetLastError();
}

bool mla_supported(int32_t D_qk, int32_t D_v, int32_t H, int32_t k) {
  const bool dims = (D_qk == 576 && D_v == 512) || (D_qk == 80 && D_v == 64);
  return dims && H >= 1 && H <= MLA_WAVES * MLA_HEADS_PER_WAVE && k >= 1 && k <= 8192;
}

size_t mla_smem_for(int32_t D_qk, int32_t D_v, int32_t keys_per_wg) {
  if (D_qk == 576) return mla_smem_bytes<576, 512>(keys_per_wg);
  return mla_smem_bytes<80, 64>(keys_per_wg);
}

hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t stream) {
  if (a.R <= 0) return hipSuccess;
  if (a.D_qk == 576 && a.D_v == 512) return launch_mla_t<576, 512>(a, stream);
  if (a.D_qk == 80 && a.D_v == 64) return launch_mla_t<80, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dsa
