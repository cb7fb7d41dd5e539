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

constexpr int MLA_WAVES = 8;
constexpr int MLA_THREADS = MLA_WAVES * WAVE;
constexpr int MLA_KB = 32;             // selected rows per block
constexpr int MLA_HEADS_PER_WAVE = 16;
constexpr int MLA_HT = MLA_HEADS_PER_WAVE / 16;  // 16-head MFMA tiles per wave
constexpr int MLA_STAGES = 3;          // gathered-row buffers in flight
constexpr int MLA_MAX_K = 2048;        // index entries per workgroup (LDS row list)
constexpr float MLA_HEADROOM = 15.0f;  // log2 headroom of fp16 probabilities above the reference

template <int DQK, int DV>
struct MlaCfg {
  static constexpr int DQK_PAD = (DQK + 31) / 32 * 32;
  static constexpr int NKS = DQK_PAD / 32;          // k-steps of the QK^T product
  static constexpr int NDT = DV / 16;               // 16-wide value tiles
  static constexpr int RC = DQK_PAD / 8;            // 16-byte chunks per gathered row
  static constexpr int SWZ = RC % 8 == 0 ? 8 : (RC % 4 == 0 ? 4 : 1);  // XOR swizzle span (chunks)
  static constexpr int SLOTS = MLA_KB * RC;         // 16-byte slots per stage
  static constexpr int K_BYTES = SLOTS * 16;
  static constexpr int DMA_INSTR = SLOTS / WAVE;    // wave-wide 1 KiB transfers per block
  static constexpr int DMA_MAX_PER_WAVE = (DMA_INSTR + MLA_WAVES - 1) / MLA_WAVES;
  static constexpr int VT_STRIDE = MLA_KB * 2 + 8;  // bytes per fp16 value column
  static constexpr int VT_BYTES = DV * VT_STRIDE;
  static constexpr int CONV_ITEMS = (DV / 8) * (MLA_KB / 4);  // (16-byte column chunk, 4-key group)
  static constexpr int CONV_PER_THREAD = (CONV_ITEMS + MLA_THREADS - 1) / MLA_THREADS;
  static_assert(DQK % 8 == 0 && DV % 16 == 0 && DV <= DQK, "unsupported MLA dims");
  static_assert(SLOTS % WAVE == 0, "gather slots must fill whole waves");
  // 16-byte slot of chunk c of gathered row r: rows are contiguous, chunks XOR-swizzled within
  // aligned groups of SWZ so that 8 consecutive rows at one chunk hit 8 distinct bank groups.
  static __device__ __forceinline__ int slot(int r, int c) { return r * RC + (c ^ (r & (SWZ - 1))); }
};

template <int DQK, int DV>
size_t mla_smem_bytes(int32_t keys_per_wg) {
  using C = MlaCfg<DQK, DV>;
  (void)keys_per_wg;
  return (size_t)MLA_STAGES * C::K_BYTES + C::VT_BYTES + (size_t)(MLA_MAX_K + 4 + MLA_MAX_K / MLA_KB) * sizeof(int32_t);
}

// One wave-wide global -> LDS transfer: lane l's 16 bytes at gaddr land at lds_base + 16 l.
// Issued as inline assembly so that the compiler does not serialise later LDS reads behind it;
// completion is awaited explicitly (vmcnt) before the barrier that publishes the data.
__device__ __forceinline__ void dma_16B(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(gaddr) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most n of this wave's vector-memory operations are pending (n wave-uniform, small).
__device__ __forceinline__ void wait_vmcnt_pending(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    default: wait_vmcnt<9>(); break;
  }
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
  uint8_t* Kbuf = smem;                                                  // [STAGES][SLOTS] x 16 B
  uint8_t* Vt = smem + MLA_STAGES * C::K_BYTES;                          // [DV][VT_STRIDE] fp16
  int32_t* phys = reinterpret_cast<int32_t*>(Vt + C::VT_BYTES);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
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
  // validity bit mask of every 32-entry block (bit i: entry 32 b + i is gathered and attended)
  uint32_t* vmask_lds = reinterpret_cast<uint32_t*>(phys + MLA_MAX_K + 4);
  for (int base = wave * WAVE; base < (cnt + 63) / 64 * 64; base += MLA_WAVES * WAVE) {
    const int i = base + lane;
    bool v = false;
    if (i < cnt) {
      const int32_t li = idx[r * k + i0 + i];
      v = li >= 0 && li < n;
    }
    const uint64_t bits = __ballot(v);
    if (lane == 0) {
      vmask_lds[base / 32] = (uint32_t)bits;
      if (base + 32 < cnt) vmask_lds[base / 32 + 1] = (uint32_t)(bits >> 32);
    }
  }
  // Skipped entries are gathered from a row that certainly holds finite data (the sequence's
  // first key) and masked out of the softmax.
  const int32_t safe_row = (int32_t)map(0);
  // zero the padding chunks of every stage once; the gather never writes them
  if (C::DQK_PAD > DQK) {
    for (int p = tid; p < MLA_STAGES * MLA_KB * C::RC; p += MLA_THREADS) {
      const int st = p / (MLA_KB * C::RC), rr = (p / C::RC) % MLA_KB, c = p % C::RC;
      if (c * 8 >= DQK)
        *reinterpret_cast<v4i*>(Kbuf + st * C::K_BYTES + C::slot(rr, c) * 16) = (v4i){0, 0, 0, 0};
    }
  }

  // queries of this wave's 32 heads, as B operands of S^T = K Q^T
  const bool active = wave * MLA_HEADS_PER_WAVE < H;
  s16x8 Qf[MLA_HT][C::NKS];
#pragma unroll
  for (int ht = 0; ht < MLA_HT; ++ht) {
    const int h = wave * MLA_HEADS_PER_WAVE + ht * 16 + j16;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      const int col = ks * 32 + g * 8;
      const bool ok = h < H && col < DQK;
      s16x8 v = *reinterpret_cast<const s16x8*>(q + (r * H + (ok ? h : 0)) * (int64_t)DQK + (ok ? col : 0));
      if (!ok) v = (s16x8){0, 0, 0, 0, 0, 0, 0, 0};
      asm volatile("" : "+v"(v));  // keep the queries resident: no re-load from memory per block
      Qf[ht][ks] = v;
    }
  }
  __syncthreads();

  const uint32_t kbuf_lds = lds_addr(Kbuf);
  const int my_dma = (C::DMA_INSTR - wave + MLA_WAVES - 1) / MLA_WAVES;  // this wave's transfers per block
  // Byte offset in a stage of the K fragment (step ks, key tile c) this lane reads: chunk 4 ks + g
  // of row 16 c + j16.  The swizzle XORs the low log2(SWZ) chunk bits with the row, so the offset is
  // one of two per-lane bases (by the parity of ks when SWZ is 8) plus a compile-time constant, and
  // no per-step address has to stay live.
  static_assert(C::SWZ == 8 || C::SWZ == 4 || C::SWZ == 1, "swizzle span");
  const int xr = j16 & (C::SWZ - 1);
  const int abase0 = (j16 * C::RC + (g ^ xr)) * 16;            // even ks (and every ks when SWZ <= 4)
  const int abase1 = (j16 * C::RC + ((4 + g) ^ xr)) * 16;      // odd ks when SWZ == 8
  auto afrag_off = [&](int ks, int c) -> int {
    if (C::SWZ == 8)
      return ((ks & 1) ? abase1 : abase0) + (ks >> 1) * 128 + c * 16 * C::RC * 16;
    return abase0 + ks * 64 + c * 16 * C::RC * 16;
  };
  auto gather = [&](int blk) {
    const uint32_t base = kbuf_lds + (uint32_t)((blk % MLA_STAGES) * C::K_BYTES);
    for (int i = wave; i < C::DMA_INSTR; i += MLA_WAVES) {
      const int s = i * WAVE + lane;
      const int rr = s / C::RC;
      const int c = (s % C::RC) ^ (rr & (C::SWZ - 1));
      const int e = blk * MLA_KB + rr;
      const int32_t pr = e < cnt ? phys[e] : -1;
      const uint16_t* src = kv + (int64_t)(pr >= 0 ? pr : safe_row) * DQK + c * 8;
      if (C::DQK_PAD == DQK || c * 8 < DQK) dma_16B(src, base + (uint32_t)(i * WAVE * 16));
    }
  };

  v4f O[C::NDT][MLA_HT];
  // Softmax reference: fixed at the first block holding a valid entry (per head).  Later blocks
  // may exceed it by up to 2^15 in probability, which fp16 still holds, so the accumulators are
  // never rescaled.  If any head goes further, the workgroup runs the token again with the now
  // known exact maximum as the reference (probabilities <= 1); the accumulators are only ever
  // zeroed, accumulated by MFMA and read once at the end.
  float mref[MLA_HT], mlane[MLA_HT], lsum[MLA_HT];  // mlane: this lane's running maximum
#pragma unroll
  for (int ht = 0; ht < MLA_HT; ++ht) mlane[ht] = -INFINITY;
  const int nblk = (cnt + MLA_KB - 1) / MLA_KB;
  int32_t* overflow_flag = phys + MLA_MAX_K;  // one int after the row list
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int ht = 0; ht < MLA_HT; ++ht) O[dt][ht] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ht = 0; ht < MLA_HT; ++ht) lsum[ht] = 0.f;
    if (pass) {  // exact row maximum of pass 0, reduced over the lanes holding each head
#pragma unroll
      for (int ht = 0; ht < MLA_HT; ++ht) {
        float m = mlane[ht];
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        mref[ht] = m;
      }
    } else {
#pragma unroll
      for (int ht = 0; ht < MLA_HT; ++ht) mref[ht] = INFINITY;  // unset: probabilities are 0 until a valid entry
    }
    bool have_ref = pass != 0;  // wave-uniform: every head of a wave gets its reference together
    bool overflow = false;

    if (nblk > 0) gather(0);
    if (nblk > 1) gather(1);
    for (int blk = 0; blk < nblk; ++blk) {
      const uint8_t* Kst = Kbuf + (blk % MLA_STAGES) * C::K_BYTES;
      // this wave's transfers of block blk are done once at most those of blk + 1 are pending
      if (blk + 1 < nblk)
        wait_vmcnt_pending(my_dma);
      else
        wait_vmcnt<0>();
      __syncthreads();
      if (blk + 2 < nblk) gather(blk + 2);

      // ---- fp16 V^T of this block (read from the gathered rows)
#pragma unroll
      for (int it = 0; it < C::CONV_PER_THREAD; ++it) {
        const int p = tid + it * MLA_THREADS;
        if (C::CONV_ITEMS % MLA_THREADS == 0 || p < C::CONV_ITEMS) {
          const int kg = p % (MLA_KB / 4), c8 = p / (MLA_KB / 4);
          v4i rows[4];
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) rows[kk] = *reinterpret_cast<const v4i*>(Kst + C::slot(kg * 4 + kk, c8) * 16);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            s16x4 col;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
              const uint32_t word = (uint32_t)rows[kk][i >> 1];
              const uint16_t bb = (i & 1) ? (uint16_t)(word >> 16) : (uint16_t)(word & 0xFFFFu);
              col[kk] = __builtin_bit_cast(short, (_Float16)bf16_to_f32(bb));
            }
            *reinterpret_cast<s16x4*>(Vt + (c8 * 8 + i) * C::VT_STRIDE + kg * 8) = col;
          }
        }
      }

      // ---- S^T[key][head] for 2 key tiles x 2 head tiles; the K fragments of step ks + 1 are
      // requested before the MFMAs of step ks so that LDS latency hides behind them
      v4f sc[2][MLA_HT];
      if (active) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int ht = 0; ht < MLA_HT; ++ht) sc[c][ht] = (v4f){0.f, 0.f, 0.f, 0.f};
        s16x8 Acur[2], Anext[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) Acur[c] = *reinterpret_cast<const s16x8*>(Kst + afrag_off(0, c));
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
          if (ks + 1 < C::NKS) {
#pragma unroll
            for (int c = 0; c < 2; ++c) Anext[c] = *reinterpret_cast<const s16x8*>(Kst + afrag_off(ks + 1, c));
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 LDS reads
          }
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int ht = 0; ht < MLA_HT; ++ht) sc[c][ht] = mfma_bf16_16x16x32(Acur[c], Qf[ht][ks], sc[c][ht]);
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * MLA_HT, 0);  // the step's MFMAs
          if (ks + 1 < C::NKS) {
            Acur[0] = Anext[0];
            Acur[1] = Anext[1];
          }
        }
      }
      __syncthreads();  // V^T complete
      if (!active) continue;

      // ---- scaled logits (log2 units), masked entries at -inf
      const uint32_t vm = vmask_lds[blk];
      const uint32_t vbits = ((vm >> (4 * g)) & 0xFu) | (((vm >> (16 + 4 * g)) & 0xFu) << 4);  // bit 4c + rr
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const bool valid = (vbits >> (c * 4 + rr)) & 1u;
#pragma unroll
          for (int ht = 0; ht < MLA_HT; ++ht) {
            const float v = valid ? sc[c][ht][rr] * scale_log2 : -INFINITY;
            sc[c][ht][rr] = v;
            mlane[ht] = fmaxf(mlane[ht], v);
          }
        }
      if (!have_ref && vm != 0u) {  // wave-uniform: the block mask is shared by all lanes
        // first block with a valid entry: its maximum becomes the reference
#pragma unroll
        for (int ht = 0; ht < MLA_HT; ++ht) {
          float m = mlane[ht];
          m = fmaxf(m, __shfl_xor(m, 16));
          m = fmaxf(m, __shfl_xor(m, 32));
          mref[ht] = m;
        }
        have_ref = true;
      }
      // ---- probabilities (fp16) packed as the B operand of out^T = V^T P^T
      s16x8 Bp[MLA_HT];
#pragma unroll
      for (int ht = 0; ht < MLA_HT; ++ht) {
        overflow |= mlane[ht] > mref[ht] + MLA_HEADROOM;
        float pr[8];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const float p = __builtin_amdgcn_exp2f(sc[c][ht][rr] - mref[ht]);  // exp2(-inf) = 0
            pr[c * 4 + rr] = p;
            lsum[ht] += p;
          }
#pragma unroll
        for (int i = 0; i < 8; ++i) Bp[ht][i] = __builtin_bit_cast(short, (_Float16)pr[i]);
      }
      // ---- out^T[d][head] += V^T[d][key] P^T[key][head], value fragments requested one tile ahead
      auto vfrag = [&](int dt) {
        const uint8_t* vrow = Vt + (dt * 16 + j16) * C::VT_STRIDE;
        const s16x4 lo = *reinterpret_cast<const s16x4*>(vrow + g * 8);
        const s16x4 hi = *reinterpret_cast<const s16x4*>(vrow + 32 + g * 8);
        return (s16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      };
      constexpr int VLA = 2;  // value fragments in flight
      s16x8 Vf[VLA];
#pragma unroll
      for (int i = 0; i < VLA - 1; ++i) Vf[i] = vfrag(i);
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) {
        if (dt + VLA - 1 < C::NDT) {
          Vf[(dt + VLA - 1) % VLA] = vfrag(dt + VLA - 1);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);  // LDS read (one ds_read2)
        }
#pragma unroll
        for (int ht = 0; ht < MLA_HT; ++ht) O[dt][ht] = mfma_f16_16x16x32(Vf[dt % VLA], Bp[ht], O[dt][ht]);
        __builtin_amdgcn_sched_group_barrier(0x008, MLA_HT, 1);  // the tile's MFMAs
      }
    }
    // does any wave need the exact-maximum pass?
    if (pass == 0) {
      if (tid == 0) *overflow_flag = 0;
      __syncthreads();
      if (active && __any(overflow)) *overflow_flag = 1;
      __syncthreads();
      if (*overflow_flag == 0) break;
      __syncthreads();
    }
  }
  wait_vmcnt<0>();
  if (!active) return;

  // ---- normalise and store
#pragma unroll
  for (int ht = 0; ht < MLA_HT; ++ht) {
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
  return dims && H >= 1 && H <= MLA_WAVES * MLA_HEADS_PER_WAVE && k >= 1 && k <= MLA_MAX_K;
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
