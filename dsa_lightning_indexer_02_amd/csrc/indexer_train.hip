// Training signal of the lightning indexer and its backward (DeepSeek-V3.2-Exp summary page,
// section "Method", continued pre-training: a dense warm-up stage trains only the indexer,
// against a KL-divergence target given by the main attention; the sparse stage keeps the
// indexer on its own graph).  The pages give no formula; the kernels compute:
//
//   p[t,s]  = (1/H) sum_h softmax_s( sm_scale * q[t,h,:] . kv[s,:] )     over s < n_t
//   pi[t,s] = softmax_s( I[t,s] ),   loss[t] = KL(p || pi) = sum_s p (log p - log pi)
//   dI[t,s] = pi[t,s] - p[t,s]
//
// and, for any dI, the gradients through I[t,s] = sum_j w[t,j] ReLU(z), z = q_I[t,j] . k_I[s]
// with the FP8 quantization passed straight through (q_I = qs dec(q8), k_I = ks dec(k8)):
//
//   dw[t,j] = sum_s dI[t,s] max(0, z),   dq[t,j,:] = w[t,j] sum_{s: z>0} dI[t,s] k_I[s,:],
//   dk[s,:] = sum_{t,j: z>0} dI[t,s] w[t,j] q_I[t,j,:].
//
// The target is the main attention over every visible key, so the loss kernel is a dense causal
// QK^T over the 576-wide latent rows (bf16 MFMA), run twice: pass 1 finds each head's
// log-normaliser, pass 2 sums the normalised probabilities over the heads and forms the loss and
// dI.  The backward recomputes z with bf16 MFMA from the FP8 codes (exact in bf16) and feeds the
// masked gradient tile, split into a bf16 high part and a bf16 remainder, straight from the
// accumulator layout into the next MFMA as its A operand.
#include "dsa_internal.hpp"

namespace dsa {

constexpr float KL_LOG2E = 1.4426950408889634f;
constexpr float KL_LN2 = 0.69314718055994531f;
constexpr float KL_NEG = -1.0e30f;  // start of a running maximum: finite and below every score

// ---------------------------------------------------------------------------------------
// Loss.  A workgroup takes two consecutive query rows (their causal ranges differ by one key)
// and eight waves: wave (row, group) holds the queries of 32 heads of its row in registers for
// the whole contraction (A operand of S = Q K^T, 32x32x16 MFMA), so the accumulator of a key
// block gives each lane one key and 16 heads.  Blocks of 32 latent rows are copied HBM/L2 ->
// LDS by DMA, KL_STAGES deep with one barrier per block, and shared by both rows.  The copies are
// issued by the six waves of groups 1..3; the first wave of each row, which reads the row's scores
// and writes its results, issues none, so waiting for its own loads never waits for the key stream.
// ---------------------------------------------------------------------------------------
constexpr int KL_TOK = 2;
constexpr int KL_GROUPS = 4;  // 32-head groups per row: H <= 128
constexpr int KL_WAVES = KL_TOK * KL_GROUPS;
constexpr int KL_THREADS = KL_WAVES * WAVE;
constexpr int KL_KB = 32;
constexpr int KL_STAGES = 4;
constexpr int KL_ISSUERS = KL_WAVES - KL_TOK;  // waves with grp != 0

template <int P>  // a compile-time pass number
struct PassTag {
  static constexpr int value = P;
};

template <int NKS>  // NKS 16-column contraction steps: the latent row padded to 16 NKS columns
struct KlCfg {
  static constexpr int DP = 16 * NKS;
  static constexpr int RC = DP / 8;  // 16-byte chunks per row (even)
  static constexpr int SWZ = RC % 8 == 0 ? 8 : (RC % 4 == 0 ? 4 : 2);
  // Chunk XOR of staged row r (within aligned groups of SWZ chunks).  gfx950's LDS serves a
  // 16-byte-per-lane read 16 lanes at a time over 64 four-byte banks; a 576-wide row moves the
  // bank map by half the banks, so the 16 rows of one fragment-read pass are conflict-free when
  // rows of equal parity get distinct XORs mod 8 (row bits 1-3 do that, row bits 0-2 do not).
  static __device__ __forceinline__ int swz(int r) { return ((((r >> 1) & 1) << 2) | ((r >> 2) & 3)) & (SWZ - 1); }
  static constexpr int SLOTS = KL_KB * RC;  // a multiple of 64
  static constexpr int K_BYTES = SLOTS * 16;
  static constexpr int DMA_INSTR = SLOTS / WAVE;
  static constexpr int RED_FLOATS = 2 * KL_TOK * KL_GROUPS * KL_KB;
  static constexpr size_t SMEM =
      (size_t)KL_STAGES * K_BYTES + (RED_FLOATS + KL_TOK * KL_GROUPS * 2) * sizeof(float);
};

// Running log-sum-exp in log2 units: l = sum 2^(v - m).  v = -inf adds nothing.
__device__ __forceinline__ void lse_push(float& m, float& l, float v) {
  const float d = v - m;
  const float e = __builtin_amdgcn_exp2f(-fabsf(d));
  l = d > 0.f ? fmaf(l, e, 1.0f) : l + e;
  m = fmaxf(m, v);
}
__device__ __forceinline__ void lse_merge(float& m, float& l, float mo, float lo) {
  const float mn = fmaxf(m, mo);
  l = l * __builtin_amdgcn_exp2f(m - mn) + lo * __builtin_amdgcn_exp2f(mo - mn);
  m = mn;
}

template <int NKS>
__global__ __launch_bounds__(KL_THREADS, 1) void indexer_kl_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, int64_t T, int64_t S, int32_t H,
    int32_t D, float scale_log2, int64_t q_start, const float* logits, int64_t ld, float* dlogits,
    float* __restrict__ loss) {
  using C = KlCfg<NKS>;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* Kbuf = smem;                                                   // [STAGES][SLOTS] x 16 B
  float* red = reinterpret_cast<float*>(smem + KL_STAGES * C::K_BYTES);  // [2][TOK][GROUPS][KB]
  float* rowstat = red + C::RED_FLOATS;                                   // [TOK][GROUPS][2]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tok = wave / KL_GROUPS, grp = wave % KL_GROUPS;
  const int l32 = lane & 31, lh = lane >> 5;
  const int64_t pair = (int64_t)gridDim.x - 1 - blockIdx.x;  // latest rows (most keys) first
  const int64_t t = pair * KL_TOK + tok;
  const bool row_ok = t < T;
  const int64_t n = row_ok ? min(S, q_start + t + 1) : 0;
  const int64_t n_max = min(S, q_start + min(pair * KL_TOK + KL_TOK, T));
  const int nblk = (int)((n_max + KL_KB - 1) / KL_KB);
  const int ngrp = (H + 31) / 32;
  const bool active = row_ok && grp < ngrp;  // wave-uniform
  const float* Irow = logits + (row_ok ? t : 0) * ld;

  // ---- log-normaliser of the row's index scores (log2 units), over the row's four waves
  {
    float m = KL_NEG, l = 0.f;
    for (int64_t s = grp * WAVE + lane; s < n; s += KL_GROUPS * WAVE) lse_push(m, l, Irow[s] * KL_LOG2E);
    for (int o = 32; o > 0; o >>= 1) lse_merge(m, l, __shfl_xor(m, o), __shfl_xor(l, o));
    if (lane == 0) {
      rowstat[(tok * KL_GROUPS + grp) * 2] = m;
      rowstat[(tok * KL_GROUPS + grp) * 2 + 1] = l;
    }
  }
  // padding chunks of every stage are zero (the DMA never writes them)
  if (C::DP > D) {
    for (int p = tid; p < KL_STAGES * C::SLOTS; p += KL_THREADS) {
      const int sl = p % C::SLOTS, r = sl / C::RC, c = (sl % C::RC) ^ C::swz(r);
      if (c * 8 >= D) *reinterpret_cast<v4i*>(Kbuf + p * 16) = (v4i){0, 0, 0, 0};
    }
  }
  __syncthreads();
  float lse_i2;
  {
    float m = KL_NEG, l = 0.f;
    for (int g = 0; g < KL_GROUPS; ++g)
      lse_merge(m, l, rowstat[(tok * KL_GROUPS + g) * 2], rowstat[(tok * KL_GROUPS + g) * 2 + 1]);
    lse_i2 = m + __builtin_amdgcn_logf(l);
  }

  // queries of this wave's 32 heads: lane supplies head 32 grp + l32, columns 16 ks + 8 lh .. + 7
  const int head = grp * 32 + l32;
  s16x8 Qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int col = 16 * ks + 8 * lh;
    s16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (active && head < H && col < D) v = *reinterpret_cast<const s16x8*>(q + (t * H + head) * (int64_t)D + col);
    asm volatile("" : "+v"(v));  // resident for both passes
    Qf[ks] = v;
  }

  const uint32_t kbuf_lds = lds_offset(Kbuf);
  const int issuer = tok * (KL_GROUPS - 1) + grp - 1;  // 0 .. KL_ISSUERS - 1; -1: issues nothing
  const int my_dma = grp == 0 ? 0 : (C::DMA_INSTR - issuer + KL_ISSUERS - 1) / KL_ISSUERS;
  auto issue = [&](int blk) {
    if (grp == 0) return;
    const uint32_t base = kbuf_lds + (uint32_t)((blk % KL_STAGES) * C::K_BYTES);
    if (C::RC >= WAVE && D == C::DP && (int64_t)(blk + 1) * KL_KB <= S) {  // workgroup-uniform
      // a whole block of unpadded rows is one contiguous range of the cache: slot sl (row
      // sl / RC) takes source chunk (sl % RC) ^ swz(row), and as RC is a multiple of SWZ the XOR
      // only flips bits 4-6 of the byte offset: offset = 16 sl ^ 16 swz(row).  A transfer of 64
      // slots spans at most two rows when RC >= 64.
      const uint16_t* src = kv + (int64_t)blk * KL_KB * D;
      for (int i = issuer; i < C::DMA_INSTR; i += KL_ISSUERS) {
        const int first = (i * WAVE) / C::RC;                       // uniform: the transfer's first row
        const int r = first + (lane >= (first + 1) * C::RC - i * WAVE ? 1 : 0);
        const uint32_t off = ((uint32_t)(i * WAVE + lane) << 4) ^ ((uint32_t)C::swz(r) << 4);
        lds_dma_16B_sbase(src, off, base + (uint32_t)(i * WAVE * 16));
      }
      return;
    }
    for (int i = issuer; i < C::DMA_INSTR; i += KL_ISSUERS) {
      const int sl = i * WAVE + lane;
      const int r = sl / C::RC, c = (sl % C::RC) ^ C::swz(r);
      const int64_t s = min((int64_t)blk * KL_KB + r, S - 1);
      if (c * 8 < D) lds_dma_16B(kv + s * D + c * 8, base + (uint32_t)(i * WAVE * 16));
    }
  };
  // B operand of step ks: key row l32, chunk 2 ks + lh.  XOR-ing the row swizzle into the low log2(SWZ)
  // chunk bits leaves steps SWZ / 2 apart a constant distance apart.
  constexpr int KP = C::SWZ / 2;
  const int kx = C::swz(l32);
  int kbase[KP];
#pragma unroll
  for (int u = 0; u < KP; ++u) kbase[u] = (l32 * C::RC + ((2 * u + lh) ^ kx)) * 16;
  auto koff = [&](int ks) { return kbase[ks % KP] + (ks / KP) * (2 * KP * 16); };

  float st_m[16], st_l[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    st_m[r] = KL_NEG;
    st_l[r] = 0.f;
  }
  const float inv_h = 1.0f / (float)H;
  float lacc = 0.f;  // loss of the row (log2 units), lanes 0..31 of the row's first wave
  auto finalize = [&](int blk) {
    const int64_t s = (int64_t)blk * KL_KB + l32;
    if (grp == 0 && lh == 0 && s < n) {
      const float* rb = red + ((blk & 1) * KL_TOK + tok) * KL_GROUPS * KL_KB + l32;
      float ps = 0.f;
      for (int g = 0; g < ngrp; ++g) ps += rb[g * KL_KB];
      const float p = ps * inv_h;
      const float lpi2 = fmaf(Irow[s], KL_LOG2E, -lse_i2);
      const float pi = __builtin_amdgcn_exp2f(lpi2);
      // terms below 1e-30 are negligible (and log2 of a subnormal is not reliable)
      if (p > 1e-30f) lacc += p * (__builtin_amdgcn_logf(p) - lpi2);
      dlogits[t * ld + s] = pi - p;
    }
  };

  // The two passes are separate straight-line phases: the running maxima and sums of the first and
  // the normalisers of the second are never live together, which leaves the registers for the
  // fragment look-ahead (with all three sets live the compiler serialised every LDS read with its
  // MFMA).
  float lse2[16];
  auto block_loop = [&](auto pass_tag) {
    constexpr int pass = decltype(pass_tag)::value;
    for (int b = 0; b < KL_STAGES - 1 && b < nblk; ++b) issue(b);
    for (int blk = 0; blk < nblk; ++blk) {
      // this wave's copies of block blk are done once at most those of the blocks after it are
      // pending (issued in order)
      const int later = min(KL_STAGES - 2, nblk - 1 - blk);
      vm_wait_pending(later * my_dma);
      __syncthreads();  // block blk is in LDS; every wave is done with block blk - 1
      if constexpr (pass == 1) {
        if (blk > 0 && row_ok) finalize(blk - 1);
      }
      if (blk + KL_STAGES - 1 < nblk) issue(blk + KL_STAGES - 1);
      if (!active) continue;
      const uint8_t* Kst = Kbuf + (blk % KL_STAGES) * C::K_BYTES;
      v16f acc = {};
      constexpr int LA = 3;  // fragments in flight
      s16x8 Bf[LA];
#pragma unroll
      for (int i = 0; i < LA - 1; ++i) Bf[i] = *reinterpret_cast<const s16x8*>(Kst + koff(i));
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (ks + LA - 1 < NKS) Bf[(ks + LA - 1) % LA] = *reinterpret_cast<const s16x8*>(Kst + koff(ks + LA - 1));
        __builtin_amdgcn_sched_barrier(0);  // keep the look-ahead: each product waits for its own fragment only
        acc = mfma_bf16_32x32x16(Qf[ks], Bf[ks % LA], acc);
        __builtin_amdgcn_sched_barrier(0);
      }
      // lane: key blk * KB + l32; element r: head 32 grp + 8 (r / 4) + 4 lh + r % 4
      const bool valid = (int64_t)blk * KL_KB + l32 < n;
      if constexpr (pass == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) lse_push(st_m[r], st_l[r], valid ? acc[r] * scale_log2 : -INFINITY);
      } else {
        float ps = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) ps += __builtin_amdgcn_exp2f(fmaf(acc[r], scale_log2, -lse2[r]));
        ps = valid ? ps : 0.f;
        ps += __shfl_xor(ps, 32);
        if (lh == 0) red[((blk & 1) * KL_TOK + tok) * KL_GROUPS * KL_KB + grp * KL_KB + l32] = ps;
      }
    }
  };
  block_loop(PassTag<0>{});
  // each head's normaliser: merge the 32 lanes that hold it (one key column each)
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float m = st_m[r], l = st_l[r];
    for (int o = 1; o < 32; o <<= 1) lse_merge(m, l, __shfl_xor(m, o), __shfl_xor(l, o));
    const int hh = grp * 32 + 8 * (r / 4) + 4 * lh + r % 4;
    lse2[r] = (hh < H && l > 0.f) ? m + __builtin_amdgcn_logf(l) : INFINITY;
  }
  __syncthreads();  // every stage free before the second pass refills them
  block_loop(PassTag<1>{});
  vm_wait<0>();
  __syncthreads();
  if (row_ok && nblk > 0) finalize(nblk - 1);
  if (grp == 0 && row_ok) {
    float v = lh == 0 ? lacc : 0.f;
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0) loss[t] = v * KL_LN2;
  }
}

// ---------------------------------------------------------------------------------------
// Sparse stage: the same loss over the entries of each row's index list (the attention that the
// sparse step computes, averaged over the heads, against the softmax of the listed scores).  The
// per-head normaliser is the sparse forward's log-sum-exp (an input), so one pass suffices.  One
// workgroup per row: four waves of 32 heads, the listed latent rows gathered by DMA (KLS_STAGES
// deep).  The pre-pass keeps the listed scores in LDS (so the gradient may overwrite the scores),
// then zeroes the row's visible range; each entry adds pi - p to its key's gradient (repeated keys
// accumulate).
// ---------------------------------------------------------------------------------------
constexpr int KLS_WAVES = 4;
constexpr int KLS_THREADS = KLS_WAVES * WAVE;
constexpr int KLS_STAGES = 3;
constexpr int KLS_MAX_K = 2048;

template <int NKS>
constexpr size_t kls_smem_bytes() {
  return (size_t)KLS_STAGES * KlCfg<NKS>::K_BYTES + (size_t)KLS_MAX_K * 8 +
         (2 * KL_GROUPS * KL_KB + 2 * KLS_WAVES + 2 * KLS_WAVES) * sizeof(float);
}

template <int NKS>
__global__ __launch_bounds__(KLS_THREADS, 1) void indexer_kl_sparse_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx, int32_t k,
    const float* __restrict__ lse, int64_t T, int64_t S, int32_t H, int32_t D, float scale_log2, int64_t q_start,
    const float* logits, int64_t ld, float* dlogits, float* __restrict__ loss) {
  using C = KlCfg<NKS>;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* Kbuf = smem;                                                              // [STAGES][SLOTS] x 16 B
  int32_t* rows = reinterpret_cast<int32_t*>(smem + KLS_STAGES * C::K_BYTES);       // [k]: key or -1
  float* isel = reinterpret_cast<float*>(rows + KLS_MAX_K);                          // [k]: listed scores
  float* red = isel + KLS_MAX_K;                                                     // [2][GROUPS][KB]
  float* wstat = red + 2 * KL_GROUPS * KL_KB;                                        // [WAVES][2]
  int32_t* wlast = reinterpret_cast<int32_t*>(wstat + 2 * KLS_WAVES);                // [WAVES]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave, l32 = lane & 31, lh = lane >> 5;
  const int64_t t = blockIdx.x;
  const int64_t n = min(S, q_start + t + 1);
  const int ngrp = (H + 31) / 32;
  const bool active = grp < ngrp;

  // ---- the list, its scores (log2 units), the normaliser of the listed scores, the last entry
  float m = KL_NEG, l = 0.f;
  int last = 0;
  for (int i = tid; i < k; i += KLS_THREADS) {
    const int32_t li = idx[t * k + i];
    const bool v = li >= 0 && li < n;
    rows[i] = v ? li : -1;
    const float x = v ? logits[t * ld + li] * KL_LOG2E : 0.f;
    isel[i] = x;
    if (v) {
      lse_push(m, l, x);
      last = i + 1;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    lse_merge(m, l, __shfl_xor(m, o), __shfl_xor(l, o));
    last = max(last, __shfl_xor(last, o));
  }
  if (lane == 0) {
    wstat[2 * wave] = m;
    wstat[2 * wave + 1] = l;
    wlast[wave] = last;
  }
  __syncthreads();  // every listed score is in LDS before the row is overwritten
  float lse_i2;
  int k_used = 0;
  {
    float mm = KL_NEG, ll = 0.f;
    for (int w = 0; w < KLS_WAVES; ++w) {
      lse_merge(mm, ll, wstat[2 * w], wstat[2 * w + 1]);
      k_used = max(k_used, wlast[w]);
    }
    lse_i2 = mm + __builtin_amdgcn_logf(ll);
  }
  for (int64_t s = tid; s < n; s += KLS_THREADS) dlogits[t * ld + s] = 0.f;
  if (C::DP > D) {
    for (int p = tid; p < KLS_STAGES * C::SLOTS; p += KLS_THREADS) {
      const int sl = p % C::SLOTS, r = sl / C::RC, c = (sl % C::RC) ^ C::swz(r);
      if (c * 8 >= D) *reinterpret_cast<v4i*>(Kbuf + p * 16) = (v4i){0, 0, 0, 0};
    }
  }
  const int nblk = (k_used + KL_KB - 1) / KL_KB;

  const int head = grp * 32 + l32;
  s16x8 Qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int col = 16 * ks + 8 * lh;
    s16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (active && head < H && col < D) v = *reinterpret_cast<const s16x8*>(q + (t * H + head) * (int64_t)D + col);
    asm volatile("" : "+v"(v));
    Qf[ks] = v;
  }
  float lse2[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int hh = grp * 32 + 8 * (r / 4) + 4 * lh + r % 4;
    lse2[r] = (active && hh < H) ? lse[t * H + hh] * KL_LOG2E : INFINITY;
  }
  vm_wait<0>();     // the zeroing stores have completed before any entry's gradient is added
  __syncthreads();  // zeroed row and padding visible; list complete

  const uint32_t kbuf_lds = lds_offset(Kbuf);
  auto issue = [&](int blk) {
    const uint32_t base = kbuf_lds + (uint32_t)((blk % KLS_STAGES) * C::K_BYTES);
    for (int i = wave; i < C::DMA_INSTR; i += KLS_WAVES) {
      const int sl = i * WAVE + lane;
      const int r = sl / C::RC, c = (sl % C::RC) ^ C::swz(r);
      const int e = blk * KL_KB + r;
      const int32_t kr = e < k ? rows[e] : -1;
      const int64_t s = kr >= 0 ? kr : 0;  // skipped entries read row 0 (masked)
      if (c * 8 < D) lds_dma_16B(kv + s * D + c * 8, base + (uint32_t)(i * WAVE * 16));
    }
  };
  constexpr int KP = C::SWZ / 2;
  const int kx = C::swz(l32);
  int kbase[KP];
#pragma unroll
  for (int u = 0; u < KP; ++u) kbase[u] = (l32 * C::RC + ((2 * u + lh) ^ kx)) * 16;
  auto koff = [&](int ks) { return kbase[ks % KP] + (ks / KP) * (2 * KP * 16); };
  const int my_dma = (C::DMA_INSTR - wave + KLS_WAVES - 1) / KLS_WAVES;

  const float inv_h = 1.0f / (float)H;
  float lacc = 0.f;
  auto finalize = [&](int blk) {
    const int e = blk * KL_KB + l32;
    if (grp == 0 && lh == 0 && e < k) {
      const int32_t kr = rows[e];
      if (kr >= 0) {
        const float* rb = red + (blk & 1) * KL_GROUPS * KL_KB + l32;
        float ps = 0.f;
        for (int g = 0; g < ngrp; ++g) ps += rb[g * KL_KB];
        const float p = ps * inv_h;
        const float lpi2 = isel[e] - lse_i2;
        if (p > 1e-30f) lacc += p * (__builtin_amdgcn_logf(p) - lpi2);
        atomicAdd(dlogits + t * ld + kr, __builtin_amdgcn_exp2f(lpi2) - p);
      }
    }
  };

  for (int b = 0; b < KLS_STAGES - 1 && b < nblk; ++b) issue(b);
  for (int blk = 0; blk < nblk; ++blk) {
    vm_wait_pending(min(KLS_STAGES - 2, nblk - 1 - blk) * my_dma);
    __syncthreads();
    if (blk > 0) finalize(blk - 1);
    if (blk + KLS_STAGES - 1 < nblk) issue(blk + KLS_STAGES - 1);
    if (!active) continue;
    const uint8_t* Kst = Kbuf + (blk % KLS_STAGES) * C::K_BYTES;
    v16f acc = {};
    constexpr int LA = 3;
    s16x8 Bf[LA];
#pragma unroll
    for (int i = 0; i < LA - 1; ++i) Bf[i] = *reinterpret_cast<const s16x8*>(Kst + koff(i));
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (ks + LA - 1 < NKS) Bf[(ks + LA - 1) % LA] = *reinterpret_cast<const s16x8*>(Kst + koff(ks + LA - 1));
      acc = mfma_bf16_32x32x16(Qf[ks], Bf[ks % LA], acc);
    }
    const int e = blk * KL_KB + l32;
    const bool valid = e < k && rows[e] >= 0;
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) ps += __builtin_amdgcn_exp2f(fmaf(acc[r], scale_log2, -lse2[r]));
    ps = valid ? ps : 0.f;
    ps += __shfl_xor(ps, 32);
    if (lh == 0) red[(blk & 1) * KL_GROUPS * KL_KB + grp * KL_KB + l32] = ps;
  }
  vm_wait<0>();
  __syncthreads();
  if (nblk > 0) finalize(nblk - 1);
  if (grp == 0) {
    float v = lh == 0 ? lacc : 0.f;
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0) loss[t] = v * KL_LN2;
  }
}

// ---------------------------------------------------------------------------------------
// Backward.  z is recomputed from the FP8 codes converted to bf16 (exact) with the 16x16x32 bf16
// MFMA; the scales, the weights and dI enter in fp32.  A 16x16 accumulator holds, in lane l,
// column l % 16 and rows 4 (l / 16) + r: computing z with the rows that are contracted next on
// the M side puts them, four per lane for each of two 16-row sub-blocks, exactly where the A
// operand of the next 16x16x32 MFMA expects its eight contraction elements (element e of lane
// group g: sub-block e / 4, row 4 g + e % 4).  The matching B operand comes from the streamed
// rows in LDS (bf16, row-major) by transposing reads.  The gradient tile is split as
// hi = bf16 truncation, lo = bf16(g - hi), so hi + lo carries 16 significant bits.
// ---------------------------------------------------------------------------------------
constexpr int BW_ROWS = 16;   // owned rows of one 16x16 tile
constexpr int BW_BLK = 32;    // streamed rows per block (two sub-blocks of 16)
constexpr int BQ_WAVES = 8;   // dq / dw: 16 query rows x 2 heads per wave
constexpr int BQ_HPW = 2;
constexpr int BK_WAVES = 4;   // dk: 32 keys per wave, all heads
constexpr int BK_KPW = 32;
constexpr int BK_HC = 4;      // heads of a query block staged at once

template <int DI>
struct BwCfg {
  static constexpr int NDT = DI / 16;   // 16-column output tiles
  static constexpr int NZS = DI / 32;   // contraction steps of z
  static constexpr int STRIDE = DI * 2 + 16;  // bytes per bf16 row in LDS (pad: bank spread)
  static constexpr size_t BK_SMEM = (size_t)BK_HC * BW_BLK * STRIDE + BK_HC * BW_BLK * sizeof(float);
};

__device__ __forceinline__ void split_bf16(float v, short& hi, short& lo) {
  const uint32_t u = __float_as_uint(v) & 0xFFFF0000u;
  hi = (short)(u >> 16);
  lo = (short)f32_to_bf16(v - __uint_as_float(u));  // the difference is exact
}

// 16 FP8 codes of one row -> 16 bf16 values at dst (32 bytes, 16-byte aligned).
__device__ __forceinline__ void stage_row16(uint8_t* dst, v4i raw) {
  *reinterpret_cast<s16x8*>(dst) = e4m3x8_to_bf16((uint32_t)raw[0], (uint32_t)raw[1]);
  *reinterpret_cast<s16x8*>(dst + 16) = e4m3x8_to_bf16((uint32_t)raw[2], (uint32_t)raw[3]);
}

// B operand of a 16x16x32 MFMA over the 32 rows of a staged block (contraction = rows in the
// order of the A operand above), for output columns c0 .. c0 + 15.
template <int STRIDE>
__device__ __forceinline__ s16x8 block_columns(const uint8_t* blk, int lane, int c0) {
  const int g = (lane >> 4) & 3, a = lane & 15;
  const uint8_t* p = blk + (4 * g + (a >> 2)) * STRIDE + (c0 + 4 * (a & 3)) * 2;
  const s16x4 x0 = lds_transpose_read16(p), x1 = lds_transpose_read16(p + 16 * STRIDE);
  return (s16x8){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
}

// A operand of step zs of z over a staged block: sub-block sub, row l % 16, columns 32 zs + 8 g.
template <int STRIDE>
__device__ __forceinline__ s16x8 block_rows(const uint8_t* blk, int lane, int sub, int zs) {
  return *reinterpret_cast<const s16x8*>(blk + (16 * sub + (lane & 15)) * STRIDE + (32 * zs + 8 * (lane >> 4)) * 2);
}

// dq and dw: a workgroup owns 16 query rows and 16 heads (two per wave) and streams the keys.
template <int DI>
__global__ __launch_bounds__(BQ_WAVES * WAVE, 1) void indexer_bwd_q_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k8, const float* __restrict__ ks, int64_t T, int64_t S, int32_t H_I,
    int64_t q_start, const float* __restrict__ dI, int64_t ld, float* __restrict__ dq, float* __restrict__ dw) {
  using C = BwCfg<DI>;
  __shared__ __align__(16) uint8_t kt[BW_BLK * C::STRIDE];
  __shared__ float kss[BW_BLK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j16 = lane & 15, g = lane >> 4;
  const int64_t t0 = ((int64_t)gridDim.x - 1 - blockIdx.x) * BW_ROWS;  // latest rows first
  const int64_t t = t0 + j16;
  const bool t_ok = t < T;
  const int64_t n_t = t_ok ? min(S, q_start + t + 1) : 0;
  const int64_t n_max = min(S, q_start + min(t0 + BW_ROWS, T));
  const int jw = (blockIdx.y * BQ_WAVES + wave) * BQ_HPW;

  // owned queries, B operands of z^T = K Q^T: lane = query t, columns 32 zs + 8 g .. + 7
  s16x8 Qb[BQ_HPW][C::NZS];
#pragma unroll
  for (int h = 0; h < BQ_HPW; ++h)
#pragma unroll
    for (int zs = 0; zs < C::NZS; ++zs) {
      s16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (t_ok && jw + h < H_I) {
        const v2i raw = *reinterpret_cast<const v2i*>(q8 + (t * H_I + jw + h) * DI + 32 * zs + 8 * g);
        v = e4m3x8_to_bf16((uint32_t)raw[0], (uint32_t)raw[1]);
      }
      Qb[h][zs] = v;
    }
  v4f acc[BQ_HPW][C::NDT];
  float dwa[BQ_HPW];
#pragma unroll
  for (int h = 0; h < BQ_HPW; ++h) {
    dwa[h] = 0.f;
#pragma unroll
    for (int n = 0; n < C::NDT; ++n) acc[h][n] = (v4f){0.f, 0.f, 0.f, 0.f};
  }

  // The loads of key block kb + 32 (codes, scales, this lane's dI) are issued before the MFMAs of
  // block kb, into registers; staging them into LDS waits for the next barrier.  Loads are
  // unconditional with clamped addresses (rows start 16-byte aligned, ld is a multiple of 4).
  static_assert(BW_BLK * (DI / 16) <= BQ_WAVES * WAVE, "one 16-byte piece per thread");
  const int pr = tid / (DI / 16), pc = tid % (DI / 16);
  const bool stager = tid < BW_BLK * (DI / 16);
  const float* drow = dI + min(t, T - 1) * ld;
  v4i nraw = {0, 0, 0, 0};
  float nks = 0.f;
  v4f nd0, nd1;
  auto prefetch = [&](int64_t kb) {
    if (stager) nraw = *reinterpret_cast<const v4i*>(k8 + min(kb + pr, S - 1) * DI + pc * 16);
    if (tid < BW_BLK) nks = ks[min(kb + tid, S - 1)];
    nd0 = *reinterpret_cast<const v4f*>(drow + min(kb + 4 * g, ld - 4));
    nd1 = *reinterpret_cast<const v4f*>(drow + min(kb + 16 + 4 * g, ld - 4));
  };
  prefetch(0);
  for (int64_t kb = 0; kb < n_max; kb += BW_BLK) {
    __syncthreads();  // the previous block is consumed
    if (stager) stage_row16(kt + pr * C::STRIDE + pc * 32, nraw);
    if (tid < BW_BLK) kss[tid] = nks;
    const v4f d0 = nd0, d1 = nd1;
    __syncthreads();
    if (kb + BW_BLK < n_max) prefetch(kb + BW_BLK);
    // key factors dI[t,s] ks[s] of this lane's eight (row, key) pairs; 0 outside the causal range
    float u[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int kr = (e < 4 ? 0 : 16) + 4 * g + (e & 3);
      u[e] = kb + kr < n_t ? (e < 4 ? d0[e] : d1[e - 4]) * kss[kr] : 0.f;
    }
    s16x8 Ka[2][C::NZS], Kb[C::NDT];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int zs = 0; zs < C::NZS; ++zs) Ka[sub][zs] = block_rows<C::STRIDE>(kt, lane, sub, zs);
#pragma unroll
    for (int nt = 0; nt < C::NDT; ++nt) Kb[nt] = block_columns<C::STRIDE>(kt, lane, 16 * nt);
#pragma unroll
    for (int h = 0; h < BQ_HPW; ++h) {
      if (jw + h >= H_I) break;  // wave-uniform
      v4f z0 = {0.f, 0.f, 0.f, 0.f}, z1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int zs = 0; zs < C::NZS; ++zs) {
        z0 = mfma_bf16_16x16x32(Ka[0][zs], Qb[h][zs], z0);
        z1 = mfma_bf16_16x16x32(Ka[1][zs], Qb[h][zs], z1);
      }
      s16x8 ghi, glo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float zz = e < 4 ? z0[e] : z1[e - 4];
        dwa[h] = fmaf(u[e], fmaxf(zz, 0.f), dwa[h]);
        short hi, lo;
        split_bf16(zz > 0.f ? u[e] : 0.f, hi, lo);
        ghi[e] = hi;
        glo[e] = lo;
      }
#pragma unroll
      for (int nt = 0; nt < C::NDT; ++nt) {
        acc[h][nt] = mfma_bf16_16x16x32(ghi, Kb[nt], acc[h][nt]);
        acc[h][nt] = mfma_bf16_16x16x32(glo, Kb[nt], acc[h][nt]);
      }
    }
  }
  // dq rows t0 + 4 g + r, columns 16 nt + j16; dw row t (reduced over the four lane groups)
#pragma unroll
  for (int h = 0; h < BQ_HPW; ++h) {
    const int j = jw + h;
    if (j >= H_I) break;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t tr = t0 + 4 * g + r;
      if (tr < T) {
        const float wv = w[tr * H_I + j];
#pragma unroll
        for (int nt = 0; nt < C::NDT; ++nt) dq[(tr * H_I + j) * DI + 16 * nt + j16] = acc[h][nt][r] * wv;
      }
    }
    const float v = wave_sum_xor16_32(dwa[h]);
    if (g == 0 && t_ok) dw[t * H_I + j] = v * qs[t * H_I + j];
  }
}

// dq and dw over each row's listed keys only (the sparse stage, where dI vanishes off the index
// lists; lists with distinct entries).  A workgroup owns one query row and 64 heads (16 per wave,
// the MFMA M dimension of dq); blocks of 32 listed keys are gathered, their FP8 codes staged as
// bf16 rows, with dI[t, key] ks[key] per entry (0 for a skipped entry).
constexpr int BL_WAVES = 4;

template <int DI>
__global__ __launch_bounds__(BL_WAVES * WAVE, 2) void indexer_bwd_q_listed_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k8, const float* __restrict__ ks, int64_t T, int64_t S, int32_t H_I,
    int64_t q_start, const int32_t* __restrict__ idx, int32_t k, const float* __restrict__ dI, int64_t ld,
    float* __restrict__ dq, float* __restrict__ dw) {
  using C = BwCfg<DI>;
  __shared__ __align__(16) uint8_t kt[BW_BLK * C::STRIDE];
  __shared__ float us[BW_BLK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j16 = lane & 15, g = lane >> 4;
  const int64_t t = blockIdx.x;
  const int64_t n = min(S, q_start + t + 1);
  const int jw = (blockIdx.y * BL_WAVES + wave) * 16;  // waves past H_I still stage (zero queries)
  const int jl = jw + j16;  // this lane's head as the column of z^T = K Q^T
  // owned queries, B operands of z^T: lane = head jl, columns 32 zs + 8 g .. + 7
  s16x8 Qb[C::NZS];
#pragma unroll
  for (int zs = 0; zs < C::NZS; ++zs) {
    s16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (jl < H_I) {
      const v2i raw = *reinterpret_cast<const v2i*>(q8 + (t * H_I + jl) * DI + 32 * zs + 8 * g);
      v = e4m3x8_to_bf16((uint32_t)raw[0], (uint32_t)raw[1]);
    }
    Qb[zs] = v;
  }
  v4f acc[C::NDT];
#pragma unroll
  for (int nt = 0; nt < C::NDT; ++nt) acc[nt] = (v4f){0.f, 0.f, 0.f, 0.f};
  float dwa = 0.f;

  // Block b + 1's codes and key factors are loaded into registers before block b's MFMAs, with
  // the list entries they need read one block earlier still.  A thread stages piece pc of row
  // pr, and thread tid < 32 the key factor of row tid; skipped entries (negative or not visible)
  // load row 0 and get the factor 0.
  static_assert(BW_BLK * (DI / 16) <= BL_WAVES * WAVE, "one 16-byte piece per thread");
  const int pr = tid / (DI / 16), pc = tid % (DI / 16);
  const bool stager = tid < BW_BLK * (DI / 16);
  const int32_t* lrow = idx + t * k;
  const float* drow = dI + t * ld;
  // entries past the row's last valid one are not visited (rows with fewer visible keys than list
  // entries end in padding)
  __shared__ int32_t klast[BL_WAVES];
  int last = 0;
  for (int i = tid; i < k; i += BL_WAVES * WAVE) {
    const int32_t key = lrow[i];
    if (key >= 0 && key < n) last = i + 1;  // i grows: the thread's last valid entry
  }
  for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o));
  if (lane == 0) klast[wave] = last;
  __syncthreads();
  int k_used = 0;
  for (int w = 0; w < BL_WAVES; ++w) k_used = max(k_used, klast[w]);
  auto entry = [&](int e) -> int32_t {  // the listed key of entry e, -1 when skipped
    const int32_t key = lrow[min(e, k - 1)];
    return (e < k && key >= 0 && key < n) ? key : -1;
  };
  int32_t kp = entry(pr), ku = entry(tid & (BW_BLK - 1));  // block 0
  v4i nraw = *reinterpret_cast<const v4i*>(k8 + (int64_t)max(kp, 0) * DI + pc * 16);
  auto factor = [&](int32_t key) {  // loads are unconditional, the select comes after them
    const int32_t kk = max(key, 0);
    const float v = drow[kk] * ks[kk];
    return key >= 0 ? v : 0.f;
  };
  float nu = factor(ku);
  kp = entry(BW_BLK + pr);  // block 1
  ku = entry(BW_BLK + (tid & (BW_BLK - 1)));
  for (int e0 = 0; e0 < k_used; e0 += BW_BLK) {
    __syncthreads();  // the previous block is consumed
    if (stager) stage_row16(kt + pr * C::STRIDE + pc * 32, nraw);
    if (tid < BW_BLK) us[tid] = nu;
    __syncthreads();
    if (e0 + BW_BLK < k_used) {
      nraw = *reinterpret_cast<const v4i*>(k8 + (int64_t)max(kp, 0) * DI + pc * 16);
      nu = factor(ku);
      kp = entry(e0 + 2 * BW_BLK + pr);
      ku = entry(e0 + 2 * BW_BLK + (tid & (BW_BLK - 1)));
    }
    s16x8 Ka[2][C::NZS];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int zs = 0; zs < C::NZS; ++zs) Ka[sub][zs] = block_rows<C::STRIDE>(kt, lane, sub, zs);
    v4f z0 = {0.f, 0.f, 0.f, 0.f}, z1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int zs = 0; zs < C::NZS; ++zs) {
      z0 = mfma_bf16_16x16x32(Ka[0][zs], Qb[zs], z0);
      z1 = mfma_bf16_16x16x32(Ka[1][zs], Qb[zs], z1);
    }
    // lane: head jl, entries e0 + 4 g + r (sub-block 0) and e0 + 16 + 4 g + r (sub-block 1)
    s16x8 ghi, glo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float zz = e < 4 ? z0[e] : z1[e - 4];
      const float u = us[(e < 4 ? 0 : 16) + 4 * g + (e & 3)];
      dwa = fmaf(u, fmaxf(zz, 0.f), dwa);
      short hi, lo;
      split_bf16(zz > 0.f ? u : 0.f, hi, lo);
      ghi[e] = hi;
      glo[e] = lo;
    }
#pragma unroll
    for (int nt = 0; nt < C::NDT; ++nt) {
      const s16x8 kcol = block_columns<C::STRIDE>(kt, lane, 16 * nt);
      acc[nt] = mfma_bf16_16x16x32(ghi, kcol, acc[nt]);
      acc[nt] = mfma_bf16_16x16x32(glo, kcol, acc[nt]);
    }
  }
  // dq: heads jw + 4 g + r, columns 16 nt + j16; dw: head jl (reduced over the lane groups)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int jh = jw + 4 * g + r;
    if (jh < H_I) {
      const float wv = w[t * H_I + jh];
#pragma unroll
      for (int nt = 0; nt < C::NDT; ++nt) dq[(t * H_I + jh) * DI + 16 * nt + j16] = acc[nt][r] * wv;
    }
  }
  const float v = wave_sum_xor16_32(dwa);
  if (g == 0 && jl < H_I) dw[t * H_I + jl] = v * qs[t * H_I + jl];
}

// Queries [qc qchunk, (qc + 1) qchunk) that can see keys of key group kg (keys 128 kg ..): the
// chunk contributes a partial dk for the group iff this range is not empty.
__host__ __device__ __forceinline__ void bk_query_range(int64_t kg, int64_t qc, int64_t qchunk, int64_t T,
                                                        int64_t q_start, int64_t& tb, int64_t& te) {
  tb = max(qc * qchunk, kg * (BK_WAVES * BK_KPW) - q_start);
  te = min(T, (qc + 1) * qchunk);
}

// dk partials: a workgroup owns 128 keys (32 per wave) and streams the query rows of one chunk,
// all heads, eight heads at a time; part [nqc][S][DI].
template <int DI>
__global__ __launch_bounds__(BK_WAVES * WAVE, 2) void indexer_bwd_k_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k8, int64_t T, int64_t S, int32_t H_I, int64_t q_start,
    const float* __restrict__ dI, int64_t ld, int64_t qchunk, float* __restrict__ part) {
  using C = BwCfg<DI>;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* qt = smem;                                                          // [HC][32][STRIDE]
  float* wq = reinterpret_cast<float*>(smem + (size_t)BK_HC * BW_BLK * C::STRIDE);  // [HC][32]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j16 = lane & 15, g = lane >> 4;
  const int64_t kg = blockIdx.x, qc = blockIdx.y;
  int64_t tb0, t_end;
  bk_query_range(kg, qc, qchunk, T, q_start, tb0, t_end);
  if (tb0 >= t_end) return;  // workgroup-uniform: no partial for this chunk
  const int64_t s_w = kg * (BK_WAVES * BK_KPW) + wave * BK_KPW;

  // owned keys, B operands of z = Q K^T: lane = key s_w + 16 u + j16, columns 32 zs + 8 g .. + 7
  s16x8 Kb[2][C::NZS];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int zs = 0; zs < C::NZS; ++zs) {
      const int64_t s = min(s_w + 16 * u + j16, S - 1);
      const v2i raw = *reinterpret_cast<const v2i*>(k8 + s * DI + 32 * zs + 8 * g);
      Kb[u][zs] = e4m3x8_to_bf16((uint32_t)raw[0], (uint32_t)raw[1]);
    }
  v4f acc[2][C::NDT];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int nt = 0; nt < C::NDT; ++nt) acc[u][nt] = (v4f){0.f, 0.f, 0.f, 0.f};

  // Query codes and weights of the next (query block, head chunk) are loaded into registers before
  // the MFMAs of the current one; staging them into LDS waits for the next barrier.
  constexpr int BK_PPT = BK_HC * BW_BLK * (DI / 16) / (BK_WAVES * WAVE);  // 16-byte pieces per thread
  static_assert(BK_PPT * BK_WAVES * WAVE == BK_HC * BW_BLK * (DI / 16), "whole pieces per thread");
  static_assert(BK_HC * BW_BLK <= BK_WAVES * WAVE, "one weight per thread");
  v4i nraw[BK_PPT];
  float nwq = 0.f;
  auto prefetch = [&](int64_t tbn, int hcn) {
#pragma unroll
    for (int u = 0; u < BK_PPT; ++u) {
      const int p = tid + u * BK_WAVES * WAVE;
      const int c = p % (DI / 16), rq = (p / (DI / 16)) % BW_BLK, hh = p / (DI / 16) / BW_BLK;
      const int64_t tq = tbn + rq;
      const int j = hcn + hh;
      nraw[u] = (v4i){0, 0, 0, 0};
      if (tq < t_end && j < H_I) nraw[u] = *reinterpret_cast<const v4i*>(q8 + (tq * H_I + j) * DI + c * 16);
    }
    if (tid < BK_HC * BW_BLK) {
      const int rq = tid % BW_BLK, hh = tid / BW_BLK;
      const int64_t tq = tbn + rq;
      const int j = hcn + hh;
      nwq = (tq < t_end && j < H_I) ? w[tq * H_I + j] * qs[tq * H_I + j] : 0.f;
    }
  };
  prefetch(tb0, 0);
  for (int64_t tb = tb0; tb < t_end; tb += BW_BLK) {
    // dI of this lane's 16 (row, key) pairs; 0 outside the chunk or the causal range
    float dv[2][8];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t tq = tb + (e < 4 ? 0 : 16) + 4 * g + (e & 3);
        const int64_t s = s_w + 16 * u + j16;
        dv[u][e] = (tq < t_end && s < min(S, q_start + tq + 1)) ? dI[tq * ld + s] : 0.f;
      }
    for (int hc = 0; hc < H_I; hc += BK_HC) {
      __syncthreads();  // the previous heads are consumed
#pragma unroll
      for (int u = 0; u < BK_PPT; ++u) {
        const int p = tid + u * BK_WAVES * WAVE;
        const int c = p % (DI / 16), rq = (p / (DI / 16)) % BW_BLK, hh = p / (DI / 16) / BW_BLK;
        stage_row16(qt + (hh * BW_BLK + rq) * C::STRIDE + c * 32, nraw[u]);
      }
      if (tid < BK_HC * BW_BLK) wq[tid] = nwq;
      __syncthreads();
      // the next chunk's loads go out before this chunk's MFMAs
      if (hc + BK_HC < H_I)
        prefetch(tb, hc + BK_HC);
      else if (tb + BW_BLK < t_end)
        prefetch(tb + BW_BLK, 0);
      for (int hh = 0; hh < BK_HC && hc + hh < H_I; ++hh) {
        const uint8_t* qh = qt + hh * BW_BLK * C::STRIDE;
        s16x8 Qa[2][C::NZS];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int zs = 0; zs < C::NZS; ++zs) Qa[sub][zs] = block_rows<C::STRIDE>(qh, lane, sub, zs);
        float wv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) wv[e] = wq[hh * BW_BLK + (e < 4 ? 0 : 16) + 4 * g + (e & 3)];
        // the gradient tiles of both key tiles first, then one B fragment at a time for both
        s16x8 ghi[2], glo[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          v4f z0 = {0.f, 0.f, 0.f, 0.f}, z1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int zs = 0; zs < C::NZS; ++zs) {
            z0 = mfma_bf16_16x16x32(Qa[0][zs], Kb[u][zs], z0);
            z1 = mfma_bf16_16x16x32(Qa[1][zs], Kb[u][zs], z1);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float zz = e < 4 ? z0[e] : z1[e - 4];
            short hi, lo;
            split_bf16(zz > 0.f ? dv[u][e] * wv[e] : 0.f, hi, lo);
            ghi[u][e] = hi;
            glo[u][e] = lo;
          }
        }
#pragma unroll
        for (int nt = 0; nt < C::NDT; ++nt) {
          const s16x8 qcol = block_columns<C::STRIDE>(qh, lane, 16 * nt);
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            acc[u][nt] = mfma_bf16_16x16x32(ghi[u], qcol, acc[u][nt]);
            acc[u][nt] = mfma_bf16_16x16x32(glo[u], qcol, acc[u][nt]);
          }
        }
      }
    }
  }
  // keys s_w + 16 u + 4 g + r, columns 16 nt + j16
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t s = s_w + 16 * u + 4 * g + r;
      if (s < S) {
#pragma unroll
        for (int nt = 0; nt < C::NDT; ++nt) part[(qc * S + s) * DI + 16 * nt + j16] = acc[u][nt][r];
      }
    }
}

// dk[s] = sum of the partials of the chunks that see the key's group (0 when none does).
__global__ __launch_bounds__(256) void indexer_bwd_k_reduce_kernel(const float* __restrict__ part, int64_t S,
                                                                   int32_t DI, int64_t T, int64_t q_start,
                                                                   int64_t qchunk, int32_t nqc,
                                                                   float* __restrict__ dk) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // float4 index
  if (i * 4 >= S * DI) return;
  const int64_t s = i * 4 / DI, kg = s / (BK_WAVES * BK_KPW);
  v4f sum = {0.f, 0.f, 0.f, 0.f};
  for (int qc = 0; qc < nqc; ++qc) {
    int64_t tb, te;
    bk_query_range(kg, qc, qchunk, T, q_start, tb, te);
    if (tb < te) sum += *reinterpret_cast<const v4f*>(part + (int64_t)qc * S * DI + i * 4);
  }
  *reinterpret_cast<v4f*>(dk + i * 4) = sum;
}

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------
static const int kKlSteps[] = {2, 4, 5, 8, 12, 16, 24, 32, 36};

bool indexer_kl_supported(int32_t H, int32_t D) { return H >= 1 && H <= 128 && D >= 8 && D <= 576 && D % 8 == 0; }

template <int NKS>
static hipError_t launch_kl(const uint16_t* q, const uint16_t* kv, int64_t T, int64_t S, int32_t H, int32_t D,
                            float sm_scale, int64_t q_start, const float* logits, int64_t ld, float* dlogits,
                            float* loss, hipStream_t stream) {
  using C = KlCfg<NKS>;
  hipError_t e = set_max_dynamic_lds(reinterpret_cast<const void*>(&indexer_kl_kernel<NKS>));
  if (e != hipSuccess) return e;
  const int64_t grid = (T + KL_TOK - 1) / KL_TOK;
  return launch("indexer_kl_kernel", indexer_kl_kernel<NKS>, dim3((unsigned)grid), dim3(KL_THREADS), C::SMEM, stream,
                q, kv, T, S, H, D, sm_scale * KL_LOG2E, q_start, logits, ld, dlogits, loss);
}

hipError_t launch_indexer_kl(const uint16_t* q, const uint16_t* kv, int64_t T, int64_t S, int32_t H, int32_t D,
                             float sm_scale, int64_t q_start, const float* logits, int64_t ld, float* dlogits,
                             float* loss, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int need = (D + 15) / 16;
  int nks = 0;
  for (int c : kKlSteps)
    if (c >= need) {
      nks = c;
      break;
    }
  switch (nks) {
#define KL_CASE(N) \
  case N: return launch_kl<N>(q, kv, T, S, H, D, sm_scale, q_start, logits, ld, dlogits, loss, stream);
    KL_CASE(2) KL_CASE(4) KL_CASE(5) KL_CASE(8) KL_CASE(12) KL_CASE(16) KL_CASE(24) KL_CASE(32) KL_CASE(36)
#undef KL_CASE
    default: return hipErrorInvalidValue;
  }
}

template <int NKS>
static hipError_t launch_kl_sparse(const uint16_t* q, const uint16_t* kv, const int32_t* idx, int32_t k,
                                   const float* lse, int64_t T, int64_t S, int32_t H, int32_t D, float sm_scale,
                                   int64_t q_start, const float* logits, int64_t ld, float* dlogits, float* loss,
                                   hipStream_t stream) {
  constexpr size_t smem = kls_smem_bytes<NKS>();
  hipError_t e = set_max_dynamic_lds(reinterpret_cast<const void*>(&indexer_kl_sparse_kernel<NKS>));
  if (e != hipSuccess) return e;
  return launch("indexer_kl_sparse_kernel", indexer_kl_sparse_kernel<NKS>, dim3((unsigned)T), dim3(KLS_THREADS), smem,
                stream, q, kv, idx, k, lse, T, S, H, D, sm_scale * KL_LOG2E, q_start, logits, ld, dlogits, loss);
}

bool indexer_kl_sparse_supported(int32_t H, int32_t D, int32_t k) {
  return indexer_kl_supported(H, D) && k >= 1 && k <= KLS_MAX_K;
}

hipError_t launch_indexer_kl_sparse(const uint16_t* q, const uint16_t* kv, const int32_t* idx, int32_t k,
                                    const float* lse, int64_t T, int64_t S, int32_t H, int32_t D, float sm_scale,
                                    int64_t q_start, const float* logits, int64_t ld, float* dlogits, float* loss,
                                    hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int need = (D + 15) / 16;
  int nks = 0;
  for (int c : kKlSteps)
    if (c >= need) {
      nks = c;
      break;
    }
  switch (nks) {
#define KLS_CASE(N)                                                                                            \
  case N:                                                                                                      \
    return launch_kl_sparse<N>(q, kv, idx, k, lse, T, S, H, D, sm_scale, q_start, logits, ld, dlogits, loss, \
                               stream);
    KLS_CASE(2) KLS_CASE(4) KLS_CASE(5) KLS_CASE(8) KLS_CASE(12) KLS_CASE(16) KLS_CASE(24) KLS_CASE(32) KLS_CASE(36)
#undef KLS_CASE
    default: return hipErrorInvalidValue;
  }
}

// Query chunk of the dk partials: about 16 chunks (enough workgroups for the chip at the
// workloads' sizes), a multiple of the 32-row block.
int64_t indexer_bwd_qchunk(int64_t T) {
  const int64_t c = (T + 15) / 16;
  return std::max<int64_t>(128, (c + BW_BLK - 1) / BW_BLK * BW_BLK);
}

size_t indexer_bwd_workspace_bytes(int64_t T, int64_t S, int32_t D_I) {
  if (T <= 0 || S <= 0) return 0;
  const int64_t qchunk = indexer_bwd_qchunk(T);
  const int64_t nqc = (T + qchunk - 1) / qchunk;
  return (size_t)nqc * (size_t)S * (size_t)D_I * sizeof(float);
}

template <int DI>
static hipError_t launch_bwd(const uint8_t* q8, const float* qs, const float* w, const uint8_t* k8, const float* ks,
                             int64_t T, int64_t S, int32_t H_I, int64_t q_start, const float* dI, int64_t ld,
                             float* dq, float* dw, float* dk, void* workspace, const int32_t* idx, int32_t k,
                             hipStream_t stream) {
  using C = BwCfg<DI>;
  hipError_t e;
  if (idx) {  // dq / dw over the listed keys only
    const int hgroups = (H_I + BL_WAVES * 16 - 1) / (BL_WAVES * 16);
    e = launch("indexer_bwd_q_listed_kernel", indexer_bwd_q_listed_kernel<DI>, dim3((unsigned)T, (unsigned)hgroups),
               dim3(BL_WAVES * WAVE), 0, stream, q8, qs, w, k8, ks, T, S, H_I, q_start, idx, k, dI, ld, dq, dw);
  } else {
    const int64_t qtiles = (T + BW_ROWS - 1) / BW_ROWS;
    const int hgroups = (H_I + BQ_WAVES * BQ_HPW - 1) / (BQ_WAVES * BQ_HPW);
    e = launch("indexer_bwd_q_kernel", indexer_bwd_q_kernel<DI>, dim3((unsigned)qtiles, (unsigned)hgroups),
               dim3(BQ_WAVES * WAVE), 0, stream, q8, qs, w, k8, ks, T, S, H_I, q_start, dI, ld, dq, dw);
  }
  if (e != hipSuccess) return e;
  e = set_max_dynamic_lds(reinterpret_cast<const void*>(&indexer_bwd_k_kernel<DI>));
  if (e != hipSuccess) return e;
  const int64_t qchunk = indexer_bwd_qchunk(T);
  const int32_t nqc = (int32_t)((T + qchunk - 1) / qchunk);
  const int64_t kgroups = (S + BK_WAVES * BK_KPW - 1) / (BK_WAVES * BK_KPW);
  float* part = reinterpret_cast<float*>(workspace);
  e = launch("indexer_bwd_k_kernel", indexer_bwd_k_kernel<DI>, dim3((unsigned)kgroups, (unsigned)nqc),
             dim3(BK_WAVES * WAVE), C::BK_SMEM, stream, q8, qs, w, k8, T, S, H_I, q_start, dI, ld, qchunk, part);
  if (e != hipSuccess) return e;
  const int64_t n4 = S * DI / 4;
  return launch("indexer_bwd_k_reduce_kernel", indexer_bwd_k_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)),
                dim3(256), 0, stream, part, S, DI, T, q_start, qchunk, nqc, dk);
}

hipError_t launch_indexer_bwd(const uint8_t* q8, const float* qs, const float* w, const uint8_t* k8, const float* ks,
                              int64_t T, int64_t S, int32_t H_I, int32_t D_I, int64_t q_start, const float* dI,
                              int64_t ld, float* dq, float* dw, float* dk, void* workspace, hipStream_t stream,
                              const int32_t* idx, int32_t k) {
  if (T <= 0 || S <= 0) return hipSuccess;
  switch (D_I) {
#define BWD_CASE(N) \
  case N: return launch_bwd<N>(q8, qs, w, k8, ks, T, S, H_I, q_start, dI, ld, dq, dw, dk, workspace, idx, k, stream);
    BWD_CASE(32) BWD_CASE(64) BWD_CASE(96) BWD_CASE(128)
#undef BWD_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsa
