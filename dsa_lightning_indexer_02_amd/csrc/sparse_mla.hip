// Sparse MLA forward in MQA mode (DeepSeek-V3.2-Exp summary page, section "Method": the main
// attention reads only the top-k indexed latent KV rows, one row shared by every query head of
// a token; AMD MI355X article, section "Computational Efficiency": O(L k) core attention).
//
// For query row t, head h and the valid entries i of its index list (0 <= idx < n_t):
//   z_i = sm_scale * q[t,h,:] . kv[idx_i, :D_qk],  p = softmax(z),
//   out[t,h,:] = sum_i p_i kv[idx_i, :D_v],        lse[t,h] = log sum_i exp(z_i).
//
// One workgroup (8 waves) per query row (or per row and index split in decode).  Heads form
// groups of 32, one 32x32 MFMA tile each; every group is served by a pair of waves that split
// the contraction: wave half f holds the queries of columns [f D_qk/2, (f+1) D_qk/2) and the
// fp32 output accumulators of value columns [f D_v/2, (f+1) D_v/2).  Per block of 32 selected
// rows (gathered HBM/L2 -> LDS by DMA, row-major):
//   1. each wave forms its partial S^T = K_f Q_f^T (32x32x16 MFMA) and posts it in LDS;
//   2. each wave adds its partner's partial (addition commutes, so both hold the same S^T),
//      and computes the probabilities of its 16 entries per lane in fp16;
//   3. out^T = V^T P^T (fp16 32x32x16 MFMA): the S^T accumulator layout is the B-operand layout
//      of P^T, so probabilities never leave registers.
// Two stagings of the gathered rows.  fp16 staging (the prefill path, given a workspace): the
// rows were converted to fp16 beforehand (mla_kv_to_f16_kernel), the queries are converted as
// they are loaded, S^T is an fp16 MFMA of the same values, and step 3 takes its V^T operands
// straight from the gathered rows by transposing LDS reads; three stages rotate.  bf16 staging
// (decode, and calls without a workspace): S^T is a bf16 MFMA, and V^T is built once per block
// by all waves (transposing LDS reads, bf16 -> fp16 in registers) into an fp16 buffer whose key
// order matches the B-operand layout of P^T; two stages rotate.  Either way bf16 -> fp16 is exact
// for |x| in [2^-17, 65504].
// P is rounded to fp16 (11-bit significand) rather than bf16.  The softmax reference maximum is
// fixed at the first block holding a valid entry; a second pass with the exact row maximum runs
// only if a later block exceeds it by more than 2^15 (the fp16 headroom).
#include "dsa_internal.hpp"

namespace dsa {

constexpr int MLA_WAVES = 8;
constexpr int MLA_THREADS = MLA_WAVES * WAVE;
constexpr int MLA_KB = 32;             // selected rows per block
constexpr int MLA_GROUP_HEADS = 32;    // heads per group (one 32x32 tile), served by a wave pair
constexpr int MLA_GROUPS = MLA_WAVES / 2;
constexpr int MLA_STAGES = 2;          // gathered-row buffers in flight (bf16 staging)
constexpr int MLA_STAGES_F16 = 3;      // the same, fp16 staging (the value phase reads the stage)
constexpr int MLA_MAX_K = 2048;        // index entries per workgroup (LDS row list)
constexpr float MLA_HEADROOM = 15.0f;  // log2 headroom of fp16 probabilities above the reference

template <int DQK, int DV, bool F16 = false>
struct MlaCfg {
  static constexpr int STAGES = F16 ? MLA_STAGES_F16 : MLA_STAGES;
  static constexpr int DH = ((DQK + 1) / 2 + 15) / 16 * 16;  // q.k columns per wave of a pair
  static constexpr int DQK_PAD = 2 * DH;
  static constexpr int NKS = DH / 16;                        // 32x32x16 steps of the partial S^T
  static constexpr int DVH = DV / 2;                         // value columns per wave of a pair
  static constexpr int NDT = DVH / 32;                       // 32-wide value tiles per wave
  static constexpr int RC = DQK_PAD / 8;                     // 16-byte chunks per gathered row
  static constexpr int SWZ = RC % 8 == 0 ? 8 : (RC % 4 == 0 ? 4 : 1);  // XOR swizzle span (chunks)
  static constexpr int SLOTS = MLA_KB * RC;                  // 16-byte slots per stage
  static constexpr int K_BYTES = SLOTS * 16;
  static constexpr int DMA_INSTR = SLOTS / WAVE;             // wave-wide 1 KiB transfers per block
  static constexpr int DMA_PW = (DMA_INSTR + MLA_WAVES - 1) / MLA_WAVES;  // transfers per wave (max)
  // wide rows: per wave, the 16-bit source descriptor of each of its transfers per lane (chunk
  // byte offset in the row | 0x8000 for the transfer's second row) and the row each lane pair reads
  static constexpr int GTAB_BYTES = RC >= WAVE ? MLA_WAVES * (DMA_PW + 1) * WAVE * 2 : 0;
  static constexpr int SX_BYTES = MLA_WAVES * WAVE * 16 * 4; // partial S^T of every wave (fp32)
  static constexpr int VT_STRIDE = 2 * MLA_KB + 16;          // bytes per fp16 V^T row (one value column)
  static constexpr int VT_BYTES = F16 ? 0 : DV * VT_STRIDE;  // fp16 staging reads V from the stage
  static_assert(DQK % 8 == 0 && DV % 64 == 0 && DV <= DQK && DV <= 64 * MLA_WAVES, "unsupported MLA dims");
  static_assert(SLOTS % WAVE == 0, "gather slots must fill whole waves");
  // Chunk XOR of gathered row r.  gfx950's LDS serves a 16-byte-per-lane read 16 lanes at a time
  // over 64 four-byte banks, and a 576-wide row (288 dwords) moves the bank map by half the banks:
  // the 16 rows of one K-fragment read pass are conflict-free when rows of equal parity get
  // distinct XORs mod 8, and the transposing reads of rows 4 j .. 4 j + 3 when rows 4 j and 4 j + 2
  // differ in XOR bit 2.  (row bit 1 -> XOR bit 2, row bits 2-3 -> XOR bits 0-1) does both.
  static __host__ __device__ __forceinline__ constexpr int swz(int r) {
    return ((((r >> 1) & 1) << 2) | ((r >> 2) & 3)) & (SWZ - 1);
  }
  // 16-byte slot of chunk c of gathered row r: rows are contiguous, chunks XOR-swizzled within
  // aligned groups of SWZ.
  static __device__ __forceinline__ int slot(int r, int c) { return r * RC + (c ^ swz(r)); }
};

template <int DQK, int DV, bool F16 = false>
size_t mla_smem_bytes(int32_t keys_per_wg) {
  using C = MlaCfg<DQK, DV, F16>;
  (void)keys_per_wg;
  return (size_t)C::STAGES * C::K_BYTES + C::SX_BYTES + C::VT_BYTES +
         (size_t)(MLA_MAX_K + 4 + MLA_MAX_K / MLA_KB) * sizeof(int32_t) + C::GTAB_BYTES;
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

// Transposing LDS read (gfx950): within each group of 16 lanes, lane i receives element i % 4 of
// the 4 x 16-bit words addressed by lanes 4 j + i / 4 of its group, j = 0..3.
__device__ __forceinline__ s16x4 lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

// Four bf16 values (two packed words each) -> fp16, as one half of an MFMA operand.
__device__ __forceinline__ void bf16x4_to_f16(const s16x4 raw, s16x8& dst, int half) {
  const v2i w = __builtin_bit_cast(v2i, raw);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const float lo = __uint_as_float((uint32_t)w[e] << 16);
    const float hi = __uint_as_float((uint32_t)w[e] & 0xFFFF0000u);
    dst[4 * half + 2 * e] = __builtin_bit_cast(short, (_Float16)lo);
    dst[4 * half + 2 * e + 1] = __builtin_bit_cast(short, (_Float16)hi);
  }
}

// OFF32: every row of the latent cache lies within 4 GiB of its base, so a gathered chunk's address
// is the base plus a 32-bit offset (row * row bytes + chunk offset: one 24-bit multiply-add).
// F16: kv holds the latent rows in fp16 (mla_kv_to_f16_kernel) and the queries are converted to fp16
// as they are loaded: S^T is an fp16 MFMA (the same products: bf16 -> fp16 is exact in fp16's normal
// range), and the value phase takes its V^T operands straight from the gathered rows by transposing
// LDS reads, so no V^T buffer is built; with the stage read until the end of a block, three stages
// keep the gather two blocks ahead.
template <int DQK, int DV, bool OFF32, bool F16>
__global__ __launch_bounds__(MLA_THREADS, 1) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ table, int64_t max_blocks, int32_t block_shift, int64_t num_blocks, int32_t per_row_table,
    const int32_t* __restrict__ seq_lens, int64_t S, int64_t q_start, int32_t H, int32_t k,
    float scale_log2, int32_t nsplit, int32_t keys_per_split, uint16_t* __restrict__ out,
    float* __restrict__ out_f32, float* __restrict__ lse, float* __restrict__ part_out,
    float* __restrict__ part_lse) {
  using C = MlaCfg<DQK, DV, F16>;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* Kbuf = smem;                                                  // [STAGES][SLOTS] x 16 B
  float* Sx = reinterpret_cast<float*>(smem + C::STAGES * C::K_BYTES);   // [WAVES][4][64] x v4f
  uint8_t* Vt = smem + C::STAGES * C::K_BYTES + C::SX_BYTES;             // [DV][VT_STRIDE] fp16 (bf16 staging)
  int32_t* phys = reinterpret_cast<int32_t*>(Vt + C::VT_BYTES);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int hg = wave >> 1, hf = wave & 1;                    // head group, contraction half
  const int l32 = lane & 31, lh = lane >> 5;
  // Rows on x (up to 2^31 - 1 in one launch), latest first: rows with full lists start together
  // and walk their ascending index lists in near lockstep, so the gathered rows of the workgroups
  // in flight overlap in L2; rows shorter than their lists (which stop early) come last.
  const int64_t r = (int64_t)gridDim.x - 1 - blockIdx.x;
  const int sp = blockIdx.y;
  const int64_t n = seq_lens ? min((int64_t)max(seq_lens[r], 0), S) : min(S, q_start + r + 1);
  const int i0 = sp * keys_per_split;
  const int i1 = min(k, i0 + keys_per_split);
  const int cnt = max(i1 - i0, 0);
  const RowMap map{table ? (per_row_table ? table + r * max_blocks : table) : nullptr, block_shift, num_blocks};

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
  // The prologue overlaps its memory latencies: the index entries (four per thread) are loaded
  // first, then the block-table lookups they need, then the queries; the tables below are built
  // while the queries are in flight, and the first gathers are issued before the queries are
  // awaited.
  static_assert(MLA_MAX_K == 4 * MLA_THREADS, "four index entries per thread");
  int32_t prow4[4];
  bool valid4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = tid + j * MLA_THREADS;
    const int32_t li = i < cnt ? idx[r * k + i0 + i] : -1;
    valid4[j] = li >= 0 && li < n;
    prow4[j] = li;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) prow4[j] = valid4[j] ? (int32_t)map(prow4[j]) : -1;  // -1: skipped entry
  // queries of this wave's head group and contraction half, as B operands of S^T = K Q^T (loads
  // only: converted and pinned to registers before the block loop)
  const bool active = hg * MLA_GROUP_HEADS < H;
  const int head = hg * MLA_GROUP_HEADS + l32;
  s16x8 Qf[C::NKS];
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) {
    const int col = hf * C::DH + ks * 16 + lh * 8;
    const bool ok = head < H && col < DQK;
    Qf[ks] = *reinterpret_cast<const s16x8*>(q + (r * H + (ok ? head : 0)) * (int64_t)DQK + (ok ? col : 0));
  }
  // physical rows of the index entries, and the validity bit mask of every 32-entry block (bit i:
  // entry 32 b + i is gathered and attended)
  uint32_t* vmask_lds = reinterpret_cast<uint32_t*>(phys + MLA_MAX_K + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = tid + j * MLA_THREADS, base = wave * WAVE + j * MLA_THREADS;
    if (i < cnt) phys[i] = prow4[j];
    const uint64_t bits = __ballot(valid4[j]);
    if (lane == 0 && base < cnt) {
      vmask_lds[base / 32] = (uint32_t)bits;
      if (base + 32 < cnt) vmask_lds[base / 32 + 1] = (uint32_t)(bits >> 32);
    }
  }
  // The gather's per-lane slot arithmetic (row = slot / RC, swizzled chunk) is the same for every
  // block: each wave tabulates it once for its own transfers.
  uint16_t* gtab = reinterpret_cast<uint16_t*>(vmask_lds + MLA_MAX_K / MLA_KB);  // [WAVES][DMA_PW][64]
  uint16_t* rtab = gtab + MLA_WAVES * C::DMA_PW * WAVE;                            // [WAVES][64]
  if constexpr (C::RC >= WAVE) {
#pragma unroll
    for (int j = 0; j < C::DMA_PW; ++j) {
      const int i = wave + j * MLA_WAVES;
      if (i < C::DMA_INSTR) {
        const int sl = i * WAVE + lane;
        const int rr = sl / C::RC;
        const int c = (sl % C::RC) ^ C::swz(rr);
        gtab[(wave * C::DMA_PW + j) * WAVE + lane] =
            (uint16_t)((c * 16) | (rr != (i * WAVE) / C::RC ? 0x8000 : 0));
      }
    }
    // lane 2 j / 2 j + 1: the row of the first / last slot of transfer j (0xFFFF: no transfer)
    const int j = lane >> 1, i = wave + j * MLA_WAVES;
    rtab[wave * WAVE + lane] =
        (j < C::DMA_PW && i < C::DMA_INSTR) ? (uint16_t)((i * WAVE + (lane & 1) * (WAVE - 1)) / C::RC) : (uint16_t)0xFFFF;
  }
  // Skipped entries are gathered from a row that certainly holds finite data (the sequence's
  // first key) and masked out of the softmax.
  const int32_t safe_row = (int32_t)map(0);
  // zero the padding chunks of every stage once; the gather never writes them
  if (C::DQK_PAD > DQK) {
    for (int p = tid; p < C::STAGES * MLA_KB * C::RC; p += MLA_THREADS) {
      const int st = p / (MLA_KB * C::RC), rr = (p / C::RC) % MLA_KB, c = p % C::RC;
      if (c * 8 >= DQK)
        *reinterpret_cast<v4i*>(Kbuf + st * C::K_BYTES + C::slot(rr, c) * 16) = (v4i){0, 0, 0, 0};
    }
  }

  __syncthreads();

  const uint32_t kbuf_lds = lds_addr(Kbuf);
  const int my_dma = (C::DMA_INSTR - wave + MLA_WAVES - 1) / MLA_WAVES;  // this wave's transfers per block
  static_assert(C::SWZ == 8 || C::SWZ == 4 || C::SWZ == 1, "swizzle span");
  // K fragment of step ks (A operand): row l32, chunk cb + 2 ks.  XOR-ing the row swizzle into the low
  // log2(SWZ) chunk bits leaves steps that are SWZ chunks apart a constant distance apart, so the
  // offset is one of KP per-lane bases plus a compile-time constant.
  constexpr int KP = C::SWZ >= 2 ? C::SWZ / 2 : 1;
  const int kx = C::swz(l32);
  const int kcb = hf * (C::DH / 8) + lh;
  int kbase[KP];
#pragma unroll
  for (int u = 0; u < KP; ++u) kbase[u] = (l32 * C::RC + ((kcb + 2 * u) ^ kx)) * 16;
  auto kfrag_off = [&](int ks) { return kbase[ks % KP] + (ks / KP) * (2 * KP * 16); };
  // V^T construction: wave w converts value columns [64 w, 64 w + 64); its 16-lane group G
  // columns 64 w + 16 G + 0..15.  Transposing read j gives lane i of the group column
  // 64 w + 16 G + i at keys 4 j' + 0..3 when lane a of the group addresses row 4 j' + a / 4,
  // columns 64 w + 16 G + 4 (a % 4) .. + 3.  Keys are stored per column in the order
  // [16 m + 4 lh + 0..3, 16 m + 8 + 4 lh + 0..3] at 16-byte unit 2 m + lh, which is the order of
  // the probabilities a lane holds in elements 8 m .. 8 m + 7 of the S^T accumulator.
  const bool converts = wave * 64 < DV;
  const int tg = (lane >> 4) & 3, ti = lane & 15;
  const int trow = (lane & 15) >> 2;                                   // + 4 j'
  const int tch = (wave * 64 + 16 * tg) / 8 + ((lane & 3) >> 1);      // chunk of the addressed columns
  // row 4 jq + trow (trow < 4) has the swizzle swz(trow) ^ swz(4 jq): the two take disjoint bits
  static_assert(C::swz(4 * 3 + 3) == (C::swz(3) ^ C::swz(12)) && C::swz(4 * 2 + 1) == (C::swz(1) ^ C::swz(8)),
                "row swizzle splits into the quad and the row within it");
  const int tbase = trow * C::RC * 16 + 8 * (lane & 1);
  const int tc0 = tch ^ C::swz(trow);
  auto tr_off = [&](int jq) {  // key quad jq (a compile-time constant): rows 4 jq + 0..3
    return tbase + 16 * (tc0 ^ C::swz(4 * jq)) + 4 * jq * C::RC * 16;
  };
  uint8_t* vt_dst = Vt + (wave * 64 + 16 * tg + ti) * C::VT_STRIDE;
  // Gather of block blk.  Transfer i covers slots [64 i, 64 i + 64).  When a row holds at least
  // 64 slots that is at most two gathered rows, (64 i) / RC and (64 i + 63) / RC: gather_rows then
  // reads the physical rows of all this wave's transfers with one LDS read (lane 2 j / 2 j + 1:
  // first / last row of its j-th transfer), early enough for the value to be there when
  // gather_issue takes them by readlane.  Narrower rows look their row up per lane.
  constexpr int DMA_PW = C::DMA_PW;
  static_assert(2 * DMA_PW <= WAVE, "one lane pair per transfer");
  auto gather_rows = [&](int blk) {
    if constexpr (C::RC < WAVE) {  // narrow rows: each lane looks its row up in gather_issue
      (void)blk;
      return safe_row;
    } else {
      const int rr = rtab[wave * WAVE + lane];
      const int e = blk * MLA_KB + rr;
      int32_t pr = -1;
      if (rr != 0xFFFF && e < cnt) pr = phys[e];
      return pr >= 0 ? pr : safe_row;
    }
  };
  auto gather_issue = [&](int blk, int stage, int32_t prow) {
    const uint32_t base = kbuf_lds + (uint32_t)(stage * C::K_BYTES);
    if constexpr (C::RC < WAVE) {
      (void)prow;
      for (int i = wave; i < C::DMA_INSTR; i += MLA_WAVES) {
        const int s = i * WAVE + lane;
        const int rr = s / C::RC;
        const int c = (s % C::RC) ^ C::swz(rr);
        const int e = blk * MLA_KB + rr;
        const int32_t pr = e < cnt ? phys[e] : -1;
        const uint16_t* src = kv + (int64_t)(pr >= 0 ? pr : safe_row) * DQK + c * 8;
        if (C::DQK_PAD == DQK || c * 8 < DQK) dma_16B(src, base + (uint32_t)(i * WAVE * 16));
      }
    } else {
    static_assert(C::DQK_PAD == DQK, "every chunk of a wide row is gathered");
#pragma unroll
    for (int j = 0; j < DMA_PW; ++j) {
      const int i = wave + j * MLA_WAVES;
      // transfers whose index stays below DMA_INSTR for every wave need no test
      if (j * MLA_WAVES + MLA_WAVES - 1 < C::DMA_INSTR || i < C::DMA_INSTR) {  // wave-uniform
        const uint32_t t = gtab[(wave * DMA_PW + j) * WAVE + lane];
        const int32_t pa = __builtin_amdgcn_readlane(prow, 2 * j), pb = __builtin_amdgcn_readlane(prow, 2 * j + 1);
        const uint32_t row = (t & 0x8000u) ? (uint32_t)pb : (uint32_t)pa;
        const uint32_t lds = base + (uint32_t)(i * WAVE * 16);
        if constexpr (OFF32)
          lds_dma_16B_sbase(kv, __umul24(row, (uint32_t)(DQK * 2)) + (t & 0x7FFFu), lds);
        else
          dma_16B(reinterpret_cast<const uint8_t*>(kv) + (uint64_t)row * (DQK * 2) + (t & 0x7FFFu), lds);
      }
    }
    }
  };
  auto gather = [&](int blk) { gather_issue(blk, blk, gather_rows(blk)); };  // blocks 0 and 1: stages 0 and 1

  // fp16 staging: the V^T operand of value step (m, dt) by transposing reads of the gathered rows.
  // The 16-lane group g of the wave reads key quad 4 m + lh (k-elements 0-3; + 2 for k-elements 4-7),
  // value columns f DV/2 + 32 dt + 16 (g & 1) + 0..15: its lane a addresses row 4 quad + a / 4,
  // columns + 4 (a % 4) .. + 3, so that lane i of the group receives column + i at the quad's four
  // keys.  Per lane: one base for each (quad parity rd, dt parity); m and dt / 2 add constants.
  int vb[2][2];
  static_assert(!F16 || C::STAGES == 3, "fp16 staging rotates three stages");
  if constexpr (F16) {
    const int g = lane >> 4, a = lane & 15, t = a >> 2;
    const int y = 2 * (g & 1) + ((a & 3) >> 1);  // chunk within the 32-column tile pair half
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int rowq = 4 * (lh + 2 * rd) + t;     // row within the 16-key half (its swizzle is the row's)
      const int z = (y ^ C::swz(rowq)) & (C::SWZ - 1);
#pragma unroll
      for (int od = 0; od < 2; ++od)  // odd dt: chunk bit 2 set before the XOR
        vb[rd][od] = (rowq * C::RC + hf * (C::DVH / 8) + (z ^ (4 * od))) * 16 + 8 * (a & 1);
    }
  }
  v16f O[C::NDT];
  float mref, mlane = -INFINITY, lsum;  // mlane: this lane's running raw maximum (its head, its keys)
  // blocks up to the last one holding a valid entry (all later entries are masked: a row with fewer
  // visible keys than list entries skips its padding); one validity word per lane, the same answer
  // in every wave
  static_assert(MLA_MAX_K / MLA_KB <= WAVE, "one block word per lane");
  const int nblk_all = (cnt + MLA_KB - 1) / MLA_KB;
  const uint64_t live = __ballot(lane < nblk_all && vmask_lds[lane] != 0u);
  const int nblk = live ? 64 - __clzll(live) : 0;
  int32_t* overflow_flag = phys + MLA_MAX_K;  // one int after the row list
  const v4f* Sx_peer = reinterpret_cast<const v4f*>(Sx) + (wave ^ 1) * 4 * WAVE + lane;
  // first two gathers of the first pass, then the queries (zero outside the heads and columns,
  // fp16 for fp16 staging), pinned to registers: no re-load from memory per block
  if (nblk > 0) gather(0);
  if (nblk > 1) gather(1);
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) {
    const int col = hf * C::DH + ks * 16 + lh * 8;
    s16x8 v = Qf[ks];
    if (!(head < H && col < DQK)) v = (s16x8){0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (F16) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = __builtin_bit_cast(short, (_Float16)__uint_as_float((uint32_t)(uint16_t)v[e] << 16));
    }
    asm volatile("" : "+v"(v));
    Qf[ks] = v;
  }
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) O[dt] = (v16f){};
    lsum = 0.f;
    // pass 1: the exact row maximum of pass 0; pass 0: unset, probabilities are 0 until a valid entry
    mref = pass ? fmaxf(mlane, __shfl_xor(mlane, 32)) * scale_log2 : INFINITY;
    bool have_ref = pass != 0;  // wave-uniform: all heads of a wave get their reference together
    bool overflow = false;

    if (pass > 0) {  // the first pass issued its first gathers before the queries were awaited
      if (nblk > 0) gather(0);
      if (nblk > 1) gather(1);
    }
    int32_t next_rows = 0;  // fp16 staging: rows of the gather issued in the next block
    if constexpr (F16) next_rows = gather_rows(2);
    int cur = 0;            // fp16 staging: stage of block blk
    for (int blk = 0; blk < nblk; ++blk) {
      const uint8_t* Kst = Kbuf + (F16 ? cur : blk % MLA_STAGES) * C::K_BYTES;
      // this wave's transfers of block blk are done once at most those of blk + 1 are pending
      if (blk + 1 < nblk) {
        // every wave issues DMA_PW or DMA_PW - 1 transfers per block: two immediate waits
        if (my_dma == DMA_PW)
          wait_vmcnt<DMA_PW>();
        else
          wait_vmcnt<DMA_PW - 1>();
      } else {
        wait_vmcnt<0>();
      }
      __syncthreads();  // stage blk complete; every wave is done with block blk - 1
      if constexpr (F16) {  // the stage of block blk - 1 is free: gather block blk + 2 into it
        if (blk + 2 < nblk) gather_issue(blk + 2, cur == 0 ? 2 : cur - 1, next_rows);
        next_rows = gather_rows(blk + 3);
      }

      // ---- bf16 staging: fp16 V^T of this block (VALU + LDS work) and the partial scores (MFMA
      // work).  The two waves of a SIMD (waves w and w + 4) run them in opposite orders, so one's
      // conversion runs beside the other's MFMAs instead of both waves doing the same kind of work
      // at once.  fp16 staging has no V^T to build.
      auto vt_build = [&]() {
      if (!F16 && converts) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {  // unit u = 2 m + lh: key quads 4 m + lh and 4 m + 2 + lh
          const int m = u >> 1, hh = u & 1;
          s16x8 vv;
          bf16x4_to_f16(lds_read_tr16(Kst + tr_off(4 * m + hh)), vv, 0);
          bf16x4_to_f16(lds_read_tr16(Kst + tr_off(4 * m + 2 + hh)), vv, 1);
          *reinterpret_cast<s16x8*>(vt_dst + 16 * u) = vv;
        }
      }

      };
      // bf16 staging: row indices of the next gather, read now so that they are in registers after
      // the barrier
      if constexpr (!F16) next_rows = gather_rows(blk + 2);
      // ---- partial S^T[key][head] over this wave's contraction half; the K fragment of step
      // ks + 1 is requested before the MFMA of step ks.  MFMA runs raise the wave's issue priority
      // so that the matrix pipe is fed first when both waves of the SIMD are ready.
      v16f sc;
      auto qk = [&]() {
      if (!active) {
        asm volatile("" : "=v"(sc));  // an inactive wave never reads its scores: no zeroing
      } else {
        __builtin_amdgcn_s_setprio(2);
        constexpr int LA = 3;  // K fragments in flight (order pinned by scheduling barriers)
        s16x8 Af[LA];
#pragma unroll
        for (int i = 0; i < LA - 1; ++i) Af[i] = *reinterpret_cast<const s16x8*>(Kst + kfrag_off(i));
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
          if (ks + LA - 1 < C::NKS) Af[(ks + LA - 1) % LA] = *reinterpret_cast<const s16x8*>(Kst + kfrag_off(ks + LA - 1));
          __builtin_amdgcn_sched_barrier(0);
          // the first product takes a zero accumulator operand (no register zeroing)
          if constexpr (F16)
            sc = mfma_f16_32x32x16(Af[ks % LA], Qf[ks], ks == 0 ? (v16f){} : sc);
          else
            sc = mfma_bf16_32x32x16(Af[ks % LA], Qf[ks], ks == 0 ? (v16f){} : sc);
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        v4f* dst = reinterpret_cast<v4f*>(Sx) + wave * 4 * WAVE + lane;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          dst[qd * WAVE] = (v4f){sc[4 * qd], sc[4 * qd + 1], sc[4 * qd + 2], sc[4 * qd + 3]};
      }
      };
      if constexpr (F16) {
        qk();
        __syncthreads();  // partial scores of both halves posted
        cur = cur == C::STAGES - 1 ? 0 : cur + 1;
      } else {
        if (wave >= MLA_WAVES / 2) {
          qk();
          vt_build();
        } else {
          vt_build();
          qk();
        }
        __syncthreads();  // partial scores of both halves posted; V^T complete; stage blk no longer read
        if (blk + 2 < nblk) gather_issue(blk + 2, blk % MLA_STAGES, next_rows);
      }
      if (!active) continue;

      // ---- full raw scores (own + partner partial), masked entries at -inf.  Element 4 qd + e
      // of a lane is key 8 qd + 4 lh + e: its validity is one bit of the block mask for each half
      // of the wave, so the lane mask of every element is built by two scalar bit-field extracts.
      const uint32_t vm = __builtin_amdgcn_readfirstlane(vmask_lds[blk]);
      if (vm == 0xFFFFFFFFu) {  // wave-uniform: every entry of the block is valid (no masks)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const v4f pv = Sx_peer[qd * WAVE];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = sc[4 * qd + e] + pv[e];
            sc[4 * qd + e] = v;
            mlane = fmaxf(mlane, v);
          }
        }
      } else {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const v4f pv = Sx_peer[qd * WAVE];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int rr = 4 * qd + e;
            const int bl = 8 * qd + e;
            const uint32_t lo = (uint32_t)((int32_t)(vm << (31 - bl)) >> 31);
            const uint32_t hi = (uint32_t)((int32_t)(vm << (27 - bl)) >> 31);
            const bool valid = __builtin_amdgcn_inverse_ballot_w64(((uint64_t)hi << 32) | lo);
            const float v = valid ? sc[rr] + pv[e] : -INFINITY;
            sc[rr] = v;
            mlane = fmaxf(mlane, v);
          }
        }
      }
      if (!have_ref && vm != 0u) {  // wave-uniform: the block mask is shared by all lanes
        // first block with a valid entry: its maximum becomes the reference (log2 units; the
        // scale is positive, so the maximum commutes with it)
        mref = fmaxf(mlane, __shfl_xor(mlane, 32)) * scale_log2;
        have_ref = true;
      }
      overflow |= mlane * scale_log2 > mref + MLA_HEADROOM;
      // ---- probabilities (fp16) packed as the B operands of out^T = V^T P^T (keys 0-15, 16-31)
      s16x8 Bp[2];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[rr], scale_log2, -mref));  // exp2(-inf) = 0
        lsum += p;
        Bp[rr >> 3][rr & 7] = __builtin_bit_cast(short, (_Float16)p);
      }
      // ---- out^T[d][head] += V^T[d][key] P^T[key][head]; consecutive MFMAs use different tiles,
      // fragments are requested one step ahead
      constexpr int NSTEP = C::NDT * 2;
      const uint8_t* vsrc = Vt + (hf * C::DVH + l32) * C::VT_STRIDE + 16 * lh;
      auto vfrag = [&](int st) {  // step st: key half m = st / NDT, value tile dt = st % NDT
        const int m = st / C::NDT, dt = st % C::NDT;
        if constexpr (F16) {
          const uint8_t* p = Kst + m * 16 * C::RC * 16 + (dt >> 1) * 128;
          const s16x4 lo = lds_read_tr16(p + vb[0][dt & 1]), hi = lds_read_tr16(p + vb[1][dt & 1]);
          return (s16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
          return *reinterpret_cast<const s16x8*>(vsrc + dt * 32 * C::VT_STRIDE + 32 * m);
        }
      };
      __builtin_amdgcn_s_setprio(2);
      constexpr int LV = 3;  // V^T fragments in flight (order pinned by scheduling barriers)
      s16x8 Vf[LV];
#pragma unroll
      for (int i = 0; i < LV - 1; ++i) Vf[i] = vfrag(i);
#pragma unroll
      for (int st = 0; st < NSTEP; ++st) {
        if (st + LV - 1 < NSTEP) Vf[(st + LV - 1) % LV] = vfrag(st + LV - 1);
        __builtin_amdgcn_sched_barrier(0);
        O[st % C::NDT] = mfma_f16_32x32x16(Vf[st % LV], Bp[st / C::NDT], O[st % C::NDT]);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
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
  if (!active || head >= H) return;

  // ---- normalise and store: element rr of tile dt is value column f DV/2 + 32 dt + 8 (rr / 4)
  // + 4 lh + rr % 4 of head `head`
  const float l = lsum + __shfl_xor(lsum, 32);
  const float inv = l > 0.f ? 1.0f / l : 0.0f;
  const float lse_v = l > 0.f ? (mref + log2f(l)) * 0.69314718055994531f : -INFINITY;
  if (nsplit == 1) {
    uint16_t* orow = out + (r * H + head) * (int64_t)DV;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int d = hf * C::DVH + dt * 32 + 8 * qd + 4 * lh;
        const v4f o = (v4f){O[dt][4 * qd], O[dt][4 * qd + 1], O[dt][4 * qd + 2], O[dt][4 * qd + 3]} * inv;
        *reinterpret_cast<v2i*>(orow + d) = (v2i){(int)f32x2_to_bf16x2(o[0], o[1]), (int)f32x2_to_bf16x2(o[2], o[3])};
        if (out_f32) *reinterpret_cast<v4f*>(out_f32 + (r * H + head) * (int64_t)DV + d) = o;
      }
    if (hf == 0 && lh == 0 && lse) lse[r * H + head] = lse_v;
  } else {
    float* prow = part_out + ((r * nsplit + sp) * (int64_t)H + head) * DV;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int d = hf * C::DVH + dt * 32 + 8 * qd + 4 * lh;
        *reinterpret_cast<v4f*>(prow + d) =
            (v4f){O[dt][4 * qd], O[dt][4 * qd + 1], O[dt][4 * qd + 2], O[dt][4 * qd + 3]} * inv;
      }
    if (hf == 0 && lh == 0) part_lse[(r * nsplit + sp) * (int64_t)H + head] = lse_v;
  }
}

// Re-reduction of split partials in fp32: out = sum_s w_s out_s / sum_s w_s, w_s = exp(lse_s - max).
// One workgroup per (row, group of heads); each thread owns four consecutive output columns of
// one head, so the partial rows stream with 16-byte loads from many workgroups at once.
constexpr int COMBINE_THREADS = 256;

template <int DV>
__global__ __launch_bounds__(COMBINE_THREADS) void mla_combine_kernel(const float* __restrict__ part_out,
                                                                      const float* __restrict__ part_lse,
                                                                      int32_t nsplit, int32_t H,
                                                                      uint16_t* __restrict__ out,
                                                                      float* __restrict__ out_f32,
                                                                      float* __restrict__ lse) {
  constexpr int TPH = DV / 4;                  // threads per head
  constexpr int HPB = COMBINE_THREADS / TPH;   // heads per workgroup
  const int64_t r = blockIdx.x;
  const int h = blockIdx.y * HPB + (int)threadIdx.x / TPH;
  if (h >= H) return;
  const int d = ((int)threadIdx.x % TPH) * 4;
  const float* pl = part_lse + r * nsplit * (int64_t)H + h;           // split s at pl[s * H]
  const float* po = part_out + (r * nsplit * (int64_t)H + h) * DV + d;  // split s at po[s * H * DV]
  float m = -INFINITY;
  for (int s = 0; s < nsplit; ++s) m = fmaxf(m, pl[(int64_t)s * H]);
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (m != -INFINITY) {
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) {
      const float ls = pl[(int64_t)s * H];
      const float wgt = ls == -INFINITY ? 0.f : expf(ls - m);
      wsum += wgt;
      const v4f v = *reinterpret_cast<const v4f*>(po + (int64_t)s * H * DV);
      acc += wgt * v;
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  const v4f o = acc * inv;
  *reinterpret_cast<v2i*>(out + (r * H + h) * (int64_t)DV + d) =
      (v2i){(int)f32x2_to_bf16x2(o[0], o[1]), (int)f32x2_to_bf16x2(o[2], o[3])};
  if (out_f32) *reinterpret_cast<v4f*>(out_f32 + (r * H + h) * (int64_t)DV + d) = o;
  if (d == 0 && lse) lse[r * H + h] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
}

// fp16 copy of the latent rows for the fp16-staged attention: logical rows [0, rows) of one sequence
// (through its block table, or contiguous) -> dst [rows][D] fp16, round to nearest even (exact for
// |v| in [2^-17, 65504]; smaller magnitudes land on fp16's 2^-24 grid, larger ones overflow).
// Each thread converts 16-byte chunks (8 values), grid-stride.
constexpr int KV16_THREADS = 256;
__global__ __launch_bounds__(KV16_THREADS) void mla_kv_to_f16_kernel(const uint16_t* __restrict__ kv, RowMap map,
                                                                   int64_t rows, int32_t D,
                                                                   uint16_t* __restrict__ dst) {
  const int cpr = D / 8;  // chunks per row
  const int64_t n = rows * cpr;
  for (int64_t c = (int64_t)blockIdx.x * KV16_THREADS + threadIdx.x; c < n; c += (int64_t)gridDim.x * KV16_THREADS) {
    const int64_t row = c / cpr;
    const int ch = (int)(c - row * cpr);
    const v4i w = *reinterpret_cast<const v4i*>(kv + map(row) * D + ch * 8);
    v4i o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = (uint32_t)w[e];
      const _Float16 lo = (_Float16)__uint_as_float(u << 16), hi = (_Float16)__uint_as_float(u & 0xFFFF0000u);
      o[e] = (int)((uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16));
    }
    *reinterpret_cast<v4i*>(dst + row * D + ch * 8) = o;
  }
}

size_t mla_kv16_bytes(int64_t S, int32_t D_qk, int32_t D_v) {
  return (D_qk == 576 && D_v == 512 && S > 0) ? (size_t)S * D_qk * sizeof(uint16_t) : 0;
}

// ---------------------------------------------------------------------------------------------
template <int DQK, int DV, bool F16>
static hipError_t launch_mla_kernel(const MlaArgs& a, const uint16_t* kv, const int32_t* table, int64_t kv_rows,
                                    int nsplit, int kps, hipStream_t stream) {
  const size_t smem = mla_smem_bytes<DQK, DV, F16>(kps);
  // rows of the latent cache the gather may name: the paged pool, or the contiguous keys
  const bool off32 = (uint64_t)kv_rows * DQK * 2 <= 0xFFFFFFFFull;
  auto kernel = off32 ? sparse_mla_kernel<DQK, DV, true, F16> : sparse_mla_kernel<DQK, DV, false, F16>;
  hipError_t e = set_max_dynamic_lds((const void*)kernel);
  if (e != hipSuccess) return e;
  const float scale_log2 = a.sm_scale * 1.4426950408889634f;
  dim3 grid((unsigned)a.R, (unsigned)nsplit);
  return launch("sparse_mla_kernel", kernel, grid, dim3(MLA_THREADS), smem, stream, a.q, kv, a.idx, table,
                a.max_blocks, a.block_shift, a.num_blocks, a.per_row_table, a.seq_lens, a.S, a.q_start, a.H, a.k,
                scale_log2, nsplit, kps, a.out, a.out_f32, a.lse, a.part_out, a.part_lse);
}

template <int DQK, int DV>
static hipError_t launch_mla_t(const MlaArgs& a, hipStream_t stream) {
  const int nsplit = a.nsplit;
  const int kps = (a.k + nsplit - 1) / nsplit;
  hipError_t e;
  if constexpr (DQK == 576 && DV == 512) {
    if (a.kv_f16 && !a.per_row_table) {
      // one sequence's S rows -> contiguous fp16, then the fp16-staged kernel over them
      const int64_t chunks = a.S * (DQK / 8);
      const int64_t want = (chunks + KV16_THREADS - 1) / KV16_THREADS;
      const unsigned g = (unsigned)std::max<int64_t>(std::min<int64_t>(want, 8192), 1);  // grid-stride beyond
      e = launch("mla_kv_to_f16_kernel", mla_kv_to_f16_kernel, dim3(g), dim3(KV16_THREADS), 0,
                 stream, a.kv, RowMap{a.table, a.block_shift, a.num_blocks}, a.S, (int32_t)DQK, a.kv_f16);
      if (e != hipSuccess) return e;
      e = launch_mla_kernel<DQK, DV, true>(a, a.kv_f16, nullptr, a.S, nsplit, kps, stream);
    } else {
      e = launch_mla_kernel<DQK, DV, false>(a, a.kv, a.table, a.table ? (a.num_blocks << a.block_shift) : a.S,
                                            nsplit, kps, stream);
    }
  } else {
    e = launch_mla_kernel<DQK, DV, false>(a, a.kv, a.table, a.table ? (a.num_blocks << a.block_shift) : a.S,
                                          nsplit, kps, stream);
  }
  if (e != hipSuccess || nsplit == 1) return e;
  constexpr int HPB = COMBINE_THREADS / (DV / 4);
  return launch("mla_combine_kernel", mla_combine_kernel<DV>, dim3((unsigned)a.R, (unsigned)((a.H + HPB - 1) / HPB)),
                dim3(COMBINE_THREADS), 0, stream, a.part_out, a.part_lse, nsplit, a.H, a.out, a.out_f32, a.lse);
}

bool mla_supported(int32_t D_qk, int32_t D_v, int32_t H, int32_t k) {
  const bool dims = (D_qk == 576 && D_v == 512) || (D_qk == 80 && D_v == 64);
  return dims && H >= 1 && H <= MLA_GROUPS * MLA_GROUP_HEADS && k >= 1 && k <= MLA_MAX_K;
}

hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t stream) {
  if (a.R <= 0) return hipSuccess;
  if (a.D_qk == 576 && a.D_v == 512) return launch_mla_t<576, 512>(a, stream);
  if (a.D_qk == 80 && a.D_v == 64) return launch_mla_t<80, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dsa
