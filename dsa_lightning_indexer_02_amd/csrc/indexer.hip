// Lightning-indexer scoring on gfx950 (DeepSeek-V3.2-Exp summary page, section "Method";
// AMD MI355X DeepSeek-V3.2-Exp article, section "DeepSeek Sparse Attention (DSA)"):
//
//   I[t,s] = ks[s] * sum_j (w[t,j] * qs[t,j]) * ReLU( dec(q8[t,j,:]) . dec(k8[s,:]) )
//
// which equals sum_j w[t,j] * ReLU(q_I[t,j] . k_I[s]) for the dequantized vectors because
// the per-row scales are positive.  The FP8 dot products run on the 16x16x128 FP8 MFMA
// (one instruction covers D_I <= 128); ReLU, the weighted head sum and the key scale are
// applied in fp32 registers.  Only causally visible entries s < min(S, pos_t + 1) are written.
#include "dsa_internal.hpp"

namespace dsa {

// ---------------------------------------------------------------------------------------
// Prefill: a workgroup owns 16 consecutive query rows (the MFMA M dimension) and a range of
// keys.  The 16 rows' FP8 queries for every head sit in LDS ([head][row][128 B + pad]); the
// NW waves take disjoint 16-key tiles, keep NK tiles of keys in registers (MFMA B operand)
// and loop over the heads, so the head reduction happens inside each lane's accumulators
// without any cross-lane traffic.
// ---------------------------------------------------------------------------------------
constexpr int IDX_ROWS = 16;
constexpr int IDX_QROW_BYTES = 144;  // 128 B of codes + 16 B pad (bank spread)

// HI > 0: the head count is a compile-time constant and the head loop is fully unrolled;
// HI == 0: any head count (plain loop).
// E8: the per-row scales are power-of-two exponents (UE8M0: q_exp [T][H_I], k_exp [S], value
// 2^(e - 127)) applied inside the MFMA as its operand scales (lane l's byte scales the row or
// column l % 16 it supplies), so the epilogue weighs by w alone and applies no key scale; qs and
// ks are not read.  Otherwise the fp32 scales qs, ks are applied in the epilogue.
template <int NW, int NK, int HI, bool E8>
__global__ __launch_bounds__(NW * WAVE) void indexer_prefill_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k8, const float* __restrict__ ks, RowMap keymap, int64_t T,
    int64_t S, int32_t H_I, int32_t D_I, int64_t q_start, float* __restrict__ logits, int64_t ld,
    int64_t key_chunk, const uint8_t* __restrict__ q_exp, const uint8_t* __restrict__ k_exp) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* qtile = smem;                                                        // [H_I][16][144]
  float* wq = reinterpret_cast<float*>(smem + (size_t)H_I * IDX_ROWS * IDX_QROW_BYTES);  // [H_I][16]
  uint8_t* qe = reinterpret_cast<uint8_t*>(wq + H_I * IDX_ROWS);                // E8: [H_I][16]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int j16 = lane & 15, g = lane >> 4;
  // heaviest tiles (latest rows) first
  const int64_t tile = (int64_t)gridDim.y - 1 - blockIdx.y;
  const int64_t t0 = tile * IDX_ROWS;
  const int64_t n_max = min(S, q_start + min(t0 + IDX_ROWS, T));  // keys the tile needs
  const int64_t c0 = (int64_t)blockIdx.x * key_chunk;
  if (c0 >= n_max) return;
  const int64_t c1 = min(n_max, c0 + key_chunk);

  // ---- stage the 16 rows' queries and weights
  const int chunks_per_row = D_I >> 4;  // 16-byte pieces of one head vector
  for (int p = tid; p < H_I * IDX_ROWS * 8; p += blockDim.x) {
    const int piece = p & 7, row = (p >> 3) & (IDX_ROWS - 1), head = p >> 7;
    const int64_t t = t0 + row;
    v4i v = {0, 0, 0, 0};
    if (t < T && piece < chunks_per_row)
      v = *reinterpret_cast<const v4i*>(q8 + ((t * H_I + head) * D_I) + piece * 16);
    *reinterpret_cast<v4i*>(qtile + (head * IDX_ROWS + row) * IDX_QROW_BYTES + piece * 16) = v;
  }
  for (int p = tid; p < H_I * IDX_ROWS; p += blockDim.x) {
    const int row = p & (IDX_ROWS - 1), head = p >> 4;
    const int64_t t = t0 + row;
    if constexpr (E8) {
      wq[head * IDX_ROWS + row] = t < T ? w[t * H_I + head] : 0.0f;
      qe[head * IDX_ROWS + row] = t < T ? q_exp[t * H_I + head] : (uint8_t)127;
    } else {
      wq[head * IDX_ROWS + row] = t < T ? w[t * H_I + head] * qs[t * H_I + head] : 0.0f;
    }
  }
  __syncthreads();

  const bool klane_has_bytes = (g * 32) < D_I;
  const int64_t pass_keys = (int64_t)NW * NK * 16;
  // key tiles of one pass (MFMA B operands) and their scales (E8: exponent bytes)
  auto load_keys = [&](int64_t base, v8i (&B)[NK], float (&ksv)[NK], int (&kb)[NK]) {
#pragma unroll
    for (int kt = 0; kt < NK; ++kt) {
      const int64_t s = min(base + kt * 16 + j16, S - 1);
      const int64_t row = keymap(s);
      v8i b = {0, 0, 0, 0, 0, 0, 0, 0};
      if (klane_has_bytes) b = *reinterpret_cast<const v8i*>(k8 + row * D_I + g * 32);
      B[kt] = b;
      if constexpr (E8)
        kb[kt] = k_exp[row];
      else
        ksv[kt] = ks[row];
    }
  };
  for (int64_t base = c0 + (int64_t)wave * NK * 16; base < c1; base += pass_keys) {
    v8i B[NK];
    float ksv[NK];
    int kb[NK];
    load_keys(base, B, ksv, kb);
    v4f acc[NK];
#pragma unroll
    for (int kt = 0; kt < NK; ++kt) acc[kt] = (v4f){0.f, 0.f, 0.f, 0.f};

    auto relu_acc = [&](const v4f& wv, const v4f (&c)[NK]) {
#pragma unroll
      for (int kt = 0; kt < NK; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[kt][r] = fmaf(wv[r], __builtin_amdgcn_fmed3f(c[kt][r], 0.f, 3.402823466e38f), acc[kt][r]);
    };
    auto load_a = [&](int head) {
      return *reinterpret_cast<const v8i*>(qtile + (head * IDX_ROWS + j16) * IDX_QROW_BYTES + g * 32);
    };
    auto load_sa = [&](int head) { return E8 ? (int)qe[head * IDX_ROWS + j16] : 0; };
    auto mfma = [&](const v8i& A, int sa, int kt) {
      if constexpr (E8)
        return mfma_fp8_16x16x128_scaled(A, B[kt], (v4f){0.f, 0.f, 0.f, 0.f}, sa, kb[kt]);
      else
        return mfma_fp8_16x16x128(A, B[kt], (v4f){0.f, 0.f, 0.f, 0.f});
    };
    auto load_w = [&](int head) { return *reinterpret_cast<const v4f*>(wq + head * IDX_ROWS + 4 * g); };
    if constexpr (HI > 0) {
      // Software pipeline over the heads, two per iteration with static slots (last iteration
      // peeled, so the body has no conditions): the MFMAs of head h + 1 are issued before the
      // ReLU and weighted accumulation of head h, so the matrix core and the VALU work side by
      // side; the order is pinned with scheduling barriers.  ReLU is one med3(c, 0, FLT_MAX)
      // (the products are finite).
      static_assert(HI % 2 == 0 && HI >= 2, "even head count");
      v4f c0[NK], c1[NK];
      v8i A0 = load_a(0), A1;
      v4f w0 = load_w(0), w1;
      int s0 = load_sa(0), s1;
      auto mma = [&](const v8i& A, int sa, v4f (&c)[NK]) {
#pragma unroll
        for (int kt = 0; kt < NK; ++kt) c[kt] = mfma(A, sa, kt);
      };
      mma(A0, s0, c0);
      for (int head = 0; head < HI - 2; head += 2) {
        A1 = load_a(head + 1);
        w1 = load_w(head + 1);
        s1 = load_sa(head + 1);
        __builtin_amdgcn_sched_barrier(0);
        mma(A1, s1, c1);      // head + 1
        relu_acc(w0, c0);     // head
        __builtin_amdgcn_sched_barrier(0);
        A0 = load_a(head + 2);
        w0 = load_w(head + 2);
        s0 = load_sa(head + 2);
        __builtin_amdgcn_sched_barrier(0);
        mma(A0, s0, c0);      // head + 2
        relu_acc(w1, c1);     // head + 1
        __builtin_amdgcn_sched_barrier(0);
      }
      A1 = load_a(HI - 1);
      w1 = load_w(HI - 1);
      s1 = load_sa(HI - 1);
      __builtin_amdgcn_sched_barrier(0);
      mma(A1, s1, c1);
      relu_acc(w0, c0);
      relu_acc(w1, c1);
    } else {
      for (int head = 0; head < H_I; ++head) {
        const v8i A = load_a(head);
        const v4f wv = load_w(head);
        const int sa = load_sa(head);
        v4f c[NK];
#pragma unroll
        for (int kt = 0; kt < NK; ++kt) c[kt] = mfma(A, sa, kt);
        relu_acc(wv, c);
      }
    }
    // lane (j16, g) holds rows t0 + 4g + r for key base + 16 kt + j16
    if (base + NK * 16 <= c1 && base + NK * 16 <= q_start + t0 + 1 && t0 + IDX_ROWS <= T) {
      // every (row, key) of the pass is visible (wave-uniform): no per-element test, one row
      // pointer per r and the key tile as an immediate offset
      float* lrow = logits + (t0 + 4 * g) * ld + base + j16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int kt = 0; kt < NK; ++kt) lrow[kt * 16] = E8 ? acc[kt][r] : acc[kt][r] * ksv[kt];
        lrow += ld;
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < NK; ++kt) {
        const int64_t s = base + kt * 16 + j16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t t = t0 + 4 * g + r;
          if (t < T && s < c1 && s < q_start + t + 1) logits[t * ld + s] = E8 ? acc[kt][r] : acc[kt][r] * ksv[kt];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Decode: one query row per sequence.  The 64 (padded to a multiple of 16) heads are the MFMA
// M dimension, held in registers; a wave scores 64 keys of one sequence at a time (four 16-key
// tiles), and the head sum is a lane-local accumulation followed by a reduction over the four
// lane groups.
//
// The work is a stream of FP8 keys whose amount per sequence is only known on the device, so
// the kernel balances it itself: every workgroup forms the prefix sum of the sequences' 64-key
// group counts in LDS, and each wave of the (resident-sized) grid takes an equal contiguous
// share of the flat list of groups.  A wave resolves up to 64 of its groups at a time, one per
// lane (sequence, first key, and, when a block holds at least 64 rows so that a group never
// straddles two blocks, the group's physical row from the block table), and picks them up with
// readlane; it issues the loads of its next group before scoring the current one.  With blocks
// of fewer than 64 rows each lane looks its rows up inside the group load.
// ---------------------------------------------------------------------------------------
constexpr int IDX_DECODE_WAVES = 4;
constexpr int IDX_DECODE_THREADS = IDX_DECODE_WAVES * WAVE;
#ifndef IDX_DECODE_DEPTH
#define IDX_DECODE_DEPTH 3                 // 64-key groups in flight per wave
#endif

__device__ __forceinline__ int64_t readlane64(int64_t v, int j) {
  const int lo = __builtin_amdgcn_readlane((int)(uint32_t)v, j);
  const int hi = __builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), j);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const int lo = __builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const int hi = __builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

__device__ __forceinline__ int64_t shfl_up64(int64_t v, int o) {
  const int lo = __shfl_up((int)(uint32_t)v, o);
  const int hi = __shfl_up((int)(uint32_t)((uint64_t)v >> 32), o);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

template <int NHT>
__global__ __launch_bounds__(IDX_DECODE_THREADS, 2) void indexer_decode_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k8, const float* __restrict__ ks, const int32_t* __restrict__ table,
    int64_t max_blocks, int32_t block_shift, int64_t num_blocks, const int32_t* __restrict__ seq_lens, int32_t B,
    int32_t H_I, int32_t D_I, int64_t max_len, float* __restrict__ logits, int64_t ld) {
  extern __shared__ __align__(16) uint8_t smem[];
  int64_t* gstart = reinterpret_cast<int64_t*>(smem);                      // [B + 1] group prefix
  int32_t* nlen = reinterpret_cast<int32_t*>(smem + (size_t)(B + 1) * 8);  // [B] visible keys
  __shared__ int64_t wave_tot[IDX_DECODE_WAVES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j16 = lane & 15, g = lane >> 4;

  // ---- prefix sum of per-sequence group counts (each thread a contiguous slice of sequences)
  const int per = (B + IDX_DECODE_THREADS - 1) / IDX_DECODE_THREADS;
  const int sb0 = tid * per;
  int64_t mine = 0;
  for (int i = 0; i < per; ++i) {
    const int bb = sb0 + i;
    if (bb < B) {
      const int64_t n = min((int64_t)max(seq_lens[bb], 0), max_len);
      nlen[bb] = (int32_t)n;
      mine += (n + 63) >> 6;
    }
  }
  int64_t incl = mine;
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) {
    const int64_t t = shfl_up64(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == WAVE - 1) wave_tot[wave] = incl;
  __syncthreads();
  int64_t run = incl - mine;
  for (int v = 0; v < wave; ++v) run += wave_tot[v];
  for (int i = 0; i < per; ++i) {
    const int bb = sb0 + i;
    if (bb < B) {
      gstart[bb] = run;
      run += ((int64_t)nlen[bb] + 63) >> 6;
    }
  }
  if (tid == 0) {
    int64_t tot = 0;
    for (int v = 0; v < IDX_DECODE_WAVES; ++v) tot += wave_tot[v];
    gstart[B] = tot;
  }
  __syncthreads();

  // ---- this wave's share of the flat group list
  const int64_t total = uniform64(gstart[B]);
  const int64_t nw = (int64_t)gridDim.x * IDX_DECODE_WAVES;
  const int64_t wg = (int64_t)blockIdx.x * IDX_DECODE_WAVES + wave;
  const int64_t f_beg = total * wg / nw, f_end = total * (wg + 1) / nw;
  if (f_beg >= f_end) return;

  // lane i of the window describes flat group ws + i
  int64_t ws = f_beg;
  int32_t wb = 0, wn = 0;
  int64_t wbase = 0, wrow = 0;
  auto window = [&](int64_t start) {
    ws = start;
    const int64_t f = start + lane;
    wb = 0;
    wn = 0;
    wbase = 0;
    wrow = 0;
    if (f < f_end) {
      int lo = 0, hi = B;  // gstart[lo] <= f < gstart[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (gstart[mid] <= f) lo = mid; else hi = mid;
      }
      wb = lo;
      wn = nlen[lo];
      wbase = (f - gstart[lo]) * 64;
      wrow = wbase;
      if (table && block_shift >= 6)
        wrow = (safe_block(table[(int64_t)lo * max_blocks + (wbase >> block_shift)], num_blocks) << block_shift) |
               (wbase & ((1 << block_shift) - 1));
    }
  };

  struct Grp {
    int32_t b, n;
    int64_t base, row0;
  };
  auto get = [&](int64_t f) {
    const int j = (int)(f - ws);
    return Grp{__builtin_amdgcn_readlane(wb, j), __builtin_amdgcn_readlane(wn, j), readlane64(wbase, j),
               readlane64(wrow, j)};
  };

  v8i A[NHT];
  float wv[NHT][4];
  const bool has_bytes = (g * 32) < D_I;
  const int kofs = has_bytes ? g * 32 : D_I - 32;
  auto load_query = [&](int64_t b) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int head = ht * 16 + j16;
      v8i a = {0, 0, 0, 0, 0, 0, 0, 0};
      if (head < H_I && has_bytes) a = *reinterpret_cast<const v8i*>(q8 + ((b * H_I + head) * D_I) + g * 32);
      A[ht] = a;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int hr = ht * 16 + 4 * g + r;
        wv[ht][r] = hr < H_I ? w[b * H_I + hr] * qs[b * H_I + hr] : 0.0f;
      }
    }
    // Complete these loads here: left pending past the branch that calls this, they would make
    // the scoring after it wait for every load in flight, the next group's prefetch included.
    // (one dword of each 16-byte load; a whole-vector operand would not pass the host compile)
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) asm volatile("" ::"v"(A[ht][0]), "v"(A[ht][4]));
  };

  // keys base .. base+63 of the group (clamped to its last visible key) into registers, and the
  // scale of the one key this lane stores (key base + 16 g + j16)
  auto load = [&](const Grp& gr, v8i (&Bk)[4], float& kme) {
    int64_t row[4], rme;
    const int64_t sme = min(gr.base + g * 16 + j16, (int64_t)gr.n - 1);
    if (!table || block_shift >= 6) {
#pragma unroll
      for (int q = 0; q < 4; ++q) row[q] = gr.row0 + (min(gr.base + q * 16 + j16, (int64_t)gr.n - 1) - gr.base);
      rme = gr.row0 + (sme - gr.base);
    } else {
      const int32_t* tb = table + (int64_t)gr.b * max_blocks;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t s = min(gr.base + q * 16 + j16, (int64_t)gr.n - 1);
        row[q] = (safe_block(tb[s >> block_shift], num_blocks) << block_shift) | (s & ((1 << block_shift) - 1));
      }
      rme = (safe_block(tb[sme >> block_shift], num_blocks) << block_shift) | (sme & ((1 << block_shift) - 1));
    }
    // Every lane loads, so no per-lane branch splits the group's loads: lanes whose k-range lies
    // past D_I re-read the row's last 32 bytes (finite codes of the same key), which meet zero
    // query bytes in the MFMA.
#pragma unroll
    for (int q = 0; q < 4; ++q) Bk[q] = *reinterpret_cast<const v8i*>(k8 + row[q] * D_I + kofs);
    kme = ks[rme];
  };

  int32_t cur_b = -1;
  auto score = [&](const Grp& gr, const v8i (&Bk)[4], float kme) {
    if (gr.b != cur_b) {
      load_query(gr.b);
      cur_b = gr.b;
    }
    float res[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v4f c[NHT];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) c[ht] = mfma_fp8_16x16x128(A[ht], Bk[q], (v4f){0.f, 0.f, 0.f, 0.f});
      float acc = 0.f;
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc = fmaf(wv[ht][r], __builtin_amdgcn_fmed3f(c[ht][r], 0.f, 3.402823466e38f), acc);
      res[q] = wave_sum_xor16_32(acc);
      // computed here, not sunk into the lane-group select below (whose divergent branches
      // would otherwise wait for every load in flight)
      asm volatile("" : "+v"(res[q]));
    }
    // lane group g stores tile g: 64 consecutive keys per store
    float v = (g == 0 ? res[0] : g == 1 ? res[1] : g == 2 ? res[2] : res[3]) * kme;
    asm volatile("" : "+v"(v));  // scaled before, not inside, the store's branch
    const int64_t s = gr.base + g * 16 + j16;
    if (s < gr.n) logits[(int64_t)gr.b * ld + s] = v;
  };

  // next group's descriptor, refilling the window when it runs out
  auto advance = [&](int64_t f) {
    if (f - ws >= WAVE) window(f);
    return get(f);
  };

  // IDX_DECODE_DEPTH groups in flight per wave, in rotating register sets (the rotation is
  // unrolled so every set has fixed registers).  The loads of group f + DEPTH are issued
  // unconditionally before group f is scored (past the wave's last group they re-read the
  // current one, which is cache-hot): a load under a branch would leave the compiler's wait
  // counts for the joined paths at those of the path without it, i.e. waiting for the prefetch.
  constexpr int NB = IDX_DECODE_DEPTH + 1;
  v8i Bk[NB][4];
  float km[NB];
  Grp gq[NB];
  window(f_beg);
  gq[0] = get(f_beg);
#pragma unroll
  for (int d = 1; d < IDX_DECODE_DEPTH; ++d) gq[d] = f_beg + d < f_end ? advance(f_beg + d) : gq[d - 1];
#pragma unroll
  for (int d = 0; d < IDX_DECODE_DEPTH; ++d) load(gq[d], Bk[d], km[d]);
  for (int64_t f = f_beg;;) {
    bool done = false;
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      constexpr int D = IDX_DECODE_DEPTH;
      const int ls = (r + D) % NB;
      gq[ls] = f + D < f_end ? advance(f + D) : gq[r];
      load(gq[ls], Bk[ls], km[ls]);
      score(gq[r], Bk[r], km[r]);
      if (++f >= f_end) {
        done = true;
        break;
      }
    }
    if (done) break;
  }
}

// ---------------------------------------------------------------------------------------
size_t indexer_prefill_smem(int32_t H_I, bool e8) {
  return (size_t)H_I * IDX_ROWS * IDX_QROW_BYTES + (size_t)H_I * IDX_ROWS * sizeof(float) +
         (e8 ? (size_t)H_I * IDX_ROWS : 0);
}

int64_t indexer_prefill_max_rows() { return (int64_t)IDX_ROWS * 65536; }

template <int NW, int NK>
static hipError_t launch_indexer_prefill_cfg(const uint8_t* q8, const float* qs, const float* w,
                                  const uint8_t* k8, const float* ks, const int32_t* table,
                                  int32_t block_shift, int64_t num_blocks, int64_t T, int64_t S, int32_t H_I, int32_t D_I,
                                  int64_t q_start, float* logits, int64_t ld, hipStream_t stream,
                                  const uint8_t* q_exp, const uint8_t* k_exp) {
  const int64_t tiles = (T + IDX_ROWS - 1) / IDX_ROWS;
  const int64_t n_last = std::min<int64_t>(S, q_start + T);
  // split keys only when the tiles alone cannot fill the chip
  int64_t key_chunk = n_last;
  const int64_t unit = (int64_t)NW * NK * 16;
  if (tiles < 1024) {
    int64_t want = (1024 + tiles - 1) / tiles;
    key_chunk = std::max<int64_t>(unit, ((n_last + want - 1) / want + unit - 1) / unit * unit);
  }
  key_chunk = std::max<int64_t>(key_chunk, 1);
  const int64_t chunks = (n_last + key_chunk - 1) / key_chunk;
  dim3 grid((unsigned)chunks, (unsigned)tiles);
  const bool e8 = q_exp != nullptr;
  const size_t smem = indexer_prefill_smem(H_I, e8);
  auto kernel = e8 ? (H_I == 64 ? indexer_prefill_kernel<NW, NK, 64, true> : indexer_prefill_kernel<NW, NK, 0, true>)
                   : (H_I == 64 ? indexer_prefill_kernel<NW, NK, 64, false> : indexer_prefill_kernel<NW, NK, 0, false>);
  hipError_t e = set_max_dynamic_lds((const void*)kernel);
  if (e != hipSuccess) return e;
  return launch(e8 ? "indexer_prefill_kernel<e8m0>" : "indexer_prefill_kernel", kernel, grid,
                dim3(NW * WAVE), smem, stream, q8, qs, w, k8, ks, RowMap{table, block_shift, num_blocks},
                T, S, H_I, D_I, q_start, logits, ld, key_chunk, q_exp, k_exp);
}

hipError_t launch_indexer_prefill(const uint8_t* q8, const float* qs, const float* w,
                                  const uint8_t* k8, const float* ks, const int32_t* table,
                                  int32_t block_shift, int64_t num_blocks, int64_t T, int64_t S, int32_t H_I, int32_t D_I,
                                  int64_t q_start, float* logits, int64_t ld, hipStream_t stream,
                                  const uint8_t* q_exp, const uint8_t* k_exp) {
  if (T <= 0) return hipSuccess;
  // Long key ranges (16384 keys or more): eight waves (two per SIMD) of eight 16-key tiles, each
  // wave's VALU beside the other's MFMAs; shorter ones: twelve waves of four tiles, whose smaller
  // passes split the causal triangle into more, better balanced workgroups.
  const int64_t n_last = std::min<int64_t>(S, q_start + T);
  return n_last >= 16384 ? launch_indexer_prefill_cfg<8, 8>(q8, qs, w, k8, ks, table, block_shift, num_blocks, T, S,
                                                           H_I, D_I, q_start, logits, ld, stream, q_exp, k_exp)
                         : launch_indexer_prefill_cfg<12, 4>(q8, qs, w, k8, ks, table, block_shift, num_blocks, T, S,
                                                            H_I, D_I, q_start, logits, ld, stream, q_exp, k_exp);
}

// Dynamic LDS of the decode indexer: the group prefix [B + 1] i64 and the visible lengths [B] i32.
static size_t indexer_decode_smem(int32_t B) { return (size_t)(B + 1) * 8 + (size_t)B * 4; }
static_assert((kDecodeMaxSeqs + 1) * 8 + kDecodeMaxSeqs * 4 + 64 <= 160 * 1024,
              "the decode prefix table of the largest batch fits gfx950's LDS");

hipError_t launch_indexer_decode(const uint8_t* q8, const float* qs, const float* w,
                                 const uint8_t* k8, const float* ks, const int32_t* table,
                                 int64_t max_blocks, int32_t block_shift, int64_t num_blocks,
                                 const int32_t* seq_lens, int32_t B, int64_t max_len, int32_t H_I, int32_t D_I,
                                 float* logits, int64_t ld, hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  if (B > kDecodeMaxSeqs) return hipErrorInvalidValue;
  const int nht = (H_I + 15) / 16;
  auto kernel = nht <= 1 ? indexer_decode_kernel<1> : nht <= 2 ? indexer_decode_kernel<2> : indexer_decode_kernel<4>;
  const size_t smem = indexer_decode_smem(B);
  hipError_t e = set_max_dynamic_lds((const void*)kernel);
  if (e != hipSuccess) return e;
  // a grid of exactly the resident workgroups: the waves split the work evenly among themselves.
  // Residency = min(the register / static-LDS bound, LDS per CU / this call's dynamic LDS), from
  // values cached once per device.
  DeviceProps props;
  e = device_props(&props);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = occupancy_without_lds((const void*)kernel, IDX_DECODE_THREADS, &per_cu);
  if (e != hipSuccess) return e;
  per_cu = std::max(1, std::min<int>(per_cu, (int)(props.lds_per_cu / (smem + 64))));
  const int64_t groups_max = (int64_t)B * ((max_len + 63) / 64);
  const int64_t need = (groups_max + IDX_DECODE_WAVES - 1) / IDX_DECODE_WAVES;
  const int64_t nwg = std::max<int64_t>(1, std::min<int64_t>((int64_t)per_cu * props.cu_count, need));
  return launch("indexer_decode_kernel", kernel, dim3((unsigned)nwg), dim3(IDX_DECODE_THREADS), smem, stream, q8,
                qs, w, k8, ks, table, max_blocks, block_shift, num_blocks, seq_lens, B, H_I, D_I, max_len, logits,
                ld);
}

}  // namespace dsa
