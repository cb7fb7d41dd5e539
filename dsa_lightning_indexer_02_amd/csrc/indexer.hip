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
// twelve waves take disjoint 16-key tiles, keep NK tiles of keys in registers (MFMA B operand)
// and loop over the heads, so the head reduction happens inside each lane's accumulators
// without any cross-lane traffic.
// ---------------------------------------------------------------------------------------
constexpr int IDX_ROWS = 16;
constexpr int IDX_QROW_BYTES = 144;  // 128 B of codes + 16 B pad (bank spread)
constexpr int IDX_PREFILL_WAVES = 12;  // three waves per SIMD: VALU of one beside MFMAs of another

// HI > 0: the head count is a compile-time constant and the head loop is fully unrolled;
// HI == 0: any head count (plain loop).
template <int NK, int HI>
__global__ __launch_bounds__(IDX_PREFILL_WAVES * WAVE) void indexer_prefill_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k8, const float* __restrict__ ks, RowMap keymap, int64_t T,
    int64_t S, int32_t H_I, int32_t D_I, int64_t q_start, float* __restrict__ logits, int64_t ld,
    int64_t key_chunk) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* qtile = smem;                                                        // [H_I][16][144]
  float* wq = reinterpret_cast<float*>(smem + (size_t)H_I * IDX_ROWS * IDX_QROW_BYTES);  // [H_I][16]

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
    wq[head * IDX_ROWS + row] = t < T ? w[t * H_I + head] * qs[t * H_I + head] : 0.0f;
  }
  __syncthreads();

  const bool klane_has_bytes = (g * 32) < D_I;
  const int64_t pass_keys = (int64_t)IDX_PREFILL_WAVES * NK * 16;
  // key tiles of one pass (MFMA B operands) and their scales
  auto load_keys = [&](int64_t base, v8i (&B)[NK], float (&ksv)[NK]) {
#pragma unroll
    for (int kt = 0; kt < NK; ++kt) {
      const int64_t s = min(base + kt * 16 + j16, S - 1);
      const int64_t row = keymap(s);
      v8i b = {0, 0, 0, 0, 0, 0, 0, 0};
      if (klane_has_bytes) b = *reinterpret_cast<const v8i*>(k8 + row * D_I + g * 32);
      B[kt] = b;
      ksv[kt] = ks[row];
    }
  };
  for (int64_t base = c0 + (int64_t)wave * NK * 16; base < c1; base += pass_keys) {
    v8i B[NK];
    float ksv[NK];
    load_keys(base, B, ksv);
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
      auto mma = [&](const v8i& A, v4f (&c)[NK]) {
#pragma unroll
        for (int kt = 0; kt < NK; ++kt) c[kt] = mfma_fp8_16x16x128(A, B[kt], (v4f){0.f, 0.f, 0.f, 0.f});
      };
      mma(A0, c0);
      for (int head = 0; head < HI - 2; head += 2) {
        A1 = load_a(head + 1);
        w1 = load_w(head + 1);
        __builtin_amdgcn_sched_barrier(0);
        mma(A1, c1);          // head + 1
        relu_acc(w0, c0);     // head
        __builtin_amdgcn_sched_barrier(0);
        A0 = load_a(head + 2);
        w0 = load_w(head + 2);
        __builtin_amdgcn_sched_barrier(0);
        mma(A0, c0);          // head + 2
        relu_acc(w1, c1);     // head + 1
        __builtin_amdgcn_sched_barrier(0);
      }
      A1 = load_a(HI - 1);
      w1 = load_w(HI - 1);
      __builtin_amdgcn_sched_barrier(0);
      mma(A1, c1);
      relu_acc(w0, c0);
      relu_acc(w1, c1);
    } else {
      for (int head = 0; head < H_I; ++head) {
        const v8i A = load_a(head);
        const v4f wv = load_w(head);
        v4f c[NK];
#pragma unroll
        for (int kt = 0; kt < NK; ++kt) c[kt] = mfma_fp8_16x16x128(A, B[kt], (v4f){0.f, 0.f, 0.f, 0.f});
        relu_acc(wv, c);
      }
    }
    // lane (j16, g) holds rows t0 + 4g + r for key base + 16 kt + j16
#pragma unroll
    for (int kt = 0; kt < NK; ++kt) {
      const int64_t s = base + kt * 16 + j16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + 4 * g + r;
        if (t < T && s < c1 && s < q_start + t + 1) logits[t * ld + s] = acc[kt][r] * ksv[kt];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Decode: one query row per sequence.  The 64 (padded to a multiple of 16) heads are the MFMA
// M dimension, held in registers; the waves stream disjoint 64-key groups of the sequence's
// keys through its block table.  The head sum is a lane-local accumulation followed by a
// reduction over the four lane groups.
// ---------------------------------------------------------------------------------------
constexpr int IDX_DECODE_WAVES = 4;

template <int NHT>
__global__ __launch_bounds__(IDX_DECODE_WAVES * WAVE) void indexer_decode_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k8, const float* __restrict__ ks, const int32_t* __restrict__ table,
    int64_t max_blocks, int32_t block_shift, const int32_t* __restrict__ seq_lens, int32_t H_I,
    int32_t D_I, int64_t max_len, float* __restrict__ logits, int64_t ld, int64_t key_chunk) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j16 = lane & 15, g = lane >> 4;
  const int64_t b = blockIdx.y;
  const int64_t n = min((int64_t)max(seq_lens[b], 0), max_len);
  const int64_t c0 = (int64_t)blockIdx.x * key_chunk;
  if (c0 >= n) return;
  const int64_t c1 = min(n, c0 + key_chunk);
  const RowMap map{table ? table + b * max_blocks : nullptr, block_shift};

  v8i A[NHT];
  float wv[NHT][4];
  const bool has_bytes = (g * 32) < D_I;
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

  for (int64_t base = c0 + (int64_t)wave * 64; base < c1; base += IDX_DECODE_WAVES * 64) {
    v8i B[4];
    float ksv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t s = min(base + q * 16 + j16, n - 1);
      const int64_t row = map(s);
      v8i bb = {0, 0, 0, 0, 0, 0, 0, 0};
      if (has_bytes) bb = *reinterpret_cast<const v8i*>(k8 + row * D_I + g * 32);
      B[q] = bb;
      ksv[q] = ks[row];
    }
    float res[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float acc = 0.f;
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        const v4f c = mfma_fp8_16x16x128(A[ht], B[q], (v4f){0.f, 0.f, 0.f, 0.f});
        acc = fmaf(wv[ht][0], fmaxf(c[0], 0.f), acc);
        acc = fmaf(wv[ht][1], fmaxf(c[1], 0.f), acc);
        acc = fmaf(wv[ht][2], fmaxf(c[2], 0.f), acc);
        acc = fmaf(wv[ht][3], fmaxf(c[3], 0.f), acc);
      }
      res[q] = wave_sum_xor16_32(acc) * ksv[q];
    }
    // lane group g stores tile g: 64 consecutive keys per store
    const float v = g == 0 ? res[0] : g == 1 ? res[1] : g == 2 ? res[2] : res[3];
    const int64_t s = base + g * 16 + j16;
    if (s < c1) logits[b * ld + s] = v;
  }
}

// ---------------------------------------------------------------------------------------
size_t indexer_prefill_smem(int32_t H_I) {
  return (size_t)H_I * IDX_ROWS * IDX_QROW_BYTES + (size_t)H_I * IDX_ROWS * sizeof(float);
}

hipError_t launch_indexer_prefill(const uint8_t* q8, const float* qs, const float* w,
                                  const uint8_t* k8, const float* ks, const int32_t* table,
                                  int32_t block_shift, int64_t T, int64_t S, int32_t H_I, int32_t D_I,
                                  int64_t q_start, float* logits, int64_t ld, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  constexpr int NK = 4;
  const int64_t tiles = (T + IDX_ROWS - 1) / IDX_ROWS;
  const int64_t n_last = std::min<int64_t>(S, q_start + T);
  // split keys only when the tiles alone cannot fill the chip
  int64_t key_chunk = n_last;
  const int64_t unit = (int64_t)IDX_PREFILL_WAVES * NK * 16;
  if (tiles < 1024) {
    int64_t want = (1024 + tiles - 1) / tiles;
    key_chunk = std::max<int64_t>(unit, ((n_last + want - 1) / want + unit - 1) / unit * unit);
  }
  key_chunk = std::max<int64_t>(key_chunk, 1);
  const int64_t chunks = (n_last + key_chunk - 1) / key_chunk;
  dim3 grid((unsigned)chunks, (unsigned)tiles);
  const size_t smem = indexer_prefill_smem(H_I);
  auto kernel = H_I == 64 ? indexer_prefill_kernel<NK, 64> : indexer_prefill_kernel<NK, 0>;
  static bool attr_set[2] = {false, false};
  if (!attr_set[H_I == 64]) {
    hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set[H_I == 64] = true;
  }
  hipLaunchKernelGGL(kernel, grid, dim3(IDX_PREFILL_WAVES * WAVE), smem, stream, q8, qs, w, k8, ks,
                     RowMap{table, block_shift}, T, S, H_I, D_I, q_start, logits, ld, key_chunk);
  return hipGetLastError();
}

hipError_t launch_indexer_decode(const uint8_t* q8, const float* qs, const float* w,
                                 const uint8_t* k8, const float* ks, const int32_t* table,
                                 int64_t max_blocks, int32_t block_shift, const int32_t* seq_lens,
                                 int32_t B, int64_t max_len, int32_t H_I, int32_t D_I, float* logits,
                                 int64_t ld, hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  const int64_t key_chunk = 4096;
  dim3 grid((unsigned)((max_len + key_chunk - 1) / key_chunk), (unsigned)B);
  const int nht = (H_I + 15) / 16;
  if (nht <= 1)
    hipLaunchKernelGGL(indexer_decode_kernel<1>, grid, dim3(IDX_DECODE_WAVES * WAVE), 0, stream, q8, qs,
                       w, k8, ks, table, max_blocks, block_shift, seq_lens, H_I, D_I, max_len, logits, ld, key_chunk);
  else if (nht <= 2)
    hipLaunchKernelGGL(indexer_decode_kernel<2>, grid, dim3(IDX_DECODE_WAVES * WAVE), 0, stream, q8, qs,
                       w, k8, ks, table, max_blocks, block_shift, seq_lens, H_I, D_I, max_len, logits, ld, key_chunk);
  else
    hipLaunchKernelGGL(indexer_decode_kernel<4>, grid, dim3(IDX_DECODE_WAVES * WAVE), 0, stream, q8, qs,
                       w, k8, ks, table, max_blocks, block_shift, seq_lens, H_I, D_I, max_len, logits, ld, key_chunk);
  return hipGetLastError();
}

}  // namespace dsa
