// FP8 quantization of the indexer's query and key vectors and the paged append of new tokens
// (createthis gist page, indexer listing: the indexer casts its query and key vectors to FP8
// E4M3 along the last dimension with one scale per vector; DeepSeek-V3.2-Exp summary page,
// section "Key claims": the released indexer-logit kernels read a paged cache).
//
// A row of D bf16 values x becomes s = max_i |x_i| / 448 (1 for an all-zero row) and the codes
// e4m3(clamp(x_i / s, -448, 448)), the division correctly rounded in fp32 and the conversion
// the hardware's round-to-nearest-even pack (v_cvt_pk_fp8_f32, OCP E4M3 on gfx950).
//
// The work is a stream (2 bytes in, 1 byte + 4 bytes per row out), so a row is spread over D / 8
// lanes with 16-byte loads (D = 128: four rows per wave), its maximum reduced over those lanes.
#include "dsa_internal.hpp"

namespace dsa {

constexpr int QZ_THREADS = 256;
constexpr float QZ_FP8_MAX = 448.0f;

// Lanes per row: the power of two >= D / 8 (rows never straddle a wave).
static int qz_lanes(int32_t D) {
  int l = 1;
  while (l < D / 8) l <<= 1;
  return l;
}

// Quantize the 8 values this lane holds (x: 8 bf16 bit patterns in a v4i) of a row whose lanes
// are the aligned group of `lanes` lanes containing this one; `active`: this lane holds values.
// Returns the 8 codes (two dwords); *scale receives the row scale.  UE8M0: the scale is the
// smallest power of two 2^p >= amax / 448 (p >= -127, createthis gist page, indexer listing: the
// cast's use_ue8m0 option) and *exp8 receives p + 127.
template <bool UE8M0>
__device__ __forceinline__ v2i quantize8(v4i x, bool active, int lanes, float* scale, uint32_t* exp8) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = (uint32_t)x[i];
    v[2 * i] = __uint_as_float(w << 16);
    v[2 * i + 1] = __uint_as_float(w & 0xFFFF0000u);
  }
  float amax = 0.0f;
  if (active) {
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  for (int o = 1; o < lanes; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  float s = amax > 0.0f ? __fdiv_rn(amax, QZ_FP8_MAX) : 1.0f;
  if constexpr (UE8M0) {
    int e;
    const float m = frexpf(s, &e);  // s = m 2^e, 0.5 <= m < 1
    const int p = max(m == 0.5f ? e - 1 : e, -127);
    s = ldexpf(1.0f, p);
    *exp8 = (uint32_t)(p + 127);
  }
  *scale = s;
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(__fdiv_rn(v[i], s), -QZ_FP8_MAX), QZ_FP8_MAX);
  // value 2 h + e of a dword lands in byte 2 h + e (h: the half-word selector)
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
  return (v2i){lo, hi};
}

// Each thread takes QZ_PIECES 16-byte pieces, QZ_THREADS pieces apart (so every load
// instruction of a wave reads consecutive memory, and a row's lanes stay in one wave), and
// issues all of their loads before it converts any.
constexpr int QZ_PIECES = 4;

template <bool UE8M0>
__global__ __launch_bounds__(QZ_THREADS) void quantize_rows_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                  int32_t D, int32_t lanes, uint8_t* __restrict__ codes,
                                                                  float* __restrict__ scales,
                                                                  uint8_t* __restrict__ exps) {
  const int64_t g0 = (int64_t)blockIdx.x * QZ_THREADS * QZ_PIECES + threadIdx.x;
  v4i xv[QZ_PIECES];
  int64_t r[QZ_PIECES];
  int j[QZ_PIECES];
  bool in_row[QZ_PIECES], active[QZ_PIECES];
#pragma unroll
  for (int u = 0; u < QZ_PIECES; ++u) {
    const int64_t gl = g0 + (int64_t)u * QZ_THREADS;
    r[u] = gl / lanes;
    j[u] = (int)(gl % lanes);  // 8-value piece of the row
    in_row[u] = r[u] < rows;
    active[u] = in_row[u] && j[u] * 8 < D;
    xv[u] = (v4i){0, 0, 0, 0};
    if (active[u]) xv[u] = *reinterpret_cast<const v4i*>(x + r[u] * D + j[u] * 8);
  }
#pragma unroll
  for (int u = 0; u < QZ_PIECES; ++u) {
    float s;
    uint32_t e8 = 0;
    const v2i c = quantize8<UE8M0>(xv[u], active[u], lanes, &s, &e8);
    if (active[u]) *reinterpret_cast<v2i*>(codes + r[u] * D + j[u] * 8) = c;
    if (in_row[u] && j[u] == 0) {
      if (scales) scales[r[u]] = s;
      if constexpr (UE8M0) exps[r[u]] = (uint8_t)e8;
    }
  }
}

// One wave per token: the key's D_I / 8 lanes quantize it into the token's slot, all 64 lanes
// copy the latent row (16 bytes per lane and step).
__global__ __launch_bounds__(QZ_THREADS) void append_paged_kernel(
    uint8_t* __restrict__ k8_pool, float* __restrict__ ks_pool, uint16_t* __restrict__ kv_pool, int64_t num_blocks,
    int32_t block_shift, const int32_t* __restrict__ table, int64_t max_blocks, int32_t B,
    const int32_t* __restrict__ seq_ids, const int32_t* __restrict__ positions, int64_t n, int32_t D_I,
    int32_t D_qk, int32_t lanes, const uint16_t* __restrict__ k, const uint16_t* __restrict__ kv) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * (QZ_THREADS / WAVE) + (threadIdx.x >> 6);
  if (i >= n) return;  // wave-uniform
  const int32_t b = seq_ids[i], p = positions[i];
  if (b < 0 || b >= B || p < 0 || (int64_t)(p >> block_shift) >= max_blocks) return;
  const int32_t blk = table[(int64_t)b * max_blocks + (p >> block_shift)];
  if (blk < 0 || blk >= num_blocks) return;
  const int64_t row = ((int64_t)blk << block_shift) | (p & ((1 << block_shift) - 1));

  if (lane < lanes) {  // whole aligned groups: the reduction in quantize8 stays inside them
    const bool active = lane * 8 < D_I;
    v4i xv = {0, 0, 0, 0};
    if (active) xv = *reinterpret_cast<const v4i*>(k + i * D_I + lane * 8);
    float s;
    uint32_t e8;
    const v2i c = quantize8<false>(xv, active, lanes, &s, &e8);
    if (active) *reinterpret_cast<v2i*>(k8_pool + row * D_I + lane * 8) = c;
    if (lane == 0) ks_pool[row] = s;
  }
  const int pieces = D_qk / 8;  // 16-byte pieces of the latent row
  for (int c = lane; c < pieces; c += WAVE)
    *reinterpret_cast<v4i*>(kv_pool + row * D_qk + c * 8) = *reinterpret_cast<const v4i*>(kv + i * D_qk + c * 8);
}

bool quantize_supported(int32_t D) { return D >= 8 && D <= 512 && D % 8 == 0; }

hipError_t launch_quantize_rows(const uint16_t* x, int64_t rows, int32_t D, uint8_t* codes, float* scales,
                                uint8_t* exps, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int lanes = qz_lanes(D);
  const int64_t pieces = rows * lanes;
  const int64_t grid = (pieces + QZ_THREADS * QZ_PIECES - 1) / (QZ_THREADS * QZ_PIECES);
  if (exps)
    return launch("quantize_rows_kernel<ue8m0>", quantize_rows_kernel<true>, dim3((unsigned)grid), dim3(QZ_THREADS),
                  0, stream, x, rows, D, lanes, codes, scales, exps);
  return launch("quantize_rows_kernel", quantize_rows_kernel<false>, dim3((unsigned)grid), dim3(QZ_THREADS), 0,
                stream, x, rows, D, lanes, codes, scales, exps);
}

hipError_t launch_append_paged(uint8_t* k8_pool, float* ks_pool, uint16_t* kv_pool, int64_t num_blocks,
                               int32_t block_shift, const int32_t* table, int64_t max_blocks, int32_t B,
                               const int32_t* seq_ids, const int32_t* positions, int64_t n, int32_t D_I,
                               int32_t D_qk, const uint16_t* k, const uint16_t* kv, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t grid = (n + QZ_THREADS / WAVE - 1) / (QZ_THREADS / WAVE);
  return launch("append_paged_kernel", append_paged_kernel, dim3((unsigned)grid), dim3(QZ_THREADS), 0, stream,
                k8_pool, ks_pool, kv_pool, num_blocks, block_shift, table, max_blocks, B, seq_ids, positions, n, D_I,
                D_qk, qz_lanes(D_I), k, kv);
}

}  // namespace dsa
