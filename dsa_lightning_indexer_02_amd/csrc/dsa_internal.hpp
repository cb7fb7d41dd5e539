// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "dsa_device.hpp"
#include "host_launch.hpp"

namespace dsa {

// ---- lightning indexer
size_t indexer_prefill_smem(int32_t H_I, bool e8);
// q_exp / k_exp non-null: UE8M0 exponent scales applied in the MFMA (qs, ks unused)
// Query rows one indexer-prefill call takes: its 16-row query tiles run on the grid's second
// dimension, which gfx950 caps at 65536 workgroups.
int64_t indexer_prefill_max_rows();
hipError_t launch_indexer_prefill(const uint8_t* q8, const float* qs, const float* w, const uint8_t* k8,
                                  const float* ks, const int32_t* table, int32_t block_shift,
                                  int64_t num_blocks, int64_t T,
                                  int64_t S, int32_t H_I, int32_t D_I, int64_t q_start, float* logits,
                                  int64_t ld, hipStream_t stream, const uint8_t* q_exp = nullptr,
                                  const uint8_t* k_exp = nullptr);
// Sequences per decode call: the prefix table of per-sequence key groups sits in LDS.
constexpr int32_t kDecodeMaxSeqs = 12288;
hipError_t launch_indexer_decode(const uint8_t* q8, const float* qs, const float* w, const uint8_t* k8,
                                 const float* ks, const int32_t* table, int64_t max_blocks,
                                 int32_t block_shift, int64_t num_blocks, const int32_t* seq_lens, int32_t B,
                                 int64_t max_len,
                                 int32_t H_I, int32_t D_I, float* logits, int64_t ld, hipStream_t stream);

// ---- FP8 quantization and paged append
bool quantize_supported(int32_t D);
// exps != nullptr: power-of-two (UE8M0) scales, biased exponents written to exps (scales may be null)
hipError_t launch_quantize_rows(const uint16_t* x, int64_t rows, int32_t D, uint8_t* codes, float* scales,
                                uint8_t* exps, hipStream_t stream);
hipError_t launch_append_paged(uint8_t* k8_pool, float* ks_pool, uint16_t* kv_pool, int64_t num_blocks,
                               int32_t block_shift, const int32_t* table, int64_t max_blocks, int32_t B,
                               const int32_t* seq_ids, const int32_t* positions, int64_t n, int32_t D_I,
                               int32_t D_qk, const uint16_t* k, const uint16_t* kv, hipStream_t stream);

// ---- indexer training signal (KL loss toward the main attention) and backward
bool indexer_kl_supported(int32_t H, int32_t D);
hipError_t launch_indexer_kl(const uint16_t* q, const uint16_t* kv, int64_t T, int64_t S, int32_t H, int32_t D,
                             float sm_scale, int64_t q_start, const float* logits, int64_t ld, float* dlogits,
                             float* loss, hipStream_t stream);
bool indexer_kl_sparse_supported(int32_t H, int32_t D, int32_t k);
hipError_t launch_indexer_kl_sparse(const uint16_t* q, const uint16_t* kv, const int32_t* idx, int32_t k,
                                    const float* lse, int64_t T, int64_t S, int32_t H, int32_t D, float sm_scale,
                                    int64_t q_start, const float* logits, int64_t ld, float* dlogits, float* loss,
                                    hipStream_t stream);
size_t indexer_bwd_workspace_bytes(int64_t T, int64_t S, int32_t D_I);
// idx non-null: dq / dw over the listed keys of each row only (idx [T][k], distinct entries)
hipError_t launch_indexer_bwd(const uint8_t* q8, const float* qs, const float* w, const uint8_t* k8, const float* ks,
                              int64_t T, int64_t S, int32_t H_I, int32_t D_I, int64_t q_start, const float* dI,
                              int64_t ld, float* dq, float* dw, float* dk, void* workspace, hipStream_t stream,
                              const int32_t* idx = nullptr, int32_t k = 0);

// ---- top-k
int32_t topk_chunks(int64_t S);
size_t topk_workspace_bytes(int64_t T, int64_t S, int32_t k);
bool topk_supported(int64_t S, int32_t k);
hipError_t launch_topk(const float* logits, int64_t ld, int64_t T, int64_t S, int64_t q_start,
                       const int32_t* seq_lens, int32_t k, int32_t* indices, void* workspace,
                       hipStream_t stream);

// ---- sparse MLA
struct MlaArgs {
  const uint16_t* q;
  const uint16_t* kv;
  const int32_t* idx;
  const int32_t* table;
  int64_t max_blocks;
  int32_t block_shift;
  int64_t num_blocks;      // pool size in blocks (paged case)
  int32_t per_row_table;   // decode: row r uses table + r * max_blocks
  const int32_t* seq_lens; // decode: visible keys per row; null for prefill
  int64_t R;               // query rows
  int64_t S;
  int64_t q_start;
  int32_t H, D_qk, D_v, k;
  float sm_scale;
  int32_t nsplit;
  uint16_t* out;
  float* out_f32;
  float* lse;
  float* part_out;
  float* part_lse;
  // fp16 staging (576/512, one sequence): S x D_qk fp16 of workspace for the converted rows; null
  // selects bf16 staging
  uint16_t* kv_f16;
};
bool mla_supported(int32_t D_qk, int32_t D_v, int32_t H, int32_t k);
// workspace bytes of the fp16 copy for fp16 staging (0: that staging is not available for the dims)
size_t mla_kv16_bytes(int64_t S, int32_t D_qk, int32_t D_v);
hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t stream);

// ---- sparse MLA backward
bool mla_bwd_supported(int32_t D_qk, int32_t D_v, int32_t H, int32_t k);
size_t mla_bwd_workspace_bytes(int64_t T, int64_t S, int32_t H, int32_t k);
hipError_t launch_sparse_mla_bwd(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const float* lse,
                                 const uint16_t* dout, int64_t T, int64_t S, int32_t H, int32_t k, int64_t q_start,
                                 float sm_scale, float* dq, float* dkv, void* workspace, hipStream_t stream);

}  // namespace dsa
