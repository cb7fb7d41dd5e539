// C ABI of the DSA hot path: host-side argument validation, workspace carving and the launch
// sequence.  Every check happens before the first launch, so a failing call enqueues nothing.
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>

#include "../../include/dsa.h"
#include "dsa_internal.hpp"

namespace {

thread_local std::string g_last_error;

dsa_status_t fail(dsa_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

dsa_status_t ok() {
  g_last_error.clear();
  return DSA_OK;
}

dsa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, status, ...)        \
  do {                                    \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

#define REQUIRE_PTR(p) REQUIRE((p) != nullptr && aligned16(p), DSA_ERR_INVALID_ARGUMENT, \
                               "%s must be a non-null 16-byte aligned pointer", #p)
#define OPTIONAL_PTR(p) REQUIRE((p) == nullptr || aligned16(p), DSA_ERR_INVALID_ARGUMENT, \
                                "%s must be 16-byte aligned when given", #p)

constexpr size_t kAlign = 256;
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t ld_for(int64_t S) { return (S + 3) / 4 * 4; }

int block_shift_of(int32_t bs) {
  int s = 0;
  while ((1 << s) < bs) ++s;
  return s;
}

dsa_status_t check_indexer_dims(int32_t H_I, int32_t D_I) {
  REQUIRE(H_I >= 1 && H_I <= 64, DSA_ERR_UNSUPPORTED, "H_I=%d not in [1, 64]", H_I);
  REQUIRE(D_I == 32 || D_I == 64 || D_I == 96 || D_I == 128, DSA_ERR_UNSUPPORTED,
          "D_I=%d not in {32, 64, 96, 128}", D_I);
  return DSA_OK;
}

dsa_status_t check_mla_dims(int32_t H, int32_t D_qk, int32_t D_v, int32_t k) {
  REQUIRE(k >= 1, DSA_ERR_INVALID_ARGUMENT, "k=%d must be >= 1", k);
  REQUIRE(dsa::mla_supported(D_qk, D_v, H, k), DSA_ERR_UNSUPPORTED,
          "sparse MLA shape H=%d D_qk=%d D_v=%d k=%d not supported", H, D_qk, D_v, k);
  return DSA_OK;
}

dsa_status_t check_topk(int64_t S, int32_t k) {
  REQUIRE(k >= 1, DSA_ERR_INVALID_ARGUMENT, "k=%d must be >= 1", k);
  REQUIRE(dsa::topk_supported(S, k), DSA_ERR_UNSUPPORTED, "top-k with k=%d over rows of %lld not supported",
          k, (long long)S);
  return DSA_OK;
}

// Index-list splits per decode row: enough (B x nsplit) sparse-MLA workgroups for one per compute
// unit of an MI355X (256), each over at least 64 indices.  More splits than that only add fp32
// partial traffic (written by the attention, re-read by the combine).
int32_t decode_splits(int32_t B, int32_t k) {
  constexpr int32_t kWorkgroups = 256;
  int32_t want = (kWorkgroups + B - 1) / B;
  int32_t cap = std::max(1, k / 64);
  return std::max(1, std::min(want, cap));
}

struct PrefillLayout {
  size_t logits, indices, topk, kv16, total;
  int64_t ld;
};
PrefillLayout prefill_layout(const dsa_dims_t* d, int64_t T, int64_t S) {
  PrefillLayout L{};
  L.ld = ld_for(S);
  L.logits = 0;
  L.indices = round_up((size_t)T * L.ld * sizeof(float), kAlign);
  L.topk = L.indices + round_up((size_t)T * d->topk * sizeof(int32_t), kAlign);
  L.kv16 = L.topk + round_up(dsa::topk_workspace_bytes(T, S, d->topk), kAlign);
  L.total = L.kv16 + round_up(dsa::mla_kv16_bytes(S, d->D_qk, d->D_v), kAlign);
  return L;
}

struct DecodeLayout {
  size_t logits, indices, topk, part_out, part_lse, total;
  int64_t ld;
  int32_t nsplit;
};
DecodeLayout decode_layout(const dsa_dims_t* d, int32_t B, int64_t max_len) {
  DecodeLayout L{};
  L.ld = ld_for(max_len);
  L.nsplit = decode_splits(B, d->topk);
  L.logits = 0;
  L.indices = round_up((size_t)B * L.ld * sizeof(float), kAlign);
  L.topk = L.indices + round_up((size_t)B * d->topk * sizeof(int32_t), kAlign);
  L.part_out = L.topk + round_up(dsa::topk_workspace_bytes(B, max_len, d->topk), kAlign);
  L.part_lse = L.part_out + round_up((size_t)B * L.nsplit * d->H * d->D_v * sizeof(float), kAlign);
  L.total = L.part_lse + round_up((size_t)B * L.nsplit * d->H * sizeof(float), kAlign);
  return L;
}

dsa_status_t check_dims(const dsa_dims_t* d) {
  REQUIRE(d != nullptr, DSA_ERR_INVALID_ARGUMENT, "dims must not be NULL");
  dsa_status_t s = check_indexer_dims(d->H_I, d->D_I);
  if (s != DSA_OK) return s;
  s = check_mla_dims(d->H, d->D_qk, d->D_v, d->topk);
  if (s != DSA_OK) return s;
  REQUIRE(d->topk <= 2048, DSA_ERR_UNSUPPORTED, "topk=%d above 2048", d->topk);
  REQUIRE(d->sm_scale > 0.f, DSA_ERR_INVALID_ARGUMENT, "sm_scale must be positive");
  return DSA_OK;
}

dsa_status_t check_cache(const dsa_paged_cache_t* c, int64_t rows_needed_per_seq, int32_t seqs) {
  REQUIRE(c != nullptr, DSA_ERR_INVALID_ARGUMENT, "cache must not be NULL");
  REQUIRE_PTR(c->k8);
  REQUIRE_PTR(c->k_scale);
  REQUIRE_PTR(c->kv);
  REQUIRE_PTR(c->block_table);
  REQUIRE(c->block_size >= 1 && c->block_size <= (1 << 20) && (c->block_size & (c->block_size - 1)) == 0,
          DSA_ERR_INVALID_ARGUMENT, "block_size=%d must be a power of two", c->block_size);
  REQUIRE(c->num_blocks >= 1, DSA_ERR_INVALID_ARGUMENT, "num_blocks must be >= 1");
  REQUIRE(c->num_blocks * (int64_t)c->block_size <= INT32_MAX, DSA_ERR_UNSUPPORTED,
          "pool of %lld rows exceeds 2^31", (long long)(c->num_blocks * c->block_size));
  const int64_t blocks_needed = (rows_needed_per_seq + c->block_size - 1) / c->block_size;
  REQUIRE(c->max_blocks_per_seq >= blocks_needed, DSA_ERR_INVALID_ARGUMENT,
          "max_blocks_per_seq=%lld < %lld blocks needed", (long long)c->max_blocks_per_seq,
          (long long)blocks_needed);
  (void)seqs;
  return DSA_OK;
}

// ---- scratch of the allocation-free top-k entry point
// One file-scope device array per GPU the library runs on (held until the process ends).  Host
// code never passes the array's name to a kernel or a copy: on the host that name is a stand-in,
// not a device address.  The device address comes from hipGetSymbolAddress, once per device with
// that device current, and is kept per device.
constexpr size_t kNoallocScratchBytes = DSA_TOPK_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

std::mutex g_scratch_mutex;
std::map<int, void*> g_scratch_ptr;  // device id -> device address of that device's `scratch`

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return dsa::take_error(e);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *out = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return dsa::take_error(e);
  g_scratch_ptr.emplace(dev, p);
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* dsa_status_string(dsa_status_t s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARGUMENT: return "DSA_ERR_INVALID_ARGUMENT";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE_TOO_SMALL: return "DSA_ERR_WORKSPACE_TOO_SMALL";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
  }
  return "unknown dsa_status_t";
}

const char* dsa_last_error(void) { return g_last_error.c_str(); }

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

dsa_status_t dsa_profile_begin(hipEvent_t* events, int32_t capacity) {
  REQUIRE(events != nullptr && capacity >= 1, DSA_ERR_INVALID_ARGUMENT, "events must be non-null, capacity >= 1");
  dsa::ProfileState& ps = dsa::profile_state();
  ps.events = events;
  ps.capacity = capacity;
  ps.count = 0;
  ps.names.clear();
  return ok();
}

int32_t dsa_profile_end(void) {
  dsa::ProfileState& ps = dsa::profile_state();
  const int32_t n = ps.events ? ps.count : 0;
  ps.events = nullptr;
  ps.capacity = 0;
  return n;
}

const char* dsa_profile_kernel_name(int32_t i) {
  const dsa::ProfileState& ps = dsa::profile_state();
  if (i < 0 || i >= (int32_t)ps.names.size()) return "";
  return ps.names[i];
}

dsa_status_t dsa_indexer_logits(const uint8_t* q8, const float* q_scale, const float* w, const uint8_t* k8,
                                const float* k_scale, int64_t T, int64_t S, int32_t H_I, int32_t D_I,
                                int64_t q_start, float* logits, int64_t ld_logits, hipStream_t stream) {
  REQUIRE(T >= 0 && S >= 0 && q_start >= 0, DSA_ERR_INVALID_ARGUMENT, "negative T, S or q_start");
  REQUIRE(T <= dsa::indexer_prefill_max_rows(), DSA_ERR_UNSUPPORTED, "T=%lld exceeds %lld query rows per call",
          (long long)T, (long long)dsa::indexer_prefill_max_rows());
  dsa_status_t s = check_indexer_dims(H_I, D_I);
  if (s != DSA_OK) return s;
  if (T == 0) return ok();
  REQUIRE(S >= 1, DSA_ERR_INVALID_ARGUMENT, "S must be >= 1 when T > 0");
  REQUIRE(ld_logits >= S && ld_logits % 4 == 0, DSA_ERR_INVALID_ARGUMENT,
          "ld_logits=%lld must be >= S=%lld and a multiple of 4", (long long)ld_logits, (long long)S);
  REQUIRE_PTR(q8);
  REQUIRE_PTR(q_scale);
  REQUIRE_PTR(w);
  REQUIRE_PTR(k8);
  REQUIRE_PTR(k_scale);
  REQUIRE_PTR(logits);
  return hip_status(dsa::launch_indexer_prefill(q8, q_scale, w, k8, k_scale, nullptr, 0, 0, T, S, H_I, D_I,
                                                q_start, logits, ld_logits, stream),
                    "indexer launch");
}

dsa_status_t dsa_indexer_logits_ue8m0(const uint8_t* q8, const uint8_t* q_exp, const float* w, const uint8_t* k8,
                                      const uint8_t* k_exp, int64_t T, int64_t S, int32_t H_I, int32_t D_I,
                                      int64_t q_start, float* logits, int64_t ld_logits, hipStream_t stream) {
  REQUIRE(T >= 0 && S >= 0 && q_start >= 0, DSA_ERR_INVALID_ARGUMENT, "negative T, S or q_start");
  REQUIRE(T <= dsa::indexer_prefill_max_rows(), DSA_ERR_UNSUPPORTED, "T=%lld exceeds %lld query rows per call",
          (long long)T, (long long)dsa::indexer_prefill_max_rows());
  dsa_status_t s = check_indexer_dims(H_I, D_I);
  if (s != DSA_OK) return s;
  if (T == 0) return ok();
  REQUIRE(S >= 1, DSA_ERR_INVALID_ARGUMENT, "S must be >= 1 when T > 0");
  REQUIRE(ld_logits >= S && ld_logits % 4 == 0, DSA_ERR_INVALID_ARGUMENT,
          "ld_logits=%lld must be >= S=%lld and a multiple of 4", (long long)ld_logits, (long long)S);
  REQUIRE_PTR(q8);
  REQUIRE_PTR(q_exp);
  REQUIRE_PTR(w);
  REQUIRE_PTR(k8);
  REQUIRE_PTR(k_exp);
  REQUIRE_PTR(logits);
  return hip_status(dsa::launch_indexer_prefill(q8, nullptr, w, k8, nullptr, nullptr, 0, 0, T, S, H_I, D_I, q_start,
                                                logits, ld_logits, stream, q_exp, k_exp),
                    "indexer launch");
}

size_t dsa_topk_workspace_size(int64_t T, int64_t S, int32_t k) {
  if (T <= 0 || S <= 0 || k <= 0) return 0;
  return dsa::topk_workspace_bytes(T, S, k);
}

dsa_status_t dsa_topk(const float* logits, int64_t ld_logits, int64_t T, int64_t S, int64_t q_start, int32_t k,
                      int32_t* indices, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  REQUIRE(T >= 0 && S >= 0 && q_start >= 0, DSA_ERR_INVALID_ARGUMENT, "negative T, S or q_start");
  dsa_status_t s = check_topk(S, k);
  if (s != DSA_OK) return s;
  if (T == 0) return ok();
  REQUIRE(S >= 1, DSA_ERR_INVALID_ARGUMENT, "S must be >= 1 when T > 0");
  REQUIRE(k <= 2048 || S <= 32768, DSA_ERR_UNSUPPORTED, "k=%d above 2048 needs S <= 32768", k);
  REQUIRE(ld_logits >= S && ld_logits % 4 == 0, DSA_ERR_INVALID_ARGUMENT,
          "ld_logits=%lld must be >= S=%lld and a multiple of 4", (long long)ld_logits, (long long)S);
  REQUIRE_PTR(logits);
  REQUIRE_PTR(indices);
  const size_t need = dsa::topk_workspace_bytes(T, S, k);
  REQUIRE(workspace_bytes >= need, DSA_ERR_WORKSPACE_TOO_SMALL, "top-k workspace %zu < %zu bytes",
          workspace_bytes, need);
  if (need) REQUIRE_PTR(workspace);
  return hip_status(dsa::launch_topk(logits, ld_logits, T, S, q_start, nullptr, k, indices, workspace, stream),
                    "top-k launch");
}

dsa_status_t dsa_topk_noalloc(const float* logits, int64_t ld_logits, int64_t T, int64_t S, int64_t q_start, int32_t k,
                              int32_t* indices, hipStream_t stream) {
  REQUIRE(T >= 0 && S >= 0 && q_start >= 0, DSA_ERR_INVALID_ARGUMENT, "negative T, S or q_start");
  dsa_status_t s = check_topk(S, k);
  if (s != DSA_OK) return s;
  if (T == 0) return ok();
  REQUIRE(S >= 1, DSA_ERR_INVALID_ARGUMENT, "S must be >= 1 when T > 0");
  REQUIRE(k <= 2048 || S <= 32768, DSA_ERR_UNSUPPORTED, "k=%d above 2048 needs S <= 32768", k);
  REQUIRE(ld_logits >= S && ld_logits % 4 == 0, DSA_ERR_INVALID_ARGUMENT,
          "ld_logits=%lld must be >= S=%lld and a multiple of 4", (long long)ld_logits, (long long)S);
  REQUIRE_PTR(logits);
  REQUIRE_PTR(indices);
  const size_t need = dsa::topk_workspace_bytes(T, S, k);
  REQUIRE(need <= kNoallocScratchBytes, DSA_ERR_UNSUPPORTED,
          "dsa_topk_noalloc: %lld rows of %lld scores need %zu bytes of scratch, above its %zu-byte array "
          "(use dsa_topk with a workspace, or fewer rows per call)",
          (long long)T, (long long)S, need, kNoallocScratchBytes);
  void* ws = nullptr;
  if (need) {
    hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return hip_status(e, "scratch symbol address");
  }
  dsa::trace_call("dsa_topk_noalloc", kNoallocScratchBytes, need);
  return hip_status(dsa::launch_topk(logits, ld_logits, T, S, q_start, nullptr, k, indices, ws, stream),
                    "top-k launch");
}

size_t dsa_sparse_mla_workspace_size(int64_t T, int64_t S, int32_t H, int32_t D_qk, int32_t D_v, int32_t k) {
  if (T <= 0 || S <= 0 || H <= 0 || k <= 0) return 0;
  return round_up(dsa::mla_kv16_bytes(S, D_qk, D_v), kAlign);
}

dsa_status_t dsa_sparse_mla_fwd(const uint16_t* q, const uint16_t* kv, const int32_t* indices, int64_t T,
                                int64_t S, int32_t H, int32_t D_qk, int32_t D_v, int32_t k, int64_t q_start,
                                float sm_scale, uint16_t* out, float* out_f32, float* lse, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  REQUIRE(T >= 0 && S >= 0 && q_start >= 0, DSA_ERR_INVALID_ARGUMENT, "negative T, S or q_start");
  dsa_status_t s = check_mla_dims(H, D_qk, D_v, k);
  if (s != DSA_OK) return s;
  REQUIRE(sm_scale > 0.f, DSA_ERR_INVALID_ARGUMENT, "sm_scale must be positive");
  if (T == 0) return ok();
  REQUIRE(S >= 1, DSA_ERR_INVALID_ARGUMENT, "S must be >= 1 when T > 0");
  REQUIRE(S <= INT32_MAX, DSA_ERR_UNSUPPORTED, "S above 2^31");
  REQUIRE_PTR(q);
  REQUIRE_PTR(kv);
  REQUIRE_PTR(indices);
  REQUIRE_PTR(out);
  OPTIONAL_PTR(out_f32);
  OPTIONAL_PTR(lse);
  // a workspace selects fp16 staging where the dims have it (it must then hold the fp16 copy)
  const size_t kv16 = round_up(dsa::mla_kv16_bytes(S, D_qk, D_v), kAlign);
  if (workspace != nullptr && kv16 > 0) {
    REQUIRE(workspace_bytes >= kv16, DSA_ERR_WORKSPACE_TOO_SMALL, "sparse MLA workspace %zu < %zu bytes",
            workspace_bytes, kv16);
    REQUIRE((reinterpret_cast<uintptr_t>(workspace) % kAlign) == 0, DSA_ERR_INVALID_ARGUMENT,
            "workspace must be 256-byte aligned");
  }
  dsa::MlaArgs a{};
  a.q = q;
  a.kv = kv;
  a.idx = indices;
  a.kv_f16 = (workspace != nullptr && kv16 > 0) ? static_cast<uint16_t*>(workspace) : nullptr;
  a.R = T;
  a.S = S;
  a.q_start = q_start;
  a.H = H;
  a.D_qk = D_qk;
  a.D_v = D_v;
  a.k = k;
  a.sm_scale = sm_scale;
  a.nsplit = 1;
  a.out = out;
  a.out_f32 = out_f32;
  a.lse = lse;
  return hip_status(dsa::launch_sparse_mla(a, stream), "sparse MLA launch");
}

size_t dsa_sparse_mla_bwd_workspace_size(int64_t T, int64_t S, int32_t H, int32_t k) {
  if (T <= 0 || S <= 0 || H <= 0 || k <= 0) return 0;
  return dsa::mla_bwd_workspace_bytes(T, S, H, k);
}

dsa_status_t dsa_sparse_mla_bwd(const uint16_t* q, const uint16_t* kv, const int32_t* indices, const float* lse,
                                const uint16_t* dout, int64_t T, int64_t S, int32_t H,
                                int32_t D_qk, int32_t D_v, int32_t k, int64_t q_start, float sm_scale, float* dq,
                                float* dkv, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  REQUIRE(T >= 0 && S >= 0 && q_start >= 0, DSA_ERR_INVALID_ARGUMENT, "negative T, S or q_start");
  REQUIRE(k >= 1, DSA_ERR_INVALID_ARGUMENT, "k=%d must be >= 1", k);
  REQUIRE(dsa::mla_bwd_supported(D_qk, D_v, H, k), DSA_ERR_UNSUPPORTED,
          "sparse MLA backward with H=%d D_qk=%d D_v=%d k=%d not supported ((576, 512), 1 <= H <= 128, k <= 2048)",
          H, D_qk, D_v, k);
  REQUIRE(sm_scale > 0.f, DSA_ERR_INVALID_ARGUMENT, "sm_scale must be positive");
  if (T == 0 && S == 0) return ok();
  REQUIRE(S >= 1, DSA_ERR_INVALID_ARGUMENT, "S must be >= 1");
  REQUIRE(S <= INT32_MAX, DSA_ERR_UNSUPPORTED, "S above 2^31");
  REQUIRE_PTR(kv);
  REQUIRE_PTR(dkv);
  if (T > 0) {
    REQUIRE_PTR(q);
    REQUIRE_PTR(indices);
    REQUIRE_PTR(lse);
    REQUIRE_PTR(dout);
    REQUIRE_PTR(dq);
  }
  const size_t need = dsa::mla_bwd_workspace_bytes(T, S, H, k);
  REQUIRE(workspace_bytes >= need, DSA_ERR_WORKSPACE_TOO_SMALL, "sparse MLA backward workspace %zu < %zu bytes",
          workspace_bytes, need);
  if (need) REQUIRE_PTR(workspace);
  dsa::trace_call("dsa_sparse_mla_bwd", workspace_bytes, need);
  return hip_status(dsa::launch_sparse_mla_bwd(q, kv, indices, lse, dout, T, S, H, k, q_start, sm_scale, dq, dkv,
                                               workspace, stream),
                    "sparse MLA backward launch");
}

size_t dsa_prefill_workspace_size(const dsa_dims_t* d, int64_t T, int64_t S) {
  if (!d || T <= 0 || S <= 0 || d->topk <= 0) return 0;
  return prefill_layout(d, T, S).total;
}

dsa_status_t dsa_prefill_paged(const dsa_paged_cache_t* c, int32_t seq, const dsa_dims_t* d, int64_t T,
                               int64_t q_start, const uint8_t* q8, const float* q_scale, const float* w,
                               const uint16_t* q, uint16_t* out, float* out_f32, float* lse,
                               int32_t* indices_out, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  dsa_status_t s = check_dims(d);
  if (s != DSA_OK) return s;
  REQUIRE(T >= 0 && q_start >= 0 && seq >= 0, DSA_ERR_INVALID_ARGUMENT, "negative T, q_start or seq");
  REQUIRE(T <= dsa::indexer_prefill_max_rows(), DSA_ERR_UNSUPPORTED, "T=%lld exceeds %lld query rows per call",
          (long long)T, (long long)dsa::indexer_prefill_max_rows());
  if (T == 0) return ok();
  const int64_t S = q_start + T;
  s = check_cache(c, S, seq + 1);
  if (s != DSA_OK) return s;
  REQUIRE(S <= (int64_t)c->num_blocks * c->block_size, DSA_ERR_INVALID_ARGUMENT,
          "context of %lld keys exceeds the pool", (long long)S);
  REQUIRE_PTR(q8);
  REQUIRE_PTR(q_scale);
  REQUIRE_PTR(w);
  REQUIRE_PTR(q);
  REQUIRE_PTR(out);
  OPTIONAL_PTR(out_f32);
  OPTIONAL_PTR(lse);
  OPTIONAL_PTR(indices_out);
  const PrefillLayout L = prefill_layout(d, T, S);
  REQUIRE(workspace_bytes >= L.total, DSA_ERR_WORKSPACE_TOO_SMALL, "prefill workspace %zu < %zu bytes",
          workspace_bytes, L.total);
  REQUIRE(workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) % kAlign) == 0,
          DSA_ERR_INVALID_ARGUMENT, "workspace must be non-null and 256-byte aligned");
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* logits = reinterpret_cast<float*>(ws + L.logits);
  int32_t* idx = indices_out ? indices_out : reinterpret_cast<int32_t*>(ws + L.indices);
  const int32_t* table = c->block_table + (int64_t)seq * c->max_blocks_per_seq;
  const int shift = block_shift_of(c->block_size);

  dsa::trace_call("dsa_prefill_paged", workspace_bytes, L.total);
  hipError_t e = dsa::launch_indexer_prefill(q8, q_scale, w, c->k8, c->k_scale, table, shift, c->num_blocks, T, S,
                                             d->H_I, d->D_I, q_start, logits, L.ld, stream);
  if (e != hipSuccess) return hip_status(e, "indexer launch");
  e = dsa::launch_topk(logits, L.ld, T, S, q_start, nullptr, d->topk, idx, ws + L.topk, stream);
  if (e != hipSuccess) return hip_status(e, "top-k launch");
  dsa::MlaArgs a{};
  a.q = q;
  a.kv = c->kv;
  a.idx = idx;
  a.table = table;
  a.max_blocks = c->max_blocks_per_seq;
  a.block_shift = shift;
  a.num_blocks = c->num_blocks;
  a.per_row_table = 0;
  a.R = T;
  a.S = S;
  a.q_start = q_start;
  a.H = d->H;
  a.D_qk = d->D_qk;
  a.D_v = d->D_v;
  a.k = d->topk;
  a.sm_scale = d->sm_scale;
  a.nsplit = 1;
  a.out = out;
  a.out_f32 = out_f32;
  a.lse = lse;
  a.kv_f16 = dsa::mla_kv16_bytes(S, d->D_qk, d->D_v) > 0 ? reinterpret_cast<uint16_t*>(ws + L.kv16) : nullptr;
  return hip_status(dsa::launch_sparse_mla(a, stream), "sparse MLA launch");
}

size_t dsa_decode_workspace_size(const dsa_dims_t* d, int32_t B, int64_t max_seq_len) {
  if (!d || B <= 0 || max_seq_len <= 0 || d->topk <= 0 || d->H <= 0 || d->D_v <= 0) return 0;
  return decode_layout(d, B, max_seq_len).total;
}

dsa_status_t dsa_decode_paged(const dsa_paged_cache_t* c, int32_t B, int64_t max_seq_len, const dsa_dims_t* d,
                              const uint8_t* q8, const float* q_scale, const float* w, const uint16_t* q,
                              uint16_t* out, float* out_f32, float* lse, int32_t* indices_out, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  dsa_status_t s = check_dims(d);
  if (s != DSA_OK) return s;
  REQUIRE(B >= 0 && max_seq_len >= 0, DSA_ERR_INVALID_ARGUMENT, "negative B or max_seq_len");
  REQUIRE(B <= dsa::kDecodeMaxSeqs, DSA_ERR_UNSUPPORTED, "B=%d sequences above %d per decode call", B,
          dsa::kDecodeMaxSeqs);
  if (B == 0) return ok();
  REQUIRE(max_seq_len >= 1, DSA_ERR_INVALID_ARGUMENT, "max_seq_len must be >= 1");
  s = check_cache(c, max_seq_len, B);
  if (s != DSA_OK) return s;
  REQUIRE_PTR(c->seq_lens);
  s = check_topk(max_seq_len, d->topk);
  if (s != DSA_OK) return s;
  REQUIRE_PTR(q8);
  REQUIRE_PTR(q_scale);
  REQUIRE_PTR(w);
  REQUIRE_PTR(q);
  REQUIRE_PTR(out);
  OPTIONAL_PTR(out_f32);
  OPTIONAL_PTR(lse);
  OPTIONAL_PTR(indices_out);
  const DecodeLayout L = decode_layout(d, B, max_seq_len);
  REQUIRE(workspace_bytes >= L.total, DSA_ERR_WORKSPACE_TOO_SMALL, "decode workspace %zu < %zu bytes",
          workspace_bytes, L.total);
  REQUIRE(workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) % kAlign) == 0,
          DSA_ERR_INVALID_ARGUMENT, "workspace must be non-null and 256-byte aligned");
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* logits = reinterpret_cast<float*>(ws + L.logits);
  int32_t* idx = indices_out ? indices_out : reinterpret_cast<int32_t*>(ws + L.indices);
  const int shift = block_shift_of(c->block_size);

  dsa::trace_call("dsa_decode_paged", workspace_bytes, L.total);
  hipError_t e = dsa::launch_indexer_decode(q8, q_scale, w, c->k8, c->k_scale, c->block_table,
                                            c->max_blocks_per_seq, shift, c->num_blocks, c->seq_lens, B,
                                            max_seq_len, d->H_I, d->D_I, logits, L.ld, stream);
  if (e != hipSuccess) return hip_status(e, "decode indexer launch");
  e = dsa::launch_topk(logits, L.ld, B, max_seq_len, 0, c->seq_lens, d->topk, idx, ws + L.topk, stream);
  if (e != hipSuccess) return hip_status(e, "top-k launch");
  dsa::MlaArgs a{};
  a.q = q;
  a.kv = c->kv;
  a.idx = idx;
  a.table = c->block_table;
  a.max_blocks = c->max_blocks_per_seq;
  a.block_shift = shift;
  a.num_blocks = c->num_blocks;
  a.per_row_table = 1;
  a.seq_lens = c->seq_lens;
  a.R = B;
  a.S = max_seq_len;
  a.q_start = 0;
  a.H = d->H;
  a.D_qk = d->D_qk;
  a.D_v = d->D_v;
  a.k = d->topk;
  a.sm_scale = d->sm_scale;
  a.nsplit = L.nsplit;
  a.out = out;
  a.out_f32 = out_f32;
  a.lse = lse;
  a.part_out = reinterpret_cast<float*>(ws + L.part_out);
  a.part_lse = reinterpret_cast<float*>(ws + L.part_lse);
  return hip_status(dsa::launch_sparse_mla(a, stream), "sparse MLA launch");
}

dsa_status_t dsa_quantize_fp8_rows(const uint16_t* x, int64_t rows, int32_t D, uint8_t* codes, float* scales,
                                   hipStream_t stream) {
  REQUIRE(rows >= 0, DSA_ERR_INVALID_ARGUMENT, "negative rows");
  REQUIRE(dsa::quantize_supported(D), DSA_ERR_UNSUPPORTED, "D=%d must be a multiple of 8 in [8, 512]", D);
  if (rows == 0) return ok();
  REQUIRE_PTR(x);
  REQUIRE_PTR(codes);
  REQUIRE_PTR(scales);
  return hip_status(dsa::launch_quantize_rows(x, rows, D, codes, scales, nullptr, stream), "quantize launch");
}

dsa_status_t dsa_quantize_fp8_rows_ue8m0(const uint16_t* x, int64_t rows, int32_t D, uint8_t* codes,
                                         uint8_t* exps, float* scales, hipStream_t stream) {
  REQUIRE(rows >= 0, DSA_ERR_INVALID_ARGUMENT, "negative rows");
  REQUIRE(dsa::quantize_supported(D), DSA_ERR_UNSUPPORTED, "D=%d must be a multiple of 8 in [8, 512]", D);
  if (rows == 0) return ok();
  REQUIRE_PTR(x);
  REQUIRE_PTR(codes);
  REQUIRE_PTR(exps);
  OPTIONAL_PTR(scales);
  return hip_status(dsa::launch_quantize_rows(x, rows, D, codes, scales, exps, stream), "quantize launch");
}

dsa_status_t dsa_append_paged(const dsa_paged_cache_t* c, int32_t B, const int32_t* seq_ids,
                              const int32_t* positions, int64_t n, int32_t D_I, int32_t D_qk, const uint16_t* k,
                              const uint16_t* kv, hipStream_t stream) {
  REQUIRE(n >= 0 && B >= 0, DSA_ERR_INVALID_ARGUMENT, "negative n or B");
  REQUIRE(dsa::quantize_supported(D_I), DSA_ERR_UNSUPPORTED, "D_I=%d must be a multiple of 8 in [8, 512]", D_I);
  REQUIRE(D_qk >= 8 && D_qk % 8 == 0, DSA_ERR_UNSUPPORTED, "D_qk=%d must be a positive multiple of 8", D_qk);
  if (n == 0) return ok();
  REQUIRE(B >= 1, DSA_ERR_INVALID_ARGUMENT, "B must be >= 1 when tokens are appended");
  dsa_status_t s = check_cache(c, 1, B);
  if (s != DSA_OK) return s;
  REQUIRE_PTR(seq_ids);
  REQUIRE_PTR(positions);
  REQUIRE_PTR(k);
  REQUIRE_PTR(kv);
  // the pools of the cache are written here (the struct's const is the readers' view)
  return hip_status(dsa::launch_append_paged(const_cast<uint8_t*>(c->k8), const_cast<float*>(c->k_scale),
                                             const_cast<uint16_t*>(c->kv), c->num_blocks,
                                             block_shift_of(c->block_size), c->block_table, c->max_blocks_per_seq,
                                             B, seq_ids, positions, n, D_I, D_qk, k, kv, stream),
                    "append launch");
}

dsa_status_t dsa_indexer_kl_loss(const uint16_t* q, const uint16_t* kv, int64_t T, int64_t S, int32_t H,
                                 int32_t D_qk, float sm_scale, int64_t q_start, const float* logits,
                                 int64_t ld_logits, float* dlogits, float* loss, hipStream_t stream) {
  REQUIRE(T >= 0 && S >= 0 && q_start >= 0, DSA_ERR_INVALID_ARGUMENT, "negative T, S or q_start");
  REQUIRE(dsa::indexer_kl_supported(H, D_qk), DSA_ERR_UNSUPPORTED,
          "KL loss with H=%d, D_qk=%d not supported (1 <= H <= 128, D_qk a multiple of 8 in [8, 576])", H, D_qk);
  if (T == 0) return ok();
  REQUIRE(S >= 1, DSA_ERR_INVALID_ARGUMENT, "S must be >= 1 when T > 0");
  REQUIRE(ld_logits >= S && ld_logits % 4 == 0, DSA_ERR_INVALID_ARGUMENT,
          "ld_logits=%lld must be >= S=%lld and a multiple of 4", (long long)ld_logits, (long long)S);
  REQUIRE(sm_scale > 0.0f && sm_scale < 1.0e30f, DSA_ERR_INVALID_ARGUMENT, "sm_scale must be positive and finite");
  REQUIRE_PTR(q);
  REQUIRE_PTR(kv);
  REQUIRE_PTR(logits);
  REQUIRE_PTR(dlogits);
  REQUIRE_PTR(loss);
  return hip_status(dsa::launch_indexer_kl(q, kv, T, S, H, D_qk, sm_scale, q_start, logits, ld_logits, dlogits, loss,
                                           stream),
                    "KL loss launch");
}

dsa_status_t dsa_indexer_kl_loss_sparse(const uint16_t* q, const uint16_t* kv, const int32_t* indices, int32_t k,
                                        const float* lse, int64_t T, int64_t S, int32_t H, int32_t D_qk,
                                        float sm_scale, int64_t q_start, const float* logits, int64_t ld_logits,
                                        float* dlogits, float* loss, hipStream_t stream) {
  REQUIRE(T >= 0 && S >= 0 && q_start >= 0, DSA_ERR_INVALID_ARGUMENT, "negative T, S or q_start");
  REQUIRE(dsa::indexer_kl_sparse_supported(H, D_qk, k), DSA_ERR_UNSUPPORTED,
          "sparse KL loss with H=%d, D_qk=%d, k=%d not supported (1 <= H <= 128, D_qk a multiple of 8 in "
          "[8, 576], 1 <= k <= 2048)", H, D_qk, k);
  if (T == 0) return ok();
  REQUIRE(S >= 1, DSA_ERR_INVALID_ARGUMENT, "S must be >= 1 when T > 0");
  REQUIRE(ld_logits >= S && ld_logits % 4 == 0, DSA_ERR_INVALID_ARGUMENT,
          "ld_logits=%lld must be >= S=%lld and a multiple of 4", (long long)ld_logits, (long long)S);
  REQUIRE(sm_scale > 0.0f && sm_scale < 1.0e30f, DSA_ERR_INVALID_ARGUMENT, "sm_scale must be positive and finite");
  REQUIRE_PTR(q);
  REQUIRE_PTR(kv);
  REQUIRE_PTR(indices);
  REQUIRE_PTR(lse);
  REQUIRE_PTR(logits);
  REQUIRE_PTR(dlogits);
  REQUIRE_PTR(loss);
  return hip_status(dsa::launch_indexer_kl_sparse(q, kv, indices, k, lse, T, S, H, D_qk, sm_scale, q_start, logits,
                                                  ld_logits, dlogits, loss, stream),
                    "sparse KL loss launch");
}

size_t dsa_indexer_bwd_workspace_size(int64_t T, int64_t S, int32_t D_I) {
  if (T <= 0 || S <= 0 || D_I <= 0) return 0;
  return dsa::indexer_bwd_workspace_bytes(T, S, D_I);
}

dsa_status_t dsa_indexer_bwd(const uint8_t* q8, const float* q_scale, const float* w, const uint8_t* k8,
                             const float* k_scale, int64_t T, int64_t S, int32_t H_I, int32_t D_I, int64_t q_start,
                             const float* dlogits, int64_t ld_dlogits, float* dq, float* dw, float* dk,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  REQUIRE(T >= 0 && S >= 0 && q_start >= 0, DSA_ERR_INVALID_ARGUMENT, "negative T, S or q_start");
  dsa_status_t s = check_indexer_dims(H_I, D_I);
  if (s != DSA_OK) return s;
  if (T == 0 && S == 0) return ok();
  REQUIRE(T >= 1 && S >= 1, DSA_ERR_INVALID_ARGUMENT, "T and S must both be >= 1 (or both 0)");
  REQUIRE(ld_dlogits >= S && ld_dlogits % 4 == 0, DSA_ERR_INVALID_ARGUMENT,
          "ld_dlogits=%lld must be >= S=%lld and a multiple of 4", (long long)ld_dlogits, (long long)S);
  REQUIRE_PTR(q8);
  REQUIRE_PTR(q_scale);
  REQUIRE_PTR(w);
  REQUIRE_PTR(k8);
  REQUIRE_PTR(k_scale);
  REQUIRE_PTR(dlogits);
  REQUIRE_PTR(dq);
  REQUIRE_PTR(dw);
  REQUIRE_PTR(dk);
  const size_t need = dsa::indexer_bwd_workspace_bytes(T, S, D_I);
  REQUIRE(workspace_bytes >= need, DSA_ERR_WORKSPACE_TOO_SMALL, "indexer backward workspace %zu < %zu bytes",
          workspace_bytes, need);
  REQUIRE_PTR(workspace);
  return hip_status(dsa::launch_indexer_bwd(q8, q_scale, w, k8, k_scale, T, S, H_I, D_I, q_start, dlogits,
                                            ld_dlogits, dq, dw, dk, workspace, stream),
                    "indexer backward launch");
}

dsa_status_t dsa_indexer_bwd_listed(const uint8_t* q8, const float* q_scale, const float* w, const uint8_t* k8,
                                    const float* k_scale, int64_t T, int64_t S, int32_t H_I, int32_t D_I,
                                    int64_t q_start, const int32_t* indices, int32_t k, const float* dlogits,
                                    int64_t ld_dlogits, float* dq, float* dw, float* dk, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  REQUIRE(T >= 0 && S >= 0 && q_start >= 0, DSA_ERR_INVALID_ARGUMENT, "negative T, S or q_start");
  dsa_status_t s = check_indexer_dims(H_I, D_I);
  if (s != DSA_OK) return s;
  REQUIRE(k >= 1, DSA_ERR_INVALID_ARGUMENT, "k=%d must be >= 1", k);
  if (T == 0 && S == 0) return ok();
  REQUIRE(T >= 1 && S >= 1, DSA_ERR_INVALID_ARGUMENT, "T and S must both be >= 1 (or both 0)");
  REQUIRE(ld_dlogits >= S && ld_dlogits % 4 == 0, DSA_ERR_INVALID_ARGUMENT,
          "ld_dlogits=%lld must be >= S=%lld and a multiple of 4", (long long)ld_dlogits, (long long)S);
  REQUIRE_PTR(q8);
  REQUIRE_PTR(q_scale);
  REQUIRE_PTR(w);
  REQUIRE_PTR(k8);
  REQUIRE_PTR(k_scale);
  REQUIRE_PTR(indices);
  REQUIRE_PTR(dlogits);
  REQUIRE_PTR(dq);
  REQUIRE_PTR(dw);
  REQUIRE_PTR(dk);
  const size_t need = dsa::indexer_bwd_workspace_bytes(T, S, D_I);
  REQUIRE(workspace_bytes >= need, DSA_ERR_WORKSPACE_TOO_SMALL, "indexer backward workspace %zu < %zu bytes",
          workspace_bytes, need);
  REQUIRE_PTR(workspace);
  return hip_status(dsa::launch_indexer_bwd(q8, q_scale, w, k8, k_scale, T, S, H_I, D_I, q_start, dlogits,
                                            ld_dlogits, dq, dw, dk, workspace, stream, indices, k),
                    "indexer backward launch");
}

}  // extern "C"
