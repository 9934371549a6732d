// C ABI: argument validation and dispatch.  Every check happens before any
// HIP call, so an invalid request launches nothing (and these paths run on a
// machine without a GPU).
#include <math.h>

#include <mutex>

#include "mla_internal.h"

namespace {

// ---- the no-allocation decode's scratch -------------------------------------
// mla_decode_noalloc keeps its split-KV workspace in this array instead of a
// caller buffer.  Every GPU the library runs on holds its own copy (its own
// address) from module load until the process ends.  In host code `scratch`
// is only a stand-in for the symbol: its device address is looked up once
// per device with hipGetSymbolAddress and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call for that device, with it current).
hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

thread_local int32_t g_last_hip_error = 0;

constexpr int32_t kMaxWidth = 1024;   // d_head, d_latent + d_rope limit of the generic kernels
constexpr int32_t kMaxModel = 1 << 20; // d_model limit of the fused projection
constexpr int64_t kMaxRows = 1 << 24;  // batch x query tokens of one decode call

bool valid_dtype(int32_t t, bool allow_e4m3) {
  return t == MLA_F32 || t == MLA_BF16 || (allow_e4m3 && t == MLA_E4M3);
}

mla_status check_dims(const mla_dims* d) {
  if (!d) return MLA_ERR_NULL;
  if (d->n_heads < 1 || d->d_head < 1 || d->d_latent < 1 || d->d_rope < 0 || d->block_size < 1)
    return MLA_ERR_SHAPE;
  if (d->d_rope % 2 != 0) return MLA_ERR_SHAPE;
  if (d->d_head > kMaxWidth || d->d_latent + d->d_rope > kMaxWidth || d->block_size > 4096)
    return MLA_ERR_SHAPE;
  if (!valid_dtype(d->act_dtype, false) || !valid_dtype(d->kv_dtype, true)) return MLA_ERR_DTYPE;
  // The decode kernels take the running maximum of raw scores and apply the
  // scale afterwards, which needs scale > 0 (a positive factor commutes with max).
  if (!isfinite(d->softmax_scale) || !(d->softmax_scale > 0.f)) return MLA_ERR_SHAPE;
  if (d->d_rope > 0 && !(d->rope_base > 0.0 && isfinite(d->rope_base))) return MLA_ERR_SHAPE;
  return MLA_OK;
}

mla_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MLA_OK;
  g_last_hip_error = static_cast<int32_t>(e);
  return MLA_ERR_HIP;
}

}  // namespace

extern "C" {

mla_status mla_absorb_q(const mla_dims* dims, int32_t batch, const void* q_c, const void* q_r,
                        const int32_t* q_pos, const void* w_uk, void* q_abs, void* stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 1) return MLA_ERR_SHAPE;
  if (!q_c || !q_pos || !w_uk || !q_abs || (dims->d_rope > 0 && !q_r)) return MLA_ERR_NULL;
  return hip_status(mla::launch_absorb_q(*dims, batch, q_c, q_r, q_pos, w_uk, q_abs,
                                         static_cast<hipStream_t>(stream)));
}

mla_status mla_cache_append(const mla_dims* dims, int32_t n_tokens, const void* c_kv,
                            const void* k_r, const int32_t* pos, const int64_t* slot,
                            int64_t num_pages, void* kv_cache, float* kv_scale, void* stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (n_tokens < 0 || num_pages < 1) return MLA_ERR_SHAPE;
  if (n_tokens == 0) return MLA_OK;
  if (!c_kv || !pos || !slot || !kv_cache || (dims->d_rope > 0 && !k_r)) return MLA_ERR_NULL;
  if (dims->kv_dtype == MLA_E4M3 && !kv_scale) return MLA_ERR_NULL;
  return hip_status(mla::launch_cache_append(*dims, n_tokens, c_kv, k_r, pos, slot, kv_cache,
                                             kv_scale, static_cast<hipStream_t>(stream)));
}

mla_status mla_absorb_q_append(const mla_dims* dims, int32_t batch, const void* q_c, const void* q_r,
                               const int32_t* q_pos, const void* w_uk, void* q_abs, int32_t n_tokens,
                               const void* c_kv, const void* k_r, const int32_t* pos, const int64_t* slot,
                               int64_t num_pages, void* kv_cache, float* kv_scale, void* stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 1 || n_tokens < 0 || num_pages < 1) return MLA_ERR_SHAPE;
  if (!q_c || !q_pos || !w_uk || !q_abs || (dims->d_rope > 0 && !q_r)) return MLA_ERR_NULL;
  if (n_tokens > 0) {
    if (!c_kv || !pos || !slot || !kv_cache || (dims->d_rope > 0 && !k_r)) return MLA_ERR_NULL;
    if (dims->kv_dtype == MLA_E4M3 && !kv_scale) return MLA_ERR_NULL;
  }
  const mla::AppendArgs app{n_tokens, c_kv, k_r, pos, slot, kv_cache, kv_scale};
  return hip_status(mla::launch_absorb_q_append(*dims, batch, q_c, q_r, q_pos, w_uk, q_abs, app,
                                                static_cast<hipStream_t>(stream)));
}

size_t mla_decode_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t num_splits) {
  if (check_dims(dims) != MLA_OK || batch < 1 || num_splits < 0 || num_splits > 65536) return 0;
  return mla::plan_decode(*dims, batch, num_splits).ws_bytes;
}

mla_status mla_decode(const mla_dims* dims, int32_t batch, const void* q_abs, const void* kv_cache,
                      const float* kv_scale, const int32_t* block_table, int32_t max_pages,
                      const int32_t* seq_lens, int32_t num_splits, void* workspace,
                      size_t workspace_bytes, void* o_lat, float* lse, void* stream) {
  return mla_decode_window(dims, batch, q_abs, kv_cache, kv_scale, block_table, max_pages, seq_lens, nullptr,
                           num_splits, workspace, workspace_bytes, o_lat, lse, stream);
}

mla_status mla_decode_window(const mla_dims* dims, int32_t batch, const void* q_abs, const void* kv_cache,
                             const float* kv_scale, const int32_t* block_table, int32_t max_pages,
                             const int32_t* seq_lens, const int32_t* seq_starts, int32_t num_splits,
                             void* workspace, size_t workspace_bytes, void* o_lat, float* lse, void* stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 1 || max_pages < 1 || num_splits < 0 || num_splits > 65536) return MLA_ERR_SHAPE;
  if (!q_abs || !kv_cache || !block_table || !seq_lens || !workspace || !o_lat) return MLA_ERR_NULL;
  if (dims->kv_dtype == MLA_E4M3 && !kv_scale) return MLA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return MLA_ERR_WORKSPACE;
  const mla::DecodePlan plan = mla::plan_decode(*dims, batch, num_splits);
  if (workspace_bytes < plan.ws_bytes) return MLA_ERR_WORKSPACE;
  return hip_status(mla::launch_decode(*dims, plan, batch, q_abs, kv_cache, kv_scale, block_table,
                                       max_pages, 1, seq_lens, seq_starts, workspace, o_lat, lse,
                                       static_cast<hipStream_t>(stream)));
}

mla_status mla_decode_noalloc(const mla_dims* dims, int32_t batch, const void* q_abs, const void* kv_cache,
                              const float* kv_scale, const int32_t* block_table, int32_t max_pages,
                              const int32_t* seq_lens, const int32_t* seq_starts, int32_t num_splits, void* o_lat,
                              float* lse, void* stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 1 || max_pages < 1 || num_splits < 0 || num_splits > 65536) return MLA_ERR_SHAPE;
  if (!q_abs || !kv_cache || !block_table || !seq_lens || !o_lat) return MLA_ERR_NULL;
  if (dims->kv_dtype == MLA_E4M3 && !kv_scale) return MLA_ERR_NULL;
  const mla::DecodePlan plan = mla::plan_decode(*dims, batch, num_splits);
  if (plan.ws_bytes > kScratchBytes) return MLA_ERR_WORKSPACE;   // checked before any HIP call
  void* ws = nullptr;
  hipError_t e = scratch_on_current_device(&ws);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(mla::launch_decode(*dims, plan, batch, q_abs, kv_cache, kv_scale, block_table, max_pages, 1,
                                       seq_lens, seq_starts, ws, o_lat, lse, static_cast<hipStream_t>(stream)));
}

size_t mla_decode_multi_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t q_len, int32_t num_splits) {
  if (check_dims(dims) != MLA_OK || batch < 1 || q_len < 1 || (int64_t)batch * q_len > kMaxRows ||
      num_splits < 0 || num_splits > 65536)
    return 0;
  return mla::multi_extra_bytes(batch, q_len) + mla::plan_decode(*dims, batch * q_len, num_splits).ws_bytes;
}

mla_status mla_decode_multi(const mla_dims* dims, int32_t batch, int32_t q_len, const void* q_abs,
                            const void* kv_cache, const float* kv_scale, const int32_t* block_table,
                            int32_t max_pages, const int32_t* seq_lens, const int32_t* seq_starts,
                            int32_t num_splits, void* workspace, size_t workspace_bytes, void* o_lat, float* lse,
                            void* stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 1 || q_len < 1 || (int64_t)batch * q_len > kMaxRows || max_pages < 1 || num_splits < 0 ||
      num_splits > 65536)
    return MLA_ERR_SHAPE;
  if (!q_abs || !kv_cache || !block_table || !seq_lens || !workspace || !o_lat) return MLA_ERR_NULL;
  if (dims->kv_dtype == MLA_E4M3 && !kv_scale) return MLA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return MLA_ERR_WORKSPACE;
  const int32_t rows = batch * q_len;
  const mla::DecodePlan plan = mla::plan_decode(*dims, rows, num_splits);
  if (workspace_bytes < mla::multi_extra_bytes(batch, q_len) + plan.ws_bytes) return MLA_ERR_WORKSPACE;
  return hip_status(mla::launch_decode_multi(*dims, plan, batch, q_len, q_abs, kv_cache, kv_scale, block_table,
                                             max_pages, seq_lens, seq_starts, workspace, o_lat, lse,
                                             static_cast<hipStream_t>(stream)));
}

mla_status mla_up_v(const mla_dims* dims, int32_t batch, const void* o_lat, const void* w_uv,
                    void* out, void* stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 1) return MLA_ERR_SHAPE;
  if (!o_lat || !w_uv || !out) return MLA_ERR_NULL;
  return hip_status(mla::launch_up_v(*dims, batch, o_lat, w_uv, out, static_cast<hipStream_t>(stream)));
}

size_t mla_kv_project_workspace_bytes(const mla_dims* dims, int32_t n_tokens, int32_t d_model) {
  if (check_dims(dims) != MLA_OK || n_tokens < 0 || d_model < 1 || d_model > kMaxModel) return 0;
  return mla::kv_project_workspace_bytes(*dims, n_tokens, d_model);
}

mla_status mla_kv_project_append(const mla_dims* dims, int32_t n_tokens, int32_t d_model, const void* h,
                                 const void* w_dkv, const void* w_kr, const int32_t* pos, const int64_t* slot,
                                 int64_t num_pages, void* kv_cache, float* kv_scale, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  mla_status st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (n_tokens < 0 || num_pages < 1 || d_model < 1 || d_model > kMaxModel) return MLA_ERR_SHAPE;
  if (n_tokens == 0) return MLA_OK;
  if (!h || !w_dkv || !pos || !slot || !kv_cache || !workspace || (dims->d_rope > 0 && !w_kr))
    return MLA_ERR_NULL;
  if (dims->kv_dtype == MLA_E4M3 && !kv_scale) return MLA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0 ||
      workspace_bytes < mla::kv_project_workspace_bytes(*dims, n_tokens, d_model))
    return MLA_ERR_WORKSPACE;
  return hip_status(mla::launch_kv_project_append(*dims, n_tokens, d_model, h, w_dkv, w_kr, pos, slot, kv_cache,
                                                  kv_scale, workspace, static_cast<hipStream_t>(stream)));
}

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "required pointer is NULL";
    case MLA_ERR_SHAPE: return "size out of range or unsupported";
    case MLA_ERR_DTYPE: return "unknown or unsupported dtype";
    case MLA_ERR_WORKSPACE: return "workspace too small or misaligned";
    case MLA_ERR_UNSUPPORTED: return "no kernel for this request";
    case MLA_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t mla_last_hip_error(void) { return g_last_hip_error; }

int32_t mla_abi_version(void) { return 1; }

}  // extern "C"
