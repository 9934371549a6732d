// Internal launcher interface between the C ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include "../../include/mla.h"

namespace mla {

// Compute units the launch geometry is planned for when the runtime cannot
// report them (MI355X: 256).
constexpr int kNumCU = 256;
// Compute units of the current device (a partitioned MI355X reports fewer),
// queried once per device; kNumCU when there is no device to ask.
int device_cu_count();

// An append carried by the absorb_q launch (mla_absorb_q_append).
struct AppendArgs {
  int32_t T;
  const void* c_kv;
  const void* k_r;
  const int32_t* pos;
  const int64_t* slot;
  void* cache;
  float* kv_scale;
};

enum DecodeKernel { kDecodeGeneric = 0, kDecodeH64 = 1, kDecodeFp8 = 2 };

struct DecodePlan {
  int32_t parts;          // W: KV chunks the flattened page list is cut into
  int32_t head_groups;    // workgroups per part (heads split across them)
  DecodeKernel kernel;    // which decode kernel the dims select
  size_t ws_bytes;        // workspace needed
};

DecodePlan plan_decode(const mla_dims& d, int32_t batch, int32_t num_splits);

hipError_t launch_absorb_q(const mla_dims& d, int32_t B, const void* q_c, const void* q_r,
                           const int32_t* pos, const void* w_uk, void* q_abs, hipStream_t s);
hipError_t launch_cache_append(const mla_dims& d, int32_t T, const void* c_kv, const void* k_r,
                               const int32_t* pos, const int64_t* slot, void* cache,
                               float* kv_scale, hipStream_t s);
hipError_t launch_absorb_q_append(const mla_dims& d, int32_t B, const void* q_c, const void* q_r,
                                  const int32_t* q_pos, const void* w_uk, void* q_abs, const AppendArgs& app,
                                  hipStream_t s);
hipError_t launch_decode(const mla_dims& d, const DecodePlan& plan, int32_t B, const void* q_abs,
                         const void* cache, const float* kv_scale, const int32_t* block_table,
                         int32_t max_pages, int32_t bt_div, const int32_t* seq_lens,
                         const int32_t* seq_starts, void* ws, void* o_lat, float* lse, hipStream_t s);
hipError_t launch_up_v(const mla_dims& d, int32_t B, const void* o_lat, const void* w_uv, void* out,
                       hipStream_t s);

// q query tokens per sequence: B * q virtual sequences (see k_generic.hip);
// the workspace holds multi_extra_bytes of lengths, then the decode's own.
size_t multi_extra_bytes(int32_t B, int32_t q);
hipError_t launch_decode_multi(const mla_dims& d, const DecodePlan& plan, int32_t B, int32_t q, const void* q_abs,
                               const void* cache, const float* kv_scale, const int32_t* block_table,
                               int32_t max_pages, const int32_t* seq_lens, const int32_t* seq_starts, void* ws,
                               void* o_lat, float* lse, hipStream_t s);

size_t kv_project_workspace_bytes(const mla_dims& d, int32_t T, int32_t dm);
hipError_t launch_kv_project_append(const mla_dims& d, int32_t T, int32_t dm, const void* h, const void* w_dkv,
                                    const void* w_kr, const int32_t* pos, const int64_t* slot, void* cache,
                                    float* kv_scale, void* ws, hipStream_t s);

hipError_t launch_combine(const mla_dims& d, const DecodePlan& plan, int32_t B, const int32_t* seq_lens,
                          const int32_t* seq_starts, const float* ws_o, const float* ws_lse, const int64_t* ws_tbl,
                          void* o_lat, float* lse, hipStream_t s);


// MFMA projections (bf16); *handled = false when the shapes or alignments are
// not covered (for absorb_q, including those of the carried append, if any),
// and the caller then runs the generic kernels.
hipError_t launch_absorb_q_mfma(const mla_dims& d, int32_t B, const void* q_c, const void* q_r,
                                const int32_t* pos, const void* w_uk, void* q_abs, hipStream_t s,
                                bool* handled, const AppendArgs* append = nullptr);
hipError_t launch_up_v_mfma(const mla_dims& d, int32_t B, const void* o_lat, const void* w_uv, void* out,
                            hipStream_t s, bool* handled);

// Whether the MFMA decode kernels handle these dims.  E4M3 cache in 16-head
// groups (k_decode_fp8.hip, when n_h is not a multiple of 64):
bool fp8_decode_supported(const mla_dims& d);
hipError_t launch_decode_fp8(const mla_dims& d, const DecodePlan& plan, int32_t B, const void* q_abs,
                             const void* cache, const float* kv_scale, const int32_t* block_table,
                             int32_t max_pages, int32_t bt_div, const int32_t* seq_lens,
                             const int32_t* seq_starts, float* ws_o, float* ws_lse, int64_t* ws_tbl, void* o_lat,
                             float* lse, hipStream_t s);
// bf16 cache at 64-head multiples: each wave owns 32 heads and half of every
// page (k_decode_h64w.hip).
bool h64w_decode_supported(const mla_dims& d);
hipError_t launch_decode_h64w(const mla_dims& d, const DecodePlan& plan, int32_t B, const void* q_abs,
                              const void* cache, const int32_t* block_table, int32_t max_pages, int32_t bt_div,
                              const int32_t* seq_lens, const int32_t* seq_starts, float* ws_o, float* ws_lse,
                              int64_t* ws_tbl, void* o_lat, float* lse, hipStream_t s);
// E4M3 cache at 64-head multiples, codes converted to bf16 in registers
// (k_decode_e4m3_h64.hip).
bool e4m3_h64_decode_supported(const mla_dims& d);
hipError_t launch_decode_e4m3_h64(const mla_dims& d, const DecodePlan& plan, int32_t B,
                                  const void* q_abs, const void* cache, const float* kv_scale,
                                  const int32_t* block_table, int32_t max_pages, int32_t bt_div,
                                  const int32_t* seq_lens, const int32_t* seq_starts, float* ws_o,
                                  float* ws_lse, int64_t* ws_tbl, void* o_lat, float* lse, hipStream_t s);

}  // namespace mla
