// Fused down-projection, RoPE and append of new tokens (the step before
// attention):
//   c_kv[t] = W_DKV h[t]    k_R[t] = W_KR h[t]     (float32 accumulation,
//                                                   rounded to the activation type)
//   cache[slot[t]] = [c_kv[t] || RoPE(k_R[t], pos[t])], written exactly as
//   mla_cache_append writes those rounded c_kv and k_R.
// Source: keybo.xyz page, section "第一步，训练时" (c_kv = W_DKV x, the latent
// is all that is cached) and section "RoPE 为什么必须解耦" (k_R = RoPE(W_KR x),
// rotated before it is cached); dgblog.top page, section "1. 下采样（压缩）".
//
// DeepSeek-V2 rows from bfloat16 activations: two kernels.  The projection is
// weight-streaming (each weight byte is used by the T tokens and nothing
// else), so it is cut into 36 blocks of 16 output features x KS slices of
// d_model, one wave each, on v_mfma_f32_16x16x32_bf16 with the weight as the
// A operand and the tokens as B; each wave stores float32 partial sums.  The
// second kernel (one workgroup per token) adds the KS partials, rounds to bf16 and
// writes the row with the same code as the 576-wide append.  Any other shape
// or alignment: one workgroup per token computes the rounded c_kv and k_R into
// the workspace and the ordinary append kernel writes them.
//
// 16x16x32 operand layouts (lane l, g = l / 16, s = l % 16):
//   A: A[s][8g + e]      B: B[8g + e][s]      D: D[4g + r][s], r = 0..3
#include <algorithm>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kRow = 576;                       // d_c + d_R of the MFMA path
constexpr int kFeatBlocks = kRow / 16;          // 36
constexpr int kSliceSteps = 8;                  // 32-wide k-steps per slice: 20 slices (720 waves) at d_model 5120

// part[j][t][f] = sum over k in slice j (kSteps x 32 wide) of W[f][k] h[t][k],
// f < 512 from W_DKV, f >= 512 from W_KR.  Grid (36, slices), one wave.  All
// of the slice's weight fragments are loaded before the first MFMA (they
// stay in registers for every 16-token block), and each block's token
// fragments likewise, so a wave waits for memory once per block.
template <int kSteps>
__global__ void __launch_bounds__(64) kv_proj_partial(int32_t T, int32_t dm, const uint16_t* __restrict__ h,
                                                      const uint16_t* __restrict__ w_dkv,
                                                      const uint16_t* __restrict__ w_kr,
                                                      float* __restrict__ part) {
  const int lane = threadIdx.x, g = lane >> 4, s = lane & 15;
  const int f0 = 16 * blockIdx.x, f = f0 + s;
  const uint16_t* wrow = f < 512 ? w_dkv + (int64_t)f * dm : w_kr + (int64_t)(f - 512) * dm;
  const int k0 = blockIdx.y * (32 * kSteps);
  bf16x8 a[kSteps];
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int k = k0 + 32 * i;
    a[i] = k < dm ? *reinterpret_cast<const bf16x8*>(wrow + k + 8 * g) : bf16x8{};
  }
  for (int tb = 0; tb < T; tb += 16) {
    const uint16_t* hrow = h + (int64_t)min(tb + s, T - 1) * dm;   // rows past T: read a real row, not stored
    bf16x8 b[kSteps];
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      const int k = k0 + 32 * i;
      b[i] = k < dm ? *reinterpret_cast<const bf16x8*>(hrow + k + 8 * g) : bf16x8{};
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kSteps; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[i], acc, 0, 0, 0);
    if (tb + s < T)                                  // D[4g + r][s]: features f0 + 4g + r of token tb + s
      *reinterpret_cast<f32x4*>(part + ((int64_t)blockIdx.y * T + tb + s) * kRow + f0 + 4 * g) = acc;
  }
}

// Sum of the KS partials of token t, rounded to bf16, then the cache row.
// Four waves per token: wave w adds slices w, w + 4, ... (up to kPerWave of
// them, all loads in flight together), the four sums meet in LDS and wave 0
// writes the row.
constexpr int kPerWave = 8;                     // so KS <= 32 (d_model <= 8192 at 256-wide slices)
template <bool kE4M3>
__global__ void __launch_bounds__(256) kv_proj_finish(int32_t T, int32_t KS, const float* __restrict__ part,
                                                      const int32_t* __restrict__ pos,
                                                      const int64_t* __restrict__ slot, void* __restrict__ cache,
                                                      float* __restrict__ kv_scale, double log2_base) {
  __shared__ f32x4 red[3][2][64];
  __shared__ f32x2 redk[3][64];
  const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x4 x0[kPerWave], x1[kPerWave];
  f32x2 y[kPerWave];
#pragma unroll
  for (int i = 0; i < kPerWave; ++i) {
    const int j = min(wave + 4 * i, KS - 1);
    const float* pr = part + ((int64_t)j * T + t) * kRow;
    x0[i] = *reinterpret_cast<const f32x4*>(pr + 8 * lane);
    x1[i] = *reinterpret_cast<const f32x4*>(pr + 8 * lane + 4);
    // every lane loads (lanes >= 32 re-read pair 31 and drop it), so that no
    // load sits in a branch whose join would wait for it
    y[i] = *reinterpret_cast<const f32x2*>(pr + 512 + 2 * min(lane, 31));
  }
  // the RoPE angle of pair `lane` (float64 sine and cosine) while the partial
  // sums are in flight
  double rc = 0.0, rs = 0.0;
  if (wave == 0 && lane < 32) rope_angle(pos[t], lane, 64, log2_base, &rc, &rs);
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
  f32x2 kr = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kPerWave; ++i)
    if (wave + 4 * i < KS) {
      c0 += x0[i];
      c1 += x1[i];
      kr += y[i];
    }
  if (wave > 0) {
    red[wave - 1][0][lane] = c0;
    red[wave - 1][1][lane] = c1;
    redk[wave - 1][lane] = kr;
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    c0 += red[w][0][lane];
    c1 += red[w][1][lane];
    kr += redk[w][lane];
  }
  const u32x4_t c = {pack2_bf16(c0[0], c0[1]), pack2_bf16(c0[2], c0[3]), pack2_bf16(c1[0], c1[1]),
                     pack2_bf16(c1[2], c1[3])};
  append_row_576_cs<kE4M3>(c, pack2_bf16(kr[0], kr[1]), rc, rs, slot[t], cache, kv_scale, lane);
}

// Any shape: one workgroup per token, thread o computes output features o,
// o + 256, ...; results rounded to the activation type into c_out / k_out.
template <typename TA>
__global__ void __launch_bounds__(256) kv_proj_generic(int32_t dm, int32_t d_c, int32_t d_R,
                                                       const TA* __restrict__ h, const TA* __restrict__ w_dkv,
                                                       const TA* __restrict__ w_kr, TA* __restrict__ c_out,
                                                       TA* __restrict__ k_out) {
  const int t = blockIdx.x;
  for (int o = threadIdx.x; o < d_c + d_R; o += blockDim.x) {
    const TA* w = o < d_c ? w_dkv + (int64_t)o * dm : w_kr + (int64_t)(o - d_c) * dm;
    float acc = 0.f;
    for (int k = 0; k < dm; ++k) acc = __builtin_fmaf(io<TA>::load(w, k), io<TA>::load(h, (int64_t)t * dm + k), acc);
    if (o < d_c) io<TA>::store(c_out, (int64_t)t * d_c + o, acc);
    else io<TA>::store(k_out, (int64_t)t * d_R + (o - d_c), acc);
  }
}

struct ProjPlan {
  bool mfma;
  int32_t ks, kc;
  size_t mfma_bytes, generic_bytes;
};

ProjPlan plan_proj(const mla_dims& d, int32_t T, int32_t dm) {
  ProjPlan p{};
  p.kc = 32 * kSliceSteps;
  p.ks = (dm + p.kc - 1) / p.kc;
  p.mfma = d.act_dtype == MLA_BF16 && d.d_latent == 512 && d.d_rope == 64 && dm % 32 == 0 &&
           p.ks <= 4 * kPerWave && (d.kv_dtype == MLA_BF16 || d.kv_dtype == MLA_E4M3);
  p.mfma_bytes = p.mfma ? (size_t)p.ks * T * kRow * sizeof(float) : 0;
  const size_t es = d.act_dtype == MLA_F32 ? 4 : 2;
  const size_t cb = ((size_t)T * d.d_latent * es + 255) & ~(size_t)255;
  p.generic_bytes = cb + (size_t)T * d.d_rope * es;
  return p;
}

}  // namespace

size_t kv_project_workspace_bytes(const mla_dims& d, int32_t T, int32_t dm) {
  const ProjPlan p = plan_proj(d, T, dm);
  return std::max<size_t>(256, std::max(p.mfma_bytes, p.generic_bytes));
}

hipError_t launch_kv_project_append(const mla_dims& d, int32_t T, int32_t dm, const void* h, const void* w_dkv,
                                    const void* w_kr, const int32_t* pos, const int64_t* slot, void* cache,
                                    float* kv_scale, void* ws, hipStream_t s) {
  const ProjPlan p = plan_proj(d, T, dm);
  const bool aligned = (reinterpret_cast<uintptr_t>(h) | reinterpret_cast<uintptr_t>(w_dkv) |
                        reinterpret_cast<uintptr_t>(w_kr) | reinterpret_cast<uintptr_t>(cache)) % 16 == 0;
  if (p.mfma && aligned) {
    float* part = static_cast<float*>(ws);
    kv_proj_partial<kSliceSteps><<<dim3(kFeatBlocks, p.ks), 64, 0, s>>>(T, dm, static_cast<const uint16_t*>(h),
                                                                        static_cast<const uint16_t*>(w_dkv),
                                                                        static_cast<const uint16_t*>(w_kr), part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (d.kv_dtype == MLA_BF16)
      kv_proj_finish<false><<<T, 256, 0, s>>>(T, p.ks, part, pos, slot, cache, kv_scale, std::log2(d.rope_base));
    else
      kv_proj_finish<true><<<T, 256, 0, s>>>(T, p.ks, part, pos, slot, cache, kv_scale, std::log2(d.rope_base));
    return hipGetLastError();
  }
  const size_t es = d.act_dtype == MLA_F32 ? 4 : 2;
  char* c_out = static_cast<char*>(ws);
  char* k_out = c_out + (((size_t)T * d.d_latent * es + 255) & ~(size_t)255);
  if (d.act_dtype == MLA_F32)
    kv_proj_generic<float><<<T, 256, 0, s>>>(dm, d.d_latent, d.d_rope, static_cast<const float*>(h),
                                             static_cast<const float*>(w_dkv), static_cast<const float*>(w_kr),
                                             reinterpret_cast<float*>(c_out), reinterpret_cast<float*>(k_out));
  else
    kv_proj_generic<bf16_t><<<T, 256, 0, s>>>(dm, d.d_latent, d.d_rope, static_cast<const bf16_t*>(h),
                                              static_cast<const bf16_t*>(w_dkv), static_cast<const bf16_t*>(w_kr),
                                              reinterpret_cast<bf16_t*>(c_out), reinterpret_cast<bf16_t*>(k_out));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_cache_append(d, T, c_out, k_out, pos, slot, cache, kv_scale, s);
}

}  // namespace mla
