// Generic kernels: any head/latent/RoPE widths, float32 or bfloat16 activations,
// float32 / bfloat16 / E4M3 cache.  Plain FMA arithmetic; the MFMA decode
// kernels for DeepSeek-V2 shapes live in k_decode_h64w.hip (bf16 cache),
// k_decode_e4m3_h64.hip and k_decode_fp8.hip (E4M3 cache).
#include <cmath>

#include <atomic>

#include "mla_device.h"
#include "mla_internal.h"

#include <math.h>

namespace mla {

// ---------------------------------------------------------------------------
// absorb_q: q_abs[b,h,:d_c] = W_UK[h]^T q_c[b,h]; q_abs[b,h,d_c:] = RoPE(q_r[b,h], pos[b])
// (score identity with W_UK moved onto the query side)
// grid (n_h, ceil(d_c/256), ceil(B/kBB)), block 256
// ---------------------------------------------------------------------------
constexpr int kBB = 16;

template <typename T>
__global__ void __launch_bounds__(256) absorb_q_generic(int32_t B, int32_t n_h, int32_t d_h,
                                                        int32_t d_c, int32_t d_R,
                                                        const T* __restrict__ q_c,
                                                        const T* __restrict__ q_r,
                                                        const int32_t* __restrict__ pos,
                                                        const T* __restrict__ w_uk,
                                                        T* __restrict__ q_abs, double log2_base) {
  extern __shared__ float sq[];  // [kBB][d_h]
  const int h = blockIdx.x;
  const int c = blockIdx.y * blockDim.x + threadIdx.x;
  const int b0 = blockIdx.z * kBB;
  const int nb = min(kBB, B - b0);
  const int64_t D = d_c + d_R;
  for (int i = threadIdx.x; i < kBB * d_h; i += blockDim.x) {
    int bb = i / d_h, k = i % d_h;
    sq[i] = bb < nb ? io<T>::load(q_c, ((int64_t)(b0 + bb) * n_h + h) * d_h + k) : 0.f;
  }
  __syncthreads();
  if (c < d_c) {
    float acc[kBB];
#pragma unroll
    for (int bb = 0; bb < kBB; ++bb) acc[bb] = 0.f;
    for (int i = 0; i < d_h; ++i) {
      float w = io<T>::load(w_uk, ((int64_t)h * d_h + i) * d_c + c);
#pragma unroll
      for (int bb = 0; bb < kBB; ++bb) acc[bb] += w * sq[bb * d_h + i];
    }
#pragma unroll
    for (int bb = 0; bb < kBB; ++bb)
      if (bb < nb) io<T>::store(q_abs, ((int64_t)(b0 + bb) * n_h + h) * D + c, acc[bb]);
  }
  if (blockIdx.y == 0 && d_R > 0) {
    const int half = d_R / 2;
    for (int i = threadIdx.x; i < nb * half; i += blockDim.x) {
      int bb = i / half, p = i % half;
      int64_t src = ((int64_t)(b0 + bb) * n_h + h) * d_R + 2 * p;
      float y0, y1;
      rope_pair(io<T>::load(q_r, src), io<T>::load(q_r, src + 1), pos[b0 + bb], p, d_R, log2_base, &y0, &y1);
      int64_t dst = ((int64_t)(b0 + bb) * n_h + h) * D + d_c + 2 * p;
      io<T>::store(q_abs, dst, y0);
      io<T>::store(q_abs, dst + 1, y1);
    }
  }
}

// ---------------------------------------------------------------------------
// cache_append: one wave per new token.  row = [c_kv || RoPE(k_r, pos)],
// written to the slot's page/offset; E4M3 rows get one float32 scale.
// ---------------------------------------------------------------------------
constexpr int kMaxRowPerLane = 32;  // D <= 2048

template <typename T, int KV>
__global__ void __launch_bounds__(64) cache_append_generic(int32_t d_c, int32_t d_R,
                                                           const T* __restrict__ c_kv,
                                                           const T* __restrict__ k_r,
                                                           const int32_t* __restrict__ pos,
                                                           const int64_t* __restrict__ slot,
                                                           void* __restrict__ cache,
                                                           float* __restrict__ kv_scale,
                                                           double log2_base) {
  const int t = blockIdx.x, lane = threadIdx.x;
  const int D = d_c + d_R;
  const int64_t s = slot[t];
  const int32_t p = pos[t];
  float v[kMaxRowPerLane];
  int n = 0;
  for (int e = lane; e < D; e += 64, ++n) {
    float x;
    if (e < d_c) {
      x = io<T>::load(c_kv, (int64_t)t * d_c + e);
    } else {
      int r = e - d_c, pr = r >> 1;
      float y0, y1;
      rope_pair(io<T>::load(k_r, (int64_t)t * d_R + 2 * pr), io<T>::load(k_r, (int64_t)t * d_R + 2 * pr + 1),
                p, pr, d_R, log2_base, &y0, &y1);
      x = (r & 1) ? y1 : y0;
    }
    v[n] = x;
  }
  if constexpr (KV == MLA_F32) {
    float* dst = static_cast<float*>(cache) + s * D;
    n = 0;
    for (int e = lane; e < D; e += 64, ++n) dst[e] = v[n];
  } else if constexpr (KV == MLA_BF16) {
    uint16_t* dst = static_cast<uint16_t*>(cache) + s * D;
    n = 0;
    for (int e = lane; e < D; e += 64, ++n) dst[e] = f32_to_bf16(v[n]);
  } else {
    float amax = 0.f;
    for (int i = 0; i < n; ++i) amax = fmaxf(amax, fabsf(v[i]));
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float sc = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    uint8_t* dst = static_cast<uint8_t*>(cache) + s * D;
    n = 0;
    for (int e = lane; e < D; e += 64, ++n) dst[e] = static_cast<uint8_t>(f32_to_e4m3(__fdiv_rn(v[n], sc)));
    if (lane == 0) kv_scale[s] = sc;
  }
}

// The DeepSeek-V2 row (d_c = 512, d_R = 64) from bfloat16 inputs: lane l
// holds latent elements 8l..8l+7 (one 16-B load) and, for l < 32, RoPE pair
// l, so the row takes one load and one store instruction per part.  A bf16
// cache receives the latent bits unchanged (bf16 -> float -> bf16 is exact).
template <int KV>
__global__ void __launch_bounds__(64) cache_append_576(const uint16_t* __restrict__ c_kv,
                                                       const uint16_t* __restrict__ k_r,
                                                       const int32_t* __restrict__ pos,
                                                       const int64_t* __restrict__ slot,
                                                       void* __restrict__ cache,
                                                       float* __restrict__ kv_scale, double log2_base) {
  const int t = blockIdx.x, lane = threadIdx.x;
  const u32x4_t c = *reinterpret_cast<const u32x4_t*>(c_kv + (int64_t)t * 512 + 8 * lane);
  uint32_t kp = 0;
  if (lane < 32) kp = *reinterpret_cast<const uint32_t*>(k_r + (int64_t)t * 64 + 2 * lane);
  append_row_576<KV == MLA_E4M3>(c, kp, pos[t], slot[t], cache, kv_scale, log2_base, lane);
}

// ---------------------------------------------------------------------------
// decode (generic): one workgroup per (part, head); 16-token sub-tiles staged
// in LDS as float32; single-pass online softmax; per-segment result either
// final (segment = whole sequence) or a partial for the log-sum-exp merge.
// ---------------------------------------------------------------------------
constexpr int kGenMaxD = 1024;
constexpr int kGenRows = 16;

template <typename TQ, int KV>
__global__ void __launch_bounds__(256) decode_generic(
    int32_t B, int32_t n_h, int32_t d_c, int32_t d_R, int32_t bs, int32_t W, float scale,
    const TQ* __restrict__ q_abs, const void* __restrict__ cache, const float* __restrict__ kv_scale,
    const int32_t* __restrict__ block_table, int32_t max_pages, int32_t bt_div,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ seq_starts, float* __restrict__ ws_o,
    float* __restrict__ ws_lse, int64_t* __restrict__ ws_tbl, TQ* __restrict__ o_lat, float* __restrict__ lse) {
  __shared__ int32_t scan[257];
  __shared__ float tile[kGenRows * kGenMaxD];
  __shared__ float q[kGenMaxD];
  __shared__ float sc[kGenRows];
  const int w = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int D = d_c + d_R;
  int32_t chunk;
  page_prefix(seq_lens, seq_starts, B, bs, scan, &chunk);
  const int64_t P = scan[blockDim.x];
  if (P == 0) return;
  const int64_t x1 = part_start(w + 1, P, W);
  int64_t x = part_start(w, P, W);
  constexpr int kCols = kGenMaxD / 256;
  while (x < x1) {
    int32_t b;
    int64_t first;
    locate_page(seq_lens, seq_starts, B, bs, scan, chunk, x, &b, &first);
    // window [st, L): pages from fp = st / bs on; L and jp count from there,
    // and the first lo rows of page fp lie before the window
    const int32_t st = seq_start(seq_starts, b);
    const int32_t fp = st / bs, lo = st - fp * bs;
    const int32_t L = seq_lens[b] - fp * bs;
    const int64_t np = window_pages(seq_lens[b], st, bs);
    const int64_t jp0 = x - first;
    const int64_t jp1 = min(np, jp0 + (x1 - x));
    if (jp0 == 0 && h == 0 && tid < 4) {                         // the merge's part range of sequence b
      const int64_t v[4] = {w, part_of_page(first + np - 1, P, W), np, P};
      ws_tbl[4 * (int64_t)b + tid] = v[tid];
    }
    __syncthreads();
    for (int i = tid; i < D; i += blockDim.x) q[i] = io<TQ>::load(q_abs, ((int64_t)b * n_h + h) * D + i);
    float m = -INFINITY, l = 0.f;
    float acc[kCols];
#pragma unroll
    for (int k = 0; k < kCols; ++k) acc[k] = 0.f;
    for (int64_t jp = jp0; jp < jp1; ++jp) {
      const int64_t page = block_table[(int64_t)(b / bt_div) * max_pages + fp + jp];
      const int ntok = (int)min<int64_t>(bs, (int64_t)L - jp * bs);
      const int tlo = jp == 0 ? lo : 0;                          // rows before the window: masked, zeroed
      for (int t0 = tlo & ~(kGenRows - 1); t0 < ntok; t0 += kGenRows) {
        const int nt = min(kGenRows, ntok - t0);
        __syncthreads();
        for (int i = tid; i < nt * D; i += blockDim.x) {
          int r = i / D, e = i % D;
          int64_t sl = page * bs + t0 + r;
          float val;
          if (t0 + r < tlo) val = 0.f;
          else if constexpr (KV == MLA_F32) val = static_cast<const float*>(cache)[sl * D + e];
          else if constexpr (KV == MLA_BF16) val = bf16_to_f32(static_cast<const uint16_t*>(cache)[sl * D + e]);
          else val = e4m3_to_f32(static_cast<const uint8_t*>(cache)[sl * D + e]) * kv_scale[sl];
          tile[r * D + e] = val;
        }
        __syncthreads();
        {
          const int r = tid / 16, sub = tid % 16;
          float part = 0.f;
          if (r < nt)
            for (int e = sub; e < D; e += 16) part += q[e] * tile[r * D + e];
          for (int off = 8; off > 0; off >>= 1) part += __shfl_xor(part, off, 16);
          if (sub == 0) sc[r] = (r < nt && t0 + r >= tlo) ? part * scale : -INFINITY;
        }
        __syncthreads();
        float mt = -INFINITY;
        for (int r = 0; r < nt; ++r) mt = fmaxf(mt, sc[r]);
        const float m_new = fmaxf(m, mt);
        const float alpha = expf(m - m_new);
        float p[kGenRows];
        float ps = 0.f;
        for (int r = 0; r < kGenRows; ++r) {
          p[r] = r < nt ? expf(sc[r] - m_new) : 0.f;
          ps += p[r];
        }
        l = l * alpha + ps;
#pragma unroll
        for (int k = 0; k < kCols; ++k) {
          const int c = tid + 256 * k;
          if (c < d_c) {
            float a = acc[k] * alpha;
            for (int r = 0; r < nt; ++r) a += p[r] * tile[r * D + c];
            acc[k] = a;
          }
        }
        m = m_new;
      }
    }
    const bool whole = (jp0 == 0 && jp1 == np);
    const float inv_l = 1.f / l;
    const float lse_v = m + logf(l);
#pragma unroll
    for (int k = 0; k < kCols; ++k) {
      const int c = tid + 256 * k;
      if (c < d_c) {
        if (whole) io<TQ>::store(o_lat, ((int64_t)b * n_h + h) * d_c + c, acc[k] * inv_l);
        else ws_o[(((int64_t)w + b) * n_h + h) * d_c + c] = acc[k] * inv_l;
      }
    }
    if (tid == 0) {
      if (whole) { if (lse) lse[(int64_t)b * n_h + h] = lse_v; }
      else ws_lse[((int64_t)w + b) * n_h + h] = lse_v;
    }
    x += jp1 - jp0;
  }
}

// ---------------------------------------------------------------------------
// combine: log-sum-exp merge of a sequence's segment partials.
// grid (B, n_h), block 64 (one wave); lane handles 4-column groups of the
// latent row.  Sequences with a single segment were written by the decode
// kernel; empty sequences get o_lat = 0, lse = -inf here.
// ---------------------------------------------------------------------------
constexpr int kCombMaxSeg = 64;   // segments merged per pass (more are folded in passes)

template <typename TO>
__global__ void __launch_bounds__(64) combine_kernel(int32_t B, int32_t n_h, int32_t d_c, int32_t bs,
                                                     int32_t W, const int32_t* __restrict__ seq_lens,
                                                     const int32_t* __restrict__ seq_starts,
                                                     const float* __restrict__ ws_o,
                                                     const float* __restrict__ ws_lse,
                                                     const int64_t* __restrict__ ws_tbl,
                                                     TO* __restrict__ o_lat, float* __restrict__ lse) {
  __shared__ float wgt[kCombMaxSeg];
  __shared__ int32_t slot[kCombMaxSeg];
  const int b = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  // part range of a sequence with pages: written by the decode kernel (ws_tbl)
  const int64_t np = window_pages(seq_lens[b], seq_start(seq_starts, b), bs);
  const int64_t row = (int64_t)b * n_h + h;
  if (np == 0) {
    for (int c = lane; c < d_c; c += 64) io<TO>::store(o_lat, row * d_c + c, 0.f);
    if (lane == 0 && lse) lse[row] = -INFINITY;
    return;
  }
  const int64_t w0 = ws_tbl[4 * (int64_t)b], w1 = ws_tbl[4 * (int64_t)b + 1], P = ws_tbl[4 * (int64_t)b + 3];
  if (w0 == w1) return;
  const int64_t nparts = w1 - w0 + 1;
  if (nparts <= 64 && d_c % 4 == 0 && d_c <= 1024) {
    // One lane per part: its lse (-inf for a part without pages) and weight,
    // then the partial rows four parts at a time with all their loads in
    // flight together (three dependent memory round trips in all).
    float e = -INFINITY;
    if (lane < nparts) {
      const int64_t w = w0 + lane;
      if (part_start(w, P, W) < part_start(w + 1, P, W)) e = ws_lse[(w + b) * n_h + h];
    }
    float M = e;
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float wl = e == -INFINITY ? 0.f : expf(e - M);
    float denom = wl;
    for (int off = 32; off > 0; off >>= 1) denom += __shfl_xor(denom, off);
    const int ncol4 = d_c / 4;
    float4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = 0; k0 < nparts; k0 += 4) {
      float wk[4];
      float4 v[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = min<int64_t>(k0 + i, nparts - 1);
        wk[i] = k0 + i < nparts ? __shfl(wl, k) : 0.f;
        const float4* src = reinterpret_cast<const float4*>(ws_o + ((w0 + k + b) * n_h + h) * d_c);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c4 = lane + 64 * j;
          v[i][j] = (wk[i] != 0.f && c4 < ncol4) ? src[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[j].x += wk[i] * v[i][j].x; acc[j].y += wk[i] * v[i][j].y;
          acc[j].z += wk[i] * v[i][j].z; acc[j].w += wk[i] * v[i][j].w;
        }
    }
    const float inv = 1.f / denom;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c4 = lane + 64 * j;
      if (c4 < ncol4) {
        io<TO>::store(o_lat, row * d_c + 4 * c4 + 0, acc[j].x * inv);
        io<TO>::store(o_lat, row * d_c + 4 * c4 + 1, acc[j].y * inv);
        io<TO>::store(o_lat, row * d_c + 4 * c4 + 2, acc[j].z * inv);
        io<TO>::store(o_lat, row * d_c + 4 * c4 + 3, acc[j].w * inv);
      }
    }
    if (lane == 0 && lse) lse[row] = M + logf(denom);
    return;
  }
  // reference max over the non-empty parts (parts inside [w0, w1] can be empty
  // when there are more parts than pages)
  float M = -INFINITY;
  for (int64_t w = w0 + lane; w <= w1; w += 64)
    if (part_start(w, P, W) < part_start(w + 1, P, W)) M = fmaxf(M, ws_lse[(w + b) * n_h + h]);
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float denom = 0.f;
  const int ncol4 = (d_c % 4 == 0) ? d_c / 4 : 0;   // float4 path needs 16-byte rows
  float4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t base = w0; base <= w1; base += kCombMaxSeg) {
    const int nseg = (int)min<int64_t>(kCombMaxSeg, w1 + 1 - base);
    __syncthreads();
    if (lane < nseg) {
      const int64_t w = base + lane;
      const bool live = part_start(w, P, W) < part_start(w + 1, P, W);
      wgt[lane] = live ? expf(ws_lse[(w + b) * n_h + h] - M) : 0.f;
      slot[lane] = (int32_t)(w + b);
    }
    __syncthreads();
    for (int k = 0; k < nseg; ++k) {
      const float wk = wgt[k];
      denom += wk;
      if (wk == 0.f) continue;
      const float4* src = reinterpret_cast<const float4*>(ws_o + ((int64_t)slot[k] * n_h + h) * d_c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c4 = lane + 64 * j;
        if (c4 < ncol4) {
          const float4 v = src[c4];
          acc[j].x += wk * v.x; acc[j].y += wk * v.y; acc[j].z += wk * v.z; acc[j].w += wk * v.w;
        }
      }
    }
  }
  const float inv = 1.f / denom;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c4 = lane + 64 * j;
    if (c4 < ncol4) {
      io<TO>::store(o_lat, row * d_c + 4 * c4 + 0, acc[j].x * inv);
      io<TO>::store(o_lat, row * d_c + 4 * c4 + 1, acc[j].y * inv);
      io<TO>::store(o_lat, row * d_c + 4 * c4 + 2, acc[j].z * inv);
      io<TO>::store(o_lat, row * d_c + 4 * c4 + 3, acc[j].w * inv);
    }
  }
  for (int c = 4 * ncol4 + lane; c < d_c; c += 64) {       // d_c not a multiple of 4
    float o = 0.f;
    for (int64_t w = w0; w <= w1; ++w)
      if (part_start(w, P, W) < part_start(w + 1, P, W))
        o += expf(ws_lse[(w + b) * n_h + h] - M) * ws_o[((w + b) * n_h + h) * d_c + c];
    io<TO>::store(o_lat, row * d_c + c, o * inv);
  }
  if (lane == 0 && lse) lse[row] = M + logf(denom);
}

// ---------------------------------------------------------------------------
// up_v (generic): out[b,h,i] = W_UV[h,i,:] . o_lat[b,h,:]
// grid (n_h, ceil(B/kBB)), block 256 (4 waves, rows i strided by 4)
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) up_v_generic(int32_t B, int32_t n_h, int32_t d_h, int32_t d_c,
                                                    const T* __restrict__ o_lat,
                                                    const T* __restrict__ w_uv, T* __restrict__ out) {
  extern __shared__ float so[];  // [kBB][d_c]
  const int h = blockIdx.x, b0 = blockIdx.y * kBB, nb = min(kBB, B - b0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kBB * d_c; i += blockDim.x) {
    int bb = i / d_c, c = i % d_c;
    so[i] = bb < nb ? io<T>::load(o_lat, ((int64_t)(b0 + bb) * n_h + h) * d_c + c) : 0.f;
  }
  __syncthreads();
  for (int i = wave; i < d_h; i += 4) {
    for (int bb = 0; bb < nb; ++bb) {
      float a = 0.f;
      for (int c = lane; c < d_c; c += 64) a += io<T>::load(w_uv, ((int64_t)h * d_h + i) * d_c + c) * so[bb * d_c + c];
      for (int off = 32; off > 0; off >>= 1) a += __shfl_xor(a, off);
      if (lane == 0) io<T>::store(out, ((int64_t)(b0 + bb) * n_h + h) * d_h + i, a);
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_absorb_q(const mla_dims& d, int32_t B, const void* q_c, const void* q_r,
                           const int32_t* pos, const void* w_uk, void* q_abs, hipStream_t s) {
  bool handled = false;
  hipError_t e = launch_absorb_q_mfma(d, B, q_c, q_r, pos, w_uk, q_abs, s, &handled);
  if (handled || e != hipSuccess) return e;
  dim3 grid(d.n_heads, (d.d_latent + 255) / 256, (B + kBB - 1) / kBB);
  size_t shm = sizeof(float) * kBB * d.d_head;
  if (d.act_dtype == MLA_F32)
    absorb_q_generic<float><<<grid, 256, shm, s>>>(B, d.n_heads, d.d_head, d.d_latent, d.d_rope,
        (const float*)q_c, (const float*)q_r, pos, (const float*)w_uk, (float*)q_abs, std::log2(d.rope_base));
  else
    absorb_q_generic<bf16_t><<<grid, 256, shm, s>>>(B, d.n_heads, d.d_head, d.d_latent, d.d_rope,
        (const bf16_t*)q_c, (const bf16_t*)q_r, pos, (const bf16_t*)w_uk, (bf16_t*)q_abs, std::log2(d.rope_base));
  return hipGetLastError();
}

template <typename T>
static void append_dispatch(const mla_dims& d, int32_t T_, const void* c_kv, const void* k_r,
                            const int32_t* pos, const int64_t* slot, void* cache, float* kv_scale,
                            hipStream_t s) {
  const T* c = static_cast<const T*>(c_kv);
  const T* k = static_cast<const T*>(k_r);
  if (d.kv_dtype == MLA_F32)
    cache_append_generic<T, MLA_F32><<<T_, 64, 0, s>>>(d.d_latent, d.d_rope, c, k, pos, slot, cache, kv_scale, std::log2(d.rope_base));
  else if (d.kv_dtype == MLA_BF16)
    cache_append_generic<T, MLA_BF16><<<T_, 64, 0, s>>>(d.d_latent, d.d_rope, c, k, pos, slot, cache, kv_scale, std::log2(d.rope_base));
  else
    cache_append_generic<T, MLA_E4M3><<<T_, 64, 0, s>>>(d.d_latent, d.d_rope, c, k, pos, slot, cache, kv_scale, std::log2(d.rope_base));
}

hipError_t launch_cache_append(const mla_dims& d, int32_t T_, const void* c_kv, const void* k_r,
                               const int32_t* pos, const int64_t* slot, void* cache,
                               float* kv_scale, hipStream_t s) {
  const bool aligned = (reinterpret_cast<uintptr_t>(c_kv) & 15u) == 0 && (reinterpret_cast<uintptr_t>(k_r) & 3u) == 0 &&
                       (reinterpret_cast<uintptr_t>(cache) & 15u) == 0;
  if (d.act_dtype == MLA_BF16 && d.d_latent == 512 && d.d_rope == 64 && aligned &&
      (d.kv_dtype == MLA_BF16 || d.kv_dtype == MLA_E4M3)) {
    auto c = static_cast<const uint16_t*>(c_kv);
    auto k = static_cast<const uint16_t*>(k_r);
    if (d.kv_dtype == MLA_BF16)
      cache_append_576<MLA_BF16><<<T_, 64, 0, s>>>(c, k, pos, slot, cache, kv_scale, std::log2(d.rope_base));
    else
      cache_append_576<MLA_E4M3><<<T_, 64, 0, s>>>(c, k, pos, slot, cache, kv_scale, std::log2(d.rope_base));
    return hipGetLastError();
  }
  if (d.act_dtype == MLA_F32) append_dispatch<float>(d, T_, c_kv, k_r, pos, slot, cache, kv_scale, s);
  else append_dispatch<bf16_t>(d, T_, c_kv, k_r, pos, slot, cache, kv_scale, s);
  return hipGetLastError();
}

hipError_t launch_absorb_q_append(const mla_dims& d, int32_t B, const void* q_c, const void* q_r,
                                  const int32_t* q_pos, const void* w_uk, void* q_abs, const AppendArgs& app,
                                  hipStream_t s) {
  bool handled = false;
  if (app.T > 0) {
    hipError_t e = launch_absorb_q_mfma(d, B, q_c, q_r, q_pos, w_uk, q_abs, s, &handled, &app);
    if (handled || e != hipSuccess) return e;
  }
  hipError_t e = launch_absorb_q(d, B, q_c, q_r, q_pos, w_uk, q_abs, s);   // separately when not covered
  if (e != hipSuccess || app.T == 0) return e;
  return launch_cache_append(d, app.T, app.c_kv, app.k_r, app.pos, app.slot, app.cache, app.kv_scale, s);
}

hipError_t launch_combine(const mla_dims& d, const DecodePlan& plan, int32_t B, const int32_t* seq_lens,
                          const int32_t* seq_starts, const float* ws_o, const float* ws_lse, const int64_t* ws_tbl,
                          void* o_lat, float* lse, hipStream_t s) {
  dim3 grid(B, d.n_heads);
  if (d.act_dtype == MLA_F32)
    combine_kernel<float><<<grid, 64, 0, s>>>(B, d.n_heads, d.d_latent, d.block_size, plan.parts, seq_lens,
                                               seq_starts, ws_o, ws_lse, ws_tbl, static_cast<float*>(o_lat), lse);
  else
    combine_kernel<bf16_t><<<grid, 64, 0, s>>>(B, d.n_heads, d.d_latent, d.block_size, plan.parts, seq_lens,
                                                seq_starts, ws_o, ws_lse, ws_tbl, static_cast<bf16_t*>(o_lat), lse);
  return hipGetLastError();
}

template <typename TQ>
static void decode_generic_dispatch(const mla_dims& d, const DecodePlan& plan, int32_t B,
                                    const void* q_abs, const void* cache, const float* kv_scale,
                                    const int32_t* bt, int32_t max_pages, int32_t bt_div,
                                    const int32_t* seq_lens, const int32_t* seq_starts, float* ws_o,
                                    float* ws_lse, int64_t* ws_tbl, void* o_lat, float* lse, hipStream_t s) {
  dim3 grid(plan.parts, d.n_heads);
  const TQ* q = static_cast<const TQ*>(q_abs);
  TQ* o = static_cast<TQ*>(o_lat);
  if (d.kv_dtype == MLA_F32)
    decode_generic<TQ, MLA_F32><<<grid, 256, 0, s>>>(B, d.n_heads, d.d_latent, d.d_rope, d.block_size, plan.parts,
        d.softmax_scale, q, cache, kv_scale, bt, max_pages, bt_div, seq_lens, seq_starts, ws_o, ws_lse, ws_tbl, o, lse);
  else if (d.kv_dtype == MLA_BF16)
    decode_generic<TQ, MLA_BF16><<<grid, 256, 0, s>>>(B, d.n_heads, d.d_latent, d.d_rope, d.block_size, plan.parts,
        d.softmax_scale, q, cache, kv_scale, bt, max_pages, bt_div, seq_lens, seq_starts, ws_o, ws_lse, ws_tbl, o, lse);
  else
    decode_generic<TQ, MLA_E4M3><<<grid, 256, 0, s>>>(B, d.n_heads, d.d_latent, d.d_rope, d.block_size, plan.parts,
        d.softmax_scale, q, cache, kv_scale, bt, max_pages, bt_div, seq_lens, seq_starts, ws_o, ws_lse, ws_tbl, o, lse);
  combine_kernel<TQ><<<dim3(B, d.n_heads), 64, 0, s>>>(B, d.n_heads, d.d_latent, d.block_size, plan.parts,
      seq_lens, seq_starts, ws_o, ws_lse, ws_tbl, o, lse);
}

static void workspace_split(const mla_dims& d, const DecodePlan& plan, int32_t B, void* ws,
                            float** ws_o, float** ws_lse, int64_t** ws_tbl) {
  const size_t slots = (size_t)plan.parts + B;
  size_t o_bytes = slots * d.n_heads * d.d_latent * sizeof(float);
  o_bytes = (o_bytes + 255) & ~(size_t)255;
  size_t l_bytes = slots * d.n_heads * sizeof(float);
  l_bytes = (l_bytes + 255) & ~(size_t)255;
  *ws_o = static_cast<float*>(ws);
  *ws_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + o_bytes);
  *ws_tbl = reinterpret_cast<int64_t*>(static_cast<char*>(ws) + o_bytes + l_bytes);
}

int device_cu_count() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> known[kMaxDev];            // 0: not asked yet
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();                         // leave no error behind for a later launch check
    return kNumCU;
  }
  int n = known[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = kNumCU;
  }
  known[dev].store(n, std::memory_order_relaxed);
  return n;
}

DecodePlan plan_decode(const mla_dims& d, int32_t batch, int32_t num_splits) {
  DecodePlan p{};
  p.kernel = h64w_decode_supported(d) || e4m3_h64_decode_supported(d) ? kDecodeH64
             : fp8_decode_supported(d)                              ? kDecodeFp8
                                                                    : kDecodeGeneric;
  p.head_groups = p.kernel == kDecodeH64 ? d.n_heads / 64 : p.kernel == kDecodeFp8 ? d.n_heads / 16 : d.n_heads;
  // one workgroup per CU for the MFMA kernels; the generic kernel runs 4 per CU
  const int32_t cus = device_cu_count();
  int32_t autos = p.kernel != kDecodeGeneric ? (cus / p.head_groups) : (cus * 4) / d.n_heads;
  p.parts = num_splits > 0 ? num_splits : (autos > 0 ? autos : 1);
  const size_t slots = (size_t)p.parts + batch;
  size_t o_bytes = slots * d.n_heads * d.d_latent * sizeof(float);
  o_bytes = (o_bytes + 255) & ~(size_t)255;
  size_t l_bytes = slots * d.n_heads * sizeof(float);
  l_bytes = (l_bytes + 255) & ~(size_t)255;
  p.ws_bytes = o_bytes + l_bytes + (size_t)batch * 4 * sizeof(int64_t);   // + per-sequence part range
  return p;
}

hipError_t launch_decode(const mla_dims& d, const DecodePlan& plan, int32_t B, const void* q_abs,
                         const void* cache, const float* kv_scale, const int32_t* block_table,
                         int32_t max_pages, int32_t bt_div, const int32_t* seq_lens,
                         const int32_t* seq_starts, void* ws, void* o_lat, float* lse, hipStream_t s) {
  float *ws_o, *ws_lse;
  int64_t* ws_tbl;
  workspace_split(d, plan, B, ws, &ws_o, &ws_lse, &ws_tbl);
  // the MFMA kernel loads 16-byte fragments and stores 8-byte groups
  const bool aligned = (reinterpret_cast<uintptr_t>(q_abs) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(cache) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(o_lat) % 8 == 0);
  if (plan.kernel == kDecodeH64 && aligned && h64w_decode_supported(d))
    return launch_decode_h64w(d, plan, B, q_abs, cache, block_table, max_pages, bt_div, seq_lens, seq_starts, ws_o,
                              ws_lse, ws_tbl, o_lat, lse, s);
  if (plan.kernel == kDecodeH64 && aligned && e4m3_h64_decode_supported(d) &&
      reinterpret_cast<uintptr_t>(kv_scale) % 4 == 0)
    return launch_decode_e4m3_h64(d, plan, B, q_abs, cache, kv_scale, block_table, max_pages, bt_div, seq_lens,
                              seq_starts, ws_o, ws_lse, ws_tbl, o_lat, lse, s);
  if (plan.kernel == kDecodeFp8 && aligned && reinterpret_cast<uintptr_t>(kv_scale) % 16 == 0)
    return launch_decode_fp8(d, plan, B, q_abs, cache, kv_scale, block_table, max_pages, bt_div, seq_lens,
                             seq_starts, ws_o, ws_lse, ws_tbl, o_lat, lse, s);
  if (d.act_dtype == MLA_F32)
    decode_generic_dispatch<float>(d, plan, B, q_abs, cache, kv_scale, block_table, max_pages, bt_div,
                                   seq_lens, seq_starts, ws_o, ws_lse, ws_tbl, o_lat, lse, s);
  else
    decode_generic_dispatch<bf16_t>(d, plan, B, q_abs, cache, kv_scale, block_table, max_pages, bt_div,
                                    seq_lens, seq_starts, ws_o, ws_lse, ws_tbl, o_lat, lse, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Several query tokens per sequence (a chunk of new tokens): query i of
// sequence b sits at position L_b - q + i and attends to the rows up to its
// own, i.e. it is the decode of a sequence of length L_b - q + 1 + i over
// the same pages.  Each (b, i) becomes such a sequence, b * q + i, with
// block-table row b; these lengths and starts are written to the workspace.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) expand_queries(int32_t B, int32_t q, const int32_t* __restrict__ seq_lens,
                                                      const int32_t* __restrict__ seq_starts,
                                                      int32_t* __restrict__ v_lens, int32_t* __restrict__ v_starts) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)B * q) return;
  const int32_t b = static_cast<int32_t>(i / q), j = static_cast<int32_t>(i - (int64_t)b * q);
  v_lens[i] = max(0, seq_lens[b] - q + 1 + j);
  v_starts[i] = seq_starts ? seq_starts[b] : 0;
}

size_t multi_extra_bytes(int32_t B, int32_t q) { return (2 * (size_t)B * q * sizeof(int32_t) + 255) & ~(size_t)255; }

hipError_t launch_decode_multi(const mla_dims& d, const DecodePlan& plan, int32_t B, int32_t q, const void* q_abs,
                               const void* cache, const float* kv_scale, const int32_t* block_table,
                               int32_t max_pages, const int32_t* seq_lens, const int32_t* seq_starts, void* ws,
                               void* o_lat, float* lse, hipStream_t s) {
  int32_t* v_lens = static_cast<int32_t*>(ws);
  int32_t* v_starts = v_lens + (size_t)B * q;
  const int64_t n = (int64_t)B * q;
  expand_queries<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(B, q, seq_lens, seq_starts, v_lens,
                                                                         v_starts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode(d, plan, B * q, q_abs, cache, kv_scale, block_table, max_pages, q, v_lens, v_starts,
                       static_cast<char*>(ws) + multi_extra_bytes(B, q), o_lat, lse, s);
}

hipError_t launch_up_v(const mla_dims& d, int32_t B, const void* o_lat, const void* w_uv, void* out,
                       hipStream_t s) {
  bool handled = false;
  hipError_t e = launch_up_v_mfma(d, B, o_lat, w_uv, out, s, &handled);
  if (handled || e != hipSuccess) return e;
  dim3 grid(d.n_heads, (B + kBB - 1) / kBB);
  size_t shm = sizeof(float) * kBB * d.d_latent;
  if (d.act_dtype == MLA_F32)
    up_v_generic<float><<<grid, 256, shm, s>>>(B, d.n_heads, d.d_head, d.d_latent,
        (const float*)o_lat, (const float*)w_uv, (float*)out);
  else
    up_v_generic<bf16_t><<<grid, 256, shm, s>>>(B, d.n_heads, d.d_head, d.d_latent,
        (const bf16_t*)o_lat, (const bf16_t*)w_uv, (bf16_t*)out);
  return hipGetLastError();
}

}  // namespace mla
