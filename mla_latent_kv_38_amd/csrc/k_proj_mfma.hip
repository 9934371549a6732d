// MFMA kernels for the two per-head projections around latent attention
// (bfloat16 activations, float32 accumulation):
//   absorb_q   q_abs[b,h,:d_c] = W_UK[h]^T q_c[b,h]   contraction over d_h (rows of W_UK[h])
//   up_v       out[b,h,:]      = W_UV[h] o_lat[b,h]    contraction over d_c (columns of W_UV[h])
// Both are weight-streaming products (every weight byte is used by each of the
// batch rows and by nothing else), so they are bound by HBM reads of the
// weights.  Each is computed transposed, D[out dim x batch] = W' . X^T, with
// v_mfma_f32_16x16x32_bf16: the weight is the A operand (16 output features
// per block), the batch the N operand (16 rows per block), so a lane ends up
// holding 4 consecutive output features of one batch row (one 8-byte store).
//
// 16x16x32 operand layouts (lane l, group g = l / 16, s = l % 16):
//   A: A[s][8g + e], e = 0..7      B: B[8g + e][s]      D: D[4g + r][s], r = 0..3
#include <algorithm>
#include <cmath>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define LDSP __attribute__((address_space(3)))


__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// absorb_q.  Workgroup = (head h, block of 128 latent columns); 4 waves, wave w
// owns columns 32w..32w+31 of the block (two 16-column A blocks).  W_UK[h]'s
// [d_h x 128] tile is staged in LDS row-major and read transposed with
// ds_read_b64_tr_b16, so each lane gets 8 consecutive contraction indices of
// one column; the A fragments are then reused for every batch block.  The
// RoPE half of q_abs is spread over the head's workgroups.
// ---------------------------------------------------------------------------
constexpr int kAbsCols = 128;
constexpr int kAbsRowB = kAbsCols * 2 + 16;     // padded LDS row (bytes)

// The batch may be split over workgroups too (grid z): workgroup z takes
// rows [z bpw, (z+1) bpw), at most kMaxBlk blocks of 16, all of whose q_C
// fragments are loaded together with the weight tile.
constexpr int kMaxBlk = 4;

// An independent append of new 576-wide rows can ride along in the same
// launch (mla_absorb_q_append): the workgroups past the absorb grid (row y = 0)
// each write four rows, one per wave, with the append's own row writer.
struct AppendJob {
  int32_t T;                       // rows to append (0: none)
  int32_t e4m3;                    // cache type: E4M3 (1) or bf16 (0)
  const uint16_t* c_kv;
  const uint16_t* k_r;
  const int32_t* pos;
  const int64_t* slot;
  void* cache;
  float* kv_scale;
};

template <int kKs>   // d_h / 32
__global__ void __launch_bounds__(256) absorb_q_mfma(int32_t B, int32_t bpw, int32_t n_h, int32_t d_c, int32_t d_R,
                                                     const uint16_t* __restrict__ q_c,
                                                     const uint16_t* __restrict__ q_r,
                                                     const int32_t* __restrict__ pos,
                                                     const uint16_t* __restrict__ w_uk,
                                                     uint16_t* __restrict__ q_abs, double log2_base,
                                                     AppendJob app) {
  constexpr int d_h = 32 * kKs;
  __shared__ __attribute__((aligned(16))) char tile[d_h * kAbsRowB];
  const int cblocks = d_c / kAbsCols;
  if (blockIdx.x >= n_h * cblocks) {                             // the ride-along append
    const int t = 4 * (blockIdx.x - n_h * cblocks) + (threadIdx.x >> 6), ln = threadIdx.x & 63;
    if (blockIdx.y != 0 || t >= app.T) return;
    const u32x4_t c = *reinterpret_cast<const u32x4_t*>(app.c_kv + (int64_t)t * 512 + 8 * ln);
    uint32_t kp = 0;
    if (ln < 32) kp = *reinterpret_cast<const uint32_t*>(app.k_r + (int64_t)t * 64 + 2 * ln);
    if (app.e4m3) append_row_576<true>(c, kp, app.pos[t], app.slot[t], app.cache, app.kv_scale, log2_base, ln);
    else append_row_576<false>(c, kp, app.pos[t], app.slot[t], app.cache, app.kv_scale, log2_base, ln);
    return;
  }
  // Workgroup i runs on XCD i % 8.  When the head count is a multiple of 8,
  // the column blocks of a head go to one XCD, so its q_C rows are fetched
  // from HBM once (their L2 is shared).
  int h, cb;
  if ((n_h & 7) == 0) {
    const int j = blockIdx.x >> 3;
    h = (j / cblocks) * 8 + (blockIdx.x & 7);
    cb = j % cblocks;
  } else {
    h = blockIdx.x / cblocks;
    cb = blockIdx.x % cblocks;
  }
  const int c0 = cb * kAbsCols;
  const int b_lo = blockIdx.y * bpw, b_hi = min(B, b_lo + bpw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, s = lane & 15;
  const int64_t D = d_c + d_R;

  // RoPE half of q_abs for this workgroup's batch rows, pairs spread over the
  // head's column-block workgroups (pair i on thread i mod (256 cblocks)).
  // The inputs of a thread's first kRopePer pairs are loaded before the
  // weight tile, so their float64 rotations run while the tile is in flight.
  constexpr int kRopePer = 4;
  const int half = d_R / 2;
  const int npairs = (b_hi - b_lo) * half;
  const int stride = cblocks * 256;
  const int i_first = cb * 256 + tid;
  float rx[kRopePer][2];
  int32_t rpos[kRopePer];
#pragma unroll
  for (int k = 0; k < kRopePer; ++k) {
    // every thread loads (a thread past the last pair re-reads that pair and
    // drops it), so that no load sits in a branch whose join would wait for it
    const int i = min(i_first + k * stride, npairs - 1);
    const int bb = b_lo + i / half, p = i % half;
    const int64_t src = ((int64_t)bb * n_h + h) * d_R + 2 * p;
    rx[k][0] = bf16_to_f32(q_r[src]);
    rx[k][1] = bf16_to_f32(q_r[src + 1]);
    rpos[k] = pos[bb];
  }
  auto rope_store = [&](int i, float x0, float x1, int32_t ps) {
    const int bb = b_lo + i / half, p = i % half;
    float y0, y1;
    rope_pair(x0, x1, ps, p, d_R, log2_base, &y0, &y1);
    *reinterpret_cast<uint32_t*>(q_abs + ((int64_t)bb * n_h + h) * D + d_c + 2 * p) = pack2_bf16(y0, y1);
  };

  // q_C rows of the workgroup's batch blocks, in flight together with the weight tile
  const int nblk = (b_hi - b_lo + 15) / 16;
  bf16x8 qf[kMaxBlk][kKs];
#pragma unroll
  for (int k = 0; k < kMaxBlk; ++k) {
    const int b = b_lo + 16 * k + s;
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
      if (k < nblk && b < b_hi)
        qf[k][ks] = *reinterpret_cast<const bf16x8*>(q_c + ((int64_t)b * n_h + h) * d_h + 32 * ks + 8 * g);
      else
        qf[k][ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
  }

  // stage W_UK[h][:, c0:c0+128] (d_h rows of 256 B): all loads first, then the LDS writes
  {
    constexpr int kPer = d_h * 16 / 256;
    u32x4 v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int c = tid + 256 * j, row = c >> 4, ch = c & 15;
      v[j] = *reinterpret_cast<const u32x4*>(w_uk + ((int64_t)h * d_h + row) * d_c + c0 + 8 * ch);
    }
#pragma unroll
    for (int k = 0; k < kRopePer; ++k)
      if (i_first + k * stride < npairs) rope_store(i_first + k * stride, rx[k][0], rx[k][1], rpos[k]);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int c = tid + 256 * j, row = c >> 4, ch = c & 15;
      *reinterpret_cast<LDSP u32x4*>((LDSP char*)tile + row * kAbsRowB + ch * 16) = v[j];
    }
  }
  for (int i = i_first + kRopePer * stride; i < npairs; i += stride) {
    const int bb = b_lo + i / half, p = i % half;
    const int64_t src = ((int64_t)bb * n_h + h) * d_R + 2 * p;
    rope_store(i, bf16_to_f32(q_r[src]), bf16_to_f32(q_r[src + 1]), pos[bb]);
  }
  __syncthreads();

  // A fragments: A[m][k] = W[k][c0 + 32 wave + 16 mb + m].  In each 16-lane
  // group, source lane s names row 8g + s/4 (+4 for the second read) and
  // columns 4(s%4)..+3; lane s receives column s of the four rows.
  bf16x8 af[2][kKs];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
      const int row = 32 * ks + 8 * g + (s >> 2);
      const int col = 32 * wave + 16 * mb + 4 * (s & 3);
      const LDSP char* p = (LDSP char*)tile + row * kAbsRowB + col * 2;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDSP s16x4*)p);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDSP s16x4*)(p + 4 * kAbsRowB));
      af[mb][ks] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }

#pragma unroll
  for (int k = 0; k < kMaxBlk; ++k) {
    if (k >= nblk) break;
    const int b = b_lo + 16 * k + s;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) acc = mfma16(af[mb][ks], qf[k][ks], acc);
      if (b < b_hi) {
        const int c = c0 + 32 * wave + 16 * mb + 4 * g;
        *reinterpret_cast<u32x2*>(q_abs + ((int64_t)b * n_h + h) * D + c) =
            u32x2{pack2_bf16(acc[0], acc[1]), pack2_bf16(acc[2], acc[3])};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// up_v.  Workgroup = (head h, block of 64 output features); 4 waves, wave w
// owns features 16w..16w+15 of the block and holds their W_UV rows (all of
// d_c) as A fragments straight from global memory (16 B per lane per step).
// Per batch block of 16 rows, o_lat[b0:b0+16, h, :] is staged once in LDS
// and read by all four waves.
// ---------------------------------------------------------------------------
template <int kKs>   // d_c / 32
__global__ void __launch_bounds__(256) up_v_mfma(int32_t B, int32_t bpw, int32_t n_h, int32_t d_h,
                                                 const uint16_t* __restrict__ o_lat,
                                                 const uint16_t* __restrict__ w_uv,
                                                 uint16_t* __restrict__ out) {
  constexpr int d_c = 32 * kKs;
  constexpr int kRowB = d_c * 2 + 16;
  __shared__ __attribute__((aligned(16))) char otile[2][16 * kRowB];   // double-buffered batch blocks
  const int iblocks = d_h / 64;
  // the feature blocks of a head on one XCD (as in absorb_q): its o_lat rows
  // come from HBM once
  int h, ib;
  if ((n_h & 7) == 0) {
    const int j = blockIdx.x >> 3;
    h = (j / iblocks) * 8 + (blockIdx.x & 7);
    ib = j % iblocks;
  } else {
    h = blockIdx.x / iblocks;
    ib = blockIdx.x % iblocks;
  }
  const int b_lo = blockIdx.y * bpw, b_hi = min(B, b_lo + bpw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, s = lane & 15;
  const int i0 = 64 * ib + 16 * wave;

  constexpr int kChunks = 16 * d_c / 8;           // 16-byte chunks of one o_lat tile
  constexpr int kPer = (kChunks + 255) / 256;
  auto load_tile = [&](int b0, u32x4 (&v)[kPer]) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int c = tid + 256 * j, row = c / (d_c / 8), ch = c % (d_c / 8);
      v[j] = u32x4{0u, 0u, 0u, 0u};
      if (c < kChunks && b0 + row < b_hi)
        v[j] = *reinterpret_cast<const u32x4*>(o_lat + ((int64_t)(b0 + row) * n_h + h) * d_c + 8 * ch);
    }
  };
  auto store_tile = [&](int buf, const u32x4 (&v)[kPer]) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int c = tid + 256 * j, row = c / (d_c / 8), ch = c % (d_c / 8);
      if (c < kChunks) *reinterpret_cast<LDSP u32x4*>((LDSP char*)otile[buf] + row * kRowB + ch * 16) = v[j];
    }
  };

  u32x4 v[kPer];
  load_tile(b_lo, v);                             // first o_lat block in flight with the weights
  bf16x8 af[kKs];
  {
    const uint16_t* wrow = w_uv + ((int64_t)h * d_h + i0 + s) * d_c + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) af[ks] = *reinterpret_cast<const bf16x8*>(wrow + 32 * ks);
  }
  store_tile(0, v);
  int buf = 0;
  for (int b0 = b_lo; b0 < b_hi; b0 += 16, buf ^= 1) {
    const bool more = b0 + 16 < b_hi;
    if (more) load_tile(b0 + 16, v);              // next block in flight during this one
    __syncthreads();                              // block b0 staged; the other buffer free
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
      const bf16x8 xf = *reinterpret_cast<const LDSP bf16x8*>((LDSP char*)otile[buf] + s * kRowB + (32 * ks + 8 * g) * 2);
      acc = mfma16(af[ks], xf, acc);
    }
    const int b = b0 + s;
    if (b < b_hi)
      *reinterpret_cast<u32x2*>(out + ((int64_t)b * n_h + h) * d_h + i0 + 4 * g) =
          u32x2{pack2_bf16(acc[0], acc[1]), pack2_bf16(acc[2], acc[3])};
    if (more) store_tile(buf ^ 1, v);
  }
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

hipError_t launch_absorb_q_mfma(const mla_dims& d, int32_t B, const void* q_c, const void* q_r,
                                const int32_t* pos, const void* w_uk, void* q_abs, hipStream_t s,
                                bool* handled, const AppendArgs* append) {
  *handled = false;
  AppendJob app{};
  if (append) {                    // only the 576-wide bf16-input append rides along
    if (!(d.d_latent == 512 && d.d_rope == 64 && (d.kv_dtype == MLA_BF16 || d.kv_dtype == MLA_E4M3) &&
          aligned16(append->c_kv) && aligned16(append->cache) && (reinterpret_cast<uintptr_t>(append->k_r) & 3u) == 0))
      return hipSuccess;
    app = AppendJob{append->T, d.kv_dtype == MLA_E4M3, static_cast<const uint16_t*>(append->c_kv),
                    static_cast<const uint16_t*>(append->k_r), append->pos, append->slot, append->cache,
                    append->kv_scale};
  }
  const int D = d.d_latent + d.d_rope;
  if (d.act_dtype != MLA_BF16 || d.d_latent % kAbsCols != 0 || d.d_head % 32 != 0 || D % 4 != 0 ||
      !aligned16(q_c) || !aligned16(w_uk) || !aligned16(q_abs) || (reinterpret_cast<uintptr_t>(q_r) & 3u))
    return hipSuccess;
  // Split the batch over workgroups until the grid fills the chip (at most
  // kMaxBlk blocks of 16 rows per workgroup).
  const int wgs = d.n_heads * (d.d_latent / kAbsCols);
  const int nblocks = (B + 15) / 16;
  int nsplit = std::max((nblocks + kMaxBlk - 1) / kMaxBlk, std::min(nblocks, (256 + wgs - 1) / wgs));
  const int bpw = 16 * ((nblocks + nsplit - 1) / nsplit);
  nsplit = (B + bpw - 1) / bpw;
  // (append workgroups padded to a multiple of 8, so that workgroup x of every
  // grid row runs on XCD x % 8; the extra ones have no row and return)
  const dim3 grid(wgs + (((app.T + 3) / 4 + 7) & ~7), nsplit);
  auto qc = static_cast<const uint16_t*>(q_c);
  auto qr = static_cast<const uint16_t*>(q_r);
  auto w = static_cast<const uint16_t*>(w_uk);
  auto qa = static_cast<uint16_t*>(q_abs);
  switch (d.d_head) {
    case 64:  absorb_q_mfma<2><<<grid, 256, 0, s>>>(B, bpw, d.n_heads, d.d_latent, d.d_rope, qc, qr, pos, w, qa, std::log2(d.rope_base), app); break;
    case 128: absorb_q_mfma<4><<<grid, 256, 0, s>>>(B, bpw, d.n_heads, d.d_latent, d.d_rope, qc, qr, pos, w, qa, std::log2(d.rope_base), app); break;
    case 192: absorb_q_mfma<6><<<grid, 256, 0, s>>>(B, bpw, d.n_heads, d.d_latent, d.d_rope, qc, qr, pos, w, qa, std::log2(d.rope_base), app); break;
    case 256: absorb_q_mfma<8><<<grid, 256, 0, s>>>(B, bpw, d.n_heads, d.d_latent, d.d_rope, qc, qr, pos, w, qa, std::log2(d.rope_base), app); break;
    default: return hipSuccess;
  }
  *handled = true;
  return hipGetLastError();
}

hipError_t launch_up_v_mfma(const mla_dims& d, int32_t B, const void* o_lat, const void* w_uv, void* out,
                            hipStream_t s, bool* handled) {
  *handled = false;
  if (d.act_dtype != MLA_BF16 || d.d_head % 64 != 0 || !aligned16(o_lat) || !aligned16(w_uv) ||
      (reinterpret_cast<uintptr_t>(out) & 7u))
    return hipSuccess;
  // Split the batch over workgroups until the grid fills the chip.
  const int wgs = d.n_heads * (d.d_head / 64);
  const int nblocks = (B + 15) / 16;
  const int nsplit0 = std::min(nblocks, (256 + wgs - 1) / wgs);
  const int bpw = 16 * ((nblocks + nsplit0 - 1) / nsplit0);
  const dim3 grid(wgs, (B + bpw - 1) / bpw);
  auto o = static_cast<const uint16_t*>(o_lat);
  auto w = static_cast<const uint16_t*>(w_uv);
  auto y = static_cast<uint16_t*>(out);
  switch (d.d_latent) {
    case 128: up_v_mfma<4><<<grid, 256, 0, s>>>(B, bpw, d.n_heads, d.d_head, o, w, y); break;
    case 256: up_v_mfma<8><<<grid, 256, 0, s>>>(B, bpw, d.n_heads, d.d_head, o, w, y); break;
    case 512: up_v_mfma<16><<<grid, 256, 0, s>>>(B, bpw, d.n_heads, d.d_head, o, w, y); break;
    default: return hipSuccess;
  }
  *handled = true;
  return hipGetLastError();
}

}  // namespace mla
