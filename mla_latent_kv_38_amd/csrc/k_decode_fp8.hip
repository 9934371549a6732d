// MFMA decode over an E4M3 latent cache: d_c = 512, d_R = 64 (rows of 576
// bytes plus one float32 scale per token), 64-token pages, bfloat16 queries,
// n_h a multiple of 16 (one workgroup per part and 16-head group).
//
// Dequantisation factors out of both contractions: with row = s_t * c~_t,
//   score_t = s_t * (q . c~_t)   and   o = sum_t (p_t s_t) c~_t / sum_t p_t,
// so the kernel converts the E4M3 codes to bfloat16 exactly (every E4M3 value
// is a bfloat16 value) and applies s_t to the score and to P in float32.
//
// Per page (one workgroup = 4 waves on one CU):
//   * the 36 KiB of codes and 256 B of scales arrive by direct loads into one
//     of two staging buffers (the next page is in flight meanwhile);
//   * a conversion pass writes the bf16 tile (64 rows padded to 73 x 16 B),
//     zeroing rows past the end of the sequence;
//   * wave w owns tokens 16w..16w+15 of every page with its own online
//     softmax state, so no score or maximum crosses waves:
//       QK  S^T[16 tok x 16 heads] = C . Q^T: 18 v_mfma_f32_16x16x32_bf16,
//           Q^T in registers;
//       PV  O^T[512 x 16 heads] += V^T[512 x 16 tok] . P^T: 32
//           v_mfma_f32_16x16x16_bf16, V^T by ds_read_b64_tr_b16 and P^T taken
//           straight from the QK result registers (the D layout of the score
//           MFMA is the B layout of the PV MFMA).
// At the end of a segment the four waves' states are merged through LDS.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
#define LDSP __attribute__((address_space(3)))

constexpr int kD = 576;
constexpr int kDc = 512;
constexpr int kBs = 64;
constexpr int kHeads = 16;                  // heads per workgroup
constexpr int kRowB = 1168;                 // bf16 tile row: 1152 B + 16 pad
constexpr int kF8B = kBs * kD;              // 36864 B of codes per page = 36 x 1 KiB
constexpr float kTau = 8.0f;                // lazy-rescale threshold (log2 units)

__shared__ __attribute__((aligned(1024))) char g_f8a[kF8B];
__shared__ __attribute__((aligned(1024))) char g_f8b[kF8B];
__shared__ __attribute__((aligned(256))) float g_sca[kBs];
__shared__ __attribute__((aligned(256))) float g_scb[kBs];
__shared__ __attribute__((aligned(1024))) char g_tile[kBs * kRowB];
__shared__ int32_t g_lens[256];
__shared__ float g_xm[4][kHeads];           // per-wave reference max (segment merge)
__shared__ float g_xl[4][kHeads];           // per-wave row sums

// Two E4M3 codes (the low or high half of a dword) -> two bfloat16 in one
// instruction: the scaled conversion with scale 1.0, exact for every code
// (each E4M3 value is a bfloat16 value; checked on the device against the
// float32 conversion for all 65 536 code pairs).
template <bool kHi>
__device__ __forceinline__ uint32_t cvt_pair(uint32_t codes) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, kHi));
}

// One page: codes (36 x 64 lanes x 16 B; wave w issues k = w, w+4, ...) and,
// from wave 0, the 64 scales (64 lanes x 4 B).
__device__ __forceinline__ void dma_page(const char* src, const float* ssrc, LDSP char* dst,
                                         LDSP float* sdst, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    const int k = wave + 4 * i;
    dma16(src, 1024 * k + 16 * lane, dst + 1024 * k);
  }
  if (wave == 0) dma4(reinterpret_cast<const char*>(ssrc), 4 * lane, sdst);
}

// Codes -> bfloat16 tile.  Thread t converts 16-byte chunks t + 256 i of the
// page (row c / 36, chunk c % 36); rows at or past nvalid are written as zeros
// so that masked tokens contribute exact zeros to PV.
__device__ __forceinline__ void convert_page(const LDSP char* __restrict__ f8, LDSP char* __restrict__ tile,
                                             int nvalid, int tid) {
#pragma unroll
  for (int i0 = 0; i0 < 9; i0 += 3) {
  u32x4 v[9];
#pragma unroll
  for (int i = i0; i < i0 + 3; ++i) {
    const int c = tid + 256 * i, row = c / 36, ch = c - 36 * row;
    v[i] = *reinterpret_cast<const LDSP u32x4*>(f8 + row * kD + ch * 16);
  }
#pragma unroll
  for (int i = i0; i < i0 + 3; ++i) {
    const int c = tid + 256 * i, row = c / 36, ch = c - 36 * row;
    const uint32_t keep = row < nvalid ? 0xFFFFFFFFu : 0u;     // branch-free zeroing of rows past the end
    u32x4 lo = {cvt_pair<false>(v[i][0]), cvt_pair<true>(v[i][0]), cvt_pair<false>(v[i][1]), cvt_pair<true>(v[i][1])};
    u32x4 hi = {cvt_pair<false>(v[i][2]), cvt_pair<true>(v[i][2]), cvt_pair<false>(v[i][3]), cvt_pair<true>(v[i][3])};
    lo &= keep;
    hi &= keep;
    LDSP char* dst = tile + row * kRowB + ch * 32;
    *reinterpret_cast<LDSP u32x4*>(dst) = lo;
    *reinterpret_cast<LDSP u32x4*>(dst + 16) = hi;
  }
  }
}

struct State {                     // one wave's running state for its token block
  f32x4 o[32];                     // O^T blocks: columns 16 cb + 4 g + r, head s (AGPRs)
  float m_ref, l_part;             // reference max (log2 units) of head s; partial row sum
};

// QK, softmax and PV of one page for wave w's 16 tokens (tile already in LDS).
__device__ __forceinline__ void page_compute(const LDSP char* __restrict__ tile, const LDSP float* __restrict__ sc,
                                             const bf16x8 (&qf)[18], int wave, int lane, int nvalid,
                                             float s2, State& st) {
  const int g = lane >> 4, s = lane & 15;
  // S^T[tok 16w + 4g + r][head s]
  f32x4 S = {0.f, 0.f, 0.f, 0.f};
  {
    const LDSP char* ap = tile + (16 * wave + s) * kRowB + g * 16;
    bf16x8 af[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) af[k] = *reinterpret_cast<const LDSP bf16x8*>(ap + 64 * k);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(S) : "v"(af[ks & 3]), "a"(qf[ks]));
      if (ks + 4 < 18) af[ks & 3] = *reinterpret_cast<const LDSP bf16x8*>(ap + 64 * (ks + 4));
    }
    asm volatile("s_nop 7\n s_nop 7\n s_nop 1" ::: "memory");   // MFMA result -> VALU
  }
  float v[4], scl[4];
  float mb = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 16 * wave + 4 * g + r;
    scl[r] = sc[t];
    v[r] = t < nvalid ? S[r] * s2 * scl[r] : -INFINITY;
    mb = fmaxf(mb, v[r]);
  }
  mb = max_xor32(max_xor16(mb));
  float alpha = 1.f;
  if (mb > st.m_ref + kTau) {
    alpha = __builtin_amdgcn_exp2f(st.m_ref - mb);
    st.m_ref = mb;
  }
  float p[4], ps = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 16 * wave + 4 * g + r;
    const float e = t < nvalid ? __builtin_amdgcn_exp2f(v[r] - st.m_ref) : 0.f;
    ps += e;
    p[r] = t < nvalid ? e * scl[r] : 0.f;
  }
  st.l_part = st.l_part * alpha + ps;
  if (__any(alpha != 1.f)) {
    asm volatile("s_nop 7\n s_nop 7\n s_nop 1" ::: "memory");  // previous page's MFMAs -> VALU
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) st.o[cb] *= alpha;
  }
  const u32x2 pk = {pack2_bf16(p[0], p[1]), pack2_bf16(p[2], p[3])};
  const s16x4 pf = __builtin_bit_cast(s16x4, pk);
  // V^T[16 cols x 16 tok]: in each 16-lane group, source lane s' names row
  // 16w + 4g + s'/4 and columns 16 cb + 4 (s'%4) .. +3; lane s receives column s.
  const LDSP char* vp = tile + (16 * wave + 4 * g + (s >> 2)) * kRowB + 4 * (s & 3) * 2;
  // V^T fragments kVPre blocks ahead; the accumulators live in AGPRs (the
  // MFMA reads and writes them there), which leaves the VGPRs for the reads.
  constexpr int kVPre = 8;
  s16x4 vf[kVPre];
#pragma unroll
  for (int k = 0; k < kVPre; ++k) vf[k] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDSP s16x4*)(vp + 32 * k));
  asm volatile("s_nop 4" ::: "memory");                          // P (VALU) -> MFMA source
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) {
    asm volatile("v_mfma_f32_16x16x16_bf16 %0, %1, %2, %0" : "+a"(st.o[cb]) : "v"(vf[cb % kVPre]), "v"(pf));
    if (cb + kVPre < 32) vf[cb % kVPre] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDSP s16x4*)(vp + 32 * (cb + kVPre)));
  }
}

// One page.  kEven selects the staging buffers statically (page jp in A, the
// next page's loads into B, or the reverse), so the compiler can see that the
// in-flight loads never alias what this page reads.
template <bool kEven>
__device__ __forceinline__ void page_iter(int64_t jp, int64_t jp1, int32_t L, const int32_t* bt,
                                          int32_t& pg_next, const char* cbase, const float* kv_scale,
                                          const bf16x8 (&qf)[18], int wave, int lane, int tid, float s2,
                                          State& st) {
  LDSP char* cur = kEven ? (LDSP char*)g_f8a : (LDSP char*)g_f8b;
  LDSP char* nxt = kEven ? (LDSP char*)g_f8b : (LDSP char*)g_f8a;
  LDSP float* csc = kEven ? (LDSP float*)g_sca : (LDSP float*)g_scb;
  LDSP float* nsc = kEven ? (LDSP float*)g_scb : (LDSP float*)g_sca;
  const int nvalid = (int)min<int64_t>(kBs, (int64_t)L - jp * kBs);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");             // this wave's loads of page jp
  barrier_lds();                                                // everyone's; tile free again
  if (jp + 1 < jp1) {                                           // page jp+1 (its id was read one page ago)
    const int64_t pg = pg_next;
    dma_page(cbase + pg * kF8B, kv_scale + pg * kBs, nxt, nsc, wave, lane);
  }
  const int32_t pg_after = jp + 2 < jp1 ? bt[jp + 2] : 0;      // in flight during this page
  convert_page(cur, (LDSP char*)g_tile, nvalid, tid);
  barrier_lds();                                                // tile ready
  page_compute((const LDSP char*)g_tile, csc, qf, wave, lane, nvalid, s2, st);
  pg_next = pg_after;
}

__global__ void __launch_bounds__(256, 1) decode_fp8_h16(
    int32_t B, int32_t n_h, int32_t W, int32_t HG, float s2,
    const uint16_t* __restrict__ q_abs, const uint8_t* __restrict__ cache, const float* __restrict__ kv_scale,
    const int32_t* __restrict__ block_table, int32_t max_pages, const int32_t* __restrict__ seq_lens,
    float* __restrict__ ws_o, float* __restrict__ ws_lse, uint16_t* __restrict__ o_lat,
    float* __restrict__ lse) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, s = lane & 15;

  // XCD x (workgroup i runs on XCD i % 8) takes the contiguous parts
  // [x ppx, (x+1) ppx) with all their head groups.
  const int ppx = (W + 7) / 8;
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int hg = j % HG;
  const int part = xcd * ppx + j / HG;
  if (part >= W) return;

  const PartRange pr = locate_part(seq_lens, B, kBs, part, W, g_lens);
  const int32_t chunk = pr.chunk;
  auto seq_len = [&](int32_t bb) { return chunk == 1 ? g_lens[bb] : seq_lens[bb]; };
  const int64_t x1 = pr.x1;
  int64_t x = pr.x0;
  if (x >= x1) return;
  int32_t b = pr.b;
  int64_t first = pr.first;

  const char* cbase = reinterpret_cast<const char*>(cache);
  for (;;) {
    const int32_t L = seq_len(b);
    const int64_t np = pages_of(L, kBs);
    const int64_t jp0 = x - first;
    const int64_t jp1 = min(np, jp0 + (x1 - x));
    const int32_t* bt = block_table + (int64_t)b * max_pages;

    {
      const int64_t pg = bt[jp0];
      dma_page(cbase + pg * kF8B, kv_scale + pg * kBs, (LDSP char*)g_f8a, (LDSP float*)g_sca, wave, lane);
    }
    bf16x8 qf[18];                                              // Q^T, pinned in AGPRs
    {
      const bf16x8* qsrc = reinterpret_cast<const bf16x8*>(
          q_abs + ((int64_t)b * n_h + (int64_t)hg * kHeads + s) * kD + 8 * g);
      bf16x8 t[18];
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) t[ks] = qsrc[4 * ks];
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) asm volatile("" : "=a"(qf[ks]) : "0"(t[ks]));
    }
    State st;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) st.o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m_ref = -INFINITY;
    st.l_part = 0.f;

    int32_t pg_next = jp0 + 1 < jp1 ? bt[jp0 + 1] : 0;
    for (int64_t jp = jp0; jp < jp1; jp += 2) {
      page_iter<true>(jp, jp1, L, bt, pg_next, cbase, kv_scale, qf, wave, lane, tid, s2, st);
      if (jp + 1 < jp1) page_iter<false>(jp + 1, jp1, L, bt, pg_next, cbase, kv_scale, qf, wave, lane, tid, s2, st);
    }

    // ---- merge the four waves' states, normalise, store ----------------------
    asm volatile("s_nop 7\n s_nop 7\n s_nop 1" ::: "memory");    // MFMA results -> VALU
    float lw = st.l_part;
    lw += __shfl_xor(lw, 16);
    lw += __shfl_xor(lw, 32);
    __syncthreads();                                            // every wave done with the tile
    if (g == 0) { g_xm[wave][s] = st.m_ref; g_xl[wave][s] = lw; }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, g_xm[w][s]);
    float Lsum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = g_xm[w][s];
      Lsum += mw == -INFINITY ? 0.f : g_xl[w][s] * __builtin_amdgcn_exp2f(mw - M);
    }
    const float fw = (st.m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.m_ref - M)) / Lsum;
    // wave w's scaled O^T into region w (register order: [cb][lane] float4)
    auto region = [](int w) -> LDSP f32x4* {
      LDSP char* r = w == 0 ? (LDSP char*)g_tile : w == 1 ? (LDSP char*)g_tile + 32768
                   : w == 2 ? (LDSP char*)g_f8a : (LDSP char*)g_f8b;
      return reinterpret_cast<LDSP f32x4*>(r);
    };
    {
      LDSP f32x4* dst = region(wave);
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) dst[cb * 64 + lane] = st.o[cb] * fw;
    }
    __syncthreads();
    const bool whole = (jp0 == 0 && jp1 == np);
    const int64_t head = (int64_t)hg * kHeads + s;
#pragma unroll 2
    for (int k = 0; k < 8; ++k) {                               // wave w stores column blocks 8w..8w+7
      const int cb = 8 * wave + k;
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; ++w) o += region(w)[cb * 64 + lane];
      const int col = 16 * cb + 4 * g;
      if (whole)
        *reinterpret_cast<u32x2*>(o_lat + ((int64_t)b * n_h + head) * kDc + col) =
            u32x2{pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3])};
      else
        *reinterpret_cast<f32x4*>(ws_o + (((int64_t)part + b) * n_h + head) * kDc + col) = o;
    }
    if (wave == 0 && g == 0) {
      const float lse_v = (M + __log2f(Lsum)) * 0.69314718055994531f;
      if (whole) { if (lse) lse[(int64_t)b * n_h + head] = lse_v; }
      else ws_lse[((int64_t)part + b) * n_h + head] = lse_v;
    }

    x += jp1 - jp0;
    if (x >= x1) break;
    do { ++b; } while (pages_of(seq_len(b), kBs) == 0);
    first = x;
    __syncthreads();                                            // regions read before the next DMA
  }
}

}  // namespace

bool fp8_decode_supported(const mla_dims& d) {
  return d.act_dtype == MLA_BF16 && d.kv_dtype == MLA_E4M3 && d.d_latent == kDc && d.d_rope == 64 &&
         d.block_size == kBs && d.n_heads % kHeads == 0;
}

hipError_t launch_decode_fp8(const mla_dims& d, const DecodePlan& plan, int32_t B, const void* q_abs,
                             const void* cache, const float* kv_scale, const int32_t* block_table,
                             int32_t max_pages, const int32_t* seq_lens, float* ws_o, float* ws_lse,
                             void* o_lat, float* lse, hipStream_t s) {
  const int HG = d.n_heads / kHeads;
  const int W = plan.parts;
  const int grid = ((W + 7) / 8) * 8 * HG;                      // 8 XCDs x ceil(W/8) parts x HG
  const float s2 = d.softmax_scale * 1.4426950408889634f;
  decode_fp8_h16<<<grid, 256, 0, s>>>(B, d.n_heads, W, HG, s2, static_cast<const uint16_t*>(q_abs),
                                      static_cast<const uint8_t*>(cache), kv_scale, block_table, max_pages,
                                      seq_lens, ws_o, ws_lse, static_cast<uint16_t*>(o_lat), lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine(d, plan, B, seq_lens, ws_o, ws_lse, o_lat, lse, s);
}

}  // namespace mla
