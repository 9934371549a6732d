// MFMA decode over an E4M3 latent cache: d_c = 512, d_R = 64 (rows of 576
// bytes plus one float32 scale per token), 64-token pages, bfloat16 queries,
// n_h a multiple of 16 (one workgroup per part and 16-head group).
//
// Dequantisation factors out of both contractions: with row = s_t * c~_t,
//   score_t = s_t * (q . c~_t)   and   o = sum_t (p_t s_t) c~_t / sum_t p_t,
// so the kernel converts E4M3 codes to bfloat16 exactly (every E4M3 value is
// a bfloat16 value) right before each MFMA and applies s_t to the score and
// to P in float32.
//
// Pages stream HBM -> LDS by direct loads through a ring of four slots
// (codes in rows padded to 37 x 16 B, plus the 64 scales).  The page loop
// takes two pages per step, from two slots, while the next two pages load
// into the other two.  Wave w owns tokens 16w..16w+15 of every page with its
// own online softmax state, so no score or maximum crosses waves and a step
// needs one barrier:
//   QK  S^T[16 tok x 16 heads] = C . Q^T per page: 18
//       v_mfma_f32_16x16x32_bf16, the two pages' chains interleaved, the A
//       fragments read as 8 codes per lane and converted in registers, Q^T
//       in AGPRs;
//   PV  O^T[512 x 16 heads] += V^T[512 x 32 tok] . P^T: 32
//       v_mfma_f32_16x16x32_bf16 over the wave's 16 tokens of both pages,
//       accumulators in AGPRs; V^T comes from ds_read_b64_tr_b8 (one read
//       per page gives two 16-column blocks of the wave's tokens), converted
//       in registers; P^T is taken straight from the QK result registers (the
//       D layout of the score MFMA, two pages side by side, is the B layout
//       of the PV MFMA).
// At the end of a segment the four waves' states are merged through LDS.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
#define LDSP __attribute__((address_space(3)))

constexpr int kD = 576;
constexpr int kDc = 512;
constexpr int kBs = 64;
constexpr int kHeads = 16;                  // heads per workgroup
constexpr int kRowF = 592;                  // LDS code row: 576 B + 16 pad (37 x 16 B)
constexpr int kSlotB = kBs * kRowF;         // 37888 B = 37 x 1 KiB
constexpr int kRing = 4;
constexpr int64_t kPageG = (int64_t)kBs * kD;  // 36864 B of codes per page in memory
constexpr float kTau = 8.0f;                // lazy-rescale threshold (log2 units)

__shared__ __attribute__((aligned(1024))) char g_ring[kRing * kSlotB];
__shared__ __attribute__((aligned(256))) float g_sc[kRing][kBs];
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
__device__ __forceinline__ bf16x8 cvt8(i32x2 c) {      // 8 codes -> 8 bfloat16
  return __builtin_bit_cast(bf16x8, u32x4{cvt_pair<false>(c[0]), cvt_pair<true>(c[0]),
                                          cvt_pair<false>(c[1]), cvt_pair<true>(c[1])});
}

// Page loads: LDS slot position q = 64 k + lane of a ring slot holds code row
// q / 37, 16-B chunk q % 37 (chunk 36 is row padding and re-reads offset 0).
// Wave w issues loads k = w, w + 4, ... (10 for wave 0, 9 otherwise, 37 in
// all); wave 0 also loads the 64 scales.  The per-lane source offsets are the
// same for every page, so they are computed once and kept in AGPRs.
__device__ __forceinline__ int page_loads(int wave) { return wave == 0 ? 11 : 9; }   // vmcnt per page

__device__ __forceinline__ void page_offsets(int wave, int lane, uint32_t (&off)[10]) {
  const int q0 = 64 * wave + lane;
  int row = q0 / 37, ch = q0 - 37 * row;
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint32_t o = (row < kBs && ch != 36) ? static_cast<uint32_t>(row * kD + ch * 16) : 0u;
    asm volatile("" : "=a"(off[i]) : "0"(o));
    row += 6;                                    // 256 positions = 6 rows + 34 chunks
    ch += 34;
    if (ch >= 37) { ch -= 37; row += 1; }
  }
}

__device__ __forceinline__ void load_page(const char* src_u, const float* ssrc, int slot, const uint32_t (&off)[10],
                                          int wave, int lane) {
  const uint32_t m0 = uniform_lds((LDSP char*)g_ring + slot * kSlotB);
#pragma unroll
  for (int i = 0; i < 10; ++i)
    if (wave + 4 * i < 37) dma16_u(src_u, off[i], m0 + 1024 * (wave + 4 * i));
  if (wave == 0) dma4(reinterpret_cast<const char*>(ssrc), 4 * lane, (LDSP float*)g_sc[slot]);
}

// Wait until at most `pending` of this wave's loads are in flight (a whole
// number of pages: 9 or 11 loads each).
__device__ __forceinline__ void wait_loads(int pending) {
  switch (pending) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
    case 18: asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); break;
    case 22: asm volatile("s_waitcnt vmcnt(22)" ::: "memory"); break;
    case 27: asm volatile("s_waitcnt vmcnt(27)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(33)" ::: "memory"); break;
  }
}

struct State {                     // one wave's running state for its token block
  f32x4 o[32];                     // O^T blocks: columns 16 cb + 4 g + r, head s (AGPRs)
  float m_ref, l_part;             // reference max (log2 units) of head s; partial row sum
};

// QK, softmax and PV of two pages a and b of the segment for wave w's 16
// tokens of each (codes in slots `ca`, `cb`).  A step without a second page
// passes nvb = 0: every token of b is masked, so its half of every operand is
// zero whatever its slot holds.  The PV contraction runs over 32
// tokens per v_mfma_f32_16x16x32_bf16: contraction index 8g + e stands for
// token 16w + 4g + e of page a when e < 4 and token 16w + 4g + e - 4 of
// page b when e >= 4, which is where the QK results of lane (g, s) put them.
__device__ __forceinline__ void pair_compute(const LDSP char* __restrict__ ca, const LDSP char* __restrict__ cb,
                                             const LDSP float* __restrict__ sca, const LDSP float* __restrict__ scb,
                                             const bf16x8 (&qf)[18], int wave, int lane, int nva, int loa, int nvb,
                                             float s2, State& st) {
  const int g = lane >> 4, s = lane & 15;
  // S^T[tok 16w + 4g + r][head s] of each page; lane (g, s) reads token row
  // 16w + s, codes 32 ks + 8g..+7.  The two pages' chains are independent.
  f32x4 S0 = {0.f, 0.f, 0.f, 0.f}, S1 = {0.f, 0.f, 0.f, 0.f};
  {
    const int ro = (16 * wave + s) * kRowF + g * 8;
    const LDSP char* ap = ca + ro;
    const LDSP char* bp = cb + ro;
    constexpr int kPre = 6;
    i32x2 af[kPre], bf[kPre];
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      af[k] = *reinterpret_cast<const LDSP i32x2*>(ap + 32 * k);
      bf[k] = *reinterpret_cast<const LDSP i32x2*>(bp + 32 * k);
    }
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const bf16x8 a = cvt8(af[ks % kPre]);
      if (ks + kPre < 18) af[ks % kPre] = *reinterpret_cast<const LDSP i32x2*>(ap + 32 * (ks + kPre));
      asm volatile("s_nop 1\n v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(S0) : "v"(a), "a"(qf[ks]));
      const bf16x8 b = cvt8(bf[ks % kPre]);
      if (ks + kPre < 18) bf[ks % kPre] = *reinterpret_cast<const LDSP i32x2*>(bp + 32 * (ks + kPre));
      asm volatile("s_nop 1\n v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(S1) : "v"(b), "a"(qf[ks]));
    }
    asm volatile("s_nop 7\n s_nop 7\n s_nop 1" ::: "memory");   // MFMA results -> VALU
  }
  float v[8], scl[8];
  float mb = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 16 * wave + 4 * g + r;
    scl[r] = sca[t];
    v[r] = (t < nva && t >= loa) ? S0[r] * s2 * scl[r] : -INFINITY;
    scl[4 + r] = scb[t];
    v[4 + r] = t < nvb ? S1[r] * s2 * scl[4 + r] : -INFINITY;
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) mb = fmaxf(mb, v[r]);
  mb = max_xor32(max_xor16(mb));
  float alpha = 1.f;
  if (mb > st.m_ref + kTau) {
    alpha = __builtin_amdgcn_exp2f(st.m_ref - mb);
    st.m_ref = mb;
  }
  float p[8], ps = 0.f;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const bool ok = v[r] != -INFINITY;
    const float e = ok ? __builtin_amdgcn_exp2f(v[r] - st.m_ref) : 0.f;
    ps += e;
    p[r] = ok ? e * scl[r] : 0.f;
  }
  st.l_part = st.l_part * alpha + ps;
  if (__any(alpha != 1.f)) {
    asm volatile("s_nop 7\n s_nop 7\n s_nop 1" ::: "memory");  // previous MFMAs -> VALU
#pragma unroll
    for (int c = 0; c < 32; ++c) st.o[c] *= alpha;
  }
  const bf16x8 pf = __builtin_bit_cast(
      bf16x8, u32x4{pack2_bf16(p[0], p[1]), pack2_bf16(p[2], p[3]), pack2_bf16(p[4], p[5]), pack2_bf16(p[6], p[7])});

  // V^T: in each 16-lane group g, source lane j names token row 16w + 4g +
  // (j/2 mod 4) and the 8 columns 32 c + 8 (j mod 2) + 16 (j/8); lane s then
  // receives, for tokens 16w + 4g + e, e = 0..3, column 32 c + s (first dword)
  // and column 32 c + 16 + s (second dword), one read per page.  Rows outside
  // the window (past the end of the sequence or before its start) are zeroed
  // after conversion (their codes may be anything).
  const int jj = lane & 15;
  const int vo = (16 * wave + 4 * g + ((jj >> 1) & 3)) * kRowF + 8 * (jj & 1) + 16 * (jj >> 3);
  const LDSP char* vpa = ca + vo;
  const LDSP char* vpb = cb + vo;
  const int t0 = 16 * wave + 4 * g;
  auto keep_a = [&](int t) { return t >= loa && t < nva; };
  auto keep_b = [&](int t) { return t < nvb; };
  const uint32_t ka01 = (keep_a(t0) ? 0x0000FFFFu : 0u) | (keep_a(t0 + 1) ? 0xFFFF0000u : 0u);
  const uint32_t ka23 = (keep_a(t0 + 2) ? 0x0000FFFFu : 0u) | (keep_a(t0 + 3) ? 0xFFFF0000u : 0u);
  const uint32_t kb01 = (keep_b(t0) ? 0x0000FFFFu : 0u) | (keep_b(t0 + 1) ? 0xFFFF0000u : 0u);
  const uint32_t kb23 = (keep_b(t0 + 2) ? 0x0000FFFFu : 0u) | (keep_b(t0 + 3) ? 0xFFFF0000u : 0u);
  constexpr int kVPre = 4;
  i32x2 va[kVPre], vb[kVPre];
#pragma unroll
  for (int k = 0; k < kVPre; ++k) {
    va[k] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDSP i32x2*)(vpa + 32 * k));
    vb[k] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDSP i32x2*)(vpb + 32 * k));
  }
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const i32x2 wa = va[c % kVPre];
    const i32x2 wb = vb[c % kVPre];
    if (c + kVPre < 16) {
      va[c % kVPre] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDSP i32x2*)(vpa + 32 * (c + kVPre)));
      vb[c % kVPre] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDSP i32x2*)(vpb + 32 * (c + kVPre)));
    }
    const uint32_t b00 = cvt_pair<false>(wb[0]) & kb01, b01 = cvt_pair<true>(wb[0]) & kb23;
    const uint32_t b10 = cvt_pair<false>(wb[1]) & kb01, b11 = cvt_pair<true>(wb[1]) & kb23;
    const bf16x8 a0 =
        __builtin_bit_cast(bf16x8, u32x4{cvt_pair<false>(wa[0]) & ka01, cvt_pair<true>(wa[0]) & ka23, b00, b01});
    const bf16x8 a1 =
        __builtin_bit_cast(bf16x8, u32x4{cvt_pair<false>(wa[1]) & ka01, cvt_pair<true>(wa[1]) & ka23, b10, b11});
    asm volatile("s_nop 1\n v_mfma_f32_16x16x32_bf16 %0, %2, %4, %0\n v_mfma_f32_16x16x32_bf16 %1, %3, %4, %1"
                 : "+a"(st.o[2 * c]), "+a"(st.o[2 * c + 1]) : "v"(a0), "v"(a1), "v"(pf));
  }
}

__global__ void __launch_bounds__(256, 1) decode_fp8_h16(
    int32_t B, int32_t n_h, int32_t W, int32_t HG, float s2,
    const uint16_t* __restrict__ q_abs, const uint8_t* __restrict__ cache, const float* __restrict__ kv_scale,
    const int32_t* __restrict__ block_table, int32_t max_pages, int32_t bt_div,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ seq_starts, float* __restrict__ ws_o,
    float* __restrict__ ws_lse, int64_t* __restrict__ ws_tbl, uint16_t* __restrict__ o_lat,
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

  const PartRange pr = locate_part(seq_lens, seq_starts, B, kBs, part, W, g_lens);
  const int32_t chunk = pr.chunk;
  auto seq_len = [&](int32_t bb) { return chunk == 1 ? g_lens[bb] : seq_lens[bb]; };
  const int64_t x1 = pr.x1;
  int64_t x = pr.x0;
  if (x >= x1) return;
  int32_t b = __builtin_amdgcn_readfirstlane(pr.b);
  int64_t first = pr.first;

  uint32_t off[10];
  page_offsets(wave, lane, off);
  const char* cbase = reinterpret_cast<const char*>(cache);
  const int nper = page_loads(wave);
  for (;;) {
    // The window [st0, L) of sequence b: its pages start at page fp; L and the
    // page indices count from there; the first lo rows of that page lie
    // before the window.
    const int32_t st0 = __builtin_amdgcn_readfirstlane(seq_start(seq_starts, b));
    const int32_t fp = st0 / kBs, lo = st0 - fp * kBs;
    const int32_t L = __builtin_amdgcn_readfirstlane(seq_len(b)) - fp * kBs;
    const int64_t np = window_pages(L + fp * kBs, st0, kBs);
    const int64_t jp0 = x - first;
    const int64_t jp1 = min(np, jp0 + (x1 - x));
    const int n = static_cast<int>(jp1 - jp0);                  // pages of this segment
    const int32_t* bt = block_table + (int64_t)(b / bt_div) * max_pages + fp;   // bt_div sequences per row
    if (jp0 == 0 && hg == 0 && tid < 4) {                       // the merge's part range of sequence b
      const int64_t v[4] = {part, part_of_page(first + np - 1, pr.P, W), np, pr.P};
      ws_tbl[4 * (int64_t)b + tid] = v[tid];
    }

    // The segment's first three pages into slots 0-2, and this head group's
    // 16 query rows (18 KiB, contiguous in q_abs) into slot 3, which is free
    // until page 3 is issued: queries and pages arrive in one round trip.
    const int npre = min(3, n);
    {
      int32_t pid[3];
      sload3_i32(bt + jp0, bt + jp0 + min(1, n - 1), bt + jp0 + min(2, n - 1), &pid[0], &pid[1], &pid[2]);
      const char* q_u = uniform(reinterpret_cast<const char*>(q_abs + ((int64_t)b * n_h + (int64_t)hg * kHeads) * kD));
      const uint32_t q_m0 = uniform_lds((LDSP char*)g_ring + 3 * kSlotB);
#pragma unroll
      for (int i = 0; i < 5; ++i)
        if (wave + 4 * i < 18) dma16_u(q_u, 1024 * (wave + 4 * i) + 16 * lane, q_m0 + 1024 * (wave + 4 * i));
#pragma unroll
      for (int i = 0; i < 3; ++i)
        if (i < npre)
          load_page(uniform(cbase + (int64_t)pid[i] * kPageG), kv_scale + (int64_t)pid[i] * kBs, i, off, wave, lane);
    }
    wait_loads(nper * npre);                                    // this wave's query loads
    barrier_lds();
    bf16x8 qf[18];                                              // Q^T of heads 16 hg + s, pinned in AGPRs
    {
      const LDSP char* qrow = (LDSP char*)g_ring + 3 * kSlotB + s * (kD * 2) + 16 * g;
      bf16x8 t[18];
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) t[ks] = *reinterpret_cast<const LDSP bf16x8*>(qrow + 64 * ks);
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) asm volatile("" : "=a"(qf[ks]) : "0"(t[ks]));
    }
    auto issue = [&](int i) {                                   // page i of the segment into slot i % 4
      const int32_t pg = sload_i32(bt + jp0 + i);
      load_page(uniform(cbase + (int64_t)pg * kPageG), kv_scale + (int64_t)pg * kBs, i & 3, off, wave, lane);
    };

    State st;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) st.o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m_ref = -INFINITY;
    st.l_part = 0.f;

    // Two pages per step: pages 2k and 2k+1 are computed from slots (2k) % 4
    // and (2k+1) % 4 while pages 2k+2 and 2k+3 load into the other two (page 2
    // went out with the queries; page 3 goes into the query slot once every
    // wave holds its queries).
    for (int k = 0; 2 * k < n; ++k) {
      const int ia = 2 * k, ib = ia + 1;
      wait_loads(k == 0 && n > 2 ? nper : 0);                   // this wave's loads of pages ia, ib
      barrier_lds();                                            // everyone's; slots of the previous pair free
      if (ia + 2 >= 3 && ia + 2 < n) issue(ia + 2);
      if (ib + 2 < n) issue(ib + 2);
      const int nva = (int)min<int64_t>(kBs, (int64_t)L - (jp0 + ia) * kBs);
      const int loa = jp0 + ia == 0 ? lo : 0;
      const LDSP char* sa = (const LDSP char*)g_ring + (ia & 3) * kSlotB;
      const LDSP char* sb = (const LDSP char*)g_ring + (ib & 3) * kSlotB;
      const int nvb = ib < n ? (int)min<int64_t>(kBs, (int64_t)L - (jp0 + ib) * kBs) : 0;
      pair_compute(sa, sb, (const LDSP float*)g_sc[ia & 3], (const LDSP float*)g_sc[ib & 3], qf, wave, lane,
                   nva, loa, nvb, s2, st);
    }

    // ---- merge the four waves' states, normalise, store ----------------------
    asm volatile("s_nop 7\n s_nop 7\n s_nop 1" ::: "memory");    // MFMA results -> VALU
    const float lw = sum_xor32(sum_xor16(st.l_part));
    __syncthreads();                                            // every wave done with the ring
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
    // wave w's scaled O^T into ring slot w (register order: [cb][lane] float4, 32 KiB)
    {
      LDSP f32x4* dst = reinterpret_cast<LDSP f32x4*>((LDSP char*)g_ring + wave * kSlotB);
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
      for (int w = 0; w < 4; ++w) o += reinterpret_cast<const LDSP f32x4*>((LDSP char*)g_ring + w * kSlotB)[cb * 64 + lane];
      const int col = 16 * cb + 4 * g;
      if (whole)
        *reinterpret_cast<u32x2*>(o_lat + ((int64_t)b * n_h + head) * kDc + col) =
            u32x2{pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3])};
      else
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(ws_o + (((int64_t)part + b) * n_h + head) * kDc + col));
    }
    if (wave == 0 && g == 0) {
      const float lse_v = (M + __log2f(Lsum)) * 0.69314718055994531f;
      if (whole) { if (lse) lse[(int64_t)b * n_h + head] = lse_v; }
      else __builtin_nontemporal_store(lse_v, ws_lse + ((int64_t)part + b) * n_h + head);
    }

    x += jp1 - jp0;
    if (x >= x1) break;
    do { ++b; } while (window_pages(__builtin_amdgcn_readfirstlane(seq_len(b)),
                                    __builtin_amdgcn_readfirstlane(seq_start(seq_starts, b)), kBs) == 0);
    first = x;
    __syncthreads();                                            // slots read before the next loads
  }
}

}  // namespace

bool fp8_decode_supported(const mla_dims& d) {
  return d.act_dtype == MLA_BF16 && d.kv_dtype == MLA_E4M3 && d.d_latent == kDc && d.d_rope == 64 &&
         d.block_size == kBs && d.n_heads % kHeads == 0;
}

hipError_t launch_decode_fp8(const mla_dims& d, const DecodePlan& plan, int32_t B, const void* q_abs,
                             const void* cache, const float* kv_scale, const int32_t* block_table,
                             int32_t max_pages, int32_t bt_div, const int32_t* seq_lens,
                             const int32_t* seq_starts, float* ws_o, float* ws_lse, int64_t* ws_tbl, void* o_lat,
                             float* lse, hipStream_t s) {
  const int HG = d.n_heads / kHeads;
  const int W = plan.parts;
  const int grid = ((W + 7) / 8) * 8 * HG;                      // 8 XCDs x ceil(W/8) parts x HG
  const float s2 = d.softmax_scale * 1.4426950408889634f;
  decode_fp8_h16<<<grid, 256, 0, s>>>(B, d.n_heads, W, HG, s2, static_cast<const uint16_t*>(q_abs),
                                      static_cast<const uint8_t*>(cache), kv_scale, block_table, max_pages,
                                      bt_div, seq_lens, seq_starts, ws_o, ws_lse, ws_tbl,
                                      static_cast<uint16_t*>(o_lat), lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine(d, plan, B, seq_lens, seq_starts, ws_o, ws_lse, ws_tbl, o_lat, lse, s);
}

}  // namespace mla
