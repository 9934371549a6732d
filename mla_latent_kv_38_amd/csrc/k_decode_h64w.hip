// MFMA decode for DeepSeek-V2 shapes with a bfloat16 cache: d_c = 512,
// d_R = 64 (rows of 576), 64-token pages, n_h a multiple of 64.  Source:
// keybo.xyz page, section "第二步，推理时的吸收" (scores of the absorbed query
// against the cached latent, softmax, the weighted latent sum) and section
// "RoPE 为什么必须解耦" (the score is the sum over the latent and the RoPE
// part of the row); dgblog.top page, section "3. 一个聪明的优化".
//
// Work decomposition.  The batch's pages are flattened and cut into parts
// (mla_device.h); one workgroup of four waves handles one part for 64 heads,
// streaming its pages HBM -> LDS with direct-to-LDS loads (double-buffered).
// Wave w owns head block hb = w & 1 (32 heads) and token half th = w >> 1
// (32 of every page's 64 rows), and keeps its own online softmax over that
// half:
//   QK  S^T[32 tok x 32 heads] = C[32 x 576] Q^T: 36 MFMA 32x32x16 bf16, the
//       rows read from LDS, Q^T resident in registers.
//   softmax  per head in the lane that holds it (and its partner lane l^32),
//       entirely inside the wave; the reference maximum moves only when a
//       half page exceeds it by 2^8 (log2 units), so the accumulators are
//       rarely rescaled.
//   PV  O^T[512 x 32 heads] += V^T[512 x 32 tok] P^T[32 tok x 32 heads]: 32
//       MFMAs, V^T by transposed LDS reads of the same rows, P^T straight
//       from the score registers (the output layout of the QK product is the
//       B-operand layout of the PV product once the rows are permuted; the
//       token order is a contraction index, so any order is exact).
// The two token halves of a head block are merged once per segment through
// LDS.  The only barrier per page guards the page buffers.
//
// LDS page buffer: the 64 latent rows at a stride of 1040 B (1024 + 16), then
// the 64 RoPE parts in eight 1 KiB blocks at a stride of 1152 B, each holding
// eight tokens' 128 B with the 16-B chunks of token t XOR-permuted by t % 8.
// Every direct load then has a per-lane source offset that does not change
// from page to page, and the QK reads (16 rows, one 16-B column) and the
// transposed PV reads (4 rows x 32 columns) each cover all 64 banks once.
#include <utility>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
#define LDSP __attribute__((address_space(3)))

constexpr int kD = 576;
constexpr int kDc = 512;
constexpr int kBs = 64;
constexpr int kRowG = kD * 2;               // 1152 B: a cache row in global memory
constexpr int kPageG = kBs * kRowG;         // 73728 B: a page in global memory
constexpr int kLatRow = 1040;               // latent row in LDS: 1024 B + 16 pad
constexpr int kLatB = kBs * kLatRow;        // 66560
constexpr int kRopeBlk = 1152;              // RoPE block in LDS: 8 tokens x 128 B + 128 pad
constexpr int kBufB = kLatB + 8 * kRopeBlk; // 75776 B per page buffer
constexpr float kTau = 8.0f;                // lazy-rescale threshold (log2 units)

__shared__ __attribute__((aligned(1024))) char g_buf0[kBufB];
__shared__ __attribute__((aligned(1024))) char g_buf1[kBufB];
__shared__ __attribute__((aligned(16))) float g_xm[2 * 64];   // per token half: reference max of each head
__shared__ __attribute__((aligned(16))) float g_xl[2 * 64];   // per token half: row sum of each head
__shared__ int32_t g_lens[256];                               // seq_lens, when the batch has <= 256
__shared__ __attribute__((aligned(16))) int64_t g_seg[4];    // segment state: next page x, part end x1, first, b

// The segment record is read through a pointer the compiler cannot see
// through, so that it is re-read from LDS at every segment start instead of
// being kept in registers across the page loop.
__device__ __forceinline__ LDSP int64_t* seg_rec() {
  uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDSP int64_t*)g_seg));
  asm volatile("" : "+v"(a));
  return (LDSP int64_t*)(uintptr_t)a;
}

struct Lane {
  int lane, wave, l32, hi, hb, th, hg_part;
  uint32_t a_lat;        // QK: this lane's latent row and 16-B half of a k-step
  uint32_t a_rope[4];    // QK: the four RoPE k-steps
  uint32_t tr;           // PV: transposed-read base
  uint32_t v_lat, v_rope;  // direct loads: per-lane source offsets
};

// ---- optional cycle stamps -------------------------------------------------
// Built with -DMLA_CYCLE_STAMPS (mla_latent_kv_38_amd/cycle_stamps.py does so
// into a separate library), the kernel accumulates s_memtime stamps around
// its phases and wave 0 of each workgroup writes them to mla_stamp_buf;
// without it every macro below is empty and the code is unchanged.
#ifdef MLA_CYCLE_STAMPS
struct Stamps {
  unsigned long long wait = 0, bar = 0, qk = 0, sm = 0, pv = 0, pages = 0, ep = 0;
  unsigned long long t_start = 0, rt_start = 0, t_locate = 0, t_qissue = 0, t_loop = 0;
};
#define ST_NOW(v) const unsigned long long v = __builtin_amdgcn_s_memtime()
#define ST_ADD(o, f, a, b) ((o).f += (b) - (a))
#define ST_SET(o, f, v) ((o).f = (v))
#define ST_SET_ONCE(o, f, v) ((o).f = (o).f ? (o).f : (v))
#define ST_ARG , Stamps& stm
#define ST_PASS , stm
constexpr int kStampFields = 14;
constexpr int kStampGroups = 4096;
__device__ unsigned long long mla_stamp_buf[kStampGroups * kStampFields];
#else
struct Stamps {};
#define ST_NOW(v)
#define ST_ADD(o, f, a, b)
#define ST_SET(o, f, v)
#define ST_SET_ONCE(o, f, v)
#define ST_ARG
#define ST_PASS
#endif

// Token (row of the page) that MFMA row m of token half th stands for.  With
// m = 16u + 8e + 4h + a this is 32 th + 16u + 4a + 2e + h: the QK output
// register r = 8u + 4e + a of lane half h is then the score of row
// 32 th + 16u + 4a + 2e + h, and the PV k-step u takes P from registers
// 8u .. 8u + 7 with V^T rows 16u + 4a + 2e + h (a = 0..3 per transposed
// read, e = read index): four rows four apart per read.
__device__ __forceinline__ int row_of(int th, int m) {
  const int u = m >> 4, e = (m >> 3) & 1, h = (m >> 2) & 1, a = m & 3;
  return 32 * th + 16 * u + 4 * a + 2 * e + h;
}

// The matrix products are written as inline asm so that the scores and the
// operands stay in VGPRs and the 256 accumulator registers of O^T in AGPRs.
// Hazards the asm has to respect itself (the compiler does not look inside):
// a 32x32x16 product's result is read by other instructions only after 18
// wait states; a VGPR written by a VALU instruction is read by a product
// after at least 2 (5 are given below).
#define MFMA_QK0(S, a, b) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(S) : "v"(a), "v"(b))
#define MFMA_QK(S, a, b) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(S) : "v"(a), "v"(b))
#define MFMA_PV(O, a, b) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(O) : "v"(a), "v"(b))
#define MFMA_PV_AFTER_VALU(O, a, b) \
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(O) : "v"(a), "v"(b))
#define MFMA_RESULT_WAIT() asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory")

// The accumulators are touched outside the products only through these, one
// register at a time, so that the compiler never needs a VGPR copy of them
// (with 256 of them in AGPRs it would have to spill).
#define AGPR_SCALE(x, s)                                                                               \
  do {                                                                                                 \
    float t_;                                                                                          \
    asm volatile("v_accvgpr_read_b32 %0, %1\n\tv_mul_f32 %0, %0, %2\n\tv_accvgpr_write_b32 %1, %0" \
                 : "=&v"(t_), "+a"(x) : "v"(s));                                                      \
  } while (0)
__device__ __forceinline__ float agpr_read(float x) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(x));
  return v;
}

struct Acc {
  f32x16 o[16];          // O^T: 16 blocks of 32 latent columns x 32 heads
  float m_ref, l_own;    // reference max (log2 units) and this lane's row sum
};

// Where a wave's 18 direct loads of a page go: its 16 latent rows start at
// row 32 th + 16 hb (source `src`, LDS `lat`), its two RoPE blocks at block
// 4 th + 2 hb, whose source rows start at the same place (LDS `rope`).
struct PageDst {
  const char* src;       // wave-uniform (SGPRs)
  uint32_t lat, rope;    // LDS byte addresses, wave-uniform
};

__device__ __forceinline__ PageDst page_dst(const Lane& ln, const char* page, uint32_t buf_u) {
  // the wave's row base is rederived at each call from an opaque copy of the
  // wave index: kept alive instead, it ends up spilled across the page loop
  int w = ln.wave;
  asm volatile("" : "+s"(w));
  const int r16 = (2 * (w >> 1) + (w & 1)) * 16;       // 32 th + 16 hb
  PageDst d;
  d.src = uniform(page + r16 * kRowG);
  d.lat = __builtin_amdgcn_readfirstlane(buf_u + r16 * kLatRow);
  d.rope = __builtin_amdgcn_readfirstlane(buf_u + kLatB + (r16 >> 3) * kRopeBlk);
  return d;
}

// One 1 KiB direct load: global (src + voff + kSrc) -> LDS (base + kLds +
// 16 lane).  The offsets are immediates, so no address is kept per load.
template <int kSrc, int kLds>
__device__ __forceinline__ void dma_imm(const char* src, uint32_t voff, uint32_t base) {
  uint32_t v;
  asm volatile("s_add_u32 m0, %3, %5\n\t"
               "v_add_u32 %0, %4, %1\n\t"
               "global_load_lds_dwordx4 %0, %2"
               : "=&v"(v) : "v"(voff), "s"(src), "s"(base), "n"(kSrc), "n"(kLds) : "memory", "m0", "scc");
}

// load i (0..17) of this wave's share of a page
template <int i>
__device__ __forceinline__ void issue_load(const Lane& ln, const PageDst& d) {
  if constexpr (i < 16) dma_imm<i * kRowG, i * kLatRow>(d.src, ln.v_lat, d.lat);
  else dma_imm<(i - 16) * 8 * kRowG, (i - 16) * kRopeBlk>(d.src, ln.v_rope, d.rope);
}
// f(std::integral_constant<int, 0>) .. f(..., N - 1>), in order
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef short s16x8 __attribute__((ext_vector_type(8)));

// PV of one page for one wave: O^T[512 x 32 heads] += V^T P^T over the wave's
// 32 rows, with the wave's share of the next page's loads when kDma.  On a
// page with rows outside [lo, nvalid) (kMask) those rows of V^T are zeroed in
// registers: P is 0 there, but 0 times a non-finite value is not.
template <bool kMask, bool kDma>
__device__ __forceinline__ void pv_page(const Lane& ln, const LDSP char* __restrict__ buf, const PageDst& nd,
                                        const bf16x8 (&pb)[2], int nvalid, int lo, Acc& acc) {
  u32x4 vmask[2];
  if (kMask) {
    int tb = 32 * ln.th + ln.hi;
    asm volatile("" : "+v"(tb));
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t m = 0;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int i = 2 * j + h2;                    // element of the A fragment
          const int t = tb + 16 * u + 4 * (i & 3) + 2 * (i >> 2);
          if (t >= lo && t < nvalid) m |= 0xFFFFu << (16 * h2);
        }
        vmask[u][j] = m;
      }
  }
  auto vload = [&](int cb, int u) {
    const LDSP char* vp = buf + ln.tr + 16 * kLatRow * u + 64 * cb;
    const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDSP s16x4*)vp);
    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDSP s16x4*)(vp + 2 * kLatRow));
    return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  constexpr int kPre = 4;
  s16x8 vf[kPre];
#pragma unroll
  for (int s = 0; s < kPre; ++s) vf[s] = vload(s >> 1, s & 1);
  static_for<32>([&](auto S_) {
    constexpr int s = S_;
    constexpr int cb = s >> 1, u = s & 1;
    if constexpr (kMask) {
      const u32x4 raw = __builtin_bit_cast(u32x4, vf[s % kPre]) & vmask[u];
      const bf16x8 a = __builtin_bit_cast(bf16x8, raw);
      MFMA_PV_AFTER_VALU(acc.o[cb], a, pb[u]);
    } else if constexpr (s == 0) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, vf[0]);
      MFMA_PV_AFTER_VALU(acc.o[cb], a, pb[u]);        // P was just written by VALU instructions
    } else {
      const bf16x8 a = __builtin_bit_cast(bf16x8, vf[s % kPre]);
      MFMA_PV(acc.o[cb], a, pb[u]);
    }
    if constexpr (s + kPre < 32) vf[s % kPre] = vload((s + kPre) >> 1, (s + kPre) & 1);
    if constexpr (kDma && (s & 1) == 0) issue_load<(s >> 1)>(ln, nd);
  });
  if constexpr (kDma) {
    issue_load<16>(ln, nd);
    issue_load<17>(ln, nd);
  }
}

// S^T[32 tok x 32 heads] for one wave's token half: 36 products fed from LDS
// four fragments ahead, Q^T from registers; with kDma the wave's 18 loads of
// the next page go out beside them.
template <bool kDma>
__device__ __forceinline__ f32x16 qk_page(const Lane& ln, const LDSP char* __restrict__ buf, const PageDst& nd,
                                          const bf16x8 (&qf)[36]) {
  f32x16 S;
  constexpr int kPre = 4;
  bf16x8 af[kPre];
  auto aload = [&](int kb) {
    const uint32_t off = kb < 32 ? ln.a_lat + 32 * kb : ln.a_rope[kb - 32];
    return *(const LDSP bf16x8*)(buf + off);
  };
#pragma unroll
  for (int kb = 0; kb < kPre; ++kb) af[kb] = aload(kb);
  static_for<36>([&](auto KB) {
    constexpr int kb = KB;
    if constexpr (kb == 0) MFMA_QK0(S, af[0], qf[0]);
    else MFMA_QK(S, af[kb % kPre], qf[kb]);
    if constexpr (kb + kPre < 36) af[kb % kPre] = aload(kb + kPre);
    if constexpr (kDma && (kb & 1) == 0) issue_load<(kb >> 1)>(ln, nd);
  });
  MFMA_RESULT_WAIT();
  return S;
}

// One page for one wave.  The wave's share of the next page's loads goes out
// during QK; on a segment's last page the loads re-read the segment's query
// rows (resident in L2) into the free buffer, so every page runs the same
// code.  (The two head-group workgroups of a part request the same lines at
// about the same time; the L2 serves the second request from the first fill.)
__device__ __forceinline__ void page_step(const Lane& ln, const LDSP char* __restrict__ buf, bool fresh,
                                          const PageDst& nd, const bf16x8 (&qf)[36], int nvalid, int lo, float s2,
                                          Acc& acc ST_ARG) {

  // ---- QK ----------------------------------------------------------------
  ST_NOW(t0);
  f32x16 S = qk_page<true>(ln, buf, nd, qf);
  ST_NOW(t1);
  ST_ADD(stm, qk, t0, t1);

  // ---- softmax (inside the wave) -----------------------------------------
  const bool partial = nvalid < kBs || lo > 0;
  if (partial) {
    // (token indices from an opaque base: computed here, on the rare partial
    // page, rather than hoisted out of the loop into 16 registers)
    int tb = 32 * ln.th + ln.hi;
    asm volatile("" : "+v"(tb));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = tb + 16 * (r >> 3) + 4 * (r & 3) + 2 * ((r >> 2) & 1);
      if (t >= nvalid || t < lo) S[r] = -INFINITY;
    }
  }
  float mloc = fmaxf(fmaxf(fmaxf(S[0], S[1]), fmaxf(S[2], S[3])), fmaxf(fmaxf(S[4], S[5]), fmaxf(S[6], S[7])));
  mloc = fmaxf(mloc, fmaxf(fmaxf(fmaxf(S[8], S[9]), fmaxf(S[10], S[11])),
                           fmaxf(fmaxf(S[12], S[13]), fmaxf(S[14], S[15]))));
  const float mc = max_xor32(mloc) * s2;          // this half page's max of the head, log2 units
  const bool need = mc > acc.m_ref + kTau;
  if (__builtin_amdgcn_ballot_w64(need)) {
    const float alpha = need ? __builtin_amdgcn_exp2f(acc.m_ref - mc) : 1.f;   // m_ref = -inf: 0
    if (need) acc.m_ref = mc;
    acc.l_own *= alpha;
    if (!fresh) {                                   // (the accumulators are still 0 on a segment's first page)
#pragma unroll
      for (int cb = 0; cb < 16; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e) AGPR_SCALE(acc.o[cb][e], alpha);
    }
  }
  // rows masked in every page so far leave m_ref at -inf; their P is 0
  const float mr = acc.m_ref == -INFINITY ? 0.f : acc.m_ref;
  float ps = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    S[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], s2, -mr));
    ps += S[r];
  }
  acc.l_own += ps;
  bf16x8 pb[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    pb[u] = __builtin_bit_cast(bf16x8, u32x4{pack2_bf16(S[8 * u], S[8 * u + 1]), pack2_bf16(S[8 * u + 2], S[8 * u + 3]),
                                             pack2_bf16(S[8 * u + 4], S[8 * u + 5]),
                                             pack2_bf16(S[8 * u + 6], S[8 * u + 7])});

  // ---- PV: 16 column blocks x 2 k-steps ----------------------------------
  ST_NOW(t2);
  ST_ADD(stm, sm, t1, t2);
  if (partial) pv_page<true, false>(ln, buf, nd, pb, nvalid, lo, acc);
  else pv_page<false, false>(ln, buf, nd, pb, nvalid, lo, acc);
#ifdef MLA_CYCLE_STAMPS
  MFMA_RESULT_WAIT();                                  // (the products' time, not just their issue)
#endif
  ST_NOW(t3);
  ST_ADD(stm, pv, t2, t3);
}

// Segment epilogue helpers (the token half TH is a template argument so that
// every accumulator index is a constant and the accumulators stay in
// registers).  give_half: this wave's accumulators of the partner's column
// blocks 8 (1 - TH) .. +7 into the exchange area.  take_and_store: our blocks
// 8 TH .. +7 and the partner's, each with its weight (sc, sc_p: the two
// halves' shares of the row sum over it), summed and stored as bf16: to o_lat (whole: row of head `head`) or as the partial in
// register order (chunk ((hb*2 + th)*8 + c)*2 + qq; lane l's 16 B = columns
// 32cb + 16qq + 4hi + {0..3, 8..11} of head 32hb + l%32).
template <int TH>
__device__ __forceinline__ void give_half(const Acc& acc, LDSP float* xch, int lane) {
  LDSP float* dst = xch + (1 - TH) * (8 * 16 * 64);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const f32x16& o = acc.o[8 * (1 - TH) + c];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)   // raw accumulators (the receiver scales them)
      *(LDSP f32x4*)(dst + ((c * 4 + r4) * 64 + lane) * 4) =
          f32x4{agpr_read(o[4 * r4]), agpr_read(o[4 * r4 + 1]), agpr_read(o[4 * r4 + 2]), agpr_read(o[4 * r4 + 3])};
  }
}

template <int TH>
__device__ __forceinline__ void take_and_store(const Acc& acc, float sc, float sc_p, const LDSP float* xch,
                                               const Lane& ln, bool whole, uint16_t* dst) {
  const LDSP float* src = xch + TH * (8 * 16 * 64);
  // every read of the partner's blocks goes out before the first use: the
  // accumulator reads below are volatile asm, which the compiler does not
  // move loads across, so reads left inside the loop would each wait their
  // full LDS latency
  f32x4 tp[8][4];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) tp[c][r4] = *(const LDSP f32x4*)(src + ((c * 4 + r4) * 64 + ln.lane) * 4);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    constexpr int kCb0 = 8 * TH;
    float v[16];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 t = tp[c][r4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * r4 + e] = __builtin_fmaf(agpr_read(acc.o[kCb0 + c][4 * r4 + e]), sc, t[e] * sc_p);
    }
    if (whole) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = 32 * (kCb0 + c) + 8 * q + 4 * ln.hi;
        *reinterpret_cast<u32x2*>(dst + col) =
            u32x2{pack2_bf16(v[4 * q], v[4 * q + 1]), pack2_bf16(v[4 * q + 2], v[4 * q + 3])};
      }
    } else {
#pragma unroll
      for (int qq = 0; qq < 2; ++qq)
        __builtin_nontemporal_store(
            u32x4{pack2_bf16(v[8 * qq], v[8 * qq + 1]), pack2_bf16(v[8 * qq + 2], v[8 * qq + 3]),
                  pack2_bf16(v[8 * qq + 4], v[8 * qq + 5]), pack2_bf16(v[8 * qq + 6], v[8 * qq + 7])},
            reinterpret_cast<u32x4*>(dst + ((((ln.hb * 2 + TH) * 8 + c) * 2 + qq) * 64 + ln.lane) * 8));
    }
  }
}

template <int kCnt>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kCnt) : "memory");
}

// a wave-uniform 64-bit value into SGPRs
__device__ __forceinline__ int64_t sgpr64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

__global__ void __launch_bounds__(256, 1) decode_h64w(
    int32_t B, int32_t n_h, int32_t W, int32_t HG, float s2, const uint16_t* __restrict__ q_abs,
    const void* __restrict__ cache, const int32_t* __restrict__ block_table, int32_t max_pages, int32_t bt_div,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ seq_starts, float* __restrict__ ws_o,
    float* __restrict__ ws_lse, int64_t* __restrict__ ws_tbl, uint16_t* __restrict__ o_lat,
    float* __restrict__ lse) {
#ifdef MLA_CYCLE_STAMPS
  Stamps stm;
  stm.t_start = __builtin_amdgcn_s_memtime();
  stm.rt_start = __builtin_amdgcn_s_memrealtime();
#endif
  Lane ln;
  const int tid = threadIdx.x;
  ln.lane = tid & 63;
  ln.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  ln.l32 = ln.lane & 31;
  ln.hi = ln.lane >> 5;
  ln.hb = ln.wave & 1;
  ln.th = ln.wave >> 1;

  // Workgroup i runs on XCD i % 8; XCD x takes the contiguous parts
  // [x ppx, (x+1) ppx) with all their head groups, so the head groups of a
  // part read each page through the same L2.
  const int ppx = (W + 7) / 8;
  const int xcd = blockIdx.x & 7, jw = blockIdx.x >> 3;
  const int hg = jw % HG;
  ln.hg_part = hg & 1;
  const int part = xcd * ppx + jw / HG;
  if (part >= W) return;

  {
    const int row = row_of(ln.th, ln.l32);
    ln.a_lat = row * kLatRow + 16 * ln.hi;
    const int blk = row >> 3, t8 = row & 7;
#pragma unroll
    for (int k = 0; k < 4; ++k) ln.a_rope[k] = kLatB + blk * kRopeBlk + 128 * t8 + 16 * ((2 * k + ln.hi) ^ t8);
    const int g = ln.lane >> 4, sg = ln.lane & 15;
    ln.tr = (32 * ln.th + 4 * (sg >> 2) + ln.hi) * kLatRow + 32 * (g & 1) + 8 * (sg & 3);
    ln.v_lat = 16 * ln.lane;
    const int tq = ln.lane >> 3, s = ln.lane & 7;
    ln.v_rope = tq * kRowG + 1024 + 16 * (s ^ tq);
  }

  const PartRange pr = locate_part(seq_lens, seq_starts, B, kBs, part, W, g_lens);
  ST_NOW(t_loc);
  ST_SET(stm, t_locate, t_loc);
  if (pr.x0 >= pr.x1) return;
  const bool lens_in_lds = pr.chunk == 1;
  const int64_t P = pr.P;
  auto seq_len = [&](int32_t bb) -> int32_t {   // from LDS (batches of up to 256) or global memory
    int32_t v;
    if (lens_in_lds) v = ((const LDSP int32_t*)g_lens)[bb & 255];
    else v = __builtin_nontemporal_load(seq_lens + bb);
    return v;
  };
  // The segment state lives in LDS between segments (read at a segment's
  // start, written at its end), so that nothing of it stays in registers
  // across the page loop.
  if (threadIdx.x == 0) {
    LDSP int64_t* r = (LDSP int64_t*)g_seg;
    r[0] = pr.x0;
    r[1] = pr.x1;
    r[2] = pr.first;
    r[3] = pr.b;
  }
  __syncthreads();
  const char* cbase = reinterpret_cast<const char*>(cache);

  for (;;) {
    const LDSP int64_t* rec = seg_rec();
    const int64_t x = rec[0], x1 = rec[1], first = rec[2];
    const int32_t b = static_cast<int32_t>(rec[3]);
    const int32_t st = seq_start(seq_starts, b);
    const int32_t fp = st / kBs, lo = st - fp * kBs;
    const int32_t Lb = seq_len(b);
    const int32_t L = Lb - fp * kBs;
    const int64_t np = window_pages(Lb, st, kBs);
    const int64_t jp0 = x - first;
    const int64_t jp1 = min(np, jp0 + (x1 - x));
    int32_t btd = bt_div;                                // opaque: no divider state kept across segments
    asm volatile("" : "+s"(btd));
    const int32_t* bt = block_table + (int64_t)(btd == 1 ? b : b / btd) * max_pages + fp;

    // This head group's 64 absorbed query rows (contiguous in q_abs, the same
    // 64 x 1152 B shape as a page) come into buffer 1 laid out like a page,
    // by the same 1 KiB direct loads; then the first page into buffer 0.  The
    // queries need no page id, so they go out first.
    {
      int32_t hg_o = hg;                                 // opaque: the row address is not hoisted
      asm volatile("" : "+s"(hg_o));
      const PageDst dq = page_dst(ln, reinterpret_cast<const char*>(q_abs + ((int64_t)b * n_h + (int64_t)hg_o * 64) * kD),
                                  uniform_lds((LDSP char*)g_buf1));
      static_for<18>([&](auto I) { issue_load<I>(ln, dq); });
    }
    ST_NOW(t_qi);
    ST_SET_ONCE(stm, t_qissue, t_qi);
    int32_t pg0, pg_next;                                // ids of the first two pages, one round trip
    sload2_i32(bt + jp0, bt + (jp0 + 1 < jp1 ? jp0 + 1 : jp0), &pg0, &pg_next);
    {
      const PageDst d0 = page_dst(ln, cbase + (int64_t)pg0 * kPageG, uniform_lds((LDSP char*)g_buf0));
      static_for<18>([&](auto I) { issue_load<I>(ln, d0); });
    }
    if (jp0 == 0 && hg == 0 && threadIdx.x < 4) {                // the merge's part range of sequence b
      // (written once the loads are out: its operands may come from scratch)
      int64_t Po = sgpr64(P);                            // opaque, as above
      int t = threadIdx.x;
      asm volatile("" : "+s"(Po));
      asm volatile("" : "+v"(t));
      const int64_t lp = part_of_page(first + np - 1, Po, W);
      ws_tbl[4 * (int64_t)b + t] = t == 0 ? (int64_t)part : t == 1 ? lp : t == 2 ? np : Po;
    }
    Acc acc;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) acc.o[cb] = f32x16{};
    acc.m_ref = -INFINITY;
    acc.l_own = 0.f;
    // Q^T fragments of this wave's 32 heads from buffer 1: head 32 hb + l%32
    // sits where a page keeps row 32 hb + l%32, so the QK read offsets of that
    // row serve (the first page keeps landing meanwhile: direct loads complete
    // in order, so waiting for all but the last 18 waits for the queries only)
    wait_vm<18>();
    __syncthreads();
    bf16x8 qf[36];
    {
      const LDSP char* qb = (const LDSP char*)g_buf1;
      int lq = ln.lane;                                  // opaque: these addresses are not hoisted
      asm volatile("" : "+v"(lq));
      const int h = 32 * ln.hb + (lq & 31);
      const uint32_t q_lat = h * kLatRow + 16 * (lq >> 5);
      const int blk = h >> 3, t8 = h & 7;
#pragma unroll
      for (int kb = 0; kb < 36; ++kb) {
        const uint32_t off = kb < 32 ? q_lat + 32 * kb : kLatB + blk * kRopeBlk + 128 * t8 + 16 * ((2 * (kb - 32) + (lq >> 5)) ^ t8);
        qf[kb] = *(const LDSP bf16x8*)(qb + off);
      }
#pragma unroll
      for (int kb = 0; kb < 36; ++kb) asm volatile("" ::"v"(qf[kb]));   // in registers before buffer 1 is reused
    }
    __syncthreads();                                     // buffer 1 free for the second page

    ST_NOW(t_lp);
    ST_SET_ONCE(stm, t_loop, t_lp);
    const int32_t j0 = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(jp0));
    const int32_t j1 = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(jp1));
    const int32_t Lu = __builtin_amdgcn_readfirstlane(L);
    const char* qrows = reinterpret_cast<const char*>(q_abs + ((int64_t)b * n_h + (int64_t)hg * 64) * kD);
    for (int32_t jp = j0; jp < j1; ++jp) {
      const bool even = ((jp - j0) & 1) == 0;
      const LDSP char* buf = even ? (const LDSP char*)g_buf0 : (const LDSP char*)g_buf1;
      const uint32_t nbuf_u = uniform_lds(even ? (LDSP char*)g_buf1 : (LDSP char*)g_buf0);
      ST_NOW(tw0);
      wait_vm<0>();                                      // this wave's loads of page jp (and the queries)
      ST_NOW(tw1);
      __syncthreads();                                   // every wave's loads landed; page jp-1 consumed
      ST_NOW(tw2);
      ST_ADD(stm, wait, tw0, tw1);
      ST_ADD(stm, bar, tw1, tw2);
      ST_ADD(stm, pages, 0, 1);
      const bool more = jp + 1 < j1;
      const PageDst nd = page_dst(ln, more ? cbase + (int64_t)pg_next * kPageG : qrows, nbuf_u);
      // id two ahead, read during this page (constant address space: a scalar load)
      const int32_t pg2 = jp + 2 < j1 ? ((const __attribute__((address_space(4))) int32_t*)bt)[jp + 2] : 0;
      const int nvalid = min(kBs, Lu - jp * kBs);
      const int plo = jp == 0 ? lo : 0;
      page_step(ln, buf, jp == j0, nd, qf, nvalid, plo, s2, acc ST_PASS);
      pg_next = pg2;
    }
    wait_vm<0>();                                        // the last page's loads (query rows) landed

    ST_NOW(te0);
    // ---- segment epilogue: merge the token halves, normalise, store ---------
    MFMA_RESULT_WAIT();                                  // last products' results
    // The epilogue's per-lane addresses are derived from an opaque copy of the
    // lane index, so that the compiler computes them here instead of keeping
    // dozens of them alive (and spilled) across the whole segment loop.
    Lane le = ln;
    asm volatile("" : "+v"(le.lane));
    asm volatile("" : "+s"(le.wave));
    le.l32 = le.lane & 31;
    le.hi = le.lane >> 5;
    le.hb = le.wave & 1;
    le.th = le.wave >> 1;
    const float l_half = sum_xor32(acc.l_own);
    if (le.hi == 0) {
      g_xm[le.th * 64 + le.hb * 32 + le.l32] = acc.m_ref;
      g_xl[le.th * 64 + le.hb * 32 + le.l32] = l_half;
    }
    __syncthreads();                                     // also: every wave is done with the page buffers
    const float m_o = g_xm[(1 - le.th) * 64 + le.hb * 32 + le.l32];
    const float l_o = g_xl[(1 - le.th) * 64 + le.hb * 32 + le.l32];
    const float M = fmaxf(acc.m_ref, m_o);               // finite: the segment holds a row of the window
    const float f_own = __builtin_amdgcn_exp2f(acc.m_ref - M), f_o = __builtin_amdgcn_exp2f(m_o - M);
    const float lt = l_half * f_own + l_o * f_o;
    const float sc = f_own / lt, sc_p = f_o / lt;     // this wave's and the partner's weights
    // hand the partner the column blocks it stores (8 (1 - th) .. +7 of this
    // wave's contribution, float32, register order) and take ours from it
    uint32_t xaddr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(le.hb == 0 ? g_buf0 : g_buf1));
    asm volatile("" : "+v"(xaddr));                      // (addressed per lane + immediate, not hoisted)
    LDSP float* xch = (LDSP float*)(uintptr_t)xaddr;
    if (le.th == 0) give_half<0>(acc, xch, le.lane);
    else give_half<1>(acc, xch, le.lane);
    __syncthreads();
    const bool whole = (jp0 == 0 && jp1 == np);
    const int64_t head = (int64_t)hg * 64 + le.hb * 32 + le.l32;
    if (le.th == 0 && le.hi == 0) {
      const float lse_v = (M + __log2f(lt)) * 0.69314718055994531f;
      if (whole) { if (lse) lse[(int64_t)b * n_h + head] = lse_v; }
      else __builtin_nontemporal_store(lse_v, ws_lse + ((int64_t)part + b) * n_h + head);
    }
    uint16_t* dst = whole ? o_lat + ((int64_t)b * n_h + head) * kDc
                          : reinterpret_cast<uint16_t*>(ws_o) + (((int64_t)part + b) * n_h + (int64_t)hg * 64) * kDc;
    if (le.th == 0) take_and_store<0>(acc, sc, sc_p, xch, ln, whole, dst);
    else take_and_store<1>(acc, sc, sc_p, xch, ln, whole, dst);

    ST_NOW(te1);
    ST_ADD(stm, ep, te0, te1);
    const int64_t xn = x + (jp1 - jp0);
    if (xn >= x1) break;
    int32_t bn = b;
    do { ++bn; } while (window_pages(seq_len(bn), seq_start(seq_starts, bn), kBs) == 0);
    __syncthreads();                                     // exchange area and g_seg read before they change
    if (threadIdx.x == 0) {
      LDSP int64_t* r = seg_rec();
      r[0] = xn;
      r[2] = xn;
      r[3] = bn;
    }
    __syncthreads();
  }
#ifdef MLA_CYCLE_STAMPS
  if (tid == 0 && blockIdx.x < kStampGroups) {
    unsigned long long* o = mla_stamp_buf + (int64_t)blockIdx.x * kStampFields;
    const unsigned long long t_end = __builtin_amdgcn_s_memtime(), rt_end = __builtin_amdgcn_s_memrealtime();
    const unsigned long long v[kStampFields] = {t_end - stm.t_start, stm.t_locate - stm.t_start,
                                                stm.t_qissue - stm.t_start, stm.t_loop - stm.t_start, stm.wait,
                                                stm.bar, stm.qk, stm.sm, stm.pv, stm.pages, stm.ep, stm.rt_start,
                                                rt_end, 1};
    for (int i = 0; i < kStampFields; ++i) o[i] = v[i];
  }
#endif
}

// ---------------------------------------------------------------------------
// Merge of the split-KV partials of decode_h64w.  A partial (slot, 64-head
// group) is 64 KiB of bfloat16 in the register order above, already divided
// by its own row sum; its log-sum-exp (float32) is in ws_lse.  One workgroup
// per (sequence, head group, 4 of the 64 chunks); thread (wave q4, lane l)
// owns one 16-B piece of each partial.  Parts are merged kN at a time with a
// running maximum, all kN loads of a batch in flight together:
//   o_lat = sum_k e^(lse_k - M) o_k / sum_k e^(lse_k - M),  lse = M + ln(sum).
// kN is 2, 4 or 8 by the sequence's part count, so that a sequence split in
// two or four parts (ragged batches, several query tokens) issues no loads
// beyond its parts.
// ---------------------------------------------------------------------------
struct MergeState {
  f32x4 a0, a1;
  float m, d;
};

template <int kN>
__device__ __forceinline__ void merge_parts(MergeState& st, int64_t w0, int64_t w1, int32_t b, int64_t P, int32_t W,
                                            bool all_live, const uint16_t* __restrict__ ws16, int64_t off,
                                            const float* __restrict__ lse_col, int32_t n_h) {
  for (int64_t base = w0; base <= w1; base += kN) {
    f32x4 v0[kN], v1[kN];
    float e[kN];
#pragma unroll
    for (int jj = 0; jj < kN; ++jj) {                 // part w0 always holds a page: dead parts read it
      const int64_t w = base + jj;
      const bool live = w <= w1 && (all_live || part_start(w, P, W) < part_start(w + 1, P, W));
      const int64_t slot = (live ? w : w0) + b;
      const u32x4 raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ws16 + slot * n_h * kDc + off));
      v0[jj] = f32x4{__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                     __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
      v1[jj] = f32x4{__uint_as_float(raw.z << 16), __uint_as_float(raw.z & 0xffff0000u),
                     __uint_as_float(raw.w << 16), __uint_as_float(raw.w & 0xffff0000u)};
      e[jj] = live ? lse_col[slot * n_h] : -INFINITY;
    }
    float n = st.m;
#pragma unroll
    for (int jj = 0; jj < kN; ++jj) n = fmaxf(n, e[jj]);
    const float a = n == st.m ? 1.f : __expf(st.m - n);
    st.a0 *= a;
    st.a1 *= a;
    st.d *= a;
    st.m = n;
#pragma unroll
    for (int jj = 0; jj < kN; ++jj) {
      const float x = e[jj] == -INFINITY ? 0.f : __expf(e[jj] - st.m);
      st.d += x;
      st.a0 += x * v0[jj];
      st.a1 += x * v1[jj];
    }
  }
}

__global__ void __launch_bounds__(256) combine_h64w(int32_t B, int32_t n_h, int32_t W, int32_t HG,
                                                    const int32_t* __restrict__ seq_lens,
                                                    const int32_t* __restrict__ seq_starts,
                                                    const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
                                                    const int64_t* __restrict__ ws_tbl, uint16_t* __restrict__ o_lat,
                                                    float* __restrict__ lse) {
  const int per_seq = HG * 16;
  const int32_t b = blockIdx.x / per_seq;
  const int r = blockIdx.x % per_seq;
  const int hg = r / 16, wc = r % 16;
  const int tid = threadIdx.x, lane = tid & 63, q4 = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int c = wc * 4 + q4;                          // chunk of the partial
  const int hb = c >> 5, th = (c >> 4) & 1, cl = (c >> 1) & 7, qq = c & 1;
  const int col = 32 * (8 * th + cl) + 16 * qq + 4 * hi;
  const int hh = 32 * hb + l32;                       // head within the group
  const int64_t head = (int64_t)b * n_h + (int64_t)hg * 64 + hh;
  // the part range is loaded together with the length (it is only stale for
  // an empty sequence, which no part covers and which does not read it)
  u32x4 wr;
  u32x2 pr;
  int32_t len;
  asm volatile("s_load_dwordx4 %0, %3, 0x0\n\t"
               "s_load_dwordx2 %1, %3, 0x18\n\t"
               "s_load_dword %2, %4, 0x0\n\t"
               "s_waitcnt lgkmcnt(0)"
               : "=&s"(wr), "=&s"(pr), "=&s"(len)
               : "s"(ws_tbl + 4 * (int64_t)b), "s"(seq_lens + b)
               : "memory");
  const int64_t w0 = static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(wr[1])) << 32) |
                                          static_cast<uint32_t>(wr[0]));
  const int64_t w1 = static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(wr[3])) << 32) |
                                          static_cast<uint32_t>(wr[2]));
  const int64_t P = static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(pr[1])) << 32) |
                                         static_cast<uint32_t>(pr[0]));
  const int64_t np = window_pages(len, seq_start(seq_starts, b), kBs);
  if (np == 0) {                                      // empty sequence: zero output, lse = -inf
    *reinterpret_cast<u32x2*>(o_lat + head * kDc + col) = u32x2{0u, 0u};
    *reinterpret_cast<u32x2*>(o_lat + head * kDc + col + 8) = u32x2{0u, 0u};
    if (c == 0 && hi == 0 && lse) {
      lse[head] = -INFINITY;
      lse[head + 32] = -INFINITY;
    }
    return;
  }
  if (w0 == w1) return;                               // one part: written by the decode kernel
  const bool all_live = P >= W;
  const uint16_t* ws16 = reinterpret_cast<const uint16_t*>(ws_o);
  const int64_t off = (int64_t)hg * 64 * kDc + (c * 64 + lane) * 8;
  const float* lse_col = ws_lse + (int64_t)hg * 64 + hh;
  MergeState st{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, -INFINITY, 0.f};
  const int64_t nparts = w1 - w0 + 1;                 // wave-uniform: one branch for the workgroup
  if (nparts <= 2) merge_parts<2>(st, w0, w1, b, P, W, all_live, ws16, off, lse_col, n_h);
  else if (nparts <= 4) merge_parts<4>(st, w0, w1, b, P, W, all_live, ws16, off, lse_col, n_h);
  else merge_parts<8>(st, w0, w1, b, P, W, all_live, ws16, off, lse_col, n_h);
  const f32x4 a0 = st.a0, a1 = st.a1;
  const float m = st.m, d = st.d;
  const float inv = 1.f / d;
  *reinterpret_cast<u32x2*>(o_lat + head * kDc + col) =
      u32x2{pack2_bf16(a0[0] * inv, a0[1] * inv), pack2_bf16(a0[2] * inv, a0[3] * inv)};
  *reinterpret_cast<u32x2*>(o_lat + head * kDc + col + 8) =
      u32x2{pack2_bf16(a1[0] * inv, a1[1] * inv), pack2_bf16(a1[2] * inv, a1[3] * inv)};
  if (c == 0 && hi == 0 && lse) lse[head] = m + __logf(d);
  if (c == 32 && hi == 0 && lse) lse[head] = m + __logf(d);
}

}  // namespace

bool h64w_decode_supported(const mla_dims& d) {
  return d.act_dtype == MLA_BF16 && d.kv_dtype == MLA_BF16 && d.d_latent == kDc && d.d_rope == 64 &&
         d.block_size == kBs && d.n_heads % 64 == 0;
}

hipError_t launch_decode_h64w(const mla_dims& d, const DecodePlan& plan, int32_t B, const void* q_abs,
                              const void* cache, const int32_t* block_table, int32_t max_pages, int32_t bt_div,
                              const int32_t* seq_lens, const int32_t* seq_starts, float* ws_o, float* ws_lse,
                              int64_t* ws_tbl, void* o_lat, float* lse, hipStream_t s) {
  const int HG = d.n_heads / 64;
  const int W = plan.parts;
  const int grid = ((W + 7) / 8) * 8 * HG;
  const float s2 = d.softmax_scale * 1.4426950408889634f;
  decode_h64w<<<grid, 256, 0, s>>>(B, d.n_heads, W, HG, s2, static_cast<const uint16_t*>(q_abs), cache, block_table,
                                   max_pages, bt_div, seq_lens, seq_starts, ws_o, ws_lse, ws_tbl,
                                   static_cast<uint16_t*>(o_lat), lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  combine_h64w<<<B * HG * 16, 256, 0, s>>>(B, d.n_heads, W, HG, seq_lens, seq_starts, ws_o, ws_lse, ws_tbl,
                                           static_cast<uint16_t*>(o_lat), lse);
  return hipGetLastError();
}

#ifdef MLA_CYCLE_STAMPS
// Readers of the stamps (only in the stamped build).
extern "C" int mla_stamps_read(void* host, size_t bytes) {
  return static_cast<int>(hipMemcpyFromSymbol(host, HIP_SYMBOL(mla_stamp_buf), bytes, 0, hipMemcpyDeviceToHost));
}
extern "C" int mla_stamps_fields() { return kStampFields; }
#endif

}  // namespace mla
