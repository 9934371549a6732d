// 64-head decode over an E4M3 cache at DeepSeek-V2 shapes: d_c = 512,
// d_R = 64 (rows of 576 codes, one float32 scale per row), 64-token pages,
// bfloat16 queries, n_h a multiple of 64.  Source: keybo.xyz page, section
// "第二步，推理时的吸收" (scores against the cached latent with the absorbed
// query, softmax, the weighted latent sum) and dgblog.top page, section
// "3. 一个聪明的优化：上采样矩阵可以"吸收""; the E4M3 row is code x per-row scale
// (keybo.xyz page, section "所以 cache 逻辑到底哪里要重写"), which factors out of
// both contractions.
//
// Work decomposition.  The batch's pages are flattened and cut into parts
// (see mla_device.h); one workgroup handles one part for 64 heads.  A
// workgroup is 4 waves on one CU; it streams its pages HBM -> LDS with
// direct-to-LDS loads (double-buffered) and every code row is read from LDS
// by all 64 heads:
//   QK  wave w scores head block hb = w & 1 (32 heads) against token half
//       th = w >> 1 of the page: S^T[32 tok x 32 heads] = C[32 x 576] Q^T,
//       36 MFMA 32x32x16 bf16 on 8-code groups converted exactly to bf16 in
//       registers, Q^T resident in AGPRs; the row scale multiplies the scores.
//   softmax  per head (one lane), page max shared between the two token-half
//       waves through LDS; the reference max only moves when the page max
//       exceeds it by 2^8 (scores are in log2 units), so rescaling the
//       accumulators is rare; P times the row scale goes to LDS as bf16.
//   PV  wave w accumulates O^T[128 latent columns x 64 heads] =
//       V^T[128 x 64 tok] P^T[64 tok x 64 heads]: 32 MFMAs per page; V^T
//       comes from ds_read_b64_tr_b8 on the code rows, converted the same
//       way, each V fragment feeding two head blocks.
// Code rows are padded to 37 x 16 B in LDS, the queries (staged once per
// segment) to 73 x 16 B; the token order inside each MFMA is permuted to
// match the reads (it is a contraction index, so any order is exact).
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
#define LDSP __attribute__((address_space(3)))

constexpr int kD = 576;
constexpr int kDc = 512;
constexpr int kBs = 64;
constexpr int kRowB = 1168;                 // query row in LDS: 1152 bytes + 16 pad (73 x 16 B)
constexpr int kPageB = kBs * kRowB;         // 74752 = 73 x 1 KiB: a page buffer (64 padded query rows)
constexpr int kPtRowB = 144;                // P^T row: 64 bf16 + 16 pad
constexpr float kTau = 8.0f;                // lazy-rescale threshold (log2 units)
constexpr int kCodePageB = kBs * kD;        // 36864: one page of E4M3 codes in the cache
constexpr int kRowC = 592;                  // E4M3 row in LDS: 576 codes + 16 pad (37 x 16 B)
constexpr int kCodeRowsB = kBs * kRowC;     // 37888; the page's 64 float32 scales follow
static_assert(kCodeRowsB + kBs * 4 <= kPageB, "an E4M3 page fits a page buffer");


// The head group's 64 absorbed query rows (64 x 1152 B, contiguous in q_abs)
// go into a page buffer with rows padded to 73 x 16 B: 73 direct loads of
// 64 lanes x 16 B, LDS slot s = 64 k + lane holding row s / 73, 16-B chunk
// s % 73 (chunk 72 is padding and re-reads chunk 0).  Wave w issues loads
// k = w, w + 4, ... (19 for wave 0, 18 for the others); the lane's (row,
// chunk) advances by 256 slots = 3 rows + 37 chunks per load.  The offsets
// are the same for every segment, so each lane's 19 are computed once per
// workgroup and kept in AGPRs (free beside the queries).
__device__ __forceinline__ int dma_count(int wave) { return wave == 0 ? 19 : 18; }

__device__ __forceinline__ void dma_offsets(int wave, int lane, uint32_t (&offa)[19]) {
  const int s0 = 64 * wave + lane;
  int row = s0 / 73, ch = s0 - 73 * (s0 / 73);
#pragma unroll
  for (int i = 0; i < 19; ++i) {
    const uint32_t off = static_cast<uint32_t>(row * (kD * 2) + (ch == 72 ? 0 : ch * 16));
    asm volatile("" : "=a"(offa[i]) : "0"(off));
    ch += 37;
    row += 3;
    if (ch >= 73) { ch -= 73; row += 1; }
  }
}

// Two E4M3 codes (the low or high half of a dword) -> two bfloat16: the
// scaled conversion with scale 1.0 is exact for every code (each E4M3 value
// is a bfloat16 value).
template <bool kHi>
__device__ __forceinline__ uint32_t cvt_pair(uint32_t codes) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, kHi));
}

__device__ __forceinline__ bf16x8 cvt8(u32x2 c) {      // 8 codes -> 8 bfloat16, in order
  return __builtin_bit_cast(bf16x8, u32x4{cvt_pair<false>(c[0]), cvt_pair<true>(c[0]), cvt_pair<false>(c[1]),
                                          cvt_pair<true>(c[1])});
}

// Copy one E4M3 page (64 x 576 codes, then 64 float32 scales) into a page
// buffer with rows padded to 37 x 16 B: LDS slot q = 64 k + lane holds row
// q / 37, 16-B chunk q % 37 (chunk 36 is padding and re-reads chunk 0);
// 37 direct loads, wave w issuing k = w, w + 4, ...; wave 0 also loads the
// scales.  Per wave: 10 loads (wave 0: 11 with the scales) or 9.
__device__ __forceinline__ void dma_code_page(const char* src_u, uint32_t dst_u, const char* ssrc,
                                              LDSP char* sdst, int wave, int lane) {
  const int q0 = 64 * wave + lane;
  int row = q0 / 37, ch = q0 - 37 * (q0 / 37);
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    if (wave + 4 * i < 37)
      dma16_u(src_u, static_cast<uint32_t>(row * kD + (ch == 36 ? 0 : 16 * ch)), dst_u + 1024u * (wave + 4 * i));
    row += 6;                                        // 256 slots = 6 rows + 34 chunks
    ch += 34;
    if (ch >= 37) { ch -= 37; row += 1; }
  }
  if (wave == 0) dma4(ssrc, 4 * lane, sdst);
}

// S^T for one wave from an E4M3 page: as qk_page, with each 8-code A
// fragment converted in registers just before its MFMA.  A lane reads 16
// codes at a time (row tok, bytes 32 j + 16 hi), the fragments of MFMAs
// 2 j and 2 j + 1, so the contraction index of MFMA 2 j + e2, lane half hi,
// element e is 32 j + 16 hi + 8 e2 + e (the query fragments follow the same
// order).  The 16-byte reads of 16 token rows 592 B apart cover all 64
// banks once; 8-byte reads would meet 2-way conflicts.
__device__ __forceinline__ f32x16 qk_page_e4m3(const LDSP char* __restrict__ ap, const bf16x8 (&qf)[36]) {
  f32x16 S;
  constexpr int kPre = 2;                       // 16-code reads in flight (4 MFMAs)
  u32x4 cf[kPre];
#pragma unroll
  for (int j = 0; j < kPre; ++j) cf[j] = *(const LDSP u32x4*)(ap + 32 * j);
#pragma unroll
  for (int kb = 0; kb < 36; ++kb) {
    const int j = kb >> 1;
    const u32x4 w = cf[j % kPre];
    const bf16x8 a = (kb & 1) ? cvt8(u32x2{w[2], w[3]}) : cvt8(u32x2{w[0], w[1]});
    if ((kb & 1) && j + kPre < 18) cf[j % kPre] = *(const LDSP u32x4*)(ap + 32 * (j + kPre));
    if (kb == 0)
      asm volatile("s_nop 1\n v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(S) : "v"(a), "a"(qf[0]));
    else
      asm volatile("s_nop 1\n v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(S) : "v"(a), "a"(qf[kb]));
  }
  asm volatile("s_nop 7\n s_nop 7\n s_nop 3" ::: "memory");       // MFMA result -> VALU
  return S;
}

// Two page buffers, the P^T tile and the exchange area are separate LDS
// objects: with every buffer reference static, the compiler can tell the
// next page's direct loads never alias the current page's reads and adds no
// waits of its own.
__shared__ __attribute__((aligned(1024))) char g_page0[kPageB];
__shared__ __attribute__((aligned(1024))) char g_page1[kPageB];
__shared__ __attribute__((aligned(16))) char g_pt[64 * kPtRowB];
__shared__ __attribute__((aligned(16))) float g_xm[2 * 64];   // page max per token half
__shared__ __attribute__((aligned(16))) float g_xa[64];       // alpha per head
__shared__ __attribute__((aligned(16))) float g_xl[2 * 64];   // row sums per token half
__shared__ __attribute__((aligned(16))) float g_xf[64];       // final reference max
__shared__ int32_t g_lens[256];                               // seq_lens, when the batch has <= 256
__shared__ __attribute__((aligned(16))) int32_t g_xneed[4];   // per wave: its page half needs a new reference

struct Lane {                      // per-lane constants
  int wave, lane, l32, hi, hb, th;
  int a_off, pt_row, tr_off;
};

struct Acc {                       // per-segment running state of one wave
  f32x16 o[4][2];
  float m_ref, l_own;
};

// One page: the next page's loads, QK, softmax, PV.
// buf (read) and nbuf (direct-load target) are __restrict__: the compiler
// then knows the in-flight loads into nbuf never alias reads of buf and adds
// no waits of its own (the explicit vmcnt + barrier at the top orders them).
//
// The buffers hold code rows of 592 B and the page's scales; both
// contractions convert their fragments in registers, and the per-token scale
// s_t multiplies the scores and P (row = s_t * codes).
__device__ __forceinline__ void page_step(const Lane& ln, LDSP char* __restrict__ buf,
                                          LDSP char* __restrict__ nbuf,
                                          bool dma, const char* cbase, const int32_t* bt_after,
                                          int32_t& pg_after, const bf16x8 (&qf)[36], int nvalid, int lo,
                                          float s2, Acc& acc, const char* sbase) {
  LDSP char* pt = (LDSP char*)g_pt;
  float* xm = g_xm;
  float* xa = g_xa;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();                                               // this page landed; previous one consumed
  asm volatile("" : "+v"(pg_after));                             // its load (one page ago) has landed
  const char* nsrc_u = uniform(cbase + (int64_t)pg_after * kCodePageB);   // next page
  const uint32_t nbuf_u = uniform_lds(nbuf);
  const int32_t pg2 = bt_after ? *bt_after : 0;                  // page id two ahead, read during this page

  if (dma)                                                        // next page's codes and scales, now
    dma_code_page(nsrc_u, nbuf_u, sbase + (int64_t)pg_after * (kBs * 4), nbuf + kCodeRowsB, ln.wave, ln.lane);

  f32x16 S = qk_page_e4m3(buf + ln.a_off, qf);

  // E4M3: score_t = s_t (q . codes_t); the scale of a masked row is taken
  // as 0 so that whatever its slot holds cannot reach P.
  float sct[16];
  {
    const LDSP float* sc = (const LDSP float*)(buf + kCodeRowsB);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ra = r >> 2;
      const int t = 32 * ln.th + 16 * (ra >> 1) + 2 * (ra & 1) + ln.hi + 4 * (r & 3);
      sct[r] = (t >= nvalid || t < lo) ? 0.f : sc[t];
      S[r] *= sct[r];
    }
  }

  // Scores stay raw (s2 > 0 commutes with the maximum); rows past the end of
  // the sequence, and rows before the start of its window, are -inf.  P below
  // is exp2(S s2 - m) in one fma per score.
  if (nvalid < kBs || lo > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ra = r >> 2;
      const int t = 32 * ln.th + 16 * (ra >> 1) + 2 * (ra & 1) + ln.hi + 4 * (r & 3);
      if (t >= nvalid || t < lo) S[r] = -INFINITY;
    }
  }
  float mloc = fmaxf(fmaxf(fmaxf(S[0], S[1]), fmaxf(S[2], S[3])), fmaxf(fmaxf(S[4], S[5]), fmaxf(S[6], S[7])));
  mloc = fmaxf(mloc, fmaxf(fmaxf(fmaxf(S[8], S[9]), fmaxf(S[10], S[11])),
                           fmaxf(fmaxf(S[12], S[13]), fmaxf(S[14], S[15]))));
  mloc = max_xor32(mloc) * s2;
  if (ln.hi == 0) xm[ln.th * 64 + ln.hb * 32 + ln.l32] = mloc;
  // Optimistic P: computed with the current reference maximum.  Only if some
  // token half of the page exceeds it by more than 2^tau (always on a
  // segment's first page, rarely after) do all waves redo P below with the
  // page maximum, exactly as the lazy rule prescribes; the common page thus
  // needs one barrier between QK and PV instead of two.
  const int need = __any(mloc > acc.m_ref + kTau);
  if (ln.lane == 0) g_xneed[ln.wave] = need;
  float ps = 0.f;
  // P^T slot order: within each 16-token k-step, slot 8 h + e holds token
  // 2 e + h, so that the transposed V reads of one lane half touch rows of one
  // parity (conflict-free banks, see tr_off).  Score register r is token
  // 16 (r >> 3) + 2 ((r >> 2) & 1) + hi + 4 (r & 3) of the wave's half, so a
  // lane's 8 registers 8 kb .. 8 kb + 7 fill slots 8 hi .. 8 hi + 7 of k-step
  // 2 th + kb in the order r = 8 kb + {0, 4, 1, 5, 2, 6, 3, 7}: one 16-B write.
  auto make_p = [&]() {
    ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      uint32_t pk[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r0 = 8 * kb + q, r1 = r0 + 4;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r0], s2, -acc.m_ref));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r1], s2, -acc.m_ref));
        ps += p0 + p1;
        pk[q] = pack2_bf16(p0 * sct[r0], p1 * sct[r1]);
      }
      const int slot = 16 * (2 * ln.th + kb) + 8 * ln.hi;
      *(LDSP u32x4*)(pt + ln.pt_row + slot * 2) = u32x4{pk[0], pk[1], pk[2], pk[3]};
    }
  };
  make_p();
  if (nvalid < kBs || lo > 0) {                                  // masked rows: zero the latent codes
    for (int i = threadIdx.x; i < (kBs - nvalid + lo) * 32; i += 256) {
      const int k = i >> 5, ch = i & 31;
      const int row = k < lo ? k : nvalid + (k - lo);
      *(LDSP u32x4*)(buf + row * kRowC + ch * 16) = u32x4{0u, 0u, 0u, 0u};
    }
  }
  barrier_lds();                                                 // P^T, page maxima and flags visible
  // The flags and the first PV operands in one LDS round trip: the flags are
  // read first (LDS reads return in order), V^T and P^T of step 0 behind them.
  const LDSP char* vbase = buf + ln.tr_off;
  auto pload = [&](int ks, int h2) {
    return *(const LDSP bf16x8*)(pt + (32 * h2 + ln.l32) * kPtRowB + (16 * ks + 8 * ln.hi) * 2);
  };
  auto vraw = [&](int step) {            // V^T by transposed byte reads
    const int ks = step >> 2, cb = step & 3;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                         (LDSP i32x2*)(vbase + 16 * ks * kRowC + 32 * cb)));
  };
  const u32x4 flags = *(const LDSP u32x4*)g_xneed;
  u32x2 rcur = vraw(0);
  bf16x8 pc0 = pload(0, 0), pc1 = pload(0, 1);
  const bool slow = (flags[0] | flags[1] | flags[2] | flags[3]) != 0;
  float alpha = 1.f;
  if (slow) {
    const float mpage = fmaxf(mloc, xm[(1 - ln.th) * 64 + ln.hb * 32 + ln.l32]);
    if (mpage > acc.m_ref + kTau) {
      alpha = __builtin_amdgcn_exp2f(acc.m_ref - mpage);
      acc.m_ref = mpage;
    }
    make_p();
    if (ln.th == 0 && ln.hi == 0) xa[ln.hb * 32 + ln.l32] = alpha;
    barrier_lds();                                               // P^T and alpha visible
    pc0 = pload(0, 0);                                           // P^T was rewritten
    pc1 = pload(0, 1);
  }
  acc.l_own = acc.l_own * alpha + ps;

  // ---- PV: 16 steps (k-step ks, column block cb), one step of prefetch ------
  const float al0 = slow ? xa[ln.l32] : 1.f, al1 = slow ? xa[32 + ln.l32] : 1.f;
  if (slow && __any(al0 != 1.f || al1 != 1.f)) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) { acc.o[cb][0][r] *= al0; acc.o[cb][1][r] *= al1; }
    asm volatile("s_nop 2" ::: "memory");                        // VALU -> MFMA source
  }
  {                                      // V^T converted before each MFMA pair
    bf16x8 pn0 = pc0, pn1 = pc1;
#pragma unroll
    for (int step = 0; step < 16; ++step) {
      const int cb = step & 3;
      u32x2 rnext = rcur;
      if (step + 1 < 16) rnext = vraw(step + 1);
      if (cb == 0 && step + 4 < 16) { pn0 = pload((step >> 2) + 1, 0); pn1 = pload((step >> 2) + 1, 1); }
      const bf16x8 v = cvt8(rcur);
      asm volatile("s_nop 1\n v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n"
                   "v_mfma_f32_32x32x16_bf16 %1, %2, %4, %1"
                   : "+v"(acc.o[cb][0]), "+v"(acc.o[cb][1]) : "v"(v), "v"(pc0), "v"(pc1));
      rcur = rnext;
      if (cb == 3) { pc0 = pn0; pc1 = pn1; }
    }
  }
  pg_after = pg2;
}

__global__ void __launch_bounds__(256, 1) decode_e4m3_h64(
    int32_t B, int32_t n_h, int32_t W, int32_t HG, float s2,
    const uint16_t* __restrict__ q_abs, const void* __restrict__ cache, const float* __restrict__ kv_scale,
    const int32_t* __restrict__ block_table, int32_t max_pages, int32_t bt_div,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ seq_starts, float* __restrict__ ws_o,
    float* __restrict__ ws_lse, int64_t* __restrict__ ws_tbl, uint16_t* __restrict__ o_lat,
    float* __restrict__ lse) {
  Lane ln;
  const int tid = threadIdx.x;
  ln.lane = tid & 63;
  ln.wave = __builtin_amdgcn_readfirstlane(tid >> 6);          // uniform within the wave
  ln.l32 = ln.lane & 31;
  ln.hi = ln.lane >> 5;
  ln.hb = ln.wave & 1;
  ln.th = ln.wave >> 1;

  // Workgroup i runs on XCD i % 8.  XCD x takes the contiguous parts
  // [x ppx, (x+1) ppx) with all their head groups, so the two head groups of
  // a part read each page through the same L2, and the parts of one sequence
  // (which share its query rows) mostly sit on one XCD.
  const int ppx = (W + 7) / 8;
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int hg = j % HG;
  const int part = xcd * ppx + j / HG;
  if (part >= W) return;

  // QK A operand: lane reads token row tok(l32) of its half, 16-B chunk hi of each k-step
  {
    const int i = ln.l32, a = i >> 3, q = i & 3, bq = (i >> 2) & 1;
    const int tok = 32 * ln.th + 16 * (a >> 1) + 2 * (a & 1) + bq + 4 * q;
    ln.a_off = tok * kRowC + ln.hi * 16;
  }
  ln.pt_row = (ln.hb * 32 + ln.l32) * kPtRowB;
  {
    // PV transposed byte reads: within a 16-lane group, source lane sg names
    // token row T(sg / 2) and the 8 codes at column 16 (g & 1) + 8 (sg & 1)
    // of the wave's block; lane s then receives column 16 (g & 1) + s of
    // rows T(0..7), the token order of the P^T slots 8 hi .. 8 hi + 7:
    // T(e) = 2 e + hi.  Rows of one parity, 592 B = 148 banks apart, start
    // 8 banks apart modulo 64, so the two 16-lane groups of a lane half
    // (columns 0-15 and 16-31, 4 banks apart) cover the 64 banks once.
    const int g = ln.lane >> 4, sg = ln.lane & 15, e = sg >> 1;
    ln.tr_off = (2 * e + ln.hi) * kRowC + 128 * ln.wave + 16 * (g & 1) + 8 * (sg & 1);
  }

  // (these do not depend on the part: computed while the locator's load is in flight)
  uint32_t offa[19];                                             // this lane's query-load offsets (AGPRs)
  dma_offsets(ln.wave, ln.lane, offa);
  const int ndma = dma_count(ln.wave);

  const PartRange pr = locate_part(seq_lens, seq_starts, B, kBs, part, W, g_lens);
  const int32_t chunk = pr.chunk;
  auto seq_len = [&](int32_t bb) { return chunk == 1 ? g_lens[bb] : seq_lens[bb]; };
  const int64_t x1 = pr.x1;
  int64_t x = pr.x0;
  if (x >= x1) return;
  int32_t b = pr.b;
  int64_t first = pr.first;
  const char* cbase = reinterpret_cast<const char*>(cache);
  const char* sbase = reinterpret_cast<const char*>(kv_scale);

  for (;;) {
    // The window [st, L) of sequence b: its pages start at page fp; L and the
    // page indices below count from there, and the first lo rows of that
    // page lie before the window.
    const int32_t st = seq_start(seq_starts, b);
    const int32_t fp = st / kBs, lo = st - fp * kBs;
    const int32_t L = seq_len(b) - fp * kBs;
    const int64_t np = window_pages(seq_len(b), st, kBs);
    const int64_t jp0 = x - first;
    const int64_t jp1 = min(np, jp0 + (x1 - x));
    const int32_t* bt = block_table + (int64_t)(b / bt_div) * max_pages + fp;   // bt_div sequences per row
    if (jp0 == 0 && hg == 0 && threadIdx.x < 4) {                // the merge's part range of sequence b
      const int64_t v[4] = {part, part_of_page(first + np - 1, pr.P, W), np, pr.P};
      ws_tbl[4 * (int64_t)b + threadIdx.x] = v[threadIdx.x];
    }

    // First page into buffer 0 and this head group's 64 absorbed query rows
    // (contiguous in q_abs, 64 x 1152 B) into buffer 1, both by 1 KiB direct
    // loads (the page by its own walk).
    int32_t pg0, pg_next;
    Acc acc;                                                     // cleared while the first loads are in flight
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc.o[cb][h2][r] = 0.f;
    acc.m_ref = -INFINITY;
    acc.l_own = 0.f;
    {                                                            // queries first: they need no page id
      const char* qsrc_u = uniform(reinterpret_cast<const char*>(q_abs + ((int64_t)b * n_h + (int64_t)hg * 64) * kD));
      const uint32_t q_m0 = uniform_lds((LDSP char*)g_page1);
#pragma unroll
      for (int i = 0; i < 19; ++i)
        if (i < ndma) dma16_u(qsrc_u, offa[i], q_m0 + 1024 * (ln.wave + 4 * i));
      // ids of the first two pages in one round trip (the second is read only
      // when the segment has it)
      sload2_i32(bt + jp0, bt + (jp0 + 1 < jp1 ? jp0 + 1 : jp0), &pg0, &pg_next);
      const char* src_u = uniform(cbase + (int64_t)pg0 * kCodePageB);
      dma_code_page(src_u, uniform_lds((LDSP char*)g_page0), sbase + (int64_t)pg0 * (kBs * 4),
                    (LDSP char*)g_page0 + kCodeRowsB, ln.wave, ln.lane);
    }
    // Wait for this wave's query loads only (issued before the page's, and
    // direct loads complete in order): the first page keeps landing while
    // the queries are read into registers; its own wait is at the page top.
    if (ln.wave == 0) asm volatile("s_waitcnt vmcnt(11)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    barrier_lds();
    // Q^T fragments stay in AGPRs for the whole segment (the MFMAs read them there)
    bf16x8 qf[36];
    {
      const LDSP char* qrow = (LDSP char*)g_page1 + (ln.hb * 32 + ln.l32) * kRowB;
      bf16x8 t[36];
#pragma unroll
      for (int kb = 0; kb < 36; ++kb)               // contraction order of qk_page_e4m3
        t[kb] = *(const LDSP bf16x8*)(qrow + 64 * (kb >> 1) + 32 * ln.hi + 16 * (kb & 1));
#pragma unroll
      for (int kb = 0; kb < 36; ++kb) asm volatile("" : "=a"(qf[kb]) : "0"(t[kb]));
    }
    barrier_lds();                                               // buffer 1 free again (page 0 may still land)


    // Page indices are wave-uniform 32-bit values (SGPRs): the loop control
    // costs scalar instructions only.
    const int32_t j0 = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(jp0));
    const int32_t j1 = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(jp1));
    const int32_t Lu = __builtin_amdgcn_readfirstlane(L);
    for (int32_t jp = j0; jp < j1; ++jp) {
      const bool even = ((jp - j0) & 1) == 0;
      LDSP char* buf = even ? (LDSP char*)g_page0 : (LDSP char*)g_page1;
      LDSP char* nbuf = even ? (LDSP char*)g_page1 : (LDSP char*)g_page0;
      const int nvalid = min(kBs, Lu - jp * kBs);                 // jp * 64 < L: no overflow
      const bool more = jp + 1 < j1;
      page_step(ln, buf, nbuf, more, cbase, jp + 2 < j1 ? bt + jp + 2 : nullptr, pg_next, qf, nvalid,
                jp == 0 ? lo : 0, s2, acc, sbase);
    }

    // ---- segment epilogue: normalise and store ------------------------------
    asm volatile("s_nop 7\n s_nop 7\n s_nop 3" ::: "memory");   // MFMA result -> VALU
    __syncthreads();
    const float l_lane = sum_xor32(acc.l_own);
    if (ln.hi == 0) {
      g_xl[ln.th * 64 + ln.hb * 32 + ln.l32] = l_lane;
      if (ln.th == 0) g_xf[ln.hb * 32 + ln.l32] = acc.m_ref;
    }
    __syncthreads();
    const bool whole = (jp0 == 0 && jp1 == np);
    float inv[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int hh = h2 * 32 + ln.l32;
      const float lt = g_xl[hh] + g_xl[64 + hh];
      inv[h2] = 1.f / lt;
      const float lse_v = (g_xf[hh] + __log2f(lt)) * 0.69314718055994531f;
      const int64_t head = (int64_t)hg * 64 + hh;
      if (ln.wave == 0 && ln.hi == 0) {
        if (whole) { if (lse) lse[(int64_t)b * n_h + head] = lse_v; }
        else __builtin_nontemporal_store(lse_v, ws_lse + ((int64_t)part + b) * n_h + head);
      }
    }
    if (whole) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int col = 128 * ln.wave + 32 * cb + 8 * q4 + 4 * ln.hi;
            const f32x16& o = acc.o[cb][h2];
            *reinterpret_cast<u32x2*>(o_lat + ((int64_t)b * n_h + (int64_t)hg * 64 + h2 * 32 + ln.l32) * kDc + col) =
                u32x2{pack2_bf16(o[4 * q4] * inv[h2], o[4 * q4 + 1] * inv[h2]),
                      pack2_bf16(o[4 * q4 + 2] * inv[h2], o[4 * q4 + 3] * inv[h2])};
          }
    } else {                                                     // bf16 partial, quad (w*4+cb)*4+q4: 64 lanes x 16 B
      uint16_t* wp = reinterpret_cast<uint16_t*>(ws_o) + (((int64_t)part + b) * n_h + (int64_t)hg * 64) * kDc +
                     ln.lane * 8;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x16& o0 = acc.o[cb][0];
          const f32x16& o1 = acc.o[cb][1];
          __builtin_nontemporal_store(u32x4{pack2_bf16(o0[4 * q4] * inv[0], o0[4 * q4 + 1] * inv[0]),
                                            pack2_bf16(o0[4 * q4 + 2] * inv[0], o0[4 * q4 + 3] * inv[0]),
                                            pack2_bf16(o1[4 * q4] * inv[1], o1[4 * q4 + 1] * inv[1]),
                                            pack2_bf16(o1[4 * q4 + 2] * inv[1], o1[4 * q4 + 3] * inv[1])},
                                      reinterpret_cast<u32x4*>(wp + ((ln.wave * 4 + cb) * 4 + q4) * 512));
        }
    }

    x += jp1 - jp0;
    if (x >= x1) break;
    do { ++b; } while (window_pages(seq_len(b), seq_start(seq_starts, b), kBs) == 0);
    first = x;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Merge of the split-KV partials of decode_e4m3_h64.  A partial (slot, 64-head
// group) is 64 KiB of bfloat16 in register order: quad (w*4 + cb)*4 + q4
// holds, for lane l, 16 B: latent columns 128w + 32cb + 8q4 + 4(l/32) .. +3
// of head l%32, then the same columns of head 32 + l%32, already divided by
// the partial's own row sum; its log-sum-exp (float32) is in ws_lse.
// Workgroup = (sequence, head group, wave-column block w*4+cb); thread
// (q4, l) owns one 16-B chunk of each partial.  Parts are merged with a
// running maximum, a batch of loads in flight at once and no LDS or barrier
// after the page count:
//   o_lat = sum_k e^(lse_k - M) o_k / sum_k e^(lse_k - M),  lse = M + ln(sum).
// ---------------------------------------------------------------------------
// Parts are merged kN at a time (2, 4 or 8 by the sequence's part count, so
// that a sequence split in two or four parts issues no loads beyond its
// parts), all kN loads of a batch in flight together; each thread carries
// two heads (l32 and 32 + l32).
struct MergeState2 {
  f32x4 acc0, acc1;
  float m0, m1, d0, d1;
};

template <int kN>
__device__ __forceinline__ void merge_parts(MergeState2& st, int64_t w0, int64_t w1, int32_t b, int hg, int64_t P,
                                            int32_t W, bool all_live, const uint16_t* __restrict__ ws16, int off,
                                            const float* __restrict__ ws_lse, int32_t n_h, int l32) {
  for (int64_t base = w0; base <= w1; base += kN) {
    f32x4 v0[kN], v1[kN];
    float e0[kN], e1[kN];
#pragma unroll
    for (int jj = 0; jj < kN; ++jj) {              // part w0 always holds a page: dead parts read it
      const int64_t w = base + jj;
      const bool live = w <= w1 && (all_live || part_start(w, P, W) < part_start(w + 1, P, W));
      const int64_t slot = (live ? w : w0) + b;
      const u32x4 raw = *reinterpret_cast<const u32x4*>(ws16 + (slot * n_h + (int64_t)hg * 64) * kDc + off);
      v0[jj] = f32x4{__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                     __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
      v1[jj] = f32x4{__uint_as_float(raw.z << 16), __uint_as_float(raw.z & 0xffff0000u),
                     __uint_as_float(raw.w << 16), __uint_as_float(raw.w & 0xffff0000u)};
      const float* ls = ws_lse + slot * n_h + (int64_t)hg * 64;
      e0[jj] = live ? ls[l32] : -INFINITY;
      e1[jj] = live ? ls[32 + l32] : -INFINITY;
    }
    float n0 = st.m0, n1 = st.m1;
#pragma unroll
    for (int jj = 0; jj < kN; ++jj) { n0 = fmaxf(n0, e0[jj]); n1 = fmaxf(n1, e1[jj]); }
    const float a0 = n0 == st.m0 ? 1.f : __expf(st.m0 - n0), a1 = n1 == st.m1 ? 1.f : __expf(st.m1 - n1);
    st.acc0 *= a0; st.d0 *= a0; st.m0 = n0;
    st.acc1 *= a1; st.d1 *= a1; st.m1 = n1;
#pragma unroll
    for (int jj = 0; jj < kN; ++jj) {
      const float x0 = e0[jj] == -INFINITY ? 0.f : __expf(e0[jj] - st.m0);
      const float x1 = e1[jj] == -INFINITY ? 0.f : __expf(e1[jj] - st.m1);
      st.d0 += x0; st.d1 += x1;
      st.acc0 += x0 * v0[jj];
      st.acc1 += x1 * v1[jj];
    }
  }
}

// One (sequence b, head group hg, wave-column block wc) of the merge.
__device__ __forceinline__ void combine_item(int32_t b, int hg, int wc, int32_t n_h, int32_t W, int64_t P,
                                             int64_t np, int64_t w0, int64_t w1, const float* __restrict__ ws_o,
                                             const float* __restrict__ ws_lse, uint16_t* __restrict__ o_lat,
                                             float* __restrict__ lse) {
  const int tid = threadIdx.x, lane = tid & 63, q4 = tid >> 6, l32 = lane & 31;
  const int64_t head0 = (int64_t)b * n_h + (int64_t)hg * 64;
  const int col0 = 128 * (wc >> 2) + 32 * (wc & 3);
  if (np == 0) {                                   // empty sequence: zero output, lse = -inf
    for (int i = tid; i < 64 * 8; i += 256) {
      const int hh = i >> 3, c4 = i & 7;
      *reinterpret_cast<u32x2*>(o_lat + (head0 + hh) * kDc + col0 + 4 * c4) = u32x2{0u, 0u};
    }
    if (wc == 0 && tid < 64 && lse) lse[head0 + tid] = -INFINITY;
    return;
  }
  if (w0 == w1) return;                            // one part: written by the decode kernel

  const bool all_live = P >= W;                    // every part holds a page unless parts outnumber pages
  const int off = (wc * 4 + q4) * 512 + lane * 8;
  const uint16_t* ws16 = reinterpret_cast<const uint16_t*>(ws_o);
  MergeState2 st{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, -INFINITY, -INFINITY, 0.f, 0.f};
  const int64_t nparts = w1 - w0 + 1;              // the same for the whole workgroup
  if (nparts <= 2) merge_parts<2>(st, w0, w1, b, hg, P, W, all_live, ws16, off, ws_lse, n_h, l32);
  else if (nparts <= 4) merge_parts<4>(st, w0, w1, b, hg, P, W, all_live, ws16, off, ws_lse, n_h, l32);
  else merge_parts<8>(st, w0, w1, b, hg, P, W, all_live, ws16, off, ws_lse, n_h, l32);
  const f32x4 acc0 = st.acc0, acc1 = st.acc1;
  const float m0 = st.m0, m1 = st.m1, d0 = st.d0, d1 = st.d1;
  const int col = col0 + 8 * q4 + 4 * (lane >> 5);
  const float i0 = 1.f / d0, i1 = 1.f / d1;
  *reinterpret_cast<u32x2*>(o_lat + (head0 + l32) * kDc + col) =
      u32x2{pack2_bf16(acc0[0] * i0, acc0[1] * i0), pack2_bf16(acc0[2] * i0, acc0[3] * i0)};
  *reinterpret_cast<u32x2*>(o_lat + (head0 + 32 + l32) * kDc + col) =
      u32x2{pack2_bf16(acc1[0] * i1, acc1[1] * i1), pack2_bf16(acc1[2] * i1, acc1[3] * i1)};
  if (wc == 0 && tid < 32 && lse) {
    lse[head0 + l32] = m0 + __logf(d0);
    lse[head0 + 32 + l32] = m1 + __logf(d1);
  }
}

// One workgroup per (sequence, head group, wave-column block); the
// sequence's part range comes from the decode kernel (ws_tbl).  (Placing each workgroup on the XCD
// whose L2 the partials were written through measured no faster than this
// plain order once the search it needed was counted.)
__global__ void __launch_bounds__(256) combine_h64(int32_t B, int32_t n_h, int32_t W, int32_t HG,
                                                   const int32_t* __restrict__ seq_lens,
                                                   const int32_t* __restrict__ seq_starts,
                                                   const float* __restrict__ ws_o,
                                                   const float* __restrict__ ws_lse,
                                                   const int64_t* __restrict__ ws_tbl,
                                                   uint16_t* __restrict__ o_lat, float* __restrict__ lse) {
  const int per_seq = HG * 16;
  const int32_t b = blockIdx.x / per_seq;
  const int r = blockIdx.x % per_seq;
  // A sequence with pages has its part range in ws_tbl (written by the decode
  // workgroup that took its first page); an empty one is known from its length.
  const int64_t np = window_pages(seq_lens[b], seq_start(seq_starts, b), kBs);
  const int64_t w0 = np > 0 ? ws_tbl[4 * (int64_t)b] : 0;
  const int64_t w1 = np > 0 ? ws_tbl[4 * (int64_t)b + 1] : 0;
  const int64_t P = np > 0 ? ws_tbl[4 * (int64_t)b + 3] : 0;
  combine_item(b, r / 16, r % 16, n_h, W, P, np, w0, w1, ws_o, ws_lse, o_lat, lse);
}

}  // namespace

bool e4m3_h64_decode_supported(const mla_dims& d) {
  return d.act_dtype == MLA_BF16 && d.kv_dtype == MLA_E4M3 && d.d_latent == kDc && d.d_rope == 64 &&
         d.block_size == kBs && d.n_heads % 64 == 0;
}

hipError_t launch_decode_e4m3_h64(const mla_dims& d, const DecodePlan& plan, int32_t B,
                                  const void* q_abs, const void* cache, const float* kv_scale,
                                  const int32_t* block_table, int32_t max_pages, int32_t bt_div,
                                  const int32_t* seq_lens, const int32_t* seq_starts, float* ws_o,
                                  float* ws_lse, int64_t* ws_tbl, void* o_lat, float* lse, hipStream_t s) {
  const int HG = d.n_heads / 64;
  const int W = plan.parts;
  const int grid = ((W + 7) / 8) * 8 * HG;                  // 8 XCDs x ceil(W/8) parts x HG
  const float s2 = d.softmax_scale * 1.4426950408889634f;
  decode_e4m3_h64<<<grid, 256, 0, s>>>(B, d.n_heads, W, HG, s2, static_cast<const uint16_t*>(q_abs), cache,
                                       kv_scale, block_table, max_pages, bt_div, seq_lens, seq_starts, ws_o,
                                       ws_lse, ws_tbl, static_cast<uint16_t*>(o_lat), lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  combine_h64<<<B * HG * 16, 256, 0, s>>>(B, d.n_heads, W, HG, seq_lens, seq_starts, ws_o, ws_lse, ws_tbl,
                                          static_cast<uint16_t*>(o_lat), lse);
  return hipGetLastError();
}

}  // namespace mla
