// Device helpers shared by the library's kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

namespace mla {

// ---- storage types ---------------------------------------------------------
struct bf16_t { uint16_t bits; };
struct e4m3_t { uint8_t bits; };

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// float32 -> bfloat16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two floats -> packed bfloat16 pair (low half = a), round to nearest even,
// by the hardware conversion (one instruction).
typedef __bf16 mla_bf16x2 __attribute__((ext_vector_type(2)));
typedef float mla_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((mla_f32x2){a, b}, mla_bf16x2));
}

// Reductions across lanes l, l ^ 32 (and l ^ 16) of a wave without going
// through LDS: the lane-swap instructions exchange the 32-lane halves (the
// odd and even 16-lane rows) of two registers; with both operands equal, the
// two results hold each lane's value and its partner's.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// E4M3 (OCP): exponent bias 7, 3 mantissa bits, subnormals m * 2^-9, max 448.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t s = (c >> 7) & 1u, e = (c >> 3) & 0xFu, m = c & 7u;
  float mag = (e == 0) ? static_cast<float>(m) * 0.001953125f  // m * 2^-9
                       : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return s ? -mag : mag;
}
// float32 -> E4M3 code: nearest, ties to even, saturating at +-448.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  uint32_t u = __float_as_uint(y);
  uint32_t sign = (u >> 31) << 7;
  uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E00000u) {                 // |y| >= 448
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {           // |y| < 2^-6: subnormal grid of step 2^-9
    float m = __builtin_rintf(__uint_as_float(a) * 512.0f);   // exact scaling, RNE
    code = static_cast<uint32_t>(m);      // m == 8 is the smallest normal, code 0x08
  } else {
    uint32_t q = a >> 20;                 // exponent and top 3 mantissa bits
    uint32_t rem = a & 0xFFFFFu;
    q += (rem > 0x80000u) || (rem == 0x80000u && (q & 1u));
    code = q - (120u << 3);               // rebias 127 -> 7
    if (code > 0x7Eu) code = 0x7Eu;       // rounding up past 448 saturates
  }
  return code | sign;
}

template <typename T> struct io;
template <> struct io<float> {
  __device__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct io<bf16_t> {
  __device__ static float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i].bits); }
  __device__ static void store(bf16_t* p, int64_t i, float v) { p[i].bits = f32_to_bf16(v); }
};

// RoPE of one pair (x0, x1) at position pos, frequency index i of d_rope/2:
// angle = pos * base^(-2i/d_rope), with the frequency formed as
// 2^(-(2i/d_rope) log2(base)) (the caller passes log2(base), computed once on
// the host); angle, sine, cosine and rotation in float64 without
// contraction, result rounded to float32.
__device__ __forceinline__ void rope_angle(int32_t pos, int i, int d_rope, double log2_base, double* c, double* s) {
#pragma clang fp contract(off)
  const double inv = exp2(-(2.0 * static_cast<double>(i) / static_cast<double>(d_rope)) * log2_base);
  const double ang = static_cast<double>(pos) * inv;
  sincos(ang, s, c);
}
__device__ __forceinline__ void rope_rotate(float x0, float x1, double c, double s, float* y0, float* y1) {
#pragma clang fp contract(off)
  const double a = static_cast<double>(x0), b = static_cast<double>(x1);
  const double r0 = a * c - b * s;
  const double r1 = a * s + b * c;
  *y0 = static_cast<float>(r0);
  *y1 = static_cast<float>(r1);
}
__device__ __forceinline__ void rope_pair(float x0, float x1, int32_t pos, int i, int d_rope,
                                          double log2_base, float* y0, float* y1) {
  double c, s;
  rope_angle(pos, i, d_rope, log2_base, &c, &s);
  rope_rotate(x0, x1, c, s, y0, y1);
}

// Workgroup barrier that waits only for this wave's LDS operations.  Direct
// global->LDS loads (counted by vmcnt) stay in flight across it; whoever reads
// their destination waits with an explicit vmcnt before its own barrier.
// (__syncthreads() would also wait for every such load to land.)
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Direct global -> LDS loads (LDS address = M0 + size * lane), issued from
// inline asm so that the compiler adds no waits of its own for them: every
// reader waits with an explicit vmcnt and a barrier.
__device__ __forceinline__ const char* uniform(const char* p) {   // wave-uniform pointer into SGPRs
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ void dma16(const char* base, uint32_t voff, const __attribute__((address_space(3))) void* dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst)));
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" :: "s"(m0), "v"(voff), "s"(uniform(base)) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const char* base, uint32_t voff, const __attribute__((address_space(3))) void* dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst)));
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" :: "s"(m0), "v"(voff), "s"(uniform(base)) : "memory", "m0");
}

// The same with a source base and an LDS address the caller has already made
// wave-uniform (SGPRs), so each load costs no extra scalar moves.
__device__ __forceinline__ void dma16_u(const char* ubase, uint32_t voff, uint32_t um0) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" :: "s"(um0), "v"(voff), "s"(ubase) : "memory", "m0");
}
__device__ __forceinline__ uint32_t uniform_lds(const __attribute__((address_space(3))) void* p) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p)));
}

// Scalar load of one int32 at a wave-uniform address; waits for itself (the
// wait covers only scalar and LDS operations, never the vector loads in flight).
__device__ __forceinline__ int32_t sload_i32(const int32_t* p) {
  int32_t v;
  const char* u = uniform(reinterpret_cast<const char*>(p));
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(u) : "memory");
  return v;
}
// Three such loads in flight together.
__device__ __forceinline__ void sload3_i32(const int32_t* p, const int32_t* q, const int32_t* r, int32_t* a,
                                           int32_t* b, int32_t* c) {
  int32_t va, vb, vc;
  const char* up = uniform(reinterpret_cast<const char*>(p));
  const char* uq = uniform(reinterpret_cast<const char*>(q));
  const char* ur = uniform(reinterpret_cast<const char*>(r));
  asm volatile("s_load_dword %0, %3, 0x0\n\ts_load_dword %1, %4, 0x0\n\ts_load_dword %2, %5, 0x0\n\t"
               "s_waitcnt lgkmcnt(0)"
               : "=&s"(va), "=&s"(vb), "=&s"(vc) : "s"(up), "s"(uq), "s"(ur) : "memory");
  *a = va;
  *b = vb;
  *c = vc;
}
// Two such loads in flight together (one memory round trip for both).
__device__ __forceinline__ void sload2_i32(const int32_t* p, const int32_t* q, int32_t* a, int32_t* b) {
  int32_t va, vb;
  const char* up = uniform(reinterpret_cast<const char*>(p));
  const char* uq = uniform(reinterpret_cast<const char*>(q));
  asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
               : "=&s"(va), "=&s"(vb) : "s"(up), "s"(uq) : "memory");
  *a = va;
  *b = vb;
}

// ---- split-KV schedule -----------------------------------------------------
// The batch's pages are flattened in sequence order (sequence b owns the
// pages of its window, see window_pages below) and cut into `parts` contiguous
// ranges: part w covers [floor(w P / W), floor((w+1) P / W)).  A (part,
// sequence) overlap is a segment; its partial result lives in slot w + b.
// floor(a / b) for 0 <= a < 2^53 and 1 <= b < 2^31: the float64 quotient is
// within one of it and is corrected to the exact value (cheaper than the
// 64-bit integer division routine).
__device__ __forceinline__ int64_t div_floor53(int64_t a, int64_t b) {
  int64_t q = static_cast<int64_t>(static_cast<double>(a) / static_cast<double>(b));
  if (q * b > a) --q;
  else if ((q + 1) * b <= a) ++q;
  return q;
}
// (W <= 65536 parts, P < 2^31 pages: every product below stays under 2^48)
__device__ __forceinline__ int64_t part_start(int64_t w, int64_t P, int64_t W) { return div_floor53(w * P, W); }
__device__ __forceinline__ int64_t part_of_page(int64_t x, int64_t P, int64_t W) {
  return div_floor53((x + 1) * W - 1, P);
}
__device__ __forceinline__ int32_t pages_of(int32_t L, int32_t bs) { return (L + bs - 1) / bs; }

// Sliding window: sequence b attends to its tokens [start_b, L_b) (start_b = 0
// when seq_starts is null).  Its pages in the flattened list are the pages
// from start_b / bs up to the one holding token L_b - 1; an empty window has
// none.
__device__ __forceinline__ int32_t seq_start(const int32_t* seq_starts, int32_t b) {
  return seq_starts ? seq_starts[b] : 0;
}
__device__ __forceinline__ int32_t window_pages(int32_t L, int32_t start, int32_t bs) {
  return start >= L ? 0 : pages_of(L, bs) - start / bs;
}

// Block-wide page prefix over sequences.  `scan` is __shared__ scratch of
// blockDim.x + 1 ints (blockDim.x a multiple of 64, at most 1024).  After the
// call scan[t] = pages of sequences before thread t's chunk
// [t*chunk, (t+1)*chunk) and scan[blockDim.x] = total P.  With one sequence
// per thread (chunk == 1) and lens_lds non-null, lens_lds[b] = seq_lens[b]
// for every b < B, so later lookups need not go back to global memory.
__device__ __forceinline__ void page_prefix(const int32_t* seq_lens, const int32_t* seq_starts, int32_t B,
                                            int32_t bs, int32_t* scan, int32_t* chunk_out,
                                            int32_t* lens_lds = nullptr) {
  __shared__ int32_t wave_tot[16];
  const int nt = blockDim.x, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int32_t chunk = (B + nt - 1) / nt;
  int32_t s = 0;
  if (chunk == 1) {
    const int32_t L = t < B ? seq_lens[t] : 0;
    if (lens_lds && t < B) lens_lds[t] = L;
    s = t < B ? window_pages(L, seq_start(seq_starts, t), bs) : 0;
  } else {
    for (int32_t b = t * chunk; b < min(B, (t + 1) * chunk); ++b)
      s += window_pages(seq_lens[b], seq_start(seq_starts, b), bs);
  }
  int32_t v = s;                         // inclusive scan inside the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63) wave_tot[wv] = v;
  __syncthreads();
  int32_t carry = 0;
  for (int w = 0; w < wv; ++w) carry += wave_tot[w];
  scan[t + 1] = v + carry;
  if (t == 0) scan[0] = 0;
  __syncthreads();
  *chunk_out = chunk;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts of
// 1, 2, 4 and 8 lanes inside each 16-lane row, then the last lane of row 0
// (row 2) added to row 1 (row 3) and the last lane of row 1 to rows 2 and 3.
__device__ __forceinline__ int32_t wave_incl_scan(int32_t v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 -> rows 2, 3
  return v;
}

// Maximum over the 64 lanes of a wave, returned in every lane: the DPP scan
// pattern of wave_incl_scan with max, then lane 63 read back.
__device__ __forceinline__ float wave_max_all(float x) {
  int v = __float_as_int(x);
  const int ninf = __float_as_int(-INFINITY);
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(ninf, v, 0x111, 0xf, 0xf, false))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(ninf, v, 0x112, 0xf, 0xf, false))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(ninf, v, 0x114, 0xf, 0xf, false))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(ninf, v, 0x118, 0xf, 0xf, false))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(ninf, v, 0x142, 0xa, 0xf, false))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(ninf, v, 0x143, 0xc, 0xf, false))));
  return __int_as_float(__builtin_amdgcn_readlane(v, 63));
}

// One 576-wide cache row (d_c = 512, d_R = 64) from bfloat16 inputs, written
// by one wave: lane l holds latent elements 8l..8l+7 (c, bf16 bits) and, for
// l < 32, the unrotated RoPE pair l (kp, two bf16) with the cosine and sine
// of its angle (rc, rs from rope_angle).  A bf16 cache receives
// the latent bits unchanged (bf16 -> float -> bf16 is exact) and the rotated
// pair rounded once; an E4M3 cache receives e4m3(x / s) with s = amax / 448
// over the whole row (1 for an all-zero row), s stored in kv_scale[slot].
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
template <bool kE4M3>
__device__ __forceinline__ void append_row_576_cs(u32x4_t c, uint32_t kp, double rc, double rs, int64_t sl,
                                                  void* cache, float* kv_scale, int lane) {
  constexpr int kDc = 512, kDr = 64, kD = 576;
  float y0 = 0.f, y1 = 0.f;
  if (lane < kDr / 2)
    rope_rotate(bf16_to_f32(static_cast<uint16_t>(kp & 0xFFFFu)), bf16_to_f32(static_cast<uint16_t>(kp >> 16)), rc, rs,
                &y0, &y1);
  if constexpr (!kE4M3) {
    uint16_t* dst = static_cast<uint16_t*>(cache) + sl * kD;
    *reinterpret_cast<u32x4_t*>(dst + 8 * lane) = c;
    if (lane < kDr / 2)
      *reinterpret_cast<uint32_t*>(dst + kDc + 2 * lane) =
          static_cast<uint32_t>(f32_to_bf16(y0)) | (static_cast<uint32_t>(f32_to_bf16(y1)) << 16);
  } else {
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(c[i] << 16);
      x[2 * i + 1] = __uint_as_float(c[i] & 0xFFFF0000u);
    }
    float amax = fmaxf(fabsf(y0), fabsf(y1));
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = wave_max_all(amax);
    const float sc = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    uint8_t* dst = static_cast<uint8_t*>(cache) + sl * kD;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= f32_to_e4m3(__fdiv_rn(x[i], sc)) << (8 * i);
      hi |= f32_to_e4m3(__fdiv_rn(x[4 + i], sc)) << (8 * i);
    }
    *reinterpret_cast<u32x2_t*>(dst + 8 * lane) = u32x2_t{lo, hi};
    if (lane < kDr / 2)
      *reinterpret_cast<uint16_t*>(dst + kDc + 2 * lane) =
          static_cast<uint16_t>(f32_to_e4m3(__fdiv_rn(y0, sc)) | (f32_to_e4m3(__fdiv_rn(y1, sc)) << 8));
    if (lane == 0) kv_scale[sl] = sc;
  }
}

// The same row with the RoPE angle computed here (lanes < 32, pair = lane).
template <bool kE4M3>
__device__ __forceinline__ void append_row_576(u32x4_t c, uint32_t kp, int32_t p, int64_t sl, void* cache,
                                               float* kv_scale, double log2_base, int lane) {
  double rc = 0.0, rs = 0.0;
  if (lane < 32) rope_angle(p, lane, 64, log2_base, &rc, &rs);
  append_row_576_cs<kE4M3>(c, kp, rc, rs, sl, cache, kv_scale, lane);
}

// The part of the split-KV schedule one workgroup needs, in two barriers and
// no search: the total page count P, the part's page range [x0, x1) and, when
// the part is not empty, the sequence b owning page x0 and that sequence's
// first flattened page.  Thread t sums the pages of sequences
// [t*chunk, (t+1)*chunk); the thread whose range holds x0 publishes it.  With
// one sequence per thread (chunk == 1) and lens_lds non-null, lens_lds[b] =
// seq_lens[b] for every b < B afterwards.  Must be called by the whole block.
struct PartRange {
  int64_t P, x0, x1, first;
  int32_t b, chunk;
};
__device__ __forceinline__ PartRange locate_part(const int32_t* seq_lens, const int32_t* seq_starts, int32_t B,
                                                 int32_t bs, int64_t part, int64_t W, int32_t* lens_lds) {
  __shared__ int32_t wave_tot[16];
  __shared__ int64_t owner[2];
  const int nt = blockDim.x, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  PartRange r;
  r.chunk = (B + nt - 1) / nt;
  int32_t s = 0;
  if (r.chunk == 1) {
    const int32_t L = t < B ? seq_lens[t] : 0;
    if (lens_lds && t < B) lens_lds[t] = L;
    s = t < B ? window_pages(L, seq_start(seq_starts, t), bs) : 0;
  } else {
    for (int32_t b = t * r.chunk; b < min(B, (t + 1) * r.chunk); ++b)
      s += window_pages(seq_lens[b], seq_start(seq_starts, b), bs);
  }
  const int32_t v = wave_incl_scan(s);
  if (lane == 63) wave_tot[wv] = v;
  __syncthreads();
  int64_t carry = 0, total = 0;
  for (int w = 0; w < nt / 64; ++w) {
    const int32_t c = wave_tot[w];
    carry += w < wv ? c : 0;
    total += c;
  }
  r.P = total;
  r.x0 = part_start(part, r.P, W);
  r.x1 = part_start(part + 1, r.P, W);
  const int64_t incl = carry + v, excl = incl - s;
  if (s > 0 && excl <= r.x0 && r.x0 < incl) {        // one thread when x0 < P
    owner[0] = t;
    owner[1] = excl;
  }
  __syncthreads();
  r.b = 0;
  r.first = 0;
  if (r.x0 < r.x1) {
    int32_t b = static_cast<int32_t>(owner[0]) * r.chunk;
    int64_t first = owner[1];
    if (r.chunk > 1) {
      for (;;) {
        const int32_t np = window_pages(seq_lens[b], seq_start(seq_starts, b), bs);
        if (r.x0 < first + np) break;
        first += np;
        ++b;
      }
    }
    r.b = b;
    r.first = first;
  }
  return r;
}

// Total page count P, and the first flattened page and page count of one
// sequence b, in two barriers.  Must be called by the whole block.
struct SeqPages {
  int64_t P, first, np;
};
__device__ __forceinline__ SeqPages seq_pages(const int32_t* seq_lens, const int32_t* seq_starts, int32_t B,
                                              int32_t bs, int32_t b) {
  __shared__ int32_t wave_tot[16];
  __shared__ int64_t found[2];
  const int nt = blockDim.x, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int32_t chunk = (B + nt - 1) / nt;
  const int32_t b0 = t * chunk, b1 = min(B, b0 + chunk);
  int32_t s = 0, before = 0, mine = 0;                 // pages of the chunk, of its part before b, of b
  for (int32_t i = b0; i < b1; ++i) {
    const int32_t np = window_pages(seq_lens[i], seq_start(seq_starts, i), bs);
    before += i < b ? np : 0;
    mine += i == b ? np : 0;
    s += np;
  }
  const int32_t v = wave_incl_scan(s);
  if (lane == 63) wave_tot[wv] = v;
  __syncthreads();
  int64_t carry = 0, total = 0;
  for (int w = 0; w < nt / 64; ++w) {
    const int32_t c = wave_tot[w];
    carry += w < wv ? c : 0;
    total += c;
  }
  if (b0 <= b && b < b1) {                             // the thread whose chunk holds b
    found[0] = carry + v - s + before;
    found[1] = mine;
  }
  __syncthreads();
  SeqPages r;
  r.P = total;
  r.first = found[0];
  r.np = found[1];
  return r;
}

// Sequence owning flattened page x (0 <= x < P), and that sequence's first page.
__device__ __forceinline__ void locate_page(const int32_t* seq_lens, const int32_t* seq_starts, int32_t B,
                                            int32_t bs, const int32_t* scan, int32_t chunk, int64_t x,
                                            int32_t* b_out, int64_t* first_out) {
  int lo = 0, hi = blockDim.x;            // scan[lo] <= x < scan[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (scan[mid] <= x) lo = mid; else hi = mid;
  }
  if (chunk == 1) {                       // lo is the sequence (empty ones share its prefix)
    *b_out = lo;
    *first_out = scan[lo];
    return;
  }
  int64_t first = scan[lo];
  int32_t b = lo * chunk;
  for (;;) {
    int32_t np = window_pages(seq_lens[b], seq_start(seq_starts, b), bs);
    if (x < first + np) break;
    first += np;
    ++b;
  }
  *b_out = b;
  *first_out = first;
}

}  // namespace mla
