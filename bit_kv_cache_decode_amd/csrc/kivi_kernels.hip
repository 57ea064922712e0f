// HIP kernels for KIVI-style quantized-KV decode on gfx950 (MI355X).
//
// Method (pages cited by title and section):
//   * discosf KIVI tutorial, section 3.1: keys are quantized in groups of G
//     tokens per channel, the newest tokens stay in an fp16 window until R of
//     them have accumulated, then the window is quantized and emptied.
//   * unite.ai KV cache quantization axis-selection guide, section on what
//     quantization error is made of: uniform quantizer with the group
//     minimum as zero-point and step = range / (2^B - 1), round to nearest.
//     Keys section: per-channel key groups.  Values section: per-token value
//     groups; the output is the softmax-weighted sum of the values.  Section
//     on why the KV cache matters: every generated token reads the whole
//     cache, so decode is bound by HBM bandwidth.
//
// Buffer layouts are the ones documented in include/kivi.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "kivi_internal.h"

namespace kivi {
namespace {

constexpr int kD = 128;        // head_dim covered by the compiled kernels
constexpr int kThreads = 256;  // 4 waves of 64
// Decode shape and pipelining: waves per workgroup and workgroups per
// compute unit (shared with the host-side work split), hence waves per SIMD;
// how waves set their
// issue priority (0 never, 1 from their own progress fraction, 2 from their
// lead over the slowest wave of the workgroup).
#ifndef KIVI_DECODE_PRIORITY
#define KIVI_DECODE_PRIORITY 2
#endif
constexpr int kDecodeWaves = kDecodeWavesPerWorkgroup;
constexpr int kDecodeThreads = 64 * kDecodeWaves;
constexpr int kDecodeWavesPerSimd = kDecodeWorkgroupsPerCU * kDecodeWaves / 4;

using half_t = _Float16;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ wave helpers

__device__ __forceinline__ uint32_t u4_get(const uint4 &v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// c ? a : b on values (a conditional on two uint4 lvalues can become a
// select of their addresses, forcing them into scratch memory)
__device__ __forceinline__ uint4 sel4(bool c, uint4 a, uint4 b) {
  return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N consecutive lanes (N in 2, 4, 8, 16, 32);
// every lane of a group receives the group sum.  DPP: quad_perm xor1 / xor2,
// then half-row mirror (lane i <-> 7 - i) and row mirror (lane i <-> 15 - i);
// for 32, a swizzle swaps the two rows of each half wave (lane i <-> i ^ 16).
template <int N>
__device__ __forceinline__ float lane_group_sum(float v) {
  v += dpp<0xB1>(v);
  if constexpr (N >= 4) v += dpp<0x4E>(v);
  if constexpr (N >= 8) v += dpp<0x141>(v);
  if constexpr (N >= 16) v += dpp<0x140>(v);
  if constexpr (N >= 32)  // bitmask mode: and 0x1F, or 0, xor 0x10
    v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
  return v;
}

// Packed fp16 maximum / minimum of two half2 words (v_pk_max_f16 / v_pk_min_f16).
__device__ __forceinline__ uint32_t pk_max16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(half2_t, a),
                                                                __builtin_bit_cast(half2_t, b)));
}

__device__ __forceinline__ uint32_t pk_min16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(half2_t, a),
                                                                __builtin_bit_cast(half2_t, b)));
}

__device__ __forceinline__ uint32_t neg16x2(uint32_t v) { return v ^ 0x80008000u; }
__device__ __forceinline__ uint32_t swap16(uint32_t v) { return (v >> 16) | (v << 16); }

template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

// Packed fp16 maximum over aligned groups of N consecutive lanes (as
// lane_group_sum).
template <int N>
__device__ __forceinline__ uint32_t lane_group_pkmax(uint32_t v) {
  v = pk_max16(v, dppu<0xB1>(v));
  if constexpr (N >= 4) v = pk_max16(v, dppu<0x4E>(v));
  if constexpr (N >= 8) v = pk_max16(v, dppu<0x141>(v));
  if constexpr (N >= 16) v = pk_max16(v, dppu<0x140>(v));
  return v;
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Whole-wave sum / maximum, the same value in every lane: DPP within each
// row of 16 lanes (as lane_group_sum), then the four rows' lanes 0, 16, 32
// and 48 read as scalars.
__device__ __forceinline__ float row_sum16(float v) { return lane_group_sum<16>(v); }

__device__ __forceinline__ float lane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// ---------------------------------------------------------------- encoder
// The fixed fp32 sequence of the quantizer (header comment of kivi.h): no
// contraction, IEEE division, round half to even.
#pragma clang fp contract(off)

constexpr float kFastOffsetMax = 128.0f;

struct GroupParams {
  float mn;  // canonical minimum (zero-point)
  float s;   // stored step as fp32
  float rs;  // fast-path multiplier: 1 / s within one ulp, 0 when s == 0;
             // NaN (every code exact) when s is an fp16 subnormal or
             // |mn / s| is large (see quant_code)
  float nm;  // fast-path offset: -(mn * rs) rounded once
  half_t zero16, scale16;
};

__device__ __forceinline__ GroupParams group_params(float mn_raw, float mx_raw, float levels) {
  GroupParams g;
  g.mn = mn_raw + 0.0f;  // -0 -> +0
  const float mx = mx_raw + 0.0f;
  const float step = (mx - g.mn) / levels;
  g.scale16 = (half_t)step;  // round to nearest even
  g.s = (float)g.scale16;
  g.rs = g.s == 0.0f ? 0.0f : g.s < 0x1p-14f ? __builtin_nanf("") : __builtin_amdgcn_rcpf(g.s);
  const float m = g.mn * g.rs;
  g.nm = -m;
  if (!(fabsf(m) <= kFastOffsetMax)) g.rs = __builtin_nanf("");
  g.zero16 = (half_t)g.mn;   // exact: mn is an fp16 value
  return g;
}

// Codes are clamp(rint((x - mn) / s), 0, top) with x - mn rounded once and
// an IEEE division (code_exact).  The fast path computes q' = x * rs + nm in
// one fused multiply-add (rs = 1 / s within one ulp, 0 when s == 0, which
// gives code 0 as required; nm = -(mn * rs) rounded once) and takes rint(q')
// unless q' lies within 2^-16 (B <= 4) or 2^-13 (B = 8) of a half-integer,
// where that one code takes the division instead:
//  * the true quotient q = (x - mn) / s is below 2^B (x - mn is at most the
//    group's range and s is the range over the levels, rounded to fp16 with
//    a relative error of at most 2^-11).  q' differs from q by at most
//    q 2^-23 (the reciprocal) + |mn rs| 2^-24 (nm) + q' 2^-24 (the fma's one
//    rounding), and the exact path's own quotient from q by at most q 2^-23
//    (its two roundings).  With |mn rs| <= 128 (kFastOffsetMax; a larger
//    offset sets rs to NaN, so every code of the group is exact) the sum is
//    below 1.3e-5 < 2^-16 for q < 16 and below 8.5e-5 < 2^-13 for q < 256:
//    away from the half-integers by the margin, q' and the exact quotient
//    round to the same integer.  q' - rint(q') is exact (Sterbenz).
//  * the clamp: with a normal fp16 step (s >= 2^-14) q' is at most
//    top (1 + 2^-10) + 2^-13 < top + 1/2, so rint never passes top and the
//    fast path needs no clamp; at x = mn, |q'| is below 2^-17.  A subnormal
//    step has rs = NaN, and a NaN q' takes the exact path.
// Exact ties are common with fp16 data (x - mn and s are short fp16
// multiples), so the exact path is taken per code, not per word.
// Codes enter the word as two fp32 sums, one per half word, of
// c * 2^(B * i): integers below 2^16, so the sums are exact.
template <int BITS>
constexpr float near_half() {
  return BITS <= 4 ? 0.5f - 0x1p-16f : 0.5f - 0x1p-13f;
}

__device__ __forceinline__ float code_exact(float x, float mn, float s) {
  return s == 0.0f ? 0.0f : rintf((x - mn) / s);
}

// One code of a group {mn, s, rs, nm}: the fast product, or the division
// for a product near a half-integer (or NaN).
template <int BITS>
__device__ __forceinline__ float quant_code(float x, float mn, float s, float rs, float nm) {
  const float q = fmaf(x, rs, nm);
  const float c = rintf(q);
  if (!(fabsf(q - c) <= near_half<BITS>()))
    return fminf(code_exact(x, mn, s), (float)((1 << BITS) - 1));
  return c;
}

template <int BITS, int CPW>
struct CodeWord {
  float lo = 0.0f, hi = 0.0f;
  float dev = 0.0f;  // add_fast: the largest |q' - rint(q')| so far
  __device__ __forceinline__ void put(int i, float c) {
    const float f = (float)(1u << (BITS * (i % (CPW / 2))));
    if (i < CPW / 2)
      lo = fmaf(c, f, lo);
    else
      hi = fmaf(c, f, hi);
  }
  // code i of the word: channel value x of a group {mn, s, rs, nm}
  __device__ __forceinline__ void add(int i, float x, float mn, float s, float rs, float nm) {
    put(i, quant_code<BITS>(x, mn, s, rs, nm));
  }
  // code i by the fast product alone
  __device__ __forceinline__ void add_fast(int i, float x, float rs, float nm) {
    const float q = fmaf(x, rs, nm);
    const float c = rintf(q);
    dev = fmaxf(dev, fabsf(q - c));
    put(i, c);
  }
  // every add_fast code is the one quant_code gives: none lies near a
  // half-integer, and none is NaN (a NaN product makes its sum NaN, while
  // fmaxf passes over it)
  __device__ __forceinline__ bool fast_ok() const {
    return dev <= near_half<BITS>() && lo == lo && hi == hi;
  }
  __device__ __forceinline__ uint32_t word() const {
    return (uint32_t)lo | ((uint32_t)hi << (BITS * (CPW / 2)));
  }
};

// One code word of CPW channel values x(i) with groups par(i) = {mn, s,
// rs, nm}: every code by the fast product, and the word once more code by
// code (quant_code) only when one of them needs the division.  One test
// per word instead of a branch per code.
template <int BITS, int CPW, typename X, typename P>
__device__ __forceinline__ uint32_t encode_word(X x, P par) {
  CodeWord<BITS, CPW> fw;
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const float4 p = par(i);
    fw.add_fast(i, x(i), p.z, p.w);
  }
  if (!fw.fast_ok()) {
    fw = CodeWord<BITS, CPW>();
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const float4 p = par(i);
      fw.add(i, x(i), p.x, p.y, p.z, p.w);
    }
  }
  return fw.word();
}

#pragma clang fp contract(on)

struct EncodeArgs {
  const half_t *src_k, *src_v;  // [batch][heads][src_tokens][D]
  int src_tokens;
  uint32_t *k_codes, *v_codes;
  half_t *k_scale, *k_zero, *v_scale, *v_zero;
  half_t *k_res, *v_res;         // window [batch][heads][R][D] (prefill writes it)
  int32_t *q_len, *r_len;
  const int32_t *len, *res;      // prefill: prompt lengths, window sizes (res may be null)
  uint32_t *status, *tickets;
  int heads, R, cap, prefill;
  // value queue (discosf KIVI tutorial, section 3.2): values leave an fp16
  // queue of the newest R one token at a time, quantized as they leave; the
  // queue is a ring in the value window (token t in slot t mod R).  Prefill
  // then quantizes only the first max(0, len - R) values.
  int vq;
};

// Window size and validity of one prompt, identical in every prefill kernel.
__device__ __forceinline__ bool prefill_split(const EncodeArgs &a, int b, int G, int *n_out,
                                              int *r_out) {
  const int n = a.len[b];
  const int r = a.res ? a.res[b] : (n >= 0 ? n % G : -1);
  *n_out = n;
  *r_out = r;
  return n >= 0 && n <= a.src_tokens && r >= 0 && r <= a.R && r <= n && ((n - r) % G) == 0;
}

__device__ __forceinline__ bool flush_ok(int ql, int rl, int G, int R, int cap) {
  return rl == R && ql >= 0 && (ql % G) == 0 && ql + R <= cap;
}

// Prefill: one workgroup quantizes one tile of G tokens of one
// (sequence, head): keys per channel over the G tokens, values per token
// over G channels, and packs both into the tiled code layout.  Both tiles
// are loaded up front; threads 0..127 then take the 128 key groups and
// threads 128..255 the 128 value groups.
template <int BITS, int G>
__global__ __launch_bounds__(kThreads) void encode_kernel(EncodeArgs a) {
  constexpr int W = kD * BITS / 32, CPW = 32 / BITS;
  constexpr float kTop = (float)((1 << BITS) - 1);
  static_assert(G * (kD / G) == kD && kD == 128, "128 key groups and 128 value groups per tile");
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;

  int n, r;
  const bool ok = prefill_split(a, b, G, &n, &r) && n - r <= a.cap;
  const int ntiles = ok ? (n - r) / G : 0;
  const int dst0 = 0;
  if (tile >= ntiles) return;

  __shared__ half_t xk[G][kD + 8], xv[G][kD + 8];
  __shared__ float4 kpar[kD], vpar[kD];  // {mn, s, rs, nm} per key channel / value group

  const size_t bh = (size_t)b * a.heads + h;
  const size_t src_off = (bh * a.src_tokens + (size_t)tile * G) * kD;
  const size_t ktile = bh * (size_t)(a.cap / G) + (size_t)(dst0 / G) + tile;

  {
    constexpr int N = G * (kD / 8);  // uint4 per tile
    static_assert(N % kThreads == 0, "whole passes");
    const uint4 *sk = reinterpret_cast<const uint4 *>(a.src_k + src_off);
    const uint4 *sv = reinterpret_cast<const uint4 *>(a.src_v + src_off);
    uint4 rk[N / kThreads], rv[N / kThreads];
#pragma unroll
    for (int i = 0; i < N / kThreads; ++i) {
      rk[i] = sk[tid + i * kThreads];
      rv[i] = sv[tid + i * kThreads];
    }
#pragma unroll
    for (int i = 0; i < N / kThreads; ++i) {
      const int e = tid + i * kThreads, t = e / (kD / 8), c = e % (kD / 8);
      *reinterpret_cast<uint4 *>(&xk[t][c * 8]) = rk[i];
      *reinterpret_cast<uint4 *>(&xv[t][c * 8]) = rv[i];
    }
  }
  __syncthreads();

  if (tid < kD) {
    // key group: channel tid over the G tokens
    float mn = INFINITY, mx = -INFINITY;
    for (int t = 0; t < G; ++t) {
      const float x = (float)xk[t][tid];
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    const GroupParams g = group_params(mn, mx, kTop);
    a.k_zero[ktile * kD + tid] = g.zero16;
    a.k_scale[ktile * kD + tid] = g.scale16;
    kpar[tid] = make_float4(g.mn, g.s, g.rs, g.nm);
  } else {
    // value group: token t, channels j*G .. j*G+G-1; stored tiled like the
    // codes, [tile][group][token]
    const int e = tid - kD, j = e / G, t = e % G;
    float mn = INFINITY, mx = -INFINITY;
    for (int c = 0; c < G; ++c) {
      const float x = (float)xv[t][j * G + c];
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    GroupParams g = group_params(mn, mx, kTop);
    if (a.vq && tile * G + t >= n - a.R) {
      // value queue: this token's value is still in the fp16 queue; its
      // group stays zero (step 0, zero-point 0, codes 0)
      g.mn = 0.0f;
      g.s = 0.0f;
      g.rs = 0.0f;
      g.nm = 0.0f;
      g.zero16 = (half_t)0.0f;
      g.scale16 = (half_t)0.0f;
    }
    a.v_zero[ktile * kD + e] = g.zero16;
    a.v_scale[ktile * kD + e] = g.scale16;
    vpar[e] = make_float4(g.mn, g.s, g.rs, g.nm);
  }
  __syncthreads();

  for (int wi = tid; wi < W * G; wi += kThreads) {
    const int w = wi / G, t = wi % G;
    const int gi = ((w * CPW) / G) * G + t;
    const float4 vp = vpar[gi];
    const uint32_t wk = encode_word<BITS, CPW>([&](int i) { return (float)xk[t][w * CPW + i]; },
                                               [&](int i) { return kpar[w * CPW + i]; });
    const uint32_t wv = encode_word<BITS, CPW>([&](int i) { return (float)xv[t][w * CPW + i]; },
                                               [&](int) { return vp; });
    a.k_codes[ktile * (W * G) + wi] = wk;
    a.v_codes[ktile * (W * G) + wi] = wv;
  }
}

// Quantize window tokens [blk0, blk1) of one (sequence, head) into
// quantized slots from ql + blk0 on.  The loads of a block of TB tokens (a
// multiple of G) are all issued up front, tile by tile; each tile of G
// tokens is then staged in LDS as soon as its own loads have arrived, its
// key groups (two channels per item) and value groups are computed, then its
// code words, while the later tiles' loads are still in flight.  Token rnew
// of the window is taken from knew / vnew (one fp16 row each) instead of the
// cache when those are given: the token an append in the same kernel has
// just written.  NTHREADS threads take part.
template <int G, int TB>
struct FlushSmem {
  static constexpr int NB = TB / G >= 2 ? 2 : 1;  // tile buffers
  half_t x[NB][2][G][kD + 8];                     // [buffer][key, value][token][channel]
  float4 kp[NB][kD], vp[NB][kD];                  // {minimum, step, 1 / step, offset}
};

// A 16-byte piece of a window row, read once by the flush: non-temporal
// unless KIVI_FLUSH_NT is 0.
#ifndef KIVI_FLUSH_NT
#define KIVI_FLUSH_NT 1
#endif
__device__ __forceinline__ uint4 load_window_row(const uint4 *p) {
#if KIVI_FLUSH_NT
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  const u4v v = __builtin_nontemporal_load(reinterpret_cast<const u4v *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *p;
#endif
}

template <int BITS, int G, int TB, int NTHREADS, bool VALUES = true>
__device__ __forceinline__ void flush_window(const EncodeArgs &a, size_t bh, int ql, int tid,
                                             FlushSmem<G, TB> &fs, int rnew, const uint4 *knew,
                                             const uint4 *vnew, int blk0, int blk1) {
  constexpr int W = kD * BITS / 32, CPW = 32 / BITS;
  constexpr float kTop = (float)((1 << BITS) - 1);
  constexpr int NTB = TB / G;                           // tiles per block
  constexpr int TE = G * (kD / 8);                      // uint4 per tile and operand
  constexpr int PE = 2 * TE / NTHREADS;                 // uint4 per thread and tile
  constexpr int NB = FlushSmem<G, TB>::NB;
  static_assert(TB % G == 0 && PE >= 1 && PE * NTHREADS == 2 * TE, "whole tiles per pass");
  const uint4 *src[2] = {reinterpret_cast<const uint4 *>(a.k_res + bh * a.R * kD),
                         reinterpret_cast<const uint4 *>(a.v_res + bh * a.R * kD)};
  const uint4 *fresh_row[2] = {knew, vnew};

  for (int blk = blk0; blk < blk1; blk += TB) {
    const int nt = min(TB, blk1 - blk) / G;  // tiles in this block
    uint4 r[NTB][PE];
#pragma unroll
    for (int tl = 0; tl < NTB; ++tl) {
#pragma unroll
      for (int i = 0; i < PE; ++i) {
        const int e = tid + i * NTHREADS, op = e / TE, f = e % TE;
        const int t = blk + min(tl, nt - 1) * G + f / (kD / 8);  // clamped: unused past nt
        if (VALUES || op == 0) r[tl][i] = load_window_row(&src[op][(size_t)t * (kD / 8) + f % (kD / 8)]);
      }
    }
#pragma unroll
    for (int tl = 0; tl < NTB; ++tl) {
      if (tl >= nt) break;
      const int bf = tl % NB;
      const size_t tile = bh * (size_t)(a.cap / G) + (size_t)((ql + blk) / G) + tl;
#pragma unroll
      for (int i = 0; i < PE; ++i) {
        const int e = tid + i * NTHREADS, op = e / TE, f = e % TE;
        const int t = f / (kD / 8), c = f % (kD / 8);
        uint4 val = r[tl][i];
        if (knew != nullptr && blk + tl * G + t == rnew) val = fresh_row[op][c];
        if (VALUES || op == 0) *reinterpret_cast<uint4 *>(&fs.x[bf][op][t][c * 8]) = val;
      }
      __syncthreads();
      for (int gi = tid; gi < kD / 2 + (VALUES ? kD : 0); gi += NTHREADS) {
        if (gi < kD / 2) {
          // key groups: channels 2 * gi and 2 * gi + 1 over the tile's G tokens
          const int c = 2 * gi;
          float mn0 = INFINITY, mx0 = -INFINITY, mn1 = INFINITY, mx1 = -INFINITY;
#pragma unroll 8
          for (int t = 0; t < G; ++t) {
            const half2_t x2 = *reinterpret_cast<const half2_t *>(&fs.x[bf][0][t][c]);
            const float x0 = (float)x2.x, x1 = (float)x2.y;
            mn0 = fminf(mn0, x0);
            mx0 = fmaxf(mx0, x0);
            mn1 = fminf(mn1, x1);
            mx1 = fmaxf(mx1, x1);
          }
          const GroupParams g0 = group_params(mn0, mx0, kTop), g1 = group_params(mn1, mx1, kTop);
          *reinterpret_cast<half2_t *>(a.k_zero + tile * kD + c) = half2_t{g0.zero16, g1.zero16};
          *reinterpret_cast<half2_t *>(a.k_scale + tile * kD + c) = half2_t{g0.scale16, g1.scale16};
          fs.kp[bf][c] = make_float4(g0.mn, g0.s, g0.rs, g0.nm);
          fs.kp[bf][c + 1] = make_float4(g1.mn, g1.s, g1.rs, g1.nm);
        } else {
          // value groups: group e / G, token e % G, in the tiled
          // [tile][group][token] order of the value zero-points
          const int e = gi - kD / 2, j = e / G, t = e % G;
          float mn = INFINITY, mx = -INFINITY;
#pragma unroll
          for (int c = 0; c < G; c += 8) {
            const uint4 u = *reinterpret_cast<const uint4 *>(&fs.x[bf][1][t][j * G + c]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const half2_t x2 = __builtin_bit_cast(half2_t, u4_get(u, q));
              mn = fminf(mn, fminf((float)x2.x, (float)x2.y));
              mx = fmaxf(mx, fmaxf((float)x2.x, (float)x2.y));
            }
          }
          const GroupParams g = group_params(mn, mx, kTop);
          a.v_zero[tile * kD + e] = g.zero16;
          a.v_scale[tile * kD + e] = g.scale16;
          fs.vp[bf][e] = make_float4(g.mn, g.s, g.rs, g.nm);
        }
      }
      __syncthreads();
      for (int wi = tid; wi < (VALUES ? 2 : 1) * W * G; wi += NTHREADS) {
        // key words first, then value words; word (w, t) holds channels
        // w * CPW .. w * CPW + CPW - 1 of token t
        const int op = wi / (W * G), w = (wi / G) % W, t = wi % G;
        float x[CPW];
        if constexpr (CPW >= 8) {
#pragma unroll
          for (int i = 0; i < CPW; i += 8) {
            const uint4 u = *reinterpret_cast<const uint4 *>(&fs.x[bf][op][t][w * CPW + i]);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const half2_t x2 = __builtin_bit_cast(half2_t, u4_get(u, q / 2));
              x[i + q] = (q & 1) ? (float)x2.y : (float)x2.x;
            }
          }
        } else {  // B = 8: four channels per word
          const uint2 u = *reinterpret_cast<const uint2 *>(&fs.x[bf][op][t][w * CPW]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const half2_t x2 = __builtin_bit_cast(half2_t, q < 2 ? u.x : u.y);
            x[q] = (q & 1) ? (float)x2.y : (float)x2.x;
          }
        }
        // (code by code: the word-level test of encode_word holds more
        // registers, which measured slower here at B = 8)
        CodeWord<BITS, CPW> fw;
        if (op == 0) {
#pragma unroll
          for (int i = 0; i < CPW; ++i) {
            const float4 kq = fs.kp[bf][w * CPW + i];
            fw.add(i, x[i], kq.x, kq.y, kq.z, kq.w);
          }
          a.k_codes[tile * (W * G) + (wi % (W * G))] = fw.word();
        } else {
          const float4 v = fs.vp[bf][((w * CPW) / G) * G + t];
#pragma unroll
          for (int i = 0; i < CPW; ++i) fw.add(i, x[i], v.x, v.y, v.z, v.w);
          a.v_codes[tile * (W * G) + (wi % (W * G))] = fw.word();
        }
      }
      if (NB == 1) __syncthreads();  // a single buffer is rewritten by the next tile
    }
    __syncthreads();
  }
}

// Flush: grid (R / (G P), heads, batch); one workgroup of P x 256 threads
// quantizes P tiles of G window tokens of one (sequence, head), 256 threads
// per tile (P below, chosen by the launcher).  Thread 0 reads b's lengths
// and hands them to the other threads through LDS behind a barrier, then
// takes one of sequence b's tickets (the atomic's latency hides behind the
// window loads); the workgroup that took the last one (every workgroup of
// the sequence has read the lengths by then, and none reads them again)
// sets q_len[b] += R, r_len[b] = 0 and clears the ticket when it is done.
// A ticket at or past the count means the counter did not start at zero
// (cache->tickets not initialised): KIVI_ST_TICKETS, and no commit.
constexpr int kFlushThreads = 256;
// Window tiles a flush workgroup takes side by side (at most).  Two measured
// best: the workgroup dispatcher starts about 230 workgroups per microsecond,
// so 1024 tile-sized workgroups take 4.4 us only to start; two tiles per
// workgroup halve that, four cost more in residency than they save.
#ifndef KIVI_FLUSH_P
#define KIVI_FLUSH_P 2
#endif

template <int BITS, int G, int P, bool VALUES = true>
__global__ __launch_bounds__(kFlushThreads * P) void flush_kernel(EncodeArgs a) {
  const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int part = tid / kFlushThreads, tile = blockIdx.x * P + part;
  __shared__ int lens[2];
  if (tid == 0) {
    lens[0] = a.q_len[b];
    lens[1] = a.r_len[b];
  }
  __syncthreads();
  const int ql = lens[0], rl = lens[1];
  if (!flush_ok(ql, rl, G, a.R, a.cap)) {
    if (rl == a.R && blockIdx.x == 0 && h == 0 && tid == 0)
      atomicOr(a.status, (ql < 0 || ql % G) ? KIVI_ST_BAD_LENGTH : KIVI_ST_CAPACITY);
    return;
  }
  uint32_t ticket = 0;
  const uint32_t n_tickets = (uint32_t)(a.heads * (a.R / G / P));
  if (tid == 0)
    ticket = __hip_atomic_fetch_add(a.tickets + (size_t)b * kTicketStride, 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
  // P tiles side by side, kFlushThreads threads and one LDS block each; they
  // pass the same barriers in step (P divides the window's tile count)
  __shared__ FlushSmem<G, G> fs[P];
  flush_window<BITS, G, G, kFlushThreads, VALUES>(a, (size_t)b * a.heads + h, ql,
                                                  tid % kFlushThreads, fs[part], -1, nullptr,
                                                  nullptr, tile * G, tile * G + G);
  if (tid == 0 && ticket == n_tickets - 1) {
    a.q_len[b] = ql + a.R;
    a.r_len[b] = 0;
    a.tickets[(size_t)b * kTicketStride] = 0u;
  }
  if (tid == 0 && ticket >= n_tickets) atomicOr(a.status, KIVI_ST_TICKETS);
}

// Prefill: copy the window part [n - r, n) of each valid prompt to slots [0, r).
__global__ __launch_bounds__(kThreads) void prefill_window_kernel(EncodeArgs a, int G) {
  const int h = blockIdx.x, b = blockIdx.y;
  int n, r;
  if (!prefill_split(a, b, G, &n, &r) || n - r > a.cap) return;
  const size_t bh = (size_t)b * a.heads + h;
  const size_t src = (bh * a.src_tokens + (size_t)(n - r)) * kD;
  const size_t dst = bh * (size_t)a.R * kD;
  for (int i = threadIdx.x; i < r * (kD / 8); i += kThreads) {
    reinterpret_cast<uint4 *>(a.k_res + dst)[i] = reinterpret_cast<const uint4 *>(a.src_k + src)[i];
    if (!a.vq)
      reinterpret_cast<uint4 *>(a.v_res + dst)[i] = reinterpret_cast<const uint4 *>(a.src_v + src)[i];
  }
  if (a.vq) {
    // the newest min(n, R) values, token t in ring slot t mod R
    const int v0 = max(0, n - a.R);
    const size_t vsrc = bh * a.src_tokens * kD;
    for (int i = threadIdx.x; i < (n - v0) * (kD / 8); i += kThreads) {
      const int t = v0 + i / (kD / 8), c = i % (kD / 8);
      reinterpret_cast<uint4 *>(a.v_res + dst + (size_t)(t % a.R) * kD)[c] =
          reinterpret_cast<const uint4 *>(a.src_v + vsrc + (size_t)t * kD)[c];
    }
  }
}

// Prefill commit: lengths and status, after the encode and window kernels.
__global__ void prefill_commit_kernel(EncodeArgs a, int batch, int G) {
  for (int b = threadIdx.x; b < batch; b += blockDim.x) {
    int n, r;
    const bool ok = prefill_split(a, b, G, &n, &r);
    if (ok && n - r <= a.cap) {
      a.q_len[b] = n - r;
      a.r_len[b] = r;
    } else {
      a.q_len[b] = 0;
      a.r_len[b] = 0;
      atomicOr(a.status, ok ? KIVI_ST_CAPACITY : KIVI_ST_BAD_LENGTH);
    }
  }
}

// ----------------------------------------------------------------- append
// One workgroup of 1024 threads per sequence copies the new token of every
// head into window slot r_len[b] (one 16-byte piece of a key or value row
// per thread and pass), then bumps r_len[b].  Every thread reads r_len[b]
// before the barrier and only thread 0 writes it after, so no thread sees
// the new value.
constexpr int kAppendThreads = 1024;

__global__ __launch_bounds__(kAppendThreads) void append_kernel(
    const half_t *k_new, const half_t *v_new, half_t *k_res, half_t *v_res, int32_t *r_len,
    uint32_t *status, int heads, int R) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int r = r_len[b];
  __syncthreads();
  if (r < 0 || r >= R) {
    if (tid == 0) atomicOr(status, r < 0 ? KIVI_ST_BAD_LENGTH : KIVI_ST_RESIDUAL_FULL);
    return;
  }
  constexpr int V = kD / 8;  // uint4 per row
  const int n = heads * V;   // uint4 per operand and sequence
  for (int i = tid; i < 2 * n; i += kAppendThreads) {
    const int e = i < n ? i : i - n;
    const size_t bh = (size_t)b * heads + e / V;
    const uint4 x = reinterpret_cast<const uint4 *>(i < n ? k_new : v_new)[(size_t)b * n + e];
    reinterpret_cast<uint4 *>(i < n ? k_res : v_res)[(bh * R + r) * V + e % V] = x;
  }
  __syncthreads();
  if (tid == 0) r_len[b] = r + 1;
}

// ------------------------------------------------------ value-queue append
// The value queue (discosf KIVI tutorial, section 3.2): the value window is
// a ring of R slots holding the newest min(T, R) values (token t in slot
// t mod R, T = q_len + r_len tokens in all).  Appending token T: its key goes
// to key-window slot r_len (as in append_kernel); once the ring is full
// (T >= R) the value in slot T mod R -- token T - R, the oldest -- is
// quantized on its own (D / G groups of G channels) into value position
// T - R of the tiles, then the slot takes the new value.  One workgroup of
// 16 waves per sequence, a wave per head at a time; lane i holds channels
// 2i and 2i + 1.  Every thread reads the lengths before the barrier that
// precedes thread 0's update of r_len.
constexpr int kAppendVqThreads = 1024;

template <int BITS, int G>
__global__ __launch_bounds__(kAppendVqThreads) void append_vq_kernel(EncodeArgs a,
                                                                     const half_t *k_new,
                                                                     const half_t *v_new) {
  constexpr int W = kD * BITS / 32, CPW = 32 / BITS, LPW = CPW / 2, LPG = G / 2;
  constexpr float kTop = (float)((1 << BITS) - 1);
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ql = a.q_len[b], r = a.r_len[b];
  __syncthreads();
  if (r < 0 || r >= a.R || ql < 0 || ql % G || ql > a.cap) {
    if (tid == 0)
      atomicOr(a.status, (r >= a.R && ql >= 0 && ql % G == 0 && ql <= a.cap)
                             ? KIVI_ST_RESIDUAL_FULL : KIVI_ST_BAD_LENGTH);
    return;
  }
  const int T = ql + r, slot = T % a.R, te = T - a.R;
  const size_t tiles = (size_t)(a.cap / G);
  for (int h = wv; h < a.heads; h += kAppendVqThreads / 64) {
    const size_t bh = (size_t)b * a.heads + h;
    uint32_t *vrow = reinterpret_cast<uint32_t *>(a.v_res + (bh * a.R + slot) * kD);
    if (te >= 0) {
      const half2_t x2 = __builtin_bit_cast(half2_t, vrow[lane]);
      const float x0 = (float)x2.x, x1 = (float)x2.y;
      float mn = fminf(x0, x1), mx = fmaxf(x0, x1);
#pragma unroll
      for (int o = 1; o < LPG; o <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, o));
        mx = fmaxf(mx, __shfl_xor(mx, o));
      }
      const GroupParams g = group_params(mn, mx, kTop);
      const uint32_t c0 = (uint32_t)fminf(code_exact(x0, g.mn, g.s), kTop);
      const uint32_t c1 = (uint32_t)fminf(code_exact(x1, g.mn, g.s), kTop);
      uint32_t word = (c0 << ((2 * lane) % CPW * BITS)) | (c1 << ((2 * lane + 1) % CPW * BITS));
#pragma unroll
      for (int o = 1; o < LPW; o <<= 1) word |= (uint32_t)__shfl_xor((int)word, o);
      const size_t tile = bh * tiles + (size_t)(te / G);
      if (lane % LPW == 0) a.v_codes[(tile * W + lane / LPW) * G + te % G] = word;
      if (lane % LPG == 0) {
        a.v_zero[tile * kD + (lane / LPG) * G + te % G] = g.zero16;
        a.v_scale[tile * kD + (lane / LPG) * G + te % G] = g.scale16;
      }
    }
    // the slot's old value has been read (same lanes, same addresses)
    vrow[lane] = reinterpret_cast<const uint32_t *>(v_new + bh * kD)[lane];
    reinterpret_cast<uint32_t *>(a.k_res + (bh * a.R + r) * kD)[lane] =
        reinterpret_cast<const uint32_t *>(k_new + bh * kD)[lane];
  }
  __syncthreads();
  if (tid == 0) a.r_len[b] = r + 1;
}

// ----------------------------------------------------------------- decode
//
// Grid (splits, heads, batch), kDecodeWaves (8) waves per workgroup: one
// workgroup per compute unit (two waves per SIMD) with two sub-chunks of
// loads in flight per wave, or, on grids larger than the chip, one sub-chunk
// in flight and a register footprint small enough for two or three
// workgroups per compute unit.  The 8 * splits waves of one (sequence,
// head) share its work: quantized sub-chunks of 64 (B=2) or 32 (B=4) tokens
// are dealt round-robin to the waves, and each wave also takes an equal
// slice of the fp16 window tokens, computed last.  Every wave works on its
// own (no block barrier until the end) and sets its issue priority from
// its lead over the slowest wave of its workgroup (the slowest issues
// first); every lane keeps its own
// online-softmax state (running max, sum, value sums) for the tokens it
// sees.  At the end the lanes and waves of the workgroup are combined in
// LDS (max m, sum l, unnormalised value sums, in log2 units).  With one
// workgroup per (sequence, head) that is the output; otherwise each
// workgroup publishes its partial state to the workspace and the one that
// takes the last ticket of its (sequence, head) merges all partials by
// log-sum-exp rescaling and writes the output.
//
// Dequantization is folded into the dot products:
//   score_t = sum_d q'_d * K_hat[t,d]
//           = sum_d (q'_d * s_{g,d}) * c_{t,d} + sum_d q'_d * z_{g,d}
//   out_d   = sum_t p_t * (z_{t,j} + s_{t,j} * c_{t,d})
//           = sum_t (p_t * s_{t,j}) * c_{t,d} + sum_t p_t * z_{t,j}
// with q' = sm_scale * log2(e) * q, so that p_t = exp2(score_t - max).
//
// Code conversion: one AND of a packed word keeps, in each 16-bit half, the
// code of one channel at its bit offset e (e < 10, inside the fp16 mantissa;
// the upper channels of each half are first shifted down).  Each half is
// then an fp16 subnormal equal to c * 2^(e - 24), exactly, and
// v_fma_mix_f32 converts it inside the fused multiply-add.  The factor
// 2^(24 - e) is folded into the key multipliers, and taken out of the value
// sums at the end (window values enter the sums pre-multiplied by
// 2^(e - 24)).

struct DecodeArgs {
  const uint32_t *k_codes, *v_codes;
  const half_t *k_scale, *k_zero, *v_scale, *v_zero, *k_res, *v_res;
  const int32_t *q_len, *r_len;
  uint32_t *status;
  const half_t *q;
  const half_t *k_new, *v_new;  // whole-step kernel only
  float *out, *part;
  uint32_t *tickets;
  float qscale;  // sm_scale * log2(e)
  int heads, R, cap, splits, win_per_wave, part_stride;
  int lpt_batch;  // > 0: workgroups take the sequences longest first (of a batch this size)
  double rope_log2_base;  // log2 of the rotary base (ROPE kernels only)
  // fp16 sink tokens [batch][heads][n_sink][D] (every decode variant: plain,
  // rotary and whole step; n_sink 0 when there is none), sink_per_wave of
  // them per wave
  const half_t *k_sink, *v_sink;
  int n_sink, sink_per_wave;
};

// Sub-chunks in flight per wave in the plain decode on grids of at most one
// workgroup per compute unit.
#ifndef KIVI_WIDE_DEPTH
#define KIVI_WIDE_DEPTH 2
#endif
constexpr int kMaxSplits = 128;
constexpr int kPartHead = 4;   // m, l, 2 pad floats before the 128 values



template <int BITS, int G>
struct DecCfg {
  static constexpr int W = kD * BITS / 32;     // words per token
  static constexpr int CPW = 32 / BITS;        // channels per word
  static constexpr int HP = CPW / 2;           // code pairs per word
  static constexpr int SUB = 512 / W;          // tokens per sub-chunk
  static constexpr int TQS = 64 / W;           // token quads per wave-load
  static constexpr int TPL = 4 * TQS;          // tokens per wave-load
  static constexpr int NL = SUB / TPL;         // wave-loads per sub-chunk and operand
  static constexpr int NVG = kD / G;            // value groups per token
  static constexpr int NTS = SUB >= G ? SUB / G : 1;  // key tiles a sub-chunk touches
  static constexpr int QPW = CPW + 4;          // padded LDS stride of one word's multipliers
  static_assert(NL == 2, "two 16-byte loads per lane per sub-chunk and operand");
  static_assert(G % TPL == 0, "a wave-load stays inside one tile");
};

template <int BITS, int G, bool ROPE = false>
struct DecSmem {
  using C = DecCfg<BITS, G>;
  struct {
    float acc[kDecodeWaves][4][kD];  // [wave][row][channel]
    float bias[kDecodeWaves][4][32]; // [wave][row][word]
    float m[kDecodeWaves], l[kDecodeWaves];
  } fin;
  union {
    struct {
      float qs[kD];                     // sm_scale * log2(e) * q
      float qp[C::NTS][C::W * C::QPW];  // key multipliers, word-padded (ROPE: steps)
      float cz[C::NTS][C::W];
    } wave[kDecodeWaves];
    struct {
      float m[kMaxSplits], l[kMaxSplits];
    } mg;
  } u;
  int ticket;
  int lens[2];             // whole step: the sequence's lengths, read once
  int prog[kDecodeWaves];  // sub-chunks each wave has started (issue priority)
  // ROPE: key zero-points of the touched tiles, word-padded like qp (kept
  // out of the per-wave staging above so that its layout, and the 16-byte
  // alignment of every wave's multipliers, is the same with or without)
  alignas(16) float zz[ROPE ? kDecodeWaves : 1][ROPE ? C::NTS : 1][ROPE ? C::W * C::QPW : 1];
};

__device__ __forceinline__ void store_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_agent(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float mix_lo(float a, uint32_t m, float c) {
  return fmaf(a, (float)__builtin_bit_cast(half2_t, m).x, c);
}

__device__ __forceinline__ float mix_hi(float a, uint32_t m, float c) {
  return fmaf(a, (float)__builtin_bit_cast(half2_t, m).y, c);
}

// Bit offset of channel i's code inside its 16-bit half after extraction.
template <int BITS>
__device__ __forceinline__ int code_offset(int i) {
  constexpr int HP = 16 / BITS;
  const int p = i % HP;
  if constexpr (BITS == 2) return p <= 4 ? 2 * p : 2 * (p - 5);
  else if constexpr (BITS == 4) return p <= 1 ? 4 * p : 4 * (p - 2);
  else return 0;  // B = 8: the low byte of a half, or the high one shifted down
}

// 2^(24 - e) for channel i of a word: the factor between an extracted code's
// fp16 value and the code.
template <int BITS>
__device__ __forceinline__ float code_factor(int i) {
  return __builtin_ldexpf(1.0f, 24 - code_offset<BITS>(i));
}

// Word u masked to code pair p (channels p and p + HP), each half holding its
// code at bit offset code_offset(p).  uh is u shifted right by 10 (B = 2) or
// 8 (B = 4, 8), which brings the upper pairs of each half into the mantissa.
template <int BITS, int P>
__device__ __forceinline__ uint32_t pair_bits(uint32_t u, uint32_t uh) {
  if constexpr (BITS == 2) {
    if constexpr (P <= 4) return u & (0x00030003u << (2 * P));
    else return uh & (0x00030003u << (2 * (P - 5)));
  } else if constexpr (BITS == 4) {
    if constexpr (P <= 1) return u & (0x000F000Fu << (4 * P));
    else return uh & (0x000F000Fu << (4 * (P - 2)));
  } else {
    if constexpr (P == 0) return u & 0x00FF00FFu;
    else return uh & 0x00FF00FFu;
  }
}

template <int BITS>
__device__ __forceinline__ uint32_t upper_pairs(uint32_t u) {
  return u >> (BITS == 2 ? 10 : 8);
}

// Adds q[i] * code_i * 2^(e_i - 24) over the word's channels to a0 (the
// channels of the low halves) and a1 (the high halves'); a0 and a1 may be
// the same accumulator.
template <int BITS, int P = 0>
__device__ __forceinline__ void dot_pairs(uint32_t u, uint32_t uh, const float *q, float &a0,
                                          float &a1) {
  constexpr int HP = 16 / BITS;
  if constexpr (P < HP) {
    const uint32_t m = pair_bits<BITS, P>(u, uh);
    a0 = mix_lo(q[P], m, a0);
    a1 = mix_hi(q[P + HP], m, a1);
    dot_pairs<BITS, P + 1>(u, uh, q, a0, a1);
  }
}

template <int BITS>
// One chain per word: a lane scores four independent tokens at a time, which
// is parallelism enough, and splitting a word's products over two chains
// cost one more instruction per word (7B layer 25.2 -> 24.5-25.0 us).
__device__ __forceinline__ float dot_word(uint32_t u, const float *q, float c0) {
  float a = c0;
  dot_pairs<BITS>(u, upper_pairs<BITS>(u), q, a, a);
  return a;
}

// acc[i] += pp * code_i * 2^(e_i - 24) over the word's channels.
template <int BITS, int P = 0>
__device__ __forceinline__ void axpy_pairs(uint32_t u, uint32_t uh, float pp, float *acc) {
  constexpr int HP = 16 / BITS;
  if constexpr (P < HP) {
    const uint32_t m = pair_bits<BITS, P>(u, uh);
    acc[P] = mix_lo(pp, m, acc[P]);
    acc[P + HP] = mix_hi(pp, m, acc[P + HP]);
    axpy_pairs<BITS, P + 1>(u, uh, pp, acc);
  }
}


// Combine the per-lane states of one wave and publish them to sm.fin.
// CPW: channels per lane; WPR: lanes per token slot; FOLD8: lanes l and l^8
// hold the same channels (two slots per 16-lane row).  Each published row
// covers all kD channels: one per 16-lane row of the wave, except with 32
// lanes per slot (B = 8), where row r is slot r and only rows 0 and 1 are
// written (publish_rows).
template <int WPR>
constexpr int publish_rows() {
  return WPR == 32 ? 2 : 4;
}

template <int CPW, int WPR, bool FOLD8>
__device__ __forceinline__ void wave_publish(float (&fin_acc)[4][kD], float (&fin_bias)[4][32],
                                             float &fin_m, float &fin_l, float m, float l,
                                             float *acc, float bias) {
  const int lane = threadIdx.x & 63;
  const int w = lane % WPR, row = WPR == 32 ? lane >> 5 : lane >> 4;
  const float M = wave_max(m);
  const float e = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
#pragma unroll
  for (int i = 0; i < CPW; ++i) acc[i] *= e;
  bias *= e;
  const float lw = wave_sum(w == 0 ? l * e : 0.0f);
  if constexpr (FOLD8) {
#pragma unroll
    for (int i = 0; i < CPW; ++i) acc[i] += dpp<0x128>(acc[i]);  // row_ror:8
    bias += dpp<0x128>(bias);
  }
  if (!FOLD8 || (lane & 8) == 0) {
#pragma unroll
    for (int i = 0; i < CPW; i += 4)
      *reinterpret_cast<float4 *>(&fin_acc[row][w * CPW + i]) =
          make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
    fin_bias[row][w] = bias;
  }
  if (lane == 0) {
    fin_m = M;
    fin_l = lw;
  }
}

// ------------------------------------------------------- decode: streaming
// All decode loads are raw buffer loads.  A descriptor covers one
// (sequence, head) region of one array; the per-lane part of an offset is a
// loop-invariant VGPR and the per-sub-chunk part a wave-uniform SGPR, so
// issuing loads needs no vector instructions.  A descriptor with zero
// records makes every load through it return 0 without touching memory.
using rsrc_t = __amdgpu_buffer_rsrc_t;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// Cache policy of the decode's loads (the buffer instructions' auxiliary
// bits: 1 sc0, 2 nt).  At B = 2 every byte the decode reads is read once
// per call, and non-temporal loads measured faster than plain ones
// (HIP-graph timings of 30 launches, alternating, one box): 7B layer 26.1
// -> 24.3 us, 13B layer 33.5 -> 30.7, ragged batch 64 203 -> 192, 131072
// tokens 78.9 -> 76.9.  At B = 4 and 8 they measured slower (7B shape at
// B = 8: 59.8 -> 91.8 us; at B = 4: 34.1 -> 35.4 us; sc0 alone and plain
// loads within noise of each other), so those widths keep sc0 alone.
#ifndef KIVI_DECODE_LOAD_AUX
#define KIVI_DECODE_LOAD_AUX 3
#endif
#ifndef KIVI_DECODE_LOAD_AUX_WIDE
#define KIVI_DECODE_LOAD_AUX_WIDE 1
#endif
constexpr int kLoadAux = KIVI_DECODE_LOAD_AUX;

template <int BITS>
constexpr int load_aux() {
  return BITS == 2 ? KIVI_DECODE_LOAD_AUX : KIVI_DECODE_LOAD_AUX_WIDE;
}

template <int AUX = kLoadAux>
__device__ __forceinline__ uint32_t bload1(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, AUX);
}

template <int AUX = kLoadAux>
__device__ __forceinline__ uint2 bload2(rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, AUX);
  return make_uint2(v.x, v.y);
}

template <int AUX = kLoadAux>
__device__ __forceinline__ uint4 bload4(rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, AUX);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Registers holding every load of one sub-chunk of one wave.
template <int BITS, int G>
struct SubLoads {
  using C = DecCfg<BITS, G>;
  uint4 kc[C::NL], vc[C::NL];      // key and value codes
  uint32_t ks[C::NTS], kz[C::NTS]; // key steps / zero-points of 2 channels per touched tile
  uint2 vs[C::NL], vz[C::NL];      // value steps / zero-points of this lane's 4 tokens
};

// Wave-uniform v_exp_f32: 2^x (0 for x = -inf).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Per-lane online-softmax state of one wave.
template <int CPW>
struct LaneState {
  float m, l, bias;
  float acc[CPW];
};

// How far (log2 units) a score may exceed a lane's reference m before the
// lane moves m up.  The softmax only needs acc, l and bias to share one
// reference, not that it be the running maximum: with m lagging by at most
// this much, every weight 2^(s - m) stays below 2^8, far inside fp32, and the
// per-wave rescale of the accumulators (taken whenever any of the wave's
// lanes moves) runs after the first sub-chunk only where a score jumps by
// more than 8, instead of on most sub-chunks of a long stream.
constexpr float kMaxLag = 8.0f;

// Fold new scores s[0..N) into the state: if any lane's scores pass its
// reference by more than kMaxLag, every lane rescales (by 1 where its own
// reference did not move).
template <int CPW, int N>
__device__ __forceinline__ void update_max(LaneState<CPW> &st, const float *s) {
  float mc = st.m;
#pragma unroll
  for (int i = 0; i < N; ++i) mc = fmaxf(mc, s[i]);
  const bool grow = mc > st.m + kMaxLag;  // always on a lane's first finite score
  if (__ballot(grow) != 0) {
    // 1 where this lane's reference did not move, 0 on its first tokens
    // (m = -inf)
    const float corr = grow ? exp2_fast(st.m - mc) : 1.0f;
    st.m = grow ? mc : st.m;
    st.l *= corr;
    st.bias *= corr;
#pragma unroll
    for (int i = 0; i < CPW; ++i) st.acc[i] *= corr;
  }
}

// Issue priority of a wave that has done `done` of its `total` sub-chunks:
// 3 at the start, falling to 0 near the end.  The SIMD's arbiter prefers
// higher priority and then older waves; without this the older wave of a
// SIMD races ahead and the younger one finishes alone, its memory latency
// then no longer hidden by any other wave.  With it, the waves sharing a
// SIMD stay within about a quarter of their work of each other.
__device__ __forceinline__ void set_progress_priority(int done, int total) {
  const int lvl = total > 0 ? 3 - min(3, (4 * done) / total) : 0;
  if (lvl >= 3) __builtin_amdgcn_s_setprio(3);
  else if (lvl == 2) __builtin_amdgcn_s_setprio(2);
  else if (lvl == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Issue priority from the wave's lead over the slowest wave of its
// workgroup: each wave posts the number of sub-chunks it has started in
// prog[wave]; the slowest gets 3, one less per sub-chunk of lead.  With the
// fraction-based levels above the waves of a SIMD still drift a quarter of
// their work apart (on 32 sub-chunks per wave, the younger four waves ended
// 6 µs after the older four in a 50 µs compute-only run).  Priority only
// orders issue, never results; an unwritten slot at the start (left over in
// LDS) can only mis-set a priority until every wave has posted once.
__device__ __forceinline__ void set_lead_priority(int *prog, int wv, int lane, int done) {
  if (lane == 0) prog[wv] = done;
  int v = lane < kDecodeWaves ? prog[lane] : 0x7fffffff;
  v = min(v, (int)dppu<0xB1>((uint32_t)v));
  v = min(v, (int)dppu<0x4E>((uint32_t)v));
  v = min(v, (int)dppu<0x141>((uint32_t)v));
  const int lead = done - __builtin_amdgcn_readlane(v, 0);
  if (lead <= 0) __builtin_amdgcn_s_setprio(3);
  else if (lead == 1) __builtin_amdgcn_s_setprio(2);
  else if (lead == 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Per-wave stream over the quantized tokens of one (sequence, head): this
// wave's sub-chunks are gw, gw + nw, gw + 2 nw, ... (n of them).
template <int BITS, int G>
struct QuantStream {
  using C = DecCfg<BITS, G>;
  const void *kc, *vc, *ks, *kz, *vs, *vz;  // (sequence, head) regions
  uint32_t code_bytes, meta_bytes;          // region sizes
  uint32_t code_voff, vmeta_voff, kmeta_voff;  // per-lane byte offsets inside a tile
  int ql, last_tile, gw, nw, n;

  __device__ __forceinline__ int t0(int c) const { return (gw + c * nw) * C::SUB; }

  // Issue every load of sub-chunk c, back to back.  For c >= n the loads go
  // through zero-record descriptors (no memory traffic).  Token indices past
  // the last valid one are clamped to valid ones; their data is never used.
  // `extra` (zero) is added to every per-lane offset: a zero computed from
  // another load's data makes these loads wait for that one.
  __device__ __forceinline__ void issue(SubLoads<BITS, G> &b, int c, uint32_t extra = 0u) const {
    constexpr int A = load_aux<BITS>();
    const bool live = c < n;
    const uint32_t cb = live ? code_bytes : 0u, mb = live ? meta_bytes : 0u;
    const int T0 = live ? t0(c) : 0;
    const int nvl = max(1, min(C::NL, (ql - T0) / C::TPL));
    const int tile0 = T0 / G;
    const rsrc_t rks = make_rsrc(ks, mb), rkz = make_rsrc(kz, mb);
    const rsrc_t rkc = make_rsrc(kc, cb), rvc = make_rsrc(vc, cb);
    const rsrc_t rvs = make_rsrc(vs, mb), rvz = make_rsrc(vz, mb);
#pragma unroll
    for (int k = 0; k < C::NTS; ++k) {
      const uint32_t so = (uint32_t)max(0, min(tile0 + k, last_tile)) * (kD * 2);
      b.ks[k] = bload1<A>(rks, kmeta_voff + extra, so);
      b.kz[k] = bload1<A>(rkz, kmeta_voff + extra, so);
    }
#pragma unroll
    for (int j = 0; j < C::NL; ++j) {
      const int t = T0 + min(j, nvl - 1) * C::TPL;
      b.kc[j] = bload4<A>(rkc, code_voff + extra, (uint32_t)((t / G) * (C::W * G) + t % G) * 4);
    }
#pragma unroll
    for (int j = 0; j < C::NL; ++j) {
      const int t = T0 + min(j, nvl - 1) * C::TPL;
      b.vc[j] = bload4<A>(rvc, code_voff + extra, (uint32_t)((t / G) * (C::W * G) + t % G) * 4);
      const uint32_t mo = (uint32_t)((t / G) * kD + t % G) * 2;
      b.vs[j] = bload2<A>(rvs, vmeta_voff + extra, mo);
      b.vz[j] = bload2<A>(rvz, vmeta_voff + extra, mo);
    }
  }

  // Sub-chunk c's loads before the lengths are known (ql, last_tile and n
  // unset), as if the cache held tokens up to the sub-chunk's end: when
  // t0(c) + SUB <= ql these are exactly the loads of issue(b, c).  A
  // sub-chunk that does not fit below cap reads zeros through zero-record
  // descriptors, so no address leaves the (sequence, head) region.
  __device__ __forceinline__ void issue_whole(SubLoads<BITS, G> &b, int c, int cap) const {
    constexpr int A = load_aux<BITS>();
    const bool fits = t0(c) + C::SUB <= cap;
    const uint32_t cb = fits ? code_bytes : 0u, mb = fits ? meta_bytes : 0u;
    const int T0 = fits ? t0(c) : 0;
    const int tile0 = T0 / G;
    const rsrc_t rks = make_rsrc(ks, mb), rkz = make_rsrc(kz, mb);
    const rsrc_t rkc = make_rsrc(kc, cb), rvc = make_rsrc(vc, cb);
    const rsrc_t rvs = make_rsrc(vs, mb), rvz = make_rsrc(vz, mb);
#pragma unroll
    for (int k = 0; k < C::NTS; ++k) {
      const uint32_t so = (uint32_t)(tile0 + k) * (kD * 2);
      b.ks[k] = bload1<A>(rks, kmeta_voff, so);
      b.kz[k] = bload1<A>(rkz, kmeta_voff, so);
    }
#pragma unroll
    for (int j = 0; j < C::NL; ++j) {
      const int t = T0 + j * C::TPL;
      b.kc[j] = bload4<A>(rkc, code_voff, (uint32_t)((t / G) * (C::W * G) + t % G) * 4);
    }
#pragma unroll
    for (int j = 0; j < C::NL; ++j) {
      const int t = T0 + j * C::TPL;
      b.vc[j] = bload4<A>(rvc, code_voff, (uint32_t)((t / G) * (C::W * G) + t % G) * 4);
      const uint32_t mo = (uint32_t)((t / G) * kD + t % G) * 2;
      b.vs[j] = bload2<A>(rvs, vmeta_voff, mo);
      b.vz[j] = bload2<A>(rvz, vmeta_voff, mo);
    }
  }
};

// ------------------------------------------ decode: keys stored pre-rotation
// Keys quantized before the rotary embedding and rotated after
// dequantization: key token t (position t in the sequence, window tokens
// after the quantized ones) is rotated by angle t * theta_f in channel pair
// f = (2f, 2f + 1), theta_f = base^(-2f/D), and the query arrives rotated.
// Rather than rotating every key, the score uses the query turned back by
// the key's angle: q . R(t) k = (R(t)^T q) . k = u_t . k, per pair
//   u[2f] = q[2f] cos + q[2f+1] sin,  u[2f+1] = q[2f+1] cos - q[2f] sin.
// The dequantization k = z + c * s then folds in as with unrotated keys, per
// token instead of per key group: score = sum_d u_d z_d + sum_d (u_d s_d) c_d.
// A lane's angles come from revolutions frac(t * theta_f / 2 pi) formed in
// fp64 (exact enough at any 32-bit position) and the hardware sine and
// cosine; the next three tokens of a lane's quad step u by the fixed
// rotation R(theta_f)^T in fp32.
template <int CPW>
struct RopeLane {
  const float *q;         // the lane's rotated query channels (x sm_scale log2 e), in LDS
  double rev[CPW / 2];    // theta_f / (2 pi) of the lane's pairs
  float cs[CPW / 2], sn[CPW / 2];  // cos and sin of theta_f
  int pos0;               // position of the sequence's first cache token

  // first channel c0 of the lane; qs: the wave's scaled query in LDS
  __device__ __forceinline__ void init(const float *qs, int c0, double log2_base, int p0) {
    q = qs + c0;
    pos0 = p0;
#pragma unroll
    for (int j = 0; j < CPW / 2; ++j) {
      const int f = c0 / 2 + j;
      const double th = exp2(-(2.0 * f / kD) * log2_base);
      rev[j] = th * 0.15915494309189535;  // 1 / (2 pi)
      cs[j] = (float)cos(th);
      sn[j] = (float)sin(th);
    }
  }
  // u = the query turned back by the angles of cache token p (position
  // pos0 + p)
  __device__ __forceinline__ void at(float (&u)[CPW], int p) const {
#pragma unroll
    for (int j = 0; j < CPW / 2; ++j) {
      double x = (double)(pos0 + p) * rev[j];
      x -= floor(x);
      const float xf = (float)x;
      const float c = __builtin_amdgcn_cosf(xf), s = __builtin_amdgcn_sinf(xf);
      const float2 qq = *reinterpret_cast<const float2 *>(q + 2 * j);
      u[2 * j] = fmaf(qq.x, c, qq.y * s);
      u[2 * j + 1] = fmaf(qq.y, c, -(qq.x * s));
    }
  }
  // u for the next position
  __device__ __forceinline__ void step(float (&u)[CPW]) const {
#pragma unroll
    for (int j = 0; j < CPW / 2; ++j) {
      const float a = u[2 * j], b = u[2 * j + 1];
      u[2 * j] = fmaf(a, cs[j], b * sn[j]);
      u[2 * j + 1] = fmaf(b, cs[j], -(a * sn[j]));
    }
  }
};

// kh[i] = z[i] + sv[i] * (channel i's code as a masked half) over a word's
// channels: the key dequantized (sv is the step times the code-offset
// factor, as staged for the pre-rotation scores).
template <int BITS, int P = 0>
__device__ __forceinline__ void dequant_word(uint32_t u, uint32_t uh, const float *sv,
                                             const float *z, float *kh) {
  constexpr int HP = 16 / BITS;
  if constexpr (P < HP) {
    const uint32_t m = pair_bits<BITS, P>(u, uh);
    kh[P] = mix_lo(sv[P], m, z[P]);
    kh[P + HP] = mix_hi(sv[P + HP], m, z[P + HP]);
    dequant_word<BITS, P + 1>(u, uh, sv, z, kh);
  }
}

// Scores of one sub-chunk with keys stored pre-rotation: staging of the
// touched tiles' steps (times the code-offset factor) and zero-points in
// LDS, then per token u, the multipliers u * s and the bias u . z.
template <int BITS, int G>
__device__ __forceinline__ void rope_scores(const SubLoads<BITS, G> &b, int T0, int nvl, int lane,
                                            float (&qp)[DecCfg<BITS, G>::NTS][DecCfg<BITS, G>::W *
                                                                             DecCfg<BITS, G>::QPW],
                                            float (&zz)[DecCfg<BITS, G>::NTS][DecCfg<BITS, G>::W *
                                                                             DecCfg<BITS, G>::QPW],
                                            const RopeLane<DecCfg<BITS, G>::CPW> &rl,
                                            float (&s)[DecCfg<BITS, G>::NL * 4]) {
  using C = DecCfg<BITS, G>;
  const int w = lane % C::W, slot = lane / C::W;
  const int d0 = 2 * lane;
  const int qpo = (d0 / C::CPW) * C::QPW + d0 % C::CPW;
#pragma unroll
  for (int k = 0; k < C::NTS; ++k) {
    qp[k][qpo] = mix_lo(code_factor<BITS>(d0 % C::CPW), b.ks[k], 0.0f);
    qp[k][qpo + 1] = mix_hi(code_factor<BITS>((d0 + 1) % C::CPW), b.ks[k], 0.0f);
    const half2_t z2 = __builtin_bit_cast(half2_t, b.kz[k]);
    zz[k][qpo] = (float)z2.x;
    zz[k][qpo + 1] = (float)z2.y;
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < C::NL; ++j) {
    if (j < nvl) {
      const int k = ((T0 % G) + j * C::TPL) / G;
      float u[C::CPW], kh[C::CPW];
      rl.at(u, T0 + j * C::TPL + 4 * slot);  // the first token of the lane's quad
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i > 0) rl.step(u);
        // the token's key channels, dequantized (z + s * c, the code taken as
        // the subnormal half it is after masking, the step carrying the
        // offset factor), then dotted with u
        const uint32_t word = u4_get(b.kc[j], i);
        dequant_word<BITS>(word, upper_pairs<BITS>(word), &qp[k][w * C::QPW], &zz[k][w * C::QPW],
                           kh);
        float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int d = 0; d < C::CPW; d += 2) {
          a0 = fmaf(u[d], kh[d], a0);
          a1 = fmaf(u[d + 1], kh[d + 1], a1);
        }
        s[4 * j + i] = lane_group_sum<C::W>(a0 + a1);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[4 * j + i] = -INFINITY;
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// Scores of one sub-chunk (every lane of a token slot ends with the full
// sums): staging of q'' = qsf * s and the zero terms of the touched tiles in
// LDS, then one dot product per token and word.
template <int BITS, int G>
__device__ __forceinline__ void plain_scores(const SubLoads<BITS, G> &b, int T0, int nvl, int lane,
                                             float qs0, float qs1, float qf0, float qf1,
                                             float (&qp)[DecCfg<BITS, G>::NTS][DecCfg<BITS, G>::W *
                                                                              DecCfg<BITS, G>::QPW],
                                             float (&cz)[DecCfg<BITS, G>::NTS][DecCfg<BITS, G>::W],
                                             float (&s)[DecCfg<BITS, G>::NL * 4]) {
  using C = DecCfg<BITS, G>;
  const int w = lane % C::W;
  const int d0 = 2 * lane;
  const int qpo = (d0 / C::CPW) * C::QPW + d0 % C::CPW;
#pragma unroll
  for (int k = 0; k < C::NTS; ++k) {
    qp[k][qpo] = mix_lo(qf0, b.ks[k], 0.0f);
    qp[k][qpo + 1] = mix_hi(qf1, b.ks[k], 0.0f);
    float zc = mix_lo(qs0, b.kz[k], mix_hi(qs1, b.kz[k], 0.0f));
    zc = lane_group_sum<C::CPW / 2>(zc);
    if ((lane % (C::CPW / 2)) == 0) cz[k][lane / (C::CPW / 2)] = zc;
  }
  __builtin_amdgcn_wave_barrier();

#pragma unroll
  for (int j = 0; j < C::NL; ++j) {
    if (j < nvl) {
      const int k = ((T0 % G) + j * C::TPL) / G;
      float qv[C::CPW];
#pragma unroll
      for (int i = 0; i < C::CPW; i += 4) {
        const float4 t4 = *reinterpret_cast<const float4 *>(&qp[k][w * C::QPW + i]);
        qv[i] = t4.x;
        qv[i + 1] = t4.y;
        qv[i + 2] = t4.z;
        qv[i + 3] = t4.w;
      }
      const float c0 = cz[k][w];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s[4 * j + i] = lane_group_sum<C::W>(dot_word<BITS>(u4_get(b.kc[j], i), qv, c0));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[4 * j + i] = -INFINITY;
    }
  }
  __builtin_amdgcn_wave_barrier();
}

template <int BITS, int G, bool ROPE = false>
__device__ __forceinline__ void process_sub(const SubLoads<BITS, G> &b, int T0, int ql, int lane,
                                            float qs0, float qs1, float qf0, float qf1,
                                            float (&qp)[DecCfg<BITS, G>::NTS][DecCfg<BITS, G>::W *
                                                                             DecCfg<BITS, G>::QPW],
                                            float (&cz)[DecCfg<BITS, G>::NTS][DecCfg<BITS, G>::W],
                                            LaneState<DecCfg<BITS, G>::CPW> &st,
                                            float (*zz)[DecCfg<BITS, G>::W * DecCfg<BITS, G>::QPW] =
                                                nullptr,
                                            const RopeLane<DecCfg<BITS, G>::CPW> *rl = nullptr) {
  using C = DecCfg<BITS, G>;
  const int nvl = min(C::NL, (ql - T0) / C::TPL);
  float s[C::NL * 4];
  if constexpr (ROPE) {
    rope_scores<BITS, G>(b, T0, nvl, lane, qp, *reinterpret_cast<float(*)[C::NTS][C::W * C::QPW]>(zz),
                         *rl, s);
  } else {
    plain_scores<BITS, G>(b, T0, nvl, lane, qs0, qs1, qf0, qf1, qp, cz, s);
  }

  update_max<C::CPW, C::NL * 4>(st, s);

  // ---- weighted value sum
#pragma unroll
  for (int j = 0; j < C::NL; ++j) {
    if (j < nvl) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2_fast(s[4 * j + i] - st.m);
        st.l += p;
        const uint32_t sw = i < 2 ? b.vs[j].x : b.vs[j].y;
        const uint32_t zw = i < 2 ? b.vz[j].x : b.vz[j].y;
        const float pp = (i & 1) ? mix_hi(p, sw, 0.0f) : mix_lo(p, sw, 0.0f);
        st.bias = (i & 1) ? mix_hi(p, zw, st.bias) : mix_lo(p, zw, st.bias);
        const uint32_t u = u4_get(b.vc[j], i);
        axpy_pairs<BITS>(u, upper_pairs<BITS>(u), pp, st.acc);
      }
    }
  }
}

// ------------------------------------------------------- decode: fp16 window
// Window tokens of one wave, one token per lane slot per step: lane
// (slot, w) holds channels w * CPW .. w * CPW + CPW - 1 of token
// begin + step * STEP + slot.  The loads of the first PF steps are issued
// before any quantized load, so they are the first to arrive.
template <int BITS, int G>
struct WinCfg {
  using C = DecCfg<BITS, G>;
  // a lane's CPW fp16 channels of one token: 16-byte vectors, or one 8-byte
  // vector when CPW = 4 (B = 8)
  static constexpr bool WIDE = C::CPW >= 8;
  using Vec = typename std::conditional<WIDE, uint4, uint2>::type;
  static constexpr int NV = WIDE ? C::CPW / 8 : 1;  // vectors per lane and token
  static constexpr int WPV = WIDE ? 4 : 2;         // half2 words per vector
  static constexpr int STEP = C::TQS;              // tokens per step
  static constexpr int PF = 16 / STEP;             // steps loaded up front (16 tokens)
};

__device__ __forceinline__ uint32_t vec_get(const uint4 &v, int i) { return u4_get(v, i); }
__device__ __forceinline__ uint32_t vec_get(const uint2 &v, int i) { return i == 0 ? v.x : v.y; }

template <int BITS, int G>
struct WinStep {
  typename WinCfg<BITS, G>::Vec k[WinCfg<BITS, G>::NV], v[WinCfg<BITS, G>::NV];
};

template <int BITS, int G>
struct WinStream {
  using WC = WinCfg<BITS, G>;
  const void *kr, *vr;  // (sequence, head) window rows
  uint32_t bytes;       // rows at or past this wave's end read as 0
  uint32_t lane_voff;   // byte offset of this lane's channels in its token row
  int begin, end;

  __device__ __forceinline__ void issue(WinStep<BITS, G> &x, int step) const {
    const rsrc_t rk = make_rsrc(kr, bytes), rv = make_rsrc(vr, bytes);
    const uint32_t vo = lane_voff + (uint32_t)(begin + step * WC::STEP) * (kD * 2);
    if constexpr (WC::WIDE) {
#pragma unroll
      for (int v = 0; v < WC::NV; ++v) x.k[v] = bload4<load_aux<BITS>()>(rk, vo + 16 * v, 0);
#pragma unroll
      for (int v = 0; v < WC::NV; ++v) x.v[v] = bload4<load_aux<BITS>()>(rv, vo + 16 * v, 0);
    } else {
      x.k[0] = bload2<load_aux<BITS>()>(rk, vo, 0);
      x.v[0] = bload2<load_aux<BITS>()>(rv, vo, 0);
    }
  }
  // one operand only (0 keys, 1 values), 16-byte rows (WIDE)
  __device__ __forceinline__ void issue_one(WinStep<BITS, G> &x, int step, int op) const {
    static_assert(WC::WIDE, "16-byte row pieces");
    const rsrc_t r = make_rsrc(op == 0 ? kr : vr, bytes);
    const uint32_t vo = lane_voff + (uint32_t)(begin + step * WC::STEP) * (kD * 2);
#pragma unroll
    for (int v = 0; v < WC::NV; ++v) (op == 0 ? x.k[v] : x.v[v]) = bload4(r, vo + 16 * v, 0);
  }
};

template <int BITS, int G>
__device__ __forceinline__ void window_step(const WinStep<BITS, G> &x, bool valid, const float *qv,
                                            LaneState<DecCfg<BITS, G>::CPW> &st) {
  using C = DecCfg<BITS, G>;
  using WC = WinCfg<BITS, G>;
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int v = 0; v < WC::NV; ++v) {
#pragma unroll
    for (int e = 0; e < WC::WPV; ++e) {
      const uint32_t u = vec_get(x.k[v], e);
      a0 = mix_lo(qv[8 * v + 2 * e], u, a0);
      a1 = mix_hi(qv[8 * v + 2 * e + 1], u, a1);
    }
  }
  float s = lane_group_sum<C::W>(a0 + a1);
  s = valid ? s : -INFINITY;
  update_max<C::CPW, 1>(st, &s);
  // absent tokens contribute 0 (and the lane's max may still be -inf)
  const float p = s > -INFINITY ? exp2_fast(s - st.m) : 0.0f;
  st.l += p;
#pragma unroll
  for (int v = 0; v < WC::NV; ++v) {
#pragma unroll
    for (int e = 0; e < WC::WPV; ++e) {
      // value sums hold channel values times 2^(e - 24) (see above)
      const uint32_t u = vec_get(x.v[v], e);
      const int c0 = 8 * v + 2 * e;
      st.acc[c0] = mix_lo(p * __builtin_ldexpf(1.0f, code_offset<BITS>(c0) - 24), u, st.acc[c0]);
      st.acc[c0 + 1] =
          mix_hi(p * __builtin_ldexpf(1.0f, code_offset<BITS>(c0 + 1) - 24), u, st.acc[c0 + 1]);
    }
  }
}

// --------------------------------------------- value queue: token by token
// With a value queue the context splits into tokens [0, vq) with quantized
// keys and values, [vq, q_len) with quantized keys and fp16 values (in the
// ring) and [q_len, T) with fp16 keys (the key window) and values.  The
// quantized stream covers whole key groups below vq; the rest, [qlq, T)
// with qlq = G * floor(vq / G), at most R + G - 1 tokens, is taken token by
// token: lane (slot, w) loads or dequantizes channels w * CPW .. of its
// token's key and value, each from wherever that token has it.

// CPW consecutive fp16 values at p (aligned to 2 * CPW bytes) as floats
template <int CPW>
__device__ __forceinline__ void load_halves(const half_t *p, float (&x)[CPW]) {
  if constexpr (CPW == 4) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const half2_t h = __builtin_bit_cast(half2_t, i < 2 ? u.x : u.y);
      x[i] = (i & 1) ? (float)h.y : (float)h.x;
    }
  } else {
#pragma unroll
    for (int v = 0; v < CPW / 8; ++v) {
      const uint4 u = reinterpret_cast<const uint4 *>(p)[v];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const half2_t h = __builtin_bit_cast(half2_t, u4_get(u, e));
        x[8 * v + 2 * e] = (float)h.x;
        x[8 * v + 2 * e + 1] = (float)h.y;
      }
    }
  }
}

template <int BITS, int G>
__device__ __forceinline__ void vq_token(const DecodeArgs &a, size_t bh, int t, bool valid, int ql,
                                         int vqn, int w, const float *qv,
                                         LaneState<DecCfg<BITS, G>::CPW> &st) {
  using C = DecCfg<BITS, G>;
  constexpr uint32_t kMask = (1u << BITS) - 1u;
  const size_t tps = (size_t)(a.cap / G);
  const size_t tile = bh * tps + (size_t)(t / G);
  const int pos = t % G;
  float k[C::CPW], v[C::CPW];
  if (t < ql) {  // quantized key: z + c * s per channel
    const uint32_t word = a.k_codes[(tile * C::W + w) * G + pos];
    float z[C::CPW], sc[C::CPW];
    load_halves<C::CPW>(a.k_zero + tile * kD + w * C::CPW, z);
    load_halves<C::CPW>(a.k_scale + tile * kD + w * C::CPW, sc);
#pragma unroll
    for (int i = 0; i < C::CPW; ++i) k[i] = fmaf((float)((word >> (i * BITS)) & kMask), sc[i], z[i]);
  } else {
    load_halves<C::CPW>(a.k_res + (bh * a.R + (t - ql)) * kD + w * C::CPW, k);
  }
  if (t < vqn) {  // quantized value: one group per token
    const uint32_t word = a.v_codes[(tile * C::W + w) * G + pos];
    const int j = (w * C::CPW) / G;
    const float z = (float)a.v_zero[tile * kD + j * G + pos];
    const float sc = (float)a.v_scale[tile * kD + j * G + pos];
#pragma unroll
    for (int i = 0; i < C::CPW; ++i) v[i] = fmaf((float)((word >> (i * BITS)) & kMask), sc, z);
  } else {
    load_halves<C::CPW>(a.v_res + (bh * a.R + (t % a.R)) * kD + w * C::CPW, v);
  }
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int d = 0; d < C::CPW; d += 2) {
    a0 = fmaf(qv[d], k[d], a0);
    a1 = fmaf(qv[d + 1], k[d + 1], a1);
  }
  float s = lane_group_sum<C::W>(a0 + a1);
  s = valid ? s : -INFINITY;
  update_max<C::CPW, 1>(st, &s);
  const float p = s > -INFINITY ? exp2_fast(s - st.m) : 0.0f;
  st.l += p;
  // value sums hold channel values times 2^(e - 24), as the window's do
#pragma unroll
  for (int i = 0; i < C::CPW; ++i)
    st.acc[i] = fmaf(p * __builtin_ldexpf(1.0f, code_offset<BITS>(i) - 24), v[i], st.acc[i]);
}

// ------------------------------------------ whole step: flush from registers
// When the step's append fills the window and every wave holds all of its
// window tokens in its prefetched registers (at most 16 per wave, R <= 128),
// the flush quantizes them from those registers instead of reading the
// window again.  Lane (slot, w) holds channels w * CPW .. w * CPW + CPW - 1
// of one token per step: exactly one key code word and one value code word.
//   values: a value group (one token, G channels) is G / CPW consecutive
//   lanes, whose minimum and maximum meet by DPP; no other wave is needed.
//   keys: a key group (one channel over the G tokens of a tile) is spread
//   over the slots and steps of the tile's G / wpw waves.  Before its
//   quantized stream, each lane reduces its own steps and stores
//   (-minimum, maximum) of its channel pairs in LDS, and each wave counts
//   itself in (a release increment of a workgroup counter).  After its
//   stream, a wave that sees every wave counted in (an acquire read)
//   reduces its tile's partials over the tile's waves and slots itself, one
//   channel pair per lane, into parameters of its own, which its lanes read
//   back for their CPW channels to encode the key words; the tile's first
//   wave writes the parameters to the cache.  No workgroup barrier is
//   involved, and the work overlaps the slower waves' streams; a wave that
//   finds the count short (it never has in practice: the partials are
//   posted long before any stream ends) does the same after the
//   workgroup's combine barrier instead.
// Minima travel negated, so that one packed fp16 maximum reduces both.

template <int BITS, int G>
struct RegFlushSmem {
  uint32_t part[kDecodeWaves][DecCfg<BITS, G>::TQS][kD / 2][2];  // [wave][slot][pair]{-min, max}
  float4 prm[kDecodeWaves][kD];  // [wave][channel]{min, step, 1/step, offset} of the wave's tile
  uint32_t arrived;              // waves whose key partials are posted
};

// LDS of the whole-step flush: the register path's, or the window-reading
// path's for longer windows (never both in one launch).
template <int BITS, int G>
union FusedFlushSmem {
  RegFlushSmem<BITS, G> reg;
  FlushSmem<G, G> lds;
};

template <int BITS, int G>
__device__ __forceinline__ FusedFlushSmem<BITS, G> &fused_flush_smem() {
  __shared__ FusedFlushSmem<BITS, G> u;
  return u;
}

// One code word from a lane's CPW fp16 channels; par(i) gives channel i's
// group {minimum, step, 1 / step, offset}.
template <int BITS, int NV, typename Par>
__device__ __forceinline__ uint32_t encode_lane_word(const uint4 (&x)[NV], Par par) {
  constexpr int CPW = 8 * NV;
  return encode_word<BITS, CPW>(
      [&](int i) {
        const half2_t h = __builtin_bit_cast(half2_t, u4_get(x[i / 8], (i % 8) / 2));
        return (i & 1) ? (float)h.y : (float)h.x;
      },
      par);
}

// Before the stream: the lane's key partials to LDS.
template <int BITS, int G>
__device__ __forceinline__ void flush_regs_key_partials(RegFlushSmem<BITS, G> &rf,
                                                        const WinStep<BITS, G> (&x)[WinCfg<BITS, G>::PF],
                                                        int wsteps, int wv, int w, int slot) {
  using WC = WinCfg<BITS, G>;
  constexpr int HW = 4 * WC::NV;  // half2 words per lane and operand
  uint32_t kmn[HW], kmx[HW];
#pragma unroll
  for (int h = 0; h < HW; ++h) kmn[h] = kmx[h] = u4_get(x[0].k[h / 4], h % 4);
#pragma unroll
  for (int i = 1; i < WC::PF; ++i)
    if (i < wsteps) {
#pragma unroll
      for (int h = 0; h < HW; ++h) {
        kmn[h] = pk_min16(kmn[h], u4_get(x[i].k[h / 4], h % 4));
        kmx[h] = pk_max16(kmx[h], u4_get(x[i].k[h / 4], h % 4));
      }
    }
  uint4 *dst = reinterpret_cast<uint4 *>(&rf.part[wv][slot][w * HW][0]);
#pragma unroll
  for (int j = 0; j < HW / 2; ++j)
    dst[j] = make_uint4(neg16x2(kmn[2 * j]), kmx[2 * j], neg16x2(kmn[2 * j + 1]), kmx[2 * j + 1]);
}

// The lane's value groups and value code words (one per step).  tile0 is the
// window's first tile in the cache; the wave's tokens [begin, begin + wsteps
// * STEP) lie in one tile.
template <int BITS, int G>
__device__ __forceinline__ void flush_regs_values(const EncodeArgs &ea,
                                                  const WinStep<BITS, G> (&x)[WinCfg<BITS, G>::PF],
                                                  int wsteps, size_t tile0, int begin, int w,
                                                  int slot) {
  using C = DecCfg<BITS, G>;
  using WC = WinCfg<BITS, G>;
  constexpr int NV = WC::NV, HW = 4 * NV;  // half2 words per lane and operand
  constexpr int LG = G / C::CPW;           // lanes per value group
  constexpr float kTop = (float)((1 << BITS) - 1);
#pragma unroll
  for (int i = 0; i < WC::PF; ++i)
    if (i < wsteps) {
      const int t = begin + i * WC::STEP + slot;  // window token
      uint32_t mn = u4_get(x[i].v[0], 0), mx = mn;
#pragma unroll
      for (int h = 1; h < HW; ++h) {
        mn = pk_min16(mn, u4_get(x[i].v[h / 4], h % 4));
        mx = pk_max16(mx, u4_get(x[i].v[h / 4], h % 4));
      }
      const uint32_t nm = pk_max16(neg16x2(mn), swap16(neg16x2(mn)));
      const uint32_t xm = pk_max16(mx, swap16(mx));
      const half2_t r =
          __builtin_bit_cast(half2_t, lane_group_pkmax<LG>((nm & 0xFFFFu) | (xm & 0xFFFF0000u)));
      const GroupParams g = group_params(-(float)r.x, (float)r.y, kTop);
      const size_t tile = tile0 + (size_t)(t / G);
      const int e = ((w * C::CPW) / G) * G + t % G;  // [group][token] inside the tile
      if (w % LG == 0) {
        ea.v_zero[tile * kD + e] = g.zero16;
        ea.v_scale[tile * kD + e] = g.scale16;
      }
      const float4 gp = make_float4(g.mn, g.s, g.rs, g.nm);
      ea.v_codes[tile * (C::W * G) + w * G + t % G] =
          encode_lane_word<BITS, NV>(x[i].v, [&](int) { return gp; });
    }
}

// One wave: the parameters of key tile T (every one of its kD / 2 channel
// pairs, lane cp taking pair cp) from the partials of the tile's nwt waves,
// into the wave's own slot of rf.prm / rf.step; with `publish`, also to the
// cache.
template <int BITS, int G>
__device__ __forceinline__ void flush_regs_tile_params(const EncodeArgs &ea,
                                                       RegFlushSmem<BITS, G> &rf, size_t tile0,
                                                       int T, int nwt, int wv, int cp,
                                                       bool publish) {
  using C = DecCfg<BITS, G>;
  constexpr float kTop = (float)((1 << BITS) - 1);
  const int u0 = T * nwt;
  uint32_t nmn = rf.part[u0][0][cp][0], mx = rf.part[u0][0][cp][1];
  for (int u = u0; u < u0 + nwt; ++u) {
    uint2 pv[C::TQS];
#pragma unroll
    for (int sl = 0; sl < C::TQS; ++sl)
      pv[sl] = *reinterpret_cast<const uint2 *>(&rf.part[u][sl][cp][0]);
#pragma unroll
    for (int sl = 0; sl < C::TQS; ++sl) {
      nmn = pk_max16(nmn, pv[sl].x);
      mx = pk_max16(mx, pv[sl].y);
    }
  }
  const half2_t hn = __builtin_bit_cast(half2_t, nmn), hx = __builtin_bit_cast(half2_t, mx);
  const GroupParams g0 = group_params(-(float)hn.x, (float)hx.x, kTop);
  const GroupParams g1 = group_params(-(float)hn.y, (float)hx.y, kTop);
  const int c = 2 * cp;
  rf.prm[wv][c] = make_float4(g0.mn, g0.s, g0.rs, g0.nm);
  rf.prm[wv][c + 1] = make_float4(g1.mn, g1.s, g1.rs, g1.nm);
  if (publish) {
    *reinterpret_cast<half2_t *>(ea.k_zero + (tile0 + T) * kD + c) = half2_t{g0.zero16, g1.zero16};
    *reinterpret_cast<half2_t *>(ea.k_scale + (tile0 + T) * kD + c) =
        half2_t{g0.scale16, g1.scale16};
  }
}

// The lane's key code words (one per step), from the parameters this wave
// computed for its tile.
template <int BITS, int G>
__device__ __forceinline__ void flush_regs_keys(const EncodeArgs &ea, const RegFlushSmem<BITS, G> &rf,
                                                const WinStep<BITS, G> (&x)[WinCfg<BITS, G>::PF],
                                                int wsteps, size_t tile0, int begin, int wv, int w,
                                                int slot) {
  using C = DecCfg<BITS, G>;
  using WC = WinCfg<BITS, G>;
  const int T = begin / G;
  const float4 *pr = &rf.prm[wv][w * C::CPW];
#pragma unroll
  for (int i = 0; i < WC::PF; ++i)
    if (i < wsteps) {
      const int t = begin + i * WC::STEP + slot;
      ea.k_codes[(tile0 + T) * (C::W * G) + w * G + t % G] =
          encode_lane_word<BITS, WC::NV>(x[i].k, [&](int c) { return pr[c]; });
    }
}

// Flush by key waves and value waves (discosf KIVI tutorial, section 3.1:
// once R tokens have collected, keys are quantized per channel over G
// tokens, values per token over G channels), B = 2 or 4, R <= 128.  Grid
// (heads, batch), one workgroup of 8 waves per full window; waves 0-3 take
// the keys, waves 4-7 the values, 32 window tokens each (waves past R / 32
// idle):
//  * key wave k holds tokens [32k, 32k + 32) column-wise, lane l taking
//    channels 2l and 2l + 1 of every token (one 4-byte load per token), so
//    the pair's minimum and maximum are in-lane packed fp16 reductions; with
//    G > 32 the tile's G / 32 key waves merge theirs through LDS behind the
//    workgroup's one barrier.  Its 2B code bits per token are packed 16 / B
//    tokens to a register, and the 16 / B lanes of each code word exchange
//    them (a transpose in log2(16 / B) lane-exchange stages), after which
//    lane j of a word's group holds that word for token j of the register;
//  * value wave v holds tokens [32v, 32v + 32) row-wise, as the whole-step
//    kernel does (flush_regs_values: groups and words per token, no LDS).
// Codes follow the same quantizer as the other encoders (group_params,
// quant_code).  Lengths, tickets and the
// commit are those of flush_kernel.  VALUES false: keys only (the value
// queue's flush).
constexpr int kFlushKeyWaves = 4;
constexpr int kFlushTokensPerWave = 32;

// One stage of the code-word transpose: lanes d apart swap chunks of cs
// bits (the odd chunks of the lane with bit d clear for the even chunks of
// its partner).
template <int D, int CS>
__device__ __forceinline__ uint32_t transpose_stage(uint32_t mine, int lane) {
  uint32_t other;
  if constexpr (D == 4)
    other = (uint32_t)__builtin_amdgcn_ds_swizzle((int)mine, 0x101F);  // lane ^ 4
  else if constexpr (D == 2)
    other = dppu<0x4E>(mine);  // lane ^ 2
  else
    other = dppu<0xB1>(mine);  // lane ^ 1
  constexpr uint32_t even = CS == 16 ? 0x0000FFFFu : CS == 8 ? 0x00FF00FFu : 0x0F0F0F0Fu;
  const bool clear = (lane & D) == 0;
  const uint32_t rot = __builtin_amdgcn_alignbit(other, other, clear ? 32 - CS : CS);
  const uint32_t keep = clear ? even : ~even;
  return (mine & keep) | (rot & ~keep);
}

template <int BITS>
__device__ __forceinline__ uint32_t transpose_words(uint32_t v, int lane) {
  if constexpr (BITS == 2) {
    v = transpose_stage<4, 16>(v, lane);
    v = transpose_stage<2, 8>(v, lane);
    return transpose_stage<1, 4>(v, lane);
  } else {
    v = transpose_stage<2, 16>(v, lane);
    return transpose_stage<1, 8>(v, lane);
  }
}

template <int BITS, int G, bool VALUES>
__global__ __launch_bounds__(kDecodeThreads, 3 * kDecodeWavesPerSimd) void flush_split_kernel(
    EncodeArgs a) {
  using C = DecCfg<BITS, G>;
  using WC = WinCfg<BITS, G>;
  static_assert(BITS == 2 || BITS == 4, "16 / B tokens per register, 16 / B lanes per word");
  static_assert(kDecodeWaves == 2 * kFlushKeyWaves, "four key waves and four value waves");
  constexpr int K = G / kFlushTokensPerWave;  // key waves per tile
  constexpr int TPR = 16 / BITS;              // tokens per register (= lanes per word)
  constexpr int NREG = kFlushTokensPerWave / TPR;
  constexpr float kTop = (float)((1 << BITS) - 1);
  __shared__ uint2 part[kFlushKeyWaves][64];  // [key wave][pair]{-min, max}
  __shared__ int lens[2];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  if (tid == 0) {
    lens[0] = a.q_len[b];
    lens[1] = a.r_len[b];
  }
  __syncthreads();
  const int ql = lens[0], rl = lens[1];
  if (!flush_ok(ql, rl, G, a.R, a.cap)) {
    if (rl == a.R && h == 0 && tid == 0)
      atomicOr(a.status, (ql < 0 || ql % G) ? KIVI_ST_BAD_LENGTH : KIVI_ST_CAPACITY);
    return;
  }
  uint32_t ticket = 0;
  if (tid == 0)
    ticket = __hip_atomic_fetch_add(a.tickets + (size_t)b * kTicketStride, 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
  const size_t bh = (size_t)b * a.heads + h;
  const size_t tile0 = bh * (size_t)(a.cap / G) + (size_t)(ql / G);
  const bool keys = wv < kFlushKeyWaves;
  const int t0 = (keys ? wv : wv - kFlushKeyWaves) * kFlushTokensPerWave;  // first window token
  const bool busy = t0 < a.R;

  if (keys) {
    // ---- key wave: channels 2 lane, 2 lane + 1 of tokens t0 .. t0 + 31
    uint32_t xr[kFlushTokensPerWave];
    const rsrc_t rk = make_rsrc(a.k_res + bh * a.R * kD, busy ? (uint32_t)a.R * kD * 2 : 0u);
#pragma unroll
    for (int r = 0; r < kFlushTokensPerWave; ++r)
      xr[r] = bload1(rk, (uint32_t)lane * 4, (uint32_t)(t0 + r) * (kD * 2));
    uint32_t mn = xr[0], mx = xr[0];
#pragma unroll
    for (int r = 1; r < kFlushTokensPerWave; ++r) {
      mn = pk_min16(mn, xr[r]);
      mx = pk_max16(mx, xr[r]);
    }
    uint32_t nmn = neg16x2(mn);
    if constexpr (K > 1) {
      part[wv][lane] = make_uint2(nmn, mx);
      __syncthreads();
      const int u0 = (wv / K) * K;
#pragma unroll
      for (int u = 0; u < K; ++u) {
        const uint2 pv = part[u0 + u][lane];
        nmn = pk_max16(nmn, pv.x);
        mx = pk_max16(mx, pv.y);
      }
    }
    if (!busy) return;
    const half2_t hn = __builtin_bit_cast(half2_t, nmn), hx = __builtin_bit_cast(half2_t, mx);
    const GroupParams g0 = group_params(-(float)hn.x, (float)hx.x, kTop);
    const GroupParams g1 = group_params(-(float)hn.y, (float)hx.y, kTop);
    const int T = t0 / G;  // the tile within the window
    if (wv % K == 0) {
      *reinterpret_cast<half2_t *>(a.k_zero + (tile0 + T) * kD + 2 * lane) =
          half2_t{g0.zero16, g1.zero16};
      *reinterpret_cast<half2_t *>(a.k_scale + (tile0 + T) * kD + 2 * lane) =
          half2_t{g0.scale16, g1.scale16};
    }
    const int w = lane / TPR, j = lane % TPR;
    uint32_t *dst = a.k_codes + (tile0 + T) * (size_t)(C::W * G) + (size_t)w * G + (t0 % G) + j;
#pragma unroll
    for (int c = 0; c < NREG; ++c) {
      // tokens c TPR .. c TPR + TPR - 1: 2B bits each, in two fp32 sums of
      // TPR / 2 tokens (16-bit integers, exact), then one register
      // (every code by the fast product first, and the register once more
      // code by code only when one of them needs the division, as
      // encode_word does)
      float lo = 0.0f, hi = 0.0f, dev = 0.0f;
      auto put = [&](int k, float c0, float c1) {
        const float f = (float)(1u << (2 * BITS * (k % (TPR / 2))));
        const float pair = fmaf(c1, (float)(1 << BITS), c0);
        if (k < TPR / 2)
          lo = fmaf(pair, f, lo);
        else
          hi = fmaf(pair, f, hi);
      };
#pragma unroll
      for (int k = 0; k < TPR; ++k) {
        const half2_t x = __builtin_bit_cast(half2_t, xr[c * TPR + k]);
        const float q0 = fmaf((float)x.x, g0.rs, g0.nm), q1 = fmaf((float)x.y, g1.rs, g1.nm);
        const float c0 = rintf(q0), c1 = rintf(q1);
        dev = fmaxf(dev, fmaxf(fabsf(q0 - c0), fabsf(q1 - c1)));
        put(k, c0, c1);
      }
      if (!(dev <= near_half<BITS>() && lo == lo && hi == hi)) {
        lo = hi = 0.0f;
#pragma unroll
        for (int k = 0; k < TPR; ++k) {
          const half2_t x = __builtin_bit_cast(half2_t, xr[c * TPR + k]);
          put(k, quant_code<BITS>((float)x.x, g0.mn, g0.s, g0.rs, g0.nm),
              quant_code<BITS>((float)x.y, g1.mn, g1.s, g1.rs, g1.nm));
        }
      }
      const uint32_t reg = (uint32_t)lo | ((uint32_t)hi << 16);
      dst[c * TPR] = transpose_words<BITS>(reg, lane);
    }
  } else {
    // ---- value wave: tokens t0 .. t0 + 31 row-wise, two halves of PF steps
    const int w = lane % C::W, slot = lane / C::W;
    WinStream<BITS, G> ws[2];
    WinStep<BITS, G> x[2][WC::PF];
    if (VALUES && busy) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        ws[hf].kr = a.k_res + bh * a.R * kD;
        ws[hf].vr = a.v_res + bh * a.R * kD;
        ws[hf].begin = t0 + 16 * hf;
        ws[hf].end = min(a.R, ws[hf].begin + 16);
        ws[hf].bytes = (uint32_t)ws[hf].end * (kD * 2);
        ws[hf].lane_voff = (uint32_t)(slot * kD + w * C::CPW) * 2;
#pragma unroll
        for (int i = 0; i < WC::PF; ++i) ws[hf].issue_one(x[hf][i], i, 1);
      }
    }
    if constexpr (K > 1) __syncthreads();  // the key waves' one barrier
    if (VALUES && busy) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        flush_regs_values<BITS, G>(a, x[hf], WC::PF, tile0, ws[hf].begin, w, slot);
    }
  }
  if (tid == 0 && ticket == (uint32_t)a.heads - 1) {
    a.q_len[b] = ql + a.R;
    a.r_len[b] = 0;
    a.tickets[(size_t)b * kTicketStride] = 0u;
  }
  if (tid == 0 && ticket >= (uint32_t)a.heads) atomicOr(a.status, KIVI_ST_TICKETS);
}

// ---- the end of a decode workgroup
// Its waves' published states combined into the workgroup's (channel tid):
// the maximum M of the log2 scores, the softmax sum L and the output
// channel's weighted sum, both relative to M.  Every published value is
// read first, then reduced: one LDS round trip instead of one per wave.
// (Every wave published finite sums, zeros without tokens, so all can be
// read before any test.)
struct WgState {
  float M, L, acc;
};

template <int BITS, int G, typename Fin>
__device__ __forceinline__ WgState combine_waves(const Fin &fin, int tid) {
  using C = DecCfg<BITS, G>;
  constexpr int NR = publish_rows<C::W>();
  float fm[kDecodeWaves], fl[kDecodeWaves];
  float ra[kDecodeWaves][NR], rb[kDecodeWaves][NR];
#pragma unroll
  for (int x = 0; x < kDecodeWaves; ++x) {
    fm[x] = fin.m[x];
    fl[x] = fin.l[x];
  }
  const int ch = tid < kD ? tid : 0;
#pragma unroll
  for (int x = 0; x < kDecodeWaves; ++x)
#pragma unroll
    for (int y = 0; y < NR; ++y) {
      ra[x][y] = fin.acc[x][y][ch];
      rb[x][y] = fin.bias[x][y][ch / C::CPW];
    }
  WgState w{-INFINITY, 0.0f, 0.0f};
#pragma unroll
  for (int x = 0; x < kDecodeWaves; ++x)
    if (fl[x] > 0.0f) w.M = fmaxf(w.M, fm[x]);
  if (w.M != -INFINITY) {
    const float cf = code_factor<BITS>(ch % C::CPW);
#pragma unroll
    for (int x = 0; x < kDecodeWaves; ++x) {
      const float ex = fl[x] > 0.0f ? exp2_fast(fm[x] - w.M) : 0.0f;
      w.L += ex * fl[x];
      float sa = 0.0f, sb = 0.0f;
#pragma unroll
      for (int y = 0; y < NR; ++y) {
        sa += ra[x][y];
        sb += rb[x][y];
      }
      w.acc += ex * fmaf(sa, cf, sb);
    }
  }
  return w;
}

// Several workgroups per (sequence, head): publish this one's state, take a
// ticket, and in the workgroup with the last ticket merge all partials.
template <typename Sm>
__device__ __forceinline__ void finish_splits(const DecodeArgs &a, Sm &sm, const WgState &wg,
                                              size_t bh, int split, int S, int tid) {
  const float M = wg.M, L = wg.L, acc_out = wg.acc;
  // The partial state is written with device-scope atomic stores, which the
  // gfx950 caches keep coherent across XCDs by themselves (they write
  // through to the device coherence point).  Waiting for their completion,
  // then a barrier, then a device-scope ticket, orders them before the
  // ticket without a device-wide release fence, whose L2 write-back and
  // invalidate would otherwise run once per wave on a shared L2.
  float *P = a.part + (bh * S + split) * (size_t)a.part_stride;
  if (L > 0.0f && tid < kD) store_agent(P + kPartHead + tid, acc_out);
  if (tid == 0) {
    store_agent(P, M);
    store_agent(P + 1, L);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (tid == 0)
    sm.ticket = (int)__hip_atomic_fetch_add(a.tickets + bh * kTicketStride, 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (sm.ticket != S - 1) {
    // a ticket at or past the split count: the workspace's counter did not
    // start at zero (workspace not initialised), so no workgroup can tell it
    // is the last; the caller is told through the status word
    if (tid == 0 && (uint32_t)sm.ticket >= (uint32_t)S) atomicOr(a.status, KIVI_ST_TICKETS);
    return;
  }

  // ---- last workgroup of this (sequence, head): merge all partials, read
  // with device-scope atomic loads (coherent with the stores above)
  const float *P0 = a.part + bh * S * (size_t)a.part_stride;
  if (tid < S) {
    sm.u.mg.m[tid] = load_agent(P0 + (size_t)tid * a.part_stride);
    sm.u.mg.l[tid] = load_agent(P0 + (size_t)tid * a.part_stride + 1);
  }
  __syncthreads();
  if (tid < kD) {
    float mx = -INFINITY;
    for (int s = 0; s < S; ++s)
      if (sm.u.mg.l[s] > 0.0f) mx = fmaxf(mx, sm.u.mg.m[s]);
    float lsum = 0.0f, macc = 0.0f;
    for (int s = 0; s < S; ++s) {
      const float e = sm.u.mg.l[s] > 0.0f ? exp2_fast(sm.u.mg.m[s] - mx) : 0.0f;
      lsum += e * sm.u.mg.l[s];
      if (e != 0.0f)
        macc = fmaf(e, load_agent(P0 + (size_t)s * a.part_stride + kPartHead + tid), macc);
    }
    a.out[bh * kD + tid] = lsum > 0.0f ? macc / lsum : 0.0f;
  }
  if (tid == 0)
    __hip_atomic_store(a.tickets + bh * kTicketStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Longest first: the index of the sequence of rank r when the batch is
// ordered by its bytes (quantized tokens, plus 8 per window token, whose fp16
// rows weigh about 8 times as much), longest first, ties by index.  The
// ranks are a permutation, so every sequence still gets every workgroup of
// its own; workgroups are dispatched in grid order, so the longest
// sequences start first and the shortest end the launch.
constexpr int kLptMax = 256;
__device__ __forceinline__ int lpt_sequence(const DecodeArgs &a, int r, int tid, int *lens_s,
                                            int *order_s) {
  const int n = a.lpt_batch;
  for (int i = tid; i < n; i += kDecodeThreads) lens_s[i] = a.q_len[i] + 8 * a.r_len[i];
  __syncthreads();
  for (int i = tid; i < n; i += kDecodeThreads) {
    const int li = lens_s[i];
    int rk = 0;
    for (int j = 0; j < n; ++j) {
      const int lj = lens_s[j];
      rk += (lj > li || (lj == li && j < i)) ? 1 : 0;
    }
    order_s[rk] = i;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(order_s[r]);
}

// DEPTH: sub-chunks whose loads each wave keeps in flight.  2 when the grid
// is one workgroup per compute unit; 1 when it is larger, where the smaller
// register footprint lets three workgroups share a compute unit (measured on
// the 13B layer, 640 workgroups: 37 us at depth 1 against 45 us at depth 2;
// on the 7B layer, 256 workgroups, depth 2 is the faster).  Depth 1 asks for
// six waves per SIMD, which caps it at 80 VGPRs (registers are allocated in
// blocks of 8 out of 512): at 82 it held only five, two workgroups per
// compute unit, and the 13B layer's last 128 workgroups ran as a second
// round (per-workgroup timestamps: started at 22 us); with three per
// compute unit all 640 start at once (37.7 -> 34.3 us).
// ROPE: keys are stored before the rotary embedding (RopeLane above).
// VQ: the cache keeps a value queue (vq_token above).
template <int BITS, int G, bool FUSED, int DEPTH, bool ROPE = false, bool VQ = false>
__global__ __launch_bounds__(kDecodeThreads, DEPTH == 1 ? (ROPE || VQ ? 2 : 3) * kDecodeWavesPerSimd : kDecodeWavesPerSimd) void decode_kernel(
    DecodeArgs a, EncodeArgs ea) {
  constexpr int kDecodeDepth = DEPTH;
  using C = DecCfg<BITS, G>;
  using WC = WinCfg<BITS, G>;
  static_assert(!FUSED || WC::WIDE, "the whole-step kernel holds window rows as 16-byte vectors");
  static_assert(!(FUSED && ROPE), "keys stored pre-rotation: the step is three kernels");
  static_assert(!(VQ && (FUSED || ROPE)), "the value queue has the plain decode only");
  __shared__ DecSmem<BITS, G, ROPE> sm;
  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const int split = blockIdx.x, h = blockIdx.y;
  int b = blockIdx.z;
  if constexpr (!FUSED) {
    __shared__ int lpt_lens[kLptMax], lpt_order[kLptMax];
    if (a.lpt_batch > 0) b = lpt_sequence(a, blockIdx.z, threadIdx.x, lpt_lens, lpt_order);
  }
  const size_t bh = (size_t)b * a.heads + h;
  const int S = a.splits;

  // ---- this wave's share: quantized sub-chunks gw, gw + nw, ... and
  // window tokens [gw * win_per_wave, (gw + 1) * win_per_wave)
  const int w = lane % C::W, slot = lane / C::W;
  const int jg = (w * C::CPW) / G;
  const size_t tps = (size_t)(a.cap / G);
  QuantStream<BITS, G> qs;
  qs.kc = a.k_codes + bh * tps * (C::W * G);
  qs.vc = a.v_codes + bh * tps * (C::W * G);
  qs.ks = a.k_scale + bh * tps * kD;
  qs.kz = a.k_zero + bh * tps * kD;
  qs.vs = a.v_scale + bh * tps * kD;
  qs.vz = a.v_zero + bh * tps * kD;
  qs.code_bytes = (uint32_t)(tps * (C::W * G) * 4);
  qs.meta_bytes = (uint32_t)(tps * kD * 2);
  qs.code_voff = (uint32_t)(w * G + 4 * slot) * 4;
  qs.vmeta_voff = (uint32_t)(jg * G + 4 * slot) * 2;
  qs.kmeta_voff = (uint32_t)lane * 4;
  qs.gw = split * kDecodeWaves + wv;
  qs.nw = kDecodeWaves * S;
  const uint32_t qraw = bload1(make_rsrc(a.q + bh * kD, kD * 2), (uint32_t)lane * 4, 0);
  // Every decode, the whole step included, requests its first sub-chunk
  // before the lengths arrive (their load is a round trip at the start of
  // every wave, through LDS and a barrier in the whole step), as if the cache
  // held it whole; it is requested again below when it does not.
  SubLoads<BITS, G> ring[kDecodeDepth];
  qs.issue_whole(ring[0], 0, a.cap);

  int ql, rl;
  if constexpr (FUSED) {
    // the lengths this kernel commits: thread 0 reads them and hands them to
    // every wave behind a barrier, so every read of them in this workgroup
    // comes before its ticket (and so before any workgroup commits)
    if (tid == 0) {
      sm.lens[0] = a.q_len[b];
      sm.lens[1] = a.r_len[b];
      fused_flush_smem<BITS, G>().reg.arrived = 0u;
    }
    __syncthreads();
    ql = sm.lens[0];
    rl = sm.lens[1];
  } else {
    // both loads out before either is waited for
    ql = a.q_len[b];
    rl = a.r_len[b];
    __builtin_amdgcn_sched_barrier(0);
  }
  // Whole step (FUSED, one workgroup per (sequence, head)): append the new
  // token at window slot rnew, decode over the window including it, and
  // flush the window if that filled it; the same results as the three
  // separate calls.  The new token's row is written to the cache, and used
  // from registers wherever this kernel needs it.
  const int ql0 = ql;
  int rl1 = rl;  // window length after the append (FUSED)
  int rnew = -1;
  bool flush = false, commit = false;
  uint32_t ticket = 0;
  const uint4 *knew = nullptr, *vnew = nullptr;
  if constexpr (FUSED) {
    knew = reinterpret_cast<const uint4 *>(a.k_new + bh * kD);
    vnew = reinterpret_cast<const uint4 *>(a.v_new + bh * kD);
    if (rl >= 0 && rl < a.R) {
      // the row itself is written from the registers that hold it for the
      // attention (store_new below), not by a load and a store here, whose
      // wait would stall the first wave at the start
      rnew = rl;
      rl += 1;
      commit = true;
    } else if (h == 0 && tid == 0) {
      atomicOr(a.status, rl < 0 ? KIVI_ST_BAD_LENGTH : KIVI_ST_RESIDUAL_FULL);
    }
    flush = flush_ok(ql, rl, G, a.R, a.cap);
    if (!flush && rl == a.R && h == 0 && tid == 0)
      atomicOr(a.status, (ql < 0 || ql % G) ? KIVI_ST_BAD_LENGTH : KIVI_ST_CAPACITY);
    commit = commit || flush;
    rl1 = rl;
    // every workgroup of the sequence takes a ticket once it has read the
    // lengths; the one with the last ticket writes the new lengths at the end
    if (commit && tid == 0)
      ticket = __hip_atomic_fetch_add(ea.tickets + (size_t)b * kTicketStride, 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
  }
  // (one test of both lengths, so that neither load waits on the other)
  const bool lens_ok = (ql >= 0) & (ql <= a.cap) & ((ql % G) == 0) & (rl >= 0) & (rl <= a.R);
  if (!lens_ok) {
    if (split == 0 && h == 0 && tid == 0) atomicOr(a.status, KIVI_ST_BAD_LENGTH);
    ql = 0;
    rl = 0;
  }

  // value queue: values are quantized for tokens [0, vqn); the quantized
  // stream covers the whole key groups below that, [0, qlq)
  [[maybe_unused]] int vqn = 0;
  int qlq = ql;
  if constexpr (VQ) {
    vqn = max(0, ql + rl - a.R);
    qlq = (vqn / G) * G;
  }

  qs.ql = qlq;
  qs.last_tile = qlq / G - 1;
  qs.n = qs.gw * C::SUB < qlq ? (qlq - qs.gw * C::SUB + qs.nw * C::SUB - 1) / (qs.nw * C::SUB) : 0;

  WinStream<BITS, G> ws;
  ws.kr = a.k_res + bh * a.R * kD;
  ws.vr = a.v_res + bh * a.R * kD;
  ws.begin = qs.gw * a.win_per_wave;
  ws.end = VQ ? ws.begin : min(rl, ws.begin + a.win_per_wave);  // VQ: no window pass
  ws.bytes = (uint32_t)max(0, ws.end) * (kD * 2);
  ws.lane_voff = (uint32_t)(slot * kD + w * C::CPW) * 2;
  const int wsteps = ws.end > ws.begin ? (ws.end - ws.begin + WC::STEP - 1) / WC::STEP : 0;


  // The query (every wave reads it: lane i holds channels 2i, 2i + 1),
  // then kDecodeDepth quantized sub-chunks.  Each sub-chunk's registers are
  // refilled with sub-chunk c + kDecodeDepth as soon as sub-chunk c is done,
  // so kDecodeDepth - 1 stay in flight while one is computed.  The fp16
  // window tokens come last: their loads are issued once the quantized
  // loads are all out, and they are computed after the quantized tokens.
  // (Issuing everything up front would not help: the memory system serves
  // all waves' requests interleaved, so the first data a wave needs would
  // arrive no sooner than the rest.)
  // Except in a whole step whose append fills a window of at most 128
  // tokens ("early"): there the window comes first -- its loads right after
  // the first sub-chunk's (requested before the lengths), then its
  // attention and the whole flush (quantized from the window registers)
  // while the first quantized sub-chunks are in flight; after the last
  // quantized byte, the flush's arithmetic would run with HBM idle.
  [[maybe_unused]] const size_t tile0 = bh * tps + (size_t)(ql0 / G);
  bool early = false;
  if constexpr (FUSED) early = flush && a.win_per_wave <= 16;

  // FUSED: this lane's channels of the appended token, loaded unconditionally
  // (a load under a branch would make the compiler wait for every load in
  // flight after it)
  [[maybe_unused]] WinStep<BITS, G> xnew;
  if constexpr (FUSED) {
#pragma unroll
    for (int v = 0; v < WC::NV; ++v) {
      xnew.k[v] = knew[(w * C::CPW) / 8 + v];
      xnew.v[v] = vnew[(w * C::CPW) / 8 + v];
    }
  }
  WinStep<BITS, G> wpf[WC::PF];
  if (early) {
#pragma unroll
    for (int i = 0; i < WC::PF; ++i) ws.issue(wpf[i], i);
  }
  // Only the first sub-chunk's loads are out so far (again now where the
  // sequence ends inside it); the rest of the ring follows once it has
  // arrived (below).  Every wave requesting its whole ring at the start
  // makes the memory system serve all of it interleaved, so the first
  // sub-chunk would arrive no sooner than the others; with half the request
  // the waves start computing earlier (7B layer 25.4 -> 24.8 us, 131072
  // tokens at B=2 80.3 -> 77.9 us, alternating runs on one box).
  if (qs.t0(0) + C::SUB > qs.ql) qs.issue(ring[0], 0);

  auto &stg = sm.u.wave[wv];
#if KIVI_DECODE_PRIORITY == 2
  if (lane == 0) sm.prog[wv] = 0;
#endif
  const half2_t hq = __builtin_bit_cast(half2_t, qraw);
  const float qs0 = (float)hq.x * a.qscale, qs1 = (float)hq.y * a.qscale;
  const float qf0 = qs0 * code_factor<BITS>((2 * lane) % C::CPW);
  const float qf1 = qs1 * code_factor<BITS>((2 * lane + 1) % C::CPW);
  stg.qs[2 * lane] = qs0;  // for the window tokens
  stg.qs[2 * lane + 1] = qs1;
  [[maybe_unused]] RopeLane<C::CPW> rope;
  if constexpr (ROPE) {
    __builtin_amdgcn_wave_barrier();
    rope.init(stg.qs, w * C::CPW, a.rope_log2_base, a.n_sink);
  }
  auto *zz = reinterpret_cast<float(*)[C::W * C::QPW]>(&sm.zz[ROPE ? wv : 0][0][0]);

  LaneState<C::CPW> st;
  st.m = -INFINITY;
  st.l = 0.0f;
  st.bias = 0.0f;
#pragma unroll
  for (int i = 0; i < C::CPW; ++i) st.acc[i] = 0.0f;

  // the wave's window tokens; the appended token (FUSED) comes from
  // registers, not from the cache
  auto window = [&]() {
    if (wsteps <= 0) return;
    __builtin_amdgcn_wave_barrier();
    float qv[C::CPW];
#pragma unroll
    for (int i = 0; i < C::CPW; ++i) qv[i] = stg.qs[w * C::CPW + i];
    auto fresh = [&](WinStep<BITS, G> &x, int i) {
      if constexpr (FUSED) {
        const bool hit = ws.begin + i * WC::STEP + slot == rnew;
#pragma unroll
        for (int v = 0; v < WC::NV; ++v) {
          x.k[v] = sel4(hit, xnew.k[v], x.k[v]);
          x.v[v] = sel4(hit, xnew.v[v], x.v[v]);
        }
      }
    };
    // keys stored pre-rotation: the query turned back by the token's
    // position (quantized tokens first, so window slot r is position ql + r)
    auto step = [&](const WinStep<BITS, G> &x, int i) {
      const int r = ws.begin + i * WC::STEP + slot;
      if constexpr (ROPE) {
        float u[C::CPW];
        rope.at(u, ql + r);
        window_step<BITS, G>(x, r < ws.end, u, st);
      } else {
        window_step<BITS, G>(x, r < ws.end, qv, st);
      }
    };
#pragma unroll
    for (int i = 0; i < WC::PF; ++i)
      if (i < wsteps) {
        fresh(wpf[i], i);
        step(wpf[i], i);
      }
    for (int i = WC::PF; i < wsteps; ++i) {  // windows longer than the prefetched steps
      WinStep<BITS, G> x;
      ws.issue(x, i);
      fresh(x, i);
      step(x, i);
    }
  };

  // FUSED: the appended row into window slot rnew of the cache, from the
  // registers of wave 0's first token slot (lane w holds channels w * CPW ..)
  [[maybe_unused]] auto store_new = [&]() {
    if constexpr (FUSED) {
      if (rnew >= 0 && wv == 0 && slot == 0) {
        uint4 *kd = reinterpret_cast<uint4 *>(ea.k_res + (bh * a.R + rnew) * kD + w * C::CPW);
        uint4 *vd = reinterpret_cast<uint4 *>(ea.v_res + (bh * a.R + rnew) * kD + w * C::CPW);
#pragma unroll
        for (int v = 0; v < WC::NV; ++v) {
          kd[v] = xnew.k[v];
          vd[v] = xnew.v[v];
        }
      }
    }
  };

  // Whole rounds of kDecodeDepth sub-chunks (no branch inside a round, so
  // the wait before each sub-chunk only covers its own loads), then the
  // remaining n mod kDecodeDepth, whose loads are already in flight.
  int c0 = 0;
  // FUSED, early: this wave's key partials before its stream (its window
  // rows arrive ahead of its first sub-chunk, so waiting for them costs
  // nothing), then the wave counts itself in
  [[maybe_unused]] const int nwt = a.win_per_wave > 0 ? G / a.win_per_wave : 1;
  [[maybe_unused]] const int tileT = ws.begin / G;
  [[maybe_unused]] bool keys_done = true;
  // this wave's key tile parameters and key words, if every wave has posted
  // its key partials (an acquire read of the count)
  [[maybe_unused]] auto try_keys = [&]() {
    if constexpr (FUSED) {
      auto &rf = fused_flush_smem<BITS, G>().reg;
      const uint32_t in = (uint32_t)__builtin_amdgcn_readfirstlane((int)__hip_atomic_load(
          &rf.arrived, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
      if (in != (uint32_t)kDecodeWaves) return false;
      flush_regs_tile_params<BITS, G>(ea, rf, tile0, tileT, nwt, wv, lane, wv % nwt == 0);
      flush_regs_keys<BITS, G>(ea, rf, wpf, wsteps, tile0, ws.begin, wv, w, slot);
    }
    return true;
  };
  if constexpr (FUSED) {
    if (early) {
      auto &rf = fused_flush_smem<BITS, G>().reg;
      // the appended token's row replaces its slot's stale one first (the
      // window pass does the same later; doing it twice is harmless)
#pragma unroll
      for (int i = 0; i < WC::PF; ++i) {
        const bool hit = ws.begin + i * WC::STEP + slot == rnew;
#pragma unroll
        for (int v = 0; v < WC::NV; ++v) {
          wpf[i].k[v] = sel4(hit, xnew.k[v], wpf[i].k[v]);
          wpf[i].v[v] = sel4(hit, xnew.v[v], wpf[i].v[v]);
        }
      }
      if (wsteps > 0) flush_regs_key_partials<BITS, G>(rf, wpf, wsteps, wv, w, slot);
      if (lane == 0)
        __hip_atomic_fetch_add(&rf.arrived, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      // then, while the first sub-chunk is in flight (the vector units would
      // otherwise wait for it), the window's attention, the flush's value
      // words, and its key words if every wave has posted its partials
      // (else after the stream, or after the combine barrier)
      window();
      store_new();
      if (wsteps > 0) {
        flush_regs_values<BITS, G>(ea, wpf, wsteps, tile0, ws.begin, w, slot);
        keys_done = try_keys();
      }
    }
  }
  if constexpr (kDecodeDepth > 1) {
    // the rest of the ring once sub-chunk 0 is in: an offset of zero that
    // depends on its last load
    uint32_t z;
    asm volatile("v_and_b32 %0, 0, %1" : "=v"(z) : "v"(ring[0].vz[C::NL - 1].y));
#pragma unroll
    for (int k = 1; k < kDecodeDepth; ++k) qs.issue(ring[k], k, z);
  }
  for (; c0 + kDecodeDepth <= qs.n; c0 += kDecodeDepth) {
#pragma unroll
    for (int k = 0; k < kDecodeDepth; ++k) {
#if KIVI_DECODE_PRIORITY == 2
      set_lead_priority(sm.prog, wv, lane, c0 + k);
#elif KIVI_DECODE_PRIORITY
      set_progress_priority(c0 + k, qs.n);
#endif
      process_sub<BITS, G, ROPE>(ring[k], qs.t0(c0 + k), qs.ql, lane, qs0, qs1, qf0, qf1, stg.qp,
                                 stg.cz, st, zz, &rope);
      qs.issue(ring[k], c0 + k + kDecodeDepth);
    }
  }
  if (!early) {
#pragma unroll
    for (int i = 0; i < WC::PF; ++i) ws.issue(wpf[i], i);
  }
#pragma unroll
  for (int k = 0; k < kDecodeDepth - 1; ++k)
    if (c0 + k < qs.n) {
#if KIVI_DECODE_PRIORITY == 2
      set_lead_priority(sm.prog, wv, lane, c0 + k);
#elif KIVI_DECODE_PRIORITY
      set_progress_priority(c0 + k, qs.n);
#endif
      process_sub<BITS, G, ROPE>(ring[k], qs.t0(c0 + k), qs.ql, lane, qs0, qs1, qf0, qf1, stg.qp,
                                 stg.cz, st, zz, &rope);
    }
#if KIVI_DECODE_PRIORITY
  __builtin_amdgcn_s_setprio(0);
#endif
  if constexpr (VQ) {
    // tokens [qlq, T) one at a time, this wave's share of them
    const int ub = qs.gw * a.win_per_wave, ue = min(ql + rl - qlq, ub + a.win_per_wave);
    if (ue > ub) {
      __builtin_amdgcn_wave_barrier();
      float qv[C::CPW];
#pragma unroll
      for (int i = 0; i < C::CPW; ++i) qv[i] = stg.qs[w * C::CPW + i];
      for (int u0 = ub; u0 < ue; u0 += WC::STEP) {
        const int u = u0 + slot;
        const bool valid = u < ue;
        vq_token<BITS, G>(a, bh, qlq + (valid ? u : ub), valid, ql, vqn, w, qv, st);
      }
    }
  } else if (!early) {
    window();
    store_new();
  } else if constexpr (FUSED) {
    // early: the key words, if the partials were not all posted before the
    // stream
    if (!keys_done) keys_done = try_keys();
  }
  // fp16 sink tokens (the sequence's first tokens, kept unquantized ahead of
  // the quantized ones, at positions 0 .. n_sink - 1): this wave's share
  // [gw * sink_per_wave, ...), one load round trip per step (set up here, so
  // that nothing of it is live during the quantized stream)
  {
    const int sb = qs.gw * a.sink_per_wave, se = min(a.n_sink, sb + a.sink_per_wave);
    if (se > sb) {
      WinStream<BITS, G> ss;
      ss.kr = a.k_sink + bh * a.n_sink * kD;
      ss.vr = a.v_sink + bh * a.n_sink * kD;
      ss.begin = sb;
      ss.end = se;
      ss.bytes = (uint32_t)se * (kD * 2);
      ss.lane_voff = (uint32_t)(slot * kD + w * C::CPW) * 2;
      __builtin_amdgcn_wave_barrier();
      float qv[C::CPW];
#pragma unroll
      for (int i = 0; i < C::CPW; ++i) qv[i] = stg.qs[w * C::CPW + i];
      for (int i = 0; sb + i * WC::STEP < se; ++i) {
        WinStep<BITS, G> x;
        ss.issue(x, i);
        const int r = sb + i * WC::STEP + slot;
        if constexpr (ROPE) {
          float u[C::CPW];
          rope.at(u, r - a.n_sink);  // position r
          window_step<BITS, G>(x, r < se, u, st);
        } else {
          window_step<BITS, G>(x, r < se, qv, st);
        }
      }
    }
  }
  wave_publish<C::CPW, C::W, C::W == 8>(sm.fin.acc[wv], sm.fin.bias[wv], sm.fin.m[wv],
                                         sm.fin.l[wv], st.m, st.l, st.acc, st.bias);
  __syncthreads();
  // one workgroup per (sequence, head): only the threads that write an
  // output channel combine (the rest would only read LDS); in the whole step
  // the others go on to its commit and, where needed, its flush
  if constexpr (!FUSED) {
    if (S == 1 && tid >= kD) return;
  }

  const WgState wg = (FUSED && tid >= kD) ? WgState{-INFINITY, 0.0f, 0.0f}
                                          : combine_waves<BITS, G>(sm.fin, tid);
  const float L = wg.L, acc_out = wg.acc;
  if (S == 1) {  // the workgroup saw every token: finish here
    if (tid < kD) a.out[bh * kD + tid] = L > 0.0f ? acc_out / L : 0.0f;
    if constexpr (FUSED) {
      if (early) {
        // a wave that found the partials count short finishes its keys here,
        // after the combine barrier (every wave posted before its stream)
        if (!keys_done) {
          auto &rf = fused_flush_smem<BITS, G>().reg;
          flush_regs_tile_params<BITS, G>(ea, rf, tile0, tileT, nwt, wv, lane, wv % nwt == 0);
          flush_regs_keys<BITS, G>(ea, rf, wpf, wsteps, tile0, ws.begin, wv, w, slot);
        }
      } else if (flush) {
        // longer windows: read again (mostly L2 hits, this workgroup has
        // just read them) and quantized through LDS
        flush_window<BITS, G, G, kDecodeThreads>(ea, bh, ql0, tid, fused_flush_smem<BITS, G>().lds,
                                                 rnew, knew, vnew, 0, a.R);
      }
      if (commit && tid == 0 && ticket == (uint32_t)a.heads - 1) {
        ea.q_len[b] = flush ? ql0 + a.R : ql0;
        ea.r_len[b] = flush ? 0 : rl1;
        ea.tickets[(size_t)b * kTicketStride] = 0u;
      }
      // a counter that did not start at zero: no commit, and the caller is told
      if (commit && tid == 0 && ticket >= (uint32_t)a.heads) atomicOr(a.status, KIVI_ST_TICKETS);
    }
    return;
  }

  finish_splits(a, sm, wg, bh, split, S, tid);
}

// --------------------------------------------- decode: two words per lane
// The plain decode at B = 2 and 4 with two sub-chunks in flight and no sink
// tokens, in a second lane layout.  decode_kernel's lane holds one code word
// of each of 8 tokens per sub-chunk; here lane (q, p) holds words 2p and
// 2p + 1 (channels 2p CPW .. 2p CPW + 2 CPW - 1) of the 4 tokens 4q .. 4q + 3.
// The arithmetic per code is the same; what is done once per token and lane
// (the score's reduction over the token's lanes, its exponential, the
// softmax sum, the value group's step and zero-point products) is done for
// half as many tokens.  The bytes read, the loads' policy, the sub-chunk
// order, the window, the combine and the split merge are decode_kernel's;
// the window pass takes one token per quad of lanes.
template <int BITS, int G>
struct PairCfg {
  using C = DecCfg<BITS, G>;
  static constexpr int PW = C::W / 2;     // lanes per token
  static constexpr int NQ = 64 / PW;      // token quads per sub-chunk (= window tokens per step)
  static constexpr int CPL = 2 * C::CPW;  // channels per lane
  static constexpr int NVW = CPL / 8;     // 16-byte fp16 vectors per lane and window row
  static constexpr int PFW = 16 / NQ;     // window steps loaded after the stream (16 tokens)
  static_assert(BITS == 2 || BITS == 4, "two code words per lane");
  static_assert(4 * NQ == C::SUB, "one token quad per lane group fills a sub-chunk");
  static_assert(C::SUB % G == 0 || G % C::SUB == 0, "sub-chunks and tiles nest");
};

// Registers holding every load of one sub-chunk of one wave.
template <int BITS, int G>
struct PairLoads {
  using C = DecCfg<BITS, G>;
  uint4 kc[2], vc[2];               // words 2p and 2p + 1 of the lane's 4 tokens
  uint32_t ks[C::NTS], kz[C::NTS];  // key groups of 2 channels of each touched tile
  uint2 vs, vz;                     // the lane's value group for its 4 tokens
};

template <int BITS, int G>
struct PairStream {
  using C = DecCfg<BITS, G>;
  const void *kc, *vc, *ks, *kz, *vs, *vz;  // (sequence, head) regions
  uint32_t code_bytes, meta_bytes;          // region sizes
  // per-lane byte offsets of word 2p of the lane's first token, and of its
  // value group, within a sub-chunk; the "c" pair moves a lane past the
  // first tile back into it (a last sub-chunk of one valid tile, G < SUB)
  uint32_t code_voff, code_voffc, vmeta_voff, vmeta_voffc, kmeta_voff;
  int ql, last_tile, gw, nw, n;

  __device__ __forceinline__ int t0(int c) const { return (gw + c * nw) * C::SUB; }

  // Every load of sub-chunk c (zero-record descriptors for c >= n).  In a
  // sub-chunk that ends past ql, the lanes whose tokens lie past it load the
  // first tile's tokens instead (valid data; their scores are masked).
  __device__ __forceinline__ void issue(PairLoads<BITS, G> &b, int c, uint32_t extra = 0u) const {
    constexpr int A = load_aux<BITS>();
    const bool live = c < n;
    const uint32_t cb = live ? code_bytes : 0u, mb = live ? meta_bytes : 0u;
    const int T0 = live ? t0(c) : 0;
    const bool whole = T0 + C::SUB <= ql;
    const int tile0 = T0 / G;
    const rsrc_t rks = make_rsrc(ks, mb), rkz = make_rsrc(kz, mb);
    const rsrc_t rkc = make_rsrc(kc, cb), rvc = make_rsrc(vc, cb);
    const rsrc_t rvs = make_rsrc(vs, mb), rvz = make_rsrc(vz, mb);
#pragma unroll
    for (int k = 0; k < C::NTS; ++k) {
      const uint32_t so = (uint32_t)max(0, min(tile0 + k, last_tile)) * (kD * 2);
      b.ks[k] = bload1<A>(rks, kmeta_voff + extra, so);
      b.kz[k] = bload1<A>(rkz, kmeta_voff + extra, so);
    }
    const uint32_t cv = (whole ? code_voff : code_voffc) + extra;
    const uint32_t cs = (uint32_t)(tile0 * (C::W * G) + T0 % G) * 4;
    b.kc[0] = bload4<A>(rkc, cv, cs);
    b.kc[1] = bload4<A>(rkc, cv + G * 4, cs);
    b.vc[0] = bload4<A>(rvc, cv, cs);
    b.vc[1] = bload4<A>(rvc, cv + G * 4, cs);
    const uint32_t mv = (whole ? vmeta_voff : vmeta_voffc) + extra;
    const uint32_t ms = (uint32_t)(tile0 * kD + T0 % G) * 2;
    b.vs = bload2<A>(rvs, mv, ms);
    b.vz = bload2<A>(rvz, mv, ms);
  }

  // Sub-chunk c before the lengths are known, as QuantStream::issue_whole:
  // the loads of issue(b, c) whenever t0(c) + SUB <= ql; zeros (zero-record
  // descriptors) when the sub-chunk does not fit below cap.
  __device__ __forceinline__ void issue_whole(PairLoads<BITS, G> &b, int c, int cap) const {
    constexpr int A = load_aux<BITS>();
    const bool fits = t0(c) + C::SUB <= cap;
    const uint32_t cb = fits ? code_bytes : 0u, mb = fits ? meta_bytes : 0u;
    const int T0 = fits ? t0(c) : 0;
    const int tile0 = T0 / G;
    const rsrc_t rks = make_rsrc(ks, mb), rkz = make_rsrc(kz, mb);
    const rsrc_t rkc = make_rsrc(kc, cb), rvc = make_rsrc(vc, cb);
    const rsrc_t rvs = make_rsrc(vs, mb), rvz = make_rsrc(vz, mb);
#pragma unroll
    for (int k = 0; k < C::NTS; ++k) {
      const uint32_t so = (uint32_t)(tile0 + k) * (kD * 2);
      b.ks[k] = bload1<A>(rks, kmeta_voff, so);
      b.kz[k] = bload1<A>(rkz, kmeta_voff, so);
    }
    const uint32_t cs = (uint32_t)(tile0 * (C::W * G) + T0 % G) * 4;
    b.kc[0] = bload4<A>(rkc, code_voff, cs);
    b.kc[1] = bload4<A>(rkc, code_voff + G * 4, cs);
    b.vc[0] = bload4<A>(rvc, code_voff, cs);
    b.vc[1] = bload4<A>(rvc, code_voff + G * 4, cs);
    const uint32_t ms = (uint32_t)(tile0 * kD + T0 % G) * 2;
    b.vs = bload2<A>(rvs, vmeta_voff, ms);
    b.vz = bload2<A>(rvz, vmeta_voff, ms);
  }
};

// One sub-chunk: key multipliers staged as decode_kernel does (the lane's
// two channels of every touched tile), then the lane's 4 scores (both words
// in one accumulation chain, reduced over the token's PW lanes), the online
// softmax, and the weighted value sums of both words.  MASK: the sub-chunk
// may end past ql (its lanes past ql score -inf and add nothing).
template <int BITS, int G, bool MASK>
__device__ __forceinline__ void process_pair(
    const PairLoads<BITS, G> &b, int T0, int ql, int lane, float qf0, float qf1, float qs0,
    float qs1, float (&qp)[DecCfg<BITS, G>::NTS][DecCfg<BITS, G>::W * DecCfg<BITS, G>::QPW],
    float (&cz)[DecCfg<BITS, G>::NTS][DecCfg<BITS, G>::W], LaneState<PairCfg<BITS, G>::CPL> &st) {
  using C = DecCfg<BITS, G>;
  using P = PairCfg<BITS, G>;
  const int d0 = 2 * lane;
  const int qpo = (d0 / C::CPW) * C::QPW + d0 % C::CPW;
#pragma unroll
  for (int k = 0; k < C::NTS; ++k) {
    qp[k][qpo] = mix_lo(qf0, b.ks[k], 0.0f);
    qp[k][qpo + 1] = mix_hi(qf1, b.ks[k], 0.0f);
    float zc = mix_lo(qs0, b.kz[k], mix_hi(qs1, b.kz[k], 0.0f));
    zc = lane_group_sum<C::CPW / 2>(zc);
    if ((lane % (C::CPW / 2)) == 0) cz[k][lane / (C::CPW / 2)] = zc;
  }
  __builtin_amdgcn_wave_barrier();

  const int p = lane % P::PW, q = lane / P::PW;
  const int k = ((T0 % G) + 4 * q) / G;  // the lane's tile within the sub-chunk
  // word 2p of the 4 tokens first, then word 2p + 1: each half waits only
  // for its own load
  float s[4];
  const float c0 = cz[k][2 * p] + cz[k][2 * p + 1];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float qv[C::CPW];
#pragma unroll
    for (int i = 0; i < C::CPW; i += 4) {
      const float4 t4 = *reinterpret_cast<const float4 *>(&qp[k][(2 * p + h) * C::QPW + i]);
      qv[i] = t4.x;
      qv[i + 1] = t4.y;
      qv[i + 2] = t4.z;
      qv[i + 3] = t4.w;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = dot_word<BITS>(u4_get(b.kc[h], i), qv, h == 0 ? c0 : s[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = lane_group_sum<P::PW>(s[i]);
  __builtin_amdgcn_wave_barrier();
  [[maybe_unused]] bool ok = true;
  if constexpr (MASK) {
    ok = T0 + 4 * q < ql;
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = ok ? s[i] : -INFINITY;
  }

  update_max<P::CPL, 4>(st, s);

  float pp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float pr = exp2_fast(s[i] - st.m);
    if constexpr (MASK) pr = ok ? pr : 0.0f;  // (-inf - -inf is NaN)
    st.l += pr;
    const uint32_t sw = i < 2 ? b.vs.x : b.vs.y;
    const uint32_t zw = i < 2 ? b.vz.x : b.vz.y;
    pp[i] = (i & 1) ? mix_hi(pr, sw, 0.0f) : mix_lo(pr, sw, 0.0f);
    st.bias = (i & 1) ? mix_hi(pr, zw, st.bias) : mix_lo(pr, zw, st.bias);
  }
  // word 2p of the 4 tokens, then word 2p + 1
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u = u4_get(b.vc[h], i);
      axpy_pairs<BITS>(u, upper_pairs<BITS>(u), pp[i], st.acc + h * C::CPW);
    }
}

// Window rows in the pair layout: lane (q, p) takes channels 2p CPW ..
// 2p CPW + 2 CPW - 1 of token begin + step NQ + q.
template <int BITS, int G>
struct PairWinStep {
  uint4 k[PairCfg<BITS, G>::NVW], v[PairCfg<BITS, G>::NVW];
};

template <int BITS, int G>
struct PairWin {
  using P = PairCfg<BITS, G>;
  const void *kr, *vr;  // (sequence, head) window rows
  uint32_t bytes;       // rows at or past this wave's end read as 0
  uint32_t lane_voff;   // byte offset of the lane's channels in its token row
  int begin, end;

  __device__ __forceinline__ void issue(PairWinStep<BITS, G> &x, int step) const {
    const rsrc_t rk = make_rsrc(kr, bytes), rv = make_rsrc(vr, bytes);
    const uint32_t vo = lane_voff + (uint32_t)(begin + step * P::NQ) * (kD * 2);
#pragma unroll
    for (int v = 0; v < P::NVW; ++v) x.k[v] = bload4<load_aux<BITS>()>(rk, vo + 16 * v, 0);
#pragma unroll
    for (int v = 0; v < P::NVW; ++v) x.v[v] = bload4<load_aux<BITS>()>(rv, vo + 16 * v, 0);
  }
};

template <int BITS, int G>
__device__ __forceinline__ void pair_window_step(const PairWinStep<BITS, G> &x, bool valid,
                                                 const float *qv,
                                                 LaneState<PairCfg<BITS, G>::CPL> &st) {
  using C = DecCfg<BITS, G>;
  using P = PairCfg<BITS, G>;
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int v = 0; v < P::NVW; ++v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = u4_get(x.k[v], e);
      a0 = mix_lo(qv[8 * v + 2 * e], u, a0);
      a1 = mix_hi(qv[8 * v + 2 * e + 1], u, a1);
    }
  }
  float s = lane_group_sum<P::PW>(a0 + a1);
  s = valid ? s : -INFINITY;
  update_max<P::CPL, 1>(st, &s);
  const float pr = s > -INFINITY ? exp2_fast(s - st.m) : 0.0f;
  st.l += pr;
#pragma unroll
  for (int v = 0; v < P::NVW; ++v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // value sums hold channel values times 2^(e - 24), e the channel's
      // code offset within its word (see the quantized tokens)
      const uint32_t u = u4_get(x.v[v], e);
      const int c = 8 * v + 2 * e;
      st.acc[c] = mix_lo(pr * __builtin_ldexpf(1.0f, code_offset<BITS>(c % C::CPW) - 24), u,
                         st.acc[c]);
      st.acc[c + 1] = mix_hi(pr * __builtin_ldexpf(1.0f, code_offset<BITS>((c + 1) % C::CPW) - 24),
                             u, st.acc[c + 1]);
    }
  }
}

// One wave's state to the workgroup's LDS, in decode_kernel's published
// form (row r: every channel, from the lanes of row r): rescale to the
// wave's maximum, then sum the token quads of each 16-lane row (lane q PW +
// p; rotations by 4 and 8 lanes within the row, or by 8 alone at PW = 8).
template <int BITS, int G>
__device__ __forceinline__ void pair_publish(float (&fin_acc)[4][kD], float (&fin_bias)[4][32],
                                             float &fin_m, float &fin_l,
                                             LaneState<PairCfg<BITS, G>::CPL> &st) {
  using C = DecCfg<BITS, G>;
  using P = PairCfg<BITS, G>;
  const int lane = threadIdx.x & 63;
  const int p = lane % P::PW, row = lane >> 4;
  const float M = wave_max(st.m);
  const float e = (st.m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(st.m - M);
  float bias = st.bias * e;
  const float lw = wave_sum(p == 0 ? st.l * e : 0.0f);
#pragma unroll
  for (int i = 0; i < P::CPL; ++i) {
    float v = st.acc[i] * e;
    if constexpr (P::PW == 4) v += dpp<0x124>(v);  // row_ror:4
    v += dpp<0x128>(v);                             // row_ror:8
    st.acc[i] = v;
  }
  if constexpr (P::PW == 4) bias += dpp<0x124>(bias);
  bias += dpp<0x128>(bias);
  if ((lane & 15) < P::PW) {
#pragma unroll
    for (int i = 0; i < P::CPL; i += 4)
      *reinterpret_cast<float4 *>(&fin_acc[row][2 * p * C::CPW + i]) =
          make_float4(st.acc[i], st.acc[i + 1], st.acc[i + 2], st.acc[i + 3]);
    fin_bias[row][2 * p] = bias;
    fin_bias[row][2 * p + 1] = bias;
  }
  if (lane == 0) {
    fin_m = M;
    fin_l = lw;
  }
}

template <int BITS, int G>
__global__ __launch_bounds__(kDecodeThreads, kDecodeWavesPerSimd) void decode_pair_kernel(
    DecodeArgs a) {
  using C = DecCfg<BITS, G>;
  using P = PairCfg<BITS, G>;
  constexpr int kDepth = 2;  // a third sub-chunk in flight measured slower
  __shared__ DecSmem<BITS, G, false> sm;
  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * a.heads + h;
  const int S = a.splits;
  const int p = lane % P::PW, q = lane / P::PW, d = 4 * q;

  // ---- the stream's descriptors and this wave's first sub-chunk, before
  // the lengths (as decode_kernel)
  const size_t tps = (size_t)(a.cap / G);
  PairStream<BITS, G> qs;
  qs.kc = a.k_codes + bh * tps * (C::W * G);
  qs.vc = a.v_codes + bh * tps * (C::W * G);
  qs.ks = a.k_scale + bh * tps * kD;
  qs.kz = a.k_zero + bh * tps * kD;
  qs.vs = a.v_scale + bh * tps * kD;
  qs.vz = a.v_zero + bh * tps * kD;
  qs.code_bytes = (uint32_t)(tps * (C::W * G) * 4);
  qs.meta_bytes = (uint32_t)(tps * kD * 2);
  const int vg = (2 * p * C::CPW) / G;  // the lane's value group
  qs.code_voff = (uint32_t)((d / G) * (C::W * G) + 2 * p * G + d % G) * 4;
  qs.code_voffc = (uint32_t)(2 * p * G + d % G) * 4;
  qs.vmeta_voff = (uint32_t)((d / G) * kD + vg * G + d % G) * 2;
  qs.vmeta_voffc = (uint32_t)(vg * G + d % G) * 2;
  qs.kmeta_voff = (uint32_t)lane * 4;
  qs.gw = split * kDecodeWaves + wv;
  qs.nw = kDecodeWaves * S;
  const uint32_t qraw = bload1(make_rsrc(a.q + bh * kD, kD * 2), (uint32_t)lane * 4, 0);
  PairLoads<BITS, G> ring[kDepth];
  qs.issue_whole(ring[0], 0, a.cap);

  int ql = a.q_len[b], rl = a.r_len[b];
  __builtin_amdgcn_sched_barrier(0);
  const bool lens_ok = (ql >= 0) & (ql <= a.cap) & ((ql % G) == 0) & (rl >= 0) & (rl <= a.R);
  if (!lens_ok) {
    if (split == 0 && h == 0 && tid == 0) atomicOr(a.status, KIVI_ST_BAD_LENGTH);
    ql = 0;
    rl = 0;
  }
  qs.ql = ql;
  qs.last_tile = ql / G - 1;
  qs.n = qs.gw * C::SUB < ql ? (ql - qs.gw * C::SUB + qs.nw * C::SUB - 1) / (qs.nw * C::SUB) : 0;
  if (qs.t0(0) + C::SUB > ql) qs.issue(ring[0], 0);

  PairWin<BITS, G> ws;
  ws.kr = a.k_res + bh * a.R * kD;
  ws.vr = a.v_res + bh * a.R * kD;
  ws.begin = qs.gw * a.win_per_wave;
  ws.end = min(rl, ws.begin + a.win_per_wave);
  ws.bytes = (uint32_t)max(0, ws.end) * (kD * 2);
  ws.lane_voff = (uint32_t)(q * kD + 2 * p * C::CPW) * 2;
  const int wsteps = ws.end > ws.begin ? (ws.end - ws.begin + P::NQ - 1) / P::NQ : 0;

  auto &stg = sm.u.wave[wv];
#if KIVI_DECODE_PRIORITY == 2
  if (lane == 0) sm.prog[wv] = 0;
#endif
  const half2_t hq = __builtin_bit_cast(half2_t, qraw);
  const float qs0 = (float)hq.x * a.qscale, qs1 = (float)hq.y * a.qscale;
  const float qf0 = qs0 * code_factor<BITS>((2 * lane) % C::CPW);
  const float qf1 = qs1 * code_factor<BITS>((2 * lane + 1) % C::CPW);
  stg.qs[2 * lane] = qs0;  // for the window tokens
  stg.qs[2 * lane + 1] = qs1;

  LaneState<P::CPL> st;
  st.m = -INFINITY;
  st.l = 0.0f;
  st.bias = 0.0f;
#pragma unroll
  for (int i = 0; i < P::CPL; ++i) st.acc[i] = 0.0f;

  // a sub-chunk, masked only where one can end past ql (G < SUB)
  auto process = [&](const PairLoads<BITS, G> &bb, int c) {
    const int T0 = qs.t0(c);
    if constexpr (G < C::SUB) {
      if (T0 + C::SUB > ql) {
        process_pair<BITS, G, true>(bb, T0, ql, lane, qf0, qf1, qs0, qs1, stg.qp, stg.cz, st);
        return;
      }
    }
    process_pair<BITS, G, false>(bb, T0, ql, lane, qf0, qf1, qs0, qs1, stg.qp, stg.cz, st);
  };

  {
    // the rest of the ring once sub-chunk 0 is in
    uint32_t z;
    asm volatile("v_and_b32 %0, 0, %1" : "=v"(z) : "v"(ring[0].vz.y));
#pragma unroll
    for (int k = 1; k < kDepth; ++k) qs.issue(ring[k], k, z);
  }
  int c0 = 0;
  for (; c0 + kDepth <= qs.n; c0 += kDepth) {
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
#if KIVI_DECODE_PRIORITY == 2
      set_lead_priority(sm.prog, wv, lane, c0 + k);
#elif KIVI_DECODE_PRIORITY
      set_progress_priority(c0 + k, qs.n);
#endif
      process(ring[k], c0 + k);
      qs.issue(ring[k], c0 + k + kDepth);
    }
  }
  PairWinStep<BITS, G> wpf[P::PFW];
#pragma unroll
  for (int i = 0; i < P::PFW; ++i) ws.issue(wpf[i], i);
#pragma unroll
  for (int k = 0; k < kDepth - 1; ++k)
    if (c0 + k < qs.n) {
#if KIVI_DECODE_PRIORITY == 2
      set_lead_priority(sm.prog, wv, lane, c0 + k);
#elif KIVI_DECODE_PRIORITY
      set_progress_priority(c0 + k, qs.n);
#endif
      process(ring[k], c0 + k);
    }
#if KIVI_DECODE_PRIORITY
  __builtin_amdgcn_s_setprio(0);
#endif

  // ---- the wave's window tokens
  if (wsteps > 0) {
    __builtin_amdgcn_wave_barrier();
    float qv[P::CPL];
#pragma unroll
    for (int i = 0; i < P::CPL; ++i) qv[i] = stg.qs[2 * p * C::CPW + i];
#pragma unroll
    for (int i = 0; i < P::PFW; ++i)
      if (i < wsteps) pair_window_step<BITS, G>(wpf[i], ws.begin + i * P::NQ + q < ws.end, qv, st);
    for (int i = P::PFW; i < wsteps; ++i) {  // windows longer than the prefetched steps
      PairWinStep<BITS, G> x;
      ws.issue(x, i);
      pair_window_step<BITS, G>(x, ws.begin + i * P::NQ + q < ws.end, qv, st);
    }
  }

  pair_publish<BITS, G>(sm.fin.acc[wv], sm.fin.bias[wv], sm.fin.m[wv], sm.fin.l[wv], st);
  __syncthreads();
  if (S == 1 && tid >= kD) return;  // only the output channels' threads combine
  const WgState wg = combine_waves<BITS, G>(sm.fin, tid);
  if (S == 1) {
    if (tid < kD) a.out[bh * kD + tid] = wg.L > 0.0f ? wg.acc / wg.L : 0.0f;
    return;
  }
  finish_splits(a, sm, wg, bh, split, S, tid);
}

// ------------------------------------------------ measurement: stream read
// Reads a buffer once and folds it into one word per wave: the HBM read rate
// this chip sustains for a given size and grid, the ceiling the decode's
// rate is compared with.  Workgroup i streams its own contiguous slice (as a
// decode workgroup streams its (sequence, head)) through a buffer
// descriptor bounded by the slice, with the decode's load policy (kLoadAux),
// kStreamUnroll 16-byte loads in flight per lane, the lanes of a wave on
// consecutive 16-byte pieces.  Measured on 114.5 MB: plain global loads
// 20.7 us at best, these 18.3 us.
constexpr int kStreamThreads = 512;
constexpr int kStreamUnroll = 8;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const char *src, size_t bytes,
                                                                     size_t per_wg,
                                                                     uint32_t *sink) {
  const size_t begin = (size_t)blockIdx.x * per_wg;
  const uint32_t len = (uint32_t)(begin < bytes ? min(bytes - begin, per_wg) : 0);
  const rsrc_t r = make_rsrc(src + (begin < bytes ? begin : 0), len);
  constexpr uint32_t kStep = kStreamThreads * 16;
  uint32_t x = 0;
  for (uint32_t o = threadIdx.x * 16; o < len; o += kStep * kStreamUnroll) {
    uint4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = bload4(r, o + (uint32_t)u * kStep, 0);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off);
  if ((threadIdx.x & 63) == 0) sink[(size_t)blockIdx.x * (kStreamThreads / 64) + threadIdx.x / 64] = x;
}

// Zero-fill n 32-bit words (a kernel, not a memset, so that a caller may
// capture it in a HIP graph).
__global__ __launch_bounds__(kThreads) void fill_zero_kernel(uint32_t *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (size_t)gridDim.x * kThreads)
    p[i] = 0u;
}

// An empty cache: lengths, ticket counters and the status word zero.
__global__ __launch_bounds__(kThreads) void cache_init_kernel(int32_t *q_len, int32_t *r_len,
                                                              uint32_t *tickets, uint32_t *status,
                                                              int batch) {
  for (int i = threadIdx.x; i < batch * kTicketStride; i += kThreads) {
    tickets[i] = 0u;
    if (i < batch) {
      q_len[i] = 0;
      r_len[i] = 0;
    }
  }
  if (threadIdx.x == 0) *status = 0u;
}

template <int BITS, int G>
int launch_encode_t(const EncodeArgs &ea, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((encode_kernel<BITS, G>), grid, dim3(kThreads), 0, st, ea);
  return (int)hipGetLastError();
}

int launch_encode(int bits, int G, const EncodeArgs &ea, dim3 grid, hipStream_t st) {
  if (bits == 2 && G == 32) return launch_encode_t<2, 32>(ea, grid, st);
  if (bits == 2 && G == 64) return launch_encode_t<2, 64>(ea, grid, st);
  if (bits == 2 && G == 128) return launch_encode_t<2, 128>(ea, grid, st);
  if (bits == 4 && G == 32) return launch_encode_t<4, 32>(ea, grid, st);
  if (bits == 4 && G == 64) return launch_encode_t<4, 64>(ea, grid, st);
  if (bits == 4 && G == 128) return launch_encode_t<4, 128>(ea, grid, st);
  if (bits == 8 && G == 32) return launch_encode_t<8, 32>(ea, grid, st);
  if (bits == 8 && G == 64) return launch_encode_t<8, 64>(ea, grid, st);
  if (bits == 8 && G == 128) return launch_encode_t<8, 128>(ea, grid, st);
  return (int)hipErrorInvalidValue;
}

template <int BITS, int G>
int launch_decode_t(const DecodeArgs &da, const EncodeArgs &ea, bool fused, int depth, dim3 grid,
                    hipStream_t st, bool rope, bool vq) {
  const dim3 blk(kDecodeThreads);
  if (vq) {  // value queue: the plain decode with the token-by-token tail
    if (fused || rope) return (int)hipErrorInvalidValue;
    if (depth == 1)
      hipLaunchKernelGGL((decode_kernel<BITS, G, false, 1, false, true>), grid, blk, 0, st, da, ea);
    else
      hipLaunchKernelGGL((decode_kernel<BITS, G, false, 2, false, true>), grid, blk, 0, st, da, ea);
    return (int)hipGetLastError();
  }
  if (rope) {
    // keys stored pre-rotation (never the whole step).  At B=2 always two
    // sub-chunks in flight: only that register budget (one workgroup per
    // compute unit) holds the rotation's per-lane state without spilling.
    // At B=4 and 8 large grids take depth 1 at two workgroups per compute
    // unit (108 and 79 VGPRs), as the plain decode does.
    if (fused) return (int)hipErrorInvalidValue;
    if constexpr (BITS >= 4) {
      if (depth == 1) {
        hipLaunchKernelGGL((decode_kernel<BITS, G, false, 1, true>), grid, blk, 0, st, da, ea);
        return (int)hipGetLastError();
      }
    }
    hipLaunchKernelGGL((decode_kernel<BITS, G, false, 2, true>), grid, blk, 0, st, da, ea);
    return (int)hipGetLastError();
  }
  if (fused) {  // one workgroup per compute unit (launch_decode_step)
    if constexpr (BITS == 8) return (int)hipErrorInvalidValue;  // three kernels instead
    else hipLaunchKernelGGL((decode_kernel<BITS, G, true, 2>), grid, blk, 0, st, da, ea);
  } else if (depth == 1) {
    hipLaunchKernelGGL((decode_kernel<BITS, G, false, 1>), grid, blk, 0, st, da, ea);
  } else {
#ifndef KIVI_PAIR
#define KIVI_PAIR 1
#endif
    // two sub-chunks in flight, no sink tokens, and by capacity at least 16
    // sub-chunks per wave: two code words per lane (on the long-context
    // workload 74.2 -> 69.1 us at B=2 and 108.9 -> 104.4 us at B=4; on the
    // 7B layer, 8 sub-chunks per wave, 23.5 against 23.9 us, and on one head
    // 4.9 against 5.5 us, where decode_kernel stays)
    if constexpr (KIVI_PAIR && BITS != 8 && KIVI_WIDE_DEPTH == 2) {
      if (da.n_sink == 0 &&
          da.cap / DecCfg<BITS, G>::SUB >= 16 * kDecodeWaves * da.splits) {
        hipLaunchKernelGGL((decode_pair_kernel<BITS, G>), grid, blk, 0, st, da);
        return (int)hipGetLastError();
      }
    }
    hipLaunchKernelGGL((decode_kernel<BITS, G, false, KIVI_WIDE_DEPTH>), grid, blk, 0, st, da, ea);
  }
  return (int)hipGetLastError();
}

EncodeArgs encode_args(const kivi_dims &d, const kivi_cache &c) {
  EncodeArgs ea{};
  ea.k_codes = static_cast<uint32_t *>(c.k_codes);
  ea.v_codes = static_cast<uint32_t *>(c.v_codes);
  ea.k_scale = static_cast<half_t *>(c.k_scale);
  ea.k_zero = static_cast<half_t *>(c.k_zero);
  ea.v_scale = static_cast<half_t *>(c.v_scale);
  ea.v_zero = static_cast<half_t *>(c.v_zero);
  ea.k_res = static_cast<half_t *>(c.k_res);
  ea.v_res = static_cast<half_t *>(c.v_res);
  ea.q_len = c.q_len;
  ea.r_len = c.r_len;
  ea.status = c.status;
  ea.tickets = c.tickets;
  ea.heads = d.heads;
  ea.R = d.residual;
  ea.cap = d.capacity;
  return ea;
}

}  // namespace

int launch_append(const kivi_dims &d, const kivi_cache &c, const void *k_new, const void *v_new,
                  void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(append_kernel, dim3(d.batch), dim3(kAppendThreads), 0, st,
                     static_cast<const half_t *>(k_new), static_cast<const half_t *>(v_new),
                     static_cast<half_t *>(c.k_res), static_cast<half_t *>(c.v_res), c.r_len,
                     c.status, d.heads, d.residual);
  return (int)hipGetLastError();
}

// P tiles per workgroup: up to 128 window tokens (the LDS of P tile blocks);
// VALUES false: keys only (the value queue's flush)
template <int BITS, int G, bool VALUES>
int launch_flush_p(const EncodeArgs &ea, dim3 grid, int P, hipStream_t st) {
  if constexpr (4 * G <= 128) {
    if (P == 4) {
      hipLaunchKernelGGL((flush_kernel<BITS, G, 4, VALUES>), grid, dim3(4 * kFlushThreads), 0, st,
                         ea);
      return (int)hipGetLastError();
    }
  }
  if constexpr (2 * G <= 128) {
    if (P == 2) {
      hipLaunchKernelGGL((flush_kernel<BITS, G, 2, VALUES>), grid, dim3(2 * kFlushThreads), 0, st,
                         ea);
      return (int)hipGetLastError();
    }
  }
  if (P != 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL((flush_kernel<BITS, G, 1, VALUES>), grid, dim3(kFlushThreads), 0, st, ea);
  return (int)hipGetLastError();
}

template <int BITS, int G>
int launch_flush_t(const EncodeArgs &ea, dim3 grid, int P, hipStream_t st, bool keys_only) {
  return keys_only ? launch_flush_p<BITS, G, false>(ea, grid, P, st)
                   : launch_flush_p<BITS, G, true>(ea, grid, P, st);
}

// The key-wave / value-wave flush: one workgroup per (sequence, head).
template <int BITS, int G>
int launch_flush_split(const EncodeArgs &ea, const kivi_dims &d, hipStream_t st, bool keys_only) {
  const dim3 grid(d.heads, d.batch), blk(kDecodeThreads);
  if (keys_only)
    hipLaunchKernelGGL((flush_split_kernel<BITS, G, false>), grid, blk, 0, st, ea);
  else
    hipLaunchKernelGGL((flush_split_kernel<BITS, G, true>), grid, blk, 0, st, ea);
  return (int)hipGetLastError();
}

#ifndef KIVI_FLUSH_SPLIT
#define KIVI_FLUSH_SPLIT 1
#endif

int launch_flush_any(const kivi_dims &d, const kivi_cache &c, void *stream, bool keys_only) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  EncodeArgs ea = encode_args(d, c);
  ea.src_k = ea.k_res;
  ea.src_v = ea.v_res;
  ea.src_tokens = d.residual;
  ea.prefill = 0;
  const int G = d.group, tiles = d.residual / G;
  // B = 2 or 4, windows of at most 128 tokens: key waves and value waves
  if (KIVI_FLUSH_SPLIT && d.bits != 8 && d.residual <= kFlushKeyWaves * kFlushTokensPerWave &&
      kDecodeWaves == 2 * kFlushKeyWaves) {
    if (d.bits == 2 && G == 32) return launch_flush_split<2, 32>(ea, d, st, keys_only);
    if (d.bits == 2 && G == 64) return launch_flush_split<2, 64>(ea, d, st, keys_only);
    if (d.bits == 2 && G == 128) return launch_flush_split<2, 128>(ea, d, st, keys_only);
    if (d.bits == 4 && G == 32) return launch_flush_split<4, 32>(ea, d, st, keys_only);
    if (d.bits == 4 && G == 64) return launch_flush_split<4, 64>(ea, d, st, keys_only);
    if (d.bits == 4 && G == 128) return launch_flush_split<4, 128>(ea, d, st, keys_only);
  }
  // tiles side by side per workgroup: the most of 4, 2, 1 that divides the
  // window's tiles and keeps to 128 tokens
  const int pmax = min(KIVI_FLUSH_P, 128 / G);
  const int P = tiles % 4 == 0 && pmax >= 4 ? 4 : tiles % 2 == 0 && pmax >= 2 ? 2 : 1;
  const dim3 grid(tiles / P, d.heads, d.batch);
  const bool k = keys_only;
  if (d.bits == 2 && G == 32) return launch_flush_t<2, 32>(ea, grid, P, st, k);
  if (d.bits == 2 && G == 64) return launch_flush_t<2, 64>(ea, grid, P, st, k);
  if (d.bits == 2 && G == 128) return launch_flush_t<2, 128>(ea, grid, P, st, k);
  if (d.bits == 4 && G == 32) return launch_flush_t<4, 32>(ea, grid, P, st, k);
  if (d.bits == 4 && G == 64) return launch_flush_t<4, 64>(ea, grid, P, st, k);
  if (d.bits == 4 && G == 128) return launch_flush_t<4, 128>(ea, grid, P, st, k);
  if (d.bits == 8 && G == 32) return launch_flush_t<8, 32>(ea, grid, P, st, k);
  if (d.bits == 8 && G == 64) return launch_flush_t<8, 64>(ea, grid, P, st, k);
  if (d.bits == 8 && G == 128) return launch_flush_t<8, 128>(ea, grid, P, st, k);
  return (int)hipErrorInvalidValue;
}

int launch_flush(const kivi_dims &d, const kivi_cache &c, void *stream) {
  return launch_flush_any(d, c, stream, false);
}

int launch_flush_keys(const kivi_dims &d, const kivi_cache &c, void *stream) {
  return launch_flush_any(d, c, stream, true);
}

template <int BITS, int G>
int launch_append_vq_t(const EncodeArgs &ea, int batch, const void *k_new, const void *v_new,
                       hipStream_t st) {
  hipLaunchKernelGGL((append_vq_kernel<BITS, G>), dim3(batch), dim3(kAppendVqThreads), 0, st, ea,
                     static_cast<const half_t *>(k_new), static_cast<const half_t *>(v_new));
  return (int)hipGetLastError();
}

int launch_append_vq(const kivi_dims &d, const kivi_cache &c, const void *k_new,
                     const void *v_new, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const EncodeArgs ea = encode_args(d, c);
  const int G = d.group;
  if (d.bits == 2 && G == 32) return launch_append_vq_t<2, 32>(ea, d.batch, k_new, v_new, st);
  if (d.bits == 2 && G == 64) return launch_append_vq_t<2, 64>(ea, d.batch, k_new, v_new, st);
  if (d.bits == 2 && G == 128) return launch_append_vq_t<2, 128>(ea, d.batch, k_new, v_new, st);
  if (d.bits == 4 && G == 32) return launch_append_vq_t<4, 32>(ea, d.batch, k_new, v_new, st);
  if (d.bits == 4 && G == 64) return launch_append_vq_t<4, 64>(ea, d.batch, k_new, v_new, st);
  if (d.bits == 4 && G == 128) return launch_append_vq_t<4, 128>(ea, d.batch, k_new, v_new, st);
  if (d.bits == 8 && G == 32) return launch_append_vq_t<8, 32>(ea, d.batch, k_new, v_new, st);
  if (d.bits == 8 && G == 64) return launch_append_vq_t<8, 64>(ea, d.batch, k_new, v_new, st);
  if (d.bits == 8 && G == 128) return launch_append_vq_t<8, 128>(ea, d.batch, k_new, v_new, st);
  return (int)hipErrorInvalidValue;
}

int launch_prefill(const kivi_dims &d, const kivi_cache &c, const void *k, const void *v,
                   int32_t src_len, const int32_t *len, const int32_t *res, void *stream,
                   bool value_queue) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  EncodeArgs ea = encode_args(d, c);
  ea.vq = value_queue ? 1 : 0;
  ea.src_k = static_cast<const half_t *>(k);
  ea.src_v = static_cast<const half_t *>(v);
  ea.src_tokens = src_len;
  ea.len = len;
  ea.res = res;
  ea.prefill = 1;
  const int tiles = src_len / d.group;
  if (tiles > 0) {
    int rc = launch_encode(d.bits, d.group, ea, dim3(tiles, d.heads, d.batch), st);
    if (rc) return rc;
  }
  hipLaunchKernelGGL(prefill_window_kernel, dim3(d.heads, d.batch), dim3(kThreads), 0, st, ea,
                     d.group);
  int rc = (int)hipGetLastError();
  if (rc) return rc;
  hipLaunchKernelGGL(prefill_commit_kernel, dim3(1), dim3(kThreads), 0, st, ea, d.batch, d.group);
  return (int)hipGetLastError();
}

namespace {

DecodeArgs decode_args(const kivi_dims &d, const kivi_cache &c, const DecodePlan &p, const void *q,
                       float *out, float sm_scale, void *workspace) {
  DecodeArgs da{};
  da.k_codes = static_cast<const uint32_t *>(c.k_codes);
  da.v_codes = static_cast<const uint32_t *>(c.v_codes);
  da.k_scale = static_cast<const half_t *>(c.k_scale);
  da.k_zero = static_cast<const half_t *>(c.k_zero);
  da.v_scale = static_cast<const half_t *>(c.v_scale);
  da.v_zero = static_cast<const half_t *>(c.v_zero);
  da.k_res = static_cast<const half_t *>(c.k_res);
  da.v_res = static_cast<const half_t *>(c.v_res);
  da.q_len = c.q_len;
  da.r_len = c.r_len;
  da.status = c.status;
  da.q = static_cast<const half_t *>(q);
  da.out = out;
  da.part = static_cast<float *>(workspace);
  da.tickets = reinterpret_cast<uint32_t *>(static_cast<char *>(workspace) + p.counters_off);
  da.qscale = sm_scale * 1.4426950408889634f;
  da.heads = d.heads;
  da.R = d.residual;
  da.cap = d.capacity;
  da.splits = p.splits;
  da.win_per_wave = p.win_per_wave;
  da.part_stride = (int)p.part_floats;
  // more workgroups than the grid's resident slots (three per compute unit
  // at depth 1): ragged batches end with their shortest sequences (batch 64
  // of 1024..8192 tokens: 197.2 -> 189.2 us; a batch of equal lengths keeps
  // its order, ties going by index)
  da.lpt_batch = (d.batch > 1 && d.batch <= kLptMax &&
                  (long)d.batch * d.heads * p.splits > 3L * 256) ? d.batch : 0;
  return da;
}

// n_sink fp16 sink tokens, shared over all waves of all splits
void set_sink(DecodeArgs &da, const DecodePlan &p, const void *k_sink, const void *v_sink,
              int n_sink) {
  if (n_sink <= 0) return;
  const int waves = kDecodeWaves * p.splits;
  da.k_sink = static_cast<const half_t *>(k_sink);
  da.v_sink = static_cast<const half_t *>(v_sink);
  da.n_sink = n_sink;
  da.sink_per_wave = ((n_sink + waves - 1) / waves + 7) / 8 * 8;
}

int launch_decode_any(const kivi_dims &d, const DecodeArgs &da, const EncodeArgs &ea, bool fused,
                      int depth, hipStream_t st, bool rope = false, bool vq = false) {
  const dim3 grid(da.splits, d.heads, d.batch);
  const int G = d.group;
  if (d.bits == 2 && G == 32) return launch_decode_t<2, 32>(da, ea, fused, depth, grid, st, rope, vq);
  if (d.bits == 2 && G == 64) return launch_decode_t<2, 64>(da, ea, fused, depth, grid, st, rope, vq);
  if (d.bits == 2 && G == 128) return launch_decode_t<2, 128>(da, ea, fused, depth, grid, st, rope, vq);
  if (d.bits == 4 && G == 32) return launch_decode_t<4, 32>(da, ea, fused, depth, grid, st, rope, vq);
  if (d.bits == 4 && G == 64) return launch_decode_t<4, 64>(da, ea, fused, depth, grid, st, rope, vq);
  if (d.bits == 4 && G == 128) return launch_decode_t<4, 128>(da, ea, fused, depth, grid, st, rope, vq);
  if (d.bits == 8 && G == 32) return launch_decode_t<8, 32>(da, ea, fused, depth, grid, st, rope, vq);
  if (d.bits == 8 && G == 64) return launch_decode_t<8, 64>(da, ea, fused, depth, grid, st, rope, vq);
  if (d.bits == 8 && G == 128) return launch_decode_t<8, 128>(da, ea, fused, depth, grid, st, rope, vq);
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_cache_init(const kivi_dims &d, const kivi_cache &c, void *stream) {
  hipLaunchKernelGGL(cache_init_kernel, dim3(1), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), c.q_len, c.r_len, c.tickets, c.status,
                     d.batch);
  return (int)hipGetLastError();
}

int launch_fill_zero(void *p, size_t bytes, void *stream) {
  const size_t n = bytes / 4;
  if (n == 0) return 0;
  const size_t blocks = std::min<size_t>((n + kThreads - 1) / kThreads, 1024);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint32_t *>(p), n);
  return (int)hipGetLastError();
}

int launch_stream_read(const void *src, size_t bytes, int workgroups, uint32_t *sink,
                       void *stream) {
  // slices of whole 16-byte pieces, each below 4 GiB (32-bit buffer offsets)
  const size_t per_wg = ((bytes + (size_t)workgroups - 1) / (size_t)workgroups + 15) / 16 * 16;
  if (per_wg >= ((size_t)1 << 32)) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kStreamThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char *>(src), bytes,
                     per_wg, sink);
  return (int)hipGetLastError();
}

int launch_decode(const kivi_dims &d, const kivi_cache &c, const DecodePlan &p, const void *q,
                  float *out, float sm_scale, void *workspace, void *stream) {
  const DecodeArgs da = decode_args(d, c, p, q, out, sm_scale, workspace);
  return launch_decode_any(d, da, encode_args(d, c), false, p.depth,
                           static_cast<hipStream_t>(stream));
}

// ------------------------------------------- allocation-free decode scratch
// One array per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is used.  A static
// __device__ array starts zero-filled; the counters are cleared once more at
// that set-up, by a kernel on the caller's stream, and every decode leaves
// them zero.
namespace {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;

struct ScratchSlot {
  std::once_flag once;
  void *ptr = nullptr;
  int rc = 0;
};

ScratchSlot g_scratch[kMaxDevices];

// The device address of this GPU's scratch (nullptr on failure), set up on
// the first call made on each device.
void *scratch_for_current_device(hipStream_t st, int *rc) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *rc = e != hipSuccess ? (int)e : -1;
    return nullptr;
  }
  ScratchSlot &slot = g_scratch[dev];
  std::call_once(slot.once, [&]() {
    void *ptr = nullptr;
    const hipError_t ge = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (ge != hipSuccess || ptr == nullptr) {
      slot.rc = ge != hipSuccess ? (int)ge : -1;
      return;
    }
    const size_t n = kNoAllocTicketBytes / 4;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, st, static_cast<uint32_t *>(ptr), n);
    const hipError_t le = hipGetLastError();
    if (le != hipSuccess) {
      slot.rc = (int)le;
      return;
    }
    slot.ptr = ptr;
  });
  *rc = slot.rc;
  return slot.ptr;
}

}  // namespace

int launch_decode_noalloc(const kivi_dims &d, const kivi_cache &c, const DecodePlan &p,
                          const void *q, float *out, float sm_scale, void *stream) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  int rc = 0;
  char *base = static_cast<char *>(scratch_for_current_device(st, &rc));
  if (base == nullptr) return rc != 0 ? rc : -1;
  // counters first (fixed place), partials after them; the sizes were checked
  // against the array by the caller
  DecodeArgs da = decode_args(d, c, p, q, out, sm_scale, base + kNoAllocTicketBytes);
  da.tickets = reinterpret_cast<uint32_t *>(base);
  return launch_decode_any(d, da, encode_args(d, c), false, p.depth, st);
}

int launch_decode_vq(const kivi_dims &d, const kivi_cache &c, const DecodePlan &p, const void *q,
                     float *out, float sm_scale, void *workspace, void *stream) {
  DecodeArgs da = decode_args(d, c, p, q, out, sm_scale, workspace);
  // the token-by-token tail: at most R + G - 1 tokens over all waves
  const int waves = kDecodeWaves * p.splits;
  da.win_per_wave = ((d.residual + d.group + waves - 1) / waves + 7) / 8 * 8;
  return launch_decode_any(d, da, encode_args(d, c), false, p.depth,
                           static_cast<hipStream_t>(stream), false, true);
}

int launch_decode_sink(const kivi_dims &d, const kivi_cache &c, const DecodePlan &p,
                       const void *k_sink, const void *v_sink, int n_sink, const void *q,
                       float *out, float sm_scale, double rope_base, void *workspace,
                       void *stream) {
  DecodeArgs da = decode_args(d, c, p, q, out, sm_scale, workspace);
  const bool rope = rope_base != 0.0;
  if (rope) da.rope_log2_base = log2(rope_base);
  set_sink(da, p, k_sink, v_sink, n_sink);
  return launch_decode_any(d, da, encode_args(d, c), false, p.depth,
                           static_cast<hipStream_t>(stream), rope);
}

int launch_decode_rope(const kivi_dims &d, const kivi_cache &c, const DecodePlan &p,
                       const void *q, float *out, float sm_scale, double rope_base,
                       void *workspace, void *stream) {
  DecodeArgs da = decode_args(d, c, p, q, out, sm_scale, workspace);
  da.rope_log2_base = log2(rope_base);
  return launch_decode_any(d, da, encode_args(d, c), false, p.depth,
                           static_cast<hipStream_t>(stream), true);
}

int launch_decode_step(const kivi_dims &d, const kivi_cache &c, const DecodePlan &p,
                       const void *k_new, const void *v_new, const void *k_sink,
                       const void *v_sink, int n_sink, const void *q, float *out,
                       float sm_scale, void *workspace, void *stream) {
  if (!step_in_one_kernel(d, p)) {
    int rc = launch_append(d, c, k_new, v_new, stream);
    if (rc) return rc;
    rc = launch_decode_sink(d, c, p, k_sink, v_sink, n_sink, q, out, sm_scale, 0.0, workspace,
                            stream);
    if (rc) return rc;
    return launch_flush(d, c, stream);
  }
  DecodeArgs da = decode_args(d, c, p, q, out, sm_scale, workspace);
  da.k_new = static_cast<const half_t *>(k_new);
  da.v_new = static_cast<const half_t *>(v_new);
  set_sink(da, p, k_sink, v_sink, n_sink);
  return launch_decode_any(d, da, encode_args(d, c), true, p.depth,
                           static_cast<hipStream_t>(stream));
}

}  // namespace kivi
