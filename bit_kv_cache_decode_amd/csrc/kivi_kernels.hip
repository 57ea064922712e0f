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

#include "kivi_internal.h"

namespace kivi {
namespace {

constexpr int kD = 128;        // head_dim covered by the compiled kernels
constexpr int kThreads = 256;  // 4 waves of 64

using half_t = _Float16;

// ------------------------------------------------------------ wave helpers

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N consecutive lanes (N in 2, 4, 8, 16); every
// lane of a group receives the group sum.  DPP: quad_perm xor1 / xor2, then
// half-row mirror (lane i <-> 7 - i) and row mirror (lane i <-> 15 - i).
template <int N>
__device__ __forceinline__ float lane_group_sum(float v) {
  v += dpp<0xB1>(v);
  if constexpr (N >= 4) v += dpp<0x4E>(v);
  if constexpr (N >= 8) v += dpp<0x141>(v);
  if constexpr (N >= 16) v += dpp<0x140>(v);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Block-wide sums of N values; `red` is shared scratch of 4 * N floats.
template <int N>
__device__ __forceinline__ void block_sum(float (&v)[N], float *red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = wave_sum(v[k]);
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < N; ++k) red[wv * N + k] = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = red[k] + red[N + k] + red[2 * N + k] + red[3 * N + k];
  __syncthreads();
}

__device__ __forceinline__ float block_max(float v, float *red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  v = wave_max(v);
  if (lane == 0) red[wv] = v;
  __syncthreads();
  v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return v;
}

// ---------------------------------------------------------------- encoder
// The fixed fp32 sequence of the quantizer (header comment of kivi.h): no
// contraction, IEEE division, round half to even.
#pragma clang fp contract(off)

struct GroupParams {
  float mn;  // canonical minimum (zero-point)
  float s;   // stored step as fp32
  half_t zero16, scale16;
};

__device__ __forceinline__ GroupParams group_params(float mn_raw, float mx_raw, float levels) {
  GroupParams g;
  g.mn = mn_raw + 0.0f;  // -0 -> +0
  const float mx = mx_raw + 0.0f;
  const float step = (mx - g.mn) / levels;
  g.scale16 = (half_t)step;  // round to nearest even
  g.s = (float)g.scale16;
  g.zero16 = (half_t)g.mn;   // exact: mn is an fp16 value
  return g;
}

__device__ __forceinline__ uint32_t encode_one(float x, float mn, float s, float top) {
  if (s == 0.0f) return 0u;
  float c = rintf((x - mn) / s);
  c = fminf(fmaxf(c, 0.0f), top);
  return (uint32_t)c;
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
  uint32_t *status;
  int heads, R, cap, prefill;
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

template <int G>
__device__ __forceinline__ void load_tile(half_t (*xs)[kD + 8], const half_t *src) {
  for (int i = threadIdx.x; i < G * (kD / 8); i += kThreads) {
    const int t = i / (kD / 8), c = i % (kD / 8);
    *reinterpret_cast<uint4 *>(&xs[t][c * 8]) =
        *reinterpret_cast<const uint4 *>(src + (size_t)t * kD + c * 8);
  }
}

// One workgroup quantizes one tile of G tokens of one (sequence, head):
// keys per channel over the G tokens, values per token over G channels, and
// packs both into the tiled code layout.
template <int BITS, int G>
__global__ __launch_bounds__(kThreads) void encode_kernel(EncodeArgs a) {
  constexpr int W = kD * BITS / 32, CPW = 32 / BITS, NVG = kD / G;
  constexpr float kTop = (float)((1 << BITS) - 1);
  static_assert(G * NVG == kD, "one value group per thread");
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;

  int ntiles, dst0;
  if (a.prefill) {
    int n, r;
    const bool ok = prefill_split(a, b, G, &n, &r) && n - r <= a.cap;
    ntiles = ok ? (n - r) / G : 0;
    dst0 = 0;
  } else {
    const int ql = a.q_len[b], rl = a.r_len[b];
    ntiles = flush_ok(ql, rl, G, a.R, a.cap) ? a.R / G : 0;
    dst0 = ql;
  }
  if (tile >= ntiles) return;

  __shared__ half_t xs[G][kD + 8];
  __shared__ float gmn[kD], gst[kD];

  const size_t bh = (size_t)b * a.heads + h;
  const size_t src_off = (bh * a.src_tokens + (size_t)tile * G) * kD;
  const size_t ktile = bh * (size_t)(a.cap / G) + (size_t)(dst0 / G) + tile;

  // ---- keys: one group per channel over the G tokens of the tile
  load_tile<G>(xs, a.src_k + src_off);
  __syncthreads();
  if (tid < kD) {
    float mn = INFINITY, mx = -INFINITY;
    for (int t = 0; t < G; ++t) {
      const float x = (float)xs[t][tid];
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    const GroupParams g = group_params(mn, mx, kTop);
    a.k_zero[ktile * kD + tid] = g.zero16;
    a.k_scale[ktile * kD + tid] = g.scale16;
    gmn[tid] = g.mn;
    gst[tid] = g.s;
  }
  __syncthreads();
  for (int wi = tid; wi < W * G; wi += kThreads) {
    const int w = wi / G, t = wi % G;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int c = w * CPW + i;
      word |= encode_one((float)xs[t][c], gmn[c], gst[c], kTop) << (i * BITS);
    }
    a.k_codes[ktile * (W * G) + wi] = word;
  }
  __syncthreads();

  // ---- values: one group per (token, G consecutive channels)
  load_tile<G>(xs, a.src_v + src_off);
  __syncthreads();
  // value zero-points and steps are tiled like the codes: [tile][group][token]
  if (tid < kD) {
    const int j = tid / G, t = tid % G;
    float mn = INFINITY, mx = -INFINITY;
    for (int c = 0; c < G; ++c) {
      const float x = (float)xs[t][j * G + c];
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    const GroupParams g = group_params(mn, mx, kTop);
    a.v_zero[ktile * kD + tid] = g.zero16;
    a.v_scale[ktile * kD + tid] = g.scale16;
    gmn[tid] = g.mn;
    gst[tid] = g.s;
  }
  __syncthreads();
  for (int wi = tid; wi < W * G; wi += kThreads) {
    const int w = wi / G, t = wi % G;
    const int gi = ((w * CPW) / G) * G + t;
    const float mn = gmn[gi], s = gst[gi];
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < CPW; ++i)
      word |= encode_one((float)xs[t][w * CPW + i], mn, s, kTop) << (i * BITS);
    a.v_codes[ktile * (W * G) + wi] = word;
  }
}

// Flush commit: runs after encode_kernel on the same stream, so no encode
// workgroup can observe the updated lengths.
__global__ void flush_commit_kernel(EncodeArgs a, int batch, int G) {
  for (int b = threadIdx.x; b < batch; b += blockDim.x) {
    const int ql = a.q_len[b], rl = a.r_len[b];
    if (rl != a.R) continue;
    if (flush_ok(ql, rl, G, a.R, a.cap)) {
      a.q_len[b] = ql + a.R;
      a.r_len[b] = 0;
    } else {
      atomicOr(a.status, (ql < 0 || ql % G) ? KIVI_ST_BAD_LENGTH : KIVI_ST_CAPACITY);
    }
  }
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
    reinterpret_cast<uint4 *>(a.v_res + dst)[i] = reinterpret_cast<const uint4 *>(a.src_v + src)[i];
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
// One workgroup per sequence copies the new token of every head into window
// slot r_len[b], then bumps r_len[b].  Every thread reads r_len[b] before the
// barrier and only thread 0 writes it after, so no thread sees the new value.
__global__ __launch_bounds__(kThreads) void append_kernel(const half_t *k_new, const half_t *v_new,
                                                          half_t *k_res, half_t *v_res,
                                                          int32_t *r_len, uint32_t *status,
                                                          int heads, int R) {
  const int b = blockIdx.x;
  const int r = r_len[b];
  __syncthreads();
  if (r < 0 || r >= R) {
    if (threadIdx.x == 0) atomicOr(status, r < 0 ? KIVI_ST_BAD_LENGTH : KIVI_ST_RESIDUAL_FULL);
    return;
  }
  constexpr int V = kD / 8;  // uint4 per row
  for (int i = threadIdx.x; i < heads * V; i += kThreads) {
    const int h = i / V, c = i % V;
    const size_t bh = (size_t)b * heads + h;
    const size_t src = bh * V + c;
    const size_t dst = (bh * R + r) * V + c;
    reinterpret_cast<uint4 *>(k_res)[dst] = reinterpret_cast<const uint4 *>(k_new)[src];
    reinterpret_cast<uint4 *>(v_res)[dst] = reinterpret_cast<const uint4 *>(v_new)[src];
  }
  __syncthreads();
  if (threadIdx.x == 0) r_len[b] = r + 1;
}

// ----------------------------------------------------------------- decode
//
// Grid (splits, heads, batch), 256 threads = 4 waves.  Split s < sq is a
// quantized split: its waves walk 128-token (B=2) or 64-token (B=4)
// sub-chunks of the quantized tokens, sub-chunk i of the split going to wave
// i % 4.  Split s >= sq is a window split over 128 fp16 window tokens, 32 per
// wave.  Every wave works on its own (no block barrier until the end); every
// lane keeps its own online-softmax state (running max, sum, value sums) for
// the tokens it sees.  At the end the lanes and waves of the workgroup are
// combined in LDS into one partial state (max m, sum l, unnormalised value
// sums) in log2 units, published to the workspace; the workgroup that takes
// the last ticket of its (sequence, head) merges all partials by log-sum-exp
// rescaling and writes the output.
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
// sums at the end.

struct DecodeArgs {
  const uint32_t *k_codes, *v_codes;
  const half_t *k_scale, *k_zero, *v_scale, *v_zero, *k_res, *v_res;
  const int32_t *q_len, *r_len;
  uint32_t *status;
  const half_t *q;
  float *out, *part;
  uint32_t *tickets;
  float qscale;  // sm_scale * log2(e)
  int heads, R, cap, kw, sq, nr, part_stride;
};

constexpr int kMaxSplits = 128;
constexpr int kPartHead = 4;   // m, l, 2 pad floats before the 128 values
constexpr int kWinWave = 32;   // window tokens per wave
constexpr int kWinRound = 16;  // window tokens per wave per round

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

template <int BITS, int G>
struct DecCfg {
  static constexpr int W = kD * BITS / 32;     // words per token
  static constexpr int CPW = 32 / BITS;        // channels per word
  static constexpr int HP = CPW / 2;           // code pairs per word
  static constexpr int SUB = 1024 / W;         // tokens per sub-chunk
  static constexpr int TQS = 64 / W;           // token quads per wave-load
  static constexpr int TPL = 4 * TQS;          // tokens per wave-load
  static constexpr int NL = SUB / TPL;         // wave-loads per sub-chunk and operand
  static constexpr int NVG = kD / G;            // value groups per token
  static constexpr int NTS = SUB >= G ? SUB / G : 1;  // key tiles a sub-chunk touches
  static_assert(NL == 4, "four 16-byte loads per lane per sub-chunk and operand");
  static_assert(G % TPL == 0, "a wave-load stays inside one tile");
};

template <int BITS, int G>
struct DecSmem {
  using C = DecCfg<BITS, G>;
  float qs[kD];   // sm_scale * log2(e) * q
  float qsf[kD];  // qs times the code-position factor 2^(24 - e) of each channel
  struct {
    float acc[4][4][kD];  // [wave][row][channel]
    float bias[4][4][16]; // [wave][row][word]
    float m[4], l[4];
  } fin;
  union {
    struct {
      float qp[C::NTS][kD];
      float cz[C::NTS][C::W];
    } wave[4];
    struct {
      float m[kMaxSplits], l[kMaxSplits], e[kMaxSplits];
      float acc[8][kD];
    } mg;
  } u;
  float red[32];
  int ticket;
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
  else return p <= 1 ? 4 * p : 4 * (p - 2);
}

// 2^(24 - e) for channel i of a word: the factor between an extracted code's
// fp16 value and the code.
template <int BITS>
__device__ __forceinline__ float code_factor(int i) {
  return __builtin_ldexpf(1.0f, 24 - code_offset<BITS>(i));
}

// Word u masked to code pair p (channels p and p + HP), each half holding its
// code at bit offset code_offset(p).  uh is u shifted right by 10 (B = 2) or
// 8 (B = 4), which brings the upper pairs of each half into the mantissa.
template <int BITS, int P>
__device__ __forceinline__ uint32_t pair_bits(uint32_t u, uint32_t uh) {
  if constexpr (BITS == 2) {
    if constexpr (P <= 4) return u & (0x00030003u << (2 * P));
    else return uh & (0x00030003u << (2 * (P - 5)));
  } else {
    if constexpr (P <= 1) return u & (0x000F000Fu << (4 * P));
    else return uh & (0x000F000Fu << (4 * (P - 2)));
  }
}

template <int BITS>
__device__ __forceinline__ uint32_t upper_pairs(uint32_t u) {
  return u >> (BITS == 2 ? 10 : 8);
}

// c0 + sum_i q[i] * code_i * 2^(e_i - 24) over the word's channels.
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
__device__ __forceinline__ float dot_word(uint32_t u, const float *q, float c0) {
  float a0 = c0, a1 = 0.0f;
  dot_pairs<BITS>(u, upper_pairs<BITS>(u), q, a0, a1);
  return a0 + a1;
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

__device__ __forceinline__ uint32_t u4_get(const uint4 &v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Combine the per-lane states of one wave and publish them to sm.fin.
// CPW: channels per lane; WPR: lanes per token slot; FOLD8: lanes l and l^8
// hold the same channels (two slots per 16-lane row).
template <int CPW, int WPR, bool FOLD8>
__device__ __forceinline__ void wave_publish(float (&fin_acc)[4][kD], float (&fin_bias)[4][16],
                                             float &fin_m, float &fin_l, float m, float l,
                                             float *acc, float bias) {
  const int lane = threadIdx.x & 63;
  const int w = lane % WPR, row = lane >> 4;
  const float M = wave_max(m);
  const float e = (m == -INFINITY) ? 0.0f : exp2f(m - M);
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

template <int BITS, int G>
__device__ __forceinline__ void quantized_split(const DecodeArgs &a, DecSmem<BITS, G> &sm, size_t bh,
                                                int split, int ql) {
  using C = DecCfg<BITS, G>;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int w = lane % C::W, slot = lane / C::W;
  const int jg = (w * C::CPW) / G;  // value group of this lane's channels
  const size_t tps = (size_t)(a.cap / G);
  const uint32_t *kcb = a.k_codes + bh * tps * (C::W * G);
  const uint32_t *vcb = a.v_codes + bh * tps * (C::W * G);
  const half_t *ksb = a.k_scale + bh * tps * kD;
  const half_t *kzb = a.k_zero + bh * tps * kD;
  const half_t *vsb = a.v_scale + bh * tps * kD;
  const half_t *vzb = a.v_zero + bh * tps * kD;
  auto &st = sm.u.wave[wv];
  const float qs0 = sm.qs[2 * lane], qs1 = sm.qs[2 * lane + 1];
  const float qf0 = sm.qsf[2 * lane], qf1 = sm.qsf[2 * lane + 1];

  float m = -INFINITY, l = 0.0f, bias = 0.0f;
  float acc[C::CPW];
#pragma unroll
  for (int i = 0; i < C::CPW; ++i) acc[i] = 0.0f;

  const int sub0 = split * 4 * a.kw;
  for (int c = 0; c < a.kw; ++c) {
    const int T0 = (sub0 + wv + 4 * c) * C::SUB;
    if (T0 >= ql) break;
    const int nvl = min(C::NL, (ql - T0) / C::TPL);
    const int tile0 = T0 / G;

    // ---- key metadata (2 channels per lane per touched tile) and key codes
    uint32_t ksr[C::NTS], kzr[C::NTS];
#pragma unroll
    for (int k = 0; k < C::NTS; ++k) {
      if ((tile0 + k) * G < ql) {
        ksr[k] = *reinterpret_cast<const uint32_t *>(ksb + (size_t)(tile0 + k) * kD + 2 * lane);
        kzr[k] = *reinterpret_cast<const uint32_t *>(kzb + (size_t)(tile0 + k) * kD + 2 * lane);
      } else {
        ksr[k] = kzr[k] = 0u;
      }
    }
    uint4 kc[C::NL];
#pragma unroll
    for (int j = 0; j < C::NL; ++j) {
      if (j < nvl) {
        const int t = T0 + j * C::TPL;
        const int tile = t / G, pos = t % G + 4 * slot;
        kc[j] = *reinterpret_cast<const uint4 *>(kcb + ((size_t)tile * C::W + w) * G + pos);
      } else {
        kc[j] = make_uint4(0u, 0u, 0u, 0u);
      }
    }

    // ---- stage q'' = qsf * s and the zero terms of the touched tiles
#pragma unroll
    for (int k = 0; k < C::NTS; ++k) {
      if ((tile0 + k) * G < ql) {
        st.qp[k][2 * lane] = mix_lo(qf0, ksr[k], 0.0f);
        st.qp[k][2 * lane + 1] = mix_hi(qf1, ksr[k], 0.0f);
        float zc = mix_lo(qs0, kzr[k], mix_hi(qs1, kzr[k], 0.0f));
        zc = lane_group_sum<C::CPW / 2>(zc);
        if ((lane % (C::CPW / 2)) == 0) st.cz[k][lane / (C::CPW / 2)] = zc;
      }
    }
    __builtin_amdgcn_wave_barrier();

    // ---- scores (every lane of a token slot ends with the full sums)
    float s[C::NL][4];
#pragma unroll
    for (int j = 0; j < C::NL; ++j) {
      if (j < nvl) {
        const int k = ((T0 % G) + j * C::TPL) / G;
        float qv[C::CPW];
#pragma unroll
        for (int i = 0; i < C::CPW; i += 4) {
          const float4 t4 = *reinterpret_cast<const float4 *>(&st.qp[k][w * C::CPW + i]);
          qv[i] = t4.x;
          qv[i + 1] = t4.y;
          qv[i + 2] = t4.z;
          qv[i + 3] = t4.w;
        }
        const float c0 = st.cz[k][w];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s[j][i] = lane_group_sum<C::W>(dot_word<BITS>(u4_get(kc[j], i), qv, c0));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) s[j][i] = -INFINITY;
      }
    }
    __builtin_amdgcn_wave_barrier();

    // ---- value codes and this lane's value-group metadata
    uint4 vc[C::NL];
    uint2 vsr[C::NL], vzr[C::NL];
#pragma unroll
    for (int j = 0; j < C::NL; ++j) {
      if (j < nvl) {
        const int t = T0 + j * C::TPL;
        const int tile = t / G, pos = t % G + 4 * slot;
        vc[j] = *reinterpret_cast<const uint4 *>(vcb + ((size_t)tile * C::W + w) * G + pos);
        const size_t mo = ((size_t)tile * C::NVG + jg) * G + pos;
        vsr[j] = *reinterpret_cast<const uint2 *>(vsb + mo);
        vzr[j] = *reinterpret_cast<const uint2 *>(vzb + mo);
      } else {
        vc[j] = make_uint4(0u, 0u, 0u, 0u);
        vsr[j] = vzr[j] = make_uint2(0u, 0u);
      }
    }

    // ---- per-lane online softmax over this lane's tokens
    float mc = m;
#pragma unroll
    for (int j = 0; j < C::NL; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) mc = fmaxf(mc, s[j][i]);
    const float corr = exp2f(m - mc);  // 0 on the first sub-chunk (m = -inf)
    m = mc;
    l *= corr;
    bias *= corr;
#pragma unroll
    for (int i = 0; i < C::CPW; ++i) acc[i] *= corr;

    // ---- weighted value sum
#pragma unroll
    for (int j = 0; j < C::NL; ++j) {
      if (j < nvl) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = exp2f(s[j][i] - m);
          l += p;
          const uint32_t sw = i < 2 ? vsr[j].x : vsr[j].y;
          const uint32_t zw = i < 2 ? vzr[j].x : vzr[j].y;
          const float pp = (i & 1) ? mix_hi(p, sw, 0.0f) : mix_lo(p, sw, 0.0f);
          bias = (i & 1) ? mix_hi(p, zw, bias) : mix_lo(p, zw, bias);
          const uint32_t u = u4_get(vc[j], i);
          axpy_pairs<BITS>(u, upper_pairs<BITS>(u), pp, acc);
        }
      }
    }
  }
  wave_publish<C::CPW, C::W, C::W == 8>(sm.fin.acc[wv], sm.fin.bias[wv], sm.fin.m[wv],
                                         sm.fin.l[wv], m, l, acc, bias);
}

// Window split: up to 128 fp16 window tokens, 32 per wave in two rounds of
// 16; 16 lanes per token, 8 channels per lane.
template <int BITS, int G>
__device__ __forceinline__ void window_split(const DecodeArgs &a, DecSmem<BITS, G> &sm, size_t bh,
                                             int rs, int rl) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int slot = lane >> 4, part = lane & 15;
  float qv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) qv[i] = sm.qs[part * 8 + i];
  float m = -INFINITY, l = 0.0f;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  for (int r = 0; r < kWinWave / kWinRound; ++r) {
    const int t0 = rs + wv * kWinWave + r * kWinRound;
    const int n = min(kWinRound, rl - t0);
    if (n <= 0) break;
    uint4 kx[4], vx[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tok = j * 4 + slot;
      if (tok < n) {
        const size_t off = (bh * a.R + t0 + tok) * kD + part * 8;
        kx[j] = *reinterpret_cast<const uint4 *>(a.k_res + off);
        vx[j] = *reinterpret_cast<const uint4 *>(a.v_res + off);
      } else {
        kx[j] = vx[j] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    float s[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j * 4 < n) {
        float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t u = u4_get(kx[j], i);
          a0 = mix_lo(qv[2 * i], u, a0);
          a1 = mix_hi(qv[2 * i + 1], u, a1);
        }
        const float t = lane_group_sum<16>(a0 + a1);
        s[j] = (j * 4 + slot < n) ? t : -INFINITY;
      } else {
        s[j] = -INFINITY;
      }
    }
    float mc = m;
#pragma unroll
    for (int j = 0; j < 4; ++j) mc = fmaxf(mc, s[j]);
    if (mc != -INFINITY) {
      const float corr = exp2f(m - mc);
      m = mc;
      l *= corr;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= corr;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = exp2f(s[j] - m);  // 0 for absent tokens
        l += p;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t u = u4_get(vx[j], i);
          acc[2 * i] = mix_lo(p, u, acc[2 * i]);
          acc[2 * i + 1] = mix_hi(p, u, acc[2 * i + 1]);
        }
      }
    }
  }
  wave_publish<8, 16, false>(sm.fin.acc[wv], sm.fin.bias[wv], sm.fin.m[wv], sm.fin.l[wv], m, l,
                             acc, 0.0f);
}

template <int BITS, int G>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  using C = DecCfg<BITS, G>;
  __shared__ DecSmem<BITS, G> sm;
  const int tid = threadIdx.x;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bh = (size_t)b * a.heads + h;
  const int S = a.sq + a.nr;

  int ql = a.q_len[b], rl = a.r_len[b];
  if (!(ql >= 0 && ql <= a.cap && (ql % G) == 0 && rl >= 0 && rl <= a.R)) {
    if (split == 0 && h == 0 && tid == 0) atomicOr(a.status, KIVI_ST_BAD_LENGTH);
    ql = 0;
    rl = 0;
  }
  const bool quant = split < a.sq;
  if (tid < kD / 2) {
    const uint32_t r = reinterpret_cast<const uint32_t *>(a.q + bh * kD)[tid];
    const half2_t hq = __builtin_bit_cast(half2_t, r);
    const float q0 = (float)hq.x * a.qscale, q1 = (float)hq.y * a.qscale;
    sm.qs[2 * tid] = q0;
    sm.qs[2 * tid + 1] = q1;
    sm.qsf[2 * tid] = q0 * code_factor<BITS>((2 * tid) % C::CPW);
    sm.qsf[2 * tid + 1] = q1 * code_factor<BITS>((2 * tid + 1) % C::CPW);
  }
  __syncthreads();

  if (quant) quantized_split<BITS, G>(a, sm, bh, split, ql);
  else window_split<BITS, G>(a, sm, bh, (split - a.sq) * 4 * kWinWave, rl);
  __syncthreads();

  // ---- combine the four waves into the workgroup's partial state
  float M = -INFINITY;
#pragma unroll
  for (int x = 0; x < 4; ++x)
    if (sm.fin.l[x] > 0.0f) M = fmaxf(M, sm.fin.m[x]);
  float L = 0.0f, acc_out = 0.0f;
  if (M != -INFINITY) {
    const int cpw = quant ? C::CPW : 8;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const float e = sm.fin.l[x] > 0.0f ? exp2f(sm.fin.m[x] - M) : 0.0f;
      L += e * sm.fin.l[x];
      if (tid < kD && e != 0.0f) {
        float sa = 0.0f, sb = 0.0f;
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          sa += sm.fin.acc[x][y][tid];
          sb += sm.fin.bias[x][y][tid / cpw];
        }
        acc_out += e * (quant ? fmaf(sa, code_factor<BITS>(tid % C::CPW), sb) : sa);
      }
    }
  }

  // ---- publish the partial state and take a ticket
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
    sm.ticket = (int)__hip_atomic_fetch_add(a.tickets + bh, 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (sm.ticket != S - 1) return;

  // ---- last workgroup of this (sequence, head): merge all partials, read
  // with device-scope atomic loads (coherent with the stores above)
  const float *P0 = a.part + bh * S * (size_t)a.part_stride;
  for (int s = tid; s < S; s += kThreads) {
    sm.u.mg.m[s] = load_agent(P0 + (size_t)s * a.part_stride);
    sm.u.mg.l[s] = load_agent(P0 + (size_t)s * a.part_stride + 1);
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int s = tid; s < S; s += kThreads)
    if (sm.u.mg.l[s] > 0.0f) mx = fmaxf(mx, sm.u.mg.m[s]);
  mx = block_max(mx, sm.red);
  float lsum[1] = {0.0f};
  for (int s = tid; s < S; s += kThreads) {
    const float e = sm.u.mg.l[s] > 0.0f ? exp2f(sm.u.mg.m[s] - mx) : 0.0f;
    sm.u.mg.e[s] = e;
    lsum[0] += e * sm.u.mg.l[s];
  }
  block_sum<1>(lsum, sm.red);
  const int cq = tid & 31, sl = tid >> 5;
  float A[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int s = sl; s < S; s += 8) {
    const float e = sm.u.mg.e[s];
    if (e != 0.0f) {
      const float *src = P0 + (size_t)s * a.part_stride + kPartHead + 4 * cq;
#pragma unroll
      for (int i = 0; i < 4; ++i) A[i] = fmaf(e, load_agent(src + i), A[i]);
    }
  }
  *reinterpret_cast<float4 *>(&sm.u.mg.acc[sl][4 * cq]) = make_float4(A[0], A[1], A[2], A[3]);
  __syncthreads();
  if (tid < kD) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += sm.u.mg.acc[i][tid];
    a.out[bh * kD + tid] = lsum[0] > 0.0f ? s / lsum[0] : 0.0f;
  }
  if (tid == 0) __hip_atomic_store(a.tickets + bh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  return (int)hipErrorInvalidValue;
}

template <int BITS, int G>
int launch_decode_t(const DecodeArgs &da, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<BITS, G>), grid, dim3(kThreads), 0, st, da);
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
  ea.heads = d.heads;
  ea.R = d.residual;
  ea.cap = d.capacity;
  return ea;
}

}  // namespace

int launch_append(const kivi_dims &d, const kivi_cache &c, const void *k_new, const void *v_new,
                  void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(append_kernel, dim3(d.batch), dim3(kThreads), 0, st,
                     static_cast<const half_t *>(k_new), static_cast<const half_t *>(v_new),
                     static_cast<half_t *>(c.k_res), static_cast<half_t *>(c.v_res), c.r_len,
                     c.status, d.heads, d.residual);
  return (int)hipGetLastError();
}

int launch_flush(const kivi_dims &d, const kivi_cache &c, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  EncodeArgs ea = encode_args(d, c);
  ea.src_k = ea.k_res;
  ea.src_v = ea.v_res;
  ea.src_tokens = d.residual;
  ea.prefill = 0;
  int rc = launch_encode(d.bits, d.group, ea, dim3(d.residual / d.group, d.heads, d.batch), st);
  if (rc) return rc;
  hipLaunchKernelGGL(flush_commit_kernel, dim3(1), dim3(kThreads), 0, st, ea, d.batch, d.group);
  return (int)hipGetLastError();
}

int launch_prefill(const kivi_dims &d, const kivi_cache &c, const void *k, const void *v,
                   int32_t src_len, const int32_t *len, const int32_t *res, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  EncodeArgs ea = encode_args(d, c);
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

int launch_decode(const kivi_dims &d, const kivi_cache &c, const DecodePlan &p, const void *q,
                  float *out, float sm_scale, void *workspace, void *stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
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
  da.kw = p.kw;
  da.sq = p.sq;
  da.nr = p.nr;
  da.part_stride = (int)p.part_floats;
  const dim3 grid(p.splits, d.heads, d.batch);
  const int G = d.group;
  if (d.bits == 2 && G == 32) return launch_decode_t<2, 32>(da, grid, st);
  if (d.bits == 2 && G == 64) return launch_decode_t<2, 64>(da, grid, st);
  if (d.bits == 2 && G == 128) return launch_decode_t<2, 128>(da, grid, st);
  if (d.bits == 4 && G == 32) return launch_decode_t<4, 32>(da, grid, st);
  if (d.bits == 4 && G == 64) return launch_decode_t<4, 64>(da, grid, st);
  if (d.bits == 4 && G == 128) return launch_decode_t<4, 128>(da, grid, st);
  return (int)hipErrorInvalidValue;
}

}  // namespace kivi
