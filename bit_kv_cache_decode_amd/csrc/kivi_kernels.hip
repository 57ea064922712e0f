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
  const size_t vtok0 = bh * (size_t)a.cap + dst0 + (size_t)tile * G;
  if (tid < kD) {
    const int t = tid / NVG, j = tid % NVG;
    float mn = INFINITY, mx = -INFINITY;
    for (int c = 0; c < G; ++c) {
      const float x = (float)xs[t][j * G + c];
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    const GroupParams g = group_params(mn, mx, kTop);
    a.v_zero[vtok0 * NVG + tid] = g.zero16;
    a.v_scale[vtok0 * NVG + tid] = g.scale16;
    gmn[tid] = g.mn;
    gst[tid] = g.s;
  }
  __syncthreads();
  for (int wi = tid; wi < W * G; wi += kThreads) {
    const int w = wi / G, t = wi % G;
    const int gi = t * NVG + (w * CPW) / G;
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
// Grid (splits, heads, batch), 256 threads.  Split s < sq covers quantized
// tokens [s * kper * CH, (s + 1) * kper * CH) in chunks of CH tokens; split
// s >= sq covers window tokens [(s - sq) * 64, ...).  Each split produces the
// partial softmax state (max m, sum l, unnormalised weighted value sum) in
// log2 units, writes it to the workspace and takes a ticket; the workgroup
// that takes the last ticket of its (sequence, head) merges all partials by
// log-sum-exp rescaling and writes the output, then resets the ticket.
//
// Dequantization is folded into the dot products:
//   score_t = sum_d q'_d * K_hat[t,d]
//           = sum_d (q'_d * s_{g,d}) * c_{t,d} + sum_d q'_d * z_{g,d}
//   out_d   = sum_t p_t * (z_{t,j} + s_{t,j} * c_{t,d})
//           = sum_t (p_t * s_{t,j}) * c_{t,d} + sum_t p_t * z_{t,j}
// with q' = sm_scale * log2(e) * q, so that p_t = exp2(score_t - max).
// Codes are converted with a byte mask and v_cvt_f32_ubyteN: the mask keeps
// one code per byte, shifted left by B*k bits; the factor 2^(B*k) is folded
// into the per-channel multipliers (keys) or removed from the accumulators
// at the end (values).

struct DecodeArgs {
  const uint32_t *k_codes, *v_codes;
  const half_t *k_scale, *k_zero, *v_scale, *v_zero, *k_res, *v_res;
  const int32_t *q_len, *r_len;
  uint32_t *status;
  const half_t *q;
  float *out, *part;
  uint32_t *tickets;
  float qscale;  // sm_scale * log2(e)
  int heads, R, cap, kper, sq, nr, win_chunk, part_stride;
};

constexpr int kMaxSplits = 128;
constexpr int kPartHead = 4;  // m, l, 2 pad floats before the 128 values

template <int BITS, int G>
struct DecCfg {
  static constexpr int W = kD * BITS / 32;      // words per token
  static constexpr int CPW = 32 / BITS;         // channels per word
  static constexpr int CH = BITS == 2 ? 512 : 256;  // tokens per chunk
  static constexpr int NT = CH / G;             // tiles per chunk
  static constexpr int TQS = 64 / W;            // token quads per wave-load
  static constexpr int LPT = G * W / 256;       // wave-loads per tile
  static constexpr int NL = CH * W / 1024;      // wave-loads per wave per chunk
  static constexpr int NVG = kD / G;            // value groups per token
  static constexpr int TPT = CH / kThreads;     // chunk tokens per thread
  static constexpr int KTW = (NT + 3) / 4;      // key tiles staged per wave
  static_assert(NL == 4, "four 16-byte loads per lane per chunk");
  static_assert(LPT >= 1 && TPT >= 1, "bad tiling");
};

template <int BITS, int G>
struct DecSmem {
  using C = DecCfg<BITS, G>;
  float qs[kD];
  float sc[C::CH];
  float cz[C::NT][C::W];
  float vbias[C::NVG];
  float red[4 * 8];
  int ticket;
  union {
    struct {
      float qp[C::NT][kD];
      float pv[C::NVG][C::CH];
    } s;
    float accred[4][4][kD];
    struct {
      float m[kMaxSplits], l[kMaxSplits], e[kMaxSplits];
      float acc[8][kD];
    } mg;
  } u;
};

// Keeps the compiler from folding the byte mask into per-code bit-field
// extracts: with the masked word opaque, each (m >> 8j) & 0xff conversion
// becomes a single v_cvt_f32_ubyte{j} of the whole word.
__device__ __forceinline__ uint32_t opaque(uint32_t m) {
  __asm__("" : "+v"(m));
  return m;
}

__device__ __forceinline__ void store_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_agent(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Power-of-two factor of channel d's code inside its byte: 2^(B * k).
template <int BITS>
__device__ __forceinline__ float inv_pos_scale(int d) {
  if constexpr (BITS == 2) {
    const int k = d & 3;
    return k == 0 ? 1.0f : k == 1 ? 0.25f : k == 2 ? 0.0625f : 0.015625f;
  } else {
    return (d & 1) ? 0.0625f : 1.0f;
  }
}

// acc + sum over the word's channels of q[i] * code_i * 2^(B * pos_i).
template <int BITS>
__device__ __forceinline__ float dot_word(uint32_t u, const float *q, float acc) {
  if constexpr (BITS == 2) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t m = opaque(u & (0x03030303u << (2 * k)));
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = fmaf(q[4 * j + k], (float)((m >> (8 * j)) & 0xFFu), acc);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t m = opaque(u & (0x0F0F0F0Fu << (4 * k)));
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = fmaf(q[2 * j + k], (float)((m >> (8 * j)) & 0xFFu), acc);
    }
  }
  return acc;
}

// acc[i] += p * code_i * 2^(B * pos_i) over the word's channels.
template <int BITS>
__device__ __forceinline__ void axpy_word(uint32_t u, float p, float *acc) {
  if constexpr (BITS == 2) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t m = opaque(u & (0x03030303u << (2 * k)));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[4 * j + k] = fmaf(p, (float)((m >> (8 * j)) & 0xFFu), acc[4 * j + k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t m = opaque(u & (0x0F0F0F0Fu << (4 * k)));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[2 * j + k] = fmaf(p, (float)((m >> (8 * j)) & 0xFFu), acc[2 * j + k]);
    }
  }
}

__device__ __forceinline__ uint32_t u4_get(const uint4 &v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <int NVG>
__device__ __forceinline__ void load_vmeta(const half_t *p, float (&out)[NVG]) {
  if constexpr (NVG == 4) {
    const uint2 r = *reinterpret_cast<const uint2 *>(p);
    const half_t *h = reinterpret_cast<const half_t *>(&r);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = (float)h[i];
  } else if constexpr (NVG == 2) {
    const uint32_t r = *reinterpret_cast<const uint32_t *>(p);
    const half_t *h = reinterpret_cast<const half_t *>(&r);
    out[0] = (float)h[0];
    out[1] = (float)h[1];
  } else {
    out[0] = (float)p[0];
  }
}

// Quantized split: chunks of CH tokens with an online softmax across chunks.
// Leaves M, L (log2-domain running max and sum) and, for threads < 128, the
// unnormalised output of channel tid in *acc_out.
template <int BITS, int G>
__device__ __forceinline__ void quantized_split(const DecodeArgs &a, DecSmem<BITS, G> &sm, size_t bh,
                                                int split, int ql, float &M, float &L,
                                                float &acc_out) {
  using C = DecCfg<BITS, G>;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int w = lane % C::W, slot = lane / C::W;
  float acc[C::CPW];
#pragma unroll
  for (int i = 0; i < C::CPW; ++i) acc[i] = 0.0f;
  if (tid < C::NVG) sm.vbias[tid] = 0.0f;

  const int tok_begin = split * a.kper * C::CH;
  const size_t tiles_per_seq = (size_t)(a.cap / G);
  bool any = false;
  for (int c = 0; c < a.kper; ++c) {
    const int t0 = tok_begin + c * C::CH;
    const int ntok = min(C::CH, ql - t0);
    if (ntok <= 0) break;
    any = true;
    const int ntv = ntok / G;
    const size_t tile0 = bh * tiles_per_seq + t0 / G;

    // ---- issue every load of the chunk: key meta, value meta, codes
    uint32_t ksr[C::KTW], kzr[C::KTW];
#pragma unroll
    for (int i = 0; i < C::KTW; ++i) {
      const int g = wv + 4 * i;
      if (g < ntv) {
        const size_t off = (tile0 + g) * kD + 2 * lane;
        ksr[i] = *reinterpret_cast<const uint32_t *>(a.k_scale + off);
        kzr[i] = *reinterpret_cast<const uint32_t *>(a.k_zero + off);
      } else {
        ksr[i] = kzr[i] = 0u;
      }
    }
    float vsr[C::TPT][C::NVG], vzr[C::TPT][C::NVG];
#pragma unroll
    for (int i = 0; i < C::TPT; ++i) {
      const int t = tid + kThreads * i;
      if (t < ntok) {
        const size_t off = (bh * a.cap + t0 + t) * C::NVG;
        load_vmeta<C::NVG>(a.v_scale + off, vsr[i]);
        load_vmeta<C::NVG>(a.v_zero + off, vzr[i]);
      } else {
#pragma unroll
        for (int j = 0; j < C::NVG; ++j) vsr[i][j] = vzr[i][j] = 0.0f;
      }
    }
    uint4 kc[C::NL], vc[C::NL];
#pragma unroll
    for (int j = 0; j < C::NL; ++j) {
      const int n = wv * C::NL + j, tile = n / C::LPT;
      const int tq = (n % C::LPT) * C::TQS + slot;
      if (tile < ntv) {
        const size_t off = (tile0 + tile) * (C::W * G) + w * G + 4 * tq;
        kc[j] = *reinterpret_cast<const uint4 *>(a.k_codes + off);
        vc[j] = *reinterpret_cast<const uint4 *>(a.v_codes + off);
      } else {
        kc[j] = vc[j] = make_uint4(0u, 0u, 0u, 0u);
      }
    }

    // ---- key staging: q'_{g,d} = qs_d * s_{g,d} / 2^(B*pos), zero term per word
#pragma unroll
    for (int i = 0; i < C::KTW; ++i) {
      const int g = wv + 4 * i;
      if (g < ntv) {
        const half_t *hs = reinterpret_cast<const half_t *>(&ksr[i]);
        const half_t *hz = reinterpret_cast<const half_t *>(&kzr[i]);
        const int d0 = 2 * lane;
        const float q0 = sm.qs[d0], q1 = sm.qs[d0 + 1];
        sm.u.s.qp[g][d0] = q0 * (float)hs[0] * inv_pos_scale<BITS>(d0);
        sm.u.s.qp[g][d0 + 1] = q1 * (float)hs[1] * inv_pos_scale<BITS>(d0 + 1);
        float zc = q0 * (float)hz[0] + q1 * (float)hz[1];
        zc = lane_group_sum<C::CPW / 2>(zc);
        if ((lane % (C::CPW / 2)) == 0) sm.cz[g][lane / (C::CPW / 2)] = zc;
      }
    }
    __syncthreads();

    // ---- scores of the chunk
#pragma unroll
    for (int j = 0; j < C::NL; ++j) {
      const int n = wv * C::NL + j, tile = n / C::LPT;
      if (tile < ntv) {
        const int tq = (n % C::LPT) * C::TQS + slot;
        float qv[C::CPW];
#pragma unroll
        for (int i = 0; i < C::CPW; i += 4) {
          const float4 t4 = *reinterpret_cast<const float4 *>(&sm.u.s.qp[tile][w * C::CPW + i]);
          qv[i] = t4.x;
          qv[i + 1] = t4.y;
          qv[i + 2] = t4.z;
          qv[i + 3] = t4.w;
        }
        const float c0 = sm.cz[tile][w];
        float s4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) s4[i] = lane_group_sum<C::W>(dot_word<BITS>(u4_get(kc[j], i), qv, c0));
        if (w == 0)
          *reinterpret_cast<float4 *>(&sm.sc[tile * G + 4 * tq]) = make_float4(s4[0], s4[1], s4[2], s4[3]);
      }
    }
    __syncthreads();

    // ---- chunk softmax (online across chunks), value staging
    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < C::TPT; ++i) {
      const int t = tid + kThreads * i;
      if (t < ntok) mloc = fmaxf(mloc, sm.sc[t]);
    }
    mloc = block_max(mloc, sm.red);
    const float Mn = fmaxf(M, mloc);
    const float corr = exp2f(M - Mn);  // 0 on the first chunk (M = -inf)
    float sums[1 + C::NVG];
#pragma unroll
    for (int j = 0; j <= C::NVG; ++j) sums[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < C::TPT; ++i) {
      const int t = tid + kThreads * i;
      if (t < ntok) {
        const float p = exp2f(sm.sc[t] - Mn);
        sums[0] += p;
#pragma unroll
        for (int j = 0; j < C::NVG; ++j) {
          sm.u.s.pv[j][t] = p * vsr[i][j];
          sums[1 + j] += p * vzr[i][j];
        }
      }
    }
    block_sum<1 + C::NVG>(sums, sm.red);  // also orders the pv writes before the reads below
    L = L * corr + sums[0];
    M = Mn;
    if (tid < C::NVG) sm.vbias[tid] = sm.vbias[tid] * corr + sums[1 + tid];
#pragma unroll
    for (int i = 0; i < C::CPW; ++i) acc[i] *= corr;

    // ---- weighted value sum
#pragma unroll
    for (int j = 0; j < C::NL; ++j) {
      const int n = wv * C::NL + j, tile = n / C::LPT;
      if (tile < ntv) {
        const int tq = (n % C::LPT) * C::TQS + slot;
        const int jg = (w * C::CPW) / G;
        const float4 pp = *reinterpret_cast<const float4 *>(&sm.u.s.pv[jg][tile * G + 4 * tq]);
        axpy_word<BITS>(vc[j].x, pp.x, acc);
        axpy_word<BITS>(vc[j].y, pp.y, acc);
        axpy_word<BITS>(vc[j].z, pp.z, acc);
        axpy_word<BITS>(vc[j].w, pp.w, acc);
      }
    }
    __syncthreads();  // qp / pv / sc are rewritten by the next chunk
  }
  if (!any) return;

  // ---- reduce the per-lane channel sums over lanes and waves
  const int row = lane >> 4;
  if constexpr (C::W == 8) {
#pragma unroll
    for (int i = 0; i < C::CPW; ++i) acc[i] += dpp<0x128>(acc[i]);  // row_ror:8 pairs lanes l, l^8
    if ((lane & 8) == 0) {
#pragma unroll
      for (int i = 0; i < C::CPW; i += 4)
        *reinterpret_cast<float4 *>(&sm.u.accred[wv][row][w * C::CPW + i]) =
            make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < C::CPW; i += 4)
      *reinterpret_cast<float4 *>(&sm.u.accred[wv][row][w * C::CPW + i]) =
          make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
  }
  __syncthreads();
  if (tid < kD) {
    float s = 0.0f;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) s += sm.u.accred[x][y][tid];
    acc_out = s * inv_pos_scale<BITS>(tid) + sm.vbias[tid / G];
  }
}

// Window split: up to 64 fp16 tokens, 16 lanes per token (8 channels each).
template <int BITS, int G>
__device__ __forceinline__ void window_split(const DecodeArgs &a, DecSmem<BITS, G> &sm, size_t bh,
                                             int rs, int n, float &M, float &L, float &acc_out) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int slot = lane >> 4, part = lane & 15;
  const half_t *kr = a.k_res + (bh * a.R + rs) * kD;
  const half_t *vr = a.v_res + (bh * a.R + rs) * kD;
  uint4 kx[4], vx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = (wv * 4 + j) * 4 + slot;
    if (tok < n) {
      kx[j] = *reinterpret_cast<const uint4 *>(kr + (size_t)tok * kD + part * 8);
      vx[j] = *reinterpret_cast<const uint4 *>(vr + (size_t)tok * kD + part * 8);
    } else {
      kx[j] = vx[j] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  float qv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) qv[i] = sm.qs[part * 8 + i];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if ((wv * 4 + j) * 4 < n) {
      const int tok = (wv * 4 + j) * 4 + slot;
      const half_t *hk = reinterpret_cast<const half_t *>(&kx[j]);
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) s = fmaf(qv[i], (float)hk[i], s);
      s = lane_group_sum<16>(s);
      if (part == 0 && tok < n) sm.sc[tok] = s;
    }
  }
  __syncthreads();
  float m = tid < n ? sm.sc[tid] : -INFINITY;
  m = block_max(m, sm.red);
  float sums[1] = {0.0f};
  if (tid < n) {
    const float p = exp2f(sm.sc[tid] - m);
    sm.sc[tid] = p;
    sums[0] = p;
  }
  block_sum<1>(sums, sm.red);
  M = m;
  L = sums[0];
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = (wv * 4 + j) * 4 + slot;
    if (tok < n) {
      const float p = sm.sc[tok];
      const half_t *hv = reinterpret_cast<const half_t *>(&vx[j]);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(p, (float)hv[i], acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; i += 4)
    *reinterpret_cast<float4 *>(&sm.u.accred[wv][slot][part * 8 + i]) =
        make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
  __syncthreads();
  if (tid < kD) {
    float s = 0.0f;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) s += sm.u.accred[x][y][tid];
    acc_out = s;
  }
}

template <int BITS, int G>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
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
  if (tid < kD / 2) {
    const uint32_t r = reinterpret_cast<const uint32_t *>(a.q + bh * kD)[tid];
    const half_t *hq = reinterpret_cast<const half_t *>(&r);
    sm.qs[2 * tid] = (float)hq[0] * a.qscale;
    sm.qs[2 * tid + 1] = (float)hq[1] * a.qscale;
  }
  __syncthreads();

  float M = -INFINITY, L = 0.0f, acc_out = 0.0f;
  if (split < a.sq) {
    quantized_split<BITS, G>(a, sm, bh, split, ql, M, L, acc_out);
  } else {
    const int rs = (split - a.sq) * a.win_chunk;
    const int n = min(a.win_chunk, rl - rs);
    if (n > 0) window_split<BITS, G>(a, sm, bh, rs, n, M, L, acc_out);
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
  da.kper = p.kper;
  da.sq = p.sq;
  da.nr = p.nr;
  da.win_chunk = p.win_chunk;
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
