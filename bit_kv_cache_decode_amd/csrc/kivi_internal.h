// Internal interface between the C ABI layer (kivi_api.cpp) and the HIP
// kernels (kivi_kernels.hip).  Not installed; not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/kivi.h"

namespace kivi {

// Decode workgroup shape: waves per workgroup (a multiple of 4, spread
// evenly over the 4 SIMDs of a compute unit) and resident workgroups per
// compute unit; the kernel is compiled for the resulting waves per SIMD.
#ifndef KIVI_DECODE_WAVES
#define KIVI_DECODE_WAVES 8
#endif
#ifndef KIVI_DECODE_WG_PER_CU
#define KIVI_DECODE_WG_PER_CU 1
#endif
constexpr int kDecodeWavesPerWorkgroup = KIVI_DECODE_WAVES;
// Ticket counters (workspace and cache) sit 256 bytes apart: device-scope
// atomics on one cache line are serialized, so counters that many
// workgroups hit at once must not share a line.
constexpr int kTicketStride = 64;
constexpr int kDecodeWorkgroupsPerCU = KIVI_DECODE_WG_PER_CU;

// Decode work split.  Each (sequence, head) gets `splits` workgroups of
// kDecodeWavesPerWorkgroup waves.  Its quantized tokens are walked in sub-chunks of `sub` tokens
// (512 / words-per-token: two 16-byte loads per lane per operand), dealt
// round-robin to the waves; each wave also takes `win_per_wave`
// consecutive fp16 window tokens (a multiple of 8).  The workgroups' partial softmax states are
// merged by the last workgroup of that (sequence, head) to finish.
struct DecodePlan {
  int sub;           // quantized tokens per sub-chunk
  int splits;        // workgroups per (sequence, head)
  int win_per_wave;  // window tokens per wave (multiple of 8)
  int depth;         // sub-chunks in flight per wave: 2 when the grid is at most one workgroup
                     // per compute unit, else 1 (several workgroups then share a compute unit)
  size_t part_floats;     // floats of partial state per split (4 + D)
  size_t counters_off;    // byte offset of the per-(sequence, head) tickets
  size_t bytes;           // total workspace bytes
};

DecodePlan decode_plan(const kivi_dims &d);

// Whether kivi_decode_step runs as the single whole-step kernel: it needs one
// workgroup per (sequence, head), and holds many more registers than the
// decode alone, so it only pays while the grid is one workgroup per compute
// unit (depth 2), and is not compiled for B = 8 (four channels per lane).
// Otherwise the step is the three kernels.
inline bool step_in_one_kernel(const kivi_dims &d, const DecodePlan &p) {
  return p.splits == 1 && p.depth == 2 && d.bits != 8;
}

// Kernel launchers (return a hipError_t value as int, 0 on success).
int launch_append(const kivi_dims &d, const kivi_cache &c, const void *k_new,
                  const void *v_new, void *stream);
int launch_flush(const kivi_dims &d, const kivi_cache &c, void *stream);
int launch_prefill(const kivi_dims &d, const kivi_cache &c, const void *k,
                   const void *v, int32_t src_len, const int32_t *len,
                   const int32_t *res, void *stream, bool value_queue);
// Value queue: key flush only, and the append that moves the oldest value
// out of the queue.
int launch_flush_keys(const kivi_dims &d, const kivi_cache &c, void *stream);
int launch_append_vq(const kivi_dims &d, const kivi_cache &c, const void *k_new,
                     const void *v_new, void *stream);
int launch_decode_vq(const kivi_dims &d, const kivi_cache &c, const DecodePlan &p, const void *q,
                     float *out, float sm_scale, void *workspace, void *stream);
int launch_decode(const kivi_dims &d, const kivi_cache &c, const DecodePlan &p,
                  const void *q, float *out, float sm_scale, void *workspace,
                  void *stream);
// Allocation-free decode (kivi_decode_attn_noalloc): its split partials and
// counters live in one file-scope device array of kNoAllocScratchBytes per
// GPU.  The counters take the first kNoAllocTicketBytes at a fixed place (one
// 256-byte line per (sequence, head), at most kNoAllocPairs pairs), so no
// call's partials ever land where a later call expects zeroed counters; the
// partials follow.
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
constexpr size_t kNoAllocTicketBytes = (size_t)1 << 20;
constexpr long kNoAllocPairs = (long)(kNoAllocTicketBytes / (kTicketStride * 4));

// 0, a hipError_t value, or -1 when the device array's address could not be
// obtained.
int launch_decode_noalloc(const kivi_dims &d, const kivi_cache &c, const DecodePlan &p,
                          const void *q, float *out, float sm_scale, void *stream);

int launch_cache_init(const kivi_dims &d, const kivi_cache &c, void *stream);
int launch_fill_zero(void *p, size_t bytes, void *stream);
int launch_stream_read(const void *src, size_t bytes, int workgroups, uint32_t *sink,
                       void *stream);
int launch_decode_sink(const kivi_dims &d, const kivi_cache &c, const DecodePlan &p,
                       const void *k_sink, const void *v_sink, int n_sink, const void *q,
                       float *out, float sm_scale, double rope_base, void *workspace,
                       void *stream);
int launch_decode_rope(const kivi_dims &d, const kivi_cache &c, const DecodePlan &p,
                       const void *q, float *out, float sm_scale, double rope_base,
                       void *workspace, void *stream);
int launch_decode_step(const kivi_dims &d, const kivi_cache &c, const DecodePlan &p,
                       const void *k_new, const void *v_new, const void *k_sink,
                       const void *v_sink, int n_sink, const void *q, float *out,
                       float sm_scale, void *workspace, void *stream);

}  // namespace kivi
