// C ABI of libkivi: argument validation, the decode work split, and calls
// into the kernel launchers.  Host-only C++ (no HIP headers): everything that
// touches the device is in kivi_kernels.hip.
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "kivi_internal.h"

namespace kivi {
namespace {

// Resident decode workgroups on the device: 256 compute units (MI355X) x
// the decode kernel's workgroups per compute unit.
constexpr long kWorkgroupSlots = 256L * kDecodeWorkgroupsPerCU;
// Fixed cost of one decode workgroup (prologue, combine, publish, merge) in
// units of one sub-chunk per wave, for choosing the split count.
constexpr double kWorkgroupOverhead = 2.0;
constexpr int kMaxSplits = 64;
constexpr int kMaxResidual = 4096;
constexpr int32_t kMaxStreamWorkgroups = 1 << 20;
constexpr int32_t kMaxSink = 4096;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool supported(const kivi_dims &d) {
  // one (sequence, head) region of any cache array must stay below 2 GiB
  // (32-bit buffer offsets in the decode kernel)
  const long code_bytes = (long)d.capacity * (d.head_dim * d.bits / 32) * 4;
  return d.head_dim == 128 && (d.group == 32 || d.group == 64 || d.group == 128) &&
         d.residual <= kMaxResidual && code_bytes < (1L << 31);
}

int check_dims(const kivi_dims *d) {
  if (!d) return KIVI_EINVAL;
  const int rc = kivi_validate_dims(d);
  if (rc != KIVI_OK) return rc;
  return supported(*d) ? KIVI_OK : KIVI_EUNSUPPORTED;
}

// Non-null and aligned: the kernels move fp16 rows, codes and scales in
// 16-byte vectors, and 32-bit lengths, counters and outputs one by one.
bool a16(const void *p) { return p && ((uintptr_t)p & 15) == 0; }
bool a4(const void *p) { return p && ((uintptr_t)p & 3) == 0; }

bool cache_ok(const kivi_cache *c) {
  return c && a16(c->k_codes) && a16(c->k_scale) && a16(c->k_zero) && a16(c->v_codes) &&
         a16(c->v_scale) && a16(c->v_zero) && a16(c->k_res) && a16(c->v_res) && a4(c->q_len) &&
         a4(c->r_len) && a4(c->status) && a4(c->tickets);
}

int hip_rc(int rc) { return rc == 0 ? KIVI_OK : KIVI_EHIP; }

}  // namespace

DecodePlan decode_plan(const kivi_dims &d) {
  DecodePlan p{};
  const int words = d.head_dim * d.bits / 32;
  p.sub = 512 / words;
  const long bh = (long)d.batch * d.heads;
  const long nsub = (d.capacity + p.sub - 1) / p.sub;
  // Split count: minimise (rounds of resident workgroups) x (per-workgroup
  // time), per-workgroup time = its share of sub-chunks per wave plus a
  // fixed overhead; the first (smallest) split count wins ties.
  int best = 1;
  double best_cost = 0.0;
  for (int s = 1; s <= kMaxSplits; ++s) {
    const long waves = (long)kDecodeWavesPerWorkgroup * s;
    if (s > 1 && nsub < waves) break;  // at least one sub-chunk per wave
    const long rounds = (bh * s + kWorkgroupSlots - 1) / kWorkgroupSlots;
    const double cost = (double)rounds * ((double)nsub / (double)waves + kWorkgroupOverhead);
    if (s == 1 || cost < best_cost - 1e-9) {
      best = s;
      best_cost = cost;
    }
  }
  p.splits = best;
  p.depth = bh * p.splits > kWorkgroupSlots ? 1 : 2;
  const long waves = (long)kDecodeWavesPerWorkgroup * p.splits;
  p.win_per_wave = (int)(((d.residual + waves - 1) / waves + 7) / 8 * 8);
  p.part_floats = 4 + (size_t)d.head_dim;
  const size_t parts = (size_t)bh * p.splits * p.part_floats * sizeof(float);
  p.counters_off = round_up(parts, 256);
  p.bytes = p.counters_off + (size_t)bh * kTicketStride * sizeof(uint32_t);
  return p;
}

}  // namespace kivi

extern "C" {

int kivi_validate_dims(const kivi_dims *d) {
  if (!d) return KIVI_EINVAL;
  if (d->batch <= 0 || d->heads <= 0 || d->head_dim <= 0 || d->group <= 0 || d->residual <= 0 ||
      d->capacity < 0)
    return KIVI_EINVAL;
  if (d->bits != 2 && d->bits != 4 && d->bits != 8) return KIVI_EINVAL;
  if (d->head_dim % d->group || d->residual % d->group || d->capacity % d->group)
    return KIVI_EINVAL;
  if ((d->head_dim * d->bits) % 32) return KIVI_EINVAL;
  return KIVI_OK;
}

int kivi_cache_init(const kivi_dims *dims, const kivi_cache *cache, void *stream) {
  const int rc = kivi::check_dims(dims);
  if (rc != KIVI_OK) return rc;
  if (!kivi::cache_ok(cache)) return KIVI_EINVAL;
  return kivi::hip_rc(kivi::launch_cache_init(*dims, *cache, stream));
}

int kivi_workspace_init(const kivi_dims *dims, void *workspace, size_t workspace_bytes,
                        void *stream) {
  const int rc = kivi::check_dims(dims);
  if (rc != KIVI_OK) return rc;
  if (!kivi::a16(workspace)) return KIVI_EINVAL;
  const kivi::DecodePlan p = kivi::decode_plan(*dims);
  if (workspace_bytes < p.bytes) return KIVI_ENOSPC;
  return kivi::hip_rc(kivi::launch_fill_zero(static_cast<char *>(workspace) + p.counters_off,
                                             p.bytes - p.counters_off, stream));
}

int kivi_append_kv(const kivi_dims *dims, const kivi_cache *cache, const void *k_new,
                   const void *v_new, void *stream) {
  const int rc = kivi::check_dims(dims);
  if (rc != KIVI_OK) return rc;
  if (!kivi::cache_ok(cache) || !kivi::a16(k_new) || !kivi::a16(v_new)) return KIVI_EINVAL;
  return kivi::hip_rc(kivi::launch_append(*dims, *cache, k_new, v_new, stream));
}

int kivi_flush_residual(const kivi_dims *dims, const kivi_cache *cache, void *stream) {
  const int rc = kivi::check_dims(dims);
  if (rc != KIVI_OK) return rc;
  if (!kivi::cache_ok(cache)) return KIVI_EINVAL;
  return kivi::hip_rc(kivi::launch_flush(*dims, *cache, stream));
}

int kivi_prefill(const kivi_dims *dims, const kivi_cache *cache, const void *k, const void *v,
                 int32_t src_len, const int32_t *len, const int32_t *res, void *stream) {
  const int rc = kivi::check_dims(dims);
  if (rc != KIVI_OK) return rc;
  if (!kivi::cache_ok(cache) || !kivi::a4(len) || src_len < 0) return KIVI_EINVAL;
  if (res && !kivi::a4(res)) return KIVI_EINVAL;
  if (src_len > 0 && (!kivi::a16(k) || !kivi::a16(v))) return KIVI_EINVAL;
  return kivi::hip_rc(kivi::launch_prefill(*dims, *cache, k, v, src_len, len, res, stream, false));
}

int kivi_prefill_vq(const kivi_dims *dims, const kivi_cache *cache, const void *k, const void *v,
                    int32_t src_len, const int32_t *len, const int32_t *res, void *stream) {
  const int rc = kivi::check_dims(dims);
  if (rc != KIVI_OK) return rc;
  if (!kivi::cache_ok(cache) || !kivi::a4(len) || src_len < 0) return KIVI_EINVAL;
  if (res && !kivi::a4(res)) return KIVI_EINVAL;
  if (src_len > 0 && (!kivi::a16(k) || !kivi::a16(v))) return KIVI_EINVAL;
  return kivi::hip_rc(kivi::launch_prefill(*dims, *cache, k, v, src_len, len, res, stream, true));
}

int kivi_append_kv_vq(const kivi_dims *dims, const kivi_cache *cache, const void *k_new,
                      const void *v_new, void *stream) {
  const int rc = kivi::check_dims(dims);
  if (rc != KIVI_OK) return rc;
  if (!kivi::cache_ok(cache) || !kivi::a16(k_new) || !kivi::a16(v_new)) return KIVI_EINVAL;
  return kivi::hip_rc(kivi::launch_append_vq(*dims, *cache, k_new, v_new, stream));
}

int kivi_flush_residual_vq(const kivi_dims *dims, const kivi_cache *cache, void *stream) {
  const int rc = kivi::check_dims(dims);
  if (rc != KIVI_OK) return rc;
  if (!kivi::cache_ok(cache)) return KIVI_EINVAL;
  return kivi::hip_rc(kivi::launch_flush_keys(*dims, *cache, stream));
}

int kivi_decode_attn_vq(const kivi_dims *dims, const kivi_cache *cache, const void *q, float *out,
                        float sm_scale, void *workspace, size_t workspace_bytes, void *stream) {
  const int rc = kivi::check_dims(dims);
  if (rc != KIVI_OK) return rc;
  if (!kivi::cache_ok(cache) || !kivi::a16(q) || !kivi::a4(out) || !kivi::a16(workspace))
    return KIVI_EINVAL;
  if (!(sm_scale == sm_scale) || sm_scale == 1.0f / 0.0f || sm_scale == -1.0f / 0.0f)
    return KIVI_EINVAL;
  const kivi::DecodePlan p = kivi::decode_plan(*dims);
  if (workspace_bytes < p.bytes) return KIVI_ENOSPC;
  return kivi::hip_rc(kivi::launch_decode_vq(*dims, *cache, p, q, out, sm_scale, workspace, stream));
}

size_t kivi_decode_workspace_bytes(const kivi_dims *dims) {
  if (kivi::check_dims(dims) != KIVI_OK) return 0;
  return kivi::decode_plan(*dims).bytes;
}

int kivi_decode_splits(const kivi_dims *dims) {
  const int rc = kivi::check_dims(dims);
  if (rc != KIVI_OK) return rc;
  return kivi::decode_plan(*dims).splits;
}

int kivi_decode_step_kernels(const kivi_dims *dims) {
  const int rc = kivi::check_dims(dims);
  if (rc != KIVI_OK) return rc;
  return kivi::step_in_one_kernel(*dims, kivi::decode_plan(*dims)) ? 1 : 3;
}

int kivi_decode_attn(const kivi_dims *dims, const kivi_cache *cache, const void *q, float *out,
                     float sm_scale, void *workspace, size_t workspace_bytes, void *stream) {
  const int rc = kivi::check_dims(dims);
  if (rc != KIVI_OK) return rc;
  if (!kivi::cache_ok(cache) || !kivi::a16(q) || !kivi::a4(out) || !kivi::a16(workspace))
    return KIVI_EINVAL;
  if (!(sm_scale == sm_scale) || sm_scale == 1.0f / 0.0f || sm_scale == -1.0f / 0.0f)
    return KIVI_EINVAL;
  const kivi::DecodePlan p = kivi::decode_plan(*dims);
  if (workspace_bytes < p.bytes) return KIVI_ENOSPC;
  return kivi::hip_rc(kivi::launch_decode(*dims, *cache, p, q, out, sm_scale, workspace, stream));
}

int kivi_decode_attn_noalloc(const kivi_dims *dims, const kivi_cache *cache, const void *q,
                             float *out, float sm_scale, void *stream) {
  const int rc = kivi::check_dims(dims);
  if (rc != KIVI_OK) return rc;
  if (!kivi::cache_ok(cache) || !kivi::a16(q) || !kivi::a4(out)) return KIVI_EINVAL;
  if (!(sm_scale == sm_scale) || sm_scale == 1.0f / 0.0f || sm_scale == -1.0f / 0.0f)
    return KIVI_EINVAL;
  const kivi::DecodePlan p = kivi::decode_plan(*dims);
  const long pairs = (long)dims->batch * dims->heads;
  const size_t parts = (size_t)pairs * p.splits * p.part_floats * sizeof(float);
  if (pairs > kivi::kNoAllocPairs ||
      parts > kivi::kNoAllocScratchBytes - kivi::kNoAllocTicketBytes)
    return KIVI_ENOSPC;
  return kivi::hip_rc(kivi::launch_decode_noalloc(*dims, *cache, p, q, out, sm_scale, stream));
}

int kivi_decode_attn_sink(const kivi_dims *dims, const kivi_cache *cache, const void *k_sink,
                          const void *v_sink, int32_t n_sink, const void *q, float *out,
                          float sm_scale, double rope_base, void *workspace,
                          size_t workspace_bytes, void *stream) {
  const int rc = kivi::check_dims(dims);
  if (rc != KIVI_OK) return rc;
  if (!kivi::cache_ok(cache) || !kivi::a16(q) || !kivi::a4(out) || !kivi::a16(workspace))
    return KIVI_EINVAL;
  if (!(sm_scale == sm_scale) || sm_scale == 1.0f / 0.0f || sm_scale == -1.0f / 0.0f)
    return KIVI_EINVAL;
  if (n_sink < 0 || n_sink > kivi::kMaxSink ||
      (n_sink > 0 && (!kivi::a16(k_sink) || !kivi::a16(v_sink))))
    return KIVI_EINVAL;
  if (rope_base != 0.0 && (!(rope_base > 1.0) || rope_base == 1.0 / 0.0)) return KIVI_EINVAL;
  const kivi::DecodePlan p = kivi::decode_plan(*dims);
  if (workspace_bytes < p.bytes) return KIVI_ENOSPC;
  return kivi::hip_rc(kivi::launch_decode_sink(*dims, *cache, p, k_sink, v_sink, n_sink, q, out,
                                               sm_scale, rope_base, workspace, stream));
}

int kivi_decode_attn_rope(const kivi_dims *dims, const kivi_cache *cache, const void *q,
                          float *out, float sm_scale, double rope_base, void *workspace,
                          size_t workspace_bytes, void *stream) {
  const int rc = kivi::check_dims(dims);
  if (rc != KIVI_OK) return rc;
  if (!kivi::cache_ok(cache) || !kivi::a16(q) || !kivi::a4(out) || !kivi::a16(workspace))
    return KIVI_EINVAL;
  if (!(sm_scale == sm_scale) || sm_scale == 1.0f / 0.0f || sm_scale == -1.0f / 0.0f)
    return KIVI_EINVAL;
  if (!(rope_base > 1.0) || rope_base == 1.0 / 0.0) return KIVI_EINVAL;
  const kivi::DecodePlan p = kivi::decode_plan(*dims);
  if (workspace_bytes < p.bytes) return KIVI_ENOSPC;
  return kivi::hip_rc(kivi::launch_decode_rope(*dims, *cache, p, q, out, sm_scale, rope_base,
                                               workspace, stream));
}

}  // extern "C"

namespace kivi {
namespace {

int decode_step(const kivi_dims *dims, const kivi_cache *cache, const void *k_new,
                const void *v_new, const void *k_sink, const void *v_sink, int32_t n_sink,
                const void *q, float *out, float sm_scale, void *workspace,
                size_t workspace_bytes, void *stream) {
  const int rc = check_dims(dims);
  if (rc != KIVI_OK) return rc;
  if (!cache_ok(cache) || !a16(k_new) || !a16(v_new) || !a16(q) || !a4(out) || !a16(workspace))
    return KIVI_EINVAL;
  if (!(sm_scale == sm_scale) || sm_scale == 1.0f / 0.0f || sm_scale == -1.0f / 0.0f)
    return KIVI_EINVAL;
  if (n_sink < 0 || n_sink > kMaxSink || (n_sink > 0 && (!a16(k_sink) || !a16(v_sink))))
    return KIVI_EINVAL;
  const DecodePlan p = decode_plan(*dims);
  if (workspace_bytes < p.bytes) return KIVI_ENOSPC;
  return hip_rc(launch_decode_step(*dims, *cache, p, k_new, v_new, k_sink, v_sink, n_sink, q,
                                   out, sm_scale, workspace, stream));
}

}  // namespace
}  // namespace kivi

extern "C" {

int kivi_decode_step(const kivi_dims *dims, const kivi_cache *cache, const void *k_new,
                     const void *v_new, const void *q, float *out, float sm_scale,
                     void *workspace, size_t workspace_bytes, void *stream) {
  return kivi::decode_step(dims, cache, k_new, v_new, nullptr, nullptr, 0, q, out, sm_scale,
                           workspace, workspace_bytes, stream);
}

int kivi_decode_step_sink(const kivi_dims *dims, const kivi_cache *cache, const void *k_new,
                          const void *v_new, const void *k_sink, const void *v_sink,
                          int32_t n_sink, const void *q, float *out, float sm_scale,
                          void *workspace, size_t workspace_bytes, void *stream) {
  return kivi::decode_step(dims, cache, k_new, v_new, k_sink, v_sink, n_sink, q, out, sm_scale,
                           workspace, workspace_bytes, stream);
}

int kivi_stream_read(const void *src, size_t bytes, int32_t workgroups, uint32_t *sink,
                     void *stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 || ((uintptr_t)src) % 16) return KIVI_EINVAL;
  if (workgroups < 1 || workgroups > kivi::kMaxStreamWorkgroups) return KIVI_EINVAL;
  return kivi::hip_rc(kivi::launch_stream_read(src, bytes, workgroups, sink, stream));
}

const char *kivi_strerror(int code) {
  switch (code) {
    case KIVI_OK: return "success";
    case KIVI_EINVAL: return "invalid argument";
    case KIVI_ENOSPC: return "workspace too small";
    case KIVI_EHIP: return "HIP kernel launch failed";
    case KIVI_EUNSUPPORTED: return "dimensions not covered by the compiled kernels";
    default: return "unknown error";
  }
}

}  // extern "C"
