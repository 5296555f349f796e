// C ABI of libmala: argument validation, workspace carving and launches.
// Every entry point either enqueues all of its work on the caller's stream
// and returns MALA_OK, or enqueues nothing and returns an error status.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "mala_internal.h"

namespace {

thread_local char g_err[512] = "";

mala_status fail(mala_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool debug_sync() {
  static const bool on = [] {
    const char* e = std::getenv("MALA_DEBUG_SYNC");
    return e != nullptr && e[0] == '1';
  }();
  return on;
}

mala_status finish(hipError_t e, hipStream_t st, const char* what) {
  if (e == hipSuccess && debug_sync()) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(MALA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  g_err[0] = '\0';
  return MALA_OK;
}

size_t elem_size(int32_t dtype) { return dtype == MALA_BF16 ? 2 : 4; }

constexpr size_t kWsAlign = 256;
size_t round_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Validates a prefill problem; fills `s`.
mala_status check_problem(const mala_problem* p, mala::Shape* s) {
  if (p == nullptr) return fail(MALA_ERR_INVALID_ARG, "problem is NULL");
  if (p->batch < 1 || p->n_q_heads < 1 || p->n_kv_heads < 1)
    return fail(MALA_ERR_INVALID_ARG, "batch, n_q_heads and n_kv_heads must be >= 1");
  if (p->n_q_heads % p->n_kv_heads != 0)
    return fail(MALA_ERR_INVALID_ARG, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)",
                p->n_q_heads, p->n_kv_heads);
  if (p->n_q < 0 || p->n_k < 0) return fail(MALA_ERR_INVALID_ARG, "n_q and n_k must be >= 0");
  if (p->n_q > 0 && p->n_k == 0)
    return fail(MALA_ERR_INVALID_ARG, "n_k must be >= 1 when n_q >= 1");
  if (p->causal && p->n_q > p->n_k)
    return fail(MALA_ERR_INVALID_ARG, "causal attention needs n_q (%d) <= n_k (%d)", p->n_q,
                p->n_k);
  if (p->dtype != MALA_F32 && p->dtype != MALA_BF16)
    return fail(MALA_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(MALA_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", p->head_dim);
  if (!std::isfinite(p->tau) || p->tau < 0.f)
    return fail(MALA_ERR_INVALID_ARG, "tau must be finite and >= 0");
  if (!std::isfinite(p->softmax_scale) || p->softmax_scale <= 0.f)
    return fail(MALA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (p->flags & ~(MALA_FLAG_FAST_GRAD | MALA_FLAG_GATE_PASS))
    return fail(MALA_ERR_INVALID_ARG, "unknown flags 0x%x", (unsigned)p->flags);
  const size_t es = elem_size(p->dtype);
  if ((size_t)p->n_q * p->head_dim * es >= (1ull << 31) ||
      (size_t)p->n_k * p->head_dim * es >= (1ull << 31))
    return fail(MALA_ERR_UNSUPPORTED, "a per-head slice exceeds 2 GiB");
  const double gridq = (double)((p->n_q + 255) / 256) * p->batch * p->n_q_heads;
  const double gridk = (double)((p->n_k + 63) / 64) * p->batch * p->n_kv_heads;
  if (gridq >= 2147483647.0 || gridk >= 2147483647.0)
    return fail(MALA_ERR_UNSUPPORTED, "problem too large for one launch");
  s->batch = p->batch;
  s->hq = p->n_q_heads;
  s->hkv = p->n_kv_heads;
  s->nq = p->n_q;
  s->nk = p->n_k;
  s->d = p->head_dim;
  s->group = p->n_q_heads / p->n_kv_heads;
  s->dtype = p->dtype;
  s->flags = p->flags;
  s->causal = p->causal ? 1 : 0;
  s->offset = p->n_k - p->n_q;
  s->scale_log2 = p->softmax_scale * 1.4426950408889634f;
  s->log2_tau = p->tau > 0.f ? std::log2(p->tau) : -INFINITY;
  s->scale = (double)p->softmax_scale;
  s->log_tau = p->tau > 0.f ? std::log((double)p->tau) : -INFINITY;
  return MALA_OK;
}

mala_status check_ptr(const void* ptr, const char* name, bool needed) {
  if (!needed) return MALA_OK;
  if (ptr == nullptr) return fail(MALA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(ptr, 16)) return fail(MALA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return MALA_OK;
}

#define MALA_TRY(x)                   \
  do {                                \
    const mala_status st_ = (x);      \
    if (st_ != MALA_OK) return st_;   \
  } while (0)

size_t bwd_ws_bytes(const mala::Shape& s) {
  return round_up(mala::bwd_ws_d_floats(s) * sizeof(float)) +
         round_up(mala::bwd_bits_words(s) * sizeof(uint32_t)) +
         round_up(mala::bwd_part_floats(s) * sizeof(float)) +
         round_up(mala::bwd_plan_ints(s) * sizeof(int32_t));
}

// Keys per split for a checked decode problem (the rule mala_decode_split_keys
// documents).
int split_keys(const mala_decode_problem* p) {
  int64_t split = mala::kDecChunk;
  if (p->split_keys > 0) {
    split = p->split_keys;
  } else if (p->split_keys == MALA_DECODE_SPLIT_AUTO) {
    const int64_t heads = (int64_t)p->batch * p->n_kv_heads;
    const int64_t target = heads >= 1024 ? 1 : 1024 / heads;   // splits per (sequence, KV head)
    const int64_t unit = (int64_t)mala::kDecChunk * target;
    split = (int64_t)mala::kDecChunk * ((p->max_n_k + unit - 1) / unit);
    if (split < mala::kDecChunk) split = mala::kDecChunk;
  }
  const int64_t whole = ((int64_t)p->max_n_k + mala::kDecBk - 1) / mala::kDecBk * mala::kDecBk;
  return (int)(split < whole ? split : whole);
}

mala_status check_decode(const mala_decode_problem* p, mala::DecodeShape* s) {
  if (p == nullptr) return fail(MALA_ERR_INVALID_ARG, "problem is NULL");
  if (p->batch < 1 || p->n_q_heads < 1 || p->n_kv_heads < 1)
    return fail(MALA_ERR_INVALID_ARG, "batch, n_q_heads and n_kv_heads must be >= 1");
  if (p->n_q_heads % p->n_kv_heads != 0)
    return fail(MALA_ERR_INVALID_ARG, "n_q_heads is not a multiple of n_kv_heads");
  if (p->n_q_heads / p->n_kv_heads > 16)
    return fail(MALA_ERR_UNSUPPORTED, "more than 16 query heads per KV head");
  if (p->dtype != MALA_F32 && p->dtype != MALA_BF16)
    return fail(MALA_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
  if (p->dtype == MALA_BF16 ? p->head_dim != 128 : (p->head_dim != 64 && p->head_dim != 128))
    return fail(MALA_ERR_UNSUPPORTED, "head_dim %d is not supported for this dtype", p->head_dim);
  if (p->cache_capacity < 1 || p->max_n_k < 1 || p->max_n_k > p->cache_capacity)
    return fail(MALA_ERR_INVALID_ARG, "need 1 <= max_n_k <= cache_capacity");
  if ((size_t)p->cache_capacity * p->head_dim * elem_size(p->dtype) >= (1ull << 31))
    return fail(MALA_ERR_UNSUPPORTED, "a per-head cache slice exceeds 2 GiB");
  if (!std::isfinite(p->tau) || p->tau < 0.f)
    return fail(MALA_ERR_INVALID_ARG, "tau must be finite and >= 0");
  if (!std::isfinite(p->softmax_scale) || p->softmax_scale <= 0.f)
    return fail(MALA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if ((int64_t)p->batch * p->n_kv_heads > 65535)
    return fail(MALA_ERR_UNSUPPORTED,
                "batch x n_kv_heads (%lld) exceeds 65535, the launch grid's second dimension",
                (long long)p->batch * p->n_kv_heads);
  if (p->split_keys < MALA_DECODE_SPLIT_AUTO || (p->split_keys > 0 && p->split_keys % mala::kDecBk))
    return fail(MALA_ERR_INVALID_ARG,
                "split_keys must be 0, MALA_DECODE_SPLIT_AUTO or a positive multiple of %d",
                mala::kDecBk);
  s->batch = p->batch;
  s->hq = p->n_q_heads;
  s->hkv = p->n_kv_heads;
  s->d = p->head_dim;
  s->group = p->n_q_heads / p->n_kv_heads;
  s->cap = p->cache_capacity;
  s->max_nk = p->max_n_k;
  s->chunk = split_keys(p);
  s->n_chunks = (p->max_n_k + s->chunk - 1) / s->chunk;
  s->wps = (s->chunk / mala::kDecBk + 31) / 32;
  // long splits (bf16) that would leave fewer split workgroups than the
  // chip's 256 compute units run as three parallel passes, when a group's
  // decision words fit the gate kernel's LDS (16 heads x 256 words)
  const int tpc = s->chunk / mala::kDecBk;
  s->staged = p->dtype == MALA_BF16 && s->chunk > 1024 &&
              (int64_t)s->n_chunks * p->batch * p->n_kv_heads < 256 && s->wps <= 256;
  s->tpart = tpc;
  s->ppc = 1;
  if (s->staged) {
    // parts of four tiles, one per wave of the P V workgroup: kept tiles
    // cluster (sinks, the recent band), and a part never walks more than
    // one of them per wave; empty parts exit at once and the merge skips them
    s->tpart = 4;
    s->ppc = (tpc + 3) / 4;
  }
  s->n_parts = s->n_chunks * s->ppc;
  s->scale_log2 = p->softmax_scale * 1.4426950408889634f;
  s->log2_tau = p->tau > 0.f ? std::log2(p->tau) : -INFINITY;
  s->scale = (double)p->softmax_scale;
  s->log_tau = p->tau > 0.f ? std::log((double)p->tau) : -INFINITY;
  return MALA_OK;
}

// nested: the backward on the forward's retained support (mala_bwd_nested);
// fwd_mask is the forward's tile mask, read by the bf16 gate pass only.
// fwd_kept (mala_bwd_auto): the forward's kept-tile counters, from which the
// bf16 backward chooses its walk on the device; the problem then takes the
// gate-pass workspace.
mala_status bwd_impl(int stages, const mala_problem* p, const void* q, const void* k,
                     const void* v, const void* o, const float* lse, const void* d_o, void* dq,
                     void* dk, void* dv, void* workspace, size_t ws_bytes, int8_t* tile_mask,
                     int32_t* kept_tiles, void* stream, bool nested = false,
                     const int8_t* fwd_mask = nullptr, const int32_t* fwd_kept = nullptr) {
  mala::Shape s;
  MALA_TRY(check_problem(p, &s));
  const bool rows = s.nq > 0;
  const bool autosel = fwd_kept != nullptr;
  if (autosel) {
    if (s.flags & MALA_FLAG_GATE_PASS)
      return fail(MALA_ERR_INVALID_ARG, "mala_bwd_auto chooses the walk: MALA_FLAG_GATE_PASS must not be set");
    if (s.dtype_is_bf16()) s.flags |= MALA_FLAG_GATE_PASS;
  }
  if (nested) {
    if (!(s.flags & MALA_FLAG_GATE_PASS))
      return fail(MALA_ERR_INVALID_ARG, "mala_bwd_nested needs MALA_FLAG_GATE_PASS in p->flags");
    if (rows && fwd_mask == nullptr) return fail(MALA_ERR_INVALID_ARG, "fwd_tile_mask is NULL");
  }
  MALA_TRY(check_ptr(q, "q", rows));
  MALA_TRY(check_ptr(k, "k", true));
  MALA_TRY(check_ptr(v, "v", true));
  MALA_TRY(check_ptr(o, "o", rows));
  MALA_TRY(check_ptr(lse, "lse", rows));
  MALA_TRY(check_ptr(d_o, "d_o", rows));
  MALA_TRY(check_ptr(dq, "dq", rows));
  MALA_TRY(check_ptr(dk, "dk", true));
  MALA_TRY(check_ptr(dv, "dv", true));
  const size_t need = bwd_ws_bytes(s);
  if (workspace == nullptr || ws_bytes < need)
    return fail(MALA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required",
                workspace ? ws_bytes : 0, need);
  if (!aligned(workspace, kWsAlign))
    return fail(MALA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  float* ws_d = (float*)workspace;
  uint32_t* ws_bits =
      (uint32_t*)((char*)workspace + round_up(mala::bwd_ws_d_floats(s) * sizeof(float)));
  float* ws_part = (float*)((char*)ws_bits + round_up(mala::bwd_bits_words(s) * sizeof(uint32_t)));
  int32_t* ws_plan = (int32_t*)((char*)ws_part + round_up(mala::bwd_part_floats(s) * sizeof(float)));
  hipError_t e;
  if (s.dtype_is_bf16())
    e = mala::launch_bwd_bf16(s, q, k, v, o, lse, d_o, dq, dk, dv, ws_d, ws_bits, ws_part, ws_plan,
                              nested ? fwd_mask : nullptr, tile_mask, kept_tiles, st, stages,
                              rows ? fwd_kept : nullptr);
  else
    e = mala::launch_bwd_f32(s, (const float*)q, (const float*)k, (const float*)v,
                             (const float*)o, lse, (const float*)d_o, (float*)dq, (float*)dk,
                             (float*)dv, ws_d, ws_bits, tile_mask, kept_tiles, st, stages);
  return finish(e, st, "mala_bwd launch");
}

mala_status decode_impl(int stages, const mala_decode_problem* p, const void* q,
                        const void* k_cache, const void* v_cache, const int32_t* seqlens_k,
                        void* o, float* lse, void* workspace, size_t ws_bytes, int8_t* tile_mask,
                        int32_t* kept_tiles, void* stream) {
  mala::DecodeShape s;
  MALA_TRY(check_decode(p, &s));
  MALA_TRY(check_ptr(q, "q", true));
  MALA_TRY(check_ptr(k_cache, "k_cache", true));
  MALA_TRY(check_ptr(v_cache, "v_cache", true));
  MALA_TRY(check_ptr(o, "o", true));
  MALA_TRY(check_ptr(lse, "lse", true));
  if (seqlens_k == nullptr) return fail(MALA_ERR_INVALID_ARG, "seqlens_k is NULL");
  const size_t need = round_up(mala::decode_ws_floats(s) * sizeof(float));
  if (workspace == nullptr || ws_bytes < need)
    return fail(MALA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required",
                workspace ? ws_bytes : 0, need);
  if (!aligned(workspace, kWsAlign))
    return fail(MALA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (p->dtype == MALA_BF16)
    e = mala::launch_decode_bf16(s, q, k_cache, v_cache, seqlens_k, o, lse, (float*)workspace,
                                 tile_mask, kept_tiles, st, stages);
  else
    e = mala::launch_decode_f32(s, (const float*)q, (const float*)k_cache,
                                (const float*)v_cache, seqlens_k, (float*)o, lse,
                                (float*)workspace, tile_mask, kept_tiles, st, stages);
  return finish(e, st, "mala_decode launch");
}

// Device scratch of mala_decode_noalloc: one copy in each GPU the library
// runs on, held until the process ends. In host code `scratch` names a
// host-side stand-in, not the device array: host code uses only the device
// address looked up below.
static __device__ __align__(256) unsigned char scratch[MALA_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`, looked up on the first call on
// that device (every lookup yields the same address, so racing first calls
// are harmless).
mala_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MALA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MALA_ERR_UNSUPPORTED, "device %d is past the %d devices the scratch covers", dev,
                kMaxDevices);
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(MALA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return MALA_OK;
}

}  // namespace

extern "C" {

mala_status mala_get_tiling(int32_t op, int32_t dtype, int32_t head_dim, int32_t* bq,
                            int32_t* bk, int32_t* chunk) {
  (void)dtype;
  (void)head_dim;
  if (bq == nullptr || bk == nullptr || chunk == nullptr)
    return fail(MALA_ERR_INVALID_ARG, "output pointer is NULL");
  switch (op) {
    case MALA_OP_FWD: *bq = mala::kFwdBq; *bk = mala::kFwdBk; *chunk = 0; break;
    case MALA_OP_BWD: *bq = mala::kBwdBq; *bk = mala::kBwdBk; *chunk = 0; break;
    case MALA_OP_DECODE: *bq = 1; *bk = mala::kDecBk; *chunk = mala::kDecChunk; break;
    default: return fail(MALA_ERR_INVALID_ARG, "unknown op %d", op);
  }
  return MALA_OK;
}

mala_status mala_fwd(const mala_problem* p, const void* q, const void* k, const void* v, void* o,
                     float* lse, int8_t* tile_mask, int32_t* kept_tiles, void* stream) {
  mala::Shape s;
  MALA_TRY(check_problem(p, &s));
  const bool rows = s.nq > 0;
  MALA_TRY(check_ptr(q, "q", rows));
  MALA_TRY(check_ptr(k, "k", rows));
  MALA_TRY(check_ptr(v, "v", rows));
  MALA_TRY(check_ptr(o, "o", rows));
  MALA_TRY(check_ptr(lse, "lse", rows));
  if (!rows) return finish(hipSuccess, (hipStream_t)stream, "mala_fwd");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (s.dtype_is_bf16())
    e = mala::launch_fwd_bf16(s, q, k, v, o, lse, tile_mask, kept_tiles, st);
  else
    e = mala::launch_fwd_f32(s, (const float*)q, (const float*)k, (const float*)v, (float*)o, lse,
                             tile_mask, kept_tiles, st);
  return finish(e, st, "mala_fwd launch");
}

size_t mala_bwd_workspace_size(const mala_problem* p) {
  mala::Shape s;
  if (check_problem(p, &s) != MALA_OK) return 0;
  return bwd_ws_bytes(s);
}

mala_status mala_bwd(const mala_problem* p, const void* q, const void* k, const void* v,
                     const void* o, const float* lse, const void* d_o, void* dq, void* dk,
                     void* dv, void* workspace, size_t ws_bytes, int8_t* tile_mask,
                     int32_t* kept_tiles, void* stream) {
  return bwd_impl(mala::kStagesAll, p, q, k, v, o, lse, d_o, dq, dk, dv, workspace, ws_bytes,
                  tile_mask, kept_tiles, stream);
}

mala_status mala_bwd_nested(const mala_problem* p, const void* q, const void* k, const void* v,
                            const void* o, const float* lse, const void* d_o,
                            const int8_t* fwd_tile_mask, void* dq, void* dk, void* dv,
                            void* workspace, size_t ws_bytes, int8_t* tile_mask,
                            int32_t* kept_tiles, void* stream) {
  return bwd_impl(mala::kStagesAll, p, q, k, v, o, lse, d_o, dq, dk, dv, workspace, ws_bytes,
                  tile_mask, kept_tiles, stream, true, fwd_tile_mask);
}

mala_status mala_bwd_auto(const mala_problem* p, const void* q, const void* k, const void* v,
                          const void* o, const float* lse, const void* d_o,
                          const int32_t* fwd_kept_tiles, void* dq, void* dk, void* dv,
                          void* workspace, size_t ws_bytes, int8_t* tile_mask, int32_t* kept_tiles,
                          void* stream) {
  if (p != nullptr && p->n_q > 0 && fwd_kept_tiles == nullptr)
    return fail(MALA_ERR_INVALID_ARG, "fwd_kept_tiles is NULL");
  // the pointer marks the mode even when there are no query rows
  static const int32_t kNoRows = 0;
  return bwd_impl(mala::kStagesAll, p, q, k, v, o, lse, d_o, dq, dk, dv, workspace, ws_bytes,
                  tile_mask, kept_tiles, stream, false, nullptr,
                  fwd_kept_tiles != nullptr ? fwd_kept_tiles : &kNoRows);
}

mala_status mala_bwd_stage(int32_t stage, const mala_problem* p, const void* q, const void* k,
                           const void* v, const void* o, const float* lse, const void* d_o,
                           void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                           int8_t* tile_mask, int32_t* kept_tiles, void* stream) {
  if (stage < MALA_BWD_PREP || stage > MALA_BWD_DQ)
    return fail(MALA_ERR_INVALID_ARG, "unknown backward stage %d", stage);
  return bwd_impl(1 << stage, p, q, k, v, o, lse, d_o, dq, dk, dv, workspace, ws_bytes,
                  tile_mask, kept_tiles, stream);
}

int32_t mala_decode_split_keys(const mala_decode_problem* p) {
  mala::DecodeShape s;
  if (check_decode(p, &s) != MALA_OK) return 0;
  return s.chunk;
}

size_t mala_decode_workspace_size(const mala_decode_problem* p) {
  mala::DecodeShape s;
  if (check_decode(p, &s) != MALA_OK) return 0;
  return round_up(mala::decode_ws_floats(s) * sizeof(float));
}

mala_status mala_decode(const mala_decode_problem* p, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* seqlens_k, void* o, float* lse,
                        void* workspace, size_t ws_bytes, int8_t* tile_mask, int32_t* kept_tiles,
                        void* stream) {
  return decode_impl(mala::kStageMain | mala::kStageCombine, p, q, k_cache, v_cache, seqlens_k, o,
                     lse, workspace, ws_bytes, tile_mask, kept_tiles, stream);
}

mala_status mala_decode_stage(int32_t stage, const mala_decode_problem* p, const void* q,
                              const void* k_cache, const void* v_cache, const int32_t* seqlens_k,
                              void* o, float* lse, void* workspace, size_t ws_bytes,
                              int8_t* tile_mask, int32_t* kept_tiles, void* stream) {
  if (stage != MALA_DECODE_SPLIT && stage != MALA_DECODE_COMBINE)
    return fail(MALA_ERR_INVALID_ARG, "unknown decode stage %d", stage);
  return decode_impl(stage == MALA_DECODE_SPLIT ? mala::kStageMain : mala::kStageCombine, p, q,
                     k_cache, v_cache, seqlens_k, o, lse, workspace, ws_bytes, tile_mask,
                     kept_tiles, stream);
}

mala_status mala_decode_noalloc(const mala_decode_problem* p, const void* q,
                                const void* k_cache, const void* v_cache,
                                const int32_t* seqlens_k, void* o, float* lse,
                                int8_t* tile_mask, int32_t* kept_tiles, void* stream) {
  mala::DecodeShape s;
  MALA_TRY(check_decode(p, &s));
  const size_t need = round_up(mala::decode_ws_floats(s) * sizeof(float));
  if (need > MALA_DECODE_NOALLOC_SCRATCH_BYTES)
    return fail(MALA_ERR_UNSUPPORTED,
                "this decode problem needs %zu bytes of scratch; mala_decode_noalloc holds %zu "
                "(use mala_decode with a workspace)",
                need, (size_t)MALA_DECODE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  MALA_TRY(scratch_of_current_device(&ws));
  return decode_impl(mala::kStageMain | mala::kStageCombine, p, q, k_cache, v_cache, seqlens_k, o,
                     lse, ws, MALA_DECODE_NOALLOC_SCRATCH_BYTES, tile_mask, kept_tiles, stream);
}

const char* mala_last_error(void) { return g_err; }

const char* mala_version(void) { return "libmala 0.1.0 (gfx950)"; }

}  // extern "C"
