// Internal declarations shared by the host layer and the kernel sources of libmala.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mala.h"

namespace mala {

// Decision partition (exposed through mala_get_tiling).
constexpr int kFwdBq = 32;      // query rows per forward decision block (one wave)
constexpr int kFwdBk = 64;      // keys per forward tile
constexpr int kBwdBq = 32;      // query rows per backward tile
constexpr int kBwdBk = 16;      // keys per backward tile (refines the forward tile)
constexpr int kDecBk = 64;      // keys per decode tile
constexpr int kDecChunk = 256;  // default keys per decode split

// Everything a kernel needs about one prefill/training problem.
struct Shape {
  int batch, hq, hkv, nq, nk, d, group;
  int dtype;         // mala_dtype
  int flags;         // MALA_FLAG_*
  int causal;
  int offset;        // n_k - n_q (bottom-right causal alignment)
  float scale_log2;  // softmax_scale * log2(e): scores in base 2
  float log2_tau;    // log2(tau), -inf when tau == 0
  double scale;      // softmax scale (fp64 copies for the fp32-input kernels)
  double log_tau;    // ln(tau), -inf when tau == 0
  bool dtype_is_bf16() const { return dtype == MALA_BF16; }
};

struct DecodeShape {
  int batch, hq, hkv, d, group, cap, max_nk;
  int chunk;         // keys per split, a multiple of kDecBk
  int n_chunks;      // ceil(max_nk / chunk)
  int wps;           // decision-bit words per split: ceil(chunk / kDecBk / 32)
  // Long splits (bf16) run as three parallel passes instead of one workgroup
  // walking the whole split: tile statistics, the gate replay per head, and
  // P V over the kept tiles in parts of tpart tiles (ppc parts per split).
  // The merge then sees n_parts = n_chunks * ppc partial states per head
  // (n_parts = n_chunks for the one-kernel path).
  int staged;        // nonzero: the three-pass path
  int tpart, ppc, n_parts;
  float scale_log2;
  float log2_tau;
  double scale;
  double log_tau;
};

// Split-KV decode workspace, in 4-byte words: the partial states (base 2,
// scale folded in) as the (m, S) pairs of every (sequence * query head,
// split), then the unnormalized outputs O of every (sequence * query head,
// split); then the split's decisions, wps words each (bit t of word i: tile
// 32 i + t of the split): per (sequence * query head, split) the kept-tile
// bits of the head, per (sequence * KV head, split) the bits of the tiles
// whose V was read. The merge kernel turns the bits into the kept-tile
// counters, so the split kernel needs no atomics.
// The (m, S) region is padded to 256 bytes so that the partial outputs are
// 16-byte aligned.
// Partial states are indexed by part (split c, part p: c * ppc + p); the
// decision bits by split.
__host__ __device__ inline size_t dec_ms_words(const DecodeShape& s) {
  return ((size_t)s.batch * s.hq * s.n_parts * 2 + 63) / 64 * 64;
}
__host__ __device__ inline size_t dec_ms_at(const DecodeShape& s, size_t bh, int part) {
  return (bh * (size_t)s.n_parts + part) * 2;
}
__host__ __device__ inline size_t dec_o_at(const DecodeShape& s, size_t bh, int part) {
  return dec_ms_words(s) + (bh * (size_t)s.n_parts + part) * s.d;
}
__host__ __device__ inline size_t dec_kbits_at(const DecodeShape& s, size_t bh, int c) {
  return dec_ms_words(s) + (size_t)s.batch * s.hq * s.n_parts * s.d +
         (bh * (size_t)s.n_chunks + c) * s.wps;
}
__host__ __device__ inline size_t dec_vbits_at(const DecodeShape& s, size_t bkv, int c) {
  return dec_ms_words(s) + (size_t)s.batch * s.hq * s.n_parts * s.d +
         (size_t)s.batch * s.hq * s.n_chunks * s.wps + (bkv * (size_t)s.n_chunks + c) * s.wps;
}
// three-pass path only: (tile max, tile sum) per (sequence * query head,
// split, tile), base 2, as float2 (the offset is even)
__host__ __device__ inline size_t dec_stats_at(const DecodeShape& s, size_t bh, int c, int t) {
  const size_t base = (dec_vbits_at(s, (size_t)s.batch * s.hkv, 0) + 1) / 2 * 2;
  return base + ((bh * (size_t)s.n_chunks + c) * (s.chunk / kDecBk) + t) * 2;
}

// Stage masks of the multi-kernel operations.
constexpr int kStagePrep = 1;      // backward: D = rowsum(O o dO), clear bits/counters
constexpr int kStageMain = 2;      // backward: dK/dV kernel; decode: split kernel
constexpr int kStageDq = 4;        // backward: dQ kernel
constexpr int kStageCombine = 4;   // decode: merge kernel
constexpr int kStagesAll = 7;

// Launchers (return hipGetLastError() of the launch).
hipError_t launch_fwd_bf16(const Shape& s, const void* q, const void* k, const void* v, void* o,
                           float* lse, int8_t* mask, int32_t* kept, hipStream_t st);
hipError_t launch_fwd_f32(const Shape& s, const float* q, const float* k, const float* v, float* o,
                          float* lse, int8_t* mask, int32_t* kept, hipStream_t st);

hipError_t launch_bwd_bf16(const Shape& s, const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* d_o, void* dq, void* dk,
                           void* dv, float* ws_d, uint32_t* ws_bits, float* ws_part,
                           int32_t* ws_plan, const int8_t* fwd_mask, int8_t* mask, int32_t* kept, hipStream_t st,
                           int stages, const int32_t* fwd_kept = nullptr);
hipError_t launch_bwd_f32(const Shape& s, const float* q, const float* k, const float* v,
                          const float* o, const float* lse, const float* d_o, float* dq, float* dk,
                          float* dv, float* ws_d, uint32_t* ws_bits, int8_t* mask, int32_t* kept,
                          hipStream_t st, int stages);

hipError_t launch_decode_bf16(const DecodeShape& s, const void* q, const void* kc, const void* vc,
                              const int32_t* seqlens, void* o, float* lse, float* ws,
                              int8_t* mask, int32_t* kept, hipStream_t st, int stages);
hipError_t launch_decode_f32(const DecodeShape& s, const float* q, const float* kc,
                             const float* vc, const int32_t* seqlens, float* o, float* lse,
                             float* ws, int8_t* mask, int32_t* kept, hipStream_t st, int stages);

// Small helpers (fill kernels instead of memsets, so the calls stay capturable).
hipError_t launch_fill_i32(int32_t* p, int32_t value, size_t n, hipStream_t st);
hipError_t launch_fill_i8(int8_t* p, int8_t value, size_t n, hipStream_t st);
hipError_t launch_decode_combine_bf16(const DecodeShape& s, const float* ws, void* o, float* lse,
                                      int32_t* kept, hipStream_t st);
hipError_t launch_decode_combine_f32(const DecodeShape& s, const float* ws, float* o, float* lse,
                                     int32_t* kept, hipStream_t st);

// Workspace layouts.
size_t bwd_ws_d_floats(const Shape& s);    // D = rowsum(O o dO), fp32 [B, Hq, Nq]
size_t bwd_bits_words(const Shape& s);     // backward decisions, one bit per tile
size_t bwd_part_floats(const Shape& s);    // gate pass: fp32 dK, dV partials [2, B, Hq, N_k, D]
size_t bwd_plan_ints(const Shape& s);      // gate pass: kept pairs per [B, Hkv, 128-key block]
size_t decode_ws_floats(const DecodeShape& s);

}  // namespace mala
