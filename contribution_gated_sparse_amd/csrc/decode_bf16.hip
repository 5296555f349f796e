// MALA split-KV decode for bf16 caches on gfx950 (Sec. 2.4; App. A.1
// "Fused decoding execution").
//
// One workgroup handles one 256-key split of one (sequence, KV head) for all
// query heads of the group (up to 16, packed as MFMA columns). Wave w owns the
// split's tile w (64 keys):
//   1. it reads its K tile straight from HBM in the 16x16x32 MFMA operand
//      layout and scores it against every head (score discovery: all keys);
//   2. per-head tile max and tile sum are exchanged through LDS; every wave
//      then replays the split's gate sequence (newest tile first, state
//      starting empty, L = N_k) from those statistics, which is exactly the
//      forward rule of Eq. 3 on a one-row block per head;
//   3. only a tile kept by at least one head loads its V tile (transposed
//      through a wave-private LDS slab) and runs P V on the MFMA; heads that
//      skipped it contribute P = 0;
//   4. the four waves' partial outputs are summed in LDS and the split writes
//      its partial state (m, l, O) in base 2.
// A second kernel merges the splits with the normalizer-aware reduction.
#include "mala_device.h"
#include "mala_internal.h"

namespace mala {
namespace {

constexpr int kChunk = 256;
constexpr int kTile = 64;
constexpr int kMaxGroup = 16;

// Position of key x inside a 32-key group of the V^T slab: matches the order
// in which one 32-key k-step of P^T is held (keys 4g..4g+3 then 16+4g..16+4g+3
// for lane group g), given by the 16x16 accumulator layout of S^T.
__device__ __forceinline__ int dec_pos(int x) {
  return (x & ~31) + 8 * ((x & 15) >> 2) + 4 * ((x >> 4) & 1) + (x & 3);
}

union alignas(16) DecSlab {
  bf16 vt[128][kTile + 8];            // V^T of the wave's tile
  float ored[128][kMaxGroup];         // then the wave's partial O^T
};
struct alignas(16) DecSmem {
  DecSlab slab[4];                    // one per wave
  float tmax[4][kMaxGroup];           // per (tile, head) max, base 2
  float tsum[4][kMaxGroup];           // per (tile, head) sum of 2^(s - max)
};

__global__ __launch_bounds__(256, 2) void decode_split_kernel(
    DecodeShape s, const bf16* __restrict__ Qd, const bf16* __restrict__ Kc,
    const bf16* __restrict__ Vc, const int32_t* __restrict__ seqlens, float* __restrict__ ws,
    int8_t* __restrict__ mask, int32_t* __restrict__ kept) {
  constexpr int D = 128;
  __shared__ DecSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j16 = lane & 15, g = lane >> 4;
  const int c = blockIdx.x;
  const int b = blockIdx.y / s.hkv, hk = blockIdx.y % s.hkv;
  const int G = s.group;
  int nk = seqlens[b];
  nk = max(1, min(nk, min(s.max_nk, s.cap)));
  const int tpc = kChunk / kTile;

  const int c0 = c * kChunk;
  const int ntile = c0 >= nk ? 0 : min(tpc, (nk - c0 + kTile - 1) / kTile);
  const size_t part_stride = (size_t)s.n_chunks * (D + 2);
  if (ntile == 0) {
    // split past the end of this sequence: no contribution
    if (tid < G) {
      float* p = ws + ((size_t)b * s.hq + hk * G + tid) * part_stride + (size_t)c * (D + 2);
      p[0] = kNegInf;
      p[1] = 0.f;
    }
    if (mask != nullptr && tid < G * tpc)
      mask[(((size_t)b * s.hq + hk * G + tid / tpc) * s.n_chunks + c) * tpc + tid % tpc] = -1;
    return;
  }

  // rows at or past N_k read as zeros (the cache may hold anything there)
  const size_t crow0 = ((size_t)b * s.hkv + hk) * (size_t)s.cap;
  const auto krs = make_rsrc(Kc + crow0 * D, (uint32_t)((size_t)nk * D * 2));
  const auto vrs = make_rsrc(Vc + crow0 * D, (uint32_t)((size_t)nk * D * 2));
  const int key0 = c0 + w * kTile;
  const bool has_keys = key0 < nk;

  // ---- score discovery for this wave's tile: S^T[key][head], 4 blocks of 16 keys
  f32x4 sacc[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) sacc[kb][r] = 0.f;
  if (has_keys) {
    bf16x8 qb[D / 32];
    const bf16* qrow = Qd + ((size_t)b * s.hq + hk * G + min(j16, G - 1)) * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) qb[t] = j16 < G ? load16(qrow + 32 * t + 8 * g) : zero8();
    bf16x8 ka[4][D / 32];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
        ka[kb][t] = buf_load16(krs, (uint32_t)((key0 + 16 * kb + j16) * D + 32 * t + 8 * g) * 2);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int t = 0; t < D / 32; ++t) sacc[kb] = mfma16(ka[kb][t], qb[t], sacc[kb]);
  }
  // lane (head j16, group g) holds keys key0 + 16kb + 4g + r
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + 16 * kb + 4 * g + r;
      const float v = key < nk ? sacc[kb][r] * s.scale_log2 : kNegInf;
      sacc[kb][r] = v;
      mx = fmaxf(mx, v);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  float sm_ = 0.f;
  if (mx > kNegInf) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm_ += fast_exp2(sacc[kb][r] - mx);
  }
  sm_ += __shfl_xor(sm_, 16, 64);
  sm_ += __shfl_xor(sm_, 32, 64);
  if (g == 0) {
    sm.tmax[w][j16] = mx;
    sm.tsum[w][j16] = sm_;
  }
  __syncthreads();

  // ---- the split's gate: newest tile first, empty state, L = N_k (Eq. 3)
  const float c2 = s.log2_tau - fast_log2((float)nk);
  float M = kNegInf, S = 0.f;
  uint32_t keepbits = 0;            // bit t: this lane's head keeps tile t
  for (int t = ntile - 1; t >= 0; --t) {
    const float tm = sm.tmax[t][j16], ts = sm.tsum[t][j16];
    const bool keep = (S == 0.f) || (tm - (M + fast_log2(S)) >= c2);
    if (keep) {
      const float mn = fmaxf(M, tm);
      S = S * fast_exp2(M - mn) + ts * fast_exp2(tm - mn);
      M = mn;
      keepbits |= 1u << t;
    }
  }
  const bool head_ok = j16 < G;
  const bool mine = head_ok && ((keepbits >> w) & 1u);
  const uint64_t vote = __builtin_amdgcn_ballot_w64(mine);
  const bool tile_kept = has_keys && vote != 0;

  if (w == 0 && g == 0 && head_ok) {
    const size_t bh = (size_t)b * s.hq + hk * G + j16;
    if (mask != nullptr)
      for (int t = 0; t < tpc; ++t)
        mask[(bh * s.n_chunks + c) * tpc + t] = t < ntile ? (int8_t)((keepbits >> t) & 1u) : (int8_t)-1;
    if (kept != nullptr) atomicAdd(&kept[(size_t)b * (s.hq + s.hkv) + hk * G + j16], __popc(keepbits));
  }
  if (kept != nullptr && lane == 0 && tile_kept)
    atomicAdd(&kept[(size_t)b * (s.hq + s.hkv) + s.hq + hk], 1);

  // ---- kept tile: V load (HBM) -> transposed LDS slab -> P V on the MFMA
  if (tile_kept) {
    const int dc = lane & 15, kq = lane >> 4;        // 16-byte column chunk, 16-key group
    bf16x8 vr[16];
#pragma unroll
    for (int p = 0; p < 16; ++p)
      vr[p] = buf_load16(vrs, (uint32_t)((key0 + 16 * kq + p) * D + 8 * dc) * 2);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pos = dec_pos(16 * kq + 4 * u);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x4 x = {vr[4 * u][e], vr[4 * u + 1][e], vr[4 * u + 2][e], vr[4 * u + 3][e]};
        *reinterpret_cast<bf16x4*>(&sm.slab[w].vt[8 * dc + e][pos]) = x;
      }
    }
  }
  __syncthreads();
  f32x4 oacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) oacc[db][r] = 0.f;
  if (tile_kept) {
    // P^T as the B operand: lane (head j16, group g) holds keys of one 32-key step
    bf16x8 pb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float sv = sacc[2 * ks + (e >> 2)][e & 3];
        pb[ks][e] = (bf16)(mine ? fast_exp2(sv - M) : 0.f);
      }
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        oacc[db] = mfma16(load16(&sm.slab[w].vt[16 * db + j16][32 * ks + 8 * g]), pb[ks], oacc[db]);
  }
  __syncthreads();
  // O^T[d = 16db + 4g + r][head j16]
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.slab[w].ored[16 * db + 4 * g + r][j16] = oacc[db][r];
  __syncthreads();

  // ---- sum the four waves and write the split's partial state
  for (int idx = tid; idx < D * G; idx += 256) {
    const int hh = idx / D, d = idx % D;
    const float o = sm.slab[0].ored[d][hh] + sm.slab[1].ored[d][hh] + sm.slab[2].ored[d][hh] +
                    sm.slab[3].ored[d][hh];
    float* p = ws + ((size_t)b * s.hq + hk * G + hh) * part_stride + (size_t)c * (D + 2);
    p[2 + d] = o;
  }
  if (w == 0 && g == 0 && head_ok) {
    float* p = ws + ((size_t)b * s.hq + hk * G + j16) * part_stride + (size_t)c * (D + 2);
    p[0] = M;
    p[1] = S;
  }
}

// Merge the split partial states of one (sequence, head): z = log sum_c Z_c,
// O = sum_c Z_c O_c / sum_c Z_c (the standard online-softmax reduction).
template <typename OutT>
__global__ __launch_bounds__(256) void decode_combine_kernel(int hq, int d, int n_chunks,
                                                             const float* __restrict__ ws,
                                                             OutT* __restrict__ o,
                                                             float* __restrict__ lse) {
  const int bh = blockIdx.x;
  const float* part = ws + (size_t)bh * n_chunks * (d + 2);
  __shared__ float red[256];
  __shared__ float acc[8][32];
  const int tid = threadIdx.x;
  float mx = kNegInf;
  for (int c = tid; c < n_chunks; c += 256) mx = fmaxf(mx, part[(size_t)c * (d + 2)]);
  red[tid] = mx;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st) red[tid] = fmaxf(red[tid], red[tid + st]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float den = 0.f;
  for (int c = tid; c < n_chunks; c += 256) {
    const float m = part[(size_t)c * (d + 2)];
    if (m > kNegInf) den += part[(size_t)c * (d + 2) + 1] * fast_exp2(m - M);
  }
  red[tid] = den;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st) red[tid] += red[tid + st];
    __syncthreads();
  }
  const float Z = red[0];
  const int dd = blockIdx.y * 32 + (tid & 31), cl = tid >> 5;
  float num = 0.f;
  if (dd < d)
    for (int c = cl; c < n_chunks; c += 8) {
      const float m = part[(size_t)c * (d + 2)];
      if (m > kNegInf) num += part[(size_t)c * (d + 2) + 2 + dd] * fast_exp2(m - M);
    }
  acc[cl][tid & 31] = num;
  __syncthreads();
  if (tid < 32 && dd < d) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) t += acc[k][tid];
    o[(size_t)bh * d + dd] = (OutT)(Z > 0.f ? t / Z : 0.f);
  }
  if (blockIdx.y == 0 && tid == 0) lse[bh] = Z > 0.f ? (M + fast_log2(Z)) * kLn2 : kNegInf;
  (void)hq;
}

}  // namespace

size_t decode_ws_floats(const DecodeShape& s) {
  return (size_t)s.batch * s.hq * s.n_chunks * (s.d + 2);
}

hipError_t launch_decode_combine_bf16(const DecodeShape& s, const float* ws, void* o, float* lse,
                                      hipStream_t st) {
  hipLaunchKernelGGL(decode_combine_kernel<bf16>, dim3(s.batch * s.hq, (s.d + 31) / 32),
                     dim3(256), 0, st, s.hq, s.d, s.n_chunks, ws, (bf16*)o, lse);
  return hipGetLastError();
}
hipError_t launch_decode_combine_f32(const DecodeShape& s, const float* ws, float* o, float* lse,
                                     hipStream_t st) {
  hipLaunchKernelGGL(decode_combine_kernel<float>, dim3(s.batch * s.hq, (s.d + 31) / 32),
                     dim3(256), 0, st, s.hq, s.d, s.n_chunks, ws, o, lse);
  return hipGetLastError();
}

hipError_t launch_decode_bf16(const DecodeShape& s, const void* q, const void* kc, const void* vc,
                              const int32_t* seqlens, void* o, float* lse, float* ws,
                              int8_t* mask, int32_t* kept, hipStream_t st, int stages) {
  if (stages & kStageMain) {
    if (kept != nullptr) {
      hipError_t e = launch_fill_i32(kept, 0, (size_t)s.batch * (s.hq + s.hkv), st);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(decode_split_kernel, dim3(s.n_chunks, s.batch * s.hkv), dim3(256), 0, st,
                       s, (const bf16*)q, (const bf16*)kc, (const bf16*)vc, seqlens, ws, mask,
                       kept);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kStageCombine) return launch_decode_combine_bf16(s, ws, o, lse, st);
  return hipSuccess;
}

}  // namespace mala
