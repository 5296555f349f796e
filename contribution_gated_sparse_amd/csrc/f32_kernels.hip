// MALA for fp32 inputs: straightforward VALU kernels (one lane per query row
// or per key) with the same decision partition and workspace formats as the
// bf16 MFMA kernels. Scores, exponentials, logarithms and the softmax state
// are evaluated in fp64 (inputs and outputs stay fp32), so the fp32 path is
// accurate to a few fp32 ulps of its outputs. They serve fp32 problems, which
// are small in this library's use (the tiny causal configuration); the bf16
// kernels are the performance path.
#include <type_traits>
#include "mala_device.h"
#include "mala_internal.h"

namespace mala {
namespace {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}
// ballot restricted to the 32 lanes of this lane's half
__device__ __forceinline__ bool half_any(bool p) {
  const uint64_t m = __builtin_amdgcn_ballot_w64(p);
  const int half = (threadIdx.x & 63) >> 5;
  return ((m >> (32 * half)) & 0xffffffffull) != 0;
}
// ballot restricted to the 16 lanes of this lane's quarter
__device__ __forceinline__ bool quarter_any(bool p) {
  const uint64_t m = __builtin_amdgcn_ballot_w64(p);
  const int qtr = (threadIdx.x & 63) >> 4;
  return ((m >> (16 * qtr)) & 0xffffull) != 0;
}

// ---------------------------------------------------------------- forward
// Block = 64 lanes = 64 query rows = two 32-row decision blocks (lanes 0-31,
// 32-63). Key tiles of 64 keys, descending from each half's diagonal.
template <int D>
__global__ __launch_bounds__(64) void fwd_f32_kernel(Shape s, const float* __restrict__ Q,
                                                     const float* __restrict__ K,
                                                     const float* __restrict__ V,
                                                     float* __restrict__ O, float* __restrict__ LSE,
                                                     int8_t* __restrict__ mask,
                                                     int32_t* __restrict__ kept, int n_blk) {
  __shared__ float ks[64][D];
  __shared__ float vs[64][D];
  const int t = threadIdx.x, half = t >> 5;
  const int bh_count = s.batch * s.hq;
  const int blk = n_blk - 1 - (int)(blockIdx.x / bh_count);
  const int bh = (int)(blockIdx.x % bh_count);
  const int b = bh / s.hq, h = bh % s.hq, hk = h / s.group;
  const size_t qrow0 = (size_t)bh * s.nq, krow0 = ((size_t)b * s.hkv + hk) * (size_t)s.nk;
  const int q0 = blk * 64, q = q0 + t;
  const bool valid = q < s.nq;
  const int tr = (s.nq + 31) / 32, tc = (s.nk + 63) / 64;
  auto top_of = [&](int first) {
    if (first >= s.nq) return -1;
    const int last = min(first + 31, s.nq - 1);
    const int lk = s.causal ? min(last + s.offset, s.nk - 1) : s.nk - 1;
    return lk / 64;
  };
  const int top_h = top_of(q0 + 32 * half);
  const int top_b = max(top_of(q0), top_of(q0 + 32));

  float qr[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qr[e] = valid ? Q[(qrow0 + q) * D + e] : 0.f;
    o[e] = 0.f;
  }
  const double scale = s.scale;
  const double cth = s.log_tau - log(s.causal ? (double)(q + s.offset + 1) : (double)s.nk);
  double m = -HUGE_VAL, lsum = 0.0;
  int nk_kept = 0;
  for (int j = top_b; j >= 0; --j) {
    __syncthreads();
    const int key = j * 64 + t;
#pragma unroll 8
    for (int e = 0; e < D; ++e) {
      ks[t][e] = key < s.nk ? K[(krow0 + key) * D + e] : 0.f;
      vs[t][e] = key < s.nk ? V[(krow0 + key) * D + e] : 0.f;
    }
    __syncthreads();
    const bool active = j <= top_h;
    double sc[64];
    double tm = -HUGE_VAL;
    for (int k = 0; k < 64; ++k) {
      double acc = 0.0;
#pragma unroll 16
      for (int e = 0; e < D; ++e) acc = fma((double)qr[e], (double)ks[k][e], acc);
      const int kk = j * 64 + k;
      const bool ok = valid && kk < s.nk && (!s.causal || kk <= q + s.offset);
      sc[k] = ok ? acc * scale : -HUGE_VAL;
      tm = fmax(tm, sc[k]);
    }
    const bool constrained = active && valid && tm > -HUGE_VAL;
    const bool row_keeps = constrained && (lsum == 0.0 || tm - (m + log(lsum)) >= cth);
    const bool keep = active && half_any(row_keeps);
    if (keep) {
      const double mn = fmax(m, tm);
      const double mu = mn == -HUGE_VAL ? 0.0 : mn;
      const double alpha = exp(m - mu);
      double rs = 0.0;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] *= (float)alpha;
      for (int k = 0; k < 64; ++k) {
        const double p = exp(sc[k] - mu);
        rs += p;
        const float pf = (float)p;
#pragma unroll
        for (int e = 0; e < D; ++e) o[e] = fmaf(pf, vs[k][e], o[e]);
      }
      lsum = alpha * lsum + rs;
      m = mn;
      ++nk_kept;
    }
    if (active && (t & 31) == 0 && mask != nullptr)
      mask[((size_t)bh * tr + (q0 >> 5) + half) * tc + j] = keep ? 1 : 0;
  }
  if (top_h < 0) return;
  const int i32 = (q0 >> 5) + half;
  if ((t & 31) == 0) {
    if (mask != nullptr)
      for (int jj = top_h + 1; jj < tc; ++jj) mask[((size_t)bh * tr + i32) * tc + jj] = -1;
    if (kept != nullptr) kept[(size_t)bh * tr + i32] = nk_kept;
  }
  if (!valid) return;
  const float inv = lsum > 0.0 ? (float)(1.0 / lsum) : 0.f;
#pragma unroll
  for (int e = 0; e < D; ++e) O[(qrow0 + q) * D + e] = o[e] * inv;
  LSE[qrow0 + q] = lsum > 0.0 ? (float)(m + log(lsum)) : kNegInf;
}

// ---------------------------------------------------------------- backward
__global__ __launch_bounds__(256) void bwd_prep_f32_kernel(int rows, int d, const float* O,
                                                           const float* dO, float* Dq,
                                                           uint32_t* bits, size_t nwords,
                                                           int32_t* kept, size_t nkept,
                                                           int8_t* mask, size_t nmask) {
  const size_t gtid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t nthr = (size_t)gridDim.x * blockDim.x;
  for (size_t i = gtid; i < nwords; i += nthr) bits[i] = 0u;
  if (kept != nullptr)
    for (size_t i = gtid; i < nkept; i += nthr) kept[i] = 0;
  if (mask != nullptr)
    for (size_t i = gtid; i < nmask; i += nthr) mask[i] = -1;
  for (size_t r = gtid; r < (size_t)rows; r += nthr) {
    double acc = 0.0;     // D feeds dP - D, which cancels: sum in fp64
    for (int e = 0; e < d; ++e) acc = fma((double)O[r * d + e], (double)dO[r * d + e], acc);
    Dq[r] = (float)acc;
  }
}

// Key-major dK/dV: block = 64 lanes = 64 keys = four 16-key decision columns.
template <int D>
__global__ __launch_bounds__(64) void bwd_dkdv_f32_kernel(
    Shape s, const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dq,
    float* __restrict__ dK, float* __restrict__ dV, uint32_t* __restrict__ bits,
    int8_t* __restrict__ mask, int32_t* __restrict__ kept) {
  // dK and dV accumulate in fp64, 64 columns per pass over the rows (two
  // passes at d = 128, which recompute S and dP; the decisions are written
  // in the first)
  constexpr int DA = 64, NPASS = D / DA;
  __shared__ float kv[2][64][D + 1];
  __shared__ float qs[32][D];
  __shared__ float os[32][D];
  __shared__ double zz[32], uu[32], dd[32];
  const int t = threadIdx.x, qtr = t >> 4;
  const int bk_count = s.batch * s.hkv;
  const int J = (int)(blockIdx.x / bk_count);
  const int bkv = (int)(blockIdx.x % bk_count);
  const int b = bkv / s.hkv, hk = bkv % s.hkv;
  const size_t krow0 = ((size_t)b * s.hkv + hk) * (size_t)s.nk;
  const int key = J * 64 + t;
  const int tr = (s.nq + 31) / 32, tc = (s.nk + 15) / 16, words = (tc + 31) / 32;
  for (int e = 0; e < D; ++e) {
    kv[0][t][e] = key < s.nk ? K[(krow0 + key) * D + e] : 0.f;
    kv[1][t][e] = key < s.nk ? V[(krow0 + key) * D + e] : 0.f;
  }
  const int kc0 = J * 64 + 16 * qtr;           // first key of this lane's column
  int i_start = 0;
  if (s.causal) {
    const int need = J * 64 - s.offset;
    i_start = need <= 0 ? 0 : need / 32;
  }
  for (int pass = 0; pass < NPASS; ++pass) {
  const int ca = pass * DA;                    // first accumulated column
  double dk[DA], dv[DA];
#pragma unroll
  for (int e = 0; e < DA; ++e) { dk[e] = 0.0; dv[e] = 0.0; }
  for (int hh = 0; hh < s.group; ++hh) {
    const int h = hk * s.group + hh;
    const size_t bh = (size_t)b * s.hq + h, qrow0 = bh * s.nq;
    for (int i = i_start; i < tr; ++i) {
      __syncthreads();
      const int r = t & 31, c0 = (t >> 5) * (D / 2);
      const int qrow = i * 32 + r;
      for (int e = c0; e < c0 + D / 2; ++e) {
        qs[r][e] = qrow < s.nq ? Q[(qrow0 + qrow) * D + e] : 0.f;
        os[r][e] = qrow < s.nq ? dO[(qrow0 + qrow) * D + e] : 0.f;
      }
      if (t < 32) {
        const double L = s.causal ? (double)(qrow + s.offset + 1) : (double)s.nk;
        const double z = qrow < s.nq ? (double)LSE[qrow0 + qrow] : 0.0;
        zz[t] = z;
        uu[t] = z + (s.log_tau - log(L));        // skip iff s < z + log(tau / L) everywhere
        dd[t] = qrow < s.nq ? (double)Dq[qrow0 + qrow] : 0.0;
      }
      __syncthreads();
      const int r0 = i * 32;
      const bool legal_tile = r0 < s.nq && kc0 < s.nk &&
                              (!s.causal || kc0 <= min(r0 + 31, s.nq - 1) + s.offset);
      double sc[32];
      double x = -HUGE_VAL;
      for (int qq = 0; qq < 32; ++qq) {
        double acc = 0.0;
#pragma unroll 16
        for (int e = 0; e < D; ++e) acc = fma((double)kv[0][t][e], (double)qs[qq][e], acc);
        const int qi = r0 + qq;
        const bool ok = qi < s.nq && key < s.nk && (!s.causal || key <= qi + s.offset);
        sc[qq] = ok ? acc * s.scale : -HUGE_VAL;
        if (ok) x = fmax(x, sc[qq] - uu[qq]);
      }
      const bool keep = legal_tile && quarter_any(x >= 0.0);
      if (pass == 0 && legal_tile && (t & 15) == 0) {
        const int j16 = kc0 / 16;
        if (keep) atomicOr(&bits[(bh * tr + i) * words + (j16 >> 5)], 1u << (j16 & 31));
        if (mask != nullptr) mask[(bh * tr + i) * tc + j16] = keep ? 1 : 0;
        if (keep && kept != nullptr) atomicAdd(&kept[bh * tr + i], 1);
      }
      if (keep) {
        for (int qq = 0; qq < 32; ++qq) {
          const double p = exp(sc[qq] - zz[qq]);
          double dp = 0.0;
#pragma unroll 16
          for (int e = 0; e < D; ++e) dp = fma((double)kv[1][t][e], (double)os[qq][e], dp);
          const double ds = p * (dp - dd[qq]);
#pragma unroll
          for (int e = 0; e < DA; ++e) {
            dv[e] += p * (double)os[qq][ca + e];
            dk[e] += ds * (double)qs[qq][ca + e];
          }
        }
      }
    }
  }
  if (key < s.nk) {
#pragma unroll
    for (int e = 0; e < DA; ++e) {
      dK[(krow0 + key) * D + ca + e] = (float)(dk[e] * s.scale);
      dV[(krow0 + key) * D + ca + e] = (float)dv[e];
    }
  }
  }
}

// Query-major dQ over the kept tiles recorded by the dK/dV kernel.
template <int D>
__global__ __launch_bounds__(64) void bwd_dq_f32_kernel(
    Shape s, const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dq,
    float* __restrict__ dQ, const uint32_t* __restrict__ bits) {
  // dQ accumulates in fp64, 64 columns per pass over the keys (two passes
  // at d = 128, which recompute S and dP)
  constexpr int DA = 64, NPASS = D / DA;
  __shared__ float dorow[64][D + 1];
  __shared__ float ks[16][D];
  __shared__ float vs[16][D];
  const int t = threadIdx.x, half = t >> 5;
  const int bh_count = s.batch * s.hq;
  const int blk = (int)(blockIdx.x / bh_count);
  const int bh = (int)(blockIdx.x % bh_count);
  const int b = bh / s.hq, h = bh % s.hq, hk = h / s.group;
  const size_t qrow0 = (size_t)bh * s.nq, krow0 = ((size_t)b * s.hkv + hk) * (size_t)s.nk;
  const int q = blk * 64 + t;
  const bool valid = q < s.nq;
  const int tr = (s.nq + 31) / 32, tc = (s.nk + 15) / 16, words = (tc + 31) / 32;
  float qr[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qr[e] = valid ? Q[(qrow0 + q) * D + e] : 0.f;
    dorow[t][e] = valid ? dO[(qrow0 + q) * D + e] : 0.f;
  }
  const double z = valid ? (double)LSE[qrow0 + q] : 0.0;
  const double dd = valid ? (double)Dq[qrow0 + q] : 0.0;
  const int i32 = min(blk * 2 + half, tr - 1);
  const uint32_t* mybits = bits + ((size_t)bh * tr + i32) * words;
  for (int pass = 0; pass < NPASS; ++pass) {
  const int ca = pass * DA;                    // first accumulated column
  double dq[DA];
#pragma unroll
  for (int e = 0; e < DA; ++e) dq[e] = 0.0;
  for (int j = 0; j < tc; ++j) {
    __syncthreads();
    const int r = t & 15, c0 = (t >> 4) * (D / 4);
    const int kk = j * 16 + r;
    for (int e = c0; e < c0 + D / 4; ++e) {
      ks[r][e] = kk < s.nk ? K[(krow0 + kk) * D + e] : 0.f;
      vs[r][e] = kk < s.nk ? V[(krow0 + kk) * D + e] : 0.f;
    }
    __syncthreads();
    const bool keep = valid && ((mybits[j >> 5] >> (j & 31)) & 1u);
    if (!keep) continue;
    for (int k = 0; k < 16; ++k) {
      const int key = j * 16 + k;
      if (!(key < s.nk && (!s.causal || key <= q + s.offset))) continue;
      double acc = 0.0, dp = 0.0;
#pragma unroll 16
      for (int e = 0; e < D; ++e) {
        acc = fma((double)qr[e], (double)ks[k][e], acc);
        dp = fma((double)dorow[t][e], (double)vs[k][e], dp);
      }
      const double p = exp(acc * s.scale - z);
      const double ds = p * (dp - dd);
#pragma unroll
      for (int e = 0; e < DA; ++e) dq[e] += ds * (double)ks[k][ca + e];
    }
  }
  if (valid) {
#pragma unroll
    for (int e = 0; e < DA; ++e) dQ[(qrow0 + q) * D + ca + e] = (float)(dq[e] * s.scale);
  }
  }
}

// ---------------------------------------------------------------- decode
// Block = one wave for one (split, sequence, KV head); lane = key of a tile;
// every query head of the group is gated separately, and a tile's V is read
// when at least one head keeps it. The partial state is written in base 2
// (the format the combine kernel shared with the bf16 path expects).
__device__ __forceinline__ double wave_max_d(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmax(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <int D>
__global__ __launch_bounds__(64) void decode_split_f32_kernel(
    DecodeShape s, const float* __restrict__ Qd, const float* __restrict__ Kc,
    const float* __restrict__ Vc, const int32_t* __restrict__ seqlens, float* __restrict__ ws,
    int8_t* __restrict__ mask) {
  constexpr int kMaxG = 16;
  __shared__ float qs[kMaxG][D];
  __shared__ double ps[kMaxG][64];
  __shared__ double st_m[kMaxG], st_s[kMaxG];
  __shared__ uint32_t st_bits[kMaxG];
  const int t = threadIdx.x, c = blockIdx.x;
  const int b = blockIdx.y / s.hkv, hk = blockIdx.y % s.hkv, G = s.group;
  int nk = seqlens[b];
  nk = max(1, min(nk, min(s.max_nk, s.cap)));
  const int tpc = s.chunk / 64;    // tiles per split
  const int c0 = c * s.chunk;
  const int ntile = c0 >= nk ? 0 : min(tpc, (nk - c0 + 63) / 64);
  const size_t crow0 = ((size_t)b * s.hkv + hk) * (size_t)s.cap;
  const size_t bh0 = (size_t)b * s.hq + hk * G;
  uint32_t* wbits = reinterpret_cast<uint32_t*>(ws);
  for (int hh = 0; hh < G; ++hh)
    for (int e = t; e < D; e += 64) qs[hh][e] = Qd[(bh0 + hh) * D + e];
  if (t < kMaxG) { st_m[t] = -HUGE_VAL; st_s[t] = 0.0; st_bits[t] = 0u; }
  // decision words and mask entries of tiles past the sequence's end
  for (int x = (ntile + 31) / 32 + t; x < s.wps; x += 64) {
    for (int hh = 0; hh < G; ++hh) wbits[dec_kbits_at(s, bh0 + hh, c) + x] = 0u;
    wbits[dec_vbits_at(s, blockIdx.y, c) + x] = 0u;
  }
  if (mask != nullptr)
    for (int x = t; x < G * (tpc - ntile); x += 64)
      mask[((bh0 + x / (tpc - ntile)) * s.n_chunks + c) * tpc + ntile + x % (tpc - ntile)] = -1;
  __syncthreads();
  const double cth = s.log_tau - log((double)nk);
  double o0[kMaxG], o1[kMaxG];
#pragma unroll
  for (int hh = 0; hh < kMaxG; ++hh) { o0[hh] = 0.0; o1[hh] = 0.0; }
  uint32_t vbits = 0;               // bit tt: tile tt's V was read
  for (int tt = ntile - 1; tt >= 0; --tt) {
    const int key = c0 + 64 * tt + t;
    const bool ok = key < nk;
    bool any_keep = false;
    double alpha[kMaxG];
#pragma unroll
    for (int hh = 0; hh < kMaxG; ++hh) {
      alpha[hh] = 1.0;
      if (hh >= G) continue;
      double acc = 0.0;
      if (ok)
        for (int e = 0; e < D; ++e) acc = fma((double)qs[hh][e], (double)Kc[(crow0 + key) * D + e], acc);
      const double sv = ok ? acc * s.scale : -HUGE_VAL;
      const double tm = wave_max_d(sv);
      const double M = st_m[hh], S = st_s[hh];
      const bool keep = (S == 0.0) || (tm - (M + log(S)) >= cth);
      double p = 0.0;
      if (keep) {
        const double mn = fmax(M, tm);
        alpha[hh] = exp(M - mn);
        p = exp(sv - mn);
        const double tot = wave_sum_d(p);
        __syncthreads();
        if (t == 0) {
          st_s[hh] = S * alpha[hh] + tot;
          st_m[hh] = mn;
          st_bits[hh] |= 1u << (tt & 31);
        }
        any_keep = true;
      }
      if (t == 0 && mask != nullptr)
        mask[((bh0 + hh) * s.n_chunks + c) * tpc + tt] = keep ? 1 : 0;
      ps[hh][t] = p;
      __syncthreads();
    }
    if (any_keep) {
      vbits |= 1u << (tt & 31);
#pragma unroll
      for (int hh = 0; hh < kMaxG; ++hh) { o0[hh] *= alpha[hh]; o1[hh] *= alpha[hh]; }
      for (int k = 0; k < 64; ++k) {
        const int kk = c0 + 64 * tt + k;
        if (kk >= nk) break;
        const double v0 = t < D ? (double)Vc[(crow0 + kk) * D + t] : 0.0;
        const double v1 = t + 64 < D ? (double)Vc[(crow0 + kk) * D + t + 64] : 0.0;
#pragma unroll
        for (int hh = 0; hh < kMaxG; ++hh) {
          if (hh >= G) continue;
          o0[hh] = fma(ps[hh][k], v0, o0[hh]);
          o1[hh] = fma(ps[hh][k], v1, o1[hh]);
        }
      }
    }
    __syncthreads();
    if ((tt & 31) == 0) {           // the lowest tile of a 32-tile word: flush it
      if (t < G) {
        wbits[dec_kbits_at(s, bh0 + t, c) + tt / 32] = st_bits[t];
        st_bits[t] = 0u;
      }
      if (t == 0) wbits[dec_vbits_at(s, blockIdx.y, c) + tt / 32] = vbits;
      vbits = 0u;
    }
    __syncthreads();
  }
  const double log2e = 1.4426950408889634;
#pragma unroll
  for (int hh = 0; hh < kMaxG; ++hh) {
    if (hh >= G) continue;
    const size_t bhh = (size_t)b * s.hq + hk * G + hh;
    float* pms = ws + dec_ms_at(s, bhh, c);
    float* po = ws + dec_o_at(s, bhh, c);
    // base-2 partial state with the scale folded in: m2 = m*log2e, O and S
    // unnormalized relative to 2^m2 (the combine kernel's format)
    if (t == 0) {
      pms[0] = ntile ? (float)(st_m[hh] * log2e) : kNegInf;
      pms[1] = ntile ? (float)st_s[hh] : 0.f;
    }
    if (t < D) po[t] = (float)o0[hh];
    if (t + 64 < D) po[t + 64] = (float)o1[hh];
  }
}

__global__ void fill_i32_kernel(int32_t* p, int32_t v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}
__global__ void fill_i8_kernel(int8_t* p, int8_t v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

unsigned grid_for(size_t n) {
  size_t g = (n + 255) / 256;
  if (g < 1) g = 1;
  if (g > 4096) g = 4096;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, int32_t value, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(grid_for(n)), dim3(256), 0, st, p, value, n);
  return hipGetLastError();
}
hipError_t launch_fill_i8(int8_t* p, int8_t value, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i8_kernel, dim3(grid_for(n)), dim3(256), 0, st, p, value, n);
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const Shape& s, const float* q, const float* k, const float* v, float* o,
                          float* lse, int8_t* mask, int32_t* kept, hipStream_t st) {
  const int n_blk = (s.nq + 63) / 64;
  const dim3 grid((unsigned)(n_blk * s.batch * s.hq));
  if (grid.x == 0) return hipSuccess;
  if (s.d == 128)
    hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, dim3(64), 0, st, s, q, k, v, o, lse, mask, kept,
                       n_blk);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, dim3(64), 0, st, s, q, k, v, o, lse, mask, kept,
                       n_blk);
  return hipGetLastError();
}

hipError_t launch_bwd_f32(const Shape& s, const float* q, const float* k, const float* v,
                          const float* o, const float* lse, const float* d_o, float* dq, float* dk,
                          float* dv, float* ws_d, uint32_t* ws_bits, int8_t* mask, int32_t* kept,
                          hipStream_t st, int stages) {
  const int rows = s.batch * s.hq * s.nq;
  const size_t nwords = bwd_bits_words(s);
  const size_t tr = (s.nq + 31) / 32, tc = (s.nk + 15) / 16;
  const size_t nkept = (size_t)s.batch * s.hq * tr;
  const size_t nmask = mask ? (size_t)s.batch * s.hq * tr * tc : 0;
  size_t work = (size_t)rows;
  if (nwords > work) work = nwords;
  if (nmask > work) work = nmask;
  if (stages & kStagePrep)
    hipLaunchKernelGGL(bwd_prep_f32_kernel, dim3(grid_for(work)), dim3(256), 0, st, rows, s.d, o,
                       d_o, ws_d, ws_bits, nwords, kept, nkept, mask, nmask);
  dim3 g1((unsigned)(((s.nk + 63) / 64) * s.batch * s.hkv));
  dim3 g2((unsigned)(((s.nq + 63) / 64) * s.batch * s.hq));
  if (!(stages & kStageMain)) g1.x = 0;
  if (!(stages & kStageDq)) g2.x = 0;
  if (s.d == 128) {
    if (g1.x)
      hipLaunchKernelGGL(bwd_dkdv_f32_kernel<128>, g1, dim3(64), 0, st, s, q, k, v, d_o, lse,
                         ws_d, dk, dv, ws_bits, mask, kept);
    if (g2.x)
      hipLaunchKernelGGL(bwd_dq_f32_kernel<128>, g2, dim3(64), 0, st, s, q, k, v, d_o, lse, ws_d,
                         dq, ws_bits);
  } else {
    if (g1.x)
      hipLaunchKernelGGL(bwd_dkdv_f32_kernel<64>, g1, dim3(64), 0, st, s, q, k, v, d_o, lse,
                         ws_d, dk, dv, ws_bits, mask, kept);
    if (g2.x)
      hipLaunchKernelGGL(bwd_dq_f32_kernel<64>, g2, dim3(64), 0, st, s, q, k, v, d_o, lse, ws_d,
                         dq, ws_bits);
  }
  return hipGetLastError();
}

hipError_t launch_decode_f32(const DecodeShape& s, const float* q, const float* kc,
                             const float* vc, const int32_t* seqlens, float* o, float* lse,
                             float* ws, int8_t* mask, int32_t* kept, hipStream_t st, int stages) {
  if (stages & kStageMain) {
  const dim3 grid(s.n_chunks, s.batch * s.hkv);
  if (s.d == 128)
    hipLaunchKernelGGL(decode_split_f32_kernel<128>, grid, dim3(64), 0, st, s, q, kc, vc, seqlens,
                       ws, mask);
  else
    hipLaunchKernelGGL(decode_split_f32_kernel<64>, grid, dim3(64), 0, st, s, q, kc, vc, seqlens,
                       ws, mask);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  }
  if (stages & kStageCombine) return launch_decode_combine_f32(s, ws, o, lse, kept, st);
  return hipSuccess;
}

}  // namespace mala
