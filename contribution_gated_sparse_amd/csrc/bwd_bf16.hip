// MALA backward for bf16 inputs on gfx950 (Algorithm 2; Sec. 2.2 "Offline
// Sparse Probability"; App. A.1 "Fused backward execution").
//
// Three kernels by default:
//   1. bwd_prep:  D_q = rowsum(O o dO) in fp32, and clears the decision bits
//                 and the kept-tile counters.
//   2. bwd_dkdv:  key-major. A workgroup owns 128 keys of one KV head (8 waves
//                 x 16 keys) and walks every query head of the group and every
//                 64-row query step from the diagonal down the sequence. Each
//                 wave recomputes S = Q K^T for its 16 keys and the step's 64
//                 rows, applies the offline gate (Eq. 4) to each of its two
//                 32 x 16 tiles against the saved z_q, and only for kept tiles
//                 reads the staged dO rows and forms P = exp(S - z), dP = dO V^T,
//                 dS = P o (dP - D) and accumulates dV += P^T dO and
//                 dK += dS^T Q on chip. The decisions are written as one bit
//                 per tile.
//   3. bwd_dq:    query-major. A workgroup owns 256 query rows (8 waves x 32);
//                 each wave reads the decision bits of its rows and, for kept
//                 tiles only, recomputes S, P, dP, dS and accumulates
//                 dQ += dS K on chip. No atomics on dQ. It also counts the
//                 kept tiles of each 32-row block from the bits.
// Both kernels see the same decisions, so dQ, dK and dV use one support.
//
// With MALA_FLAG_GATE_PASS the decisions come first instead, for inputs on
// which few tiles are kept:
//   bwd_gate:     query-major; forms every legal score and writes the
//                 decision bits (Eq. 4). Given the forward's tile mask
//                 (mala_bwd_nested), only the scores of the tiles the
//                 forward kept: the others meet the skip condition
//                 (nested support, Sec. 2.2).
//   bwd_plan:     counts each key block's kept (query head, 64-row step)
//                 pairs over its KV head's group.
//   bwd_dkdv (gated): walks over the steps that hold a kept tile of the
//                 workgroup; nothing is staged for the others. A light key
//                 block is one walk over the group's heads, writing dK, dV;
//                 a heavy one a walk per query head, into fp32 partials.
//   bwd_dkdv_finalize: sums the heavy blocks' partials into dK, dV.
// bwd_dq is the same kernel in both modes.
//
// dS enters the dK and dQ products as a bf16 MFMA operand. dK takes it as one
// bf16 operand. For dQ it is by default split into hi = bf16(dS) and
// lo = bf16(dS - hi) and both halves are multiplied (two MFMAs), which
// carries dS to ~16 significant bits: a row of dS sums to zero over the full
// support (sum_k dS_qk = 0), so dQ_q = sum_k dS_qk k_k is a sum of terms that
// largely cancel, and a single bf16 rounding of dS would leave errors of ~2^-9
// of the terms rather than of the result. A column of dS has no such
// identity, and dK keeps its error well inside the same bound with one
// rounding. MALA_FLAG_FAST_GRAD skips the lo half in dQ as well.
#include <algorithm>
#include <type_traits>

#include "mala_device.h"
#include "mala_internal.h"

namespace mala {
namespace {

constexpr int kBQ = 32;     // query rows per backward decision tile
constexpr int kBK = 16;     // keys per backward decision tile

// ---------------------------------------------------------------- prep
__global__ __launch_bounds__(256) void bwd_prep_kernel(int rows, int d, const bf16* __restrict__ O,
                                                       const bf16* __restrict__ dO,
                                                       float* __restrict__ Dq, uint32_t* bits,
                                                       size_t nbits_words, int32_t* kept,
                                                       size_t nkept, int8_t* mask, size_t nmask) {
  const size_t gtid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t nthr = (size_t)gridDim.x * blockDim.x;
  for (size_t i = gtid; i < nbits_words; i += nthr) bits[i] = 0u;
  if (kept != nullptr)
    for (size_t i = gtid; i < nkept; i += nthr) kept[i] = 0;
  if (mask != nullptr)
    for (size_t i = gtid; i < nmask; i += nthr) mask[i] = -1;   // not a legal tile
  // 16-byte chunks: d / 8 consecutive lanes per row (a power of two that
  // divides 64, so a row never straddles two waves' ranges)
  const int lane = threadIdx.x & 63;
  const int cpr = d >> 3;
  const size_t nchunks = (size_t)rows * cpr;
  const size_t wave = gtid >> 6, nwave = nthr >> 6;
  for (size_t base = wave * 64; base < nchunks; base += nwave * 64) {
    const size_t c = base + lane;
    float acc = 0.f;
    if (c < nchunks) {
      const bf16x8 o = load16(O + 8 * c), g = load16(dO + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
    }
    for (int off = cpr >> 1; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (c < nchunks && (lane & (cpr - 1)) == 0) Dq[c / cpr] = acc;
  }
}

// ---------------------------------------------------------------- dK, dV
// A workgroup owns 128 keys of one KV head: 8 waves x 16 keys. Each wave keeps
// its K and V rows in registers as the B operands of S = Q K^T and
// dP = dO V^T (16x16x32 MFMA) and accumulates dK^T, dV^T (64 registers).
// The query side streams through LDS in 64-row steps (one barrier each): Q and
// dO rows, double-buffered; their transposes, the A operands of dK^T = Q^T dS
// and dV^T = dO^T P, come from the same row-major tiles through transposing
// LDS reads. A step is two 32-row halves, and one backward decision covers a
// half: 32 query rows x the wave's 16 keys. The 8 waves' decisions of a half
// form one byte of the decision bit rows (the workgroup's 8 consecutive
// 16-key columns); it is gathered in LDS and written with one plain store by
// the workgroup that owns it.
//
// Row layout at D = 128. The default walk (kSwz) keeps unpadded 256-byte
// rows with 16-byte chunk c of row r at chunk c xor f(r mod 16),
// f(r) = r xor (2r mod 16): the 16-byte row reads and the transposing reads
// of the 16x16x32 operand layouts both run at the conflict-free rate, and on
// inputs where most tiles skip the walk runs about 4% faster than with padded
// rows (gradients bit-identical). The gated walks keep padded rows of 176
// (also conflict-free): the swizzle's per-lane chunk offsets cost them 11
// registers and 1-2%.
template <int D, bool kGated = false>
struct alignas(16) DkdvSmem {
  static constexpr bool kSwz = D == 128 && !kGated;
  static constexpr int kStride = kSwz ? 128 : (D == 128 ? 176 : 80);
  // physical 16-byte chunk of chunk c in row r
  static __device__ __forceinline__ int ch(int r, int c) {
    if constexpr (kSwz) {
      r &= 15;
      return c ^ (r ^ ((2 * r) & 15));
    }
    return c;
  }
  bf16 q[2][64][kStride];
  bf16 dout[2][64][kStride];
  alignas(16) float z2[2][64];  // z_q * log2 e
  float u2[2][64];              // z_q * log2 e + log2(tau / L_q): skip iff s2 < u2 everywhere
  float dd[2][64];              // -D_q (the dP accumulators start from it)
  uint32_t keep[2];             // [buf] bit w / 8 + w: wave w kept its first / second half
};

// Gated walks (MALA_FLAG_GATE_PASS): a key block whose KV head's group of
// query heads keeps at most kGroupWalkPairs (head, 64-row step) pairs is
// walked by one workgroup over all the group's heads, which writes dK and dV
// directly; a block with more is walked per head in parallel, into fp32
// partials that the finalize kernel sums. Both kernels take the choice from
// the same count of the decision bits.
constexpr int kGroupWalkPairs = 32;

// Kept (query head, 64-row step) pairs of KV head (b, hk)'s group for key
// block J (128 keys): a pair is kept when either 32-row half of the step
// holds a kept tile of the block, i.e. byte J of bit row 2 i or 2 i + 1 is
// nonzero. The workgroup's waves add their counts through red (one int per
// wave); every thread returns the total.
__device__ int group_kept_pairs(const Shape& s, const uint8_t* bit_bytes, int b, int hk, int J,
                                int i_start, int* red) {
  const int tr32 = (s.nq + kBQ - 1) / kBQ, tr64 = (s.nq + 63) / 64;
  const uint32_t rstride = (uint32_t)(((s.nk + kBK - 1) / kBK + 31) / 32) * 4u;
  const int nsteps = tr64 - i_start;
  const int pairs = s.group * nsteps;
  const uint32_t span = (uint32_t)(s.group * tr32) * rstride;   // 0 without query rows
  const auto rs = make_rsrc(bit_bytes + ((size_t)b * s.hq + (size_t)hk * s.group) * tr32 * rstride + J,
                            span > (uint32_t)J ? span - (uint32_t)J : 0u);
  // four pairs per thread and pass, their loads issued together; a pair
  // past the group reads row 0 and is not counted
  int c = 0;
  const int bd = (int)blockDim.x;
  for (int t0 = (int)threadIdx.x; t0 < pairs; t0 += 4 * bd) {
    uint32_t lo[4], hi[4];
    bool in[4], two[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + u * bd;
      in[u] = t < pairs;
      const int tt = in[u] ? t : 0;
      const int hs = tt / nsteps, i = i_start + tt % nsteps;
      const uint32_t r = (uint32_t)(hs * tr32 + 2 * i);
      lo[u] = __builtin_amdgcn_raw_buffer_load_b8(rs, r * rstride, 0, 0);
      hi[u] = __builtin_amdgcn_raw_buffer_load_b8(rs, (r + 1) * rstride, 0, 0);
      two[u] = 2 * i + 1 < tr32;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) c += in[u] && (lo[u] | (two[u] ? hi[u] : 0u)) != 0u ? 1 : 0;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  int total = 0;
  for (int k = 0; k < (int)(blockDim.x >> 6); ++k) total += red[k];
  __syncthreads();
  return total;
}

// Automatic walk choice (mala_bwd_auto): both walks' kernels are launched
// and a workgroup of the walk not taken returns at once. take: the flag the
// choice kernel wrote (1: the gate-pass walks, 0: the default walk), or
// nullptr outside that mode.
__device__ __forceinline__ bool walk_not_taken(const int32_t* take, int mine) {
  return take != nullptr && __builtin_amdgcn_readfirstlane(*take) != mine;
}

// The choice. counts: the sampled gate's kept and legal 16-key columns per
// workgroup (n_slots pairs); from a sample of at least kMinSampleCols legal
// columns, the gate-pass walks are taken when fewer than 60% were kept.
// Otherwise the forward's counters decide: the gate-pass walks when the
// forward kept fewer than 70% of its legal tiles (fwd_kept: kept tiles per
// (b, h, 32-row block), n entries; legal: the forward's legal tiles, a
// function of the shape counted on the host); they are read only then. One
// workgroup of 1024 threads; each thread issues its loads of a round before
// it adds.
constexpr long long kMinSampleCols = 256;

__device__ __forceinline__ long long block_sum_1024(long long x, long long* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  long long t = 0;
#pragma unroll
  for (int u = 0; u < 16; ++u) t += red[u];
  return t;
}

__global__ __launch_bounds__(1024) void bwd_choose_kernel(const int32_t* __restrict__ fwd_kept,
                                                          long long n, long long legal,
                                                          const uint32_t* __restrict__ counts,
                                                          long long n_slots,
                                                          int32_t* __restrict__ take) {
  __shared__ long long red[16];
  long long sk = 0, sl = 0;
  for (long long x0 = 0; x0 < n_slots; x0 += 4 * 1024) {
    uint32_t a[4], c[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const long long x = x0 + u * 1024 + threadIdx.x;
      a[u] = x < n_slots ? counts[2 * x] : 0u;
      c[u] = x < n_slots ? counts[2 * x + 1] : 0u;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sk += a[u];
      sl += c[u];
    }
  }
  sk = block_sum_1024(sk, red);
  sl = block_sum_1024(sl, red);
  if (sl >= kMinSampleCols) {
    if (threadIdx.x == 0) *take = 10 * sk < 6 * sl ? 1 : 0;
    return;
  }
  long long kept = 0;
  for (long long x0 = 0; x0 < n; x0 += 8 * 1024) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const long long x = x0 + u * 1024 + threadIdx.x;
      v[u] = x < n ? fwd_kept[x] : 0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) kept += v[u];
  }
  kept = block_sum_1024(kept, red);
  if (threadIdx.x == 0) *take = 10 * kept < 7 * legal ? 1 : 0;
}

// First 64-row step with a legal entry for the first key of 128-key block J.
__device__ __forceinline__ int block_first_step(const Shape& s, int J) {
  if (!s.causal) return 0;
  const int need = J * 128 - s.offset;
  return need <= 0 ? 0 : need / 64;
}

// The gated walks' plan: kept pairs of every (batch, KV head, 128-key block),
// one workgroup (one wave) each; plan[(b * Hkv + hk) * n_kb + J].
__global__ __launch_bounds__(64) void bwd_plan_kernel(Shape s, const uint32_t* __restrict__ bits,
                                                      int32_t* __restrict__ plan,
                                                      const int32_t* __restrict__ take) {
  if (walk_not_taken(take, 1)) return;
  __shared__ int red[1];
  const int n_kb = (s.nk + 127) / 128;
  const int J = (int)(blockIdx.x % n_kb), bkv = (int)(blockIdx.x / n_kb);
  const int c = group_kept_pairs(s, reinterpret_cast<const uint8_t*>(bits), bkv / s.hkv,
                                 bkv % s.hkv, J, block_first_step(s, J), red);
  if (threadIdx.x == 0) plan[blockIdx.x] = c;
}

template <int D, bool kGated>
__global__ __launch_bounds__(512, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkdv_kernel(
    Shape s, const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dq,
    bf16* __restrict__ dK, bf16* __restrict__ dV, uint32_t* __restrict__ bits,
    int8_t* __restrict__ mask, float* __restrict__ part, const int32_t* __restrict__ plan,
    const int32_t* __restrict__ take) {
  if (walk_not_taken(take, kGated ? 1 : 0)) return;
  using Smem = DkdvSmem<D, kGated>;
  __shared__ Smem sm;
  constexpr int ST = Smem::kStride;
  constexpr int KS = D / 32;      // 32-wide k-steps over d (16x16x32 MFMA)
  constexpr int DB = D / 16;      // 16-row blocks of dK^T / dV^T
  constexpr int CPR = D / 8;      // 16-byte chunks per row
  constexpr int RPP = 512 / CPR;  // staged rows per pass of the 512 threads
  constexpr int NPASS = 64 / RPP;

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int bk_count = s.batch * s.hkv;
  // workgroups per key block: one, walking the whole group; or (gated) one
  // per query head, each walking its head into fp32 partials that the
  // finalize kernel sums (heavy blocks), or one of them walking the group
  // (light blocks)
  const int nsub = kGated ? s.group : 1;
  const int J = (int)(blockIdx.x / (bk_count * nsub));  // key block (0 = longest)
  const int rem = (int)(blockIdx.x % (bk_count * nsub));
  const int bkv = rem / nsub, hsub = rem % nsub;
  const int b = bkv / s.hkv, hk = bkv % s.hkv;
  // gated: a block walked per head (into partials) or by one workgroup over
  // the group; which workgroup takes a group walk rotates with the block, so
  // that the walking ones spread over the XCDs (the dispatcher deals
  // consecutive workgroups to consecutive XCDs)
  bool gsplit = false;
  if constexpr (kGated) {
    const int n_kb = (s.nk + 127) / 128;
    gsplit = plan[bkv * n_kb + J] > kGroupWalkPairs;
    if (!gsplit && hsub != (J + bkv) % s.group) return;
  }
  const int kw0 = J * 128 + w * kBK;                   // this wave's first key
  const size_t krow0 = ((size_t)b * s.hkv + hk) * (size_t)s.nk;
  const int tr32 = (s.nq + kBQ - 1) / kBQ;
  const int tr64 = (s.nq + 63) / 64;
  const int tc16 = (s.nk + kBK - 1) / kBK;
  const int words = (tc16 + 31) / 32;
  const int key = kw0 + l16;
  uint8_t* const bit_bytes = reinterpret_cast<uint8_t*>(bits);

  // K and V rows of this wave as B operands: lane (key l16, group g) holds
  // row[32 t + 8 g .. + 7]; rows past N_k read as zeros.
  bf16x8 kr[KS], vr[KS];
  {
    const auto krs = make_rsrc(K + krow0 * D, (uint32_t)((size_t)s.nk * D * 2));
    const auto vrs = make_rsrc(V + krow0 * D, (uint32_t)((size_t)s.nk * D * 2));
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      kr[t] = buf_load16(krs, (uint32_t)(key * D + 32 * t + 8 * g) * 2);
      vr[t] = buf_load16(vrs, (uint32_t)(key * D + 32 * t + 8 * g) * 2);
    }
  }
  f32x4 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) { dk[db][r] = 0.f; dv[db][r] = 0.f; }

  const int i_start = block_first_step(s, J);   // first 64-row step with a legal entry
  const int total = s.group * (tr64 - i_start);   // (head, 64-row step) pairs of the default walk

  // staging: 64 rows x CPR chunks of Q and of dO, NPASS chunks each per thread.
  // The buffer resources span one query head (rows past N_q read as zeros)
  // and are rebuilt only when the walk moves to the next head.
  const int srow = tid / CPR, sc = tid % CPR;
  const uint32_t toff = (uint32_t)(srow * D + 8 * sc) * 2;   // this thread's chunk in a step
  const uint32_t head_bytes = (uint32_t)((size_t)s.nq * D * 2);
  auto head_row0 = [&](int h) { return ((size_t)b * s.hq + h) * (size_t)s.nq; };
  bf16x8 qreg[NPASS], oreg[NPASS];
  float zreg = 0.f, dreg = 0.f;
  auto load_step = [&](__amdgpu_buffer_rsrc_t qrs, __amdgpu_buffer_rsrc_t ors, int h, int i) {
    const uint32_t off0 = toff + (uint32_t)(i * 64) * (uint32_t)(D * 2);
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const uint32_t off = off0 + (uint32_t)(p * RPP * D * 2);
      qreg[p] = buf_load16(qrs, off);
      oreg[p] = buf_load16(ors, off);
    }
    if (tid < 64) {
      const size_t qrow0 = head_row0(h);
      const int q = i * 64 + tid;
      zreg = q < s.nq ? LSE[qrow0 + q] : 0.f;
      dreg = q < s.nq ? Dq[qrow0 + q] : 0.f;
    }
  };
  auto store_step = [&](int buf, int i) {
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      store16(&sm.q[buf][p * RPP + srow][8 * Smem::ch(p * RPP + srow, sc)], qreg[p]);
      store16(&sm.dout[buf][p * RPP + srow][8 * Smem::ch(p * RPP + srow, sc)], oreg[p]);
    }
    if (tid < 64) {
      const int q = i * 64 + tid;
      const float L = s.causal ? (float)(q + s.offset + 1) : (float)s.nk;
      const float z2 = zreg * 1.4426950408889634f;
      sm.z2[buf][tid] = z2;
      sm.u2[buf][tid] = z2 + (s.log2_tau - fast_log2(L));
      sm.dd[buf][tid] = -dreg;
    }
  };
  // the previous step's decision word (byte 0: first half, byte 1: second
  // half) -> bit rows (b, h, 2 i + half), byte J
  auto flush_keep = [&](int buf, int h, int i) {
    if (tid < 2 && 2 * i + tid < tr32) {
      const size_t bh = (size_t)b * s.hq + h;
      bit_bytes[(bh * tr32 + 2 * i + tid) * (size_t)words * 4 + J] = (uint8_t)(sm.keep[buf] >> (8 * tid));
      if (tid == 0) sm.keep[buf] = 0u;
    }
  };

  // the post-score path of one kept 32 x 16 tile (rows 32 half .. + 31 of
  // the step in LDS buffer bf; s0, s1: its scores, illegal entries -inf):
  // P, dP, dS and the dV, dK products
  // transposing read of this lane's 8 bytes of a 32-row half (tile: its
  // first row): row r0 + l16 / 4, columns 16 db + 4 (l16 mod 4) .. + 3
  auto trd = [&](const bf16* tile, int r0, int db) {
    const int r = r0 + (l16 >> 2), c = 2 * db + ((l16 & 3) >> 1);
    return lds_read_tr_at(tile + r * ST + 8 * Smem::ch(r, c) + 4 * (l16 & 1));
  };
  auto kept_tile = [&](int bf, int half, f32x4 s0, f32x4 s1) {
    const int lr = 32 * half;                        // first row of the half in the LDS tile
    f32x4 sh[2] = {s0, s1};
    // Row-major dO rows (A operand of dP): row 16 qb + l16, columns 32 t + 8 g .. + 7.
    bf16x8 orow[KS][2];
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) orow[t][qb] = load16(&sm.dout[bf][lr + 16 * qb + l16][8 * Smem::ch(l16, 4 * t + g)]);
    // dO^T and Q^T, the A operands of dV^T = dO^T P and dK^T = Q^T dS,
    // through transposing reads: element e < 4 is query row 4g + e,
    // e >= 4 is row 16 + 4g + (e - 4), for column 16 db + l16.
    bf16x8 ocol[DB], qcol[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
      ocol[db] = cat8(trd(&sm.dout[bf][lr][0], 4 * g, db), trd(&sm.dout[bf][lr][0], 16 + 4 * g, db));
#pragma unroll
    for (int db = 0; db < DB; ++db)
      qcol[db] = cat8(trd(&sm.q[bf][lr][0], 4 * g, db), trd(&sm.q[bf][lr][0], 16 + 4 * g, db));
    // ---- P = exp(S - z) (B operand over the 32 query rows, in the row
    // order of the transposing reads); it does not wait for dP
    bf16x8 pb, dsb;
    float pv[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const f32x4 z = *reinterpret_cast<const f32x4*>(&sm.z2[bf][lr + 16 * qb + 4 * g]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[qb][r] = fast_exp2(fmaf(sh[qb][r], s.scale_log2, -z[r]));
        pb[4 * qb + r] = (bf16)pv[qb][r];
      }
    }
    // ---- dP - D = dO V^T - D (the accumulators start at -D) and
    // dV^T += dO^T P, independent products
    f32x4 dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) dp[qb] = *reinterpret_cast<const f32x4*>(&sm.dd[bf][lr + 16 * qb + 4 * g]);
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) dp[qb] = mfma16(orow[t][qb], vr[t], dp[qb]);
#pragma unroll
    for (int db = 0; db < DB; ++db) dv[db] = mfma16(ocol[db], pb, dv[db]);
    // ---- dS = P o (dP - D), then dK^T += Q^T dS
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 4; ++r) dsb[4 * qb + r] = (bf16)(pv[qb][r] * dp[qb][r]);
#pragma unroll
    for (int db = 0; db < DB; ++db) dk[db] = mfma16(qcol[db], dsb, dk[db]);
  };

  // Steps on which both halves hold only legal entries for this wave's keys
  // (all 64 rows below N_q, all 16 keys below N_k and, when causal, on or
  // below the diagonal) skip the legality and boundary tests.
  const bool keys_in = kw0 + kBK <= s.nk;
  int i_lo = 0;
  if (s.causal) {
    const int need = kw0 + kBK - 1 - s.offset;
    i_lo = need <= 0 ? 0 : (need + 63) / 64;
  }
  const int i_hi = s.nq / 64;

  if constexpr (!kGated) {
  if (tid < 2) sm.keep[tid] = 0u;
  int h = hk * s.group, i = i_start;                   // current step
  int hl = h;                                          // head of the staging resources
  auto lq = make_rsrc(Q + head_row0(h) * D, head_bytes);
  auto lo = make_rsrc(dO + head_row0(h) * D, head_bytes);
  if (total > 0) {
    load_step(lq, lo, h, i);
    store_step(0, i);
  }
#pragma unroll
  for (int t = 0; t < KS; ++t) {
    settle(kr[t]);
    settle(vr[t]);
  }
  __syncthreads();

  int prev_h = 0, prev_i = -1;
  for (int it = 0; it < total; ++it) {
    const int buf = it & 1;
    int hn = h, in = i + 1;                            // next step
    if (in == tr64) { in = i_start; ++hn; }
    const bool more = it + 1 < total;
    if (hn != hl) {
      // the next head, or past the group after the last step: then a
      // zero-sized range, so the staging loads return zeros and touch nothing
      hl = hn;
      lq = make_rsrc(Q + head_row0(more ? hn : h) * D, more ? head_bytes : 0u);
      lo = make_rsrc(dO + head_row0(more ? hn : h) * D, more ? head_bytes : 0u);
    }
    // the decision store goes out before the staging loads: the loads' wait
    // at the end of the step then covers it, instead of the next step's
    // loads waiting for it
    if (prev_i >= 0) flush_keep(buf ^ 1, prev_h, prev_i);
    // unconditional, so that the wait for these loads at the end of the step
    // is the only one (after the last step they stage zeros into the idle buffer)
    load_step(lq, lo, more ? hn : h, more ? in : i);
    bool legal[2] = {true, true}, bnd[2] = {false, false};
    if (!(keys_in && i >= i_lo && i < i_hi)) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int r0 = i * 64 + 32 * half;
        legal[half] = r0 < s.nq && kw0 < s.nk && (!s.causal || kw0 <= min(r0 + 31, s.nq - 1) + s.offset);
        bnd[half] = (r0 + 32 > s.nq) || (kw0 + kBK > s.nk) || (s.causal && kw0 + kBK - 1 > r0 + s.offset);
      }
    }
    // ---- S = Q K^T over the whole 64-row step and both halves' gates come
    // first: a skipped half then costs its Q reads and score products only,
    // and the products of the two halves overlap.
    if (legal[0] || legal[1]) {
      // lane (key l16, group g), regs = queries 16 qb + 4 g + r of the step
      f32x4 sacc[4], uu[4];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        uu[qb] = *reinterpret_cast<const f32x4*>(&sm.u2[buf][16 * qb + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[qb][r] = 0.f;
      }
      {
        bf16x8 qrow[KS][4];
#pragma unroll
        for (int t = 0; t < KS; ++t)
#pragma unroll
          for (int qb = 0; qb < 4; ++qb) qrow[t][qb] = load16(&sm.q[buf][16 * qb + l16][8 * Smem::ch(l16, 4 * t + g)]);
#pragma unroll
        for (int t = 0; t < KS; ++t)
#pragma unroll
          for (int qb = 0; qb < 4; ++qb) sacc[qb] = mfma16(qrow[t][qb], kr[t], sacc[qb]);
      }
      // ---- offline gate, Eq. 4, per half: skip iff S - z < log(tau / L) on
      // every legal entry of its 32 x 16 tile
      uint32_t kept_halves = 0u;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if (!legal[half]) continue;
        float x = kNegInf;
        if (!bnd[half]) {                              // wave-uniform: every entry legal
#pragma unroll
          for (int qh = 0; qh < 2; ++qh)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              x = fmaxf(x, fmaf(sacc[2 * half + qh][r], s.scale_log2, -uu[2 * half + qh][r]));
        } else {
          const int r0 = i * 64 + 32 * half;
#pragma unroll
          for (int qh = 0; qh < 2; ++qh)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int qb = 2 * half + qh;
              const int q = r0 + 16 * qh + 4 * g + r;
              const bool ok = (q < s.nq) & (key < s.nk) & ((key <= q + s.offset) | (s.causal == 0));
              sacc[qb][r] = ok ? sacc[qb][r] : kNegInf;   // P = 0 on illegal entries
              x = fmaxf(x, ok ? fmaf(sacc[qb][r], s.scale_log2, -uu[qb][r]) : kNegInf);
            }
        }
        if (__builtin_amdgcn_ballot_w64(x >= 0.f) != 0) kept_halves |= 1u << half;
      }
      if (kept_halves != 0u && lane == 0)
        atomicOr(&sm.keep[buf], ((kept_halves & 1u) << w) | ((kept_halves >> 1) << (8 + w)));
      if (mask != nullptr && lane == 0) {
        const size_t bh = (size_t)b * s.hq + h;
#pragma unroll
        for (int half = 0; half < 2; ++half)
          if (legal[half])
            mask[(bh * tr32 + 2 * i + half) * tc16 + kw0 / kBK] = (int8_t)((kept_halves >> half) & 1u);
      }
      if (kept_halves & 1u) kept_tile(buf, 0, sacc[0], sacc[1]);
      if (kept_halves & 2u) kept_tile(buf, 1, sacc[2], sacc[3]);
    }
    prev_h = h;
    prev_i = i;
    store_step(buf ^ 1, more ? in : i);
    h = hn;
    i = in;
    __syncthreads();
  }
  if (prev_i >= 0) flush_keep((total - 1) & 1, prev_h, prev_i);
  } else {
    // ---- decisions from the gate pass: only steps that hold a kept tile of
    // this workgroup are staged; a wave forms scores only for its kept tiles.
    // A light block is one walk over the group's heads, a heavy one a walk
    // per head (kGroupWalkPairs). Step t of a walk over nh heads from h0 is
    // head h0 + t / nsteps, row step i_start + t % nsteps.
    const int nsteps = tr64 - i_start;
    const int h0 = hk * s.group + (gsplit ? hsub : 0);
    const int nh = gsplit ? 1 : s.group;
    const int tot = nh * nsteps;
    // decision bytes J of the walk's bit rows; bytes past the last row read 0
    const uint32_t rstride = (uint32_t)words * 4u;
    const uint32_t span = (uint32_t)(nh * tr32) * rstride;        // 0 without query rows
    const auto drs = make_rsrc(bit_bytes + ((size_t)b * s.hq + h0) * tr32 * rstride + J,
                               span > (uint32_t)J ? span - (uint32_t)J : 0u);
    // look-ahead: the bytes of 512 steps are fetched at once; lane k of
    // window x holds the two bytes (rows 2 i, 2 i + 1) of step
    // la_base + 64 x + k, so a walk waits on the bit rows once per 512 steps
    uint32_t la_val[8];
    int la_base = -512;
    auto la_fill = [&](int t0) {
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int t = t0 + 64 * x + lane;
        const int hs = t / nsteps, i = i_start + t % nsteps;
        const uint32_t r = (uint32_t)(hs * tr32 + 2 * i);
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b8(drs, r * rstride, 0, 0);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b8(drs, (r + 1) * rstride, 0, 0);
        la_val[x] = lo | (2 * i + 1 < tr32 ? hi << 8 : 0u);
      }
      la_base = t0;
    };
    // the first step at or after t with a kept tile (tot if none) and its bytes
    auto next_kept = [&](int t, uint32_t& v) {
      while (t < tot) {
        if (t >= la_base + 512) la_fill(t);
        const int off = t - la_base, x = off >> 6, bit = off & 63;
        uint32_t sel = la_val[0];
#pragma unroll
        for (int k = 1; k < 8; ++k) sel = x == k ? la_val[k] : sel;
        const uint64_t m = __builtin_amdgcn_ballot_w64(sel != 0u) >> bit;
        if (m != 0u) {
          const int adv = (int)__builtin_ctzll(m);
          v = __builtin_amdgcn_readlane(sel, bit + adv);
          return t + adv < tot ? t + adv : tot;
        }
        t = la_base + 64 * (x + 1);
      }
      v = 0u;
      return tot;
    };

    // a step's Q and dO rows, z and D, in registers: two sets, so that the
    // loads of the step after next are in flight while a step is processed
    // (a sparse step is short against the memory latency); z and D through
    // bounded loads that every wave issues, so no load sits in a branch
    struct StepRegs {
      bf16x8 q[NPASS], o[NPASS];
      float z, d;
    };
    // step t of the walk -> (head, row step)
    auto pair_of = [&](int t, int& hh, int& i) {
      const int hs = t / nsteps;
      hh = h0 + hs;
      i = i_start + t - hs * nsteps;
    };
    auto gload = [&](StepRegs& R, int hh, int i) {
      const auto lq = make_rsrc(Q + head_row0(hh) * D, head_bytes);
      const auto lo = make_rsrc(dO + head_row0(hh) * D, head_bytes);
      const auto lz = make_rsrc(LSE + head_row0(hh), (uint32_t)s.nq * 4u);
      const auto ld = make_rsrc(Dq + head_row0(hh), (uint32_t)s.nq * 4u);
      const uint32_t off0 = toff + (uint32_t)(i * 64) * (uint32_t)(D * 2);
#pragma unroll
      for (int p = 0; p < NPASS; ++p) {
        const uint32_t off = off0 + (uint32_t)(p * RPP * D * 2);
        R.q[p] = buf_load16(lq, off);
        R.o[p] = buf_load16(lo, off);
      }
      const uint32_t roff = (uint32_t)(i * 64 + lane) * 4u;
      R.z = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lz, roff, 0, 0));
      R.d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ld, roff, 0, 0));
    };
    auto gstore = [&](const StepRegs& R, int bf) {
#pragma unroll
      for (int p = 0; p < NPASS; ++p) {
        store16(&sm.q[bf][p * RPP + srow][8 * Smem::ch(p * RPP + srow, sc)], R.q[p]);
        store16(&sm.dout[bf][p * RPP + srow][8 * Smem::ch(p * RPP + srow, sc)], R.o[p]);
      }
      if (tid < 64) {
        sm.z2[bf][tid] = R.z * 1.4426950408889634f;
        sm.dd[bf][tid] = -R.d;
      }
    };
    // this wave's kept halves of step i (decision bytes v), staged in bf
    auto step_tiles = [&](int bf, int i, uint32_t v) {
      const uint32_t mine = ((v >> w) & 1u) | (((v >> (8 + w)) & 1u) << 1);
      if (mine == 0u) return;
      bool bnd[2] = {false, false};
      if (!(keys_in && i >= i_lo && i < i_hi)) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int r0 = i * 64 + 32 * half;
          bnd[half] = (r0 + 32 > s.nq) || (kw0 + kBK > s.nk) || (s.causal && kw0 + kBK - 1 > r0 + s.offset);
        }
      }
      f32x4 sacc[4];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[qb][r] = 0.f;
      {
        bf16x8 qrow[KS][4];
#pragma unroll
        for (int k = 0; k < KS; ++k)
#pragma unroll
          for (int qb = 0; qb < 4; ++qb) qrow[k][qb] = load16(&sm.q[bf][16 * qb + l16][8 * Smem::ch(l16, 4 * k + g)]);
#pragma unroll
        for (int k = 0; k < KS; ++k)
#pragma unroll
          for (int qb = 0; qb < 4; ++qb) sacc[qb] = mfma16(qrow[k][qb], kr[k], sacc[qb]);
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if (!bnd[half]) continue;
        const int r0 = i * 64 + 32 * half;
#pragma unroll
        for (int qh = 0; qh < 2; ++qh)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int q = r0 + 16 * qh + 4 * g + r;
            const bool ok = (q < s.nq) & (key < s.nk) & ((key <= q + s.offset) | (s.causal == 0));
            sacc[2 * half + qh][r] = ok ? sacc[2 * half + qh][r] : kNegInf;   // P = 0 there
          }
      }
      if (mine & 1u) kept_tile(bf, 0, sacc[0], sacc[1]);
      if (mine & 2u) kept_tile(bf, 1, sacc[2], sacc[3]);
    };

    // t: the step in LDS buffer buf; tn: the next kept step, in flight in
    // one register set; tnn: the one after, loaded into the other set while
    // t is processed. Past the last kept step the loads repeat a staged step.
    StepRegs ra, rb;
    uint32_t v = 0u, vn = 0u, vnn = 0u;
    int t = next_kept(0, v);
    int h = h0, i = i_start;
    if (t < tot) pair_of(t, h, i);
    gload(ra, h, i);
    gstore(ra, 0);
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      settle(kr[k]);
      settle(vr[k]);
    }
    int tn = t < tot ? next_kept(t + 1, vn) : tot;
    int hn = h, in = i;
    if (tn < tot) pair_of(tn, hn, in);
    gload(ra, hn, in);
    __syncthreads();
    int buf = 0;
    while (t < tot) {
      int tnn = tn < tot ? next_kept(tn + 1, vnn) : tot;
      int hnn = hn, inn = in;
      if (tnn < tot) pair_of(tnn, hnn, inn);
      gload(rb, hnn, inn);
      step_tiles(buf, i, v);
      gstore(ra, buf ^ 1);
      __syncthreads();
      buf ^= 1;
      t = tn; i = in; v = vn;
      tn = tnn; hn = hnn; in = inn; vn = vnn;
      if (t >= tot) break;
      tnn = tn < tot ? next_kept(tn + 1, vnn) : tot;
      hnn = hn;
      inn = in;
      if (tnn < tot) pair_of(tnn, hnn, inn);
      gload(ra, hnn, inn);
      step_tiles(buf, i, v);
      gstore(rb, buf ^ 1);
      __syncthreads();
      buf ^= 1;
      t = tn; i = in; v = vn;
      tn = tnn; hn = hnn; in = inn; vn = vnn;
    }
  }

  // ---- store dK = scale * sum dS^T Q and dV (summed over the group's heads):
  // lane (key l16, group g) holds d = 16 db + 4 g + r
  if (key >= s.nk) return;
  if (kGated && gsplit) {
    // this walk's head only: fp32 partials [2][B][Hq][N_k][D] (dK unscaled)
    const size_t prow = ((size_t)b * s.hq + hk * s.group + hsub) * (size_t)s.nk + key;
    float* pk = part + prow * D;
    float* pv = part + ((size_t)s.batch * s.hq * s.nk + prow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      *reinterpret_cast<f32x4*>(pk + 16 * db + 4 * g) = dk[db];
      *reinterpret_cast<f32x4*>(pv + 16 * db + 4 * g) = dv[db];
    }
    return;
  }
  bf16* dkr = dK + (krow0 + key) * D;
  bf16* dvr = dV + (krow0 + key) * D;
  const float sc_nat = s.scale_log2 * 0.69314718055994531f;   // softmax scale
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    bf16x4 a = {(bf16)(dk[db][0] * sc_nat), (bf16)(dk[db][1] * sc_nat),
                (bf16)(dk[db][2] * sc_nat), (bf16)(dk[db][3] * sc_nat)};
    bf16x4 c = {(bf16)dv[db][0], (bf16)dv[db][1], (bf16)dv[db][2], (bf16)dv[db][3]};
    *reinterpret_cast<bf16x4*>(dkr + 16 * db + 4 * g) = a;
    *reinterpret_cast<bf16x4*>(dvr + 16 * db + 4 * g) = c;
  }
}

// The gated walks' partials of the key blocks walked per head, summed over
// each KV head's group of query heads (in head order, so the result does not
// depend on scheduling): dK = scale * sum, dV = sum, in bf16. A workgroup per
// (batch, KV head, 128-key block); blocks walked as one group are already
// written.
__global__ __launch_bounds__(256) void bwd_dkdv_finalize_kernel(Shape s, const float* __restrict__ part,
                                                                const int32_t* __restrict__ plan,
                                                                bf16* __restrict__ dK,
                                                                bf16* __restrict__ dV,
                                                                const int32_t* __restrict__ take) {
  if (walk_not_taken(take, 1)) return;
  const int n_kb = (s.nk + 127) / 128;
  const int J = (int)(blockIdx.x % n_kb);
  const int bkv = (int)(blockIdx.x / n_kb);
  const int b = bkv / s.hkv, hk = bkv % s.hkv;
  if (plan[blockIdx.x] <= kGroupWalkPairs) return;
  const int k0 = J * 128, nkeys = min(128, s.nk - k0);
  const size_t per_head = (size_t)s.nk * s.d;                 // floats of one head's partial
  const size_t dv_off = (size_t)s.batch * s.hq * per_head;
  const size_t p0 = ((size_t)b * s.hq + (size_t)hk * s.group) * per_head + (size_t)k0 * s.d;
  const size_t o0 = ((size_t)b * s.hkv + hk) * per_head + (size_t)k0 * s.d;
  const float sc_nat = s.scale_log2 * 0.69314718055994531f;
  for (int c = (int)threadIdx.x; c < nkeys * s.d / 4; c += (int)blockDim.x) {
    const size_t e = 4 * (size_t)c;
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, v = {0.f, 0.f, 0.f, 0.f};
    for (int hs = 0; hs < s.group; ++hs) {
      a += *reinterpret_cast<const f32x4*>(part + p0 + hs * per_head + e);
      v += *reinterpret_cast<const f32x4*>(part + dv_off + p0 + hs * per_head + e);
    }
    const bf16x4 ka = {(bf16)(a[0] * sc_nat), (bf16)(a[1] * sc_nat), (bf16)(a[2] * sc_nat),
                       (bf16)(a[3] * sc_nat)};
    const bf16x4 va = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    *reinterpret_cast<bf16x4*>(dK + o0 + e) = ka;
    *reinterpret_cast<bf16x4*>(dV + o0 + e) = va;
  }
}

// ---------------------------------------------------------------- gate pass
// For inputs on which few tiles are kept (MALA_FLAG_GATE_PASS): the offline
// gate (Eq. 4) of every legal 32 x 16 backward tile, taken in a query-major
// pass before dK/dV, so that dK/dV stages and processes only the steps that
// hold a kept tile (a skipped tile then costs no dO load, App. A.1). Every
// legal score is still formed, here. The layout is the forward's: a
// workgroup owns 256 query rows of one (batch, query head), wave w rows
// [32 w, 32 w + 32), one backward decision row; K tiles of 64 keys are
// double-buffered in LDS and shared by the 8 waves; S^T = K Q^T with the
// 32x32x16 MFMA and Q^T in registers, so every lane owns one query row and
// compares against its own z_q. The decisions of the wave's row go out as
// whole 32-bit words of the bit rows, one plain store each.
template <int D>
struct alignas(16) GateSmem {
  bf16 k[2][64][D + 8];   // conflict-free 16-byte row reads (32x32x16 A layout)
};

// kSample (mala_bwd_auto): the same scores and votes on every rowstride-th
// 256-row block (the grid has a workgroup for each of those only) and there
// on the tiles j with j = phase (mod stride), where the phase varies with the
// workgroup; nothing is written but the workgroup's counts of kept and legal
// 16-key columns, to counts[2 blockIdx.x] and counts[2 blockIdx.x + 1].
template <int D, bool kNested, bool kSample = false>
__global__ __launch_bounds__(512, 1) void bwd_gate_kernel(Shape s, const bf16* __restrict__ Q,
                                                          const bf16* __restrict__ K,
                                                          const float* __restrict__ LSE,
                                                          uint32_t* __restrict__ bits,
                                                          int8_t* __restrict__ mask, int n_qb,
                                                          const int8_t* __restrict__ fmask,
                                                          const int32_t* __restrict__ take,
                                                          uint32_t* __restrict__ counts,
                                                          int stride, int rowstride) {
  if (walk_not_taken(take, 1)) return;
  __shared__ GateSmem<D> sm;
  constexpr int KT = D / 16;              // 16-wide k-steps of the QK contraction
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int RPP = 512 / CPR;          // K rows per load pass
  constexpr int KPASS = 64 / RPP;
  static_assert(kFwdBq == 32 && kFwdBk == 64, "a wave's rows and a K tile are one forward tile");

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int bh_count = s.batch * s.hq;
  // longest blocks first
  const int I = n_qb - 1 - (kSample ? rowstride : 1) * (int)(blockIdx.x / bh_count);
  const int bh = xcd_head((int)(blockIdx.x % bh_count), s.batch * s.hkv, s.group);
  const int b = bh / s.hq, h = bh % s.hq, hk = h / s.group;
  const size_t qrow0 = (size_t)bh * (size_t)s.nq;
  const size_t krow0 = ((size_t)b * s.hkv + hk) * (size_t)s.nk;
  const int tr32 = (s.nq + kBQ - 1) / kBQ;
  const int tc16 = (s.nk + kBK - 1) / kBK;
  const int words = (tc16 + 31) / 32;

  const int q0 = I * 256 + 32 * w;
  const bool active = q0 < s.nq;
  auto top_tile = [&](int last_row) {
    const int lastkey = s.causal ? min(last_row + s.offset, s.nk - 1) : s.nk - 1;
    return lastkey / 64;
  };
  const int top_b = top_tile(min(I * 256 + 255, s.nq - 1));
  const int top_w = active ? top_tile(min(q0 + 31, s.nq - 1)) : -1;
  const size_t brow = (size_t)bh * tr32 + (active ? q0 / kBQ : 0);   // this wave's bit row

  // ---- the tiles to score. By default every legal tile. Nested (Sec. 2.2):
  // a tile the forward skipped also meets the backward skip condition, so
  // only the forward's kept tiles are scored; the forward's decision block
  // r of the workgroup is exactly wave r's 32 rows, and its tile j is key
  // tile j here. The walk visits the tiles some wave's forward row kept, in
  // descending order, through a 64-tile window of the workgroup's 8 mask
  // rows held as ballots: bit i of `la_any` is tile la_base - i kept by some
  // row, of `la_own` kept by this wave's row.
  const int ftr = (s.nq + kFwdBq - 1) / kFwdBq, ftc = (s.nk + kFwdBk - 1) / kFwdBk;
  const int8_t* frow = kNested ? fmask + ((size_t)bh * ftr + 8 * I) * ftc : nullptr;
  const int nfr = min(8, ftr - 8 * I);     // forward rows of the workgroup (>= 1)
  uint64_t la_any = 0u, la_own = 0u;
  int la_base = -1;
  auto la_fill = [&](int base) {
    const int t = base - lane;
    bool any = false, own = false;
    if (t >= 0) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const bool kept = r < nfr && frow[(size_t)r * ftc + t] == 1;
        any = any || kept;
        own = own || (r == w && kept);
      }
    }
    la_any = __builtin_amdgcn_ballot_w64(any);
    la_own = __builtin_amdgcn_ballot_w64(own);
    la_base = base;
  };
  const int phase = (int)((7u * (uint32_t)I + 3u * (uint32_t)bh) % (uint32_t)stride);
  // the highest tile <= j to visit (-1: none) and whether this wave scores it
  auto next_tile = [&](int j, bool& own) -> int {
    if constexpr (kSample) {
      own = true;
      if (j < 0) return -1;
      const int jj = j - ((j - phase) % stride + stride) % stride;
      return jj >= 0 ? jj : -1;
    } else if constexpr (!kNested) {
      own = true;
      return j;
    } else {
      while (j >= 0) {
        if (j > la_base || j < la_base - 63) la_fill(j);
        const int sh = la_base - j;
        const uint64_t m = la_any >> sh;
        if (m != 0u) {
          const int jn = j - (int)__builtin_ctzll(m);
          own = ((la_own >> (la_base - jn)) & 1u) != 0u;
          return jn;
        }
        j = la_base - 64;
      }
      own = false;
      return -1;
    }
  };

  const auto qrs = make_rsrc(Q + qrow0 * D, (uint32_t)((size_t)s.nq * D * 2));
  const auto krs = make_rsrc(K + krow0 * D, (uint32_t)((size_t)s.nk * D * 2));
  // Q^T as the B operand: lane (query l32, half hf) holds Q[q][16t + 8hf .. +7]
  const int q = q0 + l32;
  const bool rvalid = q < s.nq;
  bf16x8 qr[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) qr[t] = buf_load16(qrs, (uint32_t)(q * D + 16 * t + 8 * hf) * 2);
  // the row's threshold in base 2, as dK/dV forms it: skip iff s2 < u2 on
  // every legal entry (u2 = +inf for rows past N_q: never kept)
  float u2 = __builtin_inff();
  if (rvalid) {
    const float L = s.causal ? (float)(q + s.offset + 1) : (float)s.nk;
    u2 = LSE[qrow0 + q] * 1.4426950408889634f + (s.log2_tau - fast_log2(L));
  }
  // the same test on the raw scores: keep iff max S >= u2 / (scale log2 e)
  // over a column's legal entries; the threshold is finite, so a column
  // without a legal entry (max -inf) is never kept, even at tau = 0
  const float thr = fmaxf(u2 / s.scale_log2, -3.402823466e38f);

  // a column is legal for the wave's rows iff its first key is visible to
  // the wave's last row
  auto legal_col = [&](int col) {
    const int kc0 = 16 * col;
    return col < tc16 && kc0 < s.nk &&
           (!s.causal || kc0 <= min(q0 + 31, s.nq - 1) + s.offset);
  };
  if constexpr (kNested) {
    // diagnostic mask: legal columns of the tiles this wave's forward row
    // did not keep are skipped; the walk writes the others
    if (mask != nullptr && active) {
      const int8_t* orow = frow + (size_t)w * ftc;
      for (int col = lane; col < 4 * (top_w + 1); col += 64)
        if (legal_col(col) && orow[col >> 2] != 1) mask[brow * tc16 + col] = 0;
    }
  }

  bf16x8 kreg[KPASS];
  const int kc = tid % CPR, krr = tid / CPR;
  auto load_tile = [&](int j) {
#pragma unroll
    for (int p = 0; p < KPASS; ++p)
      kreg[p] = buf_load16(krs, (uint32_t)((j * 64 + p * RPP + krr) * D + 8 * kc) * 2);
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int p = 0; p < KPASS; ++p) store16(&sm.k[buf][p * RPP + krr][8 * kc], kreg[p]);
  };
  bool own = false;
  int j = top_b >= 0 ? next_tile(top_b, own) : -1;
  if (j >= 0) {
    load_tile(j);
    store_tile(0);
  }
#pragma unroll
  for (int t = 0; t < KT; ++t) settle(qr[t]);
  float thr_s = thr;
  settle(thr_s);
  __syncthreads();

  uint32_t word = 0u;            // decisions of columns 32 (j / 8) .. + 31 of this wave's row
  uint32_t n_kept = 0u, n_legal = 0u;   // kSample: this wave's column counts
  int buf = 0;
  while (j >= 0) {
    bool own_n = false;
    const int jn = j > 0 ? next_tile(j - 1, own_n) : -1;
    if (jn >= 0) load_tile(jn);
    if (active && own && j <= top_w) {
      // ---- S^T[key][query], 64 keys x 32 queries: register r of block kb is
      // key 32 kb + 8 (r / 4) + 4 hf + r % 4
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
      bf16x8 ka[KT][2];
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) ka[t][kb] = load16(&sm.k[buf][32 * kb + l32][16 * t + 8 * hf]);
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sacc[kb] = mfma32(ka[t][kb], qr[t], sacc[kb]);
      const int key0 = j * 64;
      if ((key0 + 64 > s.nk) || (q0 + 32 > s.nq) || (s.causal && key0 + 63 > q0 + s.offset)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
            const bool ok = rvalid && key < s.nk && (!s.causal || key <= q + s.offset);
            if (!ok) sacc[kb][r] = kNegInf;
          }
      }
      // ---- offline gate, Eq. 4, per 16-key column c = keys 16 c .. + 15
      // of the tile: registers 8 (c % 2) .. + 7 of block c / 2
      uint32_t keep4 = 0u;                             // bit c: column c kept
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float x = kNegInf;
#pragma unroll
        for (int r = 0; r < 8; ++r) x = fmaxf(x, sacc[c >> 1][8 * (c & 1) + r]);
        if (__builtin_amdgcn_ballot_w64(x >= thr_s) != 0) keep4 |= 1u << c;
      }
      if constexpr (kSample) {
        // a column without a legal entry is never kept (its scores are -inf)
        n_kept += (uint32_t)__builtin_popcount(keep4);
#pragma unroll
        for (int c = 0; c < 4; ++c) n_legal += legal_col(4 * j + c) ? 1u : 0u;
      }
      word |= keep4 << ((4 * j) & 31);
      if (!kSample && mask != nullptr && lane == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (legal_col(4 * j + c)) mask[brow * tc16 + 4 * j + c] = (int8_t)((keep4 >> c) & 1u);
      }
    }
    // the word of columns 32 (j / 8) .. is complete once the walk leaves it;
    // the bit rows start cleared, so only words with a kept column are written
    if (jn < 0 || (jn >> 3) != (j >> 3)) {
      if (!kSample && active && lane == 0 && word != 0u) bits[brow * words + (j >> 3)] = word;
      word = 0u;
    }
    if (jn >= 0) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    j = jn;
    own = own_n;
  }
  if constexpr (kSample) {
    __shared__ uint32_t cnt[2][8];
    if (lane == 0) {
      cnt[0][w] = n_kept;
      cnt[1][w] = n_legal;
    }
    __syncthreads();
    if (tid < 2) {
      uint32_t t = 0u;
#pragma unroll
      for (int x = 0; x < 8; ++x) t += cnt[tid][x];
      counts[2 * (size_t)blockIdx.x + tid] = t;
    }
  }
}

// d = 128, every legal tile (the gate pass): the walk above with the K tiles
// staged by LDS-DMA loads two tiles ahead in three buffers, as in the forward
// (fwd_bf16.hip): step j reads buffer j % 3, fills the buffer that held tile
// j + 1 with tile j - 2, waits only for tile j - 1's loads and meets the other
// waves at an LDS-only barrier. The walk starts at a tile with j % 3 == 2 (at
// most two past the top, which no wave scores) so that the steps run in the
// fixed buffer order 2, 1, 0. K chunk c of row r sits at c ^ (r % 16), which
// keeps the 16-byte row reads conflict-free.
__global__ __launch_bounds__(512, 1) void bwd_gate_d128_kernel(Shape s, const bf16* __restrict__ Q,
                                                               const bf16* __restrict__ K,
                                                               const float* __restrict__ LSE,
                                                               uint32_t* __restrict__ bits,
                                                               int8_t* __restrict__ mask, int n_qb,
                                                               const int8_t* __restrict__ /*fmask*/,
                                                               const int32_t* __restrict__ take,
                                                               uint32_t* __restrict__ /*counts*/,
                                                               int /*stride*/, int /*rowstride*/) {
  if (walk_not_taken(take, 1)) return;
  constexpr int D = 128;
  constexpr int KT = D / 16;
  constexpr int TILE = 64 * D;
  constexpr uint32_t TILE_BYTES = TILE * 2;
  __shared__ __attribute__((aligned(16))) bf16 k0[TILE], k1[TILE], k2[TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int bh_count = s.batch * s.hq;
  const int I = n_qb - 1 - (int)(blockIdx.x / bh_count);     // longest blocks first
  const int bh = xcd_head((int)(blockIdx.x % bh_count), s.batch * s.hkv, s.group);
  const int b = bh / s.hq, h = bh % s.hq, hk = h / s.group;
  const size_t qrow0 = (size_t)bh * (size_t)s.nq;
  const size_t krow0 = ((size_t)b * s.hkv + hk) * (size_t)s.nk;
  const int tr32 = (s.nq + kBQ - 1) / kBQ;
  const int tc16 = (s.nk + kBK - 1) / kBK;
  const int words = (tc16 + 31) / 32;

  const int q0 = I * 256 + 32 * w;
  const bool active = q0 < s.nq;
  auto top_tile = [&](int last_row) {
    const int lastkey = s.causal ? min(last_row + s.offset, s.nk - 1) : s.nk - 1;
    return lastkey / 64;
  };
  const int top_b = top_tile(min(I * 256 + 255, s.nq - 1));
  const int top_w = active ? top_tile(min(q0 + 31, s.nq - 1)) : -1;
  const size_t brow = (size_t)bh * tr32 + (active ? q0 / kBQ : 0);   // this wave's bit row

  const auto qrs = make_rsrc(Q + qrow0 * D, (uint32_t)((size_t)s.nq * D * 2));
  const auto krs = make_rsrc(K + krow0 * D, (uint32_t)((size_t)s.nk * D * 2));
  const int q = q0 + l32;
  const bool rvalid = q < s.nq;
  bf16x8 qr[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) qr[t] = buf_load16(qrs, (uint32_t)(q * D + 16 * t + 8 * hf) * 2);
  float u2 = __builtin_inff();
  if (rvalid) {
    const float L = s.causal ? (float)(q + s.offset + 1) : (float)s.nk;
    u2 = LSE[qrow0 + q] * 1.4426950408889634f + (s.log2_tau - fast_log2(L));
  }
  const float thr = fmaxf(u2 / s.scale_log2, -3.402823466e38f);
  auto legal_col = [&](int col) {
    const int kc0 = 16 * col;
    return col < tc16 && kc0 < s.nk &&
           (!s.causal || kc0 <= min(q0 + 31, s.nq - 1) + s.offset);
  };

  // DMA: wave w stages rows 8 w .. 8 w + 7 of a tile, four per instruction;
  // lane l fills slot l % 16 of row 8 w + 4 p + l / 16 with global chunk
  // (l % 16) ^ (row % 16)
  uint32_t kvo[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int row = 8 * w + 4 * p + (lane >> 4);
    kvo[p] = (uint32_t)(row * D + 8 * ((lane & 15) ^ (row & 15))) * 2;
  }
  auto dma_k = [&](bf16* dst, int j) {
#pragma unroll
    for (int p = 0; p < 2; ++p) dma16(krs, dst + (8 * w + 4 * p) * D, kvo[p] + (uint32_t)j * TILE_BYTES);
  };
  const int ky = hf ^ (l32 & 15);   // row 32 kb + l32, chunk 2t + hf at slot 2t ^ ky

  uint32_t word = 0u;            // decisions of columns 32 (j / 8) .. + 31 of this wave's row
  float thr_s = thr;
  auto step = [&](auto which, int j) {
    constexpr int P = decltype(which)::value;   // j % 3
    constexpr int PN = (P + 1) % 3;              // (j - 2) % 3
    const bf16* const kt = P == 0 ? k0 : P == 1 ? k1 : k2;
    dma_k(PN == 0 ? k0 : PN == 1 ? k1 : k2, max(j - 2, 0));
    if (active && j <= top_w) {
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
      bf16x8 ka[KT][2];
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) ka[t][kb] = load16(kt + (32 * kb + l32) * D + 8 * ((2 * t) ^ ky));
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sacc[kb] = mfma32(ka[t][kb], qr[t], sacc[kb]);
      const int key0 = j * 64;
      if ((key0 + 64 > s.nk) || (q0 + 32 > s.nq) || (s.causal && key0 + 63 > q0 + s.offset)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
            const bool ok = rvalid && key < s.nk && (!s.causal || key <= q + s.offset);
            sacc[kb][r] = ok ? sacc[kb][r] : kNegInf;
          }
      }
      // ---- offline gate, Eq. 4, per 16-key column c = keys 16 c .. + 15
      uint32_t keep4 = 0u;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float x = kNegInf;
#pragma unroll
        for (int r = 0; r < 8; ++r) x = fmaxf(x, sacc[c >> 1][8 * (c & 1) + r]);
        if (__builtin_amdgcn_ballot_w64(x >= thr_s) != 0) keep4 |= 1u << c;
      }
      word |= keep4 << ((4 * j) & 31);
      if (mask != nullptr && lane == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (legal_col(4 * j + c)) mask[brow * tc16 + 4 * j + c] = (int8_t)((keep4 >> c) & 1u);
      }
    }
    // the word of columns 32 (j / 8) .. is complete once the walk leaves it;
    // the bit rows start cleared, so only words with a kept column are written
    if ((j & 7) == 0) {
      if (active && lane == 0 && word != 0u) bits[brow * words + (j >> 3)] = word;
      word = 0u;
    }
    // tile j - 1's loads (issued one step back) have landed once at most this
    // step's two remain
    wait_vm<2>();
    lds_barrier();
  };

  if (top_b >= 0) {
    const int j0 = top_b + (2 - top_b % 3);
    dma_k(k2, j0);
    dma_k(k1, j0 - 1);
#pragma unroll
    for (int t = 0; t < KT; ++t) settle(qr[t]);
    settle(thr_s);
    wait_vm<0>();
    __syncthreads();
    for (int j = j0; j >= 2; j -= 3) {
      step(std::integral_constant<int, 2>(), j);
      step(std::integral_constant<int, 1>(), j - 1);
      step(std::integral_constant<int, 0>(), j - 2);
    }
    wait_vm<0>();
  }
}

// ---------------------------------------------------------------- dQ
// A workgroup owns 256 query rows (8 waves x 32) of one (batch, query head).
// Key tiles of 64 rows (K and V, row-major) stream through LDS, only those
// that some wave of the block keeps; K^T, the A operand of dQ^T = K^T dS^T,
// comes from the K tile through transposing reads. This kernel stages the
// tiles through registers into double-buffered LDS and serves d = 64; the
// d = 128 kernel below stages them by LDS-DMA loads two tiles ahead.
//
// The K tile is read both as rows (16-byte reads, S^T = K Q^T) and through
// transposing reads (K^T). No single row stride serves both without bank
// conflicts, so K uses a stride of 160 (transposing reads conflict-free) and
// permutes the 16-byte chunks of each row: chunk c of row r is stored at
// chunk c ^ ((r / 4) % 4), which spreads 16 consecutive rows of one chunk
// over all 64 banks. V is only read as rows (stride 136).
template <int D>
struct alignas(16) DqSmem {
  static constexpr int kStrideK = D + 32;
  static constexpr int kStrideV = D + 8;
  bf16 k[2][64][kStrideK];
  bf16 v[2][64][kStrideV];
};
// column (bf16 index) of element chunk `c` of K tile row `r`, after the swizzle
__device__ __forceinline__ int kswz(int r, int c) { return 8 * (c ^ ((r >> 2) & 3)); }

template <int D, bool kSplit>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(
    Shape s, const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dq,
    bf16* __restrict__ dQ, const uint32_t* __restrict__ bits, int32_t* __restrict__ kept,
    int n_qb) {
  __shared__ DqSmem<D> sm;
  extern __shared__ uint32_t need[];   // ceil(tiles / 32) words, sized at launch
  constexpr int SK = DqSmem<D>::kStrideK, SV = DqSmem<D>::kStrideV;
  constexpr int KT = D / 16, DB = D / 32, CPR = D / 8;
  constexpr int RPP = 512 / CPR;            // rows per load pass
  constexpr int KPASS = 64 / RPP;

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int gg = lane >> 4, i16 = lane & 15;
  const int bh_count = s.batch * s.hq;
  const int I = n_qb - 1 - (int)(blockIdx.x / bh_count);
  const int bh = xcd_head((int)(blockIdx.x % bh_count), s.batch * s.hkv, s.group);
  const int b = bh / s.hq, h = bh % s.hq, hk = h / s.group;
  const size_t qrow0 = (size_t)bh * (size_t)s.nq;
  const size_t krow0 = ((size_t)b * s.hkv + hk) * (size_t)s.nk;
  const int tr32 = (s.nq + kBQ - 1) / kBQ;
  const int tc16 = (s.nk + kBK - 1) / kBK;
  const int words = (tc16 + 31) / 32;
  const int q0 = I * 256 + w * 32;
  const bool active = q0 < s.nq;
  const int q = q0 + l32;

  const auto qrs = make_rsrc(Q + qrow0 * D, (uint32_t)((size_t)s.nq * D * 2));
  const auto ors = make_rsrc(dO + qrow0 * D, (uint32_t)((size_t)s.nq * D * 2));
  const auto krs = make_rsrc(K + krow0 * D, (uint32_t)((size_t)s.nk * D * 2));
  const auto vrs = make_rsrc(V + krow0 * D, (uint32_t)((size_t)s.nk * D * 2));

  bf16x8 qr[KT], orr[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    qr[t] = buf_load16(qrs, (uint32_t)(q * D + 16 * t + 8 * hf) * 2);
    orr[t] = buf_load16(ors, (uint32_t)(q * D + 16 * t + 8 * hf) * 2);
  }
  const float z2 = q < s.nq ? LSE[qrow0 + q] * 1.4426950408889634f : 0.f;
  const float dd = q < s.nq ? Dq[qrow0 + q] : 0.f;
  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.f;

  // key tiles (64 keys) that may be legal for the block's last row
  const int last_row = min(I * 256 + 255, s.nq - 1);
  const int lastkey = s.causal ? min(last_row + s.offset, s.nk - 1) : s.nk - 1;
  const int ntiles = lastkey < 0 ? 0 : lastkey / 64 + 1;
  const uint32_t* mybits = bits + ((size_t)bh * tr32 + (active ? q0 / kBQ : 0)) * words;

  // kept backward tiles of this wave's 32-row block: the population count of
  // its decision bits
  if (kept != nullptr && active) {
    int cnt = 0;
    for (int x = lane; x < words; x += 64) cnt += __popc(mybits[x]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
    if (lane == 0) kept[(size_t)bh * tr32 + q0 / kBQ] = cnt;
  }

  bf16x8 kreg[KPASS], vreg[KPASS];
  const int kc = tid % CPR, kr = tid / CPR;
  auto load_tile = [&](int j) {
#pragma unroll
    for (int p = 0; p < KPASS; ++p) {
      const uint32_t off = (uint32_t)((j * 64 + p * RPP + kr) * D + 8 * kc) * 2;
      kreg[p] = buf_load16(krs, off);
      vreg[p] = buf_load16(vrs, off);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int p = 0; p < KPASS; ++p) {
      const int row = p * RPP + kr;
      store16(&sm.k[buf][row][kswz(row, kc)], kreg[p]);
      store16(&sm.v[buf][row][8 * kc], vreg[p]);
    }
  };
  // decision bits of tile j (64 keys = four 16-key columns) for one 32-row block
  auto tile_bits = [&](const uint32_t* row_bits, int j) -> uint32_t {
    return (row_bits[(4 * j) >> 5] >> ((4 * j) & 31)) & 15u;
  };
  // Tiles some wave of the block keeps, as a bitmap in LDS (bit t: some
  // 32-row block of the workgroup keeps a column of 64-key tile t), built
  // once by all threads so that skipped tiles cost no memory round trip.
  const int nrb = min(8, (s.nq - I * 256 + 31) / 32);   // valid 32-row blocks
  const uint32_t* blockbits = bits + ((size_t)bh * tr32 + I * 8) * words;
  const int nneed = (ntiles + 31) / 32;
  for (int x = tid; x < nneed; x += 512) need[x] = 0u;
  __syncthreads();
  for (int t = tid; t < ntiles; t += 512) {
    uint32_t any = 0;
#pragma unroll
    for (int ww = 0; ww < 8; ++ww)
      if (ww < nrb) any |= tile_bits(blockbits + (size_t)ww * words, t);
    if (any) atomicOr(&need[t >> 5], 1u << (t & 31));
  }
  __syncthreads();
  // largest needed tile index <= j, or -1
  auto next_needed = [&](int j) -> int {
    while (j >= 0) {
      const uint32_t w = __builtin_amdgcn_readfirstlane(need[j >> 5]) &
                         (0xffffffffu >> (31 - (j & 31)));
      if (w != 0u) return (j & ~31) + 31 - __clz(w);
      j = (j & ~31) - 1;
    }
    return -1;
  };

  // walk only the tiles some wave needs; stage each one in LDS. The staging
  // buffer alternates per staged tile (not per tile index: skipped tiles are
  // jumped over, so index parity would reuse the buffer being read).
  int j = next_needed(ntiles - 1);
  int jn = j < 0 ? -1 : next_needed(j - 1);            // next needed tile
  int buf = 0;
  if (j >= 0) {
    load_tile(j);
    store_tile(buf);
  }
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    settle(qr[t]);
    settle(orr[t]);
  }
  __syncthreads();
  uint32_t wd = j >= 0 && active ? tile_bits(mybits, j) : 0u;   // this wave's columns of tile j
  while (j >= 0) {
    // prefetch tile jn and its column bits for this wave; both are consumed
    // at the end of this iteration
    if (jn >= 0) load_tile(jn);
    const uint32_t wd_next = jn >= 0 && active ? tile_bits(mybits, jn) : 0u;

    if (active) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const uint32_t cols = (wd >> (2 * half)) & 3u;   // the half's two 16-key columns
        if (cols == 0) continue;
        const int key0 = j * 64 + 32 * half;
        // ---- S^T = K Q^T and dP^T = V dO^T: lane (query l32, half hf), regs = keys
        const int krow = 32 * half + l32;
        // dP^T accumulates from -D_q: dS = P o (dP - D) takes no subtraction
        f32x16 sacc, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) { sacc[r] = 0.f; dp[r] = -dd; }
        // K and V row operands, read four ahead of their products: the
        // schedule is pinned to four LDS reads, then alternating product and
        // read, so the two product chains (S^T, dP^T) hide the read latency
        bf16x8 ka_[KT], va_[KT];
#pragma unroll
        for (int t = 0; t < KT; ++t) {
          ka_[t] = load16(&sm.k[buf][krow][kswz(krow, 2 * t + hf)]);
          va_[t] = load16(&sm.v[buf][krow][16 * t + 8 * hf]);
        }
#pragma unroll
        for (int t = 0; t < KT; ++t) {
          sacc = mfma32(ka_[t], qr[t], sacc);
          dp = mfma32(va_[t], orr[t], dp);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);       // 4 LDS reads
#pragma unroll
        for (int u = 0; u < 2 * KT - 4; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // 1 MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // 1 LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);       // last 4 MFMAs
        const bool boundary = (key0 + 32 > s.nk) || (q0 + 32 > s.nq) ||
                              (s.causal && key0 + 31 > q0 + s.offset);
        if (boundary) {                                // wave-uniform: mask illegal entries
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = key0 + 8 * (r >> 2) + 4 * hf + (r & 3);
            const bool ok = (kk < s.nk) & (q < s.nq) & ((kk <= q + s.offset) | (s.causal == 0));
            sacc[r] = ok ? sacc[r] : kNegInf;
          }
        }
        // key offset 8(r/4) + 4hf + r%4 lies in column r / 8 of the half: a
        // skipped column contributes P = 0 (wave-uniform, rare when dense)
        if (cols != 3u) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (!((cols >> (r >> 3)) & 1u)) sacc[r] = kNegInf;
        }
        bf16x8 dsb[2], dsl[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(sacc[r], s.scale_log2, -z2));
          const float ds = p * dp[r];
          const bf16 hi = (bf16)ds;
          dsb[r >> 3][r & 7] = hi;
          if constexpr (kSplit) dsl[r >> 3][r & 7] = (bf16)(ds - (float)hi);
        }
        // ---- dQ^T += K^T dS^T; K^T element e of lane (d, hf) is key
        // 16t + 4hf + e (e < 4) or 16t + 8 + 4hf + (e - 4). Lane i16 of a
        // 16-lane group reads row r0 + i16 / 4, columns c0 + 4 (i16 % 4)..+3,
        // where the chunk holding them is permuted by the swizzle.
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int r0 = 32 * half + 16 * t + 4 * hf;
            const int c = 4 * db + 2 * (gg & 1) + ((i16 & 3) >> 1);   // 16-byte chunk
            const int within = 4 * (i16 & 1);
            const int ra = r0 + (i16 >> 2), rb = r0 + 8 + (i16 >> 2);
            const bf16x8 ka = cat8(lds_read_tr_at(&sm.k[buf][ra][kswz(ra, c) + within]),
                                   lds_read_tr_at(&sm.k[buf][rb][kswz(rb, c) + within]));
            dq[db] = mfma32(ka, dsb[t], dq[db]);
            if constexpr (kSplit) dq[db] = mfma32(ka, dsl[t], dq[db]);
          }
      }
    }
    if (jn >= 0) store_tile(buf ^ 1);
    const int jnn = jn < 1 ? -1 : next_needed(jn - 1);   // the needed tile after jn
    __syncthreads();
    buf ^= 1;
    j = jn;
    jn = jnn;
    wd = wd_next;
  }

  if (!active || q >= s.nq) return;
  const float sc_nat = s.scale_log2 * 0.69314718055994531f;
  bf16* row = dQ + (qrow0 + q) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 y = {(bf16)(dq[db][4 * g] * sc_nat), (bf16)(dq[db][4 * g + 1] * sc_nat),
                  (bf16)(dq[db][4 * g + 2] * sc_nat), (bf16)(dq[db][4 * g + 3] * sc_nat)};
      *reinterpret_cast<bf16x4*>(row + 32 * db + 8 * g + 4 * hf) = y;
    }
}


// d = 128: the same walk with the K and V tiles staged by LDS-DMA buffer
// loads (global memory straight into LDS: no registers, no LDS stores) two
// needed tiles ahead, in three buffers. Step n reads buffer n % 3, issues the
// DMA of the needed tile two ahead into the buffer that held the previous
// one, and before an LDS-only barrier waits only for the next tile's loads,
// issued one step earlier. The buffers are six separate LDS arrays and the
// walk runs its steps in the fixed order 0, 1, 2, so each read names its
// array at compile time and the compiler's DMA wait covers only reads of the
// array a DMA fills.
//
// Both tiles are unpadded (256-byte rows) with 16-byte chunk c of row r at
// c ^ f(r % 16), f(r) = r ^ 4 (r % 4): among the row permutations timed on
// this LDS for these two access patterns, it runs the K row reads and the
// K^T transposing reads at the conflict-free rate (f(r) = r halves the
// transposing reads' rate); V, read as rows only, shares it.
__device__ __forceinline__ int dq_swz(int r) { return r ^ ((r & 3) << 2); }

template <bool kSplit>
__global__ __launch_bounds__(512, 1) void bwd_dq_d128_kernel(
    Shape s, const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dq,
    bf16* __restrict__ dQ, const uint32_t* __restrict__ bits, int32_t* __restrict__ kept,
    int n_qb) {
  constexpr int D = 128;
  constexpr int KT = D / 16, DB = D / 32;
  constexpr int TILE = 64 * D;
  constexpr uint32_t TILE_BYTES = TILE * 2;
  __shared__ __attribute__((aligned(16))) bf16 k0[TILE], k1[TILE], k2[TILE], v0[TILE], v1[TILE], v2[TILE];
  extern __shared__ uint32_t need[];   // ceil(tiles / 32) words, sized at launch

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int gg = lane >> 4, i16 = lane & 15;
  const int bh_count = s.batch * s.hq;
  const int I = n_qb - 1 - (int)(blockIdx.x / bh_count);
  const int bh = xcd_head((int)(blockIdx.x % bh_count), s.batch * s.hkv, s.group);
  const int b = bh / s.hq, h = bh % s.hq, hk = h / s.group;
  const size_t qrow0 = (size_t)bh * (size_t)s.nq;
  const size_t krow0 = ((size_t)b * s.hkv + hk) * (size_t)s.nk;
  const int tr32 = (s.nq + kBQ - 1) / kBQ;
  const int tc16 = (s.nk + kBK - 1) / kBK;
  const int words = (tc16 + 31) / 32;
  const int q0 = I * 256 + w * 32;
  const bool active = q0 < s.nq;
  const int q = q0 + l32;

  const auto qrs = make_rsrc(Q + qrow0 * D, (uint32_t)((size_t)s.nq * D * 2));
  const auto ors = make_rsrc(dO + qrow0 * D, (uint32_t)((size_t)s.nq * D * 2));
  const auto krs = make_rsrc(K + krow0 * D, (uint32_t)((size_t)s.nk * D * 2));
  const auto vrs = make_rsrc(V + krow0 * D, (uint32_t)((size_t)s.nk * D * 2));
  // zero-sized: the loads of a step past the walk return zeros and touch nothing
  const auto krs0 = make_rsrc(K + krow0 * D, 0u);
  const auto vrs0 = make_rsrc(V + krow0 * D, 0u);

  bf16x8 qr[KT], orr[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    qr[t] = buf_load16(qrs, (uint32_t)(q * D + 16 * t + 8 * hf) * 2);
    orr[t] = buf_load16(ors, (uint32_t)(q * D + 16 * t + 8 * hf) * 2);
  }
  const float z2 = q < s.nq ? LSE[qrow0 + q] * 1.4426950408889634f : 0.f;
  const float dd = q < s.nq ? Dq[qrow0 + q] : 0.f;
  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.f;

  const int last_row = min(I * 256 + 255, s.nq - 1);
  const int lastkey = s.causal ? min(last_row + s.offset, s.nk - 1) : s.nk - 1;
  const int ntiles = lastkey < 0 ? 0 : lastkey / 64 + 1;
  const uint32_t* mybits = bits + ((size_t)bh * tr32 + (active ? q0 / kBQ : 0)) * words;

  if (kept != nullptr && active) {
    int cnt = 0;
    for (int x = lane; x < words; x += 64) cnt += __popc(mybits[x]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
    if (lane == 0) kept[(size_t)bh * tr32 + q0 / kBQ] = cnt;
  }

  auto tile_bits = [&](const uint32_t* row_bits, int j) -> uint32_t {
    return (row_bits[(4 * j) >> 5] >> ((4 * j) & 31)) & 15u;
  };
  const int nrb = min(8, (s.nq - I * 256 + 31) / 32);
  const uint32_t* blockbits = bits + ((size_t)bh * tr32 + I * 8) * words;
  const int nneed = (ntiles + 31) / 32;
  for (int x = tid; x < nneed; x += 512) need[x] = 0u;
  __syncthreads();
  for (int t = tid; t < ntiles; t += 512) {
    uint32_t any = 0;
#pragma unroll
    for (int ww = 0; ww < 8; ++ww)
      if (ww < nrb) any |= tile_bits(blockbits + (size_t)ww * words, t);
    if (any) atomicOr(&need[t >> 5], 1u << (t & 31));
  }
  __syncthreads();
  auto next_needed = [&](int j) -> int {
    while (j >= 0) {
      const uint32_t wv = __builtin_amdgcn_readfirstlane(need[j >> 5]) &
                          (0xffffffffu >> (31 - (j & 31)));
      if (wv != 0u) return (j & ~31) + 31 - __clz(wv);
      j = (j & ~31) - 1;
    }
    return -1;
  };

  // ---- DMA: wave w fills rows 8 w .. 8 w + 7 of a tile, four per
  // instruction; lane l fills slot l % 16 of row 8 w + 4 p + l / 16 with
  // global chunk (l % 16) ^ f(row % 16)
  uint32_t dvo[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int row = 8 * w + 4 * p + (lane >> 4);
    dvo[p] = (uint32_t)(row * D + 8 * ((lane & 15) ^ dq_swz(row & 15))) * 2;
  }
  auto dma_tile = [&](bf16* kd, bf16* vd, int j) {
    const bool live = j >= 0;
    const auto kr_ = live ? krs : krs0;
    const auto vr_ = live ? vrs : vrs0;
    const uint32_t off = (uint32_t)(live ? j : 0) * TILE_BYTES;
#pragma unroll
    for (int p = 0; p < 2; ++p) dma16(kr_, kd + (8 * w + 4 * p) * D, dvo[p] + off);
#pragma unroll
    for (int p = 0; p < 2; ++p) dma16(vr_, vd + (8 * w + 4 * p) * D, dvo[p] + off);
  };

  // ---- LDS addressing (bytes). Row reads: row 32 half + l32, chunk 2t + hf,
  // at slot 2 t ^ Y. Transposing reads: row 32 half + 16 t + 4 hf + i16 / 4
  // (+ 8), chunk 4 db + cc, half i16 % 2, at slot 4 db ^ Z (^ 8 for the + 8
  // rows, f(r + 8) = f(r) ^ 8).
  const int Y = hf ^ dq_swz(l32 & 15);
  const int cc = 2 * (gg & 1) + ((i16 & 3) >> 1);
  const int rt = 4 * hf + (i16 >> 2);
  const int Z = cc ^ dq_swz(rt);
  int ra[KT], ta[DB];
#pragma unroll
  for (int t = 0; t < KT; ++t) ra[t] = l32 * 256 + ((16 * Y) ^ (32 * t));
#pragma unroll
  for (int db = 0; db < DB; ++db) ta[db] = rt * 256 + ((16 * Z) ^ (64 * db)) + 8 * (i16 & 1);
  auto rowrd = [&](const bf16* tile, int R, int t) {
    return load16(reinterpret_cast<const char*>(tile) + R * 256 + ra[t]);
  };
  auto trrd = [&](const bf16* tile, int R, int db) {
    return lds_read_tr_at(reinterpret_cast<const bf16*>(reinterpret_cast<const char*>(tile) + R * 256 + ta[db]));
  };
  // the same eight rows further down: slot bit 3 flips (byte bit 7)
  auto trrd8 = [&](const bf16* tile, int R, int db) {
    return lds_read_tr_at(
        reinterpret_cast<const bf16*>(reinterpret_cast<const char*>(tile) + R * 256 + 2048 + (ta[db] ^ 128)));
  };

  // one step at needed tile j (buffer B); jnn: the needed tile two ahead
  auto step = [&](auto bc, int j, int jnn, uint32_t wd) {
    constexpr int B = decltype(bc)::value;
    constexpr int B2 = (B + 2) % 3;
    const bf16* const kt = B == 0 ? k0 : B == 1 ? k1 : k2;
    const bf16* const vt = B == 0 ? v0 : B == 1 ? v1 : v2;
    dma_tile(B2 == 0 ? k0 : B2 == 1 ? k1 : k2, B2 == 0 ? v0 : B2 == 1 ? v1 : v2, jnn);
    if (active && j >= 0) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const uint32_t cols = (wd >> (2 * half)) & 3u;
        if (cols == 0) continue;
        const int key0 = j * 64 + 32 * half;
        // dP^T accumulates from -D_q: dS = P o (dP - D) takes no subtraction
        f32x16 sacc, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) { sacc[r] = 0.f; dp[r] = -dd; }
        bf16x8 ka_[KT], va_[KT];
#pragma unroll
        for (int t = 0; t < KT; ++t) {
          ka_[t] = rowrd(kt, 32 * half, t);
          va_[t] = rowrd(vt, 32 * half, t);
        }
#pragma unroll
        for (int t = 0; t < KT; ++t) {
          sacc = mfma32(ka_[t], qr[t], sacc);
          dp = mfma32(va_[t], orr[t], dp);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int u = 0; u < 2 * KT - 4; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        const bool boundary = (key0 + 32 > s.nk) || (q0 + 32 > s.nq) ||
                              (s.causal && key0 + 31 > q0 + s.offset);
        if (boundary) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = key0 + 8 * (r >> 2) + 4 * hf + (r & 3);
            const bool ok = (kk < s.nk) & (q < s.nq) & ((kk <= q + s.offset) | (s.causal == 0));
            sacc[r] = ok ? sacc[r] : kNegInf;
          }
        }
        if (cols != 3u) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[r] = ((cols >> (r >> 3)) & 1u) ? sacc[r] : kNegInf;
        }
        bf16x8 dsb[2], dsl[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(sacc[r], s.scale_log2, -z2));
          const float ds = p * dp[r];
          const bf16 hi = (bf16)ds;
          dsb[r >> 3][r & 7] = hi;
          if constexpr (kSplit) dsl[r >> 3][r & 7] = (bf16)(ds - (float)hi);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int R = 32 * half + 16 * t;
            const bf16x8 ka = cat8(trrd(kt, R, db), trrd8(kt, R, db));
            dq[db] = mfma32(ka, dsb[t], dq[db]);
            if constexpr (kSplit) dq[db] = mfma32(ka, dsl[t], dq[db]);
          }
      }
    }
    wait_vm<4>();
    lds_barrier();
  };

  // walk the needed tiles from the top; (j, jn, jnn) the current one and the
  // next two
  int j = next_needed(ntiles - 1);
  if (j >= 0) {
    int jn = next_needed(j - 1);
    dma_tile(k0, v0, j);
    dma_tile(k1, v1, jn);
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      settle(qr[t]);
      settle(orr[t]);
    }
    wait_vm<0>();
    __syncthreads();
    int jnn = jn < 1 ? -1 : next_needed(jn - 1);
    uint32_t wd = active ? tile_bits(mybits, j) : 0u;
    auto advance = [&]() {
      j = jn;
      jn = jnn;
      jnn = jn < 1 ? -1 : next_needed(jn - 1);
      wd = j >= 0 && active ? tile_bits(mybits, j) : 0u;
    };
    while (true) {
      step(std::integral_constant<int, 0>(), j, jnn, wd);
      advance();
      if (j < 0) break;
      step(std::integral_constant<int, 1>(), j, jnn, wd);
      advance();
      if (j < 0) break;
      step(std::integral_constant<int, 2>(), j, jnn, wd);
      advance();
      if (j < 0) break;
    }
    wait_vm<0>();
  }

  if (!active || q >= s.nq) return;
  const float sc_nat = s.scale_log2 * 0.69314718055994531f;
  bf16* row = dQ + (qrow0 + q) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 y = {(bf16)(dq[db][4 * g] * sc_nat), (bf16)(dq[db][4 * g + 1] * sc_nat),
                  (bf16)(dq[db][4 * g + 2] * sc_nat), (bf16)(dq[db][4 * g + 3] * sc_nat)};
      *reinterpret_cast<bf16x4*>(row + 32 * db + 8 * g + 4 * hf) = y;
    }
}

}  // namespace

size_t bwd_ws_d_floats(const Shape& s) { return (size_t)s.batch * s.hq * s.nq; }

size_t bwd_part_floats(const Shape& s) {
  if (!s.dtype_is_bf16() || !(s.flags & MALA_FLAG_GATE_PASS)) return 0;
  return 2 * (size_t)s.batch * s.hq * s.nk * s.d;
}

size_t bwd_plan_entries(const Shape& s) { return (size_t)s.batch * s.hkv * ((s.nk + 127) / 128); }

// the sampled gate of mala_bwd_auto: every rowstride-th 256-row block of
// every head (about 256 workgroups, one round of the chip), one key tile in
// `stride` of each walk (about 8 tiles); both 1 for small problems, where
// the sample is the whole gate
void sample_strides(const Shape& s, int* rowstride, int* stride) {
  const long long groups = (long long)((s.nq + 255) / 256) * s.batch * s.hq;
  *rowstride = (int)std::max(1LL, groups / 256);
  *stride = std::max(1, ((s.nk + 63) / 64) / 16);
}

// workgroups of the query-major gate kernels: 256 rows of one head each
size_t bwd_gate_groups(const Shape& s) { return (size_t)((s.nq + 255) / 256) * s.batch * s.hq; }

size_t bwd_plan_ints(const Shape& s) {
  if (!s.dtype_is_bf16() || !(s.flags & MALA_FLAG_GATE_PASS)) return 0;
  // the plan, the walk choice, and the sampled gate's two counts per workgroup
  return bwd_plan_entries(s) + 1 + 2 * bwd_gate_groups(s);
}

size_t bwd_bits_words(const Shape& s) {
  const size_t tr = (s.nq + kBQ - 1) / kBQ, tc = (s.nk + kBK - 1) / kBK;
  return (size_t)s.batch * s.hq * tr * ((tc + 31) / 32);
}

hipError_t launch_bwd_bf16(const Shape& s, const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* d_o, void* dq, void* dk,
                           void* dv, float* ws_d, uint32_t* ws_bits, float* ws_part,
                           int32_t* ws_plan, const int8_t* fwd_mask, int8_t* mask, int32_t* kept,
                           hipStream_t st, int stages, const int32_t* fwd_kept) {
  const int rows = s.batch * s.hq * s.nq;
  const size_t nwords = bwd_bits_words(s);
  const size_t nkept = (size_t)s.batch * s.hq * ((s.nq + kBQ - 1) / kBQ);
  if (stages & kStagePrep) {
    const size_t nmask =
        mask ? (size_t)s.batch * s.hq * ((s.nq + kBQ - 1) / kBQ) * ((s.nk + kBK - 1) / kBK) : 0;
    size_t work = (size_t)rows * (s.d / 8) / 64;   // waves: 64 16-byte chunks of O, dO each
    if (nwords / 64 > work) work = nwords / 64;
    if (nmask / 64 > work) work = nmask / 64;
    size_t blocks = (work + 3) / 4 + 1;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, st, rows, s.d,
                       (const bf16*)o, (const bf16*)d_o, ws_d, ws_bits, nwords, kept, nkept,
                       mask, nmask);
  }
  const int n_kb = (s.nk + 127) / 128;
  const dim3 g1((unsigned)(n_kb * s.batch * s.hkv));
  const int n_qb = (s.nq + 255) / 256;
  const dim3 g2((unsigned)(n_qb * s.batch * s.hq));
  // MALA_FLAG_GATE_PASS: the gate pass writes the decisions, and dK/dV
  // visits only the steps that hold a kept tile. fwd_kept (mala_bwd_auto):
  // both walks are launched, and the choice kernel's flag (after the plan
  // entries) lets the workgroups of one of them run
  const bool gated = (s.flags & MALA_FLAG_GATE_PASS) != 0;
  const bool choose = fwd_kept != nullptr && gated;
  const int32_t* take = nullptr;
  if (choose && (stages & kStageMain)) {
    // the forward's legal tiles: per 32-row block, the 64-key tiles up to
    // the one that holds its last row's last visible key
    const int ftr = (s.nq + kFwdBq - 1) / kFwdBq;
    long long legal = 0;
    for (int i = 0; i < ftr; ++i) {
      const int last = std::min(i * kFwdBq + kFwdBq - 1, s.nq - 1);
      const int lastkey = s.causal ? std::min(last + s.offset, s.nk - 1) : s.nk - 1;
      legal += lastkey < 0 ? 0 : lastkey / kFwdBk + 1;
    }
    legal *= (long long)s.batch * s.hq;
    int32_t* flag = ws_plan + bwd_plan_entries(s);
    uint32_t* slots = reinterpret_cast<uint32_t*>(flag + 1);
    // the backward's own decisions on a sample: about 256 workgroups of the
    // gate kernel (every rowstride-th 256-row block of every head), each on
    // about 8 key tiles of its walk (one in `stride`)
    int rowstride, stride;
    sample_strides(s, &rowstride, &stride);
    const dim3 gs((unsigned)(((n_qb + rowstride - 1) / rowstride) * s.batch * s.hq));
    if (gs.x) {
      if (s.d == 128)
        hipLaunchKernelGGL((bwd_gate_kernel<128, false, true>), gs, dim3(512), 0, st, s,
                           (const bf16*)q, (const bf16*)k, lse, (uint32_t*)nullptr,
                           (int8_t*)nullptr, n_qb, (const int8_t*)nullptr,
                           (const int32_t*)nullptr, slots, stride, rowstride);
      else
        hipLaunchKernelGGL((bwd_gate_kernel<64, false, true>), gs, dim3(512), 0, st, s,
                           (const bf16*)q, (const bf16*)k, lse, (uint32_t*)nullptr,
                           (int8_t*)nullptr, n_qb, (const int8_t*)nullptr,
                           (const int32_t*)nullptr, slots, stride, rowstride);
    }
    hipLaunchKernelGGL(bwd_choose_kernel, dim3(1), dim3(1024), 0, st, fwd_kept,
                       (long long)s.batch * s.hq * ftr, legal, (const uint32_t*)slots,
                       (long long)gs.x, flag);
    take = flag;
  }
  auto launch = [&](auto gate, auto gate_nested, auto dkdv, auto dkdv_gated, auto dqk) {
    if (choose && g1.x && (stages & kStageMain)) {
      // the default walk; its workgroups return unless the flag is 0
      hipLaunchKernelGGL(dkdv, g1, dim3(512), 0, st, s, (const bf16*)q, (const bf16*)k,
                         (const bf16*)v, (const bf16*)d_o, lse, ws_d, (bf16*)dk, (bf16*)dv,
                         ws_bits, mask, (float*)nullptr, (const int32_t*)nullptr, take);
    }
    if (gated && (stages & kStageMain)) {
      // decisions (on the forward's kept tiles only, given its mask), then
      // one walk per (key block, query head), then the sums
      if (g2.x && fwd_mask != nullptr)
        hipLaunchKernelGGL(gate_nested, g2, dim3(512), 0, st, s, (const bf16*)q, (const bf16*)k,
                           lse, ws_bits, mask, n_qb, fwd_mask, take, (uint32_t*)nullptr, 1, 1);
      else if (g2.x)
        hipLaunchKernelGGL(gate, g2, dim3(512), 0, st, s, (const bf16*)q, (const bf16*)k, lse,
                           ws_bits, mask, n_qb, (const int8_t*)nullptr, take, (uint32_t*)nullptr, 1,
                           1);
      // the kept pairs of each key block choose its walks
      if (g1.x)
        hipLaunchKernelGGL(bwd_plan_kernel, g1, dim3(64), 0, st, s, (const uint32_t*)ws_bits,
                           ws_plan, take);
      const dim3 g1h((unsigned)(g1.x * s.group));
      if (g1h.x)
        hipLaunchKernelGGL(dkdv_gated, g1h, dim3(512), 0, st, s, (const bf16*)q, (const bf16*)k,
                           (const bf16*)v, (const bf16*)d_o, lse, ws_d, (bf16*)dk, (bf16*)dv,
                           ws_bits, mask, ws_part, (const int32_t*)ws_plan, take);
      if (g1.x)
        hipLaunchKernelGGL(bwd_dkdv_finalize_kernel, g1, dim3(256), 0, st, s,
                           (const float*)ws_part, (const int32_t*)ws_plan, (bf16*)dk, (bf16*)dv,
                           take);
    } else if (g1.x && (stages & kStageMain)) {
      hipLaunchKernelGGL(dkdv, g1, dim3(512), 0, st, s, (const bf16*)q, (const bf16*)k,
                         (const bf16*)v, (const bf16*)d_o, lse, ws_d, (bf16*)dk, (bf16*)dv,
                         ws_bits, mask, (float*)nullptr, (const int32_t*)nullptr,
                         (const int32_t*)nullptr);
    }
    // dynamic LDS: the needed-tile bitmap, one bit per 64-key tile
    const size_t need_bytes = (size_t)((s.nk + 64 * 32 - 1) / (64 * 32)) * 4;
    if (g2.x && (stages & kStageDq))
      hipLaunchKernelGGL(dqk, g2, dim3(512), need_bytes, st, s, (const bf16*)q, (const bf16*)k,
                         (const bf16*)v, (const bf16*)d_o, lse, ws_d, (bf16*)dq, ws_bits, kept,
                         n_qb);
  };
  const bool split = !(s.flags & MALA_FLAG_FAST_GRAD);
  if (s.d == 128) {
    if (split)
      launch(bwd_gate_d128_kernel, bwd_gate_kernel<128, true>, bwd_dkdv_kernel<128, false>,
             bwd_dkdv_kernel<128, true>, bwd_dq_d128_kernel<true>);
    else
      launch(bwd_gate_d128_kernel, bwd_gate_kernel<128, true>, bwd_dkdv_kernel<128, false>,
             bwd_dkdv_kernel<128, true>, bwd_dq_d128_kernel<false>);
  } else {
    if (split)
      launch(bwd_gate_kernel<64, false>, bwd_gate_kernel<64, true>, bwd_dkdv_kernel<64, false>,
             bwd_dkdv_kernel<64, true>, bwd_dq_kernel<64, true>);
    else
      launch(bwd_gate_kernel<64, false>, bwd_gate_kernel<64, true>, bwd_dkdv_kernel<64, false>,
             bwd_dkdv_kernel<64, true>, bwd_dq_kernel<64, false>);
  }
  return hipGetLastError();
}

}  // namespace mala
