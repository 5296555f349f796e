// MALA split-KV decode for bf16 caches on gfx950 (Sec. 2.4; App. A.1
// "Fused decoding execution").
//
// One workgroup handles one split of one (sequence, KV head) for all query
// heads of the group (up to 16, packed as MFMA columns). The split's tiles
// (64 keys each) are visited newest first in groups of four, one tile per
// wave, with the split's running state (M, S) carried from group to group:
//   1. each wave reads its K tile straight from HBM in the 16x16x32 MFMA
//      operand layout and scores it against every head (score discovery:
//      all keys);
//   2. per-head tile max and tile sum are exchanged through LDS; every wave
//      then replays the group's gate sequence (newest tile first) from those
//      statistics and the running state, which is exactly the forward rule of
//      Eq. 3 on a one-row block per head with L = N_k;
//   3. only a tile kept by at least one head loads its V tile; each 32-key
//      half of it is staged row-major in a wave-private LDS slab and read back
//      transposed (ds_read_b64_tr_b16) as the A operand of O^T += V^T P^T;
//      heads that skipped the tile contribute P = 0. P is taken against the
//      running maximum, and a wave's partial output is rescaled when a group
//      raises it (the online-softmax update);
//   4. the four waves' partial outputs are summed in LDS and the split writes
//      its partial state (m, S, O) in base 2.
// With the default 256-key split a workgroup is one group. The small LDS
// footprint (37 KB) and 144 registers let three workgroups share a CU, so the
// K and V streams of several splits are in flight at once.
// A second kernel merges the splits with the normalizer-aware reduction.
#include "mala_device.h"
#include "mala_internal.h"

namespace mala {
namespace {

constexpr int kTile = 64;
constexpr int kMaxGroup = 16;
constexpr int kSlabStride = 144;      // bf16; conflict-free transposing reads (16x16x32 layout)

union alignas(16) DecSlab {
  bf16 v[32][kSlabStride];            // one 32-key half of the wave's V tile, row-major
  float o[kMaxGroup][128 + 4];        // then the wave's partial O, [head][d]
};
struct alignas(16) DecSmem {
  DecSlab slab[4];                    // one per wave
  float tmax[4][kMaxGroup];           // per (tile of the group, head) max, base 2
  float tsum[4][kMaxGroup];           // per (tile of the group, head) sum of 2^(s - max)
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void decode_split_kernel(
    DecodeShape s, const bf16* __restrict__ Qd, const bf16* __restrict__ Kc,
    const bf16* __restrict__ Vc, const int32_t* __restrict__ seqlens, float* __restrict__ ws,
    int8_t* __restrict__ mask) {
  constexpr int D = 128;
  __shared__ DecSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j16 = lane & 15, g = lane >> 4;
  const int c = blockIdx.x;
  const int b = blockIdx.y / s.hkv, hk = blockIdx.y % s.hkv;
  const int G = s.group;
  int nk = seqlens[b];
  nk = max(1, min(nk, min(s.max_nk, s.cap)));
  const int tpc = s.chunk / kTile;                     // tiles per split
  const int c0 = c * s.chunk;
  const int ntile = c0 >= nk ? 0 : min(tpc, (nk - c0 + kTile - 1) / kTile);
  const int ngroup = (ntile + 3) / 4;
  const size_t bh0 = (size_t)b * s.hq + hk * G;        // first query head of the group
  uint32_t* wbits = reinterpret_cast<uint32_t*>(ws);
  const bool head_ok = j16 < G;

  // decision words and mask entries no group of this split visits: tiles
  // from 4 * ngroup on (all of them for a split past the end of the sequence)
  for (int x = (4 * ngroup) / 32 + tid; x < s.wps; x += 256) {
    for (int hh = 0; hh < G; ++hh) wbits[dec_kbits_at(s, bh0 + hh, c) + x] = 0u;
    wbits[dec_vbits_at(s, blockIdx.y, c) + x] = 0u;
  }
  if (mask != nullptr)
    for (int x = tid; x < G * (tpc - 4 * ngroup); x += 256) {
      const int hh = x / (tpc - 4 * ngroup), t = 4 * ngroup + x % (tpc - 4 * ngroup);
      mask[((bh0 + hh) * s.n_chunks + c) * tpc + t] = -1;
    }
  if (ntile == 0) {
    // split past the end of this sequence: no contribution
    if (tid < G) {
      float* pms = ws + dec_ms_at(s, bh0 + tid, c);
      pms[0] = kNegInf;
      pms[1] = 0.f;
    }
    for (int idx = tid; idx < D * G; idx += 256) ws[dec_o_at(s, bh0 + idx / D, c) + idx % D] = 0.f;
    return;
  }

  // rows at or past N_k read as zeros (the cache may hold anything there)
  const size_t crow0 = ((size_t)b * s.hkv + hk) * (size_t)s.cap;
  const auto krs = make_rsrc(Kc + crow0 * D, (uint32_t)((size_t)nk * D * 2));
  const auto vrs = make_rsrc(Vc + crow0 * D, (uint32_t)((size_t)nk * D * 2));
  const bf16* qrow = Qd + (bh0 + min(j16, G - 1)) * D;
  const float c2 = s.log2_tau - fast_log2((float)nk);
  float M = kNegInf, S = 0.f;       // the split's running state for head j16
  uint32_t kword = 0u, vword = 0u;  // decision bits of the current 32-tile word
  f32x4 oacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) oacc[db][r] = 0.f;

  for (int grp = ngroup - 1; grp >= 0; --grp) {
    const int tw = 4 * grp + w;                        // this wave's tile
    const int key0 = c0 + tw * kTile;
    const bool has_keys = tw < ntile;

    // ---- score discovery for this wave's tile: S^T[key][head], 4 blocks of 16 keys
    f32x4 sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) sacc[kb][r] = 0.f;
    if (has_keys) {
      // the group's queries as the B operand: lane (head j16, group g) holds
      // q[32 t + 8 g .. + 7] (read again per group: cache-resident, and not
      // held in registers across the V phase)
      bf16x8 qb[D / 32];
#pragma unroll
      for (int t = 0; t < D / 32; ++t) qb[t] = head_ok ? load16(qrow + 32 * t + 8 * g) : zero8();
      // the whole tile's K operands in one round trip (64 registers: the
      // kernel runs three workgroups per CU rather than four, which measured
      // faster than two dependent halves at four)
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
    __syncthreads();                // the previous group's statistics have been read
    if (g == 0) {
      sm.tmax[w][j16] = mx;
      sm.tsum[w][j16] = sm_;
    }
    __syncthreads();

    // ---- the group's gate, newest tile first, continuing the split's state (Eq. 3)
    const float m_prev = M;
    uint32_t keepbits = 0;          // bit tt: head j16 keeps tile 4 grp + tt
    for (int tt = 3; tt >= 0; --tt) {
      if (4 * grp + tt >= ntile) continue;
      const float tm = sm.tmax[tt][j16], ts = sm.tsum[tt][j16];
      const bool keep = (S == 0.f) || (tm - (M + fast_log2(S)) >= c2);
      if (keep) {
        const float mn = fmaxf(M, tm);
        S = S * fast_exp2(M - mn) + ts * fast_exp2(tm - mn);
        M = mn;
        keepbits |= 1u << tt;
      }
    }
    const bool mine = head_ok && ((keepbits >> w) & 1u);
    const uint64_t vote = __builtin_amdgcn_ballot_w64(mine);
    const bool tile_kept = has_keys && vote != 0;

    // decisions: the head's kept-tile bits and the bits of V tiles read
    // (counted by the merge kernel), one 32-tile word at a time
    const int sh = (4 * grp) & 31;
    kword |= (head_ok ? keepbits : 0u) << sh;
    uint32_t vb = head_ok ? keepbits : 0u;   // tile tt's V is read iff some head keeps it
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) vb |= __shfl_xor(vb, off, 64);
    vword |= vb << sh;
    // (addresses as a wave-uniform base plus a 32-bit lane offset)
    if (w == 0 && g == 0 && head_ok && mask != nullptr) {
      int8_t* mrow = mask + (bh0 * s.n_chunks + c) * tpc;
      for (int tt = 0; tt < 4; ++tt) {
        const int t = 4 * grp + tt;
        if (t < tpc)
          mrow[(uint32_t)(j16 * s.n_chunks * tpc + t)] =
              t < ntile ? (int8_t)((keepbits >> tt) & 1u) : (int8_t)-1;
      }
    }
    if (sh == 0) {                  // the lowest group of its word: flush the word
      const int word = (4 * grp) >> 5;
      if (w == 0 && g == 0 && head_ok) {
        int jh = j16;               // formed here, not kept live across the loop
        asm volatile("" : "+v"(jh));
        (wbits + dec_kbits_at(s, bh0, c))[(uint32_t)(jh * s.n_chunks * s.wps + word)] = kword;
      }
      if (w == 0 && lane == 0) wbits[dec_vbits_at(s, blockIdx.y, c) + word] = vword;
      kword = 0u;
      vword = 0u;
    }

    // a group that raised the running maximum rescales the partial output
    if (M != m_prev) {
      const float a = fast_exp2(m_prev - M);        // 0 while the state was empty
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[db][r] *= a;
    }

    // ---- kept tile: V load (HBM), then per 32-key half: row-major LDS slab ->
    // transposing reads -> P V on the MFMA. Lane (chunk dc, group kq) loads key
    // 32 (p / 8) + 8 kq + p % 8 into vr[p], 16 bytes at column chunk dc.
    if (tile_kept) {
      // P^T as the B operand of 32-key step ks: element e < 4 is key
      // 32 ks + 4 g + e, e >= 4 is key 32 ks + 16 + 4 g + (e - 4); formed
      // before the V loads so that the scores are dead during the V phase
      bf16x8 pb[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float sv = sacc[2 * ks + (e >> 2)][e & 3];
          pb[ks][e] = (bf16)(mine ? fast_exp2(sv - M) : 0.f);
        }
      const int dc = lane & 15, kq = lane >> 4;
      bf16x8 vr[16];
#pragma unroll
      for (int p = 0; p < 16; ++p)
        vr[p] = buf_load16(vrs, (uint32_t)((key0 + 32 * (p >> 3) + 8 * kq + (p & 7)) * D + 8 * dc) * 2);
      bf16* slab = &sm.slab[w].v[0][0];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        // the slab is private to the wave, and a wave's LDS operations complete
        // in order: the previous half's reads are done before these writes land
#pragma unroll
        for (int p = 0; p < 8; ++p) store16(slab + (8 * kq + p) * kSlabStride + 8 * dc, vr[8 * ks + p]);
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
          const bf16x8 va = cat8(lds_read_tr(slab, kSlabStride, 4 * g, 16 * db, j16),
                                 lds_read_tr(slab, kSlabStride, 16 + 4 * g, 16 * db, j16));
          oacc[db] = mfma16(va, pb[ks], oacc[db]);
        }
      }
    }
  }
  __syncthreads();                  // every wave is done with its slab's V rows
  // O^T[d = 16db + 4g + r][head j16] -> slab as O[head][d]
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
    *reinterpret_cast<f32x4*>(&sm.slab[w].o[j16][16 * db + 4 * g]) = oacc[db];
  __syncthreads();

  // ---- sum the four waves and write the split's partial state
  for (int idx = tid; idx < D * G; idx += 256) {
    const int hh = idx / D, d = idx % D;
    const float o = sm.slab[0].o[hh][d] + sm.slab[1].o[hh][d] + sm.slab[2].o[hh][d] +
                    sm.slab[3].o[hh][d];
    ws[dec_o_at(s, bh0 + hh, c) + d] = o;
  }
  if (w == 0 && g == 0 && head_ok) {
    float* pms = ws + dec_ms_at(s, bh0 + j16, c);
    pms[0] = M;
    pms[1] = S;
  }
}

// ---------------------------------------------------------------- long splits
// With splits longer than 1024 keys and fewer split workgroups than the
// chip's 256 compute units (one split per sequence, say), each workgroup of
// the one-kernel path would walk many tile groups in sequence on a mostly
// idle chip. Such splits run as three parallel passes that take the same
// decisions:
//   1. decode_stats_kernel: one wave per tile scores the tile against every
//      head of the group and stores each head's tile maximum and tile sum
//      (exactly the statistics the one-kernel path exchanges through LDS);
//   2. decode_gate_kernel: one wave per (query head, split) replays the
//      split's gate, newest tile first, from those statistics. A 64-lane
//      ballot over the next 64 tiles finds the newest tile the current state
//      keeps, so a run of skipped tiles costs one step; a prefix log-sum-exp
//      scan over the window finds where a run of kept tiles ends, so such a
//      run costs one step too. The state is updated only by kept tiles, as in
//      Eq. 3. It writes the decision bits, the mask and the split's final
//      (M, S);
//   3. decode_pv_kernel: parts of four tiles in parallel; a wave takes a
//      tile that some head keeps, scores it again, forms P against the
//      split's final maximum and accumulates P V. The first part of a split
//      holds the split's maximum and sum, every other part with a kept tile
//      the maximum, so the merge kernel sums those parts without rescaling;
//      it skips the empty ones, which write nothing.

__global__ __launch_bounds__(256, 4) void decode_stats_kernel(
    DecodeShape s, const bf16* __restrict__ Qd, const bf16* __restrict__ Kc,
    const int32_t* __restrict__ seqlens, float* __restrict__ ws) {
  constexpr int D = 128;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j16 = lane & 15, g = lane >> 4;
  const int b = blockIdx.y / s.hkv, hk = blockIdx.y % s.hkv;
  const int G = s.group;
  int nk = seqlens[b];
  nk = max(1, min(nk, min(s.max_nk, s.cap)));
  const int tpc = s.chunk / kTile;
  const int ta = 4 * blockIdx.x + w;                   // tile index from position 0
  const int c = ta / tpc, t = ta % tpc;
  const int key0 = ta * kTile;
  if (c >= s.n_chunks || key0 >= nk) return;           // wave-uniform; no barrier below
  const size_t bh0 = (size_t)b * s.hq + hk * G;
  const size_t crow0 = ((size_t)b * s.hkv + hk) * (size_t)s.cap;
  const auto krs = make_rsrc(Kc + crow0 * D, (uint32_t)((size_t)nk * D * 2));
  bf16x8 qb[D / 32];
  const bf16* qrow = Qd + (bh0 + min(j16, G - 1)) * D;
#pragma unroll
  for (int u = 0; u < D / 32; ++u) qb[u] = j16 < G ? load16(qrow + 32 * u + 8 * g) : zero8();
  f32x4 sacc[4];
  bf16x8 ka[4][D / 32];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int u = 0; u < D / 32; ++u) {
      ka[kb][u] = buf_load16(krs, (uint32_t)((key0 + 16 * kb + j16) * D + 32 * u + 8 * g) * 2);
    }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) sacc[kb][r] = 0.f;
#pragma unroll
    for (int u = 0; u < D / 32; ++u) sacc[kb] = mfma16(ka[kb][u], qb[u], sacc[kb]);
  }
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
  if (g == 0 && j16 < G)
    *reinterpret_cast<float2*>(ws + dec_stats_at(s, bh0 + j16, c, t)) = make_float2(mx, sm_);
}

constexpr int kGateWords = 256;       // decision words per head a gate workgroup holds
constexpr int kGateWin = 8;           // 64-tile windows of statistics loaded per batch

// lane i's value of x, i wave-uniform (v_readlane: no LDS round trip)
__device__ __forceinline__ float lane_of(float x, int i) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), i));
}

__global__ __launch_bounds__(1024) void decode_gate_kernel(DecodeShape s,
                                                           const int32_t* __restrict__ seqlens,
                                                           float* __restrict__ ws,
                                                           int8_t* __restrict__ mask) {
  __shared__ uint32_t kb[kMaxGroup][kGateWords];
  __shared__ float2 stl[kMaxGroup][kGateWin][64];     // each wave's current batch of statistics
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = blockIdx.x;
  const int b = blockIdx.y / s.hkv, hk = blockIdx.y % s.hkv;
  const int G = s.group;
  int nk = seqlens[b];
  nk = max(1, min(nk, min(s.max_nk, s.cap)));
  const int tpc = s.chunk / kTile;
  const int c0 = c * s.chunk;
  const int ntile = c0 >= nk ? 0 : min(tpc, (nk - c0 + kTile - 1) / kTile);
  const size_t bh0 = (size_t)b * s.hq + hk * G;
  const size_t bh = bh0 + w;                           // wave w: query head w of the group
  uint32_t* wbits = reinterpret_cast<uint32_t*>(ws);
  for (int x = lane; x < s.wps; x += 64) kb[w][x] = 0u;

  // ---- replay the split's gate (Eq. 3, newest tile first, empty state)
  float M = kNegInf, S = 0.f;
  const float2* st = reinterpret_cast<const float2*>(ws + dec_stats_at(s, bh, c, 0));
  const float c2 = s.log2_tau - fast_log2((float)nk);
  // Lane i of window k of a batch holds tile base - 64 k - i. A batch is
  // parked in the wave's slice of LDS (a wave's LDS accesses complete in
  // order, so no barrier), the next one is loaded into registers meanwhile,
  // and the windows are replayed by a loop that reads them back.
  float2 nxt[kGateWin];
#pragma unroll
  for (int k = 0; k < kGateWin; ++k) {
    const int t = ntile - 1 - 64 * k - lane;
    nxt[k] = t >= 0 ? st[t] : make_float2(kNegInf, 0.f);
  }
  for (int base = ntile - 1; base >= 0; base -= 64 * kGateWin) {
#pragma unroll
    for (int k = 0; k < kGateWin; ++k) {
      stl[w][k][lane] = nxt[k];
      const int t = base - 64 * (kGateWin + k) - lane;
      nxt[k] = t >= 0 ? st[t] : make_float2(kNegInf, 0.f);
    }
#pragma unroll 1
    for (int k = 0; k < kGateWin; ++k) {
      const int wb = base - 64 * k;                    // tile of lane 0
      if (wb < 0) break;
      const int last = min(63, wb);                    // last lane holding a tile
      const float2 wv = stl[w][k][lane];
      const float tmv = wv.x, tsv = wv.y;
      int off = 0;                                     // lanes below off are decided
      while (off <= last) {
        // the newest undecided tile, tested against the state exactly as in
        // the one-kernel path
        const float tm0 = lane_of(tmv, off);
        const bool keep0 = S == 0.f || tm0 - (M + fast_log2(S)) >= c2;
        if (keep0) {
          // A run of kept tiles: if every tile before lane i is kept, the state
          // lane i is tested against is the state combined with those tiles,
          // an exclusive prefix of the window. The first lane that fails that
          // test is the first tile of the run that is skipped.
          const bool cand = lane >= off && lane <= last;
          float m = cand ? tmv : kNegInf, z = cand ? tsv : 0.f;
#pragma unroll
          for (int d = 1; d < 64; d <<= 1) {           // inclusive log-sum-exp scan
            const float mu = __shfl_up(m, d, 64), zu = __shfl_up(z, d, 64);
            if (lane >= d) {
              const float mn = fmaxf(m, mu);
              z = (mu == kNegInf ? 0.f : zu * fast_exp2(mu - mn)) +
                  (m == kNegInf ? 0.f : z * fast_exp2(m - mn));
              m = mn;
            }
          }
          float me = __shfl_up(m, 1, 64), ze = __shfl_up(z, 1, 64);   // exclusive
          if (lane == 0) { me = kNegInf; ze = 0.f; }
          const float um = fmaxf(M, me);
          const float us = (M == kNegInf ? 0.f : S * fast_exp2(M - um)) +
                           (me == kNegInf ? 0.f : ze * fast_exp2(me - um));
          const bool pass = us == 0.f || tmv - (um + fast_log2(us)) >= c2;
          const uint64_t bal = __builtin_amdgcn_ballot_w64(cand && !pass);
          const int j = bal ? (int)__builtin_ctzll(bal) : last + 1;   // first skipped lane
          if (cand && lane < j) {
            const int t = wb - lane;
            atomicOr(&kb[w][t >> 5], 1u << (t & 31));
          }
          if (j <= last) {                             // lane j is skipped: its state carries on
            M = lane_of(um, j);
            S = lane_of(us, j);
          } else {                                     // the whole rest of the window is kept
            const float ml = lane_of(m, last), zl = lane_of(z, last);
            const float mn = fmaxf(M, ml);
            S = (M == kNegInf ? 0.f : S * fast_exp2(M - mn)) + zl * fast_exp2(ml - mn);
            M = mn;
          }
          off = j + 1;
        } else {
          // a run of skipped tiles: the newest later tile the state keeps
          const bool cand = lane > off && lane <= last;
          const bool keep = cand && tmv - (M + fast_log2(S)) >= c2;
          const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
          if (bal == 0) break;                         // the rest of the window is skipped
          const int i = (int)__builtin_ctzll(bal);
          const float tm = lane_of(tmv, i), ts = lane_of(tsv, i);
          const float mn = fmaxf(M, tm);
          S = S * fast_exp2(M - mn) + ts * fast_exp2(tm - mn);
          M = mn;
          const int t = wb - i;
          if (lane == 0) kb[w][t >> 5] |= 1u << (t & 31);
          off = i + 1;
        }
      }
    }
  }
  // the split's state: its sum in the first part, its maximum in the first
  // part and in every part that holds a tile the head keeps; a later part
  // without one is empty (m = -inf: the merge reads nothing of it)
  __syncthreads();
  for (int p = lane; p < s.ppc; p += 64) {
    bool any = p == 0;
    for (int t = p * s.tpart; t < min((p + 1) * s.tpart, ntile) && !any; ++t)
      any = (kb[w][t >> 5] >> (t & 31)) & 1u;
    float* pms = ws + dec_ms_at(s, bh, c * s.ppc + p);
    pms[0] = any ? M : kNegInf;
    pms[1] = p == 0 ? S : 0.f;
  }
  // decision words of every head, the V-read words (some head keeps the
  // tile) and the mask
  for (int x = tid; x < s.wps; x += blockDim.x) {
    uint32_t v = 0u;
    for (int hh = 0; hh < G; ++hh) {
      const uint32_t k = kb[hh][x];
      wbits[dec_kbits_at(s, bh0 + hh, c) + x] = k;
      v |= k;
    }
    wbits[dec_vbits_at(s, blockIdx.y, c) + x] = v;
  }
  if (mask != nullptr)
    for (int x = tid; x < G * tpc; x += blockDim.x) {
      const int hh = x / tpc, t = x % tpc;
      mask[((bh0 + hh) * s.n_chunks + c) * tpc + t] =
          t < ntile ? (int8_t)((kb[hh][t >> 5] >> (t & 31)) & 1u) : (int8_t)-1;
    }
}

__global__ __launch_bounds__(256, 4) void decode_pv_kernel(
    DecodeShape s, const bf16* __restrict__ Qd, const bf16* __restrict__ Kc,
    const bf16* __restrict__ Vc, const int32_t* __restrict__ seqlens, float* __restrict__ ws) {
  constexpr int D = 128;
  __shared__ DecSlab slab[4];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j16 = lane & 15, g = lane >> 4;
  const int part = blockIdx.x, c = part / s.ppc, p = part % s.ppc;
  const int b = blockIdx.y / s.hkv, hk = blockIdx.y % s.hkv;
  const int G = s.group;
  int nk = seqlens[b];
  nk = max(1, min(nk, min(s.max_nk, s.cap)));
  const int tpc = s.chunk / kTile;
  const int c0 = c * s.chunk;
  const int ntile = c0 >= nk ? 0 : min(tpc, (nk - c0 + kTile - 1) / kTile);
  const int t_lo = p * s.tpart, t_hi = min(t_lo + s.tpart, ntile);
  const size_t bh0 = (size_t)b * s.hq + hk * G;
  const bool head_ok = j16 < G;
  const uint32_t* wbits = reinterpret_cast<const uint32_t*>(ws);
  const uint32_t* vw = wbits + dec_vbits_at(s, blockIdx.y, c);
  const uint32_t* kw = wbits + dec_kbits_at(s, bh0 + min(j16, G - 1), c);
  const float Mh = ws[dec_ms_at(s, bh0 + min(j16, G - 1), part)];   // the split's maximum
  const size_t crow0 = ((size_t)b * s.hkv + hk) * (size_t)s.cap;
  const auto krs = make_rsrc(Kc + crow0 * D, (uint32_t)((size_t)nk * D * 2));
  const auto vrs = make_rsrc(Vc + crow0 * D, (uint32_t)((size_t)nk * D * 2));
  const bf16* qrow = Qd + (bh0 + min(j16, G - 1)) * D;
  f32x4 oacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) oacc[db][r] = 0.f;

  // the part's V-read words, each loaded once: bits t_lo .. t_hi - 1
  auto part_bits = [&](int x) -> uint32_t {
    const int lo = max(t_lo - 32 * x, 0), hi = min(t_hi - 32 * x, 32);
    const uint32_t m = (hi >= 32 ? ~0u : (1u << hi) - 1u) & ~((1u << lo) - 1u);
    return vw[x] & m;
  };
  const int x_lo = t_lo >> 5, x_hi = t_hi > t_lo ? (t_hi - 1) >> 5 : x_lo - 1;
  if (p > 0) {
    // an empty later part (no head keeps a tile of it) is skipped by the merge
    uint32_t any = 0u;
    for (int x = x_lo; x <= x_hi; ++x) any |= part_bits(x);
    if (any == 0u) return;                             // uniform over the workgroup
  }
  // wave w takes the part's tiles t_lo + w, t_lo + w + 4, ...: in every word
  // the bits congruent to t_lo + w modulo 4
  const uint32_t mine_mod4 = 0x11111111u << ((t_lo + w) & 3);
  for (int x = x_lo; x <= x_hi; ++x) {
    uint32_t todo = part_bits(x) & mine_mod4;
    if (todo == 0u) continue;
    const uint32_t kword = kw[x];                      // this lane's head
    while (todo != 0u) {                               // wave-uniform; no barrier inside
      const int t = 32 * x + __builtin_ctz(todo);
      todo &= todo - 1u;
      const bool mine = head_ok && ((kword >> (t & 31)) & 1u);
      const int key0 = c0 + t * kTile;
      // ---- the tile's scores again (as pass 1), then P against the split's maximum
      f32x4 sacc[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[kb][r] = 0.f;
      {
        bf16x8 qb[D / 32];
#pragma unroll
        for (int u = 0; u < D / 32; ++u) qb[u] = head_ok ? load16(qrow + 32 * u + 8 * g) : zero8();
#pragma unroll
        for (int hk2 = 0; hk2 < 2; ++hk2) {
          bf16x8 ka[2][D / 32];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int u = 0; u < D / 32; ++u)
              ka[kb][u] = buf_load16(
                  krs, (uint32_t)((key0 + 16 * (2 * hk2 + kb) + j16) * D + 32 * u + 8 * g) * 2);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int u = 0; u < D / 32; ++u)
              sacc[2 * hk2 + kb] = mfma16(ka[kb][u], qb[u], sacc[2 * hk2 + kb]);
        }
      }
      bf16x8 pb[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int kb = 2 * ks + (e >> 2), r = e & 3;
          const int key = key0 + 16 * kb + 4 * g + r;
          const float sv = key < nk ? sacc[kb][r] * s.scale_log2 : kNegInf;
          pb[ks][e] = (bf16)(mine ? fast_exp2(sv - Mh) : 0.f);
        }
      // ---- V (HBM) -> wave-private slab -> transposing reads -> P V
      const int dc = lane & 15, kq = lane >> 4;
      bf16x8 vr[16];
#pragma unroll
      for (int q = 0; q < 16; ++q)
        vr[q] = buf_load16(vrs, (uint32_t)((key0 + 32 * (q >> 3) + 8 * kq + (q & 7)) * D + 8 * dc) * 2);
      bf16* sl = &slab[w].v[0][0];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int q = 0; q < 8; ++q) store16(sl + (8 * kq + q) * kSlabStride + 8 * dc, vr[8 * ks + q]);
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
          const bf16x8 va = cat8(lds_read_tr(sl, kSlabStride, 4 * g, 16 * db, j16),
                                 lds_read_tr(sl, kSlabStride, 16 + 4 * g, 16 * db, j16));
          oacc[db] = mfma16(va, pb[ks], oacc[db]);
        }
      }
    }
  }
  __syncthreads();                  // every wave is done with its slab's V rows
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
    *reinterpret_cast<f32x4*>(&slab[w].o[j16][16 * db + 4 * g]) = oacc[db];
  __syncthreads();
  for (int idx = tid; idx < D * G; idx += 256) {
    const int hh = idx / D, d = idx % D;
    ws[dec_o_at(s, bh0 + hh, part) + d] =
        slab[0].o[hh][d] + slab[1].o[hh][d] + slab[2].o[hh][d] + slab[3].o[hh][d];
  }
}

// Merge the split partial states of one (sequence, head), 32 output columns
// per workgroup: z = log sum_c Z_c, O = sum_c Z_c O_c / sum_c Z_c (the
// standard online-softmax reduction), in one pass over the partials. Thread
// (split lane cl, column quad dq) folds splits cl, cl + 32, ... into a
// running (max, normalizer, output) with rescaling, sixteen splits in
// flight per thread; the 32 split lanes are then merged the same way in LDS.
template <typename OutT, bool kSkipEmpty>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeShape s,
                                                             const float* __restrict__ ws,
                                                             OutT* __restrict__ o,
                                                             float* __restrict__ lse,
                                                             int32_t* __restrict__ kept) {
  __shared__ float sm_m[32], sm_z[32];
  __shared__ f32x4 sm_o[32][8];
  __shared__ int sm_cnt[4][2];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int nc = s.n_parts;                            // partial states per head
  const float* ms = ws + dec_ms_at(s, bh, 0);
  const int cl = tid >> 3, dq = tid & 7;
  const int d0 = blockIdx.y * 32 + 4 * dq;            // this thread's 4 columns
  const bool dok = d0 < s.d;                            // d is a multiple of 32
  const float* po = ws + dec_o_at(s, bh, 0) + (dok ? d0 : 0);
  // kept-tile counters from the splits' decision bits, counted by every
  // thread of the first column block, their loads issued ahead of the merge
  // loads:
  // [b][h] for the head, [b][Hq + g] (by the group's first head) for the V
  // tiles of KV head g
  const bool count = kept != nullptr && blockIdx.y == 0;
  const int cb_ = bh / s.hq, ch_ = bh % s.hq, chk_ = ch_ / s.group;
  const bool vhead = ch_ % s.group == 0;
  int nh = 0, nv = 0;
  // a head's (and a KV head's) words of all splits are contiguous; the first
  // kCw words per thread are loaded here, together, so that their round trip
  // overlaps the merge loads' (the counts are taken after the fold), and any
  // further words in a loop at the end
  constexpr int kCw = 4;
  const int nwords = count ? s.n_chunks * s.wps : 0;
  const uint32_t* wbits = reinterpret_cast<const uint32_t*>(ws);
  const uint32_t* hb = wbits + dec_kbits_at(s, bh, 0);
  const uint32_t* vbw = wbits + dec_vbits_at(s, (size_t)cb_ * s.hkv + chk_, 0);
  // bounded buffer loads: words past the range read as zero, with no branch
  // (a guarded plain load would wait for each word in turn)
  const auto hrs = make_rsrc(hb, (uint32_t)nwords * 4u);
  const auto vrs = make_rsrc(vbw, vhead ? (uint32_t)nwords * 4u : 0u);
  uint32_t hw[kCw], vw[kCw];
#pragma unroll
  for (int u = 0; u < kCw; ++u) {
    const uint32_t off = (uint32_t)(tid + 256 * u) * 4u;
    hw[u] = __builtin_amdgcn_raw_buffer_load_b32(hrs, off, 0, 0);
    vw[u] = __builtin_amdgcn_raw_buffer_load_b32(vrs, off, 0, 0);
  }
  float mrun = kNegInf, zrun = 0.f;
  f32x4 orun = {0.f, 0.f, 0.f, 0.f};
  auto fold = [&](float m, float z, f32x4 x) {
    const float mn = fmaxf(mrun, m);
    const float a = mrun == kNegInf ? 0.f : fast_exp2(mrun - mn);
    const float w = m == kNegInf ? 0.f : fast_exp2(m - mn);
    zrun = zrun * a + z * w;
#pragma unroll
    for (int e = 0; e < 4; ++e) orun[e] = orun[e] * a + x[e] * w;
    mrun = mn;
  };
  constexpr int kU = 16;                               // splits in flight per thread
  int k = cl;
  for (; k + (kU - 1) * 32 < nc; k += kU * 32) {
    float2 mz[kU];
    f32x4 x[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) mz[u] = *reinterpret_cast<const float2*>(ms + 2 * (k + 32 * u));
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      // the three-pass path leaves the output of an empty part unwritten
      const bool rd = !kSkipEmpty || mz[u].x != kNegInf;
      x[u] = rd ? *reinterpret_cast<const f32x4*>(po + (size_t)(k + 32 * u) * s.d)
                : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) fold(mz[u].x, mz[u].y, x[u]);
  }
  for (; k < nc; k += 32) {
    const float2 mz = *reinterpret_cast<const float2*>(ms + 2 * k);
    const bool rd = !kSkipEmpty || mz.x != kNegInf;
    fold(mz.x, mz.y, rd ? *reinterpret_cast<const f32x4*>(po + (size_t)k * s.d)
                        : f32x4{0.f, 0.f, 0.f, 0.f});
  }
  if (dq == 0) { sm_m[cl] = mrun; sm_z[cl] = zrun; }
  sm_o[cl][dq] = orun;
  if (count) {
#pragma unroll
    for (int u = 0; u < kCw; ++u) {
      nh += __popc(hw[u]);
      nv += __popc(vw[u]);
    }
    for (int x = tid + 256 * kCw; x < nwords; x += 256) {
      nh += __popc(hb[x]);
      if (vhead) nv += __popc(vbw[x]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      nh += __shfl_xor(nh, off, 64);
      nv += __shfl_xor(nv, off, 64);
    }
    if ((tid & 63) == 0) { sm_cnt[tid >> 6][0] = nh; sm_cnt[tid >> 6][1] = nv; }
  }
  __syncthreads();
  if (count && tid == 0) {
    const size_t base = (size_t)cb_ * (s.hq + s.hkv);
    kept[base + ch_] = sm_cnt[0][0] + sm_cnt[1][0] + sm_cnt[2][0] + sm_cnt[3][0];
    if (vhead) kept[base + s.hq + chk_] = sm_cnt[0][1] + sm_cnt[1][1] + sm_cnt[2][1] + sm_cnt[3][1];
  }
  if (tid < 32) {
    float M = kNegInf;
#pragma unroll 8
    for (int j = 0; j < 32; ++j) M = fmaxf(M, sm_m[j]);
    float Z = 0.f, t = 0.f;
#pragma unroll 8
    for (int j = 0; j < 32; ++j) {
      const float w = sm_m[j] == kNegInf ? 0.f : fast_exp2(sm_m[j] - M);
      Z += sm_z[j] * w;
      t += sm_o[j][tid >> 2][tid & 3] * w;
    }
    const int d = blockIdx.y * 32 + tid;
    if (d < s.d) o[(size_t)bh * s.d + d] = (OutT)(Z > 0.f ? t / Z : 0.f);
    if (blockIdx.y == 0 && tid == 0) lse[bh] = Z > 0.f ? (M + fast_log2(Z)) * kLn2 : kNegInf;
  }
}

}  // namespace

size_t decode_ws_floats(const DecodeShape& s) {
  return s.staged ? dec_stats_at(s, (size_t)s.batch * s.hq, 0, 0)
                  : dec_vbits_at(s, (size_t)s.batch * s.hkv, 0);
}

hipError_t launch_decode_combine_bf16(const DecodeShape& s, const float* ws, void* o, float* lse,
                                      int32_t* kept, hipStream_t st) {
  const dim3 grid(s.batch * s.hq, (s.d + 31) / 32);
  if (s.staged)
    hipLaunchKernelGGL((decode_combine_kernel<bf16, true>), grid, dim3(256), 0, st, s, ws,
                       (bf16*)o, lse, kept);
  else
    hipLaunchKernelGGL((decode_combine_kernel<bf16, false>), grid, dim3(256), 0, st, s, ws,
                       (bf16*)o, lse, kept);
  return hipGetLastError();
}
hipError_t launch_decode_combine_f32(const DecodeShape& s, const float* ws, float* o, float* lse,
                                     int32_t* kept, hipStream_t st) {
  hipLaunchKernelGGL((decode_combine_kernel<float, false>), dim3(s.batch * s.hq, (s.d + 31) / 32),
                     dim3(256), 0, st, s, ws, o, lse, kept);
  return hipGetLastError();
}

hipError_t launch_decode_bf16(const DecodeShape& s, const void* q, const void* kc, const void* vc,
                              const int32_t* seqlens, void* o, float* lse, float* ws,
                              int8_t* mask, int32_t* kept, hipStream_t st, int stages) {
  if (stages & kStageMain) {
    const unsigned bkv = (unsigned)(s.batch * s.hkv);
    if (s.staged) {
      const int tiles = s.n_chunks * (s.chunk / kTile);
      hipLaunchKernelGGL(decode_stats_kernel, dim3((tiles + 3) / 4, bkv), dim3(256), 0, st, s,
                         (const bf16*)q, (const bf16*)kc, seqlens, ws);
      hipLaunchKernelGGL(decode_gate_kernel, dim3(s.n_chunks, bkv), dim3(64 * s.group), 0, st, s,
                         seqlens, ws, mask);
      hipLaunchKernelGGL(decode_pv_kernel, dim3(s.n_parts, bkv), dim3(256), 0, st, s,
                         (const bf16*)q, (const bf16*)kc, (const bf16*)vc, seqlens, ws);
    } else {
      hipLaunchKernelGGL(decode_split_kernel, dim3(s.n_chunks, bkv), dim3(256), 0, st, s,
                         (const bf16*)q, (const bf16*)kc, (const bf16*)vc, seqlens, ws, mask);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kStageCombine) return launch_decode_combine_bf16(s, ws, o, lse, kept, st);
  return hipSuccess;
}

}  // namespace mala
