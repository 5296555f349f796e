// MALA forward for bf16 inputs on gfx950: the online gate (Eq. 3) inside a
// tiled flash-style loop (Algorithm 1; App. A.1 "Fused forward execution").
//
// Work decomposition
//   - one workgroup = 8 waves = 256 query rows of one (batch, query head);
//     wave w owns query rows [q0, q0 + 32), which is one decision block
//     (B_q = 32), so the keep/skip vote of a tile is a wave ballot;
//   - key tiles of B_k = 64 keys are visited from the diagonal down to tile 0;
//     K_j and V_j (both row-major) are staged in LDS and shared by the 8
//     waves, one barrier per tile. At d = 64 the LDS is double-buffered and
//     the next tile is prefetched into registers with buffer loads (zero past
//     the end of the sequence) while the current one is consumed; at d = 128
//     (the second kernel below) three LDS buffers are filled by LDS-DMA loads
//     two tiles ahead;
//   - V^T, the A operand of O^T += V^T P^T, comes from the row-major V tile
//     through transposing LDS reads (ds_read_b64_tr_b16), so V is staged
//     row-major as it is; at d = 128 the V tile is unpadded, its 16-byte
//     chunks XOR-swizzled by row (chunk c of row r at c ^ 4 (r % 4)), which
//     keeps the transposing reads conflict-free in 16 KB per tile;
//   - scores are formed transposed, S^T = K Q^T, with the 32x32x16 bf16 MFMA,
//     so each lane owns one query column: the row max and row sum are in-lane
//     reductions plus one permlane32 swap;
//   - a wave that skips a tile leaves m, l and O untouched and issues no
//     exponentials and no P V MFMAs (Algorithm 1, "skip block");
//   - scores are kept in base 2 (scale * log2 e folded into one FMA); the gate
//     is Eq. 3 multiplied by log2 e;
//   - the running max is moved lazily: only when a row max exceeds it by more
//     than kLazy (base 2), so the 64 O accumulators are rarely rescaled. The
//     pair (m, l) still represents log Z = m + log l exactly (Eq. 1).
#include <type_traits>

#include "mala_device.h"
#include "mala_internal.h"

namespace mala {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerBlock = kWaves * kRowsPerWave;   // 256
constexpr int kBK = 64;
constexpr float kLazy = 8.0f;

template <int D>
struct FwdSmem {
  // row strides (bf16): 16-byte reads of K rows (32x32x16 A layout) are
  // conflict-free at D + 8; transposing reads of V (the same layout, taken
  // down the columns) are conflict-free at D + 32
  bf16 k[2][kBK][D + 8];
  alignas(16) bf16 v[2][kBK][D + 32];
};

// d = 128: element offset of V tile row r, 8-element chunk c, in the swizzled
// layout. A transposing read of the P V product covers, per 32 lanes, rows
// r0 .. r0 + 3 (r0 a multiple of 4) and the four chunks 4 db .. 4 db + 3,
// which the swizzle spreads over all 64 banks.
__device__ __forceinline__ int v_swz(int r, int c) { return r * 128 + ((c ^ (4 * (r & 3))) << 3); }

// register-staged kernel (launched for d = 64)

template <int D>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(
    Shape s, const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int8_t* __restrict__ mask,
    int32_t* __restrict__ kept, int n_qb) {
  __shared__ FwdSmem<D> sm;
  constexpr int KT = D / 16;              // 16-wide k-steps of the QK contraction
  constexpr int DB = D / 32;              // 32-row blocks of O^T
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int RPP = kThreads / CPR;     // K rows per load pass
  constexpr int KPASS = kBK / RPP;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int bh_count = s.batch * s.hq;
  const int I = n_qb - 1 - (int)(blockIdx.x / bh_count);     // longest blocks first
  const int bh = xcd_head((int)(blockIdx.x % bh_count), s.batch * s.hkv, s.group);
  const int b = bh / s.hq, h = bh % s.hq;
  const int hk = h / s.group;
  const size_t qrow0 = ((size_t)b * s.hq + h) * (size_t)s.nq;
  const size_t krow0 = ((size_t)b * s.hkv + hk) * (size_t)s.nk;
  const int tr = (s.nq + kRowsPerWave - 1) / kRowsPerWave;
  const int tc = (s.nk + kBK - 1) / kBK;

  const int q0 = I * kRowsPerBlock + w * kRowsPerWave;
  const bool active = q0 < s.nq;
  auto top_tile = [&](int last_row) {
    const int lastkey = s.causal ? min(last_row + s.offset, s.nk - 1) : s.nk - 1;
    return lastkey / kBK;
  };
  const int top_b = top_tile(min(I * kRowsPerBlock + kRowsPerBlock - 1, s.nq - 1));
  const int top_w = active ? top_tile(min(q0 + kRowsPerWave - 1, s.nq - 1)) : -1;

  const auto qrs = make_rsrc(Q + qrow0 * D, (uint32_t)((size_t)s.nq * D * 2));
  const auto krs = make_rsrc(K + krow0 * D, (uint32_t)((size_t)s.nk * D * 2));
  const auto vrs = make_rsrc(V + krow0 * D, (uint32_t)((size_t)s.nk * D * 2));

  // Q^T as the B operand: lane (query l32, half hf) holds Q[q][16t + 8hf .. +7].
  const int q = q0 + l32;
  const bool rvalid = q < s.nq;
  bf16x8 qr[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) qr[t] = buf_load16(qrs, (uint32_t)(q * D + 16 * t + 8 * hf) * 2);
  const float c2 = s.log2_tau - fast_log2(s.causal ? (float)(q + s.offset + 1) : (float)s.nk);
  float m2 = kNegInf, lsum = 0.f;
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;

  constexpr int SV = D + 32;
  const int i16 = lane & 15, gg = lane >> 4;
  bf16x8 kreg[KPASS], vreg[KPASS];
  const int kc = tid % CPR, kr = tid / CPR;
  auto load_tile = [&](int j) {
#pragma unroll
    for (int p = 0; p < KPASS; ++p)
      kreg[p] = buf_load16(krs, (uint32_t)((j * kBK + p * RPP + kr) * D + 8 * kc) * 2);
#pragma unroll
    for (int p = 0; p < KPASS; ++p)
      vreg[p] = buf_load16(vrs, (uint32_t)((j * kBK + p * RPP + kr) * D + 8 * kc) * 2);
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int p = 0; p < KPASS; ++p) {
      store16(&sm.k[buf][p * RPP + kr][8 * kc], kreg[p]);
      store16(&sm.v[buf][p * RPP + kr][8 * kc], vreg[p]);
    }
  };

  int nkept = 0;
  if (top_b >= 0) {
    load_tile(top_b);
    store_tile(top_b & 1);
  }
#pragma unroll
  for (int t = 0; t < KT; ++t) settle(qr[t]);
  __syncthreads();

  for (int j = top_b; j >= 0; --j) {
    const int buf = j & 1;
    if (j > 0) load_tile(j - 1);

    if (active && j <= top_w) {
      // ---- score discovery: S^T[key][query], 64 keys x 32 queries
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
      // K row operands four reads ahead of their products (pinned interleave:
      // four LDS reads, then alternating product and read)
      bf16x8 ka[KT][2];
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) ka[t][kb] = load16(&sm.k[buf][32 * kb + l32][16 * t + 8 * hf]);
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sacc[kb] = mfma32(ka[t][kb], qr[t], sacc[kb]);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int u = 0; u < 2 * KT - 4; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      // ---- causal mask at the diagonal and the ragged key tail
      const int key0 = j * kBK;
      if ((key0 + kBK > s.nk) || (s.causal && key0 + kBK - 1 > q0 + s.offset)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
            const bool ok = key < s.nk && (!s.causal || key <= q + s.offset);
            if (!ok) sacc[kb][r] = kNegInf;
          }
      }
      // ---- gate, Eq. 3: skip iff rowmax(S) - m - log l < log(tau / L) for
      // every valid row with a legal key; l = 0 (nothing retained) keeps.
      float x = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) x = fmaxf(x, sacc[kb][r]);
      const float tm = max_halves(x) * s.scale_log2;
      const bool constrained = rvalid && tm > kNegInf;
      const bool row_keeps =
          constrained && (lsum == 0.f || tm - (m2 + fast_log2(lsum)) >= c2);
      const bool keep = wave_any(row_keeps);
      if (keep) {
        // ---- online softmax update and P V (Algorithm 1, kept branch)
        const bool need = tm > m2 + kLazy;
        if (wave_any(need)) {
          const float alpha = need ? fast_exp2(m2 - tm) : 1.f;
          if (need) m2 = tm;
          lsum *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
        const float mu = (m2 == kNegInf) ? 0.f : m2;
        bf16x8 pb[4];
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(sacc[kb][r], s.scale_log2, -mu));
            rs += p;
            pb[2 * kb + (r >> 3)][r & 7] = (bf16)p;
          }
        lsum += sum_halves(rs);
        // V^T element e of lane (d, hf) is key 16t + 4hf + e (e < 4) or
        // 16t + 8 + 4hf + (e - 4): the key order in which pb[t] holds P^T
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int r0 = 16 * t + 4 * hf, c0 = 32 * db + 16 * (gg & 1);
            const bf16x8 va = cat8(lds_read_tr(&sm.v[buf][0][0], SV, r0, c0, i16),
                                   lds_read_tr(&sm.v[buf][0][0], SV, r0 + 8, c0, i16));
            oacc[db] = mfma32(va, pb[t], oacc[db]);
          }
        ++nkept;
      }
      if (mask != nullptr && lane == 0)
        mask[((size_t)bh * tr + (q0 / kRowsPerWave)) * tc + j] = keep ? 1 : 0;
    }

    if (j > 0) store_tile((j - 1) & 1);
    __syncthreads();
  }

  if (!active) return;
  const int i = q0 / kRowsPerWave;
  if (mask != nullptr)
    for (int jj = top_w + 1 + lane; jj < tc; jj += 64) mask[((size_t)bh * tr + i) * tc + jj] = -1;
  if (kept != nullptr && lane == 0) kept[(size_t)bh * tr + i] = nkept;

  // ---- epilogue: O <- O / l and z = m + log l (Algorithm 1, final update)
  if (!rvalid) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  bf16* orow = O + (qrow0 + q) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 y = {(bf16)(oacc[db][4 * g + 0] * inv), (bf16)(oacc[db][4 * g + 1] * inv),
                  (bf16)(oacc[db][4 * g + 2] * inv), (bf16)(oacc[db][4 * g + 3] * inv)};
      *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * g + 4 * hf) = y;
    }
  if (hf == 0) LSE[qrow0 + q] = lsum > 0.f ? (m2 + fast_log2(lsum)) * kLn2 : kNegInf;
}


// ---------------------------------------------------------------------------
// d = 128: the same walk with the K and V tiles staged by LDS-DMA buffer loads
// (global memory straight into LDS: no registers, no LDS stores) two tiles
// ahead, in three buffers. Step j reads the pair of buffer j % 3, issues the
// DMA of tile j - 2 into the pair that held tile j + 1, and before its barrier
// waits only for tile j - 1's loads (issued one step earlier); the barrier is
// an LDS-only one, so the newest loads stay in flight across it.
//
// The buffers are six separate LDS arrays and the loop runs the steps in the
// fixed order 2, 1, 0, so each read names its array at compile time and the
// compiler's DMA wait covers only reads of the array the DMA fills. Both
// tiles are unpadded with 16-byte chunks XOR-swizzled by row: K chunk c of
// row r at c ^ (r % 16), so the 16-byte reads of 16 consecutive rows cover all
// 64 banks, and V chunk c of row r at c ^ 4 (r % 4) (v_swz).
constexpr int kD128 = 128;


__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_d128_kernel(
    Shape s, const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int8_t* __restrict__ mask,
    int32_t* __restrict__ kept, int n_qb) {
  constexpr int D = kD128;
  constexpr int KT = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = kBK * D;                       // elements per tile
  constexpr uint32_t TILE_BYTES = TILE * 2;
  __shared__ __attribute__((aligned(16))) bf16 k0[TILE], k1[TILE], k2[TILE], v0[TILE], v1[TILE], v2[TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int bh_count = s.batch * s.hq;
  const int I = n_qb - 1 - (int)(blockIdx.x / bh_count);
  const int bh = xcd_head((int)(blockIdx.x % bh_count), s.batch * s.hkv, s.group);
  const int b = bh / s.hq, h = bh % s.hq;
  const int hk = h / s.group;
  const size_t qrow0 = ((size_t)b * s.hq + h) * (size_t)s.nq;
  const size_t krow0 = ((size_t)b * s.hkv + hk) * (size_t)s.nk;
  const int tr = (s.nq + kRowsPerWave - 1) / kRowsPerWave;
  const int tc = (s.nk + kBK - 1) / kBK;

  const int q0 = I * kRowsPerBlock + w * kRowsPerWave;
  const bool active = q0 < s.nq;
  auto top_tile = [&](int last_row) {
    const int lastkey = s.causal ? min(last_row + s.offset, s.nk - 1) : s.nk - 1;
    return lastkey / kBK;
  };
  const int top_b = top_tile(min(I * kRowsPerBlock + kRowsPerBlock - 1, s.nq - 1));
  const int top_w = active ? top_tile(min(q0 + kRowsPerWave - 1, s.nq - 1)) : -1;

  const auto qrs = make_rsrc(Q + qrow0 * D, (uint32_t)((size_t)s.nq * D * 2));
  const auto krs = make_rsrc(K + krow0 * D, (uint32_t)((size_t)s.nk * D * 2));
  const auto vrs = make_rsrc(V + krow0 * D, (uint32_t)((size_t)s.nk * D * 2));

  const int q = q0 + l32;
  const bool rvalid = q < s.nq;
  bf16x8 qr[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) qr[t] = buf_load16(qrs, (uint32_t)(q * D + 16 * t + 8 * hf) * 2);
  const float c2 = s.log2_tau - fast_log2(s.causal ? (float)(q + s.offset + 1) : (float)s.nk);
  float m2 = kNegInf, lsum = 0.f;
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;

  // DMA: wave w stages rows 8w .. 8w + 7 of a tile, four per instruction;
  // lane l fills LDS chunk l % 16 of row 8w + 4p + l / 16 with global chunk
  // (l % 16) ^ swizzle(row). Every row of a visited tile is written, rows past
  // the end of the sequence as zeros (they meet P = 0).
  const int dpos = lane & 15;
  uint32_t kvo[2], vvo[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int row = 8 * w + 4 * p + (lane >> 4);
    kvo[p] = (uint32_t)(row * D + 8 * (dpos ^ (row & 15))) * 2;
    vvo[p] = (uint32_t)(row * D + 8 * (dpos ^ (4 * (row & 3)))) * 2;
  }
  auto dma_tile = [&](bf16* kd, bf16* vd, int j) {
#pragma unroll
    for (int p = 0; p < 2; ++p) dma16(krs, kd + (8 * w + 4 * p) * D, kvo[p] + (uint32_t)j * TILE_BYTES);
#pragma unroll
    for (int p = 0; p < 2; ++p) dma16(vrs, vd + (8 * w + 4 * p) * D, vvo[p] + (uint32_t)j * TILE_BYTES);
  };

  // K row reads: row 32 kb + l32, chunk 2t + hf, at (2t + hf) ^ (l32 % 16)
  const int ky = hf ^ (l32 & 15);
  // this lane's transposing-read offsets into the V tile, one per 32-column
  // block db: lane i16 of a 16-lane group reads row 16 t + 4 hf + i16 / 4
  // (+ 8), columns 32 db + 16 (gg % 2) + 4 (i16 % 4) .. + 3, i.e. chunk
  // 4 db + 2 (gg % 2) + (i16 % 4) / 2, half i16 % 2; the swizzle depends on
  // the row only through i16 / 4, so the steps t and the +8 rows are fixed
  // offsets from these
  const int i16 = lane & 15, gg = lane >> 4;
  int voff[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
    voff[db] = v_swz(4 * hf + (i16 >> 2), 4 * db + 2 * (gg & 1) + ((i16 & 3) >> 1)) + 4 * (i16 & 1);

  int nkept = 0;
  // one step of the walk at tile j, whose K and V sit in the pair j % 3
  auto step = [&](auto which, int j) {
    constexpr int P = decltype(which)::value;   // j % 3
    constexpr int PN = (P + 1) % 3;              // (j - 2) % 3
    const bf16* const kt = P == 0 ? k0 : P == 1 ? k1 : k2;
    const bf16* const vt = P == 0 ? v0 : P == 1 ? v1 : v2;
    // tile j - 2 into the pair that held tile j + 1; in the last two steps
    // tile 0 again, into a pair no step reads any more (one DMA pattern in
    // every step keeps the compiler's wait bookkeeping exact)
    dma_tile(PN == 0 ? k0 : PN == 1 ? k1 : k2, PN == 0 ? v0 : PN == 1 ? v1 : v2, max(j - 2, 0));

    if (active && j <= top_w) {
      // ---- score discovery: S^T[key][query], 64 keys x 32 queries
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
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int u = 0; u < 2 * KT - 4; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      // ---- causal mask at the diagonal and the ragged key tail
      const int key0 = j * kBK;
      if ((key0 + kBK > s.nk) || (s.causal && key0 + kBK - 1 > q0 + s.offset)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
            const bool ok = key < s.nk && (!s.causal || key <= q + s.offset);
            sacc[kb][r] = ok ? sacc[kb][r] : kNegInf;
          }
      }
      // ---- gate, Eq. 3
      float x = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) x = fmaxf(x, sacc[kb][r]);
      const float tm = max_halves(x) * s.scale_log2;
      const bool constrained = rvalid && tm > kNegInf;
      const bool row_keeps =
          constrained && (lsum == 0.f || tm - (m2 + fast_log2(lsum)) >= c2);
      const bool keep = wave_any(row_keeps);
      if (keep) {
        const bool need = tm > m2 + kLazy;
        if (wave_any(need)) {
          const float alpha = need ? fast_exp2(m2 - tm) : 1.f;
          if (need) m2 = tm;
          lsum *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
        const float mu = (m2 == kNegInf) ? 0.f : m2;
        bf16x8 pb[4];
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(sacc[kb][r], s.scale_log2, -mu));
            rs += p;
            pb[2 * kb + (r >> 3)][r & 7] = (bf16)p;
          }
        lsum += sum_halves(rs);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x8 va = cat8(lds_read_tr_at(vt + voff[db] + 16 * t * D),
                                   lds_read_tr_at(vt + voff[db] + (16 * t + 8) * D));
            oacc[db] = mfma32(va, pb[t], oacc[db]);
          }
        ++nkept;
      }
      if (mask != nullptr && lane == 0)
        mask[((size_t)bh * tr + (q0 / kRowsPerWave)) * tc + j] = keep ? 1 : 0;
    }
    // tile j - 1's DMAs (issued one step back) have landed once at most
    // this step's four remain
    wait_vm<4>();
    lds_barrier();
  };

  if (top_b >= 0) {
    // the walk starts at the first tile at or above the top with j % 3 == 2
    // (at most two tiles past the top, which no wave reaches), so that the
    // steps run in the fixed buffer order 2, 1, 0
    const int j0 = top_b + (2 - top_b % 3);
    dma_tile(k2, v2, j0);
    dma_tile(k1, v1, j0 - 1);
#pragma unroll
    for (int t = 0; t < KT; ++t) settle(qr[t]);
    wait_vm<0>();
    __syncthreads();
    for (int j = j0; j >= 2; j -= 3) {
      step(std::integral_constant<int, 2>(), j);
      step(std::integral_constant<int, 1>(), j - 1);
      step(std::integral_constant<int, 0>(), j - 2);
    }
    wait_vm<0>();
  }

  if (!active) return;
  const int i = q0 / kRowsPerWave;
  if (mask != nullptr)
    for (int jj = top_w + 1 + lane; jj < tc; jj += 64) mask[((size_t)bh * tr + i) * tc + jj] = -1;
  if (kept != nullptr && lane == 0) kept[(size_t)bh * tr + i] = nkept;

  // ---- epilogue: O <- O / l and z = m + log l (Algorithm 1, final update)
  if (!rvalid) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  bf16* orow = O + (qrow0 + q) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 y = {(bf16)(oacc[db][4 * g + 0] * inv), (bf16)(oacc[db][4 * g + 1] * inv),
                  (bf16)(oacc[db][4 * g + 2] * inv), (bf16)(oacc[db][4 * g + 3] * inv)};
      *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * g + 4 * hf) = y;
    }
  if (hf == 0) LSE[qrow0 + q] = lsum > 0.f ? (m2 + fast_log2(lsum)) * kLn2 : kNegInf;
}

}  // namespace

hipError_t launch_fwd_bf16(const Shape& s, const void* q, const void* k, const void* v, void* o,
                           float* lse, int8_t* mask, int32_t* kept, hipStream_t st) {
  const int n_qb = (s.nq + kRowsPerBlock - 1) / kRowsPerBlock;
  const dim3 grid((unsigned)(n_qb * s.batch * s.hq));
  if (grid.x == 0) return hipSuccess;
  if (s.d == 128)
    hipLaunchKernelGGL(fwd_bf16_d128_kernel, grid, dim3(kThreads), 0, st, s, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, (bf16*)o, lse, mask, kept, n_qb);
  else
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, grid, dim3(kThreads), 0, st, s, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, (bf16*)o, lse, mask, kept, n_qb);
  return hipGetLastError();
}

}  // namespace mala
