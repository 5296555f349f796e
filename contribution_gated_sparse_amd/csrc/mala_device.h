// Device helpers for the gfx950 (CDNA4) kernels of libmala.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mala {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309417f;

// D(32x32) += A(32x16) * B(16x32), bf16 in, fp32 accumulate.
// Lane l holds A[l%32][8(l/32)+e], B[8(l/32)+e][l%32] for e = 0..7, and
// D[8(r/4) + 4(l/32) + r%4][l%32] in accumulator register r.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// D(16x16) += A(16x32) * B(32x16). Lane l holds A[l%16][8(l/16)+e],
// B[8(l/16)+e][l%16], D[4(l/16)+r][l%16].
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of lane (l % 32) and of lane (l % 32) + 32, in every lane.
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

__device__ __forceinline__ bf16x8 load16(const void* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void store16(void* p, bf16x8 v) {
  *reinterpret_cast<bf16x8*>(p) = v;
}

// Registers loaded before a loop and read inside it: the waitcnt insertion
// does not carry "already arrived" around the loop back edge, so every use in
// the loop would wait on the vector-memory counter, which by then also counts
// the loop's own prefetches. Touching the registers once here (an empty asm
// that reads and redefines them) makes that wait happen once, before the loop.
__device__ __forceinline__ void settle(bf16x8& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void settle(float& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (bf16)0.0f;
  return z;
}

// Transposing LDS read (ds_read_b64_tr_b16). In every group of 16 lanes,
// lane j supplies the address of row (r0 + j / 4), columns c0 + 4 (j % 4) ..
// + 3 of a row-major bf16 tile; lane i then receives tile[r0 + e][c0 + i]
// for e = 0..3: four consecutive rows of one column, which is the k-major
// order an MFMA A operand needs when the tile is stored the other way round.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
__device__ __forceinline__ bf16x4 lds_read_tr_at(const bf16* p) {   // p: this lane's 8 bytes
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(__attribute__((address_space(3))) void*)(p));
  return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* tile, int stride, int r0, int c0, int j) {
  return lds_read_tr_at(tile + (r0 + (j >> 2)) * stride + c0 + 4 * (j & 3));
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return (bf16x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

}  // namespace mala

namespace mala {

// Buffer resource over [base, base + bytes): loads past the end return zeros,
// which pads ragged tiles without branches.
// Query-major grids: the (batch, query head) index bh that the workgroup at
// position p (0 <= p < B * H_q) of a row block runs. Workgroups are dealt to
// the 8 XCDs in turn. When B * H_kv is a multiple of 8, so is B * H_q, and
// p mod 8 names the workgroup's XCD: the query heads of one KV head then all
// take positions of one XCD and share its L2 for their K/V stream. Otherwise
// p is bh. A bijection on [0, B * H_q).
__device__ __forceinline__ int xcd_head(int p, int n_bkv, int group) {
  if ((n_bkv & 7) != 0) return p;
  const int x = p & 7, q = p >> 3;
  return ((q / group) * 8 + x) * group + q % group;
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ bf16x8 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// LDS-DMA: one 16-byte buffer load per lane straight into LDS. Lane l writes
// bytes [16 l, 16 l + 16) of the 1 KB block at lds (wave-uniform) with the 16
// bytes at voff of rs (zeros past the end of the buffer). The loads count in
// the vector-memory counter like any other load and complete in order with
// them; the LDS block is written when the count says so.
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, bf16* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, voff, 0, 0, 0);
}
// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0f70 | N);
}
// barrier for LDS traffic only: waits for this wave's LDS reads and writes,
// not for its loads in flight (the DMAs stay outstanding across it)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace mala
