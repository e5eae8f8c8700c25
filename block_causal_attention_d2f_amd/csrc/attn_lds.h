// Shared pieces of the bf16 attention kernels (attn_bf16.hip, attn_gqa.hip):
// vector types, the LDS row swizzle, the direct HBM -> LDS loads, the LDS
// stage buffers and the tile barrier.
#pragma once

#include <type_traits>

#include "d2f_internal.h"

namespace d2f {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;
template <int V> using ic = std::integral_constant<int, V>;

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;
// s_waitcnt immediates: vmcnt(0) alone, and vmcnt(0) with lgkmcnt(0).
constexpr int kVmcntZero = 0x0F70;
constexpr int kVmLgkmZero = 0x0070;
// Largest excess (base-2 units) of a score over the running reference max
// before the reference is raised: probabilities stay below 2^kSlack.
constexpr float kSlack = 8.0f;

// Swizzle of 16-byte chunk positions within an LDS row (chunk c of row n is
// stored at position c ^ swz(n)).  The gfx950 LDS serves 256 bytes (64 banks)
// per cycle; the swizzle makes both read patterns of the kernel conflict-free
// -- the K fragment reads (ds_read_b128: 16 consecutive rows, one chunk each)
// and the transposed V reads (ds_read_b64_tr_b16: 16 rows, two adjacent
// chunks each) -- as measured with the SQ_LDS_BANK_CONFLICT counter on
// MI355X.  For the transposed reads, each group of 8 rows must spread its
// chunk pairs {2d, 2d+1} over 8 different pair positions.
//   D = 128 (256-byte rows): n -> 2 (n mod 8), with bit 3 of n adding 9 (xor).
//   D = 64 (128-byte rows, two per 256-byte bank line): n -> n & 6.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return ((row & 7) << 1) ^ (((row >> 3) & 1) * 9);
  else return row & 6;
}

// Direct 16-byte load HBM -> LDS (global_load_lds_dwordx4): lane l's bytes at
// base + voff land at LDS address lds_addr + 16 l; base and lds_addr are
// wave-uniform.  Issued as inline assembly so that the compiler, which cannot
// tell which LDS stage such a load targets, does not hold every later LDS
// read until all of them have landed; completion is awaited explicitly (the
// load counter, then a barrier) before a stage is read.  M0 carries the LDS
// address (nothing else in these kernels uses M0); an LDS DMA must not read
// M0 in the cycle after a scalar write to it, hence the s_nop.
// The nt form marks the lines non-temporal: used when every K/V tile of the
// launch is read by exactly one unit (no two query tiles share a KV head's
// keys), so the stream is not worth keeping in L2 or the Infinity Cache.
// (Measured on MI355X: the batched ragged workload's attention 128.8 ->
// 118.6 us per layer, a 32K prefix 106.0 -> 99.8 us, a 512-token prefix
// 13.3 -> 12.5 us.)
__device__ __forceinline__ void load_lds16(const void* base, int voff, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %0"
               :
               : "s"(base), "v"(voff), "s"(lds_addr)
               : "memory", "m0");
}
__device__ __forceinline__ void load_lds16_nt(const void* base, int voff, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %0 nt"
               :
               : "s"(base), "v"(voff), "s"(lds_addr)
               : "memory", "m0");
}
// One 16-byte K or V load of the tile loader; SHARED (a.remap: query tiles
// of one KV head re-read its tiles from L2) keeps the default cache policy.
// The policy is a template argument, fixed per launch: a runtime choice put a
// branch around every load of the tile loop, and the kernels instantiated
// per policy are 3-6% faster on the grouped-query shapes and up to 1% on the
// KV-read-bound ones (measured on MI355X).
template <bool SHARED>
__device__ __forceinline__ void load_kv16(const void* base, int voff, unsigned lds_addr) {
  if constexpr (SHARED) load_lds16(base, voff, lds_addr);
  else load_lds16_nt(base, voff, lds_addr);
}

// LDS stage J of the tile ring: [K tile][V tile], rows of 2D bytes.
template <int J, int BYTES>
__device__ __forceinline__ char* stage_buf() {
  __shared__ __attribute__((aligned(16))) char buf[BYTES];
  return buf;
}

// Workgroup barrier after this wave's own direct loads have landed and its
// LDS reads have returned.  The waits are explicit, so the barrier carries no
// fence of its own (a fence would also wait for the tile just issued); the
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(kVmLgkmZero);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace
}  // namespace d2f
