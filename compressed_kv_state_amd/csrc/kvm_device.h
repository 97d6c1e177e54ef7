// Device helpers shared by the gfx950 kernel sources of the Key-Value Means
// layer (types, lane exchanges, MFMA wrappers, barriers).  Internal.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvm {
namespace {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kInf = __builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;

// 2^x with the hardware instruction alone (no denormal-range fix-up): softmax
// arguments are <= 8 here, and a result that would be denormal (x < -126)
// contributes nothing next to the running maximum's weight 1.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T> struct Is;
template <> struct Is<float> { static constexpr bool bf = false; };
template <> struct Is<bf16> { static constexpr bool bf = true; };

// Read-form key storage type: fp16 on the bf16 path (LayerNorm output, bounded), float on
// the fp32 path.  Read-form values (rho * u, unbounded) are stored in the input type.
template <typename T> struct Rd;
template <> struct Rd<float> { using type = float; };
template <> struct Rd<bf16> { using type = f16; };

__device__ __forceinline__ float tof(float x) { return x; }
__device__ __forceinline__ float tof(bf16 x) { return (float)x; }
__device__ __forceinline__ float tof(f16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T fromf(float x) { return (T)x; }

// Value held by the lane 32 positions away (l ^ 32).
__device__ __forceinline__ uint32_t partner_u32(uint32_t x) {
  auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}
__device__ __forceinline__ float partner_f(float x) { return __uint_as_float(partner_u32(__float_as_uint(x))); }
__device__ __forceinline__ int partner_i(int x) { return (int)partner_u32((uint32_t)x); }

// Value held by lane l ^ M (M < 32): DPP within groups of four lanes for M = 1
// and 2, a swizzle (XOR mode, no memory access) otherwise.  Every lane of the
// group of 2M lanes must be active.
template <int M>
__device__ __forceinline__ int xor_lane(int x) {
  static_assert(M > 0 && M < 32, "lane mask");
  if constexpr (M == 1) return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  else if constexpr (M == 2) return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  else return __builtin_amdgcn_ds_swizzle(x, 0x1F | (M << 10));
}
template <int M>
__device__ __forceinline__ float xor_lane(float x) { return __int_as_float(xor_lane<M>(__float_as_int(x))); }
// sum over the four lanes of a group
__device__ __forceinline__ float quad_sum(float x) {
  x += xor_lane<1>(x);
  return x + xor_lane<2>(x);
}
// Lane moves that stay in the vector ALU (no LDS round trip), for sums and
// maxima over aligned lane groups, where any pairing that joins the group's
// halves will do: DPP row_half_mirror (lane i of 8 takes lane 7 - i: joins the
// two quads), row_mirror (lane i of 16 takes lane 15 - i: joins the two
// halves of 8) and row_ror:8 (lane i of 16 takes lane i + 8 mod 16: joins
// lanes 8 apart); the two rows of 16 of each half-wave, and the two half-waves,
// are joined by the permlane swaps.  Every lane of the group must be active.
template <int CTRL, typename V>
__device__ __forceinline__ V dpp_mov(V x) {
  static_assert(sizeof(V) == 4, "32-bit lanes");
  return __builtin_bit_cast(V, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// {the value of this lane's row of 16, the value of the paired row} (rows 2r, 2r + 1)
template <typename V>
__device__ __forceinline__ void row_pair(V x, V& a, V& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  a = __builtin_bit_cast(V, (uint32_t)r[0]);
  b = __builtin_bit_cast(V, (uint32_t)r[1]);
}
template <typename V>
__device__ __forceinline__ void half_pair(V x, V& a, V& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  a = __builtin_bit_cast(V, (uint32_t)r[0]);
  b = __builtin_bit_cast(V, (uint32_t)r[1]);
}

// sum over each aligned group of P consecutive lanes (P a power of two <= 64);
// every lane of a group gets the same bits
template <int P, typename V>
__device__ __forceinline__ V group_sum(V x) {
  static_assert(P >= 1 && P <= 64 && (P & (P - 1)) == 0, "lanes per group");
  if constexpr (P >= 2) x += xor_lane<1>(x);
  if constexpr (P >= 4) x += xor_lane<2>(x);
  if constexpr (P >= 8) x += dpp_mov<0x141>(x);   // row_half_mirror
  if constexpr (P >= 16) x += dpp_mov<0x140>(x);  // row_mirror
  if constexpr (P >= 32) {
    V a, b;
    row_pair(x, a, b);
    x = a + b;
  }
  if constexpr (P >= 64) {
    V a, b;
    half_pair(x, a, b);
    x = a + b;
  }
  return x;
}

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void copy16(void* dst, const void* src) {
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}
__device__ __forceinline__ void zero16(void* dst) { *reinterpret_cast<uint4*>(dst) = make_uint4(0, 0, 0, 0); }

// Barrier that orders LDS only: each wave waits for its own LDS accesses
// (lgkmcnt(0); vmcnt and expcnt left at their maxima) and meets the others.
// Outstanding global loads and global->LDS transfers stay in flight.  (A
// release fence on LDS would make the compiler wait for every transfer in
// flight into any LDS variable; the empty asm statements keep the compiler
// from moving memory accesses across the barrier instead.)
// A pointer the whole wave shares, moved to scalar registers: memory
// instructions then take it as their scalar base plus a 32-bit per-lane
// offset instead of a 64-bit per-lane address.
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<P*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Barrier that publishes data brought in by global->LDS transfers.  Such a
// transfer writes LDS when its vector-memory counter retires, and a
// workgroup-scope barrier does not wait for vector memory on this target, so
// each wave first waits for all of its own transfers (vmcnt(0); the immediate
// leaves expcnt and lgkmcnt at their maxima).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void dma_barrier() {
  wait_vmem();
  __syncthreads();
}

// Total order on floats (NaN included) so that a rank count always selects
// exactly m items.
__device__ __forceinline__ uint32_t ordered(float x) {
  uint32_t b = __float_as_uint(x + 0.0f);  // -0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

}  // namespace
}  // namespace kvm
