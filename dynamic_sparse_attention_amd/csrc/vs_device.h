// vs_device.h — gfx950 device helpers shared by the Vertical-Slash kernels.
//
// Matrix-core tiles are 32x32 outputs (v_mfma_f32_32x32x16_bf16 for bf16
// operands, v_mfma_f32_32x32x2f32 for fp32 operands), fp32 accumulation.
// Operand and result layouts of a 32x32xK instruction on a 64-lane wave
// (KPL = k values a lane supplies, K = 2*KPL):
//   A (32 x K):  lane L holds A[L%32][(L/32)*KPL + s], s < KPL
//   B (K x 32):  lane L holds B[(L/32)*KPL + s][L%32]
//   C (32 x 32): lane L, register i holds C[8*(i/4) + 4*(L/32) + i%4][L%32]
// A result tile can feed the next product as its B operand without any data
// movement if the rows of the first product are permuted by slot_perm():
// register i of a lane then holds exactly the k slot that the B operand of
// the second product wants from that lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 64;  // query/key block (the slash granularity)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T>
struct Mfma;

template <>
struct Mfma<__bf16> {
  static constexpr int KPL = 8;
  typedef bf16x8 frag;
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // KPL consecutive fp32 values rounded (nearest-even) to one operand.
  __device__ __forceinline__ static frag pack(const float* x) {
    frag r;
#pragma unroll
    for (int s = 0; s < 8; ++s) r[s] = (__bf16)x[s];
    return r;
  }
};

template <>
struct Mfma<float> {
  static constexpr int KPL = 1;
  typedef float frag;
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag pack(const float* x) { return x[0]; }
};

// Row index (0..31) of C register i in a lane of half h = L/32.
__device__ __forceinline__ constexpr int c_row(int i, int h) { return 8 * (i / 4) + 4 * h + (i % 4); }

// slot_perm<KPL>(m): the actual row that A-operand slot m must load so that
// register i = c.. of the result is the (i/KPL)-th k chunk's element i%KPL of
// the lane's half, i.e. actual row (i/KPL)*2*KPL + h*KPL + i%KPL.
template <int KPL>
__device__ __forceinline__ constexpr int slot_perm(int m) {
  const int i = 4 * (m / 8) + (m % 4);
  const int h = (m / 4) & 1;
  return (i / KPL) * 2 * KPL + h * KPL + (i % KPL);
}

// Actual row carried by register i of a lane in half h (inverse view of slot_perm).
template <int KPL>
__device__ __forceinline__ constexpr int reg_row(int i, int h) {
  return (i / KPL) * 2 * KPL + h * KPL + (i % KPL);
}

template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag load_frag(const T* p) {
  return *reinterpret_cast<const typename Mfma<T>::frag*>(p);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding and leaves the other counters alone (gfx9 layout:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// ... and one that waits for every LDS access of this wave (lgkmcnt 0).
constexpr int lgkmcnt_wait0() { return 15 | (3 << 14) | (7 << 4); }

// 16 bytes per lane from global memory straight into LDS: lane L's bytes land
// at lds_base + 16 * L (lds_base wave-uniform).  Written as inline assembly so
// that the compiler does not track it: it would otherwise make every later
// LDS read of the same array wait for all such loads in flight, which defeats
// multi-buffering.  The caller waits for completion itself (vmcnt; the loads
// return in issue order) before reading the data.
__device__ __forceinline__ void dma_lds16(const void* gptr, const void* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds_base);
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(gptr), "{m0}"(m0) : "memory");
}

// Same, addressed as a wave-uniform 64-bit base plus a per-lane 32-bit byte
// offset (no 64-bit address arithmetic per lane), into LDS at byte address
// m0 (wave-uniform, from lds_addr()).
__device__ __forceinline__ void dma_lds16_so(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}

// LDS byte address of a pointer into a __shared__ array, wave-uniform.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p);
}

// Combine every lane's value with lane i ^ 32's (the two halves of a wave):
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second, so with both operands x the pair holds x[i] and
// x[i ^ 32] in every lane, without a round trip through LDS.  (Written as
// inline assembly: the compiler builtin returns the first register twice.)
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float half_max(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float half_sum(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return a + b;
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

// Segment layout of one batch row, in blocks, passed by value to kernels.
struct SegTable {
  int n_seg;
  int start_blk[129];  // VS_MAX_SEGMENTS + 1 block offsets
};

__device__ __forceinline__ int seg_of_block(const SegTable& st, int blk) {
  int s = 0;
  while (s + 1 < st.n_seg && st.start_blk[s + 1] <= blk) ++s;
  return s;
}

// Ordered, deterministic compaction of one flag per thread across a block of
// NT threads (NT/64 waves).  Returns this thread's slot (valid if flag) and
// writes the block total to *total.  wsum is LDS scratch of NT/64 ints.
template <int NT>
__device__ __forceinline__ int block_compact(bool flag, int* wsum, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint64_t m = __ballot(flag);
  const int inwave = __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
  if (lane == 0) wsum[wave] = __popcll(m);
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int c = wsum[w];
    before += (w < wave) ? c : 0;
    tot += c;
  }
  *total = __builtin_amdgcn_readfirstlane(tot);  // uniform: keep it (and what derives from it) scalar
  return before + inwave;
}

}  // namespace vs
