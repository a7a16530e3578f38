// Device helpers shared by the KPool-DSA kernels: storage types, bf16 rounding, MFMA wrappers, paging.
//
// gfx950 matrix-core operand layouts used throughout (wave64; "g" = lane group):
//   16x16 family (v_mfma_f32_16x16x32_bf16: 8 bf16 per lane; v_mfma_f32_16x16x4_f32: 1 float per lane)
//     A[m][k]: lane l holds row m = l % 16, k-group g = l / 16 (4 groups)
//     B[k][n]: lane l holds col n = l % 16, k-group g = l / 16
//     D[m][n]: lane l, element i (0..3) holds row m = 4 * (l / 16) + i, col n = l % 16
//   32x32 family (v_mfma_f32_32x32x16_bf16: 8 bf16 per lane; v_mfma_f32_32x32x2_f32: 1 float per lane)
//     A[m][k]: lane l holds row m = l % 32, k-group g = l / 32 (2 groups)
//     B[k][n]: lane l holds col n = l % 32, k-group g = l / 32
//     D[m][n]: lane l, element i (0..15) holds row m = 8 * (i / 4) + 4 * (l / 32) + (i % 4), col n = l % 32
// Within a k-group the hardware pairs A's element e with B's element e, so which logical k index each
// (group, element) slot carries is ours to choose, as long as A and B agree.  The kernels pick it so every
// lane reads contiguous memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
// 16-byte staging registers.  A native vector type, not HIP's uint4 struct: copies of that struct-with-union
// can keep whole staging arrays out of registers (in scratch).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// bf16 storage is raw 16-bit patterns.
struct bf16 {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round-to-nearest-even fp32 -> bf16 (gfx950 v_cvt_pk_bf16_f32 under the default rounding mode).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two fp32 values -> two RNE bf16 in one dword (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// 2^x on the hardware exp unit (v_exp_f32, about 1 ulp; results below the normal range flush to zero).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <class T>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int kpl = 1;  // k elements per lane per MFMA
  typedef float frag;
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static float to_f32(float v) { return v; }
  __device__ __forceinline__ static float from_f32(float v) { return v; }
  __device__ __forceinline__ static frag frag_load(const float* p) { return *p; }
  __device__ __forceinline__ static frag frag_zero() { return 0.f; }
};

template <>
struct Elem<bf16> {
  static constexpr int kpl = 8;
  typedef bf16x8 frag;
  __device__ __forceinline__ static float to_f32(bf16 v) { return bf16_to_f32(v.bits); }
  __device__ __forceinline__ static bf16 from_f32(float v) { return bf16{f32_to_bf16(v)}; }
  __device__ __forceinline__ static frag frag_load(const bf16* p) { return *reinterpret_cast<const frag*>(p); }
  __device__ __forceinline__ static frag frag_zero() { return __builtin_bit_cast(frag, u32x4{0, 0, 0, 0}); }
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// One channel of a pooled index key: z_j = gate_j + ape_j, a = softmax_j(z), pooled = sum_j a_j key_j, computed in
// fp32 as key_0 + sum_j a_j (key_j - key_0) -- equal in exact arithmetic, and exactly key_0 when the pool's keys are
// equal.  kr, gr, ar point at channel c of token 0 of the pool's keys, gates and ape (stride D between tokens); gr and
// ar may be NULL (zero gate logits / zero position term; both NULL: the plain mean).  Every kernel that pools uses
// this function, so a pooled key has one value wherever it is computed.
template <class T>
__device__ __forceinline__ float pool_channel(const T* __restrict__ kr, const T* __restrict__ gr,
                                              const T* __restrict__ ar, int P, int D) {
  if (P == 4 && gr && ar) {
    // the model's pool size: every load issued before the first is used (one memory round trip, not one per
    // token), then the same operations in the same order as the loops below
    float k[4], z[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      k[j] = Elem<T>::to_f32(kr[j * D]);
      z[j] = Elem<T>::to_f32(gr[j * D]) + Elem<T>::to_f32(ar[j * D]);
    }
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) m = fmaxf(m, z[j]);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e = __expf(z[j] - m);
      den += e;
      num += e * (k[j] - k[0]);
    }
    return k[0] + num / den;
  }
  const float k0 = Elem<T>::to_f32(kr[0]);
  float den = 0.f, num = 0.f;
  if (gr && ar) {  // straight-line loops for the learned pooling
    float m = -INFINITY;
    for (int j = 0; j < P; ++j) m = fmaxf(m, Elem<T>::to_f32(gr[j * D]) + Elem<T>::to_f32(ar[j * D]));
    for (int j = 0; j < P; ++j) {
      const float e = __expf(Elem<T>::to_f32(gr[j * D]) + Elem<T>::to_f32(ar[j * D]) - m);
      den += e;
      num += e * (Elem<T>::to_f32(kr[j * D]) - k0);
    }
  } else {
    auto z = [&](int j) __attribute__((always_inline)) {
      return (gr ? Elem<T>::to_f32(gr[j * D]) : 0.f) + (ar ? Elem<T>::to_f32(ar[j * D]) : 0.f);
    };
    float m = -INFINITY;
    for (int j = 0; j < P; ++j) m = fmaxf(m, z(j));
    for (int j = 0; j < P; ++j) {
      const float e = __expf(z(j) - m);
      den += e;
      num += e * (Elem<T>::to_f32(kr[j * D]) - k0);
    }
  }
  return k0 + num / den;
}

// Row index (in units of rows of `rows_per_page` per page) of logical row `r` of sequence row `seq`.
__device__ __forceinline__ int64_t paged_row(const int32_t* __restrict__ bt, int bt_stride, int seq, int r,
                                             int log2_rows_per_page) {
  const int page = bt[int64_t(seq) * bt_stride + (r >> log2_rows_per_page)];
  return (int64_t(page) << log2_rows_per_page) + (r & ((1 << log2_rows_per_page) - 1));
}

// Order-preserving uint32 image of an fp32 score; -0.0 is mapped to +0.0 first.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Cross-lane step on the DPP paths (no LDS): `old` is what a lane keeps when its source lane is outside its 16-lane
// row.  Controls: quad_perm [1,0,3,2] = 0xB1 and [2,3,0,1] = 0x4E, row_shr:n = 0x110 + n, row_mirror = 0x140,
// row_half_mirror = 0x141.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(old), int(v), CTRL, 0xF, 0xF, false));
}

// Inclusive prefix sum over the lanes of the wave (row scans by DPP, then the row totals by readlane); `total`
// gets the wave's sum (uniform).
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t v, uint32_t& total) {
  v += dpp_u32<0x111>(0u, v);
  v += dpp_u32<0x112>(0u, v);
  v += dpp_u32<0x114>(0u, v);
  v += dpp_u32<0x118>(0u, v);  // inclusive within each 16-lane row
  const uint32_t r0 = uint32_t(__builtin_amdgcn_readlane(int(v), 15));
  const uint32_t r1 = uint32_t(__builtin_amdgcn_readlane(int(v), 31));
  const uint32_t r2 = uint32_t(__builtin_amdgcn_readlane(int(v), 47));
  const uint32_t r3 = uint32_t(__builtin_amdgcn_readlane(int(v), 63));
  const int row = (threadIdx.x & 63) >> 4;
  total = r0 + r1 + r2 + r3;
  return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// LDS byte offset of a pointer into shared memory, and a load from such an offset
__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}
template <class F>
__device__ __forceinline__ F lds_load(uint32_t off) {
  return *reinterpret_cast<__attribute__((address_space(3))) const F*>(uintptr_t(off));
}

// One wave-wide 16-byte direct load from global memory into LDS: lane l's 16 bytes at `src` land at LDS byte
// offset lds + 16 l.  Written as assembly so the compiler adds no waits of its own: callers wait with explicit
// vector-memory counts.  (The compiler's own builtin for this load makes it wait for every outstanding load --
// vmcnt(0) -- before the next barrier or LDS read, which would serialise the pipelines built on it.)  The
// instruction writes no VGPR; M0 carries the LDS offset (one wait state after it is written).
// M0 is a reserved register and the compiler does not preserve one named in a clobber list, so this is safe only
// while compiled code keeps no value of its own in M0 across these statements.  None of these kernels leads it to
// use M0 at all (no indirect register indexing, messages, GWS or append / consume LDS operations): the compiled
// code's only M0 writes are these statements', which tests/test_m0_usage.py checks on the generated assembly.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt immediate that waits until at most n vector-memory operations are outstanding (lgkm and exp free)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

}  // namespace kp

