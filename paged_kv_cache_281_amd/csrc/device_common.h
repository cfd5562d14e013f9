// Device-side helpers for the gfx950 kernels: raw vector types, element traits,
// MFMA / dot2 wrappers and wave-level shuffles.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>
#include <type_traits>

namespace pkv {

typedef unsigned int u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

// exp2 on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Reductions across the four 16-lane rows of a wave with the gfx950 lane-swap
// instructions (no LDS traffic).  xor16: rows (0,1) and (2,3); xor32: rows (0,2), (1,3).
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Reductions within each 16-lane row through DPP: partners lane^15, lane^7, lane^3,
// lane^1 (row mirror, half-row mirror, two quad permutations) span the row.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<0x140>(v));  // row_mirror
  v = fmaxf(v, dpp<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp<0x1B>(v));   // quad_perm [3,2,1,0]
  v = fmaxf(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
  return v;
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<0x140>(v);
  v += dpp<0x141>(v);
  v += dpp<0x1B>(v);
  v += dpp<0xB1>(v);
  return v;
}

// True in every lane when `pred` holds in any active lane (wave-uniform).
__device__ __forceinline__ bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }
__device__ __forceinline__ float shfl_idx(float v, int src) { return __shfl(v, src, 64); }
__device__ __forceinline__ u32 shfl_idx_u(u32 v, int src) {
  return static_cast<u32>(__shfl(static_cast<int>(v), src, 64));
}

// Element traits.  Storage is handled as raw bits; arithmetic is fp32.
struct BF16 {
  static constexpr int kBytes = 2;
  typedef uint16_t Bits;
  __device__ static __forceinline__ u32 pack2(float a, float b) {
    bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(u32, v);
  }
  __device__ static __forceinline__ float lo(u32 w) { return __uint_as_float(w << 16); }
  __device__ static __forceinline__ float hi(u32 w) { return __uint_as_float(w & 0xffff0000u); }
  __device__ static __forceinline__ float dot2(u32 a, u32 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
  }
  // 16x16x32 MFMA, A/B = 8 elements per lane
  __device__ static __forceinline__ f32x4 mfma_k32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // 16x16x16 MFMA, A/B = 4 elements per lane
  __device__ static __forceinline__ f32x4 mfma_k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ Bits from_float(float f) {
    return __builtin_bit_cast(Bits, static_cast<__bf16>(f));
  }
};

struct F16 {
  static constexpr int kBytes = 2;
  typedef uint16_t Bits;
  __device__ static __forceinline__ u32 pack2(float a, float b) {
    f16x2 v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
    return __builtin_bit_cast(u32, v);
  }
  __device__ static __forceinline__ float lo(u32 w) {
    return static_cast<float>(__builtin_bit_cast(f16x2, w)[0]);
  }
  __device__ static __forceinline__ float hi(u32 w) {
    return static_cast<float>(__builtin_bit_cast(f16x2, w)[1]);
  }
  __device__ static __forceinline__ float dot2(u32 a, u32 b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
  }
  __device__ static __forceinline__ f32x4 mfma_k32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 mfma_k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ Bits from_float(float f) {
    return __builtin_bit_cast(Bits, static_cast<_Float16>(f));
  }
};

struct F32 {
  static constexpr int kBytes = 4;
  typedef float Bits;
  __device__ static __forceinline__ Bits from_float(float f) { return f; }
};

// Runs load/compute over units w, w+NW, w+2*NW, ... < nunits with two register
// buffers: while unit i is computed, unit i+1 is in flight.  The scheduling fences
// keep each prefetch issued before the compute it overlaps.  The caller has already
// issued the loads of the first unit into A.
#define PKV_FENCE() __builtin_amdgcn_sched_barrier(0)
template <int NW, class Buf, class Load, class Compute>
__device__ __forceinline__ void pipeline2(int w, int nunits, Buf& A, Load&& load, Compute&& compute) {
  const int n = nunits > w ? (nunits - w + NW - 1) / NW : 0;
  Buf B;
  int i = 0;
  for (; i + 2 < n; i += 2) {
    const int u = w + i * NW;
    load(u + NW, B);
    PKV_FENCE();
    compute(u, A);
    PKV_FENCE();
    load(u + 2 * NW, A);
    PKV_FENCE();
    compute(u + NW, B);
    PKV_FENCE();
  }
  const int u = w + i * NW;
  if (n - i == 2) {
    load(u + NW, B);
    PKV_FENCE();
    compute(u, A);
    PKV_FENCE();
    compute(u + NW, B);
  } else if (n - i == 1) {
    compute(u, A);
  }
}

// The same with a runtime stride: units start, start + stride, ... < nunits.
template <class Buf, class Load, class Compute>
__device__ __forceinline__ void pipeline2s(int start, int stride, int nunits, Buf& A, Load&& load,
                                           Compute&& compute) {
  const int n = nunits > start ? (nunits - start + stride - 1) / stride : 0;
  Buf B;
  int i = 0;
  for (; i + 2 < n; i += 2) {
    const int u = start + i * stride;
    load(u + stride, B);
    PKV_FENCE();
    compute(u, A);
    PKV_FENCE();
    load(u + 2 * stride, A);
    PKV_FENCE();
    compute(u + stride, B);
    PKV_FENCE();
  }
  const int u = start + i * stride;
  if (n - i == 2) {
    load(u + stride, B);
    PKV_FENCE();
    compute(u, A);
    PKV_FENCE();
    compute(u + stride, B);
  } else if (n - i == 1) {
    compute(u, A);
  }
}

// Block tables.  Flat (Tab = int or uint16_t): entry j of sequence b is
// tables[b * W + j].  Two-level (Tab = TwoLevel): the sequence's row of the directory,
// dir[b * (W / LEAF) ..], names for every run of LEAF entries the leaf that holds them,
// and leaf l is the int32 entries tables[l * LEAF .. l * LEAF + LEAF).  table_row
// returns the address of entry e of sequence b; entries up to the end of e's leaf (or
// row) follow it.  Two-level lookups cost one more (scalar) load.
struct TwoLevel {};
template <class Tab> struct TabEntry { typedef Tab type; };
template <> struct TabEntry<TwoLevel> { typedef int type; };

template <class Tab, int LEAF>
__device__ __forceinline__ const typename TabEntry<Tab>::type* table_row(const void* tables, const int* dir, int b,
                                                                         int W, int e) {
  if constexpr (std::is_same<Tab, TwoLevel>::value) {
    const int leaf = dir[static_cast<int64_t>(b) * (W / LEAF) + e / LEAF];
    return static_cast<const int*>(tables) + static_cast<int64_t>(leaf) * LEAF + e % LEAF;
  } else {
    return static_cast<const Tab*>(tables) + static_cast<int64_t>(b) * W + e;
  }
}

// Entry e of sequence b's table loaded through the scalar cache (b and e must be
// uniform over the wave): 32-bit entries (flat int32 or two-level) are read from the
// constant address space, so the load is counted apart from the vector-memory loads in
// flight; 16-bit entries use an ordinary load.
template <class Tab, int LEAF>
__device__ __forceinline__ int table_entry_uniform(const void* tables, const int* dir, int b, int W, int e) {
  typedef const __attribute__((address_space(4))) int* cint;
  if constexpr (std::is_same<Tab, TwoLevel>::value) {
    const int leaf = ((cint)(dir))[static_cast<int64_t>(b) * (W / LEAF) + e / LEAF];
    return ((cint)(static_cast<const int*>(tables)))[static_cast<int64_t>(leaf) * LEAF + e % LEAF];
  } else if constexpr (std::is_same<Tab, int>::value) {
    return ((cint)(static_cast<const int*>(tables)))[static_cast<int64_t>(b) * W + e];
  } else {
    return static_cast<int>(*table_row<Tab, LEAF>(tables, dir, b, W, e));
  }
}

}  // namespace pkv
