// Device helpers shared by the gfx950 kernels of libseed: storage types, 16-byte vector
// loads/stores with conversion to fp32, and cross-lane sums inside a 64-wide wavefront.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace seed {

constexpr int kWave = 64;

// Storage type for a dtype code (0 = fp32, 1 = bf16 and 2 = IEEE fp16, both held as raw
// 16-bit words).
template <int DT> struct Stor;
template <> struct Stor<0> { using T = float; };
template <> struct Stor<1> { using T = uint16_t; };
template <> struct Stor<2> { using T = uint16_t; };
template <int DT> using stor_t = typename Stor<DT>::T;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Round to nearest even (v_cvt_f16_f32 in the default rounding mode); beyond the fp16 range the
// result is an infinity.
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

template <int DT> __device__ __forceinline__ float to_f32(stor_t<DT> x);
template <> __device__ __forceinline__ float to_f32<0>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<1>(uint16_t x) { return bf16_to_f32(x); }
template <> __device__ __forceinline__ float to_f32<2>(uint16_t x) { return f16_to_f32(x); }

template <int DT> __device__ __forceinline__ stor_t<DT> from_f32(float x);
template <> __device__ __forceinline__ float from_f32<0>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t from_f32<1>(float x) { return f32_to_bf16(x); }
template <> __device__ __forceinline__ uint16_t from_f32<2>(float x) { return f32_to_f16(x); }

// The two 16-bit elements of a 32-bit word (element 0 in the low half) of dtype DT (1 or 2),
// and the word two values round to.
template <int DT> __device__ __forceinline__ float lo16(uint32_t w) {
  if constexpr (DT == 1) return __uint_as_float(w << 16);
  else return f16_to_f32(static_cast<uint16_t>(w & 0xffffu));
}
template <int DT> __device__ __forceinline__ float hi16(uint32_t w) {
  if constexpr (DT == 1) return __uint_as_float(w & 0xffff0000u);
  else return f16_to_f32(static_cast<uint16_t>(w >> 16));
}
template <int DT> __device__ __forceinline__ uint32_t pack2(float a, float b) {
  return static_cast<uint32_t>(from_f32<DT>(a)) | (static_cast<uint32_t>(from_f32<DT>(b)) << 16);
}

// Load N consecutive elements of storage dtype DT into fp32 registers. N * sizeof(T) must be
// a multiple of 4 and the address aligned to it; wide accesses are used where possible.
template <int DT, int N>
__device__ __forceinline__ void load_f32(const stor_t<DT>* __restrict__ p, float (&out)[N]) {
  if constexpr (DT == 0) {
    static_assert(N % 4 == 0 || N == 1 || N == 2, "fp32 vector width");
    if constexpr (N % 4 == 0) {
#pragma unroll
      for (int c = 0; c < N / 4; ++c) {
        float4 v = reinterpret_cast<const float4*>(p)[c];
        out[4 * c + 0] = v.x; out[4 * c + 1] = v.y; out[4 * c + 2] = v.z; out[4 * c + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < N; ++e) out[e] = p[e];
    }
  } else if constexpr (N == 1) {
    out[0] = to_f32<DT>(p[0]);
  } else {
    static_assert(N % 2 == 0, "16-bit vector width");
    if constexpr (N % 8 == 0) {
#pragma unroll
      for (int c = 0; c < N / 8; ++c) {
        uint4 v = reinterpret_cast<const uint4*>(p)[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          out[8 * c + 2 * e] = lo16<DT>(w[e]);
          out[8 * c + 2 * e + 1] = hi16<DT>(w[e]);
        }
      }
    } else if constexpr (N % 4 == 0) {
#pragma unroll
      for (int c = 0; c < N / 4; ++c) {
        uint2 v = reinterpret_cast<const uint2*>(p)[c];
        out[4 * c + 0] = lo16<DT>(v.x);
        out[4 * c + 1] = hi16<DT>(v.x);
        out[4 * c + 2] = lo16<DT>(v.y);
        out[4 * c + 3] = hi16<DT>(v.y);
      }
    } else {
#pragma unroll
      for (int c = 0; c < N / 2; ++c) {
        uint32_t v = reinterpret_cast<const uint32_t*>(p)[c];
        out[2 * c] = lo16<DT>(v);
        out[2 * c + 1] = hi16<DT>(v);
      }
    }
  }
}

// Store N fp32 values as storage dtype DT (bf16, fp16: round to nearest even).
template <int DT, int N>
__device__ __forceinline__ void store_f32(stor_t<DT>* __restrict__ p, const float (&in)[N]) {
  if constexpr (DT == 0) {
    if constexpr (N % 4 == 0) {
#pragma unroll
      for (int c = 0; c < N / 4; ++c)
        reinterpret_cast<float4*>(p)[c] =
            make_float4(in[4 * c], in[4 * c + 1], in[4 * c + 2], in[4 * c + 3]);
    } else {
#pragma unroll
      for (int e = 0; e < N; ++e) p[e] = in[e];
    }
  } else if constexpr (N == 1) {
    p[0] = from_f32<DT>(in[0]);
  } else {
    static_assert(N % 2 == 0, "16-bit vector width");
    uint32_t w[N / 2];
#pragma unroll
    for (int e = 0; e < N / 2; ++e) w[e] = pack2<DT>(in[2 * e], in[2 * e + 1]);
    if constexpr (N % 8 == 0) {
#pragma unroll
      for (int c = 0; c < N / 8; ++c)
        reinterpret_cast<uint4*>(p)[c] = make_uint4(w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]);
    } else if constexpr (N % 4 == 0) {
#pragma unroll
      for (int c = 0; c < N / 4; ++c) reinterpret_cast<uint2*>(p)[c] = make_uint2(w[2 * c], w[2 * c + 1]);
    } else {
#pragma unroll
      for (int c = 0; c < N / 2; ++c) reinterpret_cast<uint32_t*>(p)[c] = w[c];
    }
  }
}

// ---- cross-lane sums -------------------------------------------------------------------------
// DPP controls: quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2),
// row_half_mirror (i <-> 7 - i inside 8 lanes), row_mirror (i <-> 15 - i inside 16 lanes).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of W consecutive lanes; every lane of a group gets the group's sum.
// Must be called with all 64 lanes active.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "group width");
  if constexpr (W >= 2) v += dpp<0xB1>(v);
  if constexpr (W >= 4) v += dpp<0x4E>(v);
  if constexpr (W >= 8) v += dpp<0x141>(v);
  if constexpr (W >= 16) v += dpp<0x140>(v);
  if constexpr (W >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (W >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// Sum over lanes that share (lane % W): i.e. across the 64 / W groups of width W.
template <int W>
__device__ __forceinline__ float across_groups_sum(float v) {
  if constexpr (W <= 1) v += __shfl_xor(v, 1, 64);
  if constexpr (W <= 2) v += __shfl_xor(v, 2, 64);
  if constexpr (W <= 4) v += __shfl_xor(v, 4, 64);
  if constexpr (W <= 8) v += __shfl_xor(v, 8, 64);
  if constexpr (W <= 16) v += __shfl_xor(v, 16, 64);
  if constexpr (W <= 32) v += __shfl_xor(v, 32, 64);
  return v;
}

// v_permlane32_swap: lanes 32..63 of x trade places with lanes 0..31 of y.
__device__ __forceinline__ void lane_swap32(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}

// v_permlane16_swap: the odd 16-lane rows of x trade places with the even rows of y.
__device__ __forceinline__ void lane_swap16(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}

// Sum over all 64 lanes; every lane gets it.
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  float x = v, y = v;
  lane_swap16(x, y);
  v = x + y;
  x = v;
  y = v;
  lane_swap32(x, y);
  return x + y;
}

// Orders LDS traffic between lanes of one wavefront (LDS operations of a wave execute in
// order; this keeps the compiler from moving them across the exchange point).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace seed
