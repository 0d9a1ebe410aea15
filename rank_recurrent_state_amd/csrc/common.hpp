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

// ---- stochastic rounding ------------------------------------------------------------------------
// Random bits: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
// 1, 2, 3", SC'11): ten rounds, each two 32 x 32 -> 64-bit products of counter words 0 and 2 with
// the round multipliers, the halves recombined with words 1 and 3 and the key; the key is bumped
// by the Weyl increments between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u, kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    if (i > 0) {
      k0 += kW0;
      k1 += kW1;
    }
    const uint32_t hi0 = __umulhi(kM0, c.x), lo0 = kM0 * c.x;
    const uint32_t hi1 = __umulhi(kM1, c.z), lo1 = kM1 * c.z;
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// Store sites of the factors (part of the random-number counter).
enum SrSite : uint32_t {
  kSiteDecodeU = 0, kSiteDecodeV = 1, kSiteCompressU = 2, kSiteCompressV = 3,
  kSiteFromDenseU = 4, kSiteFromDenseV = 5, kSiteFoldU = 6
};

// The Philox output of one group of eight consecutive elements of a stored column: key
// (rng_key, 0), counter (element / 8, site << 16 | aux << 8 | slot, unit, window count).
__device__ __forceinline__ uint4 sr_group(uint32_t rng_key, uint32_t site, uint32_t aux, int slot, int64_t unit,
                                          uint32_t window, int elem) {
  const uint4 c = make_uint4(static_cast<uint32_t>(elem) >> 3, (site << 16) | (aux << 8) | static_cast<uint32_t>(slot),
                             static_cast<uint32_t>(unit), window);
  return philox4x32_10(c, rng_key, 0u);
}

// The 16-bit draw of element e (0..7) of a group: half (e % 2) of word e / 2.
__device__ __forceinline__ uint32_t draw16(const uint4& w, int e) {
  const uint32_t x = (e >> 1) == 0 ? w.x : ((e >> 1) == 1 ? w.y : ((e >> 1) == 2 ? w.z : w.w));
  return (e & 1) ? (x >> 16) : (x & 0xffffu);
}

// Stochastic rounding of x to the 16-bit format DT with the draw r (0 .. 65535): the neighbour
// away from zero is taken exactly when r < 65536 f, f the fractional distance of x from its
// neighbour towards zero. Every step below is exact in fp32.
template <int DT> __device__ __forceinline__ uint16_t round_sr(float x, uint32_t r);
template <> __device__ __forceinline__ uint16_t round_sr<1>(float x, uint32_t r) {
  // bf16 is the upper half of the fp32 encoding: f = (low half) / 65536
  const uint32_t b = __float_as_uint(x);
  return static_cast<uint16_t>((b >> 16) + (r < (b & 0xffffu) ? 1u : 0u));
}
template <> __device__ __forceinline__ uint16_t round_sr<2>(float x, uint32_t r) {
  // the neighbour towards zero by the round-towards-zero conversion, the other one a unit of
  // the last place further out (65504 rounds to itself: its outer neighbour is the infinity)
  const auto h2 = __builtin_amdgcn_cvt_pkrtz(x, 0.f);
  const uint16_t lo = __builtin_bit_cast(uint16_t, h2[0]);
  const float flo = static_cast<float>(h2[0]);
  const float fhi = f16_to_f32(static_cast<uint16_t>(lo + 1u));
  const float d = fabsf(x) - fabsf(flo);             // exact (the two are within a factor 2)
  const float span = fabsf(fhi) - fabsf(flo);        // a power of two, or infinite
  return (static_cast<float>(r) * span < d * 65536.f) ? static_cast<uint16_t>(lo + 1u) : lo;
}

// Store N fp32 values as the 16-bit format DT with stochastic rounding; r[e] is element e's draw.
template <int DT, int N>
__device__ __forceinline__ void store_sr(stor_t<DT>* __restrict__ p, const float (&in)[N], const uint32_t (&r)[N]) {
  static_assert(DT == 1 || DT == 2, "stochastic rounding stores 16-bit formats");
  if constexpr (N == 1) {
    p[0] = round_sr<DT>(in[0], r[0]);
  } else {
    static_assert(N % 2 == 0, "16-bit vector width");
    uint32_t w[N / 2];
#pragma unroll
    for (int e = 0; e < N / 2; ++e)
      w[e] = static_cast<uint32_t>(round_sr<DT>(in[2 * e], r[2 * e])) |
             (static_cast<uint32_t>(round_sr<DT>(in[2 * e + 1], r[2 * e + 1])) << 16);
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
