// Device helpers shared by the gfx950 kernels: 16-byte vectors, streaming
// (non-temporal) accesses, the trapezoid weight, and bf16/f32 conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan_internal.h"

namespace tdp {

// 16-byte vector as a native clang vector: HIP's uint4 wrapper (a union)
// keeps arrays of it out of registers, which would serialize the loads.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming accesses: every byte is read once and written once, and the
// written tiles are consumed only after the denoiser has run, so loads and
// stores carry the non-temporal hint (they do not displace other data in
// L2 and the Infinity Cache).
template <typename T>
__device__ inline T ld_nt(const T* p) { return __builtin_nontemporal_load(p); }
template <typename T>
__device__ inline void st_nt(T* p, T v) { __builtin_nontemporal_store(v, p); }

// 1-D trapezoid of tile i of n (`size` cells, overlap o) at local cell l:
// (l+1)/(o+1) on a left ramp, (size-l)/(o+1) on a right ramp, 1 elsewhere.
// The kernels run guarded plans only (size >= 2o), where the two ramps never
// meet, so one division with the numerator chosen per case gives every
// value ((o+1)/(o+1) is exactly 1).  fp32 division is built correctly
// rounded, so each value equals the host plan's window bit for bit.
__device__ inline float ramp(int n, int o, int i, int l, int size) {
  const int num = (i > 0 && l < o) ? l + 1 : (i < n - 1 && l >= size - o) ? size - l : o + 1;
  return (float)num / (float)(o + 1);
}
__device__ inline float ramp_weight(const AxisSplit& ax, int i, int l, int size) {
  return ramp(ax.n, ax.o, i, l, size);
}

// ---------------------------------------------------------------------------
// bf16 / f32 vectors
// ---------------------------------------------------------------------------

template <int IN>  // IN = TDP_BF16 or TDP_F32
struct InVec;
template <>
struct InVec<TDP_BF16> {
  static constexpr int E = 8;
  __device__ static inline void unpack(const u32x4& v, float* x) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <>
struct InVec<TDP_F32> {
  static constexpr int E = 4;
  __device__ static inline void unpack(const u32x4& v, float* x) {
    x[0] = __uint_as_float(v.x);
    x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z);
    x[3] = __uint_as_float(v.w);
  }
};

// fp32 -> bf16, round to nearest even: gfx950's packed conversion
// (v_cvt_pk_bf16_f32) converts two values per instruction.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

// Store E accumulated floats as the output dtype at element offset `e`.
template <int OUT, int E>
__device__ inline void store_out(void* out, int64_t e, const float* acc);
template <>
__device__ inline void store_out<TDP_BF16, 8>(void* out, int64_t e, const float* a) {
  u32x4 v;
  v.x = pack_bf16x2(a[0], a[1]);
  v.y = pack_bf16x2(a[2], a[3]);
  v.z = pack_bf16x2(a[4], a[5]);
  v.w = pack_bf16x2(a[6], a[7]);
  st_nt(reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + e), v);
}
template <>
__device__ inline void store_out<TDP_BF16, 4>(void* out, int64_t e, const float* a) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  u32x2 v;
  v.x = pack_bf16x2(a[0], a[1]);
  v.y = pack_bf16x2(a[2], a[3]);
  st_nt(reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + e), v);
}
template <>
__device__ inline void store_out<TDP_F32, 8>(void* out, int64_t e, const float* a) {
  f32x4* o = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + e);
  st_nt(o, f32x4{a[0], a[1], a[2], a[3]});
  st_nt(o + 1, f32x4{a[4], a[5], a[6], a[7]});
}
template <>
__device__ inline void store_out<TDP_F32, 4>(void* out, int64_t e, const float* a) {
  st_nt(reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + e), f32x4{a[0], a[1], a[2], a[3]});
}

// Which elements of a row lane vv handles, for a kernel that reads a tile
// row of IN and writes an output row of OUT, V 16-byte input vectors per
// row.  By default lane vv takes input vector vv (elements [E*vv, E*vv+E)).
// `idx` is the vector index of (row, vv) in `t`; `row` the output row.
template <int IN, int OUT>
struct LaneIO {
  static constexpr int E = InVec<IN>::E;
  __device__ static inline u32x4 load(const u32x4* t, int64_t idx, int vv, int V) { return ld_nt(t + idx); }
  __device__ static inline void store(void* out, int64_t row, int vv, int V, const float* a) {
    store_out<OUT, E>(out, (row * V + vv) * (int64_t)E, a);
  }
  // The q-th 4-float group of the lane's elements in an fp32 row buffer.
  __device__ static inline f32x4* quad(float* acc, int64_t row, int vv, int V, int q) {
    return reinterpret_cast<f32x4*>(acc + (row * V + vv) * (int64_t)E) + q;
  }
};
// bf16 in, fp32 out: 32 output bytes per input vector.  Lane vv takes the
// 8-byte pieces vv and V + vv instead (elements [4vv, 4vv+4) and
// [4V+4vv, 4V+4vv+4)), so that each load and each fp32 store instruction of
// a wave covers one contiguous span rather than every other 16 bytes.
template <>
struct LaneIO<TDP_BF16, TDP_F32> {
  static constexpr int E = 8;
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  __device__ static inline u32x4 load(const u32x4* t, int64_t idx, int vv, int V) {
    const u32x2* r = reinterpret_cast<const u32x2*>(t + (idx - vv));
    const u32x2 a = ld_nt(r + vv), b = ld_nt(r + V + vv);
    return u32x4{a.x, a.y, b.x, b.y};
  }
  __device__ static inline void store(void* out, int64_t row, int vv, int V, const float* a) {
    f32x4* o = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + row * 8 * V);
    st_nt(o + vv, f32x4{a[0], a[1], a[2], a[3]});
    st_nt(o + V + vv, f32x4{a[4], a[5], a[6], a[7]});
  }
  __device__ static inline f32x4* quad(float* acc, int64_t row, int vv, int V, int q) {
    return reinterpret_cast<f32x4*>(acc + row * 8 * V) + (q ? V : 0) + vv;
  }
};

}  // namespace tdp
