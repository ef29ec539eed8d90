// Rotary position embedding at GLOBAL token positions, alone or folded into
// the zigzag permute.  Under context parallelism every rank rotates its
// tokens by their place in the whole sequence, which is why each rank must
// know the global offset of its segment ("序列与上下文并行", section 工程实践).
// The frequencies follow the sinusoidal table of "Tensor并行与算子拆分"
// (model code, PositionalEncoding): theta_k = base^(-2k/D).  Pair k holds
// elements (2k, 2k+1) (interleaved) or (k, k + D/2) (half split) and is
// rotated by phi = pos * theta_k:
//     y_a = x_a cos(phi) - x_b sin(phi),   y_b = x_a sin(phi) + x_b cos(phi).
//
// Precision: phi reaches ~1e6 rad at million-token positions, far beyond
// what a float32 product can hold to 1e-3 rad.  The angle is therefore formed
// in float64 as a fraction of a turn, pos * theta_k / (2 pi), reduced to
// [-1/2, 1/2] turns, and only that small remainder goes to float32 sincospi.
// The rotation itself is float32 (fma); bf16 results are rounded to nearest
// even.
//
// Layout: one thread owns 4 pairs of one token position and applies the same
// cos/sin to that position's rows in all B*H heads, so the angles are computed
// once per position.  Consecutive threads cover consecutive 16-byte pieces of
// a row and then consecutive rows, so loads and stores are coalesced.  The
// kernel is HBM-bound: it reads and writes each element once.
#include "cpa_internal.h"

#include <cmath>
#include <cstdint>

namespace cpa {
namespace {

__device__ __forceinline__ void load4(const __bf16* p, float (&v)[4]) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(u.x << 16);
  v[1] = __uint_as_float(u.x & 0xffff0000u);
  v[2] = __uint_as_float(u.y << 16);
  v[3] = __uint_as_float(u.y & 0xffff0000u);
}
__device__ __forceinline__ void load4(const float* p, float (&v)[4]) {
  const float4 u = *reinterpret_cast<const float4*>(p);
  v[0] = u.x;
  v[1] = u.y;
  v[2] = u.z;
  v[3] = u.w;
}
__device__ __forceinline__ void store4(__bf16* p, const float (&v)[4]) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 o = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
  *reinterpret_cast<bf16x4*>(p) = o;
}
__device__ __forceinline__ void store4(float* p, const float (&v)[4]) {
  *reinterpret_cast<float4*>(p) = float4{v[0], v[1], v[2], v[3]};
}

// Index space (rr, t, g): rr < nr rows of the position table, t < Lr
// positions per table row, g < D/8 groups of 4 pairs.  Position
// p = pos[rr * Lr + t].  Source row of head bh: gather ? bh*L + p (global
// order) : (rr*BH + bh)*Lr + t (same layout as the destination); destination
// row (rr*BH + bh)*Lr + t.
template <typename T, bool HALF>
__global__ __launch_bounds__(256) void rope_kernel(const T* src, T* dst,  // may alias (in place)
                                                   int64_t BH, int64_t L, int64_t Lr, int64_t nr,
                                                   int D, const int64_t* __restrict__ pos,
                                                   int gather, double log2_base) {
  const int G = D / 8;
  const int64_t n = nr * Lr * G;
  constexpr double INV_2PI = 0.15915494309189533577;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int g = (int)(i % G);
    const int64_t rest = i / G;
    const int64_t t = rest % Lr;
    const int64_t rr = rest / Lr;
    const int64_t p = pos[rr * Lr + t];
    float c[4], s[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = 4 * g + j;
      const double theta = exp2(-(2.0 * k / D) * log2_base);
      const double turns = (double)p * theta * INV_2PI;
      const double frac = turns - rint(turns);  // [-1/2, 1/2] turns
      sincospif((float)(2.0 * frac), &s[j], &c[j]);
    }
    // element offsets of the two 4-element pieces inside a row
    const int a0 = HALF ? 4 * g : 8 * g;
    const int b0 = HALF ? 4 * g + D / 2 : 8 * g + 4;
    for (int64_t bh = 0; bh < BH; ++bh) {
      const int64_t srow = gather ? bh * L + p : (rr * BH + bh) * Lr + t;
      const int64_t drow = (rr * BH + bh) * Lr + t;
      float x[4], y[4];
      load4(src + srow * D + a0, x);
      load4(src + srow * D + b0, y);
      float ox[4], oy[4];
      if (HALF) {  // pair j = (x[j], y[j])
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ox[j] = fmaf(x[j], c[j], -y[j] * s[j]);
          oy[j] = fmaf(x[j], s[j], y[j] * c[j]);
        }
      } else {  // pairs (x0,x1) (x2,x3) (y0,y1) (y2,y3) = k = 4g .. 4g+3
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          ox[2 * j] = fmaf(x[2 * j], c[j], -x[2 * j + 1] * s[j]);
          ox[2 * j + 1] = fmaf(x[2 * j], s[j], x[2 * j + 1] * c[j]);
          oy[2 * j] = fmaf(y[2 * j], c[j + 2], -y[2 * j + 1] * s[j + 2]);
          oy[2 * j + 1] = fmaf(y[2 * j], s[j + 2], y[2 * j + 1] * c[j + 2]);
        }
      }
      store4(dst + drow * D + a0, ox);
      store4(dst + drow * D + b0, oy);
    }
  }
}

unsigned rope_grid(int64_t n) {
  int64_t b = (n + 255) / 256;
  const int64_t cap = 256 * 8 * 8;
  if (b > cap) b = cap;
  if (b < 1) b = 1;
  return (unsigned)b;
}

template <typename T>
hipError_t rope_dispatch(const void* src, void* dst, int64_t BH, int64_t L, int64_t Lr, int64_t nr,
                         int D, const int64_t* pos, bool gather, double base, bool half,
                         hipStream_t stream) {
  const int64_t n = nr * Lr * (D / 8);
  if (n == 0 || BH == 0) return hipSuccess;
  const double lb = std::log2(base);
  if (half)
    hipLaunchKernelGGL((rope_kernel<T, true>), dim3(rope_grid(n)), dim3(256), 0, stream,
                       (const T*)src, (T*)dst, BH, L, Lr, nr, D, pos, gather ? 1 : 0, lb);
  else
    hipLaunchKernelGGL((rope_kernel<T, false>), dim3(rope_grid(n)), dim3(256), 0, stream,
                       (const T*)src, (T*)dst, BH, L, Lr, nr, D, pos, gather ? 1 : 0, lb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(const void* src, void* dst, bool bf16, int64_t BH, int64_t L, int64_t Lr,
                       int64_t nr, int D, const int64_t* pos, bool gather, double base, bool half,
                       hipStream_t stream) {
  if (bf16)
    return rope_dispatch<__bf16>(src, dst, BH, L, Lr, nr, D, pos, gather, base, half, stream);
  return rope_dispatch<float>(src, dst, BH, L, Lr, nr, D, pos, gather, base, half, stream);
}

}  // namespace cpa
