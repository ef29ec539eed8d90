// Bandwidth-bound and small-shape kernels of the ring:
//  * partial_rowwise: partial attention with one query row per thread and
//    float32 arithmetic everywhere (float32 inputs, and bf16 inputs with
//    D = 16), online softmax over the visible keys.
//  * merge: the online-softmax fold of a new partial into the running one
//    ("序列与上下文并行", section 上下文并行：注意力本身切分).
//  * permute: gather/scatter of whole rows between the global token order
//    and the rank-major zigzag order (same page, section 工程实践: the data
//    of each rank follows the CP layout).
//  * offsets check: finds the first entry of a position table that does not
//    exceed its predecessor; the attention kernels assume strictly
//    increasing positions within every block.
#include "cpa_internal.h"

#include <cmath>

namespace cpa {
namespace {

template <typename T>
__device__ __forceinline__ float ld(const T* p);
template <>
__device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld<__bf16>(const __bf16* p) { return (float)*p; }

template <typename T, int D>
__global__ __launch_bounds__(64) void partial_rowwise_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int64_t* __restrict__ q_off, const int64_t* __restrict__ k_off, float* __restrict__ O,
    float* __restrict__ lse, int64_t Lq, int64_t Lk, int causal, float scale) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t bh = blockIdx.y;
  if (t >= Lq) return;
  const T* q = Q + (bh * Lq + t) * D;
  const T* Kb = K + bh * Lk * D;
  const T* Vb = V + bh * Lk * D;
  float qv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) qv[d] = ld(q + d) * scale;
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int64_t qp = causal ? q_off[t] : 0;
  for (int64_t u = 0; u < Lk; ++u) {
    if (causal && k_off[u] > qp) break;  // positions increase: the rest is hidden too
    const T* k = Kb + u * D;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = fmaf(qv[d], ld(k + d), s);
    const T* v = Vb + u * D;
    if (s > m) {
      const float a = expf(m - s);
      l = l * a + 1.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(acc[d], a, ld(v + d));
      m = s;
    } else {
      const float p = expf(s - m);
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, ld(v + d), acc[d]);
    }
  }
  float* o = O + (bh * Lq + t) * D;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int d = 0; d < D; ++d) o[d] = acc[d] * inv;
  lse[bh * Lq + t] = l > 0.f ? m + logf(l) : -INFINITY;
}

template <typename T>
hipError_t rowwise_dispatch(const void* Q, const void* K, const void* V, const int64_t* q_off,
                            const int64_t* k_off, float* O, float* lse, int BH, int64_t Lq,
                            int64_t Lk, int D, bool causal, float scale, hipStream_t stream) {
  const dim3 grid((unsigned)((Lq + 63) / 64), (unsigned)BH);
  const T* q = (const T*)Q;
  const T* k = (const T*)K;
  const T* v = (const T*)V;
  const int c = causal ? 1 : 0;
  switch (D) {
    case 16:
      hipLaunchKernelGGL((partial_rowwise_kernel<T, 16>), grid, dim3(64), 0, stream, q, k, v,
                         q_off, k_off, O, lse, Lq, Lk, c, scale);
      break;
    case 64:
      hipLaunchKernelGGL((partial_rowwise_kernel<T, 64>), grid, dim3(64), 0, stream, q, k, v,
                         q_off, k_off, O, lse, Lq, Lk, c, scale);
      break;
    default:
      hipLaunchKernelGGL((partial_rowwise_kernel<T, 128>), grid, dim3(64), 0, stream, q, k, v,
                         q_off, k_off, O, lse, Lq, Lk, c, scale);
      break;
  }
  return hipGetLastError();
}

// One thread per 4 floats of a row.  Weights are recomputed per thread from
// the two lse values of its row (cheap next to the 4 x 3 float loads/stores).
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(float* __restrict__ O_acc,
                                                    float* __restrict__ lse_acc,
                                                    const float* __restrict__ O_new,
                                                    const float* __restrict__ lse_new,
                                                    int64_t rows) {
  constexpr int V4 = D / 4;
  const int64_t n = rows * V4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / V4;
    const float la = lse_acc[row];
    const float lb = lse_new[row];
    const float M = fmaxf(la, lb);
    float4 a = reinterpret_cast<const float4*>(O_acc)[i];
    const float4 b = reinterpret_cast<const float4*>(O_new)[i];
    float lse_out;
    if (M == -INFINITY) {
      a = make_float4(0.f, 0.f, 0.f, 0.f);
      lse_out = -INFINITY;
    } else {
      const float wa = expf(la - M);
      const float wb = expf(lb - M);
      const float inv = 1.f / (wa + wb);
      const float ca = wa * inv, cb = wb * inv;
      a.x = fmaf(ca, a.x, cb * b.x);
      a.y = fmaf(ca, a.y, cb * b.y);
      a.z = fmaf(ca, a.z, cb * b.z);
      a.w = fmaf(ca, a.w, cb * b.w);
      lse_out = M + logf(wa + wb);
    }
    reinterpret_cast<float4*>(O_acc)[i] = a;
    if (i % V4 == 0) lse_acc[row] = lse_out;
  }
}

// Each thread moves W bytes of one row; consecutive threads walk a row, then
// the next local token, so runs of a zigzag chunk stay contiguous on both sides.
template <typename W>
__global__ __launch_bounds__(256) void permute_kernel(const W* __restrict__ src, W* __restrict__ dst,
                                                      int64_t row_words, int64_t BH, int64_t L,
                                                      int64_t Lr, const int64_t* __restrict__ pos_all,
                                                      int rank_lo, int nr, int inverse) {
  const int64_t n = (int64_t)nr * BH * Lr * row_words;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t w = i % row_words;
    int64_t rest = i / row_words;
    const int64_t t = rest % Lr;
    rest /= Lr;
    const int64_t bh = rest % BH;
    const int64_t rr = rest / BH;  // rank relative to rank_lo
    const int64_t p = pos_all[(rr + rank_lo) * Lr + t];
    const int64_t g = (bh * L + p) * row_words + w;  // global-order element
    const int64_t r = i;                             // rank-major element (relative)
    if (inverse)
      dst[g] = src[r];
    else
      dst[r] = src[g];
  }
}

// first_bad <- rows * n: the "every table increases" answer that the check
// lowers with an atomic minimum (a fill kernel, not a memset, so that the
// pair can be captured in a graph).
__global__ void offsets_init_kernel(unsigned long long* first_bad, int64_t total) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *first_bad = (unsigned long long)total;
}

// Entry i of `rows` tables of n positions is bad if it is not the first of
// its table and does not exceed entry i - 1.
__global__ __launch_bounds__(256) void offsets_check_kernel(const int64_t* __restrict__ off,
                                                            int64_t rows, int64_t n,
                                                            unsigned long long* first_bad) {
  const int64_t total = rows * n;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    if (i % n != 0 && off[i] <= off[i - 1]) atomicMin(first_bad, (unsigned long long)i);
  }
}

unsigned grid_for(int64_t n, int per_block) {
  int64_t b = (n + per_block - 1) / per_block;
  const int64_t cap = 256 * 8 * 8;  // 8 resident blocks per CU is enough to saturate HBM
  if (b > cap) b = cap;
  if (b < 1) b = 1;
  return (unsigned)b;
}

}  // namespace

hipError_t launch_partial_rowwise(const void* Q, const void* K, const void* V, bool bf16,
                                  const int64_t* q_off, const int64_t* k_off, float* O,
                                  float* lse, int BH, int64_t Lq, int64_t Lk, int D, bool causal,
                                  float scale, hipStream_t stream) {
  if (bf16)
    return rowwise_dispatch<__bf16>(Q, K, V, q_off, k_off, O, lse, BH, Lq, Lk, D, causal, scale,
                                    stream);
  return rowwise_dispatch<float>(Q, K, V, q_off, k_off, O, lse, BH, Lq, Lk, D, causal, scale,
                                 stream);
}

hipError_t launch_merge(float* O_acc, float* lse_acc, const float* O_new, const float* lse_new,
                        int64_t rows, int D, hipStream_t stream) {
  const unsigned grid = grid_for(rows * (D / 4), 256);
  switch (D) {
    case 16:
      hipLaunchKernelGGL(merge_kernel<16>, dim3(grid), dim3(256), 0, stream, O_acc, lse_acc, O_new,
                         lse_new, rows);
      break;
    case 64:
      hipLaunchKernelGGL(merge_kernel<64>, dim3(grid), dim3(256), 0, stream, O_acc, lse_acc, O_new,
                         lse_new, rows);
      break;
    default:
      hipLaunchKernelGGL(merge_kernel<128>, dim3(grid), dim3(256), 0, stream, O_acc, lse_acc,
                         O_new, lse_new, rows);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_permute(const void* src, void* dst, int64_t row_bytes, int64_t BH, int64_t L,
                          const int64_t* pos_all, int N, int rank_lo, int rank_hi, bool inverse,
                          hipStream_t stream) {
  const int64_t Lr = L / N;
  const int nr = rank_hi - rank_lo;
  const int inv = inverse ? 1 : 0;
  if (row_bytes % 16 == 0) {
    const int64_t words = row_bytes / 16;
    const unsigned grid = grid_for(nr * BH * Lr * words, 256);
    hipLaunchKernelGGL(permute_kernel<uint4>, dim3(grid), dim3(256), 0, stream, (const uint4*)src,
                       (uint4*)dst, words, BH, L, Lr, pos_all, rank_lo, nr, inv);
  } else if (row_bytes % 8 == 0) {
    const int64_t words = row_bytes / 8;
    const unsigned grid = grid_for(nr * BH * Lr * words, 256);
    hipLaunchKernelGGL(permute_kernel<uint2>, dim3(grid), dim3(256), 0, stream, (const uint2*)src,
                       (uint2*)dst, words, BH, L, Lr, pos_all, rank_lo, nr, inv);
  } else {
    const int64_t words = row_bytes / 4;
    const unsigned grid = grid_for(nr * BH * Lr * words, 256);
    hipLaunchKernelGGL(permute_kernel<uint32_t>, dim3(grid), dim3(256), 0, stream,
                       (const uint32_t*)src, (uint32_t*)dst, words, BH, L, Lr, pos_all, rank_lo, nr,
                       inv);
  }
  return hipGetLastError();
}

hipError_t launch_check_offsets(const int64_t* off, int64_t rows, int64_t n, int64_t* first_bad,
                                hipStream_t stream) {
  unsigned long long* fb = reinterpret_cast<unsigned long long*>(first_bad);
  hipLaunchKernelGGL(offsets_init_kernel, dim3(1), dim3(64), 0, stream, fb, rows * n);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || rows * n == 0) return e;
  hipLaunchKernelGGL(offsets_check_kernel, dim3(grid_for(rows * n, 256)), dim3(256), 0, stream,
                     off, rows, n, fb);
  return hipGetLastError();
}

}  // namespace cpa
