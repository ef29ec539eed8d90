// Partial attention of one ring step on CDNA4 (gfx950): rank i's queries
// against rank j's keys/values, returning (O, lse) so that later steps can be
// folded in by online softmax ("序列与上下文并行", section
// 上下文并行：注意力本身切分).  Scores are Q K^T * scale, hidden keys get -inf,
// softmax over keys, weights times V ("Tensor并行与算子拆分", section
// 注意力的并行化优化).  Causal visibility compares global token positions
// (same page as the ring, section 工程实践: every rank knows its global offsets).
//
// Design (bf16, D = 64 or 128):
//  * One workgroup = 4 waves = 128 query rows; each wave owns 32 rows.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K (32 keys x 16 d) is the A operand read from
//    LDS, the wave's Q rows are the B operand held in registers for the whole
//    kernel.  In the 32x32 accumulator layout a lane then holds 16 keys of ONE
//    query, so the row max / row sum need only in-lane work plus one
//    permlane32 swap between the two half-waves.
//  * O is accumulated transposed, O^T += V^T P^T, so each lane again owns one
//    query row and rescaling by exp2(m_old - m_new) is lane-local.  P (fp32
//    -> bf16, round to nearest even) is the B operand straight from the score
//    registers; V^T comes from row-major V in LDS through ds_read_b64_tr_b16.
//  * K/V tiles of 64 keys are staged in LDS, double buffered, with a 16-byte
//    XOR swizzle so both operand read patterns are free of bank conflicts.
//  * Keys visible to a causal row form a prefix of the K block (positions
//    increase), so the workgroup loops only over keys below the last row's
//    bound, and only tiles that cross the first row's bound are masked per
//    element.  Rows that see no key write O = 0, lse = -inf.
//  * Workgroups are issued longest-first (last query tiles first), heads
//    fastest, so each XCD keeps working on the same heads' K/V in its L2.
#include "cpa_internal.h"

#include <cmath>

namespace cpa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int BM = 128;       // query rows per workgroup
constexpr int BN = 64;        // keys per LDS tile
constexpr int NTHREADS = 256; // 4 waves
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

template <int D>
struct Geo {
  static constexpr int CHUNKS = D / 8;                        // 16-byte chunks per row
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;           // one K or V tile
  static constexpr int LOADS = BN * CHUNKS / NTHREADS;        // chunks per thread per tile
  static constexpr int ROWS_PER_PASS = NTHREADS / CHUNKS;
};

// Physical 16-byte chunk holding logical chunk c of tile row r.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (D == 128) {
    return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
  } else {
    return c ^ ((r >> 1) & 7);
  }
}

template <int D>
__device__ __forceinline__ int lds_off(int r, int c) {
  return r * Geo<D>::ROW_BYTES + swz<D>(r, c) * 16;
}

// Number of entries <= x in the increasing array off[0, n); wave-cooperative
// 64-way search (every lane returns the same value).
__device__ int count_le(const int64_t* __restrict__ off, int64_t n, int64_t x) {
  const int lane = threadIdx.x & 63;
  int64_t lo = 0, hi = n;
  while (hi - lo > 64) {
    const int64_t step = (hi - lo + 63) / 64;
    const int64_t idx = lo + lane * step;
    const bool p = idx < hi && off[idx] <= x;
    const int c = __popcll(__ballot(p));
    if (c == 0) return (int)lo;
    const int64_t nlo = lo + (int64_t)(c - 1) * step + 1;
    const int64_t probe_c = lo + (int64_t)c * step;
    hi = probe_c < hi ? probe_c : hi;
    lo = nlo;
  }
  const int64_t idx = lo + lane;
  const bool p = idx < hi && off[idx] <= x;
  return (int)(lo + __popcll(__ballot(p)));
}

__device__ __forceinline__ float xhalf_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xhalf_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
__device__ __forceinline__ void load_tile(const __bf16* __restrict__ src, int64_t u0, int64_t Lk,
                                          u32x4 (&reg)[Geo<D>::LOADS]) {
  const int t = threadIdx.x;
  const int c = t % Geo<D>::CHUNKS;
#pragma unroll
  for (int i = 0; i < Geo<D>::LOADS; ++i) {
    const int r = t / Geo<D>::CHUNKS + i * Geo<D>::ROWS_PER_PASS;
    int64_t u = u0 + r;
    u = u < Lk ? u : Lk - 1;  // ragged tail: load a valid row, masked later
    reg[i] = *reinterpret_cast<const u32x4*>(src + u * D + c * 8);
  }
}

template <int D>
__device__ __forceinline__ void store_tile(lds_char* dst, const u32x4 (&reg)[Geo<D>::LOADS]) {
  const int t = threadIdx.x;
  const int c = t % Geo<D>::CHUNKS;
#pragma unroll
  for (int i = 0; i < Geo<D>::LOADS; ++i) {
    const int r = t / Geo<D>::CHUNKS + i * Geo<D>::ROWS_PER_PASS;
    *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(dst + lds_off<D>(r, c)) = reg[i];
  }
}

template <int D>
__global__ __launch_bounds__(NTHREADS, 2) void partial_attn_mfma_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const int64_t* __restrict__ q_off, const int64_t* __restrict__ k_off, float* __restrict__ O,
    float* __restrict__ lse, int BH, int64_t Lq, int64_t Lk, int causal, float c_log2,
    int n_qtiles) {
  using G = Geo<D>;
  __shared__ __attribute__((aligned(16))) char smem_raw[2 * 2 * G::TILE_BYTES];
  lds_char* smem = (lds_char*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int hi = lane >> 5;
  const int l32 = lane & 31;
  const int bh = blockIdx.x % BH;
  const int qt = n_qtiles - 1 - blockIdx.x / BH;
  const int64_t q_base = (int64_t)qt * BM;
  const int64_t last_row = (q_base + BM < Lq ? q_base + BM : Lq) - 1;
  const int64_t qrow = q_base + wv * 32 + l32;
  const int64_t qrow_c = qrow < Lq ? qrow : Lq - 1;

  const __bf16* Qbh = Q + (int64_t)bh * Lq * D;
  const __bf16* Kbh = K + (int64_t)bh * Lk * D;
  const __bf16* Vbh = V + (int64_t)bh * Lk * D;
  float* Obh = O + (int64_t)bh * Lq * D;
  float* lse_bh = lse + (int64_t)bh * Lq;

  int64_t n_lo = Lk, n_hi = Lk;
  int64_t my_qpos = 0;
  if (causal) {
    n_lo = count_le(k_off, Lk, q_off[q_base]);
    n_hi = count_le(k_off, Lk, q_off[last_row]);
    my_qpos = q_off[qrow_c];
  }

  if (n_hi == 0) {  // no row of this tile sees any key of this block
    if (qrow < Lq && hi == 0) lse_bh[qrow] = -INFINITY;
    if (qrow < Lq) {
      float4 z = {0.f, 0.f, 0.f, 0.f};
      for (int c = hi; c < D / 4; c += 2) reinterpret_cast<float4*>(Obh + qrow * D)[c] = z;
    }
    return;
  }

  // Q rows of this wave as the B operand: lane holds Q[qrow][kk*16 + hi*8 .. +7].
  bf16x8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    qf[kk] = *reinterpret_cast<const bf16x8*>(Qbh + qrow_c * D + kk * 16 + hi * 8);

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m2 = -INFINITY;  // running max of scaled scores, log2 units
  float lsum = 0.f;      // this lane's share of the running sum

  const int n_tiles = (int)((n_hi + BN - 1) / BN);
  u32x4 kreg[G::LOADS], vreg[G::LOADS];
  load_tile<D>(Kbh, 0, Lk, kreg);
  load_tile<D>(Vbh, 0, Lk, vreg);
  store_tile<D>(smem, kreg);
  store_tile<D>(smem + G::TILE_BYTES, vreg);
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    lds_char* Ks = smem + buf * 2 * G::TILE_BYTES;
    lds_char* Vs = Ks + G::TILE_BYTES;
    const int64_t u0 = (int64_t)it * BN;
    const bool more = it + 1 < n_tiles;
    if (more) {
      load_tile<D>(Kbh, u0 + BN, Lk, kreg);
      load_tile<D>(Vbh, u0 + BN, Lk, vreg);
    }

    // S^T for keys u0 + kb*32 + [0, 32): lane holds keys kb*32 + (r/4)*8 + hi*4 + r%4.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 a = *reinterpret_cast<__attribute__((address_space(3))) const bf16x8*>(
            Ks + lds_off<D>(kb * 32 + l32, kk * 2 + hi));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[kb], 0, 0, 0);
      }
    }

    if (u0 + BN > n_lo) {  // tile crosses a row's visibility bound or the end of the block
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t u = u0 + kb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
          const bool vis = u < Lk && (!causal || k_off[u] <= my_qpos);
          if (!vis) s[kb][r] = -INFINITY;
        }
    }

    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = xhalf_max(mx);
    const float m_new = fmaxf(m2, mx * c_log2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m2 - m_use);
    if (__ballot(m_new > m2)) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      lsum *= alpha;
    }
    m2 = m_new;

    bf16x8 pf[2][2];
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c_log2, -m_use));
        ps += p;
        pf[kb][r >> 3][r & 7] = (__bf16)p;
      }
    lsum += ps;

    // O^T += V^T P^T.  A operand: lane holds V[key slot][d = db*32 + l32] for the
    // eight key slots matching pf's registers, fetched as two transposing reads.
    const int g = lane >> 4;
    const int vrow = hi * 4 + ((lane & 15) >> 2);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int r0 = kb * 32 + half * 16 + vrow;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int ch = db * 4 + (g & 1) * 2 + ((lane >> 1) & 1);
          const int sub = (lane & 1) * 8;
          const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(Vs + lds_off<D>(r0, ch) + sub));
          const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(Vs + lds_off<D>(r0 + 8, ch) + sub));
          const i16x8 v8 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v8),
                                                            pf[kb][half], acc[db], 0, 0, 0);
        }
      }

    if (more) {
      lds_char* nK = smem + (buf ^ 1) * 2 * G::TILE_BYTES;
      store_tile<D>(nK, kreg);
      store_tile<D>(nK + G::TILE_BYTES, vreg);
    }
    __syncthreads();
  }

  const float ltot = xhalf_sum(lsum);
  if (qrow < Lq) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    float* orow = Obh + qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float4 v = {acc[db][gq * 4 + 0] * inv, acc[db][gq * 4 + 1] * inv,
                    acc[db][gq * 4 + 2] * inv, acc[db][gq * 4 + 3] * inv};
        *reinterpret_cast<float4*>(orow + db * 32 + gq * 8 + hi * 4) = v;
      }
    if (hi == 0) lse_bh[qrow] = ltot > 0.f ? (m2 + __log2f(ltot)) * LN2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_partial_mfma(const void* Q, const void* K, const void* V, const int64_t* q_off,
                               const int64_t* k_off, float* O, float* lse, int BH, int64_t Lq,
                               int64_t Lk, int D, bool causal, float scale, hipStream_t stream) {
  const int n_qtiles = (int)((Lq + BM - 1) / BM);
  const dim3 grid((unsigned)(n_qtiles * BH));
  const float c_log2 = scale * LOG2E;
  if (D == 128) {
    hipLaunchKernelGGL(partial_attn_mfma_kernel<128>, grid, dim3(NTHREADS), 0, stream,
                       (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, q_off, k_off, O, lse,
                       BH, Lq, Lk, causal ? 1 : 0, c_log2, n_qtiles);
  } else {
    hipLaunchKernelGGL(partial_attn_mfma_kernel<64>, grid, dim3(NTHREADS), 0, stream,
                       (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, q_off, k_off, O, lse,
                       BH, Lq, Lk, causal ? 1 : 0, c_log2, n_qtiles);
  }
  return hipGetLastError();
}

}  // namespace cpa
