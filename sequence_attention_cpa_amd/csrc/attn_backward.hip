// Backward of the partial attention and of a rank's ring on CDNA4 (gfx950).
//
// The gradients are the derivative of O = softmax(s) V with s = Q K^T * scale
// + mask (the attention of "Tensor并行与算子拆分", section 注意力的并行化优化),
// for an upstream gradient dO:
//     P = exp(s - lse)   dP = dO V^T   delta_t = sum_d dO[t,d] O[t,d]
//     dS = P * (dP - delta)   dQ = scale dS K   dK = scale dS^T Q   dV = P^T dO.
// Under context parallelism ("序列与上下文并行", section 上下文并行：注意力本身切分)
// the same formulas hold block by block once every query row carries its
// FINAL lse and delta, so rank i's contributions against K/V block j need only
// rank i's (Q, dO, lse, delta) and block j's (K, V).  dQ stays with rank i;
// dK_j and dV_j accumulate the contributions of every rank (in a multi-GPU
// ring they travel with K_j / V_j).
//
// Two matrix-core passes (bf16 inputs, D = 64 or 128), no atomics:
//  * dQ pass: the forward kernel's shape.  A workgroup owns 128 query rows
//    (32 per wave); K and V tiles of 32 keys stream through LDS (async copies,
//    double buffered), Q and dO rows stay in registers.  Per tile:
//    S^T = K Q^T and dP^T = V dO^T (each lane then holds 16 keys of ONE query,
//    so lse and delta are one register each), P and dS on the VALU, then
//    dQ^T += K^T dS^T with K^T read from LDS by ds_read_b64_tr_b16.  The lse
//    is known, so there is no running max and no rescaling.  The pass walks
//    the N blocks of a ring in one launch (same order as the forward).
//  * dK/dV pass: roles swapped.  A workgroup owns 128 keys; Q and dO tiles of
//    32 queries stream through LDS, with their lse and delta.  Per tile:
//    S = Q K^T and dP = dO V^T (each lane holds 16 queries of ONE key), P and
//    dS, then dV^T += dO^T P and dK^T += Q^T dS with the transposed operands
//    read by ds_read_b64_tr_b16.  Both accumulators and both resident K/V
//    rows would need about 260 registers per lane, so two waves share each
//    32-key group and split its products (P role: S, P and dV; dS role: dP,
//    dS and dK), which keeps two waves per SIMD.
// Causal visibility compares global positions (key position <= query
// position); positions increase inside every block, so a query's visible keys
// are a prefix of a block and a key's visible queries a suffix; only tiles
// that cross those bounds are masked per element.
#include "cpa_internal.h"
#include "mfma_tile.h"

#include <cmath>
#include <cstdint>
#include <type_traits>

namespace cpa {
namespace {

using namespace tile;

constexpr int NTHREADS = 256;  // 4 waves
constexpr int BM = 128;        // query rows (dQ pass) or key rows (dK/dV pass) per workgroup
static_assert(BM == cpa::kMfmaRows && NTHREADS == cpa::kMfmaThreads,
              "the host checks launch sizes with these tile constants");
constexpr float LOG2E = 1.4426950408889634f;

using I0 = std::integral_constant<int, 0>;
using I1 = std::integral_constant<int, 1>;

// Per-lane addressing of a 32-row tile of D bf16 columns in LDS, swizzled by
// swz<D>: the async copy of a tile, the row-major operand (lane = row l32,
// 8 columns starting at kk*16 + hi*8) and the transposed operand (lane = column
// d of block db, 8 consecutive rows of half `h`, as two 4-row reads).
template <int D, int NW>
struct TileAddr {
  using G = Geo<D>;
  static constexpr int NCOPY = G::TILE_BYTES / 1024;         // 1 KB copy instructions per tile
  static constexpr int IPW = NCOPY >= NW ? NCOPY / NW : 1;  // per copying wave
  static constexpr int CW = NCOPY / IPW;                    // waves that copy
  int coff[IPW];
  int crow[IPW];
  int roff[G::KK];
  int toff[G::DB][2];
  int wv;

  __device__ __forceinline__ TileAddr(int wv_, int lane) : wv(wv_) {
    const int hi = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int n = (wv % CW) * IPW + i;
      crow[i] = n * G::RPI + lane / G::CHUNKS;
      coff[i] = crow[i] * G::ROW_BYTES + swz<D>(crow[i], lane % G::CHUNKS) * 16;
    }
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk)
      roff[kk] = l32 * G::ROW_BYTES + swz<D>(l32, kk * 2 + hi) * 16;
    const int trow = hi * 4 + ((lane & 15) >> 2);
    const int tch = ((lane >> 4) & 1) * 2 + ((lane >> 1) & 1);
    const int tsub = (lane & 1) * 8;
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
      for (int p = 0; p < 2; ++p)
        toff[db][p] = (trow + 8 * p) * G::ROW_BYTES + swz<D>(trow + 8 * p, db * 4 + tch) * 16 + tsub;
  }

  // Rows [row0, row0 + 32) of a [nrows, D] matrix into `dst`; rows past the
  // end re-read the last row (callers mask them).
  __device__ __forceinline__ void copy(const __bf16* src, int64_t row0, int64_t nrows,
                                       lds_char* dst) const {
    if (wv >= CW) return;  // uniform per wave
    if (row0 + BN <= nrows) {
      const __bf16* base = src + row0 * D;
#pragma unroll
      for (int i = 0; i < IPW; ++i)
        copy16_saddr((uint32_t)coff[i], base, lds_addr(dst + (wv * IPW + i) * 1024));
    } else {
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        int64_t u = row0 + crow[i];
        u = u < nrows ? u : nrows - 1;
        const char* g = (const char*)(src + u * D) + (coff[i] - crow[i] * G::ROW_BYTES);
        copy16_vaddr(g, lds_addr(dst + (wv * IPW + i) * 1024));
      }
    }
  }

  __device__ __forceinline__ bf16x8 rows(const lds_char* t, int kk) const {
    return *reinterpret_cast<__attribute__((address_space(3))) const bf16x8*>(t + roff[kk]);
  }

  __device__ __forceinline__ bf16x8 trans(const lds_char* t, int h, int db) const {
    const lds_char* b = t + h * 16 * G::ROW_BYTES;
    const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(b + toff[db][0]));
    const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(b + toff[db][1]));
    const i16x8 v8 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    return __builtin_bit_cast(bf16x8, v8);
  }
};

// Consume registers loaded from global memory before a loop: the compiler then
// waits for those loads once, here, instead of treating them as possibly
// pending inside the loop, where its waits would also cover the asynchronous
// tile copies in flight (the hardware counts both in vmcnt).
__device__ __forceinline__ void settle(const bf16x8& x) { asm volatile("" ::"v"(x)); }

// Two phases of matrix products whose A operands come from LDS: NM1 products,
// then `between()` (the VALU work that produces the second phase's B
// operands), then NM2 products.  Operands are fetched PF products ahead
// (fetch(i) for product i), also across `between()`, so LDS latency hides
// behind the matrix work instead of stalling every product.
template <int NM1, int NM2, int PF, typename Fetch, typename Mma, typename Between>
__device__ __forceinline__ void mfma_phases(Fetch&& fetch, Mma&& mma, Between&& between) {
  constexpr int NM = NM1 + NM2;
  bf16x8 ob[PF];
#pragma unroll
  for (int i = 0; i < PF && i < NM; ++i) ob[i] = fetch(i);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    if (i == NM1) between();
    const bf16x8 cur = ob[i % PF];
    if (i + PF < NM) ob[i % PF] = fetch(i + PF);
    mma(i, cur);
  }
}

// Row offset (within a 32-row tile) of accumulator element r of a lane in
// half-wave hi, for v_mfma_f32_32x32x16 (rows of the 32x32 result).
__device__ __forceinline__ int acc_row(int r, int hi) { return (r >> 2) * 8 + hi * 4 + (r & 3); }

// exp2 reference of a row: lse * log2(e), or +inf for a row without visible
// keys (its weights are then exactly 0).
__device__ __forceinline__ float lse_ref(float l) {
  return l == -INFINITY ? INFINITY : l * LOG2E;
}

// Rows of the global-order (zigzag) layout: rank r's local row u of Lr rows
// is global row r*C + u for u < C and (2N-1-r)*C + (u - C) after, C = Lr/2.
// With C a multiple of 32, every 32-row tile is contiguous in global order.
__device__ __forceinline__ int64_t zig_row(int r, int64_t u, int64_t Lr, int nblk) {
  const int64_t C = Lr / 2;
  return u < C ? (int64_t)r * C + u : (int64_t)(2 * nblk - 1 - r) * C + (u - C);
}

// ---------------------------------------------------------------- dQ pass

// GL: Q, K, V, dO, lse, delta and dQ are the whole sequence in global token
// order ([BH, nblk * Lq, ...]); the queries are rank `first`'s rows and K/V
// block b is rank b's rows, all through zig_row.
template <int D, bool GL>
__global__ __launch_bounds__(NTHREADS, 2) void bwd_dq_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    const int64_t* __restrict__ q_off, const int64_t* __restrict__ k_off, float* __restrict__ dQ,
    int BH, int64_t Lq, int64_t Lk, int64_t kv_stride, int64_t koff_stride, int nblk, int first,
    int causal, float scale, int n_qtiles, int accumulate) {
  using G = Geo<D>;
  constexpr int TB = G::TILE_BYTES;
  constexpr int KK = G::KK;
  constexpr int DB = G::DB;
  __shared__ __attribute__((aligned(1024))) char k_lds_raw[2 * TB];
  __shared__ __attribute__((aligned(1024))) char v_lds_raw[2 * TB];
  lds_char* const Kl = (lds_char*)k_lds_raw;
  lds_char* const Vl = (lds_char*)v_lds_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5;
  const int l32 = lane & 31;
  const int bh = blockIdx.x % BH;
  const int qt = n_qtiles - 1 - blockIdx.x / BH;
  const int64_t q_base = (int64_t)qt * BM;
  const int64_t last_row = (q_base + BM < Lq ? q_base + BM : Lq) - 1;
  const int64_t qrow = q_base + wv * 32 + l32;
  const int64_t qrow_c = qrow < Lq ? qrow : Lq - 1;
  const float c_log2 = scale * LOG2E;

  const int64_t Lrow = GL ? Lq * nblk : Lq;  // rows per head of Q, dO, lse, delta, dQ
  auto qmap = [&](int64_t u) __attribute__((always_inline)) -> int64_t {
    return GL ? zig_row(first, u, Lq, nblk) : u;
  };
  // Query positions: GL rows are their own positions (the zigzag closed form).
  auto qpos = [&](int64_t u) __attribute__((always_inline)) -> int64_t {
    return GL ? qmap(u) : q_off[u];
  };
  const int64_t q_first = causal ? qpos(q_base) : 0;
  const int64_t q_last = causal ? qpos(last_row) : 0;
  const int64_t my_qpos = causal ? qpos(qrow_c) : 0;
  const int64_t qg = (int64_t)bh * Lrow + qmap(qrow_c);
  const float l2 = lse_ref(lse[qg]);
  const float dl = delta[qg];

  // Q and dO rows of this wave as B operands (lane: 8 columns of its query).
  bf16x8 qf[KK], df[KK];
  {
    const __bf16* qr = Q + qg * D;
    const __bf16* dr = dO + qg * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qf[kk] = *reinterpret_cast<const bf16x8*>(qr + kk * 16 + hi * 8);
      df[kk] = *reinterpret_cast<const bf16x8*>(dr + kk * 16 + hi * 8);
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      settle(qf[kk]);
      settle(df[kk]);
    }
  }
  const TileAddr<D, 4> ta(wv, lane);

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  const f32x16 zero16 = {};

  // Current block: K / V bases.  GL: a block's keys below C come from its
  // first chunk (base *_lo), the rest from its second (base *_hi, offset by
  // -C rows so that key u sits at base + u * D in both).
  const __bf16 *Kbh = nullptr, *Vbh = nullptr, *Kbh_hi = nullptr, *Vbh_hi = nullptr;
  const int64_t C = Lq / 2;
  int64_t n_lo = Lk, n_hi = Lk, my_n = Lk;
  int T = 0;
  // Tile t (keys [t*BN, t*BN + BN)) of the current block's K or V into LDS.
  auto copy_kv = [&](const __bf16* lo, const __bf16* hi_base, int t, lds_char* dst)
                     __attribute__((always_inline)) {
    const int64_t u0 = (int64_t)t * BN;
    ta.copy((GL && u0 >= C) ? hi_base : lo, u0, Lk, dst);
  };

  auto iter = [&](int t, auto P_) __attribute__((always_inline)) {
    constexpr int P = decltype(P_)::value;
    if (t + 1 < T) {
      copy_kv(Kbh, Kbh_hi, t + 1, Kl + (P ^ 1) * TB);
      copy_kv(Vbh, Vbh_hi, t + 1, Vl + (P ^ 1) * TB);
    }
    const lds_char* Kt = Kl + P * TB;
    const lds_char* Vt = Vl + P * TB;
    f32x16 s = zero16, dp = zero16;
    bf16x8 dsf[2];
    const int64_t u0 = (int64_t)t * BN;
    // S^T, dP^T (K and V rows alternate), then dS, then dQ^T += K^T dS^T.
    mfma_phases<2 * KK, 2 * DB, 3>(
        [&](int i) __attribute__((always_inline)) -> bf16x8 {
          if (i < 2 * KK) return ta.rows((i & 1) ? Vt : Kt, i >> 1);
          const int j = i - 2 * KK;
          return ta.trans(Kt, j / DB, j % DB);
        },
        [&](int i, const bf16x8& op) __attribute__((always_inline)) {
          if (i < 2 * KK) {
            if (i & 1)
              dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, df[i >> 1], dp, 0, 0, 0);
            else
              s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, qf[i >> 1], s, 0, 0, 0);
          } else {
            const int j = i - 2 * KK;
            acc[j % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, dsf[j / DB], acc[j % DB], 0,
                                                                  0, 0);
          }
        },
        [&]() __attribute__((always_inline)) {
          if (u0 + BN > n_lo) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (u0 + acc_row(r, hi) >= my_n) s[r] = -INFINITY;
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s[r], c_log2, -l2));
            dsf[r >> 3][r & 7] = (__bf16)(p * (dp[r] - dl));
          }
        });
    wait_copies();
    __syncthreads();
  };

  for (int sb = 0; sb < nblk; ++sb) {
    const int blk = (first + 1 + sb) % nblk;
    if constexpr (GL) {
      const int64_t lo_row = (int64_t)blk * C, hi_row = (int64_t)(2 * nblk - 1 - blk) * C - C;
      Kbh = K + ((int64_t)bh * Lrow + lo_row) * D;
      Vbh = V + ((int64_t)bh * Lrow + lo_row) * D;
      Kbh_hi = K + ((int64_t)bh * Lrow + hi_row) * D;
      Vbh_hi = V + ((int64_t)bh * Lrow + hi_row) * D;
    } else {
      Kbh = K + blk * kv_stride + (int64_t)bh * Lk * D;
      Vbh = V + blk * kv_stride + (int64_t)bh * Lk * D;
      Kbh_hi = Kbh;
      Vbh_hi = Vbh;
    }
    if (causal) {
      if constexpr (GL) {
        const int64_t C = Lk / 2;
        n_lo = zig_count_le(blk, nblk, C, q_first);
        n_hi = zig_count_le(blk, nblk, C, q_last);
        my_n = zig_count_le(blk, nblk, C, my_qpos);
      } else {
        const int64_t* kb_off = k_off + blk * koff_stride;
        n_lo = count_le(kb_off, Lk, q_first);
        n_hi = count_le(kb_off, Lk, q_last);
        int64_t lo = n_lo, hb = n_hi;
        while (lo < hb) {
          const int64_t mid = (lo + hb) >> 1;
          if (kb_off[mid] <= my_qpos) lo = mid + 1; else hb = mid;
        }
        my_n = lo;
      }
    }
    if (n_hi == 0) continue;
    T = (int)((n_hi + BN - 1) / BN);
    copy_kv(Kbh, Kbh_hi, 0, Kl);
    copy_kv(Vbh, Vbh_hi, 0, Vl);
    wait_copies();
    __syncthreads();
    int t = 0;
    for (; t + 1 < T; t += 2) {
      iter(t, I0{});
      iter(t + 1, I1{});
    }
    if (t < T) iter(t, I0{});
  }

  if (qrow < Lq) {
    float* orow = dQ + ((int64_t)bh * Lrow + qmap(qrow)) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float4* dst = reinterpret_cast<float4*>(orow + db * 32 + gq * 8 + hi * 4);
        float4 v = {acc[db][gq * 4 + 0] * scale, acc[db][gq * 4 + 1] * scale,
                    acc[db][gq * 4 + 2] * scale, acc[db][gq * 4 + 3] * scale};
        if (accumulate) {
          const float4 o = *dst;
          v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
        }
        *dst = v;
      }
  }
}

// ------------------------------------------------------------- dK/dV pass

// Eight waves per workgroup, two per SIMD, for 128 keys: waves w and w + 4
// share key group w (32 keys) and split every tile's four products evenly.
// Wave w (P role) forms S = Q K^T and P, hands P to its partner through LDS,
// and accumulates dV^T += dO^T P; wave w + 4 (dS role) forms dP = dO V^T,
// then dS = P (dP - delta) from the partner's P, and accumulates
// dK^T += Q^T dS.  A barrier in the middle of each tile publishes P.  Each
// wave keeps one 32 x D accumulator and one of K / V, so two waves fit per
// SIMD, and no product is computed twice.
// GL: all tensors in global token order ([BH, nblk * Lq, ...]); the queries
// are rank `qrank`'s rows and K/V block b (with its dK/dV rows) is rank b's,
// all through zig_row.
template <int D, bool GL>
__global__ __launch_bounds__(2 * NTHREADS, 1) void bwd_dkdv_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    const int64_t* __restrict__ q_off, const int64_t* __restrict__ k_off, float* __restrict__ dK,
    float* __restrict__ dV, int BH, int64_t Lq, int64_t Lk, int64_t kv_stride,
    int64_t koff_stride, int causal, float scale, int n_ktiles, int nblk, int qrank) {
  using G = Geo<D>;
  constexpr int TB = G::TILE_BYTES;
  constexpr int KK = G::KK;
  constexpr int DB = G::DB;
  __shared__ __attribute__((aligned(1024))) char q_lds_raw[2 * TB];
  __shared__ __attribute__((aligned(1024))) char o_lds_raw[2 * TB];
  __shared__ __attribute__((aligned(16))) float l2_lds[2][BN];
  __shared__ __attribute__((aligned(16))) float dl_lds[2][BN];
  __shared__ __attribute__((aligned(16))) float4 p_lds[4][4][64];  // [key group][r/4][lane]
  lds_char* const Ql = (lds_char*)q_lds_raw;
  lds_char* const Ol = (lds_char*)o_lds_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0 .. 7
  const int kg = wv & 3;                                     // key group
  const bool dk_role = wv >= 4;                              // dS role
  const int hi = lane >> 5;
  const int l32 = lane & 31;
  const int bh = blockIdx.x % BH;
  const int rest = blockIdx.x / BH;
  const int kt = rest % n_ktiles;
  const int blk = rest / n_ktiles;
  const int64_t k_base = (int64_t)kt * BM;
  const int64_t last_key = (k_base + BM < Lk ? k_base + BM : Lk) - 1;
  const int64_t krow = k_base + kg * 32 + l32;
  const int64_t krow_c = krow < Lk ? krow : Lk - 1;
  const float c_log2 = scale * LOG2E;

  const int64_t Lrow = GL ? Lq * nblk : Lq;  // rows per head of every tensor (GL)
  // Row of key u of this block within a head.
  auto kmap = [&](int64_t u) __attribute__((always_inline)) -> int64_t {
    return GL ? zig_row(blk, u, Lk, nblk) : u;
  };
  const __bf16* Kb = GL ? K + (int64_t)bh * Lrow * D : K + blk * kv_stride + (int64_t)bh * Lk * D;
  const __bf16* Vb = GL ? V + (int64_t)bh * Lrow * D : V + blk * kv_stride + (int64_t)bh * Lk * D;
  // The rank's Q / dO rows: GL, query u < C at Qbh + u * D (first chunk),
  // u >= C at Qbh_hi + u * D (second chunk, base offset by -C rows).
  const int64_t Cq = Lq / 2;
  const int64_t q_lo_row = GL ? (int64_t)qrank * Cq : 0;
  const int64_t q_hi_row = GL ? (int64_t)(2 * nblk - 1 - qrank) * Cq - Cq : 0;
  const __bf16* Qbh = Q + ((int64_t)bh * Lrow + q_lo_row) * D;
  const __bf16* Obh = dO + ((int64_t)bh * Lrow + q_lo_row) * D;
  const __bf16* Qbh_hi = Q + ((int64_t)bh * Lrow + q_hi_row) * D;
  const __bf16* Obh_hi = dO + ((int64_t)bh * Lrow + q_hi_row) * D;
  const float* lse_bh = lse + (int64_t)bh * Lrow;
  const float* dl_bh = delta + (int64_t)bh * Lrow;

  // Visible queries of a key form a suffix [first(u), Lq) of the query block:
  // m_lo / m_hi bound it for the workgroup's first / last key, my_first is
  // this lane's key's.
  int64_t m_lo = 0, m_hi = 0, my_first = 0;
  if (causal) {
    if constexpr (GL) {  // positions are the zigzag closed form
      m_lo = zig_count_le(qrank, nblk, Cq, kmap(k_base) - 1);
      m_hi = zig_count_le(qrank, nblk, Cq, kmap(last_key) - 1);
      my_first = zig_count_le(qrank, nblk, Cq, kmap(krow_c) - 1);
    } else {
      const int64_t* kb_off = k_off + blk * koff_stride;
      m_lo = count_le(q_off, Lq, kb_off[k_base] - 1);
      m_hi = count_le(q_off, Lq, kb_off[last_key] - 1);
      const int64_t kp = kb_off[krow_c];
      int64_t lo = m_lo, hb = m_hi;  // first t in [m_lo, m_hi] with position >= kp
      while (lo < hb) {
        const int64_t mid = (lo + hb) >> 1;
        if (q_off[mid] < kp) lo = mid + 1; else hb = mid;
      }
      my_first = lo;
    }
  }
  if (m_lo >= Lq) return;  // no query sees any key of this workgroup: nothing to add
  const int t0 = (int)(m_lo / BN);
  const int T = (int)((Lq + BN - 1) / BN);

  const TileAddr<D, 8> ta(wv, lane);
  // Query tile t (rows [t*BN, t*BN + BN)) of Q or dO into LDS.
  auto copy_q = [&](const __bf16* lo, const __bf16* hi_base, int t, lds_char* dst)
                    __attribute__((always_inline)) {
    const int64_t u0 = (int64_t)t * BN;
    ta.copy((GL && u0 >= Cq) ? hi_base : lo, u0, Lq, dst);
  };
  const f32x16 zero16 = {};

  // lse reference and delta of query tile t into LDS buffer b (first wave).
  // A tile's rows are contiguous in either layout (GL: inside one chunk), so
  // the row address is the chunk base plus the local row.
  auto stage_rows = [&](int t, int b) __attribute__((always_inline)) {
    if (tid < BN) {
      const int64_t q = (int64_t)t * BN + tid;
      const int64_t base = (GL && (int64_t)t * BN >= Cq) ? q_hi_row : q_lo_row;
      l2_lds[b][tid] = q < Lq ? lse_ref(lse_bh[base + q]) : INFINITY;
      dl_lds[b][tid] = q < Lq ? dl_bh[base + q] : 0.f;
    }
  };

  // The whole pass for one role; both roles run the same copies, staging
  // and barriers, so the workgroup stays in step.
  auto run = [&](auto DKR_) __attribute__((always_inline)) {
    constexpr bool DKR = decltype(DKR_)::value;
    // This lane's key row of K (P role) or V (dS role) as the B operand.
    bf16x8 rf[KK];
    {
      const __bf16* src = (DKR ? Vb : Kb) + kmap(krow_c) * D;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        rf[kk] = *reinterpret_cast<const bf16x8*>(src + kk * 16 + hi * 8);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) settle(rf[kk]);
    }
    f32x16 acc[DB];  // dV^T (P role) or dK^T (dS role), D x 32 keys
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
    float4* const pslot = &p_lds[kg][0][lane];

    auto iter = [&](int t, auto P_) __attribute__((always_inline)) {
      constexpr int P = decltype(P_)::value;
      if (t + 1 < T) {
        copy_q(Qbh, Qbh_hi, t + 1, Ql + (P ^ 1) * TB);
        copy_q(Obh, Obh_hi, t + 1, Ol + (P ^ 1) * TB);
      }
      const lds_char* Qt = Ql + P * TB;
      const lds_char* Ot = Ol + P * TB;
      const int64_t q0 = (int64_t)t * BN;
      // S = Q K^T (P role) or dP = dO V^T (dS role): lane holds its key's
      // 16 queries, rows acc_row(r, hi) = g*8 + hi*4 + (r & 3), r = 4g .. 4g+3.
      // Then P (published through LDS) or dS, then dV^T += dO^T P or
      // dK^T += Q^T dS.
      f32x16 x = zero16;
      bf16x8 wf[2];
      mfma_phases<KK, 2 * DB, 3>(
          [&](int i) __attribute__((always_inline)) -> bf16x8 {
            if (i < KK) return ta.rows(DKR ? Ot : Qt, i);
            const int j = i - KK;
            return ta.trans(DKR ? Qt : Ot, j / DB, j % DB);
          },
          [&](int i, const bf16x8& op) __attribute__((always_inline)) {
            if (i < KK) {
              x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, rf[i], x, 0, 0, 0);
            } else {
              const int j = i - KK;
              acc[j % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, wf[j / DB], acc[j % DB],
                                                                    0, 0, 0);
            }
          },
          [&]() __attribute__((always_inline)) {
            if constexpr (!DKR) {
              if (q0 < m_hi) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                  if (q0 + acc_row(r, hi) < my_first) x[r] = -INFINITY;
              }
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const float4 a = *reinterpret_cast<const float4*>(&l2_lds[P][g * 8 + hi * 4]);
                const float l2[4] = {a.x, a.y, a.z, a.w};
                float pv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  pv[e] = __builtin_amdgcn_exp2f(fmaf(x[g * 4 + e], c_log2, -l2[e]));
                  wf[(g * 4 + e) >> 3][(g * 4 + e) & 7] = (__bf16)pv[e];
                }
                pslot[g * 64] = float4{pv[0], pv[1], pv[2], pv[3]};
              }
            }
            __syncthreads();  // P of this tile is in LDS
            if constexpr (DKR) {
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const float4 pv = pslot[g * 64];
                const float4 b = *reinterpret_cast<const float4*>(&dl_lds[P][g * 8 + hi * 4]);
                const float p4[4] = {pv.x, pv.y, pv.z, pv.w};
                const float d4[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int r = g * 4 + e;
                  wf[r >> 3][r & 7] = (__bf16)(p4[e] * (x[r] - d4[e]));
                }
              }
            }
          });
      if (t + 1 < T) stage_rows(t + 1, P ^ 1);
      wait_copies();
      __syncthreads();
    };

    copy_q(Qbh, Qbh_hi, t0, Ql);
    copy_q(Obh, Obh_hi, t0, Ol);
    stage_rows(t0, 0);
    wait_copies();
    __syncthreads();
    int t = t0;
    for (; t + 1 < T; t += 2) {
      iter(t, I0{});
      iter(t + 1, I1{});
    }
    if (t < T) iter(t, I0{});

    if (krow < Lk) {
      float* dst = (DKR ? dK : dV) +
                   (GL ? ((int64_t)bh * Lrow + kmap(krow)) * D
                       : blk * kv_stride + ((int64_t)bh * Lk + krow) * D);
      const float f = DKR ? scale : 1.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          float4* p = reinterpret_cast<float4*>(dst + db * 32 + gq * 8 + hi * 4);
          const float4 o = *p;
          *p = float4{o.x + acc[db][gq * 4 + 0] * f, o.y + acc[db][gq * 4 + 1] * f,
                      o.z + acc[db][gq * 4 + 2] * f, o.w + acc[db][gq * 4 + 3] * f};
        }
    }
  };
  if (dk_role)
    run(std::true_type{});
  else
    run(std::false_type{});
}

// ------------------------------------------------------------- delta

template <typename T>
__device__ __forceinline__ void load8f(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8f<__bf16>(const __bf16* p, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8f<float>(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// delta[row] = sum_d dO[row, d] * O[row, d]; GS = D/8 lanes per row, each
// summing 8 products, then a butterfly over the GS lanes (GS divides 64).
// GL: the rows are rank `rank`'s share of global-order [rows / Lr heads, nblk
// * Lr, D] tensors: logical row (h, u) is physical row h * nblk * Lr + zig_row(rank, u).
template <typename T, int GS, bool GL>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const float* __restrict__ O,
                                                        const T* __restrict__ dO,
                                                        float* __restrict__ delta, int64_t rows,
                                                        int64_t Lr, int nblk, int rank) {
  constexpr int D = GS * 8;
  const int64_t per_block = 256 / GS;
  for (int64_t r0 = (int64_t)blockIdx.x * per_block; r0 < rows; r0 += (int64_t)gridDim.x * per_block) {
    const int64_t row = r0 + threadIdx.x / GS;
    const int part = threadIdx.x % GS;
    const int64_t prow =
        GL ? (row / Lr) * (Lr * nblk) + zig_row(rank, row % Lr, Lr, nblk) : row;
    float sum = 0.f;
    if (row < rows) {
      float o[8], g[8];
      load8f<float>(O + prow * D + part * 8, o);
      load8f<T>(dO + prow * D + part * 8, g);
#pragma unroll
      for (int i = 0; i < 8; ++i) sum = fmaf(o[i], g[i], sum);
    }
#pragma unroll
    for (int m = GS / 2; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, GS);
    if (row < rows && part == 0) delta[prow] = sum;
  }
}

// ------------------------------------------------------------- fp32 rows

template <typename T>
__device__ __forceinline__ float ldf(const T* p) { return (float)*p; }

// dQ of one query row per thread, fp32 arithmetic (fp32 inputs, and D = 16).
template <typename T, int D>
__global__ __launch_bounds__(64) void bwd_dq_rowwise_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    const int64_t* __restrict__ q_off, const int64_t* __restrict__ k_off, float* __restrict__ dQ,
    int64_t Lq, int64_t Lk, int causal, float scale, int accumulate) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t bh = blockIdx.y;
  if (t >= Lq) return;
  const T* q = Q + (bh * Lq + t) * D;
  const T* g = dO + (bh * Lq + t) * D;
  const T* Kb = K + bh * Lk * D;
  const T* Vb = V + bh * Lk * D;
  float qv[D], gv[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = ldf(q + d) * scale;
    gv[d] = ldf(g + d);
    acc[d] = 0.f;
  }
  const float l = lse[bh * Lq + t];
  const float dl = delta[bh * Lq + t];
  const int64_t qp = causal ? q_off[t] : 0;
  if (l != -INFINITY) {
    for (int64_t u = 0; u < Lk; ++u) {
      if (causal && k_off[u] > qp) break;
      const T* k = Kb + u * D;
      const T* v = Vb + u * D;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        s = fmaf(qv[d], ldf(k + d), s);
        dp = fmaf(gv[d], ldf(v + d), dp);
      }
      const float ds = expf(s - l) * (dp - dl);
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(ds, ldf(k + d), acc[d]);
    }
  }
  float* out = dQ + (bh * Lq + t) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) out[d] = (accumulate ? out[d] : 0.f) + acc[d] * scale;
}

// dK, dV of one key row per thread (accumulated into dK, dV), fp32 arithmetic.
template <typename T, int D>
__global__ __launch_bounds__(64) void bwd_dkdv_rowwise_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    const int64_t* __restrict__ q_off, const int64_t* __restrict__ k_off, float* __restrict__ dK,
    float* __restrict__ dV, int64_t Lq, int64_t Lk, int causal, float scale) {
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t bh = blockIdx.y;
  if (u >= Lk) return;
  const T* k = K + (bh * Lk + u) * D;
  const T* v = V + (bh * Lk + u) * D;
  float kv[D], vv[D], ak[D], av[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    kv[d] = ldf(k + d) * scale;
    vv[d] = ldf(v + d);
    ak[d] = 0.f;
    av[d] = 0.f;
  }
  int64_t t = 0;
  if (causal) {  // first query whose position is >= this key's (positions increase)
    const int64_t kp = k_off[u];
    int64_t lo = 0, hb = Lq;
    while (lo < hb) {
      const int64_t mid = (lo + hb) >> 1;
      if (q_off[mid] < kp) lo = mid + 1; else hb = mid;
    }
    t = lo;
  }
  for (; t < Lq; ++t) {
    const float l = lse[bh * Lq + t];
    if (l == -INFINITY) continue;
    const T* q = Q + (bh * Lq + t) * D;
    const T* g = dO + (bh * Lq + t) * D;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      s = fmaf(kv[d], ldf(q + d), s);
      dp = fmaf(vv[d], ldf(g + d), dp);
    }
    const float p = expf(s - l);
    const float ds = p * (dp - delta[bh * Lq + t]);
#pragma unroll
    for (int d = 0; d < D; ++d) {
      av[d] = fmaf(p, ldf(g + d), av[d]);
      ak[d] = fmaf(ds, ldf(q + d), ak[d]);
    }
  }
  float* ok = dK + (bh * Lk + u) * D;
  float* ov = dV + (bh * Lk + u) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    ok[d] += ak[d] * scale;
    ov[d] += av[d];
  }
}

unsigned grid_cap(int64_t blocks) {
  const int64_t cap = 256 * 8 * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return (unsigned)blocks;
}

template <typename T, bool GL>
hipError_t delta_dispatch(const float* O, const void* dO, int64_t rows, int D, float* delta,
                          int64_t Lr, int nblk, int rank, hipStream_t st) {
  const int GS = D / 8;
  const unsigned grid = grid_cap((rows * GS + 255) / 256);
  switch (GS) {
    case 2:
      hipLaunchKernelGGL((bwd_delta_kernel<T, 2, GL>), dim3(grid), dim3(256), 0, st, O,
                         (const T*)dO, delta, rows, Lr, nblk, rank);
      break;
    case 8:
      hipLaunchKernelGGL((bwd_delta_kernel<T, 8, GL>), dim3(grid), dim3(256), 0, st, O,
                         (const T*)dO, delta, rows, Lr, nblk, rank);
      break;
    default:
      hipLaunchKernelGGL((bwd_delta_kernel<T, 16, GL>), dim3(grid), dim3(256), 0, st, O,
                         (const T*)dO, delta, rows, Lr, nblk, rank);
      break;
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t rowwise_bwd(const void* Q, const void* K, const void* V, const void* dO,
                       const float* lse, const float* delta, const int64_t* q_off,
                       const int64_t* k_off, float* dQ, float* dK, float* dV, int BH, int64_t Lq,
                       int64_t Lk, bool causal, float scale, bool acc_dq, hipStream_t st) {
  if (Lq > 0) {
    const dim3 g((unsigned)((Lq + 63) / 64), (unsigned)BH);
    hipLaunchKernelGGL((bwd_dq_rowwise_kernel<T, D>), g, dim3(64), 0, st, (const T*)Q,
                       (const T*)K, (const T*)V, (const T*)dO, lse, delta, q_off, k_off, dQ, Lq,
                       Lk, causal ? 1 : 0, scale, acc_dq ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (Lk > 0 && Lq > 0) {
    const dim3 g((unsigned)((Lk + 63) / 64), (unsigned)BH);
    hipLaunchKernelGGL((bwd_dkdv_rowwise_kernel<T, D>), g, dim3(64), 0, st, (const T*)Q,
                       (const T*)K, (const T*)V, (const T*)dO, lse, delta, q_off, k_off, dK, dV,
                       Lq, Lk, causal ? 1 : 0, scale);
  }
  return hipGetLastError();
}

template <int D, bool GL>
hipError_t mfma_bwd(const void* Q, const void* K, const void* V, const void* dO, const float* lse,
                    const float* delta, const int64_t* q_off, const int64_t* k_off, float* dQ,
                    float* dK, float* dV, int BH, int64_t Lq, int64_t Lk, int64_t kv_stride,
                    int64_t koff_stride, int nblk, int first, bool causal, float scale,
                    bool acc_dq, hipStream_t st) {
  const int n_qtiles = (int)((Lq + BM - 1) / BM);
  const int n_ktiles = (int)((Lk + BM - 1) / BM);
  hipLaunchKernelGGL((bwd_dq_kernel<D, GL>), dim3((unsigned)(n_qtiles * BH)), dim3(NTHREADS), 0,
                     st, (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, (const __bf16*)dO,
                     lse, delta, q_off, k_off, dQ, BH, Lq, Lk, kv_stride, koff_stride, nblk,
                     first, causal ? 1 : 0, scale, n_qtiles, acc_dq ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, GL>), dim3((unsigned)(nblk * n_ktiles * BH)),
                     dim3(2 * NTHREADS), 0, st, (const __bf16*)Q, (const __bf16*)K,
                     (const __bf16*)V, (const __bf16*)dO, lse, delta, q_off, k_off, dK, dV, BH,
                     Lq, Lk, kv_stride, koff_stride, causal ? 1 : 0, scale, n_ktiles, nblk,
                     first);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_delta(const float* O, const void* dO, bool bf16, int64_t rows, int D,
                            float* delta, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  return bf16 ? delta_dispatch<__bf16, false>(O, dO, rows, D, delta, 1, 1, 0, stream)
              : delta_dispatch<float, false>(O, dO, rows, D, delta, 1, 1, 0, stream);
}

hipError_t launch_bwd_delta_share(const float* O, const void* dO, int BH, int64_t Lr, int N,
                                  int i, int D, float* delta, hipStream_t stream) {
  const int64_t rows = (int64_t)BH * Lr;
  if (rows == 0) return hipSuccess;
  return delta_dispatch<__bf16, true>(O, dO, rows, D, delta, Lr, N, i, stream);
}

hipError_t launch_bwd_mfma(const void* Q, const void* K, const void* V, const void* dO,
                           const float* lse, const float* delta, const int64_t* q_off,
                           const int64_t* k_off, float* dQ, float* dK, float* dV, int BH,
                           int64_t Lq, int64_t Lk, int64_t kv_stride, int64_t koff_stride,
                           int nblk, int first, int D, bool causal, float scale, bool acc_dq,
                           hipStream_t stream) {
  if (D == 128)
    return mfma_bwd<128, false>(Q, K, V, dO, lse, delta, q_off, k_off, dQ, dK, dV, BH, Lq, Lk,
                                kv_stride, koff_stride, nblk, first, causal, scale, acc_dq,
                                stream);
  return mfma_bwd<64, false>(Q, K, V, dO, lse, delta, q_off, k_off, dQ, dK, dV, BH, Lq, Lk,
                             kv_stride, koff_stride, nblk, first, causal, scale, acc_dq, stream);
}

hipError_t launch_bwd_share_mfma(const void* Q, const void* K, const void* V, const void* dO,
                                 const float* lse, const float* delta, float* dQ, float* dK,
                                 float* dV, int BH, int64_t Lr, int N, int i, int D, bool causal,
                                 float scale, hipStream_t stream) {
  if (D == 128)
    return mfma_bwd<128, true>(Q, K, V, dO, lse, delta, nullptr, nullptr, dQ, dK, dV, BH, Lr, Lr,
                               0, 0, N, i, causal, scale, false, stream);
  return mfma_bwd<64, true>(Q, K, V, dO, lse, delta, nullptr, nullptr, dQ, dK, dV, BH, Lr, Lr, 0,
                            0, N, i, causal, scale, false, stream);
}

hipError_t launch_bwd_rowwise(const void* Q, const void* K, const void* V, const void* dO,
                              bool bf16, const float* lse, const float* delta,
                              const int64_t* q_off, const int64_t* k_off, float* dQ, float* dK,
                              float* dV, int BH, int64_t Lq, int64_t Lk, int D, bool causal,
                              float scale, bool acc_dq, hipStream_t stream) {
#define CPA_BWD_ROWS(T, DD)                                                                     \
  return rowwise_bwd<T, DD>(Q, K, V, dO, lse, delta, q_off, k_off, dQ, dK, dV, BH, Lq, Lk, \
                            causal, scale, acc_dq, stream)
  if (bf16) CPA_BWD_ROWS(__bf16, 16);  // bf16 with D = 64 / 128 runs on the matrix cores
  if (D == 16) CPA_BWD_ROWS(float, 16);
  if (D == 64) CPA_BWD_ROWS(float, 64);
  CPA_BWD_ROWS(float, 128);
#undef CPA_BWD_ROWS
}

}  // namespace cpa
