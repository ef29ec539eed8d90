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
//    (32 per wave; 256 rows and 8 waves for shares of 8192 rows or more);
//    K and V tiles of 32 keys stream through LDS (async copies into four
//    buffers, one barrier per pair of tiles), Q and dO rows stay in
//    registers; the dP accumulator starts from -delta.  Per tile:
//    S^T = K Q^T and dP^T = V dO^T (each lane then holds 16 keys of ONE query,
//    so lse and delta are one register each), P and dS on the VALU, then
//    dQ^T += K^T dS^T with K^T read from LDS by ds_read_b64_tr_b16; the
//    exponentials issue between the dP products and half of dS between the
//    dQ products.  The lse is known, so there is no running max and no
//    rescaling.  The pass walks the N blocks of a ring in one launch (same
//    order as the forward).
//  * dK/dV pass: roles swapped.  A workgroup owns 128 keys (32 per wave);
//    Q and dO tiles of 32 queries stream through LDS, with their lse and
//    delta.  Per tile each wave computes S = Q K^T and dP = dO V^T (a lane
//    holds 16 queries of ONE key), P and dS, then dV^T += dO^T P and
//    dK^T += Q^T dS with the transposed operands read by ds_read_b64_tr_b16.
//    The exponentials issue between the dP products and dS between the dV
//    products.  K rows stay in registers and V rows in LDS, so both
//    accumulators fit at two waves per SIMD; two workgroups share a CU.
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
// Query rows per rank from which the dQ pass runs 8-wave workgroups.
constexpr int64_t kDqWideRows = 8192;
constexpr int BM = 128;        // query rows (dQ pass) or key rows (dK/dV pass) per workgroup
static_assert(BM == cpa::kMfmaRows && NTHREADS == cpa::kMfmaThreads,
              "the host checks launch sizes with these tile constants");
constexpr float LOG2E = 1.4426950408889634f;

using I0 = std::integral_constant<int, 0>;
using I1 = std::integral_constant<int, 1>;

// Per-lane addressing of a 32-row tile of D bf16 columns in LDS, in column
// blocks of W 16-byte chunks: logical chunk c of row r sits in 16-byte slot
// 32W*(c/W) + W*r + ((c%W) ^ cb_key<W>(r)).  A row-operand read (lane = row
// l32, 8 columns from kk*16 + hi*8) is then one of W/2 per-lane bases plus a
// compile-time offset, and a transposed read (lane = column d of block db,
// 8 consecutive rows of half h, as two 4-row reads) one of two; a per-element
// XOR swizzle would need KK + 2 DB offset registers.  The XOR key spreads
// each 16-lane phase of a row read and each 32-lane half of a transposed read
// over distinct banks.  Copy instruction n fills slots [64n, 64n + 64):
// 16 rows x 64 bytes (W = 4) or 8 rows x 128 bytes (W = 8, whole lines).
template <int W>
__device__ __forceinline__ int cb_key(int r) {
  if constexpr (W == 4) return (r >> 2) & 3;
  else return (((r >> 1) & 1) ? 5 : 0) ^ (((r >> 2) & 1) ? 2 : 0) ^ (((r >> 3) & 1) ? 4 : 0);
}
template <int W>
__device__ __forceinline__ int cb_slot(int r, int c) {
  return 32 * W * (c / W) + W * r + ((c % W) ^ cb_key<W>(r));
}

template <int D, int W, int NW>
struct CBTile {
  using G = Geo<D>;
  static constexpr int NCP = G::TILE_BYTES / 1024;           // 1 KB copy instructions per tile
  static constexpr int IPW = NCP >= NW ? NCP / NW : 1;       // per wave
  static constexpr int KB = W / 2;                           // row-operand bases
  static constexpr int BLK = 512 * W;                        // bytes per column block
  static_assert(NCP % NW == 0 || NW > NCP, "copy split");
  int wv, lane;
  int rbase[KB];
  int tbase[2];

  // Copy instruction n: the lane's tile row and its byte offset in global
  // memory (recomputed per copy: a few VALU instructions instead of
  // registers held across the loop).
  __device__ __forceinline__ int crow(int n) const { return (64 / W) * (n % (W / 2)) + lane / W; }
  __device__ __forceinline__ int coff(int n) const {
    const int r = crow(n);
    const int c = W * (n / (W / 2)) + ((lane % W) ^ cb_key<W>(r));
    return r * G::ROW_BYTES + c * 16;
  }

  __device__ __forceinline__ CBTile(int wv_, int lane_) : wv(wv_), lane(lane_) {
    const int hi = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int e = 0; e < KB; ++e) rbase[e] = cb_slot<W>(l32, e * 2 + hi) * 16;
    const int trow = hi * 4 + ((lane & 15) >> 2);
    const int tch = ((lane >> 4) & 1) * 2 + ((lane >> 1) & 1);
    const int tsub = (lane & 1) * 8;
#pragma unroll
    for (int e = 0; e < 2; ++e)
      tbase[e] = (W == 4 ? cb_slot<W>(trow + 8 * e, tch) : cb_slot<W>(trow, 4 * e + tch)) * 16 +
                 tsub;
  }

  // Rows [row0, row0 + 32) of a [nrows, D] matrix into the tile at LDS byte
  // address `dst` (wave-uniform, kept in scalar registers); rows past the end
  // re-read the last row (callers mask them).  Row counts are 32-bit (at most
  // 2^30 rows), so the bound checks stay on the scalar unit.
  __device__ __forceinline__ void copy(const __bf16* src, int row0, int nrows,
                                       uint32_t dst) const {
    const __bf16* base = src + (int64_t)row0 * D;
    if (row0 + BN <= nrows) {
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int n = (wv * IPW + i) % NCP;
        copy16_saddr((uint32_t)coff(n), base, dst + (uint32_t)n * 1024u);
      }
    } else {
      const int last = nrows - 1 - row0;  // last valid tile row (< 31)
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int n = (wv * IPW + i) % NCP;
        const int over = crow(n) - last;
        copy16_saddr((uint32_t)(coff(n) - (over > 0 ? over : 0) * G::ROW_BYTES), base,
                     dst + (uint32_t)n * 1024u);
      }
    }
  }

  // Row operand: lane's tile row l32, logical chunk kk*2 + hi.
  __device__ __forceinline__ bf16x8 rows(const lds_char* t, int kk) const {
    return *reinterpret_cast<__attribute__((address_space(3))) const bf16x8*>(
        t + (kk / KB) * BLK + rbase[kk % KB]);
  }

  // Transposed operand: column d of block db, rows h*16 + trow + 8p (p = 0, 1).
  __device__ __forceinline__ int taddr(int h, int db, int p) const {
    if constexpr (W == 4) return h * 1024 + db * 2048 + tbase[p];
    else return h * 2048 + (db >> 1) * 4096 + p * 1024 + tbase[p ^ (db & 1)];
  }
  __device__ __forceinline__ bf16x8 trans(const lds_char* t, int h, int db) const {
    const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(t + taddr(h, db, 0)));
    const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(t + taddr(h, db, 1)));
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
// QW waves of 32 query rows per workgroup: 4 (two workgroups per CU), or 8
// for long shares (one per CU), where every K/V tile staged in LDS then
// serves twice the rows: half the copies per product, 1.1-1.4 % off the ring
// backward at the 128k share; at 12k the wider workgroups' extra setup and
// crossing tiles cost 1.7 %, so short shares keep 4.
template <int D, bool GL, int QW>
__global__ __launch_bounds__(64 * QW, 8 / QW) void bwd_dq_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    const int64_t* __restrict__ q_off, const int64_t* __restrict__ k_off, float* __restrict__ dQ,
    int BH, int64_t Lq, int64_t Lk, int64_t kv_stride, int64_t koff_stride, int nblk, int first,
    int causal, float scale, int n_qtiles, int accumulate) {
  using G = Geo<D>;
  constexpr int TB = G::TILE_BYTES;
  constexpr int KK = G::KK;
  constexpr int DB = G::DB;
  __shared__ __attribute__((aligned(1024))) char k_lds_raw[4 * TB];
  __shared__ __attribute__((aligned(1024))) char v_lds_raw[4 * TB];
  lds_char* const Kl = (lds_char*)k_lds_raw;
  lds_char* const Vl = (lds_char*)v_lds_raw;
  // the same tiles as scalar LDS byte addresses for the copies
  const uint32_t Kl_s = __builtin_amdgcn_readfirstlane(lds_addr(Kl));
  const uint32_t Vl_s = __builtin_amdgcn_readfirstlane(lds_addr(Vl));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5;
  const int l32 = lane & 31;
  const int bh = blockIdx.x % BH;
  const int qt = n_qtiles - 1 - blockIdx.x / BH;
  const int64_t q_base = (int64_t)qt * (32 * QW);
  const int64_t last_row = (q_base + 32 * QW < Lq ? q_base + 32 * QW : Lq) - 1;
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
  f32x16 negdl;  // dP^T starts from -delta: dS = P (dP - delta) is one product
#pragma unroll
  for (int r = 0; r < 16; ++r) negdl[r] = -dl;

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
  const CBTile<D, 4, QW> ta(wv, lane);

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
  auto copy_kv = [&](const __bf16* lo, const __bf16* hi_base, int t, uint32_t dst)
                     __attribute__((always_inline)) {
    const int u0 = t * BN;  // 32-bit row counts: at most 2^30 rows
    ta.copy((GL && u0 >= (int)C) ? hi_base : lo, u0, (int)Lk, dst);
  };

  auto iter = [&](int t, auto P_) __attribute__((always_inline)) {
    // Four K/V buffers, a barrier after every odd tile: tile t sits in buffer
    // t % 4 (P), the pair (t, t+1) copies tiles t+2 and t+3 into the other
    // two buffers and waits for them before its barrier.
    constexpr int P = decltype(P_)::value;  // t % 4
    if (t + 2 < T) {
      copy_kv(Kbh, Kbh_hi, t + 2, Kl_s + ((P + 2) & 3) * TB);
      copy_kv(Vbh, Vbh_hi, t + 2, Vl_s + ((P + 2) & 3) * TB);
    }
    const lds_char* Kt = Kl + P * TB;
    const lds_char* Vt = Vl + P * TB;
    f32x16 s = zero16, dp = zero16;
    u32x4 dsf[2];  // dS^T as bf16 pairs (B operand, key halves)
    const int64_t u0 = (int64_t)t * BN;
    // Chunks, each one product with its slice of the VALU work (scheduling
    // barriers keep them in order, so the VALU issues while the matrix core
    // runs):
    //   0 .. KK-1        S^T = K Q^T
    //   KK .. 2KK-1      dP^T = V dO^T, the exponentials of 16/KK S rows each
    //   2KK .. 3KK-1     dQ^T += K^T dS^T (half, column block); dS of the
    //                    first key half before it, of the second during it
    constexpr int NM = 3 * KK, PF = 3, RPC = 16 / KK;
    static_assert(KK == 2 * DB && RPC * KK == 16, "chunk table");
    auto fetch = [&](int i) __attribute__((always_inline)) -> bf16x8 {
      if (i < KK) return ta.rows(Kt, i);
      if (i < 2 * KK) return ta.rows(Vt, i - KK);
      const int j = i - 2 * KK;
      return ta.trans(Kt, j / DB, j % DB);
    };
    auto ds_rows = [&](int r0, int r1) __attribute__((always_inline)) {
#pragma unroll
      for (int r = r0; r < r1; r += 2) {
        const float d0 = s[r] * dp[r], d1 = s[r + 1] * dp[r + 1];
        dsf[r >> 3][(r >> 1) & 3] = cvt_pk_bf16(d0, d1);
      }
    };
    bf16x8 ob[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) ob[i] = fetch(i);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i == KK) {
        __builtin_amdgcn_sched_barrier(0);
        if (u0 + BN > n_lo) {  // keys past a row's causal bound: P = 0
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (u0 + acc_row(r, hi) >= my_n) s[r] = -INFINITY;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i == 2 * KK) {
        ds_rows(0, 8);
        __builtin_amdgcn_sched_barrier(0);
      }
      const bf16x8 cur = ob[i % PF];
      if (i + PF < NM) ob[i % PF] = fetch(i + PF);
      if (i < KK) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[i], i == 0 ? zero16 : s, 0, 0, 0);
      } else if (i < 2 * KK) {
        const int c = i - KK;
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, df[c], c == 0 ? negdl : dp, 0, 0, 0);
#pragma unroll
        for (int r = c * RPC; r < (c + 1) * RPC; ++r)
          s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c_log2, -l2));
      } else {
        const int j = i - 2 * KK, h = j / DB, db = j % DB;
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, __builtin_bit_cast(bf16x8, dsf[h]),
                                                          acc[db], 0, 0, 0);
        if (h == 0) ds_rows(8 + db * (8 / DB), 8 + (db + 1) * (8 / DB));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (P & 1) {
      wait_copies();
      __syncthreads();
    }
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
    copy_kv(Kbh, Kbh_hi, 0, Kl_s);
    copy_kv(Vbh, Vbh_hi, 0, Vl_s);
    if (T > 1) {
      copy_kv(Kbh, Kbh_hi, 1, Kl_s + TB);
      copy_kv(Vbh, Vbh_hi, 1, Vl_s + TB);
    }
    wait_copies();
    __syncthreads();
    int t = 0;  // whole cycles of the four buffers, then a pair, then a single tile
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    for (; t + 3 < T; t += 4) {
      iter(t, I0{});
      iter(t + 1, I1{});
      iter(t + 2, I2{});
      iter(t + 3, I3{});
    }
    if (t + 1 < T) {
      iter(t, I0{});
      iter(t + 1, I1{});
      t += 2;
    }
    if (t < T) {  // a last single tile sits in buffer 0 or 2
      if ((t & 3) == 0) iter(t, I0{});
      else iter(t, I2{});
    }
    // the next block's first copies reuse the buffers
    wait_copies();
    __syncthreads();
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

// Four waves per workgroup, 32 keys each (128 keys), two workgroups per CU,
// so the two waves on a SIMD belong to independent workgroups and one's
// softmax arithmetic runs beside the other's matrix products.  Each wave does
// all four products of its keys against every query tile: S = Q K^T and
// dP = dO V^T (each lane then holds 16 queries of ONE key), P and dS on the
// VALU, then dV^T += dO^T P and dK^T += Q^T dS.  The wave's K rows stay in
// registers (B operand of S); its V rows are staged in LDS once (B operand
// of dP), which keeps both 32 x D accumulators in registers at two waves per
// SIMD.  Q and dO tiles stream through LDS (double buffered) with their lse
// and delta; one barrier per tile.
// GL: all tensors in global token order ([BH, nblk * Lq, ...]); the queries
// are rank `qrank`'s rows and K/V block b (with its dK/dV rows) is rank b's,
// all through zig_row.
template <int D, bool GL>
__global__ __launch_bounds__(NTHREADS, 2) void bwd_dkdv_kernel(
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
  __shared__ __attribute__((aligned(1024))) char v_lds_raw[4 * TB];  // V rows, one tile per wave
  __shared__ __attribute__((aligned(16))) float l2_lds[2][BN];
  __shared__ __attribute__((aligned(16))) float dl_lds[2][BN];
  lds_char* const Ql = (lds_char*)q_lds_raw;
  lds_char* const Ol = (lds_char*)o_lds_raw;
  // the same tiles as scalar LDS byte addresses for the copies
  const uint32_t Ql_s = __builtin_amdgcn_readfirstlane(lds_addr(Ql));
  const uint32_t Ol_s = __builtin_amdgcn_readfirstlane(lds_addr(Ol));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0 .. 3: key group
  const int hi = lane >> 5;
  const int l32 = lane & 31;
  const int bh = blockIdx.x % BH;
  const int rest = blockIdx.x / BH;
  const int kt = rest % n_ktiles;
  const int blk = rest / n_ktiles;
  const int64_t k_base = (int64_t)kt * BM;
  const int64_t last_key = (k_base + BM < Lk ? k_base + BM : Lk) - 1;
  const int64_t kw0 = k_base + wv * 32;  // first key of this wave
  const int64_t krow = kw0 + l32;
  const int64_t krow_c = krow < Lk ? krow : Lk - 1;
  const float c_log2 = scale * LOG2E;
  lds_char* const Vw = (lds_char*)v_lds_raw + wv * TB;
  const uint32_t Vw_s = __builtin_amdgcn_readfirstlane(lds_addr(Vw));

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
  const int my_first32 = (int)my_first;  // <= Lq <= 2^30
  const int t0 = (int)(m_lo / BN);
  const int T = (int)((Lq + BN - 1) / BN);

  constexpr int W = 4;
  const CBTile<D, W, 4> ta(wv, lane);
  // Query tile t (rows [t*BN, t*BN + BN)) of Q or dO into LDS.
  const int Cq32 = (int)Cq;
  const int Lq32 = (int)Lq;
  auto copy_q = [&](const __bf16* lo, const __bf16* hi_base, int t, uint32_t dst)
                    __attribute__((always_inline)) {
    const int u0 = t * BN;
    ta.copy((GL && u0 >= Cq32) ? hi_base : lo, u0, (int)Lq, dst);
  };
  const f32x16 zero16 = {};

  // lse and delta of query tile t (first wave): loaded when the tile's
  // copies are issued, written to LDS buffer b (as the exp2 reference) at the
  // end of the iteration, so the loads have the whole tile to land.  A
  // tile's rows are contiguous in either layout (GL: inside one chunk), so
  // the row address is the chunk base plus the local row.
  // (32-bit row indices: Lq <= 2^30; the per-lane part is one register.)
  float row_l = 0.f, row_d = 0.f;
  auto load_rows = [&](int t) __attribute__((always_inline)) {
    if (tid < BN) {
      const int64_t base = (GL && t * BN >= Cq32) ? q_hi_row : q_lo_row;
      const int q = t * BN + tid;
      const int qc = q < Lq32 ? q : Lq32 - 1;
      row_l = (lse_bh + base)[qc];
      row_d = (dl_bh + base)[qc];
    }
  };
  auto store_rows = [&](int t, int b) __attribute__((always_inline)) {
    if (tid < BN) {
      const bool ok = t * BN + tid < Lq32;
      l2_lds[b][tid] = ok ? lse_ref(row_l) : INFINITY;
      dl_lds[b][tid] = ok ? row_d : 0.f;
    }
  };

  // The wave's 32 V rows into its LDS tile (GL: 32 keys from a multiple of 32
  // lie in one chunk, so they are contiguous); rows past Lk re-read the last.
  {
    const CBTile<D, W, 1> tv(0, lane);
    if constexpr (GL) {
      const int64_t n = Lk - kw0;
      tv.copy(Vb + kmap(kw0 < Lk ? kw0 : Lk - 1) * D, 0, n < BN ? (n > 0 ? (int)n : 1) : BN, Vw_s);
    } else {
      tv.copy(Vb, (int)(kw0 < Lk ? kw0 : Lk - 1), (int)Lk, Vw_s);
    }
  }
  // This lane's key row of K as the B operand of S = Q K^T.
  bf16x8 kf[KK];
  {
    const __bf16* src = Kb + kmap(krow_c) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      kf[kk] = *reinterpret_cast<const bf16x8*>(src + kk * 16 + hi * 8);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) settle(kf[kk]);
  }
  f32x16 dv[DB], dk[DB];  // dV^T and dK^T, D x 32 keys
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dv[db][r] = 0.f;
      dk[db][r] = 0.f;
    }

  auto iter = [&](int t, auto P_) __attribute__((always_inline)) {
    constexpr int P = decltype(P_)::value;
    const lds_char* Qt = Ql + P * TB;
    const lds_char* Ot = Ol + P * TB;
    const int64_t q0 = (int64_t)t * BN;
    // 32 products per tile, each emitted as one chunk with its slice of the
    // VALU work so that the exponentials and dS issue while the matrix core
    // runs (scheduling barriers keep the chunks in order):
    //   chunks  0- 7  S = Q K^T (kk)
    //   chunks  8-15  dP = dO V^T (kk), exp of two S rows each
    //   chunks 16-23  dV^T += dO^T P (half, column block), dS of two rows each
    //   chunks 24-31  dK^T += Q^T dS (half, column block)
    // A operands (and dP's V rows) are read PF chunks ahead.
    constexpr int NM = 4 * KK, PF = 1;
    constexpr int RPC = 16 / KK;  // score rows per chunk of the exp and dS slices
    static_assert(KK == 2 * DB && RPC * KK == 16, "chunk table");
    using RowV = float4;  // the lse / delta values of a group of 4 rows
    f32x16 s = zero16, dp = zero16;
    u32x4 pf[2], sf[2];  // P and dS as bf16 pairs (B operands, key halves of the queries)
    // A chunk's operands: A (and dP's V rows as B), and, for the first chunk
    // of each group of 4 score rows, the group's lse references (dP chunks)
    // or deltas (dV chunks): rows 4g .. 4g + 3 are queries acc_row(4g, hi) +
    // 0 .. 3, one 16-byte read.  They are read in one go, PF chunks ahead;
    // reading the row values right after the operands keeps LDS returns (in
    // order) from making a chunk wait for a later chunk's reads.  One chunk ahead: a
    // deeper ring costs the registers that keep spill reloads (whose waits
    // also wait for the tile copies in flight) out of the loop.
    struct Ops {
      bf16x8 a, b;
      RowV rv;
    };
    auto rows_of = [&](const float(&arr)[BN], int r) __attribute__((always_inline)) -> RowV {
      return *reinterpret_cast<const RowV*>(&arr[acc_row(r & ~3, hi)]);
    };
    auto fetch = [&](int i) __attribute__((always_inline)) -> Ops {
      Ops o;
      if (i < KK) {
        o.a = ta.rows(Qt, i);
      } else if (i < 2 * KK) {
        o.a = ta.rows(Ot, i - KK);
        o.b = ta.rows(Vw, i - KK);
        if (((i - KK) * RPC) % 4 == 0) o.rv = rows_of(l2_lds[P], (i - KK) * RPC);
      } else {
        const int j = (i - 2 * KK) % (2 * DB);
        o.a = ta.trans(i < 3 * KK ? Ot : Qt, j / DB, j % DB);
        if (i < 3 * KK && ((i - 2 * KK) * RPC) % 4 == 0)
          o.rv = rows_of(dl_lds[P], (i - 2 * KK) * RPC);
      }
      return o;
    };
    auto rvel = [](const RowV& v, int e) __attribute__((always_inline)) -> float {
      return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
    };
    RowV rg;  // the current group's values
    Ops ob[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) ob[i] = fetch(i);
    // The next tile's copies issue after the first operand reads, so that
    // their address arithmetic runs while those reads are in flight.
    if (t + 1 < T) {
      copy_q(Qbh, Qbh_hi, t + 1, Ql_s + (P ^ 1) * TB);
      copy_q(Obh, Obh_hi, t + 1, Ol_s + (P ^ 1) * TB);
      load_rows(t + 1);
    }
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const Ops cur = ob[i % PF];
      if (i + PF < NM) ob[i % PF] = fetch(i + PF);
      if (i >= KK && i < 3 * KK && ((i - KK) % KK * RPC) % 4 == 0) rg = cur.rv;
      if (i < KK) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a, kf[i], i == 0 ? zero16 : s, 0, 0, 0);
      } else if (i < 2 * KK) {
        const int c = i - KK;
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a, cur.b, c == 0 ? zero16 : dp, 0, 0, 0);
        if (c == 0) {
          // The first dP product issues before the mask and the first
          // exponentials, which wait for S's last product: the matrix core
          // then has work while they wait.
          __builtin_amdgcn_sched_barrier(0);
          // hidden queries (tiles crossing a key's causal bound) get P = 0:
          // tile row u is hidden when u < my_first - q0
          if (q0 < m_hi) {
            const int lim64 = my_first32 - (int)q0;
            const int lim = lim64 < 0 ? 0 : (lim64 > BN ? BN : lim64);
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (acc_row(r, hi) < lim) s[r] = -INFINITY;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // P of rows [c RPC, (c + 1) RPC), in place of S
#pragma unroll
        for (int e = 0; e < RPC; e += 2) {
          const int r = c * RPC + e;
          s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c_log2, -rvel(rg, r & 3)));
          s[r + 1] = __builtin_amdgcn_exp2f(fmaf(s[r + 1], c_log2, -rvel(rg, (r + 1) & 3)));
          pf[r >> 3][(r >> 1) & 3] = cvt_pk_bf16(s[r], s[r + 1]);
        }
      } else if (i < 3 * KK) {
        const int j = i - 2 * KK, h = j / DB, db = j % DB;
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a, __builtin_bit_cast(bf16x8, pf[h]),
                                                         dv[db], 0, 0, 0);
        // dS of rows [j RPC, (j + 1) RPC)
#pragma unroll
        for (int e = 0; e < RPC; e += 2) {
          const int r = j * RPC + e;
          dp[r] = s[r] * (dp[r] - rvel(rg, r & 3));
          dp[r + 1] = s[r + 1] * (dp[r + 1] - rvel(rg, (r + 1) & 3));
          sf[r >> 3][(r >> 1) & 3] = cvt_pk_bf16(dp[r], dp[r + 1]);
        }
      } else {
        const int j = i - 3 * KK, h = j / DB, db = j % DB;
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a, __builtin_bit_cast(bf16x8, sf[h]),
                                                         dk[db], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_copies();
    if (t + 1 < T) store_rows(t + 1, P ^ 1);
    __syncthreads();
  };

  copy_q(Qbh, Qbh_hi, t0, Ql_s);
  copy_q(Obh, Obh_hi, t0, Ol_s);
  load_rows(t0);
  wait_copies();
  store_rows(t0, 0);
  __syncthreads();
  int t = t0;
  for (; t + 1 < T; t += 2) {
    iter(t, I0{});
    iter(t + 1, I1{});
  }
  if (t < T) iter(t, I0{});

  if (krow < Lk) {
    const int64_t row = GL ? ((int64_t)bh * Lrow + kmap(krow)) * D
                           : blk * kv_stride + ((int64_t)bh * Lk + krow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int c = db * 32 + gq * 8 + hi * 4;
        float4* pk = reinterpret_cast<float4*>(dK + row + c);
        float4* pv = reinterpret_cast<float4*>(dV + row + c);
        const float4 ok = *pk, ov = *pv;
        *pk = float4{ok.x + dk[db][gq * 4 + 0] * scale, ok.y + dk[db][gq * 4 + 1] * scale,
                     ok.z + dk[db][gq * 4 + 2] * scale, ok.w + dk[db][gq * 4 + 3] * scale};
        *pv = float4{ov.x + dv[db][gq * 4 + 0], ov.y + dv[db][gq * 4 + 1],
                     ov.z + dv[db][gq * 4 + 2], ov.w + dv[db][gq * 4 + 3]};
      }
  }
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
  const int n_ktiles = (int)((Lk + BM - 1) / BM);
  if (Lq >= kDqWideRows) {
    const int n_qtiles = (int)((Lq + 255) / 256);
    hipLaunchKernelGGL((bwd_dq_kernel<D, GL, 8>), dim3((unsigned)(n_qtiles * BH)), dim3(512), 0,
                       st, (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V,
                       (const __bf16*)dO, lse, delta, q_off, k_off, dQ, BH, Lq, Lk, kv_stride,
                       koff_stride, nblk, first, causal ? 1 : 0, scale, n_qtiles,
                       acc_dq ? 1 : 0);
  } else {
    const int n_qtiles = (int)((Lq + BM - 1) / BM);
    hipLaunchKernelGGL((bwd_dq_kernel<D, GL, 4>), dim3((unsigned)(n_qtiles * BH)),
                       dim3(NTHREADS), 0, st, (const __bf16*)Q, (const __bf16*)K,
                       (const __bf16*)V, (const __bf16*)dO, lse, delta, q_off, k_off, dQ, BH,
                       Lq, Lk, kv_stride, koff_stride, nblk, first, causal ? 1 : 0, scale,
                       n_qtiles, acc_dq ? 1 : 0);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, GL>), dim3((unsigned)(nblk * n_ktiles * BH)),
                     dim3(NTHREADS), 0, st, (const __bf16*)Q, (const __bf16*)K,
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
