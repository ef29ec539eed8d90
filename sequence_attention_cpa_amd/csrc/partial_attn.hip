// Partial attention of one ring step on CDNA4 (gfx950): rank i's queries
// against rank j's keys/values, returning (O, lse) so that later steps can be
// folded in by online softmax ("序列与上下文并行", section
// 上下文并行：注意力本身切分).  Scores are Q K^T * scale, hidden keys get -inf,
// softmax over keys, weights times V ("Tensor并行与算子拆分", section
// 注意力的并行化优化).  Causal visibility compares global token positions
// (same page as the ring, section 工程实践: every rank knows its global offsets).
//
// Design (bf16, D = 64 or 128):
//  * One workgroup = 4 waves = 128 query rows (32 per wave); two workgroups
//    per CU, so every SIMD runs two independent waves.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K (32 keys x 16 d) is the A operand read from
//    LDS, the wave's Q rows are the B operand held in registers for the whole
//    kernel.  In the 32x32 accumulator layout a lane then holds 16 keys of ONE
//    query, so the row max needs only in-lane work plus one permlane32 swap
//    between the two half-waves.
//  * O is accumulated transposed, O^T += V^T P^T, so each lane again owns one
//    query row.  P (fp32 -> bf16, round to nearest even) is the B operand
//    straight from the score registers; V^T comes from row-major V in LDS
//    through ds_read_b64_tr_b16.
//  * Software pipeline: iteration t issues the matrix work of PV(t-1) and
//    QK^T(t+1), then the exponentials of tile t, the row max of tile t+1 and
//    the rare rescale.  The operand reads from LDS run six (rank-major) or
//    four (global layout) MFMAs ahead of their use; sched_group_barrier pins
//    only that order of LDS reads and MFMAs (pinning the VALU work between the
//    MFMAs as well measured slower).
//  * K and V tiles of 32 keys live in two LDS buffers each.  Iteration t
//    starts the copies of K(t+2) and V(t) straight from global memory into
//    LDS (global_load_lds_dwordx4, no staging registers; offsets precomputed
//    per lane, base in SGPRs) and waits for them at its end.  The copy is
//    issued from inline asm so the compiler does not make every LDS read wait
//    for it.  The tile is stored in column blocks of 64 or 128 bytes with a
//    16-byte XOR inside each block (lds_slot): every operand read is one of a
//    few per-lane bases plus an immediate offset, and no read has bank
//    conflicts.  Each copy instruction writes 1 KiB of LDS contiguously.
//  * Softmax rescaling is lazy and exact: the exponent reference is an integer
//    (log2 units) raised only when a row's max outgrows it by a factor 2^32; the
//    rescale is then a power of two, applied with ldexp to O, l and the P of
//    the tile already computed but not yet multiplied into O.  O is divided by
//    the sum of the packed bf16 P (v_dot2_f32_bf16), i.e. exactly the weights
//    the PV product used, so it stays a convex combination of V rows; lse uses
//    the fp32 sum, which the bf16 rounding of a row's dominant weight would
//    otherwise bias by up to 2^-8 (relative).
//  * Keys visible to a causal row form a prefix of the K block (positions
//    increase), so the workgroup loops only over keys below the last row's
//    bound and only tiles that cross a row's bound are masked per element.
//    Rows that see no key write O = 0, lse = -inf.
//  * Workgroups are issued longest-first (last query tiles first), heads
//    fastest, so each XCD keeps working on the same heads' K/V in its L2.
#include "cpa_internal.h"
#include "mfma_tile.h"

#include <cmath>
#include <cstdint>
#include <type_traits>

namespace cpa {
namespace {

using namespace tile;

constexpr int BM = 128;        // query rows per workgroup
constexpr int NKB = BN / 32;   // 32-key MFMA blocks per tile
static_assert(NKB == 1, "the LDS tile layout holds 32 rows");
constexpr int NTHREADS = 256;  // 4 waves
static_assert(BM == cpa::kMfmaRows && NTHREADS == cpa::kMfmaThreads,
              "the host checks launch sizes with these tile constants");
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
// Lazy-rescale threshold (log2 units).  P stays below 2^33, exact in bf16
// and fp32 (their precision is relative), and the fp32 accumulators stay far
// from overflow for any |V| below 2^60 / keys; 2^8 measured 2 % slower on
// inputs with outlier rows, which rescale often.
constexpr float RESCALE_LOG2 = 32.0f;

// LDS layout of a 32-row K or V tile, in 16-byte slots, with column blocks
// of W chunks (W = 4: 64-byte blocks, W = 8: 128-byte blocks): logical chunk
// c of row r sits at slot 32W*(c/W) + W*r + ((c%W) ^ key(r)).  Column blocks
// keep every operand read at one of a few per-lane bases plus a compile-time
// offset; the XOR key spreads each 16-lane phase of the K reads and each
// 32-lane half of the transposing V reads over distinct banks.  Copy
// instruction n fills slots [64n, 64n + 64): 16 rows x 64 bytes of the tile
// (W = 4) or 8 rows x 128 bytes, whole cache lines (W = 8).
template <int W>
__device__ __forceinline__ int lds_key(int r) {
  if constexpr (W == 4) return (r >> 2) & 3;
  else return (((r >> 1) & 1) ? 5 : 0) ^ (((r >> 2) & 1) ? 2 : 0) ^ (((r >> 3) & 1) ? 4 : 0);
}
template <int W>
__device__ __forceinline__ int lds_slot(int r, int c) {
  return 32 * W * (c / W) + W * r + ((c % W) ^ lds_key<W>(r));
}

// Blocks: the queries meet nblk K/V blocks of Lk rows each, block b at
// K + b * kv_stride (V likewise) with positions k_off + b * koff_stride, in
// the order b = first + 1, first + 2, ..., first (mod nblk).  One block is one
// ring step (cpa_partial); nblk = N with first = i is rank i's whole ring, the
// running (O, max, sums) staying in registers from one block to the next.
// Visiting the rank's own block last is deliberate: in every other block a
// query tile sees either none of the keys or the same whole prefix as its
// neighbours (the zigzag chunks do not interleave), so the workgroups of a
// head sweep those blocks in step and share each K/V tile through L2; only
// the own block gives every tile a different causal prefix, after which the
// workgroups no longer run in step.
//
// GL (global layout): Q, K, V, O and lse are the whole sequence in global
// token order, [BH, N * Lq, ...], and rank r's local row u lives at global row
// zig(r, u) of the zigzag layout (chunk r for u < Lq/2, chunk 2N-1-r after),
// so the zigzag permute is folded into the addressing.  The chunk length
// Lq/2 is a multiple of 32, so every 32-row tile is contiguous in memory.
template <int D, bool GL>
__global__ __launch_bounds__(NTHREADS, 2) void partial_attn_mfma_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const int64_t* __restrict__ q_off, const int64_t* __restrict__ k_off, float* __restrict__ O,
    float* __restrict__ lse, int BH, int64_t Lq, int64_t Lk, int64_t kv_stride,
    int64_t koff_stride, int nblk, int first, int causal, float c_log2, int n_qtiles) {
  using G = Geo<D>;
  constexpr int TB = G::TILE_BYTES;
  constexpr int RB = G::ROW_BYTES;
  constexpr int KK = G::KK;
  constexpr int DB = G::DB;
  // Column-block width of the LDS tile layout, in 16-byte chunks.  The
  // global-order instantiation copies whole 128-byte lines (W = 8): there the
  // half-line copies of W = 4 measured 5-7 % slower, bound by copy latency.
  // The rank-major one runs faster with W = 4, which needs fewer base
  // registers.
  constexpr int W = GL ? 8 : 4;
  constexpr int KB = W / 2;     // K operand base registers
  constexpr int BLK = 512 * W;  // bytes per column block of a tile
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

  const int64_t C = Lq / 2;                 // chunk length (GL)
  const int64_t Lrow = GL ? Lq * nblk : Lq;  // rows per head in Q / O / lse
  // global row of rank r's local row u (GL)
  auto zig = [&](int r, int64_t u) __attribute__((always_inline)) -> int64_t {
    const bool lo = u < C;
    return (lo ? r : 2 * nblk - 1 - r) * C + (lo ? u : u - C);
  };
  const __bf16* Qbh = Q + (int64_t)bh * Lrow * D;
  float* Obh = O + (int64_t)bh * Lrow * D;
  float* lse_bh = lse + (int64_t)bh * Lrow;
  const int64_t q_first = causal ? q_off[q_base] : 0;
  const int64_t q_last = causal ? q_off[last_row] : 0;
  const int64_t my_qpos = causal ? q_off[qrow_c] : 0;

  // Current block: pointers, and the visible-key bounds.  Visible keys of a
  // causal row are a prefix [0, n) of the block (positions increase); n_lo /
  // n_hi bound it for the whole tile, my_n is this row's.
  const __bf16* Kbh = nullptr;
  const __bf16* Vbh = nullptr;
  // Indices into a block fit 32 bits (the host caps Lk at 2^30).
  int n_lo = (int)Lk, n_hi = (int)Lk, my_n = (int)Lk;
  int T = 0;

  // ---- per-lane constants -------------------------------------------------
  // Q rows of this wave as the B operand: lane holds Q[qrow][kk*16 + hi*8 .. +7].
  bf16x8 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    qf[kk] = *reinterpret_cast<const bf16x8*>(Qbh + (GL ? zig(first, qrow_c) : qrow_c) * D +
                                              kk * 16 + hi * 8);
  // K operand of kk: tile row l32, logical chunk kk*2 + hi, at byte
  // (kk / KB) * BLK + kbase[kk % KB] of the tile.
  int kbase[KB];
#pragma unroll
  for (int e = 0; e < KB; ++e) kbase[e] = lds_slot<W>(l32, e * 2 + hi) * 16;
  // V operand of (half, db): two transposing reads (p = 0, 1) of rows
  // half*16 + vrow + 8p, 8 bytes inside chunk db*4 + vch, at byte
  // vaddr(half, db, p) of the tile.
  const int vrow = hi * 4 + ((lane & 15) >> 2);
  const int vch = ((lane >> 4) & 1) * 2 + ((lane >> 1) & 1);
  const int vsub = (lane & 1) * 8;
  int vbase[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
    vbase[e] = (W == 4 ? lds_slot<W>(vrow + 8 * e, vch) : lds_slot<W>(vrow, 4 * e + vch)) * 16 +
               vsub;
  auto vaddr = [&](int half, int db, int p) __attribute__((always_inline)) -> int {
    if constexpr (W == 4) return half * 1024 + db * 2048 + vbase[p];
    else return half * 2048 + (db >> 1) * 4096 + p * 1024 + vbase[p ^ (db & 1)];
  };
  // Copy instruction n = wv*IPW + i fills LDS bytes [1024 n, 1024 n + 1024):
  // lane takes the 16-byte piece whose slot is 64 n + lane.
  int coff[G::IPW];
  int crow[G::IPW];
#pragma unroll
  for (int i = 0; i < G::IPW; ++i) {
    const int n = wv * G::IPW + i;
    crow[i] = (64 / W) * (n % (W / 2)) + lane / W;
    const int c = W * (n / (W / 2)) + ((lane % W) ^ lds_key<W>(crow[i]));
    coff[i] = crow[i] * RB + c * 16;
  }

  // GL: a block's rows below C come from the first chunk (base src), the
  // rest from the second (base src_hi, already offset by -C rows).
  const __bf16* Kbh_hi = nullptr;
  const __bf16* Vbh_hi = nullptr;
  auto copy_tile = [&](const __bf16* src, const __bf16* src_hi, int j, lds_char* dst)
                       __attribute__((always_inline)) {
    const int64_t u0 = (int64_t)j * BN;
    const __bf16* base = ((GL && u0 >= C) ? src_hi : src) + u0 * D;
    if (u0 + BN <= Lk) {
#pragma unroll
      for (int i = 0; i < G::IPW; ++i)
        copy16_saddr((uint32_t)coff[i], base, lds_addr(dst + (wv * G::IPW + i) * 1024));
    } else {  // last, ragged tile: rows past the block re-read its last row (masked later)
      const int last = (int)(Lk - 1 - u0);  // last valid tile row, 0 .. BN-2
#pragma unroll
      for (int i = 0; i < G::IPW; ++i) {
        const int over = crow[i] - last;  // rows past the end: move back by that many
        copy16_saddr((uint32_t)(coff[i] - (over > 0 ? over : 0) * RB), base,
                     lds_addr(dst + (wv * G::IPW + i) * 1024));
      }
    }
  };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  f32x16 s[2][NKB];        // scores of two tiles (S^T layout), by tile parity
  bf16x8 pf[2][NKB][2];    // bf16 P of two tiles, by tile parity
  float m2 = -INFINITY;  // exponent reference: an integer (log2 units) or -inf
  // This lane's share of the row sum of the bf16 P (normalises O) and of the
  // same sum in fp32 (gives lse), kept as 2 and 4 independent partial sums so
  // that the adds of one tile do not form one long dependent chain.
  float lsum2[2] = {0.f, 0.f};
  float lsum_f4[4] = {0.f, 0.f, 0.f, 0.f};
  const f32x16 zero16 = {};
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // Mask tile j's scores, find their row max and, when it outgrows the
  // reference, raise the reference to the next integer and rescale O, l and
  // the P of the tile computed last (`pprev`, not yet multiplied into O).
  auto finish_scores = [&](int j, f32x16 (&sj)[NKB], bf16x8 (&pprev)[NKB][2], auto HAS_PREV_)
                           __attribute__((always_inline)) {
    constexpr bool HAS_PREV = decltype(HAS_PREV_)::value;
    const int u0 = j * BN;
    if (u0 + BN > n_lo) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int u = u0 + kb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
          if (u >= my_n) sj[kb][r] = -INFINITY;
        }
    }
    float mx = sj[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sj[kb][r]);
    const float mx2 = xhalf_max(mx) * c_log2;
    if (__ballot(mx2 > m2 + RESCALE_LOG2)) {
      const float m_new = ceilf(fmaxf(m2, mx2));
      const int k = (m2 == -INFINITY || m_new == -INFINITY) ? 0 : (int)(m2 - m_new);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = __builtin_amdgcn_ldexpf(acc[db][r], k);
      lsum2[0] = __builtin_amdgcn_ldexpf(lsum2[0], k);
      lsum2[1] = __builtin_amdgcn_ldexpf(lsum2[1], k);
#pragma unroll
      for (int i = 0; i < 4; ++i) lsum_f4[i] = __builtin_amdgcn_ldexpf(lsum_f4[i], k);
      if constexpr (HAS_PREV) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              pprev[kb][h][e] = (__bf16)__builtin_amdgcn_ldexpf((float)pprev[kb][h][e], k);
      }
      m2 = m_new;
    }
  };

  // One pipeline iteration for tile t (parity P): copies of K(t+2), V(t);
  // PV(t-1) and QK^T(t+1) on the matrix cores interleaved with the exp2 of
  // tile t; then the row max of tile t+1.
  auto iter = [&](int t, auto P_, auto PV_, auto QK_) __attribute__((always_inline)) {
    constexpr int P = decltype(P_)::value;
    constexpr bool HAS_PV = decltype(PV_)::value;
    constexpr bool HAS_QK = decltype(QK_)::value;
    if (t + 2 < T) copy_tile(Kbh, Kbh_hi, t + 2, Kl + P * TB);
    copy_tile(Vbh, Vbh_hi, t, Vl + P * TB);

    const float m_use = m2 == -INFINITY ? 0.f : m2;
    const lds_char* Kt = Kl + (P ^ 1) * TB;  // K(t+1)
    const lds_char* Vt = Vl + (P ^ 1) * TB;  // V(t-1)
    constexpr int NV = HAS_PV ? 2 * NKB * DB : 0;
    constexpr int NQ = HAS_QK ? NKB * KK : 0;
    constexpr int NM = NV + NQ;
    // operands in flight ahead of the MFMA using them (chosen by measurement
    // for each layout)
    constexpr int PF = GL ? 4 : 6;
    auto fetch = [&](int i) __attribute__((always_inline)) -> bf16x8 {
      if (i < NV) {
        const int kb = i / (2 * DB), half = (i / DB) & 1, db = i % DB;
        const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(Vt + vaddr(half, db, 0)));
        const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(Vt + vaddr(half, db, 1)));
        const i16x8 v8 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        return __builtin_bit_cast(bf16x8, v8);
      }
      const int q = i - NV, kb = q / KK, kk = q % KK;
      return *reinterpret_cast<__attribute__((address_space(3))) const bf16x8*>(
          Kt + (kk / KB) * BLK + kbase[kk % KB]);
    };
    bf16x8 ob[PF];
#pragma unroll
    for (int i = 0; i < PF && i < NM; ++i) ob[i] = fetch(i);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const bf16x8 cur = ob[i % PF];
      if (i + PF < NM) ob[i % PF] = fetch(i + PF);
      if (i < NV) {
        const int kb = i / (2 * DB), half = (i / DB) & 1, db = i % DB;
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, pf[P ^ 1][kb][half], acc[db], 0,
                                                          0, 0);
      } else {
        const int q = i - NV, kb = q / KK, kk = q % KK;
        s[P ^ 1][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            cur, qf[kk], kk == 0 ? zero16 : s[P ^ 1][kb], 0, 0, 0);
      }
    }
    // Keep the operand reads PF MFMAs ahead in the final schedule as well: left
    // alone, the scheduler sinks each LDS read down to the MFMA that uses it.
#pragma unroll
    for (int i = 0; i < PF && i < NM; ++i) {
      if (i < NV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 LDS reads (V)
      else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);         // 1 LDS read (K)
    }
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA i
      if (i + PF < NM) {
        if (i + PF < NV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    // exp2 of tile t, packed to bf16; row sums of the fp32 and of the packed values.
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[P][kb][r], c_log2, -m_use));
        lsum_f4[r & 3] += p;
        pf[P][kb][r >> 3][r & 7] = (__bf16)p;
      }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pair = {pf[P][kb][h][e], pf[P][kb][h][e + 1]};
          lsum2[h] = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, lsum2[h], false);
        }
    if constexpr (HAS_QK) finish_scores(t + 1, s[P ^ 1], pf[P], std::true_type{});
    wait_copies();
    __syncthreads();
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using BT = std::true_type;
  using BF = std::false_type;

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
    const int64_t* kb_off = k_off + blk * koff_stride;
    n_lo = (int)count_le(kb_off, Lk, q_first);
    n_hi = (int)count_le(kb_off, Lk, q_last);
    int lo = n_lo, hb = n_hi;  // first u in [n_lo, n_hi) with position > my_qpos
    while (lo < hb) {
      const int mid = (lo + hb) >> 1;
      if (kb_off[mid] <= my_qpos) lo = mid + 1; else hb = mid;
    }
    my_n = lo;
  }
  if (n_hi == 0) continue;  // no row of this tile sees any key of this block
  T = (n_hi + BN - 1) / BN;

  // Prologue: K(0), K(1) into LDS; scores of tile 0.
  copy_tile(Kbh, Kbh_hi, 0, Kl);
  if (T > 1) copy_tile(Kbh, Kbh_hi, 1, Kl + TB);
  wait_copies();
  __syncthreads();
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      s[0][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *reinterpret_cast<__attribute__((address_space(3))) const bf16x8*>(
              Kl + (kk / KB) * BLK + kbase[kk % KB]),
          qf[kk], kk == 0 ? zero16 : s[0][kb], 0, 0, 0);
  finish_scores(0, s[0], pf[0], std::false_type{});
  __syncthreads();  // K(0) is read; its buffer is refilled by iteration 0

  if (T == 1) {
    iter(0, I0{}, BF{}, BF{});
  } else {
    iter(0, I0{}, BF{}, BT{});
    int t = 1;  // odd on every entry to the loop body and after it
    for (; t + 2 < T; t += 2) {
      iter(t, I1{}, BT{}, BT{});
      iter(t + 1, I0{}, BT{}, BT{});
    }
    if (t == T - 2) {  // T even: one more full iteration (odd t), then the last (even)
      iter(t, I1{}, BT{}, BT{});
      iter(t + 1, I0{}, BT{}, BF{});
    } else {           // T odd: t = T - 1 is the last
      iter(t, I1{}, BT{}, BF{});
    }
  }

  // Epilogue: PV(T-1).
  auto last_pv = [&](auto P_) __attribute__((always_inline)) {
    constexpr int P = decltype(P_)::value;
    const lds_char* Vt = Vl + P * TB;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(Vt + vaddr(half, db, 0)));
          const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(Vt + vaddr(half, db, 1)));
          const i16x8 v8 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v8),
                                                            pf[P][kb][half], acc[db], 0, 0, 0);
        }
  };
  if ((T - 1) & 1) last_pv(I1{}); else last_pv(I0{});
  __syncthreads();  // the next block refills both LDS buffers
  }  // blocks

  const float ltot = xhalf_sum(lsum2[0] + lsum2[1]);
  const float ltot_f = xhalf_sum((lsum_f4[0] + lsum_f4[1]) + (lsum_f4[2] + lsum_f4[3]));
  if (qrow < Lq) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    const int64_t orow_i = GL ? zig(first, qrow) : qrow;
    float* orow = Obh + orow_i * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const float4 v = {acc[db][gq * 4 + 0] * inv, acc[db][gq * 4 + 1] * inv,
                          acc[db][gq * 4 + 2] * inv, acc[db][gq * 4 + 3] * inv};
        *reinterpret_cast<float4*>(orow + db * 32 + gq * 8 + hi * 4) = v;
      }
    if (hi == 0) lse_bh[orow_i] = ltot_f > 0.f ? (m2 + __log2f(ltot_f)) * LN2 : -INFINITY;
  }
}

}  // namespace

namespace {
template <bool GL>
hipError_t launch_blocks(const void* Q, const void* K, const void* V, const int64_t* q_off,
                         const int64_t* k_off, float* O, float* lse, int BH, int64_t Lq,
                         int64_t Lk, int64_t kv_stride, int64_t koff_stride, int nblk, int first,
                         int D, bool causal, float scale, hipStream_t stream) {
  const int n_qtiles = (int)((Lq + BM - 1) / BM);
  const dim3 grid((unsigned)(n_qtiles * BH));
  const float c_log2 = scale * LOG2E;
  if (D == 128) {
    hipLaunchKernelGGL((partial_attn_mfma_kernel<128, GL>), grid, dim3(NTHREADS), 0, stream,
                       (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, q_off, k_off, O, lse,
                       BH, Lq, Lk, kv_stride, koff_stride, nblk, first, causal ? 1 : 0, c_log2,
                       n_qtiles);
  } else {
    hipLaunchKernelGGL((partial_attn_mfma_kernel<64, GL>), grid, dim3(NTHREADS), 0, stream,
                       (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, q_off, k_off, O, lse,
                       BH, Lq, Lk, kv_stride, koff_stride, nblk, first, causal ? 1 : 0, c_log2,
                       n_qtiles);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_partial_mfma(const void* Q, const void* K, const void* V, const int64_t* q_off,
                               const int64_t* k_off, float* O, float* lse, int BH, int64_t Lq,
                               int64_t Lk, int D, bool causal, float scale, hipStream_t stream) {
  return launch_blocks<false>(Q, K, V, q_off, k_off, O, lse, BH, Lq, Lk, 0, 0, 1, 0, D, causal,
                              scale, stream);
}

hipError_t launch_ring_mfma(const void* Q_i, const void* K_all, const void* V_all,
                            const int64_t* q_off, const int64_t* pos_all, float* O, float* lse,
                            int BH, int64_t Lr, int N, int i, int D, bool causal, float scale,
                            hipStream_t stream) {
  return launch_blocks<false>(Q_i, K_all, V_all, q_off, pos_all, O, lse, BH, Lr, Lr,
                              (int64_t)BH * Lr * D, Lr, N, i, D, causal, scale, stream);
}

hipError_t launch_share_mfma(const void* Q, const void* K, const void* V, const int64_t* pos_all,
                             float* O, float* lse, int BH, int64_t Lr, int N, int i, int D,
                             bool causal, float scale, hipStream_t stream) {
  return launch_blocks<true>(Q, K, V, pos_all + (int64_t)i * Lr, pos_all, O, lse, BH, Lr, Lr, 0,
                             Lr, N, i, D, causal, scale, stream);
}

}  // namespace cpa
