// Partial attention of the ring on CDNA4 (gfx950) matrix cores: a rank's
// queries against one or more K/V blocks, returning (O, lse) so that other
// blocks can be folded in by online softmax ("序列与上下文并行", section
// 上下文并行：注意力本身切分).  Scores are Q K^T * scale, hidden keys get -inf,
// softmax over keys, weights times V ("Tensor并行与算子拆分", section
// 注意力的并行化优化).  Causal visibility compares global token positions
// (same page as the ring, section 工程实践: every rank knows its global offsets).
//
// Design (bf16, D = 64 or 128):
//  * One workgroup = 8 waves = 256 query rows (32 per wave), one workgroup
//    per CU, two waves per SIMD.  Each K/V tile a workgroup stages in LDS
//    serves all 256 rows, which halves the L2-to-LDS traffic of four-wave
//    workgroups; at this density the part is power-limited, and bytes moved
//    cost clock.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K (32 keys x 16 d) is the A operand read from
//    LDS, the wave's Q rows are the B operand held in registers for the whole
//    kernel.  A lane then holds 16 keys of ONE query.  O is accumulated
//    transposed, O^T += V^T P^T: P (round to nearest even bf16) is the B
//    operand straight from registers, V^T comes from row-major V in LDS
//    through ds_read_b64_tr_b16.
//  * The steady loop is ONE basic block per 32-key tile: the copies of later
//    K/V tiles (branch-free: past the last full tile they re-copy it into a
//    free buffer), the 16 MFMAs of PV(t-1) and QK^T(t+1), and the softmax of
//    tile t, so the scheduler can hide the softmax arithmetic between the
//    matrix instructions.  Only the overflow check below branches, at the
//    end of the block, to a slow path that is taken a few times per row.
//  * No per-tile row max.  The exponent reference m is an integer (log2
//    units) fixed by the first tile a row sees; every later tile computes
//    P = 2^(s*c - m) directly and checks the largest of its weights (eight
//    v_max3 per lane).  A weight above 2^40 means a score outgrew the
//    reference by more than 40: the slow path then takes the tile's real
//    score max, raises m to its ceiling, rescales O and the sums by the
//    exact power of two and redoes the tile.  P stays at most 2^40, so bf16
//    P and the fp32 accumulators cannot overflow.
//  * O is divided by the sum of the bf16-rounded P (the weights the PV
//    product used), so it stays a convex combination of V rows.  That sum
//    comes from the matrix core: two 16x16x32 MFMAs per tile (half the
//    cycles of a 32x32x16 one) take the same P registers as their B operand
//    and a 0/1 mask as A (layout at the accumulator below); that costs less
//    than unpacking and adding the bf16 pairs on the VALU (and the
//    dot-product instructions stall the matrix pipe).  lse is the log of
//    that sum plus what rounding took off the largest weight each lane saw
//    (p - bf16(p)): a row that one key dominates would otherwise carry that
//    key's rounding, up to 2^-9 relative, into lse.  The largest weight
//    comes free with the overflow check (its max chain starts from the
//    running max).  An fp32 sum of all weights (16 adds per lane and tile)
//    measured 2 % slower at the 128k share and 3 % at 12k.
//  * K and V tiles live in eight LDS buffers each (128 KiB at D = 128);
//    K(t+5) and V(t+4) are copied during iteration t straight from global
//    memory into LDS (global_load_lds_dwordx4).  The workgroup meets at a
//    barrier after every second iteration only: each pair of iterations
//    waits for the copies of the pair before and publishes them to the pair
//    after, so a copy has two to four iterations to land and the waves
//    drift freely within a pair.  The first two V fragments of the next
//    iteration's PV are read before the pair's barrier (that tile was
//    published one pair earlier), so the matrix core does not wait for LDS
//    after it.
//  * Tiles are classified from the block's key positions: tiles every row of
//    the workgroup fully sees (the steady loop), and the few that cross a
//    row's causal bound or the block end.  In the global layout every tile is
//    whole and the steady loop runs the crossing tiles too, masking each
//    element by the lane's count of visible keys; the rank-major build runs
//    them in a simple, non-pipelined tail with an element mask and an exact
//    row max.  Keys visible to a causal row are a prefix of the block
//    (positions increase).  Rows that see no key write O = 0, lse = -inf.
//  * Global layout (cpa_share_forward): Q, K, V, O, lse are the whole sequence
//    in token order and rank r's local row u is global row zig(r, u) (chunk r
//    for u < C, chunk 2N-1-r after, C = L/(2N)); the positions are that same
//    closed form, so no position table is read.  With every block resident,
//    the ring's N blocks are swept as one run of keys in global order: the
//    same tiles as block by block, one copy prologue per workgroup instead of
//    one per block, contiguous tile addresses, and every long workgroup of a
//    head on the same tiles at the same time (L2 reuse).  +0.5 % at the 128k
//    share, +3.4 % at 12k against the block-by-block ring (own block last).
//  * Workgroups are issued longest-first (last query tiles first), heads
//    fastest, so each XCD keeps working on the same heads' K/V in its L2.
//  * Precise weights (PP, global layout only, opt-in): each P is split into
//    hi = bf16(P) and lo = bf16(P - hi), and the PV product runs twice per V
//    fragment, once on each part.  hi + lo carries P to a relative 2^-16, so
//    the bf16 rounding of P no longer limits O, and O is divided by the fp32
//    sum instead (no matrix-core row sums); lse and the overflow check use
//    that fp32 sum too (a sum above 2^40 takes the slow path).  It costs 8
//    MFMAs per tile (24 instead of 18 at D = 128) and about 40 VALU
//    instructions.
#include "cpa_internal.h"
#include "mfma_tile.h"

#include <cmath>
#include <cstdint>
#include <type_traits>

namespace cpa {
namespace {

using namespace tile;

// Waves per workgroup (32 query rows each); the K/V tiles a workgroup stages
// in LDS serve all of them.
constexpr int WAVES = 8;
constexpr int BM = 32 * WAVES;       // query rows per workgroup
constexpr int NTHREADS = 64 * WAVES;
static_assert(NTHREADS * cpa::kMfmaRows == BM * cpa::kMfmaThreads,
              "the host checks launch sizes with two threads per query row");
// LDS buffers per operand, and how far ahead iteration t copies: K(t +
// K_AHEAD), V(t + V_AHEAD).  With a barrier after every odd iteration, the
// pair of iterations (2q, 2q+1) reads K(2q+1..2q+2) and V(2q-1..2q+1) (the
// last one for the next pair's first PV), the copies of the pair before
// are landing and the pair's own copies go to K(2q+5..2q+6) and
// V(2q+4..2q+5): K_AHEAD = 5 and V_AHEAD = 4 are the distances at which a
// pair's copies are read two pairs later, and 6 K and 7 V tiles are in use
// at once.
constexpr int NBUF = 8;
constexpr int K_AHEAD = 5;
constexpr int V_AHEAD = 4;
static_assert(K_AHEAD + 1 <= NBUF && V_AHEAD + 3 <= NBUF, "copy would overwrite a tile in use");
// Operand reads in flight ahead of the MFMA that uses them (2 to 6 measured
// within 1.5 %; 2 is the fastest with the carried reads below).
constexpr int FWD_PF = 2;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
// A lane's largest weight of a tile above this (precise weights: its 16
// weights summing above it) sends the wave to the slow path.
constexpr float TILE_SUM_MAX = 0x1p40f;
// Reference before a row's first tile: any finite score overflows against it.
constexpr float M_INIT = -0x1p100f;

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
// running (O, reference, sums) staying in registers from one block to the
// next.  The rank's own block comes last: in every other block a query tile
// sees either none of the keys or the same whole prefix as its neighbours,
// so the workgroups of a head sweep those blocks in step and share each K/V
// tile through L2.
//
// GL (global layout): Q, K, V, O and lse are [BH, N * Lq, ...] in global
// token order; rank r's local row u is global row zig(r, u), which is also
// its position.  Lq/2 is a multiple of 32, so every 32-row tile is
// contiguous in memory and lies in one chunk.
template <int D, bool GL, int W, bool PP>
__global__ __launch_bounds__(NTHREADS, 8 / WAVES) void attn_fwd_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const int64_t* __restrict__ q_off, const int64_t* __restrict__ k_off, float* __restrict__ O,
    float* __restrict__ lse, int BH, int Lq, int Lk, int64_t kv_stride, int64_t koff_stride,
    int nblk, int rank0, int nranks, int causal, float c_log2, int n_qtiles) {
  using G = Geo<D>;
  constexpr int TB = G::TILE_BYTES;
  constexpr int RB = G::ROW_BYTES;
  constexpr int KK = G::KK;
  constexpr int DB = G::DB;
  constexpr int NCP = TB / 1024;  // 1 KiB copy instructions per tile
  constexpr int IPW = NCP / WAVES > 0 ? NCP / WAVES : 1;  // ... per wave (extra waves repeat)
  constexpr int KB = W / 2;     // K operand base registers
  constexpr int BLK = 512 * W;  // bytes per column block of a tile
  __shared__ __attribute__((aligned(1024))) char k_lds_raw[NBUF * TB];
  __shared__ __attribute__((aligned(1024))) char v_lds_raw[NBUF * TB];
  lds_char* const Kl = (lds_char*)k_lds_raw;
  lds_char* const Vl = (lds_char*)v_lds_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5;
  const int lr = lane & 31;
  // Workgroups: heads fastest, then the launch's ranks, then query tiles,
  // longest first (ranks' tiles of one index carry the same zigzag work).
  const int bh = blockIdx.x % BH;
  const int rest = blockIdx.x / BH;
  const int first = rank0 + rest % nranks;  // this workgroup's rank
  const int qt = n_qtiles - 1 - rest / nranks;
  const int q0 = qt * BM;                         // first local row of the workgroup
  const int qlast = min(q0 + BM, Lq) - 1;         // its last valid row
  const int w0 = q0 + wv * 32;                    // first local row of this wave
  const int qrow = w0 + lr;
  const int qrow_c = qrow < Lq ? qrow : Lq - 1;

  const int64_t C = Lq / 2;                     // chunk length (GL)
  const int64_t Lrow = GL ? (int64_t)Lq * nblk : Lq;  // rows per head in Q / O / lse
  // global row of rank r's local row u (GL)
  auto zig = [&](int r, int64_t u) __attribute__((always_inline)) -> int64_t {
    const bool lo = u < C;
    return (lo ? r : 2 * nblk - 1 - r) * C + (lo ? u : u - C);
  };
  auto qpos = [&](int u) __attribute__((always_inline)) -> int64_t {
    return GL ? zig(first, u) : q_off[u];
  };
  const __bf16* Qbh = Q + (int64_t)bh * Lrow * D;
  float* Obh = O + (int64_t)bh * Lrow * D;
  float* lse_bh = lse + (int64_t)bh * Lrow;
  // Positions of the workgroup's first and last rows and of this wave's
  // (waves past Lq take the last row: they compute nothing that is stored).
  const int wfirst = w0 < Lq ? w0 : Lq - 1;
  const int wlast = (w0 + 31 < Lq ? w0 + 31 : Lq - 1);
  int64_t pq_g0 = 0, pq_gl = 0, pq_w0 = 0, pq_wl = 0, my_qpos = 0;
  if (causal) {
    pq_g0 = qpos(q0);
    pq_gl = qpos(qlast);
    pq_w0 = qpos(wfirst);
    pq_wl = qpos(wlast);
    my_qpos = qpos(qrow_c);
  }

  // ---- per-lane constants -------------------------------------------------
  // Q rows of this wave as the B operand: lane holds Q[qrow][kk*16 + hi*8 .. +7].
  bf16x8 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    qf[kk] = *reinterpret_cast<const bf16x8*>(Qbh + (GL ? zig(first, qrow_c) : qrow_c) * D +
                                              kk * 16 + hi * 8);
  // K operand of kk: tile row lr, logical chunk kk*2 + hi, at byte
  // (kk / KB) * BLK + kbase[kk % KB] of the tile.
  int kbase[KB];
#pragma unroll
  for (int e = 0; e < KB; ++e) kbase[e] = lds_slot<W>(lr, e * 2 + hi) * 16;
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
  // Copy instruction n = (wv*IPW + i) % NCP fills LDS bytes [1024 n, 1024 n + 1024)
  // of a tile: lane takes the 16-byte piece whose slot is 64 n + lane.
  int coff[IPW];
  int crow[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int n = (wv * IPW + i) % NCP;
    crow[i] = (64 / W) * (n % (W / 2)) + lane / W;
    const int c = W * (n / (W / 2)) + ((lane % W) ^ lds_key<W>(crow[i]));
    coff[i] = crow[i] * RB + c * 16;
  }

  // Current K/V bases: a rank-major block, or (GL) the head's whole sequence.
  const __bf16* Kbh = nullptr;
  const __bf16* Vbh = nullptr;
  auto tile_src = [&](const __bf16* base, int j) __attribute__((always_inline)) -> const __bf16* {
    return base + (int64_t)(j * 32) * D;
  };
  auto copy_full = [&](const __bf16* src, lds_char* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < IPW; ++i)
      copy16_saddr((uint32_t)coff[i], src, lds_addr(dst + ((wv * IPW + i) % NCP) * 1024));
  };
  // Tile j that may run past the block end: rows past the end re-read the
  // block's last row (masked later).
  auto copy_any = [&](const __bf16* src, int j, lds_char* dst) __attribute__((always_inline)) {
    const int last = Lk - 1 - j * 32;  // last valid tile row
    if (last >= 31) {
      copy_full(src, dst);
    } else {
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int over = crow[i] - last;
        copy16_saddr((uint32_t)(coff[i] - (over > 0 ? over : 0) * RB), src,
                     lds_addr(dst + ((wv * IPW + i) % NCP) * 1024));
      }
    }
  };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  f32x16 s[2];            // scores of two tiles (S^T layout), by tile parity
  bf16x8 pf[2][2];        // bf16 P of two tiles, by tile parity, key halves
  bf16x8 pl[2][2];        // PP: the residuals P - hi, same indexing
  float m2 = M_INIT;      // exponent reference (log2 units): an integer after the first tile
  float L32 = 0.f;        // PP: the lane's share of the fp32 row sum; else its largest weight
  // Row sums of the bf16 P (normalise O), accumulated on the matrix core as
  // M x P^T with v_mfma_f32_16x16x32_bf16.  As its B operand, lane l's 8
  // weights of a key half are column l % 16, key group l / 16; the query of
  // lane l is l % 32, so column n of groups 0 and 2 is query n, of groups 1
  // and 3 query n + 16.  Result row 4g + j sits in element j of lanes
  // [16g, 16g + 16): mask rows 0 and 8 take groups 0 and 2, rows 4 and 12
  // groups 1 and 3 (lane l supplies row l % 16 of group l / 16), so element
  // 0 of every lane holds the sum of that lane's own query.
  f32x4 lsum = {};
  const int mrow = lane & 15;
  const __bf16 one = (mrow & 3) == 0 && ((mrow >> 2) & 1) == ((lane >> 4) & 1) ? (__bf16)1.f
                                                                                : (__bf16)0.f;
  const bf16x8 ones8 = {one, one, one, one, one, one, one, one};
  float ts32;             // the lane's largest weight of the tile (PP: fp32 tile sum)
  const f32x16 zero16 = {};

  // bf16 residuals of a packed pair: bf16(p0 - hi0), bf16(p1 - hi1), where
  // w holds hi0 in its low half and hi1 in its high half.  p - hi is exact
  // in fp32.
  auto residual = [](float p0, float p1, uint32_t w) __attribute__((always_inline)) -> uint32_t {
    const float h0 = __builtin_bit_cast(float, w << 16);
    const float h1 = __builtin_bit_cast(float, w & 0xffff0000u);
    return cvt_pk_bf16(p0 - h0, p1 - h1);
  };
  auto pack = [](const uint32_t* w, int h) __attribute__((always_inline)) -> bf16x8 {
    const u32x4 q4 = {w[4 * h], w[4 * h + 1], w[4 * h + 2], w[4 * h + 3]};
    return __builtin_bit_cast(bf16x8, q4);
  };
  // Weights of one tile at the current reference: P packed to bf16 for the
  // PV product (PP: and its residuals) and the lane's largest weight (PP:
  // the lane's fp32 sum).
  auto softmax = [&](const f32x16& sj, bf16x8 (&pj)[2], bf16x8 (&pjl)[2], float& t32)
                     __attribute__((always_inline)) {
    float a[4];
    uint32_t pw[8], lw[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sj[r], c_log2, -m2));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sj[r + 1], c_log2, -m2));
      if constexpr (PP) {
        if (r < 4) {
          a[r] = p0;
          a[r + 1] = p1;
        } else {
          a[r & 3] += p0;
          a[(r + 1) & 3] += p1;
        }
      } else {
        a[0] = r == 0 ? fmaxf(p0, p1) : fmaxf(fmaxf(a[0], p0), p1);
      }
      pw[r >> 1] = cvt_pk_bf16(p0, p1);
      if constexpr (PP) lw[r >> 1] = residual(p0, p1, pw[r >> 1]);
    }
    t32 = PP ? (a[0] + a[1]) + (a[2] + a[3]) : a[0];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      pj[h] = pack(pw, h);
      if constexpr (PP) pjl[h] = pack(lw, h);
    }
  };
  // The tile's exact row max raises the reference (to its ceiling) when it
  // is above it; O and the running sums are rescaled by the power of two,
  // then the tile's weights are recomputed.
  auto reraise = [&](const f32x16& sj, bf16x8 (&pj)[2], bf16x8 (&pjl)[2], float& t32)
                     __attribute__((always_inline)) {
    float mx = sj[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sj[r]);
    mx = xhalf_max(mx) * c_log2;
    const float m_new = mx > m2 ? ceilf(mx) : m2;
    const int k = (int)fmaxf(m2 - m_new, -1000.f);
    if (__ballot(k != 0)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = __builtin_amdgcn_ldexpf(acc[db][r], k);
      if constexpr (!PP) lsum[0] = __builtin_amdgcn_ldexpf(lsum[0], k);
      L32 = __builtin_amdgcn_ldexpf(L32, k);
    }
    m2 = m_new;
    softmax(sj, pj, pjl, t32);
  };
  // A tile that passed its check: PP adds the lane's fp32 sum to L32; with
  // bf16 weights L32 keeps the lane's largest weight so far (the slow path
  // rescales it with the sums).
  auto fold = [&](float t32) __attribute__((always_inline)) {
    if constexpr (PP) L32 += t32;
    else L32 = fmaxf(L32, t32);
  };

  auto qk_mfma = [&](const lds_char* Kt, f32x16& sj) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      sj = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *reinterpret_cast<__attribute__((address_space(3))) const bf16x8*>(
              Kt + (kk / KB) * BLK + kbase[kk % KB]),
          qf[kk], kk == 0 ? zero16 : sj, 0, 0, 0);
  };
  auto pv_mfma = [&](const lds_char* Vt, const bf16x8 (&pj)[2], const bf16x8 (&pjl)[2])
                     __attribute__((always_inline)) {
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
                                                          pj[half], acc[db], 0, 0, 0);
        if constexpr (PP)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v8),
                                                            pjl[half], acc[db], 0, 0, 0);
      }
    if constexpr (!PP) {
#pragma unroll
      for (int half = 0; half < 2; ++half)
        lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pj[half], lsum, 0, 0, 0);
    }
  };

  // GL: every block is resident and a token's position is its global index,
  // so the ring's blocks are swept as ONE run of keys in global order
  // (positions 0 .. L-1): the same tiles, one copy prologue instead of one
  // per block, and contiguous tile addresses.
  const int nsweep = GL ? 1 : nblk;
  const int LkS = GL ? (int)Lrow : Lk;  // keys of one sweep (the rank-major ring: one block)
  for (int sb = 0; sb < nsweep; ++sb) {
    const int blk = (first + 1 + sb) % nblk;
    if constexpr (GL) {
      Kbh = K + (int64_t)bh * Lrow * D;
      Vbh = V + (int64_t)bh * Lrow * D;
    } else {
      Kbh = K + blk * kv_stride + (int64_t)bh * Lk * D;
      Vbh = V + blk * kv_stride + (int64_t)bh * Lk * D;
    }
    // Tile counts.  n_main: tiles every row of the workgroup fully sees (the
    // first row sees the fewest); n_tot: tiles with a key any of its rows
    // sees.  The same per wave for the tail.
    int n_main, n_tot, w_full, w_tot;
    if (!causal) {
      n_main = w_full = LkS / 32;
      n_tot = w_tot = (LkS + 31) / 32;
    } else {
      int64_t c_g0, c_gl, c_w0, c_wl;
      if constexpr (GL) {  // keys at positions <= p: p + 1
        c_g0 = pq_g0 + 1;
        c_gl = pq_gl + 1;
        c_w0 = pq_w0 + 1;
        c_wl = pq_wl + 1;
      } else {
        const int64_t* kb_off = k_off + blk * koff_stride;
        c_g0 = count_le(kb_off, Lk, pq_g0);
        c_gl = count_le(kb_off, Lk, pq_gl);
        c_w0 = count_le(kb_off, Lk, pq_w0);
        c_wl = count_le(kb_off, Lk, pq_wl);
      }
      n_main = __builtin_amdgcn_readfirstlane((int)(c_g0 / 32));
      n_tot = __builtin_amdgcn_readfirstlane((int)((c_gl + 31) / 32));
      w_full = __builtin_amdgcn_readfirstlane((int)(c_w0 / 32));
      w_tot = __builtin_amdgcn_readfirstlane((int)((c_wl + 31) / 32));
    }
    if (w0 >= Lq) w_full = w_tot = 0;  // a wave past the last row stores nothing
    if (n_tot == 0) continue;          // no row of the workgroup sees this block (sweep)
    // GL: every tile is whole (the sweep's L is a multiple of 32), so the
    // steady loop also runs the tiles that cross a row's causal bound,
    // masking each element by the lane's count of visible keys (keys are in
    // position order); waves whose rows see none of such a tile compute it
    // with every weight 0.  The rank-major path keeps them for the tail.
    const int n_loop = GL ? n_tot : n_main;
    int my_cnt = 0;
    if constexpr (GL) {
      if (causal) my_cnt = (int)(my_qpos + 1);
    }

    // ---- steady loop over tiles [0, n_loop): every wave sees [0, n_main) ----
    if (n_loop > 0) {
      const int last = n_loop - 1;
      auto kcopy = [&](int j, int buf) __attribute__((always_inline)) {
        const int jj = j < last ? j : last;
        copy_full(tile_src(Kbh, jj), Kl + buf * TB);
      };
      auto vcopy = [&](int j, int buf) __attribute__((always_inline)) {
        const int jj = j < last ? j : last;
        copy_full(tile_src(Vbh, jj), Vl + buf * TB);
      };
#pragma unroll
      for (int j = 0; j < K_AHEAD; ++j) kcopy(j, j % NBUF);
#pragma unroll
      for (int j = 0; j < V_AHEAD; ++j) vcopy(j, j % NBUF);
      // Iteration 0 runs the same body as the others: its PV(-1) multiplies
      // zero weights into V(0), copied to the buffer tile -1 would use (so
      // that no stale LDS value can turn 0 * x into NaN); the last
      // iteration's QK^T of tile n_main reads a re-copied tile and is unused.
      vcopy(0, NBUF - 1);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pf[1][h][e] = (__bf16)0.0f;
          if constexpr (PP) pl[1][h][e] = (__bf16)0.0f;
        }
      wait_copies();
      __syncthreads();
      qk_mfma(Kl, s[0]);
      constexpr int NPV = 2 * DB;   // PV(t-1) V fragments (PP: two MFMAs each)
      constexpr int NV = NPV + (PP ? 0 : 2);  // ... and the row sums of P(t-1)
      constexpr int NM = NV + KK;   // ... and QK^T(t+1)
      // The last FWD_PF chunks of an iteration read the first V fragments of
      // the next one's PV (V(t), published a pair earlier) into the same
      // registers the next iteration starts from.
      constexpr bool CARRY = NM % FWD_PF == 0 && FWD_PF <= NPV;
      auto vfrag = [&](const lds_char* Vt, int i) __attribute__((always_inline)) -> bf16x8 {
        const int half = i / DB, db = i % DB;
        const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(Vt + vaddr(half, db, 0)));
        const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(Vt + vaddr(half, db, 1)));
        const i16x8 v8 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        return __builtin_bit_cast(bf16x8, v8);
      };
      bf16x8 ob[FWD_PF];
      if constexpr (CARRY) {
#pragma unroll
        for (int i = 0; i < FWD_PF; ++i) ob[i] = vfrag(Vl + (NBUF - 1) * TB, i);
      }

      // Iteration t: copies of K(t+5), V(t+4); PV(t-1) and QK^T(t+1) on the
      // matrix cores next to the softmax of tile t; the overflow check; the
      // barrier after odd iterations.
      auto iter = [&](int t, auto P_, auto M_, auto B_, auto PH_) __attribute__((always_inline)) {
        constexpr int P = decltype(P_)::value;
        constexpr bool MASK = decltype(M_)::value;
        constexpr bool BAR = decltype(B_)::value;
        constexpr int PH = decltype(PH_)::value;  // t % NBUF when known, else -1
        auto bufi = [&](int k) __attribute__((always_inline)) -> int {
          if constexpr (PH >= 0) return (PH + k) % NBUF;
          else return (t + k) % NBUF;
        };
        // masked tiles: tile row u of this lane's row is visible when u < lim
        int lim = 0;
        if constexpr (MASK) {
          const int l = my_cnt - t * 32;
          lim = l < 0 ? 0 : (l > 32 ? 32 : l);
        }
        kcopy(t + K_AHEAD, bufi(K_AHEAD));
        vcopy(t + V_AHEAD, bufi(V_AHEAD));
        const lds_char* Vt = Vl + bufi(NBUF - 1) * TB;  // V(t-1)
        const lds_char* Kt = Kl + bufi(1) * TB;         // K(t+1)
        const lds_char* Vn = Vl + bufi(0) * TB;         // V(t), next PV
        auto fetch = [&](int i) __attribute__((always_inline)) -> bf16x8 {
          if (i < NPV) return vfrag(Vt, i);
          if (i < NV) return ones8;
          const int kk = i - NV;
          return *reinterpret_cast<__attribute__((address_space(3))) const bf16x8*>(
              Kt + (kk / KB) * BLK + kbase[kk % KB]);
        };
        // The iteration is emitted as NM chunks, each one MFMA (its operands
        // read FWD_PF chunks ahead) and the softmax of some of the 16 score
        // elements of tile t; scheduling barriers keep the chunks in order, so
        // the exponentials issue while the matrix core is busy.
        float a4[4], pe[16];  // a4: running max of the weights (PP: four partial sums)
        uint32_t pw[8], lw[8];  // P of tile t, bf16 pairs (PP: and residual pairs)
        auto element = [&](int r) __attribute__((always_inline)) {
          if constexpr (MASK) {
            if ((r >> 2) * 8 + hi * 4 + (r & 3) >= lim) s[P][r] = -INFINITY;
          }
          pe[r] = __builtin_amdgcn_exp2f(fmaf(s[P][r], c_log2, -m2));
          if constexpr (PP) {
            if (r < 4) a4[r] = pe[r];
            else a4[r & 3] += pe[r];
          } else if (r & 1) {
            a4[0] = fmaxf(fmaxf(r == 1 ? L32 : a4[0], pe[r - 1]), pe[r]);
          }
          if (r & 1) {
            pw[r >> 1] = cvt_pk_bf16(pe[r - 1], pe[r]);
            if constexpr (PP) lw[r >> 1] = residual(pe[r - 1], pe[r], pw[r >> 1]);
          }
        };
        if constexpr (!CARRY) {
#pragma unroll
          for (int i = 0; i < FWD_PF && i < NM; ++i) ob[i] = fetch(i);
        }
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          const bf16x8 cur = ob[i % FWD_PF];
          if (i + FWD_PF < NM) ob[i % FWD_PF] = fetch(i + FWD_PF);
          else if constexpr (CARRY) ob[i % FWD_PF] = vfrag(Vn, i + FWD_PF - NM);
          if (i < NPV) {
            const int half = i / DB, db = i % DB;
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, pf[P ^ 1][half], acc[db], 0, 0,
                                                              0);
            if constexpr (PP)
              acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, pl[P ^ 1][half], acc[db], 0,
                                                                0, 0);
          } else if (i < NV) {
            lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, pf[P ^ 1][i - NPV], lsum, 0, 0, 0);
          } else {
            const int kk = i - NV;
            s[P ^ 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[kk],
                                                               kk == 0 ? zero16 : s[P ^ 1], 0, 0, 0);
          }
          // softmax elements of this chunk: [16 i / NM, 16 (i + 1) / NM)
#pragma unroll
          for (int r = (16 * i) / NM; r < (16 * (i + 1)) / NM; ++r) element(r);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (PP) ts32 = (a4[0] + a4[1]) + (a4[2] + a4[3]);
        else ts32 = a4[0];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          pf[P][h] = pack(pw, h);
          if constexpr (PP) pl[P][h] = pack(lw, h);
        }
        // With bf16 weights the max chain above started from L32, so
        // without the slow path ts32 already is the new running max.
        if (__ballot(ts32 > TILE_SUM_MAX)) {
          reraise(s[P], pf[P], pl[P], ts32);
          if constexpr (!PP) ts32 = fmaxf(ts32, L32);
        }
        if constexpr (PP) L32 += ts32;
        else L32 = ts32;
        if constexpr (BAR) {
          // Only this pair's copies may still be in flight.  A plain
          // s_barrier: the carried operand reads stay in flight across it
          // (they read a tile that no copy of the next pair overwrites); the
          // empty asm keeps the compiler from moving LDS accesses across it.
          wait_copies_but<4 * IPW>();
          asm volatile("" ::: "memory");
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::: "memory");
        }
      };
      using WITH_BAR = std::true_type;
      using NO_BAR = std::false_type;
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      using NOM = std::false_type;
      // Pairs keep the tile parity static and end at the barrier; masked
      // pairs start at an even tile (masking a tile every row fully sees
      // changes nothing).  A last, unpaired iteration needs no barrier: what
      // follows reads only tiles published before it, and waits for every
      // copy before the closing barrier.  The unmasked loop runs a whole
      // cycle of the NBUF buffers per trip, so every buffer index is a
      // constant and each LDS address is a lane register plus an immediate
      // offset (no address arithmetic per tile: 8 fewer VALU and about 15
      // fewer SALU instructions; +2.5 % at the 128k share, +3 % at 12k).
      const int n_plain = GL ? (n_main & ~1) : n_main;
      using DYN = std::integral_constant<int, -1>;
      int t = 0;
      for (; t + NBUF <= n_plain; t += NBUF) {
        iter(t, I0{}, NOM{}, NO_BAR{}, std::integral_constant<int, 0>{});
        iter(t + 1, I1{}, NOM{}, WITH_BAR{}, std::integral_constant<int, 1>{});
        iter(t + 2, I0{}, NOM{}, NO_BAR{}, std::integral_constant<int, 2>{});
        iter(t + 3, I1{}, NOM{}, WITH_BAR{}, std::integral_constant<int, 3>{});
        iter(t + 4, I0{}, NOM{}, NO_BAR{}, std::integral_constant<int, 4>{});
        iter(t + 5, I1{}, NOM{}, WITH_BAR{}, std::integral_constant<int, 5>{});
        iter(t + 6, I0{}, NOM{}, NO_BAR{}, std::integral_constant<int, 6>{});
        iter(t + 7, I1{}, NOM{}, WITH_BAR{}, std::integral_constant<int, 7>{});
      }
      for (; t + 1 < n_plain; t += 2) {
        iter(t, I0{}, NOM{}, NO_BAR{}, DYN{});
        iter(t + 1, I1{}, NOM{}, WITH_BAR{}, DYN{});
      }
      if constexpr (GL) {
        using MSK = std::true_type;
        for (; t + 1 < n_loop; t += 2) {
          iter(t, I0{}, MSK{}, NO_BAR{}, DYN{});
          iter(t + 1, I1{}, MSK{}, WITH_BAR{}, DYN{});
        }
        if (t < n_loop) iter(t, I0{}, MSK{}, NO_BAR{}, DYN{});
      } else {
        if (t < n_loop) iter(t, I0{}, NOM{}, NO_BAR{}, DYN{});
      }
      // PV(last); its V tile was published before the last pair.
      if (last & 1)
        pv_mfma(Vl + (last % NBUF) * TB, pf[1], pl[1]);
      else
        pv_mfma(Vl + (last % NBUF) * TB, pf[0], pl[0]);
      wait_copies();  // redundant re-copies may still be in flight
      __syncthreads();
    }

    // ---- tail: tiles [n_loop, n_tot), per wave full, masked or skipped ----
    if (n_tot > n_loop) {
      auto tcopy = [&](int j) __attribute__((always_inline)) {
        const int buf = j % NBUF;
        copy_any(tile_src(Kbh, j), j, Kl + buf * TB);
        copy_any(tile_src(Vbh, j), j, Vl + buf * TB);
      };
      tcopy(n_loop);
      for (int t = n_loop; t < n_tot; ++t) {
        if (t + 1 < n_tot) {
          tcopy(t + 1);
          wait_copies_but<2 * IPW>();
        } else {
          wait_copies();
        }
        __syncthreads();
        if (t < w_tot) {
          const lds_char* Kt = Kl + (t % NBUF) * TB;
          const lds_char* Vt = Vl + (t % NBUF) * TB;
          qk_mfma(Kt, s[0]);
          if (t >= w_full) {
            const int u0 = t * 32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int u = u0 + (r >> 2) * 8 + hi * 4 + (r & 3);
              bool vis = u < LkS;
              if (causal && vis) {
                int64_t kp;
                if constexpr (GL) kp = u;
                else kp = k_off[blk * koff_stride + u];
                vis = kp <= my_qpos;
              }
              if (!vis) s[0][r] = -INFINITY;
            }
          }
          reraise(s[0], pf[0], pl[0], ts32);
          fold(ts32);
          pv_mfma(Vt, pf[0], pl[0]);
        }
      }
      __syncthreads();  // the next block refills the buffers
    }
  }  // blocks

  const float l32 = xhalf_sum(L32);
  // O's normaliser: the sum of the weights the PV product used.
  const float l16 = PP ? l32 : lsum[0];
  if (qrow < Lq) {
    const float inv = l16 > 0.f ? 1.f / l16 : 0.f;
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
    // bf16 weights: add back what rounding took off each lane's largest
    // weight (the row's two lanes: xhalf_sum).
    const float l_lse =
        PP ? l32
           : l16 + xhalf_sum(L32 - __builtin_bit_cast(float, cvt_pk_bf16(L32, 0.f) << 16));
    if (hi == 0) lse_bh[orow_i] = l_lse > 0.f ? (m2 + __log2f(l_lse)) * LN2 : -INFINITY;
  }
}

template <bool GL, int W, bool PP = false>
hipError_t launch_blocks(const void* Q, const void* K, const void* V, const int64_t* q_off,
                         const int64_t* k_off, float* O, float* lse, int BH, int64_t Lq,
                         int64_t Lk, int64_t kv_stride, int64_t koff_stride, int nblk, int first,
                         int nranks, int D, bool causal, float scale, hipStream_t stream) {
  const int n_qtiles = (int)((Lq + BM - 1) / BM);
  const dim3 grid((unsigned)((int64_t)n_qtiles * BH * nranks));
  const float c_log2 = scale * LOG2E;
  if (D == 128) {
    hipLaunchKernelGGL((attn_fwd_kernel<128, GL, W, PP>), grid, dim3(NTHREADS), 0, stream,
                       (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, q_off, k_off, O, lse,
                       BH, (int)Lq, (int)Lk, kv_stride, koff_stride, nblk, first, nranks,
                       causal ? 1 : 0,
                       c_log2, n_qtiles);
  } else {
    hipLaunchKernelGGL((attn_fwd_kernel<64, GL, W, PP>), grid, dim3(NTHREADS), 0, stream,
                       (const __bf16*)Q, (const __bf16*)K, (const __bf16*)V, q_off, k_off, O, lse,
                       BH, (int)Lq, (int)Lk, kv_stride, koff_stride, nblk, first, nranks,
                       causal ? 1 : 0,
                       c_log2, n_qtiles);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_partial_mfma(const void* Q, const void* K, const void* V, const int64_t* q_off,
                               const int64_t* k_off, float* O, float* lse, int BH, int64_t Lq,
                               int64_t Lk, int D, bool causal, float scale, hipStream_t stream) {
  return launch_blocks<false, 4>(Q, K, V, q_off, k_off, O, lse, BH, Lq, Lk, 0, 0, 1, 0, 1, D,
                                 causal, scale, stream);
}

hipError_t launch_ring_mfma(const void* Q_i, const void* K_all, const void* V_all,
                            const int64_t* q_off, const int64_t* pos_all, float* O, float* lse,
                            int BH, int64_t Lr, int N, int i, int D, bool causal, float scale,
                            hipStream_t stream) {
  return launch_blocks<false, 4>(Q_i, K_all, V_all, q_off, pos_all, O, lse, BH, Lr, Lr,
                                 (int64_t)BH * Lr * D, Lr, N, i, 1, D, causal, scale, stream);
}

hipError_t launch_share_mfma(const void* Q, const void* K, const void* V, float* O, float* lse,
                             int BH, int64_t Lr, int N, int rank_lo, int nranks, int D,
                             bool causal, float scale, bool precise, hipStream_t stream) {
  if (precise)
    return launch_blocks<true, 8, true>(Q, K, V, nullptr, nullptr, O, lse, BH, Lr, Lr, 0, 0, N,
                                        rank_lo, nranks, D, causal, scale, stream);
  return launch_blocks<true, 8>(Q, K, V, nullptr, nullptr, O, lse, BH, Lr, Lr, 0, 0, N, rank_lo,
                                nranks, D, causal, scale, stream);
}

}  // namespace cpa
