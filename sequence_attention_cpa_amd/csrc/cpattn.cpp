// C-ABI layer of libcpattn: argument checks, the zigzag layout, and the ring
// driver that strings partial-attention and merge launches together.  Every
// check runs on the host before anything is enqueued; errors are returned as
// cpa_status with a per-thread message.  No exception leaves this file.
#include "cpattn.h"
#include "cpa_internal.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

// Device scratch of cpa_rank_forward_noalloc: the partial (O, lse) of one
// slice of a rank's rows.  Every GPU the library runs on holds its own copy
// for the life of the process; host code reaches it only through the address
// hipGetSymbolAddress returns for that device (the name is a host-side
// stand-in, not a device address).
constexpr size_t kNoallocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) char scratch[kNoallocScratchBytes];

namespace {

thread_local std::string g_err;

cpa_status fail(cpa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

cpa_status ok() {
  g_err.clear();
  return CPA_OK;
}

cpa_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(CPA_EHIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool supported_d(int32_t D) { return D == 16 || D == 64 || D == 128; }

// The row kernels put the (b, h) pair in grid.y, which holds at most 65535
// workgroups on every HIP target.
constexpr int64_t kMaxBH = 65535;

// A dispatch counts its work-items along x in 32 bits.  The matrix-core
// kernels (bf16, D = 64 or 128) launch cpa::kMfmaThreads threads on every
// cpa::kMfmaRows query rows of every (b, h) pair; the backward's dK/dV pass
// launches as many on every kMfmaRows key rows of every (b, h) pair and K/V
// block.  nblk_bwd = 0 checks the forward launch only.
cpa_status check_mfma_launch(cpa_dtype dt, int32_t D, int64_t BH, int64_t Lq, int64_t Lk,
                             int64_t nblk_bwd) {
  if (dt != CPA_BF16 || (D != 64 && D != 128)) return CPA_OK;
  const int64_t lim = (int64_t)UINT32_MAX;
  const int64_t qt = (Lq + cpa::kMfmaRows - 1) / cpa::kMfmaRows;
  const int64_t kt = (Lk + cpa::kMfmaRows - 1) / cpa::kMfmaRows;
  if (qt > lim / (BH * cpa::kMfmaThreads))
    return fail(CPA_ESHAPE, "launch of %lld query rows x %lld heads exceeds 2^32 work-items",
                (long long)Lq, (long long)BH);
  if (nblk_bwd > 0 && kt > lim / (BH * cpa::kMfmaThreads) / nblk_bwd)
    return fail(CPA_ESHAPE, "backward launch of %lld blocks x %lld key rows x %lld heads exceeds "
                            "2^32 work-items",
                (long long)nblk_bwd, (long long)Lk, (long long)BH);
  return CPA_OK;
}

cpa_status check_partial(const void* Q, const void* K, const void* V, cpa_dtype dt, int32_t B,
                         int32_t H, int64_t Lq, int64_t Lk, int32_t D, const int64_t* q_off,
                         const int64_t* k_off, int32_t causal, const float* O, const float* lse) {
  if (dt != CPA_BF16 && dt != CPA_F32) return fail(CPA_EDTYPE, "unknown dtype %d", (int)dt);
  if (B < 1 || H < 1) return fail(CPA_ESHAPE, "B and H must be >= 1 (B=%d, H=%d)", B, H);
  if (Lq < 0 || Lk < 0) return fail(CPA_ESHAPE, "Lq and Lk must be >= 0 (Lq=%lld, Lk=%lld)",
                                    (long long)Lq, (long long)Lk);
  if (Lq > (int64_t)1 << 30 || Lk > (int64_t)1 << 30)
    return fail(CPA_ESHAPE, "Lq and Lk are limited to 2^30 rows");
  if ((int64_t)B * H > kMaxBH) return fail(CPA_ESHAPE, "B*H is limited to %lld", (long long)kMaxBH);
  if (!supported_d(D)) return fail(CPA_EUNSUPPORTED, "head_dim %d not built (16, 64, 128)", D);
  if (Lq > 0 && (!Q || !O || !lse)) return fail(CPA_EINVAL, "null Q/O/lse pointer");
  if (Lq > 0 && Lk > 0 && (!K || !V)) return fail(CPA_EINVAL, "null K/V pointer");
  if (causal && Lq > 0 && Lk > 0 && (!q_off || !k_off))
    return fail(CPA_EINVAL, "causal attention needs q_off and k_off");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16))
    return fail(CPA_EINVAL, "Q, K, V and O must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(q_off, 8) || !aligned(k_off, 8))
    return fail(CPA_EINVAL, "lse must be 4-byte and offsets 8-byte aligned");
  return CPA_OK;
}

cpa_status enqueue_partial(const void* Q, const void* K, const void* V, cpa_dtype dt, int32_t B,
                           int32_t H, int64_t Lq, int64_t Lk, int32_t D, const int64_t* q_off,
                           const int64_t* k_off, int32_t causal, float scale, float* O, float* lse,
                           hipStream_t st) {
  if (Lq == 0) return ok();
  if (!(scale > 0.f)) scale = 1.0f / std::sqrt((float)D);
  const int BH = B * H;
  hipError_t e;
  if (Lk == 0) {
    // No keys at all: every row is empty.  The row-wise kernel writes (0, -inf)
    // without touching K/V.
    e = cpa::launch_partial_rowwise(Q, K, V, dt == CPA_BF16, q_off, k_off, O, lse, BH, Lq, 0, D,
                                    false, scale, st);
  } else if (dt == CPA_BF16 && (D == 64 || D == 128)) {
    e = cpa::launch_partial_mfma(Q, K, V, q_off, k_off, O, lse, BH, Lq, Lk, D, causal != 0, scale,
                                 st);
  } else {
    e = cpa::launch_partial_rowwise(Q, K, V, dt == CPA_BF16, q_off, k_off, O, lse, BH, Lq, Lk, D,
                                    causal != 0, scale, st);
  }
  return from_hip(e, "partial attention launch");
}

cpa_status check_rank_shape(int32_t N, int64_t L, int32_t B, int32_t H, int32_t D) {
  if (N < 1) return fail(CPA_EINVAL, "N must be >= 1 (N=%d)", N);
  if (L <= 0 || L % (2 * (int64_t)N) != 0)
    return fail(CPA_ESHAPE, "L must be > 0 and divisible by 2N (L=%lld, N=%d)", (long long)L, N);
  if (B < 1 || H < 1) return fail(CPA_ESHAPE, "B and H must be >= 1");
  if (D < 1) return fail(CPA_ESHAPE, "D must be >= 1");
  return CPA_OK;
}

cpa_status check_rope(cpa_dtype dt, int32_t B, int32_t H, int32_t D, double base,
                      int32_t pairing) {
  if (dt != CPA_BF16 && dt != CPA_F32) return fail(CPA_EDTYPE, "unknown dtype %d", (int)dt);
  if (B < 1 || H < 1) return fail(CPA_ESHAPE, "B and H must be >= 1 (B=%d, H=%d)", B, H);
  if ((int64_t)B * H > kMaxBH) return fail(CPA_ESHAPE, "B*H is limited to %lld", (long long)kMaxBH);
  if (D < 8 || D > 512 || D % 8 != 0)
    return fail(CPA_EUNSUPPORTED, "rope needs D a multiple of 8 in [8, 512] (D=%d)", D);
  if (!(base > 1.0) || !std::isfinite(base))
    return fail(CPA_EINVAL, "rope base must be finite and > 1 (base=%g)", base);
  if (pairing != CPA_ROPE_INTERLEAVED && pairing != CPA_ROPE_HALF)
    return fail(CPA_EINVAL, "unknown rope pairing %d", pairing);
  return CPA_OK;
}

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Address of `scratch` on the device that runs `stream` (the current device
// for the null stream), looked up once per device with that device current.
hipError_t noalloc_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    int prev = -1;
    hipError_t r = hipGetDevice(&prev);
    if (r == hipSuccess && prev != dev) r = hipSetDevice(dev);
    if (r == hipSuccess) r = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
    if (prev >= 0 && prev != dev) {
      const hipError_t r2 = hipSetDevice(prev);
      if (r == hipSuccess) r = r2;
    }
    g_scratch_err[dev] = r;
  });
  *out = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

}  // namespace

extern "C" {

const char* cpa_last_error(void) { return g_err.c_str(); }

const char* cpa_version(void) { return "libcpattn 0.2.0 gfx950"; }

cpa_status cpa_zigzag_layout(int64_t L, int32_t N, int64_t* out) {
  if (N < 1) return fail(CPA_EINVAL, "N must be >= 1 (N=%d)", N);
  if (L <= 0 || L % (2 * (int64_t)N) != 0)
    return fail(CPA_ESHAPE, "L must be > 0 and divisible by 2N (L=%lld, N=%d)", (long long)L, N);
  if (!out) return fail(CPA_EINVAL, "null output table");
  const int64_t C = L / (2 * (int64_t)N);
  const int64_t Lr = 2 * C;
  for (int64_t r = 0; r < N; ++r) {
    const int64_t early = r * C;                        // chunk r
    const int64_t late = (2 * (int64_t)N - 1 - r) * C;  // chunk 2N-1-r
    int64_t* row = out + r * Lr;
    for (int64_t t = 0; t < C; ++t) {
      row[t] = early + t;
      row[C + t] = late + t;
    }
  }
  return ok();
}

cpa_status cpa_partial(const void* Q, const void* K, const void* V, cpa_dtype dt, int32_t B,
                       int32_t H, int64_t Lq, int64_t Lk, int32_t D, const int64_t* q_off,
                       const int64_t* k_off, int32_t causal, float scale, float* O, float* lse,
                       void* stream) {
  cpa_status st = check_partial(Q, K, V, dt, B, H, Lq, Lk, D, q_off, k_off, causal, O, lse);
  if (st != CPA_OK) return st;
  if (Lk > 0 && (st = check_mfma_launch(dt, D, (int64_t)B * H, Lq, Lk, 0)) != CPA_OK) return st;
  return enqueue_partial(Q, K, V, dt, B, H, Lq, Lk, D, q_off, k_off, causal, scale, O, lse,
                         (hipStream_t)stream);
}

cpa_status cpa_merge(float* O_acc, float* lse_acc, const float* O_new, const float* lse_new,
                     int64_t rows, int32_t D, void* stream) {
  if (rows < 0) return fail(CPA_ESHAPE, "rows must be >= 0");
  if (!supported_d(D)) return fail(CPA_EUNSUPPORTED, "head_dim %d not built (16, 64, 128)", D);
  if (rows == 0) return ok();
  if (!O_acc || !lse_acc || !O_new || !lse_new) return fail(CPA_EINVAL, "null pointer");
  if (!aligned(O_acc, 16) || !aligned(O_new, 16)) return fail(CPA_EINVAL, "O must be 16-byte aligned");
  if (!aligned(lse_acc, 4) || !aligned(lse_new, 4)) return fail(CPA_EINVAL, "lse must be 4-byte aligned");
  return from_hip(cpa::launch_merge(O_acc, lse_acc, O_new, lse_new, rows, D, (hipStream_t)stream),
                  "merge launch");
}

size_t cpa_rank_forward_workspace(int32_t B, int32_t H, int64_t L, int32_t N, int32_t D) {
  if (N < 1 || B < 1 || H < 1 || D < 1 || L <= 0 || L % (2 * (int64_t)N) != 0) return 0;
  const size_t rows = (size_t)B * H * (size_t)(L / N);
  const size_t o_bytes = (rows * D * 4 + 255) / 256 * 256;
  const size_t l_bytes = (rows * 4 + 255) / 256 * 256;
  return o_bytes + l_bytes;
}

cpa_status cpa_rank_forward(int32_t i, int32_t N, const void* Q_i, const void* K_all,
                            const void* V_all, const int64_t* pos_all, cpa_dtype dt, int32_t B,
                            int32_t H, int64_t L, int32_t D, int32_t causal, float scale,
                            float* O_i, float* lse_i, void* ws, size_t ws_bytes, void* stream) {
  cpa_status st = check_rank_shape(N, L, B, H, D);
  if (st != CPA_OK) return st;
  if (i < 0 || i >= N) return fail(CPA_EINVAL, "rank index %d outside [0, %d)", i, N);
  if (!pos_all) return fail(CPA_EINVAL, "null pos_all");
  const int64_t Lr = L / N;
  st = check_partial(Q_i, K_all, V_all, dt, B, H, Lr, Lr, D, pos_all, pos_all, causal, O_i, lse_i);
  if (st != CPA_OK) return st;
  st = check_mfma_launch(dt, D, (int64_t)B * H, Lr, Lr, 0);
  if (st != CPA_OK) return st;
  const size_t need = cpa_rank_forward_workspace(B, H, L, N, D);
  if (N > 1) {
    if (!ws) return fail(CPA_EINVAL, "null workspace");
    if (ws_bytes < need)
      return fail(CPA_EINVAL, "workspace too small: %zu bytes, need %zu", ws_bytes, need);
    if (!aligned(ws, 256)) return fail(CPA_EINVAL, "workspace must be 256-byte aligned");
  }
  const size_t esz = dt == CPA_BF16 ? 2 : 4;
  const size_t rank_elems = (size_t)B * H * Lr * D;
  const size_t rows = (size_t)B * H * Lr;
  float* tO = (float*)ws;
  float* tl = (float*)((char*)ws + (rows * D * 4 + 255) / 256 * 256);
  hipStream_t hs = (hipStream_t)stream;
  const int64_t* q_off = pos_all + (int64_t)i * Lr;
  for (int32_t s = 0; s < N; ++s) {
    const int32_t j = (i + s) % N;  // ring order: own block first, then i+1, i+2, ...
    const char* Kj = (const char*)K_all + (size_t)j * rank_elems * esz;
    const char* Vj = (const char*)V_all + (size_t)j * rank_elems * esz;
    const int64_t* k_off = pos_all + (int64_t)j * Lr;
    if (s == 0) {
      st = enqueue_partial(Q_i, Kj, Vj, dt, B, H, Lr, Lr, D, q_off, k_off, causal, scale, O_i,
                           lse_i, hs);
      if (st != CPA_OK) return st;
    } else {
      st = enqueue_partial(Q_i, Kj, Vj, dt, B, H, Lr, Lr, D, q_off, k_off, causal, scale, tO, tl,
                           hs);
      if (st != CPA_OK) return st;
      st = from_hip(cpa::launch_merge(O_i, lse_i, tO, tl, (int64_t)rows, D, hs), "merge launch");
      if (st != CPA_OK) return st;
    }
  }
  return ok();
}

cpa_status cpa_rank_forward_noalloc(int32_t i, int32_t N, const void* Q_i, const void* K_all,
                                    const void* V_all, const int64_t* pos_all, cpa_dtype dt,
                                    int32_t B, int32_t H, int64_t L, int32_t D, int32_t causal,
                                    float scale, float* O_i, float* lse_i, void* stream) {
  cpa_status st = check_rank_shape(N, L, B, H, D);
  if (st != CPA_OK) return st;
  if (i < 0 || i >= N) return fail(CPA_EINVAL, "rank index %d outside [0, %d)", i, N);
  if (!pos_all) return fail(CPA_EINVAL, "null pos_all");
  const int64_t Lr = L / N;
  st = check_partial(Q_i, K_all, V_all, dt, B, H, Lr, Lr, D, pos_all, pos_all, causal, O_i, lse_i);
  if (st != CPA_OK) return st;
  st = check_mfma_launch(dt, D, (int64_t)B * H, Lr, Lr, 0);
  if (st != CPA_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  char* ws = nullptr;
  if (N > 1) {
    void* p = nullptr;
    const hipError_t e = noalloc_scratch(hs, &p);
    if (e != hipSuccess) return from_hip(e, "device scratch lookup");
    ws = (char*)p;
  }
  // The partial of a slice fits the scratch: whole heads at a time when a
  // head does (O at the start, lse 256-byte aligned after it), else row
  // ranges of one head.
  const int64_t cap = (int64_t)((kNoallocScratchBytes - 512) / ((size_t)(D + 1) * 4));
  const int64_t BH = (int64_t)B * H;
  const int64_t heads_per = Lr <= cap ? (BH < cap / Lr ? BH : cap / Lr) : 1;
  const int64_t rows_per = Lr <= cap ? Lr : cap;
  const size_t esz = dt == CPA_BF16 ? 2 : 4;
  for (int64_t h0 = 0; h0 < BH; h0 += heads_per) {
    const int64_t nh = BH - h0 < heads_per ? BH - h0 : heads_per;
    for (int64_t r0 = 0; r0 < Lr; r0 += rows_per) {
      const int64_t nr = Lr - r0 < rows_per ? Lr - r0 : rows_per;
      const int64_t row0 = h0 * Lr + r0;  // first O row of the slice
      const char* Qs = (const char*)Q_i + (size_t)row0 * D * esz;
      float* Os = O_i + row0 * D;
      float* ls = lse_i + row0;
      const int64_t* q_off = pos_all + (int64_t)i * Lr + r0;
      float* tO = (float*)ws;
      float* tl = (float*)(ws + ((size_t)(nh * nr) * D * 4 + 255) / 256 * 256);
      for (int32_t s = 0; s < N; ++s) {
        const int32_t j = (i + s) % N;  // ring order: own block first, then i+1, i+2, ...
        const size_t blk = ((size_t)j * BH + h0) * Lr * D * esz;
        const char* Kj = (const char*)K_all + blk;
        const char* Vj = (const char*)V_all + blk;
        const int64_t* k_off = pos_all + (int64_t)j * Lr;
        st = enqueue_partial(Qs, Kj, Vj, dt, 1, (int32_t)nh, nr, Lr, D, q_off, k_off, causal,
                             scale, s == 0 ? Os : tO, s == 0 ? ls : tl, hs);
        if (st != CPA_OK) return st;
        if (s > 0) {
          st = from_hip(cpa::launch_merge(Os, ls, tO, tl, nh * nr, D, hs), "merge launch");
          if (st != CPA_OK) return st;
        }
      }
    }
  }
  return ok();
}

cpa_status cpa_rank_forward_fused(int32_t i, int32_t N, const void* Q_i, const void* K_all,
                                  const void* V_all, const int64_t* pos_all, cpa_dtype dt,
                                  int32_t B, int32_t H, int64_t L, int32_t D, int32_t causal,
                                  float scale, float* O_i, float* lse_i, void* stream) {
  cpa_status st = check_rank_shape(N, L, B, H, D);
  if (st != CPA_OK) return st;
  if (i < 0 || i >= N) return fail(CPA_EINVAL, "rank index %d outside [0, %d)", i, N);
  if (!pos_all) return fail(CPA_EINVAL, "null pos_all");
  const int64_t Lr = L / N;
  st = check_partial(Q_i, K_all, V_all, dt, B, H, Lr, Lr, D, pos_all, pos_all, causal, O_i, lse_i);
  if (st != CPA_OK) return st;
  st = check_mfma_launch(dt, D, (int64_t)B * H, Lr, Lr, 0);
  if (st != CPA_OK) return st;
  if (dt != CPA_BF16 || (D != 64 && D != 128))
    return fail(CPA_EUNSUPPORTED, "fused ring needs bf16 with D = 64 or 128 (use cpa_rank_forward)");
  if (!(scale > 0.f)) scale = 1.0f / std::sqrt((float)D);
  return from_hip(cpa::launch_ring_mfma(Q_i, K_all, V_all, pos_all + (int64_t)i * Lr, pos_all, O_i,
                                        lse_i, B * H, Lr, N, i, D, causal != 0, scale,
                                        (hipStream_t)stream),
                  "fused ring launch");
}

cpa_status cpa_zigzag_permute(const void* src, void* dst, int32_t elem_bytes, int32_t B,
                              int32_t H, int64_t L, int32_t D, const int64_t* pos_all, int32_t N,
                              int32_t rank_lo, int32_t rank_hi, int32_t inverse, void* stream) {
  if (elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8)
    return fail(CPA_EDTYPE, "elem_bytes must be 2, 4 or 8 (got %d)", elem_bytes);
  cpa_status st = check_rank_shape(N, L, B, H, D);
  if (st != CPA_OK) return st;
  if (rank_lo < 0 || rank_hi > N || rank_lo >= rank_hi)
    return fail(CPA_EINVAL, "rank range [%d, %d) invalid for N=%d", rank_lo, rank_hi, N);
  const int64_t row_bytes = (int64_t)D * elem_bytes;
  if (row_bytes % 4 != 0) return fail(CPA_ESHAPE, "row bytes D*elem_bytes must be a multiple of 4");
  if (!src || !dst || !pos_all) return fail(CPA_EINVAL, "null pointer");
  if (!aligned(src, 16) || !aligned(dst, 16)) return fail(CPA_EINVAL, "src/dst must be 16-byte aligned");
  if (!aligned(pos_all, 8)) return fail(CPA_EINVAL, "pos_all must be 8-byte aligned");
  return from_hip(cpa::launch_permute(src, dst, row_bytes, (int64_t)B * H, L, pos_all, N, rank_lo,
                                      rank_hi, inverse != 0, (hipStream_t)stream),
                  "permute launch");
}

cpa_status cpa_check_offsets(const int64_t* off, int64_t rows, int64_t n, int64_t* first_bad,
                             void* stream) {
  if (rows < 0 || n < 0) return fail(CPA_ESHAPE, "rows and n must be >= 0 (rows=%lld, n=%lld)",
                                     (long long)rows, (long long)n);
  if (n > 0 && rows > ((int64_t)1 << 62) / n)
    return fail(CPA_ESHAPE, "rows * n is limited to 2^62 entries");
  if (!first_bad) return fail(CPA_EINVAL, "null first_bad");
  if (rows * n > 0 && !off) return fail(CPA_EINVAL, "null offset table");
  if (!aligned(off, 8) || !aligned(first_bad, 8))
    return fail(CPA_EINVAL, "off and first_bad must be 8-byte aligned");
  return from_hip(cpa::launch_check_offsets(off, rows, n, first_bad, (hipStream_t)stream),
                  "offsets check launch");
}

cpa_status cpa_rope(const void* x, void* y, cpa_dtype dt, int32_t B, int32_t H, int64_t rows,
                    int32_t D, const int64_t* pos, double base, int32_t pairing, void* stream) {
  cpa_status st = check_rope(dt, B, H, D, base, pairing);
  if (st != CPA_OK) return st;
  if (rows < 0) return fail(CPA_ESHAPE, "rows must be >= 0 (rows=%lld)", (long long)rows);
  if (rows == 0) return ok();
  if (!x || !y || !pos) return fail(CPA_EINVAL, "null pointer");
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(CPA_EINVAL, "x/y must be 16-byte aligned");
  if (!aligned(pos, 8)) return fail(CPA_EINVAL, "pos must be 8-byte aligned");
  return from_hip(cpa::launch_rope(x, y, dt == CPA_BF16, (int64_t)B * H, rows, rows, 1, D, pos,
                                   false, base, pairing == CPA_ROPE_HALF, (hipStream_t)stream),
                  "rope launch");
}

cpa_status cpa_zigzag_permute_rope(const void* src, void* dst, cpa_dtype dt, int32_t B, int32_t H,
                                   int64_t L, int32_t D, const int64_t* pos_all, int32_t N,
                                   int32_t rank_lo, int32_t rank_hi, double base, int32_t pairing,
                                   void* stream) {
  cpa_status st = check_rope(dt, B, H, D, base, pairing);
  if (st != CPA_OK) return st;
  st = check_rank_shape(N, L, B, H, D);
  if (st != CPA_OK) return st;
  if (rank_lo < 0 || rank_hi > N || rank_lo >= rank_hi)
    return fail(CPA_EINVAL, "rank range [%d, %d) invalid for N=%d", rank_lo, rank_hi, N);
  if (!src || !dst || !pos_all) return fail(CPA_EINVAL, "null pointer");
  if (!aligned(src, 16) || !aligned(dst, 16)) return fail(CPA_EINVAL, "src/dst must be 16-byte aligned");
  if (!aligned(pos_all, 8)) return fail(CPA_EINVAL, "pos_all must be 8-byte aligned");
  const int64_t Lr = L / N;
  return from_hip(cpa::launch_rope(src, dst, dt == CPA_BF16, (int64_t)B * H, L, Lr,
                                   rank_hi - rank_lo, D, pos_all + (int64_t)rank_lo * Lr, true,
                                   base, pairing == CPA_ROPE_HALF, (hipStream_t)stream),
                  "permute+rope launch");
}

namespace {

cpa_status share_forward(const void* Q, const void* K, const void* V, cpa_dtype dt, int32_t B,
                         int32_t H, int64_t L, int32_t D, int32_t N, int32_t rank_lo,
                         int32_t rank_hi, int32_t causal, float scale, float* O, float* lse,
                         bool precise, void* stream) {
  if (dt != CPA_BF16 && dt != CPA_F32) return fail(CPA_EDTYPE, "unknown dtype %d", (int)dt);
  cpa_status st = check_rank_shape(N, L, B, H, D);
  if (st != CPA_OK) return st;
  if (rank_lo < 0 || rank_hi > N || rank_lo >= rank_hi)
    return fail(CPA_EINVAL, "rank range [%d, %d) invalid for N=%d", rank_lo, rank_hi, N);
  const int64_t Lr = L / N;
  if (dt != CPA_BF16 || (D != 64 && D != 128))
    return fail(CPA_EUNSUPPORTED, "the global-layout ring runs bf16 with D = 64 or 128");
  if ((Lr / 2) % 32 != 0)
    return fail(CPA_EUNSUPPORTED, "the global-layout ring needs chunks L/(2N) that are multiples "
                                  "of 32 (L=%lld, N=%d); use the rank-major path",
                (long long)L, N);
  if (Lr > ((int64_t)1 << 30)) return fail(CPA_ESHAPE, "L/N is limited to 2^30 rows");
  if ((int64_t)B * H > kMaxBH) return fail(CPA_ESHAPE, "B*H is limited to %lld", (long long)kMaxBH);
  // one launch covers every selected rank
  st = check_mfma_launch(dt, D, (int64_t)B * H * (rank_hi - rank_lo), Lr, Lr, 0);
  if (st != CPA_OK) return st;
  if (!Q || !K || !V || !O || !lse) return fail(CPA_EINVAL, "null pointer");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16))
    return fail(CPA_EINVAL, "Q, K, V and O must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(CPA_EINVAL, "lse must be 4-byte aligned");
  if (!(scale > 0.f)) scale = 1.0f / std::sqrt((float)D);
  return from_hip(cpa::launch_share_mfma(Q, K, V, O, lse, B * H, Lr, N, rank_lo,
                                         rank_hi - rank_lo, D, causal != 0, scale, precise,
                                         (hipStream_t)stream),
                  "global-layout ring launch");
}

}  // namespace

cpa_status cpa_share_forward(const void* Q, const void* K, const void* V, cpa_dtype dt, int32_t B,
                             int32_t H, int64_t L, int32_t D, int32_t N,
                             int32_t rank_lo, int32_t rank_hi, int32_t causal, float scale,
                             float* O, float* lse, void* stream) {
  return share_forward(Q, K, V, dt, B, H, L, D, N, rank_lo, rank_hi, causal, scale, O, lse, false,
                       stream);
}

cpa_status cpa_share_forward_precise(const void* Q, const void* K, const void* V, cpa_dtype dt,
                                     int32_t B, int32_t H, int64_t L, int32_t D, int32_t N,
                                     int32_t rank_lo, int32_t rank_hi, int32_t causal,
                                     float scale, float* O, float* lse, void* stream) {
  return share_forward(Q, K, V, dt, B, H, L, D, N, rank_lo, rank_hi, causal, scale, O, lse, true,
                       stream);
}

cpa_status cpa_backward_delta(const float* O, const void* dO, cpa_dtype dt, int64_t rows,
                              int32_t D, float* delta, void* stream) {
  if (dt != CPA_BF16 && dt != CPA_F32) return fail(CPA_EDTYPE, "unknown dtype %d", (int)dt);
  if (rows < 0) return fail(CPA_ESHAPE, "rows must be >= 0");
  if (!supported_d(D)) return fail(CPA_EUNSUPPORTED, "head_dim %d not built (16, 64, 128)", D);
  if (rows == 0) return ok();
  if (!O || !dO || !delta) return fail(CPA_EINVAL, "null pointer");
  if (!aligned(O, 16) || !aligned(dO, 16) || !aligned(delta, 4))
    return fail(CPA_EINVAL, "O and dO must be 16-byte aligned, delta 4-byte");
  return from_hip(cpa::launch_bwd_delta(O, dO, dt == CPA_BF16, rows, D, delta,
                                        (hipStream_t)stream),
                  "backward delta launch");
}

cpa_status cpa_partial_backward(const void* Q, const void* K, const void* V, const void* dO,
                                const float* lse, const float* delta, cpa_dtype dt, int32_t B,
                                int32_t H, int64_t Lq, int64_t Lk, int32_t D,
                                const int64_t* q_off, const int64_t* k_off, int32_t causal,
                                float scale, float* dQ, float* dK, float* dV, void* stream) {
  cpa_status st = check_partial(Q, K, V, dt, B, H, Lq, Lk, D, q_off, k_off, causal, dQ, lse);
  if (st != CPA_OK) return st;
  if (Lq == 0 || Lk == 0) return ok();  // no pair: every contribution is zero
  st = check_mfma_launch(dt, D, (int64_t)B * H, Lq, Lk, 1);
  if (st != CPA_OK) return st;
  if (!dO || !delta || !dK || !dV) return fail(CPA_EINVAL, "null dO/delta/dK/dV pointer");
  if (!aligned(dO, 16) || !aligned(dK, 16) || !aligned(dV, 16) || !aligned(delta, 4))
    return fail(CPA_EINVAL, "dO, dK and dV must be 16-byte aligned, delta 4-byte");
  if (!(scale > 0.f)) scale = 1.0f / std::sqrt((float)D);
  const int BH = B * H;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (dt == CPA_BF16 && (D == 64 || D == 128))
    e = cpa::launch_bwd_mfma(Q, K, V, dO, lse, delta, q_off, k_off, dQ, dK, dV, BH, Lq, Lk, 0, 0,
                             1, 0, D, causal != 0, scale, true, s);
  else
    e = cpa::launch_bwd_rowwise(Q, K, V, dO, dt == CPA_BF16, lse, delta, q_off, k_off, dQ, dK, dV,
                                BH, Lq, Lk, D, causal != 0, scale, true, s);
  return from_hip(e, "partial backward launch");
}

cpa_status cpa_rank_backward(int32_t i, int32_t N, const void* Q_i, const void* K_all,
                             const void* V_all, const int64_t* pos_all, const float* O_i,
                             const void* dO_i, const float* lse_i, cpa_dtype dt, int32_t B,
                             int32_t H, int64_t L, int32_t D, int32_t causal, float scale,
                             float* dQ_i, float* dK_all, float* dV_all, float* delta_i,
                             void* stream) {
  cpa_status st = check_rank_shape(N, L, B, H, D);
  if (st != CPA_OK) return st;
  if (i < 0 || i >= N) return fail(CPA_EINVAL, "rank index %d outside [0, %d)", i, N);
  const int64_t Lr = L / N;
  if (!pos_all) return fail(CPA_EINVAL, "null pos_all");
  st = check_partial(Q_i, K_all, V_all, dt, B, H, Lr, Lr, D, pos_all, pos_all, causal, dQ_i,
                     lse_i);
  if (st != CPA_OK) return st;
  st = check_mfma_launch(dt, D, (int64_t)B * H, Lr, Lr, N);
  if (st != CPA_OK) return st;
  if (!O_i || !dO_i || !dK_all || !dV_all || !delta_i)
    return fail(CPA_EINVAL, "null O/dO/dK/dV/delta pointer");
  if (!aligned(O_i, 16) || !aligned(dO_i, 16) || !aligned(dK_all, 16) || !aligned(dV_all, 16) ||
      !aligned(delta_i, 4))
    return fail(CPA_EINVAL, "O, dO, dK and dV must be 16-byte aligned, delta 4-byte");
  if (!(scale > 0.f)) scale = 1.0f / std::sqrt((float)D);
  const int BH = B * H;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = cpa::launch_bwd_delta(O_i, dO_i, dt == CPA_BF16, (int64_t)BH * Lr, D, delta_i, s);
  if (e != hipSuccess) return from_hip(e, "backward delta launch");
  const int64_t* q_off = pos_all + (int64_t)i * Lr;
  const int64_t blk = (int64_t)BH * Lr * D;  // elements per rank block
  const size_t eb = dt == CPA_BF16 ? 2 : 4;
  if (dt == CPA_BF16 && (D == 64 || D == 128)) {
    e = cpa::launch_bwd_mfma(Q_i, K_all, V_all, dO_i, lse_i, delta_i, q_off, pos_all, dQ_i,
                             dK_all, dV_all, BH, Lr, Lr, blk, Lr, N, i, D, causal != 0, scale,
                             false, s);
    return from_hip(e, "ring backward launch");
  }
  for (int32_t step = 0; step < N; ++step) {
    const int32_t j = (i + step) % N;
    const char* Kj = (const char*)K_all + (size_t)j * blk * eb;
    const char* Vj = (const char*)V_all + (size_t)j * blk * eb;
    e = cpa::launch_bwd_rowwise(Q_i, Kj, Vj, dO_i, dt == CPA_BF16, lse_i, delta_i, q_off,
                                pos_all + (int64_t)j * Lr, dQ_i, dK_all + j * blk,
                                dV_all + j * blk, BH, Lr, Lr, D, causal != 0, scale, step > 0, s);
    if (e != hipSuccess) return from_hip(e, "ring backward launch");
  }
  return ok();
}

cpa_status cpa_share_backward(const void* Q, const void* K, const void* V, const float* O,
                              const void* dO, const float* lse, cpa_dtype dt,
                              int32_t B, int32_t H, int64_t L, int32_t D, int32_t N,
                              int32_t rank_lo, int32_t rank_hi, int32_t causal, float scale,
                              float* dQ, float* dK, float* dV, float* delta, void* stream) {
  if (dt != CPA_BF16 && dt != CPA_F32) return fail(CPA_EDTYPE, "unknown dtype %d", (int)dt);
  cpa_status st = check_rank_shape(N, L, B, H, D);
  if (st != CPA_OK) return st;
  if (rank_lo < 0 || rank_hi > N || rank_lo >= rank_hi)
    return fail(CPA_EINVAL, "rank range [%d, %d) invalid for N=%d", rank_lo, rank_hi, N);
  const int64_t Lr = L / N;
  if (dt != CPA_BF16 || (D != 64 && D != 128))
    return fail(CPA_EUNSUPPORTED, "the global-layout backward runs bf16 with D = 64 or 128");
  if ((Lr / 2) % 32 != 0)
    return fail(CPA_EUNSUPPORTED, "the global-layout backward needs chunks L/(2N) that are "
                                  "multiples of 32 (L=%lld, N=%d); use the rank-major path",
                (long long)L, N);
  if (Lr > ((int64_t)1 << 30)) return fail(CPA_ESHAPE, "L/N is limited to 2^30 rows");
  if ((int64_t)B * H > kMaxBH) return fail(CPA_ESHAPE, "B*H is limited to %lld", (long long)kMaxBH);
  st = check_mfma_launch(dt, D, (int64_t)B * H, Lr, Lr, N);
  if (st != CPA_OK) return st;
  if (!Q || !K || !V || !O || !dO || !lse || !dQ || !dK || !dV || !delta)
    return fail(CPA_EINVAL, "null pointer");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) ||
      !aligned(dO, 16) || !aligned(dQ, 16) || !aligned(dK, 16) || !aligned(dV, 16))
    return fail(CPA_EINVAL, "Q, K, V, O, dO, dQ, dK and dV must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(delta, 4))
    return fail(CPA_EINVAL, "lse and delta must be 4-byte aligned");
  if (!(scale > 0.f)) scale = 1.0f / std::sqrt((float)D);
  const int BH = B * H;
  hipStream_t s = (hipStream_t)stream;
  for (int32_t r = rank_lo; r < rank_hi; ++r) {
    hipError_t e = cpa::launch_bwd_delta_share(O, dO, BH, Lr, N, r, D, delta, s);
    if (e != hipSuccess) return from_hip(e, "backward delta launch");
    e = cpa::launch_bwd_share_mfma(Q, K, V, dO, lse, delta, dQ, dK, dV, BH, Lr, N, r, D,
                                   causal != 0, scale, s);
    if (e != hipSuccess) return from_hip(e, "global-layout ring backward launch");
  }
  return ok();
}

}  // extern "C"
