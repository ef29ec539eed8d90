// Internal launch interface between the C-ABI host layer (cpattn.cpp) and the
// HIP kernels.  Arguments are already validated by the caller; each launcher
// enqueues on `stream` and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace cpa {

// Launch shape of the matrix-core kernels (partial_attn.hip, attn_backward.hip
// assert that they match): threads per workgroup, and query rows (forward, dQ
// pass) or key rows (dK/dV pass, twice the threads) per workgroup.
constexpr int kMfmaThreads = 256;
constexpr int kMfmaRows = 128;

// Partial attention, bf16 inputs on the matrix cores (D = 64 or 128).
hipError_t launch_partial_mfma(const void* Q, const void* K, const void* V,
                               const int64_t* q_off, const int64_t* k_off, float* O,
                               float* lse, int BH, int64_t Lq, int64_t Lk, int D, bool causal,
                               float scale, hipStream_t stream);

// Rank i's whole ring in one launch: Q_i [BH, Lr, D] against the N blocks of
// rank-major K_all / V_all [N, BH, Lr, D] (positions pos_all [N, Lr]) in the
// order i+1, ..., i+N-1, i, online-softmax state kept in registers (D = 64 or 128).
hipError_t launch_ring_mfma(const void* Q_i, const void* K_all, const void* V_all,
                            const int64_t* q_off, const int64_t* pos_all, float* O, float* lse,
                            int BH, int64_t Lr, int N, int i, int D, bool causal, float scale,
                            hipStream_t stream);

// The whole rings of ranks [rank_lo, rank_lo + nranks) in one launch on
// global-order data: Q, K, V [BH, N*Lr, D] and O, lse [BH, N*Lr, ...] in
// global token order, rank r's local row u at zigzag row zig(r, u), which is
// also its position (the causal bounds are that closed form).  Requires
// Lr/2 % 32 == 0; writes only those ranks' rows.
hipError_t launch_share_mfma(const void* Q, const void* K, const void* V, float* O, float* lse,
                             int BH, int64_t Lr, int N, int rank_lo, int nranks, int D,
                             bool causal, float scale, bool precise, hipStream_t stream);

// Partial attention, one query row per thread, fp32 arithmetic throughout
// (fp32 inputs, and bf16 inputs with D = 16).
hipError_t launch_partial_rowwise(const void* Q, const void* K, const void* V, bool bf16,
                                  const int64_t* q_off, const int64_t* k_off, float* O,
                                  float* lse, int BH, int64_t Lq, int64_t Lk, int D, bool causal,
                                  float scale, hipStream_t stream);

// In-place online-softmax merge of `rows` rows of D floats.
hipError_t launch_merge(float* O_acc, float* lse_acc, const float* O_new, const float* lse_new,
                        int64_t rows, int D, hipStream_t stream);

// Row gather/scatter between [BH, L, row_bytes] and rank-major [nr, BH, L/N, row_bytes].
hipError_t launch_permute(const void* src, void* dst, int64_t row_bytes, int64_t BH, int64_t L,
                          const int64_t* pos_all, int N, int rank_lo, int rank_hi, bool inverse,
                          hipStream_t stream);

// first_bad <- smallest i with i % n != 0 and off[i] <= off[i - 1] over
// `rows` tables of n positions, or rows * n if there is none.
hipError_t launch_check_offsets(const int64_t* off, int64_t rows, int64_t n, int64_t* first_bad,
                                hipStream_t stream);

// Rotary position embedding of rows at given global positions (D % 8 == 0).
// Index space: nr x Lr positions pos[rr*Lr + t]; destination rows
// (rr*BH + bh)*Lr + t of [nr, BH, Lr, D]; source rows bh*L + p of global
// [BH, L, D] when `gather`, else the destination's own layout (may alias dst).
hipError_t launch_rope(const void* src, void* dst, bool bf16, int64_t BH, int64_t L, int64_t Lr,
                       int64_t nr, int D, const int64_t* pos, bool gather, double base, bool half,
                       hipStream_t stream);

// Backward: delta[r] = sum_d dO[r, d] O[r, d] for `rows` rows (D in {16, 64, 128}).
hipError_t launch_bwd_delta(const float* O, const void* dO, bool bf16, int64_t rows, int D,
                            float* delta, hipStream_t stream);

// Backward on the matrix cores (bf16, D = 64 or 128): dQ of the queries over
// nblk K/V blocks (block b at K + b*kv_stride, positions k_off + b*koff_stride,
// visited first+1, ..., first), written or added (acc_dq), and every block's
// dK / dV contributions added into dK / dV (same block layout, fp32).
hipError_t launch_bwd_mfma(const void* Q, const void* K, const void* V, const void* dO,
                           const float* lse, const float* delta, const int64_t* q_off,
                           const int64_t* k_off, float* dQ, float* dK, float* dV, int BH,
                           int64_t Lq, int64_t Lk, int64_t kv_stride, int64_t koff_stride,
                           int nblk, int first, int D, bool causal, float scale, bool acc_dq,
                           hipStream_t stream);

// Backward of ranks' shares on global-order data (bf16, D = 64 or 128, Lr/2
// % 32 == 0): tensors are [BH, N*Lr, ...] in global token order and rank r's
// local row u is global row zig(r, u).  delta of rank i's rows; then rank
// i's dQ (written) and its contributions to every block's dK / dV (added).
// Positions are the zigzag closed form (a row's global index).
hipError_t launch_bwd_delta_share(const float* O, const void* dO, int BH, int64_t Lr, int N,
                                  int i, int D, float* delta, hipStream_t stream);
hipError_t launch_bwd_share_mfma(const void* Q, const void* K, const void* V, const void* dO,
                                 const float* lse, const float* delta, float* dQ, float* dK,
                                 float* dV, int BH, int64_t Lr, int N, int i, int D, bool causal,
                                 float scale, hipStream_t stream);

// Backward of one block, one row per thread in fp32 (fp32 inputs; bf16 with D = 16).
hipError_t launch_bwd_rowwise(const void* Q, const void* K, const void* V, const void* dO,
                              bool bf16, const float* lse, const float* delta,
                              const int64_t* q_off, const int64_t* k_off, float* dQ, float* dK,
                              float* dV, int BH, int64_t Lq, int64_t Lk, int D, bool causal,
                              float scale, bool acc_dq, hipStream_t stream);

}  // namespace cpa
