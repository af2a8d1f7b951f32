// internal.h -- launch interfaces shared by the host library and the kernels
// of the W4A16 MoE layer. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Bucketing: stable counting sort of valid (token, slot) pairs by local expert.
// launch_align: one work-group; E <= kMaxExperts. launch_align_multi: the
// same result from many work-groups (three launches), with
// align_scratch_ints(P, E) int32 of scratch.
constexpr int kMaxExperts = 512;
hipError_t launch_align(const int32_t* topk_ids, int64_t P, int32_t E, int32_t base,
                        int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
                        int32_t* n_padded, hipStream_t stream);
int64_t align_scratch_ints(int64_t P, int32_t E);
hipError_t launch_align_multi(const int32_t* topk_ids, int64_t P, int32_t E, int32_t base,
                              int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
                              int32_t* n_padded, int32_t* scratch, hipStream_t stream);

// Operands of one grouped-GEMM launch (routed blocks followed by shared-expert
// row tiles). Widths are in elements.
struct GemmParams {
  // routed part
  const uint16_t* a_routed;     // gate_up: x [T, H]; down: h [rows, I] (sorted order)
  const int32_t* sorted_ids;    // [max_blocks * bm]
  const int32_t* block_expert;  // [max_blocks]
  const int32_t* n_padded;      // [1]
  const int32_t* packed;        // int4 codes [E, Nw, K/8]
  const uint16_t* scales;       // bf16 [E, Nw, K/32]
  int32_t max_blocks;
  // shared part (absent when wshared == nullptr)
  const uint16_t* a_shared;     // gate_up: x [T, H]; down: hs [T, I]
  const uint16_t* wshared;      // bf16 [Nw, K]
  // outputs
  uint16_t* h_routed;           // gate_up: h [max_blocks * bm, I]
  uint16_t* h_shared;           // gate_up: hs [T, I]
  float* y_routed;              // down: y [T*k, H], row = pair id
  float* y_shared;              // down: s [T, H]
  // sizes
  int64_t T;
  int64_t P;                    // T * k (sentinel value)
  int32_t k;
  int32_t K;                    // reduction width (H for gate_up, I for down)
  int32_t I;                    // intermediate width
  int32_t N;                    // output width (I for gate_up, H for down)
  uint32_t nibble_mask;         // 0x0F0F0F0F (a run-time value on purpose)
};

hipError_t launch_gate_up(const GemmParams& p, int32_t block_m, hipStream_t stream);
hipError_t launch_down(const GemmParams& p, int32_t block_m, hipStream_t stream);

// Small-batch variants (buckets padded to 4 rows; see gemm_small.hip).
// small_batch_fits: whether their staged scales fit in LDS for these widths.
bool small_batch_fits(int32_t hidden, int32_t inter);
hipError_t launch_gate_up_small(const GemmParams& p, hipStream_t stream);
hipError_t launch_down_small(const GemmParams& p, hipStream_t stream);

// Routed int4 experts in 128-row blocks (prefill-sized batches; see
// gemm_prefill.hip). prefill_fits: whether the widths suit its tiles.
bool prefill_fits(int32_t hidden, int32_t inter);
int32_t prefill_block_m();  // bucket rows per block of that path
hipError_t launch_gate_up_prefill(const GemmParams& p, hipStream_t stream);
hipError_t launch_down_prefill(const GemmParams& p, hipStream_t stream);

// Router step: for each of T tokens, the k largest of S fp32 scores (equal
// scores: lower expert first), descending, and weights = softmax over them.
constexpr int32_t kMaxScored = 1024;  // scores per token (experts of the model)
hipError_t launch_route(const float* scores, int64_t T, int32_t S, int32_t k, int32_t* topk_ids,
                        float* topk_weights, hipStream_t stream);
// Dense bf16 GEMM of the shared expert (hipBLASLt; see shared_blas.cpp):
// out [T, rows] fp32 = act [T, K] . weights [rows, K]^T, with
// kSharedBlasWorkspace bytes of library workspace. hipErrorNotSupported when
// the library offers no algorithm for the shape (nothing was launched).
constexpr size_t kSharedBlasWorkspace = size_t(32) << 20;
hipError_t launch_shared_blas(const uint16_t* weights, const uint16_t* act, float* out,
                              int64_t rows, int64_t T, int64_t K, void* workspace,
                              hipStream_t stream);
// h [T, I] bf16 = silu(gu[:, :I]) * gu[:, I:] from fp32 gu [T, 2I].
hipError_t launch_swiglu(const float* gu, uint16_t* h, int64_t T, int32_t I, hipStream_t stream);
// out[t] = bf16(s[t] + sum_j valid * w[t,j] * y[t*k+j]), fp32 sum in slot order.
hipError_t launch_combine(const float* y, const float* s, const int32_t* topk_ids,
                          const float* topk_weights, uint16_t* out, int64_t T, int32_t H,
                          int32_t k, int32_t E, int32_t base, hipStream_t stream);

}  // namespace moe
