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
// The split form (one work-group): experts with at most tau pairs are
// bucketed into the second set of arrays with block size block_m2, the others
// into the first; each set as launch_align would bucket its experts alone.
hipError_t launch_align_split(const int32_t* topk_ids, int64_t P, int32_t E, int32_t base,
                              int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
                              int32_t* n_padded, int32_t tau, int32_t block_m2,
                              int32_t* sorted2, int32_t* block_expert2, int32_t* n_padded2,
                              hipStream_t stream);
int64_t align_scratch_ints(int64_t P, int32_t E);
hipError_t launch_align_multi(const int32_t* topk_ids, int64_t P, int32_t E, int32_t base,
                              int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
                              int32_t* n_padded, int32_t* scratch, hipStream_t stream);

// Operands of one grouped-GEMM launch (routed blocks followed by shared-expert
// row tiles). Widths are in elements.
struct GemmParams {
  // routed part
  const uint16_t* a_routed;     // gate_up: x [T, H]; down: h [rows, I] (sorted order)
                                // (96-row blocks: fp16, scaled by 2^-a_exp)
  const int32_t* a_exp;         // 96-row blocks: gate_up: kx [T]; down: kr [rows]
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
  int32_t* h_exp;               // 96-row blocks, gate_up: kh [max_blocks * bm, n_htiles]
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
  int32_t n_htiles;             // 96-row blocks: ceil(I / kHTile)
  uint32_t nibble_mask;         // 0x0F0F0F0F (a run-time value on purpose)
  int32_t prepacked;            // packed/scales in the prepacked layout (below)
  // Small-batch gate_up with at most kLocalPairs pairs (local_route != 0):
  // the work-groups bucket the pairs themselves
  // from topk_ids (in the bucketing kernel's order; the input sorted_ids,
  // block_expert and n_padded are not read), and one of them writes the
  // bucketing to the *_out arrays for the launches that follow.
  int32_t local_route;
  const int32_t* topk_ids;      // [T, k]
  int32_t n_experts;            // local experts
  int32_t expert_base;          // global id of local expert 0
  int32_t* sorted_out;          // [max_blocks * 4]
  int32_t* block_expert_out;    // [max_blocks]
  int32_t* n_padded_out;        // [1]
};

// (each routed work-group buckets all pairs before its first weight load:
// worth it only while that is a few lane steps)
constexpr int32_t kLocalPairs = 16;
constexpr int32_t kLocalTokens = 8;  // tokens of the launch instance that does it

// ---- prepacked weights ------------------------------------------------------
// The layout moe_w4a16_prepack writes, per expert and matrix (W13: Nw = 2I
// rows, K = H; W2: Nw = H, K = I). Rows are grouped in tiles of kPackRows (the
// prefill kernel's work-group rows; W13 rows in the order that kernel takes
// them: per 64-row wave slice, 16 gate rows, the next 16 gate rows, then the
// 32 matching up rows). Within a tile:
//   codes:  [K / 128 chunks][kPackRows rows][4 groups x 16 bytes]
//   scales: [ceil(K / 512) periods][kPackRows rows][16 groups x 2 bytes],
//           zero past the last group
// so that each 128-input chunk of a tile (32 KB of codes), and each 16-group
// period of its scales (16 KB), is contiguous. Requires Nw % kPackRows == 0
// and K % 128 == 0.
constexpr int kPackRows = 512;
constexpr int kPackChunk = 128;  // inputs per chunk

struct PackPos {
  int32_t tile, row;  // tile of the weight row and its row inside the tile
};
__host__ __device__ inline PackPos pack_pos(bool w13, int32_t I, int32_t n) {
  if (!w13) return PackPos{n / kPackRows, n % kPackRows};
  const int32_t up = n >= I ? 2 : 0;
  const int32_t c = up ? n - I : n;
  const int32_t cc = c % (kPackRows / 2);
  const int32_t w = cc / 32, s = (cc % 32) / 16 + up, r = cc % 16;
  return PackPos{c / (kPackRows / 2), 64 * w + 16 * s + r};
}
__host__ __device__ inline int32_t pack_chunks(int32_t K) { return K / kPackChunk; }
__host__ __device__ inline int32_t pack_periods(int32_t K) { return (K / 32 + 15) / 16; }
// bytes of one expert's codes / scales
__host__ __device__ inline int64_t pack_code_bytes(int32_t Nw, int32_t K) {
  return (int64_t)Nw * (K / 2);
}
__host__ __device__ inline int64_t pack_scale_bytes(int32_t Nw, int32_t K) {
  return (int64_t)Nw * pack_periods(K) * 32;
}
// byte offset (inside one expert) of group g (32 inputs) of weight row n
__host__ __device__ inline int64_t pack_code_offset(bool w13, int32_t I, int32_t K, int32_t n,
                                                    int32_t g) {
  const PackPos q = pack_pos(w13, I, n);
  return (((int64_t)q.tile * pack_chunks(K) + g / 4) * kPackRows + q.row) * 64 + 16 * (g % 4);
}
__host__ __device__ inline int64_t pack_scale_offset(bool w13, int32_t I, int32_t K, int32_t n,
                                                     int32_t g) {
  const PackPos q = pack_pos(w13, I, n);
  return (((int64_t)q.tile * pack_periods(K) + g / 16) * kPackRows + q.row) * 32 + 2 * (g % 16);
}
// One-time repack of an int4 matrix [E, Nw, K/8] and its bf16 scales
// [E, Nw, K/32] into the layout above.
hipError_t launch_prepack(const int32_t* packed, const uint16_t* scales, int32_t E, int32_t Nw,
                          int32_t K, bool w13, int32_t I, uint8_t* codes_out,
                          uint8_t* scales_out, hipStream_t stream);

// Small-batch variants (buckets padded to 4 rows; see gemm_small.hip).
// small_batch_fits: whether their staged scales fit in LDS for these widths.
bool small_batch_fits(int32_t hidden, int32_t inter);
hipError_t launch_gate_up_small(const GemmParams& p, hipStream_t stream);
hipError_t launch_down_small(const GemmParams& p, hipStream_t stream);

// Routed int4 experts in 96-row blocks, with the bf16 shared expert's tiles
// in the same launches (every batch past the small-batch regime; see
// gemm_prefill.hip). Any hidden and inter that are multiples of 128;
// prefill_fits: whether they are whole tiles (the prepacked layout needs it).
// The routed products run in fp16: launch_x16 first converts x [T, H] (bf16)
// into x16 (fp16, scaled per token by 2^-kx[t]); gate_up writes h in fp16
// with one exponent per (row, kHTile columns).
constexpr int32_t kHTile = 256;
bool prefill_fits(int32_t hidden, int32_t inter);
int32_t prefill_block_m();  // bucket rows per block of that path
hipError_t launch_x16(const uint16_t* x, uint16_t* x16, int32_t* kx, int64_t T, int32_t H,
                      hipStream_t stream);
// Between the launches: each bucketed row's h tiles rescaled to the row's
// largest exponent kr[row] (rows below *n_padded of `rows`).
hipError_t launch_h_rescale(uint16_t* h, const int32_t* kh, int32_t* kr, const int32_t* n_padded,
                            int64_t rows, int32_t I, int32_t n_htiles, hipStream_t stream);
hipError_t launch_gate_up_prefill(const GemmParams& p, hipStream_t stream);
hipError_t launch_down_prefill(const GemmParams& p, hipStream_t stream);

// Router step: for each of T tokens, the k largest of S fp32 scores (equal
// scores: lower expert first), descending, and weights = softmax over them.
constexpr int32_t kMaxScored = 1024;  // scores per token (experts of the model)
hipError_t launch_route(const float* scores, int64_t T, int32_t S, int32_t k, int32_t* topk_ids,
                        float* topk_weights, hipStream_t stream);
// out[t] = bf16(s[t] + sum_j valid * w[t,j] * y[t*k+j]), fp32 sum in slot order.
hipError_t launch_combine(const float* y, const float* s, const int32_t* topk_ids,
                          const float* topk_weights, uint16_t* out, int64_t T, int32_t H,
                          int32_t k, int32_t E, int32_t base, hipStream_t stream);

}  // namespace moe
