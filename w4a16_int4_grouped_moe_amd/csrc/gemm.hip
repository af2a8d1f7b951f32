// gemm.hip -- grouped W4A16 GEMMs of the routed-expert MoE layer (gfx950).
//
// Two launches per layer:
//   gate_up: h[row] = silu(x_row . W1_e) * (x_row . W3_e) for every bucketed row
//            (W13_e rows [0, I) are the gate W1, rows [I, 2I) the up W3), SwiGLU
//            fused into the epilogue, h stored as bf16 in bucket order;
//   down:    y[pair] = h[row] . W2_e, fp32, scattered to the row's (token, slot).
// Each launch also carries the bf16 shared expert's tiles (same MLP on every
// token, bf16 weights), after the routed tiles.
//
// The routed weights are INT4 codes, eight per 32-bit word along the input
// dimension (field i at bits 4i..4i+3, value field - 8), with one bf16 scale per
// 32 inputs of a row (Kimi-K2.6 catalog entry, QUANT and PARAMS paragraphs).
//
// Work-group tile (256 threads = 4 waves): BM bucketed rows of one expert x
// 64 h columns (gate_up; 64 gate + 64 up weight rows) or x 128 output columns
// (down). K advances in chunks of 128 (four groups of 32):
//   * the BM x 128 activation chunk is gathered from HBM with 16-byte loads into
//     a double-buffered LDS tile (rows beyond the valid ones are zero);
//   * every wave streams its own two 16-row weight slices with one 16-byte
//     load per lane per slice: lane (r = lane%16, q = lane/16) holds the four
//     words of group q of weight row r, i.e. each weight row is read as 64
//     contiguous bytes per chunk;
//   * the words are dequantised in registers to bf16 (u - 8) * s and fed to
//     v_mfma_f32_16x16x32_bf16: MFMA step j takes word j of every lane, so its
//     32-long reduction spans one 8-input slice of each of the four groups --
//     the matching activations are read from LDS at the same offsets;
//   * the next chunk's global loads are issued before the current chunk's
//     MFMAs (register double buffering).
// Row sub-tiles of 16 that hold only bucket padding are skipped.
#include "internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBK = 128;          // inputs per K chunk (four groups of 32)
constexpr int kLdsRow = kBK + 8;  // bf16 per LDS row; 16-byte pad spreads banks

enum { kGateUp = 0, kDown = 1 };

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) {
  return __builtin_bit_cast(float, bits << 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// the eight codes of one word -> eight bf16 weights (u - 8) * s in input order.
// (u - 8) * s is exact in fp32 (4-bit times 8-bit significands); one rounding
// to bf16 follows.
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float s, float neg8s) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = fmaf((float)((w >> (8 * i)) & 15u), s, neg8s);
    const float hi = fmaf((float)((w >> (8 * i + 4)) & 15u), s, neg8s);
    r[i] = pack_bf16x2(lo, hi);
  }
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  // silu(g) * u = g * u / (1 + exp(-g))
  return g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// One work-group tile. INT4 selects the routed (int4 + scales) or the shared
// (bf16) weight format.
template <int BM, int PHASE, bool INT4>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, int mblk, int tile,
                                          uint16_t (*As)[BM * kLdsRow]) {
  constexpr int kMsub = BM / 16;
  constexpr int kLoadsA = BM / 16;  // 16-byte A loads per thread per chunk
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 15;
  const int lq = lane >> 4;
  const int K = p.K;
  const int nchunks = K / kBK;
  const int64_t row0 = (int64_t)mblk * BM;

  // ---- rows of this tile ------------------------------------------------
  int e = 0;
  int n_valid;
  if (INT4) {
    e = p.block_expert[mblk];
    int valid_lane = 0;
    if (lane < BM) valid_lane = p.sorted_ids[row0 + lane] < p.P;
    n_valid = __popcll(__ballot(valid_lane));
  } else {
    n_valid = (p.T - row0 < BM) ? (int)(p.T - row0) : BM;
  }
  const int msub = (n_valid + 15) >> 4;

  // A source rows handled by this thread (nullptr = zero row)
  const uint16_t* arow[kLoadsA];
  const int acol = (tid & 15) * 8;  // bf16 offset inside the chunk
#pragma unroll
  for (int i = 0; i < kLoadsA; ++i) {
    const int r = (tid >> 4) + 16 * i;
    const uint16_t* src = nullptr;
    if (r < msub * 16) {
      if (PHASE == kGateUp) {
        if (INT4) {
          const int32_t pair = p.sorted_ids[row0 + r];
          if (pair < p.P) src = p.a_routed + (int64_t)(pair / p.k) * K;
        } else if (row0 + r < p.T) {
          src = p.a_shared + (row0 + r) * K;
        }
      } else {
        if (INT4) src = p.a_routed + (row0 + r) * K;
        else if (row0 + r < p.T) src = p.a_shared + (row0 + r) * K;
      }
    }
    arow[i] = src;
  }

  // ---- weight rows of this lane ----------------------------------------
  int wrow[2];
  if (PHASE == kGateUp) {
    const int c = tile * 64 + 16 * wave + lr;
    wrow[0] = c;        // gate
    wrow[1] = p.I + c;  // up
  } else {
    wrow[0] = tile * 128 + 32 * wave + lr;
    wrow[1] = wrow[0] + 16;
  }
  const int Nw = (PHASE == kGateUp) ? 2 * p.I : p.N;
  const int32_t* wq[2];
  const uint16_t* ws[2];
  const uint16_t* wb[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if (INT4) {
      const int64_t r = (int64_t)e * Nw + wrow[s];
      wq[s] = p.packed + r * (K / 8) + 4 * lq;
      ws[s] = p.scales + r * (K / 32) + lq;
    } else {
      wb[s] = p.wshared + (int64_t)wrow[s] * K + 32 * lq;
    }
  }

  // ---- register buffers --------------------------------------------------
  u32x4 a_reg[kLoadsA];
  u32x4 bq_reg[2];       // int4: four words (one group) per slice
  uint32_t sc_reg[2];    // int4: scale bits
  u32x4 bb_reg[2][4];    // bf16: 32 weights per slice

  auto load_chunk = [&](int ch) {
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i) {
      a_reg[i] = arow[i] ? *reinterpret_cast<const u32x4*>(arow[i] + ch * kBK + acol)
                         : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (INT4) {
        bq_reg[s] = *reinterpret_cast<const u32x4*>(wq[s] + ch * 16);
        sc_reg[s] = ws[s][ch * 4];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bb_reg[s][j] = *reinterpret_cast<const u32x4*>(wb[s] + ch * kBK + 8 * j);
      }
    }
  };

  f32x4 acc[kMsub][2];
#pragma unroll
  for (int mi = 0; mi < kMsub; ++mi)
#pragma unroll
    for (int s = 0; s < 2; ++s) acc[mi][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_chunk(0);
  for (int ch = 0; ch < nchunks; ++ch) {
    uint16_t* buf = As[ch & 1];
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i) {
      const int r = (tid >> 4) + 16 * i;
      *reinterpret_cast<u32x4*>(buf + r * kLdsRow + acol) = a_reg[i];
    }
    // weights of this chunk -> bf16 fragments
    bf16x8 bw[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (INT4) {
        const float sc = bf16_to_f32(sc_reg[s]);
        const float n8 = -8.0f * sc;
#pragma unroll
        for (int j = 0; j < 4; ++j) bw[s][j] = dequant8(bq_reg[s][j], sc, n8);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) bw[s][j] = __builtin_bit_cast(bf16x8, bb_reg[s][j]);
      }
    }
    __syncthreads();
    if (ch + 1 < nchunks) load_chunk(ch + 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int mi = 0; mi < kMsub; ++mi) {
        if (mi < msub) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              buf + (mi * 16 + lr) * kLdsRow + 32 * lq + 8 * j);
          acc[mi][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bw[0][j], acc[mi][0], 0, 0, 0);
          acc[mi][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bw[1][j], acc[mi][1], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue: lane holds rows 4*lq + i of each 16-row sub-tile, column lr
  if (PHASE == kGateUp) {
    const int col = tile * 64 + 16 * wave + lr;
#pragma unroll
    for (int mi = 0; mi < kMsub; ++mi) {
      if (mi >= msub) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = row0 + mi * 16 + 4 * lq + i;
        const float hv = silu_mul(acc[mi][0][i], acc[mi][1][i]);
        const uint16_t hb = (uint16_t)(pack_bf16x2(hv, 0.f) & 0xFFFFu);
        if (INT4) p.h_routed[r * p.I + col] = hb;
        else if (r < p.T) p.h_shared[r * p.I + col] = hb;
      }
    }
  } else {
#pragma unroll
    for (int mi = 0; mi < kMsub; ++mi) {
      if (mi >= msub) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = row0 + mi * 16 + 4 * lq + i;
        float* dst = nullptr;
        if (INT4) {
          const int32_t pair = p.sorted_ids[r];
          if (pair < p.P) dst = p.y_routed + (int64_t)pair * p.N;
        } else if (r < p.T) {
          dst = p.y_shared + r * p.N;
        }
        if (dst) {
#pragma unroll
          for (int s = 0; s < 2; ++s) dst[wrow[s]] = acc[mi][s][i];
        }
      }
    }
  }
}

template <int BM, int PHASE>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kLdsRow];
  constexpr int kCols = (PHASE == kGateUp) ? 64 : 128;
  const int n_tiles = p.N / kCols;
  const int routed = p.max_blocks * n_tiles;
  int bid = blockIdx.x;
  if (bid < routed) {
    const int mblk = bid / n_tiles;
    const int tile = bid - mblk * n_tiles;
    if ((int64_t)mblk * BM >= *p.n_padded) return;
    gemm_tile<BM, PHASE, true>(p, mblk, tile, As);
  } else {
    bid -= routed;
    const int mblk = bid / n_tiles;
    const int tile = bid - mblk * n_tiles;
    gemm_tile<BM, PHASE, false>(p, mblk, tile, As);
  }
}

template <int BM, int PHASE>
hipError_t launch(const GemmParams& p, hipStream_t stream) {
  constexpr int kCols = (PHASE == kGateUp) ? 64 : 128;
  const int n_tiles = p.N / kCols;
  const int64_t shared_blocks = p.wshared ? (p.T + BM - 1) / BM : 0;
  const int64_t grid = ((int64_t)p.max_blocks + shared_blocks) * n_tiles;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  GemmParams args = p;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&grouped_gemm_kernel<BM, PHASE>),
                         dim3((unsigned)grid), dim3(kThreads), kargs, 0, stream);
}

}  // namespace

hipError_t launch_gate_up(const GemmParams& p, int32_t block_m, hipStream_t stream) {
  if (block_m == 16) return launch<16, kGateUp>(p, stream);
  if (block_m == 64) return launch<64, kGateUp>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_down(const GemmParams& p, int32_t block_m, hipStream_t stream) {
  if (block_m == 16) return launch<16, kDown>(p, stream);
  if (block_m == 64) return launch<64, kDown>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace moe
