// gemm.hip -- grouped W4A16 GEMMs of the routed-expert MoE layer (gfx950),
// tiled path for many rows per expert (prefill, skewed and expert-parallel
// batches).
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
// 4 * 16 * NSUB weight rows; for gate_up half of every wave's NSUB 16-row
// sub-tiles are gate rows and half the matching up rows. K advances in chunks of
// 128 (four groups of 32):
//   * the BM x 128 activation chunk is gathered from HBM with 16-byte loads into
//     a double-buffered LDS tile (rows past the valid ones are not loaded);
//   * every wave streams its own NSUB weight sub-tiles with one 16-byte load
//     per lane and sub-tile: lane (r = lane%16, q = lane/16) holds the four
//     words of group q of weight row r, i.e. each weight row is read as 64
//     contiguous bytes per chunk;
//   * the words are dequantised in registers to bf16 (u - 8) * s and fed to
//     v_mfma_f32_16x16x32_bf16: MFMA step j takes word j of every lane, so its
//     32-long reduction spans one 8-input slice of each of the four groups --
//     the matching activations are read from LDS at the same offsets. Each
//     dequantised fragment serves all BM / 16 row sub-tiles, so the
//     dequantisation cost is shared by up to BM rows;
//   * the next chunk's global loads are issued before the current chunk's
//     MFMAs (register double buffering).
// Row sub-tiles of 16 that hold only bucket padding are skipped.
#include "internal.h"

namespace moe {
namespace {

// cache policy bits of the int4 weight loads
#ifndef MOE_TILED_AUX
#define MOE_TILED_AUX 0
#endif
constexpr int kTiledAux = MOE_TILED_AUX;

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

// The eight codes of one word -> eight bf16 weights (u - 8) * s in input order.
// Even fields are masked into the four bytes of one register and odd fields
// into another, so each code converts with one v_cvt_f32_ubyte{0..3};
// (u - 8) * s = fma(u, s, -8 s) is exact in fp32 (4-bit times 8-bit
// significands) and is rounded once to bf16. `mask` is 0x0F0F0F0F, passed at
// run time so that the compiler keeps the byte form.
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, uint32_t mask, float s, float neg8s) {
  const uint32_t ev = w & mask;
  const uint32_t od = (w >> 4) & mask;
  u32x4 r;
  r[0] = pack_bf16x2(fmaf((float)(ev & 0xFFu), s, neg8s), fmaf((float)(od & 0xFFu), s, neg8s));
  r[1] = pack_bf16x2(fmaf((float)((ev >> 8) & 0xFFu), s, neg8s),
                     fmaf((float)((od >> 8) & 0xFFu), s, neg8s));
  r[2] = pack_bf16x2(fmaf((float)((ev >> 16) & 0xFFu), s, neg8s),
                     fmaf((float)((od >> 16) & 0xFFu), s, neg8s));
  r[3] = pack_bf16x2(fmaf((float)(ev >> 24), s, neg8s), fmaf((float)(od >> 24), s, neg8s));
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  // silu(g) * u = g * u / (1 + exp(-g))
  return g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

template <int PHASE, int NSUB>
constexpr int tile_cols() {  // output columns of one work-group
  return PHASE == kGateUp ? 4 * 16 * NSUB / 2 : 4 * 16 * NSUB;
}

constexpr int kBufferFlags = 0x00020000;   // raw buffer resource, dword 3
constexpr uint32_t kNoRow = 0x80000000u;   // buffer offset past any tensor: loads 0

// A wave-uniform byte offset for the scalar offset field of a buffer load;
// readfirstlane makes it an SGPR value, so the compiler emits one load instead
// of a loop over distinct lane values.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// One work-group tile. INT4 selects the routed (int4 + scales) or the shared
// (bf16) weight format.
template <int BM, int PHASE, int NSUB, bool INT4>
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

  // ---- rows of this tile: bucket padding sits at the end of the block --------
  int e = 0;
  int n_valid;
  if (INT4) {
    e = p.block_expert[mblk];
    n_valid = 0;
#pragma unroll
    for (int h = 0; h < (BM + 63) / 64; ++h) {
      const int r = 64 * h + lane;
      const int valid = r < BM ? (p.sorted_ids[row0 + r] < p.P) : 0;
      n_valid += __popcll(__ballot(valid));
    }
  } else {
    n_valid = (p.T - row0 < BM) ? (int)(p.T - row0) : BM;
  }
  const int msub = (n_valid + 15) >> 4;

  // ---- activation rows this thread stages (byte offsets; kNoRow loads 0) ---
  const uint16_t* abase;
  int64_t arows;
  if (PHASE == kGateUp) {
    abase = INT4 ? p.a_routed : p.a_shared;
    arows = p.T;
  } else {
    abase = INT4 ? p.a_routed : p.a_shared;
    arows = INT4 ? (int64_t)p.max_blocks * BM : p.T;
  }
  const __amdgpu_buffer_rsrc_t ares =
      __builtin_amdgcn_make_buffer_rsrc((void*)abase, 0, (int)(arows * K * 2), kBufferFlags);
  const int acol = (tid & 15) * 8;  // bf16 offset inside the chunk
  uint32_t aoff[kLoadsA];
#pragma unroll
  for (int i = 0; i < kLoadsA; ++i) {
    const int r = (tid >> 4) + 16 * i;
    int64_t src = -1;
    if (r < msub * 16) {
      if (PHASE == kGateUp && INT4) {
        const int32_t pair = p.sorted_ids[row0 + r];
        if (pair < p.P) src = pair / p.k;
      } else if (INT4 || row0 + r < p.T) {
        src = row0 + r;
      }
    }
    aoff[i] = src < 0 ? kNoRow : (uint32_t)((src * K + acol) * 2);
  }

  // ---- weight rows of this lane ----------------------------------------
  int wrow[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    if (PHASE == kGateUp) {
      const int c = tile * tile_cols<PHASE, NSUB>() + wave * (8 * NSUB) + 16 * (s % (NSUB / 2)) + lr;
      wrow[s] = s < NSUB / 2 ? c : p.I + c;  // gate, then the matching up rows
    } else {
      wrow[s] = tile * tile_cols<PHASE, NSUB>() + wave * (16 * NSUB) + 16 * s + lr;
    }
  }
  const int Nw = (PHASE == kGateUp) ? 2 * p.I : p.N;
  __amdgpu_buffer_rsrc_t wres, sres;
  if (INT4) {
    const int64_t r0 = (int64_t)e * Nw;
    wres = __builtin_amdgcn_make_buffer_rsrc((void*)(p.packed + r0 * (K / 8)), 0,
                                             Nw * (K / 8) * 4, kBufferFlags);
    sres = __builtin_amdgcn_make_buffer_rsrc((void*)(p.scales + r0 * (K / 32)), 0,
                                             Nw * (K / 32) * 2, kBufferFlags);
  } else {
    wres = __builtin_amdgcn_make_buffer_rsrc((void*)p.wshared, 0, Nw * K * 2, kBufferFlags);
    sres = wres;
  }
  uint32_t woff[NSUB], soff[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    woff[s] = INT4 ? (uint32_t)((wrow[s] * (K / 8) + 4 * lq) * 4)
                   : (uint32_t)((wrow[s] * K + 32 * lq) * 2);
    soff[s] = (uint32_t)((wrow[s] * (K / 32) + lq) * 2);
  }

  // ---- register buffers --------------------------------------------------
  u32x4 a_reg[kLoadsA];
  u32x4 bq_reg[NSUB][INT4 ? 1 : 4];  // int4: four words (one group); bf16: 32 weights
  uint32_t sc_reg[NSUB];             // int4: scale bits

  // Chunk ch's loads. Past the last chunk the scalar offset lies beyond every
  // buffer (the loads return zeros without traffic), so that the prefetch is
  // issued unconditionally: a conditional one makes the compiler's wait
  // before each use also cover the loads just issued.
  auto cofs = [&](int ch, int bytes) { return uniform(ch < nchunks ? ch * bytes : (int)kNoRow); };
  auto load_chunk = [&](int ch) {
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i)
      a_reg[i] = __builtin_amdgcn_raw_buffer_load_b128(ares, aoff[i], cofs(ch, kBK * 2), 0);
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      if (INT4) {
        bq_reg[s][0] = __builtin_amdgcn_raw_buffer_load_b128(wres, woff[s], cofs(ch, 64), kTiledAux);
        sc_reg[s] = __builtin_amdgcn_raw_buffer_load_b16(sres, soff[s], cofs(ch, 8), 0);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bq_reg[s][j] = __builtin_amdgcn_raw_buffer_load_b128(wres, woff[s] + 16 * j, cofs(ch, kBK * 2), 0);
      }
    }
  };

  f32x4 acc[kMsub][NSUB];
#pragma unroll
  for (int mi = 0; mi < kMsub; ++mi)
#pragma unroll
    for (int s = 0; s < NSUB; ++s) acc[mi][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_chunk(0);
  for (int ch = 0; ch < nchunks; ++ch) {
    uint16_t* buf = As[ch & 1];
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i) {
      const int r = (tid >> 4) + 16 * i;
      if (r < msub * 16) *reinterpret_cast<u32x4*>(buf + r * kLdsRow + acol) = a_reg[i];
    }
    // this chunk's weights stay in registers while the next chunk loads
    u32x4 wq[NSUB][INT4 ? 1 : 4];
    float sc[NSUB], n8[NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
#pragma unroll
      for (int q = 0; q < (INT4 ? 1 : 4); ++q) wq[s][q] = bq_reg[s][q];
      sc[s] = bf16_to_f32(sc_reg[s]);
      n8[s] = -8.0f * sc[s];
    }
    __syncthreads();
    load_chunk(ch + 1);
    // keep the prefetch ahead of the MFMAs (the scheduler would sink it)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 bw[NSUB];
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
        bw[s] = INT4 ? dequant8(wq[s][0][j], p.nibble_mask, sc[s], n8[s])
                     : __builtin_bit_cast(bf16x8, wq[s][INT4 ? 0 : j]);
#pragma unroll
      for (int mi = 0; mi < kMsub; ++mi) {
        if (mi < msub) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              buf + (mi * 16 + lr) * kLdsRow + 32 * lq + 8 * j);
#pragma unroll
          for (int s = 0; s < NSUB; ++s)
            acc[mi][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bw[s], acc[mi][s], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue: lane holds rows 4*lq + i of each 16-row sub-tile, column lr
  if (PHASE == kGateUp) {
#pragma unroll
    for (int s = 0; s < NSUB / 2; ++s) {
      const int col = wrow[s];
#pragma unroll
      for (int mi = 0; mi < kMsub; ++mi) {
        if (mi >= msub) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t r = row0 + mi * 16 + 4 * lq + i;
          const float hv = silu_mul(acc[mi][s][i], acc[mi][s + NSUB / 2][i]);
          const uint16_t hb = (uint16_t)(pack_bf16x2(hv, 0.f) & 0xFFFFu);
          if (INT4) p.h_routed[r * p.I + col] = hb;
          else if (r < p.T) p.h_shared[r * p.I + col] = hb;
        }
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
          for (int s = 0; s < NSUB; ++s) dst[wrow[s]] = acc[mi][s][i];
        }
      }
    }
  }
}

// Work-groups: routed (max_blocks x tiles of NSUB sub-tiles per wave) first,
// then the shared expert's (row blocks of BM tokens x tiles of NSUBS), both
// block-major. (Remapping work-group ids so that each XCD runs a contiguous
// range of items was measured slower on MI355X than the default round-robin
// placement, for this kernel and for the small-batch one.)
template <int BM, int PHASE, int NSUB, int NSUBS>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kLdsRow];
  const int n_tiles = p.N / tile_cols<PHASE, NSUB>();
  const int routed = p.max_blocks * n_tiles;
  int bid = blockIdx.x;
  if (bid < routed) {
    const int mblk = bid / n_tiles;
    const int tile = bid - mblk * n_tiles;
    if ((int64_t)mblk * BM >= *p.n_padded) return;
    gemm_tile<BM, PHASE, NSUB, true>(p, mblk, tile, As);
  } else {
    bid -= routed;
    const int ns = p.N / tile_cols<PHASE, NSUBS>();
    const int mblk = bid / ns;
    const int tile = bid - mblk * ns;
    gemm_tile<BM, PHASE, NSUBS, false>(p, mblk, tile, As);
  }
}

template <int BM, int PHASE, int NSUB, int NSUBS>
hipError_t launch(const GemmParams& p, hipStream_t stream) {
  if (p.N % tile_cols<PHASE, NSUB>() != 0 || p.N % tile_cols<PHASE, NSUBS>() != 0)
    return hipErrorInvalidValue;
  const int64_t routed = (int64_t)p.max_blocks * (p.N / tile_cols<PHASE, NSUB>());
  const int64_t shared = p.wshared ? (p.T + BM - 1) / BM * (p.N / tile_cols<PHASE, NSUBS>()) : 0;
  const int64_t grid = routed + shared;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  GemmParams args = p;
  void* kargs[] = {&args};
  return hipLaunchKernel(
      reinterpret_cast<const void*>(&grouped_gemm_kernel<BM, PHASE, NSUB, NSUBS>),
      dim3((unsigned)grid), dim3(kThreads), kargs, 0, stream);
}

}  // namespace

// 16- and 64-row blocks (the sizes the layer call picks for this kernel), two
// column sub-tiles per wave.
hipError_t launch_gate_up(const GemmParams& p, int32_t block_m, hipStream_t stream) {
  if (block_m == 16) return launch<16, kGateUp, 2, 2>(p, stream);
  if (block_m == 64) return launch<64, kGateUp, 2, 2>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_down(const GemmParams& p, int32_t block_m, hipStream_t stream) {
  if (block_m == 16) return launch<16, kDown, 2, 2>(p, stream);
  if (block_m == 64) return launch<64, kDown, 2, 2>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace moe
