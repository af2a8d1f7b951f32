// gemm_small.hip -- grouped W4A16 GEMMs for small token counts (decode), gfx950.
//
// Same two launches as gemm.hip (gate_up with fused SwiGLU, then down), for
// buckets of at most four rows per expert block. In this regime the layer is
// bound by the HBM stream of int4 weights, so the kernel is built around that
// stream and around a cheap, exact dequantisation.
//
// Work decomposition. A work-group (4 waves) takes one 4-row block and four
// consecutive slices of weight rows; each wave owns one slice of NR row-sets of
// four rows (for gate_up half of them gate rows, half the matching up rows).
// K advances 16 groups of 32 (512 inputs) per iteration.
//
// Data movement per iteration:
//  * weights: each wave streams its own rows, one 16-byte buffer load per lane
//    and row-set: lane l = 4*kp + j reads group kp of row j of the row-set, so a
//    load reads 256 contiguous bytes of each of four rows;
//  * activations and scales are shared by the four waves: the work-group loads
//    them once, each thread one coalesced 16-byte piece of each, into LDS
//    (double buffered, one barrier per iteration). Activations are written in
//    MFMA fragment order, already permuted for the dequantised weights, so a
//    wave reads its operands with linear, conflict-free ds_read_b128.
//
// Arithmetic: v_mfma_f32_4x4x4_16b_bf16 with its 16 blocks laid along K (block
// kp = group kp of the iteration): A = the four token rows, B = four weight
// rows, so activations are not replicated across lanes; the 16 k-parts are
// summed across lanes once, after the K loop. Dequantisation has no multiply:
// a 4-bit field u OR-ed into the bf16 pattern 0x4300 is exactly the bf16 value
// 128 + u (one shift and one v_bitop3 per pair of fields i, i+4), activations
// are permuted to the same (0,4,1,5 | 2,6,3,7) order, and each group's MFMA
// chain starts from C0 = -136 * sum(x over the group) -- an MFMA chain of the
// same activations against the constant bf16 -136 -- so it yields exactly
// sum x * (u - 8); the group's bf16 scale then multiplies it in fp32 (the
// weight is never rounded). The bf16 shared expert uses the same structure
// with its weights taken as they are (natural order, no scales).
#include <algorithm>

#include "internal.h"

namespace moe {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#ifndef MOE_SMALL_NR
#define MOE_SMALL_NR 4  // int4 row-sets per wave
#endif

constexpr int kThreads = 256;  // four waves
constexpr int kWaves = kThreads / 64;
#ifndef MOE_SMALL_NR_DOWN
#define MOE_SMALL_NR_DOWN MOE_SMALL_NR
#endif
#ifndef MOE_SMALL_TOKBLOCKS
#define MOE_SMALL_TOKBLOCKS 2  // 4-token blocks per shared-expert work-group
#endif

constexpr int kNR = MOE_SMALL_NR;            // gate_up
constexpr int kNRDown = MOE_SMALL_NR_DOWN;   // down
#ifndef MOE_SMALL_NRS
#define MOE_SMALL_NRS 2
#endif
constexpr int kNRS = MOE_SMALL_NRS;  // bf16 shared-expert row-sets per wave
constexpr int kTokBlocks = MOE_SMALL_TOKBLOCKS;
#ifndef MOE_SMALL_TOKBLOCKS_LARGE
#define MOE_SMALL_TOKBLOCKS_LARGE 4
#endif
constexpr int kTokBlocksLarge = MOE_SMALL_TOKBLOCKS_LARGE;  // for batches beyond 4 kTokBlocks

// occupancy target (waves per SIMD) of a launch whose int4 waves hold NR row-sets
#ifndef MOE_SMALL_WAVES
#define MOE_SMALL_WAVES 4
#endif
constexpr int waves_per_simd(int nr) { return nr >= 8 ? 2 : MOE_SMALL_WAVES; }
#ifndef MOE_SMALL_DEPTH
#define MOE_SMALL_DEPTH 1
#endif
constexpr int kSmallDepth = MOE_SMALL_DEPTH;  // int4 weight iterations in flight
constexpr int kGroupsPerIt = 16;  // k-parts = MFMA blocks
constexpr uint32_t kMagic = 0x43004300u;   // bf16 128.0 in both halves
constexpr uint32_t kNeg136 = 0xC308C308u;  // bf16 -136.0 in both halves
constexpr int kBufferFlags = 0x00020000;   // raw buffer resource, dword 3
constexpr int kXBytes = 4 * 64 * 16;       // activation fragments per iteration
constexpr int kOutOfRange = (int)0x80000000u;  // buffer offset past any resource: reads 0
constexpr int kScaleBatch = 8;             // scale pieces in flight per thread while staging
// cache policy bits of the buffer loads: int4 weights, their scales and the
// bf16 shared weights
#ifndef MOE_STREAM_AUX
#define MOE_STREAM_AUX 2  // nt: the weight stream bypasses cache retention
#endif
#ifndef MOE_SCALE_AUX
#define MOE_SCALE_AUX 0
#endif
#ifndef MOE_SHARED_AUX
#define MOE_SHARED_AUX 0
#endif
constexpr int kStreamAux = MOE_STREAM_AUX;
constexpr int kScaleAux = MOE_SCALE_AUX;
constexpr int kSharedAux = MOE_SHARED_AUX;

// A wave-uniform byte offset for the scalar offset field of a buffer load;
// readfirstlane makes it an SGPR value, so the compiler emits one load instead
// of a loop over distinct lane values.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

enum { kGateUp = 0, kDown = 1 };

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) {
  return __builtin_bit_cast(float, bits << 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ f32x4 mfma4(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4, a),
                                                __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// (a & m) | c in one v_bitop3_b32 (truth table 0xEA over (a, m, c)). The
// intrinsic keeps the 32-bit form; written as plain and/or, the compiler splits
// it into 16-bit halves to match the MFMA operand type.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, m, c, 0xEA);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Pairwise exchanges of lanes l and l ^ m: both lanes add the same two
// rounded terms, so every lane of a class ends with bit-identical sums, and a
// result's rounding does not depend on which lane (i.e. which bucket row) it
// is read from. A rotation would add the terms in lane-dependent orders, and
// an add contracted with the multiply before it (an FMA) would round one
// lane's own term but not its partner's; hence no contraction here.
__device__ __forceinline__ float add_xor4(float v) {  // ds_swizzle, xor mask 4
#pragma clang fp contract(off)
  return v + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                   0x101F));
}
__device__ __forceinline__ float add_xor8(float v) {  // DPP row_ror:8 = xor 8 in a row
#pragma clang fp contract(off)
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ float add_xor(float v, int m) {  // m = 16 or 32
#pragma clang fp contract(off)
  return v + __shfl_xor(v, m);
}

// sum over the 16 k-parts: lanes with equal lane % 4
__device__ __forceinline__ float kpart_sum(float v) {
  v = add_xor8(add_xor4(v));
  return add_xor(add_xor(v, 16), 32);
}

// Output columns per wave slice: gate_up slices cover 2*NR h columns (NR/2
// gate + NR/2 up row-sets), down slices cover 4*NR output columns.
template <int PHASE, int NR>
constexpr int slice_cols() {
  static_assert(PHASE != kGateUp || NR % 2 == 0,
                "a gate_up slice pairs NR / 2 gate row-sets with NR / 2 up row-sets");
  return PHASE == kGateUp ? 2 * NR : 4 * NR;
}

// weight row of row-set rs, row j, of wave slice `slice`
template <int PHASE, int NR>
__device__ __forceinline__ int weight_row(const GemmParams& p, int slice, int rs, int j) {
  if (PHASE == kGateUp) {
    const int c0 = slice * (2 * NR);
    return (rs < NR / 2) ? c0 + 4 * rs + j : p.I + c0 + 4 * (rs - NR / 2) + j;
  }
  return slice * (4 * NR) + 4 * rs + j;
}

// LDS of one pipeline stage: the activation fragments of NB 4-token blocks.
template <int NB>
constexpr int stage_bytes() { return NB * kXBytes; }

// LDS bytes per weight row of the int4 scales, staged once for the whole K:
// an odd number of 32-byte units (one unit = the 16 groups of one iteration),
// so that the four rows j = lane % 4 read by a wave fall in distinct banks.
__host__ __device__ inline int scale_row_bytes(int K) {
  const int niters = (K / 32 + kGroupsPerIt - 1) / kGroupsPerIt;
  return 32 * (niters | 1);
}

// One iteration of an int4 work item: 16 groups of K against NR row-sets of
// four weight rows (w: this lane's code words, group kp of row j of each
// row-set), activations from the LDS stage of the iteration, each group's
// scale from sread (row-set rs at + 4 rs srow, iteration it at + 32 it).
template <int NR>
__device__ __forceinline__ void int4_step(const u32x4 (&w)[NR], const uint8_t* stage,
                                          const uint8_t* sread, int srow, int it,
                                          f32x4 (&acc)[NR]) {
  const int lane = threadIdx.x & 63;
  u32x4 xf[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) xf[q] = *reinterpret_cast<const u32x4*>(stage + q * 1024 + lane * 16);
  // C0 = -136 * (sum of the group's activations), per token row
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f};
  const u32x2 neg136 = {kNeg136, kNeg136};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    c0 = mfma4(u32x2{xf[q][0], xf[q][1]}, neg136, c0);
    c0 = mfma4(u32x2{xf[q][2], xf[q][3]}, neg136, c0);
  }
  // NR independent chains, interleaved so that consecutive MFMAs never
  // depend on each other
  f32x4 t[NR];
#pragma unroll
  for (int rs = 0; rs < NR; ++rs) t[rs] = c0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    u32x2 b0[NR], b1[NR];
#pragma unroll
    for (int rs = 0; rs < NR; ++rs) {
      const uint32_t v = w[rs][q];
      b0[rs] = u32x2{and_or(v, 0x000F000Fu, kMagic), and_or(v >> 4, 0x000F000Fu, kMagic)};
      b1[rs] = u32x2{and_or(v >> 8, 0x000F000Fu, kMagic), and_or(v >> 12, 0x000F000Fu, kMagic)};
    }
#pragma unroll
    for (int rs = 0; rs < NR; ++rs) t[rs] = mfma4(u32x2{xf[q][0], xf[q][1]}, b0[rs], t[rs]);
#pragma unroll
    for (int rs = 0; rs < NR; ++rs) t[rs] = mfma4(u32x2{xf[q][2], xf[q][3]}, b1[rs], t[rs]);
  }
#pragma unroll
  for (int rs = 0; rs < NR; ++rs) {
    const uint32_t sb = *reinterpret_cast<const uint16_t*>(sread + rs * 4 * srow + it * 32);
    acc[rs] += bf16_to_f32(sb) * t[rs];
  }
}

// NB blocks of four rows starting at row0 (NB > 1 only for the bf16 shared
// expert: its weights are then read once for 4 NB tokens).
template <int PHASE, int NR, bool INT4, int NB, int DEPTH, bool PK = false>
__device__ __forceinline__ void small_tile(const GemmParams& p, int64_t row0, int slice0,
                                           uint8_t* lds) {
  static_assert(INT4 ? NB == 1 : NB >= 1, "int4 work items hold one block");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kp = lane >> 2;  // k-part: group offset inside an iteration
  const int j = lane & 3;    // token row (A) and weight row in a row-set (B)
  const int slice = slice0 + wave;
  const int K = p.K;
  const int ngroups = K / 32;
  const int niters = (ngroups + kGroupsPerIt - 1) / kGroupsPerIt;
  const int tail = ngroups % kGroupsPerIt;  // groups of the last iteration if partial
  constexpr int kRowsWG = kWaves * 4 * NR;  // weight rows of the work-group

  // ---- activation staging: thread t -> token row t/64, 16-byte piece t%64 ---
  // piece c of the row's 1 KB chunk = group c/4, quarter c%4 -> fragment slot
  // [c%4][lane 4 (c/4) + token]. Rows without data (bucket padding, rows past
  // the last token of the shared expert) read a real row instead: their
  // results are never stored and MFMA rows depend only on their own input row.
  const int xt = tid >> 6;
  const int xc = tid & 63;
  const uint16_t* abase;
  int64_t arows;
  int xoff[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    int64_t arow;
    if (INT4) {
      if (PHASE == kGateUp) {
        const int32_t pair = p.sorted_ids[row0 + xt];
        arow = pair < p.P ? pair / p.k : 0;
        abase = p.a_routed;
        arows = p.T;
      } else {
        arow = row0 + xt;
        abase = p.a_routed;
        arows = (int64_t)p.max_blocks * 4;
      }
    } else {
      const int64_t r = row0 + 4 * b + xt;
      arow = r < p.T ? r : p.T - 1;
      abase = p.a_shared;
      arows = p.T;
    }
    xoff[b] = (int)(arow * K) * 2 + xc * 16;
  }
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)abase, 0, (int)(arows * K * 2), kBufferFlags);
  const int xdst = (xc & 3) * 1024 + ((xc >> 2) * 4 + xt) * 16;
  const bool xzero_tail = (xc >> 2) >= tail;  // only used in a partial iteration

  // ---- scales (int4): all groups of the work-group's rows, staged once ------
  // Row r of the work-group (wave r / 4NR, row-set and row r % 4NR) is read as
  // 2 niters pieces of 16 bytes (8 groups each), contiguous in memory, and kept
  // in LDS for the whole K loop; groups past the end of K are zero.
  const int Nw = (PHASE == kGateUp) ? 2 * p.I : p.N;
  const int srow = scale_row_bytes(K);
  uint8_t* const slds = lds + 2 * stage_bytes<NB>();
  const int e = INT4 ? p.block_expert[row0 / 4] : 0;
  // prepacked weights (see internal.h): tiles of kPackRows rows, each 128-input
  // chunk of a tile and each 16-group scale period of it one contiguous run
  constexpr bool packed_layout = INT4 && PK;
  auto stage_scales = [&]() {
    const int64_t r0 = (int64_t)e * Nw;
    const __amdgpu_buffer_rsrc_t sres =
        packed_layout
            ? __builtin_amdgcn_make_buffer_rsrc(
                  (void*)(reinterpret_cast<const uint8_t*>(p.scales) +
                          e * pack_scale_bytes(Nw, K)),
                  0, (int)pack_scale_bytes(Nw, K), kBufferFlags)
            : __builtin_amdgcn_make_buffer_rsrc((void*)(p.scales + r0 * (K / 32)), 0,
                                                Nw * (K / 32) * 2, kBufferFlags);
    const int ppr = 2 * niters;  // pieces per row
    const int npieces = kRowsWG * ppr;
    auto batch = [&](int base) {
      u32x4 v[kScaleBatch];
#pragma unroll
      for (int u = 0; u < kScaleBatch; ++u) {
        // loads of a work-group-uniform range only; a thread without a piece
        // inside it reads out of range
        if (base + u * kThreads >= npieces) break;
        const int i = base + u * kThreads + tid;
        const int r = i / ppr, pc = i - r * ppr;
        int off = kOutOfRange;
        if (i < npieces && pc * 8 < ngroups) {
          const int w = r / (4 * NR), lr = r % (4 * NR);
          const int n = weight_row<PHASE, NR>(p, slice0 + w, lr / 4, lr % 4);
          off = packed_layout ? (int)pack_scale_offset(PHASE == kGateUp, p.I, K, n, pc * 8)
                              : (n * (K / 32) + pc * 8) * 2;
        }
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(sres, off, 0, kScaleAux);
      }
#pragma unroll
      for (int u = 0; u < kScaleBatch; ++u) {
        if (base + u * kThreads >= npieces) break;
        const int i = base + u * kThreads + tid;
        if (i < npieces) {
          const int r = i / ppr, pc = i - r * ppr;
          const int valid = ngroups - pc * 8;  // groups of the piece inside K
          u32x4 sv = v[u];
          if (valid < 8) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              const uint32_t lo = 2 * h < valid ? (sv[h] & 0xFFFFu) : 0u;
              const uint32_t hi = 2 * h + 1 < valid ? (sv[h] & 0xFFFF0000u) : 0u;
              sv[h] = lo | hi;
            }
          }
          *reinterpret_cast<u32x4*>(slds + r * srow + pc * 16) = sv;
        }
      }
    };
    // the first batch (every K up to 8192 for 64 rows) as straight-line code:
    // a loop around it would make the compiler wait at its head for all loads
    // in flight, including the first iteration's operands
    batch(0);
    for (int base = kScaleBatch * kThreads; base < npieces; base += kScaleBatch * kThreads)
      batch(base);
  };

  // ---- weights of this lane ----------------------------------------------
  __amdgpu_buffer_rsrc_t wres;
  if (INT4) {
    const int64_t r0 = (int64_t)e * Nw;
    wres = __builtin_amdgcn_make_buffer_rsrc((void*)(p.packed + r0 * (K / 8)), 0,
                                             Nw * (K / 8) * 4, kBufferFlags);
  } else {
    wres = __builtin_amdgcn_make_buffer_rsrc((void*)p.wshared, 0, Nw * K * 2, kBufferFlags);
  }
  // lane (kp, j): group kp of iteration it of row j of each row-set; the
  // iteration adds wstep bytes (checkpoint layout: 16 groups of the row;
  // prepacked: four chunks of the tile)
  int woff[NR];
#pragma unroll
  for (int rs = 0; rs < NR; ++rs) {
    const int row = weight_row<PHASE, NR>(p, slice, rs, j);
    woff[rs] = !INT4          ? (row * K + 32 * kp) * 2
               : packed_layout ? (int)pack_code_offset(PHASE == kGateUp, p.I, K, row, kp)
                               : (row * (K / 8) + 4 * kp) * 4;
  }
  const int wstep = packed_layout ? (kGroupsPerIt / 4) * kPackRows * 64 : kGroupsPerIt * 16;
  // this lane's scales: row (wave, 4 rs + j), group kp of the iteration
  const uint8_t* const sread = slds + (wave * 4 * NR + j) * srow + kp * 2;

  // scalar byte offset of iteration `it` for a stride of `bytes` per iteration;
  // past the last iteration an offset beyond any buffer, so that the prefetch
  // can be issued unconditionally (a conditional one makes the compiler's wait
  // before each use also cover the prefetch) and reads zeros without traffic
  auto kofs = [&](int it, int bytes) { return uniform(it < niters ? it * bytes : kOutOfRange); };

  struct Frag {
    u32x4 w[NR][INT4 ? 1 : 4];  // int4: 4 words; bf16: 32 weights
  };
  auto load_w = [&](Frag& f, int it) {
#pragma unroll
    for (int rs = 0; rs < NR; ++rs) {
      if (INT4) {
        f.w[rs][0] = __builtin_amdgcn_raw_buffer_load_b128(wres, woff[rs], kofs(it, wstep),
                                                           kStreamAux);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          f.w[rs][q] = __builtin_amdgcn_raw_buffer_load_b128(wres, woff[rs] + 16 * q,
                                                             kofs(it, kGroupsPerIt * 64), kSharedAux);
      }
    }
    // Groups past the end of K (a partial last iteration) need no masking:
    // their staged activations are zero, so int4 codes (always finite once
    // dequantised) contribute exactly zero, and so do the bf16 weights that
    // follow in memory (a non-finite one there already makes its own row, and
    // with it the layer output, non-finite).
  };

  // shared stage registers: one activation piece per token block
  u32x4 xs_reg[NB];
  auto load_shared = [&](int it) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
      xs_reg[b] = __builtin_amdgcn_raw_buffer_load_b128(xres, xoff[b], kofs(it, kGroupsPerIt * 64), 0);
  };
  auto store_shared = [&](uint8_t* stage, int it) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      u32x4 v = xs_reg[b];
      if (tail && it == niters - 1 && xzero_tail) v = u32x4{0, 0, 0, 0};
      if (INT4) {  // (x0..x7) -> (x0,x4,x1,x5 | x2,x6,x3,x7)
        v = u32x4{__builtin_amdgcn_perm(v[2], v[0], 0x05040100u),
                  __builtin_amdgcn_perm(v[2], v[0], 0x07060302u),
                  __builtin_amdgcn_perm(v[3], v[1], 0x05040100u),
                  __builtin_amdgcn_perm(v[3], v[1], 0x07060302u)};
      }
      *reinterpret_cast<u32x4*>(stage + b * kXBytes + xdst) = v;
    }
  };

  f32x4 acc[NB][NR];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int rs = 0; rs < NR; ++rs) acc[b][rs] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Frag& f, const uint8_t* stage, int it) {
    if (INT4) {
      u32x4 w[NR];
#pragma unroll
      for (int rs = 0; rs < NR; ++rs) w[rs] = f.w[rs][0];
      int4_step<NR>(w, stage, sread, srow, it, acc[0]);
    } else {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        u32x4 xf[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          xf[q] = *reinterpret_cast<const u32x4*>(stage + b * kXBytes + q * 1024 + lane * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int rs = 0; rs < NR; ++rs)
            acc[b][rs] = mfma4(u32x2{xf[q][0], xf[q][1]}, u32x2{f.w[rs][q][0], f.w[rs][q][1]},
                               acc[b][rs]);
#pragma unroll
          for (int rs = 0; rs < NR; ++rs)
            acc[b][rs] = mfma4(u32x2{xf[q][2], xf[q][3]}, u32x2{f.w[rs][q][2], f.w[rs][q][3]},
                               acc[b][rs]);
        }
      }
    }
  };

  // ---- pipeline: the weights of DEPTH iterations and the activations of the
  // next one are in flight while an iteration is computed (a ring of DEPTH + 1
  // weight stages, two activation stages in LDS) --------------------------------
  uint8_t* const st[2] = {lds, lds + stage_bytes<NB>()};
  Frag f[DEPTH + 1];
  load_shared(0);
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    load_w(f[d], d);
    __builtin_amdgcn_sched_barrier(0);  // keep the iterations' loads in issue order
  }
  // the scales are fetched together with the first iterations' operands
  if (INT4) stage_scales();
  store_shared(st[0], 0);
  __syncthreads();
  // (the scheduling barriers keep the prefetch ahead of the computation: left
  // free, the scheduler sinks the loads below it to save registers)
  constexpr int kPeriod = (DEPTH + 1) % 2 ? 2 * (DEPTH + 1) : DEPTH + 1;
  for (int it0 = 0; it0 < niters; it0 += kPeriod) {
#pragma unroll
    for (int u = 0; u < kPeriod; ++u) {
      const int it = it0 + u;
      load_shared(it + 1);
      load_w(f[(u + DEPTH) % (DEPTH + 1)], it + DEPTH);
      __builtin_amdgcn_sched_barrier(0);
      compute(f[u % (DEPTH + 1)], st[u % 2], it);
      if (it + 1 >= niters) break;
      store_shared(st[(u + 1) % 2], it + 1);
      __syncthreads();
    }
  }

  // ---- per block: sum the k-parts (every lane then holds all NR x 4 results
  // of its row j) and store ----------------------------------------------------
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int64_t rb = row0 + 4 * b;
#pragma unroll
    for (int rs = 0; rs < NR; ++rs)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[b][rs][r] = kpart_sum(acc[b][rs][r]);

    // lane (kp, j) writes token row r = kp % 4 of row-sets kp / 4 + 4 t
    const int r = kp & 3;
    auto pick = [&](int rs) -> float {
      float v = acc[b][rs][0];
      v = (r == 1) ? acc[b][rs][1] : v;
      v = (r == 2) ? acc[b][rs][2] : v;
      v = (r == 3) ? acc[b][rs][3] : v;
      return v;
    };
    if (PHASE == kGateUp) {
#pragma unroll
      for (int t = 0; t < (NR / 2 + 3) / 4; ++t) {
        const int rsg = (kp >> 2) + 4 * t;
        if (rsg >= NR / 2) continue;
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int rs = 0; rs < NR / 2; ++rs) {
          if (rs == rsg) {
            g = pick(rs);
            u = pick(rs + NR / 2);
          }
        }
        const int col = slice * (2 * NR) + 4 * rsg + j;
        const uint16_t hb = (uint16_t)(pack_bf16x2(silu_mul(g, u), 0.f) & 0xFFFFu);
        if (INT4) {
          p.h_routed[(rb + r) * p.I + col] = hb;
        } else if (rb + r < p.T) {
          p.h_shared[(rb + r) * p.I + col] = hb;
        }
      }
    } else {
      float* dst = nullptr;
      if (INT4) {
        const int32_t pair = p.sorted_ids[rb + r];
        if (pair < p.P) dst = p.y_routed + (int64_t)pair * p.N;
      } else if (rb + r < p.T) {
        dst = p.y_shared + (rb + r) * p.N;
      }
#pragma unroll
      for (int t = 0; t < (NR + 3) / 4; ++t) {
        const int rsd = (kp >> 2) + 4 * t;
        if (rsd >= NR) continue;
        float v = 0.f;
#pragma unroll
        for (int rs = 0; rs < NR; ++rs)
          if (rs == rsd) v = pick(rs);
        if (dst) dst[slice * (4 * NR) + 4 * rsd + j] = v;
      }
    }
  }
}

// ---- local bucketing (decode path with at most kLocalPairs pairs) -----------
// One wave buckets the pairs q < P (lane q holds pair q) in the align kernel's
// order: local experts ascending, each bucket's pairs in ascending pair order,
// padded with the sentinel P to a multiple of 4 rows. Every bucket holds a
// pair, so there are at most P blocks and 4 P rows. sids (kLocalRows entries)
// and bexp (kLocalPairs entries) are the caller's LDS arrays; returns the
// block count (the same value in every lane).
constexpr int kLocalRows = 4 * kLocalPairs;
__device__ __forceinline__ int local_buckets(const int32_t* __restrict__ ids, int P, int E,
                                             int base, int32_t* sids, int32_t* bexp) {
  const int lane = threadIdx.x & 63;
  int e = -1;
  if (lane < P) {
    const int v = ids[lane] - base;
    e = (unsigned)v < (unsigned)E ? v : -1;
  }
  for (int r = lane; r < kLocalRows; r += 64) sids[r] = P;
  // the pairs of this lane's expert: how many, and how many come before it
  int cnt = 0, rank = 0;
  for (int q = 0; q < P; ++q) {
    const int eq = __builtin_amdgcn_readlane(e, q);
    if (e >= 0 && eq == e) {
      ++cnt;
      rank += q < lane ? 1 : 0;
    }
  }
  const int padded = (cnt + 3) & ~3;
  const int lead = (e >= 0 && rank == 0) ? 1 : 0;  // first pair of its expert
  // bucket start: the padded sizes of the smaller experts
  int off = 0, total = 0;
  for (int q = 0; q < P; ++q) {
    if (__builtin_amdgcn_readlane(lead, q)) {
      const int eq = __builtin_amdgcn_readlane(e, q);
      const int pq = __builtin_amdgcn_readlane(padded, q);
      off += eq < e ? pq : 0;
      total += pq;
    }
  }
  // (a wave's LDS stores land in issue order: the positions overwrite the
  // sentinels)
  if (e >= 0) sids[off + rank] = lane;
  if (lead)
    for (int b = 0; b < padded / 4; ++b) bexp[off / 4 + b] = e;
  return __builtin_amdgcn_readfirstlane(total) >> 2;
}

// One work-group = one block of rows x 4 consecutive wave slices, numbered
// block-major (consecutive work-groups stream consecutive rows of one expert;
// the default round-robin placement then spreads them over the XCDs). The
// shared expert's work-groups (TB 4-token blocks each: every such group of
// tokens reads the shared weights once) come first: each streams twice the
// bytes of a routed one (bf16 weights), so starting them first keeps them out
// of the kernel's tail. Routed work-groups (one 4-row bucket block each)
// follow. In small grids the shared work-groups are moved (place_shared).
// PK: the routed weights are in the prepacked layout (a separate instance, so
// that traces tell the two apart)
// Where the shared expert's work-groups sit in the grid. Work-groups go to the
// 8 XCDs in id order, round-robin, and within an XCD to its 32 CUs in turn, so
// id i lands on CU slot (i / 8) % 32 of XCD i % 8, and each run of 256 ids puts
// one work-group on every CU. A small grid (at most three work-groups per CU,
// all resident at once) gives the CU slots below (G % 256) / 8 one work-group
// more than the others; the shared expert's work-groups, which stream about
// twice the bytes of a routed one, are then placed at ids [G % 256, G % 256 +
// shared) of the first run, which reach the other CU slots. A CU streams at a
// bounded rate, so the launch lasts as long as its most loaded CU: for one
// token (128 shared and 512 routed work-groups) the most loaded CUs carry 717
// or 774 KB instead of 975 KB. Larger grids keep the shared work-groups first,
// out of the kernel's tail (and grids below one work-group per CU need no
// placement). The result is a permutation of work-group ids.
constexpr int64_t kChipCUs = 256;
__device__ __forceinline__ int64_t place_shared(int64_t bid, int64_t shared) {
  const int64_t grid = gridDim.x;
  const int64_t s0 = grid % kChipCUs;
  if (grid < kChipCUs || grid > 3 * kChipCUs || s0 + shared > kChipCUs) return bid;
  if (bid < s0) return bid + shared;      // routed work-groups before them
  if (bid < s0 + shared) return bid - s0;  // the shared expert's
  return bid;                              // routed work-groups after them
}

template <int PHASE, int NR, int NRS, int TB, bool PK>
__global__ __launch_bounds__(kThreads, waves_per_simd(NR)) void small_gemm_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // small_lds_bytes
  const int ns = p.N / slice_cols<PHASE, NRS>() / kWaves;
  const int64_t shared = p.wshared ? (p.T + 4 * TB - 1) / (4 * TB) * ns : 0;
  const int64_t bid = place_shared(blockIdx.x, shared);
  if (bid < shared) {
    const int64_t tg = bid / ns;
    const int s = (int)(bid - tg * ns);
    small_tile<PHASE, NRS, false, TB, 1>(p, tg * 4 * TB, s * kWaves, lds);
  } else {
    const int wg_slices = p.N / slice_cols<PHASE, NR>() / kWaves;
    const int64_t b2 = bid - shared;
    const int64_t blk = b2 / wg_slices;
    const int s = (int)(b2 - blk * wg_slices);
    // (local routing runs with at most kLocalTokens tokens, i.e. in the
    // kTokBlocks instance)
    static_assert(kLocalTokens <= 4 * kTokBlocks, "local routing instance");
    if constexpr (PHASE == kGateUp && TB == kTokBlocks) {
      if (p.local_route) {  // the work-group buckets the pairs itself
        __shared__ int32_t lsids[kLocalRows];
        __shared__ int32_t lbexp[kLocalPairs];
        __shared__ int32_t lnb;
        if (blk >= kLocalPairs) return;
        const bool writer = blk == 0 && s == 0;
        if (threadIdx.x < 64) {
          const int nb = local_buckets(p.topk_ids, (int)p.P, p.n_experts, p.expert_base, lsids,
                                       lbexp);
          if (threadIdx.x == 0) lnb = nb;
        }
        __syncthreads();
        const int nb = lnb;
        if (writer) {  // the table for the down and combine launches
          for (int i = threadIdx.x; i < 4 * nb; i += kThreads) p.sorted_out[i] = lsids[i];
          for (int i = threadIdx.x; i < nb; i += kThreads) p.block_expert_out[i] = lbexp[i];
          if (threadIdx.x == 0) *p.n_padded_out = 4 * nb;
        }
        if (blk >= nb) return;
        GemmParams q = p;
        q.sorted_ids = lsids;
        q.block_expert = lbexp;
        small_tile<PHASE, NR, true, 1, kSmallDepth, PK>(q, blk * 4, s * kWaves, lds);
        return;
      }
    }
    if (blk * 4 >= *p.n_padded) return;
    small_tile<PHASE, NR, true, 1, kSmallDepth, PK>(p, blk * 4, s * kWaves, lds);
  }
}

// ---------------------------------------------------------------------------
// Streamed down projection (int4 part) for 512 < K <= 2048, e.g. I = 2048.
// With K that short, a work item of small_tile runs only K / 512 iterations
// between its prologue (staging, first loads) and its epilogue, and the
// stream drains at every item. Here a work-group takes nsg consecutive slice
// groups (4 NR x 4 weight rows each) of one 4-row bucket block instead: the
// block's activations for all of K are staged in LDS once, the scales per
// slice group (double buffered, one barrier per slice group), and the weight
// prefetch runs on across slice groups, so that the stream does not stop
// until the work-group's last rows. Arithmetic and numerics are small_tile's.
// ---------------------------------------------------------------------------
constexpr int kStreamMaxIters = 4;  // K <= 2048: every activation stage in LDS at once
#ifndef MOE_STREAM_SG
#define MOE_STREAM_SG 4
#endif
constexpr int kStreamSG = MOE_STREAM_SG;  // most slice groups per work-group

template <int NR>
constexpr int stream_rows() { return kWaves * 4 * NR; }  // weight rows of a slice group

template <int NR>
int stream_lds_bytes(int K) {
  const int niters = (K / 32 + kGroupsPerIt - 1) / kGroupsPerIt;
  return niters * kXBytes + 2 * stream_rows<NR>() * scale_row_bytes(K);
}

template <int NR, int DEPTH, bool PK>
__device__ __forceinline__ void down_stream_tile(const GemmParams& p, int64_t row0, int sg0,
                                                 int nsg, uint8_t* lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kp = lane >> 2;
  const int j = lane & 3;
  const int K = p.K;
  const int ngroups = K / 32;
  const int niters = (ngroups + kGroupsPerIt - 1) / kGroupsPerIt;  // <= kStreamMaxIters
  const int tail = ngroups % kGroupsPerIt;
  constexpr int kRows = stream_rows<NR>();
  const int srow = scale_row_bytes(K);
  const int rowbytes = K / 2;
  uint8_t* const act = lds;  // [niters][kXBytes]
  uint8_t* const sbuf = lds + niters * kXBytes;  // [2][kRows][srow]

  const int e = p.block_expert[row0 / 4];
  const int64_t r0 = (int64_t)e * p.N;
  constexpr bool packed_layout = PK;  // see internal.h
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.packed + r0 * (K / 8)), 0, p.N * rowbytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t sres =
      packed_layout
          ? __builtin_amdgcn_make_buffer_rsrc(
                (void*)(reinterpret_cast<const uint8_t*>(p.scales) + e * pack_scale_bytes(p.N, K)),
                0, (int)pack_scale_bytes(p.N, K), kBufferFlags)
          : __builtin_amdgcn_make_buffer_rsrc((void*)(p.scales + r0 * (K / 32)), 0,
                                              p.N * (K / 32) * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.a_routed, 0, (int)((int64_t)p.max_blocks * 4 * K * 2), kBufferFlags);

  // this lane's weights: row-set rs, row j, group kp. Checkpoint layout: the
  // offset in slice group 0, plus kRows rows per slice group and 16 groups per
  // iteration. Prepacked layout (down rows in tiles of kPackRows, kRows
  // dividing it): the offset inside a slice group's rows of a tile, plus the
  // slice group's place (its tile, its rows in the tile) and four chunks of
  // the tile per iteration.
  static_assert(kPackRows % kRows == 0, "slice groups inside prepacked tiles");
  int woff[NR];
#pragma unroll
  for (int rs = 0; rs < NR; ++rs) {
    const int l = wave * 4 * NR + 4 * rs + j;  // row inside the slice group
    woff[rs] = packed_layout ? (int)pack_code_offset(false, 0, K, l, kp)
                             : ((sg0 * kRows + l) * (K / 8) + 4 * kp) * 4;
  }
  auto group_base = [&](int sg) {  // uniform: bytes of slice group sg0 + sg
    if (!packed_layout) return sg * kRows * rowbytes;
    const int sgg = sg0 + sg;
    constexpr int kPerTile = kPackRows / kRows;
    return (sgg / kPerTile) * pack_chunks(K) * kPackRows * 64 + (sgg % kPerTile) * kRows * 64;
  };
  const int wstep = packed_layout ? (kGroupsPerIt / 4) * kPackRows * 64 : kGroupsPerIt * 16;
  // the prefetch position (slice group, iteration) and its loads; past the
  // work-group's last iteration an offset beyond the buffer (reads zeros)
  int pf_sg = 0, pf_it = 0;
  auto load_next = [&](u32x4 (&w)[NR]) {
    const int off = uniform(pf_sg < nsg ? group_base(pf_sg) + pf_it * wstep : kOutOfRange);
#pragma unroll
    for (int rs = 0; rs < NR; ++rs)
      w[rs] = __builtin_amdgcn_raw_buffer_load_b128(wres, woff[rs], off, kStreamAux);
    if (++pf_it == niters) {
      pf_it = 0;
      ++pf_sg;
    }
  };

  // scales of slice group sg: kRows rows x 2 niters pieces of 16 bytes
  const int ppr = 2 * niters;
  const int npieces = kRows * ppr;
  constexpr int kSP = (kRows * 2 * kStreamMaxIters + kThreads - 1) / kThreads;
  u32x4 sv[kSP];
  auto load_scales = [&](int sg) {
#pragma unroll
    for (int u = 0; u < kSP; ++u) {
      const int i = u * kThreads + tid;
      const int r = i / ppr, pc = i - r * ppr;
      int off = kOutOfRange;
      if (i < npieces && pc * 8 < ngroups) {
        const int n = (sg0 + sg) * kRows + r;
        off = packed_layout ? (int)pack_scale_offset(false, 0, K, n, pc * 8)
                            : (n * (K / 32) + pc * 8) * 2;
      }
      sv[u] = __builtin_amdgcn_raw_buffer_load_b128(sres, off, 0, kScaleAux);
    }
  };
  auto store_scales = [&](uint8_t* sb) {
#pragma unroll
    for (int u = 0; u < kSP; ++u) {
      const int i = u * kThreads + tid;
      if (i < npieces) {
        const int r = i / ppr, pc = i - r * ppr;
        const int valid = ngroups - pc * 8;  // groups of the piece inside K
        u32x4 v = sv[u];
        if (valid < 8) {
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const uint32_t lo = 2 * h < valid ? (v[h] & 0xFFFFu) : 0u;
            const uint32_t hi = 2 * h + 1 < valid ? (v[h] & 0xFFFF0000u) : 0u;
            v[h] = lo | hi;
          }
        }
        *reinterpret_cast<u32x4*>(sb + r * srow + pc * 16) = v;
      }
    }
  };

  struct Frag {
    u32x4 w[NR];
  };
  Frag f[DEPTH + 1];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    load_next(f[d].w);
    __builtin_amdgcn_sched_barrier(0);  // keep the iterations' loads in issue order
  }

  // activations of the block for all of K: thread t -> token row t / 64,
  // piece t % 64 of each iteration's 1 KB (the fragment slots of small_tile)
  const int xt = tid >> 6;
  const int xc = tid & 63;
  const int xoff = (int)((row0 + xt) * K) * 2 + xc * 16;
  u32x4 xv[kStreamMaxIters];
#pragma unroll
  for (int it = 0; it < kStreamMaxIters; ++it)
    xv[it] = __builtin_amdgcn_raw_buffer_load_b128(xres, xoff,
                                                   uniform(it < niters ? it * 1024 : kOutOfRange), 0);
  load_scales(0);
  // the pair of token row r = kp % 4 (every slice group stores to it)
  const int r = kp & 3;
  const int32_t pair = p.sorted_ids[row0 + r];
  float* const dst = pair < p.P ? p.y_routed + (int64_t)pair * p.N : nullptr;

  const int xdst = (xc & 3) * 1024 + ((xc >> 2) * 4 + xt) * 16;
#pragma unroll
  for (int it = 0; it < kStreamMaxIters; ++it) {
    if (it >= niters) break;
    u32x4 v = xv[it];
    if (tail && it == niters - 1 && (xc >> 2) >= tail) v = u32x4{0, 0, 0, 0};
    // (x0..x7) -> (x0,x4,x1,x5 | x2,x6,x3,x7), the codes' field order
    v = u32x4{__builtin_amdgcn_perm(v[2], v[0], 0x05040100u),
              __builtin_amdgcn_perm(v[2], v[0], 0x07060302u),
              __builtin_amdgcn_perm(v[3], v[1], 0x05040100u),
              __builtin_amdgcn_perm(v[3], v[1], 0x07060302u)};
    *reinterpret_cast<u32x4*>(act + it * kXBytes + xdst) = v;
  }
  store_scales(sbuf);
  if (nsg > 1) load_scales(1);  // in flight during slice group 0
  __syncthreads();

  f32x4 acc[NR];
#pragma unroll
  for (int rs = 0; rs < NR; ++rs) acc[rs] = f32x4{0.f, 0.f, 0.f, 0.f};
  // this lane's scales: row (wave, 4 rs + j), group kp of the iteration
  const int sread_off = (wave * 4 * NR + j) * srow + kp * 2;

  // sum the k-parts of slice group sg and store its 4 NR columns per wave
  auto finish = [&](int sg) {
#pragma unroll
    for (int rs = 0; rs < NR; ++rs)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[rs][q] = kpart_sum(acc[rs][q]);
    const int col0 = ((sg0 + sg) * kWaves + wave) * (4 * NR);
#pragma unroll
    for (int t = 0; t < (NR + 3) / 4; ++t) {
      const int rsd = (kp >> 2) + 4 * t;
      if (rsd >= NR) continue;
      float v = 0.f;
#pragma unroll
      for (int rs = 0; rs < NR; ++rs) {
        if (rs == rsd) {
          v = acc[rs][0];
          v = (r == 1) ? acc[rs][1] : v;
          v = (r == 2) ? acc[rs][2] : v;
          v = (r == 3) ? acc[rs][3] : v;
        }
      }
      if (dst) dst[col0 + 4 * rsd + j] = v;
    }
#pragma unroll
    for (int rs = 0; rs < NR; ++rs) acc[rs] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  constexpr int kPeriod = (DEPTH + 1) % 2 ? 2 * (DEPTH + 1) : DEPTH + 1;
  const int total = nsg * niters;
  int it = 0, sg = 0;
  for (int i0 = 0; i0 < total; i0 += kPeriod) {
#pragma unroll
    for (int u = 0; u < kPeriod; ++u) {
      load_next(f[(u + DEPTH) % (DEPTH + 1)].w);
      __builtin_amdgcn_sched_barrier(0);
      int4_step<NR>(f[u % (DEPTH + 1)].w, act + it * kXBytes,
                    sbuf + (sg & 1) * kRows * srow + sread_off, srow, it, acc);
      if (++it == niters) {
        finish(sg);
        it = 0;
        ++sg;
        if (sg < nsg) {
          store_scales(sbuf + (sg & 1) * kRows * srow);
          __syncthreads();
          if (sg + 1 < nsg) load_scales(sg + 1);
        }
      }
      if (i0 + u + 1 >= total) break;
    }
  }
}

// Shared-expert work-groups first (as in small_gemm_kernel), then routed ones:
// each 4-row bucket block is split into runs of `sgs` slice groups.
template <int NR, int NRS, int TB, bool PK>
__global__ __launch_bounds__(kThreads, waves_per_simd(NR)) void stream_down_kernel(GemmParams p,
                                                                                   int sgs) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // stream_down_lds_bytes
  const int64_t bid = blockIdx.x;
  const int ns = p.N / slice_cols<kDown, NRS>() / kWaves;
  const int64_t shared = p.wshared ? (p.T + 4 * TB - 1) / (4 * TB) * ns : 0;
  if (bid < shared) {
    const int64_t tg = bid / ns;
    const int s = (int)(bid - tg * ns);
    small_tile<kDown, NRS, false, TB, 1>(p, tg * 4 * TB, s * kWaves, lds);
  } else {
    const int groups = p.N / stream_rows<NR>();
    const int runs = (groups + sgs - 1) / sgs;
    const int64_t b2 = bid - shared;
    const int64_t blk = b2 / runs;
    const int q = (int)(b2 - blk * runs);
    if (blk * 4 >= *p.n_padded) return;
    const int sg0 = q * sgs;
    down_stream_tile<NR, kSmallDepth, PK>(p, blk * 4, sg0, min(sgs, groups - sg0), lds);
  }
}

// ---------------------------------------------------------------------------
// Narrow reductions (down projection with I <= 512, e.g. one GPU's share of a
// tensor-parallel split). The whole of K (at most 16 groups) fits in one MFMA
// instruction's 16 blocks, so K is no longer the streamed dimension: each lane
// loads its activations once (registers, no LDS, no barrier), and the waves
// stream weight rows instead, the next step's rows in flight while the current
// ones are computed. With KG = 16 / RC blocks per copy, block kp holds group
// kp % KG of row-set copy kp / KG: one instruction covers RC row-sets of four
// rows, and the k-parts are summed across the KG blocks of each copy at every
// step. Groups past K (I = 384) are read out of range, i.e. as zeros.
// ---------------------------------------------------------------------------
template <int KG>
__device__ __forceinline__ float kpart_sum_narrow(float v) {
  v = add_xor8(add_xor4(v));
  if (KG >= 8) v = add_xor(v, 16);
  if (KG >= 16) v = add_xor(v, 32);
  return v;
}

#ifndef MOE_NARROW_STEPS
#define MOE_NARROW_STEPS 4
#endif
constexpr int kNarrowSteps = MOE_NARROW_STEPS;  // row steps per work-group
#ifndef MOE_NARROW_DEPTH
#define MOE_NARROW_DEPTH 3
#endif
constexpr int kNarrowDepth = MOE_NARROW_DEPTH;  // int4 steps in flight ahead

// weight rows of one wave step
template <int KG, int NR>
constexpr int narrow_rows() { return 4 * NR * (16 / KG); }

// NB blocks of four rows (routed: one 4-row bucket block; shared: NB blocks of
// consecutive tokens) against the weight rows of kNarrowSteps wave steps from
// n0 (fewer where N ends first: a wave takes the steps that start below N).
template <int KG, int NR, bool INT4, int NB, int DEPTH, bool PK = false>
__device__ __forceinline__ void narrow_tile(const GemmParams& p, int64_t row0, int n0) {
  constexpr int RC = 16 / KG;
  constexpr int RW = narrow_rows<KG, NR>();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // steps of this wave: those whose RW rows start below N (N is a multiple of RW)
  const int avail = p.N - n0 - wave * RW;
  const int nsteps =
      uniform(avail <= 0 ? 0 : min(kNarrowSteps, (avail + kWaves * RW - 1) / (kWaves * RW)));
  const int kp = lane >> 2;
  const int j = lane & 3;
  const int c = kp / KG;
  const int g = kp % KG;
  const int K = p.K;
  const bool gvalid = g < K / 32;

  // ---- activations: group g of token row j, once; (x0..x7) permuted to
  // (x0,x4,x1,x5 | x2,x6,x3,x7) for the int4 codes' field order --------------
  const uint16_t* abase = INT4 ? p.a_routed : p.a_shared;
  const int64_t arows = INT4 ? (int64_t)p.max_blocks * 4 : p.T;
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)abase, 0, (int)(arows * K * 2), kBufferFlags);
  u32x4 xf[NB][4];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    int64_t arow = row0 + 4 * b + j;
    if (!INT4 && arow >= p.T) arow = p.T - 1;  // never stored
    const int off = gvalid ? (int)(arow * K + 32 * g) * 2 : kOutOfRange;
#pragma unroll
    for (int q = 0; q < 4; ++q) xf[b][q] = __builtin_amdgcn_raw_buffer_load_b128(xres, off, 16 * q, 0);
  }
  // (permuted below, after the first weight loads are issued)
  // the pair of token row r, read before the weights for the same reason
  const int r = g & 3;
  int32_t pair = 0;
  if (INT4) pair = p.sorted_ids[row0 + r];

  // ---- weight rows of this lane: row-set rs, copy c, row j ------------------
  const int Nw = p.N;
  const int e = INT4 ? p.block_expert[row0 / 4] : 0;
  const int64_t r0 = (int64_t)e * Nw;
  // prepacked weights (see internal.h): a step's kWaves * RW rows lie in one
  // tile (the work-group's first row is a multiple of kPackRows), so a lane's
  // offset is its place in the step's rows plus the step's uniform base
  constexpr bool packed_layout = INT4 && PK;
  __amdgpu_buffer_rsrc_t wres, sres;
  if (INT4) {
    wres = __builtin_amdgcn_make_buffer_rsrc((void*)(p.packed + r0 * (K / 8)), 0,
                                             Nw * (K / 8) * 4, kBufferFlags);
    sres = packed_layout
               ? __builtin_amdgcn_make_buffer_rsrc(
                     (void*)(reinterpret_cast<const uint8_t*>(p.scales) +
                             e * pack_scale_bytes(Nw, K)),
                     0, (int)pack_scale_bytes(Nw, K), kBufferFlags)
               : __builtin_amdgcn_make_buffer_rsrc((void*)(p.scales + r0 * (K / 32)), 0,
                                                   Nw * (K / 32) * 2, kBufferFlags);
  } else {
    wres = __builtin_amdgcn_make_buffer_rsrc((void*)p.wshared, 0, Nw * K * 2, kBufferFlags);
    sres = wres;
  }
  auto row_of = [&](int step, int rs) {
    return n0 + (step * kWaves + wave) * RW + 4 * (rs * RC + c) + j;
  };
  static_assert(kPackRows % (kWaves * RW) == 0, "narrow steps inside prepacked tiles");
  int woff[NR], soff[NR];
#pragma unroll
  for (int rs = 0; rs < NR; ++rs) {
    const int row = row_of(0, rs);
    const int lr = row - n0;  // row inside the step
    if (packed_layout) {
      woff[rs] = gvalid ? (int)pack_code_offset(false, 0, K, lr, g) : kOutOfRange;
      soff[rs] = gvalid ? (int)pack_scale_offset(false, 0, K, lr, g) : kOutOfRange;
    } else {
      woff[rs] = !gvalid ? kOutOfRange : INT4 ? (row * (K / 8) + 4 * g) * 4 : (row * K + 32 * g) * 2;
      soff[rs] = gvalid ? (row * (K / 32) + g) * 2 : kOutOfRange;
    }
  }
  const int wstep = kWaves * RW * (INT4 ? K / 2 : 2 * K);  // bytes per step
  const int sstep = kWaves * RW * (K / 32) * 2;
  auto sofs = [&](int step, int bytes) {
    return uniform(step < nsteps ? step * bytes : kOutOfRange);
  };
  // prepacked: the uniform base of step `step` (its first row's tile and row)
  auto pofs = [&](int step, int tile_bytes, int row_bytes) {
    const int rb = n0 + step * kWaves * RW;
    return uniform(step < nsteps
                       ? (rb / kPackRows) * tile_bytes + (rb % kPackRows) * row_bytes
                       : kOutOfRange);
  };
  const int ptile_w = pack_chunks(K) * kPackRows * 64, ptile_s = pack_periods(K) * kPackRows * 32;

  struct Frag {
    u32x4 w[NR][INT4 ? 1 : 4];
    uint32_t s[INT4 ? NR : 1];
  };
  auto load = [&](Frag& f, int step) {
#pragma unroll
    for (int rs = 0; rs < NR; ++rs) {
      if (INT4) {
        f.w[rs][0] = __builtin_amdgcn_raw_buffer_load_b128(
            wres, woff[rs], packed_layout ? pofs(step, ptile_w, 64) : sofs(step, wstep),
            kStreamAux);
        f.s[rs] = __builtin_amdgcn_raw_buffer_load_b16(
            sres, soff[rs], packed_layout ? pofs(step, ptile_s, 32) : sofs(step, sstep),
            kScaleAux);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          f.w[rs][q] = __builtin_amdgcn_raw_buffer_load_b128(wres, woff[rs] + 16 * q,
                                                             sofs(step, wstep), kSharedAux);
      }
    }
  };

  // ring of DEPTH + 1 register stages: the loads of DEPTH steps are in flight
  // while a step is computed (past nsteps they read out of range: no traffic)
  Frag f[DEPTH + 1];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    load(f[d], d);
    // keep the steps' loads in issue order, so that a step waits for its own
    // loads only
    __builtin_amdgcn_sched_barrier(0);
  }

  f32x4 c0 = {0.f, 0.f, 0.f, 0.f};
  if (INT4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 v = xf[0][q];
      xf[0][q] = u32x4{__builtin_amdgcn_perm(v[2], v[0], 0x05040100u),
                       __builtin_amdgcn_perm(v[2], v[0], 0x07060302u),
                       __builtin_amdgcn_perm(v[3], v[1], 0x05040100u),
                       __builtin_amdgcn_perm(v[3], v[1], 0x07060302u)};
    }
    const u32x2 neg136 = {kNeg136, kNeg136};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c0 = mfma4(u32x2{xf[0][q][0], xf[0][q][1]}, neg136, c0);
      c0 = mfma4(u32x2{xf[0][q][2], xf[0][q][3]}, neg136, c0);
    }
  }

  // lane (g, j) of copy c stores token row g % 4 of row-sets g / 4 + (KG / 4) t
  constexpr int kStores = (NR * 4 + KG - 1) / KG;

  auto compute_store = [&](const Frag& f, int step) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      f32x4 v[NR];
      if (INT4) {
#pragma unroll
        for (int rs = 0; rs < NR; ++rs) v[rs] = c0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u32x2 b0[NR], b1[NR];
#pragma unroll
          for (int rs = 0; rs < NR; ++rs) {
            const uint32_t w = f.w[rs][0][q];
            b0[rs] = u32x2{and_or(w, 0x000F000Fu, kMagic), and_or(w >> 4, 0x000F000Fu, kMagic)};
            b1[rs] = u32x2{and_or(w >> 8, 0x000F000Fu, kMagic),
                           and_or(w >> 12, 0x000F000Fu, kMagic)};
          }
#pragma unroll
          for (int rs = 0; rs < NR; ++rs)
            v[rs] = mfma4(u32x2{xf[0][q][0], xf[0][q][1]}, b0[rs], v[rs]);
#pragma unroll
          for (int rs = 0; rs < NR; ++rs)
            v[rs] = mfma4(u32x2{xf[0][q][2], xf[0][q][3]}, b1[rs], v[rs]);
        }
#pragma unroll
        for (int rs = 0; rs < NR; ++rs) v[rs] *= bf16_to_f32(f.s[rs]);
      } else {
#pragma unroll
        for (int rs = 0; rs < NR; ++rs) v[rs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int rs = 0; rs < NR; ++rs)
            v[rs] = mfma4(u32x2{xf[b][q][0], xf[b][q][1]}, u32x2{f.w[rs][q][0], f.w[rs][q][1]},
                          v[rs]);
#pragma unroll
          for (int rs = 0; rs < NR; ++rs)
            v[rs] = mfma4(u32x2{xf[b][q][2], xf[b][q][3]}, u32x2{f.w[rs][q][2], f.w[rs][q][3]},
                          v[rs]);
        }
      }
#pragma unroll
      for (int rs = 0; rs < NR; ++rs)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[rs][i] = kpart_sum_narrow<KG>(v[rs][i]);

      float* dst = nullptr;
      if (INT4) {
        if (pair < p.P) dst = p.y_routed + (int64_t)pair * p.N;
      } else {
        const int64_t tok = row0 + 4 * b + r;
        if (tok < p.T) dst = p.y_shared + tok * p.N;
      }
#pragma unroll
      for (int t = 0; t < kStores; ++t) {
        const int rsd = (g >> 2) + (KG / 4) * t;
        if (rsd >= NR) continue;
        float val = 0.f;
#pragma unroll
        for (int rs = 0; rs < NR; ++rs) {
          if (rs == rsd) {
            val = v[rs][0];
            val = (r == 1) ? v[rs][1] : val;
            val = (r == 2) ? v[rs][2] : val;
            val = (r == 3) ? v[rs][3] : val;
          }
        }
        if (dst) dst[row_of(step, rsd)] = val;
      }
    }
  };

#pragma unroll
  for (int step = 0; step < kNarrowSteps; ++step) {
    if (step >= nsteps) break;
    if (step + DEPTH < kNarrowSteps) load(f[(step + DEPTH) % (DEPTH + 1)], step + DEPTH);
    __builtin_amdgcn_sched_barrier(0);
    compute_store(f[step % (DEPTH + 1)], step);
  }
}

// Work-groups: shared-expert items first (kTokBlocks 4-token blocks each),
// then routed 4-row bucket blocks; each takes kNarrowSteps wave steps of
// consecutive weight rows.
#ifndef MOE_NARROW_WAVES
#define MOE_NARROW_WAVES 3
#endif
template <int KG, int NR, int NRS, bool PK>
__global__ __launch_bounds__(kThreads, MOE_NARROW_WAVES) void narrow_down_kernel(GemmParams p) {
  const int64_t bid = blockIdx.x;
  constexpr int kRowsWGs = kNarrowSteps * kWaves * narrow_rows<KG, NRS>();
  constexpr int kRowsWG = kNarrowSteps * kWaves * narrow_rows<KG, NR>();
  const int cs = (p.N + kRowsWGs - 1) / kRowsWGs;
  const int64_t shared = p.wshared ? (p.T + 4 * kTokBlocks - 1) / (4 * kTokBlocks) * cs : 0;
  if (bid < shared) {
    const int64_t tg = bid / cs;
    const int n0 = (int)(bid - tg * cs) * kRowsWGs;
    narrow_tile<KG, NRS, false, kTokBlocks, 1>(p, tg * 4 * kTokBlocks, n0);
  } else {
    const int cr = (p.N + kRowsWG - 1) / kRowsWG;
    const int64_t b2 = bid - shared;
    const int64_t blk = b2 / cr;
    const int n0 = (int)(b2 - blk * cr) * kRowsWG;
    if (blk * 4 >= *p.n_padded) return;
    narrow_tile<KG, NR, true, 1, kNarrowDepth, PK>(p, blk * 4, n0);
  }
}

#ifndef MOE_NARROW_NR
#define MOE_NARROW_NR 4
#endif
#ifndef MOE_NARROW_NRS
#define MOE_NARROW_NRS 2
#endif

template <int KG>
hipError_t launch_narrow(const GemmParams& p, hipStream_t stream) {
  constexpr int NR = MOE_NARROW_NR, NRS = MOE_NARROW_NRS;
  // whole wave steps only (a work-group's last step may hold fewer waves)
  if (p.N % narrow_rows<KG, NR>() || p.N % narrow_rows<KG, NRS>() || p.K > 512 || p.K % 32)
    return hipErrorInvalidValue;
  constexpr int kRowsWGs = kNarrowSteps * kWaves * narrow_rows<KG, NRS>();
  constexpr int kRowsWG = kNarrowSteps * kWaves * narrow_rows<KG, NR>();
  const int64_t routed = (int64_t)p.max_blocks * ((p.N + kRowsWG - 1) / kRowsWG);
  const int64_t shared = p.wshared ? (p.T + 4 * kTokBlocks - 1) / (4 * kTokBlocks) *
                                         ((p.N + kRowsWGs - 1) / kRowsWGs)
                                   : 0;
  const int64_t grid = routed + shared;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  GemmParams args = p;
  void* kargs[] = {&args};
  const void* fn = p.prepacked
                       ? reinterpret_cast<const void*>(&narrow_down_kernel<KG, NR, NRS, true>)
                       : reinterpret_cast<const void*>(&narrow_down_kernel<KG, NR, NRS, false>);
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kThreads), kargs, 0, stream);
}

// Dynamic LDS of a launch: two activation stages (of the larger of the routed
// and the shared work items) and, for the routed ones, the staged scales.
template <int NR, int TB = kTokBlocksLarge>
int small_lds_bytes(int K) {
  const int routed = 2 * stage_bytes<1>() + kWaves * 4 * NR * scale_row_bytes(K);
  const int shared = 2 * stage_bytes<TB>();
  return routed > shared ? routed : shared;
}
constexpr int kMaxLds = 64 * 1024;

template <int PHASE, int NR, int NRS, int TB>
hipError_t launch_small_tb(const GemmParams& p, hipStream_t stream) {
  // every work-group holds whole 4-slice groups: N must split evenly
  if (p.N % (slice_cols<PHASE, NR>() * kWaves) || p.N % (slice_cols<PHASE, NRS>() * kWaves))
    return hipErrorInvalidValue;
  const int lds = small_lds_bytes<NR, TB>(p.K);
  if (lds > kMaxLds) return hipErrorInvalidValue;
  const int64_t routed = (int64_t)p.max_blocks * (p.N / slice_cols<PHASE, NR>() / kWaves);
  const int64_t shared = p.wshared ? (p.T + 4 * TB - 1) / (4 * TB) *
                                         (p.N / slice_cols<PHASE, NRS>() / kWaves)
                                   : 0;
  const int64_t grid = routed + shared;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  GemmParams args = p;
  void* kargs[] = {&args};
  const void* fn = p.prepacked
                       ? reinterpret_cast<const void*>(&small_gemm_kernel<PHASE, NR, NRS, TB, true>)
                       : reinterpret_cast<const void*>(&small_gemm_kernel<PHASE, NR, NRS, TB, false>);
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kThreads), kargs, (size_t)lds, stream);
}

// A few tokens: the shared weights are read once per 4 kTokBlocks tokens by
// many small work-groups; more tokens: once per 4 kTokBlocksLarge tokens,
// fewer re-reads of the shared weights for the same per-weight arithmetic.
template <int PHASE, int NR, int NRS>
hipError_t launch_small(const GemmParams& p, hipStream_t stream) {
  if (p.T > 4 * kTokBlocks) return launch_small_tb<PHASE, NR, NRS, kTokBlocksLarge>(p, stream);
  return launch_small_tb<PHASE, NR, NRS, kTokBlocks>(p, stream);
}

// Streamed down launch. Slice groups per routed work-group: enough routed
// work-groups to hold about kStreamTargetWG of them (the bucket count is not
// known on the host; min(pairs, experts) estimates it), at most kStreamSG.
#ifndef MOE_STREAM_TARGET_WG
#define MOE_STREAM_TARGET_WG 2048
#endif
constexpr int64_t kStreamTargetWG = MOE_STREAM_TARGET_WG;
#ifndef MOE_STREAM_ONE_ROUND
#define MOE_STREAM_ONE_ROUND 1
#endif
constexpr bool kStreamOneRound = MOE_STREAM_ONE_ROUND != 0;
constexpr int64_t kCUs = 256;  // MI355X compute units

template <int NR, int NRS, int TB>
hipError_t launch_stream_down(const GemmParams& p, hipStream_t stream) {
  if (p.N % stream_rows<NR>() || p.N % (slice_cols<kDown, NRS>() * kWaves) || p.K % 32)
    return hipErrorInvalidValue;
  const int routed_lds = stream_lds_bytes<NR>(p.K);
  const int shared_lds = 2 * stage_bytes<TB>();
  const int lds = routed_lds > shared_lds ? routed_lds : shared_lds;
  if (lds > kMaxLds) return hipErrorInvalidValue;
  const int groups = p.N / stream_rows<NR>();
  const int64_t est_blocks = std::max<int64_t>(1, std::min<int64_t>(p.P, p.max_blocks));
  int sgs = (int)std::min<int64_t>(kStreamSG, est_blocks * groups / kStreamTargetWG);
  if (sgs < 1) sgs = 1;
  const int64_t shared = p.wshared ? (p.T + 4 * TB - 1) / (4 * TB) *
                                         (p.N / slice_cols<kDown, NRS>() / kWaves)
                                   : 0;
  if (kStreamOneRound) {
    // a grid a little over one round of resident work-groups ends with a
    // second round of a few work-groups that start late: take more slice
    // groups per work-group where that fits the grid in one round
    const int64_t slots = (int64_t)kCUs * 4 * waves_per_simd(NR) / kWaves;
    auto grid_of = [&](int g) { return est_blocks * ((groups + g - 1) / g) + shared; };
    if (grid_of(sgs) > slots)
      for (int g = sgs + 1; g <= kStreamSG; ++g)
        if (grid_of(g) <= slots) {
          sgs = g;
          break;
        }
  }
  const int64_t routed = (int64_t)p.max_blocks * ((groups + sgs - 1) / sgs);
  const int64_t grid = routed + shared;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  GemmParams args = p;
  void* kargs[] = {&args, &sgs};
  const void* fn = p.prepacked
                       ? reinterpret_cast<const void*>(&stream_down_kernel<NR, NRS, TB, true>)
                       : reinterpret_cast<const void*>(&stream_down_kernel<NR, NRS, TB, false>);
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kThreads), kargs, (size_t)lds, stream);
}

}  // namespace

bool small_batch_fits(int32_t hidden, int32_t inter) {
  return small_lds_bytes<kNR>(hidden) <= kMaxLds && small_lds_bytes<kNRDown>(inter) <= kMaxLds;
}

hipError_t launch_gate_up_small(const GemmParams& p, hipStream_t stream) {
  return launch_small<kGateUp, kNR, kNRS>(p, stream);
}

hipError_t launch_down_small(const GemmParams& p, hipStream_t stream) {
  if (p.K <= 128) return launch_narrow<4>(p, stream);
  if (p.K <= 256) return launch_narrow<8>(p, stream);
  if (p.K <= 512) return launch_narrow<16>(p, stream);
  if (p.K <= 32 * kGroupsPerIt * kStreamMaxIters) {
    if (p.T > 4 * kTokBlocks) return launch_stream_down<kNRDown, kNRS, kTokBlocksLarge>(p, stream);
    return launch_stream_down<kNRDown, kNRS, kTokBlocks>(p, stream);
  }
  return launch_small<kDown, kNRDown, kNRS>(p, stream);
}

}  // namespace moe
