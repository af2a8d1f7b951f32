// gemm_prefill.hip -- grouped W4A16 GEMMs for many rows per expert (gfx950):
// the int4 routed experts of every batch past the decode regime, in 96-row
// bucket blocks, and the bf16 shared expert in 96-token tiles of the same
// launches.
//
// Two launches per layer (after the bucketing and the activation conversion
// below): gate_up with the SwiGLU epilogue, then down. Here the layer is a
// dense contraction per expert (about 85 rows each for 4096 tokens, top-8 of
// 384), so the kernel is built around keeping the MFMA pipes fed: every
// dequantised weight serves all rows of the block, and the int4 operands
// arrive through LDS without holding registers while in flight.
//
// Numerics: the int4 weights are exact. A code u of a group with scale s
// (Kimi-K2.6 catalog entry, QUANT paragraph: symmetric, group 32) is the value
// (u - 8) * s; with s a bf16 (8 significant bits) and |u - 8| <= 8 the product
// has at most 11 significant bits, which is exactly an fp16; the kernel's
// single-fma dequantisation (dequant8) gets it exactly for
// 2^-17 <= |s| <= 2720. So the routed products run on v_mfma_f32_16x16x32_f16:
//  * activations x are converted once per call to fp16 with one power-of-two
//    scale per token (x16_kernel: the largest |x| of the token lands in
//    [2^14, 2^15)), which is exact for every value down to 2^-32 of the
//    token's largest;
//  * the SwiGLU output h is rounded once to fp16 with one power-of-two scale
//    per (row, 256-column tile of gate_up); between the two launches
//    h_rescale_kernel brings each row's tiles to the row's largest scale
//    (exact except values below 2^-38 of the row's largest);
//  * the accumulators are fp32; the scales come back in the epilogues (exact
//    power-of-two multiplies).
// The bf16 shared expert keeps bf16 operands (bf16 MFMA, x as given, its h
// rounded to bf16).
//
// Routed work-group (512 threads = 8 waves): one block of up to kBM bucketed
// rows x 512 weight rows (a column tile; where K is only a few chunks, several
// consecutive tiles of the block in turn, prefill_tiles_kernel). Every wave
// owns four 16-row weight sub-tiles (gate_up: two gate sub-tiles and the two
// matching up sub-tiles) and computes them for all of the block's rows, so
// each weight is dequantised exactly once per block. K advances in chunks of
// 128 inputs (four 32-input groups):
//  * activations: a ring of kBM x 128 chunks in LDS, copied straight from
//    HBM (buffer loads with an LDS destination); a row's 16 pieces of 16
//    bytes are permuted, piece c of row r at slot c ^ f(r & 15) where f swaps
//    the two 2-bit halves of its argument, so that the fragment reads (16 rows
//    at one k offset per 16 lanes) are free of bank conflicts on gfx950
//    16-byte LDS reads (the simpler XOR forms are not);
//  * weights, checkpoint layout, one tile per work-group (block_tile_w): each
//    wave copies its own 64 rows into its own 8 KB of LDS in stages of 256
//    inputs, one whole 128-byte line per row, and reads its fragments into
//    registers at the start of the stage; the activation ring holds three
//    chunks, each copied two chunks ahead; the copies of a chunk go out a few
//    at a time between its MFMA steps;
//  * weights, prepacked layout or several tiles per work-group (block_tile):
//    lane (r = lane % 16, q = lane / 16) loads group q of row r of each of its
//    four sub-tiles straight into registers (16 bytes each), a ring of four
//    chunks; the activation ring holds four chunks, three ahead;
//  * scales: per wave, the groups of its rows for a stage (or a period of four
//    chunks), loaded into registers, stored to the wave's LDS area and read
//    back at the start of the stage;
//  * the words are dequantised to fp16 (u - 8) * s and fed to the MFMA: step j
//    of a chunk takes word j of every lane, so its 32-long reduction covers one
//    8-input slice of each of the four groups; the matching activations are
//    read at those offsets. The dequantisation (VALU) is interleaved with the
//    MFMAs.
// One barrier per chunk, which also frees the activation slot that the next
// copies overwrite. Barriers are raw s_barrier with explicit waits (the fence
// of __syncthreads() would also wait for the copies just issued). The number
// of 16-row sub-tiles holding bucket rows is a template parameter of the K
// loop, so the loop body is straight-line code. Widths that are not whole
// tiles (hidden % 512, inter % 256) run masked: weight rows past the width
// read zeros and their outputs are not stored.
//
// Shared-expert work-group: 128 tokens x 512 weight rows of the bf16 weights,
// both operands through LDS in stages of 64 inputs (see shared_tile).
#include "internal.h"

namespace moe {
namespace {

// cache policy bits of the int4 weight copies: the default policy in the
// checkpoint layout (the rest of each line is read a chunk later and should
// stay in L2), non-temporal in the prepacked layout (every line is used whole
// by one copy)
#ifndef MOE_PREFILL_AUX
#define MOE_PREFILL_AUX 0
#endif
constexpr int kPrefillAux = MOE_PREFILL_AUX;
// instruction scheduling of an MFMA step: 1 = activation reads, then one
// MFMA per two VALU instructions; 2 = compiler's order within each step;
// 0 = compiler's order across steps
#ifndef MOE_PREFILL_SCHED
#define MOE_PREFILL_SCHED 1
#endif
constexpr int kPrefillSched = MOE_PREFILL_SCHED;
#ifndef MOE_PREFILL_PRIO
#define MOE_PREFILL_PRIO 0
#endif
constexpr int kPrefillPrio = MOE_PREFILL_PRIO;  // wave priority around a sub-tile's MFMAs
constexpr int kPrefillPackedAux = 2;

typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

#ifndef MOE_PREFILL_MAX_SUBTILES
#define MOE_PREFILL_MAX_SUBTILES 6
#endif

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxMS = MOE_PREFILL_MAX_SUBTILES;  // 16-row sub-tiles per block
constexpr int kBM = 16 * kMaxMS;           // bucket rows per block
constexpr int kNSub = 4;                   // 16-row weight sub-tiles per wave
constexpr int kBN = kWaves * kNSub * 16;   // weight rows per work-group
constexpr int kKC = 128;                   // inputs per chunk
constexpr int kSPeriod = 4;                // chunks per scale buffer
constexpr int kABytes = kBM * kKC * 2;     // activation chunk in LDS
constexpr int kWRowBytes = kKC / 2;        // int4 bytes of a weight row per chunk
constexpr int kWBytes = kBN * kWRowBytes;
constexpr int kSRowBytes = kSPeriod * 4 * 2;  // scale bytes of one row per buffer
constexpr int kSBytes = kBN * kSRowBytes;
constexpr int kBufferFlags = 0x00020000;   // raw buffer resource, dword 3
static_assert(kBN == kPackRows && kKC == kPackChunk, "tiles of the prepacked layout");
static_assert(kHTile == kBN / 2, "h exponent tiles are the gate_up column tiles");
constexpr uint32_t kNoRow = 0x80000000u;   // offset past any buffer: loads 0
#ifndef MOE_PREFILL_ODD_SUBTILES
#define MOE_PREFILL_ODD_SUBTILES 1
#endif
// blocks of 33-48 and 65-80 rows run the K loop for 3 and 5 sub-tiles
// (otherwise 4 and 6)
constexpr bool kOddSubtiles = MOE_PREFILL_ODD_SUBTILES != 0;
#ifndef MOE_PREFILL_ONE_SUBTILE
#define MOE_PREFILL_ONE_SUBTILE 1
#endif
// blocks of at most 16 rows (an expert's last rows, the few-pair experts of
// skewed batches) run the K loop for one sub-tile (otherwise two)
constexpr bool kOneSubtile = MOE_PREFILL_ONE_SUBTILE != 0;
#ifndef MOE_PREFILL_WLDS
#define MOE_PREFILL_WLDS 1
#endif
// checkpoint-layout blocks of one tile per work-group stage their weights
// through LDS in whole lines (block_tile_w); otherwise straight into
// registers (block_tile)
constexpr bool kWeightsLds = MOE_PREFILL_WLDS != 0;
#ifndef MOE_PREFILL_WLDS_AUX
#define MOE_PREFILL_WLDS_AUX 2
#endif
// cache policy of those whole-line weight copies: non-temporal (each line is
// used once, by one copy; kept out of the way of the activation chunks that
// the block's other column tiles read from L2)
constexpr int kWLdsAux = MOE_PREFILL_WLDS_AUX;
#ifndef MOE_PREFILL_STEP_PRIO
#define MOE_PREFILL_STEP_PRIO 1
#endif
constexpr bool kStepPrio = MOE_PREFILL_STEP_PRIO != 0;
#ifndef MOE_PREFILL_WLDS_SCHED
#define MOE_PREFILL_WLDS_SCHED 0
#endif
// instruction order of an MFMA step in that tile (as kPrefillSched); the
// compiler's own order measured 2-3% faster there than the fixed interleave
constexpr int kWLdsSched = MOE_PREFILL_WLDS_SCHED;
#ifndef MOE_SHARED_TOKENS
#define MOE_SHARED_TOKENS 128
#endif
constexpr int kSBM = MOE_SHARED_TOKENS;    // tokens per shared-expert work-group
static_assert(kSBM % 32 == 0 && kSBM <= 128, "shared token block: 2..8 sub-tiles");
constexpr int kSKC = 64;                   // inputs per shared-expert stage
constexpr int kSRow = kSKC * 2;            // bytes of a row per stage: one 128-byte line

enum { kGateUp = 0, kDown = 1 };

// the routed blocks' ring of four activation chunks (kBM rows x 128 inputs);
// the shared-expert tiles stage their weights in the first (sized for them)
// and their activations in the next two. Each buffer is an object of its
// own: the compiler then sees that a buffer load into one (an LDS write it
// tracks with the vector-memory counter) does not alias LDS reads of
// another, and does not wait for the copies just issued before the next
// reads.
constexpr int kSWBytes = kWaves * 64 * kSRow;  // shared-expert weight stage
__shared__ __attribute__((aligned(1024))) uint8_t lds_a0[kSWBytes > kABytes ? kSWBytes : kABytes];
__shared__ __attribute__((aligned(1024))) uint8_t lds_a1[kABytes];
__shared__ __attribute__((aligned(1024))) uint8_t lds_a2[kABytes];
__shared__ __attribute__((aligned(1024))) uint8_t lds_a3[kABytes];
// per wave: the bf16 scales of its 64 weight rows, 16 groups (four chunks)
// per row; only the wave itself writes and reads its buffer (ordinary LDS
// stores of registers: a copy with an LDS destination into it would make the
// compiler wait for every copy in flight before reading it)
constexpr int kScRow = 32;                   // bytes per row and period
constexpr int kScBuf = 64 * kScRow;          // one wave's buffer
__shared__ __attribute__((aligned(1024))) uint8_t lds_sc[kWaves][kScBuf];
// per block row: the exponent of its activation scale (gate_up: the token's;
// down: the row's largest h tile exponent), the h tile exponent being chosen,
// and the per-wave maxima it is chosen from
__shared__ int32_t lds_rexp[kBM];
// down, staged epilogue: the pair id of each block row (the y row it writes)
__shared__ int32_t lds_rpair[kBM];
__shared__ int32_t lds_rkh[kBM];
__shared__ float lds_rmax[kWaves][kBM];

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) {
  return __builtin_bit_cast(float, bits << 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// (a & m) | c in one v_bitop3_b32 (truth table 0xEA over (a, m, c)).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, m, c, 0xEA);
}

// A bf16 group scale as an fp16 pair (exact for 2^-17 <= |s| <= 65504).
__device__ __forceinline__ h16x2 scale_pair(uint32_t bits) {
  const _Float16 h = (_Float16)bf16_to_f32(bits);
  return h16x2{h, h};
}

#ifndef MOE_DEQUANT_FMA
#define MOE_DEQUANT_FMA 1
#endif
// 1: the single-fma dequantisation below (12 VALU per word); 0: subtract,
// then multiply (13)
constexpr bool kDequantFma = MOE_DEQUANT_FMA != 0;

// A group's scale s as an fp16 pair and the pair -24 s (the offset of the
// single-fma form below; exact for |s| <= 2720, i.e. 24 |s| <= 65504).
struct GroupScale {
  h16x2 s, c;
};
__device__ __forceinline__ GroupScale group_scale(uint32_t bits) {
  const h16x2 s = scale_pair(bits);
  const h16x2 m24 = {(_Float16)-24.0f, (_Float16)-24.0f};
  return {s, s * m24};
}

// The eight codes of one word -> eight fp16 weights (u - 8) * s, in the order
// of fields 0, 4, 1, 5, 2, 6, 3, 7 (activations are stored in the same order).
// Single-fma form: each field is shifted to bits 6-9 of its 16-bit half, right
// below the implicit bit, and OR-ed into the fp16 pattern 0x4C00 (16.0): the
// value is exactly 16 + u. fma(16 + u, s, -24 s) is (u - 8) * s before its
// one rounding, and that product is exact in fp16 (at most 11 significant
// bits), so the weight is exact whenever -24 s is: 2^-17 <= |s| <= 2720.
// 12 VALU instructions per word (four shifts, four v_bitop3, four packed
// fp16 fma). Two-step form: a field in bits 0-3 of a half OR-ed into 0x6400
// is 1024 + u, one in bits 4-7 gives 1024 + 16 u; (1024 + u) - 1032 and
// (1024 + 16 u) / 16 - 72 are exactly u - 8, then times s (exact for
// 2^-17 <= |s| < 2^13); 13 instructions (one shift, four v_bitop3, four
// packed add/fma, four packed multiplies).
__device__ __forceinline__ h16x8 dequant8(uint32_t w, const GroupScale& g) {
  h16x2 q0, q1, q2, q3;
  if (kDequantFma) {
    constexpr uint32_t kField = 0x03C003C0u, k16 = 0x4C004C00u;
    q0 = __builtin_elementwise_fma(__builtin_bit_cast(h16x2, and_or(w << 6, kField, k16)), g.s,
                                   g.c);  // u0, u4
    q1 = __builtin_elementwise_fma(__builtin_bit_cast(h16x2, and_or(w << 2, kField, k16)), g.s,
                                   g.c);  // u1, u5
    q2 = __builtin_elementwise_fma(__builtin_bit_cast(h16x2, and_or(w >> 2, kField, k16)), g.s,
                                   g.c);  // u2, u6
    q3 = __builtin_elementwise_fma(__builtin_bit_cast(h16x2, and_or(w >> 6, kField, k16)), g.s,
                                   g.c);  // u3, u7
  } else {
    const uint32_t w8 = w >> 8;
    const h16x2 c1032 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h16x2 c16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h16x2 c72 = {(_Float16)-72.0f, (_Float16)-72.0f};
    const h16x2 h0 = __builtin_bit_cast(h16x2, and_or(w, 0x000F000Fu, 0x64006400u));   // u0, u4
    const h16x2 h1 = __builtin_bit_cast(h16x2, and_or(w, 0x00F000F0u, 0x64006400u));   // u1, u5
    const h16x2 h2 = __builtin_bit_cast(h16x2, and_or(w8, 0x000F000Fu, 0x64006400u));  // u2, u6
    const h16x2 h3 = __builtin_bit_cast(h16x2, and_or(w8, 0x00F000F0u, 0x64006400u));  // u3, u7
    q0 = (h0 + c1032) * g.s;
    q1 = __builtin_elementwise_fma(h1, c16, c72) * g.s;
    q2 = (h2 + c1032) * g.s;
    q3 = __builtin_elementwise_fma(h3, c16, c72) * g.s;
  }
  return h16x8{q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
}

// Position of input c inside its stored 8-element piece: fields 0..7 are
// stored in the order 0, 4, 1, 5, 2, 6, 3, 7.
__device__ __forceinline__ int perm_pos(int c) {
  const int j = c & 7;
  return (c & ~7) | ((j & 3) << 1) | (j >> 2);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Exponent k with m * 2^-k in [2^14, 2^15) for a positive finite m; 0
// otherwise (zero rows; rows holding inf or NaN keep them).
__device__ __forceinline__ int scale_exp(float m) {
  if (!(m > 0.f) || !(m <= 3.0e38f)) return 0;
  return __builtin_amdgcn_frexp_expf(m) - 15;
}

// largest value over the 16 lanes of a row of the wave (lanes 16q..16q+15)
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, __shfl_xor(v, 1, 16));
  v = fmaxf(v, __shfl_xor(v, 2, 16));
  v = fmaxf(v, __shfl_xor(v, 4, 16));
  v = fmaxf(v, __shfl_xor(v, 8, 16));
  return v;
}

// s_waitcnt with only the vector-memory counter limited (lgkm and exp left
// unconstrained), and with the LDS counter at zero.
template <int N>
__device__ __forceinline__ void wait_vm() {
  // gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

template <int PHASE>
constexpr int tile_cols() { return PHASE == kGateUp ? kBN / 2 : kBN; }

// Permutation of the sixteen 16-byte pieces of activation row r in LDS.
__device__ __forceinline__ int aslot(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// Permutation of the 16-byte pieces of a 128-byte row staged in LDS (the
// shared-expert operands, the routed weights of the LDS-staged tile): piece
// P of row r sits in slot P ^ sswz(r), so that 16 rows read at one piece
// fall in distinct banks.
__device__ __forceinline__ int sswz(int r) { return (r >> 1) & 7; }

// Output column (h column for gate_up, y column for down) of work-group row
// R = 64 wave + 16 sub-tile + r; gate_up sub-tiles 0, 1 are gate rows, 2, 3
// the matching up rows.
template <int PHASE>
__device__ __forceinline__ int out_col(int tile, int R) {
  const int w = R >> 6, s = (R >> 4) & 3, r = R & 15;
  if (PHASE == kGateUp) return tile * (kBN / 2) + w * 32 + 16 * (s & 1) + r;
  return tile * kBN + w * 64 + 16 * s + r;
}
// Weight row of work-group row R, or -1 past the width.
template <int PHASE>
__device__ __forceinline__ int weight_row(const GemmParams& p, int tile, int R) {
  const int c = out_col<PHASE>(tile, R);
  if (PHASE == kGateUp) {
    if (c >= p.I) return -1;
    return ((R >> 4) & 3) < 2 ? c : p.I + c;  // gate rows, then the matching up rows
  }
  return c < p.N ? c : -1;
}

// ---- the x conversion --------------------------------------------------------
// x16[t] = fp16(x[t] * 2^-kx[t]) in the stored piece order, kx[t] chosen from
// the token's largest finite |x| (one work-group per token).
constexpr int kConvThreads = 256;

__global__ __launch_bounds__(kConvThreads) void x16_kernel(const uint16_t* __restrict__ x,
                                                           uint16_t* __restrict__ x16,
                                                           int32_t* __restrict__ kx, int H) {
  __shared__ uint32_t wmax[kConvThreads / 64];
  const int64_t t = blockIdx.x;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + t * H);
  u32x4* dst = reinterpret_cast<u32x4*>(x16 + t * H);
  const int npieces = H / 8;
  uint32_t m = 0;
  for (int g = threadIdx.x; g < npieces; g += kConvThreads) {
    const u32x4 v = src[g];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t lo = v[d] & 0x7FFFu, hi = (v[d] >> 16) & 0x7FFFu;
      if (lo < 0x7F80u) m = max(m, lo);  // finite values only
      if (hi < 0x7F80u) m = max(m, hi);
    }
  }
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const int k = scale_exp(bf16_to_f32(m));
  if (threadIdx.x == 0) kx[t] = k;
  for (int g = threadIdx.x; g < npieces; g += kConvThreads) {
    const u32x4 v = src[g];
    _Float16 h[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      h[2 * d] = (_Float16)__builtin_ldexpf(bf16_to_f32(v[d] & 0xFFFFu), -k);
      h[2 * d + 1] = (_Float16)__builtin_ldexpf(bf16_to_f32(v[d] >> 16), -k);
    }
    // stored order: inputs 0, 4, 1, 5, 2, 6, 3, 7 of the piece
    const h16x8 o = {h[0], h[4], h[1], h[5], h[2], h[6], h[3], h[7]};
    dst[g] = __builtin_bit_cast(u32x4, o);
  }
}

// ---- the h rescale between the launches ----------------------------------------
// For every bucketed row r below n_padded: kr[r] = the largest of its tile
// exponents kh[r][.], and each tile's fp16 values times 2^(kh - kr) in place
// (a power of two <= 1: exact unless the value falls below fp16's range,
// i.e. below 2^-38 of the row's largest). One work-group per row.
__global__ __launch_bounds__(kConvThreads) void h_rescale_kernel(uint16_t* __restrict__ h,
                                                                const int32_t* __restrict__ kh,
                                                                int32_t* __restrict__ kr,
                                                                const int32_t* __restrict__ n_padded,
                                                                int I, int n_htiles) {
  const int64_t r = blockIdx.x;
  if (r >= *n_padded) return;
  const int32_t* k = kh + r * n_htiles;
  int m = k[0];
  for (int j = 1; j < n_htiles; ++j) m = max(m, k[j]);
  if (threadIdx.x == 0) kr[r] = m;
  u32x4* row = reinterpret_cast<u32x4*>(h + r * I);
  for (int g = threadIdx.x; g < I / 8; g += kConvThreads) {
    const int d = k[g * 8 / kHTile] - m;
    if (d == 0) continue;
    // (the whole 16-byte piece is reinterpreted at once: a bit_cast of a
    // single element of an ext_vector value miscompiles with this compiler,
    // reading element 0 for every element)
    const _Float16 f = (_Float16)__builtin_ldexpf(1.0f, d);
    const h16x8 f8 = {f, f, f, f, f, f, f, f};
    row[g] = __builtin_bit_cast(u32x4, __builtin_bit_cast(h16x8, row[g]) * f8);
  }
}

// ---- routed blocks: activation copies and row exponents -------------------------
// A block's activations reach LDS in chunks of kBM rows x 128 inputs (256
// bytes per row); copy instruction u covers LDS rows 4u..4u+3 (16 lanes per
// row, 16 bytes each: whole lines), kAPW instructions per wave and chunk.
constexpr int kAPW = kBM / 4 / kWaves;
static_assert((kBM / 4) % kWaves == 0, "activation copies per wave");

template <int PHASE>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_act_rsrc(const GemmParams& p) {
  return __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.a_routed, 0,
      (int)((PHASE == kGateUp ? p.T : (int64_t)p.max_blocks * kBM) * p.K * 2), kBufferFlags);
}

// Source offsets of this lane's activation copies: row 4 (kAPW wave + i) +
// lane / 16, piece lane % 16 stored at the permuted slot; rows past the
// block's sub-tiles and padding rows read zeros.
template <int PHASE, int MS>
__device__ __forceinline__ void block_act_offsets(const GemmParams& p, int64_t row0,
                                                  uint32_t (&aoff)[kAPW]) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < kAPW; ++i) {
    const int row = 4 * (kAPW * wave + i) + (lane >> 4);
    const int piece = (lane & 15) ^ aslot(row & 15);
    int64_t src = -1;
    if (row < MS * 16) {
      if (PHASE == kGateUp) {
        const int32_t pair = p.sorted_ids[row0 + row];
        if (pair < p.P) src = pair / p.k;
      } else {
        src = row0 + row;
      }
    }
    aoff[i] = src < 0 ? kNoRow : (uint32_t)((src * p.K + piece * 8) * 2);
  }
}

// Per-row activation exponents for the epilogue (gate_up: the token's; down:
// the row's, after h_rescale_kernel), into lds_rexp.
template <int PHASE, int MS, bool STAGE = false>
__device__ __forceinline__ void block_row_exps(const GemmParams& p, int64_t row0) {
  const int tid = threadIdx.x;
  if (tid < kBM) {
    int v = 0;
    if (PHASE == kGateUp) {
      const int32_t pair = p.sorted_ids[row0 + tid];
      if (pair < p.P) v = p.a_exp[pair / p.k];
    } else if (tid < MS * 16) {
      v = p.a_exp[row0 + tid];
    }
    lds_rexp[tid] = v;
    if (PHASE == kDown && STAGE) lds_rpair[tid] = tid < MS * 16 ? p.sorted_ids[row0 + tid] : INT32_MAX;
  }
}

// Epilogue of a routed block tile: lane holds rows 4 lq + i of each 16-row
// sub-tile, column lr. STAGE: the wave's 8 KB of lds_a0 is free (every copy
// into LDS has landed and every wave is past its last fragment read), and the
// outputs go through it so that each lane stores 16 bytes of a row at a time:
// one store instruction per 16 rows x 16 columns of fp32 (or 32 of fp16)
// instead of one per 4 rows x 16 columns. (A vector-memory instruction costs
// its 64 addresses whatever their width; the 2- and 4-byte stores of the
// plain form made these epilogues a sixth of a short tile's time.)
constexpr int kStageRow = 20;  // fp32 per staged row of 16 columns (padded: the
                               // writes of the four row groups fall in distinct banks)
constexpr int kStageRowH = 40; // fp16 per staged row of 32 h columns (padded likewise)
template <int PHASE, int MS, bool STAGE>
__device__ __forceinline__ void block_epilogue(const GemmParams& p, f32x4 (&acc)[MS][kNSub],
                                               int64_t row0, int ctile) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int lr = lane & 15;
  const int lq = lane >> 4;
  if (PHASE == kGateUp) {
    // h = silu(g) * u at the true scale (activations came scaled by 2^-kx),
    // then one power-of-two scale per row of the tile, from the row's
    // largest |h| over the tile's 256 columns
    float rmax[MS][4];
#pragma unroll
    for (int mi = 0; mi < MS; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kx = lds_rexp[mi * 16 + 4 * lq + i];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const float g = __builtin_ldexpf(acc[mi][s][i], kx);
          const float u = __builtin_ldexpf(acc[mi][s + 2][i], kx);
          acc[mi][s][i] = silu_mul(g, u);
        }
        rmax[mi][i] = max16(fmaxf(fabsf(acc[mi][0][i]), fabsf(acc[mi][1][i])));
      }
    if (lr == 0) {
#pragma unroll
      for (int mi = 0; mi < MS; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) lds_rmax[wave][mi * 16 + 4 * lq + i] = rmax[mi][i];
    }
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    if (tid < MS * 16) {
      float m = lds_rmax[0][tid];
#pragma unroll
      for (int w2 = 1; w2 < kWaves; ++w2) m = fmaxf(m, lds_rmax[w2][tid]);
      const int kh = scale_exp(m);
      lds_rkh[tid] = kh;
      p.h_exp[(row0 + tid) * p.n_htiles + ctile] = kh;
    }
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    _Float16* h16 = reinterpret_cast<_Float16*>(p.h_routed);
    if (STAGE) {
      // the wave's 32 h columns of each row, in the stored order
      _Float16* st = reinterpret_cast<_Float16*>(lds_a0 + wave * 8192);
      static_assert(kBM * kStageRowH * 2 <= 8192, "h staging area");
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int pc = perm_pos(16 * s + lr);
#pragma unroll
        for (int mi = 0; mi < MS; ++mi)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = mi * 16 + 4 * lq + i;
            st[r * kStageRowH + pc] = (_Float16)__builtin_ldexpf(acc[mi][s][i], -lds_rkh[r]);
          }
      }
      const int col0 = ctile * (kBN / 2) + wave * 32;  // the wave's 32 columns lie all
      if (col0 < p.I) {                                // inside the width or all past it
        // piece q = 64 u + lane: row q / 4, 8 stored positions 8 (q % 4) ..
#pragma unroll
        for (int u = 0; u < MS; ++u) {
          const int q = 64 * u + lane;
          const int r = q >> 2, g = q & 3;
          const u32x4 v = *reinterpret_cast<const u32x4*>(st + r * kStageRowH + 8 * g);
          *reinterpret_cast<u32x4*>(h16 + (row0 + r) * p.I + col0 + 8 * g) = v;
        }
      }
      return;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int col = ctile * (kBN / 2) + wave * 32 + 16 * s + lr;
      if (col >= p.I) continue;
      const int pc = perm_pos(col);
#pragma unroll
      for (int mi = 0; mi < MS; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = mi * 16 + 4 * lq + i;
          h16[(row0 + r) * p.I + pc] = (_Float16)__builtin_ldexpf(acc[mi][s][i], -lds_rkh[r]);
        }
    }
  } else if (STAGE) {
    // one 16-column sub-tile at a time: all rows of it through the wave's LDS
    // area, then 16 bytes (4 columns of a row) per lane
    float* st = reinterpret_cast<float*>(lds_a0 + wave * 8192);
    static_assert(kBM * kStageRow * 4 <= 8192, "y staging area");
    const int colw = ctile * kBN + wave * 64;  // the wave's 64 columns lie all inside
    if (colw >= p.N) return;                   // the width or all past it
#pragma unroll
    for (int s = 0; s < kNSub; ++s) {
#pragma unroll
      for (int mi = 0; mi < MS; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = mi * 16 + 4 * lq + i;
          st[r * kStageRow + lr] = __builtin_ldexpf(acc[mi][s][i], lds_rexp[r]);
        }
      // piece q = 64 u + lane: row q / 4, columns 4 (q % 4) ..
#pragma unroll
      for (int u = 0; u < MS; ++u) {
        const int q = 64 * u + lane;
        const int r = q >> 2, g = q & 3;
        const f32x4 v = *reinterpret_cast<const f32x4*>(st + r * kStageRow + 4 * g);
        const int32_t pair = lds_rpair[r];
        if (pair < p.P)
          *reinterpret_cast<f32x4*>(p.y_routed + (int64_t)pair * p.N + colw + 16 * s + 4 * g) = v;
      }
    }
  } else {
#pragma unroll
    for (int mi = 0; mi < MS; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mi * 16 + 4 * lq + i;
        const int64_t row = row0 + r;
        const int32_t pair = p.sorted_ids[row];
        if (pair >= p.P) continue;
        const int kr = lds_rexp[r];
        float* dst = p.y_routed + (int64_t)pair * p.N;
#pragma unroll
        for (int s = 0; s < kNSub; ++s) {
          const int col = ctile * kBN + wave * 64 + 16 * s + lr;
          if (col < p.N) dst[col] = __builtin_ldexpf(acc[mi][s][i], kr);
        }
      }
  }
}

// ---- routed int4 blocks ---------------------------------------------------------
// K advances in chunks of 128 inputs (four groups of 32). Each wave streams
// its own 64 weight rows straight into registers: lane (lr, lq) loads group
// lq of row 16 s + lr of each sub-tile s (16 bytes; the four lanes of a row
// read its 64 bytes of the chunk), three chunks ahead of their use, in a ring
// of four register sets. The activations (kBM rows x 128 inputs) reach LDS
// through buffer loads with an LDS destination, also three chunks ahead, in a
// ring of four buffers. Each wave copies the bf16 scales of its rows into its
// own LDS area, 16 groups (32 bytes) per row every four chunks. MFMA step j of
// a chunk takes word j of every lane, so its 32-long reduction covers one
// 8-input slice of each of the four groups; the matching activations are read
// at piece 4 lq + j of each row. One barrier per chunk, which also frees the
// activation buffer that the next copies overwrite. The down phase's
// activations are the h rows in fp16 with one exponent per row
// (h_rescale_kernel brings each row's tiles to its largest exponent between
// the two launches).
constexpr int kRing = 4;          // chunk slots in flight: the one computed + 3 ahead
template <int PHASE, int MS, bool PK, bool MT>
__device__ __forceinline__ void block_tile(const GemmParams& p, int mblk, int tile, int ntl_arg) {
  const int ntl = MT ? ntl_arg : 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int lr = lane & 15;
  const int lq = lane >> 4;
  const int K = p.K;
  const int nch = K / kKC;                   // 128-input chunks
  const int nkp = (nch + kRing - 1) / kRing * kRing;  // chunk slots per tile
  const int64_t row0 = (int64_t)mblk * kBM;
  const int e = p.block_expert[mblk];
  const int Nw = (PHASE == kGateUp) ? 2 * p.I : p.N;
  const int64_t wbase = (int64_t)e * Nw;

  const __amdgpu_buffer_rsrc_t ares = block_act_rsrc<PHASE>(p);
  uint32_t aoff[kAPW];
  block_act_offsets<PHASE, MS>(p, row0, aoff);
  // slot c of tile t; past the tiles or the chunks, offsets past any buffer
  // (zeros; the copies are issued all the same, so that every chunk waits on
  // the same number of loads)
  auto copy_a = [&](uint8_t* dst, int t, int c) {
    const int so = uniform(t < ntl && c < nch ? c * kKC * 2 : (int)kNoRow);
#pragma unroll
    for (int i = 0; i < kAPW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ares, (lds_ptr)(dst + (kAPW * wave + i) * 1024), 16,
                                               aoff[i], so, 0, 0);
  };

  // ---- weights into registers, scales into the wave's LDS area ---------------
  constexpr bool packed_layout = PK;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.packed + wbase * (K / 8)), 0, Nw * (K / 8) * 4, kBufferFlags);
  const int nper = (nch + kSPeriod - 1) / kSPeriod;  // scale periods (4 chunks)
  const __amdgpu_buffer_rsrc_t sres =
      packed_layout
          ? __builtin_amdgcn_make_buffer_rsrc(
                (void*)(reinterpret_cast<const uint8_t*>(p.scales) + e * pack_scale_bytes(Nw, K)),
                0, (int)pack_scale_bytes(Nw, K), kBufferFlags)
          : __builtin_amdgcn_make_buffer_rsrc((void*)(p.scales + wbase * (K / 32)), 0,
                                              Nw * (K / 32) * 2, kBufferFlags);
  uint32_t woff[kNSub];
#pragma unroll
  for (int s = 0; s < kNSub; ++s) {
    const int R = wave * 64 + 16 * s + lr;
    const int n = weight_row<PHASE>(p, tile, R);
    woff[s] = n < 0 ? kNoRow
              : packed_layout ? (uint32_t)(((tile * nch) * kBN + R) * kWRowBytes + 16 * lq)
                              : (uint32_t)(n * (K / 2) + 16 * lq);
  }
  // scales: instruction i of a period copies the 32 bytes (16 groups) of the
  // wave's rows 32 i + lane / 2
  uint32_t scoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int R = wave * 64 + 32 * i + (lane >> 1);
    const int n = weight_row<PHASE>(p, tile, R);
    scoff[i] = n < 0 ? kNoRow
               : packed_layout ? (uint32_t)(((tile * nper) * kBN + R) * kSRowBytes + 16 * (lane & 1))
                               : (uint32_t)(n * (K / 32) * 2 + 16 * (lane & 1));
  }
  // bytes from one tile's weights (scales) to the next tile's (whole tiles only)
  const int wtile = packed_layout ? nch * kWBytes : tile_cols<PHASE>() * (K / 2);
  const int stile = packed_layout ? nper * kSBytes : tile_cols<PHASE>() * (K / 16);
  auto load_w = [&](u32x4 (&d)[kNSub], int t, int c) {
    const int so = uniform(t < ntl && c < nch
                               ? t * wtile + (packed_layout ? c * kWBytes : c * kWRowBytes)
                               : (int)kNoRow);
    const int aux = PK ? kPrefillPackedAux : kPrefillAux;
#pragma unroll
    for (int s = 0; s < kNSub; ++s)
      d[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, woff[s], so, aux));
  };
  // the scales of period lp (chunks 4 lp .. 4 lp + 3) of tile t: loaded
  // into registers, then stored to the wave's LDS buffer
  auto load_sc = [&](u32x4 (&r)[2], int t, int lp) {
    const int so = uniform(t < ntl && lp < nper
                               ? t * stile + (packed_layout ? lp * kSBytes : lp * kScRow)
                               : (int)kNoRow);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(sres, scoff[i], so, 0));
  };
  auto store_sc = [&](const u32x4 (&r)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4*>(lds_sc[wave] + i * 1024 + lane * 16) = r[i];
  };

  block_row_exps<PHASE, MS>(p, row0);  // made visible by the first barrier

  f32x4 acc[MS][kNSub];
#pragma unroll
  for (int mi = 0; mi < MS; ++mi)
#pragma unroll
    for (int s = 0; s < kNSub; ++s) acc[mi][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  // activations: row 16 mi + lr, piece 4 lq + j (permuted slot)
  const int aread = lr * (kKC * 2);
  // Four MFMA steps per chunk: the activation fragments are read first, then
  // each sub-tile's weights are dequantised under the previous one's MFMAs.
  // this lane's scales of a period, two bf16 per register: [sub-tile][chunk
  // pair of the period]
  uint32_t scr[kNSub][kSPeriod / 2];
  auto read_sc = [&]() {
    const uint8_t* sbuf = lds_sc[wave] + lr * kScRow + 2 * lq;
#pragma unroll
    for (int s = 0; s < kNSub; ++s)
#pragma unroll
      for (int q = 0; q < kSPeriod; q += 2) {
        const uint32_t lo = *reinterpret_cast<const uint16_t*>(sbuf + 16 * s * kScRow + 8 * q);
        const uint32_t hi = *reinterpret_cast<const uint16_t*>(sbuf + 16 * s * kScRow + 8 * q + 8);
        scr[s][q / 2] = lo | (hi << 16);
      }
  };
  auto compute = [&](const uint8_t* abuf, const u32x4 (&w)[kNSub], int q) {
    GroupScale sc[kNSub];
#pragma unroll
    for (int s = 0; s < kNSub; ++s)
      sc[s] = group_scale((q & 1) ? scr[s][q / 2] >> 16 : scr[s][q / 2] & 0xFFFFu);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h16x8 a[MS];
      const int apc = aread + (((4 * lq + j) ^ aslot(lr)) * 16);
#pragma unroll
      for (int mi = 0; mi < MS; ++mi)
        a[mi] = *reinterpret_cast<const h16x8*>(abuf + mi * 16 * (kKC * 2) + apc);
#pragma unroll
      for (int s = 0; s < kNSub; ++s) {
        const h16x8 b = dequant8(w[s][j], sc[s]);
        if (kPrefillPrio) __builtin_amdgcn_s_setprio(kPrefillPrio);
#pragma unroll
        for (int mi = 0; mi < MS; ++mi)
          acc[mi][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mi], b, acc[mi][s], 0, 0, 0);
        if (kPrefillPrio) __builtin_amdgcn_s_setprio(0);
      }
      if (kPrefillSched == 1) {
        __builtin_amdgcn_sched_group_barrier(0x100, MS, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x002, kDequantFma ? 12 : 13, 0);  // VALU: first sub-tile's weights
#pragma unroll
        for (int i = 0; i < MS * kNSub; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
      } else if (kPrefillSched == 2) {
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // One chunk slot c (ring position q = c % 4): the activation copies of
  // slot c + 3 (into the LDS slot freed by the previous barrier) and, at even
  // positions, the weights of slots c + 2 and c + 3 (into the two register
  // stages of slots c - 2 and c - 1) are issued first, then slot c's MFMAs.
  // Loading a pair of slots' weights together requests both 64-byte halves
  // of each weight row's 128-byte line at once, so the line is fetched once
  // (loaded a slot apart, the second half often found the line evicted).
  // The scales of period p (slots 4p .. 4p + 3) are loaded into registers
  // in slot 4p - 3 (position 1), stored to the wave's LDS buffer in slot
  // 4p - 1 (position 3), after the wave read period p - 1's scales from it in
  // slot 4p - 4 (position 0; a wave's LDS accesses are done in order), and
  // read into registers in slot 4p.
  // Loads issued per position (in this order): 0: weights 2 kNSub,
  // activations kAPW; 1: scales 2, activations; 2: weights 2 kNSub,
  // activations; 3: activations. Before the barrier of slot c, slot c + 1's
  // weights and activations must have landed; the loads issued after the
  // later of the two may stay in flight:
  //   position 0: after slot c + 1's activations (issued at position 2):
  //               kAPW + (2 kNSub + kAPW) = 14
  //   position 1: after its weights (position 0): kNSub + kAPW + 2 + kAPW = 12
  //   position 2: after its activations (position 0): 2 + kAPW + 2 kNSub + kAPW = 16
  //   position 3: after its weights (position 2): kNSub + kAPW + kAPW = 10
  static_assert(kAPW == 3 && kNSub == 4, "wait counts");
  u32x4 sreg[2];  // the next period's scales, between positions 1 and 3
  // The ring position q = c % 4 is a compile-time constant at every call,
  // and so is each activation buffer's identity.
  auto chunk = [&](int t, int c, int q, uint8_t* abuf, uint8_t* aprev,
                   const u32x4 (&wcur)[kNSub], u32x4 (&wn2)[kNSub], u32x4 (&wn3)[kNSub]) {
    auto next = [&](int d, int& tt, int& cc) {  // slot c + d as (tile, slot)
      const int cd = c + d;
      tt = cd < nkp ? t : t + 1;
      cc = cd < nkp ? cd : cd - nkp;
    };
    int t2, c2, t3, c3;
    next(2, t2, c2);
    next(3, t3, c3);
    if (q == 0) read_sc();
    __builtin_amdgcn_sched_barrier(0);
    if (q == 1) load_sc(sreg, t3, c3 / kSPeriod);
    if ((q & 1) == 0) {
      load_w(wn2, t2, c2);
      load_w(wn3, t3, c3);
    }
    copy_a(aprev, t3, c3);
    __builtin_amdgcn_sched_barrier(0);
    if (c < nch) compute(abuf, wcur, q);
    if (q == 3) store_sc(sreg);
    if (q == 0) wait_vm<14>();
    else if (q == 1) wait_vm<12>();
    else if (q == 2) wait_vm<16>();
    else wait_vm<10>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
  };

  // ---- pipeline -------------------------------------------------------------
  // slots 0, 1, 2 (and the first scale period) in flight, slot 0 landed
  u32x4 w0[kNSub], w1[kNSub], w2[kNSub], w3[kNSub];
  // slot 0's and 1's weights, slots 0, 1 and 2's activations in flight, slot
  // 0's landed (slots 1 and 2's activations may stay in flight)
  load_sc(sreg, 0, 0);
  load_w(w0, 0, 0);
  load_w(w1, 0, 1);
  copy_a(lds_a0, 0, 0);
  copy_a(lds_a1, 0, 1);
  copy_a(lds_a2, 0, 2);
  store_sc(sreg);
  wait_vm<2 * kAPW>();
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  // the ring's four positions in turn (whole rounds per tile); with several
  // tiles the copy stream runs on from one tile into the next and the
  // accumulators restart at zero for each tile
  for (int t = 0; t < ntl; ++t) {
    for (int c = 0; c < nkp; c += kRing) {
      chunk(t, c, 0, lds_a0, lds_a3, w0, w2, w3);
      chunk(t, c + 1, 1, lds_a1, lds_a0, w1, w2, w3);  // (no weight loads)
      chunk(t, c + 2, 2, lds_a2, lds_a1, w2, w0, w1);
      chunk(t, c + 3, 3, lds_a3, lds_a2, w3, w0, w1);  // (no weight loads)
    }
    block_epilogue<PHASE, MS, false>(p, acc, row0, tile + t);
    if (!MT) break;
#pragma unroll
    for (int mi = 0; mi < MS; ++mi)
#pragma unroll
      for (int s = 0; s < kNSub; ++s) acc[mi][s] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// ---- routed int4 blocks, weights through LDS ---------------------------------------
// The checkpoint layout's weight rows are 4096 bytes apart, and a chunk takes
// 64 bytes of each: loaded straight into MFMA registers (16 rows per load)
// that is half of each 128-byte line per load, a load shape that runs at a
// quarter of the whole-line rate, and the line's other half is often fetched
// again a chunk later. This form stages the weights through LDS in stages of
// 256 inputs, one whole 128-byte line per row: each wave copies its own 64
// rows (8 copies of 8 rows x 128 bytes, LDS destination, the 16-byte piece
// P ^ sswz(r) of row r into slot P as in the shared-expert tiles) into its
// own 8 KB of lds_a0, and at the start of the stage reads its fragments
// (lane (lr, lq) of sub-tile s: groups lq and lq + 4 of row 16 s + lr, 16
// bytes each) into registers before it copies the next stage into the same
// place; no other wave reads them, so they need no barrier. The stage's two
// 128-input chunks run as before: chunk h takes group lq + 4 h of each lane,
// MFMA step j word j of it. The activations take the three other LDS
// buffers, a ring of three chunks (each copied two chunks ahead); the scales
// of a stage (8 groups of each of the wave's rows, 16 bytes) are loaded into
// registers one stage ahead, stored to the wave's LDS area with groups q and
// q + 4 in word q, and read back at the stage's start. One barrier per chunk.
template <int PHASE, int MS>
__device__ __forceinline__ void block_tile_w(const GemmParams& p, int mblk, int tile) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int lr = lane & 15;
  const int lq = lane >> 4;
  const int K = p.K;
  const int nch = K / kKC;        // 128-input chunks
  const int nst = (nch + 1) / 2;  // 256-input weight stages (an odd chunk count
                                  // leaves the last stage's second half unused)
  const int64_t row0 = (int64_t)mblk * kBM;
  const int e = p.block_expert[mblk];
  const int Nw = (PHASE == kGateUp) ? 2 * p.I : p.N;
  const int64_t wbase = (int64_t)e * Nw;

  const __amdgpu_buffer_rsrc_t ares = block_act_rsrc<PHASE>(p);
  uint32_t aoff[kAPW];
  block_act_offsets<PHASE, MS>(p, row0, aoff);
  // chunk c; past the chunks, offsets past any buffer (zeros; issued all the
  // same, so that every chunk waits on the same number of loads)
  auto copy_a = [&](uint8_t* dst, int c) {
    const int so = uniform(c < nch ? c * kKC * 2 : (int)kNoRow);
#pragma unroll
    for (int i = 0; i < kAPW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ares, (lds_ptr)(dst + (kAPW * wave + i) * 1024), 16,
                                               aoff[i], so, 0, 0);
  };

  // weights: copy i covers the wave's rows 8 i .. 8 i + 7 (lane / 8), lane
  // % 8 the slot
  constexpr int kWRow = 2 * kKC / 2;  // bytes of a row per stage: 128
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.packed + wbase * (K / 8)), 0, Nw * (K / 8) * 4, kBufferFlags);
  // The weight row of the wave's row 8 i + r is n0 + 8 i + r, except that
  // gate_up's rows 32..63 (the up sub-tiles) continue at I + n0: a lane
  // offset (row r, its slot's piece; the swizzle of row 8 i + r is that of
  // row 8 (i % 2) + r) and a uniform offset per copy. Widths are multiples of
  // 128, so a wave's 64 rows are all inside the width or all past it.
  const int n0 = weight_row<PHASE>(p, tile, wave * 64);
  uint32_t wlane[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * i + (lane >> 3);
    wlane[i] = n0 < 0 ? kNoRow
                      : (uint32_t)((n0 + (lane >> 3)) * (K / 2) + 16 * ((lane & 7) ^ sswz(r)));
  }
  const int wup = PHASE == kGateUp ? (p.I - 32) * (K / 2) : 0;
  uint8_t* const wbuf = lds_a0 + wave * (64 * kWRow);
  auto copy_w = [&](int st, int i) {  // copy i (rows 8 i ..) of stage st
    const int so = uniform(st < nst ? st * kWRow + 8 * i * (K / 2) + (i >= 4 ? wup : 0) : (int)kNoRow);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, (lds_ptr)(wbuf + i * 1024), 16, wlane[i & 1], so,
                                             0, kWLdsAux);
  };
  // scales: lane l loads the 16 bytes (8 groups) of the wave's row l
  const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.scales + wbase * (K / 32)), 0, Nw * (K / 32) * 2, kBufferFlags);
  const int nsc = weight_row<PHASE>(p, tile, wave * 64 + lane);
  const uint32_t scoff = nsc < 0 ? kNoRow : (uint32_t)(nsc * (K / 16));
  auto load_sc = [&](int st) {
    const int so = uniform(st < nst ? st * 16 : (int)kNoRow);
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(sres, scoff, so, 0));
  };
  uint8_t* const scbuf = lds_sc[wave];
  auto store_sc = [&](const u32x4 v) {
    // word q: groups q (low half) and q + 4 (high half)
    const u32x4 o = {(v[0] & 0xFFFFu) | (v[2] << 16), (v[0] >> 16) | (v[2] & 0xFFFF0000u),
                     (v[1] & 0xFFFFu) | (v[3] << 16), (v[1] >> 16) | (v[3] & 0xFFFF0000u)};
    *reinterpret_cast<u32x4*>(scbuf + lane * 16) = o;
  };

  f32x4 acc[MS][kNSub];
#pragma unroll
  for (int mi = 0; mi < MS; ++mi)
#pragma unroll
    for (int s = 0; s < kNSub; ++s) acc[mi][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int aread = lr * (kKC * 2);
  const int wrd = lr * kWRow;
  const int pw0 = 16 * ((0 + lq) ^ sswz(lr));  // sswz(16 s + lr) == sswz(lr)
  const int pw1 = 16 * ((4 + lq) ^ sswz(lr));
  u32x4 w[2][kNSub];     // the stage's weight fragments: [chunk][sub-tile]
  uint32_t scr[kNSub];   // the stage's scales: groups lq, lq + 4 of each sub-tile row
  u32x4 sreg;            // the next stage's scales, in flight
  auto read_stage = [&]() {
#pragma unroll
    for (int s = 0; s < kNSub; ++s) {
      w[0][s] = *reinterpret_cast<const u32x4*>(wbuf + s * 16 * kWRow + wrd + pw0);
      w[1][s] = *reinterpret_cast<const u32x4*>(wbuf + s * 16 * kWRow + wrd + pw1);
      scr[s] = *reinterpret_cast<const uint32_t*>(scbuf + (16 * s + lr) * 16 + 4 * lq);
    }
  };
  // issue(j) runs before MFMA step j (the copies spread over the chunk)
  auto compute = [&](const uint8_t* abuf, int h, auto&& issue) {
    GroupScale sc[kNSub];
#pragma unroll
    for (int s = 0; s < kNSub; ++s) sc[s] = group_scale(h ? scr[s] >> 16 : scr[s] & 0xFFFFu);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // the two waves of a SIMD share its issue slots, and the older one
      // wins ties: with one priority the younger one falls behind and the
      // older one then idles at the chunk's barrier; a priority that drops
      // with each step lets the wave that is behind catch up
      if (kStepPrio) {
        if (j == 0) __builtin_amdgcn_s_setprio(3);
        else if (j == 1) __builtin_amdgcn_s_setprio(2);
        else if (j == 2) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      }
      issue(j);
      __builtin_amdgcn_sched_barrier(0);
      // activation fragments: row 16 mi + lr, piece 4 lq + j
      h16x8 a[MS];
      const int apc = aread + (((4 * lq + j) ^ aslot(lr)) * 16);
#pragma unroll
      for (int mi = 0; mi < MS; ++mi)
        a[mi] = *reinterpret_cast<const h16x8*>(abuf + mi * 16 * (kKC * 2) + apc);
#pragma unroll
      for (int s = 0; s < kNSub; ++s) {
        const h16x8 b = dequant8(w[h][s][j], sc[s]);
#pragma unroll
        for (int mi = 0; mi < MS; ++mi)
          acc[mi][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mi], b, acc[mi][s], 0, 0, 0);
      }
      if (kWLdsSched == 1) {
        __builtin_amdgcn_sched_group_barrier(0x100, MS, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x002, kDequantFma ? 12 : 13, 0);  // VALU: first sub-tile's weights
#pragma unroll
        for (int i = 0; i < MS * kNSub; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
      } else if (kWLdsSched == 2) {
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Chunk c = 2 n + h of stage n, its activations in abuf, chunk c + 2's
  // copied into anext (freed by the previous barrier). The copies are spread
  // over the chunk's four MFMA steps: issued all at once, the eight waves'
  // copies fill the compute unit's vector-memory queue and every wave stalls
  // on issue while its MFMAs wait. Loads issued per chunk, in this order:
  // before step 0 chunk c + 2's activations (kAPW); for h = 0 then the
  // weights of stage n + 1, two copies before each step, and the scales of
  // stage n + 1 (1) before step 3. Before the barrier, chunk c + 1's
  // activations (and for h = 1 the next stage's weights and scales, issued
  // after them in chunk c - 1) must have landed; the loads issued after them
  // may stay in flight: h = 0: kAPW + 8 + 1 = 12; h = 1: kAPW = 3.
  static_assert(kAPW == 3, "wait counts");
  auto chunk = [&](int c, int h, const uint8_t* abuf, uint8_t* anext) {
    const int n = c >> 1;
    if (h == 0) {
      read_stage();
      wait_lgkm0();  // the fragments are in registers before the copies overwrite them
      __builtin_amdgcn_sched_barrier(0);
    }
    auto issue = [&](int j) {
      if (j == 0) copy_a(anext, c + 2);
      if (h == 0) {
        copy_w(n + 1, 2 * j);
        copy_w(n + 1, 2 * j + 1);
        if (j == 3) sreg = load_sc(n + 1);
      }
    };
    if (c < nch) {
      compute(abuf, h, issue);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) issue(j);
    }
    if (h == 1) store_sc(sreg);  // after this stage's read_stage (a wave's LDS accesses are in order)
    if (h == 0) wait_vm<12>();
    else wait_vm<3>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
  };

  block_row_exps<PHASE, MS, true>(p, row0);  // made visible by the first barrier
  // stage 0's scales and weights, chunks 0 and 1's activations; chunk 0 and
  // the weights landed before the first barrier
  sreg = load_sc(0);
#pragma unroll
  for (int i = 0; i < 8; ++i) copy_w(0, i);
  copy_a(lds_a1, 0);
  copy_a(lds_a2, 1);
  store_sc(sreg);
  wait_vm<kAPW>();
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  // chunk c sits in buffer c % 3 (lds_a1, lds_a2, lds_a3)
  for (int c = 0;; c += 6) {
    // (already true here; stated so that the compiler's wait insertion, which
    // merges the loop entry with the back edge, knows that only chunk c + 1's
    // copies are in flight and adds no wait before chunk c's reads)
    wait_vm<kAPW>();
    chunk(c, 0, lds_a1, lds_a3);
    chunk(c + 1, 1, lds_a2, lds_a1);
    if (c + 2 >= nch) break;
    chunk(c + 2, 0, lds_a3, lds_a2);
    chunk(c + 3, 1, lds_a1, lds_a3);
    if (c + 4 >= nch) break;
    chunk(c + 4, 0, lds_a2, lds_a1);
    chunk(c + 5, 1, lds_a3, lds_a2);
    if (c + 6 >= nch) break;
  }
  wait_vm<0>();  // the copies past the last chunk (zeros) are done with LDS
  block_epilogue<PHASE, MS, true>(p, acc, row0, tile);
}

// ---- shared-expert tiles (bf16 weights) -----------------------------------------
// A work-group: 96 tokens (t0..) x 512 weight rows of the shared expert's
// gate/up [2I, H] (gate_up; sub-tiles as in the routed blocks) or down [H, I].
// Both operands go through LDS in stages of 64 inputs, one 128-byte line per
// row: the activations (x or the shared h, bf16, 12 KB, two buffers) and the
// weights (64 KB, one buffer; each wave copies and reads only its own 64
// rows). Every copy instruction covers 8 rows x 128 bytes, whole lines: a
// load that takes half of each line it touches runs at a quarter of the
// rate. A lane copies the 16-byte piece p ^ sw(r) of row r into slot p
// (sw(r) = (r >> 1) & 7), so that the fragment reads (16 rows at one piece)
// fall in distinct banks. Per stage: the activation copies of the next stage
// (into the other buffer) after the barrier, the wave's weight fragments,
// then its weight copies of the next stage (they run under the activation
// reads, the MFMAs and the next barrier), the activation fragments, the MFMAs.

template <int PHASE, int MS>
__device__ __forceinline__ void shared_tile(const GemmParams& p, int64_t t0, int tile) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int lr = lane & 15;
  const int lq = lane >> 4;
  const int K = p.K;
  const int nst = K / kSKC;  // even: K is a multiple of 128
  const int Nw = (PHASE == kGateUp) ? 2 * p.I : p.N;

  // activations: copy i (rows 8 i ..) by wave i % 8
  constexpr int kACopies = 2 * MS;
  constexpr int kAPerWave = (kACopies + kWaves - 1) / kWaves;
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.a_shared, 0, (int)(p.T * K * 2), kBufferFlags);
  uint32_t aoff[kAPerWave];
#pragma unroll
  for (int u = 0; u < kAPerWave; ++u) {
    const int i = wave + kWaves * u;
    const int row = 8 * i + (lane >> 3);
    const int64_t tok = t0 + row;
    aoff[u] = (i < kACopies && tok < p.T)
                  ? (uint32_t)((tok * K + 8 * ((lane & 7) ^ sswz(row))) * 2)
                  : kNoRow;
  }
  // weights: the wave's 64 rows, copy i covers rows 8 i ..
  const __amdgpu_buffer_rsrc_t wres =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.wshared, 0, Nw * K * 2, kBufferFlags);
  uint32_t woff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 8 * i + (lane >> 3);
    const int n = weight_row<PHASE>(p, tile, wave * 64 + row);
    woff[i] = n < 0 ? kNoRow : (uint32_t)((n * K + 8 * ((lane & 7) ^ sswz(row))) * 2);
  }
  static_assert(kABytes >= kSBM * kSRow, "activation stage");
  uint8_t* const wbuf = lds_a0 + wave * (64 * kSRow);
  auto copy_a = [&](uint8_t* abuf, int st) {
    const int so = uniform(st * kSRow);
#pragma unroll
    for (int u = 0; u < kAPerWave; ++u) {
      const int i = wave + kWaves * u;
      if (kACopies % kWaves == 0 || i < kACopies)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ares, (lds_ptr)(abuf + i * 1024), 16, aoff[u], so,
                                                 0, 0);
    }
  };
  auto copy_w = [&](int st) {
    const int so = uniform(st * kSRow);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, (lds_ptr)(wbuf + i * 1024), 16, woff[i], so, 0,
                                               0);
  };

  f32x4 acc[MS][kNSub];
#pragma unroll
  for (int mi = 0; mi < MS; ++mi)
#pragma unroll
    for (int s = 0; s < kNSub; ++s) acc[mi][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment of step j (inputs 32 j + 8 lq .. + 8 of the stage), row lr of
  // a 16-row sub-tile
  const int rbase = lr * kSRow;
  const int pc0 = 16 * ((0 + lq) ^ sswz(lr));
  const int pc1 = 16 * ((4 + lq) ^ sswz(lr));

  auto stage = [&](int st, const uint8_t* acur, uint8_t* anext) {
    wait_vm<0>();
    __builtin_amdgcn_s_barrier();  // the stage's copies landed; the other
                                   // activation buffer's reads are done
    __builtin_amdgcn_sched_barrier(0);
    if (st + 1 < nst) copy_a(anext, st + 1);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 a[2][MS], b[2][kNSub];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int s = 0; s < kNSub; ++s)
        b[j][s] = *reinterpret_cast<const bf16x8*>(wbuf + s * 16 * kSRow + rbase + (j ? pc1 : pc0));
    wait_lgkm0();
    __builtin_amdgcn_sched_barrier(0);
    if (st + 1 < nst) copy_w(st + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int mi = 0; mi < MS; ++mi)
        a[j][mi] = *reinterpret_cast<const bf16x8*>(acur + mi * 16 * kSRow + rbase + (j ? pc1 : pc0));
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int mi = 0; mi < MS; ++mi)
#pragma unroll
        for (int s = 0; s < kNSub; ++s)
          acc[mi][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j][mi], b[j][s], acc[mi][s], 0, 0,
                                                               0);
  };
  copy_a(lds_a1, 0);
  copy_w(0);
  for (int st = 0; st < nst; st += 2) {
    stage(st, lds_a1, lds_a2);
    stage(st + 1, lds_a2, lds_a1);
  }
  wait_lgkm0();

  // epilogue: lane holds rows 4 lq + i of each sub-tile, column lr
  if (PHASE == kGateUp) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int col = tile * (kBN / 2) + wave * 32 + 16 * s + lr;
      if (col >= p.I) continue;
#pragma unroll
      for (int mi = 0; mi < MS; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t tok = t0 + mi * 16 + 4 * lq + i;
          if (tok >= p.T) continue;
          const float hv = silu_mul(acc[mi][s][i], acc[mi][s + 2][i]);
          p.h_shared[tok * p.I + col] = (uint16_t)(pack_bf16x2(hv, 0.f) & 0xFFFFu);
        }
    }
  } else {
#pragma unroll
    for (int mi = 0; mi < MS; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t tok = t0 + mi * 16 + 4 * lq + i;
        if (tok >= p.T) continue;
        float* dst = p.y_shared + tok * p.N;
#pragma unroll
        for (int s = 0; s < kNSub; ++s) {
          const int col = tile * kBN + wave * 64 + 16 * s + lr;
          if (col < p.N) dst[col] = acc[mi][s][i];
        }
      }
  }
}

// Work-groups: all column tiles of block b run on XCD b % 8. Work-groups are
// dispatched round-robin over the 8 XCDs in id order, so the s-th work-group
// that XCD x receives (id 8 s + x) takes tile s % n_tiles of block
// 8 (s / n_tiles) + x: a block's activations are fetched into one XCD's L2 and
// shared by its tiles there, and the blocks past the last bucket (which exit
// at once) are spread evenly over the XCDs. The grid holds a multiple of 8
// blocks.
constexpr int kXcds = 8;

// The block's rows, rounded up to whole 16-row sub-tiles, select the K loop.
template <int PHASE, bool PK, bool MT>
__device__ __forceinline__ void run_block(const GemmParams& p, int mblk, int tile, int ntl) {
  // bucket rows of the block (padding sits at its end), in 16-row sub-tiles
  const int64_t row0 = (int64_t)mblk * kBM;
  const int lane = threadIdx.x & 63;
  int n_valid = 0;
#pragma unroll
  for (int h = 0; h < (kBM + 63) / 64; ++h) {
    const int r = 64 * h + lane;
    n_valid += __popcll(__ballot(r < kBM && p.sorted_ids[row0 + r] < p.P));
  }
  const int msub = uniform((n_valid + 15) >> 4);
  if constexpr (kWeightsLds && !PK && !MT) {
    if (kOddSubtiles && kMaxMS == 6 && msub == 3) block_tile_w<PHASE, 3>(p, mblk, tile);
    else if (kOddSubtiles && kMaxMS == 6 && msub == 5) block_tile_w<PHASE, 5>(p, mblk, tile);
    else if (kOneSubtile && msub <= 1) block_tile_w<PHASE, 1>(p, mblk, tile);
    else if (msub <= 2) block_tile_w<PHASE, 2>(p, mblk, tile);
    else if (msub <= 4 || kMaxMS < 6) block_tile_w<PHASE, (kMaxMS < 4 ? kMaxMS : 4)>(p, mblk, tile);
    else if (msub <= 6 || kMaxMS < 8) block_tile_w<PHASE, (kMaxMS < 6 ? kMaxMS : 6)>(p, mblk, tile);
    else block_tile_w<PHASE, kMaxMS>(p, mblk, tile);
    return;
  }
  if (kOddSubtiles && kMaxMS == 6 && (msub == 3 || msub == 5)) {
    if (msub == 3) block_tile<PHASE, 3, PK, MT>(p, mblk, tile, ntl);
    else block_tile<PHASE, 5, PK, MT>(p, mblk, tile, ntl);
    return;
  }
  if (kOneSubtile && msub <= 1) block_tile<PHASE, 1, PK, MT>(p, mblk, tile, ntl);
  else if (msub <= 2) block_tile<PHASE, 2, PK, MT>(p, mblk, tile, ntl);
  else if (msub <= 4 || kMaxMS < 6) block_tile<PHASE, (kMaxMS < 4 ? kMaxMS : 4), PK, MT>(p, mblk, tile, ntl);
  else if (msub <= 6 || kMaxMS < 8) block_tile<PHASE, (kMaxMS < 6 ? kMaxMS : 6), PK, MT>(p, mblk, tile, ntl);
  else block_tile<PHASE, kMaxMS, PK, MT>(p, mblk, tile, ntl);
}

// The shared expert's work-groups: tile s % n_tiles of token block s / n_tiles
// (consecutive work-groups share a token block, as the routed ones share a
// bucket block).
template <int PHASE>
__device__ __forceinline__ void run_shared(const GemmParams& p, int sid, int n_tiles) {
  const int tb = sid / n_tiles;
  const int tile = sid - tb * n_tiles;
  const int64_t t0 = (int64_t)tb * kSBM;
  const int64_t rows = p.T - t0 < kSBM ? p.T - t0 : kSBM;
  if (rows <= 32) shared_tile<PHASE, 2>(p, t0, tile);
  else if (rows <= 64) shared_tile<PHASE, 4>(p, t0, tile);
  else if (rows <= 96 || kSBM <= 96) shared_tile<PHASE, 6>(p, t0, tile);
  else shared_tile<PHASE, kSBM / 16>(p, t0, tile);
}

// Shared-expert work-groups first (ids below n_shared), then one per
// (block, column tile). PK: the weights are in the prepacked layout (a
// separate instance, so that traces tell the two apart).
template <int PHASE, bool PK>
__global__ __launch_bounds__(kThreads, 1) void prefill_gemm_kernel(GemmParams p, int n_shared) {
  const int n_tiles = (p.N + tile_cols<PHASE>() - 1) / tile_cols<PHASE>();
  if ((int)blockIdx.x < n_shared) {
    run_shared<PHASE>(p, blockIdx.x, n_tiles);
    return;
  }
  const int id = blockIdx.x - n_shared;
  const int x = id % kXcds;
  const int sx = id / kXcds;
  const int mblk = (sx / n_tiles) * kXcds + x;
  const int tile = sx - (sx / n_tiles) * n_tiles;
  if (mblk >= p.max_blocks || (int64_t)mblk * kBM >= *p.n_padded) return;
  run_block<PHASE, PK, false>(p, mblk, tile, 1);
}

// Short K (a few chunks per tile, e.g. the down projection of one GPU's share
// of a tensor-parallel layer): a work-group takes up to tpw_max consecutive
// column tiles of its block, and its copy stream runs on from one tile into
// the next, so that each tile no longer starts with an empty pipeline and
// ends with its stores alone. The grid holds one work-group per (block, tile);
// the tiles per work-group are chosen from the real block count (the grid's
// is an upper bound), as many as still leave six work-groups per CU, and the
// work-groups past the last group exit at once. Whole tiles and an even chunk
// count only.
template <int PHASE, bool PK>
__global__ __launch_bounds__(kThreads, 1) void prefill_tiles_kernel(GemmParams p, int n_shared,
                                                                   int tpw_max) {
  const int n_tiles = p.N / tile_cols<PHASE>();
  if ((int)blockIdx.x < n_shared) {
    run_shared<PHASE>(p, blockIdx.x, n_tiles);
    return;
  }
  const int id = blockIdx.x - n_shared;
  const int64_t nblk = *p.n_padded / kBM;
  int tpw = 1;
  for (int c = tpw_max; c > 1; c >>= 1)
    if (nblk * ((n_tiles + c - 1) / c) >= 6 * 256) {
      tpw = c;
      break;
    }
  const int ngrp = (n_tiles + tpw - 1) / tpw;  // groups of tpw consecutive tiles
  const int x = id % kXcds;
  const int sx = id / kXcds;
  const int mblk = (sx / ngrp) * kXcds + x;
  const int tile = (sx - (sx / ngrp) * ngrp) * tpw;
  if (mblk >= p.max_blocks || (int64_t)mblk * kBM >= *p.n_padded) return;
  run_block<PHASE, PK, true>(p, mblk, tile, min(tpw, n_tiles - tile));
}

template <int PHASE>
hipError_t launch(const GemmParams& p, hipStream_t stream) {
  if (p.K % kKC != 0) return hipErrorInvalidValue;
  // buffer resources hold 32-bit byte sizes
  const int64_t arows = PHASE == kGateUp ? p.T : (int64_t)p.max_blocks * kBM;
  const int64_t nw = PHASE == kGateUp ? 2 * (int64_t)p.I : p.N;
  if (arows * p.K * 2 > 0x7fffffff || nw * p.K * 2 > 0x7fffffff || p.T * p.K * 2 > 0x7fffffff)
    return hipErrorInvalidValue;
  const int64_t blocks = ((int64_t)p.max_blocks + kXcds - 1) / kXcds * kXcds;
  const int n_tiles = (p.N + tile_cols<PHASE>() - 1) / tile_cols<PHASE>();
  const int nch = p.K / kKC;
  const int64_t n_shared64 = p.wshared ? (p.T + kSBM - 1) / kSBM * n_tiles : 0;
  // several tiles per work-group only where a tile is a few chunks long
  // (at most 16 chunks per work-group, at most four tiles), over whole tiles
  // and an even chunk count
  int tpw = 1;
  if (p.N % tile_cols<PHASE>() == 0 && nch % 2 == 0)
    while (2 * tpw * nch <= 16 && 2 * tpw <= 4) tpw *= 2;
  const int64_t grid = n_shared64 + blocks * n_tiles;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  GemmParams args = p;
  int n_shared = (int)n_shared64;
  if (tpw == 1) {
    void* kargs[] = {&args, &n_shared};
    const void* fn = p.prepacked
                         ? reinterpret_cast<const void*>(&prefill_gemm_kernel<PHASE, true>)
                         : reinterpret_cast<const void*>(&prefill_gemm_kernel<PHASE, false>);
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kThreads), kargs, 0, stream);
  }
  void* kargs[] = {&args, &n_shared, &tpw};
  const void* fn = p.prepacked
                       ? reinterpret_cast<const void*>(&prefill_tiles_kernel<PHASE, true>)
                       : reinterpret_cast<const void*>(&prefill_tiles_kernel<PHASE, false>);
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kThreads), kargs, 0, stream);
}

}  // namespace

int32_t prefill_block_m() { return kBM; }

bool prefill_fits(int32_t hidden, int32_t inter) {
  return inter % tile_cols<kGateUp>() == 0 && hidden % tile_cols<kDown>() == 0 &&
         hidden % kKC == 0 && inter % kKC == 0;
}

hipError_t launch_x16(const uint16_t* x, uint16_t* x16, int32_t* kx, int64_t T, int32_t H,
                      hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (H % 8 || T > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(x16_kernel, dim3((unsigned)T), dim3(kConvThreads), 0, stream, x, x16, kx, H);
  return hipGetLastError();
}

hipError_t launch_h_rescale(uint16_t* h, const int32_t* kh, int32_t* kr, const int32_t* n_padded,
                            int64_t rows, int32_t I, int32_t n_htiles, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (I % 8 || rows > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(h_rescale_kernel, dim3((unsigned)rows), dim3(kConvThreads), 0, stream, h, kh,
                     kr, n_padded, I, n_htiles);
  return hipGetLastError();
}

hipError_t launch_gate_up_prefill(const GemmParams& p, hipStream_t stream) {
  return launch<kGateUp>(p, stream);
}

hipError_t launch_down_prefill(const GemmParams& p, hipStream_t stream) {
  return launch<kDown>(p, stream);
}

}  // namespace moe
