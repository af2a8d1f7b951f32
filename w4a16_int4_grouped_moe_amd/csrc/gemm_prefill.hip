// gemm_prefill.hip -- grouped W4A16 GEMMs for many rows per expert (gfx950):
// the int4 routed experts of prefill-sized batches, 96-row bucket blocks.
//
// Same two launches as the other GEMM paths (gate_up with the SwiGLU epilogue,
// then down), for blocks of 96 bucketed rows of one expert. Here the layer is
// a dense contraction per expert (about 85 rows each for 4096 tokens, top-8 of
// 384), so the kernel is built around keeping the MFMA pipes fed: every
// dequantised weight serves all rows of the block, and all operands arrive
// through LDS without holding registers while in flight.
//
// Work-group (512 threads = 8 waves): one block of up to kBM bucketed rows x
// 512 weight rows (a column tile; where K is only a few chunks, several
// consecutive tiles of the block in turn, prefill_tiles_kernel). Every wave owns four 16-row weight sub-tiles (gate_up: two
// gate sub-tiles and the two matching up sub-tiles) and computes them for all
// of the block's rows, so each weight is dequantised exactly once per block.
// K advances in chunks of 128 inputs (four 32-input groups). All operands reach
// LDS through 16-byte buffer loads with an LDS destination (no registers held
// while in flight), so registers hold only accumulators and the fragments of
// one MFMA step:
//  * activations: the kBM x 128 chunk, double buffered; a row's 16 pieces of 16
//    bytes are permuted, piece c of row r at slot c ^ f(r & 15) where f swaps
//    the two 2-bit halves of its argument, so that the fragment reads (16 rows
//    at one k offset per 16 lanes) are free of bank conflicts;
//  * weights: the 512 rows x 64 bytes (four groups of 32 codes) of the chunk,
//    double buffered, the four groups of row r permuted by (r >> 1) & 3 for the
//    same reason; lane (r = lane % 16, q = lane / 16) of a wave reads group q of
//    row r of each of its sub-tiles;
//    (both permutations measured free of bank conflicts on gfx950 16-byte LDS
//    reads, where the simpler XOR forms are not)
//  * scales: 16 groups (4 chunks) of each of the 512 rows, two buffers that
//    alternate every 4 chunks;
//  * the words are dequantised to bf16 (u - 8) * s and fed to
//    v_mfma_f32_16x16x32_bf16: MFMA step j of a chunk takes word j of every
//    lane, so its 32-long reduction covers one 8-input slice of each of the
//    four groups; the matching activations are read at those offsets. The
//    next step's dequantisation (VALU) is interleaved with this step's MFMAs.
// One barrier per chunk: the copies of chunk c + 1 are issued during the first
// MFMA step of chunk c and waited for after it. Barriers are raw s_barrier with explicit
// waits (the fence of __syncthreads() would also wait for the copies just
// issued). The number of 16-row sub-tiles holding bucket rows (even, after
// rounding up) is a template parameter of the K loop, so the loop body is
// straight-line code.
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
constexpr int kPrefillPackedAux = 2;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
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
constexpr uint32_t kNoRow = 0x80000000u;   // offset past any buffer: loads 0

enum { kGateUp = 0, kDown = 1 };

__shared__ __attribute__((aligned(1024))) uint8_t lds_a0[kABytes];
__shared__ __attribute__((aligned(1024))) uint8_t lds_a1[kABytes];
__shared__ __attribute__((aligned(1024))) uint8_t lds_w0[kWBytes];
__shared__ __attribute__((aligned(1024))) uint8_t lds_w1[kWBytes];
__shared__ __attribute__((aligned(1024))) uint8_t lds_s0[kSBytes];
__shared__ __attribute__((aligned(1024))) uint8_t lds_s1[kSBytes];

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

// Per-group dequantisation constants: the scale s, -1032 s, s / 16 and -72 s.
struct GroupScale {
  float s, c1032, s16, c72;
};
__device__ __forceinline__ GroupScale group_scale(float s) {
  return GroupScale{s, -1032.0f * s, 0.0625f * s, -72.0f * s};
}

// The eight codes of one word -> eight bf16 weights (u - 8) * s in input order.
// A field in bits 0-3 of a 16-bit half OR-ed into the fp16 pattern 0x6400 is
// exactly the fp16 value 1024 + u, a field in bits 4-7 gives 1024 + 16 u, so
// the word's low byte pair (fields 0, 4 and 1, 5) needs no shift and its high
// byte pair (fields 2, 6 and 3, 7) one shift by 8: one shift and four
// v_bitop3 per word. One mixed fp16/fp32 FMA per code, fma(1024 + u, s,
// -1032 s) or fma(1024 + 16 u, s / 16, -72 s), gives (u - 8) * s exactly in
// fp32 (the products have at most 19 significant bits, and s / 16, 1032 s and
// 72 s are exact), which is rounded once to bf16.
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, const GroupScale& g) {
  const uint32_t w8 = w >> 8;
  const h16x2 h0 = __builtin_bit_cast(h16x2, and_or(w, 0x000F000Fu, 0x64006400u));   // u0, u4
  const h16x2 h1 = __builtin_bit_cast(h16x2, and_or(w, 0x00F000F0u, 0x64006400u));   // u1, u5
  const h16x2 h2 = __builtin_bit_cast(h16x2, and_or(w8, 0x000F000Fu, 0x64006400u));  // u2, u6
  const h16x2 h3 = __builtin_bit_cast(h16x2, and_or(w8, 0x00F000F0u, 0x64006400u));  // u3, u7
  const f32x2 v0 = {fmaf((float)h0[0], g.s, g.c1032), fmaf((float)h0[1], g.s, g.c1032)};
  const f32x2 v1 = {fmaf((float)h1[0], g.s16, g.c72), fmaf((float)h1[1], g.s16, g.c72)};
  const f32x2 v2 = {fmaf((float)h2[0], g.s, g.c1032), fmaf((float)h2[1], g.s, g.c1032)};
  const f32x2 v3 = {fmaf((float)h3[0], g.s16, g.c72), fmaf((float)h3[1], g.s16, g.c72)};
  u32x4 r;
  r[0] = pack_bf16x2(v0[0], v1[0]);
  r[1] = pack_bf16x2(v2[0], v3[0]);
  r[2] = pack_bf16x2(v0[1], v1[1]);
  r[3] = pack_bf16x2(v2[1], v3[1]);
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// s_waitcnt with only the vector-memory counter limited (lgkm and exp left
// unconstrained), and with both vector-memory and LDS counters at zero.
template <int N>
__device__ __forceinline__ void wait_vm() {
  // gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  static_assert(N >= 0 && N < 16, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

template <int PHASE>
constexpr int tile_cols() { return PHASE == kGateUp ? kBN / 2 : kBN; }

// Permutations of 16-byte pieces in LDS: the four groups of weight row R, the
// sixteen pieces of activation row r.
__device__ __forceinline__ int wslot(int R) { return (R >> 1) & 3; }
__device__ __forceinline__ int aslot(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Weight row of work-group row R = 64 wave + 16 sub-tile + r.
template <int PHASE>
__device__ __forceinline__ int weight_row(const GemmParams& p, int tile, int R) {
  const int w = R >> 6, s = (R >> 4) & 3, r = R & 15;
  if (PHASE == kGateUp) {
    const int c = tile * (kBN / 2) + w * 32 + 16 * (s & 1) + r;
    return s < 2 ? c : p.I + c;  // gate rows, then the matching up rows
  }
  return tile * kBN + w * 64 + 16 * s + r;
}

// MT: the work-group computes ntl consecutive column tiles of the block
// (otherwise exactly one: ntl is then the constant 1)
template <int PHASE, int MS, bool PK, bool MT>
__device__ __forceinline__ void block_tile(const GemmParams& p, int mblk, int tile, int ntl_arg) {
  const int ntl = MT ? ntl_arg : 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int lr = lane & 15;
  const int lq = lane >> 4;
  const int K = p.K;
  const int nch = K / kKC;
  const int64_t row0 = (int64_t)mblk * kBM;
  const int e = p.block_expert[mblk];
  const int Nw = (PHASE == kGateUp) ? 2 * p.I : p.N;
  const int64_t wbase = (int64_t)e * Nw;

  // ---- activation copies: instruction t covers LDS rows 4t..4t+3 ------------
  constexpr int kACopies = kBM / 4;                        // per work-group
  constexpr int kAPerWave = (kACopies + kWaves - 1) / kWaves;
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.a_routed, 0,
      (int)((PHASE == kGateUp ? p.T : (int64_t)p.max_blocks * kBM) * K * 2), kBufferFlags);
  uint32_t aoff[kAPerWave];
#pragma unroll
  for (int i = 0; i < kAPerWave; ++i) {
    const int t = kAPerWave * wave + i;
    const int row = 4 * t + (lane >> 4);
    const int piece = (lane & 15) ^ aslot(row & 15);
    int64_t src = -1;
    if (t < kACopies && row < MS * 16) {
      if (PHASE == kGateUp) {
        const int32_t pair = p.sorted_ids[row0 + row];
        if (pair < p.P) src = pair / p.k;
      } else {
        src = row0 + row;
      }
    }
    aoff[i] = src < 0 ? kNoRow : (uint32_t)((src * K + piece * 8) * 2);
  }
  // copies are addressed by (tile t of the work-group's tiles, chunk c of it);
  // past the last tile an offset beyond any buffer (loads zeros)
  auto copy_a = [&](uint8_t* dst, int t, int c) {
    const int so = uniform(t < ntl ? c * kKC * 2 : (int)kNoRow);
#pragma unroll
    for (int i = 0; i < kAPerWave; ++i) {
      const int t = kAPerWave * wave + i;
      if (kACopies % kWaves == 0 || t < kACopies)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ares, (lds_ptr)(dst + t * 1024), 16, aoff[i], so, 0, 0);
    }
  };

  // ---- weight copies: instruction u covers rows 16u..16u+15 (64 B each) ------
  // Checkpoint layout: row R's 64 bytes of chunk ch at ch * 64 in its row of
  // K / 2 bytes. Prepacked layout: the tile's chunk is one 32 KB run (rows of
  // 64 bytes), so an instruction reads 1 KB of whole lines.
  constexpr bool packed_layout = PK;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.packed + wbase * (K / 8)), 0, Nw * (K / 8) * 4, kBufferFlags);
  uint32_t woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int R = 16 * (4 * wave + i) + (lane >> 2);
    const int g = (lane & 3) ^ wslot(R);
    woff[i] = packed_layout
                  ? (uint32_t)(((tile * nch) * kBN + R) * kWRowBytes + 16 * g)
                  : (uint32_t)((weight_row<PHASE>(p, tile, R) * (K / 8) + 4 * g) * 4);
  }
  const int wstep = packed_layout ? kWBytes : kWRowBytes;  // bytes per chunk
  // bytes from one tile's weights to the next tile's
  const int wtile = packed_layout ? nch * kWBytes : tile_cols<PHASE>() * (K / 2);
  auto copy_w = [&](uint8_t* dst, int t, int c) {
    const int so = uniform(t < ntl ? t * wtile + c * wstep : (int)kNoRow);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, (lds_ptr)(dst + (4 * wave + i) * 1024), 16,
                                               woff[i], so, 0, PK ? kPrefillPackedAux : kPrefillAux);
  };

  // ---- scale copies: instruction v covers rows 32v..32v+31 (32 B each) -------
  // (prepacked: a period of the tile is one 16 KB run; its periods are the
  // four-chunk periods here)
  static_assert(kSPeriod * kKC == 16 * 32, "scale periods of the prepacked layout");
  const int nper = (nch + kSPeriod - 1) / kSPeriod;
  const __amdgpu_buffer_rsrc_t sres =
      packed_layout
          ? __builtin_amdgcn_make_buffer_rsrc(
                (void*)(reinterpret_cast<const uint8_t*>(p.scales) + e * pack_scale_bytes(Nw, K)),
                0, (int)pack_scale_bytes(Nw, K), kBufferFlags)
          : __builtin_amdgcn_make_buffer_rsrc((void*)(p.scales + wbase * (K / 32)), 0,
                                              Nw * (K / 32) * 2, kBufferFlags);
  uint32_t soff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int R = 32 * (2 * wave + i) + (lane >> 1);
    soff[i] = packed_layout
                  ? (uint32_t)(((tile * nper) * kBN + R) * kSRowBytes + 16 * (lane & 1))
                  : (uint32_t)((weight_row<PHASE>(p, tile, R) * (K / 32) + 8 * (lane & 1)) * 2);
  }
  const int sstep = packed_layout ? kSBytes : kSRowBytes;  // bytes per period
  const int stile = packed_layout ? nper * kSBytes : tile_cols<PHASE>() * (K / 16);
  auto copy_s = [&](uint8_t* dst, int t, int lp) {
    const int so = uniform(t < ntl ? t * stile + lp * sstep : (int)kNoRow);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sres, (lds_ptr)(dst + (2 * wave + i) * 1024), 16,
                                               soff[i], so, 0, 0);
  };

  // ---- this lane's LDS read offsets -----------------------------------------
  // weights: row R = 64 wave + 16 s + lr, group lq (permuted slot)
  int wread[kNSub];
#pragma unroll
  for (int s = 0; s < kNSub; ++s) {
    const int R = wave * 64 + 16 * s + lr;
    wread[s] = R * kWRowBytes + (lq ^ wslot(R)) * 16;
  }
  // scales: row R, group 4 (chunk % 4) + lq
  const int sread = (wave * 64 + lr) * kSRowBytes + lq * 2;
  constexpr int kMaxCopies = kAPerWave + 4 + 2;  // copy instructions per wave and chunk
  // activations: row 16 mi + lr, piece 4 lq + j (permuted slot)
  const int aread = lr * (kKC * 2);

  f32x4 acc[MS][kNSub];
#pragma unroll
  for (int mi = 0; mi < MS; ++mi)
#pragma unroll
    for (int s = 0; s < kNSub; ++s) acc[mi][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  // issue_copies() is called in the first MFMA step; the scheduler spreads its
  // copy instructions between that step's MFMAs.
  auto compute = [&](const uint8_t* abuf, const u32x4 (&w)[kNSub], const float (&sc)[kNSub],
                     auto&& issue_copies) {
    GroupScale gs[kNSub];
#pragma unroll
    for (int s = 0; s < kNSub; ++s) gs[s] = group_scale(sc[s]);
    bf16x8 bw[2][kNSub];  // this step's and the next step's weights
#pragma unroll
    for (int s = 0; s < kNSub; ++s) bw[0][s] = dequant8(w[s][0], gs[s]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 a[MS];
      const int apiece = ((4 * lq + j) ^ aslot(lr)) * 16;  // inputs 32 lq + 8 j
#pragma unroll
      for (int mi = 0; mi < MS; ++mi)
        a[mi] = *reinterpret_cast<const bf16x8*>(abuf + mi * 16 * (kKC * 2) + aread + apiece);
      if (j < 3) {
#pragma unroll
        for (int s = 0; s < kNSub; ++s)
          bw[(j + 1) & 1][s] = dequant8(w[s][j + 1], gs[s]);
      }
#pragma unroll
      for (int mi = 0; mi < MS; ++mi)
#pragma unroll
        for (int s = 0; s < kNSub; ++s)
          acc[mi][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mi], bw[j & 1][s], acc[mi][s], 0, 0, 0);
      if (j == 0) issue_copies();
      // interleave: the activation reads first, then one MFMA per three VALU
      // instructions of the next step's dequantisation, and in the first step
      // one copy after each of the first MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, MS, 0);  // DS read
#pragma unroll
      for (int i = 0; i < MS * kNSub; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
        if (j == 0 && i < kMaxCopies) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto read_scales = [&](float (&sc)[kNSub], int t, int c) {
    const int per = t * nper + c / kSPeriod;  // period count across the tiles
    const uint8_t* sb = (per & 1) ? lds_s1 : lds_s0;
    const int g = (c % kSPeriod) * 8;  // bytes: 4 groups per chunk
#pragma unroll
    for (int s = 0; s < kNSub; ++s)
      sc[s] = bf16_to_f32(*reinterpret_cast<const uint16_t*>(sb + sread + s * 16 * kSRowBytes + g));
  };

  // The chunk's scales and this wave's weight words are read from LDS first;
  // the weight buffer is then free (each wave copies and reads only its own
  // rows), so the copy of chunk ch + 2 goes into it in this chunk: weights are
  // fetched two chunks ahead, activations (shared by all waves, buffer freed
  // by the barrier) one chunk ahead. The copies are issued between the first
  // step's MFMAs, not as one burst after the barrier: a burst from all eight
  // waves at once stalls them on issue with no MFMA work in flight.
  auto chunk = [&](int t, int c, uint8_t* abuf, uint8_t* anext, uint8_t* wbuf) {
    float sc[kNSub];
    read_scales(sc, t, c);
    u32x4 w[kNSub];
#pragma unroll
    for (int s = 0; s < kNSub; ++s) w[s] = *reinterpret_cast<const u32x4*>(wbuf + wread[s]);
    wait_lgkm0();
    __builtin_amdgcn_sched_barrier(0);
    // the chunk after this one and the one after that (nch is even, so a
    // tile boundary falls between two chunks of a pair)
    const int t1 = c + 1 < nch ? t : t + 1, c1 = c + 1 < nch ? c + 1 : 0;
    const int t2 = c + 2 < nch ? t : t + 1, c2 = c + 2 < nch ? c + 2 : c + 2 - nch;
    // the next scale period, at the first chunk of each period
    const int lp = c / kSPeriod;
    const int tn = lp + 1 < nper ? t : t + 1, lpn = lp + 1 < nper ? lp + 1 : 0;
    const bool new_s = c % kSPeriod == 0 && tn < ntl;
    const int pbuf = (t * nper + lp + 1) & 1;
    compute(abuf, w, sc, [&]() {
      copy_a(anext, t1, c1);
      copy_w(wbuf, t2, c2);
      if (new_s) copy_s(pbuf ? lds_s1 : lds_s0, tn, lpn);
    });
    // activations and weights of chunk ch + 1 in LDS (the copies of chunk
    // ch + 2's weights and of the next scales may stay in flight); this
    // chunk's LDS reads done before its activation buffer is overwritten
    if (new_s) wait_vm<6>();
    else wait_vm<4>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
  };

  // ---- pipeline -----------------------------------------------------------
  copy_w(lds_w0, 0, 0);
  copy_w(lds_w1, 0, 1);
  copy_a(lds_a0, 0, 0);
  copy_s(lds_s0, 0, 0);
  wait_vm<0>();
  __builtin_amdgcn_s_barrier();
  // ---- epilogue: lane holds rows 4 lq + i of each 16-row sub-tile, column lr
  auto epilogue = [&](int ctile) {
    if (PHASE == kGateUp) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int col = ctile * (kBN / 2) + wave * 32 + 16 * s + lr;
#pragma unroll
        for (int mi = 0; mi < MS; ++mi)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t r = row0 + mi * 16 + 4 * lq + i;
            const float hv = silu_mul(acc[mi][s][i], acc[mi][s + 2][i]);
            p.h_routed[r * p.I + col] = (uint16_t)(pack_bf16x2(hv, 0.f) & 0xFFFFu);
          }
      }
    } else {
#pragma unroll
      for (int mi = 0; mi < MS; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t r = row0 + mi * 16 + 4 * lq + i;
          const int32_t pair = p.sorted_ids[r];
          if (pair >= p.P) continue;
          float* dst = p.y_routed + (int64_t)pair * p.N + ctile * kBN + wave * 64 + lr;
#pragma unroll
          for (int s = 0; s < kNSub; ++s) dst[16 * s] = acc[mi][s][i];
        }
    }
  };

  // whole pairs (the chunk count is even; a loop with a second exit between
  // the halves makes the register allocator move the accumulators)
  if (!MT) {
    for (int c = 0; c < nch; c += 2) {
      chunk(0, c, lds_a0, lds_a1, lds_w0);
      chunk(0, c + 1, lds_a1, lds_a0, lds_w1);
    }
    epilogue(tile);
    return;
  }
  // several tiles: they follow each other without a break in the copy
  // stream (the last chunks of a tile already fetch the next tile's first
  // ones); the accumulators restart at zero for each tile
  for (int t = 0; t < ntl; ++t) {
    for (int c = 0; c < nch; c += 2) {
      chunk(t, c, lds_a0, lds_a1, lds_w0);
      chunk(t, c + 1, lds_a1, lds_a0, lds_w1);
    }
    epilogue(tile + t);
#pragma unroll
    for (int mi = 0; mi < MS; ++mi)
#pragma unroll
      for (int s = 0; s < kNSub; ++s) acc[mi][s] = f32x4{0.f, 0.f, 0.f, 0.f};
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
  if (msub <= 2) block_tile<PHASE, 2, PK, MT>(p, mblk, tile, ntl);
  else if (msub <= 4 || kMaxMS < 6) block_tile<PHASE, (kMaxMS < 4 ? kMaxMS : 4), PK, MT>(p, mblk, tile, ntl);
  else if (msub <= 6 || kMaxMS < 8) block_tile<PHASE, (kMaxMS < 6 ? kMaxMS : 6), PK, MT>(p, mblk, tile, ntl);
  else block_tile<PHASE, kMaxMS, PK, MT>(p, mblk, tile, ntl);
}

// One work-group per (block, column tile). PK: the weights are in the
// prepacked layout (a separate instance, so that traces tell the two apart).
template <int PHASE, bool PK>
__global__ __launch_bounds__(kThreads, 1) void prefill_gemm_kernel(GemmParams p) {
  const int n_tiles = p.N / tile_cols<PHASE>();
  const int x = blockIdx.x % kXcds;
  const int sx = blockIdx.x / kXcds;
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
// work-groups past the last group exit at once.
template <int PHASE, bool PK>
__global__ __launch_bounds__(kThreads, 1) void prefill_tiles_kernel(GemmParams p, int tpw_max) {
  const int n_tiles = p.N / tile_cols<PHASE>();
  const int64_t nblk = *p.n_padded / kBM;
  int tpw = 1;
  for (int c = tpw_max; c > 1; c >>= 1)
    if (nblk * ((n_tiles + c - 1) / c) >= 6 * 256) {
      tpw = c;
      break;
    }
  const int ngrp = (n_tiles + tpw - 1) / tpw;  // groups of tpw consecutive tiles
  const int x = blockIdx.x % kXcds;
  const int sx = blockIdx.x / kXcds;
  const int mblk = (sx / ngrp) * kXcds + x;
  const int tile = (sx - (sx / ngrp) * ngrp) * tpw;
  if (mblk >= p.max_blocks || (int64_t)mblk * kBM >= *p.n_padded) return;
  run_block<PHASE, PK, true>(p, mblk, tile, min(tpw, n_tiles - tile));
}

template <int PHASE>
hipError_t launch(const GemmParams& p, hipStream_t stream) {
  if (p.N % tile_cols<PHASE>() != 0 || p.K % (2 * kKC) != 0) return hipErrorInvalidValue;
  // buffer resources hold 32-bit byte sizes
  const int64_t arows = PHASE == kGateUp ? p.T : (int64_t)p.max_blocks * kBM;
  const int64_t nw = PHASE == kGateUp ? 2 * (int64_t)p.I : p.N;
  if (arows * p.K * 2 > 0x7fffffff || nw * p.K / 2 > 0x7fffffff) return hipErrorInvalidValue;
  const int64_t blocks = ((int64_t)p.max_blocks + kXcds - 1) / kXcds * kXcds;
  const int n_tiles = p.N / tile_cols<PHASE>();
  const int nch = p.K / kKC;
  // several tiles per work-group only where a tile is a few chunks long
  // (at most 16 chunks per work-group, at most four tiles)
  int tpw = 1;
  while (2 * tpw * nch <= 16 && 2 * tpw <= 4) tpw *= 2;
  const int64_t grid = blocks * n_tiles;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  GemmParams args = p;
  if (tpw == 1) {
    void* kargs[] = {&args};
    const void* fn = p.prepacked
                         ? reinterpret_cast<const void*>(&prefill_gemm_kernel<PHASE, true>)
                         : reinterpret_cast<const void*>(&prefill_gemm_kernel<PHASE, false>);
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kThreads), kargs, 0, stream);
  }
  void* kargs[] = {&args, &tpw};
  const void* fn = p.prepacked
                       ? reinterpret_cast<const void*>(&prefill_tiles_kernel<PHASE, true>)
                       : reinterpret_cast<const void*>(&prefill_tiles_kernel<PHASE, false>);
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kThreads), kargs, 0, stream);
}

}  // namespace

int32_t prefill_block_m() { return kBM; }

bool prefill_fits(int32_t hidden, int32_t inter) {
  return inter % tile_cols<kGateUp>() == 0 && hidden % tile_cols<kDown>() == 0 &&
         hidden % (2 * kKC) == 0 && inter % (2 * kKC) == 0;
}

hipError_t launch_gate_up_prefill(const GemmParams& p, hipStream_t stream) {
  return launch<kGateUp>(p, stream);
}

hipError_t launch_down_prefill(const GemmParams& p, hipStream_t stream) {
  return launch<kDown>(p, stream);
}

}  // namespace moe
