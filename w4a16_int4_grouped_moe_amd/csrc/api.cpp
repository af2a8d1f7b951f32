// api.cpp -- host side of the W4A16 MoE C ABI: argument validation, workspace
// layout and the launch sequence align -> gate_up(+SwiGLU) -> down -> combine.
// Every check runs before the first launch; nothing is allocated and the host
// never waits on the device.
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/moe_w4a16.h"
#include "internal.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kMaxPairs = 0x7ffffffe;  // T*k and the sentinel T*k fit in int32

thread_local char g_status_msg[256];

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

static_assert(moe::kMaxExperts == MOE_MAX_EXPERTS,
              "the bucketing kernels size their tables for MOE_MAX_EXPERTS");

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

int32_t choose_block_m(const moe_w4a16_problem* p);
int64_t sorted_capacity(const moe_w4a16_problem* p, int32_t bm);

// Buffer resources of the kernels hold 32-bit byte sizes, and their
// out-of-range offsets (2^31) must lie past every buffer: every array a
// kernel addresses through one stays below 2 GiB.
constexpr int64_t kMaxResource = 0x7fffffff;

int check_problem(const moe_w4a16_problem* p) {
  if (!p) return MOE_ERR_NULL;
  if (p->group_size != 32) return MOE_ERR_UNSUPPORTED;
  if (p->num_tokens < 0 || p->hidden <= 0 || p->inter <= 0 || p->num_experts <= 0 ||
      p->top_k <= 0 || p->top_k > MOE_MAX_TOP_K || p->expert_base < 0)
    return MOE_ERR_SHAPE;
  if (p->hidden % 128 != 0 || p->inter % 128 != 0) return MOE_ERR_SHAPE;
  if (p->num_experts > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)p->expert_base + p->num_experts > 0x7fffffff) return MOE_ERR_SHAPE;
  if (p->num_tokens > kMaxPairs / p->top_k) return MOE_ERR_SHAPE;
  const int64_t H = p->hidden, I = p->inter;
  // one bf16 matrix of the shared expert, one expert's int4 matrices
  if (2 * I * H * 2 > kMaxResource) return MOE_ERR_UNSUPPORTED;
  if (p->num_tokens > 0 && choose_block_m(p) != 4) {
    // 96-row blocks: x (bf16 and fp16) and the bucketed h rows (fp16)
    if (p->num_tokens * H * 2 > kMaxResource) return MOE_ERR_UNSUPPORTED;
    if (sorted_capacity(p, choose_block_m(p)) * I * 2 > kMaxResource) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

int64_t sorted_capacity(const moe_w4a16_problem* p, int32_t bm) {
  const int64_t P = p->num_tokens * p->top_k;
  const int64_t emin = P < p->num_experts ? P : p->num_experts;
  return P + emin * (bm - 1);
}

int32_t choose_block_m(const moe_w4a16_problem* p) {
  // About one row per expert (decode): 4-row buckets and the weight-streaming
  // small-batch kernels. Beyond that the block kernel's 96-row buckets
  // (measured faster than 16- and 64-row blocks from a few rows per expert
  // on, and with skewed routing).
  const int64_t P = p->num_tokens * p->top_k;
  const int64_t E = p->num_experts;
  if (P <= 4 * E && moe::small_batch_fits(p->hidden, p->inter)) return 4;
  return moe::prefill_block_m();
}

// Bucketing in many work-groups (three launches) from this many pairs on.
#ifndef MOE_ALIGN_MULTI_MIN
#define MOE_ALIGN_MULTI_MIN 8192
#endif
constexpr int64_t kAlignMultiMin = MOE_ALIGN_MULTI_MIN;

// 96-row problems bucketed in one work-group (fewer than kAlignMultiMin
// pairs): experts with at most this many pairs go to 4-row buckets and the
// small-batch kernels, which stream an expert's weights about 1.6x faster
// than a 96-row block kernel holding a few rows (measured: 2.7 vs 4.5 us per
// expert); beyond 4 pairs a second 4-row bucket would read the weights twice.
#ifndef MOE_SPLIT_MAX_PAIRS
#define MOE_SPLIT_MAX_PAIRS 4
#endif
constexpr int32_t kSplitMaxPairs = MOE_SPLIT_MAX_PAIRS;

bool split_buckets(const moe_w4a16_problem* p, int32_t bm) {
  const int64_t P = p->num_tokens * p->top_k;
  return kSplitMaxPairs > 0 && bm == moe::prefill_block_m() && P > 0 && P < kAlignMultiMin &&
         moe::small_batch_fits(p->hidden, p->inter);
}

struct Layout {
  size_t sorted_ids, block_expert, meta, h, y, hs, s, align_scratch, x16, kx, kh, kr, total;
  // split bucketing: the 4-row set (its ids, block map, count, bf16 h rows)
  size_t sorted2, block2, meta2, h2;
  int64_t cap_rows, cap_rows2;
  int32_t max_blocks, bm, n_htiles, max_blocks2;
  bool split;
};

Layout layout(const moe_w4a16_problem* p) {
  Layout L{};
  L.bm = choose_block_m(p);
  L.cap_rows = sorted_capacity(p, L.bm);
  L.max_blocks = (int32_t)(L.cap_rows / L.bm);
  L.n_htiles = (p->inter + moe::kHTile - 1) / moe::kHTile;
  const size_t T = (size_t)p->num_tokens, H = (size_t)p->hidden, I = (size_t)p->inter;
  const size_t P = T * (size_t)p->top_k;
  size_t o = 0;
  L.sorted_ids = o; o = round_up(o + 4 * (size_t)L.cap_rows);
  L.block_expert = o; o = round_up(o + 4 * (size_t)L.max_blocks);
  L.meta = o; o = round_up(o + 64);
  L.h = o; o = round_up(o + 2 * (size_t)L.max_blocks * L.bm * I);
  L.y = o; o = round_up(o + 4 * P * H);
  L.hs = o; o = round_up(o + 2 * T * I);
  L.s = o; o = round_up(o + 4 * T * H);
  L.align_scratch = o;
  if ((int64_t)P >= kAlignMultiMin)
    o = round_up(o + 4 * (size_t)moe::align_scratch_ints((int64_t)P, p->num_experts));
  // 96-row blocks: x in fp16 with its per-token exponents, the per-(row,
  // tile) exponents of h
  L.x16 = L.kx = L.kh = L.kr = o;
  if (L.bm == moe::prefill_block_m()) {
    L.x16 = o; o = round_up(o + 2 * T * H);
    L.kx = o; o = round_up(o + 4 * T);
    L.kh = o; o = round_up(o + 4 * (size_t)L.cap_rows * L.n_htiles);
    L.kr = o; o = round_up(o + 4 * (size_t)L.cap_rows);
  }
  L.split = split_buckets(p, L.bm);
  L.sorted2 = L.block2 = L.meta2 = L.h2 = o;
  if (L.split) {
    // an expert of the 4-row set holds at most kSplitMaxPairs pairs: at most
    // ceil(kSplitMaxPairs / 4) blocks each (the launches over this set size
    // their grids by it, and its blocks past the count exit at once)
    const int64_t P64 = (int64_t)P, E64 = p->num_experts;
    const int64_t per = (kSplitMaxPairs + 3) / 4;
    L.cap_rows2 = std::min<int64_t>(sorted_capacity(p, 4), 4 * per * std::min(E64, P64));
    L.max_blocks2 = (int32_t)(L.cap_rows2 / 4);
    L.sorted2 = o; o = round_up(o + 4 * (size_t)L.cap_rows2);
    L.block2 = o; o = round_up(o + 4 * (size_t)L.max_blocks2);
    L.meta2 = o; o = round_up(o + 64);
    L.h2 = o; o = round_up(o + 2 * (size_t)L.cap_rows2 * I);
  }
  L.total = o;
  return L;
}

int hip_status(hipError_t err) {
  if (err == hipSuccess) return MOE_OK;
  snprintf(g_status_msg, sizeof g_status_msg, "HIP error %d (%s): %s", (int)err,
           hipGetErrorName(err), hipGetErrorString(err));
  return MOE_ERR_HIP;
}

}  // namespace

extern "C" {

int moe_w4a16_workspace_size(const moe_w4a16_problem* p, size_t* bytes) {
  const int st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_NULL;
  *bytes = p->num_tokens == 0 ? 0 : layout(p).total;
  return MOE_OK;
}

int moe_w4a16_forward_block_m(const moe_w4a16_problem* p, int32_t* block_m) {
  const int st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!block_m) return MOE_ERR_NULL;
  *block_m = choose_block_m(p);
  return MOE_OK;
}

int moe_w4a16_forward_split_max_pairs(const moe_w4a16_problem* p, int32_t* max_pairs) {
  const int st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!max_pairs) return MOE_ERR_NULL;
  *max_pairs = split_buckets(p, choose_block_m(p)) ? kSplitMaxPairs : 0;
  return MOE_OK;
}

int moe_w4a16_align_capacity(const moe_w4a16_problem* p, int32_t block_m,
                             int64_t* sorted_cap, int64_t* block_cap) {
  const int st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!sorted_cap || !block_cap) return MOE_ERR_NULL;
  if (block_m < 1 || block_m > 1024) return MOE_ERR_SHAPE;
  *sorted_cap = sorted_capacity(p, block_m);
  *block_cap = *sorted_cap / block_m;
  return MOE_OK;
}

int moe_w4a16_align_scratch_size(const moe_w4a16_problem* p, size_t* bytes) {
  const int st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_NULL;
  *bytes = 4 * (size_t)moe::align_scratch_ints(p->num_tokens * p->top_k, p->num_experts);
  return MOE_OK;
}

int moe_w4a16_align(const int32_t* topk_ids, const moe_w4a16_problem* p, int32_t block_m,
                    int32_t* sorted_ids, int64_t sorted_cap, int32_t* block_expert,
                    int64_t block_cap, int32_t* n_padded, void* scratch, size_t scratch_bytes,
                    void* stream) {
  const int st = check_problem(p);
  if (st != MOE_OK) return st;
  if (block_m < 1 || block_m > 1024) return MOE_ERR_SHAPE;
  if (!n_padded) return MOE_ERR_NULL;
  const int64_t need = sorted_capacity(p, block_m);
  if (p->num_tokens > 0 && (!topk_ids || !sorted_ids || !block_expert)) return MOE_ERR_NULL;
  if (!aligned16(topk_ids) || !aligned16(sorted_ids) || !aligned16(block_expert) ||
      !aligned16(n_padded))
    return MOE_ERR_ALIGNMENT;
  if (sorted_cap < need || block_cap < need / block_m) return MOE_ERR_WORKSPACE;
  const int64_t P = p->num_tokens * p->top_k;
  if (scratch) {
    if (!aligned16(scratch)) return MOE_ERR_ALIGNMENT;
    if (scratch_bytes < 4 * (size_t)moe::align_scratch_ints(P, p->num_experts))
      return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_align_multi(topk_ids, P, p->num_experts, p->expert_base,
                                              block_m, sorted_ids, block_expert, n_padded,
                                              static_cast<int32_t*>(scratch), (hipStream_t)stream));
  }
  return hip_status(moe::launch_align(topk_ids, P, p->num_experts, p->expert_base, block_m,
                                      sorted_ids, block_expert, n_padded, (hipStream_t)stream));
}

// The layer call's argument checks (before any launch). own_workspace: the
// workspace is the library's device array (not checked here).
static int check_forward(const void* x, const int32_t* topk_ids, const float* topk_weights,
                         const int32_t* packed_w13, const void* scales_w13,
                         const int32_t* packed_w2, const void* scales_w2, const void* shared_w,
                         const void* out, const moe_w4a16_problem* p, const void* workspace,
                         size_t workspace_bytes, bool own_workspace = false) {
  const int st = check_problem(p);
  if (st != MOE_OK) return st;
  if (p->num_tokens == 0) return MOE_OK;
  if (!x || !topk_ids || !topk_weights || !packed_w13 || !scales_w13 || !packed_w2 ||
      !scales_w2 || !out || (!workspace && !own_workspace))
    return MOE_ERR_NULL;
  const void* ptrs[] = {x, topk_ids, topk_weights, packed_w13, scales_w13,
                        packed_w2, scales_w2, shared_w, out, own_workspace ? nullptr : workspace};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return MOE_ERR_ALIGNMENT;
  if (workspace_bytes < layout(p).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

static int forward_impl(const void* x, const int32_t* topk_ids, const float* topk_weights,
                        const int32_t* packed_w13, const void* scales_w13,
                        const int32_t* packed_w2, const void* scales_w2, const void* shared_w,
                        void* out, const moe_w4a16_problem* p, void* workspace,
                        size_t workspace_bytes, void* stream, void* const* events,
                        bool prepacked = false) {
  const int st = check_forward(x, topk_ids, topk_weights, packed_w13, scales_w13, packed_w2,
                               scales_w2, shared_w, out, p, workspace, workspace_bytes);
  if (st != MOE_OK || p->num_tokens == 0) return st;
  const Layout L = layout(p);

  char* ws = static_cast<char*>(workspace);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted_ids);
  int32_t* blk = reinterpret_cast<int32_t*>(ws + L.block_expert);
  int32_t* n_padded = reinterpret_cast<int32_t*>(ws + L.meta);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.h);
  float* y = reinterpret_cast<float*>(ws + L.y);
  uint16_t* hs = reinterpret_cast<uint16_t*>(ws + L.hs);
  float* s = reinterpret_cast<float*>(ws + L.s);
  hipStream_t strm = (hipStream_t)stream;

  const int64_t T = p->num_tokens;
  const int32_t H = p->hidden, I = p->inter, E = p->num_experts, k = p->top_k;
  const uint16_t* sw = static_cast<const uint16_t*>(shared_w);

  auto mark = [&](int i) -> hipError_t {  // stage_events[i], if given
    if (events && events[i]) return hipEventRecord((hipEvent_t)events[i], strm);
    return hipSuccess;
  };
  hipError_t err = mark(0);
  if (err != hipSuccess) return hip_status(err);
  // A few pairs: the gate_up launch buckets them itself (no bucketing launch).
  const bool local = L.bm == 4 && T * k <= moe::kLocalPairs && T <= moe::kLocalTokens;
  if (local)
    err = hipSuccess;
  else if (T * k >= kAlignMultiMin)
    err = moe::launch_align_multi(topk_ids, T * k, E, p->expert_base, L.bm, sorted, blk, n_padded,
                                  reinterpret_cast<int32_t*>(ws + L.align_scratch), strm);
  else if (L.split)
    err = moe::launch_align_split(topk_ids, T * k, E, p->expert_base, L.bm, sorted, blk, n_padded,
                                  kSplitMaxPairs, 4, reinterpret_cast<int32_t*>(ws + L.sorted2),
                                  reinterpret_cast<int32_t*>(ws + L.block2),
                                  reinterpret_cast<int32_t*>(ws + L.meta2), strm);
  else
    err = moe::launch_align(topk_ids, T * k, E, p->expert_base, L.bm, sorted, blk, n_padded, strm);
  if (err != hipSuccess) return hip_status(err);

  // One GEMM phase: a single launch that carries the routed experts and the
  // shared expert (split bucketing: first a small-batch launch over the
  // 4-row buckets, without the shared expert). Event `after_routed` follows.
  auto gemm = [&](const moe::GemmParams& gp, bool gate_up, int after_routed) -> hipError_t {
    hipError_t e = hipSuccess;
    if (L.split) {
      moe::GemmParams g4 = gp;
      g4.sorted_ids = reinterpret_cast<const int32_t*>(ws + L.sorted2);
      g4.block_expert = reinterpret_cast<const int32_t*>(ws + L.block2);
      g4.n_padded = reinterpret_cast<const int32_t*>(ws + L.meta2);
      g4.max_blocks = L.max_blocks2;
      g4.wshared = nullptr;
      g4.a_exp = nullptr;
      g4.h_exp = nullptr;
      uint16_t* h2 = reinterpret_cast<uint16_t*>(ws + L.h2);
      if (gate_up) {
        g4.a_routed = static_cast<const uint16_t*>(x);
        g4.h_routed = h2;
        e = moe::launch_gate_up_small(g4, strm);
      } else {
        g4.a_routed = h2;
        e = moe::launch_down_small(g4, strm);
      }
      if (e != hipSuccess) return e;
    }
    if (L.bm == 4)
      e = gate_up ? moe::launch_gate_up_small(gp, strm) : moe::launch_down_small(gp, strm);
    else
      e = gate_up ? moe::launch_gate_up_prefill(gp, strm) : moe::launch_down_prefill(gp, strm);
    return e != hipSuccess ? e : mark(after_routed);
  };

  moe::GemmParams g{};
  g.sorted_ids = sorted;
  g.block_expert = blk;
  g.n_padded = n_padded;
  g.max_blocks = L.max_blocks;
  g.T = T;
  g.P = T * k;
  g.k = k;
  g.I = I;
  g.nibble_mask = 0x0F0F0F0Fu;
  g.prepacked = prepacked ? 1 : 0;
  g.n_htiles = L.n_htiles;
  g.local_route = local ? 1 : 0;
  g.topk_ids = topk_ids;
  g.n_experts = E;
  g.expert_base = p->expert_base;
  g.sorted_out = sorted;
  g.block_expert_out = blk;
  g.n_padded_out = n_padded;
  const bool blocks96 = L.bm == moe::prefill_block_m();
  uint16_t* x16 = reinterpret_cast<uint16_t*>(ws + L.x16);
  int32_t* kx = reinterpret_cast<int32_t*>(ws + L.kx);
  int32_t* kh = reinterpret_cast<int32_t*>(ws + L.kh);
  int32_t* kr = reinterpret_cast<int32_t*>(ws + L.kr);

  // gate_up + SwiGLU (96-row blocks: on x in fp16, converted with the
  // bucketing's stage, before event 1)
  if (blocks96) {
    err = moe::launch_x16(static_cast<const uint16_t*>(x), x16, kx, T, H, strm);
    if (err != hipSuccess) return hip_status(err);
  }
  if ((err = mark(1)) != hipSuccess) return hip_status(err);
  g.a_routed = blocks96 ? x16 : static_cast<const uint16_t*>(x);
  g.a_exp = kx;
  g.h_exp = kh;
  g.packed = packed_w13;
  g.scales = static_cast<const uint16_t*>(scales_w13);
  g.a_shared = static_cast<const uint16_t*>(x);
  g.wshared = sw;
  g.h_routed = h;
  g.h_shared = hs;
  g.K = H;
  g.N = I;
  err = gemm(g, true, 5);
  if (err != hipSuccess) return hip_status(err);
  g.local_route = 0;

  // down (96-row blocks: h rows brought to one exponent per row first)
  if (blocks96) {
    err = moe::launch_h_rescale(h, kh, kr, n_padded, L.cap_rows, I, L.n_htiles, strm);
    if (err != hipSuccess) return hip_status(err);
  }
  g.a_routed = h;
  g.a_exp = kr;
  g.h_exp = nullptr;
  g.packed = packed_w2;
  g.scales = static_cast<const uint16_t*>(scales_w2);
  g.a_shared = hs;
  g.wshared = sw ? sw + (size_t)2 * I * H : nullptr;
  g.y_routed = y;
  g.y_shared = s;
  g.K = I;
  g.N = H;
  if ((err = mark(2)) != hipSuccess) return hip_status(err);
  err = gemm(g, false, 6);
  if (err != hipSuccess) return hip_status(err);

  if ((err = mark(3)) != hipSuccess) return hip_status(err);
  err = moe::launch_combine(y, sw ? s : nullptr, topk_ids, topk_weights,
                            static_cast<uint16_t*>(out), T, H, k, E, p->expert_base, strm);
  if (err != hipSuccess) return hip_status(err);
  return hip_status(mark(4));
}

int moe_w4a16_forward(const void* x, const int32_t* topk_ids, const float* topk_weights,
                      const int32_t* packed_w13, const void* scales_w13,
                      const int32_t* packed_w2, const void* scales_w2, const void* shared_w,
                      void* out, const moe_w4a16_problem* p, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return forward_impl(x, topk_ids, topk_weights, packed_w13, scales_w13, packed_w2, scales_w2,
                      shared_w, out, p, workspace, workspace_bytes, stream, nullptr);
}

}  // extern "C"

// ---- the allocation-free variant ------------------------------------------------
// Its workspace is this file-scope device array (one per GPU, held until the
// process ends). In host code `scratch` is only a host-side stand-in for the
// symbol: its device address comes from hipGetSymbolAddress, once per device,
// and only that address is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device

// The address of the current device's scratch array (resolved on the first
// call on that device, with the device current), or NULL with *err set.
void* scratch_address(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int moe_w4a16_noalloc_workspace_limit(size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL;
  *bytes = MOE_NOALLOC_SCRATCH_BYTES;
  return MOE_OK;
}

int moe_w4a16_forward_noalloc(const void* x, const int32_t* topk_ids, const float* topk_weights,
                              const int32_t* packed_w13, const void* scales_w13,
                              const int32_t* packed_w2, const void* scales_w2,
                              const void* shared_w, void* out, const moe_w4a16_problem* p,
                              void* stream) {
  const int st = check_forward(x, topk_ids, topk_weights, packed_w13, scales_w13, packed_w2,
                               scales_w2, shared_w, out, p, nullptr,
                               (size_t)MOE_NOALLOC_SCRATCH_BYTES, true);
  if (st != MOE_OK || p->num_tokens == 0) return st;
  hipError_t err = hipSuccess;
  void* ws = scratch_address(&err);
  if (!ws) return hip_status(err);
  return forward_impl(x, topk_ids, topk_weights, packed_w13, scales_w13, packed_w2, scales_w2,
                      shared_w, out, p, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int moe_w4a16_forward_timed(const void* x, const int32_t* topk_ids, const float* topk_weights,
                            const int32_t* packed_w13, const void* scales_w13,
                            const int32_t* packed_w2, const void* scales_w2,
                            const void* shared_w, void* out, const moe_w4a16_problem* p,
                            void* workspace, size_t workspace_bytes, void* stream,
                            void* const* stage_events) {
  return forward_impl(x, topk_ids, topk_weights, packed_w13, scales_w13, packed_w2, scales_w2,
                      shared_w, out, p, workspace, workspace_bytes, stream, stage_events);
}

// ---- prepacked weights --------------------------------------------------------
// Buffer: W13 codes, W13 scales, W2 codes, W2 scales of all local experts, each
// region 256-byte aligned, in the layout of internal.h.
struct PackLayout {
  size_t w13, s13, w2, s2, total;
};

static PackLayout pack_layout(const moe_w4a16_problem* p) {
  const size_t E = (size_t)p->num_experts;
  const int32_t H = p->hidden, I = p->inter;
  PackLayout L{};
  size_t o = 0;
  L.w13 = o; o = round_up(o + E * (size_t)moe::pack_code_bytes(2 * I, H));
  L.s13 = o; o = round_up(o + E * (size_t)moe::pack_scale_bytes(2 * I, H));
  L.w2 = o; o = round_up(o + E * (size_t)moe::pack_code_bytes(H, I));
  L.s2 = o; o = round_up(o + E * (size_t)moe::pack_scale_bytes(H, I));
  L.total = o;
  return L;
}

// Widths the prepacked layout serves: every batch size must run on the
// small-batch (with the narrow down kernel) and prefill kernels, which read
// it; the tiled kernel, used where the prefill tiles do not fit, does not.
static int check_prepack_problem(const moe_w4a16_problem* p) {
  const int st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!moe::prefill_fits(p->hidden, p->inter)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int moe_w4a16_prepack_size(const moe_w4a16_problem* p, size_t* bytes) {
  const int st = check_prepack_problem(p);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_NULL;
  *bytes = pack_layout(p).total;
  return MOE_OK;
}

int moe_w4a16_prepack(const int32_t* packed_w13, const void* scales_w13,
                      const int32_t* packed_w2, const void* scales_w2,
                      const moe_w4a16_problem* p, void* prepacked, size_t prepacked_bytes,
                      void* stream) {
  const int st = check_prepack_problem(p);
  if (st != MOE_OK) return st;
  if (!packed_w13 || !scales_w13 || !packed_w2 || !scales_w2 || !prepacked) return MOE_ERR_NULL;
  const void* ptrs[] = {packed_w13, scales_w13, packed_w2, scales_w2, prepacked};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return MOE_ERR_ALIGNMENT;
  const PackLayout L = pack_layout(p);
  if (prepacked_bytes < L.total) return MOE_ERR_WORKSPACE;
  uint8_t* b = static_cast<uint8_t*>(prepacked);
  const int32_t E = p->num_experts, H = p->hidden, I = p->inter;
  hipStream_t strm = (hipStream_t)stream;
  hipError_t err = moe::launch_prepack(packed_w13, static_cast<const uint16_t*>(scales_w13), E,
                                       2 * I, H, true, I, b + L.w13, b + L.s13, strm);
  if (err != hipSuccess) return hip_status(err);
  return hip_status(moe::launch_prepack(packed_w2, static_cast<const uint16_t*>(scales_w2), E, H,
                                        I, false, I, b + L.w2, b + L.s2, strm));
}

static int forward_prepacked_impl(const void* x, const int32_t* topk_ids,
                                  const float* topk_weights, const void* prepacked,
                                  size_t prepacked_bytes, const void* shared_w, void* out,
                                  const moe_w4a16_problem* p, void* workspace,
                                  size_t workspace_bytes, void* stream, void* const* events) {
  const int st = check_prepack_problem(p);
  if (st != MOE_OK) return st;
  if (p->num_tokens == 0) return MOE_OK;
  if (!prepacked) return MOE_ERR_NULL;
  if (!aligned16(prepacked)) return MOE_ERR_ALIGNMENT;
  const PackLayout L = pack_layout(p);
  if (prepacked_bytes < L.total) return MOE_ERR_WORKSPACE;
  const uint8_t* b = static_cast<const uint8_t*>(prepacked);
  return forward_impl(x, topk_ids, topk_weights, reinterpret_cast<const int32_t*>(b + L.w13),
                      b + L.s13, reinterpret_cast<const int32_t*>(b + L.w2), b + L.s2, shared_w,
                      out, p, workspace, workspace_bytes, stream, events, true);
}

int moe_w4a16_forward_prepacked(const void* x, const int32_t* topk_ids,
                                const float* topk_weights, const void* prepacked,
                                size_t prepacked_bytes, const void* shared_w, void* out,
                                const moe_w4a16_problem* p, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return forward_prepacked_impl(x, topk_ids, topk_weights, prepacked, prepacked_bytes, shared_w,
                                out, p, workspace, workspace_bytes, stream, nullptr);
}

int moe_w4a16_forward_prepacked_timed(const void* x, const int32_t* topk_ids,
                                      const float* topk_weights, const void* prepacked,
                                      size_t prepacked_bytes, const void* shared_w, void* out,
                                      const moe_w4a16_problem* p, void* workspace,
                                      size_t workspace_bytes, void* stream,
                                      void* const* stage_events) {
  return forward_prepacked_impl(x, topk_ids, topk_weights, prepacked, prepacked_bytes, shared_w,
                                out, p, workspace, workspace_bytes, stream, stage_events);
}

static int check_route(const float* scores, int32_t num_scored, const moe_w4a16_problem* p,
                       const int32_t* topk_ids, const float* topk_weights) {
  const int st = check_problem(p);
  if (st != MOE_OK) return st;
  if (num_scored < 1 || num_scored > MOE_MAX_SCORED || p->top_k > num_scored ||
      (int64_t)p->expert_base + p->num_experts > num_scored)
    return MOE_ERR_SHAPE;
  if (p->num_tokens == 0) return MOE_OK;
  if (!scores || !topk_ids || !topk_weights) return MOE_ERR_NULL;
  if (!aligned16(scores) || !aligned16(topk_ids) || !aligned16(topk_weights))
    return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

int moe_w4a16_route(const float* scores, int32_t num_scored, const moe_w4a16_problem* p,
                    int32_t* topk_ids, float* topk_weights, void* stream) {
  const int st = check_route(scores, num_scored, p, topk_ids, topk_weights);
  if (st != MOE_OK || p->num_tokens == 0) return st;
  return hip_status(moe::launch_route(scores, p->num_tokens, num_scored, p->top_k, topk_ids,
                                      topk_weights, (hipStream_t)stream));
}

int moe_w4a16_forward_scores(const void* x, const float* scores, int32_t num_scored,
                             const int32_t* packed_w13, const void* scales_w13,
                             const int32_t* packed_w2, const void* scales_w2,
                             const void* shared_w, void* out, int32_t* topk_ids,
                             float* topk_weights, const moe_w4a16_problem* p, void* workspace,
                             size_t workspace_bytes, void* stream) {
  int st = check_route(scores, num_scored, p, topk_ids, topk_weights);
  if (st != MOE_OK || p->num_tokens == 0) return st;
  // every check of the layer call runs before the router's launch
  st = check_forward(x, topk_ids, topk_weights, packed_w13, scales_w13, packed_w2, scales_w2,
                     shared_w, out, p, workspace, workspace_bytes);
  if (st != MOE_OK) return st;
  st = hip_status(moe::launch_route(scores, p->num_tokens, num_scored, p->top_k, topk_ids,
                                    topk_weights, (hipStream_t)stream));
  if (st != MOE_OK) return st;
  return forward_impl(x, topk_ids, topk_weights, packed_w13, scales_w13, packed_w2, scales_w2,
                      shared_w, out, p, workspace, workspace_bytes, stream, nullptr);
}

const char* moe_w4a16_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK: success";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: a size is out of range";
    case MOE_ERR_ALIGNMENT: return "MOE_ERR_ALIGNMENT: a device pointer is not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace or buffer too small";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: unsupported configuration";
    case MOE_ERR_HIP: return g_status_msg[0] ? g_status_msg : "MOE_ERR_HIP: a HIP call failed";
    default: return "unknown status";
  }
}

}  // extern "C"
