// Host-only stand-ins for the HIP runtime calls and kernel launchers that the
// library's host code (csrc/api.cpp) makes, so that this code can be built
// with AddressSanitizer and UndefinedBehaviorSanitizer on a machine without a
// GPU. No kernel runs. Each launcher checks that every workspace array it is
// handed lies inside the workspace the check program registered, with the
// size the kernel would address, and counts the call.
#include <hip/hip_runtime.h>

#include <cstdio>

#include "internal.h"
#include "moe_w4a16.h"

namespace stub {
const char* ws_lo = nullptr;
size_t ws_bytes = 0;
int launches = 0;
int bad = 0;
const void* scratch = nullptr;  // the allocation-free entry point's array, once known

void set_workspace(const void* p, size_t n) {
  ws_lo = static_cast<const char*>(p);
  ws_bytes = n;
}

// the next launches run in the allocation-free entry point's array (its
// address is looked up on that entry point's first call)
void select_scratch() {
  if (scratch) set_workspace(scratch, MOE_NOALLOC_SCRATCH_BYTES);
}

// [p, p + bytes) inside the registered workspace (NULL: not used)
static void in_ws(const void* p, int64_t bytes, const char* what) {
  if (!p) return;
  const char* c = static_cast<const char*>(p);
  if (bytes < 0 || c < ws_lo || c + bytes > ws_lo + ws_bytes) {
    std::fprintf(stderr, "stub: %s [%p, +%lld) outside the workspace [%p, +%zu)\n", what, p,
                 (long long)bytes, (const void*)ws_lo, ws_bytes);
    ++bad;
  }
}

static void gemm_common(const moe::GemmParams& p, int bm, bool gate_up) {
  ++launches;
  const int64_t rows = (int64_t)p.max_blocks * bm;
  if (p.local_route) {
    in_ws(p.sorted_out, 4 * rows, "sorted_out");
    in_ws(p.block_expert_out, 4 * (int64_t)p.max_blocks, "block_expert_out");
    in_ws(p.n_padded_out, 4, "n_padded_out");
  } else {
    in_ws(p.sorted_ids, 4 * rows, "sorted_ids");
    in_ws(p.block_expert, 4 * (int64_t)p.max_blocks, "block_expert");
    in_ws(p.n_padded, 4, "n_padded");
  }
  if (gate_up) {
    in_ws(p.h_routed, 2 * rows * p.I, "h");
    if (p.wshared) in_ws(p.h_shared, 2 * p.T * p.I, "shared h");
  } else {
    in_ws(p.a_routed, 2 * rows * p.K, "h (down input)");
    in_ws(p.y_routed, 4 * p.P * p.N, "y");
    if (p.wshared) in_ws(p.y_shared, 4 * p.T * p.N, "s");
  }
}
}  // namespace stub

extern "C" {
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}
const char* hipGetErrorName(hipError_t) { return "hipErrorStub"; }
const char* hipGetErrorString(hipError_t) { return "stub"; }
// the host shadow of a __device__ array stands for its device address; the
// allocation-free entry point then takes it as its workspace
hipError_t hipGetSymbolAddress(void** ptr, const void* symbol) {
  *ptr = const_cast<void*>(symbol);
  stub::scratch = symbol;
  stub::select_scratch();
  return hipSuccess;
}
}

namespace moe {
// the same values as the library's own helpers
int64_t align_scratch_ints(int64_t P, int32_t E) { return ((P + 255) / 256 + 1) * E; }
int32_t prefill_block_m() { return 96; }
bool prefill_fits(int32_t hidden, int32_t inter) {
  return inter % 256 == 0 && hidden % 512 == 0 && hidden % 128 == 0 && inter % 128 == 0;
}
bool small_batch_fits(int32_t hidden, int32_t inter) {
  auto lds = [](int K) {
    const int niters = (K / 32 + 15) / 16;
    const int routed = 2 * 4096 + 4 * 4 * 4 * 32 * (niters | 1);
    const int shared = 2 * 4 * 4096;
    return routed > shared ? routed : shared;
  };
  return lds(hidden) <= 64 * 1024 && lds(inter) <= 64 * 1024;
}

hipError_t launch_align(const int32_t*, int64_t P, int32_t E, int32_t, int32_t block_m,
                        int32_t* sorted_ids, int32_t* block_expert, int32_t* n_padded,
                        hipStream_t) {
  ++stub::launches;
  const int64_t cap = P + (P < E ? P : E) * (block_m - 1);
  stub::in_ws(sorted_ids, 4 * cap, "sorted_ids");
  stub::in_ws(block_expert, 4 * (cap / block_m), "block_expert");
  stub::in_ws(n_padded, 4, "n_padded");
  return hipSuccess;
}
hipError_t launch_align_split(const int32_t* ids, int64_t P, int32_t E, int32_t base,
                              int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
                              int32_t* n_padded, int32_t tau, int32_t block_m2, int32_t* sorted2,
                              int32_t* block_expert2, int32_t* n_padded2, hipStream_t s) {
  if (tau < 0 || block_m2 < 1) ++stub::bad;
  // the second set holds experts of at most tau pairs: ceil(tau / block_m2)
  // blocks each at most
  const int64_t emin = P < E ? P : E;
  const int64_t full = P + emin * (block_m2 - 1);
  const int64_t tight = block_m2 * ((tau + block_m2 - 1) / block_m2) * emin;
  const int64_t cap2 = full < tight ? full : tight;
  stub::in_ws(sorted2, 4 * cap2, "sorted_ids (second set)");
  stub::in_ws(block_expert2, 4 * (cap2 / block_m2), "block_expert (second set)");
  stub::in_ws(n_padded2, 4, "n_padded (second set)");
  return launch_align(ids, P, E, base, block_m, sorted_ids, block_expert, n_padded, s);
}
hipError_t launch_align_multi(const int32_t* ids, int64_t P, int32_t E, int32_t base,
                              int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
                              int32_t* n_padded, int32_t* scratch, hipStream_t s) {
  stub::in_ws(scratch, 4 * align_scratch_ints(P, E), "align scratch");
  return launch_align(ids, P, E, base, block_m, sorted_ids, block_expert, n_padded, s);
}
hipError_t launch_prepack(const int32_t*, const uint16_t*, int32_t, int32_t, int32_t, bool,
                          int32_t, uint8_t*, uint8_t*, hipStream_t) {
  ++stub::launches;
  return hipSuccess;
}
hipError_t launch_gate_up_small(const GemmParams& p, hipStream_t) {
  stub::gemm_common(p, 4, true);
  return hipSuccess;
}
hipError_t launch_down_small(const GemmParams& p, hipStream_t) {
  stub::gemm_common(p, 4, false);
  return hipSuccess;
}
hipError_t launch_gate_up_prefill(const GemmParams& p, hipStream_t) {
  stub::gemm_common(p, 96, true);
  stub::in_ws(p.a_routed, 2 * p.T * p.K, "x16");
  stub::in_ws(p.a_exp, 4 * p.T, "kx");
  stub::in_ws(p.h_exp, 4 * (int64_t)p.max_blocks * 96 * p.n_htiles, "kh");
  return hipSuccess;
}
hipError_t launch_down_prefill(const GemmParams& p, hipStream_t) {
  stub::gemm_common(p, 96, false);
  stub::in_ws(p.a_exp, 4 * (int64_t)p.max_blocks * 96, "kr");
  return hipSuccess;
}
hipError_t launch_x16(const uint16_t*, uint16_t* x16, int32_t* kx, int64_t T, int32_t H,
                      hipStream_t) {
  ++stub::launches;
  stub::in_ws(x16, 2 * T * H, "x16");
  stub::in_ws(kx, 4 * T, "kx");
  return hipSuccess;
}
hipError_t launch_h_rescale(uint16_t* h, const int32_t* kh, int32_t* kr, const int32_t* n_padded,
                            int64_t rows, int32_t I, int32_t n_htiles, hipStream_t) {
  ++stub::launches;
  stub::in_ws(h, 2 * rows * I, "h");
  stub::in_ws(kh, 4 * rows * n_htiles, "kh");
  stub::in_ws(kr, 4 * rows, "kr");
  stub::in_ws(n_padded, 4, "n_padded");
  return hipSuccess;
}
hipError_t launch_combine(const float* y, const float* s, const int32_t*, const float*,
                          uint16_t*, int64_t T, int32_t H, int32_t k, int32_t, int32_t,
                          hipStream_t) {
  ++stub::launches;
  stub::in_ws(y, 4 * T * k * H, "y");
  stub::in_ws(s, 4 * T * H, "s");
  return hipSuccess;
}
hipError_t launch_route(const float*, int64_t, int32_t, int32_t, int32_t*, float*, hipStream_t) {
  ++stub::launches;
  return hipSuccess;
}
}  // namespace moe
