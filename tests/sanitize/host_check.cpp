// Drives every entry point of the library's host code (csrc/api.cpp, built
// with the stand-ins of host_stubs.cpp) over valid and invalid problems: the
// argument checks must return the documented status before any launch, and
// valid calls must carve every workspace array inside the workspace. Built
// with AddressSanitizer and UndefinedBehaviorSanitizer; exits non-zero on the
// first failed expectation count.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "moe_w4a16.h"

namespace stub {
void set_workspace(const void* p, size_t n);
void select_scratch();
extern int launches;
extern int bad;
}  // namespace stub

static int checks = 0, fails = 0;
#define EXPECT(cond)                                              \
  do {                                                            \
    ++checks;                                                     \
    if (!(cond)) {                                                \
      fprintf(stderr, "line %d: expected %s\n", __LINE__, #cond); \
      ++fails;                                                    \
    }                                                             \
  } while (0)

// Stand-ins for device pointers: 256-byte aligned, never dereferenced.
alignas(256) static char dev[4096];
static void* D(int i) { return dev + 256 * i; }

static moe_w4a16_problem mk(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                            int32_t base = 0) {
  moe_w4a16_problem p;
  p.num_tokens = T;
  p.hidden = H;
  p.inter = I;
  p.num_experts = E;
  p.expert_base = base;
  p.top_k = k;
  p.group_size = 32;
  return p;
}

static int fwd(const moe_w4a16_problem& p, void* ws, size_t bytes, const void* shared = D(7),
               const void* x = D(0)) {
  return moe_w4a16_forward(x, (const int32_t*)D(1), (const float*)D(2), (const int32_t*)D(3),
                           D(4), (const int32_t*)D(5), D(6), shared, D(8), &p, ws, bytes,
                           nullptr);
}

static void invalid_problems() {
  size_t b = 0;
  EXPECT(moe_w4a16_workspace_size(nullptr, &b) == MOE_ERR_NULL);
  moe_w4a16_problem p = mk(4, 7168, 2048, 384, 8);
  p.group_size = 64;
  EXPECT(moe_w4a16_workspace_size(&p, &b) == MOE_ERR_UNSUPPORTED);
  EXPECT((p = mk(-1, 7168, 2048, 384, 8), moe_w4a16_workspace_size(&p, &b)) == MOE_ERR_SHAPE);
  EXPECT((p = mk(4, 100, 2048, 384, 8), moe_w4a16_workspace_size(&p, &b)) == MOE_ERR_SHAPE);
  EXPECT((p = mk(4, 7168, 2016, 384, 8), moe_w4a16_workspace_size(&p, &b)) == MOE_ERR_SHAPE);
  EXPECT((p = mk(4, 0, 2048, 384, 8), moe_w4a16_workspace_size(&p, &b)) == MOE_ERR_SHAPE);
  EXPECT((p = mk(4, 7168, 2048, 0, 8), moe_w4a16_workspace_size(&p, &b)) == MOE_ERR_SHAPE);
  EXPECT((p = mk(4, 7168, 2048, 384, 0), moe_w4a16_workspace_size(&p, &b)) == MOE_ERR_SHAPE);
  EXPECT((p = mk(4, 7168, 2048, 384, 17), moe_w4a16_workspace_size(&p, &b)) == MOE_ERR_SHAPE);
  EXPECT((p = mk(4, 7168, 2048, 513, 8), moe_w4a16_workspace_size(&p, &b)) ==
         MOE_ERR_UNSUPPORTED);
  EXPECT((p = mk(4, 7168, 2048, 384, 8, -1), moe_w4a16_workspace_size(&p, &b)) ==
         MOE_ERR_SHAPE);
  EXPECT((p = mk(4, 7168, 2048, 384, 8, 0x7fffff00), moe_w4a16_workspace_size(&p, &b)) ==
         MOE_ERR_SHAPE);
  EXPECT((p = mk(0x7ffffffe / 8 + 1, 7168, 2048, 384, 8), moe_w4a16_workspace_size(&p, &b)) ==
         MOE_ERR_SHAPE);
  // arrays a buffer resource would address beyond 2 GiB
  EXPECT((p = mk(200000, 7168, 2048, 384, 8), moe_w4a16_workspace_size(&p, &b)) ==
         MOE_ERR_UNSUPPORTED);
  EXPECT((p = mk(4, 65536, 16384, 8, 2), moe_w4a16_workspace_size(&p, &b)) ==
         MOE_ERR_UNSUPPORTED);
  // status strings of every code
  for (int s = -8; s <= 1; ++s) EXPECT(moe_w4a16_status_string(s) != nullptr);
}

// One problem through every entry point that takes it.
static void valid_problem(const moe_w4a16_problem& p) {
  size_t bytes = 0;
  EXPECT(moe_w4a16_workspace_size(&p, &bytes) == MOE_OK);
  int32_t bm = 0;
  EXPECT(moe_w4a16_forward_block_m(&p, &bm) == MOE_OK);
  EXPECT(bm == 4 || bm == 96);
  // (not zeroed: the stand-ins never touch it)
  char* const ws = static_cast<char*>(malloc(bytes + 512));
  char* w = ws + (256 - ((uintptr_t)ws & 255));
  stub::set_workspace(w, bytes);
  const int before = stub::launches;
  stub::bad = 0;
  EXPECT(fwd(p, w, bytes) == MOE_OK);
  EXPECT(fwd(p, w, bytes, nullptr) == MOE_OK);  // no shared expert
  EXPECT(stub::bad == 0);
  EXPECT(p.num_tokens == 0 ? stub::launches == before : stub::launches > before);
  void* events[7] = {};
  EXPECT(moe_w4a16_forward_timed(D(0), (const int32_t*)D(1), (const float*)D(2),
                                 (const int32_t*)D(3), D(4), (const int32_t*)D(5), D(6), D(7),
                                 D(8), &p, w, bytes, nullptr, events) == MOE_OK);
  if (p.num_tokens > 0) {
    // the range checks are live: half the workspace registered is caught
    stub::set_workspace(w, bytes / 2);
    EXPECT(fwd(p, w, bytes) == MOE_OK);
    EXPECT(stub::bad > 0);
    stub::bad = 0;
    stub::set_workspace(w, bytes);
    EXPECT(fwd(p, w, bytes - 1) == MOE_ERR_WORKSPACE);
    EXPECT(fwd(p, nullptr, bytes) == MOE_ERR_NULL);
    EXPECT(fwd(p, w, bytes, D(7), nullptr) == MOE_ERR_NULL);
    EXPECT(fwd(p, w, bytes, D(7), dev + 8) == MOE_ERR_ALIGNMENT);
    EXPECT(fwd(p, w + 8, bytes) == MOE_ERR_ALIGNMENT);
  }
  EXPECT(stub::bad == 0);

  // bucketing entry points
  int64_t scap = 0, bcap = 0;
  EXPECT(moe_w4a16_align_capacity(&p, bm, &scap, &bcap) == MOE_OK);
  size_t sbytes = 0;
  EXPECT(moe_w4a16_align_scratch_size(&p, &sbytes) == MOE_OK);
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t o_blk = up(4 * (size_t)scap), o_np = o_blk + up(4 * (size_t)bcap),
               o_scr = o_np + 256, a_bytes = o_scr + up(sbytes);
  std::vector<char> al(a_bytes + 256);
  char* a = al.data() + (256 - ((uintptr_t)al.data() & 255));
  stub::set_workspace(a, a_bytes);
  int32_t* sid = (int32_t*)a;
  int32_t* blk = (int32_t*)(a + o_blk);
  int32_t* np = (int32_t*)(a + o_np);
  void* scr = sbytes ? (void*)(a + o_scr) : nullptr;
  EXPECT(moe_w4a16_align((const int32_t*)D(1), &p, bm, sid, scap, blk, bcap, np, scr, sbytes,
                         nullptr) == MOE_OK);
  if (p.num_tokens > 0)
    EXPECT(moe_w4a16_align((const int32_t*)D(1), &p, bm, sid, scap - 1, blk, bcap, np, scr,
                           sbytes, nullptr) == MOE_ERR_WORKSPACE);
  EXPECT(moe_w4a16_align((const int32_t*)D(1), &p, 0, sid, scap, blk, bcap, np, scr, sbytes,
                         nullptr) != MOE_OK);
  EXPECT(stub::bad == 0);

  // router step
  EXPECT(moe_w4a16_route((const float*)D(2), 384 > p.top_k ? 384 : p.top_k, &p,
                         (int32_t*)D(1), (float*)D(2), nullptr) == MOE_OK);
  EXPECT(moe_w4a16_route((const float*)D(2), p.top_k - 1, &p, (int32_t*)D(1), (float*)D(2),
                         nullptr) != MOE_OK);
  stub::set_workspace(w, bytes);
  EXPECT(moe_w4a16_forward_scores(D(0), (const float*)D(2), 384, (const int32_t*)D(3), D(4),
                                  (const int32_t*)D(5), D(6), D(7), D(8), (int32_t*)D(1),
                                  (float*)D(2), &p, w, bytes, nullptr) == MOE_OK);
  EXPECT(stub::bad == 0);

  // prepacked weights: widths that are whole 512-row tiles
  size_t pk = 0;
  const int st = moe_w4a16_prepack_size(&p, &pk);
  if (st == MOE_OK) {
    EXPECT(moe_w4a16_prepack((const int32_t*)D(3), D(4), (const int32_t*)D(5), D(6), &p, D(9),
                             pk, nullptr) == MOE_OK);
    EXPECT(moe_w4a16_prepack((const int32_t*)D(3), D(4), (const int32_t*)D(5), D(6), &p, D(9),
                             pk - 1, nullptr) == MOE_ERR_WORKSPACE);
    stub::set_workspace(w, bytes);
    EXPECT(moe_w4a16_forward_prepacked(D(0), (const int32_t*)D(1), (const float*)D(2), D(9), pk,
                                       D(7), D(8), &p, w, bytes, nullptr) == MOE_OK);
    if (p.num_tokens > 0)
      EXPECT(moe_w4a16_forward_prepacked(D(0), (const int32_t*)D(1), (const float*)D(2), D(9),
                                         pk - 1, D(7), D(8), &p, w, bytes,
                                         nullptr) == MOE_ERR_WORKSPACE);
    EXPECT(stub::bad == 0);
  } else {
    EXPECT(st == MOE_ERR_UNSUPPORTED);
  }

  // allocation-free entry point: its own workspace, up to its limit
  size_t limit = 0;
  EXPECT(moe_w4a16_noalloc_workspace_limit(&limit) == MOE_OK);
  stub::select_scratch();
  const int na = moe_w4a16_forward_noalloc(D(0), (const int32_t*)D(1), (const float*)D(2),
                                           (const int32_t*)D(3), D(4), (const int32_t*)D(5),
                                           D(6), D(7), D(8), &p, nullptr);
  EXPECT(na == (bytes <= limit ? MOE_OK : MOE_ERR_WORKSPACE));
  EXPECT(stub::bad == 0);
  free(ws);
}

int main() {
  invalid_problems();
  // (T, H, I, E, k, base): decode, the bucketing inside gate_up (<= 16
  // pairs), the 96-row path with whole and masked tiles, expert base, many
  // pairs (bucketing in several launches), the tensor-parallel share, empty
  const int64_t cases[][6] = {
      {1, 7168, 2048, 384, 8, 0},  {2, 7168, 2048, 384, 8, 0},  {8, 7168, 2048, 384, 8, 0},
      {64, 7168, 2048, 384, 8, 0}, {300, 7168, 2048, 384, 8, 0}, {512, 7168, 2048, 48, 8, 0},
      {33, 640, 384, 8, 4, 0},     {97, 384, 640, 6, 2, 2},       {5, 1152, 640, 6, 3, 1},
      {1200, 1024, 256, 8, 8, 0},  {64, 7168, 256, 384, 8, 0},    {0, 7168, 2048, 384, 8, 0},
  };
  for (const auto& c : cases)
    valid_problem(mk(c[0], (int32_t)c[1], (int32_t)c[2], (int32_t)c[3], (int32_t)c[4],
                     (int32_t)c[5]));
  printf("host checks: %d, failed: %d, launches: %d\n", checks, fails, stub::launches);
  return fails ? 1 : 0;
}
