// abi_check.cpp -- drives the host side of the C ABI (argument validation,
// launch planning, the per-thread memo of the last validated call) under
// AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU (built and run
// by tests/test_sanitize_cpu.py).
//
// The library's host code calls two HIP runtime functions.  This program
// defines both: hipLaunchKernel records the launch instead of enqueuing it,
// and hipGetErrorString names the stand-in.  The kernel tables are stand-ins
// too (a non-null tag per compiled kernel, never called), so nothing here
// touches a GPU or the HIP runtime, and successful calls are exercised as
// well as rejected ones.  Pointers are fake device addresses that are never
// dereferenced.
//
// Checks, besides the sanitizers' own: every call on a grid of valid
// problems launches once with the grid and workgroup rn_describe_launch_ex
// reports, kernel arguments that match the call, and a grid that covers
// every row; a repeated call launches the same; a rejected call launches
// nothing and leaves the next call's launch intact; a seeded fuzz over
// random (mostly invalid) arguments keeps the same invariants.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <random>

#include "resnorm.h"
#include "rn_args.h"

namespace {

struct Rec {
  const void* fn;
  dim3 grid, block;
  rn::RowArgs a;
  void* stream;
  long n = 0;
} g_rec;

long g_fail = 0, g_calls = 0;

#define CHECK(cond, ...)            \
  do {                              \
    if (!(cond)) {                  \
      fprintf(stderr, __VA_ARGS__); \
      fputc('\n', stderr);          \
      ++g_fail;                     \
    }                               \
  } while (0)

}  // namespace

extern "C" hipError_t hipLaunchKernel(const void* function_address, dim3 numBlocks, dim3 dimBlocks,
                                      void** args, size_t sharedMemBytes, hipStream_t stream) {
  g_rec.fn = function_address;
  g_rec.grid = numBlocks;
  g_rec.block = dimBlocks;
  memcpy(&g_rec.a, args[0], sizeof g_rec.a);
  g_rec.stream = (void*)stream;
  ++g_rec.n;
  (void)sharedMemBytes;
  return hipSuccess;
}

extern "C" const char* hipGetErrorString(hipError_t) { return "stand-in"; }

// Kernel tables: a tag for each compiled (family, affine, shape); multi-row
// shapes exist only for the norm-only op with weight.
namespace rn {
static KernelFn tag(int family, int aff, int shape, bool nss) {
  if (shape < 0 || shape >= kNumShapes || aff < 0 || aff >= kNumAff) return nullptr;
  if (kShapes[shape].k > 1 && !(nss && aff != kAffNone)) return nullptr;
  return (KernelFn)(uintptr_t)(0x1000000 + family * 0x10000 + aff * 0x100 + shape);
}
#define RN_TABLE(name, family, nss) \
  KernelFn name(int aff, int shape) { return tag(family, aff, shape, nss); }
RN_TABLE(kernels_fused_ln_bf16, 0, false)
RN_TABLE(kernels_fused_ln_f32, 1, false)
RN_TABLE(kernels_fused_ln_fp8, 2, false)
RN_TABLE(kernels_fused_ln_gate_bf16, 3, false)
RN_TABLE(kernels_fused_ln_gate_f32, 4, false)
RN_TABLE(kernels_fused_ln_gate_fp8, 5, false)
RN_TABLE(kernels_fused_rms_bf16, 6, false)
RN_TABLE(kernels_fused_rms_f32, 7, false)
RN_TABLE(kernels_fused_rms_fp8, 8, false)
RN_TABLE(kernels_fused_rms_gate_bf16, 9, false)
RN_TABLE(kernels_fused_rms_gate_f32, 10, false)
RN_TABLE(kernels_fused_rms_gate_fp8, 11, false)
RN_TABLE(kernels_nss_ln_bf16, 12, true)
RN_TABLE(kernels_nss_ln_f32, 13, true)
RN_TABLE(kernels_nss_ln_fp8, 14, true)
RN_TABLE(kernels_nss_rms_bf16, 15, true)
RN_TABLE(kernels_nss_rms_f32, 16, true)
RN_TABLE(kernels_nss_rms_fp8, 17, true)
}  // namespace rn

namespace {

// Fake device addresses, 2^49 bytes apart (more than any tensor the ABI
// accepts), 256-byte aligned.
uintptr_t base(int i) { return ((uintptr_t)(i + 1) << 49); }

struct Call {
  bool fused = true;
  int64_t B = 1, L = 16, D = 5120;
  uint32_t flags = RN_GATE;
  rn_layout gl{RN_BCAST, 0}, sl{RN_BCAST, 0};
  float eps = 1e-6f;
  int aff_dtype = RN_DTYPE_BF16, y_dtype = RN_DTYPE_BF16;
  uintptr_t y = base(0), ro = base(1), x = base(2), res = base(3), gate = base(4), w = base(5),
            b = base(6), sc = base(7), sh = base(8), ys = base(9);
  void* stream = (void*)(uintptr_t)0x5000;

  rn_status go() const {
    rn_ext ext{aff_dtype, y_dtype, y_dtype == RN_DTYPE_FP8_E4M3 ? (void*)ys : nullptr};
    const void* pw = (flags & RN_WEIGHT) ? (void*)w : nullptr;
    const void* pb = (flags & RN_BIAS) ? (void*)b : nullptr;
    ++g_calls;
    if (fused) {
      const void* pg = (flags & RN_GATE) ? (void*)gate : nullptr;
      return resnorm_fused_fwd_ex((void*)y, (void*)ro, (void*)x, (void*)res, pg, pw, pb, (void*)sc,
                                  (void*)sh, B, L, D, flags, gl, sl, eps, &ext, stream);
    }
    return norm_scale_shift_fwd_ex((void*)y, (void*)x, pw, pb, (void*)sc, (void*)sh, B, L, D, flags, sl,
                                   eps, &ext, stream);
  }
};

// What a successful call must have launched.
void check_launch(const Call& c, long launches_before, const char* what) {
  const int64_t R = c.B * c.L;
  if (R == 0) {
    CHECK(g_rec.n == launches_before, "%s: empty problem launched", what);
    return;
  }
  CHECK(g_rec.n == launches_before + 1, "%s: %ld launches for one call", what, g_rec.n - launches_before);
  rn_ext ext{c.aff_dtype, c.y_dtype, nullptr};
  rn_launch_info info{};
  const rn_status st = rn_describe_launch_ex(c.B, c.L, c.D, c.flags, c.fused, c.gl, c.sl, &ext, &info);
  CHECK(st == RN_OK, "%s: describe_launch %d: %s", what, st, rn_last_error());
  const uint64_t gx = g_rec.grid.x, gy = g_rec.grid.y;
  CHECK(g_rec.block.x == (uint32_t)info.block_threads && g_rec.block.y == 1 && g_rec.block.z == 1,
        "%s: block %u, describe says %d", what, g_rec.block.x, info.block_threads);
  CHECK(g_rec.block.x <= 1024 && g_rec.block.x % 64 == 0, "%s: block %u", what, g_rec.block.x);
  CHECK(gx * g_rec.block.x <= UINT32_MAX && gy * g_rec.block.x <= UINT32_MAX, "%s: grid too large", what);
  CHECK(gx * gy >= (uint64_t)info.grid_blocks && (gx * gy - (uint64_t)info.grid_blocks) < gx,
        "%s: grid %llux%llu for %lld blocks", what, (unsigned long long)gx, (unsigned long long)gy,
        (long long)info.grid_blocks);
  CHECK((uint64_t)info.grid_blocks * info.rows_per_block >= (uint64_t)R, "%s: grid misses rows", what);
  CHECK(g_rec.fn != nullptr && g_rec.stream == c.stream, "%s: kernel or stream", what);
  const rn::RowArgs& a = g_rec.a;
  CHECK(a.rows == (uint32_t)R && a.L == (uint32_t)c.L && a.d == (uint32_t)c.D && a.nvec == (uint32_t)(c.D / 8),
        "%s: sizes in the kernel arguments", what);
  CHECK(a.x == (void*)c.x && a.y == (void*)c.y && a.scale == (void*)c.sc && a.shift == (void*)c.sh,
        "%s: pointers in the kernel arguments", what);
  CHECK(memcmp(&a.eps, &c.eps, sizeof a.eps) == 0, "%s: eps", what);
  CHECK(a.ss_kind == c.sl.kind, "%s: scale/shift layout", what);
  if (c.sl.kind == RN_FRAME)
    CHECK(a.ss_frames == (uint32_t)c.sl.frames && a.ss_tokens_per_frame * (uint32_t)c.sl.frames == (uint32_t)c.L,
          "%s: frames", what);
}

void valid_grid() {
  static const int64_t widths[] = {8, 16, 136, 520, 2048, 2560, 3072, 4096, 4104, 5120, 6144, 8192, 10240, 16384};
  static const int64_t rows[] = {1, 7, 16, 32, 100, 128, 129, 256, 257, 512, 513, 768, 769,
                                 1024, 1025, 1536, 1537, 3072, 65536, 90000, 176400, 6711887, 2147483647};
  for (int64_t D : widths)
    for (int64_t R : rows)
      for (int fused = 0; fused <= 1; ++fused)
        for (uint32_t flags = 0; flags < 16; ++flags) {
          if ((flags & RN_BIAS) && !(flags & RN_WEIGHT)) continue;
          if (!fused && (flags & RN_GATE)) continue;
          for (int lay = 0; lay < 3; ++lay)
            for (int dt = 0; dt < 3; ++dt) {
              Call c;
              c.fused = fused;
              c.flags = flags;
              c.D = D;
              c.B = (R % 2 == 0 && lay == 2) ? 2 : 1;
              c.L = R / c.B;
              c.sl = lay == 0 ? rn_layout{RN_BCAST, 0} : lay == 1 ? rn_layout{RN_ROW, 0}
                                                             : rn_layout{RN_FRAME, c.L % 4 == 0 ? 4 : 1};
              c.gl = (lay == 2) ? c.sl : rn_layout{RN_BCAST, 0};
              c.aff_dtype = (dt & 1) ? RN_DTYPE_F32 : RN_DTYPE_BF16;
              c.y_dtype = dt;
              char what[160];
              snprintf(what, sizeof what, "fused=%d flags=%u D=%lld B=%lld L=%lld lay=%d dt=%d", fused, flags,
                       (long long)D, (long long)c.B, (long long)c.L, lay, dt);
              long n0 = g_rec.n;
              rn_status st = c.go();
              CHECK(st == RN_OK, "%s: status %d: %s", what, st, rn_last_error());
              if (st == RN_OK) check_launch(c, n0, what);
              // the same call again (the memo): the same launch
              const Rec first = g_rec;
              n0 = g_rec.n;
              st = c.go();
              CHECK(st == RN_OK, "%s: repeat status %d", what, st);
              if (st == RN_OK) {
                check_launch(c, n0, what);
                CHECK(g_rec.fn == first.fn && g_rec.grid.x == first.grid.x && g_rec.grid.y == first.grid.y,
                      "%s: repeat launched differently", what);
              }
            }
        }
}

void rejected_calls_leave_no_trace() {
  Call good;
  good.y_dtype = RN_DTYPE_BF16;
  struct Bad {
    const char* what;
    void (*mutate)(Call&);
    rn_status want;
  } bads[] = {
      {"D % 8", [](Call& c) { c.D = 5124; }, RN_EINVAL},
      {"D too large", [](Call& c) { c.D = RN_D_MAX + 8; }, RN_EUNSUPPORTED},
      {"negative L", [](Call& c) { c.L = -1; }, RN_EINVAL},
      {"2^31 rows", [](Call& c) { c.B = 2; c.L = 1LL << 30; }, RN_EUNSUPPORTED},
      {"unknown flag", [](Call& c) { c.flags |= 1u << 7; }, RN_EINVAL},
      {"bias without weight", [](Call& c) { c.flags |= RN_BIAS; }, RN_EINVAL},
      {"bad layout", [](Call& c) { c.sl = rn_layout{7, 0}; }, RN_EINVAL},
      {"frames do not divide L", [](Call& c) { c.sl = rn_layout{RN_FRAME, 5}; }, RN_EINVAL},
      {"nan eps", [](Call& c) { c.eps = __builtin_nanf(""); }, RN_EINVAL},
      {"negative eps", [](Call& c) { c.eps = -1e-6f; }, RN_EINVAL},
      {"misaligned x", [](Call& c) { c.x += 8; }, RN_EINVAL},
      {"y overlaps x", [](Call& c) { c.y = c.x + 16; }, RN_EINVAL},
      {"residual_out overlaps shift", [](Call& c) { c.ro = c.sh; }, RN_EINVAL},
      {"bad y dtype", [](Call& c) { c.y_dtype = 9; }, RN_EINVAL},
      {"bad affine dtype", [](Call& c) { c.flags |= RN_WEIGHT; c.aff_dtype = 5; }, RN_EINVAL},
  };
  for (const Bad& bad : bads) {
    // a valid call, so the memo holds it; then the rejected variant; then the
    // valid call again, which must launch as before
    long n0 = g_rec.n;
    CHECK(good.go() == RN_OK, "%s: valid call rejected: %s", bad.what, rn_last_error());
    check_launch(good, n0, bad.what);
    Call c = good;
    bad.mutate(c);
    n0 = g_rec.n;
    const rn_status st = c.go();
    CHECK(st == bad.want, "%s: status %d, want %d (%s)", bad.what, st, bad.want, rn_last_error());
    CHECK(g_rec.n == n0, "%s: a rejected call launched", bad.what);
    CHECK(rn_last_error()[0] != '\0', "%s: no message", bad.what);
    n0 = g_rec.n;
    CHECK(good.go() == RN_OK && rn_last_error()[0] == '\0', "%s: valid call after a rejected one", bad.what);
    check_launch(good, n0, bad.what);
  }
  // exact aliasing is allowed; alternating two problems keeps each one's launch
  Call inplace = good;
  inplace.y = inplace.x;
  inplace.ro = inplace.res;
  for (int i = 0; i < 4; ++i) {
    const Call& c = (i % 2) ? inplace : good;
    long n0 = g_rec.n;
    CHECK(c.go() == RN_OK, "aliasing %d: %s", i, rn_last_error());
    check_launch(c, n0, "alternating problems");
    CHECK(g_rec.a.y == (void*)c.y && g_rec.a.residual_out == (void*)c.ro, "alternating problems: stale arguments");
  }
}

void fuzz(uint64_t seed, int n) {
  std::mt19937_64 rng(seed);
  auto pick = [&](int64_t lo, int64_t hi) { return lo + (int64_t)(rng() % (uint64_t)(hi - lo + 1)); };
  for (int i = 0; i < n; ++i) {
    Call c;
    c.fused = rng() & 1;
    c.B = pick(-2, 5) * ((rng() % 8 == 0) ? (1LL << 29) : 1);
    c.L = pick(-2, 300000) * ((rng() % 16 == 0) ? (1LL << 20) : 1);
    c.D = (rng() % 4 == 0) ? pick(-16, 20000) : 8 * pick(0, 2100);
    c.flags = (uint32_t)(rng() % 40);
    const int32_t kinds[] = {RN_BCAST, RN_ROW, RN_FRAME, 3, -1};
    c.sl = rn_layout{kinds[rng() % 5], (int32_t)pick(-3, 60)};
    c.gl = rn_layout{kinds[rng() % 5], (int32_t)pick(-3, 60)};
    const float epss[] = {1e-6f, 0.f, -0.f, 1e-2f, -1e-6f, __builtin_inff(), __builtin_nanf("")};
    c.eps = epss[rng() % 7];
    c.aff_dtype = (int)pick(-1, 3);
    c.y_dtype = (int)pick(-1, 3);
    for (uintptr_t* p : {&c.y, &c.ro, &c.x, &c.res, &c.gate, &c.w, &c.b, &c.sc, &c.sh, &c.ys}) {
      const int r = (int)(rng() % 16);
      if (r == 0) *p = 0;                        // null
      else if (r == 1) *p += 4;                  // misaligned
      else if (r == 2) *p = base(2) + 256 * (uintptr_t)pick(0, 64);  // into x
    }
    const long n0 = g_rec.n;
    const rn_status st = c.go();
    CHECK(st == RN_OK || st == RN_EINVAL || st == RN_EUNSUPPORTED, "fuzz %d: status %d", i, st);
    if (st == RN_OK) {
      char what[64];
      snprintf(what, sizeof what, "fuzz %d", i);
      check_launch(c, n0, what);
    } else {
      CHECK(g_rec.n == n0, "fuzz %d: rejected call launched", i);
      CHECK(rn_last_error()[0] != '\0', "fuzz %d: no message", i);
    }
  }
}

}  // namespace

int main() {
  valid_grid();
  rejected_calls_leave_no_trace();
  fuzz(20261203, 300000);
  printf("abi_check: %ld calls, %ld launches, %ld failures\n", g_calls, g_rec.n, g_fail);
  return g_fail ? 1 : 0;
}
